"""Mixed-precision layer plan for the Ideogram 4 DiT projections.

A policy fixes the code width of every quantized projection: the modulation
(AdaLN) and conditioning (llm_cond_proj) projections stay at 8 bits in every
policy, because the modulation's scale and tanh gate multiply the whole
residual stream; the bulk projections (attention QKV and output, MLP gate/up
and down) take the policy's bulk width (Ideogram-4-IQ4_M card, sections
"Against the pack this replaces" and "Conversion": a 3-bit bulk in the older
pack, a 4-bit bulk with --bulk-bits 4, 8-bit modulation and conditioning in
every policy). Shapes follow the Ideogram 4 paper notes (section 2.8 table:
width 4608, MLP width 12288, 34 blocks, AdaLN width 512; section 2.3:
13 x 4096 = 53248 text features). Reading taken for the modulation: each
block maps the 512-wide AdaLN embedding to 6 x 4608 values (shift, scale and
gate for the attention and MLP branches; the skinny benchmark rows use the
configured 4608-wide input instead).

Host-side bookkeeping only: it chooses widths and sizes; the projections run
through ``qlinear_forward_ex``.
"""
from __future__ import annotations

from dataclasses import dataclass

WIDTH = 4608
MLP = 12288
ADALN = 512
BLOCKS = 34
TEXT_FEATURES = 53248
GROUP = 64

# role -> "bulk" or a fixed width
_ROLE_WIDTH = {
    "attn_qkv": "bulk",
    "attn_out": "bulk",
    "mlp_gate_up": "bulk",
    "mlp_down": "bulk",
    "adaln_modulation": 8,
    "llm_cond_proj": 8,
}

POLICIES = {
    "mixed_3_8": 3,   # 3-bit bulk, 8-bit modulation and conditioning
    "mixed_4_8": 4,   # the same policy with a 4-bit bulk
    "uniform_8": 8,   # every projection at 8 bits
}


@dataclass(frozen=True)
class Projection:
    name: str
    role: str
    N: int        # output features (weight rows)
    K: int        # input features
    bits: int

    @property
    def params(self) -> int:
        return self.N * self.K

    @property
    def storage_bytes(self) -> int:
        """Packed codes plus one f16 scale and one f16 bias per 64 weights."""
        return self.N * self.K * self.bits // 8 + 4 * self.N * (self.K // GROUP)


def role_bits(policy: str, role: str, bulk_bits: int | None = None) -> int:
    """Code width of a projection role under a policy (bulk_bits overrides the bulk width)."""
    if policy not in POLICIES:
        raise ValueError(f"unknown policy {policy!r}; one of {sorted(POLICIES)}")
    if role not in _ROLE_WIDTH:
        raise ValueError(f"unknown role {role!r}; one of {sorted(_ROLE_WIDTH)}")
    w = _ROLE_WIDTH[role]
    if w != "bulk":
        return w
    bulk = POLICIES[policy] if bulk_bits is None else bulk_bits
    if bulk not in (2, 3, 4, 8):
        raise ValueError(f"bulk width must be 2, 3, 4 or 8, got {bulk}")
    return bulk


def block_projections(policy: str, bulk_bits: int | None = None) -> list[Projection]:
    """The quantized projections of one DiT block."""
    shapes = [
        ("attn_qkv", "attn_qkv", 3 * WIDTH, WIDTH),
        ("attn_out", "attn_out", WIDTH, WIDTH),
        ("mlp_gate_up", "mlp_gate_up", 2 * MLP, WIDTH),
        ("mlp_down", "mlp_down", WIDTH, MLP),
        ("adaln_modulation", "adaln_modulation", 6 * WIDTH, ADALN),
    ]
    return [Projection(n, r, N, K, role_bits(policy, r, bulk_bits)) for n, r, N, K in shapes]


def model_plan(policy: str, bulk_bits: int | None = None) -> list[Projection]:
    """Every planned projection of the DiT: 34 blocks and the conditioning projection."""
    out = []
    for b in range(BLOCKS):
        out += [Projection(f"block{b}.{p.name}", p.role, p.N, p.K, p.bits)
                for p in block_projections(policy, bulk_bits)]
    out.append(Projection("llm_cond_proj", "llm_cond_proj", WIDTH, TEXT_FEATURES,
                          role_bits(policy, "llm_cond_proj", bulk_bits)))
    return out


def bits_per_weight(plan: list[Projection]) -> float:
    """Average stored bits per weight of a plan, group overhead included."""
    return 8.0 * sum(p.storage_bytes for p in plan) / sum(p.params for p in plan)
