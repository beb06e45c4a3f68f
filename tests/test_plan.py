"""Host-side tests of the mixed-precision layer plan."""
import pytest

from group_wise_affine_qlinear_amd import plan


def test_modulation_and_conditioning_stay_8bit_in_every_policy():
    for policy in plan.POLICIES:
        assert plan.role_bits(policy, "adaln_modulation") == 8
        assert plan.role_bits(policy, "llm_cond_proj") == 8
        assert plan.role_bits(policy, "adaln_modulation", bulk_bits=3) == 8


def test_bulk_width_per_policy_and_override():
    for role in ("attn_qkv", "attn_out", "mlp_gate_up", "mlp_down"):
        assert plan.role_bits("mixed_3_8", role) == 3
        assert plan.role_bits("mixed_4_8", role) == 4
        assert plan.role_bits("mixed_3_8", role, bulk_bits=4) == 4
    with pytest.raises(ValueError):
        plan.role_bits("mixed_3_8", "attn_qkv", bulk_bits=5)
    with pytest.raises(ValueError):
        plan.role_bits("nf4", "attn_qkv")
    with pytest.raises(ValueError):
        plan.role_bits("mixed_3_8", "embedding")


def test_planned_parameters_match_the_dit_size():
    # the paper notes' table gives 9.3B DiT parameters; the planned projections
    # (34 blocks + llm_cond_proj) hold nearly all of them
    p = plan.model_plan("mixed_4_8")
    total = sum(x.params for x in p)
    assert total == 34 * (3 * 4608 * 4608 + 4608 * 4608 + 2 * 12288 * 4608 + 4608 * 12288 + 6 * 4608 * 512) \
        + 4608 * 53248
    assert 9.0e9 < total < 9.5e9


def test_bits_per_weight_closed_form():
    bulk = 34 * (3 * 4608 * 4608 + 4608 * 4608 + 2 * 12288 * 4608 + 4608 * 12288)
    eight = 34 * 6 * 4608 * 512 + 4608 * 53248
    for policy, b in (("mixed_3_8", 3), ("mixed_4_8", 4)):
        want = ((b + 0.5) * bulk + 8.5 * eight) / (bulk + eight)
        assert abs(plan.bits_per_weight(plan.model_plan(policy)) - want) < 1e-12
    assert plan.bits_per_weight(plan.model_plan("uniform_8")) == 8.5
    assert plan.bits_per_weight(plan.block_projections("mixed_3_8")[:1]) == 3.5
