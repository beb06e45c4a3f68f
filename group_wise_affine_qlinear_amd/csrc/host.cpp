// C ABI of libqlinear: argument validation, dispatch, workspace, host packer
// and host RTN quantizer. Kernels live in gemm.hip, skinny.hip and misc.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/qlinear.h"
#include "ql_kernels.h"

#define QL_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kGroup = 64;
constexpr int kMaxSkinnyM = 16;

thread_local char g_last_path[160] = "none";

void set_last_path(const char *s) {
  std::snprintf(g_last_path, sizeof(g_last_path), "%s", s);
}

bool bits_ok(int bits) { return bits == 2 || bits == 3 || bits == 4 || bits == 8; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// fp32 -> IEEE half bit pattern, round-half-to-even (overflow -> inf).
uint16_t f32_to_f16(float f) {
  uint32_t x;
  std::memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return (uint16_t)(sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u : 0u));
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // >= 65520 rounds to inf
  if (ax < 0x38800000u) {                                    // below 2^-14: subnormal or zero
    if (ax < 0x33000000u) return (uint16_t)sign;             // below 2^-25
    const uint32_t e = ax >> 23;
    const uint32_t m = (ax & 0x7FFFFFu) | 0x800000u;
    const uint32_t shift = 126u - e;                         // value / 2^-24 = m >> shift
    uint32_t q = m >> shift;
    const uint32_t rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1u);
    if (rem > half || (rem == half && (q & 1u))) ++q;
    return (uint16_t)(sign | q);
  }
  const uint32_t e = (ax >> 23) - 112u;
  const uint32_t m = ax & 0x7FFFFFu;
  uint32_t q = (e << 10) | (m >> 13);
  const uint32_t rem = m & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) ++q;
  return (uint16_t)(sign | q);
}

float f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  uint32_t x;
  if (e == 0) {
    if (m == 0) {
      x = sign;
    } else {  // subnormal: value = m * 2^-24, exact in fp32
      float v = std::ldexp((float)m, -24);
      std::memcpy(&x, &v, 4);
      x |= sign;
    }
  } else if (e == 31) {
    x = sign | 0x7F800000u | (m << 13);
  } else {
    x = sign | ((e + 112u) << 23) | (m << 13);
  }
  float f;
  std::memcpy(&f, &x, 4);
  return f;
}

// ---- scratch of qlinear_forward_noalloc: a fixed device array in this
// library's code object (each device that loads the library holds its own
// copy until the process ends). Host code never passes the array's name to a
// kernel: its device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and kept per device.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

struct ScratchAddress {
  std::once_flag once;
  void *ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchAddress g_scratch_address[kMaxDevices];

int noalloc_scratch(void **out) {
  *out = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QL_EHIP;
  ScratchAddress &s = g_scratch_address[dev];
  std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  if (s.err != hipSuccess || s.ptr == nullptr) return QL_EHIP;
  *out = s.ptr;
  return QL_OK;
}

// ---- dispatch
struct Plan {
  int path = QL_PATH_AUTO;
  int mode = QL_MODE_EXACT;
  int tile = 0;
  int splits = 1;
  int groups_per_split = 0;
  size_t ws_xsum = 0, ws_partial = 0;
  size_t ws_x16 = 0;  // fast mode: fp16 x and per-row scales
  bool online = false;  // fast mode without them: the GEMM converts x itself
  bool copy = false;  // canonical 3-bit codes: the GEMM runs on a tiled copy in the workspace
  ql::Gemm2Plan g2{};
  ql::Gemm3Plan g3{};
};

// What a call brings besides the operands; it decides which plans need no
// library scratch. scratch: a workspace is passed (scratch plans allowed);
// x16, xsum: the caller's FAST activations / EXACT group sums.
struct Caller {
  bool scratch = false, x16 = false, xsum = false;
  bool epilogue = false;  // a fused epilogue (its FAST GEMM takes prepared fp16 activations)
};

size_t ti_sizes(int tile) {
  const ql::TileInfo *t = ql::gemm_tile(tile);
  return t ? (size_t)t->bm * (size_t)t->bn : 0;
}

int env_int(const char *name, int dflt) {
  const char *v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

// Static tile table from sweeps on MI355X, with a heuristic default. Entries:
// bits (0 = any), M range, N range, K range -> tile id and split count
// (0 = heuristic split).
struct TableEntry {
  int bits;
  int64_t m_lo, m_hi, n_lo, n_hi, k_lo, k_hi;
  int tile, splits;
};
// Exact-mode large-M tiles for canonical codes, from a sweep of tiles 1, 2, 3,
// 5, 10, 11 over the DiT projection shapes on one MI355X (first match wins):
//  - 8-bit: the 128 x 128 first-generation tile (gate/up 4608x24576: 1.80 ms
//    against 2.30 ms for tile 10; down 12288->4608: 0.97 against 1.21 ms);
//  - M <= 383: the 64 x 128 tile (M=256, N=K=4608: 48 us against 52 us);
//  - larger M: the second-generation 256 x 128 tile, which stages codes and x
//    by LDS DMA (QKV 4608x13824: 0.82 ms against 0.99 ms for tile 1; 2048^2
//    2-bit sweep 16896x13824: 2.85 against 3.40 ms; llm_cond_proj with its
//    8-way K split: 0.49 against 0.60 ms).
const TableEntry kTable[] = {
    {8, 17, 1LL << 40, 1, 1LL << 40, 1, 1LL << 40, 1, 0},
    {0, 17, 383, 1, 1LL << 40, 1, 1LL << 40, 5, 0},
    {0, 384, 1LL << 40, 1, 1LL << 40, 1, 1LL << 40, 10, 0},
};

int choose_splits(int64_t tiles, int G) {
  // Fill ~2 waves of blocks on 256 CUs when the tile grid alone is small;
  // keep at least 8 groups per split.
  if (tiles >= 256 || G < 16) return 1;
  int s = (int)((512 + tiles - 1) / tiles);
  if (s > G / 8) s = G / 8;
  if (s > 16) s = 16;
  return s < 1 ? 1 : s;
}

// Large-M tiles of the FAST (gemm3.hip) and SPLIT (gemm4.hip) numerics.
constexpr int kFastTile = 20;
constexpr int kSplitTile = 30;

// Workspace bytes of a tiled copy of canonical weights (codes, then scale|bias
// words, each 256-byte aligned).
size_t repack_ws_bytes(int bits, int64_t N, int64_t K) {
  const int64_t n32 = round_up(N, 32);
  return (size_t)round_up(n32 * K * bits / 32 * 4, 256) + (size_t)round_up(n32 * (K / kGroup) * 4, 256);
}

// Plans a forward call. Automatic numerics for the large-M path: FAST, with
// its activations from the caller, from a prepass into the workspace, or
// (no workspace) converted inside the GEMM, which needs no scratch; K is
// split only with a workspace, and a grid of fewer tiles than CUs that is not
// split along K is cut into row pieces instead. Canonical 3-bit codes run
// every GEMM on a tiled copy in the workspace.
int make_plan(int bits, int64_t M, int64_t N, int64_t K, int force_path, int force_split,
              int force_tile, bool tiled, int mode, Caller c, Plan *p) {
  *p = Plan{};  // a re-plan into the same Plan keeps no field of the previous one
  const int G = (int)(K / kGroup);
  int path = force_path;
  if (path == QL_PATH_AUTO) {
    const int envp = env_int("QLINEAR_FORCE_PATH", 0);
    if (envp > 0) path = envp;
  }
  if (path == QL_PATH_AUTO) path = (M <= kMaxSkinnyM) ? QL_PATH_SKINNY : QL_PATH_GEMM;
  if (path == QL_PATH_SKINNY) {
    if (M > kMaxSkinnyM || mode == QL_MODE_FAST || mode == QL_MODE_SPLIT) return QL_EUNSUPPORTED;
    p->path = QL_PATH_SKINNY;
    p->mode = QL_MODE_EXACT;
    return QL_OK;
  }
  if (path != QL_PATH_GEMM && path != QL_PATH_SPLITK) return QL_EUNSUPPORTED;
  int tile = force_tile > 0 ? force_tile : env_int("QLINEAR_TILE", 0);
  const ql::TileInfo *forced = tile > 0 ? ql::gemm_tile(tile) : nullptr;
  if (tile > 0 && !forced) return QL_EUNSUPPORTED;
  // canonical codes on the FAST and SPLIT GEMMs are addressed with 32-bit byte offsets
  const bool canon_big = !tiled && bits != 3 && N * (K * bits / 8) > (int64_t)INT32_MAX;
  if (mode == QL_MODE_AUTO) {
    if (forced) mode = forced->gen == 3 ? QL_MODE_FAST : forced->gen == 4 ? QL_MODE_SPLIT : QL_MODE_EXACT;
    else if (canon_big) mode = QL_MODE_EXACT;
    else mode = QL_MODE_FAST;  // with no workspace and no fp16 activations the GEMM converts x itself
  }
  if (mode != QL_MODE_EXACT && mode != QL_MODE_FAST && mode != QL_MODE_SPLIT) return QL_EINVAL;
  p->mode = mode;
  // the GEMMs read 3-bit codes in the tiled layout only
  p->copy = bits == 3 && !tiled;
  if (p->copy) tiled = true;
  if (mode == QL_MODE_FAST || mode == QL_MODE_SPLIT) {
    const int gen = mode == QL_MODE_FAST ? 3 : 4;
    if (canon_big) return QL_EUNSUPPORTED;
    if (forced && forced->gen != gen) return QL_EUNSUPPORTED;
    int fs = force_split > 0 ? force_split : 0;
    if (path == QL_PATH_GEMM && force_path == QL_PATH_GEMM) fs = force_split > 0 ? force_split : 1;
    if (path == QL_PATH_SPLITK && fs < 2) fs = 2;
    if (fs <= 0 && !c.scratch) fs = 1;  // no workspace: no K split
    if (fs > G) fs = G;
    // QLINEAR_GEMM_SLOTS: resident-block count override, for tests of the
    // tail pieces and K splits on small shapes
    p->g3 = ql::gemm3_plan(M, N, G, env_int("QLINEAR_GEMM_SLOTS", 0), fs, true);
    if (path == QL_PATH_SPLITK && p->g3.splits < 2) return QL_EUNSUPPORTED;
    p->path = p->g3.splits > 1 ? QL_PATH_SPLITK : QL_PATH_GEMM;
    p->tile = gen == 3 ? kFastTile : kSplitTile;
    p->splits = p->g3.splits;
    p->groups_per_split = G > 0 ? (G + p->splits - 1) / p->splits : 0;
    // FAST activations: the caller's, else a prepass into the workspace, else
    // (no workspace) converted inside the GEMM
    if (mode == QL_MODE_FAST && !c.x16) {
      if (c.scratch || c.epilogue) p->ws_x16 = (size_t)round_up(M * K * 2, 256) + (size_t)round_up(M * 4, 256);
      else p->online = true;
    }
    p->ws_partial = p->g3.partial_bytes;
    return QL_OK;
  }
  if (forced && forced->gen >= 3) return QL_EUNSUPPORTED;
  // 3-bit codes: second-generation tiles only
  if (bits == 3 && forced && forced->gen != 2) return QL_EUNSUPPORTED;
  int splits = 0;
  if (tile <= 0) {
    for (const TableEntry &e : kTable) {
      if ((e.bits == 0 || e.bits == bits) && M >= e.m_lo && M <= e.m_hi && N >= e.n_lo && N <= e.n_hi &&
          K >= e.k_lo && K <= e.k_hi) {
        tile = e.tile;
        splits = e.splits;
        break;
      }
    }
    if (tile <= 0) tile = 1;
    // exact mode on tiled codes: the second-generation kernel (the 256-row
    // tile does not fit two blocks per CU with 8-bit codes)
    if (tiled && !ql::gemm_tile_supports_tiled(tile)) tile = bits == 8 ? 11 : 10;
  }
  const ql::TileInfo *ti = ql::gemm_tile(tile);
  if (!ti) return QL_EUNSUPPORTED;
  const int64_t tiles = ((M + ti->bm - 1) / ti->bm) * ((N + ti->bn - 1) / ti->bn);
  if (force_split > 0) splits = force_split;
  if (splits <= 0) splits = choose_splits(tiles, G);
  if (path == QL_PATH_GEMM && force_path == QL_PATH_GEMM) splits = force_split > 0 ? force_split : 1;
  if (path == QL_PATH_SPLITK && splits < 2) splits = G >= 2 ? 2 : 1;
  if (splits > G) splits = G > 0 ? G : 1;
  const int gps = G > 0 ? (G + splits - 1) / splits : 0;
  if (G > 0) splits = (G + gps - 1) / gps;  // no empty split
  if (path == QL_PATH_SPLITK && splits < 2) return QL_EUNSUPPORTED;
  p->path = splits > 1 ? QL_PATH_SPLITK : QL_PATH_GEMM;
  p->tile = tile;
  p->splits = splits;
  p->groups_per_split = gps;
  p->ws_xsum = c.xsum ? 0 : (size_t)G * (size_t)round_up(M, 256) * 4u;
  p->ws_partial = splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * 4u : 0;
  if (ti->gen == 2) {
    // QLINEAR_GEMM_SLOTS: as above
    p->g2 = ql::gemm2_plan(bits, tile, M, N, G, splits, env_int("QLINEAR_GEMM_SLOTS", 0));
    if (p->g2.sk_partial_bytes > p->ws_partial) p->ws_partial = p->g2.sk_partial_bytes;
  }
  return QL_OK;
}

// Scratch bytes a plan takes from the workspace (the tiled copy of canonical
// 3-bit codes is added by the caller, it depends on N and K).
size_t plan_ws(const Plan &p) {
  if (p.path == QL_PATH_SKINNY) return 0;
  return (size_t)round_up((int64_t)p.ws_xsum, 256) + (size_t)round_up((int64_t)p.ws_x16, 256) + p.ws_partial;
}

size_t plan_total_ws(const Plan &p, int bits, int64_t N, int64_t K) {
  const size_t need = (size_t)round_up((int64_t)plan_ws(p), 256);
  return need + (p.copy && p.path != QL_PATH_SKINNY ? repack_ws_bytes(bits, N, K) : 0);
}

int validate_forward(const ql_forward_args *a) {
  if (!a) return QL_EINVAL;
  if (!bits_ok(a->bits) || a->group != kGroup) return QL_EUNSUPPORTED;
  if (a->M < 0 || a->N < 0 || a->K < 0 || a->K % kGroup) return QL_EINVAL;
  if (a->M > (1LL << 31) - 1 || a->N > (1LL << 31) - 1 || a->K > (1LL << 30)) return QL_EINVAL;
  if (a->out_dtype != QL_OUT_F32 && a->out_dtype != QL_OUT_BF16) return QL_EINVAL;
  if (a->layout != QL_LAYOUT_CANONICAL && a->layout != QL_LAYOUT_TILED) return QL_EINVAL;
  if (a->mode != QL_MODE_AUTO && a->mode != QL_MODE_EXACT && a->mode != QL_MODE_FAST && a->mode != QL_MODE_SPLIT)
    return QL_EINVAL;
  if ((a->x16 == nullptr) != (a->rowscale == nullptr)) return QL_EINVAL;
  if (a->epilogue != QL_EPI_NONE && a->epilogue != QL_EPI_SWIGLU && a->epilogue != QL_EPI_GATE_RESIDUAL)
    return QL_EINVAL;
  if (a->epilogue != QL_EPI_NONE) {
    if (a->mode == QL_MODE_EXACT || a->mode == QL_MODE_SPLIT || a->path == QL_PATH_SKINNY ||
        a->path == QL_PATH_SPLITK || a->split_k > 1)
      return QL_EUNSUPPORTED;
    // the GLU order is a tiled repack
    if (a->epilogue == QL_EPI_SWIGLU && a->layout != QL_LAYOUT_TILED) return QL_EUNSUPPORTED;
  }
  if (a->epilogue == QL_EPI_SWIGLU && a->N % 32) return QL_EINVAL;
  if (a->epilogue == QL_EPI_GATE_RESIDUAL) {
    if (a->gate_rows < 1) return QL_EINVAL;
    if (a->M > 0 && a->N > 0 && (!a->residual || !a->gate)) return QL_EINVAL;
    if (reinterpret_cast<uintptr_t>(a->gate) & 3u) return QL_EALIGN;
    if (reinterpret_cast<uintptr_t>(a->residual) & (a->out_dtype == QL_OUT_BF16 ? 1u : 3u)) return QL_EALIGN;
  }
  if (a->M == 0 || a->N == 0) return QL_OK;
  if (!a->out) return QL_EINVAL;
  if (!aligned16(a->out)) return QL_EALIGN;
  if (a->K == 0) return QL_OK;
  const bool tiled = a->layout == QL_LAYOUT_TILED;
  if (!a->x || !a->packed_q || !a->scales || (!tiled && !a->biases)) return QL_EINVAL;
  if (!aligned16(a->x) || !aligned16(a->packed_q)) return QL_EALIGN;
  if (tiled) {
    if (reinterpret_cast<uintptr_t>(a->scales) & 3u) return QL_EALIGN;
  } else if ((reinterpret_cast<uintptr_t>(a->scales) & 1u) || (reinterpret_cast<uintptr_t>(a->biases) & 1u)) {
    return QL_EALIGN;
  }
  if (a->xsum) {
    if (a->ld_xsum < round_up(a->M, 256) || a->ld_xsum % 4) return QL_EINVAL;
    if (!aligned16(a->xsum)) return QL_EALIGN;
  }
  if (a->x16 && !aligned16(a->x16)) return QL_EALIGN;
  return QL_OK;
}

}  // namespace

QL_API int qlinear_version(void) { return 100; }

QL_API const char *qlinear_status_string(int status) {
  switch (status) {
    case QL_OK: return "ok";
    case QL_EINVAL: return "invalid argument (size, null pointer or K not a multiple of 64)";
    case QL_EALIGN: return "misaligned pointer (x, out and packed_q need 16-byte alignment)";
    case QL_EUNSUPPORTED: return "unsupported (bits must be 2, 3, 4 or 8; group 64; 3-bit needs the tiled layout; or forced path cannot serve shape)";
    case QL_EWORKSPACE: return "workspace missing or too small";
    case QL_EHIP: return "HIP runtime error";
    case QL_ERANGE: return "non-finite weight or f16 overflow of scale/bias";
    default: return "unknown status";
  }
}

QL_API int qlinear_last_path(char *buf, size_t len) {
  if (!buf || len == 0) return QL_EINVAL;
  std::snprintf(buf, len, "%s", g_last_path);
  return QL_OK;
}

QL_API size_t qlinear_packed_words(int bits, int64_t N, int64_t K) {
  if (!bits_ok(bits) || N < 0 || K < 0) return 0;
  return (size_t)N * (size_t)K * (size_t)bits / 32u;
}

QL_API size_t qlinear_workspace_bytes(int bits, int64_t M, int64_t N, int64_t K) {
  if (!bits_ok(bits) || M <= 0 || N <= 0 || K <= 0 || K % kGroup) return 0;
  // the largest need over both layouts and every numerics mode a call with a
  // workspace may run under automatic path selection
  Caller c;
  c.scratch = true;
  size_t need = 0;
  for (bool tiled : {false, true})
    for (int mode : {QL_MODE_AUTO, QL_MODE_EXACT, QL_MODE_FAST, QL_MODE_SPLIT}) {
      Plan p;
      if (make_plan(bits, M, N, K, QL_PATH_AUTO, 0, 0, tiled, mode, c, &p) != QL_OK) continue;
      need = std::max(need, plan_total_ws(p, bits, N, K));
    }
  // the fused epilogues run the FAST GEMM at every M, with no K split
  for (bool tiled : {false, true}) {
    Plan p;
    if (make_plan(bits, M, N, K, QL_PATH_GEMM, 1, 0, tiled, QL_MODE_FAST, c, &p) == QL_OK)
      need = std::max(need, plan_total_ws(p, bits, N, K));
  }
  return need;
}

QL_API size_t qlinear_forward_workspace_bytes(const ql_forward_args *a) {
  if (!a) return 0;
  // size the call as if it had a workspace: the pointer is only checked for alignment
  ql_forward_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (validate_forward(&b) != QL_OK || b.M == 0 || b.N == 0 || b.K == 0) return 0;
  Caller c;
  c.scratch = true;
  c.x16 = b.x16 != nullptr;
  c.xsum = b.xsum != nullptr;
  const bool fused = b.epilogue == QL_EPI_SWIGLU || b.epilogue == QL_EPI_GATE_RESIDUAL;
  const bool tiled = b.layout == QL_LAYOUT_TILED;
  Plan p;
  const int st = fused ? make_plan(b.bits, b.M, b.N, b.K, QL_PATH_GEMM, 1, b.tile, tiled, QL_MODE_FAST, c, &p)
                       : make_plan(b.bits, b.M, b.N, b.K, b.path, b.split_k, b.tile, tiled, b.mode, c, &p);
  return st == QL_OK ? plan_total_ws(p, b.bits, b.N, b.K) : 0;
}

QL_API int qlinear_forward_ex(const ql_forward_args *a, void *stream_v) {
  int st = validate_forward(a);
  if (st != QL_OK) return st;
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
  if (a->M == 0 || a->N == 0) {
    set_last_path("noop");
    return QL_OK;
  }
  const bool glu = a->epilogue == QL_EPI_SWIGLU;
  const bool gated = a->epilogue == QL_EPI_GATE_RESIDUAL;
  const int64_t n_out = glu ? a->N / 2 : a->N;
  if (a->K == 0 && gated) {
    // y = 0: the gated update leaves the residual stream as it is
    set_last_path("copy_residual");
    if (a->residual == a->out) return QL_OK;
    const size_t bytes = (size_t)(a->M * a->N) * (a->out_dtype == QL_OUT_BF16 ? 2 : 4);
    return hipMemcpyAsync(a->out, a->residual, bytes, hipMemcpyDeviceToDevice, stream) == hipSuccess ? QL_OK
                                                                                                   : QL_EHIP;
  }
  if (a->K == 0) {
    set_last_path("fill_zero");
    return ql::launch_fill_zero(a->out, a->M * n_out, a->out_dtype == QL_OUT_BF16, stream) == hipSuccess ? QL_OK
                                                                                                        : QL_EHIP;
  }
  Plan p;
  Caller c;
  c.scratch = a->workspace != nullptr;
  c.x16 = a->x16 != nullptr;
  c.xsum = a->xsum != nullptr;
  c.epilogue = glu || gated;
  const bool tiled_in = a->layout == QL_LAYOUT_TILED;
  // the fused epilogues run on the FAST GEMM without a K split (they need
  // finished sums), at any M
  st = (glu || gated) ? make_plan(a->bits, a->M, a->N, a->K, QL_PATH_GEMM, 1, a->tile, tiled_in, QL_MODE_FAST, c, &p)
                      : make_plan(a->bits, a->M, a->N, a->K, a->path, a->split_k, a->tile, tiled_in, a->mode, c, &p);
  if (st != QL_OK) return st;
  const int G = (int)(a->K / kGroup);
  const int out_bf16 = a->out_dtype == QL_OUT_BF16;
  char buf[160];
  if (p.path == QL_PATH_SKINNY) {
    ql::SkinnyArgs s{static_cast<const uint16_t *>(a->x),
                     a->packed_q,
                     tiled_in ? nullptr : static_cast<const uint16_t *>(a->scales),
                     tiled_in ? nullptr : static_cast<const uint16_t *>(a->biases),
                     tiled_in ? static_cast<const uint32_t *>(a->scales) : nullptr,
                     a->out, a->M, a->N, a->K, G, out_bf16, tiled_in ? 1 : 0};
    // one or two rows on canonical weights: the lane-along-K GEMV (its
    // loads read whole lines of a row); QLINEAR_NO_GEMV=1 keeps the skinny
    // kernel, for comparisons
    if (ql::gemv_chunks_per_lane(a->bits, a->M, a->K, tiled_in ? 1 : 0) > 0 && !env_int("QLINEAR_NO_GEMV", 0)) {
      std::snprintf(buf, sizeof(buf), "gemv_b%d_m%lld_canonical", a->bits, (long long)a->M);
      set_last_path(buf);
      return ql::launch_gemv(a->bits, s, stream) == hipSuccess ? QL_OK : QL_EHIP;
    }
    std::snprintf(buf, sizeof(buf), "skinny_b%d_m%lld_%s", a->bits, (long long)a->M, tiled_in ? "tiled" : "canonical");
    set_last_path(buf);
    return ql::launch_skinny(a->bits, s, stream) == hipSuccess ? QL_OK : QL_EHIP;
  }
  const bool copy = p.copy;
  const bool plan_tiled = tiled_in || copy;
  if (plan_tiled && !ql::gemm_tile_supports_tiled(p.tile)) return QL_EUNSUPPORTED;
  // scratch comes only from the caller's workspace: a plan that needs some
  // without one is refused before anything is launched
  const size_t plan_need = (size_t)round_up((int64_t)plan_ws(p), 256);
  const size_t need = plan_total_ws(p, a->bits, a->N, a->K);
  void *ws = a->workspace;
  if (need > 0) {
    if (!ws || a->workspace_bytes < need) return QL_EWORKSPACE;
    if (!aligned16(ws)) return QL_EALIGN;
  }
  ql_forward_args tiled_args;
  if (copy) {
    uint32_t *tq = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + plan_need);
    uint32_t *tsb = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(tq) +
                                                 round_up((int64_t)qlinear_tiled_words(a->bits, a->N, a->K) * 4, 256));
    if (ql::launch_repack(a->bits, a->packed_q, static_cast<const uint16_t *>(a->scales),
                          static_cast<const uint16_t *>(a->biases), a->N, a->K, 0, tq, tsb, stream) != hipSuccess)
      return QL_EHIP;
    tiled_args = *a;
    tiled_args.packed_q = tq;
    tiled_args.scales = tsb;
    tiled_args.biases = nullptr;
    tiled_args.layout = QL_LAYOUT_TILED;
    a = &tiled_args;
  }
  const bool canon = a->layout == QL_LAYOUT_CANONICAL;
  const char *lay = canon ? "canonical" : (copy ? "tiled_copy" : "tiled");
  if (p.mode == QL_MODE_FAST || p.mode == QL_MODE_SPLIT) {
    const bool fast = p.mode == QL_MODE_FAST;
    // the GEMM reads x16: the caller's fp16 activations, the prepass output
    // below, or the bf16 x itself (SPLIT, and FAST converting in the GEMM)
    const uint16_t *x16 = static_cast<const uint16_t *>(fast && !p.online ? a->x16 : a->x);
    const float *rowscale = fast && !p.online ? a->rowscale : nullptr;
    char *after = static_cast<char *>(ws) + round_up((int64_t)p.ws_x16, 256);
    if (fast && !p.online && !x16) {
      if (!ws) return QL_EWORKSPACE;  // the plan asked for it: checked above, kept as a guard
      uint16_t *x16w = static_cast<uint16_t *>(ws);
      float *rsw = reinterpret_cast<float *>(static_cast<char *>(ws) + round_up(a->M * a->K * 2, 256));
      if (ql::launch_x16(static_cast<const uint16_t *>(a->x), x16w, rsw, a->M, a->K, stream) != hipSuccess)
        return QL_EHIP;
      x16 = x16w;
      rowscale = rsw;
    }
    const bool split = p.g3.splits > 1;
    float *partial = reinterpret_cast<float *>(after);
    ql::Gemm3Args g3{x16, rowscale, a->packed_q, static_cast<const uint32_t *>(a->scales),
                     split ? static_cast<void *>(partial) : a->out,
                     a->M, a->N, a->K, G, split ? 0 : out_bf16,
                     p.g3.dp_tiles, p.g3.tail_tiles, p.g3.tail_mi, p.g3.splits, p.g3.grid_x, glu ? 1 : 0,
                     gated ? a->residual : nullptr, gated ? a->gate : nullptr,
                     gated ? (int)std::min<int64_t>(a->gate_rows, a->M) : 0,
                     canon ? 1 : 0, canon ? static_cast<const uint16_t *>(a->scales) : nullptr,
                     canon ? static_cast<const uint16_t *>(a->biases) : nullptr};
    const char *kname = p.online ? "gemm3_f16online" : fast ? "gemm3_f16" : "gemm4_bf16x2";
    if (gated)
      std::snprintf(buf, sizeof(buf), "%s_256x256_b%d%s_gate_%s", kname, a->bits, p.g3.tail_tiles > 0 ? "_tail" : "",
                    lay);
    else if (glu)
      std::snprintf(buf, sizeof(buf), "%s_256x256_b%d%s_swiglu_tiled", kname, a->bits,
                    p.g3.tail_tiles > 0 ? "_tail" : "");
    else if (split)
      std::snprintf(buf, sizeof(buf), "%s_256x256_b%d_split%d_%s", kname, a->bits, p.g3.splits, lay);
    else if (p.g3.tail_tiles > 0)
      std::snprintf(buf, sizeof(buf), "%s_256x256_b%d_tail%dx%d_%s", kname, a->bits, p.g3.tail_tiles,
                    16 / p.g3.tail_mi, lay);
    else
      std::snprintf(buf, sizeof(buf), "%s_256x256_b%d_%s", kname, a->bits, lay);
    set_last_path(buf);
    const hipError_t le = p.online ? ql::launch_gemm3_online(a->bits, g3, stream)
                          : fast     ? ql::launch_gemm3(a->bits, g3, stream)
                                     : ql::launch_gemm4(a->bits, g3, stream);
    if (le != hipSuccess) return QL_EHIP;
    if (split && ql::launch_splitk_reduce(partial, p.g3.splits, a->M, a->N, a->out, out_bf16, stream) != hipSuccess)
      return QL_EHIP;
    return QL_OK;
  }
  int64_t Mp = round_up(a->M, 256);
  float *xsum = static_cast<float *>(ws);
  float *partial = reinterpret_cast<float *>(static_cast<char *>(ws) + round_up((int64_t)p.ws_xsum, 256));
  if (a->xsum) {
    xsum = const_cast<float *>(a->xsum);
    Mp = a->ld_xsum;
  } else if (ql::launch_xsum(static_cast<const uint16_t *>(a->x), xsum, a->M, a->K, Mp, stream) != hipSuccess) {
    return QL_EHIP;
  }
  const bool tiled = a->layout == QL_LAYOUT_TILED;
  ql::GemmArgs g{static_cast<const uint16_t *>(a->x),
                 a->packed_q,
                 tiled ? nullptr : static_cast<const uint16_t *>(a->scales),
                 tiled ? nullptr : static_cast<const uint16_t *>(a->biases),
                 tiled ? static_cast<const uint32_t *>(a->scales) : nullptr,
                 xsum,
                 a->out,
                 partial,
                 a->M, a->N, a->K, Mp,
                 G,
                 p.splits,
                 p.groups_per_split,
                 out_bf16,
                 p.g2.dp_tiles, p.g2.sk_tiles, p.g2.sk_pieces, p.g2.grid_x,
                 nullptr, nullptr};
  if (p.g2.sk_tiles > 0) {
    const size_t part = (size_t)p.g2.sk_tiles * p.g2.sk_pieces * ti_sizes(p.tile);
    g.sk_partial = partial;
    g.sk_count = reinterpret_cast<int *>(reinterpret_cast<char *>(partial) + round_up((int64_t)part * 4, 256));
    if (ql::launch_fill_zero(g.sk_count, p.g2.sk_tiles, 0, stream) != hipSuccess) return QL_EHIP;
  }
  const ql::TileInfo *ti = ql::gemm_tile(p.tile);
  if (p.g2.sk_tiles > 0)
    std::snprintf(buf, sizeof(buf), "%s_b%d_split%d_tail%dx%d_%s", ti ? ti->name : "gemm", a->bits, p.splits,
                  p.g2.sk_tiles, p.g2.sk_pieces, lay);
  else
    std::snprintf(buf, sizeof(buf), "%s_b%d_split%d_%s", ti ? ti->name : "gemm", a->bits, p.splits, lay);
  set_last_path(buf);
  const hipError_t le = (ti && ti->gen == 2) ? ql::launch_gemm2(a->bits, p.tile, tiled, g, stream)
                                             : ql::launch_gemm(a->bits, p.tile, g, stream);
  if (le != hipSuccess) return QL_EHIP;
  if (p.splits > 1) {
    if (ql::launch_splitk_reduce(partial, p.splits, a->M, a->N, a->out, out_bf16, stream) != hipSuccess)
      return QL_EHIP;
  }
  return QL_OK;
}

QL_API int qlinear_forward_noalloc(const ql_forward_args *a, void *stream) {
  if (!a) return QL_EINVAL;
  if (a->workspace || a->workspace_bytes) return QL_EINVAL;
  // argument errors first, then the scratch need against the array's size,
  // both before the scratch address is looked up or anything launched
  int st = validate_forward(a);
  if (st != QL_OK) return st;
  if (qlinear_forward_workspace_bytes(a) > kNoallocScratchBytes) return QL_EWORKSPACE;
  void *ptr = nullptr;
  st = noalloc_scratch(&ptr);
  if (st != QL_OK) return st;
  ql_forward_args b = *a;
  b.workspace = ptr;
  b.workspace_bytes = kNoallocScratchBytes;
  return qlinear_forward_ex(&b, stream);
}

QL_API size_t qlinear_forward_noalloc_max_scratch(void) { return kNoallocScratchBytes; }

QL_API int64_t qlinear_group_sums_ld(int64_t M) { return M <= 0 ? 0 : round_up(M, 256); }

QL_API int qlinear_fast_activations(const void *x, int64_t M, int64_t K, void *x16, float *rowscale,
                                    void *stream) {
  if (M < 0 || K < 0 || K % kGroup) return QL_EINVAL;
  if (M == 0 || K == 0) return QL_OK;
  if (!x || !x16 || !rowscale) return QL_EINVAL;
  if (!aligned16(x) || !aligned16(x16)) return QL_EALIGN;
  set_last_path("fast_activations");
  return ql::launch_x16(static_cast<const uint16_t *>(x), static_cast<uint16_t *>(x16), rowscale, M, K,
                        reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? QL_OK
             : QL_EHIP;
}

QL_API int qlinear_fast_activations_adaln(const void *x, const float *scale, int64_t scale_rows, int64_t M, int64_t K,
                                          void *x16, float *rowscale, void *stream) {
  if (M < 0 || K < 0 || K % kGroup || scale_rows < 1) return QL_EINVAL;
  if (M == 0 || K == 0) return QL_OK;
  if (!x || !x16 || !rowscale || !scale) return QL_EINVAL;
  if (!aligned16(x) || !aligned16(x16) || !aligned16(scale)) return QL_EALIGN;
  set_last_path("fast_activations_adaln");
  return ql::launch_x16(static_cast<const uint16_t *>(x), static_cast<uint16_t *>(x16), rowscale, M, K,
                        reinterpret_cast<hipStream_t>(stream), scale, scale_rows) == hipSuccess
             ? QL_OK
             : QL_EHIP;
}

QL_API int qlinear_group_sums(const void *x, int64_t M, int64_t K, float *xsum, int64_t ld_xsum, void *stream) {
  if (M < 0 || K < 0 || K % kGroup) return QL_EINVAL;
  if (M == 0 || K == 0) return QL_OK;
  if (!x || !xsum) return QL_EINVAL;
  if (ld_xsum < round_up(M, 256) || ld_xsum % 4) return QL_EINVAL;
  if (!aligned16(x) || !aligned16(xsum)) return QL_EALIGN;
  set_last_path("group_sums");
  return ql::launch_xsum(static_cast<const uint16_t *>(x), xsum, M, K, ld_xsum,
                         reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? QL_OK
             : QL_EHIP;
}

QL_API int qlinear_forward(const void *x, const uint32_t *packed_q, const void *scales, const void *biases,
                           int bits, int group, int64_t M, int64_t N, int64_t K, float *out) {
  ql_forward_args a;
  std::memset(&a, 0, sizeof(a));
  a.x = x;
  a.packed_q = packed_q;
  a.scales = scales;
  a.biases = biases;
  a.bits = bits;
  a.group = group;
  a.M = M;
  a.N = N;
  a.K = K;
  a.out = out;
  a.out_dtype = QL_OUT_F32;
  return qlinear_forward_ex(&a, nullptr);
}

// Code k of a row sits in bits [bits*k, bits*k + bits) of the row's
// little-endian bit stream (bit i of the stream = bit i % 32 of word i / 32);
// 3-bit codes may straddle two words.
QL_API int qlinear_pack_host(const uint8_t *q, int bits, int64_t N, int64_t K, uint32_t *packed) {
  if (!bits_ok(bits)) return QL_EUNSUPPORTED;
  if (N < 0 || K < 0 || (K * bits) % 32) return QL_EINVAL;
  if (N * K > 0 && (!q || !packed)) return QL_EINVAL;
  const uint32_t lim = 1u << bits;
  for (int64_t i = 0; i < N * K; ++i)
    if (q[i] >= lim) return QL_ERANGE;
  const int64_t wr = K * bits / 32;
  for (int64_t n = 0; n < N; ++n) {
    uint32_t *row = packed + n * wr;
    for (int64_t j = 0; j < wr; ++j) row[j] = 0;
    for (int64_t k = 0; k < K; ++k) {
      const uint32_t v = q[n * K + k];
      const int64_t p = k * bits;
      const int sh = (int)(p % 32);
      row[p / 32] |= v << sh;
      if (sh + bits > 32) row[p / 32 + 1] |= v >> (32 - sh);
    }
  }
  return QL_OK;
}

QL_API int qlinear_unpack_host(const uint32_t *packed, int bits, int64_t N, int64_t K, uint8_t *q) {
  if (!bits_ok(bits)) return QL_EUNSUPPORTED;
  if (N < 0 || K < 0 || (K * bits) % 32) return QL_EINVAL;
  if (N * K > 0 && (!q || !packed)) return QL_EINVAL;
  const uint32_t mask = (1u << bits) - 1u;
  const int64_t wr = K * bits / 32;
  for (int64_t n = 0; n < N; ++n) {
    const uint32_t *row = packed + n * wr;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t p = k * bits;
      const int sh = (int)(p % 32);
      uint32_t v = row[p / 32] >> sh;
      if (sh + bits > 32) v |= row[p / 32 + 1] << (32 - sh);
      q[n * K + k] = (uint8_t)(v & mask);
    }
  }
  return QL_OK;
}

QL_API int qlinear_quantize_rtn_host(const float *w, int bits, int group, int64_t N, int64_t K, uint8_t *q,
                                     uint16_t *s16, uint16_t *b16) {
  if (!bits_ok(bits) || group != kGroup) return QL_EUNSUPPORTED;
  if (N < 0 || K < 0 || K % kGroup) return QL_EINVAL;
  if (N * K > 0 && (!w || !q || !s16 || !b16)) return QL_EINVAL;
  const int64_t G = K / kGroup;
  const float qmax = (float)((1 << bits) - 1);
  for (int64_t i = 0; i < N * K; ++i)
    if (!std::isfinite(w[i])) return QL_ERANGE;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < G; ++g) {
      const float *wp = w + n * K + g * kGroup;
      // min/max order -0 below +0 (IEEE 754-2019 minimum/maximum)
      float mn = wp[0], mx = wp[0];
      for (int k = 1; k < kGroup; ++k) {
        const float v = wp[k];
        if (v < mn || (v == mn && std::signbit(v) && !std::signbit(mn))) mn = v;
        if (v > mx || (v == mx && !std::signbit(v) && std::signbit(mx))) mx = v;
      }
      volatile float diff = mx - mn;  // keep fp32 rounding of each step explicit
      volatile float s32 = diff / qmax;
      const uint16_t sh = f32_to_f16(s32), bh = f32_to_f16(mn);
      if ((sh & 0x7C00u) == 0x7C00u || (bh & 0x7C00u) == 0x7C00u) return QL_ERANGE;
      const float sf = f16_to_f32(sh), bf = f16_to_f32(bh);
      for (int k = 0; k < kGroup; ++k) {
        uint8_t code = 0;
        if (sf != 0.f) {
          volatile float d = wp[k] - bf;
          volatile float t = d / sf;
          float r = std::nearbyint((float)t);
          if (r < 0.f) r = 0.f;
          if (r > qmax) r = qmax;
          code = (uint8_t)r;
        }
        q[n * K + g * kGroup + k] = code;
      }
      s16[n * G + g] = sh;
      b16[n * G + g] = bh;
    }
  }
  return QL_OK;
}

QL_API int qlinear_quantize_rtn(const float *w, int bits, int group, int64_t N, int64_t K, uint32_t *packed_q,
                                uint16_t *scales, uint16_t *biases, int *status_dev, void *stream) {
  if (!bits_ok(bits) || group != kGroup) return QL_EUNSUPPORTED;
  if (N < 0 || K < 0 || K % kGroup) return QL_EINVAL;
  if (N == 0 || K == 0) return QL_OK;
  if (!w || !packed_q || !scales || !biases) return QL_EINVAL;
  if (!aligned16(w) || !aligned16(packed_q)) return QL_EALIGN;
  set_last_path("quantize_rtn");
  return ql::launch_quantize(bits, w, N, K, packed_q, scales, biases, status_dev,
                             reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? QL_OK
             : QL_EHIP;
}

QL_API int qlinear_quantize_imatrix(const float *w, const float *importance, int bits, int group, int64_t N,
                                    int64_t K, uint32_t *packed_q, uint16_t *scales, uint16_t *biases,
                                    int *status_dev, void *stream) {
  if (!bits_ok(bits) || group != kGroup) return QL_EUNSUPPORTED;
  if (N < 0 || K < 0 || K % kGroup) return QL_EINVAL;
  if (N == 0 || K == 0) return QL_OK;
  if (!w || !importance || !packed_q || !scales || !biases) return QL_EINVAL;
  if (!aligned16(w) || !aligned16(importance) || !aligned16(packed_q)) return QL_EALIGN;
  set_last_path("quantize_imatrix");
  return ql::launch_quantize_imatrix(bits, w, importance, N, K, packed_q, scales, biases, status_dev,
                                     reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? QL_OK
             : QL_EHIP;
}

QL_API size_t qlinear_tiled_words(int bits, int64_t N, int64_t K) {
  if (!bits_ok(bits) || N < 0 || K < 0 || K % kGroup) return 0;
  return (size_t)round_up(N, 32) * (size_t)K * (size_t)bits / 32u;
}

QL_API size_t qlinear_tiled_sb_words(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || K % kGroup) return 0;
  return (size_t)round_up(N, 32) * (size_t)(K / kGroup);
}

QL_API int qlinear_repack(const uint32_t *packed_q, const void *scales, const void *biases, int bits, int group,
                          int64_t N, int64_t K, uint32_t *tiled_q, uint32_t *tiled_sb, void *stream) {
  if (!bits_ok(bits) || group != kGroup) return QL_EUNSUPPORTED;
  if (N < 0 || K < 0 || K % kGroup) return QL_EINVAL;
  if (N == 0 || K == 0) return QL_OK;
  if (!packed_q || !scales || !biases || !tiled_q || !tiled_sb) return QL_EINVAL;
  if (!aligned16(packed_q) || !aligned16(tiled_q) || (reinterpret_cast<uintptr_t>(tiled_sb) & 3u)) return QL_EALIGN;
  set_last_path("repack");
  return ql::launch_repack(bits, packed_q, static_cast<const uint16_t *>(scales),
                           static_cast<const uint16_t *>(biases), N, K, 0, tiled_q, tiled_sb,
                           reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? QL_OK
             : QL_EHIP;
}

QL_API int qlinear_repack_glu(const uint32_t *packed_q, const void *scales, const void *biases, int bits, int group,
                              int64_t N, int64_t K, uint32_t *tiled_q, uint32_t *tiled_sb, void *stream) {
  if (!bits_ok(bits) || group != kGroup) return QL_EUNSUPPORTED;
  if (N < 0 || K < 0 || K % kGroup || N % 32) return QL_EINVAL;
  if (N == 0 || K == 0) return QL_OK;
  if (!packed_q || !scales || !biases || !tiled_q || !tiled_sb) return QL_EINVAL;
  if (!aligned16(packed_q) || !aligned16(tiled_q) || (reinterpret_cast<uintptr_t>(tiled_sb) & 3u)) return QL_EALIGN;
  set_last_path("repack_glu");
  return ql::launch_repack(bits, packed_q, static_cast<const uint16_t *>(scales),
                           static_cast<const uint16_t *>(biases), N, K, N / 2, tiled_q, tiled_sb,
                           reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? QL_OK
             : QL_EHIP;
}

QL_API int qlinear_unrepack(const uint32_t *tiled_q, const uint32_t *tiled_sb, int bits, int group, int64_t N,
                            int64_t K, uint32_t *packed_q, void *scales, void *biases, void *stream) {
  if (!bits_ok(bits) || group != kGroup) return QL_EUNSUPPORTED;
  if (N < 0 || K < 0 || K % kGroup) return QL_EINVAL;
  if (N == 0 || K == 0) return QL_OK;
  if (!packed_q || !scales || !biases || !tiled_q || !tiled_sb) return QL_EINVAL;
  if (!aligned16(packed_q) || !aligned16(tiled_q) || (reinterpret_cast<uintptr_t>(tiled_sb) & 3u)) return QL_EALIGN;
  set_last_path("unrepack");
  return ql::launch_unrepack(bits, tiled_q, tiled_sb, N, K, 0, packed_q, static_cast<uint16_t *>(scales),
                             static_cast<uint16_t *>(biases), reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? QL_OK
             : QL_EHIP;
}

QL_API int qlinear_unrepack_glu(const uint32_t *tiled_q, const uint32_t *tiled_sb, int bits, int group, int64_t N,
                                int64_t K, uint32_t *packed_q, void *scales, void *biases, void *stream) {
  if (!bits_ok(bits) || group != kGroup) return QL_EUNSUPPORTED;
  if (N < 0 || K < 0 || K % kGroup || N % 32) return QL_EINVAL;
  if (N == 0 || K == 0) return QL_OK;
  if (!packed_q || !scales || !biases || !tiled_q || !tiled_sb) return QL_EINVAL;
  if (!aligned16(packed_q) || !aligned16(tiled_q) || (reinterpret_cast<uintptr_t>(tiled_sb) & 3u)) return QL_EALIGN;
  set_last_path("unrepack_glu");
  return ql::launch_unrepack(bits, tiled_q, tiled_sb, N, K, N / 2, packed_q, static_cast<uint16_t *>(scales),
                             static_cast<uint16_t *>(biases), reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? QL_OK
             : QL_EHIP;
}

QL_API int qlinear_dequantize(const uint32_t *packed_q, const void *scales, const void *biases, int bits,
                              int group, int64_t N, int64_t K, float *w_out, void *stream) {
  if (!bits_ok(bits) || group != kGroup) return QL_EUNSUPPORTED;
  if (N < 0 || K < 0 || K % kGroup) return QL_EINVAL;
  if (N == 0 || K == 0) return QL_OK;
  if (!packed_q || !scales || !biases || !w_out) return QL_EINVAL;
  if (!aligned16(packed_q) || !aligned16(w_out)) return QL_EALIGN;
  set_last_path("dequantize");
  return ql::launch_dequant(bits, packed_q, static_cast<const uint16_t *>(scales),
                            static_cast<const uint16_t *>(biases), N, K, w_out,
                            reinterpret_cast<hipStream_t>(stream)) == hipSuccess
             ? QL_OK
             : QL_EHIP;
}
