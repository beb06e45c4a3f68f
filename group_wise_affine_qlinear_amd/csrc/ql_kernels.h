// Internal launcher interface between the C ABI (host.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ql {

struct GemmArgs {
  const uint16_t *x;      // bf16 [M, K]
  const uint32_t *w;      // packed codes [N, K*bits/32]
  const uint16_t *s;      // f16 [N, G] (canonical layout)
  const uint16_t *b;      // f16 [N, G] (canonical layout)
  const uint32_t *sb;     // scale|bias words (tiled layout)
  const float *xsum;      // [G, Mp] per-group row sums of x
  void *out;              // [M, N] fp32 or bf16 (splits == 1)
  float *partial;         // [splits, M, N] fp32 (splits > 1)
  int64_t M, N, K, Mp;
  int G;
  int splits;
  int groups_per_split;
  int out_bf16;
  // second-generation kernel only (see Gemm2Plan)
  int dp_tiles, sk_tiles, sk_pieces, grid_x;
  float *sk_partial;      // [sk_tiles, sk_pieces, BM*BN] fp32
  int *sk_count;          // [sk_tiles], zero before the launch; left zero after it
};

struct TileInfo {
  int id, bm, bn, warps_m, warps_n;
  const char *name;
  int gen;  // 1: gemm.hip (canonical, exact), 2: gemm2.hip (either layout, exact),
            // 3: gemm3.hip (either layout, fast), 4: gemm4.hip (either layout, split bf16)
};

// GEMM tile configurations compiled into the library (id >= 1).
const TileInfo *gemm_tile(int id);
bool gemm_tile_supports_tiled(int id);
int gemm_tile_count();
size_t gemm_lds_bytes(int bits, int id);

hipError_t launch_xsum(const uint16_t *x, float *xsum, int64_t M, int64_t K, int64_t Mp,
                       hipStream_t stream);
hipError_t launch_gemm(int bits, int tile_id, const GemmArgs &a, hipStream_t stream);
// second-generation kernel (gemm2.hip), tile ids >= 10, canonical or tiled codes
hipError_t launch_gemm2(int bits, int tile_id, bool tiled, const GemmArgs &a, hipStream_t stream);
size_t gemm2_lds_bytes(int bits, int id);
// Work split of one second-generation launch over the blocks the device holds
// at once (`slots`; <= 0 queries the device): dp_tiles whole tiles, then the
// remaining sk_tiles tiles cut into sk_pieces K-ranges each when the whole
// tiles leave part of the last round idle.
struct Gemm2Plan {
  int64_t tiles;
  int dp_tiles, sk_tiles, sk_pieces, grid_x;
  size_t sk_partial_bytes;  // includes the counters, 256-byte aligned pieces
};
Gemm2Plan gemm2_plan(int bits, int tile_id, int64_t M, int64_t N, int G, int splits, int slots);
// Fast mode (gemm3.hip): fp16 x with per-row power-of-two scales, tiled codes
// dequantized to fp16 in registers, 256 x 256 block tiles.
struct Gemm3Args {
  const uint16_t *x16;    // fp16 [M, K]
  const float *rowscale;  // [M], 2^e per row
  const uint32_t *w;      // tiled codes, or canonical codes [N, K*bits/32] when canon
  const uint32_t *sb;     // tiled scale|bias words (unused when canon)
  void *out;              // [M, N] fp32 or bf16; with splits > 1 fp32 [splits, M, N]
  int64_t M, N, K;
  int G;
  int out_bf16;           // ignored when splits > 1 (partials are fp32)
  int dp_tiles;           // whole tiles, t = blockIdx.x, + gridDim.x, ...
  int tail_tiles;         // tiles after dp_tiles, cut along M into 16/tail_mi pieces
  int tail_mi;            // 16-row subtiles per piece: 2, 4 or 8
  int splits;             // K ranges (grid y)
  int grid_x;
  int glu;                // 1: GLU-ordered weights, out = silu(gate) * up, [M, N/2]
  const void *residual;   // non-null with gate: out = residual + gate[m / gate_rows] * y
  const float *gate;      // fp32 [ceil(M / gate_rows), N]
  int gate_rows;          // 1 .. M (callers clamp larger values to M)
  int canon;              // 1: canonical codes with separate f16 scales and biases
  const uint16_t *s16;    // canonical scales [N, K/64] (canon only)
  const uint16_t *b16;    // canonical biases [N, K/64] (canon only)
};
struct Gemm3Plan {
  int64_t tiles;
  int dp_tiles, tail_tiles, tail_mi, splits, grid_x;
  size_t partial_bytes;   // splits > 1: fp32 [splits, M, N]
};
// slots <= 0: one block per CU of the current device; force_splits > 0 fixes
// the K split. fill_by_pieces: with fewer tiles than slots and no K split,
// cut every tile along M into row pieces so the grid covers the CUs (needs no
// scratch, unlike a K split).
Gemm3Plan gemm3_plan(int64_t M, int64_t N, int G, int slots, int force_splits, bool fill_by_pieces = false);
// mod_scale (fp32 [ceil(M / mod_rows), K], or null): AdaLN scale, value k of
// row m taken as x * (1 + mod_scale[m / mod_rows, k]) before the conversion
hipError_t launch_x16(const uint16_t *x, uint16_t *x16, float *rowscale, int64_t M, int64_t K, hipStream_t stream,
                      const float *mod_scale = nullptr, int64_t mod_rows = 1);
hipError_t launch_gemm3(int bits, const Gemm3Args &a, hipStream_t stream);
// SPLIT numerics (gemm4.hip): same arguments, x16 holds the caller's bf16 x,
// rowscale is unused, glu and gate must be off.
hipError_t launch_gemm4(int bits, const Gemm3Args &a, hipStream_t stream);
// FAST numerics without a prepass (gemm3o.hip): x16 holds the caller's bf16
// x, converted to fp16 inside the GEMM; rowscale is unused, glu and gate must
// be off. Two launches: the GEMM, then the recomputation (SPLIT numerics) of
// any tile with a row outside the in-kernel conversion's range.
hipError_t launch_gemm3_online(int bits, const Gemm3Args &a, hipStream_t stream);

hipError_t launch_splitk_reduce(const float *partial, int splits, int64_t M, int64_t N,
                                void *out, int out_bf16, hipStream_t stream);
hipError_t launch_fill_zero(void *out, int64_t count, int out_bf16, hipStream_t stream);

struct SkinnyArgs {
  const uint16_t *x;
  const uint32_t *w;      // canonical codes, or tiled codes when tiled != 0
  const uint16_t *s;      // canonical scales (unused when tiled)
  const uint16_t *b;      // canonical biases (unused when tiled)
  const uint32_t *sb;     // tiled scale|bias words (tiled only)
  void *out;
  int64_t M, N, K;
  int G;
  int out_bf16;
  int tiled;
};
// M <= 16 only.
hipError_t launch_skinny(int bits, const SkinnyArgs &a, hipStream_t stream);
// Canonical rows, one or two rows of x (gemv.hip): chunks of 16 bytes per
// lane and row for the shape, 0 when the GEMV does not serve it.
int gemv_chunks_per_lane(int bits, int64_t M, int64_t K, int tiled);
hipError_t launch_gemv(int bits, const SkinnyArgs &a, hipStream_t stream);

// Tiled layout (see layout.hip): codes [N32][G][32 * 2*bits words], scale|bias [N32][G][32].
// glu_f > 0: GLU row order for a [gate (glu_f); up (glu_f)] weight (see layout.hip).
hipError_t launch_repack(int bits, const uint32_t *canon, const uint16_t *s, const uint16_t *b, int64_t N,
                         int64_t K, int64_t glu_f, uint32_t *tiled, uint32_t *sb, hipStream_t stream);
hipError_t launch_unrepack(int bits, const uint32_t *tiled, const uint32_t *sb, int64_t N, int64_t K, int64_t glu_f,
                           uint32_t *canon, uint16_t *s, uint16_t *b, hipStream_t stream);

hipError_t launch_dequant(int bits, const uint32_t *w, const uint16_t *s, const uint16_t *b,
                          int64_t N, int64_t K, float *out, hipStream_t stream);
hipError_t launch_quantize(int bits, const float *w, int64_t N, int64_t K, uint32_t *packed,
                           uint16_t *s, uint16_t *b, int *status, hipStream_t stream);
hipError_t launch_quantize_imatrix(int bits, const float *w, const float *imp, int64_t N, int64_t K,
                                  uint32_t *packed, uint16_t *s, uint16_t *b, int *status, hipStream_t stream);

}  // namespace ql
