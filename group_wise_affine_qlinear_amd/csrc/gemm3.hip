// FAST numerics of the large-M dequant-GEMM (fp16 weights, row-scaled fp16
// activations on fp16 MFMA; see gemm3_core.h), its activation prepass and the
// work split of a launch over the device's CUs.
#include "gemm3_core.h"

namespace ql {

namespace {

// Row exponent of the fp16 activations: the power of two 2^-e that brings the
// row's largest magnitude mx into [2^14, 2^15), e = floor(log2 mx) - 14,
// clamped to [-126, 120] so 2^e and 2^-e are normal fp32 (e = 0 for mx = 0).
__device__ __forceinline__ int row_exponent(float mx) {
  if (!(mx > 0.f)) return 0;
  const int ex = ilogbf(mx);  // exact for fp32 subnormals; INT_MAX for inf
  return ex > 134 ? 120 : min(max(ex - 14, -126), 120);
}

// Optional AdaLN scale modulation of the activations: value k of row m
// becomes x * (1 + scale[m / mod_rows, k]), in fp32 (1 + scale rounded once,
// the product rounded once), before the row maximum and the fp16 rounding.
struct Modulation {
  const float *scale;  // fp32 [ceil(M / rows), K]; null: none
  int64_t rows;        // activation rows per scale row (>= 1)
};

// The 8 (possibly modulated) fp32 values of 16-byte vector i of row m.
template <bool MOD>
__device__ __forceinline__ void load8(const u32x4 &v, const Modulation &md, int64_t m, int64_t K, int i, float (&f)[8]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f[2 * t] = bf16_lo(v[t]);
    f[2 * t + 1] = bf16_hi(v[t]);
  }
  if constexpr (MOD) {
    const float4 *sp = reinterpret_cast<const float4 *>(md.scale + (int64_t)((uint64_t)m / (uint64_t)md.rows) * K) + 2 * i;
    const float4 s0 = sp[0], s1 = sp[1];
    const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = f[j] * (1.0f + sc[j]);
  }
}

__device__ __forceinline__ u32x4 pack8_f16(const float (&f)[8], float inv) {
  u32x4 o;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const _Float16 lo = (_Float16)(f[2 * t] * inv);
    const _Float16 hi = (_Float16)(f[2 * t + 1] * inv);
    o[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return o;
}

// x (bf16) -> x16 (fp16) with a power-of-two scale per row. One block per
// row: the row's max magnitude picks e (row_exponent); every value is
// multiplied by 2^-e (exact) and rounded to fp16.
template <bool MOD>
__global__ __launch_bounds__(256) void x16_kernel(const uint16_t *x, uint16_t *x16, float *rowscale, int64_t K,
                                                  Modulation md) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x + m * K);
  u32x4 *dst = reinterpret_cast<u32x4 *>(x16 + m * K);
  const int nv = (int)(K / 8);
  float mx = 0.f;
  for (int i = threadIdx.x; i < nv; i += 256) {
    float f[8];
    load8<MOD>(src[i], md, m, K, i, f);
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(f[j]));
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = row_exponent(mx);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
  if (threadIdx.x == 0) rowscale[m] = __uint_as_float((uint32_t)(127 + e) << 23);
  for (int i = threadIdx.x; i < nv; i += 256) {
    float f[8];
    load8<MOD>(src[i], md, m, K, i, f);
    dst[i] = pack8_f16(f, inv);
  }
}

// Same conversion with one wave per row and the row held in registers (K up
// to 64*8*V): one read of x instead of two.
template <int V, bool MOD>
__global__ __launch_bounds__(256) void x16_row_kernel(const uint16_t *x, uint16_t *x16, float *rowscale, int64_t M,
                                                      int64_t K, Modulation md) {
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x + m * K);
  u32x4 *dst = reinterpret_cast<u32x4 *>(x16 + m * K);
  const int nv = (int)(K / 8);
  float f[V][8];
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = lane + 64 * j;
    if (i < nv) {
      load8<MOD>(src[i], md, m, K, i, f[j]);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) f[j][t] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) mx = fmaxf(mx, fabsf(f[j][t]));
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const int e = row_exponent(mx);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
  if (lane == 0) rowscale[m] = __uint_as_float((uint32_t)(127 + e) << 23);
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = lane + 64 * j;
    if (i >= nv) break;
    dst[i] = pack8_f16(f[j], inv);
  }
}

// CUs of the calling thread's current device (queried per call: the library
// keeps no device state).
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1)
    n = 1;
  return n;
}

}  // namespace

Gemm3Plan gemm3_plan(int64_t M, int64_t N, int G, int slots, int force_splits, bool fill_by_pieces) {
  Gemm3Plan p{};
  using g3::kBM;
  using g3::kBN;
  p.tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  p.dp_tiles = (int)p.tiles;
  p.grid_x = (int)p.tiles;
  p.splits = 1;
  if (slots <= 0) slots = device_cus();  // one block per CU
  int splits = force_splits;
  if (splits <= 0 && p.tiles * 2 <= slots && G >= 16) {
    // too few tiles for the CUs: split K, keeping >= 8 groups per range
    splits = (int)(slots / p.tiles);
    if (splits > G / 8) splits = G / 8;
    if (splits > 16) splits = 16;
  }
  if (splits > G) splits = G;
  if (splits > 1) {
    const int gps = (G + splits - 1) / splits;
    p.splits = (G + gps - 1) / gps;  // no empty range
    if (p.splits > 1) p.partial_bytes = (size_t)p.splits * (size_t)M * (size_t)N * 4u;
    return p;
  }
  if (p.tiles < slots && fill_by_pieces && M > 32) {
    // every tile in row pieces, all in one round of blocks: the most pieces
    // per tile (8, 4 or 2) that need no more blocks than slots, whole tiles
    // when even halves would not fit. A piece dequantizes its tile's whole
    // width, so its time grows much less than its rows: two rounds of small
    // pieces take longer than one of larger ones (36 tiles as 288 pieces of
    // 32 rows on 256 slots gave 32 slots two pieces each)
    int pieces = 8;
    while (pieces >= 2 && p.tiles * pieces > slots) pieces /= 2;
    if (pieces < 2) return p;
    p.dp_tiles = 0;
    p.tail_tiles = (int)p.tiles;
    p.tail_mi = 16 / pieces;
    p.grid_x = (int)p.tiles * pieces;
    return p;
  }
  if (p.tiles <= slots || p.tiles % slots == 0) return p;
  const int64_t tail = p.tiles % slots;
  int pieces = 8;
  while (pieces >= 2 && tail * pieces > slots) pieces /= 2;
  if (pieces < 2) return p;
  p.dp_tiles = (int)(p.tiles - tail);
  p.tail_tiles = (int)tail;
  p.tail_mi = 16 / pieces;
  p.grid_x = slots;
  return p;
}

namespace {
template <bool MOD>
void launch_x16_mod(const uint16_t *x, uint16_t *x16, float *rowscale, int64_t M, int64_t K, Modulation md,
                    hipStream_t stream) {
  const int64_t vecs = (K / 8 + 63) / 64;  // 16-byte vectors per lane for one wave per row
  const dim3 grid4((unsigned)((M + 3) / 4));
  if (vecs <= 4) hipLaunchKernelGGL((x16_row_kernel<4, MOD>), grid4, dim3(256), 0, stream, x, x16, rowscale, M, K, md);
  else if (vecs <= 9) hipLaunchKernelGGL((x16_row_kernel<9, MOD>), grid4, dim3(256), 0, stream, x, x16, rowscale, M, K, md);
  else if (vecs <= 16) hipLaunchKernelGGL((x16_row_kernel<16, MOD>), grid4, dim3(256), 0, stream, x, x16, rowscale, M, K, md);
  else hipLaunchKernelGGL((x16_kernel<MOD>), dim3((unsigned)M), dim3(256), 0, stream, x, x16, rowscale, K, md);
}
}  // namespace

hipError_t launch_x16(const uint16_t *x, uint16_t *x16, float *rowscale, int64_t M, int64_t K, hipStream_t stream,
                      const float *mod_scale, int64_t mod_rows) {
  if (mod_scale) launch_x16_mod<true>(x, x16, rowscale, M, K, Modulation{mod_scale, mod_rows}, stream);
  else launch_x16_mod<false>(x, x16, rowscale, M, K, Modulation{nullptr, 1}, stream);
  return hipGetLastError();
}

hipError_t launch_gemm3(int bits, const Gemm3Args &a, hipStream_t stream) {
  if (bits == 4) return g3::launch3_bits<4, false>(a, stream);
  if (bits == 8) return g3::launch3_bits<8, false>(a, stream);
  if (bits == 2) return g3::launch3_bits<2, false>(a, stream);
  if (bits == 3) return g3::launch3_bits<3, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ql
