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

// x (bf16) -> x16 (fp16) with a power-of-two scale per row. One block per
// row: the row's max magnitude picks e (row_exponent); every value is
// multiplied by 2^-e (exact) and rounded to fp16.
__global__ __launch_bounds__(256) void x16_kernel(const uint16_t *x, uint16_t *x16, float *rowscale, int64_t K) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x + m * K);
  u32x4 *dst = reinterpret_cast<u32x4 *>(x16 + m * K);
  const int nv = (int)(K / 8);
  float mx = 0.f;
  for (int i = threadIdx.x; i < nv; i += 256) {
    const u32x4 v = src[i];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      mx = fmaxf(mx, fabsf(bf16_lo(v[t])));
      mx = fmaxf(mx, fabsf(bf16_hi(v[t])));
    }
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = row_exponent(mx);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
  if (threadIdx.x == 0) rowscale[m] = __uint_as_float((uint32_t)(127 + e) << 23);
  for (int i = threadIdx.x; i < nv; i += 256) {
    const u32x4 v = src[i];
    u32x4 o;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const _Float16 lo = (_Float16)(bf16_lo(v[t]) * inv);
      const _Float16 hi = (_Float16)(bf16_hi(v[t]) * inv);
      o[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    dst[i] = o;
  }
}

// Same conversion with one wave per row and the row held in registers (K up
// to 64*8*V): one read of x instead of two.
template <int V>
__global__ __launch_bounds__(256) void x16_row_kernel(const uint16_t *x, uint16_t *x16, float *rowscale, int64_t M,
                                                      int64_t K) {
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x + m * K);
  u32x4 *dst = reinterpret_cast<u32x4 *>(x16 + m * K);
  const int nv = (int)(K / 8);
  u32x4 v[V];
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = lane + 64 * j;
    v[j] = i < nv ? src[i] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 4; ++t) mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(v[j][t])), fabsf(bf16_hi(v[j][t]))));
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const int e = row_exponent(mx);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
  if (lane == 0) rowscale[m] = __uint_as_float((uint32_t)(127 + e) << 23);
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = lane + 64 * j;
    if (i >= nv) break;
    u32x4 o;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const _Float16 lo = (_Float16)(bf16_lo(v[j][t]) * inv);
      const _Float16 hi = (_Float16)(bf16_hi(v[j][t]) * inv);
      o[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    dst[i] = o;
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
    // every tile in row pieces: the fewest pieces per tile (2, 4 or 8) that
    // give at least one block per slot
    int pieces = 2;
    while (pieces < 8 && p.tiles * pieces < slots) pieces *= 2;
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

hipError_t launch_x16(const uint16_t *x, uint16_t *x16, float *rowscale, int64_t M, int64_t K, hipStream_t stream) {
  const int64_t vecs = (K / 8 + 63) / 64;  // 16-byte vectors per lane for one wave per row
  const dim3 grid4((unsigned)((M + 3) / 4));
  if (vecs <= 4) hipLaunchKernelGGL(x16_row_kernel<4>, grid4, dim3(256), 0, stream, x, x16, rowscale, M, K);
  else if (vecs <= 9) hipLaunchKernelGGL(x16_row_kernel<9>, grid4, dim3(256), 0, stream, x, x16, rowscale, M, K);
  else if (vecs <= 16) hipLaunchKernelGGL(x16_row_kernel<16>, grid4, dim3(256), 0, stream, x, x16, rowscale, M, K);
  else hipLaunchKernelGGL(x16_kernel, dim3((unsigned)M), dim3(256), 0, stream, x, x16, rowscale, K);
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
