// Skinny-M path (M <= 16): memory-bound GEMV-like projection, e.g. the AdaLN
// modulation and timestep projections (one or a few rows of x against a wide
// weight). The kernel streams each packed weight row once from HBM with
// 16-byte loads and keeps the arithmetic on the matrix cores so the vector
// ALUs only unpack codes.
//
// Block = 4 waves on one strip of 32 output columns; wave w takes a contiguous
// quarter of the K groups, and the four partial sums are added in a fixed
// order through LDS (deterministic, no atomics). Per group and wave:
//   B: each lane loads its column's codes for half of the group (lane/32 picks
//      the half), i.e. 16 bytes of 4-bit codes = 32 codes = 4 MFMA K-steps;
//   A: lanes whose row m = lane%32 < M load the matching 32 values of x (rows
//      >= M are zero);
//   P  = sum over the 4 steps of v_mfma_f32_32x32x16_bf16(x, 128 + q)
//   P1 = the same with B = 1.0, which puts xsum[m, g] in P's register layout;
//   acc += s * P + (b - 128 s) * P1.
// Step t of lane half h covers codes 32h + 8t .. 32h + 8t + 7 of the group, so
// every MFMA stays inside one group.
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

__device__ __forceinline__ uint16_t f32_to_bf16_rne_s(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Per-lane codes of one group: 4-bit 16 B, 8-bit 32 B, 2-bit 8 B.
template <int BITS> struct LaneCodes { u32x4 v[BITS == 8 ? 2 : 1]; };

template <int BITS>
__device__ __forceinline__ LaneCodes<BITS> load_codes(const uint32_t *wrow, int g, int h) {
  LaneCodes<BITS> c;
  if constexpr (BITS == 4) {
    c.v[0] = *reinterpret_cast<const u32x4 *>(wrow + g * 8 + 4 * h);
  } else if constexpr (BITS == 8) {
    c.v[0] = *reinterpret_cast<const u32x4 *>(wrow + g * 16 + 8 * h);
    c.v[1] = *reinterpret_cast<const u32x4 *>(wrow + g * 16 + 8 * h + 4);
  } else {
    const u32x2 t = *reinterpret_cast<const u32x2 *>(wrow + g * 4 + 2 * h);
    c.v[0] = u32x4{t[0], t[1], 0u, 0u};
  }
  return c;
}

template <int BITS>
__device__ __forceinline__ bf16x8 codes_step(const LaneCodes<BITS> &c, int t) {
  if constexpr (BITS == 4) return as_bf16x8(unpack8_b4(c.v[0][t]));
  else if constexpr (BITS == 8) return as_bf16x8(unpack8_b8(c.v[t >> 1][(t & 1) * 2], c.v[t >> 1][(t & 1) * 2 + 1]));
  else return as_bf16x8(unpack8_b2(c.v[0][t >> 1], t & 1));
}

template <int BITS, int MR>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyArgs a) {
  constexpr int U = 8;  // groups of codes kept in flight per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, h = lane >> 5;
  const int64_t n0 = (int64_t)blockIdx.x * 32;
  int64_t n = n0 + col;
  if (n >= a.N) n = a.N - 1;
  const int G = a.G;
  const int gpw = (G + 3) / 4;
  const int g0 = wave * gpw;
  const int g1 = min(G, g0 + gpw);

  const bool arow = col < a.M;
  const uint16_t *xrow = a.x + (int64_t)(arow ? col : 0) * a.K + 32 * h;
  const uint32_t *wrow = a.w + n * (a.K * BITS / 32);
  const uint16_t *srow = a.s + n * G;
  const uint16_t *brow = a.b + n * G;
  const float offset = CodeOffset<BITS>::value;

  const u32x4 one4 = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8 ones = as_bf16x8(one4);

  float acc[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) acc[r] = 0.f;

  LaneCodes<BITS> wbuf[U];
  uint32_t sbbuf[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (g0 + u < g1) {
      wbuf[u] = load_codes<BITS>(wrow, g0 + u, h);
      sbbuf[u] = (uint32_t)srow[g0 + u] | ((uint32_t)brow[g0 + u] << 16);
    }
  }

  for (int gb = g0; gb < g1; gb += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int g = gb + u;
      if (g < g1) {
        const LaneCodes<BITS> cw = wbuf[u];
        const uint32_t sb = sbbuf[u];
        if (g + U < g1) {
          wbuf[u] = load_codes<BITS>(wrow, g + U, h);
          sbbuf[u] = (uint32_t)srow[g + U] | ((uint32_t)brow[g + U] << 16);
        }
        u32x4 xa[4];
        if (arow) {
#pragma unroll
          for (int t = 0; t < 4; ++t) xa[t] = *reinterpret_cast<const u32x4 *>(xrow + (int64_t)g * 64 + 8 * t);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) xa[t] = u32x4{0u, 0u, 0u, 0u};
        }
        f32x16 p = {}, p1 = {};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 av = as_bf16x8(xa[t]);
          p = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, codes_step<BITS>(cw, t), p, 0, 0, 0);
          p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, ones, p1, 0, 0, 0);
        }
        const float sf = f16_to_f32((uint16_t)(sb & 0xFFFFu));
        const float bf = __builtin_fmaf(-offset, sf, f16_to_f32((uint16_t)(sb >> 16)));
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          const float t = __builtin_fmaf(sf, p[r], acc[r]);
          acc[r] = __builtin_fmaf(bf, p1[r], t);
        }
      }
    }
  }

  __shared__ float red[4][MR][64];
#pragma unroll
  for (int r = 0; r < MR; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  if (wave == 0) {
    const int64_t nn = n0 + col;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const float v = ((red[0][r][lane] + red[1][r][lane]) + red[2][r][lane]) + red[3][r][lane];
      const int row = 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < a.M && nn < a.N) {
        if (a.out_bf16) reinterpret_cast<uint16_t *>(a.out)[(int64_t)row * a.N + nn] = f32_to_bf16_rne_s(v);
        else reinterpret_cast<float *>(a.out)[(int64_t)row * a.N + nn] = v;
      }
    }
  }
}

template <int BITS>
hipError_t launch_bits(const SkinnyArgs &a, hipStream_t stream) {
  const unsigned blocks = (unsigned)((a.N + 31) / 32);
  if (a.M <= 8) hipLaunchKernelGGL((skinny_kernel<BITS, 4>), dim3(blocks), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((skinny_kernel<BITS, 8>), dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(int bits, const SkinnyArgs &a, hipStream_t stream) {
  if (a.M > 16) return hipErrorInvalidValue;
  if (bits == 4) return launch_bits<4>(a, stream);
  if (bits == 8) return launch_bits<8>(a, stream);
  if (bits == 2) return launch_bits<2>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ql
