// Device dequantize (check path) and device load-time RTN quantizer.
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  // v_cvt_f16_f32 under the default round-to-nearest-even mode; overflow gives inf
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

__device__ __forceinline__ bool f16_finite(uint16_t h) { return (h & 0x7C00u) != 0x7C00u; }

// W_hat[n, k] = fp32(s) * q + fp32(b); s*q is exact in fp32 so the fused form
// rounds exactly once, like the plain multiply-then-add definition. One
// thread per (row, group): the group's 2*BITS words of the row's code stream.
template <int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t *w, const uint16_t *s,
                                                      const uint16_t *b, int64_t N, int64_t K,
                                                      float *out) {
  constexpr int WPG = 2 * BITS;
  const int64_t G = K / 64;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * G) return;
  const int64_t n = idx / G, g = idx % G;
  const float sf = f16_to_f32(s[n * G + g]);
  const float bf = f16_to_f32(b[n * G + g]);
  uint32_t word[WPG];
  const uint32_t *src = w + n * (K * BITS / 32) + g * WPG;
#pragma unroll
  for (int j = 0; j < WPG; ++j) word[j] = src[j];
  float *o = out + n * K + g * 64;
#pragma unroll
  for (int k = 0; k < 64; k += 4) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(sf, (float)stream_code<BITS>(word, k + e), bf);
    *reinterpret_cast<f32x4 *>(o + k) = v;
  }
}

// One thread per (row, group): min/max, f16 scale and bias, codes from the
// stored f16 values with IEEE subtract/divide and round-half-even, packed.
template <int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(const float *w, int64_t N, int64_t K,
                                                       uint32_t *packed, uint16_t *s, uint16_t *b,
                                                       int *status) {
#pragma clang fp contract(off)
  constexpr int Q = (1 << BITS) - 1;
  const int64_t G = K / 64;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * G) return;
  const int64_t n = idx / G, g = idx % G;
  const float *wp = w + n * K + g * 64;
  float mn = wp[0], mx = wp[0];
  bool bad = false;
#pragma unroll
  for (int k = 0; k < 64; k += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(wp + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = v[j];
      bad |= !__builtin_isfinite(x);
      // min/max order -0 below +0 (IEEE 754-2019 minimum/maximum)
      if (x < mn || (x == mn && __builtin_signbit(x) && !__builtin_signbit(mn))) mn = x;
      if (x > mx || (x == mx && !__builtin_signbit(x) && __builtin_signbit(mx))) mx = x;
    }
  }
  const float s32 = __fdiv_rn(__fsub_rn(mx, mn), (float)Q);
  const uint16_t s16 = f32_to_f16_bits(s32);
  const uint16_t b16 = f32_to_f16_bits(mn);
  if (bad || !f16_finite(s16) || !f16_finite(b16)) {
    if (status) *status = -6;  // QL_ERANGE
  }
  const float sf = f16_to_f32(s16), bf = f16_to_f32(b16);
  uint32_t word[2 * BITS];
#pragma unroll
  for (int j = 0; j < 2 * BITS; ++j) word[j] = 0u;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    int q = 0;
    if (sf != 0.f) {
      float t = __builtin_rintf(__fdiv_rn(__fsub_rn(wp[i], bf), sf));
      t = fminf(fmaxf(t, 0.f), (float)Q);
      q = (int)t;
    }
    stream_put<BITS>(word, i, (uint32_t)q);
  }
  uint32_t *pw = packed + n * (K * BITS / 32) + g * (2 * BITS);
#pragma unroll
  for (int j = 0; j < 2 * BITS; ++j) pw[j] = word[j];
  s[n * G + g] = s16;
  b[n * G + g] = b16;
}

// Importance-weighted fit, one thread per (row, group). Objective per group:
// E(s, b) = sum_j imp_j * (w_j - (s*q_j + b))^2 with q the RTN codes of the
// stored f16 (s, b) (Ideogram-4-IQ4_M card, section on what "IQ4" means: the
// error of input channel j weighs E[x_j^2]; the min/max RTN fit is candidate
// 0, so the result is never worse than RTN). Candidates after RTN: weighted
// least-squares lines w ~ s*l + b fitted to starting codes l = the RTN codes,
// then l = clamp(rint((w - lo) * (Q + d) / (hi - lo)), 0, Q) for 16 offsets d
// over the group's [min, max] and over the min/max of its channels with
// nonzero importance. A candidate replaces the best only with a strictly
// smaller E. fp32, one rounding per operation (plain operators under the
// no-contraction pragma below; the header helpers such as __fmul_rn may be
// fused into FMAs once inlined), sums over j in order, so every decision
// matches a plain reimplementation step for step.
template <int BITS>
__global__ __launch_bounds__(256) void quantize_imatrix_kernel(const float *w, const float *imp, int64_t N,
                                                               int64_t K, uint32_t *packed, uint16_t *s, uint16_t *b,
                                                               int *status) {
#pragma clang fp contract(off)
  constexpr float Q = (float)((1 << BITS) - 1);
  const int64_t G = K / 64;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * G) return;
  const int64_t n = idx / G, g = idx % G;
  float wv[64], av[64];
  bool bad = false, bad_imp = false;
#pragma unroll
  for (int k = 0; k < 64; k += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(w + n * K + g * 64 + k);
    const f32x4 u = *reinterpret_cast<const f32x4 *>(imp + g * 64 + k);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wv[k + j] = v[j];
      av[k + j] = u[j];
      bad |= !__builtin_isfinite(v[j]);
      bad_imp |= !(__builtin_isfinite(u[j]) && u[j] >= 0.f);
    }
  }
  // candidate 0: the min/max RTN fit (as quantize_kernel)
  float mn = wv[0], mx = wv[0], lo_a = __builtin_inff(), hi_a = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const float x = wv[j];
    if (x < mn || (x == mn && __builtin_signbit(x) && !__builtin_signbit(mn))) mn = x;
    if (x > mx || (x == mx && !__builtin_signbit(x) && __builtin_signbit(mx))) mx = x;
    if (av[j] > 0.f) {
      if (x < lo_a) lo_a = x;
      if (x > hi_a) hi_a = x;
    }
  }
  const uint16_t s0 = f32_to_f16_bits(__fdiv_rn(mx - mn, Q));
  const uint16_t b0 = f32_to_f16_bits(mn);
  if (bad || !f16_finite(s0) || !f16_finite(b0)) {
    if (status) *status = -6;  // QL_ERANGE
  }
  if (bad_imp && status) *status = -1;  // QL_EINVAL
  auto code = [&](float x, float sf, float bf) -> float {
    if (sf == 0.f) return 0.f;
    return fminf(fmaxf(__builtin_rintf(__fdiv_rn(x - bf, sf)), 0.f), Q);
  };
  auto error = [&](float sf, float bf) -> float {
    float e = 0.f;
    for (int j = 0; j < 64; ++j) {
      const float d = wv[j] - (sf * code(wv[j], sf, bf) + bf);
      e = e + av[j] * (d * d);
    }
    return e;
  };
  const float s0f = f16_to_f32(s0), b0f = f16_to_f32(b0);
  uint16_t s_best = s0, b_best = b0;
  float e_best = error(s0f, b0f);
  // candidate c: 0 = RTN codes, 1..16 = offsets over [min, max], 17..32 over the weighted range
  for (int c = 0; c <= 32; ++c) {
    if (s0f == 0.f) break;
    float lo = 0.f, inv = 0.f;
    if (c > 0) {
      const bool full = c <= 16;
      const float l0 = full ? mn : lo_a, h0 = full ? mx : hi_a;
      if (!(h0 > l0)) continue;
      const double dd = ((double)((c - 1) % 16) - 7.5) / 10.0;
      lo = l0;
      inv = __fdiv_rn(Q + (float)dd, h0 - l0);
    }
    float S0 = 0.f, S1 = 0.f, S2 = 0.f, T0 = 0.f, T1 = 0.f;
    for (int j = 0; j < 64; ++j) {
      const float l = c == 0 ? code(wv[j], s0f, b0f)
                             : fminf(fmaxf(__builtin_rintf((wv[j] - lo) * inv), 0.f), Q);
      const float al = av[j] * l;
      S0 = S0 + av[j];
      S1 = S1 + al;
      S2 = S2 + al * l;
      T0 = T0 + av[j] * wv[j];
      T1 = T1 + al * wv[j];
    }
    const float D = S0 * S2 - S1 * S1;
    if (!(D > 0.f)) continue;
    const float sc = __fdiv_rn(S0 * T1 - S1 * T0, D);
    const float bc = __fdiv_rn(S2 * T0 - S1 * T1, D);
    const uint16_t sc16 = f32_to_f16_bits(sc), bc16 = f32_to_f16_bits(bc);
    const float sf = f16_to_f32(sc16), bf = f16_to_f32(bc16);
    if (!(f16_finite(sc16) && sf > 0.f && f16_finite(bc16))) continue;
    const float e = error(sf, bf);
    if (e < e_best) {
      e_best = e;
      s_best = sc16;
      b_best = bc16;
    }
  }
  const float sf = f16_to_f32(s_best), bf = f16_to_f32(b_best);
  uint32_t word[2 * BITS];
#pragma unroll
  for (int j = 0; j < 2 * BITS; ++j) word[j] = 0u;
#pragma unroll
  for (int i = 0; i < 64; ++i) stream_put<BITS>(word, i, (uint32_t)(int)code(wv[i], sf, bf));
  uint32_t *pw = packed + n * (K * BITS / 32) + g * (2 * BITS);
#pragma unroll
  for (int j = 0; j < 2 * BITS; ++j) pw[j] = word[j];
  s[n * G + g] = s_best;
  b[n * G + g] = b_best;
}

template <int BITS>
hipError_t quantize_imatrix_bits(const float *w, const float *imp, int64_t N, int64_t K, uint32_t *packed,
                                 uint16_t *s, uint16_t *b, int *status, hipStream_t stream) {
  const int64_t threads = N * (K / 64);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(quantize_imatrix_kernel<BITS>, dim3((unsigned)blocks), dim3(256), 0, stream, w, imp, N, K,
                     packed, s, b, status);
  return hipGetLastError();
}

template <int BITS>
hipError_t dequant_bits(const uint32_t *w, const uint16_t *s, const uint16_t *b, int64_t N, int64_t K,
                        float *out, hipStream_t stream) {
  const int64_t threads = N * (K / 64);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(dequant_kernel<BITS>, dim3((unsigned)blocks), dim3(256), 0, stream, w, s, b, N, K, out);
  return hipGetLastError();
}

template <int BITS>
hipError_t quantize_bits(const float *w, int64_t N, int64_t K, uint32_t *packed, uint16_t *s,
                         uint16_t *b, int *status, hipStream_t stream) {
  const int64_t threads = N * (K / 64);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(quantize_kernel<BITS>, dim3((unsigned)blocks), dim3(256), 0, stream, w, N, K, packed,
                     s, b, status);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(int bits, const uint32_t *w, const uint16_t *s, const uint16_t *b, int64_t N,
                          int64_t K, float *out, hipStream_t stream) {
  if (bits == 4) return dequant_bits<4>(w, s, b, N, K, out, stream);
  if (bits == 8) return dequant_bits<8>(w, s, b, N, K, out, stream);
  if (bits == 2) return dequant_bits<2>(w, s, b, N, K, out, stream);
  if (bits == 3) return dequant_bits<3>(w, s, b, N, K, out, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_quantize_imatrix(int bits, const float *w, const float *imp, int64_t N, int64_t K,
                                  uint32_t *packed, uint16_t *s, uint16_t *b, int *status, hipStream_t stream) {
  if (bits == 4) return quantize_imatrix_bits<4>(w, imp, N, K, packed, s, b, status, stream);
  if (bits == 8) return quantize_imatrix_bits<8>(w, imp, N, K, packed, s, b, status, stream);
  if (bits == 2) return quantize_imatrix_bits<2>(w, imp, N, K, packed, s, b, status, stream);
  if (bits == 3) return quantize_imatrix_bits<3>(w, imp, N, K, packed, s, b, status, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_quantize(int bits, const float *w, int64_t N, int64_t K, uint32_t *packed, uint16_t *s,
                           uint16_t *b, int *status, hipStream_t stream) {
  if (bits == 4) return quantize_bits<4>(w, N, K, packed, s, b, status, stream);
  if (bits == 8) return quantize_bits<8>(w, N, K, packed, s, b, status, stream);
  if (bits == 2) return quantize_bits<2>(w, N, K, packed, s, b, status, stream);
  if (bits == 3) return quantize_bits<3>(w, N, K, packed, s, b, status, stream);
  return hipErrorInvalidValue;
}

}  // namespace ql
