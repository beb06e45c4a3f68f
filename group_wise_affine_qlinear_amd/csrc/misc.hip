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
// rounds exactly once, like the plain multiply-then-add definition.
template <int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t *w, const uint16_t *s,
                                                      const uint16_t *b, int64_t N, int64_t K,
                                                      float *out) {
  constexpr int CPW = 32 / BITS;
  constexpr uint32_t Q = (1u << BITS) - 1u;
  const int64_t wr = K / CPW;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * wr) return;
  const int64_t n = idx / wr, wi = idx % wr;
  const int64_t k0 = wi * CPW;
  const int64_t G = K / 64;
  const int64_t g = k0 / 64;
  const float sf = f16_to_f32(s[n * G + g]);
  const float bf = f16_to_f32(b[n * G + g]);
  const uint32_t word = w[idx];
  float v[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) v[j] = __builtin_fmaf(sf, (float)((word >> (BITS * j)) & Q), bf);
  float *o = out + n * K + k0;
#pragma unroll
  for (int j = 0; j < CPW; j += 4) *reinterpret_cast<f32x4 *>(o + j) = f32x4{v[j], v[j + 1], v[j + 2], v[j + 3]};
}

// One thread per (row, group): min/max, f16 scale and bias, codes from the
// stored f16 values with IEEE subtract/divide and round-half-even, packed.
template <int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(const float *w, int64_t N, int64_t K,
                                                       uint32_t *packed, uint16_t *s, uint16_t *b,
                                                       int *status) {
#pragma clang fp contract(off)
  constexpr int CPW = 32 / BITS;
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
  uint32_t *pw = packed + n * (K / CPW) + g * (64 / CPW);
#pragma unroll
  for (int j = 0; j < 64 / CPW; ++j) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      int q = 0;
      if (sf != 0.f) {
        float t = __builtin_rintf(__fdiv_rn(__fsub_rn(wp[j * CPW + i], bf), sf));
        t = fminf(fmaxf(t, 0.f), (float)Q);
        q = (int)t;
      }
      word |= (uint32_t)q << (BITS * i);
    }
    pw[j] = word;
  }
  s[n * G + g] = s16;
  b[n * G + g] = b16;
}

template <int BITS>
hipError_t dequant_bits(const uint32_t *w, const uint16_t *s, const uint16_t *b, int64_t N, int64_t K,
                        float *out, hipStream_t stream) {
  const int64_t threads = N * (K * BITS / 32);
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
  return hipErrorInvalidValue;
}

hipError_t launch_quantize(int bits, const float *w, int64_t N, int64_t K, uint32_t *packed, uint16_t *s,
                           uint16_t *b, int *status, hipStream_t stream) {
  if (bits == 4) return quantize_bits<4>(w, N, K, packed, s, b, status, stream);
  if (bits == 8) return quantize_bits<8>(w, N, K, packed, s, b, status, stream);
  if (bits == 2) return quantize_bits<2>(w, N, K, packed, s, b, status, stream);
  return hipErrorInvalidValue;
}

}  // namespace ql
