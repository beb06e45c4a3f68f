// GEMV for one or two rows of x against canonical weight rows (2-, 4- and
// 8-bit codes): the memory-bound AdaLN / timestep projections when the
// weights stay in the checkpoint's row layout.
//
// Lanes run along K. A row's codes are cut into 16-byte chunks (32 codes of
// 4-bit, 16 of 8-bit, 64 of 2-bit); lane L takes chunks L, L+64, ... of every
// row it visits, so each load instruction of a wave reads 1 KB of one row
// contiguously and every 128-byte line is used whole. Because a lane always
// covers the same chunk positions, its slice of x (and the slice sums) is
// loaded once into registers and serves every row: a block stages x in LDS
// once, its waves copy their slices out, and then loop over the rows in
// pairs (grid of a few blocks per CU; both rows' loads in flight before any
// arithmetic).
//
// Arithmetic, as the skinny kernel's EXACT numerics: codes become exact
// bf16 values c = q + off (off = 128 for 2/4-bit, 0 for 8-bit), products
// with x accumulate in fp32 through v_dot2_f32_bf16, and each chunk folds
// its scale and bias: acc += s * sum(x*c) + (b - off*s) * sum(x). The 64
// lane partials of a row are added across the wave with DPP moves, in a
// fixed order.
#include <algorithm>

#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf2;

constexpr int kThreads = 256;  // four waves

__device__ __forceinline__ float dot2(uint32_t x, uint32_t c, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, x), __builtin_bit_cast(bf2, c), acc, false);
}

// v + (v of the lane the DPP control selects); lanes of rows the row mask
// leaves out add zero
template <int CTRL, int ROWS>
__device__ __forceinline__ float add_dpp(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false);
  return v + __builtin_bit_cast(float, o);
}

// Sum of v over the 64 lanes, in lane 63, in a fixed order: pairs and quads
// (quad permutes), half rows and rows (mirrors), then row 0 into row 1 and
// row 2 into row 3 (broadcast of lane 15 of each row), then rows 0-1 into
// rows 2-3 (broadcast of lane 31).
__device__ __forceinline__ float wave_sum63(float v) {
  v = add_dpp<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
  v = add_dpp<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
  v = add_dpp<0x141, 0xF>(v);  // row_half_mirror
  v = add_dpp<0x140, 0xF>(v);  // row_mirror
  v = add_dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = add_dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne_v(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Code pairs (k, k+1) of one 16-byte chunk as bf16x2 words, in k order.
template <int BITS> struct Chunk {
  static constexpr int kCodes = 128 / BITS;  // codes per chunk
  static constexpr int kPairs = kCodes / 2;
  __device__ static void pairs(const u32x4 &w, uint32_t (&p)[kPairs]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (BITS == 4) {
        const u32x4 r = unpack8_b4(w[i]);
#pragma unroll
        for (int t = 0; t < 4; ++t) p[4 * i + t] = r[t];
      } else if constexpr (BITS == 2) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const u32x4 r = unpack8_b2(w[i], hh);
#pragma unroll
          for (int t = 0; t < 4; ++t) p[8 * i + 4 * hh + t] = r[t];
        }
      } else {
        if (i % 2 == 0) {
          const u32x4 r = unpack8_b8(w[i], w[i + 1]);
#pragma unroll
          for (int t = 0; t < 4; ++t) p[2 * i + t] = r[t];
        }
      }
    }
  }
};

// M rows of x, J chunks per lane (chunks lane + 64 j of each row, j < J),
// R weight rows per wave step.
template <int BITS, int M, int J, int R>
__global__ __launch_bounds__(kThreads) void gemv_kernel(SkinnyArgs a) {
  constexpr int kRowsPerWave = R;
  using CK = Chunk<BITS>;
  constexpr int P = CK::kPairs;
  constexpr float kOff = CodeOffset<BITS>::value;
  extern __shared__ __attribute__((aligned(16))) unsigned char xl[];  // x [M, K] bf16
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int C = (int)(a.K * BITS / 128);  // chunks per row
  const int G = a.G;
  const int64_t row_words = a.K * BITS / 32;

  // x into LDS, 16 bytes per thread and step
  {
    const int nv = (int)(M * a.K / 8);
    const u32x4 *src = reinterpret_cast<const u32x4 *>(a.x);
    for (int i = threadIdx.x; i < nv; i += kThreads) reinterpret_cast<u32x4 *>(xl)[i] = src[i];
    __syncthreads();
  }
  // this lane's slice of x: pairs (k, k+1) of chunk j, and the slice sums
  uint32_t xp[M][J][P];
  float xs[M][J];
#pragma unroll
  for (int m = 0; m < M; ++m)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + 64 * j;
      const bool ok = c < C;
      const u32x4 *src = reinterpret_cast<const u32x4 *>(xl + ((int64_t)m * a.K + (int64_t)(ok ? c : 0) * CK::kCodes) * 2);
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < P / 4; ++v) {
        const u32x4 t = ok ? src[v] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xp[m][j][4 * v + e] = t[e];
          s = dot2(t[e], 0x3F803F80u, s);  // sum of the pair (1.0, 1.0)
        }
      }
      xs[m][j] = s;
    }

  // Row groups of this wave: pr0, pr0 + stride, ...; all loads of a group
  // are issued before its arithmetic.
  struct Buf {
    u32x4 w[kRowsPerWave][J];
    uint16_t sv[kRowsPerWave][J], bv[kRowsPerWave][J];
  };
  // codes, scale and bias of a pair (rows past N clamp to N-1 and are not
  // stored; chunks past the row end read chunk 0 and are not used)
  auto load = [&](Buf &bf, int64_t pr) {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      const int64_t n = min<int64_t>(pr * kRowsPerWave + r, a.N - 1);
      const u32x4 *wr = reinterpret_cast<const u32x4 *>(a.w + n * row_words);
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = lane + 64 * j;
        const int cc = c < C ? c : 0;
        bf.w[r][j] = wr[cc];
        const int g = (int)((int64_t)cc * CK::kCodes / 64);
        bf.sv[r][j] = a.s[n * G + g];
        bf.bv[r][j] = a.b[n * G + g];
      }
    }
  };
  auto compute = [&](const Buf &bf, int64_t pr) {
#pragma unroll
    for (int r = 0; r < kRowsPerWave; ++r) {
      float acc[M];
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = 0.f;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (lane + 64 * j < C) {
          uint32_t cp[P];
          CK::pairs(bf.w[r][j], cp);
          const float s = f16_to_f32(bf.sv[r][j]);
          const float bb = __builtin_fmaf(-kOff, s, f16_to_f32(bf.bv[r][j]));
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < P; ++i) d = dot2(xp[m][j][i], cp[i], d);
            acc[m] = __builtin_fmaf(bb, xs[m][j], __builtin_fmaf(s, d, acc[m]));
          }
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = wave_sum63(acc[m]);
      const int64_t n = pr * kRowsPerWave + r;
      if (lane == 63 && n < a.N) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          if (a.out_bf16) reinterpret_cast<uint16_t *>(a.out)[(int64_t)m * a.N + n] = f32_to_bf16_rne_v(acc[m]);
          else reinterpret_cast<float *>(a.out)[(int64_t)m * a.N + n] = acc[m];
        }
      }
    }
  };
  const int64_t pairs_total = (a.N + kRowsPerWave - 1) / kRowsPerWave;
  const int64_t stride = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t pr = (int64_t)blockIdx.x * (kThreads / 64) + wave; pr < pairs_total; pr += stride) {
    Buf bf;
    load(bf, pr);
    compute(bf, pr);
  }
}

// CUs of the calling thread's current device (queried per launch: no state)
int device_cus_gemv() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n < 1)
    n = 1;
  return n;
}

template <int BITS, int M, int J>
hipError_t launch_j(const SkinnyArgs &a, hipStream_t stream) {
  // two rows per wave step: measured at N = 27648, K = 4608, one row of
  // 4-bit codes, 19.4 us against 20.2 us with four rows (3 waves per SIMD
  // instead of 4) and 24.2 us with the next pair's loads issued ahead of the
  // current pair's arithmetic (2 waves per SIMD)
  constexpr int kRowsPerWave = 2;
  auto kern = gemv_kernel<BITS, M, J, kRowsPerWave>;
  const size_t lds = (size_t)(M * a.K * 2);
  // as many blocks as the CUs hold at once (each loops over row pairs), no
  // more than the pairs need
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kern), kThreads, lds) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const int64_t need = (a.N + kRowsPerWave * (kThreads / 64) - 1) / (kRowsPerWave * (kThreads / 64));
  const unsigned blocks = (unsigned)std::min<int64_t>(need, (int64_t)per_cu * device_cus_gemv());
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <int BITS, int M>
hipError_t launch_m(const SkinnyArgs &a, int J, hipStream_t stream) {
  switch (J) {
    case 1: return launch_j<BITS, M, 1>(a, stream);
    case 2: return launch_j<BITS, M, 2>(a, stream);
    case 3: return launch_j<BITS, M, 3>(a, stream);
    case 4: return launch_j<BITS, M, 4>(a, stream);
    case 5: return launch_j<BITS, M, 5>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS>
hipError_t launch_bits(const SkinnyArgs &a, int J, hipStream_t stream) {
  return a.M == 1 ? launch_m<BITS, 1>(a, J, stream) : launch_m<BITS, 2>(a, J, stream);
}

}  // namespace

int gemv_chunks_per_lane(int bits, int64_t M, int64_t K, int tiled) {
  if (tiled || M < 1 || M > 2 || (bits != 2 && bits != 4 && bits != 8)) return 0;
  const int64_t C = K * bits / 128;
  if (C < 64) return 0;  // fewer chunks than lanes: the skinny kernel serves it
  const int64_t J = (C + 63) / 64;
  // the lane's slice of x stays in registers: at most 96 of them (M * J *
  // pairs per chunk), which keeps two or more waves per SIMD
  const int64_t pairs = 64 / bits;
  // x is staged in LDS (at most 32 KB, so four blocks share a CU)
  return (J <= 5 && M * J * pairs <= 96 && M * K * 2 <= 32768) ? (int)J : 0;
}

hipError_t launch_gemv(int bits, const SkinnyArgs &a, hipStream_t stream) {
  const int J = gemv_chunks_per_lane(bits, a.M, a.K, a.tiled);
  if (J == 0) return hipErrorInvalidValue;
  if (bits == 4) return launch_bits<4>(a, J, stream);
  if (bits == 8) return launch_bits<8>(a, J, stream);
  return launch_bits<2>(a, J, stream);
}

}  // namespace ql
