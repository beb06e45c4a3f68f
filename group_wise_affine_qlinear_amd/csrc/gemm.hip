// Large-M fused dequant-GEMM for gfx950: packed 2/4/8-bit codes, f16 scale and
// bias per 64-wide K group, bf16 activations, fp32 accumulation and output.
//
// Numerics (exact-integer operand design). The codes are fed to the bf16 MFMA
// as exact integers (offset by 128 for 2/4-bit, see CodeOffset), one 64-wide
// group at a time into a fresh accumulator P. The group's scale and bias are
// then applied in fp32:
//     acc += s[n,g] * P[m,n]  +  (b[n,g] - offset*s[n,g]) * xsum[m,g]
// where xsum[m,g] is the fp32 sum of x over the group. Since every product in
// P is exact and s*q is exact in fp32, this differs from the fp64 product
// x @ W_hat^T only by fp32 accumulation rounding.
//
// Block tile BM x BN, one K group (64) per pipeline step, two LDS stages with
// register prefetch of the next group, one barrier per step. Waves form a
// WARPS_M x WARPS_N grid; each wave owns (BM/WARPS_M) x (BN/WARPS_N) outputs as
// 16x16 MFMA subtiles (v_mfma_f32_16x16x32_bf16).
//
// Operand K mapping inside a group: the group's 64 codes are 8 blocks of 8.
// For K-chunk c (0,1) lane group h = lane/16 supplies block j = 2h + c for
// both A (x) and B (codes), so one 8-byte LDS read gives a lane both chunks of
// 4-bit codes. The MFMA sums over K, so any mapping shared by A and B is valid.
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

constexpr int kXPitch = 72;  // bf16 per LDS row of x (64 + 8 pad): conflict-free b128 reads

template <int BITS> struct WLayout;
template <> struct WLayout<4> { static constexpr int bytes = 32, pitch = 40; };
template <> struct WLayout<8> { static constexpr int bytes = 64, pitch = 80; };
template <> struct WLayout<2> { static constexpr int bytes = 16, pitch = 20; };

template <int BITS, int BM, int BN>
struct Smem {
  static constexpr int x_stage = BM * kXPitch * 2;
  static constexpr int w_stage = BN * WLayout<BITS>::pitch;
  static constexpr int sb_stage = BN * 4;
  static constexpr int xs_stage = BM * 4;
  static constexpr int x_off = 0;
  static constexpr int w_off = x_off + 2 * x_stage;
  static constexpr int s_off = w_off + ((2 * w_stage + 15) / 16) * 16;
  static constexpr int b_off = s_off + 2 * sb_stage;
  static constexpr int xs_off = b_off + 2 * sb_stage;
  static constexpr int total = xs_off + 2 * xs_stage;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int BITS, int BM, int BN, int WARPS_M, int WARPS_N>
__global__ __launch_bounds__(64 * WARPS_M * WARPS_N)
void gemm_kernel(GemmArgs a) {
  constexpr int NT = 64 * WARPS_M * WARPS_N;
  constexpr int WM = BM / WARPS_M, WN = BN / WARPS_N;
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int WB = WLayout<BITS>::bytes, WP = WLayout<BITS>::pitch;
  constexpr int XCH = BM * 8;                 // 16-byte chunks of x per group
  constexpr int XPT = (XCH + NT - 1) / NT;
  constexpr int WCH = BN * (WB / 16);         // 16-byte chunks of codes per group
  constexpr int WPT = (WCH + NT - 1) / NT;
  constexpr int XSCH = BM / 4;                // 16-byte chunks of xsum per group
  using S = Smem<BITS, BM, BN>;
  static_assert(BM % (16 * WARPS_M) == 0 && BN % (16 * WARPS_N) == 0, "tile");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WARPS_N, wn = wave % WARPS_N;
  const int r16 = lane & 15, h = lane >> 4;

  const int tiles_n = (int)((a.N + BN - 1) / BN);
  const int tiles_m = (int)((a.M + BM - 1) / BM);
  const int tile = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int tm = tile / tiles_n, tn = tile % tiles_n;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int split = blockIdx.y;
  const int g_begin = split * a.groups_per_split;
  int g_end = g_begin + a.groups_per_split;
  if (g_end > a.G) g_end = a.G;

  const int64_t wrow_words = a.K * BITS / 32;
  const float offset = CodeOffset<BITS>::value;

  // ---- register prefetch buffers
  u32x4 xr[XPT];
  u32x4 wr[WPT];
  uint16_t sr = 0, br = 0;
  u32x4 xsr = {0, 0, 0, 0};

  auto load_group = [&](int g) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = tid + i * NT;
      if (idx < XCH) {
        const int row = idx >> 3, ch = idx & 7;
        int64_t m = m0 + row;
        if (m >= a.M) m = a.M - 1;
        xr[i] = *reinterpret_cast<const u32x4 *>(a.x + m * a.K + (int64_t)g * 64 + ch * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int idx = tid + i * NT;
      if (idx < WCH) {
        const int row = idx / (WB / 16), ch = idx % (WB / 16);
        int64_t n = n0 + row;
        if (n >= a.N) n = a.N - 1;
        wr[i] = *reinterpret_cast<const u32x4 *>(a.w + n * wrow_words + (int64_t)g * (2 * BITS) + ch * 4);
      }
    }
    if (tid < BN) {
      int64_t n = n0 + tid;
      if (n >= a.N) n = a.N - 1;
      sr = a.s[n * a.G + g];
      br = a.b[n * a.G + g];
    }
    if (tid < XSCH) {
      xsr = *reinterpret_cast<const u32x4 *>(a.xsum + (int64_t)g * a.Mp + m0 + tid * 4);
    }
  };

  auto store_group = [&](int st) {
    unsigned char *xs_base = smem + S::x_off + st * S::x_stage;
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = tid + i * NT;
      if (idx < XCH) {
        const int row = idx >> 3, ch = idx & 7;
        *reinterpret_cast<u32x4 *>(xs_base + row * (kXPitch * 2) + ch * 16) = xr[i];
      }
    }
    unsigned char *w_base = smem + S::w_off + st * S::w_stage;
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int idx = tid + i * NT;
      if (idx < WCH) {
        const int row = idx / (WB / 16), ch = idx % (WB / 16);
        unsigned char *p = w_base + row * WP + ch * 16;
        if constexpr (BITS == 8) {
          *reinterpret_cast<u32x4 *>(p) = wr[i];
        } else if constexpr (BITS == 4) {
          u32x2 lo = {wr[i][0], wr[i][1]}, hi = {wr[i][2], wr[i][3]};
          *reinterpret_cast<u32x2 *>(p) = lo;
          *reinterpret_cast<u32x2 *>(p + 8) = hi;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) reinterpret_cast<uint32_t *>(p)[j] = wr[i][j];
        }
      }
    }
    if (tid < BN) {
      const float sf = f16_to_f32(sr);
      const float bf = f16_to_f32(br);
      reinterpret_cast<float *>(smem + S::s_off + st * S::sb_stage)[tid] = sf;
      reinterpret_cast<float *>(smem + S::b_off + st * S::sb_stage)[tid] = __builtin_fmaf(-offset, sf, bf);
    }
    if (tid < XSCH) {
      *reinterpret_cast<u32x4 *>(smem + S::xs_off + st * S::xs_stage + tid * 16) = xsr;
    }
  };

  f32x4 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (g_begin < g_end) {
    load_group(g_begin);
    store_group(0);
  }
  __syncthreads();

  for (int g = g_begin; g < g_end; ++g) {
    const int st = (g - g_begin) & 1;
    const bool more = (g + 1) < g_end;
    if (more) load_group(g + 1);

    const unsigned char *xl = smem + S::x_off + st * S::x_stage;
    const unsigned char *wl = smem + S::w_off + st * S::w_stage;
    const float *sl = reinterpret_cast<const float *>(smem + S::s_off + st * S::sb_stage);
    const float *bl = reinterpret_cast<const float *>(smem + S::b_off + st * S::sb_stage);
    const float *xsl = reinterpret_cast<const float *>(smem + S::xs_off + st * S::xs_stage);

    bf16x8 bq[NI][2];
    float sv[NI], bv[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int row = wn * WN + ni * 16 + r16;
      if constexpr (BITS == 4) {
        const u32x2 wv = *reinterpret_cast<const u32x2 *>(wl + row * WP + 8 * h);
        bq[ni][0] = as_bf16x8(unpack8_b4(wv[0]));
        bq[ni][1] = as_bf16x8(unpack8_b4(wv[1]));
      } else if constexpr (BITS == 8) {
        const u32x4 wv = *reinterpret_cast<const u32x4 *>(wl + row * WP + 16 * h);
        bq[ni][0] = as_bf16x8(unpack8_b8(wv[0], wv[1]));
        bq[ni][1] = as_bf16x8(unpack8_b8(wv[2], wv[3]));
      } else {
        const uint32_t wv = *reinterpret_cast<const uint32_t *>(wl + row * WP + 4 * h);
        bq[ni][0] = as_bf16x8(unpack8_b2(wv, 0));
        bq[ni][1] = as_bf16x8(unpack8_b2(wv, 1));
      }
      sv[ni] = sl[row];
      bv[ni] = bl[row];
    }

#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = wm * WM + mi * 16 + r16;
      const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(xl + row * (kXPitch * 2) + 32 * h);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(xl + row * (kXPitch * 2) + 32 * h + 16);
      const f32x4 xs = *reinterpret_cast<const f32x4 *>(xsl + wm * WM + mi * 16 + 4 * h);
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bq[ni][0], p, 0, 0, 0);
        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bq[ni][1], p, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float t = __builtin_fmaf(sv[ni], p[i], acc[mi][ni][i]);
          acc[mi][ni][i] = __builtin_fmaf(bv[ni], xs[i], t);
        }
      }
    }

    if (more) store_group(st ^ 1);
    __syncthreads();
  }

  // ---- store
  const bool to_partial = a.splits > 1;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int64_t n = n0 + wn * WN + ni * 16 + r16;
      if (n >= a.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * WM + mi * 16 + 4 * h + i;
        if (m >= a.M) continue;
        const float v = acc[mi][ni][i];
        if (to_partial) {
          a.partial[((int64_t)split * a.M + m) * a.N + n] = v;
        } else if (a.out_bf16) {
          reinterpret_cast<uint16_t *>(a.out)[m * a.N + n] = f32_to_bf16_rne(v);
        } else {
          reinterpret_cast<float *>(a.out)[m * a.N + n] = v;
        }
      }
    }
  }
}

// Per-group row sums of x: xsum[g, m] = sum_{k in group g} x[m, k] (fp32).
// Eight lanes share one (m, g): each sums 8 values, then a 3-step butterfly.
__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t *x, float *xs, int64_t M,
                                                   int64_t K, int64_t Mp) {
  const int64_t G = K / 64;
  const int64_t pair = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3;
  const int sub = threadIdx.x & 7;
  const bool valid = pair < M * G;
  const int64_t m = valid ? pair / G : 0, g = valid ? pair % G : 0;
  float sum = 0.f;
  if (valid) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(x + m * K + g * 64 + sub * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) sum += bf16_lo(v[j]) + bf16_hi(v[j]);
  }
  sum += __shfl_xor(sum, 1);
  sum += __shfl_xor(sum, 2);
  sum += __shfl_xor(sum, 4);
  if (valid && sub == 0) xs[g * Mp + m] = sum;
}

__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *partial, int splits,
                                                            int64_t count, void *out, int out_bf16) {
  const int64_t i4 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= count) return;
  if (i4 + 4 <= count) {
    f32x4 s = *reinterpret_cast<const f32x4 *>(partial + i4);
    for (int k = 1; k < splits; ++k) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(partial + (int64_t)k * count + i4);
      s += v;
    }
    if (out_bf16) {
      uint16_t *o = reinterpret_cast<uint16_t *>(out) + i4;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = f32_to_bf16_rne(s[j]);
    } else {
      *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + i4) = s;
    }
  } else {
    for (int64_t i = i4; i < count; ++i) {
      float s = partial[i];
      for (int k = 1; k < splits; ++k) s += partial[(int64_t)k * count + i];
      if (out_bf16) reinterpret_cast<uint16_t *>(out)[i] = f32_to_bf16_rne(s);
      else reinterpret_cast<float *>(out)[i] = s;
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint16_t *out, int64_t halves) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < halves) out[i] = 0u;
}

template <int BITS, int BM, int BN, int WMW, int WNW>
hipError_t launch_tile(const GemmArgs &a, hipStream_t stream) {
  using S = Smem<BITS, BM, BN>;
  auto kern = gemm_kernel<BITS, BM, BN, WMW, WNW>;
  // set on every launch (cheap; the library keeps no per-device state)
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, S::total);
  if (e != hipSuccess) return e;
  const int tiles = (int)(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN));
  dim3 grid(tiles, a.splits);
  hipLaunchKernelGGL(kern, grid, dim3(64 * WMW * WNW), S::total, stream, a);
  return hipGetLastError();
}

// id, BM, BN, WARPS_M, WARPS_N
#define QL_TILES(X)            \
  X(1, 128, 128, 2, 2)         \
  X(2, 256, 128, 4, 2)         \
  X(3, 128, 256, 2, 4)         \
  X(5, 64, 128, 1, 2)

const TileInfo kTiles[] = {
#define QL_TILE_INFO(id, bm, bn, wmw, wnw) {id, bm, bn, wmw, wnw, "gemm_" #bm "x" #bn "_w" #wmw "x" #wnw, 1},
    QL_TILES(QL_TILE_INFO)
#undef QL_TILE_INFO
    {10, 256, 128, 2, 2, "gemm2_256x128_w2x2", 2},
    {11, 128, 128, 1, 2, "gemm2_128x128_w1x2", 2},
    {20, 256, 256, 2, 4, "gemm3_f16_256x256_w2x4", 3},
    {30, 256, 256, 1, 8, "gemm4_bf16x2_256x256_w1x8", 4},
};

}  // namespace

const TileInfo *gemm_tile(int id) {
  for (const TileInfo &t : kTiles)
    if (t.id == id) return &t;
  return nullptr;
}

bool gemm_tile_supports_tiled(int id) {
  const TileInfo *t = gemm_tile(id);
  return t && t->gen >= 2;
}

int gemm_tile_count() { return (int)(sizeof(kTiles) / sizeof(kTiles[0])); }

size_t gemm_lds_bytes(int bits, int id) {
#define QL_TILE_LDS(tid, bm, bn, wmw, wnw)                   \
  if (id == tid) {                                           \
    if (bits == 4) return Smem<4, bm, bn>::total;            \
    if (bits == 8) return Smem<8, bm, bn>::total;            \
    if (bits == 2) return Smem<2, bm, bn>::total;            \
  }
  QL_TILES(QL_TILE_LDS)
#undef QL_TILE_LDS
  return 0;
}

hipError_t launch_gemm(int bits, int tile_id, const GemmArgs &a, hipStream_t stream) {
  if (tile_id >= 10 && tile_id < 20) return launch_gemm2(bits, tile_id, false, a, stream);
#define QL_TILE_LAUNCH(tid, bm, bn, wmw, wnw)                                      \
  if (tile_id == tid) {                                                            \
    if (bits == 4) return launch_tile<4, bm, bn, wmw, wnw>(a, stream);             \
    if (bits == 8) return launch_tile<8, bm, bn, wmw, wnw>(a, stream);             \
    if (bits == 2) return launch_tile<2, bm, bn, wmw, wnw>(a, stream);             \
  }
  QL_TILES(QL_TILE_LAUNCH)
#undef QL_TILE_LAUNCH
  return hipErrorInvalidValue;
}

hipError_t launch_xsum(const uint16_t *x, float *xsum, int64_t M, int64_t K, int64_t Mp,
                       hipStream_t stream) {
  const int64_t threads = M * (K / 64) * 8;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(xsum_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, xsum, M, K, Mp);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float *partial, int splits, int64_t M, int64_t N, void *out,
                                int out_bf16, hipStream_t stream) {
  const int64_t count = M * N;
  const int64_t threads = (count + 3) / 4;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, partial,
                     splits, count, out, out_bf16);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void *out, int64_t count, int out_bf16, hipStream_t stream) {
  const int64_t halves = count * (out_bf16 ? 1 : 2);
  const int64_t blocks = (halves + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<uint16_t *>(out), halves);
  return hipGetLastError();
}

}  // namespace ql
