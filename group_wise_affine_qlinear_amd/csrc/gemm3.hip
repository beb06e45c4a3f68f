// Large-M dequant-GEMM, fast mode: weights dequantized to fp16 in registers,
// fp16 MFMA with fp32 accumulation.
//
// Numerics. The exact mode (gemm2.hip) keeps the codes as integers in the MFMA
// and applies scale and bias per group on the accumulator; that costs two
// fp32 VALU ops per MFMA and bounds the kernel by vector issue. Here every
// weight is instead dequantized once per block tile and group:
//     W16[n,k] = fp16( s[n,g]*q[n,k] + b[n,g] )        (one rounding, packed
//                                                        fp16 fused multiply-add)
// and x enters as fp16 from a prepass that scales each row by a power of two
// 2^-e (e >= 0, the smallest that keeps the row below 2^15; e = 0 for any
// row already in range) so the conversion from bf16 is exact for every
// value of magnitude >= 2^-14 after scaling. The output row is multiplied back
// by 2^e. fp16 keeps 11 significant bits where bf16 keeps 8, so the only
// rounding beyond fp32 accumulation is the half-ulp (2^-11 relative) of W16:
// relative Frobenius error ~2e-4 on the pages' shapes, against 1.7e-3 for
// weights rounded to bf16. The mode requires |W| < 65504 (true for weights
// quantized from fp16-range values: W lies between b and b + (2^bits - 1)*s).
//
// Kernel. Block tile 256 x 256 with eight waves side by side, each owning all
// 256 rows and one 32-column strip (16 x 2 subtiles of v_mfma_f32_16x16x32_f16,
// 128 fp32 accumulators). A wave's strip is exactly one block of the tiled
// weight layout, so each lane loads its own codes (8 bytes per column-half for
// 4-bit) and dequantizes them straight into B fragments: every weight is
// dequantized once, with three packed fp16 ops per pair, and weights never
// pass through LDS. x (fp16) moves by LDS DMA into a ring of three 32 KB
// stages (rows of 128 bytes, 16-byte chunks XOR-swizzled by row, see xswz),
// issued 1.5 groups ahead of its use; one barrier per group, in the middle
// of the group's MFMAs, so the waves of a SIMD never idle at a group edge.
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kBM = 256, kBN = 256, kNW = 8, kNT = 64 * kNW;
constexpr int kWarpsN = 8;                       // waves side by side along N
constexpr int kWM = 256, kWN = 32, kMI = kWM / 16, kNI = kWN / 16;
constexpr int kXStage = kBM * 128;               // bytes of one x stage

__device__ __forceinline__ uint16_t f32_to_bf16_rne3(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two codes (1024 + q as fp16 bit patterns in the halves of v) -> two weights.
__device__ __forceinline__ uint32_t dq_pair(uint32_t v, h2 s2, h2 b2) {
  const h2 q = __builtin_bit_cast(h2, v) - h2{(_Float16)1024.0f, (_Float16)1024.0f};  // exact
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
}

// A lane's codes of one column and group: codes 16h .. 16h+15 (h = lane / 16),
// i.e. k-blocks 2h and 2h+1, as they sit in the tiled layout.
template <int BITS> struct LaneCodes;
// 4-bit block [h'2][col32][4 words]: words 2(h%2), +1 of half h/2, pair order
// (code 2p at bits 4p, code 2p+1 at 16 + 4p).
template <> struct LaneCodes<4> {
  static constexpr int kWords = 2;
  __device__ static constexpr uint32_t offset(int col, int h) { return (h >> 1) * 512 + col * 16 + (h & 1) * 8; }
  __device__ static h8 frag(const uint32_t (&w)[kWords], int c, h2 s2, h2 b2) {
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = dq_pair(and_or(w[c] >> (4 * p), 0x000F000Fu, 0x64006400u), s2, b2);
    return __builtin_bit_cast(h8, o);
  }
};
// 8-bit block [part2][h'2][col32][4 words]: part h%2, half h/2, little-endian.
template <> struct LaneCodes<8> {
  static constexpr int kWords = 4;
  __device__ static constexpr uint32_t offset(int col, int h) { return (h & 1) * 1024 + (h >> 1) * 512 + col * 16; }
  __device__ static h8 frag(const uint32_t (&w)[kWords], int c, h2 s2, h2 b2) {
    u32x4 o;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const uint32_t x = w[2 * c + v];
      // bytes (b0, b1) and (b2, b3) into the halves, over 0x6400 (1024)
      o[2 * v] = dq_pair(perm(0u, x, 0x0C010C00u) | 0x64006400u, s2, b2);
      o[2 * v + 1] = dq_pair(perm(0u, x, 0x0C030C02u) | 0x64006400u, s2, b2);
    }
    return __builtin_bit_cast(h8, o);
  }
};
// 2-bit block [h'2][col32][2 words]: word h%2 of half h/2, pair order (code 2p
// at bits 2p, code 2p+1 at 16 + 2p); chunk c is pairs 4c .. 4c+3.
template <> struct LaneCodes<2> {
  static constexpr int kWords = 1;
  __device__ static constexpr uint32_t offset(int col, int h) { return (h >> 1) * 256 + col * 8 + (h & 1) * 4; }
  __device__ static h8 frag(const uint32_t (&w)[kWords], int c, h2 s2, h2 b2) {
    u32x4 o;
    const uint32_t x = w[0] >> (8 * c);
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = dq_pair(and_or(x >> (2 * p), 0x00030003u, 0x64006400u), s2, b2);
    return __builtin_bit_cast(h8, o);
  }
};

// Chunk swizzle of an x stage: logical 16-byte chunk c of row r sits at
// position c ^ xswz(r). With this function the 64 lanes of an MFMA fragment
// read (16 rows, four k-blocks) spread over the banks best among the
// XOR swizzles measured on MI355X (194 B/clk/CU against 140 for c ^ (r & 7)).
__device__ __forceinline__ int xswz(int r) { return (r ^ (r >> 3)) & 7; }

template <int BITS>
__device__ __forceinline__ void tile_accumulate3(const Gemm3Args &a, unsigned char *x0, unsigned char *x1,
                                                 unsigned char *x2, int64_t m0, int64_t n0, int g_begin,
                                                 int g_end, f32x4 (&acc)[kMI][kNI]) {
  using LC = LaneCodes<BITS>;
  constexpr int WB = 64 * BITS / 8;     // code bytes of one column per group
  constexpr int BB = 32 * WB;           // bytes of one tiled block (32 columns x 1 group)
  constexpr int XPW = (kBM / 8) / kNW;  // 1 KB x copies per wave per group
  constexpr int kSteps = 2 * kMI;       // steps (c, mi) of kNI MFMAs per group
  // A fragments are read this many steps ahead of their use; the ring index
  // t % (kAhead + 1) continues across groups, whose reads ahead wrap into
  // the next stage
  constexpr int kAhead = 3;
  static_assert(kSteps % (kAhead + 1) == 0, "A-fragment ring must divide the steps of a group");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, h = lane >> 4;
  const int G = a.G;

  // x copies: copy i of this wave fills block rows (wave*XPW + i)*8 .. +7, lane L
  // row +L/8 at chunk position L & 7, which holds logical chunk
  // (L & 7) ^ xswz(row). Rows past M repeat the last row.
  const int64_t xrow = a.K * 2;
  const int64_t mrows = min<int64_t>(kBM, a.M - m0);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x16, m0 * xrow, mrows * xrow);
  uint32_t xo[XPW];
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    const int rr = (wave * XPW + i) * 8 + (lane >> 3);
    const int r = rr < mrows ? rr : (int)mrows - 1;
    xo[i] = (uint32_t)(r * xrow) + (uint32_t)(((lane & 7) ^ xswz(rr)) * 16);
  }
  // this wave's strip of the tiled codes; past N repeat the last strip
  const int64_t nstrips = (a.N + 31) / 32;
  int64_t strip = n0 / 32 + wave;
  if (strip >= nstrips) strip = nstrips - 1;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, strip * G * BB, (int64_t)G * BB);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.sb, strip * G * 128, (int64_t)G * 128);
  const uint32_t wo = LC::offset(r16, h), so = (uint32_t)(r16 * 4);
  constexpr uint32_t kColStep = LC::offset(16, 0) - LC::offset(0, 0);  // bytes per 16 columns

  auto load_codes = [&](uint32_t (&w)[kNI][LC::kWords], uint32_t (&sb)[kNI], int gv) {
    const int g = __builtin_amdgcn_readfirstlane(gv);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      if constexpr (BITS == 4) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, wo + ni * kColStep, (uint32_t)g * BB, 0);
        w[ni][0] = v[0];
        w[ni][1] = v[1];
      } else if constexpr (BITS == 8) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, wo + ni * kColStep, (uint32_t)g * BB, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t) w[ni][t] = v[t];
      } else {
        w[ni][0] = __builtin_amdgcn_raw_buffer_load_b32(wr, wo + ni * kColStep, (uint32_t)g * BB, 0);
      }
      sb[ni] = __builtin_amdgcn_raw_buffer_load_b32(sr, so + ni * 64u, (uint32_t)g * 128u, 0);
    }
  };
  auto issue_x = [&](unsigned char *X, int gv) {
    const int g = __builtin_amdgcn_readfirstlane(gv);
#pragma unroll
    for (int i = 0; i < XPW; ++i) dma16(xr, xo[i], (uint32_t)g * 128u, X + (wave * XPW + i) * 1024);
  };

  // A fragments: rows mi*16 + r16, k-block 2h + c, at chunk position
  // (2h + c) ^ xswz(mi*16 + r16) = (2h + c) ^ ((r16 ^ (r16 >> 3) ^ 2mi) & 7):
  // four lane offsets per chunk, by mi & 3
  int a_off[2][4];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) a_off[c][q] = ((2 * h + c) ^ ((r16 ^ (r16 >> 3) ^ (2 * q)) & 7)) * 16;
  const int a_base = r16 * 128;
  h8 af[kAhead + 1];
  auto read_a = [&](const unsigned char *X, int t) {
    const int c = t / kMI, mi = t % kMI;
    af[t % (kAhead + 1)] = *reinterpret_cast<const h8 *>(X + a_base + mi * 2048 + a_off[c][mi & 3]);
  };

  // B fragments of the group being multiplied, built from codes that arrived
  // one group earlier; a group past the end gets zero scale and bias, so its
  // weights are zero and its step adds nothing.
  h8 bf[kNI][2];
  uint32_t cw[kNI][LC::kWords];  // codes of the group after the one in bf
  uint32_t sbw[kNI];
  auto dequant_frag = [&](h8 (&dst)[kNI][2], bool valid, int f) {
    const int ni = f >> 1, c = f & 1;
    const uint32_t v = valid ? sbw[ni] : 0u;
    const h2 s2 = __builtin_bit_cast(h2, (v & 0xFFFFu) * 0x10001u);
    const h2 b2 = __builtin_bit_cast(h2, (v >> 16) * 0x10001u);
    dst[ni][c] = LC::frag(cw[ni], c, s2, b2);
  };

  // One group on stage X. First half: MFMAs on the fragments in hand. Then
  // one barrier, after which the next stage XN is complete and the stage of
  // the previous group (XD) is free: the x copies for two groups ahead go
  // into XD and the codes for two groups ahead are requested. Second half:
  // MFMAs, with the next group's B fragments dequantized in between and the
  // first A fragments of XN read ahead, so the next group starts without a
  // stall.
  auto step = [&](const unsigned char *X, const unsigned char *XN, unsigned char *XD, int g) {
    h8 bn[kNI][2];
    uint32_t cn[kNI][LC::kWords], sn[kNI];
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const int c = t / kMI, mi = t % kMI;
      if (t == kSteps / 2) {
        __syncthreads();
        issue_x(XD, min(g + 2, g_end - 1));
        load_codes(cn, sn, min(g + 2, g_end - 1));
      }
      if (t + kAhead < kSteps) read_a(X, t + kAhead);
      else read_a(XN, t + kAhead - kSteps);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[t % (kAhead + 1)], bf[ni][c], acc[mi][ni], 0, 0, 0);
      if (t >= kSteps / 2 && (t & 3) == 1) dequant_frag(bn, g + 1 < g_end, (t - kSteps / 2) >> 2);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      bf[ni][0] = bn[ni][0];
      bf[ni][1] = bn[ni][1];
      sbw[ni] = sn[ni];
#pragma unroll
      for (int u = 0; u < LC::kWords; ++u) cw[ni][u] = cn[ni][u];
    }
  };

#pragma unroll
  for (int i = 0; i < kMI; ++i)
#pragma unroll
    for (int j = 0; j < kNI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Groups run in threes (x stages 0, 1, 2) in straight-line code: loads for
  // a group past the end are clamped to the last group and its weights
  // dequantize to zero, so the accumulators never pass through a branch.
  if (g_begin < g_end) {
    load_codes(cw, sbw, g_begin);
    issue_x(x0, g_begin);
    issue_x(x1, min(g_begin + 1, g_end - 1));
  }
  __syncthreads();  // first two stages and the first codes have arrived
  if (g_begin < g_end) {
#pragma unroll
    for (int f = 0; f < 2 * kNI; ++f) dequant_frag(bf, true, f);
    load_codes(cw, sbw, min(g_begin + 1, g_end - 1));
#pragma unroll
    for (int t = 0; t < kAhead; ++t) read_a(x0, t);
  }
  for (int g = g_begin; g < g_end; g += 3) {
    step(x0, x1, x2, g);
    step(x1, x2, x0, g + 1);
    step(x2, x0, x1, g + 2);
  }
  __syncthreads();  // every copy has landed and every stage is free
}

template <bool OUT_BF16>
__device__ __forceinline__ void tile_store3(const Gemm3Args &a, int64_t m0, int64_t n0,
                                            const f32x4 (&acc)[kMI][kNI]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWarpsN, wn = wave % kWarpsN;  // wm == 0
  const int r16 = lane & 15, h = lane >> 4;
  const int64_t row0 = m0 + wm * kWM + 4 * h;
  const int64_t col0 = n0 + wn * kWN + r16;
  const bool full = (m0 + kBM <= a.M) && (n0 + kBN <= a.N);
#pragma unroll
  for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = row0 + mi * 16 + i;
      if (!full && m >= a.M) continue;
      const float rs = a.rowscale[m];
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        const int64_t n = col0 + ni * 16;
        if (!full && n >= a.N) continue;
        const float v = acc[mi][ni][i] * rs;
        if constexpr (OUT_BF16) reinterpret_cast<uint16_t *>(a.out)[m * a.N + n] = f32_to_bf16_rne3(v);
        else reinterpret_cast<float *>(a.out)[m * a.N + n] = v;
      }
    }
}

// One launch covers dp_tiles whole tiles (t = blockIdx.x, + gridDim.x, ...)
// and, when sk_tiles > 0, the last sk_tiles tiles cut into sk_pieces K-ranges
// that run first, one per block: with one block per CU a tile count just past
// a multiple of the CU count would otherwise leave most CUs idle for a whole
// tile time. Each piece writes an fp32 partial (thread-major, so writes and the
// later reads are contiguous); the piece that arrives last (atomic count)
// adds all partials in piece order, so the result is independent of timing,
// stores the tile and re-arms the count.
template <int BITS, bool OUT_BF16>
__global__ __launch_bounds__(kNT, 1) void gemm3_kernel(Gemm3Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char x0[kXStage];
  __shared__ __attribute__((aligned(16))) unsigned char x1[kXStage];
  __shared__ __attribute__((aligned(16))) unsigned char x2[kXStage];
  __shared__ int s_arrived;
  const int tid = threadIdx.x;
  const int tiles_n = (int)((a.N + kBN - 1) / kBN);
  f32x4 acc[kMI][kNI];

  if (a.sk_tiles > 0 && (int)blockIdx.x < a.sk_tiles * a.sk_pieces) {
    const int tail = blockIdx.x / a.sk_pieces, piece = blockIdx.x % a.sk_pieces;
    const int tile = a.dp_tiles + tail;
    const int64_t m0 = (int64_t)(tile / tiles_n) * kBM, n0 = (int64_t)(tile % tiles_n) * kBN;
    const int gpp = (a.G + a.sk_pieces - 1) / a.sk_pieces;
    const int gb = piece * gpp, ge = min(a.G, gb + gpp);
    tile_accumulate3<BITS>(a, x0, x1, x2, m0, n0, gb, ge, acc);
    float *part = a.sk_partial + (int64_t)tail * a.sk_pieces * (kBM * kBN);
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
        *reinterpret_cast<f32x4 *>(part + (int64_t)piece * (kBM * kBN) + ((mi * kNI + ni) * kNT + tid) * 4) =
            acc[mi][ni];
    __syncthreads();  // every thread's partial stores are complete
    if (tid == 0) {
      // make this block's partial visible device-wide, then count it
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      s_arrived = __hip_atomic_fetch_add(&a.sk_count[tail], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (s_arrived == a.sk_pieces - 1) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    if (s_arrived == a.sk_pieces - 1) {
#pragma unroll
      for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni) {
          const f32x4 mine = acc[mi][ni];
          const int64_t e = ((mi * kNI + ni) * kNT + tid) * 4;
          f32x4 sum = piece == 0 ? mine : *reinterpret_cast<const f32x4 *>(part + e);
          for (int p = 1; p < a.sk_pieces; ++p)
            sum += p == piece ? mine : *reinterpret_cast<const f32x4 *>(part + (int64_t)p * (kBM * kBN) + e);
          acc[mi][ni] = sum;
        }
      tile_store3<OUT_BF16>(a, m0, n0, acc);
      if (tid == 0) a.sk_count[tail] = 0;
    }
  }
  for (int t = blockIdx.x; t < a.dp_tiles; t += gridDim.x) {
    const int tile = xcd_remap(t, a.dp_tiles);
    const int64_t m0 = (int64_t)(tile / tiles_n) * kBM, n0 = (int64_t)(tile % tiles_n) * kBN;
    tile_accumulate3<BITS>(a, x0, x1, x2, m0, n0, 0, a.G, acc);
    tile_store3<OUT_BF16>(a, m0, n0, acc);
  }
}

// x (bf16) -> x16 (fp16) with a power-of-two scale per row. One block per
// row: the row's max magnitude picks e (the smallest e >= 0 with max*2^-e <
// 2^15); every value is multiplied by 2^-e (exact) and rounded to fp16.
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
  int e = 0;
  while (e < 120 && mx * __uint_as_float((uint32_t)(127 - e) << 23) >= 32768.0f) ++e;  // mx * 2^-e
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
  int e = 0;
  while (e < 120 && mx * __uint_as_float((uint32_t)(127 - e) << 23) >= 32768.0f) ++e;
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

template <int BITS>
hipError_t launch3_bits(const Gemm3Args &a, hipStream_t stream) {
  if (a.out_bf16)
    hipLaunchKernelGGL((gemm3_kernel<BITS, true>), dim3(a.grid_x), dim3(kNT), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm3_kernel<BITS, false>), dim3(a.grid_x), dim3(kNT), 0, stream, a);
  return hipGetLastError();
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
      n = 1;
    cus = n;
  }
  return cus;
}

}  // namespace

Gemm3Plan gemm3_plan(int64_t M, int64_t N, int G, int slots) {
  Gemm3Plan p{};
  p.tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  p.dp_tiles = (int)p.tiles;
  p.grid_x = (int)p.tiles;
  if (slots <= 0) slots = device_cus();  // one block per CU
  if (G < 2 || p.tiles <= slots || p.tiles % slots == 0) return p;
  const int64_t dp = (p.tiles / slots) * slots;
  const int tail = (int)(p.tiles - dp);
  int pieces = slots / tail;
  if (pieces > G) pieces = G;
  if (pieces < 2) return p;
  const int gpp = (G + pieces - 1) / pieces;
  pieces = (G + gpp - 1) / gpp;
  p.dp_tiles = (int)dp;
  p.sk_tiles = tail;
  p.sk_pieces = pieces;
  p.grid_x = slots;
  const size_t part = (size_t)tail * pieces * kBM * kBN * 4u;
  p.sk_partial_bytes = ((part + 255) / 256) * 256 + (((size_t)tail * 4u + 255) / 256) * 256;
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
  if (bits == 4) return launch3_bits<4>(a, stream);
  if (bits == 8) return launch3_bits<8>(a, stream);
  if (bits == 2) return launch3_bits<2>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ql
