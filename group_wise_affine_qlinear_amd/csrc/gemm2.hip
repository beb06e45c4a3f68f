// Large-M fused dequant-GEMM, second generation: 128x64 wave tiles fed by LDS
// DMA.
//
// Same numerics as gemm.hip (exact integer codes on bf16 MFMA, per-group fp32
// scale and bias), reorganised for gfx950 throughput:
//  * each wave owns a 128x64 output tile (8x4 subtiles of 16x16), so one
//    unpacked code fragment feeds 8 MFMA pairs and one x fragment feeds 4;
//  * global -> LDS staging uses global_load_lds_dwordx4 (each lane moves 16
//    bytes straight into LDS at base + 16*lane), so the next group's operands
//    occupy no registers while the current group is computed; the two LDS
//    stages are distinct objects and the group loop is unrolled by two, which
//    lets the compiler see that reads of one stage never wait for the copies
//    into the other;
//  * x tiles live in LDS as 128-byte rows with the 16-byte chunks XOR-swizzled
//    by row (chunk c of row r at position c ^ (r & 7)); the swizzle is applied
//    on the global side of the copy (lane L of a copy loads logical chunk
//    (L & 7) ^ (L >> 3) of its row), so fragment reads hit distinct banks;
//  * codes come either in the canonical layout or in the tiled layout of
//    layout.hip, copied verbatim; fragment reads pick the right bytes of each.
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

__device__ __forceinline__ uint16_t f32_to_bf16_rne2(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Bytes of one output column's codes per 64-wide group.
template <int BITS> struct WRow { static constexpr int bytes = 64 * BITS / 8; };

template <int BITS, int BM, int BN>
struct Stage {
  unsigned char x[BM * 128];                 // BM rows x 64 bf16, chunk-swizzled
  unsigned char w[BN * WRow<BITS>::bytes];   // codes as stored in global memory
  float xs[BM];                              // xsum of the group per row
  f32x2 sb[BN];                              // (scale, bias - offset*scale) per column
};

template <int BITS, bool TILED, int BM, int BN, int WARPS_M, int WARPS_N>
struct Gemm2Shape {
  static constexpr int NT = 64 * WARPS_M * WARPS_N;
  static constexpr int MI = BM / WARPS_M / 16, NI = BN / WARPS_N / 16;
};

// Accumulates groups [g_begin, g_end) of the BM x BN output tile at (m0, n0)
// into acc (zeroed first). Leaves both LDS stages free on return.
template <int BITS, bool TILED, int BM, int BN, int WARPS_M, int WARPS_N>
__device__ __forceinline__ void tile_accumulate(const GemmArgs &a, Stage<BITS, BM, BN> &st0,
                                                Stage<BITS, BM, BN> &st1, int64_t m0, int64_t n0,
                                                int g_begin, int g_end,
                                                f32x4 (&acc)[BM / WARPS_M / 16][BN / WARPS_N / 16]) {
  constexpr int NW = WARPS_M * WARPS_N;
  constexpr int NT = 64 * NW;
  constexpr int WM = BM / WARPS_M, WN = BN / WARPS_N;
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int WB = WRow<BITS>::bytes;
  constexpr int XCOPIES = BM / 8;              // 1 KB copies of x per group (8 rows each)
  constexpr int XPW = XCOPIES / NW;            // per wave
  constexpr int WCOPIES = BN * WB / 1024;      // 1 KB copies of codes per group
  constexpr int WPW = (WCOPIES + NW - 1) / NW;
  constexpr int BB = 32 * WB;                  // bytes of one tiled block (32 columns)
  static_assert(XCOPIES % NW == 0, "x copies must split evenly over waves");
  static_assert(BN * WB % 1024 == 0, "code tile must be whole 1 KB copies");
  static_assert(BM == 128 || BM == 256, "xsum copy covers 128 or 256 rows");
  static_assert(BN <= NT && BN % 32 == 0, "scale staging");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WARPS_N, wn = wave % WARPS_N;
  const int r16 = lane & 15, h = lane >> 4;
  const int G = a.G;
  const float offset = CodeOffset<BITS>::value;

  // ---- copy plan: buffer resources based at this block's first row / column
  // (so every per-lane offset is a small 32-bit value) and per-lane offsets
  // fixed for the whole K loop; the group step goes into the scalar offset.
  // x: copy i of this wave covers rows R = (wave*XPW + i)*8 .. R+7; lane L
  // takes row R + L/8 and logical chunk (L & 7) ^ (L >> 3). Rows past M are
  // clamped to the last row (their outputs are never stored).
  const int64_t row_bytes_x = a.K * 2;
  const int64_t mrows = min<int64_t>(BM, a.M - m0);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, m0 * row_bytes_x, mrows * row_bytes_x);
  uint32_t xo[XPW];
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    int r = (wave * XPW + i) * 8 + (lane >> 3);
    if (r >= mrows) r = (int)mrows - 1;
    xo[i] = (uint32_t)(r * row_bytes_x) + (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16);
  }
  // codes: copy j = wave + i*NW covers tile bytes e = j*1024 + 16*lane
  const int64_t nstrips = (a.N + 31) / 32;
  const int64_t row_bytes = a.K * BITS / 8;
  __amdgpu_buffer_rsrc_t wr;
  uint32_t wo[WPW];
  if constexpr (TILED) {
    const int64_t s0 = n0 / 32, ns = min<int64_t>(BN / 32, nstrips - s0);
    wr = make_rsrc(a.w, s0 * G * BB, ns * G * BB);
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
      const int j = wave + i * NW;
      const int e = (j < WCOPIES ? j : 0) * 1024 + 16 * lane;
      int st = e / BB;
      if (st >= ns) st = (int)ns - 1;
      wo[i] = (uint32_t)(st * G * BB + (e % BB));
    }
  } else {
    const int64_t nrows = min<int64_t>(BN, a.N - n0);
    wr = make_rsrc(a.w, n0 * row_bytes, nrows * row_bytes);
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
      const int j = wave + i * NW;
      const int e = (j < WCOPIES ? j : 0) * 1024 + 16 * lane;
      int r = e / WB;
      if (r >= nrows) r = (int)nrows - 1;
      wo[i] = (uint32_t)(r * row_bytes + (e % WB));
    }
  }
  const uint32_t w_gstride = TILED ? BB : WB;  // bytes per group step
  // scale / bias: thread tid < BN stages column tid through one register
  const bool sb_on = tid < BN;
  const uint16_t *sg = nullptr, *bg = nullptr;
  const uint32_t *sbg = nullptr;
  {
    const int c = sb_on ? tid : 0;
    if constexpr (TILED) {
      int64_t s = n0 / 32 + c / 32;
      if (s >= nstrips) s = nstrips - 1;
      sbg = a.sb + s * G * 32 + (c % 32);
    } else {
      int64_t n = n0 + c;
      if (n >= a.N) n = a.N - 1;
      sg = a.s + n * G;
      bg = a.b + n * G;
    }
  }
  uint32_t sbr = 0;

  auto issue = [&](Stage<BITS, BM, BN> &S, int gv) {
    const int g = __builtin_amdgcn_readfirstlane(gv);  // uniform: scalar offsets below
#pragma unroll
    for (int i = 0; i < XPW; ++i) dma16(xr, xo[i], (uint32_t)g * 128u, S.x + (wave * XPW + i) * 1024);
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
      const int j = wave + i * NW;
      if (j < WCOPIES) dma16(wr, wo[i], (uint32_t)g * w_gstride, S.w + j * 1024);
    }
    if (wave == 0 && (BM == 256 || lane < 32)) {
      // this group's xsum row block: floats 4L .. 4L+3 for lane L
      const __amdgpu_buffer_rsrc_t xsr = make_rsrc(a.xsum, ((int64_t)g * a.Mp + m0) * 4, BM * 4);
      dma16(xsr, 16u * lane, 0u, S.xs);
    }
    if (sb_on) {
      if constexpr (TILED) sbr = sbg[g * 32];
      else sbr = (uint32_t)sg[g] | ((uint32_t)bg[g] << 16);
    }
  };
  auto finish = [&](Stage<BITS, BM, BN> &S) {
    if (sb_on) {
      const float sf = f16_to_f32((uint16_t)(sbr & 0xFFFFu));
      const float bf = f16_to_f32((uint16_t)(sbr >> 16));
      S.sb[tid] = f32x2{sf, __builtin_fmaf(-offset, sf, bf)};
    }
  };

#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // fragment read offsets inside a stage (rows of subtile mi add mi*16)
  const int sw = r16 & 7;
  const int xa0 = (wm * WM + r16) * 128 + ((2 * h) ^ sw) * 16;
  const int xa1 = (wm * WM + r16) * 128 + ((2 * h + 1) ^ sw) * 16;
  const int xsa = wm * WM + 4 * h;

  auto compute = [&](const Stage<BITS, BM, BN> &S) {
    bf16x8 bq[NI][2];
    f32x2 sbv[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int col = wn * WN + ni * 16 + r16;
      // lane group h takes codes 16h .. 16h+15 of the group (k-blocks 2h, 2h+1)
      if constexpr (BITS == 4) {
        const int off = TILED ? (col / 32) * BB + (h >> 1) * 512 + (col % 32) * 16 + (h & 1) * 8 : col * WB + h * 8;
        const u32x2 wv = *reinterpret_cast<const u32x2 *>(S.w + off);
        bq[ni][0] = as_bf16x8(TILED ? unpack8_b4_pair(wv[0]) : unpack8_b4(wv[0]));
        bq[ni][1] = as_bf16x8(TILED ? unpack8_b4_pair(wv[1]) : unpack8_b4(wv[1]));
      } else if constexpr (BITS == 8) {
        const int off = TILED ? (col / 32) * BB + (h & 1) * 1024 + (h >> 1) * 512 + (col % 32) * 16 : col * WB + h * 16;
        const u32x4 wv = *reinterpret_cast<const u32x4 *>(S.w + off);
        bq[ni][0] = as_bf16x8(unpack8_b8(wv[0], wv[1]));
        bq[ni][1] = as_bf16x8(unpack8_b8(wv[2], wv[3]));
      } else if constexpr (BITS == 3) {
        // tiled only: the 2-bit block of the low bits, then the high-bit word of
        // half h/2 (pairs 8(h%2) .. +7 of this lane, bits P and 16 + P)
        static_assert(TILED, "3-bit codes are staged from the tiled layout");
        const int base = (col / 32) * BB;
        const uint32_t wv = *reinterpret_cast<const uint32_t *>(S.w + base + (h >> 1) * 256 + (col % 32) * 8 + (h & 1) * 4);
        const uint32_t hw = *reinterpret_cast<const uint32_t *>(S.w + base + 512 + (h >> 1) * 128 + (col % 32) * 4);
        const uint32_t hs = (hw >> (8 * (h & 1))) << 2;  // this lane's pair j at bits 2 + j and 18 + j
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          u32x4 r = unpack8_b2_pair(wv, c);
#pragma unroll
          for (int q = 0; q < 4; ++q) r[q] = and_or(hs >> (4 * c + q), 0x00040004u, r[q]);
          bq[ni][c] = as_bf16x8(r);
        }
      } else {
        const int off = TILED ? (col / 32) * BB + (h >> 1) * 256 + (col % 32) * 8 + (h & 1) * 4 : col * WB + h * 4;
        const uint32_t wv = *reinterpret_cast<const uint32_t *>(S.w + off);
        bq[ni][0] = as_bf16x8(TILED ? unpack8_b2_pair(wv, 0) : unpack8_b2(wv, 0));
        bq[ni][1] = as_bf16x8(TILED ? unpack8_b2_pair(wv, 1) : unpack8_b2(wv, 1));
      }
      sbv[ni] = S.sb[col];
    }
    // Software pipeline over the wave's subtile rows. Step t reads the x
    // fragments of row t+1, issues the 8 MFMAs of row t and applies the fp32
    // epilogue of row t-1 (scale) and row t (bias), so the MFMA and VALU pipes
    // work at the same time; each MFMA is paired with four VALU ops.
    bf16x8 a0[2], a1[2];
    f32x4 xs[2];
    f32x4 P[2][NI];
    auto read_a = [&](int mi, int slot) {
      // subtile rows start at multiples of 16: the swizzle term is per lane only
      a0[slot] = *reinterpret_cast<const bf16x8 *>(S.x + xa0 + mi * 2048);
      a1[slot] = *reinterpret_cast<const bf16x8 *>(S.x + xa1 + mi * 2048);
      xs[slot] = *reinterpret_cast<const f32x4 *>(&S.xs[xsa + mi * 16]);
    };
    read_a(0, 0);
#pragma unroll
    for (int t = 0; t <= MI; ++t) {
      const int cur = t & 1, nxt = cur ^ 1;
      if (t + 1 < MI) read_a(t + 1, nxt);
      if (t < MI) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          P[cur][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[cur], bq[ni][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
          P[cur][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[cur], bq[ni][1], P[cur][ni], 0, 0, 0);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][ni][i] = __builtin_fmaf(sbv[ni][1], xs[cur][i], acc[t][ni][i]);
      }
      if (t >= 1) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t - 1][ni][i] = __builtin_fmaf(sbv[ni][0], P[nxt][ni][i], acc[t - 1][ni][i]);
          // keep the update here: sinking it would hold every subtile's P live
          asm volatile("" : "+v"(acc[t - 1][ni]));
        }
      }
      if (t + 1 < MI) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // fragment reads first
      if (t < MI) {
#pragma unroll
        for (int k = 0; k < 2 * NI; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Groups run in pairs (stage 0 then stage 1) with a single loop exit; an odd
  // last group runs after the loop from stage 0.
  if (g_begin < g_end) {
    issue(st0, g_begin);
    finish(st0);
  }
  dma_barrier();
  int g = g_begin;
  for (; g + 1 < g_end; g += 2) {
    issue(st1, g + 1);
    compute(st0);
    finish(st1);
    dma_barrier();
    const bool more2 = g + 2 < g_end;
    if (more2) issue(st0, g + 2);
    compute(st1);
    if (more2) finish(st0);
    dma_barrier();
  }
  if (g < g_end) compute(st0);
  __syncthreads();  // every wave is done with both stages before they are refilled
}

// Stores a finished tile: fp32 or bf16 into out, or fp32 into the split-K
// partial buffer of `split`.
template <int BITS, bool TILED, int BM, int BN, int WARPS_M, int WARPS_N, bool OUT_BF16>
__device__ __forceinline__ void tile_store(const GemmArgs &a, int64_t m0, int64_t n0, int split,
                                           const f32x4 (&acc)[BM / WARPS_M / 16][BN / WARPS_N / 16]) {
  constexpr int WM = BM / WARPS_M, WN = BN / WARPS_N;
  constexpr int MI = WM / 16, NI = WN / 16;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WARPS_N, wn = wave % WARPS_N;
  const int r16 = lane & 15, h = lane >> 4;
  const int64_t row0 = m0 + wm * WM + 4 * h;
  const int64_t col0 = n0 + wn * WN + r16;
  const bool full = (m0 + BM <= a.M) && (n0 + BN <= a.N);
  if (a.splits > 1) {
    float *outp = a.partial + (int64_t)split * a.M * a.N;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = row0 + mi * 16 + i, n = col0 + ni * 16;
          if (full || (m < a.M && n < a.N)) outp[m * a.N + n] = acc[mi][ni][i];
        }
  } else if constexpr (OUT_BF16) {
    uint16_t *outp = reinterpret_cast<uint16_t *>(a.out);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = row0 + mi * 16 + i, n = col0 + ni * 16;
          if (full || (m < a.M && n < a.N)) outp[m * a.N + n] = f32_to_bf16_rne2(acc[mi][ni][i]);
        }
  } else {
    float *outp = reinterpret_cast<float *>(a.out);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = row0 + mi * 16 + i, n = col0 + ni * 16;
          if (full || (m < a.M && n < a.N)) outp[m * a.N + n] = acc[mi][ni][i];
        }
  }
}

// One launch covers `dp_tiles` whole tiles (tile t = blockIdx.x, blockIdx.x +
// gridDim.x, ..., split over K by blockIdx.y when splits > 1) and, when
// sk_tiles > 0, the last sk_tiles tiles cut into sk_pieces K-ranges that run
// first, one per block. A tile that does not fill the machine's last round is
// thereby spread over every block instead of leaving most of them idle. Each
// piece writes its fp32 partial to workspace; the piece that finishes last
// (atomic count) adds all partials in piece order, so the result does not
// depend on timing, stores the tile and re-arms the count.
template <int BITS, bool TILED, int BM, int BN, int WARPS_M, int WARPS_N, bool OUT_BF16>
__global__ __launch_bounds__(64 * WARPS_M * WARPS_N, 2)
void gemm2_kernel(GemmArgs a) {
  using Sh = Gemm2Shape<BITS, TILED, BM, BN, WARPS_M, WARPS_N>;
  constexpr int NT = Sh::NT, MI = Sh::MI, NI = Sh::NI;
  __shared__ __attribute__((aligned(16))) Stage<BITS, BM, BN> st0;
  __shared__ __attribute__((aligned(16))) Stage<BITS, BM, BN> st1;
  __shared__ int s_arrived;

  const int tid = threadIdx.x;
  const int tiles_n = (int)((a.N + BN - 1) / BN);
  f32x4 acc[MI][NI];

  if (a.sk_tiles > 0 && (int)blockIdx.x < a.sk_tiles * a.sk_pieces) {
    // pieces of one tail tile stay on one XCD (block ids dealt round-robin
    // over 8 XCDs) so their partials meet in one L2
    int tail, piece;
    if (a.sk_tiles % 8 == 0 && gridDim.x % 8 == 0) {
      const int x = blockIdx.x % 8, j = blockIdx.x / 8;
      tail = (j / a.sk_pieces) * 8 + x;
      piece = j % a.sk_pieces;
    } else {
      tail = blockIdx.x / a.sk_pieces;
      piece = blockIdx.x % a.sk_pieces;
    }
    const int tile = a.dp_tiles + tail;
    const int64_t m0 = (int64_t)(tile / tiles_n) * BM, n0 = (int64_t)(tile % tiles_n) * BN;
    const int gpp = (a.G + a.sk_pieces - 1) / a.sk_pieces;
    const int gb = piece * gpp, ge = min(a.G, gb + gpp);
    tile_accumulate<BITS, TILED, BM, BN, WARPS_M, WARPS_N>(a, st0, st1, m0, n0, gb, ge, acc);
    // partial in thread-major order: each (mi, ni) fragment is NT*16 contiguous bytes
    float *part = a.sk_partial + (int64_t)tail * a.sk_pieces * (BM * BN);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        *reinterpret_cast<f32x4 *>(part + (int64_t)piece * (BM * BN) + ((mi * NI + ni) * NT + tid) * 4) = acc[mi][ni];
    __threadfence();
    __syncthreads();
    if (tid == 0) s_arrived = atomicAdd(&a.sk_count[tail], 1);
    __syncthreads();
    if (s_arrived == a.sk_pieces - 1) {
      __threadfence();
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          const f32x4 mine = acc[mi][ni];
          f32x4 sum = piece == 0 ? mine : *reinterpret_cast<const f32x4 *>(part + ((mi * NI + ni) * NT + tid) * 4);
          for (int p = 1; p < a.sk_pieces; ++p) {
            const f32x4 v = p == piece ? mine
                                       : *reinterpret_cast<const f32x4 *>(part + (int64_t)p * (BM * BN) +
                                                                         ((mi * NI + ni) * NT + tid) * 4);
            sum += v;
          }
          acc[mi][ni] = sum;
        }
      tile_store<BITS, TILED, BM, BN, WARPS_M, WARPS_N, OUT_BF16>(a, m0, n0, 0, acc);
      if (tid == 0) a.sk_count[tail] = 0;
    }
  }

  const int split = blockIdx.y;
  const int g_begin = split * a.groups_per_split;
  const int g_end = min(a.G, g_begin + a.groups_per_split);
  for (int t = blockIdx.x; t < a.dp_tiles; t += gridDim.x) {
    const int tile = xcd_remap(t, a.dp_tiles);
    const int64_t m0 = (int64_t)(tile / tiles_n) * BM, n0 = (int64_t)(tile % tiles_n) * BN;
    tile_accumulate<BITS, TILED, BM, BN, WARPS_M, WARPS_N>(a, st0, st1, m0, n0, g_begin, g_end, acc);
    tile_store<BITS, TILED, BM, BN, WARPS_M, WARPS_N, OUT_BF16>(a, m0, n0, split, acc);
  }
}

template <int BITS, bool TILED, int BM, int BN, int WMW, int WNW>
hipError_t launch2(const GemmArgs &a, hipStream_t stream) {
  dim3 grid(a.grid_x, a.splits);
  if (a.out_bf16 && a.splits == 1)
    hipLaunchKernelGGL((gemm2_kernel<BITS, TILED, BM, BN, WMW, WNW, true>), grid, dim3(64 * WMW * WNW), 0, stream, a);
  else
    hipLaunchKernelGGL((gemm2_kernel<BITS, TILED, BM, BN, WMW, WNW, false>), grid, dim3(64 * WMW * WNW), 0, stream, a);
  return hipGetLastError();
}

template <int BM, int BN, int WMW, int WNW>
hipError_t launch2_any(int bits, bool tiled, const GemmArgs &a, hipStream_t stream) {
  if (bits == 4) return tiled ? launch2<4, true, BM, BN, WMW, WNW>(a, stream) : launch2<4, false, BM, BN, WMW, WNW>(a, stream);
  if (bits == 8) return tiled ? launch2<8, true, BM, BN, WMW, WNW>(a, stream) : launch2<8, false, BM, BN, WMW, WNW>(a, stream);
  if (bits == 2) return tiled ? launch2<2, true, BM, BN, WMW, WNW>(a, stream) : launch2<2, false, BM, BN, WMW, WNW>(a, stream);
  if (bits == 3) return tiled ? launch2<3, true, BM, BN, WMW, WNW>(a, stream) : hipErrorInvalidValue;
  return hipErrorInvalidValue;
}

}  // namespace

size_t gemm2_lds_bytes(int bits, int id) {
  if (id == 10)
    return 2 * (bits == 4 ? sizeof(Stage<4, 256, 128>) : bits == 8 ? sizeof(Stage<8, 256, 128>)
                : bits == 3 ? sizeof(Stage<3, 256, 128>) : sizeof(Stage<2, 256, 128>));
  if (id == 11)
    return 2 * (bits == 4 ? sizeof(Stage<4, 128, 128>) : bits == 8 ? sizeof(Stage<8, 128, 128>)
                : bits == 3 ? sizeof(Stage<3, 128, 128>) : sizeof(Stage<2, 128, 128>));
  return 0;
}

Gemm2Plan gemm2_plan(int bits, int tile_id, int64_t M, int64_t N, int G, int splits, int slots) {
  const int bm = tile_id == 10 ? 256 : 128, bn = 128;
  Gemm2Plan p{};
  p.tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  p.dp_tiles = (int)p.tiles;
  p.grid_x = (int)p.tiles;
  // This kernel is bound by per-SIMD instruction issue, not by rounds of
  // blocks: a CU with one resident block already runs at full rate, so the
  // tiles past the last full round cost their share of work either way, and
  // splitting them only adds partial traffic and fences (measured slower on
  // MI355X at 4096x4608x4608). The split runs only when a caller-side slot
  // count is given (tests of the split itself).
  if (splits > 1 || G < 2 || p.tiles < 2 || slots <= 0) return p;
  if (p.tiles <= slots || p.tiles % slots == 0) return p;
  const int64_t dp = (p.tiles / slots) * slots;
  const int tail = (int)(p.tiles - dp);
  int pieces = slots / tail;
  if (pieces > G) pieces = G;
  if (pieces < 2) return p;
  const int gpp = (G + pieces - 1) / pieces;
  pieces = (G + gpp - 1) / gpp;  // no empty piece
  p.dp_tiles = (int)dp;
  p.sk_tiles = tail;
  p.sk_pieces = pieces;
  p.grid_x = slots;
  const size_t part = (size_t)tail * pieces * bm * bn * 4u;
  p.sk_partial_bytes = ((part + 255) / 256) * 256 + (((size_t)tail * 4u + 255) / 256) * 256;
  return p;
}

hipError_t launch_gemm2(int bits, int tile_id, bool tiled, const GemmArgs &a, hipStream_t stream) {
  if (tile_id == 10) return launch2_any<256, 128, 2, 2>(bits, tiled, a, stream);
  if (tile_id == 11) return launch2_any<128, 128, 1, 2>(bits, tiled, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ql
