// Large-M dequant-GEMM, fast mode: weights dequantized to fp16 in registers,
// fp16 MFMA with fp32 accumulation.
//
// Numerics. The exact mode (gemm2.hip) keeps the codes as integers in the MFMA
// and applies scale and bias per group on the accumulator; that costs two
// fp32 VALU ops per MFMA and bounds the kernel by vector issue. Here every
// weight is instead dequantized once per block tile and group:
//     W16[n,k] = fp16( s[n,g]*q[n,k] + b[n,g] )        (one rounding, packed
//                                                        fp16 fused multiply-add)
// and x enters as fp16 from a prepass that scales each row by the power of
// two 2^-e bringing its largest magnitude into [2^14, 2^15), so the
// conversion from bf16 is exact for every value within 2^28 of the row's
// largest (scaled magnitude >= 2^-14). The output row is multiplied back by
// 2^e. fp16 keeps 11 significant bits where bf16 keeps 8, so the only
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
//
// Grid. One block per CU runs whole tiles (t, t + gridDim.x, ...). When the
// tile count is a little past a multiple of the CU count, the last tiles are
// cut along M into pieces of 32, 64 or 128 rows (same code, fewer 16-row
// subtiles per wave) that run first, so every CU does the same work and no
// partial sums are needed. When there are fewer tiles than CUs, K is split
// into ranges (blockIdx.y) that write fp32 partials for an ordered reduction.
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kBM = 256, kBN = 256, kNW = 8, kNT = 64 * kNW;
constexpr int kWN = 32, kMI = kBM / 16, kNI = kWN / 16;  // a wave: all rows x 32 columns
constexpr int kXStage = kBM * 128;               // bytes of one x stage
constexpr int kStages = 3;                       // x stages in the LDS ring

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
// i.e. k-blocks 2h and 2h+1, as they sit in the tiled layout. pair(w, c, p)
// gives word p of the B fragment of k-block 2h + c (two fp16 weights).
template <int BITS> struct LaneCodes;
// 4-bit block [h'2][col32][4 words]: words 2(h%2), +1 of half h/2, pair order
// (code 2p at bits 4p, code 2p+1 at 16 + 4p).
template <> struct LaneCodes<4> {
  static constexpr int kWords = 2;
  __device__ static constexpr uint32_t offset(int col, int h) { return (h >> 1) * 512 + col * 16 + (h & 1) * 8; }
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], int c, int p, h2 s2, h2 b2) {
    return dq_pair(and_or(w[c] >> (4 * p), 0x000F000Fu, 0x64006400u), s2, b2);
  }
};
// 8-bit block [part2][h'2][col32][4 words]: part h%2, half h/2, little-endian.
template <> struct LaneCodes<8> {
  static constexpr int kWords = 4;
  __device__ static constexpr uint32_t offset(int col, int h) { return (h & 1) * 1024 + (h >> 1) * 512 + col * 16; }
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], int c, int p, h2 s2, h2 b2) {
    // bytes (b0, b1) or (b2, b3) of word 2c + p/2 into the halves, over 0x6400 (1024)
    return dq_pair(perm(0u, w[2 * c + (p >> 1)], (p & 1) ? 0x0C030C02u : 0x0C010C00u) | 0x64006400u, s2, b2);
  }
};
// 2-bit block [h'2][col32][2 words]: word h%2 of half h/2, pair order (code 2p
// at bits 2p, code 2p+1 at 16 + 2p); chunk c is pairs 4c .. 4c+3.
template <> struct LaneCodes<2> {
  static constexpr int kWords = 1;
  __device__ static constexpr uint32_t offset(int col, int h) { return (h >> 1) * 256 + col * 8 + (h & 1) * 4; }
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], int c, int p, h2 s2, h2 b2) {
    return dq_pair(and_or(w[0] >> (8 * c + 2 * p), 0x00030003u, 0x64006400u), s2, b2);
  }
};

// 3-bit block: the 2-bit block of the low bits (word h%2 of half h/2, as
// above), then the high-bit plane [h'2][col32][1 word] at byte 512 (code 2P
// of the half at bit P, code 2P+1 at bit 16+P). w[0] is the low-bit word,
// w[1] the high-bit word of half h/2 after prep(): the lane's pairs
// 8(h%2) .. +7 moved to bits 2.. and 18.. (prep runs once per group, when
// the codes have arrived).
template <> struct LaneCodes<3> {
  static constexpr int kWords = 2;
  __device__ static constexpr uint32_t offset(int col, int h) { return (h >> 1) * 256 + col * 8 + (h & 1) * 4; }
  __device__ static constexpr uint32_t hi_offset(int col, int h) { return 512 + (h >> 1) * 128 + col * 4; }
  __device__ static uint32_t prep(uint32_t hw, int h) { return (hw >> (8 * (h & 1))) << 2; }
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], int c, int p, h2 s2, h2 b2) {
    const uint32_t lo = and_or(w[0] >> (8 * c + 2 * p), 0x00030003u, 0x64006400u);
    return dq_pair(and_or(w[1] >> (4 * c + p), 0x00040004u, lo), s2, b2);
  }
};

// Canonical layout (each row one little-endian code stream): a lane's 16
// codes 16h .. 16h+15 of its row and group are 16*BITS/8 contiguous bytes at
// row offset g*8*BITS + 2*BITS*h; the codes are in plain order, so a pair is
// gathered with one byte permute (4-bit, 2-bit) before the AND-OR. 8-bit
// bytes are already in the order LaneCodes<8> reads.
template <int BITS> struct CanonCodes;
template <> struct CanonCodes<4> {
  static constexpr int kWords = 2;
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], int c, int p, h2 s2, h2 b2) {
    // nibbles 2p, 2p+1 of word c: byte p of w and of w >> 4, low nibbles
    const uint32_t sel = 0x0C040C00u + 0x00010001u * (uint32_t)p;
    return dq_pair(and_or(perm(w[c] >> 4, w[c], sel), 0x000F000Fu, 0x64006400u), s2, b2);
  }
};
template <> struct CanonCodes<8> {
  static constexpr int kWords = 4;
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], int c, int p, h2 s2, h2 b2) {
    return LaneCodes<8>::pair(w, c, p, s2, b2);
  }
};
template <> struct CanonCodes<2> {
  static constexpr int kWords = 1;
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], int c, int p, h2 s2, h2 b2) {
    // codes 8c+2p, 8c+2p+1 at bits 16c+4p and 16c+4p+2
    const uint32_t t = w[0] >> (16 * c + 4 * p);
    return dq_pair(and_or(perm(t >> 2, t, 0x0C040C00u), 0x00030003u, 0x64006400u), s2, b2);
  }
};
template <int BITS, bool CANON> struct CodesOf { using type = LaneCodes<BITS>; };
template <int BITS> struct CodesOf<BITS, true> { using type = CanonCodes<BITS>; };

// Chunk swizzle of an x stage: logical 16-byte chunk c of row r sits at
// position c ^ xswz(r). With this function the 64 lanes of an MFMA fragment
// read (16 rows, four k-blocks) spread over the banks best among the
// XOR swizzles measured on MI355X (194 B/clk/CU against 140 for c ^ (r & 7)).
__device__ __forceinline__ int xswz(int r) { return (r ^ (r >> 3)) & 7; }

// Accumulates rows m0 .. m0 + 16*MI of the block tile at (m0, n0) over groups
// [g_begin, g_end): MI = 16 for a whole tile, fewer for a row piece.
template <int BITS, int MI, bool CANON>
__device__ __forceinline__ void tile_accumulate3(const Gemm3Args &a, unsigned char *const (&xs)[kStages], int64_t m0,
                                                 int64_t n0, int g_begin, int g_end, f32x4 (&acc)[MI][kNI]) {
  constexpr int S = kStages;
  using LC = typename CodesOf<BITS, CANON>::type;
  constexpr int WB = 64 * BITS / 8;     // code bytes of one column per group
  constexpr int BB = 32 * WB;           // bytes of one tiled block (32 columns x 1 group)
  constexpr int kRows = 16 * MI;
  constexpr int XC = kRows / 8;         // 1 KB x copies per group (8 rows each)
  constexpr int XPW = XC >= kNW ? XC / kNW : 1;  // copies per issuing wave
  static_assert(XC % kNW == 0 || kNW % XC == 0, "x copies must spread evenly over the waves");
  constexpr int kSteps = 2 * MI;        // steps (c, mi) of kNI MFMAs per group
  constexpr int kHalf = kSteps / 2;
  // A fragments are read this many steps ahead of their use; the ring index
  // t % (kAhead + 1) continues across groups, whose reads ahead wrap into
  // the next stage, which is complete only after the mid-group barrier
  constexpr int kAhead = (kSteps % 4 == 0 && kHalf >= 3) ? 3 : 1;
  static_assert(kSteps % (kAhead + 1) == 0, "A-fragment ring must divide the steps of a group");
  static_assert(kAhead <= kHalf, "reads of the next stage must follow the mid-group barrier");
  // the next group's B fragments are built in 4 * 2 * kNI pieces of one word
  // (two weights), spread over the steps of the second half so the vector
  // work sits between MFMAs instead of in bursts
  constexpr int kPieces = 8 * kNI;
  constexpr int kPerStep = (kPieces + kHalf - 1) / kHalf;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, h = lane >> 4;
  const int G = a.G;

  // x copies: copy i of this wave fills block rows (wave*XPW + i)*8 .. +7, lane L
  // row +L/8 at chunk position L & 7, which holds logical chunk
  // (L & 7) ^ xswz(row). Rows past M repeat the last row. With fewer copies
  // than waves only the first XC waves copy.
  const int64_t xrow = a.K * 2;
  const int64_t mrows = min<int64_t>(kRows, a.M - m0);
  const bool x_issuer = XC >= kNW || wave < XC;
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
  __amdgpu_buffer_rsrc_t wr, sr, br;
  uint32_t wo = 0, so = 0, who = 0;  // who: 3-bit, the lane's high-bit word
  uint32_t kColStep = 0;             // tiled: bytes per 16 columns
  uint32_t rowo[kNI] = {}, srow[kNI] = {};  // canonical: the lane's row of each column block
  if constexpr (CANON) {
    // one descriptor over all rows (uniform), the row in the lane offset;
    // rows past N repeat row N-1
    wr = make_rsrc(a.w, 0, a.N * (a.K * BITS / 8));
    sr = make_rsrc(a.s16, 0, a.N * (int64_t)G * 2);
    br = make_rsrc(a.b16, 0, a.N * (int64_t)G * 2);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const int64_t n = min<int64_t>(strip * 32 + ni * 16 + r16, a.N - 1);
      rowo[ni] = (uint32_t)(n * (a.K * BITS / 8)) + (uint32_t)(h * 2 * BITS);
      srow[ni] = (uint32_t)(n * G * 2);
    }
  } else {
    wr = make_rsrc(a.w, strip * G * BB, (int64_t)G * BB);
    sr = make_rsrc(a.sb, strip * G * 128, (int64_t)G * 128);
    br = sr;
    wo = LaneCodes<BITS>::offset(r16, h);
    so = (uint32_t)(r16 * 4);
    if constexpr (BITS == 3) who = LaneCodes<BITS>::hi_offset(r16, h);
    kColStep = LaneCodes<BITS>::offset(16, 0) - LaneCodes<BITS>::offset(0, 0);
  }

  auto load_codes = [&](uint32_t (&w)[kNI][LC::kWords], uint32_t (&sb)[kNI], uint32_t (&bb)[kNI], int gv) {
    const int g = __builtin_amdgcn_readfirstlane(gv);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      if constexpr (CANON) {
        const uint32_t go = (uint32_t)g * (8u * BITS);
        if constexpr (BITS == 4) {
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, rowo[ni], go, 0);
          w[ni][0] = v[0];
          w[ni][1] = v[1];
        } else if constexpr (BITS == 8) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, rowo[ni], go, 0);
#pragma unroll
          for (int t = 0; t < 4; ++t) w[ni][t] = v[t];
        } else {
          w[ni][0] = __builtin_amdgcn_raw_buffer_load_b32(wr, rowo[ni], go, 0);
        }
        sb[ni] = __builtin_amdgcn_raw_buffer_load_b16(sr, srow[ni], (uint32_t)g * 2u, 0);
        bb[ni] = __builtin_amdgcn_raw_buffer_load_b16(br, srow[ni], (uint32_t)g * 2u, 0);
        continue;
      }
      if constexpr (BITS == 4) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, wo + ni * kColStep, (uint32_t)g * BB, 0);
        w[ni][0] = v[0];
        w[ni][1] = v[1];
      } else if constexpr (BITS == 8) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, wo + ni * kColStep, (uint32_t)g * BB, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t) w[ni][t] = v[t];
      } else if constexpr (BITS == 3) {
        w[ni][0] = __builtin_amdgcn_raw_buffer_load_b32(wr, wo + ni * kColStep, (uint32_t)g * BB, 0);
        w[ni][1] = __builtin_amdgcn_raw_buffer_load_b32(wr, who + ni * 64u, (uint32_t)g * BB, 0);
      } else {
        w[ni][0] = __builtin_amdgcn_raw_buffer_load_b32(wr, wo + ni * kColStep, (uint32_t)g * BB, 0);
      }
      sb[ni] = __builtin_amdgcn_raw_buffer_load_b32(sr, so + ni * 64u, (uint32_t)g * 128u, 0);
      bb[ni] = 0u;
    }
  };
  auto issue_x = [&](unsigned char *X, int gv) {
    const int g = __builtin_amdgcn_readfirstlane(gv);
    if (x_issuer) {
#pragma unroll
      for (int i = 0; i < XPW; ++i) dma16(xr, xo[i], (uint32_t)g * 128u, X + (wave * XPW + i) * 1024);
    }
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
    const int c = t / MI, mi = t % MI;
    af[t % (kAhead + 1)] = *reinterpret_cast<const h8 *>(X + a_base + mi * 2048 + a_off[c][mi & 3]);
  };

  // B fragments of the group being multiplied, built from codes that arrived
  // earlier; a group past the end gets zero scale and bias, so its weights
  // are zero and its step adds nothing. Codes and scale|bias words of groups
  // g+1 .. g+S-2 are held (cq[0] = g+1); those of g+S-1 are requested in
  // group g.
  u32x4 bf[kNI][2];
  uint32_t cq[S - 1][kNI][LC::kWords];
  uint32_t sq[S - 1][kNI];   // tiled: s | b << 16; canonical: s
  uint32_t bq[S - 1][kNI];   // canonical: b (unused when tiled)
  // piece i of the B fragments from cq[0]/sq[0]: fragment (ni, c) = i / 4, word i % 4
  auto dequant_piece = [&](u32x4 (&dst)[kNI][2], bool valid, int i) {
    const int f = i >> 2, p = i & 3, ni = f >> 1, c = f & 1;
    const uint32_t v = valid ? (CANON ? (sq[0][ni] & 0xFFFFu) | (bq[0][ni] << 16) : sq[0][ni]) : 0u;
    const h2 s2 = __builtin_bit_cast(h2, (v & 0xFFFFu) * 0x10001u);
    const h2 b2 = __builtin_bit_cast(h2, (v >> 16) * 0x10001u);
    if constexpr (BITS == 3 && !CANON) {
      // the first piece of a column block (i = 8 ni) runs before its other
      // pieces: in both placements below pieces run in increasing i within a
      // column block
      if (c == 0 && p == 0) cq[0][ni][1] = LC::prep(cq[0][ni][1], h);
    }
    uint32_t r = LC::pair(cq[0][ni], c, p, s2, b2);
    asm volatile("" : "+v"(r));  // keeps the piece where it is placed, between MFMAs
    dst[ni][c][p] = r;
  };

  // One group on stage X. First half: MFMAs on the fragments in hand. Then
  // the barrier, after which the next stage XN is complete and the stage of
  // the previous group (XD) is free: the x copies for S-1 groups ahead go
  // into XD and their codes are requested. Second half: MFMAs, with the next
  // group's B fragments dequantized in between and the first A fragments of
  // XN read ahead, so the next group starts without a stall.
  auto step = [&](const unsigned char *X, const unsigned char *XN, unsigned char *XD, int g) {
    u32x4 bn[kNI][2];
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const int c = t / MI, mi = t % MI;
      if (t == kHalf) {
        dma_barrier();  // stage g+1 has landed everywhere, stage g-1 is free
        // the second half runs at raised wave priority (back to normal at the
        // end of the group): 1-1.5 % faster on the large shapes, measured
        __builtin_amdgcn_s_setprio(1);
        issue_x(XD, min(g + S - 1, g_end - 1));
        load_codes(cq[S - 2], sq[S - 2], bq[S - 2], min(g + S - 1, g_end - 1));
      }
      if (t + kAhead < kSteps) read_a(X, t + kAhead);
      else read_a(XN, t + kAhead - kSteps);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[t % (kAhead + 1)], __builtin_bit_cast(h8, bf[ni][c]),
                                                             acc[mi][ni], 0, 0, 0);
        if (t >= kHalf) {
#pragma unroll
          for (int u = 0; u < kPerStep; ++u) {
            const int i = (t - kHalf) * kPerStep + u;
            if ((u % kNI) == ni && i < kPieces) dequant_piece(bn, g + 1 < g_end, i);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      bf[ni][0] = bn[ni][0];
      bf[ni][1] = bn[ni][1];
#pragma unroll
      for (int j = 0; j + 1 < S - 1; ++j) {
        sq[j][ni] = sq[j + 1][ni];
        bq[j][ni] = bq[j + 1][ni];
#pragma unroll
        for (int u = 0; u < LC::kWords; ++u) cq[j][ni][u] = cq[j + 1][ni][u];
      }
    }
  };

#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < kNI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Groups run S at a time (one per x stage) in straight-line code: loads
  // for a group past the end are clamped to the last group and its weights
  // dequantize to zero, so the accumulators never pass through a branch.
  if (g_begin < g_end) {
    load_codes(cq[0], sq[0], bq[0], g_begin);
    issue_x(xs[0], g_begin);
    issue_x(xs[1], min(g_begin + 1, g_end - 1));
  }
  dma_barrier();  // first two stages and the first codes have arrived
  if (g_begin < g_end) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) dequant_piece(bf, true, i);
    load_codes(cq[0], sq[0], bq[0], min(g_begin + 1, g_end - 1));
    // stages and codes up to g_begin + S - 2 are in flight now; each group g
    // requests g + S - 1
#pragma unroll
    for (int j = 2; j < S - 1; ++j) {
      issue_x(xs[j], min(g_begin + j, g_end - 1));
      load_codes(cq[j - 1], sq[j - 1], bq[j - 1], min(g_begin + j, g_end - 1));
    }
#pragma unroll
    for (int t = 0; t < kAhead; ++t) read_a(xs[0], t);
  }
  for (int g = g_begin; g < g_end; g += S) {
#pragma unroll
    for (int k = 0; k < S; ++k) step(xs[k], xs[(k + 1) % S], xs[(k + S - 1) % S], g + k);
  }
  dma_barrier();  // the copies requested past the last group have landed; every stage is free
}

// silu(g) * u: g / (1 + e^-g) with the hardware exponential and reciprocal;
// e^-g overflows to +inf for g < -88 and the quotient is then -0.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Stores rows m0 .. m0 + 16*MI of a tile, times the row scales, into out
// ([M, N] fp32 or bf16). The row scales come from LDS (rs_lds[m - m0], staged
// by the caller): a global load among the stores would wait for every store
// before it, since one counter tracks both, which cost ~6 % of the kernel. With GLU-ordered weights subtile ni = 0 of a wave
// holds gate outputs and ni = 1 the up outputs of the same 16 columns
// f = 16*strip + r16 of the [M, N/2] result, which gets silu(gate) * up.
template <bool OUT_BF16, int MI>
__device__ __forceinline__ void tile_store3(const Gemm3Args &a, void *out, int64_t m0, int64_t n0,
                                            const f32x4 (&acc)[MI][kNI], const float *rs_lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, h = lane >> 4;
  const int64_t row0 = m0 + 4 * h;
  if (a.glu) {
    const int64_t F = a.N / 2;
    const int64_t f = (n0 / 32 + wave) * 16 + r16;
    if (f >= F) return;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = row0 + mi * 16 + i;
        if (m >= a.M) continue;
        const float rs = rs_lds[m - m0];
        const float v = swiglu(acc[mi][0][i] * rs, acc[mi][1][i] * rs);
        if constexpr (OUT_BF16) reinterpret_cast<uint16_t *>(out)[m * F + f] = f32_to_bf16_rne3(v);
        else reinterpret_cast<float *>(out)[m * F + f] = v;
      }
    return;
  }
  const int64_t col0 = n0 + wave * kWN + r16;
  const bool full = (m0 + 16 * MI <= a.M) && (n0 + kBN <= a.N);
  if (a.gate) {
    // gated residual update: out = residual + gate[m / gate_rows] * y, one
    // fused multiply-add in fp32; each element is read and written by the
    // same lane, so residual may be out itself. Residual and gate values are
    // read for two subtile rows at a time before their stores, so a load
    // waits behind earlier stores once per pair of subtile rows
    constexpr int CH = MI < 2 ? MI : 2;
#pragma unroll
    for (int mc = 0; mc < MI; mc += CH) {
      float rv[CH][4][kNI], gv[CH][4][kNI];
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = row0 + (mc + c) * 16 + i;
          const float *grow = a.gate + (int64_t)((uint32_t)m / (uint32_t)a.gate_rows) * a.N;
#pragma unroll
          for (int ni = 0; ni < kNI; ++ni) {
            const int64_t n = col0 + ni * 16;
            const bool ok = full || (m < a.M && n < a.N);
            if constexpr (OUT_BF16)
              rv[c][i][ni] = ok ? bf16_lo(reinterpret_cast<const uint16_t *>(a.residual)[m * a.N + n]) : 0.f;
            else
              rv[c][i][ni] = ok ? reinterpret_cast<const float *>(a.residual)[m * a.N + n] : 0.f;
            gv[c][i][ni] = ok ? grow[n] : 0.f;
          }
        }
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = row0 + (mc + c) * 16 + i;
          if (!full && m >= a.M) continue;
          const float rs = rs_lds[m - m0];
#pragma unroll
          for (int ni = 0; ni < kNI; ++ni) {
            const int64_t n = col0 + ni * 16;
            if (!full && n >= a.N) continue;
            const float y = __builtin_fmaf(gv[c][i][ni], acc[mc + c][ni][i] * rs, rv[c][i][ni]);
            if constexpr (OUT_BF16) reinterpret_cast<uint16_t *>(out)[m * a.N + n] = f32_to_bf16_rne3(y);
            else reinterpret_cast<float *>(out)[m * a.N + n] = y;
          }
        }
    }
    return;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = row0 + mi * 16 + i;
      if (!full && m >= a.M) continue;
      const float rs = rs_lds[m - m0];
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        const int64_t n = col0 + ni * 16;
        if (!full && n >= a.N) continue;
        const float v = acc[mi][ni][i] * rs;
        if constexpr (OUT_BF16) reinterpret_cast<uint16_t *>(out)[m * a.N + n] = f32_to_bf16_rne3(v);
        else reinterpret_cast<float *>(out)[m * a.N + n] = v;
      }
    }
}

// blockIdx.y = K range (a.splits of them; each writes its own fp32 slice of
// out, [splits, M, N], for an ordered reduction afterwards). Blocks
// [0, tail_tiles * 16/PMI) first run the row pieces of the last tail_tiles
// tiles (PMI 16-row subtiles each, pieces of one tile on one XCD), then every
// block takes whole tiles t = blockIdx.x, + gridDim.x, ... below dp_tiles.
// Power-of-two row scales commute exactly with the summation, so partials
// carry them already.
template <int BITS, bool OUT_BF16, int PMI, bool CANON>
__global__ __launch_bounds__(kNT, 1) void gemm3_kernel(Gemm3Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char x0[kXStage];
  __shared__ __attribute__((aligned(16))) unsigned char x1[kXStage];
  __shared__ __attribute__((aligned(16))) unsigned char x2[kXStage];
  __shared__ __attribute__((aligned(16))) float rs_lds[kBM];
  unsigned char *const xs[kStages] = {x0, x1, x2};
  // the row scales of a tile's rows: requested at the tile's start (one value
  // per thread), written to LDS once the K loop has ended (its last barrier
  // also ends every wave's reads of the previous tile's scales)
  auto tile_rs = [&](int64_t m0, int rows) -> float {
    const int64_t m = m0 + threadIdx.x;
    return (int)threadIdx.x < rows && m < a.M ? a.rowscale[m] : 0.f;
  };
  auto stage_rs = [&](float v, int rows) {
    if ((int)threadIdx.x < rows) rs_lds[threadIdx.x] = v;
    __syncthreads();
  };
  const int tiles_n = (int)((a.N + kBN - 1) / kBN);
  const int split = blockIdx.y;
  const int gps = (a.G + a.splits - 1) / a.splits;
  const int gb = split * gps, ge = min(a.G, gb + gps);
  void *out = a.splits > 1 ? static_cast<void *>(static_cast<float *>(a.out) + (int64_t)split * a.M * a.N) : a.out;

  if constexpr (PMI > 0) {
    constexpr int kPieces = 16 / PMI;
    if ((int)blockIdx.x < a.tail_tiles * kPieces) {
      const int tail = blockIdx.x % a.tail_tiles, piece = blockIdx.x / a.tail_tiles;
      const int tile = a.dp_tiles + tail;
      const int64_t m0 = (int64_t)(tile / tiles_n) * kBM + piece * 16 * PMI;
      const int64_t n0 = (int64_t)(tile % tiles_n) * kBN;
      if (m0 < a.M) {  // uniform per block
        f32x4 pacc[PMI][kNI];
        const float rs = tile_rs(m0, 16 * PMI);
        tile_accumulate3<BITS, PMI, CANON>(a, xs, m0, n0, gb, ge, pacc);
        stage_rs(rs, 16 * PMI);
        tile_store3<OUT_BF16, PMI>(a, out, m0, n0, pacc, rs_lds);
      }
    }
  }
  f32x4 acc[kMI][kNI];
  for (int t = blockIdx.x; t < a.dp_tiles; t += gridDim.x) {
    const int tile = xcd_remap(t, a.dp_tiles);
    const int64_t m0 = (int64_t)(tile / tiles_n) * kBM, n0 = (int64_t)(tile % tiles_n) * kBN;
    const float rs = tile_rs(m0, kBM);
    tile_accumulate3<BITS, kMI, CANON>(a, xs, m0, n0, gb, ge, acc);
    stage_rs(rs, kBM);
    tile_store3<OUT_BF16, kMI>(a, out, m0, n0, acc, rs_lds);
  }
}

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

template <int BITS, bool OUT_BF16, bool CANON>
void launch3_out(const Gemm3Args &a, hipStream_t stream) {
  const dim3 grid((unsigned)a.grid_x, (unsigned)a.splits);
  switch (a.tail_tiles > 0 ? a.tail_mi : 0) {
    case 2: hipLaunchKernelGGL((gemm3_kernel<BITS, OUT_BF16, 2, CANON>), grid, dim3(kNT), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((gemm3_kernel<BITS, OUT_BF16, 4, CANON>), grid, dim3(kNT), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((gemm3_kernel<BITS, OUT_BF16, 8, CANON>), grid, dim3(kNT), 0, stream, a); break;
    default: hipLaunchKernelGGL((gemm3_kernel<BITS, OUT_BF16, 0, CANON>), grid, dim3(kNT), 0, stream, a); break;
  }
}

template <int BITS, bool CANON>
void launch3_layout(const Gemm3Args &a, hipStream_t stream) {
  if (a.out_bf16 && a.splits == 1) launch3_out<BITS, true, CANON>(a, stream);
  else launch3_out<BITS, false, CANON>(a, stream);
}

template <int BITS>
hipError_t launch3_bits(const Gemm3Args &a, hipStream_t stream) {
  if (a.tail_tiles > 0 && a.tail_mi != 2 && a.tail_mi != 4 && a.tail_mi != 8) return hipErrorInvalidValue;
  if (a.splits < 1 || (a.splits > 1 && a.tail_tiles > 0)) return hipErrorInvalidValue;
  if constexpr (BITS == 3) {
    if (a.canon) return hipErrorInvalidValue;  // 3-bit codes run on tiled weights only
    launch3_layout<BITS, false>(a, stream);
  } else {
    if (a.canon) launch3_layout<BITS, true>(a, stream);
    else launch3_layout<BITS, false>(a, stream);
  }
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

Gemm3Plan gemm3_plan(int64_t M, int64_t N, int G, int slots, int force_splits) {
  Gemm3Plan p{};
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
  if (bits == 4) return launch3_bits<4>(a, stream);
  if (bits == 8) return launch3_bits<8>(a, stream);
  if (bits == 2) return launch3_bits<2>(a, stream);
  if (bits == 3) return launch3_bits<3>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ql
