// Large-M dequant-GEMM on 256 x 256 block tiles, shared by two numerics:
//
// FAST (gemm3.hip): every weight is dequantized once per block tile and group
// to fp16 with one rounding,
//     W16[n,k] = fp16( (s[n,g]*q[n,k] + b[n,g]) * 2^-c[n] )  (one rounding, packed
//                                                           fp16 fused multiply-add)
// and x enters as fp16 from a prepass that scales each row by the power of
// two 2^-e bringing its largest magnitude into [2^14, 2^15), so the
// conversion from bf16 is exact for every value within 2^28 of the row's
// largest (scaled magnitude >= 2^-14). Outputs are multiplied back by 2^e
// (row) and 2^c (column). c[n] is 0 unless the column's weights could reach
// the fp16 limit: each tile first scans its columns' scale and bias words
// for the bound max(|b|, |b + (2^bits-1)*s|) over its K range and, where
// that bound is >= 65504, takes c = floor(log2 bound) - 14, so every
// weight of any finite f16 scale and bias stays finite in fp16. fp16 keeps
// 11 significant bits where bf16 keeps 8, so the only rounding beyond fp32
// accumulation is the half-ulp (2^-11 relative) of W16: relative Frobenius
// error ~2e-4 on the pages' shapes, against 1.7e-3 for weights rounded to
// bf16.
//
// SPLIT (gemm4.hip): bf16 x straight from the caller (no prepass). Each
// weight is dequantized in fp32 exactly as the affine format defines it,
// W = s*q + b (one rounding: s*q is exact), and split into two bf16 terms
// hi = bf16(W), lo = bf16(W - hi) (both round to nearest even; W - hi is
// exact), so |W - hi - lo| <= 2^-16 |W|. Both terms go through the bf16
// MFMA against the same x fragment, accumulating in fp32: twice the matrix
// work of FAST, no activation prepass, no scratch memory and no range
// condition on x or W (bf16 has the fp32 exponent range). Relative
// Frobenius error ~1e-5.
//
// Kernel. Block tile 256 x 256 with eight waves side by side, each owning all
// 256 rows and one 32-column strip (16 x 2 subtiles of 16 x 16 x 32 MFMAs,
// 128 fp32 accumulators). A wave's strip is exactly one block of the tiled
// weight layout, so each lane loads its own codes (8 bytes per column-half for
// 4-bit) and dequantizes them straight into B fragments: every weight is
// dequantized once per tile and weights never pass through LDS. x (fp16 or
// bf16) moves by LDS DMA into a ring of three 32 KB stages (rows of 128
// bytes, 16-byte chunks XOR-swizzled by row, see xswz), issued 1.5 groups
// ahead of its use; one barrier per group, in the middle of the group's
// MFMAs, so the waves of a SIMD never idle at a group edge.
//
// Grid. One block per CU runs whole tiles (t, t + gridDim.x, ...). When the
// tile count is a little past a multiple of the CU count, the last tiles are
// cut along M into pieces of 32, 64 or 128 rows (same code, fewer 16-row
// subtiles per wave), one per block, run before the block's whole tiles on
// even blocks and after them on odd ones, so every CU does the same work, no
// partial sums are needed and the CUs do not all store their tiles at once. When there are fewer tiles than CUs, K may be
// split into ranges (blockIdx.y) that write fp32 partials for an ordered
// reduction.
#pragma once

#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace g3 {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf2;
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 256, kBN = 256, kNW = 8, kNT = 64 * kNW;
constexpr int kWN = 32, kMI = kBM / 16, kNI = kWN / 16;  // a wave: all rows x 32 columns
constexpr int kXStage = kBM * 128;               // bytes of one x stage
constexpr int kStages = 3;                       // x stages in the LDS ring
// canonical scale/bias staging in LDS: chunks of 8 groups of the tile's 256
// columns, [buffer][s, b][column][group], one f16 per dword (a 2-byte copy to
// LDS writes its value zero-extended to 4 bytes); loads run 2 chunks ahead
constexpr int kSbChunk = 8, kSbBufs = 3;
constexpr int kSbBufWords = 2 * kBN * kSbChunk;  // dwords per buffer

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

// Two codes (byte 0 and byte 2 of qp) -> hi and lo bf16 pairs of the fp32
// weights s*q + b (SPLIT numerics).
__device__ __forceinline__ void split_pair(uint32_t qp, float s, float b, uint32_t &hi, uint32_t &lo) {
  const float w0 = __builtin_fmaf((float)(qp & 0xFFu), s, b);
  const float w1 = __builtin_fmaf((float)((qp >> 16) & 0xFFu), s, b);
  const bf2 h = {(__bf16)w0, (__bf16)w1};  // v_cvt_pk_bf16_f32, round to nearest even
  const uint32_t hb = __builtin_bit_cast(uint32_t, h);
  const float r0 = w0 - __uint_as_float(hb << 16);           // exact
  const float r1 = w1 - __uint_as_float(hb & 0xFFFF0000u);   // exact
  const bf2 l = {(__bf16)r0, (__bf16)r1};
  hi = hb;
  lo = __builtin_bit_cast(uint32_t, l);
}

// A lane's codes of one column and group: codes 16h .. 16h+15 (h = lane / 16),
// i.e. k-blocks 2h and 2h+1, as they sit in the tiled layout. pair(w, c, p)
// gives word p of the FAST B fragment of k-block 2h + c (two fp16 weights);
// qpair(w, c, p) gives the same two codes in bytes 0 and 2.
template <int BITS> struct LaneCodes;
// 4-bit block [h'2][col32][4 words]: words 2(h%2), +1 of half h/2, pair order
// (code 2p at bits 4p, code 2p+1 at 16 + 4p).
template <> struct LaneCodes<4> {
  static constexpr int kWords = 2;
  __device__ static constexpr uint32_t offset(int col, int h) { return (h >> 1) * 512 + col * 16 + (h & 1) * 8; }
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], int c, int p, h2 s2, h2 b2) {
    return dq_pair(and_or(w[c] >> (4 * p), 0x000F000Fu, 0x64006400u), s2, b2);
  }
  __device__ static uint32_t qpair(const uint32_t (&w)[kWords], int c, int p) { return (w[c] >> (4 * p)) & 0x000F000Fu; }
};
// 8-bit block [part2][h'2][col32][4 words]: part h%2, half h/2, little-endian.
template <> struct LaneCodes<8> {
  static constexpr int kWords = 4;
  __device__ static constexpr uint32_t offset(int col, int h) { return (h & 1) * 1024 + (h >> 1) * 512 + col * 16; }
  __device__ static uint32_t qpair(const uint32_t (&w)[kWords], int c, int p) {
    // bytes (b0, b1) or (b2, b3) of word 2c + p/2 into bytes 0 and 2
    return perm(0u, w[2 * c + (p >> 1)], (p & 1) ? 0x0C030C02u : 0x0C010C00u);
  }
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], int c, int p, h2 s2, h2 b2) {
    return dq_pair(qpair(w, c, p) | 0x64006400u, s2, b2);
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
  __device__ static uint32_t qpair(const uint32_t (&w)[kWords], int c, int p) {
    return (w[0] >> (8 * c + 2 * p)) & 0x00030003u;
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
  __device__ static uint32_t qpair(const uint32_t (&w)[kWords], int c, int p) {
    return ((w[0] >> (8 * c + 2 * p)) & 0x00030003u) | ((w[1] >> (4 * c + p)) & 0x00040004u);
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
  __device__ static uint32_t qpair(const uint32_t (&w)[kWords], int c, int p) {
    const uint32_t sel = 0x0C040C00u + 0x00010001u * (uint32_t)p;
    return perm(w[c] >> 4, w[c], sel) & 0x000F000Fu;
  }
};
template <> struct CanonCodes<8> {
  static constexpr int kWords = 4;
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], int c, int p, h2 s2, h2 b2) {
    return LaneCodes<8>::pair(w, c, p, s2, b2);
  }
  __device__ static uint32_t qpair(const uint32_t (&w)[kWords], int c, int p) { return LaneCodes<8>::qpair(w, c, p); }
};
template <> struct CanonCodes<2> {
  static constexpr int kWords = 1;
  __device__ static uint32_t pair(const uint32_t (&w)[kWords], int c, int p, h2 s2, h2 b2) {
    // codes 8c+2p, 8c+2p+1 at bits 16c+4p and 16c+4p+2
    const uint32_t t = w[0] >> (16 * c + 4 * p);
    return dq_pair(and_or(perm(t >> 2, t, 0x0C040C00u), 0x00030003u, 0x64006400u), s2, b2);
  }
  __device__ static uint32_t qpair(const uint32_t (&w)[kWords], int c, int p) {
    const uint32_t t = w[0] >> (16 * c + 4 * p);
    return perm(t >> 2, t, 0x0C040C00u) & 0x00030003u;
  }
};
template <int BITS, bool CANON> struct CodesOf { using type = LaneCodes<BITS>; };
template <int BITS> struct CodesOf<BITS, true> { using type = CanonCodes<BITS>; };

// Chunk swizzle of an x stage: logical 16-byte chunk c of row r sits at
// position c ^ xswz(r). With this function the 64 lanes of an MFMA fragment
// read (16 rows, four k-blocks) spread over the banks best among the
// XOR swizzles measured on MI355X (194 B/clk/CU against 140 for c ^ (r & 7)).
__device__ __forceinline__ int xswz(int r) { return (r ^ (r >> 3)) & 7; }

// The part of a tile's K loop both numerics share: x copies into the stage
// ring, the lane's code and scale/bias loads, A-fragment reads. MI 16-row
// subtiles per wave (16 for a whole tile, fewer for a row piece).
template <int BITS, int MI, bool CANON>
struct TileIO {
  using LC = typename CodesOf<BITS, CANON>::type;
  static constexpr int WB = 64 * BITS / 8;     // code bytes of one column per group
  static constexpr int BB = 32 * WB;           // bytes of one tiled block (32 columns x 1 group)
  static constexpr int kRows = 16 * MI;
  static constexpr int XC = kRows / 8;         // 1 KB x copies per group (8 rows each)
  static constexpr int XPW = XC >= kNW ? XC / kNW : 1;  // copies per issuing wave
  static_assert(XC % kNW == 0 || kNW % XC == 0, "x copies must spread evenly over the waves");

  const Gemm3Args &a;
  int lane, wave, r16, h, G;
  bool x_issuer;
  // canonical scale/bias staging (see stage_issue)
  uint32_t *sbl = nullptr;
  int g_first = 0;        // first group of the tile's K range
  uint32_t st_voff = 0;   // the lane's staging offset: its row and its group within a chunk
  __amdgpu_buffer_rsrc_t xr, wr, sr, br;
  uint32_t xo[XPW];
  uint32_t wo = 0, so = 0, who = 0;  // who: 3-bit, the lane's high-bit word
  uint32_t kColStep = 0;             // tiled: bytes per 16 columns
  uint32_t rowo[kNI] = {}, srow[kNI] = {};  // canonical: the lane's row of each column block
  int a_off[2][4];
  int a_base;

  __device__ TileIO(const Gemm3Args &args, int64_t m0, int64_t n0, uint32_t *sb_lds = nullptr, int g_begin = 0)
      : a(args) {
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    r16 = lane & 15;
    h = lane >> 4;
    G = a.G;
    // x copies: copy i of this wave fills block rows (wave*XPW + i)*8 .. +7, lane L
    // row +L/8 at chunk position L & 7, which holds logical chunk
    // (L & 7) ^ xswz(row). Rows past M repeat the last row. With fewer copies
    // than waves only the first XC waves copy.
    const int64_t xrow = a.K * 2;
    const int64_t mrows = min<int64_t>(kRows, a.M - m0);
    x_issuer = XC >= kNW || wave < XC;
    xr = make_rsrc(a.x16, m0 * xrow, mrows * xrow);
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
      sbl = sb_lds;
      g_first = g_begin;
      st_voff = (uint32_t)(((n0 + (wave & 3) * 64 + (lane >> 3)) * G + (lane & 7)) * 2);
    } else {
      wr = make_rsrc(a.w, strip * G * BB, (int64_t)G * BB);
      sr = make_rsrc(a.sb, strip * G * 128, (int64_t)G * 128);
      br = sr;
      wo = LC::offset(r16, h);
      so = (uint32_t)(r16 * 4);
      if constexpr (BITS == 3) who = LaneCodes<BITS>::hi_offset(r16, h);
      kColStep = LC::offset(16, 0) - LC::offset(0, 0);
    }
    // A fragments: rows mi*16 + r16, k-block 2h + c, at chunk position
    // (2h + c) ^ xswz(mi*16 + r16) = (2h + c) ^ ((r16 ^ (r16 >> 3) ^ 2mi) & 7):
    // four lane offsets per chunk, by mi & 3
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) a_off[c][q] = ((2 * h + c) ^ ((r16 ^ (r16 >> 3) ^ (2 * q)) & 7)) * 16;
    a_base = r16 * 128;
  }

  // Codes and scale/bias of group gv for this lane's two column blocks.
  // Tiled: sb = s | b << 16, bb unused; canonical: codes only (scale and
  // bias come from the staged chunks through read_sb).
  __device__ __forceinline__ void load_codes(uint32_t (&w)[kNI][LC::kWords], uint32_t (&sb)[kNI], uint32_t (&bb)[kNI],
                                             int gv) const {
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
  }

  // Canonical: scale | bias << 16 of group gv for this lane's two column
  // blocks, from the staged chunk (see stage_issue).
  __device__ __forceinline__ void read_sb(int gv, uint32_t (&sb)[kNI]) const {
    const int rel = __builtin_amdgcn_readfirstlane(gv) - g_first;
    const uint32_t *buf = sbl + ((rel / kSbChunk) % kSbBufs) * kSbBufWords + (rel % kSbChunk);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const int col = wave * kWN + ni * 16 + r16;
      sb[ni] = buf[col * kSbChunk] | (buf[(kBN + col) * kSbChunk] << 16);
    }
  }

  __device__ __forceinline__ void issue_x(unsigned char *X, int gv) const {
    const int g = __builtin_amdgcn_readfirstlane(gv);
    if (x_issuer) {
#pragma unroll
      for (int i = 0; i < XPW; ++i) dma16(xr, xo[i], (uint32_t)g * 128u, X + (wave * XPW + i) * 1024);
    }
  }

  // Vector-memory loads load_codes issues (they follow a group's x copies).
  static constexpr int kCodeLoads = CANON ? kNI : (BITS == 3 ? 3 : 2) * kNI;

  // In-kernel fp16 activations (FAST without a prepass). Copy i of stage X
  // (the 16 bytes this lane brought in: 8 bf16 values of one row) becomes 8
  // fp16 values in place, fp16 = RTZ(x): exact for 2^-17 <= |x| <= 65504
  // (bf16 carries 8 significant bits), off by less than 2^-24 below. Only the
  // lane that copied the bytes touches them, once its own copy has landed.
  // The largest magnitude of the row seen so far is kept as a bf16 bit
  // pattern (sign cleared; integer order is value order, a NaN counts as
  // largest) in 16-bit slot i % 2 of mx[i / 2].
  static constexpr int kMxRegs = (XPW + 1) / 2;
  __device__ __forceinline__ void convert_copy(unsigned char *X, int i, uint32_t (&mx)[kMxRegs]) const {
    if (x_issuer) {
      u32x4 *p = reinterpret_cast<u32x4 *>(X + (wave * XPW + i) * 1024 + lane * 16);
      const u32x4 v = *p;
      u32x4 o;
      u16x2 m = {0, 0};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t w = v[t];
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu));
        o[t] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16),
                                                                       __uint_as_float(w & 0xFFFF0000u)));
      }
      *p = o;
      // both halves -> the copy's largest, then into its slot
      m = __builtin_elementwise_max(m, __builtin_shufflevector(m, m, 1, 0));
      const uint32_t mw = __builtin_bit_cast(uint32_t, m) & ((i & 1) ? 0xFFFF0000u : 0x0000FFFFu);
      mx[i / 2] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, mx[i / 2]),
                                                                         __builtin_bit_cast(u16x2, mw)));
    }
  }

  // Whether a row this block copied lies outside the range where the
  // unscaled fp16 activations keep FAST's accuracy: a largest magnitude above
  // 2^15 (or a non-finite value), or a nonzero largest magnitude below 2^-6
  // (values below 2^-17 round with an absolute error up to 2^-24, which must
  // stay small against the row). A row's maximum combines the 8 lanes that
  // copy it (lanes 8r .. 8r+7 of a copy) with DPP moves; the block's answer
  // comes back from a barrier.
  __device__ __forceinline__ bool rows_out_of_range(const uint32_t (&mx)[kMxRegs]) const {
    int bad = 0;
    if (x_issuer) {
#pragma unroll
      for (int r = 0; r < kMxRegs; ++r) {
        u16x2 v = __builtin_bit_cast(u16x2, mx[r]);
        v = __builtin_elementwise_max(v, __builtin_bit_cast(u16x2, __builtin_amdgcn_update_dpp(
                                                               0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
        v = __builtin_elementwise_max(v, __builtin_bit_cast(u16x2, __builtin_amdgcn_update_dpp(
                                                               0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
        v = __builtin_elementwise_max(v, __builtin_bit_cast(u16x2, __builtin_amdgcn_update_dpp(
                                                               0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          if (2 * r + hh >= XPW) continue;
          const uint32_t h16 = v[hh];
          bad |= (h16 > 0x4700u) || (h16 != 0u && h16 < 0x3C80u);
        }
      }
    }
    return __syncthreads_or(bad) != 0;
  }

  // Canonical scale/bias staging. Per-group loads of a lane's own column
  // touch 16 rows for 2 bytes each; a staging load instead covers 8 groups
  // of 8 columns (16 bytes of each row's line) and copies them straight to
  // LDS. Chunk c holds groups [g_first + 8c, +8) of the tile's 256 columns
  // in buffer c % 3: scale at [col][group], bias kBN*kSbChunk dwords further.
  // Wave w copies array w / 4 (scale, bias), columns (w % 4)*64 + 8j + L/8
  // for its load j, lane L taking group L % 8: the lanes of one load fill 64
  // consecutive dwords. The row step and the chunk's first group go in the
  // uniform offset, which the buffer range check includes: rows past N and
  // groups past the array's end read zero; groups past G of other rows read
  // the next row's values. Neither is ever used.
  // Before the K loop chunks 0-1 are copied (a wait and a barrier publish
  // them); then each group g of the loop copies load (g - g_first) % 8 of
  // chunk (g - g_first)/8 + 2. A chunk's last copy is requested six groups
  // before its first group is read (codes are read at most two groups
  // ahead), and a buffer is refilled after two barriers past the last read
  // of the chunk it held.
  __device__ __forceinline__ void stage_issue(int chunk, int j) const {
    const __amdgpu_buffer_rsrc_t r = (wave >> 2) ? br : sr;
    const uint32_t soff = (uint32_t)(8 * j * G + g_first + chunk * kSbChunk) * 2u;
    uint32_t *dst = sbl + (chunk % kSbBufs) * kSbBufWords + ((wave >> 2) * kBN + (wave & 3) * 64 + 8 * j) * kSbChunk;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 2, (int)st_voff, (int)soff, 0, 0);
  }
  __device__ void stage_prologue() const {
    if constexpr (CANON) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) stage_issue(c, j);
    }
  }
  // once per group of the K loop, after the group's barrier
  __device__ __forceinline__ void stage_step(int gv) const {
    if constexpr (CANON) {
      const int rel = __builtin_amdgcn_readfirstlane(gv) - g_first;
      stage_issue(rel / 8 + 2, rel % 8);
    }
  }

  // A fragment of step t = c*MI + mi: rows mi*16 + r16, k-block 2h + c.
  __device__ __forceinline__ h8 read_a(const unsigned char *X, int t) const {
    const int c = t / MI, mi = t % MI;
    return *reinterpret_cast<const h8 *>(X + a_base + mi * 2048 + a_off[c][mi & 3]);
  }

  // Largest |W| the column blocks of this lane can produce over groups
  // [g_begin, g_end): max over groups of max(|b|, |b + Q*s|), W lying between
  // b and b + Q*s. The four lanes of a column (h = 0..3) scan every fourth
  // group and combine their maxima.
  __device__ void column_bounds(int g_begin, int g_end, float (&bound)[kNI]) const {
    constexpr float Q = (float)((1 << BITS) - 1);
    constexpr int U = 6;
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) bound[ni] = 0.f;
    for (int g0 = g_begin + h; g0 < g_end; g0 += 4 * U) {
      uint32_t sv[U][kNI], bv[U][kNI];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // g differs between the lanes of a column: it goes into the per-lane offset
        const int g = min(g0 + 4 * u, g_end - 1);
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni) {
          if constexpr (CANON) {
            sv[u][ni] = __builtin_amdgcn_raw_buffer_load_b16(sr, srow[ni] + (uint32_t)g * 2u, 0u, 0);
            bv[u][ni] = __builtin_amdgcn_raw_buffer_load_b16(br, srow[ni] + (uint32_t)g * 2u, 0u, 0);
          } else {
            const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(sr, so + ni * 64u + (uint32_t)g * 128u, 0u, 0);
            sv[u][ni] = v & 0xFFFFu;
            bv[u][ni] = v >> 16;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int ni = 0; ni < kNI; ++ni) {
          const float s = f16_to_f32((uint16_t)sv[u][ni]), b = f16_to_f32((uint16_t)bv[u][ni]);
          bound[ni] = fmaxf(bound[ni], fmaxf(fabsf(b), fabsf(__builtin_fmaf(Q, s, b))));
        }
    }
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      bound[ni] = fmaxf(bound[ni], __shfl_xor(bound[ni], 16));
      bound[ni] = fmaxf(bound[ni], __shfl_xor(bound[ni], 32));
    }
  }
};

// FAST numerics: accumulates rows m0 .. m0 + 16*MI of the block tile at
// (m0, n0) over groups [g_begin, g_end) on fp16 MFMA; cs[ni] receives the
// power-of-two output scale 2^c of the lane's column blocks.
// ONLINE: x arrives as the caller's bf16 and each wave converts the rows it
// copied to fp16 in LDS (convert_copy) in the first half of the group before
// their first read, one copy every third MFMA step (converting them all at
// one step pushes the loop past the register file); the return value says
// whether a row fell outside the range where that keeps FAST's accuracy.
template <int BITS, int MI, bool CANON, bool ONLINE = false>
__device__ __forceinline__ bool tile_accumulate3(const Gemm3Args &a, unsigned char *const (&xs)[kStages],
                                                 uint32_t *sbl, int64_t m0, int64_t n0, int g_begin, int g_end,
                                                 f32x4 (&acc)[MI][kNI], float (&cs)[kNI]) {
  constexpr int S = kStages;
  using IO = TileIO<BITS, MI, CANON>;
  using LC = typename IO::LC;
  constexpr int kSteps = 2 * MI;        // steps (c, mi) of kNI MFMAs per group
  constexpr int kHalf = kSteps / 2;
  // A fragments are read this many steps ahead of their use; the ring index
  // t % (kAhead + 1) continues across groups, whose reads ahead wrap into
  // the next stage, which is complete only after the mid-group barrier.
  // ONLINE on tiled codes reads one step ahead: its conversion registers
  // pushed the loop past the register file, and the spills sat in the K
  // loop; the shorter ring (8 fewer VGPRs) gave M = 4608, K = 4608,
  // N = 13824 691 us against 850 and M = 4096, K = N = 4608 220 against 235
  // (outputs bit-identical). On canonical codes the same change was slower
  // (759 against 695 us, 256 against 249 us), as was FAST's (1-2 %).
  constexpr int kAhead = (kSteps % 4 == 0 && kHalf >= 3 && !(ONLINE && !CANON)) ? 3 : 1;
  // FAST on tiled codes builds each group's k-block 1 fragments during the
  // group's own first half and the next group's k-block 0 fragments during
  // its second half, so one fragment set is live instead of two (16 fewer
  // VGPRs against one more code slot): 157.3 against 160.3 us at M = 4096,
  // K = N = 4608 and 444.8 against 454.1 at K = 12288 (outputs
  // bit-identical). ONLINE ran slower with it, as did the other code widths
  // (3-bit 40 %, 2-bit 2-3 %, 8-bit up to 1 %, 2048^2 sweep shapes): there
  // the next group's whole fragment set is built during the second half.
  constexpr bool kHalfRefill = !ONLINE && !CANON && BITS == 4;
  constexpr int kRing = kHalfRefill ? S : S - 1;  // code slots
  static_assert(kSteps % (kAhead + 1) == 0, "A-fragment ring must divide the steps of a group");
  static_assert(kAhead <= kHalf, "reads of the next stage must follow the mid-group barrier");
  // the next group's B fragments are built in 4 * 2 * kNI pieces of one word
  // (two weights), spread over the steps of the second half so the vector
  // work sits between MFMAs instead of in bursts
  constexpr int kPieces = 8 * kNI;
  constexpr int kPerStep = (kPieces + kHalf - 1) / kHalf;
  // ONLINE: the step of the first half at which copy i of the next stage is converted
  constexpr auto conv_step = [](int i) { return 2 + 3 * i < kHalf - 1 ? 2 + 3 * i : kHalf - 1; };
  const IO io(a, m0, n0, sbl, g_begin);
  const int h = io.h;

  // per-column fp16 range: weights of a column whose bound reaches 65504 are
  // scaled by 2^-c before the fp16 rounding (scale and bias multiplied by an
  // exact power of two), and the column's outputs by 2^c at the store
  h2 wsc[kNI];
  {
    float bound[kNI];
    io.column_bounds(g_begin, g_end, bound);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const int c = bound[ni] < 65504.f ? 0 : max(0, min(ilogbf(bound[ni]) - 14, 30));
      cs[ni] = __uint_as_float((uint32_t)(127 + c) << 23);
      const _Float16 inv = (_Float16)__uint_as_float((uint32_t)(127 - c) << 23);
      wsc[ni] = h2{inv, inv};
    }
  }

  h8 af[kAhead + 1];
  // B fragments of the group being multiplied, built from codes that arrived
  // earlier; a group past the end gets zero scale and bias, so its weights
  // are zero and its step adds nothing. Codes and scale|bias words of groups
  // g+1 .. g+S-2 are held (cq[0] = g+1); those of g+S-1 are requested in
  // group g.
  u32x4 bf[kNI][2];
  uint32_t xmx[IO::kMxRegs] = {};  // ONLINE: largest magnitudes of the rows this lane converts
  // code ring: group g+1 .. (and group g itself with half refills) at the
  // start of group g; the last slot is requested in group g
  uint32_t cq[kRing][kNI][LC::kWords];
  uint32_t sq[kRing][kNI];   // tiled: s | b << 16
  uint32_t bq[kRing][kNI];   // unused
  uint32_t sbc[kNI];         // canonical: s | b << 16 of the group being dequantized
  // piece i of the B fragments from cq[0] and its scale/bias: fragment (ni, c) = i / 4, word i % 4
  auto dequant_piece = [&](u32x4 (&dst)[kNI][2], int slot, bool valid, int i) {
    const int f = i >> 2, p = i & 3, ni = f >> 1, c = f & 1;
    const uint32_t v = valid ? (CANON ? sbc[ni] : sq[slot][ni]) : 0u;
    // scale and bias broadcast to both halves inside the packed multiply
    // (its operand select), no separate splat
    const h2 hv = __builtin_bit_cast(h2, v);
    const h2 s2 = __builtin_shufflevector(hv, hv, 0, 0) * wsc[ni];
    const h2 b2 = __builtin_shufflevector(hv, hv, 1, 1) * wsc[ni];
    if constexpr (BITS == 3 && !CANON) {
      // the first piece of a column block (i = 8 ni) runs before its other
      // pieces: in both placements below pieces run in increasing i within a
      // column block
      if (c == 0 && p == 0) cq[slot][ni][1] = LC::prep(cq[slot][ni][1], h);
    }
    uint32_t r = LC::pair(cq[slot][ni], c, p, s2, b2);
    asm volatile("" : "+v"(r));  // keeps the piece where it is placed, between MFMAs
    dst[ni][c][p] = r;
  };
  // half refills: piece j of k-block c is word j % 4 of fragment (j / 4, c)
  auto piece_of = [](int c, int j) { return ((2 * (j >> 2) + c) << 2) | (j & 3); };

  // One group on stage X. First half: MFMAs on the fragments in hand. Then
  // the barrier, after which the next stage XN is complete and the stage of
  // the previous group (XD) is free: the x copies for S-1 groups ahead go
  // into XD and their codes are requested. Second half: MFMAs, with the next
  // group's B fragments dequantized in between and the first A fragments of
  // XN read ahead, so the next group starts without a stall.
  auto step = [&](const unsigned char *X, unsigned char *XN, unsigned char *XD, int g) {
    u32x4 bn[kNI][2];
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const int c = t / MI, mi = t % MI;
      if constexpr (ONLINE) {
        // stage g+1 was copied in the middle of group g-1, and only the
        // codes of g+1 were requested after it: once at most that many
        // vector loads are in flight, this wave's copies have landed
        if (t == conv_step(0)) {
          constexpr int n = IO::kCodeLoads;
          __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | 0xF70);
        }
#pragma unroll
        for (int i = 0; i < IO::XPW; ++i)
          if (t == conv_step(i)) io.convert_copy(XN, i, xmx);
      }
      if (t == kHalf) {
        dma_barrier();  // stage g+1 has landed everywhere, stage g-1 is free
        // the second half runs at raised wave priority (back to normal at the
        // end of the group): 1-1.5 % faster on the large shapes, measured
        __builtin_amdgcn_s_setprio(1);
        io.stage_step(g);
        io.issue_x(XD, min(g + S - 1, g_end - 1));
        // ONLINE counts the code loads issued after the copies (see above)
        if constexpr (ONLINE) __builtin_amdgcn_sched_barrier(0);
        io.load_codes(cq[kRing - 1], sq[kRing - 1], bq[kRing - 1], min(g + S - 1, g_end - 1));
      }
      // canonical: the next group's scale|bias words come from LDS early in
      // the first half, so their latency is spent under MFMAs rather than
      // in front of the first dequant piece after the barrier (the staged
      // chunk was published more than six groups before; its buffer is
      // refilled two barriers after this read at the earliest). 208 -> 194 us FAST and
      // 245 -> 228 us ONLINE at M = 4096, K = N = 4608; 570 -> 546 and
      // 673 -> 645 us at M = 4608, K = 4608, N = 13824 (outputs bit-identical).
      if constexpr (CANON && !kHalfRefill) {
        if (t == 1) io.read_sb(min(g + 1, g_end - 1), sbc);
      }
      if (t + kAhead < kSteps) af[(t + kAhead) % (kAhead + 1)] = io.read_a(X, t + kAhead);
      else af[(t + kAhead) % (kAhead + 1)] = io.read_a(XN, t + kAhead - kSteps);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[t % (kAhead + 1)], __builtin_bit_cast(h8, bf[ni][c]),
                                                             acc[mi][ni], 0, 0, 0);
        if constexpr (!kHalfRefill) {
          if (t >= kHalf) {
#pragma unroll
            for (int u = 0; u < kPerStep; ++u) {
              const int i = (t - kHalf) * kPerStep + u;
              if ((u % kNI) == ni && i < kPieces) dequant_piece(bn, 0, g + 1 < g_end, i);
            }
          }
        }
      }
      if constexpr (kHalfRefill) {
        // first half: k-block 1 of group g (slot 0), while its k-block 0 is
        // in use; second half: k-block 0 of group g+1 (slot 1)
        const int tl = t % kHalf;
        constexpr int kHP = kPieces / 2;
        constexpr int kEvery = kHalf >= kHP ? kHalf / kHP : 1;
        constexpr int kPer = kHalf >= kHP ? 1 : kHP / kHalf;
        if (tl % kEvery == 0) {
#pragma unroll
          for (int u = 0; u < kPer; ++u) {
            const int j = (tl / kEvery) * kPer + u;
            if (j < kHP) {
              if (t < kHalf) dequant_piece(bf, 0, g < g_end, piece_of(1, j));
              else dequant_piece(bf, 1, g + 1 < g_end, piece_of(0, j));
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      if constexpr (!kHalfRefill) {
        bf[ni][0] = bn[ni][0];
        bf[ni][1] = bn[ni][1];
      }
#pragma unroll
      for (int j = 0; j + 1 < kRing; ++j) {
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
  if constexpr (CANON) {
    io.stage_prologue();
    dma_barrier();  // the first staged chunks are read below
  }
  if (g_begin < g_end) {
    io.load_codes(cq[0], sq[0], bq[0], g_begin);
    io.issue_x(xs[0], g_begin);
    io.issue_x(xs[1], min(g_begin + 1, g_end - 1));
  }
  dma_barrier();  // first two stages and the first codes have arrived
  if constexpr (ONLINE) {
    // the first group's stage; the second one's is converted during the first group
#pragma unroll
    for (int i = 0; i < IO::XPW; ++i) io.convert_copy(xs[0], i, xmx);
    __syncthreads();
  }
  if (g_begin < g_end) {
    if constexpr (CANON) io.read_sb(g_begin, sbc);
    if constexpr (kHalfRefill) {
      // k-block 0 of the first group; its k-block 1 is built in its first half
#pragma unroll
      for (int j = 0; j < kPieces / 2; ++j) dequant_piece(bf, 0, true, piece_of(0, j));
    } else {
#pragma unroll
      for (int i = 0; i < kPieces; ++i) dequant_piece(bf, 0, true, i);
    }
    io.load_codes(cq[kRing - 2], sq[kRing - 2], bq[kRing - 2], min(g_begin + 1, g_end - 1));
    // stages and codes up to g_begin + S - 2 are in flight now; each group g
    // requests g + S - 1
#pragma unroll
    for (int j = 2; j < S - 1; ++j) {
      io.issue_x(xs[j], min(g_begin + j, g_end - 1));
      io.load_codes(cq[kRing - S + j], sq[kRing - S + j], bq[kRing - S + j], min(g_begin + j, g_end - 1));
    }
#pragma unroll
    for (int t = 0; t < kAhead; ++t) af[t] = io.read_a(xs[0], t);
  }
  for (int g = g_begin; g < g_end; g += S) {
#pragma unroll
    for (int k = 0; k < S; ++k) step(xs[k], xs[(k + 1) % S], xs[(k + S - 1) % S], g + k);
  }
  dma_barrier();  // the copies requested past the last group have landed; every stage is free
  if constexpr (ONLINE) return io.rows_out_of_range(xmx);
  return false;
}

// SPLIT numerics: same tile walk on bf16 MFMA with hi and lo weight
// fragments. The k-block c = 1 fragments of group g are built during the
// first half of group g (from the codes of g), the c = 0 fragments of group
// g+1 during the second half (from the codes of g+1), so each half refills
// the fragments the other half does not use and no second fragment set is
// held. Code slots: [0] = group g, [1] = group g+1, requested when group g
// starts (half a group before its first use). Each A fragment feeds four
// MFMAs, so it is read one step ahead.
template <int BITS, int MI, bool CANON>
__device__ __forceinline__ void tile_accumulate_split(const Gemm3Args &a, unsigned char *const (&xs)[kStages],
                                                      uint32_t *sbl, int64_t m0, int64_t n0, int g_begin, int g_end,
                                                      f32x4 (&acc)[MI][kNI]) {
  constexpr int S = kStages;
  using IO = TileIO<BITS, MI, CANON>;
  using LC = typename IO::LC;
  constexpr int kSteps = 2 * MI;
  constexpr int kHalf = kSteps / 2;
  constexpr int kAhead = 1;
  // 4 * kNI pieces (one word of one fragment: two weights, hi and lo) per
  // half, spread evenly over the half's steps
  constexpr int kPieces = 4 * kNI;
  constexpr int kStride = kHalf >= kPieces ? kHalf / kPieces : 1;
  constexpr int kPerStep = kHalf >= kPieces ? 1 : kPieces / kHalf;
  static_assert(kHalf >= kPieces ? kHalf % kPieces == 0 : kPieces % kHalf == 0, "pieces spread evenly");
  const IO io(a, m0, n0, sbl, g_begin);
  const int h = io.h;

  h8 af[kAhead + 1];
  u32x4 bh[kNI][2], bl[kNI][2];
  uint32_t cq[2][kNI][LC::kWords];
  uint32_t sq[2][kNI];
  uint32_t bq[2][kNI];
  float sf[kNI], bfl[kNI];  // fp32 scale and bias of the slot being dequantized

  // fp32 scale and bias of group gv (code slot `slot`); canonical: read from
  // the staged chunk here
  auto prep_slot = [&](int slot, int gv, bool valid) {
    uint32_t sbc[kNI];
    if constexpr (CANON) io.read_sb(min(gv, g_end - 1), sbc);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      const uint32_t v = valid ? (CANON ? sbc[ni] : sq[slot][ni]) : 0u;
      sf[ni] = f16_to_f32((uint16_t)(v & 0xFFFFu));
      bfl[ni] = f16_to_f32((uint16_t)(v >> 16));
    }
  };
  // piece i (fragment ni = i / 4 of k-block c, word p = i % 4) from slot
  auto dequant_piece = [&](int slot, int c, int i) {
    const int ni = i >> 2, p = i & 3;
    if constexpr (BITS == 3 && !CANON) {
      if (c == 0 && p == 0) cq[slot][ni][1] = LC::prep(cq[slot][ni][1], h);
    }
    uint32_t hi, lo;
    split_pair(LC::qpair(cq[slot][ni], c, p), sf[ni], bfl[ni], hi, lo);
    asm volatile("" : "+v"(hi), "+v"(lo));  // keeps the piece where it is placed, between MFMAs
    bh[ni][c][p] = hi;
    bl[ni][c][p] = lo;
  };

  auto step = [&](const unsigned char *X, const unsigned char *XN, unsigned char *XD, int g) {
#pragma unroll
    for (int t = 0; t < kSteps; ++t) {
      const int c = t / MI, mi = t % MI;
      const int tt = t % kHalf;
      if (t == 0) {
        io.load_codes(cq[1], sq[1], bq[1], min(g + 1, g_end - 1));
        prep_slot(0, g, g < g_end);
      }
      if (t == kHalf) {
        dma_barrier();  // stage g+1 and the codes of g+1 have landed, stage g-1 is free
        __builtin_amdgcn_s_setprio(1);
        io.stage_step(g);
        io.issue_x(XD, min(g + S - 1, g_end - 1));
        prep_slot(1, g + 1, g + 1 < g_end);
      }
      if (t + kAhead < kSteps) af[(t + kAhead) % (kAhead + 1)] = io.read_a(X, t + kAhead);
      else af[(t + kAhead) % (kAhead + 1)] = io.read_a(XN, t + kAhead - kSteps);
      const bf16x8 av = __builtin_bit_cast(bf16x8, af[t % (kAhead + 1)]);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bh[ni][c]), acc[mi][ni],
                                                              0, 0, 0);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bl[ni][c]), acc[mi][ni],
                                                              0, 0, 0);
      if (tt % kStride == 0) {
#pragma unroll
        for (int u = 0; u < kPerStep; ++u) {
          const int i = (tt / kStride) * kPerStep + u;
          if (i < kPieces) {
            if (t < kHalf) dequant_piece(0, 1, i);  // k-block 1 of group g
            else dequant_piece(1, 0, i);            // k-block 0 of group g+1
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int ni = 0; ni < kNI; ++ni) {
      sq[0][ni] = sq[1][ni];
      bq[0][ni] = bq[1][ni];
#pragma unroll
      for (int u = 0; u < LC::kWords; ++u) cq[0][ni][u] = cq[1][ni][u];
    }
  };

#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < kNI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (CANON) {
    io.stage_prologue();
    dma_barrier();  // the first staged chunks are read below
  }
  if (g_begin < g_end) {
    io.load_codes(cq[0], sq[0], bq[0], g_begin);
    io.issue_x(xs[0], g_begin);
    io.issue_x(xs[1], min(g_begin + 1, g_end - 1));
  }
  dma_barrier();  // first two stages and the codes of the first group have arrived
  if (g_begin < g_end) {
    prep_slot(0, g_begin, true);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) dequant_piece(0, 0, i);  // k-block 0 of the first group
#pragma unroll
    for (int t = 0; t < kAhead; ++t) af[t] = io.read_a(xs[0], t);
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

// Stores rows m0 .. m0 + 16*MI of a tile, times the row scales rs and the
// column scales cs, into out ([M, N] fp32 or bf16). The row scales come from
// LDS (rs_lds[m - m0], staged by the caller): a global load among the stores
// would wait for every store before it, since one counter tracks both, which
// cost ~6 % of the kernel. Without SCALED (SPLIT numerics) there are no
// scales. With GLU-ordered weights subtile ni = 0 of a wave holds gate outputs
// and ni = 1 the up outputs of the same 16 columns f = 16*strip + r16 of the
// [M, N/2] result, which gets silu(gate) * up.
template <bool OUT_BF16, int MI, bool SCALED>
__device__ __forceinline__ void tile_store3(const Gemm3Args &a, void *out, int64_t m0, int64_t n0,
                                            const f32x4 (&acc)[MI][kNI], const float *rs_lds, const float (&cs)[kNI]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, h = lane >> 4;
  const int64_t row0 = m0 + 4 * h;
  auto row_scale = [&](int64_t m) -> float {
    if constexpr (SCALED) return rs_lds[m - m0];
    else return 1.f;
  };
  auto col = [&](float v, int ni) -> float {
    if constexpr (SCALED) return v * cs[ni];
    else return v;
  };
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
        const float rs = row_scale(m);
        const float v = swiglu(col(acc[mi][0][i] * rs, 0), col(acc[mi][1][i] * rs, 1));
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
          const float rs = row_scale(m);
#pragma unroll
          for (int ni = 0; ni < kNI; ++ni) {
            const int64_t n = col0 + ni * 16;
            if (!full && n >= a.N) continue;
            const float y = __builtin_fmaf(gv[c][i][ni], col(acc[mc + c][ni][i] * rs, ni), rv[c][i][ni]);
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
      const float rs = row_scale(m);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) {
        const int64_t n = col0 + ni * 16;
        if (!full && n >= a.N) continue;
        const float v = col(acc[mi][ni][i] * rs, ni);
        if constexpr (OUT_BF16) reinterpret_cast<uint16_t *>(out)[m * a.N + n] = f32_to_bf16_rne3(v);
        else reinterpret_cast<float *>(out)[m * a.N + n] = v;
      }
    }
}

// The output slice of this block's K range (fp32 partials [splits, M, N]
// when K is split).
__device__ __forceinline__ void *out_of_split(const Gemm3Args &a) {
  return a.splits > 1 ? static_cast<void *>(static_cast<float *>(a.out) + (int64_t)blockIdx.y * a.M * a.N) : a.out;
}

// ONLINE: the mark of a tile left to the fixup kernel, a NaN in its first
// output element (m0, n0), and the fixup kernel's test for it (every thread
// reads the same element: the answer is uniform).
template <bool OUT_BF16>
__device__ __forceinline__ void mark_tile(void *out, int64_t N, int64_t m0, int64_t n0) {
  if constexpr (OUT_BF16) reinterpret_cast<uint16_t *>(out)[m0 * N + n0] = 0x7FC1u;
  else reinterpret_cast<uint32_t *>(out)[m0 * N + n0] = 0x7FC00001u;
}
template <bool OUT_BF16>
__device__ __forceinline__ bool tile_marked(const void *out, int64_t N, int64_t m0, int64_t n0) {
  if constexpr (OUT_BF16) {
    const uint32_t v = reinterpret_cast<const uint16_t *>(out)[m0 * N + n0];
    return __builtin_amdgcn_readfirstlane((v & 0x7FFFu) > 0x7F80u) != 0;
  } else {
    const uint32_t v = reinterpret_cast<const uint32_t *>(out)[m0 * N + n0];
    return __builtin_amdgcn_readfirstlane((v & 0x7FFFFFFFu) > 0x7F800000u) != 0;
  }
}

// blockIdx.y = K range (a.splits of them; each writes its own fp32 slice of
// out, [splits, M, N], for an ordered reduction afterwards). Blocks
// [0, tail_tiles * 16/PMI) run one row piece each of the last tail_tiles
// tiles (PMI 16-row subtiles each, pieces of one tile on one XCD), even
// blocks before and odd blocks after their whole tiles t = blockIdx.x,
// + gridDim.x, ... below dp_tiles.
// Power-of-two row and column scales commute exactly with the summation, so
// partials carry them already.
// ONLINE (FAST only): x16 holds the caller's bf16 x, converted to fp16 in
// LDS by the kernel (no row scales). A tile with a row outside that
// conversion's range is not stored: its first output element gets a NaN
// mark and gemm3_fixup_kernel, launched next on the same grid, recomputes
// it with SPLIT numerics. Other tiles have finite outputs (finite fp16
// operands, |x| <= 2^15), so a NaN there means a marked tile, or a NaN
// weight, whose SPLIT recomputation is NaN as well.
template <int BITS, bool OUT_BF16, int PMI, bool CANON, bool SPLIT, bool ONLINE = false>
__global__ __launch_bounds__(kNT, 1) void gemm3_kernel(Gemm3Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char x0[kXStage];
  __shared__ __attribute__((aligned(16))) unsigned char x1[kXStage];
  __shared__ __attribute__((aligned(16))) unsigned char x2[kXStage];
  __shared__ __attribute__((aligned(16))) float rs_lds[kBM];
  // canonical scale/bias staging (unused with tiled weights)
  __shared__ __attribute__((aligned(16))) uint32_t sbl[CANON ? kSbBufs * kSbBufWords : 4];
  unsigned char *const xs[kStages] = {x0, x1, x2};
  // FAST: the row scales of a tile's rows, requested at the tile's start (one
  // value per thread), written to LDS once the K loop has ended (its last
  // barrier also ends every wave's reads of the previous tile's scales)
  auto tile_rs = [&](int64_t m0, int rows) -> float {
    if constexpr (SPLIT || ONLINE) return 1.f;
    const int64_t m = m0 + threadIdx.x;
    return (int)threadIdx.x < rows && m < a.M ? a.rowscale[m] : 0.f;
  };
  auto stage_rs = [&](float v, int rows) {
    if constexpr (SPLIT) return;
    if ((int)threadIdx.x < rows) rs_lds[threadIdx.x] = v;
    __syncthreads();
  };
  auto accumulate = [&](auto &acc_, int64_t m0, int64_t n0, int gb, int ge, float (&cs)[kNI]) {
    constexpr int MI = sizeof(acc_) / sizeof(acc_[0]);
    if constexpr (SPLIT) {
      tile_accumulate_split<BITS, MI, CANON>(a, xs, sbl, m0, n0, gb, ge, acc_);
#pragma unroll
      for (int ni = 0; ni < kNI; ++ni) cs[ni] = 1.f;
      return false;
    } else {
      return tile_accumulate3<BITS, MI, CANON, ONLINE>(a, xs, sbl, m0, n0, gb, ge, acc_, cs);
    }
  };
  // ONLINE: a tile left to the fixup kernel (the flag is uniform per block)
  auto store = [&](bool redo, auto &acc_, int64_t m0, int64_t n0, const float (&cs)[kNI]) {
    constexpr int MI = sizeof(acc_) / sizeof(acc_[0]);
    if (!redo) tile_store3<OUT_BF16, MI, !SPLIT>(a, out_of_split(a), m0, n0, acc_, rs_lds, cs);
    else if (threadIdx.x == 0) mark_tile<OUT_BF16>(out_of_split(a), a.N, m0, n0);
  };
  const int tiles_n = (int)((a.N + kBN - 1) / kBN);
  const int split = blockIdx.y;
  const int gps = (a.G + a.splits - 1) / a.splits;
  const int gb = split * gps, ge = min(a.G, gb + gps);

  auto run_piece = [&]() {
    if constexpr (PMI > 0) {
      constexpr int kPieces = 16 / PMI;
      if ((int)blockIdx.x < a.tail_tiles * kPieces) {
        const int tail = blockIdx.x % a.tail_tiles, piece = blockIdx.x / a.tail_tiles;
        const int tile = a.dp_tiles + tail;
        const int64_t m0 = (int64_t)(tile / tiles_n) * kBM + piece * 16 * PMI;
        const int64_t n0 = (int64_t)(tile % tiles_n) * kBN;
        if (m0 < a.M) {  // uniform per block
          f32x4 pacc[PMI][kNI];
          float cs[kNI];
          const float rs = tile_rs(m0, 16 * PMI);
          const bool redo = accumulate(pacc, m0, n0, gb, ge, cs);
          stage_rs(rs, 16 * PMI);
          store(redo, pacc, m0, n0, cs);
        }
      }
    }
  };
  // Even blocks run their row piece before their whole tiles, odd blocks
  // after them, so half the CUs store a whole tile while the other half
  // still computes (every CU storing its 256 KB tile at the same moment
  // leaves the matrix cores idle behind the write bandwidth): 165.3 -> 161.7
  // us at M = 4096, K = N = 4608, measured.
  const bool piece_last = (blockIdx.x & 1) != 0;
  if (!piece_last) run_piece();
  f32x4 acc[kMI][kNI];
  for (int t = blockIdx.x; t < a.dp_tiles; t += gridDim.x) {
    const int tile = xcd_remap(t, a.dp_tiles);
    const int64_t m0 = (int64_t)(tile / tiles_n) * kBM, n0 = (int64_t)(tile % tiles_n) * kBN;
    float cs[kNI];
    const float rs = tile_rs(m0, kBM);
    const bool redo = accumulate(acc, m0, n0, gb, ge, cs);
    stage_rs(rs, kBM);
    store(redo, acc, m0, n0, cs);
  }
  if (piece_last) run_piece();
}

// The tiles of an ONLINE launch that gemm3_kernel left marked, recomputed
// with SPLIT numerics: same grid, same tile and row-piece walk; every other
// tile costs one load of its mark.
template <int BITS, bool OUT_BF16, int PMI, bool CANON>
__global__ __launch_bounds__(kNT, 1) void gemm3_fixup_kernel(Gemm3Args a) {
  __shared__ __attribute__((aligned(16))) unsigned char x0[kXStage];
  __shared__ __attribute__((aligned(16))) unsigned char x1[kXStage];
  __shared__ __attribute__((aligned(16))) unsigned char x2[kXStage];
  __shared__ __attribute__((aligned(16))) uint32_t sbl[CANON ? kSbBufs * kSbBufWords : 4];
  unsigned char *const xs[kStages] = {x0, x1, x2};
  const int tiles_n = (int)((a.N + kBN - 1) / kBN);
  const int split = blockIdx.y;
  const int gps = (a.G + a.splits - 1) / a.splits;
  const int gb = split * gps, ge = min(a.G, gb + gps);
  void *out = out_of_split(a);
  const float one[kNI] = {1.f, 1.f};
  if constexpr (PMI > 0) {
    constexpr int kPieces = 16 / PMI;
    if ((int)blockIdx.x < a.tail_tiles * kPieces) {
      const int tail = blockIdx.x % a.tail_tiles, piece = blockIdx.x / a.tail_tiles;
      const int tile = a.dp_tiles + tail;
      const int64_t m0 = (int64_t)(tile / tiles_n) * kBM + piece * 16 * PMI;
      const int64_t n0 = (int64_t)(tile % tiles_n) * kBN;
      if (m0 < a.M && tile_marked<OUT_BF16>(out, a.N, m0, n0)) {
        f32x4 pacc[PMI][kNI];
        tile_accumulate_split<BITS, PMI, CANON>(a, xs, sbl, m0, n0, gb, ge, pacc);
        tile_store3<OUT_BF16, PMI, false>(a, out, m0, n0, pacc, nullptr, one);
      }
    }
  }
  for (int t = blockIdx.x; t < a.dp_tiles; t += gridDim.x) {
    const int tile = xcd_remap(t, a.dp_tiles);
    const int64_t m0 = (int64_t)(tile / tiles_n) * kBM, n0 = (int64_t)(tile % tiles_n) * kBN;
    if (!tile_marked<OUT_BF16>(out, a.N, m0, n0)) continue;
    f32x4 acc[kMI][kNI];
    tile_accumulate_split<BITS, kMI, CANON>(a, xs, sbl, m0, n0, gb, ge, acc);
    tile_store3<OUT_BF16, kMI, false>(a, out, m0, n0, acc, nullptr, one);
  }
}

template <int BITS, bool OUT_BF16, bool CANON, bool SPLIT, bool ONLINE>
void launch3_out(const Gemm3Args &a, hipStream_t stream) {
  const dim3 grid((unsigned)a.grid_x, (unsigned)a.splits);
  switch (a.tail_tiles > 0 ? a.tail_mi : 0) {
    case 2: hipLaunchKernelGGL((gemm3_kernel<BITS, OUT_BF16, 2, CANON, SPLIT, ONLINE>), grid, dim3(kNT), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((gemm3_kernel<BITS, OUT_BF16, 4, CANON, SPLIT, ONLINE>), grid, dim3(kNT), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((gemm3_kernel<BITS, OUT_BF16, 8, CANON, SPLIT, ONLINE>), grid, dim3(kNT), 0, stream, a); break;
    default: hipLaunchKernelGGL((gemm3_kernel<BITS, OUT_BF16, 0, CANON, SPLIT, ONLINE>), grid, dim3(kNT), 0, stream, a); break;
  }
}

template <int BITS, bool OUT_BF16, bool CANON>
void launch3_fixup_out(const Gemm3Args &a, hipStream_t stream) {
  const dim3 grid((unsigned)a.grid_x, (unsigned)a.splits);
  switch (a.tail_tiles > 0 ? a.tail_mi : 0) {
    case 2: hipLaunchKernelGGL((gemm3_fixup_kernel<BITS, OUT_BF16, 2, CANON>), grid, dim3(kNT), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((gemm3_fixup_kernel<BITS, OUT_BF16, 4, CANON>), grid, dim3(kNT), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((gemm3_fixup_kernel<BITS, OUT_BF16, 8, CANON>), grid, dim3(kNT), 0, stream, a); break;
    default: hipLaunchKernelGGL((gemm3_fixup_kernel<BITS, OUT_BF16, 0, CANON>), grid, dim3(kNT), 0, stream, a); break;
  }
}

template <int BITS, bool CANON, bool SPLIT, bool ONLINE>
void launch3_layout(const Gemm3Args &a, hipStream_t stream) {
  const bool bf = a.out_bf16 && a.splits == 1;
  if (bf) launch3_out<BITS, true, CANON, SPLIT, ONLINE>(a, stream);
  else launch3_out<BITS, false, CANON, SPLIT, ONLINE>(a, stream);
  if constexpr (ONLINE) {
    if (bf) launch3_fixup_out<BITS, true, CANON>(a, stream);
    else launch3_fixup_out<BITS, false, CANON>(a, stream);
  }
}

template <int BITS, bool SPLIT, bool ONLINE = false>
hipError_t launch3_bits(const Gemm3Args &a, hipStream_t stream) {
  if (a.tail_tiles > 0 && a.tail_mi != 2 && a.tail_mi != 4 && a.tail_mi != 8) return hipErrorInvalidValue;
  if (a.splits < 1 || (a.splits > 1 && a.tail_tiles > 0)) return hipErrorInvalidValue;
  if constexpr (BITS == 3) {
    if (a.canon) return hipErrorInvalidValue;  // 3-bit codes run on tiled weights only
    launch3_layout<BITS, false, SPLIT, ONLINE>(a, stream);
  } else {
    if (a.canon) launch3_layout<BITS, true, SPLIT, ONLINE>(a, stream);
    else launch3_layout<BITS, false, SPLIT, ONLINE>(a, stream);
  }
  return hipGetLastError();
}

}  // namespace g3

}  // namespace ql
