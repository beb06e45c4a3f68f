// Tiled weight layout (QL_LAYOUT_TILED) and the repack / unrepack kernels.
//
// The canonical layout stores each output row's codes contiguously, so a wave
// that works on 32 columns touches 32 rows x 32 bytes per group: partial cache
// lines, which caps streaming reads well below HBM bandwidth. The tiled layout
// stores, for every strip of 32 output columns and every 64-wide K group, one
// contiguous block in the lane order of the kernels:
//
//   4-bit: 1 KB   = [h 2][col 32][4 words]   words t: codes 32h+8t .. +7
//   8-bit: 2 KB   = [part 2][h 2][col 32][4 words]  part p: codes 32h+16p .. +15
//   2-bit: 512 B  = [h 2][col 32][2 words]   words t: codes 32h+16t .. +15
//   3-bit: 768 B  = the 2-bit block of the codes' low two bits, then
//                   [h 2][col 32][1 word] of their high bits: code 32h+2P at
//                   bit P and code 32h+2P+1 at bit 16+P (P = 0..15)
//
// so lane l = 32h + col of a wave reads its 16 (or 8) bytes at l*16 and one
// load instruction covers whole cache lines. Blocks are ordered [strip][group].
// Inside a word, 2- and 4-bit codes use a pair order: code 2p sits in the low
// half and code 2p+1 in the high half at the same bit offset (4-bit: bits
// 4p and 16+4p; 2-bit: bits 2p and 16+2p), so a shift and one AND-OR give a
// pair of bf16 operands. 8-bit words keep little-endian byte order.
// Scale and bias become one uint32 per (strip, group, column): s | b << 16,
// ordered [strip][group][col]. Columns past N in the last strip are zero.
//
// GLU order (for a fused gate/up projection, rows [gate (F); up (F)], N = 2F,
// F a multiple of 16): strip j holds gate rows 16j .. 16j+15 in its columns
// 0..15 and up rows 16j .. 16j+15 in columns 16..31, so one lane of the GEMM
// ends with a gate output and the matching up output in its registers.
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

// Canonical word(s) of 8 codes -> pair-order word, 4-bit: c_i at bits 4i ->
// c_{2p} at 4p, c_{2p+1} at 16+4p.
__device__ __forceinline__ uint32_t to_pair_b4(uint32_t w) {
  uint32_t r = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    r |= ((w >> (8 * p)) & 0xFu) << (4 * p);
    r |= ((w >> (8 * p + 4)) & 0xFu) << (16 + 4 * p);
  }
  return r;
}
__device__ __forceinline__ uint32_t from_pair_b4(uint32_t r) {
  uint32_t w = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    w |= ((r >> (4 * p)) & 0xFu) << (8 * p);
    w |= ((r >> (16 + 4 * p)) & 0xFu) << (8 * p + 4);
  }
  return w;
}
// 2-bit: 16 codes, c_i at bits 2i -> c_{2p} at 2p, c_{2p+1} at 16+2p.
__device__ __forceinline__ uint32_t to_pair_b2(uint32_t w) {
  uint32_t r = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    r |= ((w >> (4 * p)) & 0x3u) << (2 * p);
    r |= ((w >> (4 * p + 2)) & 0x3u) << (16 + 2 * p);
  }
  return r;
}
__device__ __forceinline__ uint32_t from_pair_b2(uint32_t r) {
  uint32_t w = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    w |= ((r >> (2 * p)) & 0x3u) << (4 * p);
    w |= ((r >> (16 + 2 * p)) & 0x3u) << (4 * p + 2);
  }
  return w;
}

// One thread per (strip, group, column): moves that column's codes of the group
// (2*BITS words) and its scale/bias between the layouts.
// glu_f > 0: GLU order with F = glu_f (tiled column col of strip `strip`
// holds canonical row 16*strip + col, or F + 16*strip + col - 16).
template <int BITS, bool TO_TILED>
__global__ __launch_bounds__(256) void repack_kernel(const uint32_t *src, uint32_t *dst,
                                                     const uint16_t *s, const uint16_t *b,
                                                     uint32_t *sb, uint16_t *s_out,
                                                     uint16_t *b_out, int64_t N, int64_t K, int64_t glu_f) {
  constexpr int WPG = 2 * BITS;  // words of one column per group
  const int64_t G = K / 64;
  const int64_t N32 = (N + 31) / 32;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N32 * G * 32) return;
  const int col = (int)(idx % 32);
  const int64_t g = (idx / 32) % G;
  const int64_t strip = idx / (32 * G);
  const int64_t n = glu_f > 0 ? (col < 16 ? strip * 16 + col : glu_f + strip * 16 + (col - 16)) : strip * 32 + col;
  const bool real = glu_f > 0 ? strip * 16 < glu_f : n < N;
  uint32_t *tile = TO_TILED ? dst : const_cast<uint32_t *>(src);
  uint32_t *blk = tile + (strip * G + g) * (32 * WPG);
  // tiled position of canonical word j (0..WPG-1) of this column
  auto tpos = [&](int j) -> int64_t {
    if (BITS == 4) return (j >> 2) * 128 + col * 4 + (j & 3);          // h = j/4, t = j%4
    if (BITS == 8) return ((j >> 2) & 1) * 256 + (j >> 3) * 128 + col * 4 + (j & 3);  // h = j/8, part = (j/4)%2
    return (j >> 1) * 64 + col * 2 + (j & 1);                            // 2-bit: h = j/2, t = j%2
  };
  if constexpr (BITS == 3) {
    // low-bit plane words at [h][col][t] (2-bit block), high-bit plane at 128 + [h][col]
    if (TO_TILED) {
      // 8-byte loads: a group's 24 bytes start on an 8-byte boundary
      uint32_t cw[WPG];
      const u32x2 *crow = reinterpret_cast<const u32x2 *>(src + n * (K * 3 / 32) + g * WPG);
#pragma unroll
      for (int j = 0; j < WPG / 2; ++j) {
        const u32x2 v = real ? crow[j] : u32x2{0u, 0u};
        cw[2 * j] = v[0];
        cw[2 * j + 1] = v[1];
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t hi = 0;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          uint32_t lo = 0;
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            const uint32_t c0 = stream_code<3>(cw, 32 * hh + 16 * t + 2 * p);
            const uint32_t c1 = stream_code<3>(cw, 32 * hh + 16 * t + 2 * p + 1);
            lo |= ((c0 & 3u) << (2 * p)) | ((c1 & 3u) << (16 + 2 * p));
            hi |= ((c0 >> 2) << (8 * t + p)) | ((c1 >> 2) << (16 + 8 * t + p));
          }
          blk[hh * 64 + col * 2 + t] = lo;
        }
        blk[128 + hh * 32 + col] = hi;
      }
      sb[(strip * G + g) * 32 + col] = real ? ((uint32_t)s[n * G + g] | ((uint32_t)b[n * G + g] << 16)) : 0u;
    } else {
      if (!real) return;
      uint32_t cw[WPG];
#pragma unroll
      for (int j = 0; j < WPG; ++j) cw[j] = 0u;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t hi = blk[128 + hh * 32 + col];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint32_t lo = blk[hh * 64 + col * 2 + t];
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            const uint32_t c0 = ((lo >> (2 * p)) & 3u) | (((hi >> (8 * t + p)) & 1u) << 2);
            const uint32_t c1 = ((lo >> (16 + 2 * p)) & 3u) | (((hi >> (16 + 8 * t + p)) & 1u) << 2);
            stream_put<3>(cw, 32 * hh + 16 * t + 2 * p, c0);
            stream_put<3>(cw, 32 * hh + 16 * t + 2 * p + 1, c1);
          }
        }
      }
      uint32_t *crow = dst + n * (K * 3 / 32) + g * WPG;
#pragma unroll
      for (int j = 0; j < WPG; ++j) crow[j] = cw[j];
      const uint32_t v = sb[(strip * G + g) * 32 + col];
      s_out[n * G + g] = (uint16_t)(v & 0xFFFFu);
      b_out[n * G + g] = (uint16_t)(v >> 16);
    }
    return;
  }
  if (TO_TILED) {
    // 16-byte loads of the column's WPG words (rows and groups start on
    // 16-byte boundaries: packed_q is 16-byte aligned and a row holds a whole
    // number of groups) and 16- (2-bit: 8-) byte stores of consecutive tiled
    // words, so one store instruction of 32 lanes fills 512 contiguous bytes
    const u32x4 *crow = reinterpret_cast<const u32x4 *>(src + n * (K * BITS / 32) + g * WPG);
#pragma unroll
    for (int v = 0; v < WPG / 4; ++v) {
      u32x4 w = real ? crow[v] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (BITS == 4) w[e] = to_pair_b4(w[e]);
        if (BITS == 2) w[e] = to_pair_b2(w[e]);
      }
      if constexpr (BITS == 2) {
        *reinterpret_cast<u32x2 *>(blk + tpos(4 * v)) = u32x2{w[0], w[1]};
        *reinterpret_cast<u32x2 *>(blk + tpos(4 * v + 2)) = u32x2{w[2], w[3]};
      } else {
        *reinterpret_cast<u32x4 *>(blk + tpos(4 * v)) = w;
      }
    }
    sb[(strip * G + g) * 32 + col] = real ? ((uint32_t)s[n * G + g] | ((uint32_t)b[n * G + g] << 16)) : 0u;
  } else {
    if (!real) return;
    uint32_t *crow = dst + n * (K * BITS / 32) + g * WPG;
#pragma unroll
    for (int j = 0; j < WPG; ++j) {
      uint32_t w = blk[tpos(j)];
      if (BITS == 4) w = from_pair_b4(w);
      if (BITS == 2) w = from_pair_b2(w);
      crow[j] = w;
    }
    const uint32_t v = sb[(strip * G + g) * 32 + col];
    s_out[n * G + g] = (uint16_t)(v & 0xFFFFu);
    b_out[n * G + g] = (uint16_t)(v >> 16);
  }
}

template <int BITS, bool TO_TILED>
hipError_t repack_bits(const uint32_t *src, uint32_t *dst, const uint16_t *s, const uint16_t *b,
                       uint32_t *sb, uint16_t *s_out, uint16_t *b_out, int64_t N, int64_t K, int64_t glu_f,
                       hipStream_t stream) {
  const int64_t threads = ((N + 31) / 32) * (K / 64) * 32;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((repack_kernel<BITS, TO_TILED>), dim3((unsigned)blocks), dim3(256), 0, stream, src, dst, s,
                     b, sb, s_out, b_out, N, K, glu_f);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_repack(int bits, const uint32_t *canon, const uint16_t *s, const uint16_t *b, int64_t N,
                         int64_t K, int64_t glu_f, uint32_t *tiled, uint32_t *sb, hipStream_t stream) {
  if (bits == 4) return repack_bits<4, true>(canon, tiled, s, b, sb, nullptr, nullptr, N, K, glu_f, stream);
  if (bits == 8) return repack_bits<8, true>(canon, tiled, s, b, sb, nullptr, nullptr, N, K, glu_f, stream);
  if (bits == 2) return repack_bits<2, true>(canon, tiled, s, b, sb, nullptr, nullptr, N, K, glu_f, stream);
  if (bits == 3) return repack_bits<3, true>(canon, tiled, s, b, sb, nullptr, nullptr, N, K, glu_f, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_unrepack(int bits, const uint32_t *tiled, const uint32_t *sb, int64_t N, int64_t K, int64_t glu_f,
                           uint32_t *canon, uint16_t *s, uint16_t *b, hipStream_t stream) {
  uint32_t *sbm = const_cast<uint32_t *>(sb);
  if (bits == 4) return repack_bits<4, false>(tiled, canon, nullptr, nullptr, sbm, s, b, N, K, glu_f, stream);
  if (bits == 8) return repack_bits<8, false>(tiled, canon, nullptr, nullptr, sbm, s, b, N, K, glu_f, stream);
  if (bits == 2) return repack_bits<2, false>(tiled, canon, nullptr, nullptr, sbm, s, b, N, K, glu_f, stream);
  if (bits == 3) return repack_bits<3, false>(tiled, canon, nullptr, nullptr, sbm, s, b, N, K, glu_f, stream);
  return hipErrorInvalidValue;
}

}  // namespace ql
