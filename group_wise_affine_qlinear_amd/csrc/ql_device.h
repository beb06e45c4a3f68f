// Device-side helpers shared by the qlinear HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kGroup = 64;

// Codes are fed to the bf16 MFMA as exact integers. For 2- and 4-bit codes the
// bf16 bit pattern 0x4300 | q is the value 128 + q (exponent 2^7, q in the low
// mantissa bits), so one AND-OR per pair produces two operands. The offset is
// removed per group with the row sums of x: sum_k x*(128+q) = P + 128*xsum.
// 8-bit codes are converted exactly (integers <= 255 fit bf16's 8-bit
// significand) and carry no offset.
template <int BITS> struct CodeOffset { static constexpr float value = 128.0f; };  // 2, 3, 4-bit
template <> struct CodeOffset<8> { static constexpr float value = 0.0f; };

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// (a & mask) | bits in one v_and_or_b32. With both constants as literals the
// compiler emits a v_and_b32 and a v_or_b32 (a VOP3 op takes no literal), so
// the empty asm statements pin the mask to an SGPR and `bits` to a VGPR
// (loop-invariant, hoisted) and leave the compiler free to select
// v_and_or_b32 itself. The instruction must stay visible to the compiler: its
// result often feeds an MFMA directly, and the wait states required between a
// VALU write of a VGPR and an MFMA read of it are only inserted for
// instructions the compiler knows are VALU, never for an asm statement.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
  asm("" : "+s"(mask));
  asm("" : "+v"(bits));
  return (a & mask) | bits;
}

// 4-bit: word w holds codes c0..c7 (nibble i = code i). Returns four bf16
// pairs (c0,c1),(c2,c3),(c4,c5),(c6,c7) as 128 + code.
__device__ __forceinline__ u32x4 unpack8_b4(uint32_t w) {
  const uint32_t t = w >> 4;
  u32x4 r;
  // byte p of w holds (c_{2p} low nibble, c_{2p+1} high nibble); byte p of t
  // holds c_{2p+1} in its low nibble. Select w.byte_p -> byte 0, t.byte_p ->
  // byte 2, zero bytes 1 and 3, then keep the low nibble of each half.
  const uint32_t hi = 0x43004300u;
  r[0] = and_or(perm(t, w, 0x0C040C00u), 0x000F000Fu, hi);
  r[1] = and_or(perm(t, w, 0x0C050C01u), 0x000F000Fu, hi);
  r[2] = and_or(perm(t, w, 0x0C060C02u), 0x000F000Fu, hi);
  r[3] = and_or(perm(t, w, 0x0C070C03u), 0x000F000Fu, hi);
  return r;
}

// 2-bit: the 16-bit half `half` (0 or 1) of w holds codes c0..c7 (2 bits
// each). Returns four bf16 pairs as 128 + code.
__device__ __forceinline__ u32x4 unpack8_b2(uint32_t w, int half) {
  const uint32_t v = half ? (w >> 16) : w;
  const uint32_t v2 = v >> 2, v4 = v >> 4, v6 = v >> 6;
  u32x4 r;
  // byte b of v holds codes 4b..4b+3 at bits 0,2,4,6.
  const uint32_t hi = 0x43004300u;
  r[0] = and_or(perm(v2, v, 0x0C040C00u), 0x00030003u, hi);   // c0, c1
  r[1] = and_or(perm(v6, v4, 0x0C040C00u), 0x00030003u, hi);  // c2, c3
  r[2] = and_or(perm(v2, v, 0x0C050C01u), 0x00030003u, hi);   // c4, c5
  r[3] = and_or(perm(v6, v4, 0x0C050C01u), 0x00030003u, hi);  // c6, c7
  return r;
}

// 8-bit: two words hold codes c0..c7 (byte i of w0 = c_i, of w1 = c_{4+i}).
// Returns four bf16 pairs holding the codes exactly.
__device__ __forceinline__ u32x4 unpack8_b8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  // (float)(byte) lowers to v_cvt_f32_ubyte{0..3}
  const float a0 = (float)(w0 & 0xFFu), a1 = (float)((w0 >> 8) & 0xFFu);
  const float a2 = (float)((w0 >> 16) & 0xFFu), a3 = (float)(w0 >> 24);
  const float b0 = (float)(w1 & 0xFFu), b1 = (float)((w1 >> 8) & 0xFFu);
  const float b2 = (float)((w1 >> 16) & 0xFFu), b3 = (float)(w1 >> 24);
  // an integer <= 255 has a zero low half in fp32, so the high half is its bf16
  r[0] = perm(__float_as_uint(a1), __float_as_uint(a0), 0x07060302u);
  r[1] = perm(__float_as_uint(a3), __float_as_uint(a2), 0x07060302u);
  r[2] = perm(__float_as_uint(b1), __float_as_uint(b0), 0x07060302u);
  r[3] = perm(__float_as_uint(b3), __float_as_uint(b2), 0x07060302u);
  return r;
}

// Tiled layout (pair order, see layout.hip), 4-bit: word w holds code 2p in
// bits [4p, 4p+4) and code 2p+1 in bits [16+4p, 16+4p+4). Pair p is one shift
// and one AND-OR: four bf16 pairs as 128 + code.
__device__ __forceinline__ u32x4 unpack8_b4_pair(uint32_t w) {
  const uint32_t hi = 0x43004300u;
  u32x4 r;
  r[0] = and_or(w, 0x000F000Fu, hi);
  r[1] = and_or(w >> 4, 0x000F000Fu, hi);
  r[2] = and_or(w >> 8, 0x000F000Fu, hi);
  r[3] = and_or(w >> 12, 0x000F000Fu, hi);
  return r;
}

// Tiled layout, 2-bit: word w holds code 2p in bits [2p, 2p+2) and code 2p+1
// in bits [16+2p, 16+2p+2), p = 0..7; `half` selects pairs 4*half .. 4*half+3.
__device__ __forceinline__ u32x4 unpack8_b2_pair(uint32_t w, int half) {
  const uint32_t hi = 0x43004300u;
  const uint32_t v = half ? (w >> 8) : w;
  u32x4 r;
  r[0] = and_or(v, 0x00030003u, hi);
  r[1] = and_or(v >> 2, 0x00030003u, hi);
  r[2] = and_or(v >> 4, 0x00030003u, hi);
  r[3] = and_or(v >> 6, 0x00030003u, hi);
  return r;
}

// Canonical code stream: a row's codes form one little-endian bit stream
// along K, code k in stream bits [BITS*k, BITS*k + BITS), stream bit i being
// bit i % 32 of word i / 32. One 64-wide group is 2*BITS words; 3-bit codes
// 10, 21, 42 and 53 of a group straddle two words. With i a compile-time
// constant (unrolled loops) both helpers reduce to shifts and masks.
template <int BITS>
__device__ __forceinline__ uint32_t stream_code(const uint32_t (&w)[2 * BITS], int i) {
  const int p = BITS * i, j = p >> 5, sh = p & 31;
  uint32_t v = w[j] >> sh;
  if (sh + BITS > 32) v |= w[j + 1] << (32 - sh);
  return v & ((1u << BITS) - 1u);
}
template <int BITS>
__device__ __forceinline__ void stream_put(uint32_t (&w)[2 * BITS], int i, uint32_t q) {
  const int p = BITS * i, j = p >> 5, sh = p & 31;
  w[j] |= q << sh;
  if (sh + BITS > 32) w[j + 1] |= q >> (32 - sh);
}

// x >> n for n >= 0, x << -n otherwise (n a compile-time constant after
// unrolling).
__device__ __forceinline__ uint32_t shift_right(uint32_t x, int n) { return n >= 0 ? x >> n : x << -n; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over `bytes` bytes starting at base + off (stride 0,
// word 3 = the gfx9 raw-buffer format). Reads past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t off, int64_t bytes) {
  const char *p = reinterpret_cast<const char *>(base) + off;
  const int n = bytes >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), (short)0, n, 0x00020000);
}

// One 16-byte-per-lane copy buffer -> LDS: lane L's bytes (at voff + soff in
// the buffer) land at lds + 16*L. `lds` and `soff` must be wave-uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void *lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, (int)voff, (int)soff, 0, 0);
}

// Block barrier that publishes LDS filled by dma16: a copy to LDS is a vector
// memory load, counted by vmcnt until its bytes are in LDS, and the workgroup
// fence of __syncthreads() waits only for LDS operations, so each wave first
// waits for all of its own copies (and other loads) in flight.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// XCD-aware remap of a linear block id: the hardware deals consecutive block
// ids round-robin over the 8 XCDs; renumber so that each XCD receives a
// contiguous run of logical tiles (neighbouring tiles share one L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  if (nblocks % kXcd != 0) return bid;
  const int per = nblocks / kXcd;
  return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace ql
