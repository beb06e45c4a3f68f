// Skinny-M path (M <= 16): memory-bound GEMV-like projection, e.g. the AdaLN
// modulation and timestep projections (one or a few rows of x against a wide
// weight). The kernel streams each packed weight row once from HBM with
// 16-byte loads and keeps the arithmetic on the matrix cores so the vector
// ALUs only unpack codes.
//
// Block = 8 waves = 2 strips of 32 output columns x 4 K-quarters. The block
// first stages x[0:M, chunk] in LDS together with its per-group row sums, so
// the waves read activations at LDS latency while their code stream runs
// ahead in registers (4 groups in flight per lane). Per group and wave:
//   B: each lane holds its column's codes for half of the group (lane/32
//      picks the half), i.e. 16 bytes of 4-bit codes = 4 MFMA K-steps;
//   A: lanes whose row m = lane%32 < M read the matching 32 values of x from
//      LDS (rows >= M are zero);
//   P  = sum over the 4 steps of v_mfma_f32_32x32x16_bf16(x, 128 + q)
//   acc += s * P + (b - 128 s) * xsum[m, g].
// Step t of lane half h covers codes 32h + 8t .. 32h + 8t + 7 of the group, so
// every MFMA stays inside one group. The four K-quarter partial sums are added
// in a fixed order through LDS (deterministic, no atomics).
#include "ql_device.h"
#include "ql_kernels.h"

namespace ql {

namespace {

constexpr int kStrips = 2;       // 32-column strips per block
constexpr int kKSplit = 4;       // waves per strip (K quarters)
constexpr int kThreads = 64 * kStrips * kKSplit;
constexpr int kXBudget = 76 * 1024;  // LDS bytes staged per block (2 blocks per CU)

__device__ __forceinline__ uint16_t f32_to_bf16_rne_s(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Per-lane codes of one group: 4-bit 16 B, 8-bit 32 B, 2-bit 8 B, 3-bit 8 B
// of low bits + 4 B of high bits (tiled only). `p` points at the lane's first
// 16 (8) bytes; for 8-bit `p2` at its second 16 bytes, for 3-bit at its
// high-bit word.
template <int BITS> struct LaneCodes { u32x4 v[BITS == 8 ? 2 : 1]; };

template <int BITS, bool TILED>
__device__ __forceinline__ LaneCodes<BITS> load_codes(const uint32_t *p, const uint32_t *p2) {
  LaneCodes<BITS> c;
  if constexpr (BITS == 3 && !TILED) {
    // canonical 3-bit: the lane's 32 codes are 12 bytes of the row's stream
    c.v[0] = u32x4{p[0], p[1], p[2], 0u};
  } else if constexpr (BITS == 4) {
    c.v[0] = *reinterpret_cast<const u32x4 *>(p);
  } else if constexpr (BITS == 8) {
    c.v[0] = *reinterpret_cast<const u32x4 *>(p);
    c.v[1] = *reinterpret_cast<const u32x4 *>(p2);
  } else if constexpr (BITS == 3) {
    const u32x2 t = *reinterpret_cast<const u32x2 *>(p);
    c.v[0] = u32x4{t[0], t[1], *p2, 0u};
  } else {
    const u32x2 t = *reinterpret_cast<const u32x2 *>(p);
    c.v[0] = u32x4{t[0], t[1], 0u, 0u};
  }
  return c;
}

// Operand of MFMA step t (codes 32h + 8t .. +7 of the group).
template <int BITS, bool TILED>
__device__ __forceinline__ bf16x8 codes_step(const LaneCodes<BITS> &c, int t) {
  if constexpr (BITS == 4) return as_bf16x8(TILED ? unpack8_b4_pair(c.v[0][t]) : unpack8_b4(c.v[0][t]));
  else if constexpr (BITS == 8) return as_bf16x8(unpack8_b8(c.v[t >> 1][(t & 1) * 2], c.v[t >> 1][(t & 1) * 2 + 1]));
  else if constexpr (BITS == 3 && !TILED) {
    // canonical: codes 8t .. 8t+7 are stream bits 24t .. 24t+23 of the lane's
    // three words; code 2p of the step at bit 6p, code 2p+1 at bit 6p+3
    const int b = 24 * t, j = b >> 5;
    const uint32_t hi = j + 1 < 3 ? c.v[0][j + 1] : 0u;
    const uint32_t v24 = __builtin_amdgcn_alignbit(hi, c.v[0][j], (uint32_t)(b & 31));
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a0 = v24 >> (6 * p);
      r[p] = (a0 & 7u) | ((a0 << 13) & 0x00070000u) | 0x43004300u;
    }
    return as_bf16x8(r);
  } else if constexpr (BITS == 3) {
    // low two bits as 2-bit codes, then the high bit of pair P = 4t + p (bits
    // P and 16 + P of the high-bit word) into bits 2 and 18: 128 + q
    u32x4 r = unpack8_b2_pair(c.v[0][t >> 1], t & 1);
#pragma unroll
    for (int p = 0; p < 4; ++p) r[p] = and_or(shift_right(c.v[0][2], 4 * t + p - 2), 0x00040004u, r[p]);
    return as_bf16x8(r);
  }
  else return as_bf16x8(TILED ? unpack8_b2_pair(c.v[0][t >> 1], t & 1) : unpack8_b2(c.v[0][t >> 1], t & 1));
}

// Rows of x per pitch-row in LDS; the pitch adds 16 bytes so rows start in
// different banks.
__host__ __device__ constexpr int x_pitch_bytes(int chunk_groups) { return chunk_groups * 128 + 16; }

// MR = accumulator registers of the 32x32 output used: register r of lane l
// holds row 8*(r/4) + 4*(l/32) + r%4, so MR=1 covers M=1 (row 0), MR=2 M<=2,
// MR=4 M<=8, MR=8 M<=16.
// Barrier for LDS traffic only: waits for this wave's LDS operations, not for
// its global loads, so prefetched code streams stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-lane ring slot: the codes of one group plus (tiled layout) its scale and
// bias bits, whose 32 lanes of a strip read one 128-byte line.
template <int BITS, bool TILED> struct Slot {
  LaneCodes<BITS> c;
  uint32_t sb;            // tiled: s | b << 16 ; unused for canonical
};

template <int BITS, int MR, int kRing, bool TILED, int XB, int SB, int kBatch>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void skinny_kernel(SkinnyArgs a, int chunk_groups) {
  constexpr int MPAD = MR <= 4 ? 8 : 16;  // row stride of the per-group row-sum table
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int xpitch = x_pitch_bytes(chunk_groups);
  unsigned char *x_lds = smem;
  float *xs_lds = reinterpret_cast<float *>(smem + ((a.M * xpitch + 15) / 16) * 16);
  // canonical layout: scale and bias bits of the block's 64 columns for the
  // chunk, [column][group] (s) followed by the same for b
  uint16_t *s_lds = reinterpret_cast<uint16_t *>(xs_lds + chunk_groups * MPAD);
  uint16_t *b_lds = s_lds + kStrips * 32 * chunk_groups;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, h = lane >> 5;
  const int strip = blockIdx.x * kStrips + wave / kKSplit;
  const int kpart = wave % kKSplit;
  const int64_t n0 = (int64_t)strip * 32;
  int64_t n = n0 + col;
  if (n >= a.N) n = a.N - 1;
  const int G = a.G;
  const bool arow = col < a.M;
  const float offset = CodeOffset<BITS>::value;
  // code stream of this lane: group g starts at wbase + g * gstride
  const int64_t nstrips = (a.N + 31) / 32;
  const int64_t strip_c = strip < nstrips ? strip : nstrips - 1;
  const uint32_t *wbase;
  const uint32_t *sbbase;  // tiled scale|bias words of (strip, col), group g at + 32*g
  int64_t gstride;
  int off2 = 0;
  if constexpr (TILED) {
    const int l = 32 * h + col;
    gstride = 64 * BITS;  // 32 columns x 2*BITS words
    wbase = a.w + strip_c * G * gstride + (BITS == 2 || BITS == 3 ? 2 * l : 4 * l);
    sbbase = a.sb + strip_c * G * 32 + col;
    off2 = BITS == 3 ? 128 - l : 256;  // 3-bit: high-bit word 128 + l of the block
  } else {
    gstride = 2 * BITS;
    wbase = a.w + n * (a.K * BITS / 32) + (BITS == 8 ? 8 * h : (BITS == 4 ? 4 * h : (BITS == 3 ? 3 * h : 2 * h)));
    sbbase = nullptr;
    off2 = 4;
  }
  auto load_g = [&](int g) {
    Slot<BITS, TILED> sl;
    const uint32_t *p = wbase + (int64_t)g * gstride;
    sl.c = load_codes<BITS, TILED>(p, p + off2);
    if constexpr (TILED) sl.sb = sbbase[32 * g];
    else sl.sb = 0;
    return sl;
  };

  float acc[MR];
#pragma unroll
  for (int r = 0; r < MR; ++r) acc[r] = 0.f;

  for (int c0 = 0; c0 < G; c0 += chunk_groups) {
    const int cg = min(chunk_groups, G - c0);
    const int q = (cg + kKSplit - 1) / kKSplit;
    const int g0 = c0 + kpart * q;
    const int g1 = min(c0 + cg, g0 + q);
    const bool active = g0 < g1;
    const int glast = active ? g1 - 1 : c0;

    // 1) activations of the chunk: issue all staging loads first (clamped, so
    //    every thread issues exactly XB of them) ...
    const int pieces = a.M * cg * 8;
    u32x4 xv[XB];
#pragma unroll
    for (int j = 0; j < XB; ++j) {
      const int i = min(tid + j * kThreads, pieces - 1);
      const int m = i / (cg * 8), rem = i % (cg * 8);
      xv[j] = *reinterpret_cast<const u32x4 *>(a.x + (int64_t)m * a.K + (int64_t)c0 * 64 + rem * 8);
    }
    // canonical layout: scale/bias of the block's 64 columns, as words of two
    // groups (G even) or single values, also issued before the code stream
    // two-group words need an even chunk and 4-byte aligned scale/bias rows
    const bool pairs = ((G | chunk_groups) & 1) == 0 &&
                       ((reinterpret_cast<uintptr_t>(a.s) | reinterpret_cast<uintptr_t>(a.b)) & 3u) == 0;
    const int sbw = pairs ? kStrips * 32 * ((cg + 1) / 2) : kStrips * 32 * cg;  // items per array
    uint32_t sv[TILED ? 1 : SB], bv[TILED ? 1 : SB];
    if constexpr (!TILED) {
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const int i = min(tid + j * kThreads, sbw - 1);
        const int per = sbw / (kStrips * 32);
        const int c = i / per, w = i % per;
        int64_t nn = (int64_t)blockIdx.x * kStrips * 32 + c;
        if (nn >= a.N) nn = a.N - 1;
        if (pairs) {
          sv[j] = *reinterpret_cast<const uint32_t *>(a.s + nn * G + c0 + 2 * w);
          bv[j] = *reinterpret_cast<const uint32_t *>(a.b + nn * G + c0 + 2 * w);
        } else {
          sv[j] = a.s[nn * G + c0 + w];
          bv[j] = a.b[nn * G + c0 + w];
        }
      }
    }
    // 2) ... then this wave's code stream (loads are unconditional, indices
    //    clamped, so the compiler counts outstanding loads exactly) ...
    Slot<BITS, TILED> ring[kRing];
#pragma unroll
    for (int u = 0; u < kRing; ++u) ring[u] = load_g(min(g0 + u, glast));
    // 3) ... and wait only for the staging loads (they are older than the ring).
    if (c0 > 0) lds_barrier();  // previous chunk fully consumed
#pragma unroll
    for (int j = 0; j < XB; ++j) {
      const int i = tid + j * kThreads;
      if (i < pieces) {
        const int m = i / (cg * 8), rem = i % (cg * 8);
        *reinterpret_cast<u32x4 *>(x_lds + m * xpitch + rem * 16) = xv[j];
      }
    }
    if constexpr (!TILED) {
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const int i = tid + j * kThreads;
        if (i < sbw) {
          const int per = sbw / (kStrips * 32);
          const int c = i / per, w = i % per;
          if (pairs) {
            const int gl = 2 * w;
            s_lds[c * chunk_groups + gl] = (uint16_t)(sv[j] & 0xFFFFu);
            b_lds[c * chunk_groups + gl] = (uint16_t)(bv[j] & 0xFFFFu);
            if (gl + 1 < cg) {
              s_lds[c * chunk_groups + gl + 1] = (uint16_t)(sv[j] >> 16);
              b_lds[c * chunk_groups + gl + 1] = (uint16_t)(bv[j] >> 16);
            }
          } else {
            s_lds[c * chunk_groups + w] = (uint16_t)sv[j];
            b_lds[c * chunk_groups + w] = (uint16_t)bv[j];
          }
        }
      }
    }
    lds_barrier();
    // per-group row sums of the staged activations, table [group][MPAD]
    for (int i = tid; i < cg * MPAD; i += kThreads) {
      const int gl = i / MPAD, m = i % MPAD;
      float sum = 0.f;
      if (m < a.M) {
        const unsigned char *p = x_lds + m * xpitch + gl * 128;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x4 v = *reinterpret_cast<const u32x4 *>(p + 16 * j);
#pragma unroll
          for (int e = 0; e < 4; ++e) sum += bf16_lo(v[e]) + bf16_hi(v[e]);
        }
      }
      xs_lds[i] = sum;
    }
    lds_barrier();

    auto process = [&](int g, const Slot<BITS, TILED> &sl) {
      const int gl = g - c0;
      uint16_t s16, b16;
      if constexpr (TILED) {
        s16 = (uint16_t)(sl.sb & 0xFFFFu);
        b16 = (uint16_t)(sl.sb >> 16);
      } else {
        const int cc = (wave / kKSplit) * 32 + col;
        s16 = s_lds[cc * chunk_groups + gl];
        b16 = b_lds[cc * chunk_groups + gl];
      }
      u32x4 xa[4];
      if (arow) {
        const unsigned char *p = x_lds + col * xpitch + gl * 128 + 64 * h;
#pragma unroll
        for (int t = 0; t < 4; ++t) xa[t] = *reinterpret_cast<const u32x4 *>(p + 16 * t);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) xa[t] = u32x4{0u, 0u, 0u, 0u};
      }
      f32x16 pacc = {};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(xa[t]), codes_step<BITS, TILED>(sl.c, t), pacc, 0, 0, 0);
      const float sf = f16_to_f32(s16);
      const float bf = __builtin_fmaf(-offset, sf, f16_to_f32(b16));
      const float *xsr = xs_lds + gl * MPAD + 4 * h;
      float xs[MR];
      if constexpr (MR >= 4) {
        const f32x4 v0 = *reinterpret_cast<const f32x4 *>(xsr);
#pragma unroll
        for (int r = 0; r < 4; ++r) xs[r] = v0[r];
        if constexpr (MR == 8) {
          const f32x4 v1 = *reinterpret_cast<const f32x4 *>(xsr + 8);
#pragma unroll
          for (int r = 0; r < 4; ++r) xs[4 + r] = v1[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < MR; ++r) xs[r] = xsr[r];
      }
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const float t = __builtin_fmaf(sf, pacc[r], acc[r]);
        acc[r] = __builtin_fmaf(bf, xs[r], t);
      }
    };

    if (active) {
      int g = g0;
      for (; g + kRing <= g1; g += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
          // consume the slot, then refill the same registers: a new load never
          // overlaps the old value, so the ring needs no register copies
          // (a copy of a load in flight would force a wait for it). Slots are
          // refilled kBatch at a time, back to back: on canonical rows the
          // loads of kBatch consecutive groups then share their cache lines
          // while the lines are still in the vector cache.
          process(g + u, ring[u]);
          __builtin_amdgcn_sched_barrier(0);
          if (u % kBatch == kBatch - 1) {
#pragma unroll
            for (int v = u + 1 - kBatch; v <= u; ++v) ring[v] = load_g(min(g + v + kRing, glast));
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kRing; ++u)
        if (g + u < g1) process(g + u, ring[u]);
    }
  }

  // cross-wave (K-quarter) reduction through LDS, fixed order
  lds_barrier();
  float *red = reinterpret_cast<float *>(smem);  // [kStrips*kKSplit][MR][64]
#pragma unroll
  for (int r = 0; r < MR; ++r) red[(wave * MR + r) * 64 + lane] = acc[r];
  lds_barrier();
  if (kpart == 0) {
    const int64_t nn = n0 + col;
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      float v = red[(wave * MR + r) * 64 + lane];
#pragma unroll
      for (int k = 1; k < kKSplit; ++k) v += red[((wave + k) * MR + r) * 64 + lane];
      const int row = 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < a.M && nn < a.N) {
        if (a.out_bf16) reinterpret_cast<uint16_t *>(a.out)[(int64_t)row * a.N + nn] = f32_to_bf16_rne_s(v);
        else reinterpret_cast<float *>(a.out)[(int64_t)row * a.N + nn] = v;
      }
    }
  }
}

template <int BITS, int MR, bool TILED>
hipError_t launch_mr(const SkinnyArgs &a, hipStream_t stream) {
  constexpr int MPAD = MR <= 4 ? 8 : 16;
  // rows of x this instantiation serves (MR=1: 1, MR=2: 2, MR=4: 8, MR=8: 16)
  constexpr int MMAX = MR == 1 ? 1 : (MR == 2 ? 2 : (MR == 4 ? 8 : 16));
  // staging loads of x per thread (16 bytes each), issued before the code
  // stream: 9 covers 8 rows x 72 groups; one-row shapes need 2
  constexpr int XB = MMAX <= 2 ? 2 : 9;
  // equal chunks of groups such that x and its row sums fit the LDS budget
  // and the staging loads
  // canonical scale/bias staging loads per thread: 9 covers 64 columns x 72
  // groups as two-group words (even G, 4-byte aligned scale/bias), 36 groups
  // as single values
  constexpr int SB = 9;
  const bool al = ((reinterpret_cast<uintptr_t>(a.s) | reinterpret_cast<uintptr_t>(a.b)) & 3u) == 0;
  const bool pairs = !TILED && a.G % 2 == 0 && al;
  const int sbytes = TILED ? 0 : kStrips * 32 * 2 * 2;  // LDS bytes of s and b per group
  int cmax = kXBudget / (int)(a.M * 128 + MPAD * 4 + sbytes);
  const int cstage = XB * kThreads / (int)(a.M * 8);
  if (cmax > cstage) cmax = cstage;
  if (!TILED) {
    const int csb = pairs ? 2 * SB * kThreads / (kStrips * 32) : SB * kThreads / (kStrips * 32);
    if (cmax > csb) cmax = csb;
  }
  if (pairs) cmax &= ~1;  // two-group words stay inside a chunk
  if (cmax < 1) cmax = 1;
  const int nchunks = (a.G + cmax - 1) / cmax;
  const int chunk = pairs ? 2 * ((a.G / 2 + nchunks - 1) / nchunks) : (a.G + nchunks - 1) / nchunks;
  const size_t xbytes = ((size_t)a.M * x_pitch_bytes(chunk) + 15) / 16 * 16;
  const size_t red = (size_t)kStrips * kKSplit * MR * 64 * 4;
  size_t lds = xbytes + (size_t)chunk * MPAD * 4 + (size_t)chunk * sbytes;
  if (lds < red) lds = red;
  // groups of codes kept in flight per lane, bounded so the kernel stays
  // within 128 VGPRs (4 waves per SIMD, 16 per CU). Measured at N = 27648,
  // K = 4608: 4 is the best depth at one or two rows for every code width
  // (4-bit, one row: 16 us against 19 us with 8, since the kernel's 3456
  // waves already keep ~14 MB of loads in flight); 5 at up to 8 rows, 3 at 16.
  constexpr int RING_T = BITS == 8 ? (MR == 8 ? 2 : 4) : (MR == 8 ? 3 : (MR == 4 ? 5 : 4));
  // canonical rows at one or two output rows: refill in batches of groups
  // that share 128-byte lines (3/4-bit: four groups, 8-bit: two), with a
  // deeper ring at one row so a batch is in flight while the other is
  // consumed. Measured at N = 27648, K = 4608, one row: 4-bit 24.4 -> 22.3 us,
  // 3-bit 24.6 -> 22.9, 8-bit 34.1 -> 33.1; 2-bit (16-byte groups) was
  // slower batched and keeps single refills.
  constexpr bool kBatched = !TILED && MR <= 2 && BITS != 2;
  constexpr int BATCH = !kBatched ? 1 : (MR == 1 ? (BITS == 8 ? 2 : 4) : 2);
  constexpr int RING = (kBatched && MR == 1 && BITS != 8) ? 8 : RING_T;
  static_assert(RING % BATCH == 0, "the ring refills whole batches");
  auto kern = skinny_kernel<BITS, MR, RING, TILED, XB, SB, BATCH>;
  // set on every launch (cheap; the library keeps no per-device state)
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
  if (e != hipSuccess) return e;
  const unsigned blocks = (unsigned)((a.N + 32 * kStrips - 1) / (32 * kStrips));
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kThreads), lds, stream, a, chunk);
  return hipGetLastError();
}

template <int BITS, bool TILED>
hipError_t launch_layout(const SkinnyArgs &a, hipStream_t stream) {
  if (a.M == 1) return launch_mr<BITS, 1, TILED>(a, stream);
  if (a.M == 2) return launch_mr<BITS, 2, TILED>(a, stream);
  if (a.M <= 8) return launch_mr<BITS, 4, TILED>(a, stream);
  return launch_mr<BITS, 8, TILED>(a, stream);
}

template <int BITS>
hipError_t launch_bits(const SkinnyArgs &a, hipStream_t stream) {
  return a.tiled ? launch_layout<BITS, true>(a, stream) : launch_layout<BITS, false>(a, stream);
}

}  // namespace

hipError_t launch_skinny(int bits, const SkinnyArgs &a, hipStream_t stream) {
  if (a.M > 16 || a.M < 1) return hipErrorInvalidValue;
  if (bits == 4) return launch_bits<4>(a, stream);
  if (bits == 8) return launch_bits<8>(a, stream);
  if (bits == 2) return launch_bits<2>(a, stream);
  if (bits == 3) return launch_bits<3>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace ql
