/*
 * qlinear.h -- C ABI of libqlinear, an MI355X (gfx950) group-wise affine
 * quantized linear layer.
 *
 *   y[m, n] = sum_k x[m, k] * W_hat[n, k]
 *   W_hat[n, k] = scale[n, g] * q[n, k] + bias[n, g],   g = k / 64
 *
 * The format -- unsigned codes q of 2, 3, 4 or 8 bits, one f16 scale and one f16
 * bias per 64 consecutive weights of a row, i.e. half a bit of overhead per
 * weight -- is the one described by the Ideogram-4-IQ4_M model card
 * (aimarketly.com; opening section and the section on what "IQ4" means) and
 * the SceneWorks/ideogram-4-mlx model card (huggingface.co; section
 * "Versions": group-wise affine Q4/Q8, group size 64, packed). 3-bit codes
 * serve the mixed-precision packs of the IQ4_M card (3-bit DiT bulk with
 * 8-bit modulation and conditioning; sections "Against the pack this
 * replaces" and "Conversion"). They run on every path: the skinny kernel
 * reads either layout; the GEMMs read the TILED layout, so a GEMM call on
 * canonical 3-bit weights first repacks them into the workspace (one extra
 * pass over the weights per call; repack once at load with qlinear_repack to
 * avoid it).
 *
 * Conventions for every entry point:
 *  - Pointers whose name ends in _host are host memory; all others are device
 *    memory (hipMalloc'ed or torch CUDA tensors). The caller owns every buffer;
 *    the library never frees caller memory.
 *  - Arrays are row-major and contiguous.
 *      x        bf16 bit patterns, [M, K]
 *      packed_q uint32, [N, K*bits/32]; each row is one little-endian bit
 *               stream along K: code k sits in stream bits
 *               [bits*k, bits*k + bits), stream bit i being bit i % 32 of
 *               word i / 32 (so 2/4/8-bit words hold 32/bits whole codes
 *               and 3-bit codes may straddle two words; the pages say only
 *               "packed", this is the layout this library fixes)
 *      scales   f16 bit patterns, [N, K/64]
 *      biases   f16 bit patterns, [N, K/64]
 *      out      fp32 [M, N] (or bf16 with QL_OUT_BF16 in the _ex form)
 *  - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *    Device entry points only enqueue work and return; they never
 *    synchronize. Errors found before launch are returned and nothing is
 *    launched.
 *  - Return value: QL_OK (0) or a negative ql_status. No entry point aborts,
 *    exits or throws.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QL_OK = 0,
  QL_EINVAL = -1,        /* bad size, null pointer, K not a multiple of 64  */
  QL_EALIGN = -2,        /* x / out / packed_q not 16-byte aligned            */
  QL_EUNSUPPORTED = -3,  /* bits not in {2,3,4,8}, group != 64, forced path
                            that cannot serve the shape                      */
  QL_EWORKSPACE = -4,    /* caller workspace missing or too small             */
  QL_EHIP = -5,          /* a HIP runtime call or kernel launch failed        */
  QL_ERANGE = -6         /* non-finite weight, or f16 overflow of scale/bias  */
} ql_status;

typedef enum { QL_OUT_F32 = 0, QL_OUT_BF16 = 1 } ql_out_dtype;

/*
 * Weight layouts. CANONICAL is the layout described at the top of this file.
 * TILED is this library's load-time repack into the kernels' lane order (see
 * qlinear_repack): for each strip of 32 output rows and each 64-wide group the
 * codes form one contiguous block (4-bit 1 KB, 8-bit 2 KB, 2-bit 512 B, 3-bit
 * 768 B: the low two bits as a 2-bit block, then a plane of high bits) and
 * the scale and bias become one uint32 (s | b << 16) per row and group, so a
 * wave's loads cover whole cache lines. Every path reads 2/4/8-bit codes in
 * either layout directly. The large-M GEMMs read 3-bit codes in the tiled
 * layout only: a GEMM call on CANONICAL 3-bit weights first writes a tiled
 * copy of them into the workspace (one pass over the weights per call; it
 * needs a workspace, and the path name ends in "_tiled_copy"). Repack 3-bit
 * weights once at load with qlinear_repack to avoid it.
 */
typedef enum { QL_LAYOUT_CANONICAL = 0, QL_LAYOUT_TILED = 1 } ql_layout;

/*
 * Numerics of the large-M GEMM path. Every mode computes the product with the
 * weights of the format above; they differ in how the weights meet the MFMA.
 * EXACT: codes enter the bf16 MFMA as exact integers and each group's scale
 *   and bias are applied to the fp32 accumulator; the only rounding is fp32
 *   accumulation (relative Frobenius error ~1e-6 against an fp64 product).
 *   Needs per-group row sums of x: K/64 * roundup(M, 256) floats of workspace
 *   unless the caller passes them (qlinear_group_sums, xsum).
 * SPLIT: each weight is dequantized in fp32 exactly as defined above,
 *   W = s*q + b (one rounding), split into two bf16 terms hi = bf16(W) and
 *   lo = bf16(W - hi) (round to nearest even; |W - hi - lo| <= 2^-16 |W|),
 *   and both terms go through the bf16 MFMA against bf16 x with fp32
 *   accumulation (relative Frobenius error ~1e-5). Reads x as given, needs no
 *   scratch unless K is split, and holds for any finite weights and x.
 * FAST: each weight is dequantized once per block tile to fp16 with a single
 *   rounding, W16 = fp16(s*q + b), and x enters as fp16 after scaling each
 *   row by the power of two 2^-e that brings its largest magnitude into
 *   [2^14, 2^15), exact for every scaled value of magnitude >= 2^-14 (every
 *   value within 2^28 of the row's largest); outputs are scaled back by 2^e
 *   and accumulated in fp32 on fp16 MFMA. The added error is the half-ulp of
 *   fp16 on W (relative Frobenius error ~2e-4 on normal weights). A column
 *   whose weights could reach the fp16 limit (max over its groups of
 *   max(|b|, |b + (2^bits - 1)*s|) >= 65504) has its fp16 weights scaled by
 *   a power of two 2^-c and its outputs by 2^c, so any finite f16 scale and
 *   bias are served (such a column's weights are then exact to one rounding
 *   relative to its largest magnitude). Runs on either layout (canonical
 *   2/4/8-bit codes of fewer than 2^31 code bytes; slower than tiled: strided
 *   code loads). The fp16 x comes from the caller (qlinear_fast_activations,
 *   x16/rowscale), else from a prepass into M*K*2 + M*4 workspace bytes, else
 *   (no workspace, no fused epilogue) from the GEMM itself: each block
 *   converts the bf16 x it stages in LDS to fp16 by truncation, with no row
 *   scale (exact for 2^-17 <= |x| <= 2^15; below 2^-17 the error is under
 *   2^-24 per value), and every block tile or row piece holding a row whose
 *   largest magnitude is above 2^15 (or not finite), or nonzero and below
 *   2^-6, is recomputed by a second launch with SPLIT numerics. Outputs of
 *   this form equal the prepass form's bit for bit wherever every nonzero
 *   |x| is at least 2^-17 and no tile is recomputed.
 * A K split (few output tiles, long K) adds splits*M*N*4 bytes of fp32
 *   partials to any mode's workspace.
 * AUTO: FAST (EXACT for canonical codes of 2^31 bytes or more). The skinny
 *   (M <= 16) path is always EXACT and needs no workspace. Without a
 *   workspace K is never split. A grid of fewer 256 x 256 tiles than CUs that
 *   is not split along K has every tile cut into the most row pieces (8, 4 or
 *   2: 32, 64 or 128 rows) that fit one round of blocks, whole tiles when even
 *   halves would not (long-K, few-row shapes run slower than with a
 *   workspace's K split).
 */
typedef enum { QL_MODE_AUTO = 0, QL_MODE_EXACT = 1, QL_MODE_FAST = 2, QL_MODE_SPLIT = 3 } ql_mode;

/*
 * Fused epilogues.
 * SWIGLU: the weight is a gate projection stacked on an up projection, rows
 *   [gate (F); up (F)], N = 2F with F a multiple of 16, repacked with
 *   qlinear_repack_glu. The call writes out[m, f] = silu(g) * u for
 *   f < F, where g = y[m, f], u = y[m, F + f] of the product y = x W^T and
 *   silu(g) = g / (1 + exp(-g)), in fp32 (bf16 out: one RNE rounding of that
 *   value); out is [M, F]. This is the SwiGLU MLP of the DiT block
 *   (Ideogram 4 paper notes, section 2.1 pipeline and section 2.8 table).
 *   Runs the FAST GEMM without a K split at any M; needs QL_LAYOUT_TILED,
 *   mode AUTO or FAST and path AUTO or GEMM, else QL_EUNSUPPORTED; N not a
 *   multiple of 32 is QL_EINVAL.
 * GATE_RESIDUAL: the gated residual update of a DiT block branch. The call
 *   writes out[m, n] = residual[m, n] + gate[m / gate_rows, n] * y[m, n]
 *   (integer division: rows m of one sample share its gate row), computed
 *   in fp32 as one fused multiply-add (bf16 out: one RNE rounding of it).
 *   residual is [M, N] with the dtype of out and may be out itself (in-place
 *   update of the residual stream); gate is fp32 [ceil(M / gate_rows), N],
 *   the tanh gate as the modulation projection emits it; gate_rows >= 1.
 *   This is the AdaLN gate of each DiT block, taken from the timestep
 *   embedding and applied to the attention-out and MLP-down projections
 *   (Ideogram 4 paper notes, section 2.1 pipeline; Ideogram-4-IQ4_M card,
 *   Conversion section: a per-layer scale and a tanh gate). Runs the FAST
 *   GEMM without a K split at any M, on tiled or canonical weights; a missing
 *   residual or gate or gate_rows < 1 is QL_EINVAL. With K == 0 the call
 *   copies residual to out.
 */
typedef enum { QL_EPI_NONE = 0, QL_EPI_SWIGLU = 1, QL_EPI_GATE_RESIDUAL = 2 } ql_epilogue;

typedef enum {
  QL_PATH_AUTO = 0,      /* dispatch table decides                            */
  QL_PATH_SKINNY = 1,    /* wavefront GEMV kernel, M <= 16                    */
  QL_PATH_GEMM = 2,      /* fused dequant-GEMM on bf16 MFMA, no K split       */
  QL_PATH_SPLITK = 3     /* fused dequant-GEMM with split K + ordered reduce  */
} ql_path;

/* Full-form arguments of qlinear_forward_ex. Zero-initialise, then fill. */
typedef struct ql_forward_args {
  const void *x;             /* bf16 [M, K]                                  */
  const uint32_t *packed_q;  /* uint32 [N, K*bits/32]                        */
  const void *scales;        /* f16 [N, K/group]                             */
  const void *biases;        /* f16 [N, K/group]                             */
  int bits;                  /* 2, 3, 4 or 8                                 */
  int group;                 /* 64                                           */
  int64_t M, N, K;
  void *out;                 /* [M, N] ([M, N/2] with QL_EPI_SWIGLU), dtype per out_dtype */
  int out_dtype;             /* ql_out_dtype                                 */
  void *workspace;           /* device scratch owned by the caller, or NULL:
                                NULL restricts the call to plans that need
                                no scratch (see qlinear_forward_ex)         */
  size_t workspace_bytes;    /* bytes at workspace; qlinear_workspace_bytes()
                                is enough for every plan of the shape       */
  int path;                  /* ql_path; QL_PATH_AUTO unless testing         */
  int split_k;               /* 0 = auto; >0 forces the K split count        */
  int tile;                  /* 0 = auto; >0 forces a GEMM tile id (tests)   */
  const float *xsum;         /* optional: per-group row sums of x from
                                qlinear_group_sums ([K/64, ld_xsum] fp32);
                                NULL = computed inside the call             */
  int64_t ld_xsum;           /* row pitch of xsum, >= qlinear_group_sums_ld(M) */
  int layout;                /* ql_layout. For QL_LAYOUT_TILED, packed_q holds
                                the tiled codes, scales the tiled scale|bias
                                words, and biases is ignored                */
  int mode;                  /* ql_mode; FAST and SPLIT need a large-M path
                                (AUTO with M > 16, GEMM or SPLITK), else
                                QL_EUNSUPPORTED; xsum is used by EXACT only,
                                x16/rowscale by FAST only                   */
  const void *x16;           /* optional, FAST only: fp16 [M, K] activations
                                and                                         */
  const float *rowscale;     /* [M] row scales from qlinear_fast_activations
                                for this x; both NULL = computed inside the
                                call (both or neither must be given)        */
  int epilogue;              /* ql_epilogue; QL_EPI_NONE = plain y           */
  const void *residual;      /* QL_EPI_GATE_RESIDUAL: [M, N], dtype of out   */
  const float *gate;         /* QL_EPI_GATE_RESIDUAL: fp32 [ceil(M/gate_rows), N] */
  int64_t gate_rows;         /* QL_EPI_GATE_RESIDUAL: output rows per gate row */
} ql_forward_args;

/*
 * y = x @ W_hat^T with W_hat defined above, fp32 out, default stream; the
 * call of the method's spec form (x, packed_q, scales, biases, bits,
 * group, M, N, K, out) on canonical weights.
 * M, N >= 0 (0 is a no-op), K >= 0 and a multiple of 64 (K == 0 writes zeros),
 * group must be 64. The call allocates no memory and uses no scratch: M <= 16
 * runs the skinny kernel (or the GEMV), larger M the FAST GEMM converting x
 * itself, without a K split (see ql_mode; few-tile shapes run as row
 * pieces). The library holds no buffers or other state between calls, so
 * concurrent calls on different streams are independent. The one case that
 * needs scratch, canonical 3-bit codes with M > 16 (tiled copy, see
 * ql_layout), returns QL_EWORKSPACE: use qlinear_forward_ex with a workspace,
 * or repack the weights.
 */
int qlinear_forward(const void *x, const uint32_t *packed_q, const void *scales,
                    const void *biases, int bits, int group, int64_t M, int64_t N,
                    int64_t K, float *out);

/* Same product with explicit stream, workspace, output dtype, layout, numerics
 * mode, fused epilogue and forced path (tests). Scratch comes only from
 * args->workspace, which the caller owns and sizes with
 * qlinear_workspace_bytes; the library never allocates device memory and
 * never synchronizes. With a NULL workspace automatic selection keeps to
 * plans that need none (no K split; FAST converts x inside the GEMM unless
 * FAST activations are passed); a request that still needs scratch (EXACT
 * without xsum, an epilogue without x16, a forced K split, canonical 3-bit
 * GEMMs) returns QL_EWORKSPACE before anything is launched.
 * Calls that share one workspace must not overlap in time. */
int qlinear_forward_ex(const ql_forward_args *args, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * call as qlinear_forward_ex, but its scratch is a fixed 64 MiB array inside
 * the library (qlinear_forward_noalloc_max_scratch() bytes, held on every
 * device that loads the library until the process ends) instead of a caller
 * workspace. args->workspace and args->workspace_bytes must be 0 (QL_EINVAL
 * otherwise). The plan is the one qlinear_forward_ex picks with a workspace;
 * a call whose plan needs more than the array (qlinear_forward_workspace_bytes
 * > the maximum, e.g. fp16 activations of more than 64 MiB) returns
 * QL_EWORKSPACE before anything is launched. Allocates nothing and never
 * synchronizes. Every call on one device uses that device's one array, which
 * keeps the last call's contents: calls that overlap in time on one device
 * (other streams, other threads) race on it and must be serialized by the
 * caller. Whatever must start at zero is cleared by a kernel on the call's
 * stream, so the call can be captured in a HIP graph.
 */
int qlinear_forward_noalloc(const ql_forward_args *args, void *stream);

/* Bytes of the fixed scratch array of qlinear_forward_noalloc (64 MiB). */
size_t qlinear_forward_noalloc_max_scratch(void);

/*
 * Per-group row sums of the activations, xsum[g, m] = sum_{k=64g}^{64g+63}
 * x[m, k] in fp32, written to xsum with row pitch ld_xsum (layout
 * [K/64, ld_xsum]). The fused kernels fold each group's bias in as
 * bias[n, g] * xsum[m, g] (the affine form W_hat = s*q + b of the
 * Ideogram-4-IQ4_M card's section on what "IQ4" means, summed per group).
 * Several projections of the same x (e.g. Q/K/V, gate/up) can share one call
 * by passing the result in ql_forward_args.xsum. ld_xsum must be at least
 * qlinear_group_sums_ld(M); the buffer holds (K/64) * ld_xsum floats.
 */
int qlinear_group_sums(const void *x, int64_t M, int64_t K, float *xsum, int64_t ld_xsum,
                       void *stream);

/* Minimum row pitch (floats) of a group-sum buffer for M rows. */
int64_t qlinear_group_sums_ld(int64_t M);

/*
 * FAST-mode activations (see ql_mode): for each row m of the bf16 [M, K]
 * input with largest magnitude mx = max_k |x[m,k]|, e = floor(log2 mx) - 14
 * clamped to [-126, 120] (e = 0 when mx = 0), so mx * 2^-e lies in
 * [2^14, 2^15); x16[m, k] = fp16(x[m, k] * 2^-e) (round to nearest even;
 * exact for scaled magnitudes >= 2^-14) and rowscale[m] = 2^e. x16 is [M, K] fp16 (16-byte
 * aligned), rowscale [M] fp32. Several projections of the same x (Q/K/V,
 * gate/up) can share one call by passing the results in ql_forward_args.
 * Returns QL_EINVAL for bad sizes or null pointers, QL_EALIGN for misaligned
 * x or x16.
 */
int qlinear_fast_activations(const void *x, int64_t M, int64_t K, void *x16, float *rowscale, void *stream);

/*
 * FAST-mode activations of an AdaLN-modulated input (Ideogram 4 paper notes,
 * section 2.1 pipeline: each DiT block takes an AdaLN scale, with its gate,
 * from the timestep embedding; Ideogram-4-IQ4_M card, Conversion section:
 * the modulation projection emits a per-layer scale and a tanh gate). The
 * pages give no formula; the reading taken is the zero-centred one, value
 * k of row m becomes x[m, k] * (1 + scale[m / scale_rows, k]) (integer
 * division: the rows of one sample share its scale row; no shift term).
 * This call applies it on the way into fp16: in fp32, t = 1 + scale (one
 * rounding) and v = x * t (one rounding), then the row maximum, exponent e
 * and x16 = fp16(v * 2^-e) exactly as qlinear_fast_activations does for v.
 * The gate half of the modulation is the QL_EPI_GATE_RESIDUAL epilogue.
 * scale is fp32 [ceil(M / scale_rows), K], 16-byte aligned; scale_rows >= 1.
 * Returns QL_EINVAL for bad sizes or null pointers, QL_EALIGN for misaligned
 * x, x16 or scale.
 */
int qlinear_fast_activations_adaln(const void *x, const float *scale, int64_t scale_rows, int64_t M, int64_t K,
                                   void *x16, float *rowscale, void *stream);

/* Bytes of device workspace that serve every qlinear_forward_ex call of this
 * shape with automatic path, tile and split, under any numerics mode, layout
 * or epilogue (an upper bound over the plans; for 3-bit codes it includes the
 * tiled copy of canonical weights). 0 for invalid arguments. */
size_t qlinear_workspace_bytes(int bits, int64_t M, int64_t N, int64_t K);

/* Bytes of workspace the call described by args needs when it is given a
 * workspace (args->workspace and args->workspace_bytes are not read): exact
 * for forced paths, tiles and splits as well, 0 when the plan needs none or
 * the arguments are invalid. */
size_t qlinear_forward_workspace_bytes(const ql_forward_args *args);

/* Number of uint32 words of packed codes for an [N, K] weight: N*K*bits/32. */
size_t qlinear_packed_words(int bits, int64_t N, int64_t K);

/* Host packer: q_host uint8 [N, K] with values < 2^bits -> packed_host
 * uint32 [N, K*bits/32]. QL_ERANGE if a code is out of range. */
int qlinear_pack_host(const uint8_t *q_host, int bits, int64_t N, int64_t K,
                      uint32_t *packed_host);

/* Host unpacker, inverse of qlinear_pack_host. */
int qlinear_unpack_host(const uint32_t *packed_host, int bits, int64_t N, int64_t K,
                        uint8_t *q_host);

/*
 * Host min/max round-to-nearest fit (the "candidate 0" fit of the
 * Ideogram-4-IQ4_M card's section on what "IQ4" means), per row and 64-group:
 *   scale = f16_rne((max - min) / (2^bits - 1))   (fp32 subtract and divide)
 *   bias  = f16_rne(min)
 *   q     = clamp(rint_half_even((w - bias) / scale), 0, 2^bits - 1)  in fp32,
 *           q = 0 where scale == 0.
 * w_host fp32 [N, K] -> q_host uint8 [N, K], s16_host/b16_host f16 [N, K/64].
 * QL_ERANGE for a non-finite weight or an f16 overflow of scale or bias.
 */
int qlinear_quantize_rtn_host(const float *w_host, int bits, int group, int64_t N,
                              int64_t K, uint8_t *q_host, uint16_t *s16_host,
                              uint16_t *b16_host);

/*
 * Device load-time quantizer: the same fit as qlinear_quantize_rtn_host,
 * byte-identical, writing packed codes directly (no dense transient beyond w).
 * The SceneWorks/ideogram-4-mlx card (section "Provenance & attribution")
 * describes its packer as byte-equivalent to load-time quantization; this is
 * that load-time path. w fp32 [N, K] -> packed_q [N, K*bits/32], scales and
 * biases f16 [N, K/64]. Non-finite input or f16 overflow sets *status_dev
 * (an int in device memory, may be NULL) to QL_ERANGE; it is never cleared,
 * so zero it before the call.
 */
int qlinear_quantize_rtn(const float *w, int bits, int group, int64_t N, int64_t K,
                         uint32_t *packed_q, uint16_t *scales, uint16_t *biases,
                         int *status_dev, void *stream);

/*
 * Device importance-weighted fit ("imatrix"), same storage as
 * qlinear_quantize_rtn. Per (row, 64-group) it minimises
 * sum_j importance[k_j] * (w_j - W_hat_j)^2, the error weighting of the
 * Ideogram-4-IQ4_M card (section on what "IQ4" means: importance is the
 * per-input-channel mean squared activation E[x^2]); the min/max RTN fit is
 * candidate 0 and is kept unless another candidate is strictly better, so
 * the fit is never worse than RTN by that objective. The other candidates
 * (weighted least-squares lines from 33 starting code sets) are this
 * library's search, decided in fp32 with one rounding per operation.
 * importance fp32 [K], finite and >= 0 (16-byte aligned), else
 * *status_dev = QL_EINVAL; non-finite weights or f16 overflow of the RTN fit
 * set QL_ERANGE, as for qlinear_quantize_rtn. *status_dev is never cleared.
 */
int qlinear_quantize_imatrix(const float *w, const float *importance, int bits, int group,
                             int64_t N, int64_t K, uint32_t *packed_q, uint16_t *scales,
                             uint16_t *biases, int *status_dev, void *stream);

/* Device dequantize (check path) of canonical-layout weights: W_hat fp32
 * [N, K], one rounding per value, bit-identical to fp32(scale)*q + fp32(bias).
 * Tiled weights go back to the canonical layout with qlinear_unrepack first. */
int qlinear_dequantize(const uint32_t *packed_q, const void *scales, const void *biases,
                       int bits, int group, int64_t N, int64_t K, float *w_out,
                       void *stream);

/* uint32 words of tiled codes for an [N, K] weight: ceil(N/32)*32*K*bits/32. */
size_t qlinear_tiled_words(int bits, int64_t N, int64_t K);

/* uint32 words of tiled scale|bias for an [N, K] weight: ceil(N/32)*32*K/64. */
size_t qlinear_tiled_sb_words(int64_t N, int64_t K);

/*
 * Device repack, canonical -> tiled (one-time, at load). Reads packed_q
 * [N, K*bits/32], scales and biases [N, K/64]; writes tiled_q
 * (qlinear_tiled_words) and tiled_sb (qlinear_tiled_sb_words). Rows past N in
 * the last strip are zero. A bijection on the rows < N: qlinear_unrepack
 * restores the canonical arrays bit for bit.
 */
int qlinear_repack(const uint32_t *packed_q, const void *scales, const void *biases, int bits,
                   int group, int64_t N, int64_t K, uint32_t *tiled_q, uint32_t *tiled_sb,
                   void *stream);

/*
 * Device repack of a stacked gate/up weight, rows [gate (N/2); up (N/2)],
 * canonical -> tiled in GLU order (strip j holds gate rows 16j .. 16j+15,
 * then up rows 16j .. 16j+15), for QL_EPI_SWIGLU. Same array sizes as
 * qlinear_repack; N must be a multiple of 32 (QL_EINVAL otherwise).
 */
int qlinear_repack_glu(const uint32_t *packed_q, const void *scales, const void *biases, int bits,
                       int group, int64_t N, int64_t K, uint32_t *tiled_q, uint32_t *tiled_sb,
                       void *stream);

/* Inverse of qlinear_repack_glu. */
int qlinear_unrepack_glu(const uint32_t *tiled_q, const uint32_t *tiled_sb, int bits, int group,
                         int64_t N, int64_t K, uint32_t *packed_q, void *scales, void *biases,
                         void *stream);

/* Device unrepack, tiled -> canonical (inverse of qlinear_repack). */
int qlinear_unrepack(const uint32_t *tiled_q, const uint32_t *tiled_sb, int bits, int group,
                     int64_t N, int64_t K, uint32_t *packed_q, void *scales, void *biases,
                     void *stream);

/* Static description of a status code. */
const char *qlinear_status_string(int status);

/* Name of the kernel/tile/split the calling thread's last forward launched,
 * NUL-terminated into buf. Returns QL_OK or QL_EINVAL. */
int qlinear_last_path(char *buf, size_t len);

/* Library ABI version (major*100 + minor). */
int qlinear_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
