/*
 * w4a8.h -- C ABI of the MI355X (gfx950) W4A8 linear layer: 4-bit group-quantized weights times
 * int8 group-quantized activations.
 *
 * The operation (from the pages this library is written from):
 *   - "cactus PR #697: SME2 acceleration for CQ4 matmul, prefill attention, and orthogonal
 *     embeddings", section "Quantized matmul": the M=1 GEMV runs a first phase that applies a
 *     Hadamard transform to the activations and quantizes them to int8 per group, then streams
 *     packed 4-bit weight nibbles; the M>1 GEMM produces raw int32 partials that are rescaled in
 *     a vector epilogue.  The review snippet of the per-group leaf contract in the same page
 *     defines the partial: for one group and one output channel, the int32 sum over the group
 *     of activation code times weight value, with activation scale and weight scale applied by
 *     the caller.
 *   - "TensorFold PR #3215: simd_qmm on Metal: X's group sums and half operands from a prepass",
 *     section "What this changes": one prepass per call writes the per-row per-group sums of X
 *     that the 4-bit affine (scale and bias per 64-group) weights need for their bias term.
 *   - "geistlib issue #500: native W*A8 int8 GEMM for prefill", sections "Design" and "Scope":
 *     one shared activation quantization feeding both GEMV and GEMM, and a load-time repack of
 *     the weights into the kernel's layout.
 *
 * Definitions used by every entry point (x is fp32 [m][k]; weight group == activation group G):
 *   rotation    (optional) normalized Walsh-Hadamard transform of each 128-wide block of a row,
 *               fp32 butterflies with span 1, 2, ..., 64, then one multiply by fp32(1/sqrt(128))
 *   xs[g][r]    = amax / 127 (IEEE fp32 divide), amax = max |x| over group g of row r (stored
 *                 group-major); it is 0 when amax == 0 and also when amax / 127 underflows to 0
 *                 (a group of subnormals with amax <= 63 * 2^-149)
 *   xq[r][k]    = round-half-even(x / xs) (IEEE fp32 divide) clamped to [-127, 127]; every code
 *                 of a group is 0 when its xs == 0 (a subnormal xs has few significant bits, so
 *                 x / xs can pass 127 and the clamp applies)
 *   xsum[g][r]  = sum of the group's xq (int32, group-major)
 *   D[r][n][g]  = sum over k in group g of xq[r][k] * w[n][k]        (exact int32)
 *                 w = q in [-8, 7] (SYM), u in [0, 15] (AFFINE), codebook[n][j] (CODEBOOK)
 *   y[r][n]     = sum over g of xs[g][r] * ( sw[n][g] * D[r][n][g] + bw[n][g] * xsum[g][r] )
 *                 bw = 0 except AFFINE (dequantized weight = sw * u + bw); fp32 result
 *
 * Conventions
 *   - Every data pointer is a DEVICE pointer owned by the caller, except the layout struct,
 *     which lives in host memory.  No entry point allocates, frees or keeps device memory, and
 *     none keeps state between calls apart from a per-device architecture check and a
 *     thread-local error message.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is enqueued
 *     on it and the call returns without synchronizing; faults of enqueued work surface at the
 *     caller's next synchronization.
 *   - Arguments are validated on the host before any device work.  On a non-OK status nothing
 *     was enqueued (except W4A8_ERR_HIP, which reports a failed launch) and w4a8_last_error()
 *     describes the problem.
 *   - Device pointers must be 16-byte aligned; `packed` must be 256-byte aligned.
 *   - There is no fallback path: a request the kernels do not cover returns an error.
 *   - The current device must be an MI355X-class gfx950 GPU, else W4A8_ERR_DEVICE.
 */
#ifndef W4A8_H
#define W4A8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A8_OK = 0,
    W4A8_ERR_ARG = 1,          /* an argument is invalid (null, size, alignment, combination) */
    W4A8_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels implement               */
    W4A8_ERR_DEVICE = 3,       /* no device, or the current device is not gfx950             */
    W4A8_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed                 */
} w4a8_status;

typedef enum {
    W4A8_SYM_I4 = 0,       /* two's-complement 4-bit q in [-8, 7], fp16 scale per group       */
    W4A8_AFFINE_U4 = 1,    /* unsigned 4-bit u in [0, 15], fp16 scale and fp16 bias per group */
    W4A8_CODEBOOK_I4 = 2,  /* 4-bit index into a per-output-row 16-entry int8 codebook,
                              fp16 scale per group (PR #697's CQ4 codebook format)           */
    W4A8_INT8 = 3,         /* signed int8 weight, fp16 scale per group (W8A8: "geistlib issue
                              #500", sections "Scope" and "Design sketch"); codes are int8
                              [n][k], one byte per weight                                    */
    W4A8_CQ2 = 4,          /* 2-bit index into a per-output-row 4-entry int8 codebook, fp16
                              scale per group (CQ2 of PR #697's CQ1-CQ4 family; W2A8); codes
                              are uint8 [n][k/4], the index of k = 4b + i in bits 2i, 2i+1 of
                              byte b; codebook int8 [n][4]                                   */
    W4A8_CQ1 = 5,          /* 1-bit index into a per-output-row 2-entry int8 codebook, fp16
                              scale per group (CQ1); codes are uint8 [n][k/8], the index of
                              k = 8b + i in bit i of byte b; codebook int8 [n][2]            */
    W4A8_CQ3 = 6           /* 3-bit index into a per-output-row 8-entry int8 codebook, fp16
                              scale per group (CQ3); codes are uint8 [n][k], one index per
                              byte in its low 3 bits (the high bits are ignored); codebook
                              int8 [n][8]                                                    */
    /* W4A8_INT8 and the CQ1-CQ3 formats run through w4a8_gemv / w4a8_gemm / w4a8_linear (no
       fused one-row kernel); the gated, greedy-tail, partials and fp16-activation entry points
       return W4A8_ERR_UNSUPPORTED for them. */
} w4a8_format;

/* Rows of the packed weight buffer come in panels of this many output channels. */
#define W4A8_PANEL_ROWS 64

/*
 * Description of one packed weight buffer (host struct, filled by w4a8_packed_layout).
 *
 * Packed buffer (all offsets in bytes from the 256-byte aligned base, each section 256-aligned):
 *   codes     at off_codes: n_pad/64 panels; each panel is k/32 chunk columns; each chunk column
 *             is 64 rows x 16 bytes.  The 16 bytes of (row n, chunk c) hold the 32 codes of
 *             k = 32c .. 32c+31 as four dwords; dword j, byte b holds the code of k = 32c+4j+b in
 *             its low nibble and of k = 32c+16+4j+b in its high nibble.  SYM stores q's
 *             two's-complement nibble, AFFINE stores u XOR 8 (= u - 8 as a signed nibble),
 *             CODEBOOK stores the index.
 *   meta      at off_meta: per panel, per block j of 4 groups (ceil((k/group)/4) blocks), per
 *             panel row: the 4 entries of groups 4j .. 4j+3, meta_bytes bytes each (entries
 *             past the last group are zero).  SYM and CODEBOOK: the fp16 scale.  AFFINE: a
 *             dword, fp16 scale in the low half and fp16 bias in the high half.  A row's block
 *             is one 8- or 16-byte load.
 *   codebook  at off_codebook (CODEBOOK only): int8 [n_pad][16].
 * INT8, CQ2, CQ1 and CQ3 keep the panels and the meta section (SYM's) and change the codes:
 *   INT8: chunk column c holds w[n][16c .. 16c+15];  CQ2: chunk column c holds 64 k;
 *   CQ1 / CQ3: each 128 k (k padded to a multiple of 128) is 1 / 3 chunk columns in a row.
 *   Their codebooks at off_codebook: CQ2 and CQ1 one dword per row (entries in its bytes), CQ3
 *   two.  The exact bit order inside a chunk is the kernels' own (the packer writes it).
 * Rows n >= n of the padded last panel hold zero codes, zero scales and zero codebooks.
 */
typedef struct {
    int32_t format;       /* w4a8_format                                   */
    int32_t n;            /* output channels                               */
    int32_t k;            /* input channels                                */
    int32_t group;        /* 64 or 128; k % group == 0                     */
    int32_t n_pad;        /* n rounded up to a multiple of W4A8_PANEL_ROWS */
    int32_t meta_bytes;   /* 2 (SYM, CODEBOOK) or 4 (AFFINE)               */
    uint64_t bytes;       /* total size of the packed buffer               */
    uint64_t off_codes;
    uint64_t off_meta;
    uint64_t off_codebook;  /* 0 and unused unless a codebook format       */
} w4a8_layout;

/*
 * Fill *L for a weight of `n` output channels and `k` input channels.  Host only, no device
 * call.  Requires format in w4a8_format, group in {64, 128}, 1 <= n <= 2^24, group <= k <= 2^20,
 * k % group == 0.  Source: "geistlib issue #500", section "Design" (load-time repack into the
 * inner kernel's layout).
 */
w4a8_status w4a8_packed_layout(int32_t format, int32_t n, int32_t k, int32_t group,
                               w4a8_layout *L);

/*
 * Repack canonical weights into the layout described by L (a pure permutation of nibbles plus
 * the AFFINE re-encode u -> u XOR 8; scales, bias and codebook are copied).
 *   codes      uint8 [n][k/2]: two codes per byte, the low nibble holds the even k (4-bit
 *              formats); the w4a8_format comments give INT8's and the CQ formats' shapes
 *   scales_f16 uint16 [n][k/group] (IEEE binary16 bit patterns)
 *   bias_f16   uint16 [n][k/group] for AFFINE, else must be NULL
 *   codebook   int8 [n][16] for CODEBOOK, [n][4] CQ2, [n][2] CQ1, [n][8] CQ3, else NULL
 *   packed     L->bytes of device memory, written completely (padding included)
 * Source: "cactus PR #697", follow-up commits on the interleaved lm_head and on the single
 * runtime weight format (one packed format read by every kernel, built once at load).
 */
w4a8_status w4a8_pack_weights(const w4a8_layout *L, const uint8_t *codes,
                              const uint16_t *scales_f16, const uint16_t *bias_f16,
                              const int8_t *codebook, void *packed, void *stream);

/*
 * w4a8_pack_weights for weights with one scale (and, AFFINE, one bias) per output row: the row's
 * value is seen as the scale of each of its K / L->group groups, so every kernel computes
 *   y[r][n] = s[n] * sum_g xs[r][g] * D[r][n][g]   (+ b[n] * sum_g xs[r][g] * xsum[r][g], AFFINE)
 * and the packed buffer is the one w4a8_pack_weights writes from scales repeated over the groups.
 *   row_scales_f16  uint16 [n] (IEEE binary16 bit patterns)
 *   row_bias_f16    uint16 [n] for AFFINE, else must be NULL
 *   codes, codebook, packed, errors: as w4a8_pack_weights
 * Source: "cactus PR #697", the lm_head commit (the orthogonal lm_head keeps one scale per row and
 * views it as K/128 groups of 128, which is exact because a group's partial is an integer and its
 * weight scale a constant of the row).
 */
w4a8_status w4a8_pack_weights_row_scale(const w4a8_layout *L, const uint8_t *codes,
                                        const uint16_t *row_scales_f16,
                                        const uint16_t *row_bias_f16, const int8_t *codebook,
                                        void *packed, void *stream);

/*
 * The activation prepass: optional rotation, then per-row per-group int8 quantization and
 * group sums (definitions above).
 *   x       fp32 [m][k] row-major (not modified)
 *   xq      int8 [m][k] row-major
 *   xs      fp32 [k/group][m] (group-major: one group's scales for all rows are contiguous)
 *   xsum    int32 [k/group][m] (group-major)
 *   hadamard_block  0 (no rotation) or 128 (requires k % 128 == 0)
 * m == 0 is a no-op (the pointers may then be NULL).  Bit-exact: the same fp32 operations in the same order for each value as
 * the definition.  Sources: "cactus PR #697", section "Quantized matmul" (Hadamard + int8
 * activation quantization as the GEMV's first phase; 128-wide groups of the orthogonal
 * lm_head); "TensorFold PR #3215", section "What this changes" (group sums from a prepass).
 */
w4a8_status w4a8_prep(const float *x, int32_t m, int32_t k, int32_t group,
                      int32_t hadamard_block, int8_t *xq, float *xs, int32_t *xsum,
                      void *stream);

/*
 * Decode GEMV (one activation row): y[n] for n < L->n (definitions above).
 *   xq int8 [k], xs fp32 [k/group], xsum int32 [k/group] from w4a8_prep with L->group
 *   y  fp32 [L->n]
 * Source: "cactus PR #697", section "Quantized matmul" (hybrid fused GEMV, M=1, streaming
 * packed nibbles).
 */
w4a8_status w4a8_gemv(const w4a8_layout *L, const void *packed, const int8_t *xq,
                      const float *xs, const int32_t *xsum, float *y, void *stream);

/*
 * Prefill GEMM: y[r][n] for r < m, n < L->n (definitions above).
 *   xq int8 [m][k], xs fp32 [k/group][m], xsum int32 [k/group][m] from w4a8_prep
 *   y  fp32 [m][L->n]
 * m == 0 is a no-op (xq, xs, xsum and y may then be NULL).  W4A8_ERR_UNSUPPORTED when
 * m * (k/group + 16) * 4 bytes exceed 2^31 - 16.  The int32 group partials are exact; the fp32
 * sum over groups has a fixed order for given shapes and device (repeated calls give the same
 * bits), but tiles of a last, partial round over the device's CUs add their k quarters
 * separately, so the order (and the last bits) can depend on the CU count and on n and m.
 * Source: "cactus PR #697", section "Quantized matmul" (fused GEMM, M>1, raw int32 partials
 * rescaled per tile); "geistlib issue #500" (native int8 GEMM for prefill).
 */
w4a8_status w4a8_gemm(const w4a8_layout *L, const void *packed, int32_t m, const int8_t *xq,
                      const float *xs, const int32_t *xsum, float *y, void *stream);

/*
 * The whole hot path of one linear layer: the prepass of x (as w4a8_prep with L->group), then
 * the GEMV (m == 1) or the GEMM (m > 1).
 *   x               fp32 [m][L->k] row-major (not modified)
 *   hadamard_block  0 or 128, as for w4a8_prep
 *   xq, xs, xsum    the prepass outputs, laid out as for w4a8_prep (written; the GEMM reads them)
 *   y               fp32 [m][L->n]
 * m == 1 with L->k <= 16384 and L->n <= 262144 (131072 with hadamard_block 128) runs one
 * kernel: every workgroup of the GEMV quantizes the row itself into LDS with the prepass's
 * arithmetic (so xq, xs and xsum are the same bits as w4a8_prep's), which removes a launch from
 * each decode layer.  Otherwise the prepass kernel and then the GEMV or GEMM kernel are enqueued
 * on the stream.  m == 0 is a no-op (the pointers may then be NULL).
 * Source: "cactus PR #697", section "Quantized matmul" (the fused GEMV's first phase is the
 * Hadamard rotation and int8 quantization of the activations).
 */
w4a8_status w4a8_linear(const w4a8_layout *L, const void *packed, int32_t m, const float *x,
                        int32_t hadamard_block, int8_t *xq, float *xs, int32_t *xsum, float *y,
                        void *stream);

/* Activation of the gated output (w4a8_linear_glu). */
typedef enum {
    W4A8_ACT_SILU = 0,      /* v / (1 + e^-v) */
    W4A8_ACT_GELU_TANH = 1, /* v/2 * (1 + tanh(sqrt(2/pi) * (v + 0.044715 v^3))) */
    W4A8_ACT_GELU_ERF = 2   /* v/2 * (1 + erf(v / sqrt(2))) */
} w4a8_act;

/*
 * A gated feed-forward input in one call: sibling gate and up projections packed as one weight
 * matrix of L->n = 2F rows (gate rows 0..F-1, then up rows F..2F-1; F a multiple of 64, so
 * L->n % 128 == 0), one prepass of x shared by both, and
 *   y[r][f] = act(gate[r][f]) * up[r][f],  f < F,
 * written instead of the two halves.  gate and up are the fp32 outputs w4a8_linear computes
 * for those rows; act and the product are fp32 (device expf, tanhf, erff).
 *   x, hadamard_block, xq, xs, xsum  as for w4a8_linear (xq, xs and xsum are written)
 *   act   a w4a8_act
 *   y     fp32 [m][L->n / 2]
 * m == 1 with L->k <= 16384 and L->n <= 262144 (131072 with hadamard_block 128) runs one kernel
 * (the prepass fused, as for w4a8_linear); otherwise the prepass kernel, then the gated GEMV or GEMM.  m == 0 is a no-op.
 * W4A8_ERR_ARG: L->n % 128 != 0, or act not a w4a8_act.  W4A8_ERR_UNSUPPORTED: the span from a
 * gate row to its up row in the packed codes or metadata ((L->n / 2 + 64) rows) exceeds
 * 2^31 - 16 bytes, or as for w4a8_gemm.
 * Source: "cactus-compute/engine PR #750: Metal Support", the commit list (a gelu-gated
 * feed-forward pair fused into one GEMV; sibling quantized GEMVs batched into one; gelu-erf
 * and sigmoid activation codes); "geistlib issue #500", section "Design" (paired linears share
 * one activation prepass).
 */
w4a8_status w4a8_linear_glu(const w4a8_layout *L, const void *packed, int32_t m, const float *x,
                            int32_t hadamard_block, int32_t act, int8_t *xq, float *xs,
                            int32_t *xsum, float *y, void *stream);

/*
 * The gated output from prepared activations (the second half of w4a8_linear_glu):
 *   xq int8 [m][k], xs fp32 [k/group][m], xsum int32 [k/group][m] from w4a8_prep
 *   act   a w4a8_act
 *   y     fp32 [m][L->n / 2] = act(gate) * up, as for w4a8_linear_glu
 * m == 1 runs the gated GEMV, m > 1 the gated GEMM; m == 0 is a no-op.  Errors as for
 * w4a8_linear_glu.  Source: as for w4a8_linear_glu.
 */
w4a8_status w4a8_gemm_glu(const w4a8_layout *L, const void *packed, int32_t m, const int8_t *xq,
                          const float *xs, const int32_t *xsum, int32_t act, float *y,
                          void *stream);

/*
 * The greedy tail of a vocabulary head for one activation row: its logits, optionally
 * soft-capped, and the index of their maximum, with the maximum found on the GPU.
 *   x        fp32 [L->k] (one row, not modified)
 *   hadamard_block, xq, xs, xsum  as for w4a8_linear with m = 1 (xq, xs, xsum are written)
 *   softcap  c > 0: logits = c * tanh(y / c); c == 0: logits = y (y as w4a8_gemv computes it)
 *   logits   fp32 [L->n] (written)
 *   token    int32 [1]: the smallest index of the largest logit (written)
 *   value    fp32 [1]: that logit (written)
 *   work, work_bytes  device scratch of at least W4A8_ARGMAX_WORK_BYTES(L->n) bytes, 8-byte
 *            aligned: one 64-bit key per 64-row panel (no initial contents are needed; calls
 *            that overlap on one work buffer race)
 * The kernels on the stream: the GEMV, which also caps and stores the logits and stores each
 * panel's largest (logit, smaller index) key to work, with the prepass fused into it within the
 * bounds where w4a8_linear fuses it (k <= 16384 and at most 4096 panels, 2048 with the rotation;
 * workgroup 0 writes xq, xs and xsum) and a prepass kernel before it otherwise; then a
 * one-workgroup kernel that reduces the keys into token and value.  The results are the same
 * bits either way.  A one-scale-per-row head (the orthogonal lm_head) is packed with that scale
 * repeated over its 128-wide groups (group = 128): the same formula.
 * W4A8_ERR_ARG: softcap negative or not finite, token / value / work NULL or misaligned,
 * work_bytes too small.
 * Source: "cactus-compute/engine PR #750: Metal Support", the commit list (the orthogonal lm_head
 * with its softcap fused into the GPU argmax / sampling tail) and its file table (GPU-side
 * sampling and argmax helpers); "cactus PR #697", the lm_head commit (the virtual 128-wide group
 * view of one scale per row).
 */
#define W4A8_ARGMAX_WORK_BYTES(n) ((((uint64_t)(n) + 63u) / 64u) * 8u)

w4a8_status w4a8_lm_head_argmax(const w4a8_layout *L, const void *packed, const float *x,
                                int32_t hadamard_block, float softcap, int8_t *xq, float *xs,
                                int32_t *xsum, float *logits, int32_t *token, float *value,
                                void *work, uint64_t work_bytes, void *stream);

/*
 * w4a8_lm_head_argmax for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same validation, the same
 * kernels and the same results, with the panel keys in a buffer the library holds on each
 * GPU it runs on (W4A8_ARGMAX_WORK_BYTES(W4A8_NOALLOC_MAX_N) = 128 KiB, kept until the process
 * ends) instead of a caller's work buffer.  Nothing is allocated or freed: the buffer is a static
 * device array whose address is looked up once per device, on the first call there.
 *   every argument  as for w4a8_lm_head_argmax (there is no work buffer)
 * The keys need no initial contents.  Every call on one GPU shares that GPU's key buffer: calls
 * that overlap on one GPU (concurrent streams, or threads) race and may return a wrong token.
 * W4A8_ERR_UNSUPPORTED: L->n > W4A8_NOALLOC_MAX_N.  W4A8_ERR_HIP: the buffer's address lookup
 * failed.  Other errors as w4a8_lm_head_argmax.
 */
#define W4A8_NOALLOC_MAX_N (1 << 20)

w4a8_status w4a8_lm_head_argmax_noalloc(const w4a8_layout *L, const void *packed,
                                        const float *x, int32_t hadamard_block, float softcap,
                                        int8_t *xq, float *xs, int32_t *xsum, float *logits,
                                        int32_t *token, float *value, void *stream);

/*
 * The GEMV and greedy tail of w4a8_lm_head_argmax on activations already quantized by w4a8_prep
 * (m = 1): the GEMV with the tail and the key reduction, with the same logits, token and value.
 * Errors as w4a8_gemv and w4a8_lm_head_argmax.
 * Source: as w4a8_lm_head_argmax.
 */
w4a8_status w4a8_gemv_argmax(const w4a8_layout *L, const void *packed, const int8_t *xq,
                             const float *xs, const int32_t *xsum, float softcap, float *logits,
                             int32_t *token, float *value, void *work, uint64_t work_bytes,
                             void *stream);

/*
 * The fp16-activation path (W4A16): the same packed 4-bit weights times activations rounded to
 * binary16, with the affine bias term on fp32 group sums of the activations:
 *   y[r][n] = sum_g ( sw[n][g] * sum_{k in g} w_int[n][k] * xh[r][k] + bw[n][g] * S[r][g] )
 * where w_int is q (SYM) or the unsigned u (AFFINE), xh = binary16(x) rounded to nearest even,
 * and S[r][g] = ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)) in fp32, c_o the left-to-right fp32 sum of
 * the group's inputs 8o .. 8o+7.  Groups are 64 wide (L->group == 64).
 *
 * w4a8_prep_a16: the prepass.
 *   x     fp32 [m][k] row-major, 16-byte aligned (not modified); k % 64 == 0
 *   xh    binary16 [m][k], 16-byte aligned (written) in an interleaved order: within every
 *         32-wide block of a row, element 8j + h holds input k = {4j, 4j+2, 16+4j, 18+4j, 4j+1,
 *         4j+3, 17+4j, 19+4j}[h] of the block (j = 0..3)
 *   xsf   fp32 [k/64][m] group-major (written)
 *   W4A8_ERR_ARG: m < 0, group != 64, k not a positive multiple of 64 up to 2^20, NULL or
 *   misaligned pointers.  W4A8_ERR_UNSUPPORTED: m * k * 2 above 2^31 - 16.
 * w4a8_linear_a16: the prepass, then the GEMV (m == 1) or the GEMM (m > 1) on its outputs.
 *   packed, L  SYM or AFFINE with group 64 (CODEBOOK: W4A8_ERR_UNSUPPORTED)
 *   x, xh, xsf as for w4a8_prep_a16 (xh and xsf are written); y fp32 [m][L->n] (written)
 * w4a8_gemm_a16: the GEMV / GEMM alone on xh and xsf from w4a8_prep_a16.
 * Source: "TensorFold PR #3215, simd_qmm on Metal: X's group sums and half operands from a
 * prepass", section "What this changes" (the half tiles, the prepass writing X as half and the
 * group sums, the sums' fixed tree) and the "Perf" section (4-bit affine g64 weights, 128-row
 * prompt tiles).
 */
w4a8_status w4a8_prep_a16(const float *x, int32_t m, int32_t k, int32_t group, uint16_t *xh,
                          float *xsf, void *stream);
w4a8_status w4a8_linear_a16(const w4a8_layout *L, const void *packed, int32_t m, const float *x,
                            uint16_t *xh, float *xsf, float *y, void *stream);
w4a8_status w4a8_gemm_a16(const w4a8_layout *L, const void *packed, int32_t m,
                          const uint16_t *xh, const float *xsf, float *y, void *stream);

/*
 * Prefill attention over the cached int8 key/value segment of a prefill chunk.
 *
 * Cache (canonical input): for nkvh key/value heads and nkv slots of head dimension d (64, 128
 * or 256): k8, v8 int8 [nkvh][nkv][d]; ks, vs fp32 [nkvh][nkv][d/32] (one scale per 32 of the
 * head dimension); kvpos int32 [nkv], the position held by each slot (-1: empty; slots need not
 * be in position order, as in a rolled sliding-window ring).
 * Queries: q fp32 [nh][nq][d], nh a multiple of nkvh (query head h reads cache head
 * h / (nh / nkvh)); query i sits at position pos0 + i.
 * A slot at position p is seen by the query at t when p >= 0, p <= t, and window == 0 (a global
 * layer) or p < sink (attention sinks) or t - p < window.
 * Method: q8 = round-half-even(q / sq) clamped to [-127, 127], sq = max|q row| / 127 (one scale
 * per query row; q8 = 0 when sq == 0, as in the activation quantization); keys to
 * one flat scale per vector, sk = max_g ks[g], kq = round-half-even(k8 * fp32(ks[g] / sk));
 * logits S = scale * sq * sk * (q8 . kq); over blocks of 64 slots in slot order, an online
 * softmax m' = max(m, block max), alpha = e^(m - m'), P = e^(S - m'), l = alpha * l + sum P;
 * per value group g of 32 dims, P'_j = P_j * vs[j][g] quantized to u = round(P'_j / sp) in
 * 0..255 with sp = max_j P' / 255 per (query, group, block), and O_g = alpha * O_g +
 * sp * sum_j u_j * v8[j].  Results: the unnormalized O [nh][nq][d], m, l [nh][nq] (m = -inf,
 * l = 0, O = 0 for a query that sees no slot): the state a following new-token segment
 * continues from; O / l is the attention output over the cached segment.
 *
 * w4a8_attn_layout_init: host only; d in {64, 128, 256}, 1 <= nkvh, 1 <= nkv <= 2^24.
 * w4a8_attn_pack_kv: repack the canonical cache into AL->bytes of device memory (256-byte
 *   aligned): keys requantized to their flat scales ([nkvh][nblk*64][d], slot order); per block
 *   of 64 slots the values transposed ([d][64]), the slots' scales, positions (-1 past nkv) and
 *   value-group scales ([d/32][64]), all with slot jj of the block at index 32t + 16h + 4(r/8) +
 *   r%4 (t = jj/32, r = jj%32, h = (r/4)%2: the order the matrix-core output holds them), and
 *   each column's sum of the block's value codes.
 * w4a8_attn_work_bytes: the bytes of device scratch w4a8_attn_prefill needs for (nh, nq)
 *   (0 when the slot range is not split).
 * w4a8_attn_prefill: q8 int8 [nh][nq][d] and sq fp32 [nh][nq] (the query codes, written), o, m,
 *   l (written), work (w4a8_attn_work_bytes of scratch, 16-byte aligned, contents irrelevant;
 *   may be NULL when that is 0).  W4A8_ERR_ARG: nh not a positive multiple of AL->nkvh, nq < 0,
 *   pos0 / window / sink negative, scale not positive and finite, NULL or misaligned pointers,
 *   work_bytes too small.
 * Source: "cactus PR #697", section "Prefill attention" (and its test list: the attention
 * differential against a double-precision oracle, global and sliding-window layers, a rolled
 * cache with the sink exemption live, partial query tiles and key blocks).
 */
typedef struct w4a8_attn_layout {
    int32_t nkvh, nkv, d, nblk;   /* nblk = ceil(nkv / 64) */
    uint64_t bytes;               /* total size of the packed cache */
    uint64_t off_kq, off_sk, off_pos, off_vt, off_sv, off_vsum;
} w4a8_attn_layout;

w4a8_status w4a8_attn_layout_init(int32_t nkvh, int32_t nkv, int32_t d, w4a8_attn_layout *AL);
w4a8_status w4a8_attn_pack_kv(const w4a8_attn_layout *AL, const int8_t *k8, const float *ks,
                              const int8_t *v8, const float *vs, const int32_t *kvpos,
                              void *packed, void *stream);
uint64_t w4a8_attn_work_bytes(const w4a8_attn_layout *AL, int32_t nh, int32_t nq);
w4a8_status w4a8_attn_prefill(const w4a8_attn_layout *AL, const void *packed, const float *q,
                              int32_t nh, int32_t nq, int32_t pos0, int32_t window, int32_t sink,
                              float scale, int8_t *q8, float *sq, float *o, float *m, float *l,
                              void *work, uint64_t work_bytes, void *stream);

/*
 * The exact int32 partials D[r][n][g] (definitions above) written by the same kernel code as
 * the GEMV (m == 1) or the GEMM (m > 1) of the layout's format (the 4-bit formats' kernels, or
 * those of the int8 and CQ1-CQ3 weights), with the fp32 epilogue replaced by a store of D.
 *   xsum  as from w4a8_prep (the AFFINE partial is recovered from the u - 8 codes as
 *         D_u = D_(u-8) + 8 * xsum; the one-row CQ1 GEMV forms D = e0 * xsum + (e1 - e0) *
 *         (sum of the codes whose bit is set); the other formats do not read it, but it must
 *         be given)
 *   d     int32 [m][L->n][k/group]
 * Source: "cactus PR #697", review snippet of the per-group leaf contract.
 */
w4a8_status w4a8_debug_partials(const w4a8_layout *L, const void *packed, int32_t m,
                                const int8_t *xq, const int32_t *xsum, int32_t *d,
                                void *stream);

/* A static English name for a status code. */
const char *w4a8_status_string(w4a8_status s);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char *w4a8_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A8_H */
