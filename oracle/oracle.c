/*
 * oracle.c -- plain, slow, obviously-correct CPU definition of the W4A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file: only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It shares
 * no code, header, table or constant with the HIP library, and includes nothing from it.
 *
 * What it computes (sources are the four pages this project is written from):
 *
 *   rotation   "cactus PR #697, SME2 acceleration for CQ4 matmul, prefill attention, and
 *              orthogonal embeddings", section "What's in here / Quantized matmul": the fused
 *              GEMV's first phase applies a Hadamard transform to the activations before their
 *              int8 quantization; the 128-wide virtual groups of the orthogonal lm_head keep the
 *              rotation aligned with quantization groups.  Reading taken here: the normalized
 *              Sylvester-order Walsh-Hadamard transform on independent 128-wide blocks, fp32
 *              add/sub butterflies with the span doubling 1,2,...,64, then one multiply by
 *              fp32(1/sqrt(128)).
 *   quantize   same section (int8 per-group activation quantization) and the review snippet of
 *              the per-group SMOPA leaf contract (per-group int8 activations, one activation
 *              scale per group).  Reading: per row and group, amax = max|x| (exact),
 *              xs = amax / 127 as an IEEE fp32 divide, xq = round-half-even(x / xs) as an IEEE
 *              fp32 divide then rint, clamped to [-127, 127]; a group whose scale is 0 (amax == 0,
 *              or amax / 127 underflows to 0 for a group of tiny subnormals) has xs = 0 and
 *              every code 0.
 *   group sums "TensorFold PR #3215, simd_qmm on Metal: X's group sums and half operands from a
 *              prepass", section "What this changes": the prepass writes each row's per-group
 *              sums once, for the affine bias term.  Reading: the int32 sum of the int8 codes of
 *              the group (the only reading under which x_hat = xs*xq makes the bias term
 *              sum_k x_hat*bw equal xs*bw*xsum exactly).
 *   partials   PR #697's leaf contract (review snippet): a raw int32 dot product per group and
 *              output channel, partials[g][c] = sum over the group of act[k]*weight[c][k], with
 *              the activation-scale and weight-scale rescale applied by the caller.
 *   output     y[m][n] = sum over groups g of xs[m][g]*( sw[n][g]*D[m][n][g]
 *                                                      + bw[n][g]*xsum[m][g] )
 *              evaluated here in fp64 with g ascending; bw = 0 except for the affine format
 *              ("TensorFold PR #3215": 4-bit affine g64 weights, scale and bias per group,
 *              dequantized weight = scale*u + bias).
 *
 *   glu        "cactus-compute/engine PR #750: Metal Support", the commit list: the fusion-plan
 *              compiler folds a gelu-gated feed-forward pair into one transform + GEMV and
 *              sibling quantized GEMVs into one batched GEMV; the kernel commit lists gelu-erf
 *              and sigmoid activation codes.  "geistlib issue #500", section "Design": paired
 *              linears share one activation prepass.  Reading taken here: the gate and up
 *              projections are one packed linear of n = 2F output rows, gate rows first;
 *              z[r][f] = act(y[r][f]) * y[r][F + f] in fp64, act one of
 *                silu(v)      = v / (1 + exp(-v))
 *                gelu_tanh(v) = v/2 * (1 + tanh(sqrt(2/pi) * (v + 0.044715 v^3)))
 *                gelu_erf(v)  = v/2 * (1 + erf(v / sqrt(2)))
 *   fp16 path  "TensorFold PR #3215, simd_qmm on Metal: X's group sums and half operands from a
 *              prepass", section "What this changes": the prompt tiles multiply 4-bit g64
 *              weights (dequantized w = scale * u + bias) with X, either in fp32 or as half; a
 *              prepass writes X as half and each row's 64-wide group sums for the bias term,
 *              summed by the tiles' fixed tree ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)), each c a
 *              left-to-right sum of 8 consecutive inputs.  Reading taken here: xh = x rounded to
 *              the nearest binary16 (ties to even); S[r][g] = that tree over x in fp32 (fma with
 *              a unit factor is an add); y[r][n] = sum over g of ( sw * sum_k w_int * xh
 *              + bw * S ) in fp64, w_int the format's integer weight (affine: unsigned u).
 *   attention  "cactus PR #697", section "Prefill attention": the cached-int8 KV segment of a
 *              prefill chunk (fully visible by causality) with int8 QK products under one flat
 *              scale per query row and per key vector (the keys' group-scale ratios requantized
 *              into their int8 values), a masked softmax over 64-key blocks carried online, and
 *              an unsigned 8-bit P quantized per (row, value group, block) with the value group's
 *              scale folded into it; sliding window with attention-sink exemption; the new-token
 *              segment continues from the running statistics.  Readings taken here: Q codes as
 *              the activation quantization with one group per row; sk = max of the key's group
 *              scales and kq = round-half-even(k8 * fp32(ks_g / sk)) in fp32; logits
 *              scale * sq * sk * sum q8*kq; per block m' = max(m, block max), alpha = e^(m-m'),
 *              P = e^(S-m'), l = alpha*l + sum P; per value group g, P'_j = P_j * vs[j][g],
 *              sp = max P' / 255, u_j = round-half-even(P'_j / sp), O_g = alpha*O_g +
 *              sp * sum_j u_j * v8[j]; a slot at position p is seen by the query at t when
 *              p >= 0 and (no window, or p < sink, or t - p < window).
 *   lm_head    "cactus-compute/engine PR #750: Metal Support", the commit list (the orthogonal
 *              lm_head with its softcap fused into a GPU argmax / sampling tail) and the file
 *              table (GPU-side sampling and argmax helpers); "cactus PR #697", the lm_head commit
 *              (one scale per weight row viewed as K/128 virtual 128-wide groups, exactly).
 *              Reading: logits = c * tanh(y / c) for a cap c > 0, logits = y for c == 0; the
 *              greedy token is the smallest index of the largest logit.  The row-scale view is
 *              the output formula with every group scale of a row equal to the row's scale.
 *
 * Weight formats (canonical input, one byte holds two 4-bit codes, low nibble = even k):
 *   format 0 (symmetric):  code is a two's-complement q in [-8, 7]; w_int = q
 *   format 1 (affine):     code is an unsigned u in [0, 15];        w_int = u
 *   format 2 (codebook):   code is an index j in [0, 15];           w_int = codebook[n][j]
 *                          (PR #697's CQ4: 4-bit codebook indices expanded to int8 by lookup)
 *   format 3 (int8):       codes are int8 [n][k], one byte per weight; w_int = the byte
 *                          ("geistlib issue #500", sections "Scope" and "Design sketch": the
 *                          W8A8 inner kernel beside the W4A8 one, sharing the activation side;
 *                          symmetric, one fp16 scale per group)
 *   format 4 (2-bit codebook): codes uint8 [n][k/4], byte b holding the indices of k = 4b .. 4b+3
 *                          in bits 0-1, 2-3, 4-5, 6-7; w_int = codebook[n][index], a 4-entry
 *                          int8 codebook per row ("cactus PR #697": the CQ1-CQ4 codebook family,
 *                          of which this is CQ2; "geistlib issue #500", "Acceptance criteria":
 *                          W2A8 models), one fp16 scale per group
 *   format 5 (1-bit codebook, CQ1): codes uint8 [n][k/8], bit i of byte b is the index of
 *                          k = 8b + i; w_int = codebook[n][index], 2 entries per row
 *   format 6 (3-bit codebook, CQ3): codes uint8 [n][k], one index 0..7 per byte (low 3 bits);
 *                          w_int = codebook[n][index], 8 entries per row
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (no fast-math), so that every fp32
 * operation is a single IEEE-rounded operation in program order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1
#define ORACLE_OVERFLOW 2

/* ---------------------------------------------------------------- fp16 decoding -------- */

/* IEEE binary16 bit pattern -> double, exactly (every binary16 value is a double). */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int mant = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)mant, -24);               /* subnormal: mant * 2^-24 */
    } else if (expo == 31) {
        v = mant ? NAN : INFINITY;
    } else {
        v = ldexp((double)(mant | 0x400), expo - 25); /* (1024 + mant) * 2^(e-15-10) */
    }
    return sign ? -v : v;
}

/* ---------------------------------------------------------------- rotation ------------- */

/* The normalizing constant, fp32(1/sqrt(128)), computed in double and rounded once. */
static float oracle_wht_scale(int block)
{
    return (float)(1.0 / sqrt((double)block));
}

/*
 * In-place normalized Walsh-Hadamard transform of one block of `block` floats (a power of two).
 * Butterfly on pairs (j, j+h): new x[j] = x[j] + x[j+h], new x[j+h] = x[j] - x[j+h], for
 * h = 1, 2, 4, ..., block/2, then every element is multiplied by fp32(1/sqrt(block)).
 */
void oracle_wht_block(float *v, int block)
{
    for (int h = 1; h < block; h *= 2) {
        for (int i = 0; i < block; i += 2 * h) {
            for (int j = i; j < i + h; ++j) {
                float a = v[j];
                float b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
    float c = oracle_wht_scale(block);
    for (int j = 0; j < block; ++j)
        v[j] = v[j] * c;
}

/* Rotate every `block`-wide block of every row of x[m][k] in place. */
int oracle_rotate(float *x, int64_t m, int64_t k, int32_t block)
{
    if (block <= 0 || (block & (block - 1)) != 0 || k % block != 0 || m < 0)
        return ORACLE_BAD_ARGS;
    for (int64_t r = 0; r < m; ++r)
        for (int64_t b = 0; b < k / block; ++b)
            oracle_wht_block(x + r * k + b * block, block);
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- quantization --------- */

/*
 * Per row r and group g of `group` consecutive k:
 *   amax = max |x|;  xs = amax / 127 (fp32 divide);  xq = rint(x / xs) (fp32 divide, ties to even)
 *   clamped to [-127, 127];  xsum = sum of the group's codes (int32).
 *   The codes are taken only where xs > 0: when amax / 127 rounds to 0 (amax == 0, or amax at
 *   most 63 * 2^-149) the group is all zero codes with xs = 0.  When xs is itself subnormal it
 *   carries fewer significant bits, x / xs can exceed 127 and the clamp does apply.
 */
int oracle_quantize(const float *x, int64_t m, int64_t k, int32_t group,
                    int8_t *xq, float *xs, int32_t *xsum)
{
    if (group <= 0 || k % group != 0 || m < 0)
        return ORACLE_BAD_ARGS;
    int64_t ng = k / group;
    for (int64_t r = 0; r < m; ++r) {
        for (int64_t g = 0; g < ng; ++g) {
            const float *xg = x + r * k + g * group;
            int8_t *qg = xq + r * k + g * group;
            float amax = 0.0f;
            for (int i = 0; i < group; ++i) {
                float a = fabsf(xg[i]);
                if (a > amax)
                    amax = a;
            }
            float scale = amax / 127.0f;
            int32_t sum = 0;
            for (int i = 0; i < group; ++i) {
                int32_t q = 0;
                if (scale > 0.0f) {
                    float t = xg[i] / scale;
                    float rq = rintf(t);          /* round to nearest, ties to even */
                    if (rq > 127.0f) rq = 127.0f;   /* reached only with a subnormal scale */
                    if (rq < -127.0f) rq = -127.0f;
                    q = (int32_t)rq;
                }
                qg[i] = (int8_t)q;
                sum += q;
            }
            xs[r * ng + g] = scale;
            xsum[r * ng + g] = sum;
        }
    }
    return ORACLE_OK;
}

/* The whole activation prepass: copy, optional rotation, quantization. */
int oracle_prep(const float *x, int64_t m, int64_t k, int32_t group, int32_t hadamard_block,
                int8_t *xq, float *xs, int32_t *xsum)
{
    if (hadamard_block != 0 && (hadamard_block <= 0 || k % hadamard_block != 0))
        return ORACLE_BAD_ARGS;
    float *tmp = (float *)malloc((size_t)(m * k > 0 ? m * k : 1) * sizeof(float));
    if (!tmp)
        return ORACLE_BAD_ARGS;
    memcpy(tmp, x, (size_t)(m * k) * sizeof(float));
    int rc = ORACLE_OK;
    if (hadamard_block != 0)
        rc = oracle_rotate(tmp, m, k, hadamard_block);
    if (rc == ORACLE_OK)
        rc = oracle_quantize(tmp, m, k, group, xq, xs, xsum);
    free(tmp);
    return rc;
}

/* ---------------------------------------------------------------- weights -------------- */

/* The 4-bit code of weight (n, k) from the canonical byte array codes[n][k/2]. */
static int oracle_code(const uint8_t *codes, int64_t k_total, int64_t n, int64_t k)
{
    uint8_t byte = codes[n * (k_total / 2) + k / 2];
    return (k % 2 == 0) ? (byte & 0x0f) : (byte >> 4);
}

/* The integer weight of (n, k) for each format (see the file header). */
static int32_t oracle_weight_int(int format, const uint8_t *codes, const int8_t *codebook,
                                 int64_t k_total, int64_t n, int64_t k)
{
    if (format == 3)
        return (int32_t)((const int8_t *)codes)[n * k_total + k];   /* one byte per weight */
    if (format == 4) {                                             /* four indices per byte */
        int idx = (codes[n * (k_total / 4) + k / 4] >> (2 * (k % 4))) & 3;
        return (int32_t)codebook[n * 4 + idx];
    }
    if (format == 5) {                                             /* eight indices per byte */
        int idx = (codes[n * (k_total / 8) + k / 8] >> (k % 8)) & 1;
        return (int32_t)codebook[n * 2 + idx];
    }
    if (format == 6)                                               /* one index per byte */
        return (int32_t)codebook[n * 8 + (codes[n * k_total + k] & 7)];
    int c = oracle_code(codes, k_total, n, k);
    if (format == 0)
        return c >= 8 ? c - 16 : c;                 /* two's-complement nibble */
    if (format == 1)
        return c;                                   /* unsigned code */
    return (int32_t)codebook[n * 16 + c];           /* codebook lookup */
}

/* ---------------------------------------------------------------- partials, output ----- */

/*
 * D[r][n][g] = sum over k in group g of xq[r][k] * w_int[n][k], accumulated in int64 and
 * checked to fit int32.  Output layout d[m][n][k/group].
 */
int oracle_partials(int32_t format, const uint8_t *codes, const int8_t *codebook,
                    int64_t n, int64_t k, int32_t group, const int8_t *xq, int64_t m,
                    int32_t *d)
{
    if (group <= 0 || k % group != 0 || k % 2 != 0 || format < 0 || format > 6)
        return ORACLE_BAD_ARGS;
    if ((format == 2 || format >= 4) && codebook == NULL)
        return ORACLE_BAD_ARGS;
    int64_t ng = k / group;
    int overflow = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : overflow)
    for (int64_t c = 0; c < n; ++c) {
        int32_t *w = (int32_t *)malloc((size_t)k * sizeof(int32_t));
        for (int64_t kk = 0; kk < k; ++kk)
            w[kk] = oracle_weight_int(format, codes, codebook, k, c, kk);
        for (int64_t r = 0; r < m; ++r) {
            for (int64_t g = 0; g < ng; ++g) {
                int64_t acc = 0;
                for (int64_t kk = g * group; kk < (g + 1) * group; ++kk)
                    acc += (int64_t)xq[r * k + kk] * (int64_t)w[kk];
                if (acc > INT32_MAX || acc < INT32_MIN)
                    overflow = 1;
                d[(r * n + c) * ng + g] = (int32_t)acc;
            }
        }
        free(w);
    }
    return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

/*
 * y[r][n] = sum_g xs[r][g] * ( sw[n][g]*D[r][n][g] + bw[n][g]*xsum[r][g] )    (fp64, g ascending)
 * t[r][n] = sum_g |xs*sw*D| + |xs*bw*xsum|      (the magnitude of the terms, for error bounds)
 * bias_f16 is used only for format 1 (affine); it may be NULL otherwise.
 * t may be NULL.
 */
int oracle_linear(int32_t format, const uint8_t *codes, const uint16_t *scales_f16,
                  const uint16_t *bias_f16, const int8_t *codebook,
                  int64_t n, int64_t k, int32_t group,
                  const int8_t *xq, const float *xs, const int32_t *xsum, int64_t m,
                  double *y, double *t)
{
    if (group <= 0 || k % group != 0 || k % 2 != 0 || format < 0 || format > 6)
        return ORACLE_BAD_ARGS;
    if ((format == 1 && bias_f16 == NULL) || ((format == 2 || format >= 4) && codebook == NULL))
        return ORACLE_BAD_ARGS;
    int64_t ng = k / group;
    int overflow = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : overflow)
    for (int64_t c = 0; c < n; ++c) {
        int32_t *w = (int32_t *)malloc((size_t)k * sizeof(int32_t));
        for (int64_t kk = 0; kk < k; ++kk)
            w[kk] = oracle_weight_int(format, codes, codebook, k, c, kk);
        for (int64_t r = 0; r < m; ++r) {
            double acc = 0.0, mag = 0.0;
            for (int64_t g = 0; g < ng; ++g) {
                int64_t dot = 0;
                for (int64_t kk = g * group; kk < (g + 1) * group; ++kk)
                    dot += (int64_t)xq[r * k + kk] * (int64_t)w[kk];
                if (dot > INT32_MAX || dot < INT32_MIN)
                    overflow = 1;
                double a = (double)xs[r * ng + g];
                double sw = oracle_half_to_double(scales_f16[c * ng + g]);
                double bw = (format == 1) ? oracle_half_to_double(bias_f16[c * ng + g]) : 0.0;
                double main_term = a * (sw * (double)dot);
                double bias_term = a * (bw * (double)xsum[r * ng + g]);
                acc += main_term + bias_term;
                mag += fabs(main_term) + fabs(bias_term);
            }
            y[r * n + c] = acc;
            if (t)
                t[r * n + c] = mag;
        }
        free(w);
    }
    return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

/* ---------------------------------------------------------------- gated output -------- */
#define ORACLE_ACT_SILU 0
#define ORACLE_ACT_GELU_TANH 1
#define ORACLE_ACT_GELU_ERF 2

static double oracle_act(int32_t act, double v)
{
    const double pi = 3.14159265358979323846;
    if (act == ORACLE_ACT_SILU)
        return v / (1.0 + exp(-v));
    if (act == ORACLE_ACT_GELU_TANH)
        return 0.5 * v * (1.0 + tanh(sqrt(2.0 / pi) * (v + 0.044715 * v * v * v)));
    return 0.5 * v * (1.0 + erf(v / sqrt(2.0)));
}

/*
 * z[r][f] = act(y[r][f]) * y[r][F + f] for f < F = n / 2 (fp64), from the linear's y [m][n].
 * tz (may be NULL) bounds how far z moves when the two linear outputs move by at most e times
 * their term magnitudes t: |dz| <= e * tz with tz = 1.2 * |u| * t_g + |act(g)| * t_u, where 1.2
 * exceeds the largest slope of every act here (silu about 1.0998, both gelus about 1.1289).
 */
int oracle_glu(int32_t act, const double *y, const double *t, int64_t m, int64_t n,
               double *z, double *tz)
{
    if (act < ORACLE_ACT_SILU || act > ORACLE_ACT_GELU_ERF || n % 2 != 0 || m < 0)
        return ORACLE_BAD_ARGS;
    int64_t f_n = n / 2;
    for (int64_t r = 0; r < m; ++r)
        for (int64_t f = 0; f < f_n; ++f) {
            double g = y[r * n + f], u = y[r * n + f_n + f];
            double a = oracle_act(act, g);
            z[r * f_n + f] = a * u;
            if (tz && t)
                tz[r * f_n + f] = 1.2 * fabs(u) * t[r * n + f] + fabs(a) * t[r * n + f_n + f];
        }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- greedy tail ---------- */
/*
 * Per row r of y [m][n]: logits = cap * tanh(y / cap) (cap > 0) or y (cap == 0), in fp64, and
 * token[r] = the smallest index of the largest logit, value[r] = that logit.
 */
int oracle_softcap_argmax(const double *y, int64_t m, int64_t n, double cap, double *logits,
                          int64_t *token, double *value)
{
    if (n <= 0 || m < 0 || cap < 0.0)
        return ORACLE_BAD_ARGS;
    for (int64_t r = 0; r < m; ++r) {
        int64_t best = 0;
        for (int64_t c = 0; c < n; ++c) {
            double v = y[r * n + c];
            if (cap > 0.0)
                v = cap * tanh(v / cap);
            logits[r * n + c] = v;
            if (v > logits[r * n + best])
                best = c;
        }
        token[r] = best;
        value[r] = logits[r * n + best];
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- fp16 activations ----- */

/* Round a non-negative double q to the nearest integer, ties to the even one. */
static double oracle_round_half_even(double q)
{
    double fl = floor(q);
    double diff = q - fl;                           /* exact for the q used here */
    if (diff > 0.5)
        return fl + 1.0;
    if (diff < 0.5)
        return fl;
    return fmod(fl, 2.0) == 0.0 ? fl : fl + 1.0;
}

/*
 * IEEE binary16 bit pattern nearest to f, ties to even (round-to-nearest-even conversion):
 * binary16 has 10 stored fraction bits, exponents -14..15, subnormals down to 2^-24, and every
 * magnitude from 65520 (half-way between 65504 and 2^16) up rounds to infinity.
 */
uint16_t oracle_float_to_half(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (((bits >> 23) & 0xffu) == 0xffu)            /* infinity or NaN */
        return sign | 0x7c00u | ((bits & 0x7fffffu) ? 0x200u : 0u);
    double v = fabs((double)f);                     /* exact */
    if (v >= 65520.0)
        return sign | 0x7c00u;
    if (v < ldexp(1.0, -14)) {                      /* subnormal range: units of 2^-24 */
        double q = oracle_round_half_even(v * ldexp(1.0, 24));
        return sign | (uint16_t)q;                  /* q == 1024 is the smallest normal */
    }
    int ex;
    frexp(v, &ex);                                  /* v in [2^(ex-1), 2^ex) */
    int e = ex - 1;
    double q = oracle_round_half_even(ldexp(v, 10 - e));   /* in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return sign | 0x7c00u;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)q - 1024));
}

/*
 * The fp16-activation prepass: xh[r][k] = binary16(x[r][k]) (natural order) and, per row and
 * 64-wide group, S[r][g] = ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)) in fp32 with
 * c_o = (((x[8o] + x[8o+1]) + x[8o+2]) + ... ) + x[8o+7] over the group's inputs.
 * Output layouts xh[m][k], xsf[m][k/64].
 */
int oracle_prep_a16(const float *x, int64_t m, int64_t k, uint16_t *xh, float *xsf)
{
    if (m < 0 || k <= 0 || k % 64 != 0)
        return ORACLE_BAD_ARGS;
    int64_t ng = k / 64;
    for (int64_t i = 0; i < m * k; ++i)
        xh[i] = oracle_float_to_half(x[i]);
    for (int64_t r = 0; r < m; ++r) {
        for (int64_t g = 0; g < ng; ++g) {
            const float *v = x + r * k + g * 64;
            float c[8];
            for (int o = 0; o < 8; ++o) {
                float acc = v[8 * o];
                for (int i = 1; i < 8; ++i)
                    acc = acc + v[8 * o + i];
                c[o] = acc;
            }
            xsf[r * ng + g] = ((c[0] + c[1]) + (c[2] + c[3])) + ((c[4] + c[5]) + (c[6] + c[7]));
        }
    }
    return ORACLE_OK;
}

/*
 * y[r][n] = sum_g ( sw[n][g] * sum_{k in g} w_int[n][k] * xh[r][k] + bw[n][g] * S[r][g] )
 * t[r][n] = sum_g ( sum_{k in g} |sw * w_int * xh| + |bw * S| )          (fp64, g and k ascending)
 * xh holds binary16 bit patterns [m][k], xsf the fp32 group sums [m][k/group]; bias_f16 is used
 * only for format 1.  t may be NULL.
 */
int oracle_linear_a16(int32_t format, const uint8_t *codes, const uint16_t *scales_f16,
                      const uint16_t *bias_f16, const int8_t *codebook, int64_t n, int64_t k,
                      int32_t group, const uint16_t *xh, const float *xsf, int64_t m,
                      double *y, double *t)
{
    if (group <= 0 || k % group != 0 || k % 2 != 0 || format < 0 || format > 6)
        return ORACLE_BAD_ARGS;
    if ((format == 1 && bias_f16 == NULL) || (format == 2 && codebook == NULL))
        return ORACLE_BAD_ARGS;
    int64_t ng = k / group;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t c = 0; c < n; ++c) {
        double *w = (double *)malloc((size_t)k * sizeof(double));
        for (int64_t kk = 0; kk < k; ++kk)
            w[kk] = (double)oracle_weight_int(format, codes, codebook, k, c, kk);
        for (int64_t r = 0; r < m; ++r) {
            double acc = 0.0, mag = 0.0;
            for (int64_t g = 0; g < ng; ++g) {
                double sw = oracle_half_to_double(scales_f16[c * ng + g]);
                double bw = (format == 1) ? oracle_half_to_double(bias_f16[c * ng + g]) : 0.0;
                double dot = 0.0, dmag = 0.0;
                for (int64_t kk = g * group; kk < (g + 1) * group; ++kk) {
                    double p = w[kk] * oracle_half_to_double(xh[r * k + kk]);
                    dot += p;
                    dmag += fabs(p);
                }
                double bias_term = bw * (double)xsf[r * ng + g];
                acc += sw * dot + bias_term;
                mag += fabs(sw) * dmag + fabs(bias_term);
            }
            y[r * n + c] = acc;
            if (t)
                t[r * n + c] = mag;
        }
        free(w);
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- prefill attention ---- */

/*
 * Keys to one flat scale per vector: sk[j] = max_g ks[j][g]; kq[j][i] = round-half-even of
 * k8[j][i] * fp32(ks[j][g] / sk[j]) in fp32 (0 when sk == 0).  Layouts k8, kq [n][d],
 * ks [n][d/gk], sk [n].
 */
int oracle_attn_requant_k(const int8_t *k8, const float *ks, int64_t n, int64_t d, int32_t gk,
                          int8_t *kq, float *sk)
{
    if (gk <= 0 || d % gk != 0 || n < 0)
        return ORACLE_BAD_ARGS;
    int64_t ng = d / gk;
    for (int64_t j = 0; j < n; ++j) {
        float mx = 0.0f;
        for (int64_t g = 0; g < ng; ++g)
            if (ks[j * ng + g] > mx)
                mx = ks[j * ng + g];
        sk[j] = mx;
        for (int64_t i = 0; i < d; ++i) {
            float v = 0.0f;
            if (mx > 0.0f) {
                float ratio = ks[j * ng + i / gk] / mx;
                v = rintf((float)k8[j * d + i] * ratio);
            }
            kq[j * d + i] = (int8_t)v;
        }
    }
    return ORACLE_OK;
}

/* Is the cache slot at position p visible to the query at position t? */
static int oracle_attn_visible(int64_t t, int64_t p, int32_t window, int32_t sink)
{
    if (p < 0 || p > t)
        return 0;
    if (window <= 0 || p < sink)
        return 1;
    return t - p < window;
}

/*
 * The int8 method in fp64, blocks of 64 slots in slot order.  Inputs: q8 [nh][nq][d], sq
 * [nh][nq]; kq [nkvh][nkv][d], sk [nkvh][nkv]; v8 [nkvh][nkv][d], vs [nkvh][nkv][d/gv];
 * kvpos [nkv]; query i sits at position pos0 + i; query head h reads key/value head
 * h / (nh / nkvh).  Outputs: the running state o [nh][nq][d] (unnormalized), m, l [nh][nq]
 * (m = -inf and l = 0 where no slot is visible).
 */
int oracle_attn_int8(const int8_t *q8, const float *sq, int64_t nh, int64_t nq,
                     const int8_t *kq, const float *sk, const int8_t *v8, const float *vs,
                     const int32_t *kvpos, int64_t nkvh, int64_t nkv, int64_t d, int32_t gv,
                     int64_t pos0, int32_t window, int32_t sink, double scale,
                     double *o, double *m, double *l)
{
    if (nh <= 0 || nkvh <= 0 || nh % nkvh != 0 || gv <= 0 || d % gv != 0)
        return ORACLE_BAD_ARGS;
    int64_t ng = d / gv, per = nh / nkvh;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int64_t h = 0; h < nh; ++h) {
        for (int64_t i = 0; i < nq; ++i) {
            int64_t kh = h / per, t = pos0 + i;
            const int8_t *qr = q8 + (h * nq + i) * d;
            double *orow = o + (h * nq + i) * d;
            double mrun = -INFINITY, lrun = 0.0;
            double sv[64], pv[64], pg[64];
            int vis[64];
            for (int64_t c = 0; c < d; ++c)
                orow[c] = 0.0;
            for (int64_t j0 = 0; j0 < nkv; j0 += 64) {
                int64_t nb = (nkv - j0 < 64) ? nkv - j0 : 64;
                double mb = -INFINITY;
                for (int64_t jj = 0; jj < nb; ++jj) {
                    int64_t j = j0 + jj;
                    vis[jj] = oracle_attn_visible(t, kvpos[j], window, sink);
                    if (!vis[jj])
                        continue;
                    const int8_t *kr = kq + (kh * nkv + j) * d;
                    int64_t dot = 0;
                    for (int64_t c = 0; c < d; ++c)
                        dot += (int64_t)qr[c] * (int64_t)kr[c];
                    sv[jj] = scale * (double)sq[h * nq + i] * (double)sk[kh * nkv + j] * (double)dot;
                    if (sv[jj] > mb)
                        mb = sv[jj];
                }
                if (mb == -INFINITY)
                    continue;                                   /* nothing visible here */
                double mnew = mrun > mb ? mrun : mb;
                double alpha = exp(mrun - mnew);                /* 0 while mrun = -inf */
                double psum = 0.0;
                for (int64_t jj = 0; jj < nb; ++jj) {
                    pv[jj] = vis[jj] ? exp(sv[jj] - mnew) : 0.0;
                    psum += pv[jj];
                }
                lrun = lrun * alpha + psum;
                for (int64_t g = 0; g < ng; ++g) {
                    double mx = 0.0;
                    for (int64_t jj = 0; jj < nb; ++jj) {
                        pg[jj] = pv[jj] * (double)vs[(kh * nkv + j0 + jj) * ng + g];
                        if (pg[jj] > mx)
                            mx = pg[jj];
                    }
                    double sp = mx / 255.0;
                    for (int64_t c = g * gv; c < (g + 1) * gv; ++c) {
                        double acc = 0.0;
                        for (int64_t jj = 0; jj < nb; ++jj) {
                            double u = mx > 0.0 ? oracle_round_half_even(pg[jj] / sp) : 0.0;
                            acc += u * (double)v8[(kh * nkv + j0 + jj) * d + c];
                        }
                        orow[c] = orow[c] * alpha + sp * acc;
                    }
                }
                mrun = mnew;
            }
            m[h * nq + i] = mrun;
            l[h * nq + i] = lrun;
        }
    }
    return ORACLE_OK;
}

/*
 * Plain attention in fp64 on the unquantized queries and the dequantized cache (k8 * ks_g,
 * v8 * vs_g): out[h][i] = sum_j softmax_j(scale * q . k_j) v_j over the visible slots (0 when
 * none is visible).  The reference the int8 method is measured against.
 */
int oracle_attn_exact(const float *q, int64_t nh, int64_t nq, const int8_t *k8, const float *ks,
                      const int8_t *v8, const float *vs, const int32_t *kvpos, int64_t nkvh,
                      int64_t nkv, int64_t d, int32_t gk, int32_t gv, int64_t pos0,
                      int32_t window, int32_t sink, double scale, double *out)
{
    if (nh <= 0 || nkvh <= 0 || nh % nkvh != 0 || gk <= 0 || gv <= 0 || d % gk || d % gv)
        return ORACLE_BAD_ARGS;
    int64_t per = nh / nkvh, ngk = d / gk, ngv = d / gv;
#pragma omp parallel for collapse(2) schedule(dynamic, 4)
    for (int64_t h = 0; h < nh; ++h) {
        for (int64_t i = 0; i < nq; ++i) {
            int64_t kh = h / per, t = pos0 + i;
            const float *qr = q + (h * nq + i) * d;
            double *orow = out + (h * nq + i) * d;
            double *sc = (double *)malloc((size_t)(nkv > 0 ? nkv : 1) * sizeof(double));
            double mx = -INFINITY;
            for (int64_t j = 0; j < nkv; ++j) {
                sc[j] = -INFINITY;
                if (!oracle_attn_visible(t, kvpos[j], window, sink))
                    continue;
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += (double)qr[c] * (double)k8[(kh * nkv + j) * d + c] *
                           (double)ks[(kh * nkv + j) * ngk + c / gk];
                sc[j] = scale * dot;
                if (sc[j] > mx)
                    mx = sc[j];
            }
            for (int64_t c = 0; c < d; ++c)
                orow[c] = 0.0;
            if (mx != -INFINITY) {
                double den = 0.0;
                for (int64_t j = 0; j < nkv; ++j) {
                    if (sc[j] == -INFINITY)
                        continue;
                    double p = exp(sc[j] - mx);
                    den += p;
                    for (int64_t c = 0; c < d; ++c)
                        orow[c] += p * (double)v8[(kh * nkv + j) * d + c] *
                                   (double)vs[(kh * nkv + j) * ngv + c / gv];
                }
                for (int64_t c = 0; c < d; ++c)
                    orow[c] /= den;
            }
            free(sc);
        }
    }
    return ORACLE_OK;
}

/* Number of OpenMP threads a parallel region here would use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
