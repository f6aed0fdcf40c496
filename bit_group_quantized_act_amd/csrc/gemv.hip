// Decode GEMV (one activation row) over the packed 4-bit weights.
//
// Source: "cactus PR #697", section "Quantized matmul": the M=1 path is a fused GEMV whose first
// phase rotates (optionally) and quantizes the activations to int8 per group and whose second
// phase streams packed nibbles (half the bytes of expanded int8 weights); it is bound by memory
// bandwidth on the vocabulary head.  The review snippet of the per-group leaf contract defines
// the raw int32 partial per group and output channel, rescaled afterwards by activation scale
// times weight scale.
//
// MI355X design: one workgroup per 64-row panel, W wavefronts splitting the panel's groups.
// Lane r of every wavefront owns panel row r, so each load instruction of a wavefront reads one
// contiguous KiB (64 rows x 16 bytes of one 32-wide k chunk).  Per 16-byte chunk a lane does 12
// unpack ops and 8 v_dot4_i32_i8; per group it converts the int32 partial and applies xs * sw
// with one FMA.  The W partial sums of a row meet once in LDS and are added in a fixed order
// (deterministic).
//   Activations.  Every lane needs the same 32 activation codes per chunk.  The plain kernel
//   reads them from the prepass output through the scalar cache into SGPRs.  The fused kernel
//   (one launch for the whole decode layer) loads its part of the fp32 row, issues its weight
//   loads, then quantizes the row into LDS with the prepass's arithmetic (prep_quad, so the codes
//   are the same bits) while the weights are in flight; the dot products then read the codes as
//   LDS broadcasts.  Workgroup 0 also writes xq, xs and xsum.
#include "w4a8_kernels.h"

namespace w4a8 {
namespace {

constexpr int kBatchGroups = 4;   // groups whose chunks are loaded before any is consumed

template <int FMT>
__device__ __forceinline__ int dot_chunk(uint4 v, const int *__restrict__ xc, uint4 cb, int acc) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t lo, hi;
        if (FMT == kFmtCodebook) {
            lo = cb_lo(w[j], cb);
            hi = cb_hi(w[j], cb);
        } else {
            lo = lo_x16(w[j]);
            hi = hi_x16(w[j]);
        }
        acc = __builtin_amdgcn_sdot4(static_cast<int>(lo), xc[j], acc, false);
        acc = __builtin_amdgcn_sdot4(static_cast<int>(hi), xc[4 + j], acc, false);
    }
    return acc;
}

// FUSED: x is the fp32 activation row; xq/xs/xsum are outputs written by workgroup 0.
// Otherwise xq/xs/xsum are the prepass outputs (inputs here) and x is unused.
template <int FMT, int G, int W, bool PARTIALS, bool FUSED, bool ROT>
__global__ __launch_bounds__(64 * W) void gemv_kernel(const uint8_t *__restrict__ packed,
                                                      const Geom geom,
                                                      const float *__restrict__ x,
                                                      int8_t *__restrict__ xq,
                                                      float *__restrict__ xs,
                                                      int *__restrict__ xsum,
                                                      float *__restrict__ y,
                                                      int *__restrict__ d) {
    constexpr int kChunksPerGroup = G / kChunkK;
    constexpr int kLanesPerGroup = G / 4;
    constexpr int kLdsQuads = FUSED ? kFusedMaxK / 4 : 1;
    constexpr int kLdsGroups = FUSED ? kFusedMaxK / G : 1;
    __shared__ __attribute__((aligned(16))) int lds_xq[kLdsQuads];
    __shared__ float lds_xs[kLdsGroups];
    __shared__ int lds_xsum[kLdsGroups];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int p = blockIdx.x;
    const int kc = geom.k / kChunkK;
    const int ng = geom.k / G;
    const int g0 = wave * ng / W;
    const int g1 = (wave + 1) * ng / W;
    const int64_t row = (int64_t)p * kPanelRows + lane;

    const uint4 *wp = reinterpret_cast<const uint4 *>(packed + geom.off_codes) +
                      (int64_t)p * kc * kPanelRows + lane;
    const uint8_t *meta = packed + geom.off_meta +
                          ((int64_t)p * ng * kPanelRows + lane) * geom.meta_bytes;
    uint4 cb = make_uint4(0u, 0u, 0u, 0u);
    if (FMT == kFmtCodebook)
        cb = *reinterpret_cast<const uint4 *>(packed + geom.off_codebook + row * 16);

    uint4 v[kBatchGroups * kChunksPerGroup];
    // A batch always issues the same loads (slots past the wavefront's groups re-read a valid
    // chunk of the panel and are never used): with no load behind a branch, the compiler's waits
    // count exactly the loads issued after the one they wait for.
    auto load_batch = [&](int gb) {
        const int glast = max(g1 - 1, 0);
#pragma unroll
        for (int i = 0; i < kBatchGroups; ++i) {
            const int g = min(gb + i, glast);
#pragma unroll
            for (int c = 0; c < kChunksPerGroup; ++c)
                v[i * kChunksPerGroup + c] = wp[(int64_t)(g * kChunksPerGroup + c) * kPanelRows];
        }
    };
    // Fused: the thread's first activation quad is loaded before the weight batch.  Loads complete
    // in issue order, so the prepass below then waits for x only, with the whole batch still in
    // flight.  The compiler would sink an ordinary load below the batch (and then drain every
    // load before the prepass), so this one is issued by hand, ahead of the batch (the memory
    // clobber keeps the batch behind it), and waited for by hand: vmcnt(batch loads).
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
    const int nq = geom.k / 4;
    v4f xr = {0.f, 0.f, 0.f, 0.f};
    if (FUSED) {
        const float4 *xp = x4 + min(static_cast<int>(threadIdx.x), nq - 1);
        asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(xr) : "v"(xp) : "memory");
    }
    load_batch(g0);
    if (FUSED) asm volatile("s_waitcnt vmcnt(%1)" : "+v"(xr) : "n"(kBatchGroups * kChunksPerGroup));
    const float4 xv0 = make_float4(xr[0], xr[1], xr[2], xr[3]);

    const int *xq4;                 // activation codes, 4 per int
    const float *xsv;               // per-group scales
    const int *xsumv;               // per-group sums
    if (FUSED) {
        // the prepass of the row, while the first weight batch is in flight
        for (int t = threadIdx.x; t < nq; t += 64 * W) {
            float scale;
            int sum;
            const float4 xv = (t == static_cast<int>(threadIdx.x)) ? xv0 : x4[t];
            const int codes = prep_quad<G, ROT>(xv, t & 63, scale, sum);
            lds_xq[t] = codes;
            const bool leader = (t & (kLanesPerGroup - 1)) == 0;
            if (leader) {
                lds_xs[t / kLanesPerGroup] = scale;
                lds_xsum[t / kLanesPerGroup] = sum;
            }
            if (blockIdx.x == 0) {
                reinterpret_cast<int *>(xq)[t] = codes;
                if (leader) {
                    xs[t / kLanesPerGroup] = scale;
                    xsum[t / kLanesPerGroup] = sum;
                }
            }
        }
        __syncthreads();
        xq4 = lds_xq;
        xsv = lds_xs;
        xsumv = lds_xsum;
    } else {
        xq4 = reinterpret_cast<const int *>(xq);
        xsv = xs;
        xsumv = xsum;
    }

    float acc = 0.0f;    // sum over groups of xs * sw * (partial as computed, see kOut)
    float bacc = 0.0f;   // AFFINE: sum over groups of xs * xsum * bw
    for (int gb = g0; gb < g1; gb += kBatchGroups) {
        if (gb > g0) load_batch(gb);
        const int nb = min(kBatchGroups, g1 - gb);
#pragma unroll
        for (int i = 0; i < kBatchGroups; ++i) {
            if (i < nb) {
                const int g = gb + i;
                int dot = 0;
#pragma unroll
                for (int c = 0; c < kChunksPerGroup; ++c)
                    dot = dot_chunk<FMT>(v[i * kChunksPerGroup + c],
                                         xq4 + (g * kChunksPerGroup + c) * (kChunkK / 4), cb,
                                         dot);
                if (PARTIALS) {
                    // sym/affine dot is 16x the signed-code partial; affine adds back 8*xsum.
                    int part = (FMT == kFmtCodebook) ? dot : (dot >> 4);
                    if (FMT == kFmtAffine) part += 8 * xsumv[g];
                    if (row < geom.n) d[row * ng + g] = part;
                } else {
                    const float a = xsv[g];
                    if (FMT == kFmtAffine) {
                        const uint32_t mb = *reinterpret_cast<const uint32_t *>(
                            meta + (int64_t)g * kPanelRows * 4);
                        const float sw = half_bits_to_float(mb & 0xFFFFu);
                        const float bw = half_bits_to_float(mb >> 16);
                        const int s = xsumv[g];
                        // 16*D_u = dot + 128*xsum, exact in int32
                        acc = fmaf(a * sw, static_cast<float>(dot + 128 * s), acc);
                        bacc = fmaf(a * static_cast<float>(s), bw, bacc);
                    } else {
                        const uint32_t mb = *reinterpret_cast<const uint16_t *>(
                            meta + (int64_t)g * kPanelRows * 2);
                        const float sw = half_bits_to_float(mb);
                        acc = fmaf(a * sw, static_cast<float>(dot), acc);
                    }
                }
            }
        }
    }
    if (PARTIALS) return;

    // sym/affine partials were computed x16 (exact power of two, folded in once here)
    constexpr float kOut = (FMT == kFmtCodebook) ? 1.0f : 0.0625f;
    float part = acc * kOut + bacc;
    if (W == 1) {
        if (row < geom.n) y[row] = part;
        return;
    }
    __shared__ float red[W][64];
    red[wave][lane] = part;
    __syncthreads();
    if (wave == 0) {
        float s = red[0][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) s += red[w][lane];
        if (row < geom.n) y[row] = s;
    }
}

template <int FMT, int G, bool PARTIALS, bool FUSED, bool ROT>
hipError_t launch_w(const Geom &g, const uint8_t *packed, const float *x, int8_t *xq, float *xs,
                    int32_t *xsum, float *y, int32_t *d, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>(g.n_pad / kPanelRows);
    const int ng = g.k / G;
    if (ng >= 8)
        gemv_kernel<FMT, G, 8, PARTIALS, FUSED, ROT><<<grid, 512, 0, stream>>>(
            packed, g, x, xq, xs, xsum, y, d);
    else
        gemv_kernel<FMT, G, 4, PARTIALS, FUSED, ROT><<<grid, 256, 0, stream>>>(
            packed, g, x, xq, xs, xsum, y, d);
    return hipGetLastError();
}

template <int FMT, bool PARTIALS, bool FUSED, bool ROT>
hipError_t launch_g(const Geom &g, const uint8_t *packed, const float *x, int8_t *xq, float *xs,
                    int32_t *xsum, float *y, int32_t *d, hipStream_t stream) {
    if (g.group == 64)
        return launch_w<FMT, 64, PARTIALS, FUSED, ROT>(g, packed, x, xq, xs, xsum, y, d, stream);
    return launch_w<FMT, 128, PARTIALS, FUSED, ROT>(g, packed, x, xq, xs, xsum, y, d, stream);
}

template <bool PARTIALS, bool FUSED, bool ROT>
hipError_t launch_f(const Geom &g, const uint8_t *packed, const float *x, int8_t *xq, float *xs,
                    int32_t *xsum, float *y, int32_t *d, hipStream_t stream) {
    switch (g.fmt) {
    case kFmtSym:
        return launch_g<kFmtSym, PARTIALS, FUSED, ROT>(g, packed, x, xq, xs, xsum, y, d, stream);
    case kFmtAffine:
        return launch_g<kFmtAffine, PARTIALS, FUSED, ROT>(g, packed, x, xq, xs, xsum, y, d,
                                                          stream);
    default:
        return launch_g<kFmtCodebook, PARTIALS, FUSED, ROT>(g, packed, x, xq, xs, xsum, y, d,
                                                            stream);
    }
}

}  // namespace

hipError_t launch_gemv(const Geom &g, const uint8_t *packed, const int8_t *xq, const float *xs,
                       const int32_t *xsum, float *y, int32_t *d, hipStream_t stream) {
    // the plain kernel only reads its activation arguments
    int8_t *q = const_cast<int8_t *>(xq);
    float *s = const_cast<float *>(xs);
    int32_t *u = const_cast<int32_t *>(xsum);
    if (d) return launch_f<true, false, false>(g, packed, nullptr, q, s, u, nullptr, d, stream);
    return launch_f<false, false, false>(g, packed, nullptr, q, s, u, y, nullptr, stream);
}

hipError_t launch_gemv_fused(const Geom &g, const uint8_t *packed, const float *x, int hadamard,
                             int8_t *xq, float *xs, int32_t *xsum, float *y, hipStream_t stream) {
    if (hadamard) return launch_f<false, true, true>(g, packed, x, xq, xs, xsum, y, nullptr, stream);
    return launch_f<false, true, false>(g, packed, x, xq, xs, xsum, y, nullptr, stream);
}

}  // namespace w4a8
