// Decode GEMV (one activation row) over the packed 4-bit weights.
//
// Source: "cactus PR #697", section "Quantized matmul": the M=1 path streams packed nibbles (half
// the bytes of expanded int8 weights) and is bound by memory bandwidth on the vocabulary head;
// the review snippet of the per-group leaf contract defines the raw int32 partial per group and
// output channel, rescaled afterwards by activation scale times weight scale.
//
// MI355X design: one workgroup per 64-row panel, W wavefronts splitting the panel's groups.
// Lane r of every wavefront owns panel row r, so each load instruction of a wavefront reads one
// contiguous KiB (64 rows x 16 bytes of one 32-wide k chunk) and every lane needs the same 32
// activation codes, which therefore come through the scalar cache into SGPRs (no LDS, no
// cross-lane traffic in the inner loop).  Per 16-byte chunk a lane does 12 unpack ops and 8
// v_dot4_i32_i8; per group it converts the int32 partial and applies xs * sw with one FMA.  The
// W partial sums of a row meet once in LDS and are added in a fixed order (deterministic).
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

template <int FMT, int G, int W, bool PARTIALS>
__global__ __launch_bounds__(64 * W) void gemv_kernel(const uint8_t *__restrict__ packed,
                                                      const Geom geom,
                                                      const int8_t *__restrict__ xq,
                                                      const float *__restrict__ xs,
                                                      const int *__restrict__ xsum,
                                                      float *__restrict__ y,
                                                      int *__restrict__ d) {
    constexpr int kChunksPerGroup = G / kChunkK;
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
    const int *xq4 = reinterpret_cast<const int *>(xq);

    float acc = 0.0f;    // sum over groups of xs * sw * (partial as computed, see kOut)
    float bacc = 0.0f;   // AFFINE: sum over groups of xs * xsum * bw
    for (int gb = g0; gb < g1; gb += kBatchGroups) {
        const int nb = min(kBatchGroups, g1 - gb);
        uint4 v[kBatchGroups * kChunksPerGroup];
#pragma unroll
        for (int i = 0; i < kBatchGroups; ++i) {
            if (i < nb) {
#pragma unroll
                for (int c = 0; c < kChunksPerGroup; ++c)
                    v[i * kChunksPerGroup + c] =
                        wp[(int64_t)((gb + i) * kChunksPerGroup + c) * kPanelRows];
            }
        }
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
                    if (FMT == kFmtAffine) part += 8 * xsum[g];
                    if (row < geom.n) d[row * ng + g] = part;
                } else {
                    const float a = xs[g];
                    if (FMT == kFmtAffine) {
                        const uint32_t mb = *reinterpret_cast<const uint32_t *>(
                            meta + (int64_t)g * kPanelRows * 4);
                        const float sw = half_bits_to_float(mb & 0xFFFFu);
                        const float bw = half_bits_to_float(mb >> 16);
                        const int s = xsum[g];
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

template <int FMT, int G, bool PARTIALS>
hipError_t launch_w(const Geom &g, const uint8_t *packed, const int8_t *xq, const float *xs,
                    const int32_t *xsum, float *y, int32_t *d, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>(g.n_pad / kPanelRows);
    const int ng = g.k / G;
    if (ng >= 8)
        gemv_kernel<FMT, G, 8, PARTIALS><<<grid, 512, 0, stream>>>(packed, g, xq, xs, xsum, y, d);
    else
        gemv_kernel<FMT, G, 4, PARTIALS><<<grid, 256, 0, stream>>>(packed, g, xq, xs, xsum, y, d);
    return hipGetLastError();
}

template <int FMT, bool PARTIALS>
hipError_t launch_g(const Geom &g, const uint8_t *packed, const int8_t *xq, const float *xs,
                    const int32_t *xsum, float *y, int32_t *d, hipStream_t stream) {
    if (g.group == 64) return launch_w<FMT, 64, PARTIALS>(g, packed, xq, xs, xsum, y, d, stream);
    return launch_w<FMT, 128, PARTIALS>(g, packed, xq, xs, xsum, y, d, stream);
}

template <bool PARTIALS>
hipError_t launch_f(const Geom &g, const uint8_t *packed, const int8_t *xq, const float *xs,
                    const int32_t *xsum, float *y, int32_t *d, hipStream_t stream) {
    switch (g.fmt) {
    case kFmtSym: return launch_g<kFmtSym, PARTIALS>(g, packed, xq, xs, xsum, y, d, stream);
    case kFmtAffine: return launch_g<kFmtAffine, PARTIALS>(g, packed, xq, xs, xsum, y, d, stream);
    default: return launch_g<kFmtCodebook, PARTIALS>(g, packed, xq, xs, xsum, y, d, stream);
    }
}

}  // namespace

hipError_t launch_gemv(const Geom &g, const uint8_t *packed, const int8_t *xq, const float *xs,
                       const int32_t *xsum, float *y, int32_t *d, hipStream_t stream) {
    if (d) return launch_f<true>(g, packed, xq, xs, xsum, nullptr, d, stream);
    return launch_f<false>(g, packed, xq, xs, xsum, y, nullptr, stream);
}

}  // namespace w4a8
