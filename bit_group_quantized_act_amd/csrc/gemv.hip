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
//   Gated output (GLU).  For a [gate; up] linear (n = 2F, F a multiple of 64) workgroup b takes
//   rows 32 (b & 1) .. +31 of gate panel b / 2 in lanes 0..31 and the same rows of the up panel
//   F / 64 panels on in lanes 32..63: every load is still two contiguous 512-byte runs, the grid
//   and the bytes per workgroup are those of the plain GEMV, and after the cross-wavefront sum
//   lane r < 32 combines its gate value with lane r + 32's up value into act(gate) * up.
//   Greedy tail (ARGMAX).  Wavefront 0 caps each logit, stores it, and turns it into a 64-bit key
//   (an order-preserving image of the value above, the inverted row below: the largest key is
//   the largest logit at its smallest row); a butterfly gives the panel's largest key, which
//   lane 0 stores to the panel's slot of the key buffer.  A one-workgroup kernel (tail.hip)
//   then reduces the keys and decodes the token and its logit: no atomics, and nothing waits
//   on another workgroup.
#include "w4a8_kernels.h"

namespace w4a8 {
namespace {

constexpr int kRing = 4;   // groups whose loads are in flight ahead of the one consumed

template <int FMT>
__device__ __forceinline__ int dot_chunk(v4i v, const int *__restrict__ xc, uint4 cb, int acc) {
    const uint32_t w[4] = {(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
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
// XQ (fused only): activation quads per lane, enough for the wavefront's groups.
template <int FMT, int G, int W, bool PARTIALS, bool FUSED, bool ROT, int XQ, bool GLU,
          bool ARGMAX>
__global__ __launch_bounds__(64 * W) void gemv_kernel(const uint8_t *__restrict__ packed,
                                                      const Geom geom,
                                                      const float *__restrict__ x,
                                                      int8_t *__restrict__ xq,
                                                      float *__restrict__ xs,
                                                      int *__restrict__ xsum,
                                                      float *__restrict__ y,
                                                      int *__restrict__ d, int act, Tail tail) {
    static_assert(!(GLU && PARTIALS), "the gated output has no partials variant");
    static_assert(!(ARGMAX && (GLU || PARTIALS)), "the greedy tail has no gated or partials variant");
    constexpr int kChunksPerGroup = G / kChunkK;
    constexpr int kLanesPerGroup = G / 4;
    // Fused: activation quads (4 values) per lane that a wavefront quantizes, at most (the
    // launcher sizes XQ to the wavefront's groups: every one of these loads is issued).
    constexpr int kXQ = FUSED ? XQ : 1;
    constexpr int kXG = kXQ * 64 / kLanesPerGroup;           // groups per wavefront, at most
    // wavefront-private codes, scales and sums of its own groups (fused kernel)
    __shared__ __attribute__((aligned(16))) int lds_xq[FUSED ? W : 1][kXQ * 64];
    __shared__ float lds_xs[FUSED ? W : 1][kXG];
    __shared__ int lds_xsum[FUSED ? W : 1][kXG];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // GLU: the descriptors start at gate panel p and span the up panel up_pan panels on
    const int up_pan = GLU ? geom.n_pad / (2 * kPanelRows) : 0;
    const int p = GLU ? static_cast<int>(blockIdx.x >> 1) : static_cast<int>(blockIdx.x);
    const int lrow = GLU ? static_cast<int>((blockIdx.x & 1) * 32 + (lane & 31)) : lane;
    const bool up_lane = GLU && lane >= 32;
    const int npan = GLU ? up_pan + 1 : 1;
    const int kc = geom.k / kChunkK;
    const int ng = geom.k / G;
    // Wavefront w owns groups [g0, g1), split in whole metadata blocks of 4 groups (which also
    // keeps each 128-wide rotation block inside one wavefront).
    const int nblk = (ng + 3) / 4;
    const int g0 = min(ng, (wave * nblk / W) * 4);
    const int g1 = min(ng, ((wave + 1) * nblk / W) * 4);
    const int64_t row = (int64_t)(p + (up_lane ? up_pan : 0)) * kPanelRows + lrow;

    constexpr int kMetaBytes = (FMT == kFmtAffine) ? 4 : 2;
    constexpr int kRowBlk = 4 * kMetaBytes;          // one row's metadata block (4 groups)
    // the panel's codes and metadata; a load at kOOB returns zeros without a memory access
    const rsrc_t rw = make_rsrc(packed + geom.off_codes + (int64_t)p * kc * 1024,
                                (uint64_t)npan * kc * 1024);
    const rsrc_t rm = make_rsrc(packed + geom.off_meta + (int64_t)p * nblk * kPanelRows * kRowBlk,
                                (uint64_t)npan * nblk * kPanelRows * kRowBlk);
    // (GLU: the up lanes' offset to their panel; the host keeps both spans below 2^31)
    const int wlane = up_lane ? up_pan * kc * 1024 : 0;
    const int mlane = up_lane ? up_pan * nblk * kPanelRows * kRowBlk : 0;
    uint4 cb = make_uint4(0u, 0u, 0u, 0u);
    if (FMT == kFmtCodebook)
        cb = *reinterpret_cast<const uint4 *>(packed + geom.off_codebook + row * 16);

    // Ring of kRing = 4 groups (one metadata block) in flight: slot i holds a group's chunks,
    // and slot 0's load of a block's first group is preceded by the load of the block's
    // metadata (8 or 16 bytes per row) into mnext.  Loads complete in issue order, so the wait
    // for a group's chunks covers its metadata too, and the loads of the groups behind it stay
    // in flight.  Every load is issued unconditionally (a group past the wavefront's range loads
    // at kOOB: zeros, no memory traffic, never consumed): with no load behind a branch, the
    // compiler's waits count exactly the loads issued after the one they wait for.
    static_assert(kRing == 4, "a ring pass is one metadata block");
    v4i v[kRing][kChunksPerGroup];
    v4i mcur = {0, 0, 0, 0}, mnext = {0, 0, 0, 0};  // metadata blocks: this pass, the next
    auto load_group = [&](int slot, int g) {
        const bool in = g < g1;
        if (slot == 0) {
            const int mo = in ? ((g / 4) * kPanelRows + lrow) * kRowBlk + mlane : kOOB;
            if (kRowBlk == 16) {
                mnext = ld128(rm, mo);
            } else {
                const v2i m2 = ld64(rm, mo);
                mnext = v4i{m2[0], m2[1], 0, 0};
            }
        }
#pragma unroll
        for (int c = 0; c < kChunksPerGroup; ++c)
            v[slot][c] = ld128_stream(rw, in ? ((g * kChunksPerGroup + c) * kPanelRows + lrow) * 16 + wlane
                                      : kOOB);
    };
    // Issue order is pinned with scheduling barriers (loads complete in issue order, and every
    // wait above counts on it).  Fused: the lane's activation quads come first (those past the
    // wavefront's groups at kOOB), so the prepass below waits for x only, with the ring still in
    // flight behind it.
    const int qbase = g0 * kLanesPerGroup;            // first quad of the wavefront's groups
    const int nqw = (g1 - g0) * kLanesPerGroup;       // its quads
    v4i xr[kXQ];
    if (FUSED) {
        const rsrc_t rx = make_rsrc(x, (uint64_t)geom.k * 4);
#pragma unroll
        for (int i = 0; i < kXQ; ++i) {
            const int t = lane + 64 * i;
            xr[i] = ld128(rx, t < nqw ? (qbase + t) * 16 : kOOB);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
        load_group(i, g0 + i);
        __builtin_amdgcn_sched_barrier(0);
    }
    mcur = mnext;

    // activation codes (4 per int), scales and sums, indexed by the global quad / group
    const int *xq4;
    const float *xsv;
    const int *xsumv;
    if (FUSED) {
        // The prepass of the wavefront's own groups, while the ring is in flight.  A group's
        // G/4 lanes, and a rotation block's 32 lanes, are aligned runs of the wavefront that are
        // all active or all inactive.  No other wavefront reads these codes: no barrier.
#pragma unroll
        for (int i = 0; i < kXQ; ++i) {
            const int t = lane + 64 * i;
            if (t < nqw) {
                float scale;
                int sum;
                // (the whole vector is reinterpreted: clang's bit cast of one vector element
                // reads element 0 whatever the index)
                const v4f xf = __builtin_bit_cast(v4f, xr[i]);
                const float4 xv = make_float4(xf[0], xf[1], xf[2], xf[3]);
                const int codes = prep_quad<G, ROT>(xv, lane, scale, sum);
                lds_xq[wave][t] = codes;
                const bool leader = (t & (kLanesPerGroup - 1)) == 0;
                if (leader) {
                    lds_xs[wave][t / kLanesPerGroup] = scale;
                    lds_xsum[wave][t / kLanesPerGroup] = sum;
                }
                if (blockIdx.x == 0) {
                    reinterpret_cast<int *>(xq)[qbase + t] = codes;
                    if (leader) {
                        xs[g0 + t / kLanesPerGroup] = scale;
                        xsum[g0 + t / kLanesPerGroup] = sum;
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        xq4 = &lds_xq[wave][0] - qbase;
        xsv = &lds_xs[wave][0] - g0;
        xsumv = &lds_xsum[wave][0] - g0;
    } else {
        xq4 = reinterpret_cast<const int *>(xq);
        xsv = xs;
        xsumv = xsum;
    }

    float acc = 0.0f;    // sum over groups of xs * sw * (partial as computed, see kOut)
    float bacc = 0.0f;   // AFFINE: sum over groups of xs * xsum * bw
    for (int gb = g0; gb < g1; gb += kRing) {
#pragma unroll
        for (int i = 0; i < kRing; ++i) {
            const int g = gb + i;
            // the group's metadata entry: element i of the row's block (2-byte entries pack two
            // to a dword)
            const uint32_t mv = (kRowBlk == 16) ? static_cast<uint32_t>(mcur[i])
                                                : static_cast<uint32_t>(mcur[i / 2]) >> (16 * (i & 1));
            if (g < g1) {
                int dot = 0;
#pragma unroll
                for (int c = 0; c < kChunksPerGroup; ++c)
                    dot = dot_chunk<FMT>(v[i][c], xq4 + (g * kChunksPerGroup + c) * (kChunkK / 4),
                                         cb, dot);
                if (PARTIALS) {
                    // sym/affine dot is 16x the signed-code partial; affine adds back 8*xsum.
                    int part = (FMT == kFmtCodebook) ? dot : (dot >> 4);
                    if (FMT == kFmtAffine) part += 8 * xsumv[g];
                    if (row < geom.n) d[row * ng + g] = part;
                } else {
                    const float a = xsv[g];
                    const float sw = half_bits_to_float(mv & 0xFFFFu);
                    if (FMT == kFmtAffine) {
                        const float bw = half_bits_to_float(mv >> 16);
                        const int s = xsumv[g];
                        // 16*D_u = dot + 128*xsum, exact in int32
                        acc = fmaf(a * sw, static_cast<float>(dot + 128 * s), acc);
                        bacc = fmaf(a * static_cast<float>(s), bw, bacc);
                    } else {
                        acc = fmaf(a * sw, static_cast<float>(dot), acc);
                    }
                }
            }
            load_group(i, g + kRing);
            __builtin_amdgcn_sched_barrier(0);
        }
        mcur = mnext;
    }
    if (PARTIALS) return;

    // sym/affine partials were computed x16 (exact power of two, folded in once here)
    constexpr float kOut = (FMT == kFmtCodebook) ? 1.0f : 0.0625f;
    float part = acc * kOut + bacc;
    float s = part;
    if (W > 1) {
        __shared__ float red[W][64];
        red[wave][lane] = part;
        __syncthreads();
        if (wave != 0) return;
        s = red[0][lane];
#pragma unroll
        for (int w = 1; w < W; ++w) s += red[w][lane];
    }
    if (GLU) {
        const float u = __shfl(s, lane + 32, 64);   // lane r < 32: the up value of its row
        const int64_t zr = (int64_t)p * kPanelRows + lrow;
        if (lane < 32 && zr < geom.n / 2) y[zr] = act_apply(act, s) * u;
    } else if (ARGMAX) {
        float v = s;
        if (tail.cap > 0.0f) v = tail.cap * tanhf(v / tail.cap);
        v = v + 0.0f;                               // -0 becomes +0: equal logits, equal keys
        unsigned long long key = 0ull;              // below every logit's key
        if (row < geom.n) {
            y[row] = v;
            const uint32_t b = __float_as_uint(v);
            const uint32_t u = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
            key = (static_cast<unsigned long long>(u) << 32) |
                  (0xFFFFFFFFu - static_cast<uint32_t>(row));
        }
        key = wave_max_key(key);
        if (lane == 0) tail.keys[blockIdx.x] = key;
    } else if (row < geom.n) {
        y[row] = s;
    }
}

// (the gated output keeps the grid: two workgroups per gate panel, one per half of its rows)
template <int FMT, int G, int W, bool PARTIALS, bool FUSED, bool ROT, int XQ, bool GLU,
          bool ARGMAX = false>
hipError_t launch_k(const Geom &g, int act, const uint8_t *packed, const float *x, int8_t *xq,
                    float *xs, int32_t *xsum, float *y, int32_t *d, hipStream_t stream,
                    const Tail &tail = Tail{}) {
    const unsigned grid = static_cast<unsigned>(g.n_pad / kPanelRows);
    gemv_kernel<FMT, G, W, PARTIALS, FUSED, ROT, XQ, GLU, ARGMAX><<<grid, 64 * W, 0, stream>>>(
        packed, g, x, xq, xs, xsum, y, d, act, tail);
    return hipGetLastError();
}

template <int FMT, int G, int W, bool PARTIALS, bool FUSED, bool ROT, bool GLU, bool ARGMAX>
hipError_t launch_wk(const Geom &g, int act, const uint8_t *packed, const float *x, int8_t *xq,
                     float *xs, int32_t *xsum, float *y, int32_t *d, hipStream_t stream,
                     const Tail &tail) {
    if (!FUSED)
        return launch_k<FMT, G, W, PARTIALS, FUSED, ROT, 1, GLU, ARGMAX>(
            g, act, packed, x, xq, xs, xsum, y, d, stream, tail);
    // the quads of the largest wavefront share (whole metadata blocks of 4 groups)
    const int nblk = (g.k / G + 3) / 4;
    const int max_quads = (nblk + W - 1) / W * 4 * (G / 4);
    if (max_quads <= 64)
        return launch_k<FMT, G, W, PARTIALS, FUSED, ROT, 1, GLU, ARGMAX>(
            g, act, packed, x, xq, xs, xsum, y, d, stream, tail);
    if (max_quads <= 128)
        return launch_k<FMT, G, W, PARTIALS, FUSED, ROT, 2, GLU, ARGMAX>(
            g, act, packed, x, xq, xs, xsum, y, d, stream, tail);
    if (max_quads <= 256)
        return launch_k<FMT, G, W, PARTIALS, FUSED, ROT, 4, GLU, ARGMAX>(
            g, act, packed, x, xq, xs, xsum, y, d, stream, tail);
    if (max_quads <= 64 * kFusedQuadsPerLane)
        return launch_k<FMT, G, W, PARTIALS, FUSED, ROT, kFusedQuadsPerLane, GLU, ARGMAX>(
            g, act, packed, x, xq, xs, xsum, y, d, stream, tail);
    return hipErrorInvalidValue;
}

template <int FMT, int G, bool PARTIALS, bool FUSED, bool ROT, bool GLU, bool ARGMAX>
hipError_t launch_w(const Geom &g, int act, const uint8_t *packed, const float *x, int8_t *xq,
                    float *xs, int32_t *xsum, float *y, int32_t *d, hipStream_t stream,
                    const Tail &tail) {
    // W = 8 once there are 6 metadata blocks (some wavefronts may own none), else 4.  The fused
    // kernel at exactly 6 blocks takes W = 6, one block per wavefront, so that every wavefront
    // quantizes and loads (the 262144-row head at K = 1536: 33.6 -> 33.0 us; the plain kernel
    // measured no faster with 6)
    if (FUSED && (g.k / G + 3) / 4 == 6)
        return launch_wk<FMT, G, 6, PARTIALS, FUSED, ROT, GLU, ARGMAX>(g, act, packed, x, xq, xs,
                                                                      xsum, y, d, stream, tail);
    if ((g.k / G + 3) / 4 >= 6)
        return launch_wk<FMT, G, 8, PARTIALS, FUSED, ROT, GLU, ARGMAX>(g, act, packed, x, xq, xs,
                                                                      xsum, y, d, stream, tail);
    return launch_wk<FMT, G, 4, PARTIALS, FUSED, ROT, GLU, ARGMAX>(g, act, packed, x, xq, xs,
                                                                  xsum, y, d, stream, tail);
}

template <int FMT, bool PARTIALS, bool FUSED, bool ROT, bool GLU, bool ARGMAX>
hipError_t launch_g(const Geom &g, int act, const uint8_t *packed, const float *x, int8_t *xq,
                    float *xs, int32_t *xsum, float *y, int32_t *d, hipStream_t stream,
                    const Tail &tail) {
    if (g.group == 64)
        return launch_w<FMT, 64, PARTIALS, FUSED, ROT, GLU, ARGMAX>(g, act, packed, x, xq, xs,
                                                                   xsum, y, d, stream, tail);
    return launch_w<FMT, 128, PARTIALS, FUSED, ROT, GLU, ARGMAX>(g, act, packed, x, xq, xs, xsum,
                                                                y, d, stream, tail);
}

template <bool PARTIALS, bool FUSED, bool ROT, bool GLU = false, bool ARGMAX = false>
hipError_t launch_f(const Geom &g, const uint8_t *packed, const float *x, int8_t *xq, float *xs,
                    int32_t *xsum, float *y, int32_t *d, hipStream_t stream, int act = 0,
                    const Tail &tail = Tail{}) {
    switch (g.fmt) {
    case kFmtSym:
        return launch_g<kFmtSym, PARTIALS, FUSED, ROT, GLU, ARGMAX>(g, act, packed, x, xq, xs,
                                                                   xsum, y, d, stream, tail);
    case kFmtAffine:
        return launch_g<kFmtAffine, PARTIALS, FUSED, ROT, GLU, ARGMAX>(g, act, packed, x, xq, xs,
                                                                      xsum, y, d, stream, tail);
    default:
        return launch_g<kFmtCodebook, PARTIALS, FUSED, ROT, GLU, ARGMAX>(g, act, packed, x, xq, xs,
                                                                        xsum, y, d, stream, tail);
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

namespace {
template <int FMT, int G>
hipError_t launch_argmax_w(const Geom &g, const uint8_t *packed, const int8_t *xq,
                           const float *xs, const int32_t *xsum, float *y, const Tail &tail,
                           hipStream_t stream) {
    int8_t *q = const_cast<int8_t *>(xq);
    float *s = const_cast<float *>(xs);
    int32_t *u = const_cast<int32_t *>(xsum);
    if ((g.k / G + 3) / 4 >= 6)
        return launch_k<FMT, G, 8, false, false, false, 1, false, true>(g, 0, packed, nullptr, q,
                                                                        s, u, y, nullptr, stream,
                                                                        tail);
    return launch_k<FMT, G, 4, false, false, false, 1, false, true>(g, 0, packed, nullptr, q, s,
                                                                    u, y, nullptr, stream, tail);
}

template <int FMT>
hipError_t launch_argmax_g(const Geom &g, const uint8_t *packed, const int8_t *xq,
                           const float *xs, const int32_t *xsum, float *y, const Tail &tail,
                           hipStream_t stream) {
    if (g.group == 64) return launch_argmax_w<FMT, 64>(g, packed, xq, xs, xsum, y, tail, stream);
    return launch_argmax_w<FMT, 128>(g, packed, xq, xs, xsum, y, tail, stream);
}
}  // namespace

hipError_t launch_gemv_argmax(const Geom &g, const uint8_t *packed, const int8_t *xq,
                              const float *xs, const int32_t *xsum, float *y, const Tail &tail,
                              hipStream_t stream) {
    hipError_t e;
    switch (g.fmt) {
    case kFmtSym: e = launch_argmax_g<kFmtSym>(g, packed, xq, xs, xsum, y, tail, stream); break;
    case kFmtAffine:
        e = launch_argmax_g<kFmtAffine>(g, packed, xq, xs, xsum, y, tail, stream);
        break;
    default: e = launch_argmax_g<kFmtCodebook>(g, packed, xq, xs, xsum, y, tail, stream); break;
    }
    if (e != hipSuccess) return e;
    return launch_argmax_keys(tail.keys, g.n_pad / kPanelRows, tail.token, tail.value, stream);
}

hipError_t launch_gemv_argmax_fused(const Geom &g, const uint8_t *packed, const float *x,
                                    int hadamard, int8_t *xq, float *xs, int32_t *xsum, float *y,
                                    const Tail &tail, hipStream_t stream) {
    const hipError_t e =
        hadamard ? launch_f<false, true, true, false, true>(g, packed, x, xq, xs, xsum, y, nullptr,
                                                            stream, 0, tail)
                 : launch_f<false, true, false, false, true>(g, packed, x, xq, xs, xsum, y,
                                                             nullptr, stream, 0, tail);
    if (e != hipSuccess) return e;
    return launch_argmax_keys(tail.keys, g.n_pad / kPanelRows, tail.token, tail.value, stream);
}

hipError_t launch_gemv_glu(const Geom &g, int act, const uint8_t *packed, const int8_t *xq,
                           const float *xs, const int32_t *xsum, float *y, hipStream_t stream) {
    int8_t *q = const_cast<int8_t *>(xq);
    float *s = const_cast<float *>(xs);
    int32_t *u = const_cast<int32_t *>(xsum);
    return launch_f<false, false, false, true>(g, packed, nullptr, q, s, u, y, nullptr, stream,
                                               act);
}

hipError_t launch_gemv_glu_fused(const Geom &g, int act, const uint8_t *packed, const float *x,
                                 int hadamard, int8_t *xq, float *xs, int32_t *xsum, float *y,
                                 hipStream_t stream) {
    if (hadamard)
        return launch_f<false, true, true, true>(g, packed, x, xq, xs, xsum, y, nullptr, stream,
                                                 act);
    return launch_f<false, true, false, true>(g, packed, x, xq, xs, xsum, y, nullptr, stream, act);
}

}  // namespace w4a8
