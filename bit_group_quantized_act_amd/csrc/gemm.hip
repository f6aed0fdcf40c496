// Prefill GEMM (m activation rows) over the packed 4-bit weights with int8 MFMA.
//
// Sources: "cactus PR #697", section "Quantized matmul" (the M>1 fused GEMM accumulates raw int32
// partials per group in the matrix unit and rescales them per tile in a vector epilogue, with
// several accumulator tiles in flight); "geistlib issue #500", sections "Why" and "Design" (a
// native int8 GEMM removes the dequantize-to-fp32 intermediate of prefill); "TensorFold PR
// #3215" (the affine bias term uses the per-row group sums from the prepass).
//
// MI355X design.
//   Tiles.  A workgroup of 4 wavefronts owns BM activation rows (128 or 64) and BN = 128*64/BM
//   output channels; each wavefront owns 64 rows x 32 channels as two 32x32 int32 tiles that
//   share one weight fragment.  Lane l of a tile holds activation row l%32 and k half l/32; the
//   weight chunk of lane l is panel row l%32 of the wavefront's 32 channels at chunk 2q + l/32,
//   so a tile's weight fragment is two contiguous 512-byte runs of the packed panel.  The low
//   nibbles of the chunk are k 0..15 and pair with the lane's first 16 activation bytes, the
//   high nibbles k 16..31 with the next 16 (the same k on both sides, which is all the MFMA
//   needs): two v_mfma_i32_32x32x32_i8 per tile per 64-wide k step, operands straight from the
//   loads.
//   Loads.  Every operand comes through buffer loads (SGPR descriptor, one fixed VGPR offset per
//   lane, the k step in the SGPR offset), so the loop does no VALU address arithmetic, and rows
//   past m read as zeros (the descriptor's range check) instead of being predicated.  Operands
//   are prefetched in registers (weights 4 k steps ahead, activations 2) to hide latency.
//   Epilogue per group.  The int32 partials of a group are converted once and accumulated with
//   one FMA each.  Their coefficients xs[row] * sw[col] come from one fp32 outer-product MFMA
//   (v_mfma_f32_32x32x1_2b: block t = tile t), which also lands each coefficient in the lane and
//   register of its partial; the affine bias term xs*xsum[row] * (bw + 8 sw)[col] is a second
//   outer product accumulated straight into its own fp32 tile on the matrix unit.  So the VALU
//   does two operations per element and group, the matrix unit the rest.
//   Signed codes (sym q, affine u-8) enter the MFMA as 16*q (nibble moved to the byte's top);
//   the 1/16 is folded into sw, and affine's u = (u-8) + 8 is restored through the bias term.
#include "w4a8_kernels.h"

#include <type_traits>

namespace w4a8 {
namespace {

constexpr int kWaves = 4;
constexpr int kDepthA = 2;     // k steps of activation operands in flight per wavefront
constexpr int kDepthB = 4;     // k steps of weight chunks in flight per wavefront
constexpr uint32_t kRsrcCfg = 0x00020000u;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint64_t bytes) {
    const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : static_cast<uint32_t>(bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, kRsrcCfg);
}

__device__ __forceinline__ v4i ld128(rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t ld32(rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ld16(rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
}

template <int FMT>
__device__ __forceinline__ void unpack_b(v4i v, uint4 cb, v4i &lo, v4i &hi) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w = static_cast<uint32_t>(v[j]);
        if (FMT == kFmtCodebook) {
            lo[j] = static_cast<int>(cb_lo(w, cb));
            hi[j] = static_cast<int>(cb_hi(w, cb));
        } else {
            lo[j] = static_cast<int>(lo_x16(w));
            hi[j] = static_cast<int>(hi_x16(w));
        }
    }
}

template <int FMT, int G, int BM, bool PARTIALS>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t *__restrict__ packed,
                                                   const Geom geom, int m,
                                                   const int8_t *__restrict__ xq,
                                                   const float *__restrict__ xs,
                                                   const int *__restrict__ xsum,
                                                   float *__restrict__ y,
                                                   int *__restrict__ d) {
    constexpr int kWavesM = BM / 64;
    constexpr int kWavesN = kWaves / kWavesM;
    constexpr int kBN = 32 * kWavesN;
    constexpr int kStepsPerGroup = G / 64;
    static_assert(kDepthB == 4 && kDepthB % kDepthA == 0 && kDepthA % kStepsPerGroup == 0,
                  "the unrolled loop body assumes 4 weight slots aligned to groups");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int r0 = blockIdx.y * BM + wm * 64;            // first activation row of the wavefront
    const int c0 = blockIdx.x * kBN + wn * 32;           // first output channel of the wavefront
    if (r0 >= m || c0 >= geom.n_pad) return;             // no barriers below
    const int p = c0 / kPanelRows;                       // its panel
    const int prow = (c0 % kPanelRows) + (lane & 31);    // lane's channel row inside the panel
    const int k = geom.k;
    const int kc = k / kChunkK;
    const int ng = k / G;
    const int nsteps = k / 64;
    const int half = lane >> 5;
    const int r32 = lane & 31;
    const int rows = min(m - r0, 64);                    // valid rows of the wavefront
    constexpr int mb = (FMT == kFmtAffine) ? 4 : 2;       // meta bytes per channel and group

    // descriptors rebased at the wavefront's rows / panel: offsets stay far below 2^31 and
    // anything past the valid range reads as zero
    const rsrc_t rq = make_rsrc(xq + (int64_t)r0 * k, (uint64_t)rows * k);
    const rsrc_t rw = make_rsrc(packed + geom.off_codes + (int64_t)p * kc * 1024,
                                (uint64_t)kc * 1024);
    const rsrc_t rm = make_rsrc(packed + geom.off_meta + (int64_t)p * ng * kPanelRows * mb,
                                (uint64_t)ng * kPanelRows * mb);
    const rsrc_t rs = make_rsrc(xs + (int64_t)r0 * ng, (uint64_t)rows * ng * 4);
    const rsrc_t rx = make_rsrc(xsum + (int64_t)r0 * ng, (uint64_t)rows * ng * 4);

    // per-lane constant offsets (bytes); the k step goes into the SGPR offset
    const int a_off0 = r32 * k + 32 * half;                      // tile 0 row, chunk half
    const int a_off1 = a_off0 + 32 * k;                          // tile 1 row
    const int w_off = half * 1024 + prow * 16;
    const int meta_off = prow * mb;
    const int s_off = lane * ng * 4;                             // row r0 + lane (outer products)

    uint4 cb = make_uint4(0u, 0u, 0u, 0u);
    if (FMT == kFmtCodebook) {
        const uint4 *cbp = reinterpret_cast<const uint4 *>(packed + geom.off_codebook);
        cb = cbp[(int64_t)p * kPanelRows + prow];
    }

    // Two load rings: activation operands (L2 resident) kDepthA steps ahead, weight chunks and
    // their metadata (HBM) kDepthB steps ahead.  Loads are unconditional (past the last step the
    // step index is clamped, re-reading it from cache), so the counted waits stay exact.
    v4i ra[kDepthA][2][2];      // [slot][tile][16-byte half]: 32 activation bytes per tile
    float rxs[kDepthA];         // activation scale of row r0 + lane, the step's group
    int rxsum[kDepthA];         // its group sum (affine)
    v4i rb[kDepthB];            // 16 weight bytes of the lane's channel
    uint32_t rmeta[kDepthB];    // fp16 scale (| fp16 bias << 16) of the lane's channel
    auto load_a = [&](int slot, int step) {
        step = min(step, nsteps - 1);
        const int soff = step * 64;
        ra[slot][0][0] = ld128(rq, a_off0, soff);
        ra[slot][0][1] = ld128(rq, a_off0 + 16, soff);
        ra[slot][1][0] = ld128(rq, a_off1, soff);
        ra[slot][1][1] = ld128(rq, a_off1 + 16, soff);
        if (!PARTIALS) {
            const int g = step / kStepsPerGroup;
            rxs[slot] = __builtin_bit_cast(float, ld32(rs, s_off, g * 4));
            if (FMT == kFmtAffine) rxsum[slot] = static_cast<int>(ld32(rx, s_off, g * 4));
        }
    };
    auto load_b = [&](int slot, int step) {
        step = min(step, nsteps - 1);
        rb[slot] = ld128(rw, w_off, step * 2048);
        if (!PARTIALS) {
            const int g = step / kStepsPerGroup;
            rmeta[slot] = (mb == 4) ? ld32(rm, meta_off, g * kPanelRows * 4)
                                    : ld16(rm, meta_off, g * kPanelRows * 2);
        }
    };
#pragma unroll
    for (int i = 0; i < kDepthB; ++i) load_b(i, i);
#pragma unroll
    for (int i = 0; i < kDepthA; ++i) load_a(i, i);

    v32f acc = {};     // [tile][16]: fp32 output accumulators (bias term included)
    v16i dt0 = {}, dt1 = {};

    // One 64-wide k step whose operands sit in ring slots I % kDepthA and I % kDepthB; both slots
    // are refilled right after the MFMAs have taken their operands (the scheduling barriers keep
    // the compiler from sinking those loads to the end of the loop).
    auto body = [&](auto I, int s) {
        constexpr int i = decltype(I)::value;
        constexpr int sa = i % kDepthA, sb = i % kDepthB;
        constexpr bool first = (i % kStepsPerGroup) == 0;
        constexpr bool last = (i % kStepsPerGroup) == kStepsPerGroup - 1;
        v4i blo, bhi;
        unpack_b<FMT>(rb[sb], cb, blo, bhi);
        const v16i z = {};
        dt0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ra[sa][0][0], blo, first ? z : dt0, 0, 0, 0);
        dt1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ra[sa][1][0], blo, first ? z : dt1, 0, 0, 0);
        dt0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ra[sa][0][1], bhi, dt0, 0, 0, 0);
        dt1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ra[sa][1][1], bhi, dt1, 0, 0, 0);
        const uint32_t meta = rmeta[sb];
        const float xs_l = rxs[sa];
        const int xsum_l = rxsum[sa];
        __builtin_amdgcn_sched_barrier(0);
        load_b(sb, s + kDepthB);
        load_a(sa, s + kDepthA);
        __builtin_amdgcn_sched_barrier(0);
        if (!last) return;
        const int g = s / kStepsPerGroup;

        if (PARTIALS) {
            // element e of tile t: row r0 + 32t + 8(e/4) + 4*half + e%4, channel c0 + r32
            const int col = c0 + r32;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = r0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
                    const int raw = t ? dt1[e] : dt0[e];
                    if (row >= m || col >= geom.n) continue;
                    int v = (FMT == kFmtCodebook) ? raw : (raw >> 4);
                    if (FMT == kFmtAffine) v += 8 * xsum[(int64_t)row * ng + g];
                    d[((int64_t)row * geom.n + col) * ng + g] = v;
                }
            }
            return;
        }

        const float sw = half_bits_to_float(meta & 0xFFFFu);
        const float sw16 = (FMT == kFmtCodebook) ? sw : sw * 0.0625f;
        const v32f zf = {};
        const v32f coef = __builtin_amdgcn_mfma_f32_32x32x1f32(xs_l, sw16, zf, 0, 0, 0);
        if (FMT == kFmtAffine) {
            // sum_g xs*xsum[row] * (bw + 8 sw)[col]: bias plus the u = (u-8) + 8 correction
            const float b2 = fmaf(8.0f, sw, half_bits_to_float(meta >> 16));
            acc = __builtin_amdgcn_mfma_f32_32x32x1f32(xs_l * static_cast<float>(xsum_l), b2, acc,
                                                       0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            acc[e] = fmaf(static_cast<float>(dt0[e]), coef[e], acc[e]);
            acc[16 + e] = fmaf(static_cast<float>(dt1[e]), coef[16 + e], acc[16 + e]);
        }
    };

    constexpr int kUnroll = kDepthB;   // a multiple of kDepthA and of the steps per group
    int s0 = 0;
    for (; s0 + kUnroll <= nsteps; s0 += kUnroll) {
        body(std::integral_constant<int, 0>(), s0);
        body(std::integral_constant<int, 1>(), s0 + 1);
        body(std::integral_constant<int, 2>(), s0 + 2);
        body(std::integral_constant<int, 3>(), s0 + 3);
    }
    // remaining steps (fewer than kUnroll, a whole number of groups) use slots 0, 1, 2
    if (s0 < nsteps) body(std::integral_constant<int, 0>(), s0);
    if (s0 + 1 < nsteps) body(std::integral_constant<int, 1>(), s0 + 1);
    if (s0 + 2 < nsteps) body(std::integral_constant<int, 2>(), s0 + 2);
    if (PARTIALS) return;

    const int col = c0 + r32;
    if (col >= geom.n) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = r0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
            if (row >= m) continue;
            y[(int64_t)row * geom.n + col] = acc[16 * t + e];
        }
    }
}

template <int FMT, int G, bool PARTIALS>
hipError_t launch_bm(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                     const float *xs, const int32_t *xsum, float *y, int32_t *d,
                     hipStream_t stream) {
    if (m <= 64) {
        const dim3 grid(static_cast<unsigned>(g.n_pad / 128 + (g.n_pad % 128 ? 1 : 0)), 1);
        gemm_kernel<FMT, G, 64, PARTIALS><<<grid, 256, 0, stream>>>(packed, g, m, xq, xs, xsum, y, d);
    } else {
        const dim3 grid(static_cast<unsigned>(g.n_pad / 64), static_cast<unsigned>((m + 127) / 128));
        gemm_kernel<FMT, G, 128, PARTIALS><<<grid, 256, 0, stream>>>(packed, g, m, xq, xs, xsum, y, d);
    }
    return hipGetLastError();
}

template <int FMT, bool PARTIALS>
hipError_t launch_g(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                    const float *xs, const int32_t *xsum, float *y, int32_t *d,
                    hipStream_t stream) {
    if (g.group == 64) return launch_bm<FMT, 64, PARTIALS>(g, packed, m, xq, xs, xsum, y, d, stream);
    return launch_bm<FMT, 128, PARTIALS>(g, packed, m, xq, xs, xsum, y, d, stream);
}

template <bool PARTIALS>
hipError_t launch_f(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                    const float *xs, const int32_t *xsum, float *y, int32_t *d,
                    hipStream_t stream) {
    switch (g.fmt) {
    case kFmtSym: return launch_g<kFmtSym, PARTIALS>(g, packed, m, xq, xs, xsum, y, d, stream);
    case kFmtAffine:
        return launch_g<kFmtAffine, PARTIALS>(g, packed, m, xq, xs, xsum, y, d, stream);
    default: return launch_g<kFmtCodebook, PARTIALS>(g, packed, m, xq, xs, xsum, y, d, stream);
    }
}

}  // namespace

hipError_t launch_gemm(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                       const float *xs, const int32_t *xsum, float *y, int32_t *d,
                       hipStream_t stream) {
    if (m == 0) return hipSuccess;
    if (d) return launch_f<true>(g, packed, m, xq, xs, xsum, nullptr, d, stream);
    return launch_f<false>(g, packed, m, xq, xs, xsum, y, nullptr, stream);
}

}  // namespace w4a8
