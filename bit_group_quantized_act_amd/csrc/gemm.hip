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
constexpr int kDepthB = 4;       // k steps of weight chunks in flight per wavefront
constexpr int kStageSteps = 2;   // 64-wide k steps per LDS activation stage
constexpr int kStageK = 64 * kStageSteps;
constexpr int kLdsRow = kStageK + 16;   // padded LDS row of one activation stage (bytes)
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
    constexpr int mb = (FMT == kFmtAffine) ? 4 : 2;       // meta bytes per channel and group
    static_assert(kDepthB == 4 && kStageSteps == 2 && kDepthB % kStepsPerGroup == 0,
                  "the unrolled loop assumes 4 weight slots and 2-step LDS stages");
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * kLdsRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    const int m0 = blockIdx.y * BM;                      // first activation row of the workgroup
    const int r0 = m0 + wm * 64;                         // first activation row of the wavefront
    const int c0 = blockIdx.x * kBN + wn * 32;           // first output channel of the wavefront
    const bool active = r0 < m && c0 < geom.n_pad;       // wave-uniform
    const int p = c0 / kPanelRows;                       // the wavefront's panel
    const int prow = (c0 % kPanelRows) + (lane & 31);    // lane's channel row inside the panel
    const int k = geom.k;
    const int kc = k / kChunkK;
    const int ng = k / G;
    const int nsteps = k / 64;
    const int nstages = (nsteps + kStageSteps - 1) / kStageSteps;
    const int half = lane >> 5;
    const int r32 = lane & 31;
    const int rows_wg = min(m - m0, BM);                 // valid rows of the workgroup

    // Descriptors rebased at the workgroup's rows / the wavefront's panel: offsets stay far below
    // 2^31 and anything past the valid range reads as zero without touching memory.
    const rsrc_t rq = make_rsrc(xq + (int64_t)m0 * k, (uint64_t)rows_wg * k);
    const uint8_t *wbase = active ? packed + geom.off_codes + (int64_t)p * kc * 1024 : packed;
    const rsrc_t rw = make_rsrc(wbase, active ? (uint64_t)kc * 1024 : 0);
    const uint8_t *mbase =
        active ? packed + geom.off_meta + (int64_t)p * ng * kPanelRows * mb : packed;
    const rsrc_t rm = make_rsrc(mbase, active ? (uint64_t)ng * kPanelRows * mb : 0);
    const int w_off = half * 1024 + prow * 16;
    const int meta_off = prow * mb;

    uint4 cb = make_uint4(0u, 0u, 0u, 0u);
    if (FMT == kFmtCodebook && active) {
        const uint4 *cbp = reinterpret_cast<const uint4 *>(packed + geom.off_codebook);
        cb = cbp[(int64_t)p * kPanelRows + prow];
    }

    // ---- activation tiles: global -> registers -> LDS, one 128-wide k stage at a time.  Thread
    // t moves 16 bytes of row 32j + t/8 per j, eight threads per 128-byte row segment (whole
    // cache lines); LDS rows are padded to 144 bytes so the MFMA-layout reads below (32 rows at
    // one k offset per half wavefront) spread over the banks.
    constexpr int kAJ = BM / 32;
    v4i stage_regs[kAJ];
    const int a_row = tid >> 3, a_piece = tid & 7;
    auto stage_load = [&](int st) {
        st = min(st, nstages - 1);
#pragma unroll
        for (int j = 0; j < kAJ; ++j)
            stage_regs[j] = ld128(rq, (32 * j + a_row) * k + a_piece * 16, st * kStageK);
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kAJ; ++j)
            *reinterpret_cast<v4i *>(&lds_a[buf][(32 * j + a_row) * kLdsRow + a_piece * 16]) =
                stage_regs[j];
    };
    // LDS offset of this lane's MFMA operands: row wm*64 + 32t + r32, k bytes 32*half + 16*h of
    // the 64-wide step
    const int a_lds = (wm * 64 + r32) * kLdsRow + 32 * half;

    // ---- weight chunks and per-group metadata: a ring of kDepthB k steps in registers
    v4i rb[kDepthB];            // 16 weight bytes of the lane's channel
    uint32_t rmeta[kDepthB];    // fp16 scale (| fp16 bias << 16) of the lane's channel
    float rxs[kDepthB];         // activation scale of row r0 + lane, the step's group
    int rxsum[kDepthB];         // its group sum (affine)
    const int x_off = (r0 + lane) * 4;                   // row of the outer-product operands
    auto load_b = [&](int slot, int step) {
        step = min(step, nsteps - 1);
        rb[slot] = ld128(rw, w_off, step * 2048);
        if (!PARTIALS) {
            const int g = step / kStepsPerGroup;
            rmeta[slot] = (mb == 4) ? ld32(rm, meta_off, g * kPanelRows * 4)
                                    : ld16(rm, meta_off, g * kPanelRows * 2);
            // group-major scales and sums: one descriptor per group column, rows >= m read 0
            const rsrc_t rs = make_rsrc(xs + (int64_t)g * m, (uint64_t)m * 4);
            rxs[slot] = __builtin_bit_cast(float, ld32(rs, x_off, 0));
            if (FMT == kFmtAffine) {
                const rsrc_t rx = make_rsrc(xsum + (int64_t)g * m, (uint64_t)m * 4);
                rxsum[slot] = static_cast<int>(ld32(rx, x_off, 0));
            }
        }
    };

    stage_load(0);
    stage_store(0);
    stage_load(1);
#pragma unroll
    for (int i = 0; i < kDepthB; ++i) load_b(i, i);
    __syncthreads();

    v32f acc = {};     // [tile][16]: fp32 output accumulators (bias term included)
    v16i dt0 = {}, dt1 = {};

    // One 64-wide k step: weights from ring slot I, activations from LDS buffer (I/2)%2, which
    // holds stage s/2.  The ring slot is refilled right after the MFMAs have taken their operands
    // (the scheduling barriers keep the compiler from sinking those loads to the loop's end).
    auto body = [&](auto I, int s) {
        constexpr int i = decltype(I)::value;
        constexpr int buf = (i / kStageSteps) % 2;
        constexpr int sub = i % kStageSteps;
        constexpr bool first = (i % kStepsPerGroup) == 0;
        constexpr bool last = (i % kStepsPerGroup) == kStepsPerGroup - 1;
        if (!active) return;
        const uint8_t *ab = &lds_a[buf][a_lds + sub * 64];
        const v4i a00 = *reinterpret_cast<const v4i *>(ab);
        const v4i a01 = *reinterpret_cast<const v4i *>(ab + 16);
        const v4i a10 = *reinterpret_cast<const v4i *>(ab + 32 * kLdsRow);
        const v4i a11 = *reinterpret_cast<const v4i *>(ab + 32 * kLdsRow + 16);
        v4i blo, bhi;
        unpack_b<FMT>(rb[i], cb, blo, bhi);
        // everything read from ring slot i is consumed before the slot is refilled, so the refill
        // loads can land in the same registers with no copies (and no early wait)
        const uint32_t meta = rmeta[i];
        const float sw = half_bits_to_float(meta & 0xFFFFu);
        const float sw16 = (FMT == kFmtCodebook) ? sw : sw * 0.0625f;
        const float xs_l = rxs[i];
        float b2 = 0.0f, xs_sum = 0.0f;
        if (FMT == kFmtAffine) {
            b2 = fmaf(8.0f, sw, half_bits_to_float(meta >> 16));
            xs_sum = xs_l * static_cast<float>(rxsum[i]);
        }
        const v16i z = {};
        dt0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a00, blo, first ? z : dt0, 0, 0, 0);
        dt1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a10, blo, first ? z : dt1, 0, 0, 0);
        dt0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a01, bhi, dt0, 0, 0, 0);
        dt1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a11, bhi, dt1, 0, 0, 0);
        // coefficient tiles xs[row] * sw16[col] for the group's epilogue
        v32f coef = {};
        if (!PARTIALS && last) {
            const v32f zf = {};
            coef = __builtin_amdgcn_mfma_f32_32x32x1f32(xs_l, sw16, zf, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        load_b(i, s + kDepthB);
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
                    if (FMT == kFmtAffine) v += 8 * xsum[(int64_t)g * m + row];
                    d[((int64_t)row * geom.n + col) * ng + g] = v;
                }
            }
            return;
        }

        if (FMT == kFmtAffine) {
            // sum_g xs*xsum[row] * (bw + 8 sw)[col]: bias plus the u = (u-8) + 8 correction
            acc = __builtin_amdgcn_mfma_f32_32x32x1f32(xs_sum, b2, acc, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            acc[e] = fmaf(static_cast<float>(dt0[e]), coef[e], acc[e]);
            acc[16 + e] = fmaf(static_cast<float>(dt1[e]), coef[16 + e], acc[16 + e]);
        }
    };
    // After the two steps of stage st: publish stage st+1 (loaded one stage ago) into the buffer
    // stage st-1 used, fetch stage st+2, and let every wavefront see the new buffer.
    auto stage_end = [&](int st) {
        stage_store((st + 1) & 1);
        stage_load(st + 2);
        __syncthreads();
    };

    int s = 0;
    for (; s + 4 <= nsteps; s += 4) {
        body(std::integral_constant<int, 0>(), s);
        body(std::integral_constant<int, 1>(), s + 1);
        stage_end(s / 2);
        body(std::integral_constant<int, 2>(), s + 2);
        body(std::integral_constant<int, 3>(), s + 3);
        stage_end(s / 2 + 1);
    }
    // remaining steps (fewer than 4; a whole number of groups)
    if (s < nsteps) body(std::integral_constant<int, 0>(), s);
    if (s + 1 < nsteps) body(std::integral_constant<int, 1>(), s + 1);
    if (s + 2 < nsteps) {
        stage_end(s / 2);
        body(std::integral_constant<int, 2>(), s + 2);
    }
    if (PARTIALS || !active) return;

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
