// Prefill GEMM (m activation rows) over the packed 4-bit weights with int8 MFMA.
//
// Sources: "cactus PR #697", section "Quantized matmul" (the M>1 fused GEMM accumulates raw int32
// partials per group in the matrix unit and rescales them per tile in a vector epilogue, with
// several accumulator tiles in flight); "geistlib issue #500", sections "Why" and "Design" (a
// native int8 GEMM removes the dequantize-to-fp32 intermediate of prefill); "TensorFold PR
// #3215" (the affine bias term uses the per-row group sums from the prepass).
//
// MI355X design.
//   Tiles.  A workgroup of 4 wavefronts owns 64 activation rows and 128 output channels; each
//   wavefront owns all 64 rows x its own 32 channels as two 32x32 int32 tiles that share one
//   weight fragment, so no two wavefronts load the same weight bytes.  Lane l of a tile holds
//   activation row l%32 and k half l/32; the weight chunk of lane l is panel row l%32 of the
//   wavefront's 32 channels at chunk 2q + l/32, so a tile's weight fragment is two contiguous
//   512-byte runs of the packed panel.  The low nibbles of the chunk are k 0..15 and pair with
//   the lane's first 16 activation bytes, the high nibbles k 16..31 with the next 16 (the same k
//   on both sides, which is all the MFMA needs): two v_mfma_i32_32x32x32_i8 per tile per 64-wide
//   k step.  Workgroups are numbered so that each XCD (one L2) gets a contiguous run of tiles,
//   with the M tiles of one channel block adjacent: they share its weights in that L2.
//   Loads.  Every operand comes through buffer loads (SGPR descriptor, one fixed VGPR offset per
//   lane, the k step in the SGPR offset), so rows past m read as zeros (the descriptor's range
//   check) instead of being predicated.  Activations are staged through LDS in 128-wide k
//   stages from three register sets loaded three stages ahead (three LDS buffers, one barrier
//   per stage); weight chunks and per-group metadata are loaded six k steps ahead.  Loads
//   complete in issue order, so the two leads are matched (a wait for one load never forces a
//   much younger one), and no load sits behind a branch (the compiler's waits would otherwise
//   drain every load in flight): this keeps ~48 KiB of weights in flight per CU.
//   Software pipeline.  The epilogue of group g-1 runs on the VALU, tile by tile, between the
//   MFMAs of group g: the int32 partials of a tile are converted and accumulated with one FMA
//   each, and that tile's MFMAs for group g are issued right after its last read.  The FMA
//   coefficients xs[row] * sw[col] come from one fp32 outer-product MFMA
//   (v_mfma_f32_32x32x1_2b: block t = tile t) issued as soon as the previous group's
//   coefficients are consumed, which also lands each coefficient in the lane and register of
//   its partial.  The affine bias term xs*xsum[row] * (bw + 8 sw)[col] is a second outer
//   product accumulated on the matrix unit into its own fp32 tile.  So per element and group the
//   VALU does two operations and the matrix unit the rest.
//   Signed codes (sym q, affine u-8) enter the MFMA as 16*q (nibble moved to the byte's top);
//   the 1/16 is folded into sw, and affine's u = (u-8) + 8 is restored through the bias term.
#include "w4a8_kernels.h"

#include <type_traits>

namespace w4a8 {
namespace {

constexpr int BM = 64;                     // activation rows per workgroup
constexpr int kBN = 128;                   // output channels per workgroup (4 wavefronts x 32)
constexpr int kStageSteps = 2;             // 64-wide k steps per LDS activation stage
constexpr int kStageK = 64 * kStageSteps;
constexpr int kLdsRow = kStageK + 16;      // padded LDS row of one activation stage (bytes)
constexpr int kSets = 3;                   // activation stages in flight (registers and LDS)
constexpr int kLead = kSets * kStageSteps; // k steps of weights and metadata loaded ahead
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

template <int FMT, int G, bool PARTIALS>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const uint8_t *__restrict__ packed,
                                                      const Geom geom, int m,
                                                      const int8_t *__restrict__ xq,
                                                      const float *__restrict__ xs,
                                                      const int *__restrict__ xsum,
                                                      float *__restrict__ y,
                                                      int *__restrict__ d) {
    constexpr int SPG = G / 64;                          // 64-wide k steps per group
    constexpr int GPSt = kStageSteps / SPG;              // groups per activation stage
    constexpr int kMD = 16 * (FMT == kFmtAffine ? 4 : 2); // meta dwords per panel and group
    constexpr int kMB = (FMT == kFmtAffine) ? 4 : 2;     // meta bytes per channel and group
    constexpr int kAJ = BM / 32;                         // 16-byte staging loads per thread
    static_assert(kLead == 6 && kStageSteps == 2 && kLead % SPG == 0,
                  "the unrolled loop covers three stages of two k steps");
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[kSets][BM * kLdsRow];
    // per stage: activation scales and sums of the workgroup's rows ([xs|xsum][group][row]) and
    // the weight metadata of its two panels ([group][panel][row]), one dword per thread
    __shared__ uint32_t lds_x[kSets][256];
    __shared__ uint32_t lds_m[kSets][256];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wn = wave;

    // Tile of this workgroup.  When the tile count is a multiple of the 8 XCDs, workgroup b runs
    // on XCD b % 8 and takes tile (b % 8) * (T / 8) + b / 8, so each XCD walks a contiguous run.
    const int tiles_m = (m + BM - 1) / BM;
    const int tiles_n = (geom.n_pad + kBN - 1) / kBN;
    const int ntiles = tiles_m * tiles_n;
    int bid = blockIdx.x;
    if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
    const int mt = bid % tiles_m, nt = bid / tiles_m;

    const int m0 = mt * BM;                              // first activation row of the workgroup
    const int r0 = m0;                                   // first activation row of the wavefront
    const int c0 = nt * kBN + wn * 32;                   // first output channel of the wavefront
    const bool active = r0 < m && c0 < geom.n_pad;       // wave-uniform
    const int p = c0 / kPanelRows;                       // the wavefront's panel
    const int half = lane >> 5;
    const int r32 = lane & 31;
    const int prow = (c0 % kPanelRows) + r32;            // lane's channel row inside the panel
    const int k = geom.k;
    const int kc = k / kChunkK;
    const int ng = k / G;
    const int nsteps = k / 64;
    const int rows_wg = min(m - m0, BM);                 // valid rows of the workgroup

    // Descriptors rebased at the workgroup's rows / the wavefront's panel: offsets stay far below
    // 2^31 and anything past the valid range reads as zero without touching memory.
    const rsrc_t rq = make_rsrc(xq + (int64_t)m0 * k, (uint64_t)rows_wg * k);
    const uint8_t *wbase = active ? packed + geom.off_codes + (int64_t)p * kc * 1024 : packed;
    const rsrc_t rw = make_rsrc(wbase, active ? (uint64_t)kc * 1024 : 0);
    const int w_off = half * 1024 + prow * 16;

    uint4 cb = make_uint4(0u, 0u, 0u, 0u);
    if (FMT == kFmtCodebook && active) {
        const uint4 *cbp = reinterpret_cast<const uint4 *>(packed + geom.off_codebook);
        cb = cbp[(int64_t)p * kPanelRows + prow];
    }

    // ---- activation stages: global -> register set -> LDS.  Thread t moves 16 bytes of row
    // 32j + t/8 per j, eight threads per 128-byte row segment (whole cache lines).  LDS rows are
    // padded to 144 bytes so the MFMA-layout reads (32 rows at one k offset per half wavefront)
    // spread over the banks.
    v4i stage_regs[kSets][kAJ];
    uint32_t stage_x[kSets], stage_m[kSets];
    const int a_row = tid >> 3, a_piece = tid & 7;
    // Metadata staging: wave w loads xs (w < 2) or xsum (w >= 2) of group w & 1 of the stage for
    // the 64 rows (one dword per lane), and thread t loads dword t of the stage's weight metadata
    // block [group][panel][row] of the workgroup's two panels.  Loads that fall outside the data
    // get an out-of-range offset (zeros, no memory access) instead of a branch.
    constexpr uint32_t kOOB = 0x7FFFFFF0u;
    const int x_which = wave >> 1, x_j = wave & 1;
    const bool x_valid = x_j < GPSt && (x_which == 0 || FMT == kFmtAffine);
    const int m_j = tid / (2 * kMD), m_pnl = (tid / kMD) & 1, m_d = tid % kMD;
    const int wg_p0 = nt * (kBN / kPanelRows);           // first panel of the workgroup
    const int wg_np = min(kBN / kPanelRows, geom.n_pad / kPanelRows - wg_p0);
    const rsrc_t rmw = make_rsrc(packed + geom.off_meta + (int64_t)wg_p0 * ng * kPanelRows * kMB,
                                 (uint64_t)wg_np * ng * kPanelRows * kMB);
    // Every load in the main loop is issued unconditionally (a stage or step past the end reads
    // zeros through the range check, or a clamped valid address): the waits the compiler places
    // for one load then count exactly the loads issued after it, which keeps the deep prefetch
    // in flight.  A load behind a branch would make those waits drain everything.
    auto stage_load = [&](auto SET, int st) {
        constexpr int set = decltype(SET)::value;
#pragma unroll
        for (int j = 0; j < kAJ; ++j)
            stage_regs[set][j] = ld128(rq, (32 * j + a_row) * k + a_piece * 16, st * kStageK);
        const int gb = st * GPSt;                        // first group of the stage
        const int gv = max(0, min(GPSt, ng - gb));       // its groups that exist
        const float *xbase = x_which ? reinterpret_cast<const float *>(xsum) : xs;
        const rsrc_t rx = make_rsrc(xbase + (int64_t)min(gb, ng - 1) * m, (uint64_t)gv * m * 4);
        stage_x[set] = ld32(rx, x_valid ? (x_j * m + m0 + lane) * 4 : (int)kOOB, 0);
        const bool mv = m_j < gv;
        stage_m[set] = ld32(rmw, mv ? ((m_pnl * ng + gb + m_j) * kPanelRows * kMB + m_d * 4)
                                    : (int)kOOB, 0);
    };
    auto stage_store = [&](auto SET) {
        constexpr int set = decltype(SET)::value;
#pragma unroll
        for (int j = 0; j < kAJ; ++j)
            *reinterpret_cast<v4i *>(&lds_a[set][(32 * j + a_row) * kLdsRow + a_piece * 16]) =
                stage_regs[set][j];
        lds_x[set][tid] = stage_x[set];
        lds_m[set][tid] = stage_m[set];
    };
    // LDS offset of this lane's MFMA operands: row 32t + r32, k bytes 32*half + 16*h of
    // the 64-wide step
    const int a_lds = r32 * kLdsRow + 32 * half;

    // ---- weight chunks, one k step each, loaded kLead steps ahead
    v4i rb[kLead];                 // 16 weight bytes of the lane's channel
    // the current group's outer-product operands, read from the staged metadata
    float g_sw16 = 0.0f, g_xs = 0.0f, g_b2 = 0.0f, g_xsum = 0.0f;
    auto load_b = [&](int slot, int step) { rb[slot] = ld128(rw, w_off, step * 2048); };

    // prologue: stages 0..2 in flight, then weights and metadata, publish stage 0, start 3
    stage_load(std::integral_constant<int, 0>(), 0);
    stage_load(std::integral_constant<int, 1>(), 1);
    stage_load(std::integral_constant<int, 2>(), 2);
#pragma unroll
    for (int i = 0; i < kLead; ++i) load_b(i, i);
    stage_store(std::integral_constant<int, 0>());
    __syncthreads();
    stage_load(std::integral_constant<int, 0>(), 3);

    v16i dt0 = {}, dt1 = {};   // int32 partials of the current group, tiles 0 and 1
    v32f coef = {};            // [tile][16]: xs[row] * sw16[col] of the group held in dt0/dt1
    v32f acc = {};             // [tile][16]: fp32 outputs
    v32f bacc = {};            // [tile][16]: affine bias term

    // The previous group's epilogue for tile T: convert and accumulate (or store the partials).
    auto finish_tile = [&](auto TT, int g) {
        constexpr int t = decltype(TT)::value;
        const v16i &dt = t ? dt1 : dt0;
        if (PARTIALS) {
            // element e of tile t: row r0 + 32t + 8(e/4) + 4*half + e%4, channel c0 + r32
            const int col = c0 + r32;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = r0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
                if (row >= m || col >= geom.n) continue;
                int v = (FMT == kFmtCodebook) ? dt[e] : (dt[e] >> 4);
                if (FMT == kFmtAffine) v += 8 * xsum[(int64_t)g * m + row];
                d[((int64_t)row * geom.n + col) * ng + g] = v;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[16 * t + e] =
                    fmaf(static_cast<float>(dt[e]), coef[16 * t + e], acc[16 * t + e]);
        }
    };

    // Publish stage st + 1 (register set (st+1)%3) into LDS buffer (st+1)%3, which stage st - 2
    // used; once every wavefront is past the barrier, refill the set with stage st + 4.
    auto stage_end = [&](auto SET, int st) {
        stage_store(SET);
        __syncthreads();
        stage_load(SET, st + 1 + kSets);
    };

    // One 64-wide k step s = 6q + I.
    auto step = [&](auto II, int s) {
        constexpr int I = decltype(II)::value;
        constexpr int buf = I / 2;                       // LDS buffer and register set of s / 2
        constexpr int sub = I % 2;
        constexpr bool first = (I % SPG) == 0;           // first step of its group
        constexpr bool last = (I % SPG) == SPG - 1;
        if (sub == 0 && s > 0) stage_end(std::integral_constant<int, buf>(), s / 2 - 1);
        const int g = s / SPG;
        // Consume this step's ring slots first and refill them at once, so the loads for step
        // s + kLead are in flight while this step computes.
        v4i blo, bhi;
        unpack_b<FMT>(rb[I], cb, blo, bhi);
        load_b(I, s + kLead);
        if (first && !PARTIALS) {
            // group j of this stage: the lane's row scale / sum and its channel's metadata
            constexpr int j = (I % kStageSteps) / SPG;
            const int pnl = wn >> 1;
            const uint32_t meta =
                (kMB == 4) ? lds_m[buf][(j * 2 + pnl) * kPanelRows + prow]
                           : reinterpret_cast<const uint16_t *>(lds_m[buf])[(j * 2 + pnl) * kPanelRows + prow];
            const float sw = half_bits_to_float(meta & 0xFFFFu);
            g_sw16 = (FMT == kFmtCodebook) ? sw : sw * 0.0625f;
            g_xs = __builtin_bit_cast(float, lds_x[buf][j * 64 + lane]);
            if (FMT == kFmtAffine) {
                g_b2 = fmaf(8.0f, sw, half_bits_to_float(meta >> 16));
                g_xsum = g_xs * static_cast<float>(static_cast<int>(lds_x[buf][128 + j * 64 + lane]));
            }
        }
        if (s < nsteps && active) {
            const uint8_t *ab = &lds_a[buf][a_lds + sub * 64];
            const v4i a00 = *reinterpret_cast<const v4i *>(ab);
            const v4i a01 = *reinterpret_cast<const v4i *>(ab + 16);
            const v4i a10 = *reinterpret_cast<const v4i *>(ab + 32 * kLdsRow);
            const v4i a11 = *reinterpret_cast<const v4i *>(ab + 32 * kLdsRow + 16);
            const v16i z = {};
            if (first && g > 0) finish_tile(std::integral_constant<int, 0>(), g - 1);
            dt0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a00, blo, first ? z : dt0, 0, 0, 0);
            dt0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a01, bhi, dt0, 0, 0, 0);
            if (first) {
                if (g > 0) finish_tile(std::integral_constant<int, 1>(), g - 1);
                if (!PARTIALS) {
                    // coefficient tiles xs[row] * sw16[col] of group g, after the last read of
                    // group g-1's coefficients
                    const v32f zf = {};
                    coef = __builtin_amdgcn_mfma_f32_32x32x1f32(g_xs, g_sw16, zf, 0, 0, 0);
                }
            }
            dt1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a10, blo, first ? z : dt1, 0, 0, 0);
            dt1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a11, bhi, dt1, 0, 0, 0);
            if (last && FMT == kFmtAffine && !PARTIALS) {
                // sum_g xs*xsum[row] * (bw + 8 sw)[col]: bias plus the u = (u-8) + 8 correction
                bacc = __builtin_amdgcn_mfma_f32_32x32x1f32(g_xsum, g_b2, bacc, 0, 0, 0);
            }
        }
    };

    for (int s = 0; s < nsteps; s += kLead) {
        step(std::integral_constant<int, 0>(), s);
        step(std::integral_constant<int, 1>(), s + 1);
        step(std::integral_constant<int, 2>(), s + 2);
        step(std::integral_constant<int, 3>(), s + 3);
        step(std::integral_constant<int, 4>(), s + 4);
        step(std::integral_constant<int, 5>(), s + 5);
    }
    if (!active) return;
    finish_tile(std::integral_constant<int, 0>(), ng - 1);
    finish_tile(std::integral_constant<int, 1>(), ng - 1);
    if (PARTIALS) return;

    const int col = c0 + r32;
    if (col >= geom.n) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = r0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
            if (row >= m) continue;
            float v = acc[16 * t + e];
            if (FMT == kFmtAffine) v += bacc[16 * t + e];
            y[(int64_t)row * geom.n + col] = v;
        }
    }
}

template <int FMT, int G, bool PARTIALS>
hipError_t launch_bm(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                     const float *xs, const int32_t *xsum, float *y, int32_t *d,
                     hipStream_t stream) {
    const unsigned tiles =
        static_cast<unsigned>(((g.n_pad + kBN - 1) / kBN) * ((m + BM - 1) / BM));
    gemm_kernel<FMT, G, PARTIALS><<<tiles, 256, 0, stream>>>(packed, g, m, xq, xs, xsum, y, d);
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
