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
//   wavefront's 32 channels at chunk 2s + l/32, so a step's weight fragment is two contiguous
//   512-byte runs of the packed panel.  The chunk's low nibbles (k 0..15) pair with the lane's
//   first 16 activation bytes and its high nibbles (k 16..31) with the next 16: two
//   v_mfma_i32_32x32x32_i8 per tile per 64-wide k step.  Workgroups are numbered so that each
//   XCD (one L2) gets a contiguous run of tiles, the M tiles of a channel block adjacent.
//   Split tiles.  A CU's time follows how many tiles it holds, so a last round that gives only
//   some CUs one more tile costs a large part of a whole round (measured at 128 rows and k 5120:
//   512 tiles 51.5 us, 544 tiles 63 us, 768 tiles 73 us).
//   The launcher therefore splits the tiles of such a partial round: each goes to four
//   workgroups, one per 32-channel group, whose four wavefronts run one k quarter each (one
//   64-wide step per stage) and add their outputs in LDS in a fixed order.  Small layers (fewer
//   tiles than CUs) are split whole, which spreads them over four times the CUs.  A gated tile
//   splits in two (32 output channels each): wavefronts 0, 1 take the gate panel over the two k
//   halves, 2, 3 the up panel, and act(gate) * up is formed after the halves are added.
//   Stages.  The k range is cut into stages of 256.  A stage's activation rows, the activation
//   scales (and sums) of its groups and the weight metadata of the workgroup's two panels are
//   copied from memory straight into one of two LDS stage buffers by buffer loads with an LDS
//   destination (no registers, no VALU), one stage ahead.  Activation rows sit in LDS as
//   16-byte units XOR-swizzled by the row, so the MFMA operand reads of 32 rows at one k spread
//   over all banks.  Each wavefront issues the same six copies per stage, so one fixed wait
//   count (the loads issued after them) tells it its copies have landed; a barrier then tells
//   it everybody's have.  Weight chunks go to registers one stage ahead.  A load that may fall
//   outside its buffer carries its whole offset in the range-checked VGPR operand, and every
//   load past the data is aimed out of range: it returns zeros and touches no memory.
//   Occupancy.  At most 168 VGPRs and 44 KiB of LDS per workgroup let three workgroups share a
//   CU (three wavefronts per SIMD).  Measured on MI355X, that beats a register-hungrier layout
//   at two per SIMD (double-buffered partials, weights three stages ahead, three LDS buffers):
//   the step is a chain of short dependent phases (unpack, operand reads, MFMAs, epilogue)
//   that other wavefronts cover better than reordering inside one wavefront does.
//   Epilogue.  At the last k step of a group the VALU turns the group's int32 partials into
//   floats and accumulates them with one FMA each (the wait for the MFMA results is covered by
//   the other wavefronts of the SIMD).  Where the registers allow, the partials start from the
//   bit pattern of 1.5 * 2^23 rather than zero, so the float is one exact subtraction instead of
//   a slower conversion (the same value).  The FMA coefficients
//   xs[row] * sw[col] come from one fp32 outer-product MFMA (v_mfma_f32_32x32x1_2b: block t =
//   tile t), which lands each coefficient in the lane and register of its partial; the affine
//   bias term xs*xsum[row] * (bw + 8 sw)[col] is a second outer product accumulated on the
//   matrix unit.  Per element and group the VALU does two operations and the matrix unit the
//   rest.  Signed codes (sym q, affine u-8) enter the MFMA as 16*q (nibble moved to the byte's
//   top); the 1/16 is folded into sw, and affine's u = (u-8) + 8 is restored through the bias
//   term.
//   Gated output (GLU).  For a [gate; up] linear (n = 2F, F a multiple of 64) a workgroup owns
//   64 output channels: wavefronts 0 and 1 compute them from gate panel nt, wavefronts 2 and 3
//   from the up panel F / 64 panels on (the same tile count as the plain GEMM); after the k loop
//   each gate/up pair swaps half its tiles through LDS and each of the two stores one row tile
//   of act(gate) * up.
#include "w4a8_kernels.h"

#include <type_traits>

namespace w4a8 {
namespace {

constexpr int BM = 64;                      // activation rows per workgroup
constexpr int kBN = 128;                    // output channels per workgroup (4 wavefronts x 32)
constexpr int kSK = 256;                    // k per stage
constexpr int kSteps = kSK / 64;            // 64-wide k steps per stage
constexpr int kNS = 2;                      // LDS stage buffers
constexpr int kAStage = BM * kSK;           // activation bytes of a stage (16 KiB)
constexpr int kXOff = kAStage;              // xs [4 groups][64 rows] fp32, then xsum the same
constexpr int kMOff = kAStage + 2048;       // weight metadata of the workgroup's two panels
                                            // (a split workgroup: 1 KiB per wavefront)
constexpr int kStageBytes = kAStage + 6144;
// The count is exact only while the kernel makes no other vector memory access in the loop: a
// register spill (scratch loads and stores count too) would break it, so the build rejects any
// GEMM kernel that uses scratch.
// Copies and weight chunks are both issued one stage ahead: at the top of stage s a wavefront
// issues the copies of stage s+1, then its k steps issue the weight chunks of stage s+1.  Loads
// a wavefront issues between its copies of stage s and the wait at the top of stage s: the
// weight chunks of stage s.
constexpr int kVmAfterStage = kSteps;
// A split workgroup's wavefront runs one k step per stage, so one weight chunk follows the copies.
constexpr int kVmAfterSplitStage = 1;
constexpr int kSplit = 4;                   // k quarters of a split workgroup (its wavefronts)

typedef __attribute__((address_space(3))) void lds_void;

// 64 lanes x 16 bytes to LDS byte address lds_addr + 16 * lane.  The destination goes to M0, so it
// is made a scalar explicitly (otherwise the compiler wraps the copy in a loop over lanes).
__device__ __forceinline__ void copy16(rsrc_t r, uint32_t lds_addr, int voff) {
    const uint32_t a = __builtin_amdgcn_readfirstlane(lds_addr);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(uintptr_t)a, 16, voff, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    // s_waitcnt vmcnt(N), expcnt and lgkmcnt left at their maxima
    static_assert(N < 64, "vmcnt is six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
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

template <int FMT, int G, bool PARTIALS, bool GLU>
__global__ __launch_bounds__(256, 3) void gemm_kernel(const uint8_t *__restrict__ packed,
                                                      const Geom geom, int m,
                                                      const int8_t *__restrict__ xq,
                                                      const float *__restrict__ xs,
                                                      const int *__restrict__ xsum,
                                                      float *__restrict__ y,
                                                      int *__restrict__ d, int act, int nfull) {
    static_assert(!(GLU && PARTIALS), "the gated output has no partials variant");
    constexpr int SPG = G / 64;                        // k steps per group
    constexpr int GPS = kSteps / SPG;                  // groups per stage
    constexpr int kMB = (FMT == kFmtAffine) ? 4 : 2;   // metadata bytes per channel and group
    // Partials start from kPartialBias (16 more registers for the start value) except where that
    // does not fit the register budget (affine with 128-groups) and in the partials variant.
    constexpr bool kBiased = !PARTIALS && !(FMT == kFmtAffine && G == 128);
    __shared__ __attribute__((aligned(16))) uint8_t lds[kNS][kStageBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Tile of this workgroup.  Workgroups below nfull take whole tiles: when nfull is a multiple
    // of the 8 XCDs, workgroup b runs on XCD b % 8 and takes tile (b % 8) * (nfull / 8) + b / 8,
    // so each XCD walks a contiguous run.  Each tile from nfull on is split over four workgroups
    // (two, gated), one per 32-channel group of the tile; a split workgroup's four wavefronts
    // take that channel group over one k quarter each (gated: gate and up over one k half each)
    // and add their outputs in LDS at the end (fixed order).  The launcher splits the tiles of a
    // last, partial round of the CUs, which would otherwise leave a few CUs a whole extra tile.
    const int tiles_m = (m + BM - 1) / BM;
    const int tiles_n = (geom.n_pad + kBN - 1) / kBN;
    // workgroups per split tile: four (one per 32-channel group); two for the gated output (one
    // per 32 output channels, whose gate and up tiles its wavefronts share)
    constexpr int kParts = GLU ? 2 : kSplit;
    const bool split = static_cast<int>(blockIdx.x) >= nfull;   // workgroup-uniform
    int bid = blockIdx.x;
    int cgrp = 0;                                      // split: the tile's channel group
    if (split) {
        // Part p of the split tiles.  Workgroup b runs on XCD b % 8 (nfull is a multiple of 8),
        // so the parts of one channel group of one channel block (its row tiles, whose weights
        // are the same) are placed 8 apart, on one XCD: for each run of 8 (channel block,
        // channel group) units, the parts of row tile mt are parts 8 mt .. 8 mt + 7 of the run.
        // That needs the tail to be whole channel blocks (tiles_m a power of two) and a whole
        // number of runs; otherwise part p is channel group p % 4 of tile p / 4.
        const int part = bid - nfull;
        const int units = (tiles_m * tiles_n - nfull) / tiles_m * kParts;   // tail units
        const int run = 8 * tiles_m;                   // parts per run of 8 units
        if ((tiles_m & (tiles_m - 1)) == 0 && part < (units / 8) * run) {
            const int u = (part / run) * 8 + part % 8;
            const int mtp = (part % run) / 8;
            cgrp = u % kParts;
            bid = nfull + (u / kParts) * tiles_m + mtp;
        } else {
            cgrp = part % kParts;
            bid = nfull + part / kParts;
        }
    } else if ((nfull & 7) == 0) {
        bid = (bid & 7) * (nfull >> 3) + (bid >> 3);
    }
    const int mt = bid % tiles_m, nt = bid / tiles_m;
    // the wavefront's 32-channel group (gated: bit 1 the gate or up panel, bit 0 the group)
    const int wcol = !split ? wave : (GLU ? ((wave & 2) | cgrp) : cgrp);

    const int k = geom.k;
    const int ng = k / G;
    const int nblk = (ng + 3) / 4;                     // metadata blocks of 4 groups
    const int nstages = (k + kSK - 1) / kSK;
    const int m0 = mt * BM;
    const int rows_wg = min(m - m0, BM);
    const int c0 = nt * kBN + wcol * 32;               // first output channel of the wavefront
    const bool active = c0 < geom.n_pad;               // wave-uniform (workgroup-uniform: split)
    const int half = lane >> 5;
    const int r32 = lane & 31;
    const int pnl = wcol >> 1;                         // the wavefront's panel in the workgroup
    const int prow = (wcol & 1) * 32 + r32;            // the lane's channel row in that panel
    // GLU: gate panel nt (wavefronts 0, 1) and the up panel up_pan panels on (2, 3)
    const int up_pan = GLU ? geom.n_pad / (2 * kPanelRows) : 0;
    const int p = GLU ? nt + (pnl ? up_pan : 0) : (active ? c0 / kPanelRows : 0);
    const int kc = k / kChunkK;
    const int wg_p0 = GLU ? nt : nt * (kBN / kPanelRows);
    const int pstep = GLU ? up_pan : 1;                // panels between the workgroup's two
    const int wg_np = GLU ? up_pan + 1
                          : max(0, min(kBN / kPanelRows, geom.n_pad / kPanelRows - wg_p0));

    // ---- descriptors (offsets rebased per workgroup / panel stay far below 2^31)
    const rsrc_t ra = make_rsrc(xq + (int64_t)m0 * k, (uint64_t)rows_wg * k);
    const rsrc_t rw = make_rsrc(packed + geom.off_codes + (int64_t)p * kc * 1024,
                                active ? (uint64_t)kc * 1024 : 0);
    const rsrc_t rmeta = make_rsrc(packed + geom.off_meta + (int64_t)wg_p0 * nblk * 64 * 4 * kMB,
                                   (uint64_t)wg_np * nblk * 64 * 4 * kMB);
    // copy 5 of a stage: xs (even wavefronts) or xsum (odd wavefronts, affine; else xs again)
    const bool x_is_sum = (FMT == kFmtAffine || PARTIALS) && (wave & 1);
    const void *xbase = x_is_sum ? static_cast<const void *>(xsum) : static_cast<const void *>(xs);
    const rsrc_t rx = make_rsrc(xbase, xbase ? (uint64_t)ng * m * 4 : 0);

    uint4 cb = make_uint4(0u, 0u, 0u, 0u);
    if (FMT == kFmtCodebook && active)
        cb = reinterpret_cast<const uint4 *>(packed + geom.off_codebook)[(int64_t)p * 64 + prow];

    // ---- per-lane parts of the stage copies
    // Activation copy i (0..3) of this wavefront covers rows 16*wave + 4i + lane/16; lane's LDS
    // unit lane%16 of that row holds the row's k unit (lane%16) ^ (row%16).  Bytes past k need
    // no care: they meet zero weights (the weight loads past k are out of range).
    int a_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 16 * wave + 4 * i + (lane >> 4);
        a_off[i] = row * k + 16 * ((lane & 15) ^ (row & 15));
    }
    // scales/sums copy: lane holds group st*GPS + lane/16, rows 4*(lane%16) .. +3; groups past
    // the last one are out of range of the descriptor (zeros)
    const int x_off = ((lane >> 4) * m + m0 + 4 * (lane & 15)) * 4;
    // metadata copy: block (st*GPS)/4 of the workgroup's panels (2-byte entries: both panels in
    // one copy; 4-byte entries: panel wave & 1)
    const int vp = (kMB == 2) ? (lane >> 5) : (wave & 1);
    const int m_off = (kMB == 2) ? (vp * pstep * nblk * 512 + (lane & 31) * 16)
                                 : (vp * pstep * nblk * 1024 + lane * 16);
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (lds_void *)&lds[0][0]));
    auto issue_stage = [&](int st) __attribute__((always_inline)) {
        const uint32_t buf = lds_base + (st % kNS) * kStageBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            copy16(ra, buf + (16 * wave + 4 * i) * kSK, a_off[i] + st * kSK);
        copy16(rx, buf + kXOff + (x_is_sum ? 1024 : 0), x_off + st * GPS * m * 4);
        const int blk = (st * GPS) / 4;
        // (a block past the last reads the other panel's metadata or nothing: its groups have
        // zero scales xs, so nothing from them reaches the output)
        copy16(rmeta, buf + kMOff + ((kMB == 2) ? 0 : vp * 1024), m_off + blk * ((kMB == 2) ? 512 : 1024));
    };

    // ---- weight chunks: register slot s % 4 holds step s (one stage)
    constexpr int kRingSteps = kSteps;
    v4i rb[kRingSteps];
    const int w_off = (half * 64 + prow) * 16;     // steps past k are past the descriptor's range
    auto load_b = [&](int slot, int step) { rb[slot] = ld128(rw, w_off + step * 2048); };

    v16i dt[2] = {};          // [tile] int32 partials of the current group
    v32f coef = {};           // [tile][16]: xs[row] * sw16[col] of the current group
    v32f acc = {};            // [tile][16]: fp32 outputs (the affine bias term accumulates here too)
    const v32f zf = {};

    // The epilogue of group g, whose partials are in dt and coefficients in coef.
    // (PARTIALS: the int32 partials go to d instead, with the affine sums from slot gi of xbuf;
    // a split workgroup's stage past its quarter stores nothing: live false)
    auto finish = [&](int g, const uint8_t *xbuf, int gi, bool live, auto BIASED)
                      __attribute__((always_inline)) {
        constexpr bool biased = decltype(BIASED)::value;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (PARTIALS) {
                const int col = c0 + r32;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int rl = 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
                    const int row = m0 + rl;
                    if (!live || !active || g >= ng || row >= m || col >= geom.n) continue;
                    int v = (FMT == kFmtCodebook) ? dt[t][e] : (dt[t][e] >> 4);
                    if (FMT == kFmtAffine)
                        v += 8 * reinterpret_cast<const int *>(xbuf + kXOff + 1024)[gi * 64 + rl];
                    d[((int64_t)row * geom.n + col) * ng + g] = v;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float df = biased ? partial_to_float(dt[t][e])
                                            : static_cast<float>(dt[t][e]);
                    acc[16 * t + e] = fmaf(df, coef[16 * t + e], acc[16 * t + e]);
                }
            }
        }
    };
    // The outer products of a group from a stage buffer's scales and metadata: its coefficients
    // (into coef) and, affine, its bias term (into acc).  gi: the group's slot of scales and sums
    // in the stage; mi: its metadata entry.
    auto group_products = [&](const uint8_t *buf, int gi, int mi) __attribute__((always_inline)) {
        const float xsv = reinterpret_cast<const float *>(buf + kXOff)[gi * 64 + lane];
        uint32_t meta;
        if (kMB == 2)
            meta = reinterpret_cast<const uint16_t *>(buf + kMOff)[mi];
        else
            meta = reinterpret_cast<const uint32_t *>(buf + kMOff)[mi];
        const float sw = half_bits_to_float(meta & 0xFFFFu);
        const float sw16 = (FMT == kFmtCodebook) ? sw : sw * 0.0625f;
        coef = __builtin_amdgcn_mfma_f32_32x32x1f32(xsv, sw16, zf, 0, 0, 0);
        if (FMT == kFmtAffine) {
            const int xsumv = reinterpret_cast<const int *>(buf + kXOff + 1024)[gi * 64 + lane];
            const float b2 = fmaf(8.0f, sw, half_bits_to_float(meta >> 16));
            acc = __builtin_amdgcn_mfma_f32_32x32x1f32(xsv * static_cast<float>(xsumv), b2, acc,
                                                        0, 0, 0);
        }
    };

    // LDS offsets of this lane's activation operands in a stage buffer: step J, MFMA h (units
    // 4J + 2 half + h of rows r32 (tile 0) and 32 + r32 (tile 1, 32 * kSK bytes on: the swizzle
    // key row % 16 is the same)).
    int a_rd[kSteps][2];
#pragma unroll
    for (int j = 0; j < kSteps; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            a_rd[j][h] = r32 * kSK + 16 * ((4 * j + 2 * half + h) ^ (r32 & 15));

    // One 64-wide k step s = kSteps * st + J of stage st, whose LDS buffer and register-ring third
    // are B = st % 3 (compile-time).  Steps past k run on zero weights.
    auto step = [&](auto BB, auto JJ, int st) __attribute__((always_inline)) {
        constexpr int B = decltype(BB)::value;
        constexpr int J = decltype(JJ)::value;
        constexpr int sub = J % SPG;                   // step inside its group
        constexpr bool first = sub == 0;
        constexpr bool last = sub == SPG - 1;
        const int s = st * kSteps + J;
        const int g = s / SPG;
        const uint8_t *buf = lds[B];
        v4i blo, bhi;
        unpack_b<FMT>(rb[J], cb, blo, bhi);
        load_b(J, s + kRingSteps);                     // the same step one stage on
        const v4i a00 = *reinterpret_cast<const v4i *>(buf + a_rd[J][0]);
        const v4i a01 = *reinterpret_cast<const v4i *>(buf + a_rd[J][1]);
        const v4i a10 = *reinterpret_cast<const v4i *>(buf + a_rd[J][0] + 32 * kSK);
        const v4i a11 = *reinterpret_cast<const v4i *>(buf + a_rd[J][1] + 32 * kSK);
        const v16i z = kBiased ? partial_start() : v16i{};
        v16i &d0 = dt[0];
        v16i &d1 = dt[1];
        d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a00, blo, first ? z : d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a10, blo, first ? z : d1, 0, 0, 0);
        d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a01, bhi, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a11, bhi, d1, 0, 0, 0);
        if (last) {   // group g's products (its coefficients and affine bias), then its epilogue
            if (!PARTIALS) group_products(buf, g % GPS, (pnl * 64 + prow) * 4 + g % 4);
            finish(g, buf, g % GPS, true, std::integral_constant<bool, kBiased>());
        }
    };

    // Stage st: this wavefront's copies of it have landed, then everybody's have; every
    // wavefront is also done with the buffer of stage st - 1, which stage st + 1 refills.
    auto stage = [&](auto BB, int st) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vm<kVmAfterStage>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue_stage(st + 1);
        __builtin_amdgcn_sched_barrier(0);
        step(BB, std::integral_constant<int, 0>(), st);
        __builtin_amdgcn_sched_barrier(0);
        step(BB, std::integral_constant<int, 1>(), st);
        __builtin_amdgcn_sched_barrier(0);
        step(BB, std::integral_constant<int, 2>(), st);
        __builtin_amdgcn_sched_barrier(0);
        step(BB, std::integral_constant<int, 3>(), st);
    };

    if (split) {
        // ---- a split workgroup: k is cut into NSL slices (quarters; halves for the gated output,
        // whose wavefronts 0, 1 take the gate panel and 2, 3 the up panel of the same channels),
        // and wavefront w runs slice w % NSL of channel group cgrp, one 64-wide step per stage (k
        // is a multiple of NSL G and of 256, so a slice is whole steps and whole groups).  A stage
        // buffer holds the slices' steps side by side: k unit u of a row is unit u % 4 of slice
        // u / 4 (slices past NSL are left empty), so wavefront w reads the same operand offsets as
        // step w % NSL of a whole stage.  Slot q of the scales and sums holds slice q's group, and
        // the metadata region w (1 KiB) the block of wavefront w's group in its panel.  Stages
        // past the slice's end (the loop runs two at a time) load their weights, scales and
        // metadata out of range: zero weights with zero coefficients add nothing, and their
        // partials are not stored.
        constexpr int NSL = GLU ? 2 : kSplit;
        const int slice = wave % NSL;
        const int qsteps = k / (64 * NSL);                 // steps per slice
        const int sw0 = slice * qsteps;                    // the wavefront's first step in all of k
        const int sq = lane >> 4;                          // the lane's copy slice (>= NSL: empty)
        const int gq0 = sq * (ng / NSL);                   // first group of the lane's copy slice
        int sa_off[4];
    #pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * wave + 4 * i + (lane >> 4);
            const int ku = (lane & 15) ^ (row & 15);
            sa_off[i] = (ku >> 2) < NSL ? row * k + (ku >> 2) * (k / NSL) + 16 * (ku & 3) : kOOB;
        }
        const int sx_off = (m0 + 4 * (lane & 15)) * 4;
        const int sm_off = pnl * pstep * nblk * 64 * 4 * kMB + lane * 16;
        auto issue_split = [&](int st) __attribute__((always_inline)) {
            const uint32_t buf = lds_base + (st % kNS) * kStageBytes;
            const bool live = st < qsteps;
    #pragma unroll
            for (int i = 0; i < 4; ++i)
                copy16(ra, buf + (16 * wave + 4 * i) * kSK,
                       sa_off[i] == kOOB ? kOOB : sa_off[i] + 64 * st);
            const int gl = gq0 + (64 * st) / G;
            copy16(rx, buf + kXOff + (x_is_sum ? 1024 : 0),
                   live && sq < NSL ? gl * m * 4 + sx_off : kOOB);
            const int gw = slice * (ng / NSL) + (64 * st) / G;
            copy16(rmeta, buf + kMOff + wave * 1024, live ? sm_off + (gw / 4) * 64 * 4 * kMB : kOOB);
        };
        auto load_split = [&](int slot, int st) {
            rb[slot] = ld128(rw, st < qsteps ? w_off + (sw0 + st) * 2048 : kOOB);
        };
        int sa_rd[2];
    #pragma unroll
        for (int h = 0; h < 2; ++h) sa_rd[h] = r32 * kSK + 16 * ((4 * slice + 2 * half + h) ^ (r32 & 15));
        // The wavefront's step of stage st, whose LDS buffer and weight slot B = S = st % 2 are
        // compile-time (two weight chunks in flight).
        auto split_step = [&](auto BB, auto SS, int st) __attribute__((always_inline)) {
            constexpr int B = decltype(BB)::value;
            constexpr int S = decltype(SS)::value;
            constexpr int sub = S % SPG;                   // (a slice starts on a group)
            constexpr bool first = sub == 0;
            constexpr bool last = sub == SPG - 1;
            const int g = (sw0 + st) / SPG;
            const uint8_t *buf = lds[B];
            v4i blo, bhi;
            unpack_b<FMT>(rb[S], cb, blo, bhi);
            load_split(S, st + 2);                         // the slot's step two stages on
            const v4i a00 = *reinterpret_cast<const v4i *>(buf + sa_rd[0]);
            const v4i a01 = *reinterpret_cast<const v4i *>(buf + sa_rd[1]);
            const v4i a10 = *reinterpret_cast<const v4i *>(buf + sa_rd[0] + 32 * kSK);
            const v4i a11 = *reinterpret_cast<const v4i *>(buf + sa_rd[1] + 32 * kSK);
            const v16i z = {};                             // (no start-value registers here)
            v16i &d0 = dt[0];
            v16i &d1 = dt[1];
            d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a00, blo, first ? z : d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a10, blo, first ? z : d1, 0, 0, 0);
            d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a01, bhi, d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a11, bhi, d1, 0, 0, 0);
            if (last) {
                if (!PARTIALS) group_products(buf, slice, wave * (1024 / kMB) + prow * 4 + g % 4);
                finish(g, buf, slice, st < qsteps, std::false_type());
            }
        };
        auto split_stage = [&](auto BB, auto SS, int st) __attribute__((always_inline)) {
            __builtin_amdgcn_sched_barrier(0);
            wait_vm<kVmAfterSplitStage>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            issue_split(st + 1);
            __builtin_amdgcn_sched_barrier(0);
            split_step(BB, SS, st);
        };

        // ---- prologue: copies of stage 0, then the weight chunks of stages 0 and 1
        issue_split(0);
        __builtin_amdgcn_sched_barrier(0);
        load_split(0, 0);
        load_split(1, 1);
        __builtin_amdgcn_sched_barrier(0);
        for (int st = 0; st < qsteps; st += 2) {
            split_stage(std::integral_constant<int, 0>(), std::integral_constant<int, 0>(), st);
            split_stage(std::integral_constant<int, 1>(), std::integral_constant<int, 1>(), st + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (PARTIALS || !active) return;                 // (workgroup-uniform)
        // The slices' outputs meet in LDS: wavefronts 1-3 store theirs, wavefront 0 adds them
        // to its own in slice order and stores the tile (gated: gate = wavefronts 0 + 1, up =
        // 2 + 3, then act(gate) * up).
        __syncthreads();
        float *xch = reinterpret_cast<float *>(&lds[0][0]);   // [3][32][64] fp32, 24 KiB
        if (wave > 0) {
#pragma unroll
            for (int e = 0; e < 32; ++e) xch[((wave - 1) * 32 + e) * 64 + lane] = acc[e];
        }
        __syncthreads();
        if (GLU) {
            if (wave != 0) return;
            const int f_n = geom.n / 2;
            const int colz = nt * kPanelRows + prow;       // output channel, < F
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int i = 16 * t + e;
                    const int row = m0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
                    const float gate = acc[i] + xch[i * 64 + lane];
                    const float up = xch[(32 + i) * 64 + lane] + xch[(64 + i) * 64 + lane];
                    if (row < m) y[(int64_t)row * f_n + colz] = act_apply(act, gate) * up;
                }
            }
            return;
        }
        const int col = c0 + r32;
        if (wave != 0 || col >= geom.n) return;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
                float v = acc[16 * t + e];
#pragma unroll
                for (int w = 0; w < kSplit - 1; ++w) v += xch[(w * 32 + 16 * t + e) * 64 + lane];
                if (row < m) y[(int64_t)row * geom.n + col] = v;
            }
        }
        return;
    }

    // ---- prologue, in the loop's issue order: copies of stage 0, then its weight chunks
    issue_stage(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kSteps; ++j) load_b(j, j);
    __builtin_amdgcn_sched_barrier(0);

    // Stages two at a time: the LDS buffer is then compile-time.  A stage past the end runs on
    // zeros.
    for (int st = 0; st < nstages; st += 2) {
        stage(std::integral_constant<int, 0>(), st);
        stage(std::integral_constant<int, 1>(), st + 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (PARTIALS || !active) return;

    if (GLU) {
        // Gate wavefront q and up wavefront q + 2 hold the same outputs' gate and up tiles.  Every
        // wavefront is done with the stage buffers; each pair swaps half its tiles through LDS
        // (the up tile 0 to the gate wavefront, the gate tile 1 to the up wavefront), and each
        // wavefront finishes one row tile: the activations split evenly.
        __syncthreads();
        float *xch = reinterpret_cast<float *>(&lds[0][0]);   // [pnl][pair][16][64] fp32, 16 KiB
        const int q = wave & 1;
        const int give = pnl ? 0 : 16;                         // the tile this wavefront hands over
#pragma unroll
        for (int e = 0; e < 16; ++e) xch[((pnl * 2 + q) * 16 + e) * 64 + lane] = acc[give + e];
        __syncthreads();
        const int f_n = geom.n / 2;
        const int colz = nt * kPanelRows + prow;               // output channel, < F
        const int t = pnl;                                     // the row tile this wavefront stores
        const int other = ((pnl ^ 1) * 2 + q) * 16;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = m0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
            const float mine = acc[16 * t + e], theirs = xch[(other + e) * 64 + lane];
            const float g = pnl ? theirs : mine, u = pnl ? mine : theirs;
            if (row < m) y[(int64_t)row * f_n + colz] = act_apply(act, g) * u;
        }
        return;
    }

    const int col = c0 + r32;
    if (col >= geom.n) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = m0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
            if (row < m) y[(int64_t)row * geom.n + col] = acc[16 * t + e];
        }
    }
}

// The split needs k to be whole 256-wide stages and each quarter (each half, gated) whole groups.
int gemm_whole_tiles(int tiles, int k, int group, bool glu) {
    if (k % 256 != 0 || k % ((glu ? 2 : kSplit) * group) != 0) return tiles;
    return whole_tiles(tiles);
}

// (the gated output has the same tile count: 64 output channels per workgroup from 128 rows)
template <int FMT, int G, bool PARTIALS, bool GLU>
hipError_t launch_bm(const Geom &g, int act, const uint8_t *packed, int m, const int8_t *xq,
                     const float *xs, const int32_t *xsum, float *y, int32_t *d,
                     hipStream_t stream) {
    const int tiles = ((g.n_pad + kBN - 1) / kBN) * ((m + BM - 1) / BM);
    const int nfull = gemm_whole_tiles(tiles, g.k, G, GLU);
    const unsigned grid = static_cast<unsigned>(nfull + (GLU ? 2 : kSplit) * (tiles - nfull));
    gemm_kernel<FMT, G, PARTIALS, GLU><<<grid, 256, 0, stream>>>(packed, g, m, xq, xs, xsum, y,
                                                                 d, act, nfull);
    return hipGetLastError();
}

template <int FMT, bool PARTIALS, bool GLU>
hipError_t launch_g(const Geom &g, int act, const uint8_t *packed, int m, const int8_t *xq,
                    const float *xs, const int32_t *xsum, float *y, int32_t *d,
                    hipStream_t stream) {
    if (g.group == 64)
        return launch_bm<FMT, 64, PARTIALS, GLU>(g, act, packed, m, xq, xs, xsum, y, d, stream);
    return launch_bm<FMT, 128, PARTIALS, GLU>(g, act, packed, m, xq, xs, xsum, y, d, stream);
}

template <bool PARTIALS, bool GLU>
hipError_t launch_f(const Geom &g, int act, const uint8_t *packed, int m, const int8_t *xq,
                    const float *xs, const int32_t *xsum, float *y, int32_t *d,
                    hipStream_t stream) {
    switch (g.fmt) {
    case kFmtSym:
        return launch_g<kFmtSym, PARTIALS, GLU>(g, act, packed, m, xq, xs, xsum, y, d, stream);
    case kFmtAffine:
        return launch_g<kFmtAffine, PARTIALS, GLU>(g, act, packed, m, xq, xs, xsum, y, d, stream);
    default:
        return launch_g<kFmtCodebook, PARTIALS, GLU>(g, act, packed, m, xq, xs, xsum, y, d,
                                                     stream);
    }
}

}  // namespace

int device_cus() {
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cus[dev] = v;
    }
    return cus[dev];
}

int whole_tiles(int tiles) {
    const int cus = device_cus();
    if (cus <= 0) return tiles;
    const int tail = tiles % cus;
    if (tail == 0 || tail * 4 > cus * 3) return tiles;
    return tiles - tail;
}

hipError_t launch_gemm(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                       const float *xs, const int32_t *xsum, float *y, int32_t *d,
                       hipStream_t stream) {
    if (m == 0) return hipSuccess;
    if (d) return launch_f<true, false>(g, 0, packed, m, xq, xs, xsum, nullptr, d, stream);
    return launch_f<false, false>(g, 0, packed, m, xq, xs, xsum, y, nullptr, stream);
}

hipError_t launch_gemm_glu(const Geom &g, int act, const uint8_t *packed, int m,
                           const int8_t *xq, const float *xs, const int32_t *xsum, float *y,
                           hipStream_t stream) {
    if (m == 0) return hipSuccess;
    return launch_f<false, true>(g, act, packed, m, xq, xs, xsum, y, nullptr, stream);
}

}  // namespace w4a8
