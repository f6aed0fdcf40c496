// Prefill attention over the cached int8 key/value segment.
//
// Source: "cactus PR #697", section "Prefill attention": for the cached-int8 part of a prefill
// chunk (fully visible by causality), int8 QK products under one flat scale per query row and
// per key vector (the keys' group-scale ratios requantized into their int8 values), a masked
// softmax over 64-key blocks carried online, and an unsigned 8-bit P quantized per (row, value
// group, block) with the value group's scale folded in; sliding window with attention-sink
// exemption; the new-token segment continues from the running statistics (m, l) and the
// unnormalized output.
//
// MI355X design.
//   Packing (once per cache write): keys requantized to their flat scale; each 64-slot block's
//   values stored transposed ([d][slot]) with the slots in the order the MFMA output holds
//   them, so that P never moves between lanes: the QK product is computed transposed (slots as
//   rows, queries as columns, v_mfma_i32_32x32x32_i8 with the keys as A), lane (q, h) then holds
//   slots 32t + 8(e/4) + 4h + e%4 (e = 0..15) of its query, which are exactly the 16 k slots it
//   supplies as the B operand of the AV product (values^T as A).  Slot scales, positions and
//   value-group scales are stored in the same order; per block and d, the column sum of the
//   value codes.
//   AV with unsigned P on a signed MFMA: u - 128 enters the i8 product and 128 * (the block's
//   column sum) is added back in int32, exactly.
//   Kernel: a workgroup of 8 wavefronts (two per SIMD) per (query head, 32-query tile, slot
//   range).  It stages 1024 / head_dim consecutive blocks of its key/value head at a time in LDS
//   (about 145 KiB: key codes, transposed value codes, value-group scales, column sums, slot
//   positions and key scales) with buffer loads that write LDS directly, and quantizes the
//   tile's queries into LDS while those copies are in flight (the first range's workgroup also
//   writes the codes and scales out); one wait and one barrier later every operand is an LDS
//   read, with the 16-byte units of key, value and query rows XOR-swizzled so that the MFMA
//   operand reads are free of bank conflicts.  Each wavefront takes every (8 / DS)-th block of
//   the range (head_dim 256, DS = 2: half of the value groups, to keep its output state in
//   registers), keeps its own (O, m, l) and skips blocks no query of the tile sees; the
//   wavefronts merge through LDS, and ranges split over several workgroups (one workgroup per
//   CU fills the chip) merge in a second kernel, both in a fixed order.  The codes are
//   P' * (255 / max P'), one reciprocal per (row, group, block).
#include "w4a8_kernels.h"

namespace w4a8 {
namespace {

constexpr int kSlots = 64;      // slots per block
constexpr int kQT = 32;         // queries per tile
constexpr int kAW = 8;          // wavefronts per workgroup (two per SIMD)
constexpr float kNegInf = -__builtin_inff();
// Scores are kept in base-2 units (the log2(e) factor is folded into the query scale), so every
// exponential is one hardware 2^x; the statistic m is returned in natural units (times ln 2).
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr int kMergeRegs = 8;  // split states the merge holds in registers at once

// Position of slot jj (0..63) of a block in the MFMA order: subtile t = jj / 32, row r = jj % 32
// sits in lane half h = (r / 4) % 2 at element e = 4 (r / 8) + r % 4.
__device__ __forceinline__ int mfma_order(int jj) {
    const int t = jj >> 5, r = jj & 31;
    return t * 32 + ((r >> 2) & 1) * 16 + 4 * (r >> 3) + (r & 3);
}

// ---- packing

__global__ __launch_bounds__(256) void attn_pack_slots(const AttnGeom ag, const int8_t *__restrict__ k8,
                                                       const float *__restrict__ ks,
                                                       const int8_t *__restrict__ v8,
                                                       const float *__restrict__ vs,
                                                       const int32_t *__restrict__ kvpos,
                                                       uint8_t *__restrict__ out) {
#pragma clang fp contract(off)
    const int64_t t = blockIdx.x * (int64_t)256 + threadIdx.x;
    const int64_t npad = (int64_t)ag.nblk * kSlots;
    if (t >= (int64_t)ag.nkvh * npad) return;
    const int kh = static_cast<int>(t / npad);
    const int j = static_cast<int>(t % npad);
    const int d = ag.d, ng = d / 32;
    const int b = j / kSlots, idx = mfma_order(j % kSlots);
    const bool live = j < ag.nkv;
    const int64_t src = (int64_t)kh * ag.nkv + j;
    int8_t *kq = reinterpret_cast<int8_t *>(out + ag.off_kq) + ((int64_t)kh * npad + j) * d;
    float sk = 0.0f;
    if (live)
        for (int g = 0; g < ng; ++g) sk = fmaxf(sk, ks[src * ng + g]);
    for (int i = 0; i < d; ++i) {
        float v = 0.0f;
        if (live && sk > 0.0f) v = rintf(static_cast<float>(k8[src * d + i]) * (ks[src * ng + i / 32] / sk));
        kq[i] = static_cast<int8_t>(v);
    }
    const int64_t bo = ((int64_t)kh * ag.nblk + b) * kSlots + idx;
    reinterpret_cast<float *>(out + ag.off_sk)[bo] = sk;
    reinterpret_cast<int32_t *>(out + ag.off_pos)[bo] = live ? kvpos[j] : -1;
    int8_t *vt = reinterpret_cast<int8_t *>(out + ag.off_vt) + ((int64_t)kh * ag.nblk + b) * d * kSlots;
    for (int i = 0; i < d; ++i) vt[i * kSlots + idx] = live ? v8[src * d + i] : 0;
    float *sv = reinterpret_cast<float *>(out + ag.off_sv) + ((int64_t)kh * ag.nblk + b) * ng * kSlots;
    for (int g = 0; g < ng; ++g) sv[g * kSlots + idx] = live ? vs[src * ng + g] : 0.0f;
}

// column sums of a block's value codes, stored per (group, lane half, element) in the order the
// AV output tile holds the d rows: d = 32g + 8(e/4) + 4h + e%4
__global__ __launch_bounds__(256) void attn_pack_vsum(const AttnGeom ag, const int8_t *__restrict__ v8,
                                                      uint8_t *__restrict__ out) {
    const int64_t t = blockIdx.x * (int64_t)256 + threadIdx.x;
    const int d = ag.d;
    if (t >= (int64_t)ag.nkvh * ag.nblk * d) return;
    const int i = static_cast<int>(t % d);
    const int64_t kb = t / d;                                   // kh * nblk + b
    const int kh = static_cast<int>(kb / ag.nblk), b = static_cast<int>(kb % ag.nblk);
    int32_t s = 0;
    for (int jj = 0; jj < kSlots; ++jj) {
        const int j = b * kSlots + jj;
        if (j < ag.nkv) s += v8[((int64_t)kh * ag.nkv + j) * d + i];
    }
    const int g = i / 32, r = i % 32;
    const int h = (r >> 2) & 1, e = 4 * (r >> 3) + (r & 3);
    reinterpret_cast<int32_t *>(out + ag.off_vsum)[kb * d + g * 32 + h * 16 + e] = s;
}

// ---- attention

struct AttnArgs {
    const float *q;            // [nh][nq][d]
    int nh, nq, pos0, window, sink, nsplit, bps;   // bps: blocks per split
    float scale;
    int8_t *q8;                // [nh][nq][d]
    float *sq;                 // [nh][nq]
    float *o, *m, *l;          // final [nh][nq][d], [nh][nq] (nsplit == 1) ...
    float *work;               // ... or partial states: o [nsplit][nh][nq][d], then (m, l)
                               // [nsplit][nh][nq][2] (m in base-2 units)
};

__device__ __forceinline__ float wave_max32(float v) {          // max with the other lane half
    return fmaxf(v, __shfl_xor(v, 32, 64));
}

// LDS staging of NB = 1024 / D consecutive blocks of one key/value head (every region a whole
// number of KiB, about 142-148 KiB in all): key codes [NB * 64][D] and transposed value codes
// [NB][D][64] with their 16-byte units XOR-swizzled by row, value-group scales [NB][NG][64],
// value column sums [NB][D], slot positions and key scales [NB][64].
template <int D>
struct AttnStage {
    static constexpr int NB = 1024 / D;
    static constexpr int NG = D / 32;
    static constexpr int kK = NB * kSlots * D;
    static constexpr int kVT = NB * D * kSlots;
    static constexpr int kSV = NB * NG * kSlots * 4;
    static constexpr int kVS = NB * D * 4;
    static constexpr int kPS = NB * kSlots * 4;
    static constexpr int oK = 0, oVT = oK + kK, oSV = oVT + kVT, oVS = oSV + kSV;
    static constexpr int oPos = oVS + kVS, oSk = oPos + kPS, kBytes = oSk + kPS;
    static_assert(kSV % 1024 == 0 && kVS % 1024 == 0 && kPS % 1024 == 0, "whole copies");
    // A key row is D bytes (D / 16 units); 256 / D rows share one 256-byte bank period, so the
    // unit key changes every 256 / D rows: 16 lanes reading one unit of 16 rows hit 16 distinct
    // 16-byte bank groups.  Value rows are 64 bytes (4 units, 4 rows per period).
    __device__ static int kkey(int slot) { return (slot / (256 / D)) % (D / 16); }
    __device__ static int vkey(int row) { return (row >> 2) & 3; }
};

typedef __attribute__((address_space(3))) void attn_lds_void;

// 64 lanes x 16 bytes from r at the lane's offset to LDS byte address lds_addr + 16 * lane (the
// destination goes to M0, so it is made a scalar).
__device__ __forceinline__ void attn_copy16(rsrc_t r, uint32_t lds_addr, int voff) {
    const uint32_t a = __builtin_amdgcn_readfirstlane(lds_addr);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (attn_lds_void *)(uintptr_t)a, 16, voff, 0, 0, 0);
}

// DS = 2 (head_dim 256) splits the value groups over wavefront pairs: wavefront w takes groups
// (w / 2) * NG/2 .. +NG/2-1 of every second block (w % 2), so its output state is half as large
// (both of a pair compute the block's QK product and softmax, identically).
template <int D, int DS>
__global__ __launch_bounds__(64 * kAW) void attn_kernel(const AttnGeom ag,
                                                        const uint8_t *__restrict__ packed,
                                                        const AttnArgs a) {
#pragma clang fp contract(off)
    using ST = AttnStage<D>;
    constexpr int NG = D / 32;           // value groups of the head
    constexpr int NGW = NG / DS;         // value groups of this wavefront
    constexpr int BL = kAW / DS;         // wavefronts sharing a group set (one block each)
    constexpr int NB = ST::NB;
    __shared__ __attribute__((aligned(16))) uint8_t stage[ST::kBytes];
    __shared__ __attribute__((aligned(16))) uint8_t qtile[kQT * D];   // the tile's query codes
    __shared__ float qscl[kQT];                                       // and row scales
    __shared__ float xm[kAW][kQT];
    // the merge's exchange buffer reuses the staged blocks once every block is done:
    // [wavefront][group][element][lane] (a wavefront's 64 lanes store one element as 256
    // contiguous bytes, free of bank conflicts)
    static_assert(kAW * NGW * 16 * 64 * 4 <= ST::kBytes, "merge buffer inside the staged blocks");
    float *xst = reinterpret_cast<float *>(stage);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int dpart = wave / BL, blane = wave % BL;
    const int half = lane >> 5, col = lane & 31;
    const int qtiles = (a.nq + kQT - 1) / kQT;
    const int split = blockIdx.x % a.nsplit;
    const int hq = blockIdx.x / a.nsplit;                     // head * qtiles + tile
    const int head = hq / qtiles, q0 = (hq % qtiles) * kQT;
    const int kh = head / (a.nh / ag.nkvh);
    const int qi = q0 + col;                                  // this lane's query
    const bool qlive = qi < a.nq;
    // positions compare as unsigned 32-bit: pos0 + qi < 2^32, and a slot's p is checked >= 0
    // (then p <= qpos makes qpos - p exact)
    const uint32_t qpos = static_cast<uint32_t>(a.pos0) + static_cast<uint32_t>(qi);
    const uint32_t window = static_cast<uint32_t>(a.window), sink = static_cast<uint32_t>(a.sink);

    // the head's regions in the packed cache (rebased per staged chunk below)
    const uint8_t *kqh = packed + ag.off_kq + (int64_t)kh * ag.nblk * kSlots * D;
    const uint8_t *skh = packed + ag.off_sk + (int64_t)kh * ag.nblk * kSlots * 4;
    const uint8_t *posh = packed + ag.off_pos + (int64_t)kh * ag.nblk * kSlots * 4;
    const uint8_t *vth = packed + ag.off_vt + (int64_t)kh * ag.nblk * D * kSlots;
    const uint8_t *svh = packed + ag.off_sv + (int64_t)kh * ag.nblk * NG * kSlots * 4;
    const uint8_t *vsh = packed + ag.off_vsum + (int64_t)kh * ag.nblk * D * 4;
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (attn_lds_void *)&stage[0]));

    // Stage blocks cb .. cb + NB - 1: every wavefront issues every eighth 1-KiB copy of each
    // region; blocks past the head's last read past the rebased ranges and stage zeros.  The key
    // side (positions, key scales, key codes) first; the value side is issued once the key side
    // has landed and arrives while the QK products and the softmax run.
    auto stage_keys = [&](int cb) __attribute__((always_inline)) {
        const int nb = ag.nblk - cb;                           // blocks left in the head (>= 1)
        const rsrc_t rk = make_rsrc(kqh + (int64_t)cb * kSlots * D, (uint64_t)nb * kSlots * D);
        const rsrc_t rpos = make_rsrc(posh + (int64_t)cb * kSlots * 4, (uint64_t)nb * kSlots * 4);
        const rsrc_t rsk = make_rsrc(skh + (int64_t)cb * kSlots * 4, (uint64_t)nb * kSlots * 4);
        for (int c = wave; c < ST::kPS / 1024; c += kAW) {
            attn_copy16(rpos, lds0 + ST::oPos + c * 1024, c * 1024 + 16 * lane);
            attn_copy16(rsk, lds0 + ST::oSk + c * 1024, c * 1024 + 16 * lane);
        }
        for (int c = wave; c < ST::kK / 1024; c += kAW) {
            const int pb = c * 1024 + 16 * lane;
            const int slot = pb / D, u = (pb % D) / 16;
            attn_copy16(rk, lds0 + ST::oK + c * 1024, slot * D + 16 * (u ^ ST::kkey(slot % kSlots)));
        }
    };
    auto stage_values = [&](int cb) __attribute__((always_inline)) {
        const int nb = ag.nblk - cb;
        const rsrc_t rv = make_rsrc(vth + (int64_t)cb * D * kSlots, (uint64_t)nb * D * kSlots);
        const rsrc_t rsv = make_rsrc(svh + (int64_t)cb * NG * kSlots * 4, (uint64_t)nb * NG * kSlots * 4);
        const rsrc_t rvs = make_rsrc(vsh + (int64_t)cb * D * 4, (uint64_t)nb * D * 4);
        for (int c = wave; c < ST::kVT / 1024; c += kAW) {
            const int pb = c * 1024 + 16 * lane;
            const int row = pb / kSlots, u = (pb % kSlots) / 16;
            attn_copy16(rv, lds0 + ST::oVT + c * 1024, row * kSlots + 16 * (u ^ ST::vkey(row)));
        }
        for (int c = wave; c < ST::kSV / 1024; c += kAW)
            attn_copy16(rsv, lds0 + ST::oSV + c * 1024, c * 1024 + 16 * lane);
        for (int c = wave; c < ST::kVS / 1024; c += kAW)
            attn_copy16(rvs, lds0 + ST::oVS + c * 1024, c * 1024 + 16 * lane);
    };

    // The tile's query rows quantized into LDS while the first chunk's copies are in flight: a
    // row is D / 4 consecutive lanes of one wavefront, one float4 each (scale = max|row| / 127 and
    // codes round-half-even(q / scale) in fp32, as the activation quantization; a zero scale gives
    // zero codes).  The codes' 16-byte units are swizzled as the key rows'.  The first split's
    // workgroup also writes them out (q8, sq).
    auto quantize_queries = [&]() __attribute__((always_inline)) {
        constexpr int LPR = D / 4;                          // lanes per row
        constexpr int kQuads = kQT * LPR;
#pragma unroll
        for (int j0 = 0; j0 < kQuads; j0 += 64 * kAW) {
            const int j = j0 + static_cast<int>(threadIdx.x);
            const int r = j / LPR, c4 = j % LPR;
            const bool live = j < kQuads && q0 + r < a.nq;
            const int64_t qidx = ((int64_t)head * a.nq + q0 + r) * LPR + c4;
            const float4 v = live ? reinterpret_cast<const float4 *>(a.q)[qidx]
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
            float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
            for (int o = 1; o < LPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
            const float scale = amax / 127.0f;
            const float e[4] = {v.x, v.y, v.z, v.w};
            uint32_t w = 0u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int c = 0;
                if (scale > 0.0f)
                    c = static_cast<int>(fminf(fmaxf(rintf(e[i] / scale), -127.0f), 127.0f));
                w |= (static_cast<uint32_t>(c) & 0xFFu) << (8 * i);
            }
            if (j < kQuads) {
                const int u = c4 / 4;
                *reinterpret_cast<uint32_t *>(qtile + r * D + 16 * (u ^ ST::kkey(r)) + 4 * (c4 % 4)) = w;
                if (c4 == 0) qscl[r] = scale;
            }
            if (live && split == 0) {
                reinterpret_cast<uint32_t *>(a.q8)[qidx] = w;
                if (c4 == 0) a.sq[(int64_t)head * a.nq + q0 + r] = scale;
            }
        }
    };

    v4i qb[NG];                 // the lane's query codes: d = 32i + 16h .. +15 of chunk i
    float qscale = 0.0f;
    float mrun = kNegInf, lrun = 0.0f;
    v16f o[NGW];
#pragma unroll
    for (int g = 0; g < NGW; ++g)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[g][e] = 0.0f;

    // Block b (staged at local index lb), every operand from LDS: visibility, S^T = K Q^T and the
    // online softmax (qk_block, key side only), then the value products of the wavefront's groups
    // (av_block) from the probabilities and rescale factor qk_block leaves in a BlockP.
    struct BlockP {
        float p[2][16];
        float keep;
        bool live;                       // some query of the tile sees the block
    };
    auto qk_block = [&](int lb, BlockP &bp) __attribute__((always_inline)) {
        bp.live = false;
        const int *posl = reinterpret_cast<const int *>(stage + ST::oPos) + lb * kSlots;
        const float *skl = reinterpret_cast<const float *>(stage + ST::oSk) + lb * kSlots;
        // visibility of the lane's 32 slots (two subtiles of 16)
        float s[2][16];
        bool any = false;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            int pos16[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int4 pv = reinterpret_cast<const int4 *>(posl + t * 32 + half * 16)[c];
                pos16[4 * c] = pv.x; pos16[4 * c + 1] = pv.y; pos16[4 * c + 2] = pv.z;
                pos16[4 * c + 3] = pv.w;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t p = static_cast<uint32_t>(pos16[e]);
                const bool vis = qlive && pos16[e] >= 0 && p <= qpos &&
                                 (window == 0u || p < sink || qpos - p < window);
                s[t][e] = vis ? 0.0f : kNegInf;
                any |= vis;
            }
        }
        if (__builtin_amdgcn_ballot_w64(any) == 0) return;            // no query sees the block
        bp.live = true;
        // S^T = K Q^T for the block's two 32-slot subtiles
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int slot = t * 32 + col;
            const uint8_t *kr = stage + ST::oK + (lb * kSlots + slot) * D;
            const int key = ST::kkey(slot);
            v4i ka[NG];
#pragma unroll
            for (int i = 0; i < NG; ++i)
                ka[i] = *reinterpret_cast<const v4i *>(kr + 16 * ((2 * i + half) ^ key));
            v16i acc = {};
#pragma unroll
            for (int i = 0; i < NG; ++i)
                acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[i], qb[i], acc, 0, 0, 0);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float4 kv = reinterpret_cast<const float4 *>(skl + t * 32 + half * 16)[c];
                const float k4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {   // (a select: visible slots hold 0, hidden -inf)
                    const float sc = static_cast<float>(acc[4 * c + i]) * qscale * k4[i];
                    s[t][4 * c + i] = (s[t][4 * c + i] == 0.0f) ? sc : kNegInf;
                }
            }
        }
        float mb = kNegInf;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) mb = fmaxf(mb, s[t][e]);
        mb = wave_max32(mb);
        const float mnew = fmaxf(mrun, mb);
        const float alpha = (mrun == kNegInf) ? 0.0f : exp2_hw(mrun - mnew);
        float psum = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                bp.p[t][e] = (s[t][e] == kNegInf) ? 0.0f : exp2_hw(s[t][e] - mnew);
                psum += bp.p[t][e];
            }
        lrun = lrun * alpha + psum;
        mrun = (mb == kNegInf) ? mrun : mnew;
        bp.keep = (mb == kNegInf) ? 1.0f : alpha;
    };
    auto av_block = [&](int lb, const BlockP &bp) __attribute__((always_inline)) {
        if (!bp.live) return;
        const float keep = bp.keep;
        const float(&p)[2][16] = bp.p;
#pragma unroll
        for (int gi = 0; gi < NGW; ++gi) {
            const int g = dpart * NGW + gi;
            const float *svl = reinterpret_cast<const float *>(stage + ST::oSV) + (lb * NG + g) * kSlots;
            float4 sv[2][4];
            v4i va[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    sv[t][c] = reinterpret_cast<const float4 *>(svl + t * 32 + half * 16)[c];
                const int row = lb * D + 32 * g + col;
                va[t] = *reinterpret_cast<const v4i *>(stage + ST::oVT + row * kSlots +
                                                      16 * ((2 * t + half) ^ ST::vkey(row)));
            }
            // P folded with the value group's scale, quantized to u8 per (row, group, block)
            float mx = 0.0f;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float4 v = sv[t][c];
                    mx = fmaxf(mx, fmaxf(fmaxf(p[t][4 * c] * v.x, p[t][4 * c + 1] * v.y),
                                         fmaxf(p[t][4 * c + 2] * v.z, p[t][4 * c + 3] * v.w)));
                }
            mx = wave_max32(mx);
            const float sp = mx / 255.0f;         // 0 when nothing of the row is visible
            // one reciprocal per (row, group, block); u = rint(pg * rsp) lies in 0..255 since
            // pg <= mx, and every pg is 0 when mx is
            const float rsp = (mx > 0.0f) ? 255.0f / mx : 0.0f;
            v16i iacc = {};
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                uint32_t w4[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float sv4[4] = {sv[t][c].x, sv[t][c].y, sv[t][c].z, sv[t][c].w};
                    // x + (2^23 + 2^22 + 128) rounds x to the nearest integer (ties to even) in
                    // the sum's low bits, already offset by 128: the low byte is u - 128 as int8
                    uint32_t bq[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float pg = p[t][4 * c + i] * sv4[i];
                        bq[i] = __float_as_uint(pg * rsp + 12583040.0f);
                    }
                    w4[c] = __builtin_amdgcn_perm(bq[1], bq[0], 0x0C0C0400u) |
                            __builtin_amdgcn_perm(bq[3], bq[2], 0x04000C0Cu);
                }
                const v4i pb = {static_cast<int>(w4[0]), static_cast<int>(w4[1]),
                                static_cast<int>(w4[2]), static_cast<int>(w4[3])};
                iacc = __builtin_amdgcn_mfma_i32_32x32x32_i8(va[t], pb, iacc, 0, 0, 0);
            }
            const int4 *vsr = reinterpret_cast<const int4 *>(stage + ST::oVS) +
                              (lb * D + g * 32 + half * 16) / 4;
            int vs16[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int4 v = vsr[c];
                vs16[4 * c] = v.x; vs16[4 * c + 1] = v.y; vs16[4 * c + 2] = v.z;
                vs16[4 * c + 3] = v.w;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float av = static_cast<float>(iacc[e] + 128 * vs16[e]);
                o[gi][e] = fmaf(o[gi][e], keep, sp * av);
            }
        }
    };

    // The workgroup's blocks in staged chunks of NB; the wavefront takes blocks b_lo + blane,
    // + BL, ... of each chunk in order.
    const int b_lo = split * a.bps;
    const int b_hi = min(ag.nblk, b_lo + a.bps);
    constexpr int MB = (NB + BL - 1) / BL;               // blocks of a wavefront per chunk
    for (int cb = b_lo; cb < b_hi; cb += NB) {
        if (cb > b_lo) __syncthreads();                    // every wavefront is done with LDS
        stage_keys(cb);
        if (cb == b_lo) quantize_queries();
        __builtin_amdgcn_s_waitcnt(0);                     // this wavefront's copies (and loads)
        __syncthreads();                                   // everybody's
        stage_values(cb);
        if (cb == b_lo) {
#pragma unroll
            for (int i = 0; i < NG; ++i)
                qb[i] = *reinterpret_cast<const v4i *>(qtile + col * D +
                                                      16 * ((2 * i + half) ^ ST::kkey(col)));
            qscale = qlive ? qscl[col] * (a.scale * kLog2e) : 0.0f;
        }
        const int ce = min(b_hi, cb + NB);
        const int bf = cb + ((blane - (cb - b_lo)) % BL + BL) % BL;   // the wavefront's first
        BlockP bp[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            bp[i].live = false;
            if (bf + i * BL < ce) qk_block(bf + i * BL - cb, bp[i]);
        }
        __builtin_amdgcn_s_waitcnt(0);                     // the value side, everybody's
        __syncthreads();
#pragma unroll
        for (int i = 0; i < MB; ++i)
            if (bf + i * BL < ce) av_block(bf + i * BL - cb, bp[i]);
    }

    // merge the states of the BL wavefronts of each group set (fixed order): M = max m_w, each
    // scaled by 2^(m_w - M) (base-2 scores); the two group sets of DS = 2 hold the same (m, l)
    const float lw = lrun + __shfl_xor(lrun, 32, 64);
    if (half == 0) xm[wave][col] = mrun;
    __syncthreads();
    float mall = xm[dpart * BL][col];
#pragma unroll
    for (int w = 1; w < BL; ++w) mall = fmaxf(mall, xm[dpart * BL + w][col]);
    const float mine = (mrun == kNegInf) ? 0.0f : exp2_hw(mrun - mall);
    __syncthreads();
    if (half == 0) xm[wave][col] = lw * mine;
    __syncthreads();
    float lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < BL; ++w) lsum += xm[dpart * BL + w][col];
    // Every wavefront stores its scaled state; then each of the BL wavefronts of a group set
    // adds the BL states (in wavefront order) for NGW * 16 / BL of the set's elements and stores
    // them: the sums and the output stores are spread over all the wavefronts.
#pragma unroll
    for (int g = 0; g < NGW; ++g)
#pragma unroll
        for (int e = 0; e < 16; ++e) xst[((wave * NGW + g) * 16 + e) * 64 + lane] = o[g][e] * mine;
    __syncthreads();
    if (!qlive) return;
    const int64_t row = (int64_t)head * a.nq + qi;
    float *orow;
    const bool stats = dpart == 0 && blane == 0 && half == 0;
    if (a.nsplit == 1) {
        orow = a.o + row * D;
        if (stats) { a.m[row] = mall * kLn2; a.l[row] = lsum; }
    } else {
        const int64_t rows = (int64_t)a.nh * a.nq, srow = (int64_t)split * rows + row;
        orow = a.work + srow * D;
        if (stats) {
            float *ml = a.work + a.nsplit * rows * D + 2 * srow;
            ml[0] = mall;
            ml[1] = lsum;
        }
    }
    constexpr int PPW = NGW * 16 / BL;                 // elements each wavefront adds up
    static_assert(PPW * BL == NGW * 16, "the elements split evenly");
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        const int pe = blane * PPW + i;
        const int g = pe >> 4, e = pe & 15;
        float v = xst[(((dpart * BL) * NGW + g) * 16 + e) * 64 + lane];
#pragma unroll
        for (int w = 1; w < BL; ++w) v += xst[(((dpart * BL + w) * NGW + g) * 16 + e) * 64 + lane];
        orow[32 * (dpart * NGW + g) + 8 * (e >> 2) + 4 * half + (e & 3)] = v;
    }
}

// the split states of each (head, query) merged in split order; a thread per 4 columns of a row
__global__ __launch_bounds__(256) void attn_merge(int nsplit, int64_t rows, int d,
                                                  const float *__restrict__ work,
                                                  float *__restrict__ o, float *__restrict__ m,
                                                  float *__restrict__ l) {
    const int64_t t = blockIdx.x * (int64_t)256 + threadIdx.x;
    const int q4 = d / 4;
    if (t >= rows * q4) return;
    const int64_t row = t / q4;
    const int c4 = static_cast<int>(t % q4);
    const float2 *ml = reinterpret_cast<const float2 *>(work + nsplit * rows * d);
    auto part = [&](int s) { return reinterpret_cast<const float4 *>(work + (s * rows + row) * d)[c4]; };
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float mall = kNegInf, lsum = 0.0f;
    auto add = [&](float2 st, float4 v) {
        const float f = (st.x == kNegInf) ? 0.0f : exp2_hw(st.x - mall);
        acc.x += v.x * f;
        acc.y += v.y * f;
        acc.z += v.z * f;
        acc.w += v.w * f;
        lsum += st.y * f;
    };
    if (nsplit <= kMergeRegs) {
        // every split's state loaded at once (one memory round trip), then the same arithmetic
        float2 st[kMergeRegs];
        float4 v[kMergeRegs];
#pragma unroll
        for (int s = 0; s < kMergeRegs; ++s) {
            if (s < nsplit) {
                st[s] = ml[s * rows + row];
                v[s] = part(s);
            }
        }
#pragma unroll
        for (int s = 0; s < kMergeRegs; ++s)
            if (s < nsplit) mall = fmaxf(mall, st[s].x);
#pragma unroll
        for (int s = 0; s < kMergeRegs; ++s)
            if (s < nsplit) add(st[s], v[s]);
    } else {
        for (int s = 0; s < nsplit; ++s) mall = fmaxf(mall, ml[s * rows + row].x);
        for (int s = 0; s < nsplit; ++s) add(ml[s * rows + row], part(s));
    }
    reinterpret_cast<float4 *>(o)[t] = acc;
    if (c4 == 0) { m[row] = mall * kLn2; l[row] = lsum; }
}

}  // namespace

int attn_splits(int nh, int nq, int nblk) {
    // one workgroup per CU (the staged blocks fill its LDS), at most one block per wavefront of
    // a group set (four for head_dim 256)
    const int tiles = nh * ((nq + kQT - 1) / kQT);
    int s = (256 + tiles - 1) / tiles;
    s = max(1, min(s, (nblk + kAW / 2 - 1) / (kAW / 2)));
    return s;
}

hipError_t launch_attn_pack(const AttnGeom &ag, const int8_t *k8, const float *ks,
                            const int8_t *v8, const float *vs, const int32_t *kvpos,
                            uint8_t *packed, hipStream_t stream) {
    const int64_t slots = (int64_t)ag.nkvh * ag.nblk * kSlots;
    attn_pack_slots<<<static_cast<unsigned>((slots + 255) / 256), 256, 0, stream>>>(ag, k8, ks, v8, vs,
                                                                                  kvpos, packed);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t cols = (int64_t)ag.nkvh * ag.nblk * ag.d;
    attn_pack_vsum<<<static_cast<unsigned>((cols + 255) / 256), 256, 0, stream>>>(ag, v8, packed);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnGeom &ag, const uint8_t *packed, const float *q, int nh, int nq,
                       int pos0, int window, int sink, float scale, int8_t *q8, float *sq,
                       float *o, float *m, float *l, float *work, hipStream_t stream) {
    if (nq == 0) return hipSuccess;
    AttnArgs a{q, nh, nq, pos0, window, sink, attn_splits(nh, nq, ag.nblk), 0, scale, q8, sq, o, m,
               l, work};
    a.bps = (ag.nblk + a.nsplit - 1) / a.nsplit;
    const unsigned grid = static_cast<unsigned>(nh * ((nq + kQT - 1) / kQT) * a.nsplit);
    if (ag.d == 64) attn_kernel<64, 1><<<grid, 64 * kAW, 0, stream>>>(ag, packed, a);
    else if (ag.d == 128) attn_kernel<128, 1><<<grid, 64 * kAW, 0, stream>>>(ag, packed, a);
    else attn_kernel<256, 2><<<grid, 64 * kAW, 0, stream>>>(ag, packed, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nsplit == 1) return e;
    const int64_t n = (int64_t)nh * nq * ag.d / 4;
    attn_merge<<<static_cast<unsigned>((n + 255) / 256), 256, 0, stream>>>(
        a.nsplit, (int64_t)nh * nq, ag.d, work, o, m, l);
    return hipGetLastError();
}

}  // namespace w4a8
