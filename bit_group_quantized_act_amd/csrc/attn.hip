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
//   Queries: a prepass writes the int8 codes and row scales once; the attention kernel loads them.
//   Kernel: a workgroup of 4 wavefronts per (query head, 32-query tile, slot range); each
//   wavefront takes every 4th block of the range (head_dim 256: every 2nd block and half of the
//   value groups, to keep its output state in registers), keeps its own (O, m, l) and skips
//   blocks no query of the tile sees; the wavefronts merge through LDS, and ranges split over
//   several workgroups (to fill the chip) merge in a second kernel, both in a fixed order.  The
//   next value group's scales, codes and column sums load as soon as the current group's are used;
//   the codes are P' * (255 / max P'), one reciprocal per (row, group, block).  At one wavefront
//   per SIMD the waits are the cost: a block's positions and key scales load during the
//   wavefront's previous block, and its first value group right behind its key codes.
#include "w4a8_kernels.h"

namespace w4a8 {
namespace {

constexpr int kSlots = 64;      // slots per block
constexpr int kQT = 32;         // queries per tile
constexpr int kAW = 4;          // wavefronts per workgroup
constexpr float kNegInf = -__builtin_inff();
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
                               // [nsplit][nh][nq][2]
};

__device__ __forceinline__ float wave_max32(float v) {          // max with the other lane half
    return fmaxf(v, __shfl_xor(v, 32, 64));
}

// DS = 2 (head_dim 256) splits the value groups over wavefront pairs: wavefront w takes groups
// (w / 2) * NG/2 .. +NG/2-1 of every second block (w % 2), so its output state is half as large
// (both of a pair compute the block's QK product and softmax, identically).
template <int D, int DS>
__global__ __launch_bounds__(64 * kAW) void attn_kernel(const AttnGeom ag,
                                                        const uint8_t *__restrict__ packed,
                                                        const AttnArgs a) {
#pragma clang fp contract(off)
    constexpr int NG = D / 32;           // value groups of the head
    constexpr int NGW = NG / DS;         // value groups of this wavefront
    constexpr int BL = kAW / DS;         // wavefronts sharing a group set (one block each)
    __shared__ float xm[kAW][kQT];
    __shared__ float xo[kAW - 1][64][16];
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

    // the query row's int8 codes (from the query prepass), as the B operands of the QK product:
    // lane (q, h) holds d = 32i + 16h .. +15 of each 32-wide chunk i
    v4i qb[NG];
    const int64_t qrow = (int64_t)head * a.nq + (qlive ? qi : 0);
#pragma unroll
    for (int i = 0; i < NG; ++i)
        qb[i] = qlive ? *reinterpret_cast<const v4i *>(a.q8 + qrow * D + 32 * i + 16 * half)
                      : v4i{0, 0, 0, 0};
    const float sq = qlive ? a.sq[qrow] : 0.0f;
    const float qscale = sq * a.scale;

    const int8_t *kqb = reinterpret_cast<const int8_t *>(packed + ag.off_kq) + (int64_t)kh * ag.nblk * kSlots * D;
    const float *skb = reinterpret_cast<const float *>(packed + ag.off_sk) + (int64_t)kh * ag.nblk * kSlots;
    const int32_t *posb = reinterpret_cast<const int32_t *>(packed + ag.off_pos) + (int64_t)kh * ag.nblk * kSlots;
    const int8_t *vtb = reinterpret_cast<const int8_t *>(packed + ag.off_vt) + (int64_t)kh * ag.nblk * D * kSlots;
    const float *svb = reinterpret_cast<const float *>(packed + ag.off_sv) + (int64_t)kh * ag.nblk * NG * kSlots;
    const int32_t *vsb = reinterpret_cast<const int32_t *>(packed + ag.off_vsum) + (int64_t)kh * ag.nblk * D;

    float mrun = kNegInf, lrun = 0.0f;
    v16f o[NGW];
#pragma unroll
    for (int g = 0; g < NGW; ++g)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[g][e] = 0.0f;

    const int b_lo = split * a.bps;
    const int b_hi = min(ag.nblk, b_lo + a.bps);
    // a block's slot positions and key scales for the lane's 32 slots: loaded while the
    // wavefront's previous block is processed, so visibility needs no wait at a block's start
    struct KBlock {
        int4 pos[2][4];
        float4 sk[2][4];
    };
    auto load_kblock = [&](int b, KBlock &k) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int base = b * kSlots + t * 32 + half * 16;
#pragma unroll
            for (int c = 0; c < 4; ++c) k.pos[t][c] = reinterpret_cast<const int4 *>(posb + base)[c];
#pragma unroll
            for (int c = 0; c < 4; ++c) k.sk[t][c] = reinterpret_cast<const float4 *>(skb + base)[c];
        }
    };
    // block b with its positions and key scales in kc; the wavefront's next block's load into kn
    auto block = [&](int b, const KBlock &kc, KBlock &kn) {
        if (b + BL < b_hi) load_kblock(b + BL, kn);
        // visibility of the lane's 32 slots (two subtiles of 16)
        float s[2][16];
        bool any = false;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            int pos16[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int4 pv = kc.pos[t][c];
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
        // the value side of group g: its scales for the lane's 32 slots, the transposed value
        // codes (A operands) and the column sums
        struct VGroup {
            float4 sv[2][4];
            v4i va[2];
            int4 vsum[4];
        };
        auto load_group = [&](int g, VGroup &v) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const float4 *svr = reinterpret_cast<const float4 *>(
                    svb + ((int64_t)b * NG + g) * kSlots + t * 32 + half * 16);
#pragma unroll
                for (int c = 0; c < 4; ++c) v.sv[t][c] = svr[c];
                v.va[t] = *reinterpret_cast<const v4i *>(
                    vtb + ((int64_t)b * D + 32 * g + col) * kSlots + t * 32 + half * 16);
            }
            const int4 *vsr = reinterpret_cast<const int4 *>(vsb + (int64_t)b * D + g * 32 + half * 16);
#pragma unroll
            for (int c = 0; c < 4; ++c) v.vsum[c] = vsr[c];
        };
        // the key codes of both subtiles, then the first value group: its loads complete while
        // the QK product and the softmax run
        v4i ka[2][NG];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int8_t *kr = kqb + ((int64_t)b * kSlots + t * 32 + col) * D + 16 * half;
#pragma unroll
            for (int i = 0; i < NG; ++i) ka[t][i] = *reinterpret_cast<const v4i *>(kr + 32 * i);
        }
        VGroup cur;
        load_group(dpart * NGW, cur);
        // S^T = K Q^T for the block's two 32-slot subtiles
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            v16i acc = {};
#pragma unroll
            for (int i = 0; i < NG; ++i)
                acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka[t][i], qb[i], acc, 0, 0, 0);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float4 kv = kc.sk[t][c];
                const float k4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (s[t][4 * c + i] == 0.0f)
                        s[t][4 * c + i] = static_cast<float>(acc[4 * c + i]) * qscale * k4[i];
            }
        }
        float mb = kNegInf;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) mb = fmaxf(mb, s[t][e]);
        mb = wave_max32(mb);
        const float mnew = fmaxf(mrun, mb);
        const float alpha = (mrun == kNegInf) ? 0.0f : expf(mrun - mnew);
        float p[2][16];
        float psum = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                p[t][e] = (s[t][e] == kNegInf) ? 0.0f : expf(s[t][e] - mnew);
                psum += p[t][e];
            }
        lrun = lrun * alpha + psum;
        mrun = (mb == kNegInf) ? mrun : mnew;
        const float keep = (mb == kNegInf) ? 1.0f : alpha;
        // one group's operands in flight: the next group's scales and codes load as soon as the
        // current group's are consumed, overlapping its matrix product and epilogue
#pragma unroll
        for (int g = 0; g < NGW; ++g) {
            // P folded with the value group's scale, quantized to u8 per (row, group, block)
            float mx = 0.0f;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float4 sv = cur.sv[t][c];
                    mx = fmaxf(mx, fmaxf(fmaxf(p[t][4 * c] * sv.x, p[t][4 * c + 1] * sv.y),
                                         fmaxf(p[t][4 * c + 2] * sv.z, p[t][4 * c + 3] * sv.w)));
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
                    const float sv4[4] = {cur.sv[t][c].x, cur.sv[t][c].y, cur.sv[t][c].z,
                                          cur.sv[t][c].w};
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
                iacc = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.va[t], pb, iacc, 0, 0, 0);
            }
            const int vs16[16] = {cur.vsum[0].x, cur.vsum[0].y, cur.vsum[0].z, cur.vsum[0].w,
                                  cur.vsum[1].x, cur.vsum[1].y, cur.vsum[1].z, cur.vsum[1].w,
                                  cur.vsum[2].x, cur.vsum[2].y, cur.vsum[2].z, cur.vsum[2].w,
                                  cur.vsum[3].x, cur.vsum[3].y, cur.vsum[3].z, cur.vsum[3].w};
            if (g + 1 < NGW) load_group(dpart * NGW + g + 1, cur);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float av = static_cast<float>(iacc[e] + 128 * vs16[e]);
                o[g][e] = fmaf(o[g][e], keep, sp * av);
            }
        }
    };
    // the wavefront's blocks b_lo + blane, + BL, ..., two per turn with the key sides ping-ponged
    KBlock k0, k1;
    if (b_lo + blane < b_hi) load_kblock(b_lo + blane, k0);
    for (int b = b_lo + blane; b < b_hi; b += 2 * BL) {
        block(b, k0, k1);
        if (b + BL < b_hi) block(b + BL, k1, k0);
    }

    // merge the states of the BL wavefronts of each group set (fixed order): M = max m_w, each
    // scaled by e^(m_w - M); the two group sets of DS = 2 hold the same (m, l)
    const float lw = lrun + __shfl_xor(lrun, 32, 64);
    if (half == 0) xm[wave][col] = mrun;
    __syncthreads();
    float mall = xm[dpart * BL][col];
#pragma unroll
    for (int w = 1; w < BL; ++w) mall = fmaxf(mall, xm[dpart * BL + w][col]);
    const float mine = (mrun == kNegInf) ? 0.0f : expf(mrun - mall);
    __syncthreads();
    if (half == 0) xm[wave][col] = lw * mine;
    __syncthreads();
    float lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < BL; ++w) lsum += xm[dpart * BL + w][col];
#pragma unroll
    for (int g = 0; g < NGW; ++g) {
        if (blane != 0)
#pragma unroll
            for (int e = 0; e < 16; ++e) xo[dpart * (BL - 1) + blane - 1][lane][e] = o[g][e] * mine;
        __syncthreads();
        if (blane == 0) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float v = o[g][e] * mine;
#pragma unroll
                for (int w = 1; w < BL; ++w) v += xo[dpart * (BL - 1) + w - 1][lane][e];
                o[g][e] = v;
            }
        }
        __syncthreads();
    }
    if (blane != 0 || !qlive) return;
    const int64_t row = (int64_t)head * a.nq + qi;
    float *orow;
    const bool stats = dpart == 0 && half == 0;
    if (a.nsplit == 1) {
        orow = a.o + row * D;
        if (stats) { a.m[row] = mall; a.l[row] = lsum; }
    } else {
        const int64_t rows = (int64_t)a.nh * a.nq, srow = (int64_t)split * rows + row;
        orow = a.work + srow * D;
        if (stats) {
            float *ml = a.work + a.nsplit * rows * D + 2 * srow;
            ml[0] = mall;
            ml[1] = lsum;
        }
    }
#pragma unroll
    for (int g = 0; g < NGW; ++g)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            orow[32 * (dpart * NGW + g) + 8 * (e >> 2) + 4 * half + (e & 3)] = o[g][e];
}

// The query prepass: one lane per 4 inputs of a row (a row is D/4 lanes of one wavefront),
// sq = max|row| / 127 and q8 = round-half-even(q / sq) in fp32, as the activation quantization.
__global__ __launch_bounds__(256) void attn_quant_q(const float4 *__restrict__ q, int64_t quads,
                                                    int lanes_per_row, int *__restrict__ q8,
                                                    float *__restrict__ sq) {
#pragma clang fp contract(off)
    const int64_t t = blockIdx.x * (int64_t)256 + threadIdx.x;
    const bool live = t < quads;
    const float4 v = live ? q[t] : make_float4(0.f, 0.f, 0.f, 0.f);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    for (int o = 1; o < lanes_per_row; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const float scale = amax / 127.0f;
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t w = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int c = 0;
        if (scale > 0.0f) c = static_cast<int>(fminf(fmaxf(rintf(e[i] / scale), -127.0f), 127.0f));
        w |= (static_cast<uint32_t>(c) & 0xFFu) << (8 * i);
    }
    if (!live) return;
    q8[t] = static_cast<int>(w);
    if (t % lanes_per_row == 0) sq[t / lanes_per_row] = scale;
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
        const float f = (st.x == kNegInf) ? 0.0f : expf(st.x - mall);
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
    if (c4 == 0) { m[row] = mall; l[row] = lsum; }
}

}  // namespace

int attn_splits(int nh, int nq, int nblk) {
    const int tiles = nh * ((nq + kQT - 1) / kQT);
    int s = (512 + tiles - 1) / tiles;                 // aim at two workgroups per CU
    s = max(1, min(s, (nblk + kAW - 1) / kAW));        // about one block per wavefront
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
    const int64_t quads = (int64_t)nh * nq * ag.d / 4;
    attn_quant_q<<<static_cast<unsigned>((quads + 255) / 256), 256, 0, stream>>>(
        reinterpret_cast<const float4 *>(q), quads, ag.d / 4, reinterpret_cast<int *>(q8), sq);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
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
