// The fp16-activation path (W4A16): 4-bit weights in the packed format times activations
// rounded to binary16, with fp32 group sums for the affine bias term.
//
// Source: "TensorFold PR #3215, simd_qmm on Metal: X's group sums and half operands from a
// prepass", section "What this changes": the prompt tiles multiply 4-bit g64 weights
// (w = scale * u + bias) with X as half; a prepass writes X as half and each row's 64-wide group
// sums for the bias term, added by the tiles' fixed tree ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)),
// each c a left-to-right sum of 8 consecutive inputs.  Output:
//   y[r][n] = sum_g ( sw[n][g] * sum_{k in g} w_int[n][k] * xh[r][k] + bw[n][g] * S[r][g] )
// with w_int = q (symmetric, -8..7) or u (affine, 0..15): the affine code enters unsigned, so the
// bias term takes the fp32 sums of X itself, not of its halves.
//
// Interleaved halves.  Within every 32-wide block of a row, the prepass stores xh so that the
// 4-byte word 4j + e holds the two inputs that nibble pair e of the weight chunk's dword j meets
// (see the packed chunk format: byte b of dword j holds k = 4j + b low and 16 + 4j + b high):
//   word 4j+0: k 4j, 4j+2     word 4j+1: k 16+4j, 18+4j
//   word 4j+2: k 4j+1, 4j+3   word 4j+3: k 17+4j, 19+4j
// so a dword of codes becomes four half pairs with one shift, one and-or and one packed add each
// (the magic-number conversion: 0x6400 | v is the binary16 value 1024 + v), and meets four
// consecutive words of xh: one v_dot2_f32_f16 each in the GEMV, one 16-byte operand in the GEMM.
//
// MI355X design.
//   Prepass: one lane per 8 consecutive inputs (two 16-byte loads); the octet's left-to-right
//   sum, then the tree as three cross-lane adds (lanes 8 apart form a group); the halves go
//   through LDS to be written interleaved, 16 bytes per lane.
//   GEMV (one row): a workgroup per 64-row panel, 8 wavefronts taking every 8th group, lane r
//   on panel row r (each chunk load is one contiguous KiB per wavefront); four groups in flight
//   per wavefront; the row's halves and sums are wave-uniform and come through scalar loads.
//   GEMM: a workgroup owns 64 rows x 128 channels, each wavefront 64 rows x its 32 channels as
//   two 32x32 tiles sharing one weight fragment (v_mfma_f32_32x32x16_f16, four per tile and
//   group: weight dword j against the 16-byte word run 4j..4j+3).  The rows' halves are staged
//   through two LDS buffers of 128 k (XOR-swizzled 16-byte units, so the 32 rows one operand
//   read touches spread over the banks); a stage's halves, weight chunks, scales and sums are
//   loaded two stages ahead into a register ring (one stage of work does not cover the latency
//   of a load under full load).  Each group ends with acc += sw * P (one FMA per element; the
//   lane's column is fixed, so sw is one register); the affine bias of a stage's two groups is
//   one update on the matrix unit (v_mfma_f32_32x32x2_f32, k slot h = group 2s + h: rows' sums
//   times the channel's bias).  The tiles of a last, partial round over the CUs are split over
//   four workgroups (one k quarter per wavefront, outputs added in LDS in a fixed order), as in
//   the int8 GEMM.
#include "w4a8_kernels.h"

#include <type_traits>

namespace w4a8 {
namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));

constexpr int kGroupA16 = 64;

// The half pair e of code dword w (already XORed with 0x88888888, so each nibble holds
// v = code + 8 for the symmetric format and u for the affine one) as binary16 w_int values.
template <int FMT>
__device__ __forceinline__ uint32_t half_pair(uint32_t w, int e) {
    const uint32_t h = ((w >> (4 * e)) & 0x000F000Fu) | 0x64006400u;    // 1024 + v
    const _Float16 off = static_cast<_Float16>(FMT == kFmtAffine ? -1024.0f : -1032.0f);
    const h2_t r = __builtin_bit_cast(h2_t, h) + h2_t{off, off};        // exact: |w_int| <= 15
    return __builtin_bit_cast(uint32_t, r);
}

// ---- prepass

__global__ __launch_bounds__(256) void prep_a16_kernel(const float4 *__restrict__ x,
                                                       int64_t octets, int64_t m, int k,
                                                       uint4 *__restrict__ xh,
                                                       float *__restrict__ xsf) {
#pragma clang fp contract(off)
    __shared__ _Float16 tile[256 * 8];                 // the block's octets as halves, in order
    const int64_t t = blockIdx.x * (int64_t)256 + threadIdx.x;
    const bool live = t < octets;
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (live) {
        const float4 a = x[2 * t], b = x[2 * t + 1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    float c = v[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) c = c + v[i];
    // ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)): lanes 8 apart hold the group's octets in order; an
    // IEEE add is commutative, so every lane of the group ends with the same bits
    c = c + __shfl_xor(c, 1, 64);
    c = c + __shfl_xor(c, 2, 64);
    c = c + __shfl_xor(c, 4, 64);
    const int64_t per_row = k / 8;
    if (live && (t & 7) == 0) {
        const int64_t row = t / per_row;
        const int64_t g = (t % per_row) / 8;
        xsf[g * m + row] = c;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[threadIdx.x * 8 + i] = static_cast<_Float16>(v[i]);
    __syncthreads();
    if (!live) return;
    // this lane writes word run 4j..4j+3 of its 32-wide block (4 lanes per block, aligned)
    const int base = (threadIdx.x & ~3) * 8;
    const int j = threadIdx.x & 3;
    const int src[8] = {4 * j, 4 * j + 2, 16 + 4 * j, 18 + 4 * j,
                        4 * j + 1, 4 * j + 3, 17 + 4 * j, 19 + 4 * j};
    uint32_t wd[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = __builtin_bit_cast(uint16_t, tile[base + src[2 * e]]);
        const uint32_t hi = __builtin_bit_cast(uint16_t, tile[base + src[2 * e + 1]]);
        wd[e] = lo | (hi << 16);
    }
    xh[t] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
}

// ---- GEMV (one activation row)

constexpr int kA16Waves = 8;
constexpr int kA16Ring = 4;                            // groups in flight per wavefront
constexpr int kA16FusedIters = kFusedMaxK / 8 / (64 * kA16Waves);   // fused: octets per thread

// FUSED: the prepass runs in every workgroup (x is the fp32 row; xw / xsf are not read): the
// row's halves in the interleaved order and its group sums go to LDS with the prepass's own
// arithmetic, and workgroup 0 also writes them to xh_out / xsf_out.  The row's loads are issued
// before the weight loads, so the prepass waits for x only (loads complete in issue order).
template <int FMT, bool FUSED>
__global__ __launch_bounds__(64 * kA16Waves) void gemv_a16_kernel(const uint8_t *__restrict__ packed,
                                                                  const Geom geom,
                                                                  const uint32_t *__restrict__ xw,
                                                                  const float *__restrict__ xsf,
                                                                  float *__restrict__ y,
                                                                  const float *__restrict__ x,
                                                                  uint4 *__restrict__ xh_out,
                                                                  float *__restrict__ xsf_out) {
#pragma clang fp contract(off)
    constexpr int MB = (FMT == kFmtAffine) ? 4 : 2;
    __shared__ float red[kA16Waves][64];
    __shared__ __attribute__((aligned(16))) uint32_t lxw[FUSED ? kFusedMaxK / 2 : 1];
    __shared__ float lxsf[FUSED ? kFusedMaxK / kGroupA16 : 1];
    __shared__ _Float16 tile[FUSED ? 64 * kA16Waves * 8 : 1];
    const int noct = geom.k / 8;
    float4 xr[FUSED ? 2 * kA16FusedIters : 1];
    if constexpr (FUSED) {
        const rsrc_t rx = make_rsrc(x, (uint64_t)geom.k * 4);
#pragma unroll
        for (int i = 0; i < kA16FusedIters; ++i) {
            const int o = threadIdx.x + 64 * kA16Waves * i;
            xr[2 * i] = __builtin_bit_cast(float4, ld128(rx, o < noct ? o * 32 : kOOB));
            xr[2 * i + 1] = __builtin_bit_cast(float4, ld128(rx, o < noct ? o * 32 + 16 : kOOB));
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int p = blockIdx.x;
    const int kc = geom.k / kChunkK;
    const int ng = geom.k / kGroupA16;
    const int nblk = (ng + 3) / 4;
    const rsrc_t rc = make_rsrc(packed + geom.off_codes + (uint64_t)p * kc * 1024,
                                (uint64_t)kc * 1024);
    const rsrc_t rm = make_rsrc(packed + geom.off_meta + (uint64_t)p * nblk * 256 * MB,
                                (uint64_t)nblk * 256 * MB);
    auto code_off = [&](int g, int h) {
        return g < ng ? ((2 * g + h) * 64 + lane) * 16 : kOOB;
    };
    auto meta_off = [&](int g) {
        return g < ng ? (((g >> 2) * 64 + lane) * 4 + (g & 3)) * MB : kOOB;
    };
    v4i ring[kA16Ring][2];
    uint32_t meta[kA16Ring];
#pragma unroll
    for (int s = 0; s < kA16Ring; ++s) {
        const int g = wave + s * kA16Waves;
        ring[s][0] = ld128_stream(rc, code_off(g, 0));
        ring[s][1] = ld128_stream(rc, code_off(g, 1));
        meta[s] = (MB == 4) ? ld32(rm, meta_off(g)) : ld16(rm, meta_off(g));
    }
    const uint32_t *xsrc;                             // the row's halves and sums: LDS when fused
    const float *xsfsrc;
    if constexpr (FUSED) {
        // per octet as the prepass kernel: the left-to-right sum of 8, the tree over a group's 8
        // octets (8 aligned lanes, all active or all inactive), the halves through a staging tile
        // into the interleaved word order (a 32-wide block is 4 aligned lanes)
#pragma unroll
        for (int i = 0; i < kA16FusedIters; ++i) {
            const int o = threadIdx.x + 64 * kA16Waves * i;
            if (64 * kA16Waves * i >= noct) break;    // (uniform across the workgroup)
            const bool live = o < noct;
            const float4 a = xr[2 * i], b = xr[2 * i + 1];
            const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            float c = v[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) c = c + v[e];
            c = c + __shfl_xor(c, 1, 64);
            c = c + __shfl_xor(c, 2, 64);
            c = c + __shfl_xor(c, 4, 64);
            if (live && (o & 7) == 0) {
                lxsf[o / 8] = c;
                if (blockIdx.x == 0) xsf_out[o / 8] = c;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) tile[threadIdx.x * 8 + e] = static_cast<_Float16>(v[e]);
            __syncthreads();
            if (live) {
                const int base = (threadIdx.x & ~3) * 8;
                const int j = threadIdx.x & 3;
                const int src[8] = {4 * j, 4 * j + 2, 16 + 4 * j, 18 + 4 * j,
                                    4 * j + 1, 4 * j + 3, 17 + 4 * j, 19 + 4 * j};
                uint32_t wd[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = __builtin_bit_cast(uint16_t, tile[base + src[2 * e]]);
                    const uint32_t hi = __builtin_bit_cast(uint16_t, tile[base + src[2 * e + 1]]);
                    wd[e] = lo | (hi << 16);
                }
                const uint4 q = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                reinterpret_cast<uint4 *>(lxw)[o] = q;
                if (blockIdx.x == 0) xh_out[o] = q;
            }
            __syncthreads();
        }
        xsrc = lxw;
        xsfsrc = lxsf;
    } else {
        xsrc = xw;
        xsfsrc = xsf;
    }
    float acc = 0.0f;
    for (int g0 = wave; g0 < ng; g0 += kA16Ring * kA16Waves) {
#pragma unroll
        for (int s = 0; s < kA16Ring; ++s) {
            const int g = g0 + s * kA16Waves;
            if (g < ng) {
                const uint32_t *xg = xsrc + 32 * g;      // the group's 64 halves: wave-uniform
                float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // one chain per code dword
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t w = static_cast<uint32_t>(ring[s][h][j]) ^ 0x88888888u;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t wp = half_pair<FMT>(w, e);
                            d4[j] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, wp),
                                                           __builtin_bit_cast(h2_t, xg[16 * h + 4 * j + e]),
                                                           d4[j], false);
                        }
                    }
                }
                const float dot = (d4[0] + d4[1]) + (d4[2] + d4[3]);
                const float sw = half_bits_to_float(meta[s] & 0xFFFFu);
                acc = fmaf(sw, dot, acc);
                if (FMT == kFmtAffine) acc = fmaf(half_bits_to_float(meta[s] >> 16), xsfsrc[g], acc);
            }
            const int gn = g + kA16Ring * kA16Waves;
            ring[s][0] = ld128_stream(rc, code_off(gn, 0));
            ring[s][1] = ld128_stream(rc, code_off(gn, 1));
            meta[s] = (MB == 4) ? ld32(rm, meta_off(gn)) : ld16(rm, meta_off(gn));
        }
    }
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    float s = red[0][lane];
#pragma unroll
    for (int w = 1; w < kA16Waves; ++w) s += red[w][lane];
    const int row = p * kPanelRows + lane;
    if (row < geom.n) y[row] = s;
}

// ---- GEMM (several activation rows)

constexpr int kA16BN = 128;                        // channels per workgroup (4 wavefronts x 32)
constexpr int kA16SK = 128;                        // k per LDS stage (two groups)
constexpr int kA16Split = 4;                       // k quarters of a split workgroup

// Everything one LDS stage needs from memory, loaded two stages ahead: the rows' halves (four
// 16-byte units per thread), the lane's weight chunk of each of the stage's two groups, those
// groups' scale (and bias) of the lane's channel, and each tile's row sums of the lane's group
// (group 2s for lanes 0-31, 2s+1 for lanes 32-63: the two k slots of the bias update).
struct StageRegs {
    v4i a[4];
    v4i b[2];
    uint32_t meta[2];
    float sum[2];
};

// Workgroups from nfull on take a quarter of a tile each: its 32-channel group cgrp over all of
// k, the four wavefronts one k quarter each (one 32-wide chunk per stage), their outputs added in
// LDS in quarter order at the end (the launcher splits the tiles of a last, partial round).
template <int FMT>
__global__ __launch_bounds__(256, 2) void gemm_a16_kernel(const uint8_t *__restrict__ packed,
                                                          const Geom geom, int m,
                                                          const uint16_t *__restrict__ xh,
                                                          const float *__restrict__ xsf,
                                                          float *__restrict__ y, int nfull) {
    constexpr int MB = (FMT == kFmtAffine) ? 4 : 2;
    __shared__ __attribute__((aligned(16))) v4i lds[2][64 * 16];   // [buf][row][16-byte unit]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int r32 = lane & 31;

    const int mtiles = (m + 63) / 64;
    const bool split = static_cast<int>(blockIdx.x) >= nfull;   // workgroup-uniform
    int bid = blockIdx.x;
    int cgrp = 0;
    if (split) {
        cgrp = (bid - nfull) % kA16Split;
        bid = nfull + (bid - nfull) / kA16Split;
    } else if (nfull % 8 == 0) {
        bid = (bid % 8) * (nfull / 8) + bid / 8;            // consecutive tiles on one XCD
    }
    const int mt = bid % mtiles, nt = bid / mtiles;
    const int m0 = mt * 64;
    const int c0 = nt * kA16BN + (split ? cgrp : wave) * 32;   // this wavefront's first channel
    const bool wact = c0 < geom.n_pad;                      // panels are whole: all or none
    const int col = c0 + r32;
    const int p = col / kPanelRows, prow = col % kPanelRows;
    const int k = geom.k;
    const int kc = k / kChunkK;
    const int ng = k / kGroupA16;
    const int nblk = (ng + 3) / 4;
    const int nstage = (k + kA16SK - 1) / kA16SK;

    const rsrc_t rc = make_rsrc(packed + geom.off_codes + (uint64_t)(wact ? p : 0) * kc * 1024,
                                wact ? (uint64_t)kc * 1024 : 0);
    const rsrc_t rm = make_rsrc(packed + geom.off_meta + (uint64_t)(wact ? p : 0) * nblk * 256 * MB,
                                wact ? (uint64_t)nblk * 256 * MB : 0);
    const rsrc_t rx = make_rsrc(xh, (uint64_t)m * k * 2);
    const rsrc_t rs = make_rsrc(xsf, (uint64_t)ng * m * 4);

    auto load_stage = [&](int s, StageRegs &r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = i * 16 + (tid >> 4), u = tid & 15;
            const int kk = s * kA16SK + 8 * u;
            const bool ok = (m0 + rr < m) && (kk < k);
            r.a[i] = ld128(rx, ok ? ((m0 + rr) * k + kk) * 2 : kOOB);
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int g = 2 * s + st;
            r.b[st] = ld128(rc, g < ng ? ((2 * g + half) * 64 + prow) * 16 : kOOB);
            const int mo = g < ng ? (((g >> 2) * 64 + prow) * 4 + (g & 3)) * MB : kOOB;
            r.meta[st] = (MB == 4) ? ld32(rm, mo) : ld16(rm, mo);
        }
        const int gs = 2 * s + half;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int row = m0 + 32 * t + r32;
            const bool ok = FMT == kFmtAffine && gs < ng && row < m;
            r.sum[t] = __builtin_bit_cast(float, ld32(rs, ok ? (gs * m + row) * 4 : kOOB));
        }
    };
    auto store_a = [&](int buf, const StageRegs &r) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = i * 16 + (tid >> 4), u = tid & 15;
            lds[buf][rr * 16 + (u ^ (rr & 7))] = r.a[i];
        }
    };

    v16f acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
    }
    const v16f zero16 = acc[0];

    if (split) {
        // Stage s of a split workgroup holds chunk s of each k quarter: LDS unit u of a row is
        // unit u % 4 of quarter u / 4 (32 k each); wavefront q (quarter q) takes its units
        // 4q .. 4q+3, chunk q k/128 + s of its channel and group (q k/128 + s) / 2, whose
        // epilogue follows its second chunk (a quarter starts on a group: k % 256 == 0).
        const int qchunks = k / (kA16Split * 32);            // chunks per quarter
        const int c_first = wave * qchunks;
        auto load_split = [&](int s, StageRegs &r) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = i * 16 + (tid >> 4), u = tid & 15;
                const int kk = (u >> 2) * (k / kA16Split) + s * 32 + 8 * (u & 3);
                const bool ok = (m0 + rr < m) && s < qchunks;
                r.a[i] = ld128(rx, ok ? ((m0 + rr) * k + kk) * 2 : kOOB);
            }
            const int c = c_first + s;
            const int g = c >> 1;
            const bool okc = s < qchunks;
            r.b[0] = ld128(rc, okc ? (c * 64 + prow) * 16 : kOOB);
            const int mo = okc ? (((g >> 2) * 64 + prow) * 4 + (g & 3)) * MB : kOOB;
            r.meta[0] = (MB == 4) ? ld32(rm, mo) : ld16(rm, mo);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int row = m0 + 32 * t + r32;
                // the bias update's k slot 0 (lanes 0-31) carries the group, slot 1 nothing
                const bool ok = FMT == kFmtAffine && okc && half == 0 && row < m;
                r.sum[t] = __builtin_bit_cast(float, ld32(rs, ok ? (g * m + row) * 4 : kOOB));
            }
        };
        StageRegs sring[2];
        v16f part[2] = {zero16, zero16};
        load_split(0, sring[0]);
        if (qchunks > 1) load_split(1, sring[1]);
        store_a(0, sring[0]);
        __syncthreads();
        auto split_stage = [&](auto slot_c, int s) {
            constexpr int slot = decltype(slot_c)::value;
            const v4i bch = sring[slot].b[0];
            const uint32_t meta = sring[slot].meta[0];
            const float sum[2] = {sring[slot].sum[0], sring[slot].sum[1]};
            if (s + 2 < qchunks) load_split(s + 2, sring[slot]);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                // lane half h: dword 2 jj + h of the chunk against unit 4 q + 2 jj + h
                const uint32_t w = static_cast<uint32_t>(bch[2 * jj + half]) ^ 0x88888888u;
                const v4i bw4 = {static_cast<int>(half_pair<FMT>(w, 0)),
                                 static_cast<int>(half_pair<FMT>(w, 1)),
                                 static_cast<int>(half_pair<FMT>(w, 2)),
                                 static_cast<int>(half_pair<FMT>(w, 3))};
                const v8h_t bop = __builtin_bit_cast(v8h_t, bw4);
                const int unit = 4 * wave + 2 * jj + half;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int rr = 32 * t + r32;
                    const v8h_t aop =
                        __builtin_bit_cast(v8h_t, lds[slot][rr * 16 + (unit ^ (rr & 7))]);
                    part[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop, part[t], 0, 0, 0);
                }
            }
            if (s & 1) {                                   // the group's second chunk
                const float sw = half_bits_to_float(meta & 0xFFFFu);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[t][e] = fmaf(sw, part[t][e], acc[t][e]);
                    part[t] = zero16;
                }
                if (FMT == kFmtAffine) {
                    const float bw = half == 0 ? half_bits_to_float(meta >> 16) : 0.0f;
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(sum[t], bw, acc[t], 0, 0, 0);
                }
            }
            if (s + 1 < qchunks) store_a(slot ^ 1, sring[slot ^ 1]);
            __syncthreads();
        };
        for (int s = 0; s < qchunks; s += 2) {
            split_stage(std::integral_constant<int, 0>{}, s);
            split_stage(std::integral_constant<int, 1>{}, s + 1);
        }
        if (!wact) return;                                 // (workgroup-uniform)
        float *xch = reinterpret_cast<float *>(&lds[0][0]);   // [3][32][64] fp32, 24 KiB
        if (wave > 0) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e) xch[((wave - 1) * 32 + 16 * t + e) * 64 + lane] = acc[t][e];
        }
        __syncthreads();
        if (wave != 0 || col >= geom.n) return;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
                float v = acc[t][e];
#pragma unroll
                for (int w = 0; w < kA16Split - 1; ++w) v += xch[(w * 32 + 16 * t + e) * 64 + lane];
                if (row < m) y[(int64_t)row * geom.n + col] = v;
            }
        }
        return;
    }

    // stage s reads LDS buffer s & 1 and its loads sit in ring slot s & 1; at stage s the slot
    // is refilled with stage s + 2, and at its end stage s + 1's halves go to the other buffer
    StageRegs ring[2];
    load_stage(0, ring[0]);
    if (nstage > 1) load_stage(1, ring[1]);
    store_a(0, ring[0]);
    __syncthreads();

    auto stage = [&](auto slot_c, int s) {
        constexpr int slot = decltype(slot_c)::value;
        const v4i b[2] = {ring[slot].b[0], ring[slot].b[1]};
        const uint32_t meta[2] = {ring[slot].meta[0], ring[slot].meta[1]};
        const float sum[2] = {ring[slot].sum[0], ring[slot].sum[1]};
        if (s + 2 < nstage) load_stage(s + 2, ring[slot]);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const int g = 2 * s + st;
            if (g >= ng) break;
            v16f part[2] = {zero16, zero16};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = static_cast<uint32_t>(b[st][j]) ^ 0x88888888u;
                const v4i bw4 = {static_cast<int>(half_pair<FMT>(w, 0)),
                                 static_cast<int>(half_pair<FMT>(w, 1)),
                                 static_cast<int>(half_pair<FMT>(w, 2)),
                                 static_cast<int>(half_pair<FMT>(w, 3))};
                const v8h_t bop = __builtin_bit_cast(v8h_t, bw4);
                const int unit = (2 * st + half) * 4 + j;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int rr = 32 * t + r32;
                    const v8h_t aop =
                        __builtin_bit_cast(v8h_t, lds[slot][rr * 16 + (unit ^ (rr & 7))]);
                    part[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(aop, bop, part[t], 0, 0, 0);
                }
            }
            const float sw = half_bits_to_float(meta[st] & 0xFFFFu);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[t][e] = fmaf(sw, part[t][e], acc[t][e]);
            }
        }
        if (FMT == kFmtAffine) {
            // both groups' bias at once: k slot h of the update is group 2s + h
            const float bw = half_bits_to_float(meta[half] >> 16);
#pragma unroll
            for (int t = 0; t < 2; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(sum[t], bw, acc[t], 0, 0, 0);
        }
        if (s + 1 < nstage) store_a(slot ^ 1, ring[slot ^ 1]);
        __syncthreads();
    };
    for (int s = 0; s < nstage; s += 2) {
        stage(std::integral_constant<int, 0>{}, s);
        if (s + 1 < nstage) stage(std::integral_constant<int, 1>{}, s + 1);
    }

    if (!wact || col >= geom.n) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = m0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
            if (row < m) y[(int64_t)row * geom.n + col] = acc[t][e];
        }
    }
}

}  // namespace

hipError_t launch_prep_a16(const float *x, int64_t m, int k, uint16_t *xh, float *xsf,
                           hipStream_t stream) {
    const int64_t octets = m * (int64_t)k / 8;
    if (octets == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>((octets + 255) / 256);
    prep_a16_kernel<<<grid, 256, 0, stream>>>(reinterpret_cast<const float4 *>(x), octets, m, k,
                                              reinterpret_cast<uint4 *>(xh), xsf);
    return hipGetLastError();
}

hipError_t launch_linear_a16(const Geom &g, const uint8_t *packed, int m, const uint16_t *xh,
                             const float *xsf, float *y, hipStream_t stream) {
    if (m == 0) return hipSuccess;
    if (m == 1) {
        const unsigned grid = static_cast<unsigned>(g.n_pad / kPanelRows);
        const uint32_t *xw = reinterpret_cast<const uint32_t *>(xh);
        if (g.fmt == kFmtAffine)
            gemv_a16_kernel<kFmtAffine, false><<<grid, 64 * kA16Waves, 0, stream>>>(
                packed, g, xw, xsf, y, nullptr, nullptr, nullptr);
        else
            gemv_a16_kernel<kFmtSym, false><<<grid, 64 * kA16Waves, 0, stream>>>(
                packed, g, xw, xsf, y, nullptr, nullptr, nullptr);
        return hipGetLastError();
    }
    const int tiles = ((m + 63) / 64) * ((g.n_pad + kA16BN - 1) / kA16BN);
    const int nfull = (g.k % (kA16Split * kGroupA16) == 0) ? whole_tiles(tiles) : tiles;
    const unsigned grid = static_cast<unsigned>(nfull + kA16Split * (tiles - nfull));
    if (g.fmt == kFmtAffine)
        gemm_a16_kernel<kFmtAffine><<<grid, 256, 0, stream>>>(packed, g, m, xh, xsf, y, nfull);
    else
        gemm_a16_kernel<kFmtSym><<<grid, 256, 0, stream>>>(packed, g, m, xh, xsf, y, nfull);
    return hipGetLastError();
}

hipError_t launch_linear_a16_fused(const Geom &g, const uint8_t *packed, const float *x,
                                   uint16_t *xh, float *xsf, float *y, hipStream_t stream) {
    if (g.k > kFusedMaxK) return hipErrorInvalidValue;
    const unsigned grid = static_cast<unsigned>(g.n_pad / kPanelRows);
    uint4 *xh4 = reinterpret_cast<uint4 *>(xh);
    if (g.fmt == kFmtAffine)
        gemv_a16_kernel<kFmtAffine, true><<<grid, 64 * kA16Waves, 0, stream>>>(
            packed, g, nullptr, nullptr, y, x, xh4, xsf);
    else
        gemv_a16_kernel<kFmtSym, true><<<grid, 64 * kA16Waves, 0, stream>>>(
            packed, g, nullptr, nullptr, y, x, xh4, xsf);
    return hipGetLastError();
}

}  // namespace w4a8
