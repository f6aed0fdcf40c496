// Int8 weights (W8A8) and 1-, 2- and 3-bit codebook weights (CQ1, CQ2 / W2A8, CQ3), against the
// same int8 activations, scales and group sums as the 4-bit formats; all decode to int8 weights
// in registers.
//
// Source: "geistlib issue #500: native W*A8 int8 GEMM for prefill", sections "Scope" and
// "Design sketch": a W8A8 inner kernel beside the W4A8 one, both behind a load-time repack,
// sharing the activation quantization; w8a8 GEMV and GEMM entry points.
//   y[r][n] = sum_g xs[r][g] * sw[n][g] * D[r][n][g],  D = sum_{k in g} xq[r][k] * w8[n][k]
//
// Codebooks: "cactus PR #697", the CQ1-CQ4 codebook family (a b-bit index per weight into a
// per-row table of 2^b int8 entries, one fp16 scale per group; CQ4 is the 4-bit codebook
// format); "geistlib issue #500", "Acceptance criteria" (W2A8 models).
//
// Packed layouts: per 64-row panel and per k chunk, 64 rows x 16 bytes.  Int8: chunk c of row r
// is w8[r][16c .. 16c+15].  CQ2: a chunk holds 64 k as four 32-bit words in the k order
// 0-15, 32-47, 16-31, 48-63, and in a word covering k = b .. b+15 the index of k = b + 4s + j sits
// at bits 8j + 2s, so (w >> 2s) & 0x03030303 selects four consecutive weights and one v_perm
// against the row's codebook dword turns them into int8; the words' order lets a GEMM lane half
// read its two MFMA blocks of a chunk as one 8-byte run.
// CQ1 and CQ3 (bit-plane formats): a chunk covers 128 k in P planes of 64 rows x 16 bytes
// (P = 1 for CQ1, 3 for CQ3), plane-major inside the chunk so that every load of a wavefront is
// one contiguous KiB.  The bit plane: word 2h + q covers k = 64q + 16h + 4s + j at bit
// 8j + s and k = 64q + 32 + 16h + 4s + j at bit 8j + 4 + s (the halves h of MFMA blocks 2q and
// 2q + 1), so (w >> (4P + s)) & 0x01010101 is one bit of four consecutive weights and a GEMM
// lane half again reads 8 bytes.  CQ1 stores the index there; CQ3 stores index >> 2 there and
// index & 3 in planes 0 and 1 (CQ2's layout for k = 0..63 and 64..127), and one v_perm over the
// two codebook dwords (entries 0-3 in the second source, 4-7 in the first) decodes the 3-bit
// selectors.  Scales: the symmetric format's blocked metadata; codebooks: one dword per row
// (CQ1: entries in bytes 0 and 1, CQ2), two dwords per row (CQ3).
//
// MI355X design.
//   GEMV (one row): a workgroup per panel, 8 wavefronts over the groups, lane r on panel row r
//   (a chunk load is one contiguous KiB per wavefront); v_dot4_i32_i8 of the weight bytes
//   against the row's codes, which are wave-uniform and come through scalar loads; a ring of
//   256 k of groups in flight per wavefront.
//   GEMM: 64 rows x 128 channels per workgroup; each wavefront two 32x32 int32 tiles
//   (v_mfma_i32_32x32x32_i8) sharing its weight bytes, which enter the matrix unit unchanged
//   (lane (c, h) reads chunk 2j + h of its channel: k slots 16h .. 16h+15 of 32-wide block j);
//   activation codes staged through two LDS buffers of 128 k (XOR-swizzled 16-byte units), a
//   stage's codes, weight chunks, scales and activation scales loaded two stages ahead into a
//   register ring.  Each group ends with coef = xs (x) sw for both tiles as one two-block outer
//   product on the matrix unit (v_mfma_f32_32x32x1_2b_f32: block t = tile t) and
//   acc += coef * float(D): a convert and an FMA per element.
#include "w4a8_kernels.h"

#include <type_traits>

namespace w4a8 {
namespace {

constexpr int kW8Chunk = 16;        // k per 16-byte chunk
constexpr int kW8Waves = 8;
constexpr int kBitChunk = 128;      // k per chunk of the bit-plane formats
constexpr int kMinUnits = 4;        // GEMV: groups (chunks) per wavefront before panels share
constexpr int kMinGrid = 1024;      // GEMV: fewest workgroups once panels share one
constexpr int kFusedQuads = kFusedMaxK / 4 / (64 * kW8Waves);   // fused prepass: quads per thread

// The prepass fused into a one-row GEMV: every workgroup quantizes the whole row into LDS
// (workgroup 0 also writes xq, xs and xsum).  issue() loads the thread's quads and goes before
// the kernel's weight loads, so run() waits for x only (loads complete in issue order).
template <int G, bool ROT>
struct FusedPrep {
    v4i xr[kFusedQuads];
    __device__ __forceinline__ void issue(const FusedIO &io, int k) {
        const rsrc_t rx = make_rsrc(io.x, (uint64_t)k * 4);
#pragma unroll
        for (int i = 0; i < kFusedQuads; ++i) {
            const int q = threadIdx.x + 64 * kW8Waves * i;
            xr[i] = ld128(rx, q < k / 4 ? q * 16 : kOOB);
        }
    }
    // A wavefront's quads are 64 consecutive ones, so a group's G/4 lanes and a rotation block's
    // 32 are aligned runs that are all active or all inactive (k is a multiple of G and of 128).
    // lxsum (when not null) also receives the group sums
    __device__ __forceinline__ void run(const FusedIO &io, int k, int *lxq, float *lxs,
                                        int *lxsum = nullptr) {
        const int lane = threadIdx.x & 63;
#pragma unroll
        for (int i = 0; i < kFusedQuads; ++i) {
            const int q = threadIdx.x + 64 * kW8Waves * i;
            if (q < k / 4) {
                float scale;
                int sum;
                const v4f xf = __builtin_bit_cast(v4f, xr[i]);
                const int codes = prep_quad<G, ROT>(make_float4(xf[0], xf[1], xf[2], xf[3]), lane,
                                                    scale, sum);
                lxq[q] = codes;
                const bool leader = (q & (G / 4 - 1)) == 0;
                if (leader) lxs[q / (G / 4)] = scale;
                if (leader && lxsum) lxsum[q / (G / 4)] = sum;
                if (blockIdx.x == 0) {
                    reinterpret_cast<int *>(io.xq)[q] = codes;
                    if (leader) {
                        io.xs[q / (G / 4)] = scale;
                        io.xsum[q / (G / 4)] = sum;
                    }
                }
            }
        }
        __syncthreads();
    }
};

template <int FMT>
constexpr bool bit_plane = FMT == kFmtCQ1 || FMT == kFmtCQ3;
template <int FMT>
constexpr int planes = FMT == kFmtCQ3 ? 3 : 1;     // 16-byte planes per row per chunk

// ---- packing

__global__ __launch_bounds__(256) void pack_codes_w8_kernel(const int8_t *__restrict__ w8, int n,
                                                            int k, int64_t total,
                                                            uint4 *__restrict__ out) {
    const int kc = k / kW8Chunk;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int r = static_cast<int>(t % kPanelRows);
        const int64_t rest = t / kPanelRows;
        const int c = static_cast<int>(rest % kc);
        const int64_t row = (rest / kc) * kPanelRows + r;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (row < n) v = *reinterpret_cast<const uint4 *>(w8 + row * (int64_t)k + (int64_t)c * kW8Chunk);
        out[t] = v;
    }
}

__global__ __launch_bounds__(256) void pack_codes_cq2_kernel(const uint8_t *__restrict__ codes,
                                                             const int8_t *__restrict__ cb, int n,
                                                             int k, int64_t total,
                                                             uint4 *__restrict__ out,
                                                             uint32_t *__restrict__ cb_out) {
    const int kc = k / 64;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int r = static_cast<int>(t % kPanelRows);
        const int64_t rest = t / kPanelRows;
        const int c = static_cast<int>(rest % kc);
        const int64_t row = (rest / kc) * kPanelRows + r;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (row < n) {
            const uint8_t *src = codes + row * (int64_t)(k / 4) + (int64_t)c * 16;   // 64 k
            const int kq[4] = {0, 32, 16, 48};            // k offset of word position q
            for (int q = 0; q < 4; ++q)
                for (int s4 = 0; s4 < 4; ++s4)
                    for (int j = 0; j < 4; ++j) {
                        const int kk = kq[q] + 4 * s4 + j;                     // k within chunk
                        const uint32_t idx = (src[kk / 4] >> (2 * (kk % 4))) & 3u;
                        w[q] |= idx << (8 * j + 2 * s4);
                    }
        }
        out[t] = make_uint4(w[0], w[1], w[2], w[3]);
        if (c == 0) {
            uint32_t v = 0u;
            if (row < n)
                for (int e = 0; e < 4; ++e)
                    v |= static_cast<uint32_t>(static_cast<uint8_t>(cb[row * 4 + e])) << (8 * e);
            cb_out[row] = v;
        }
    }
}

template <int FMT>
__global__ __launch_bounds__(256) void pack_codes_bits_kernel(const uint8_t *__restrict__ codes,
                                                              const int8_t *__restrict__ cb,
                                                              int n, int k, int64_t total,
                                                              uint4 *__restrict__ out,
                                                              uint32_t *__restrict__ cb_out) {
    constexpr int P = planes<FMT>;
    constexpr int NE = FMT == kFmtCQ3 ? 8 : 2;         // codebook entries
    const int kc = (k + kBitChunk - 1) / kBitChunk;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int r = static_cast<int>(t % kPanelRows);
        const int64_t rest = t / kPanelRows;         // panel * kc + chunk
        const int c = static_cast<int>(rest % kc);
        const int64_t row = (rest / kc) * kPanelRows + r;
        // the index of k = 128c + kk (zero past the weight)
        auto index = [&](int kk) -> uint32_t {
            const int ka = c * kBitChunk + kk;
            if (row >= n || ka >= k) return 0u;
            if (FMT == kFmtCQ1) return (codes[row * (int64_t)(k / 8) + ka / 8] >> (ka % 8)) & 1u;
            return codes[row * (int64_t)k + ka] & 7u;
        };
        uint32_t bits[4] = {0u, 0u, 0u, 0u};
        for (int h = 0; h < 2; ++h)
            for (int q = 0; q < 2; ++q)
                for (int pb = 0; pb < 2; ++pb)                 // block 2q + pb
                    for (int s4 = 0; s4 < 4; ++s4)
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t idx = index(64 * q + 32 * pb + 16 * h + 4 * s4 + j);
                            bits[2 * h + q] |= (FMT == kFmtCQ3 ? idx >> 2 : idx)
                                               << (8 * j + 4 * pb + s4);
                        }
        uint4 *dst = out + rest * P * kPanelRows + r;
        if (FMT == kFmtCQ3) {
            const int kq[4] = {0, 32, 16, 48};            // k offset of word position q
            for (int u = 0; u < 2; ++u) {
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                for (int q = 0; q < 4; ++q)
                    for (int s4 = 0; s4 < 4; ++s4)
                        for (int j = 0; j < 4; ++j)
                            w[q] |= (index(64 * u + kq[q] + 4 * s4 + j) & 3u) << (8 * j + 2 * s4);
                dst[u * kPanelRows] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        dst[(P - 1) * kPanelRows] = make_uint4(bits[0], bits[1], bits[2], bits[3]);
        if (c == 0) {
            constexpr int CBW = NE == 8 ? 2 : 1;          // codebook dwords per row
            uint32_t v[2] = {0u, 0u};
            if (row < n)
                for (int e = 0; e < NE; ++e)
                    v[e / 4] |= static_cast<uint32_t>(static_cast<uint8_t>(cb[row * NE + e]))
                                << (8 * (e % 4));
            for (int w = 0; w < CBW; ++w) cb_out[row * CBW + w] = v[w];
        }
    }
}

// Four int8 weights of k = b + 4s .. b + 4s + 3 from a CQ2 word (the layout above).
__device__ __forceinline__ int cq2_dword(uint32_t w, int s, uint32_t cb) {
    return static_cast<int>(__builtin_amdgcn_perm(cb, cb, (w >> (2 * s)) & 0x03030303u));
}

// The four one-bit selectors at bits 8j + sh of a CQ1 bit word as bytes 0 or 1.
__device__ __forceinline__ uint32_t cq1_bits(uint32_t bw, int sh) {
    return (bw >> sh) & 0x01010101u;
}

// The bit-plane formats: four int8 weights whose one-bit selectors sit at bits 8j + sh of the
// bit word bw (CQ1), or whose low two bits sit at 8j + 2s of the crumb word w and high bit at
// 8j + sh of bw (CQ3; cb0 holds entries 0-3, cb1 entries 4-7).
__device__ __forceinline__ int cq1_dword(uint32_t bw, int sh, uint32_t cb) {
    return static_cast<int>(__builtin_amdgcn_perm(cb, cb, cq1_bits(bw, sh)));
}
__device__ __forceinline__ int cq3_dword(uint32_t w, int s, uint32_t bw, int sh, uint32_t cb0,
                                         uint32_t cb1) {
    const uint32_t sel = ((w >> (2 * s)) & 0x03030303u) | (((bw >> sh) & 0x01010101u) << 2);
    return static_cast<int>(__builtin_amdgcn_perm(cb1, cb0, sel));
}

// ---- GEMV

// wpp: wavefronts per panel (1, 2, 4 or 8); a workgroup takes 8 / wpp consecutive panels, so a
// short row still gives each wavefront several groups (or chunks) and each workgroup more bytes.
// FUSED: the prepass runs in the kernel (x in io) and xq4 / xs are not read.  PARTIALS: each
// group's int32 dot product is stored to d[row][g] in place of the fp32 epilogue.
template <int FMT, int G, bool FUSED, bool ROT, bool PARTIALS = false>
__global__ __launch_bounds__(64 * kW8Waves) void gemv_w8_kernel(const uint8_t *__restrict__ packed,
                                                                const Geom geom,
                                                                const int *__restrict__ xq4,
                                                                const float *__restrict__ xs,
                                                                float *__restrict__ y, int wpp,
                                                                const FusedIO io,
                                                                int *__restrict__ d = nullptr) {
    static_assert(!(PARTIALS && FUSED), "the partials come from the plain GEMV");
    constexpr int CK = (FMT == kFmtCQ2) ? 64 : kW8Chunk;   // k per chunk
    constexpr int CPG = G / CK;                       // chunks per group
    constexpr int RING = (FMT == kFmtCQ2) ? 4 : 256 / G;   // groups in flight per wavefront
    __shared__ float red[kW8Waves][64];
    __shared__ __attribute__((aligned(16))) int lxq[FUSED ? kFusedMaxK / 4 : 1];
    __shared__ float lxs[FUSED ? kFusedMaxK / 64 : 1];
    FusedPrep<G, ROT> fp;
    if constexpr (FUSED) fp.issue(io, geom.k);
    __builtin_amdgcn_sched_barrier(0);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wsub = wave & (wpp - 1);
    const int p = blockIdx.x * (kW8Waves / wpp) + wave / wpp;
    const bool live = p < geom.n_pad / kPanelRows;    // (the last workgroup may be partial)
    const int kc = geom.k / CK;
    const int ng = live ? geom.k / G : 0;
    const int nblk = (geom.k / G + 3) / 4;
    const int row = p * kPanelRows + lane;
    const rsrc_t rc = make_rsrc(packed + geom.off_codes + (uint64_t)(live ? p : 0) * kc * 1024,
                                live ? (uint64_t)kc * 1024 : 0);
    const rsrc_t rm = make_rsrc(packed + geom.off_meta + (uint64_t)(live ? p : 0) * nblk * 512,
                                live ? (uint64_t)nblk * 512 : 0);
    uint32_t cb = 0u;
    if (FMT == kFmtCQ2 && live)
        cb = reinterpret_cast<const uint32_t *>(packed + geom.off_codebook)[p * kPanelRows + lane];
    v4i ring[RING][CPG];
    uint32_t meta[RING];
    auto load = [&](int s, int g) {
#pragma unroll
        for (int c = 0; c < CPG; ++c)
            ring[s][c] = ld128_stream(rc, g < ng ? ((g * CPG + c) * 64 + lane) * 16 : kOOB);
        meta[s] = ld16(rm, g < ng ? (((g >> 2) * 64 + lane) * 4 + (g & 3)) * 2 : kOOB);
    };
#pragma unroll
    for (int s = 0; s < RING; ++s) load(s, wsub + s * wpp);
    const int *xsrc;                                  // the row's codes and scales: LDS when fused
    const float *xssrc;
    if constexpr (FUSED) {
        fp.run(io, geom.k, lxq, lxs);
        xsrc = lxq;
        xssrc = lxs;
    } else {
        xsrc = xq4;
        xssrc = xs;
    }
    float acc = 0.0f;
    for (int g0 = wsub; g0 < ng; g0 += RING * wpp) {
#pragma unroll
        for (int s = 0; s < RING; ++s) {
            const int g = g0 + s * wpp;
            if (g < ng) {
                const int *xg = xsrc + g * (G / 4);      // the group's codes: wave-uniform
                int d4[4] = {0, 0, 0, 0};
                if (FMT == kFmtCQ2) {
                    constexpr int kq[4] = {0, 32, 16, 48};  // k offset of word position q
#pragma unroll
                    for (int c = 0; c < CPG; ++c)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                d4[e] = __builtin_amdgcn_sdot4(
                                    cq2_dword(static_cast<uint32_t>(ring[s][c][q]), e, cb),
                                    xg[(64 * c + kq[q]) / 4 + e], d4[e], false);
                } else {
#pragma unroll
                    for (int c = 0; c < CPG; ++c)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            d4[e] = __builtin_amdgcn_sdot4(ring[s][c][e], xg[4 * c + e], d4[e], false);
                }
                const int dot = (d4[0] + d4[1]) + (d4[2] + d4[3]);
                if (PARTIALS) {
                    if (row < geom.n) d[(int64_t)row * ng + g] = dot;
                } else {
                    const float coef = xssrc[g] * half_bits_to_float(meta[s] & 0xFFFFu);
                    acc = fmaf(coef, static_cast<float>(dot), acc);
                }
            }
            load(s, g + RING * wpp);
        }
    }
    if (PARTIALS) return;                             // (every wavefront: no barrier follows)
    red[wave][lane] = acc;
    __syncthreads();
    if (wsub != 0 || !live) return;
    float s = red[wave][lane];
    for (int w = 1; w < wpp; ++w) s += red[wave + w][lane];
    if (row < geom.n) y[row] = s;
}

// One row against the bit-plane formats: a workgroup per panel, 8 wavefronts over the 128-k
// chunks, lane r on panel row r; a chunk is P 16-byte loads per lane and holds 128 / G groups.
// PARTIALS as for gemv_w8_kernel.
// CQ1 uses that a two-entry codebook is affine in its selector bit: with entries e0, e1 the
// weight is e0 + b (e1 - e0), so a group's dot product is e0 * xsum + (e1 - e0) * (the sum of the
// codes whose bit is set), the same integer.  The masked sums take one dot4 against the bits as
// 0/1 bytes, without the byte permute that looks the entries up.
template <int FMT, int G, bool FUSED, bool ROT, bool PARTIALS = false>
__global__ __launch_bounds__(64 * kW8Waves) void gemv_bits_kernel(const uint8_t *__restrict__ packed,
                                                                  const Geom geom,
                                                                  const int *__restrict__ xq4,
                                                                  const float *__restrict__ xs,
                                                                  const int *__restrict__ xsum,
                                                                  float *__restrict__ y, int wpp,
                                                                  const FusedIO io,
                                                                  int *__restrict__ d = nullptr) {
    static_assert(!(PARTIALS && FUSED), "the partials come from the plain GEMV");
    constexpr int P = planes<FMT>;
    constexpr int GPC = kBitChunk / G;                // groups per chunk (2 or 1)
    constexpr int RING = FMT == kFmtCQ3 ? 2 : 4;      // chunks in flight per wavefront
    constexpr bool kAffineBit = FMT == kFmtCQ1;
    __shared__ float red[kW8Waves][64];
    __shared__ __attribute__((aligned(16))) int lxq[FUSED ? kFusedMaxK / 4 : 1];
    __shared__ float lxs[FUSED ? kFusedMaxK / 64 : 1];
    __shared__ int lxsum[(FUSED && kAffineBit) ? kFusedMaxK / 64 : 1];
    FusedPrep<G, ROT> fp;
    if constexpr (FUSED) fp.issue(io, geom.k);
    __builtin_amdgcn_sched_barrier(0);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wsub = wave & (wpp - 1);
    const int p = blockIdx.x * (kW8Waves / wpp) + wave / wpp;
    const bool live = p < geom.n_pad / kPanelRows;    // (the last workgroup may be partial)
    const int kc = live ? (geom.k + kBitChunk - 1) / kBitChunk : 0;
    const int ng = geom.k / G;
    const int nblk = (ng + 3) / 4;
    const rsrc_t rc = make_rsrc(packed + geom.off_codes + (uint64_t)(live ? p : 0) * kc * P * 1024,
                                (uint64_t)kc * P * 1024);
    const rsrc_t rm = make_rsrc(packed + geom.off_meta + (uint64_t)(live ? p : 0) * nblk * 512,
                                live ? (uint64_t)nblk * 512 : 0);
    const int row = p * kPanelRows + lane;
    uint32_t cb0 = 0u, cb1 = 0u;
    if (FMT == kFmtCQ3 && live) {
        const uint2 v = reinterpret_cast<const uint2 *>(packed + geom.off_codebook)[row];
        cb0 = v.x;
        cb1 = v.y;
    } else if (live) {
        cb0 = reinterpret_cast<const uint32_t *>(packed + geom.off_codebook)[row];
    }
    // CQ1: entry 0 and the step to entry 1
    const int e0 = static_cast<int8_t>(cb0 & 0xFFu);
    const int step = static_cast<int>(static_cast<int8_t>((cb0 >> 8) & 0xFFu)) - e0;
    v4i ring[RING][P];
    uint32_t meta[RING];
    auto load = [&](int s, int c) {
#pragma unroll
        for (int u = 0; u < P; ++u)
            ring[s][u] = ld128_stream(rc, c < kc ? ((c * P + u) * 64 + lane) * 16 : kOOB);
        // the chunk's groups share one block of 4 (GPC * c is even when GPC = 2)
        const int g = c * GPC;
        if (GPC == 2) meta[s] = ld32(rm, c < kc ? (((g >> 2) * 64 + lane) * 4 + (g & 3)) * 2 : kOOB);
        else meta[s] = ld16(rm, c < kc ? (((g >> 2) * 64 + lane) * 4 + (g & 3)) * 2 : kOOB);
    };
#pragma unroll
    for (int s = 0; s < RING; ++s) load(s, wsub + s * wpp);
    const int *xsrc;                                  // the row's codes, scales and (CQ1) group
    const float *xssrc;                               // sums: LDS when fused
    const int *xsumsrc;
    if constexpr (FUSED) {
        fp.run(io, geom.k, lxq, lxs, kAffineBit ? lxsum : nullptr);
        xsrc = lxq;
        xssrc = lxs;
        xsumsrc = lxsum;
    } else {
        xsrc = xq4;
        xssrc = xs;
        xsumsrc = xsum;
    }
    float acc = 0.0f;
    for (int c0 = wsub; c0 < kc; c0 += RING * wpp) {
#pragma unroll
        for (int s = 0; s < RING; ++s) {
            const int c = c0 + s * wpp;
            if (c < kc) {
                int dot = 0;
#pragma unroll
                for (int gi = 0; gi < 2; ++gi) {             // the chunk's two 64-k halves
                    const int g = (c * kBitChunk + 64 * gi) / G;
                    if (g >= ng) break;                      // (a ragged last chunk)
                    const int *xg = xsrc + c * (kBitChunk / 4) + 16 * gi;  // wave-uniform
                    int d4[4] = {0, 0, 0, 0};
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int pb = 0; pb < 2; ++pb)
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                // k = 128c + 64gi + 32pb + 16h + 4e .. + 3
                                const uint32_t bw = static_cast<uint32_t>(ring[s][P - 1][2 * h + gi]);
                                int wv;
                                if (FMT == kFmtCQ3)
                                    wv = cq3_dword(static_cast<uint32_t>(ring[s][gi][pb + 2 * h]), e,
                                                   bw, 4 * pb + e, cb0, cb1);
                                else   // the bits themselves: d4 sums the selected codes
                                    wv = static_cast<int>(cq1_bits(bw, 4 * pb + e));
                                d4[e] = __builtin_amdgcn_sdot4(wv, xg[8 * pb + 4 * h + e], d4[e],
                                                               false);
                            }
                    int dgi = (d4[0] + d4[1]) + (d4[2] + d4[3]);
                    // CQ1 with 64-groups: the group's dot product from its masked sum (with
                    // 128-groups the chunk's two halves are added first, below)
                    if (kAffineBit && GPC == 2) dgi = e0 * xsumsrc[g] + step * dgi;
                    if (GPC == 2 && PARTIALS) {
                        if (row < geom.n) d[(int64_t)row * ng + g] = dgi;
                    } else if (GPC == 2) {
                        const float coef = xssrc[g] * half_bits_to_float((meta[s] >> (16 * gi)) & 0xFFFFu);
                        acc = fmaf(coef, static_cast<float>(dgi), acc);
                    } else {
                        dot += dgi;
                    }
                }
                if (kAffineBit && GPC == 1) dot = e0 * xsumsrc[c] + step * dot;
                if (GPC == 1 && PARTIALS) {
                    if (row < geom.n) d[(int64_t)row * ng + c] = dot;
                } else if (GPC == 1) {
                    const float coef = xssrc[c] * half_bits_to_float(meta[s] & 0xFFFFu);
                    acc = fmaf(coef, static_cast<float>(dot), acc);
                }
            }
            load(s, c + RING * wpp);
        }
    }
    if (PARTIALS) return;                             // (every wavefront: no barrier follows)
    red[wave][lane] = acc;
    __syncthreads();
    if (wsub != 0 || !live) return;
    float t = red[wave][lane];
    for (int w = 1; w < wpp; ++w) t += red[wave + w][lane];
    if (row < geom.n) y[row] = t;
}

// ---- GEMM

constexpr int kW8BN = 128;          // channels per workgroup (4 wavefronts x 32)
constexpr int kW8SK = 128;          // k per LDS stage: four 32-wide MFMA blocks

template <int FMT, int G>
struct W8Stage {
    static constexpr int GPS = kW8SK / G;             // groups per stage (2 or 1)
    v4i a[2];                                         // two 16-byte activation units per thread
    v2i w2[2];                                        // CQ2 / CQ3: the lane's 8 bytes of each
                                                      // chunk / crumb plane
    v2i bp;                                           // CQ1 / CQ3: the lane's 8 bytes of bits
    uint32_t meta[GPS];
    float xs[GPS];                                    // per group: the scale of the lane's row
};                                                    // (row r32 of tile `half`)

// Three workgroups per CU (12 wavefronts) where the registers allow it: the int8 variant keeps
// its 16-byte weight operands one stage ahead instead of two for that.  PARTIALS: each group's
// int32 tile is stored to d[row][col][g] in place of the fp32 epilogue (xs and y are not used).
// Split tiles (not PARTIALS): workgroups from nfull on each take one 32-channel group of a tile
// of the last, partial round over the CUs; wavefront w runs k quarter w of it, one 32-wide block
// per stage (a stage's LDS buffer holds the four quarters' blocks side by side, so wavefront w
// reads the operand offsets of block w of a whole stage), and the four outputs are added in LDS
// in quarter order.  k is a multiple of 128 and of 4 G.
// The kernels with a split path: the codebook formats with 64-groups.  (In the int8 and the
// 128-group kernels the extra path made the register allocation spill in the whole-tile loop.)
template <int FMT, int G, bool PARTIALS>
constexpr bool kW8Split = !PARTIALS && FMT != kFmtInt8 && G == 64;

template <int FMT, int G>
struct W8Split {
    v4i a[2];                                         // two 16-byte activation units per thread
    v4i w;                                            // int8: the lane's 16-byte chunk
    v2i w2[2];                                        // CQ2: chunk / CQ3: crumb planes (8 bytes)
    v2i bp;                                           // CQ1 / CQ3: the lane's 8 bytes of bits
    uint32_t meta;                                    // the block's group: weight metadata
    float xs;                                         // and the scale of the lane's row
};


// A split workgroup (see gemm_w8_kernel): 32 channels of one tile, wavefront w over k quarter w.
template <int FMT, int G>
__device__ __forceinline__ void split_tile(const uint8_t *__restrict__ packed, const Geom &geom,
                                           int m, const int8_t *__restrict__ xq,
                                           const float *__restrict__ xs, float *__restrict__ y,
                                           int nfull, v4i (*lds)[64 * 8]) {
    constexpr int BPG = G / 32;                       // 32-wide blocks per group
    constexpr int P = planes<FMT>;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int r32 = lane & 31;
    const int mtiles = (m + 63) / 64;
    const int part_id = static_cast<int>(blockIdx.x) - nfull;
    const int tile = nfull + part_id / 4;
    const int mt = tile % mtiles, nt = tile / mtiles;
    const int m0 = mt * 64;
    const int c0 = nt * kW8BN + (part_id % 4) * 32;   // the workgroup's 32 channels
    if (c0 >= geom.n_pad) return;                     // (workgroup-uniform)
    const int col = c0 + r32;
    const int p = col / kPanelRows, prow = col % kPanelRows;
    const int k = geom.k;
    const int kc = bit_plane<FMT> ? (k + kBitChunk - 1) / kBitChunk
                                  : k / ((FMT == kFmtCQ2) ? 64 : kW8Chunk);
    const int ng = k / G;
    const int nblk = (ng + 3) / 4;
    const int qk = k / 4;                             // k per quarter
    const int nst = qk / 32;                          // stages: one 32-wide block per wavefront
    const int gb0 = wave * nst;                       // the wavefront's first block in all of k
    uint32_t cb = 0u, cb1 = 0u;
    if (FMT == kFmtCQ2 || FMT == kFmtCQ1)
        cb = reinterpret_cast<const uint32_t *>(packed + geom.off_codebook)[col];
    if (FMT == kFmtCQ3) {
        const uint2 v = reinterpret_cast<const uint2 *>(packed + geom.off_codebook)[col];
        cb = v.x;
        cb1 = v.y;
    }
    const rsrc_t rc = make_rsrc(packed + geom.off_codes + (uint64_t)p * kc * P * 1024,
                                (uint64_t)kc * P * 1024);
    const rsrc_t rm = make_rsrc(packed + geom.off_meta + (uint64_t)p * nblk * 512,
                                (uint64_t)nblk * 512);
    const rsrc_t rx = make_rsrc(xq, (uint64_t)m * k);
    const rsrc_t rs = make_rsrc(xs, (uint64_t)ng * m * 4);

    // Stage s: activation unit u of a row holds quarter u / 2, k 32 s + 16 (u % 2) of it; the
    // wavefront's weights, metadata and row scale are those of its block gb0 + s.
    auto load_stage = [&](int s, W8Split<FMT, G> &r) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int rr = i * 32 + (tid >> 3), u = tid & 7;
            const int kk = (u >> 1) * qk + 32 * s + 16 * (u & 1);
            const bool ok = (m0 + rr < m) && s < nst;
            r.a[i] = ld128(rx, ok ? (m0 + rr) * k + kk : kOOB);
        }
        const int gb = gb0 + s;
        const bool okb = s < nst;
        if (FMT == kFmtInt8) {
            r.w = ld128(rc, okb ? ((2 * gb + half) * 64 + prow) * 16 : kOOB);
        } else if (FMT == kFmtCQ2) {
            r.w2[0] = ld64(rc, okb ? ((gb >> 1) * 64 + prow) * 16 + 8 * half : kOOB);
        } else {
            const int c = gb >> 2;
            if (FMT == kFmtCQ3)
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    r.w2[u] = ld64(rc, okb ? ((c * P + u) * 64 + prow) * 16 + 8 * half : kOOB);
            r.bp = ld64(rc, okb ? ((c * P + P - 1) * 64 + prow) * 16 + 8 * half : kOOB);
        }
        const int g = (gb * 32) / G;
        r.meta = ld16(rm, okb ? (((g >> 2) * 64 + prow) * 4 + (g & 3)) * 2 : kOOB);
        const int row = m0 + 32 * half + r32;
        r.xs = __builtin_bit_cast(float, ld32(rs, (okb && row < m) ? (g * m + row) * 4 : kOOB));
    };
    auto store_a = [&](int buf, const W8Split<FMT, G> &r) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int rr = i * 32 + (tid >> 3), u = tid & 7;
            lds[buf][rr * 8 + (u ^ (rr & 7))] = r.a[i];
        }
    };

    v16f acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
    v32f zero32;
#pragma unroll
    for (int e = 0; e < 32; ++e) zero32[e] = 0.0f;
    const v16i izero = {};
    v16i part[2] = {};
    W8Split<FMT, G> ring[2];
    load_stage(0, ring[0]);
    if (nst > 1) load_stage(1, ring[1]);
    store_a(0, ring[0]);
    __syncthreads();

    auto stage = [&](auto slot_c, int s) {
        constexpr int slot = decltype(slot_c)::value;
        const int gb = gb0 + s;
        // nst is a multiple of BPG (k a multiple of 4 G), so the block's place in its group is
        // that of s, and s is even in slot 0 and odd in slot 1
        const bool first = (BPG == 2) ? slot == 0 : s % BPG == 0;
        const bool last = (BPG == 2) ? slot == 1 : s % BPG == BPG - 1;
        v4i b;
        if (FMT == kFmtCQ2) {
            const uint32_t w = static_cast<uint32_t>(ring[slot].w2[0][slot]);   // word gb % 2
            b = v4i{cq2_dword(w, 0, cb), cq2_dword(w, 1, cb), cq2_dword(w, 2, cb),
                    cq2_dword(w, 3, cb)};
        } else if (bit_plane<FMT>) {
            // block j = 2q + pb of its chunk (selects, not a runtime index into the registers)
            const int j = gb & 3;
            const v2i bpv = ring[slot].bp;
            const uint32_t bw = static_cast<uint32_t>((j >> 1) ? bpv[1] : bpv[0]);
            uint32_t cw = 0u;
            if (FMT == kFmtCQ3) {
                const v2i c0v = ring[slot].w2[0], c1v = ring[slot].w2[1];
                const v2i cv = (j >> 1) ? c1v : c0v;
                cw = static_cast<uint32_t>((j & 1) ? cv[1] : cv[0]);
            }
            const int sh = 4 * (j & 1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (FMT == kFmtCQ3)
                    b[e] = cq3_dword(cw, e, bw, sh + e, cb, cb1);
                else
                    b[e] = cq1_dword(bw, sh + e, cb);
            }
        } else {
            b = ring[slot].w;
        }
        const uint32_t meta = ring[slot].meta;
        const float xsv = ring[slot].xs;
        if (s + 2 < nst) load_stage(s + 2, ring[slot]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int rr = 32 * t + r32;
            const v4i aop = lds[slot][rr * 8 + ((2 * wave + half) ^ (rr & 7))];
            part[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, b, first ? izero : part[t],
                                                            0, 0, 0);
        }
        if (last) {                                   // the group's last block: rescale
            const float sw = half_bits_to_float(meta & 0xFFFFu);
            const v32f coef = __builtin_amdgcn_mfma_f32_32x32x1f32(xsv, sw, zero32, 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    acc[t][e] = fmaf(coef[16 * t + e], static_cast<float>(part[t][e]), acc[t][e]);
        }
        if (s + 1 < nst) store_a(slot ^ 1, ring[slot ^ 1]);
        __syncthreads();
    };
    for (int s = 0; s < nst; s += 2) {
        stage(std::integral_constant<int, 0>{}, s);
        if (s + 1 < nst) stage(std::integral_constant<int, 1>{}, s + 1);
    }

    // the quarters' outputs meet in LDS, one tile at a time: wavefronts 1-3 store theirs and
    // wavefront 0 adds them to its own in quarter order
    float *xch = reinterpret_cast<float *>(&lds[0][0]);   // [3][16][64] fp32, 12 KiB
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (wave > 0) {
#pragma unroll
            for (int e = 0; e < 16; ++e) xch[((wave - 1) * 16 + e) * 64 + lane] = acc[t][e];
        }
        __syncthreads();
        if (wave == 0 && col < geom.n) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
                float v = acc[t][e];
#pragma unroll
                for (int w = 0; w < 3; ++w) v += xch[(w * 16 + e) * 64 + lane];
                if (row < m) y[(int64_t)row * geom.n + col] = v;
            }
        }
        __syncthreads();
    }
}

// SPLIT: the variant with the split path, launched only when there are split tiles (its mere
// presence slowed the whole-tile loop of some formats, 3-bit codebook 5% on the 64-row head).
template <int FMT, int G, bool PARTIALS = false, bool SPLIT = false>
__global__ __launch_bounds__(256, 3) void gemm_w8_kernel(const uint8_t *__restrict__ packed,
                                                         const Geom geom, int m,
                                                         const int8_t *__restrict__ xq,
                                                         const float *__restrict__ xs,
                                                         float *__restrict__ y,
                                                         int *__restrict__ d, int nfull) {
    constexpr int GPS = kW8SK / G;
    constexpr int BPG = G / 32;                       // MFMA blocks per group
    __shared__ __attribute__((aligned(16))) v4i lds[2][64 * 8];   // [buf][row][16-byte unit]
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = lane >> 5;
    const int r32 = lane & 31;

    const int mtiles = (m + 63) / 64;
    if constexpr (SPLIT && kW8Split<FMT, G, PARTIALS>) {
        if (static_cast<int>(blockIdx.x) >= nfull) {    // (workgroup-uniform)
            split_tile<FMT, G>(packed, geom, m, xq, xs, y, nfull, lds);
            return;
        }
    }
    int bid = blockIdx.x;
    if (nfull % 8 == 0) bid = (bid % 8) * (nfull / 8) + bid / 8;   // consecutive tiles on one XCD
    const int mt = bid % mtiles, nt = bid / mtiles;
    const int m0 = mt * 64;
    const int c0 = nt * kW8BN + wave * 32;
    const bool wact = c0 < geom.n_pad;
    const int col = c0 + r32;
    const int p = col / kPanelRows, prow = col % kPanelRows;
    const int k = geom.k;
    constexpr int P = planes<FMT>;
    const int kc = bit_plane<FMT> ? (k + kBitChunk - 1) / kBitChunk
                                  : k / ((FMT == kFmtCQ2) ? 64 : kW8Chunk);
    const int ng = k / G;
    const int nblk = (ng + 3) / 4;
    const int nstage = (k + kW8SK - 1) / kW8SK;
    uint32_t cb = 0u, cb1 = 0u;
    if ((FMT == kFmtCQ2 || FMT == kFmtCQ1) && wact)
        cb = reinterpret_cast<const uint32_t *>(packed + geom.off_codebook)[col];
    if (FMT == kFmtCQ3 && wact) {
        const uint2 v = reinterpret_cast<const uint2 *>(packed + geom.off_codebook)[col];
        cb = v.x;
        cb1 = v.y;
    }

    const rsrc_t rc = make_rsrc(packed + geom.off_codes + (uint64_t)(wact ? p : 0) * kc * P * 1024,
                                wact ? (uint64_t)kc * P * 1024 : 0);
    const rsrc_t rm = make_rsrc(packed + geom.off_meta + (uint64_t)(wact ? p : 0) * nblk * 512,
                                wact ? (uint64_t)nblk * 512 : 0);
    const rsrc_t rx = make_rsrc(xq, (uint64_t)m * k);
    const rsrc_t rs = make_rsrc(xs, PARTIALS ? 0 : (uint64_t)ng * m * 4);   // (no xs: zeros)

    auto load_stage = [&](int s, W8Stage<FMT, G> &r) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int rr = i * 32 + (tid >> 3), u = tid & 7;
            const int kk = s * kW8SK + 16 * u;
            const bool ok = (m0 + rr < m) && (kk < k);
            r.a[i] = ld128(rx, ok ? (m0 + rr) * k + kk : kOOB);
        }
        if (bit_plane<FMT>) {                         // one chunk per stage
            const bool okc = s < kc;
            if (FMT == kFmtCQ3)
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    r.w2[u] = ld64(rc, okc ? ((s * P + u) * 64 + prow) * 16 + 8 * half : kOOB);
            r.bp = ld64(rc, okc ? ((s * P + P - 1) * 64 + prow) * 16 + 8 * half : kOOB);
        } else if (FMT == kFmtCQ2) {
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const int c = 2 * s + c2;
                r.w2[c2] = ld64(rc, c < kc ? (c * 64 + prow) * 16 + 8 * half : kOOB);
            }
        }
#pragma unroll
        for (int q = 0; q < GPS; ++q) {
            const int g = s * GPS + q;
            r.meta[q] = ld16(rm, g < ng ? (((g >> 2) * 64 + prow) * 4 + (g & 3)) * 2 : kOOB);
            const int row = m0 + 32 * half + r32;
            const bool ok = g < ng && row < m;
            r.xs[q] = __builtin_bit_cast(float, ld32(rs, ok ? (g * m + row) * 4 : kOOB));
        }
    };
    auto store_a = [&](int buf, const W8Stage<FMT, G> &r) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int rr = i * 32 + (tid >> 3), u = tid & 7;
            lds[buf][rr * 8 + (u ^ (rr & 7))] = r.a[i];
        }
    };

    v16f acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
    v32f zero32;
#pragma unroll
    for (int e = 0; e < 32; ++e) zero32[e] = 0.0f;
    const v16i izero = {};
    v16i part[2] = {};

    // int8: the lane's weight chunks of the next stage (loaded one stage ahead)
    v4i wnext[4];
    auto load_w = [&](int s) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = s * (kW8SK / kW8Chunk) + 2 * j + half;
            wnext[j] = ld128(rc, c < kc ? (c * 64 + prow) * 16 : kOOB);
        }
    };
    if (FMT == kFmtInt8) load_w(0);
    W8Stage<FMT, G> ring[2];
    load_stage(0, ring[0]);
    if (nstage > 1) load_stage(1, ring[1]);
    store_a(0, ring[0]);
    __syncthreads();

    auto stage = [&](auto slot_c, int s) {
        constexpr int slot = decltype(slot_c)::value;
        v4i b[4];
        uint32_t meta[GPS];
        float xsv[GPS];
        if (FMT == kFmtCQ2) {
            // block j: word (j % 2) of the lane's 8 bytes of chunk j / 2, decoded to 16 bytes
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = static_cast<uint32_t>(ring[slot].w2[j >> 1][j & 1]);
                b[j] = v4i{cq2_dword(w, 0, cb), cq2_dword(w, 1, cb), cq2_dword(w, 2, cb),
                           cq2_dword(w, 3, cb)};
            }
        } else if (bit_plane<FMT>) {
            // block j = 2q + pb: bit word q of the lane's 8 bytes at shift 4pb; CQ3's crumbs as CQ2
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t bw = static_cast<uint32_t>(ring[slot].bp[j >> 1]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (FMT == kFmtCQ3)
                        b[j][e] = cq3_dword(static_cast<uint32_t>(ring[slot].w2[j >> 1][j & 1]), e,
                                            bw, 4 * (j & 1) + e, cb, cb1);
                    else
                        b[j][e] = cq1_dword(bw, 4 * (j & 1) + e, cb);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = wnext[j];
            if (s + 1 < nstage) load_w(s + 1);
        }
#pragma unroll
        for (int q = 0; q < GPS; ++q) {
            meta[q] = ring[slot].meta[q];
            xsv[q] = ring[slot].xs[q];
        }
        if (s + 2 < nstage) load_stage(s + 2, ring[slot]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int g = s * GPS + j / BPG;
            if (g >= ng) break;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int rr = 32 * t + r32;
                const v4i aop = lds[slot][rr * 8 + ((2 * j + half) ^ (rr & 7))];
                // the group's first block starts from zero (no separate clear)
                part[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, b[j],
                                                                (j % BPG == 0) ? izero : part[t],
                                                                0, 0, 0);
            }
            if (PARTIALS && j % BPG == BPG - 1) {     // the group's last block: store D
                if (wact && col < geom.n) {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
#pragma unroll
                        for (int e = 0; e < 16; ++e) {
                            const int row = m0 + 32 * t + 8 * (e / 4) + 4 * half + (e % 4);
                            if (row < m) d[((int64_t)row * geom.n + col) * ng + g] = part[t][e];
                        }
                }
            } else if (j % BPG == BPG - 1) {          // the group's last block: rescale
                const int q = j / BPG;
                const float sw = half_bits_to_float(meta[q] & 0xFFFFu);
                // both tiles' coefficients in one two-block outer product: block t = tile t
                const v32f coef = __builtin_amdgcn_mfma_f32_32x32x1f32(xsv[q], sw, zero32, 0, 0, 0);
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[t][e] = fmaf(coef[16 * t + e], static_cast<float>(part[t][e]),
                                         acc[t][e]);
            }
        }
        if (s + 1 < nstage) store_a(slot ^ 1, ring[slot ^ 1]);
        __syncthreads();
    };
    for (int s = 0; s < nstage; s += 2) {
        stage(std::integral_constant<int, 0>{}, s);
        if (s + 1 < nstage) stage(std::integral_constant<int, 1>{}, s + 1);
    }

    if (PARTIALS || !wact || col >= geom.n) return;
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

hipError_t launch_pack_codes_w8(const Geom &g, const int8_t *w8, uint8_t *packed,
                                hipStream_t stream) {
    const int64_t chunks = (int64_t)g.n_pad * (g.k / kW8Chunk);
    const int64_t blocks = (chunks + 255) / 256;
    pack_codes_w8_kernel<<<static_cast<unsigned>(blocks < 65536 ? blocks : 65536), 256, 0, stream>>>(
        w8, g.n, g.k, chunks, reinterpret_cast<uint4 *>(packed + g.off_codes));
    return hipGetLastError();
}

namespace {
// One-row GEMV shape: waves per panel, halved while a wavefront would get fewer than kMinUnits
// groups (chunks) and the grid keeps at least kMinGrid workgroups (4 per CU).
int gemv_wpp(const Geom &g, int *grid) {
    const bool bits = g.fmt == kFmtCQ1 || g.fmt == kFmtCQ3;
    const int units = bits ? (g.k + kBitChunk - 1) / kBitChunk : g.k / g.group;
    const int panels = g.n_pad / kPanelRows;
    int wpp = kW8Waves;
    while (wpp > 1 && units < kMinUnits * wpp) {
        const int ppw_next = kW8Waves / (wpp / 2);
        if ((panels + ppw_next - 1) / ppw_next < kMinGrid) break;
        wpp /= 2;
    }
    const int ppw = kW8Waves / wpp;
    *grid = (panels + ppw - 1) / ppw;
    return wpp;
}

template <int FMT, int G, bool FUSED, bool ROT>
void gemv_go(const Geom &g, unsigned grid, int wpp, const uint8_t *packed, const int *x4,
             const float *xs, const int *xsum, float *y, const FusedIO &io, hipStream_t stream) {
    if constexpr (bit_plane<FMT>)
        gemv_bits_kernel<FMT, G, FUSED, ROT><<<grid, 64 * kW8Waves, 0, stream>>>(packed, g, x4, xs,
                                                                                xsum, y, wpp, io);
    else
        gemv_w8_kernel<FMT, G, FUSED, ROT><<<grid, 64 * kW8Waves, 0, stream>>>(packed, g, x4, xs, y,
                                                                              wpp, io);
}

template <int FMT, bool FUSED, bool ROT>
void gemv_fmt(const Geom &g, const uint8_t *packed, const int *x4, const float *xs,
              const int *xsum, float *y, const FusedIO &io, hipStream_t stream) {
    int grid;
    const int wpp = gemv_wpp(g, &grid);
    if (g.group == 64)
        gemv_go<FMT, 64, FUSED, ROT>(g, static_cast<unsigned>(grid), wpp, packed, x4, xs, xsum, y, io,
                                     stream);
    else
        gemv_go<FMT, 128, FUSED, ROT>(g, static_cast<unsigned>(grid), wpp, packed, x4, xs, xsum, y,
                                      io, stream);
}

template <int FMT>
void gemv_fused_fmt(const Geom &g, const uint8_t *packed, int hadamard, const FusedIO &io,
                    float *y, hipStream_t stream) {
    if (hadamard == 128) gemv_fmt<FMT, true, true>(g, packed, nullptr, nullptr, nullptr, y, io, stream);
    else gemv_fmt<FMT, true, false>(g, packed, nullptr, nullptr, nullptr, y, io, stream);
}

// The partials variants: the plain GEMV (m == 1) or the GEMM with their epilogues replaced by a
// store of the int32 per-group dot products.
template <int FMT, int G>
void partials_go(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                 const int32_t *xsum, int32_t *d, hipStream_t stream) {
    if (m == 1) {
        int grid;
        const int wpp = gemv_wpp(g, &grid);
        const int *x4 = reinterpret_cast<const int *>(xq);
        if constexpr (bit_plane<FMT>)
            gemv_bits_kernel<FMT, G, false, false, true><<<grid, 64 * kW8Waves, 0, stream>>>(
                packed, g, x4, nullptr, xsum, nullptr, wpp, FusedIO{}, d);
        else
            gemv_w8_kernel<FMT, G, false, false, true><<<grid, 64 * kW8Waves, 0, stream>>>(
                packed, g, x4, nullptr, nullptr, wpp, FusedIO{}, d);
        return;
    }
    const int tiles = ((m + 63) / 64) * ((g.n_pad + kW8BN - 1) / kW8BN);
    gemm_w8_kernel<FMT, G, true><<<static_cast<unsigned>(tiles), 256, 0, stream>>>(
        packed, g, m, xq, nullptr, nullptr, d, tiles);
}

template <int FMT>
void partials_fmt(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                  const int32_t *xsum, int32_t *d, hipStream_t stream) {
    if (g.group == 64) partials_go<FMT, 64>(g, packed, m, xq, xsum, d, stream);
    else partials_go<FMT, 128>(g, packed, m, xq, xsum, d, stream);
}

template <int FMT>
hipError_t launch_w8_fmt(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                         const float *xs, const int32_t *xsum, float *y, hipStream_t stream) {
    if (m == 1) {
        gemv_fmt<FMT, false, false>(g, packed, reinterpret_cast<const int *>(xq), xs, xsum, y,
                                    FusedIO{}, stream);
        return hipGetLastError();
    }
    // the tiles of a last, partial round over the CUs split in four (k a multiple of 128 and of
    // 4 G: whole 32-wide blocks and whole groups per quarter)
    const int tiles = ((m + 63) / 64) * ((g.n_pad + kW8BN - 1) / kW8BN);
    const bool can_split = (g.group == 64) ? kW8Split<FMT, 64, false> : kW8Split<FMT, 128, false>;
    const int nfull = (can_split && g.k % 128 == 0 && g.k % (4 * g.group) == 0)
                          ? whole_tiles(tiles) : tiles;
    const unsigned grid = static_cast<unsigned>(nfull + 4 * (tiles - nfull));
    if (g.group == 128)
        gemm_w8_kernel<FMT, 128><<<grid, 256, 0, stream>>>(packed, g, m, xq, xs, y, nullptr, nfull);
    else if (nfull < tiles)
        gemm_w8_kernel<FMT, 64, false, kW8Split<FMT, 64, false>><<<grid, 256, 0, stream>>>(
            packed, g, m, xq, xs, y, nullptr, nfull);
    else
        gemm_w8_kernel<FMT, 64><<<grid, 256, 0, stream>>>(packed, g, m, xq, xs, y, nullptr, nfull);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_w8(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                     const float *xs, const int32_t *xsum, float *y, hipStream_t stream) {
    if (m == 0) return hipSuccess;
    if (g.fmt == kFmtCQ2) return launch_w8_fmt<kFmtCQ2>(g, packed, m, xq, xs, xsum, y, stream);
    if (g.fmt == kFmtCQ1) return launch_w8_fmt<kFmtCQ1>(g, packed, m, xq, xs, xsum, y, stream);
    if (g.fmt == kFmtCQ3) return launch_w8_fmt<kFmtCQ3>(g, packed, m, xq, xs, xsum, y, stream);
    return launch_w8_fmt<kFmtInt8>(g, packed, m, xq, xs, xsum, y, stream);
}

hipError_t launch_w8_partials(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                              const int32_t *xsum, int32_t *d, hipStream_t stream) {
    if (m == 0) return hipSuccess;
    if (g.fmt == kFmtCQ2) partials_fmt<kFmtCQ2>(g, packed, m, xq, xsum, d, stream);
    else if (g.fmt == kFmtCQ1) partials_fmt<kFmtCQ1>(g, packed, m, xq, xsum, d, stream);
    else if (g.fmt == kFmtCQ3) partials_fmt<kFmtCQ3>(g, packed, m, xq, xsum, d, stream);
    else partials_fmt<kFmtInt8>(g, packed, m, xq, xsum, d, stream);
    return hipGetLastError();
}

int w8_gemv_workgroups(const Geom &g) {
    int grid;
    gemv_wpp(g, &grid);
    return grid;
}

hipError_t launch_w8_fused(const Geom &g, const uint8_t *packed, const float *x, int hadamard,
                           int8_t *xq, float *xs, int32_t *xsum, float *y, hipStream_t stream) {
    if (g.k > kFusedMaxK) return hipErrorInvalidValue;
    const FusedIO io{x, xq, xs, xsum};
    if (g.fmt == kFmtCQ2) gemv_fused_fmt<kFmtCQ2>(g, packed, hadamard, io, y, stream);
    else if (g.fmt == kFmtCQ1) gemv_fused_fmt<kFmtCQ1>(g, packed, hadamard, io, y, stream);
    else if (g.fmt == kFmtCQ3) gemv_fused_fmt<kFmtCQ3>(g, packed, hadamard, io, y, stream);
    else gemv_fused_fmt<kFmtInt8>(g, packed, hadamard, io, y, stream);
    return hipGetLastError();
}

hipError_t launch_pack_cq2(const Geom &g, const uint8_t *codes, const int8_t *codebook,
                           uint8_t *packed, hipStream_t stream) {
    const int64_t chunks = (int64_t)g.n_pad * (g.k / 64);
    const int64_t blocks = (chunks + 255) / 256;
    pack_codes_cq2_kernel<<<static_cast<unsigned>(blocks < 65536 ? blocks : 65536), 256, 0, stream>>>(
        codes, codebook, g.n, g.k, chunks, reinterpret_cast<uint4 *>(packed + g.off_codes),
        reinterpret_cast<uint32_t *>(packed + g.off_codebook));
    return hipGetLastError();
}

hipError_t launch_pack_bits(const Geom &g, const uint8_t *codes, const int8_t *codebook,
                            uint8_t *packed, hipStream_t stream) {
    const int64_t chunks = (int64_t)g.n_pad * ((g.k + kBitChunk - 1) / kBitChunk);
    const int64_t blocks = (chunks + 255) / 256;
    const unsigned grid = static_cast<unsigned>(blocks < 65536 ? blocks : 65536);
    uint4 *out = reinterpret_cast<uint4 *>(packed + g.off_codes);
    uint32_t *cb_out = reinterpret_cast<uint32_t *>(packed + g.off_codebook);
    if (g.fmt == kFmtCQ3)
        pack_codes_bits_kernel<kFmtCQ3><<<grid, 256, 0, stream>>>(codes, codebook, g.n, g.k,
                                                                  chunks, out, cb_out);
    else
        pack_codes_bits_kernel<kFmtCQ1><<<grid, 256, 0, stream>>>(codes, codebook, g.n, g.k,
                                                                  chunks, out, cb_out);
    return hipGetLastError();
}

}  // namespace w4a8
