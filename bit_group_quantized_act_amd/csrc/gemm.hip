// Prefill GEMM (m activation rows) over the packed 4-bit weights with int8 MFMA.
//
// Sources: "cactus PR #697", section "Quantized matmul" (the M>1 fused GEMM accumulates raw int32
// partials per group in the matrix unit and rescales them per tile in a vector epilogue, with
// several accumulator tiles in flight); "geistlib issue #500", sections "Why" and "Design" (a
// native int8 GEMM removes the dequantize-to-fp32 intermediate of prefill); "TensorFold PR
// #3215" (the affine bias term uses the per-row group sums from the prepass).
//
// MI355X design.  A workgroup owns one 64-row weight panel and 128 activation rows; each of its 4
// wavefronts owns 32 activation rows x 64 output channels, i.e. two 32x32 int32 tiles.  For every
// 64-wide k step the wavefront loads 32 activation bytes per lane straight from global (L2
// resident: the activations are small and shared by every panel) and one 16-byte weight chunk per
// lane per tile; the nibbles become int8 in registers (x16 for signed codes, a v_perm lookup for
// codebooks) and feed two v_mfma_i32_32x32x32_i8 per tile.  Lane l holds activation row l%32 and
// k half l/32; the packed chunk of lane l is panel row 32t + l%32 at chunk 2q + l/32, so each
// tile's B fragment is two contiguous 512-byte runs.  The low nibbles of the four chunk dwords
// pair with activation dwords 0,2,4,6 and the high nibbles with 1,3,5,7 (the same k on both
// sides, which is all the MFMA needs).
//
// Epilogue per group: the coefficient tile xs[row]*sw[col] comes from one fp32 outer-product
// MFMA (v_mfma_f32_32x32x1_2b, one block per tile), which also puts each coefficient in the same
// lane/register as its int32 partial; the VALU then does one convert and one FMA per element.
// The affine bias term sum_g (xs*xsum)[row][g] * (bw + 8 sw)[col][g] is an fp32 matrix product
// over groups and runs on v_mfma_f32_32x32x2 (two groups per instruction).
#include "w4a8_kernels.h"

namespace w4a8 {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kBlockRows = kWaves * kRowsPerWave;   // activation rows per workgroup

template <int FMT>
__device__ __forceinline__ void unpack_b(uint4 v, uint4 cb, v4i &lo, v4i &hi) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (FMT == kFmtCodebook) {
            lo[j] = static_cast<int>(cb_lo(w[j], cb));
            hi[j] = static_cast<int>(cb_hi(w[j], cb));
        } else {
            lo[j] = static_cast<int>(lo_x16(w[j]));
            hi[j] = static_cast<int>(hi_x16(w[j]));
        }
    }
}

__device__ __forceinline__ float meta_scale(const uint8_t *meta, int64_t idx, int mb) {
    if (mb == 4)
        return half_bits_to_float(reinterpret_cast<const uint32_t *>(meta)[idx] & 0xFFFFu);
    return half_bits_to_float(reinterpret_cast<const uint16_t *>(meta)[idx]);
}

template <int FMT, int G, bool PARTIALS>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t *__restrict__ packed,
                                                   const Geom geom, int m,
                                                   const int8_t *__restrict__ xq,
                                                   const float *__restrict__ xs,
                                                   const int *__restrict__ xsum,
                                                   float *__restrict__ y,
                                                   int *__restrict__ d) {
    constexpr int kPairsPerGroup = G / 64;   // 64-wide k steps per group
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int p = blockIdx.x;
    const int m_base = blockIdx.y * kBlockRows + wave * kRowsPerWave;
    if (m_base >= m) return;   // whole wavefront past the last row (no barriers below)
    const int k = geom.k;
    const int kc = k / kChunkK;
    const int ng = k / G;
    const int half = lane >> 5;          // k half of the MFMA operands
    const int r32 = lane & 31;
    const int a_row = m_base + r32;      // activation row this lane loads
    const bool a_ok = a_row < m;

    const uint4 *wpan = reinterpret_cast<const uint4 *>(packed + geom.off_codes) +
                        (int64_t)p * kc * kPanelRows;
    const uint8_t *meta = packed + geom.off_meta + (int64_t)p * ng * kPanelRows * geom.meta_bytes;
    uint4 cb0 = make_uint4(0u, 0u, 0u, 0u), cb1 = cb0;
    if (FMT == kFmtCodebook) {
        const uint4 *cbp = reinterpret_cast<const uint4 *>(packed + geom.off_codebook);
        cb0 = cbp[(int64_t)p * kPanelRows + r32];
        cb1 = cbp[(int64_t)p * kPanelRows + 32 + r32];
    }
    const uint4 *arow = reinterpret_cast<const uint4 *>(xq + (int64_t)(a_ok ? a_row : 0) * k);

    v16f acc0 = {}, acc1 = {};
    v16f bacc0 = {}, bacc1 = {};

    for (int g = 0; g < ng; ++g) {
        v16i d0 = {}, d1 = {};
#pragma unroll
        for (int q = 0; q < kPairsPerGroup; ++q) {
            const int c = g * (G / kChunkK) + 2 * q + half;   // this lane's chunk
            uint4 a0 = make_uint4(0u, 0u, 0u, 0u), a1 = a0;
            if (a_ok) {
                a0 = arow[2 * c];
                a1 = arow[2 * c + 1];
            }
            const uint4 w0 = wpan[(int64_t)c * kPanelRows + r32];
            const uint4 w1 = wpan[(int64_t)c * kPanelRows + 32 + r32];
            const v4i alo = {static_cast<int>(a0.x), static_cast<int>(a0.z),
                             static_cast<int>(a1.x), static_cast<int>(a1.z)};
            const v4i ahi = {static_cast<int>(a0.y), static_cast<int>(a0.w),
                             static_cast<int>(a1.y), static_cast<int>(a1.w)};
            v4i blo0, bhi0, blo1, bhi1;
            unpack_b<FMT>(w0, cb0, blo0, bhi0);
            unpack_b<FMT>(w1, cb1, blo1, bhi1);
            d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo, blo0, d0, 0, 0, 0);
            d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi, bhi0, d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(alo, blo1, d1, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ahi, bhi1, d1, 0, 0, 0);
        }

        if (PARTIALS) {
            // output element i of a tile: row 8*(i/4) + 4*half + i%4, column r32
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m_base + 8 * (i / 4) + 4 * half + (i % 4);
                if (row >= m) continue;
                int s8 = 0;
                if (FMT == kFmtAffine) s8 = 8 * xsum[(int64_t)row * ng + g];
                int v0 = (FMT == kFmtCodebook) ? d0[i] : (d0[i] >> 4);
                int v1 = (FMT == kFmtCodebook) ? d1[i] : (d1[i] >> 4);
                const int64_t col0 = (int64_t)p * kPanelRows + r32;
                if (col0 < geom.n) d[((int64_t)row * geom.n + col0) * ng + g] = v0 + s8;
                if (col0 + 32 < geom.n) d[((int64_t)row * geom.n + col0 + 32) * ng + g] = v1 + s8;
            }
            continue;
        }

        // coefficient tiles: block t of the outer product is xs[rows] x sw16[cols 32t..32t+31];
        // lane l supplies row l%32 for both blocks and panel column l (= 32t + l%32).
        const float xs_a = a_ok ? xs[(int64_t)a_row * ng + g] : 0.0f;
        float sw = meta_scale(meta, (int64_t)g * kPanelRows + lane, geom.meta_bytes);
        if (FMT != kFmtCodebook) sw *= 0.0625f;   // the signed-code partials are 16x
        v32f coef = {};
        coef = __builtin_amdgcn_mfma_f32_32x32x1f32(xs_a, sw, coef, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            acc0[i] = fmaf(static_cast<float>(d0[i]), coef[i], acc0[i]);
            acc1[i] = fmaf(static_cast<float>(d1[i]), coef[16 + i], acc1[i]);
        }

        if (FMT == kFmtAffine && ((g & 1) || g == ng - 1)) {
            // bias term for groups (g & ~1) + half: A = xs*xsum [row][group], B = bw + 8*sw
            // [group][col]; a missing second group contributes zeros.
            const int gg = (g & ~1) + half;
            float a2 = 0.0f, b20 = 0.0f, b21 = 0.0f;
            if (gg <= g) {
                if (a_ok)
                    a2 = xs[(int64_t)a_row * ng + gg] *
                         static_cast<float>(xsum[(int64_t)a_row * ng + gg]);
                const uint32_t *m4 = reinterpret_cast<const uint32_t *>(meta);
                const uint32_t e0 = m4[(int64_t)gg * kPanelRows + r32];
                const uint32_t e1 = m4[(int64_t)gg * kPanelRows + 32 + r32];
                b20 = fmaf(8.0f, half_bits_to_float(e0 & 0xFFFFu), half_bits_to_float(e0 >> 16));
                b21 = fmaf(8.0f, half_bits_to_float(e1 & 0xFFFFu), half_bits_to_float(e1 >> 16));
            }
            bacc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a2, b20, bacc0, 0, 0, 0);
            bacc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a2, b21, bacc1, 0, 0, 0);
        }
    }
    if (PARTIALS) return;

    const int64_t col0 = (int64_t)p * kPanelRows + r32;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = m_base + 8 * (i / 4) + 4 * half + (i % 4);
        if (row >= m) continue;
        float v0 = acc0[i], v1 = acc1[i];
        if (FMT == kFmtAffine) {
            v0 += bacc0[i];
            v1 += bacc1[i];
        }
        if (col0 < geom.n) y[(int64_t)row * geom.n + col0] = v0;
        if (col0 + 32 < geom.n) y[(int64_t)row * geom.n + col0 + 32] = v1;
    }
}

template <int FMT, bool PARTIALS>
hipError_t launch_g(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                    const float *xs, const int32_t *xsum, float *y, int32_t *d,
                    hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(g.n_pad / kPanelRows),
                    static_cast<unsigned>((m + kBlockRows - 1) / kBlockRows));
    if (g.group == 64)
        gemm_kernel<FMT, 64, PARTIALS><<<grid, 256, 0, stream>>>(packed, g, m, xq, xs, xsum, y, d);
    else
        gemm_kernel<FMT, 128, PARTIALS><<<grid, 256, 0, stream>>>(packed, g, m, xq, xs, xsum, y, d);
    return hipGetLastError();
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
