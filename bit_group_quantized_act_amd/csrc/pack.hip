// Load-time weight repacker: canonical row-major 4-bit codes, fp16 scales (and fp16 biases or an
// int8 codebook) -> the one panel format that both the GEMV and the GEMM read.
//
// The pages' lesson ("cactus PR #697", follow-up commits on the interleaved lm_head and on the
// single runtime weight format): the layout is the largest single lever, one format should feed
// every kernel, and it should be built once at load.  Here a panel is 64 output rows; its bytes
// are ordered by 32-wide k chunk, then row, 16 bytes per (row, chunk); the per-group metadata is
// ordered by block of 4 groups, then row, so a row's four entries are one 8- or 16-byte load.  A decode wavefront then
// reads one contiguous KiB per chunk (one row per lane), and a 32x32x32 int8 MFMA B fragment for
// 32 rows and a 64-wide k group is two contiguous 512-byte runs.  Inside a chunk the low nibbles
// of the four dwords hold k = 0..15 and the high nibbles k = 16..31, so each half of the chunk
// pairs with one contiguous 16-byte run of activation codes (one MFMA operand, no shuffles).
#include "w4a8_kernels.h"

namespace w4a8 {
namespace {

__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t *__restrict__ codes,
                                                         int n, int k, int fmt, int64_t total,
                                                         uint4 *__restrict__ out) {
    const int kc = k / kChunkK;
    const uint32_t flip = (fmt == kFmtAffine) ? 0x8u : 0x0u;   // u -> u XOR 8 = u - 8 (signed)
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int r = static_cast<int>(t % kPanelRows);
        const int64_t rest = t / kPanelRows;
        const int c = static_cast<int>(rest % kc);
        const int64_t p = rest / kc;
        const int64_t row = p * kPanelRows + r;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        if (row < n) {
            // 16 canonical bytes: byte i holds k = 32c + 2i (low nibble) and 32c + 2i + 1 (high).
            const uint8_t *src = codes + row * (int64_t)(k / 2) + (int64_t)c * 16;
            uint8_t b[16];
            for (int i = 0; i < 16; ++i) b[i] = src[i];
            for (int j = 0; j < 4; ++j) {
                for (int byte = 0; byte < 4; ++byte) {
                    const int k_lo = 4 * j + byte, k_hi = 16 + 4 * j + byte;
                    const uint32_t q_lo = ((b[k_lo / 2] >> (4 * (k_lo & 1))) & 0xFu) ^ flip;
                    const uint32_t q_hi = ((b[k_hi / 2] >> (4 * (k_hi & 1))) & 0xFu) ^ flip;
                    w[j] |= (q_lo | (q_hi << 4)) << (8 * byte);
                }
            }
        }
        out[t] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Metadata in blocks of 4 groups: per panel, per block j, per panel row, the entries of groups
// 4j .. 4j+3 (zero past the last group), so one 8- or 16-byte load gives a row four groups.
// The scale (and bias) of (row, group g) is scales[row * row_stride + g * group_stride]: (ng, 1)
// for one value per group, (1, 0) for one value per row seen as every group's.
__global__ __launch_bounds__(256) void pack_meta_kernel(const uint16_t *__restrict__ scales,
                                                        const uint16_t *__restrict__ bias,
                                                        int n, int ng, int row_stride,
                                                        int group_stride, int64_t total,
                                                        uint8_t *__restrict__ out) {
    const int nblk = (ng + 3) / 4;
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int i = static_cast<int>(t & 3);
        const int r = static_cast<int>((t >> 2) % kPanelRows);
        const int64_t rest = (t >> 2) / kPanelRows;
        const int j = static_cast<int>(rest % nblk);
        const int64_t p = rest / nblk;
        const int64_t row = p * kPanelRows + r;
        const int g = 4 * j + i;
        const bool valid = row < n && g < ng;
        const int64_t src = row * row_stride + static_cast<int64_t>(g) * group_stride;
        const uint32_t s = valid ? scales[src] : 0u;
        if (bias) {
            const uint32_t b = valid ? bias[src] : 0u;
            reinterpret_cast<uint32_t *>(out)[t] = s | (b << 16);
        } else {
            reinterpret_cast<uint16_t *>(out)[t] = static_cast<uint16_t>(s);
        }
    }
}

__global__ __launch_bounds__(256) void pack_codebook_kernel(const int8_t *__restrict__ cb,
                                                            int n, int64_t total,
                                                            int8_t *__restrict__ out) {
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x)
        out[t] = (t / 16 < n) ? cb[t] : static_cast<int8_t>(0);
}

unsigned grid_for(int64_t total) {
    const int64_t blocks = (total + 255) / 256;
    return static_cast<unsigned>(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

hipError_t launch_pack(const Geom &g, const uint8_t *codes, const uint16_t *scales,
                       const uint16_t *bias, const int8_t *codebook, uint8_t *packed,
                       hipStream_t stream, bool row_scale) {
    hipError_t e;
    if (g.fmt == kFmtInt8) {
        e = launch_pack_codes_w8(g, reinterpret_cast<const int8_t *>(codes), packed, stream);
    } else if (g.fmt == kFmtCQ2) {
        e = launch_pack_cq2(g, codes, codebook, packed, stream);     // codes and codebooks
    } else if (g.fmt == kFmtCQ1 || g.fmt == kFmtCQ3) {
        e = launch_pack_bits(g, codes, codebook, packed, stream);    // codes and codebooks
    } else {
        const int64_t chunks = (int64_t)g.n_pad * (g.k / kChunkK);
        pack_codes_kernel<<<grid_for(chunks), 256, 0, stream>>>(
            codes, g.n, g.k, g.fmt, chunks, reinterpret_cast<uint4 *>(packed + g.off_codes));
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    const int ng = g.k / g.group;
    const int64_t metas = (int64_t)g.n_pad * ((ng + 3) / 4) * 4;
    pack_meta_kernel<<<grid_for(metas), 256, 0, stream>>>(
        scales, g.fmt == kFmtAffine ? bias : nullptr, g.n, ng, row_scale ? 1 : ng,
        row_scale ? 0 : 1, metas, packed + g.off_meta);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (g.fmt == kFmtCodebook) {
        const int64_t entries = (int64_t)g.n_pad * 16;
        pack_codebook_kernel<<<grid_for(entries), 256, 0, stream>>>(
            codebook, g.n, entries, reinterpret_cast<int8_t *>(packed + g.off_codebook));
        e = hipGetLastError();
    }
    return e;
}

}  // namespace w4a8
