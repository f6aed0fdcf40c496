// Activation prepass: optional normalized Walsh-Hadamard rotation of 128-wide blocks, then
// per-row per-group int8 quantization and int32 group sums.
//
// Sources: "cactus PR #697", section "Quantized matmul" (the GEMV's first phase rotates the
// activations with a Hadamard transform and quantizes them to int8 per group; the rotated lm_head
// keeps 128-wide groups aligned with the rotation); "TensorFold PR #3215", section "What this
// changes" (X-only per-group values, the group sums for the affine bias term, are written once
// per call by a prepass instead of being recomputed in every column tile).
//
// Mapping: the [m][k] activations are treated as a flat array of float4 quads.  Thread t owns
// floats 4t..4t+3; since k is a multiple of the group (64 or 128) and of the rotation block, a
// group is G/4 consecutive lanes of one wavefront and never straddles rows, so row * (k/G) +
// group is simply 4t/G.  Loads are 16-byte coalesced (1 KiB per wavefront), code stores 4 bytes
// per lane.  The scales and sums are stored group-major ([k/G][m]) so that a matmul epilogue reads
// one group's values for consecutive rows as one contiguous run.
//
// Bit-exactness: prep_quad (shared with the fused decode GEMV) puts every value through the same
// fp32 operations as the definition.
#include "w4a8_kernels.h"

namespace w4a8 {
namespace {

template <int G, bool ROT>
__global__ __launch_bounds__(256) void prep_kernel(const float4 *__restrict__ x, int64_t quads,
                                                   int64_t m, int ng,
                                                   int *__restrict__ xq4,
                                                   float *__restrict__ xs,
                                                   int *__restrict__ xsum) {
    constexpr int kLanesPerGroup = G / 4;
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int lane = threadIdx.x & 63;
    const bool live = t < quads;   // whole groups are live or dead together (see mapping)
    const float4 v = live ? x[t] : make_float4(0.f, 0.f, 0.f, 0.f);
    float scale;
    int sum;
    const int codes = prep_quad<G, ROT>(v, lane, scale, sum);
    if (live) {
        xq4[t] = codes;
        if ((lane & (kLanesPerGroup - 1)) == 0) {
            const int64_t f = t / kLanesPerGroup;          // row * ng + group
            const int64_t o = (f % ng) * m + f / ng;       // group-major: [group][row]
            xs[o] = scale;
            xsum[o] = sum;
        }
    }
}

}  // namespace

hipError_t launch_prep(const float *x, int64_t m, int k, int group, int hadamard,
                       int8_t *xq, float *xs, int32_t *xsum, hipStream_t stream) {
    const int64_t quads = m * (int64_t)k / 4;
    if (quads == 0) return hipSuccess;
    const unsigned grid = static_cast<unsigned>((quads + 255) / 256);
    const float4 *x4 = reinterpret_cast<const float4 *>(x);
    int *q4 = reinterpret_cast<int *>(xq);
    const int ng = k / group;
    if (group == 64) {
        if (hadamard) prep_kernel<64, true><<<grid, 256, 0, stream>>>(x4, quads, m, ng, q4, xs, xsum);
        else prep_kernel<64, false><<<grid, 256, 0, stream>>>(x4, quads, m, ng, q4, xs, xsum);
    } else {
        if (hadamard) prep_kernel<128, true><<<grid, 256, 0, stream>>>(x4, quads, m, ng, q4, xs, xsum);
        else prep_kernel<128, false><<<grid, 256, 0, stream>>>(x4, quads, m, ng, q4, xs, xsum);
    }
    return hipGetLastError();
}

}  // namespace w4a8
