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
// Bit-exactness: every value goes through the same fp32 operations as the definition.  The
// rotation's butterflies are the network with span 1, 2, ..., 64 (spans 1 and 2 inside a lane,
// 4..64 across lanes 1..16 apart), each output being a single add or subtract of the same two
// operands; then one multiply by fp32(1/sqrt(128)).  The scale is an IEEE-rounded divide by 127
// and each code an IEEE-rounded divide then round-half-even (v_rndne).  Contraction is off.
#include "w4a8_kernels.h"

namespace w4a8 {
namespace {

// 1/sqrt(128) = sqrt(2)/16 rounded to the nearest fp32: sqrt(2) rounds to 0x3FB504F3, and the
// division by 16 only moves the exponent, giving 0x3DB504F3.
constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;

template <int G, bool ROT>
__global__ __launch_bounds__(256) void prep_kernel(const float4 *__restrict__ x, int64_t quads,
                                                   int64_t m, int ng,
                                                   int *__restrict__ xq4,
                                                   float *__restrict__ xs,
                                                   int *__restrict__ xsum) {
#pragma clang fp contract(off)
    constexpr int kLanesPerGroup = G / 4;
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const int lane = threadIdx.x & 63;
    const bool live = t < quads;   // whole groups are live or dead together (see mapping)
    float4 v = live ? x[t] : make_float4(0.f, 0.f, 0.f, 0.f);
    float e[4] = {v.x, v.y, v.z, v.w};

    if (ROT) {
        float a, b;
        // span 1: (0,1), (2,3)
        a = e[0]; b = e[1]; e[0] = a + b; e[1] = a - b;
        a = e[2]; b = e[3]; e[2] = a + b; e[3] = a - b;
        // span 2: (0,2), (1,3)
        a = e[0]; b = e[2]; e[0] = a + b; e[2] = a - b;
        a = e[1]; b = e[3]; e[1] = a + b; e[3] = a - b;
        // spans 4..64: partner lane differs in bit s of the lane's position in its 128-block
#pragma unroll
        for (int s = 1; s < 32; s <<= 1) {
            const bool upper = (lane & s) != 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float other = __shfl_xor(e[i], s, 64);
                e[i] = upper ? (other - e[i]) : (e[i] + other);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = e[i] * kInvSqrt128;
    }

    float amax = fmaxf(fmaxf(fabsf(e[0]), fabsf(e[1])), fmaxf(fabsf(e[2]), fabsf(e[3])));
#pragma unroll
    for (int s = 1; s < kLanesPerGroup; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));

    const float scale = amax / 127.0f;
    int q[4] = {0, 0, 0, 0};
    if (amax > 0.0f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float r = rintf(e[i] / scale);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            q[i] = static_cast<int>(r);
        }
    }
    int sum = q[0] + q[1] + q[2] + q[3];
#pragma unroll
    for (int s = 1; s < kLanesPerGroup; s <<= 1) sum += __shfl_xor(sum, s, 64);

    if (live) {
        xq4[t] = (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) |
                 ((q[3] & 0xFF) << 24);
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
