// The last step of the greedy tail of a vocabulary head: the largest of the GEMV workgroups'
// panel keys, decoded into the token (its row) and the value (its logit).
// Source: "cactus-compute/engine PR #750: Metal Support", the commit list (the lm_head softcap
// fused into the GPU argmax tail) and its file table (GPU-side sampling and argmax helpers).
#include "w4a8_kernels.h"

namespace w4a8 {
namespace {

// One workgroup (nkeys >= 1): every lane keeps the largest of a strided slice of the keys, loading
// kKeyUnroll of them at a time so that their latencies overlap (the keys were just written by
// the GEMV and come from beyond this CU's caches); then wavefronts, then the 16 wavefront
// results in one lane.
constexpr int kKeyThreads = 1024;
constexpr int kKeyUnroll = 4;

__global__ __launch_bounds__(kKeyThreads) void argmax_keys_kernel(
        const unsigned long long *__restrict__ keys, int nkeys, int32_t *__restrict__ token,
        float *__restrict__ value) {
    __shared__ unsigned long long wave_key[kKeyThreads / 64];
    unsigned long long key = 0ull;
    for (int base = 0; base < nkeys; base += kKeyThreads * kKeyUnroll) {
        unsigned long long v[kKeyUnroll];
#pragma unroll
        for (int j = 0; j < kKeyUnroll; ++j) {
            // past the end: the last key again (a repeat cannot change the maximum), so the
            // loads need no branch and all issue before the first wait
            const int i = base + j * kKeyThreads + static_cast<int>(threadIdx.x);
            v[j] = keys[i < nkeys ? i : nkeys - 1];
        }
#pragma unroll
        for (int j = 0; j < kKeyUnroll; ++j) key = v[j] > key ? v[j] : key;
    }
    key = wave_max_key(key);
    if ((threadIdx.x & 63) == 0) wave_key[threadIdx.x >> 6] = key;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kKeyThreads / 64; ++w) key = wave_key[w] > key ? wave_key[w] : key;
        const uint32_t u = static_cast<uint32_t>(key >> 32);
        *token = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key));
        *value = __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
    }
}

}  // namespace

hipError_t launch_argmax_keys(const unsigned long long *keys, int nkeys, int32_t *token,
                              float *value, hipStream_t stream) {
    argmax_keys_kernel<<<1, kKeyThreads, 0, stream>>>(keys, nkeys, token, value);
    return hipGetLastError();
}

}  // namespace w4a8
