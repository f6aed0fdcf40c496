// A plain read of device buffers: the achievable HBM read rate that the GEMV's weight stream is
// measured against.  A measurement aid of the benchmark, built into its own library
// (libw4a8_probe.so); it is not part of the layer's C ABI.
//
// Each workgroup of 256 lanes reads one contiguous slice with 16-byte non-temporal loads, several
// in flight per lane, and folds them into a dword so the loads are kept; lane 0 of each workgroup stores the
// fold to sink[workgroup] (the result is meaningless, only the traffic matters).
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void read_kernel(const uint4 *__restrict__ buf, uint64_t n16,
                                                   uint64_t per_wg, uint32_t *__restrict__ sink) {
    const uint64_t lo = blockIdx.x * per_wg;
    const uint64_t hi = lo + per_wg < n16 ? lo + per_wg : n16;
    uint32_t acc = 0u;
    uint64_t i = lo + threadIdx.x;
    for (; i + (U - 1) * 256 < hi; i += U * 256) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(buf) + i + u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < hi; i += 256) {
        const uint4 a = buf[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    __shared__ uint32_t part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) of `buf` (16-byte aligned) with `workgroups` workgroups of
// 256 lanes, `unroll` (4, 8 or 16) loads in flight per lane; sink: uint32 [workgroups].
// Returns the hipError_t of the launch (0 on success).
int stream_probe_read(const void *buf, uint64_t bytes, uint32_t *sink, int32_t workgroups,
                      int32_t unroll, void *stream) {
    if (!buf || !sink || workgroups <= 0 || bytes % 16 != 0 ||
        (reinterpret_cast<uintptr_t>(buf) & 15) != 0 ||
        (unroll != 4 && unroll != 8 && unroll != 16))
        return static_cast<int>(hipErrorInvalidValue);
    const uint64_t n16 = bytes / 16;
    const uint64_t per_wg = (n16 + workgroups - 1) / workgroups;
    const uint4 *b = static_cast<const uint4 *>(buf);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (unroll == 4)
        read_kernel<4><<<workgroups, 256, 0, st>>>(b, n16, per_wg, sink);
    else if (unroll == 8)
        read_kernel<8><<<workgroups, 256, 0, st>>>(b, n16, per_wg, sink);
    else
        read_kernel<16><<<workgroups, 256, 0, st>>>(b, n16, per_wg, sink);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
