// Internal declarations shared by the HIP translation units of libw4a8 (not installed, not
// part of the C ABI).  Device helpers for the packed weight format live here so that the
// repacker and the two matmul kernels agree on it by construction.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace w4a8 {

constexpr int kPanelRows = 64;   // output channels per packed panel
constexpr int kChunkK = 32;      // k values per 16-byte chunk of one row
constexpr int kFmtSym = 0, kFmtAffine = 1, kFmtCodebook = 2;

// What the kernels need from a w4a8_layout (plain values, passed by value to kernels).
struct Geom {
    int fmt, n, k, group, n_pad, meta_bytes;
    uint64_t off_codes, off_meta, off_codebook;
};

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

// ---- 4-bit unpack helpers (packed chunk format: dword j, byte b holds the code of k = 4j+b in
// its low nibble and of k = 16+4j+b in its high nibble).

// Signed codes (SYM q, AFFINE u-8) as int8 bytes scaled by 16: the low nibbles moved to the top
// of each byte, and the high nibbles masked in place.  16*q is exact in int8 for q in [-8, 7].
__device__ __forceinline__ uint32_t lo_x16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t hi_x16(uint32_t w) { return w & 0xF0F0F0F0u; }

// Codebook lookup of four indices (one per byte, each 0..15) in a row's 16 int8 entries held
// as dwords c0 (entries 0-3) .. c3 (entries 12-15).  v_perm selects bytes 0..7 of a dword
// pair, so two lookups cover the halves and the index's bit 3 picks between them per byte.
__device__ __forceinline__ uint32_t cb_lookup(uint32_t idx, uint32_t c0, uint32_t c1,
                                              uint32_t c2, uint32_t c3) {
    const uint32_t sel = idx & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(c1, c0, sel);
    const uint32_t hi = __builtin_amdgcn_perm(c3, c2, sel);
    const uint32_t t = (idx >> 3) & 0x01010101u;
    const uint32_t mask = (t << 8) - t;               // 0xFF in each byte whose bit 3 is set
    return (hi & mask) | (lo & ~mask);
}
__device__ __forceinline__ uint32_t cb_lo(uint32_t w, uint4 cb) {
    return cb_lookup(w & 0x0F0F0F0Fu, cb.x, cb.y, cb.z, cb.w);
}
__device__ __forceinline__ uint32_t cb_hi(uint32_t w, uint4 cb) {
    return cb_lookup((w >> 4) & 0x0F0F0F0Fu, cb.x, cb.y, cb.z, cb.w);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// ---- launchers (each returns the hipGetLastError() of its launch)

hipError_t launch_pack(const Geom &g, const uint8_t *codes, const uint16_t *scales,
                       const uint16_t *bias, const int8_t *codebook, uint8_t *packed,
                       hipStream_t stream);

hipError_t launch_prep(const float *x, int64_t m, int k, int group, int hadamard,
                       int8_t *xq, float *xs, int32_t *xsum, hipStream_t stream);

// y != nullptr: fp32 output; d != nullptr: int32 partials instead.
hipError_t launch_gemv(const Geom &g, const uint8_t *packed, const int8_t *xq, const float *xs,
                       const int32_t *xsum, float *y, int32_t *d, hipStream_t stream);

hipError_t launch_gemm(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                       const float *xs, const int32_t *xsum, float *y, int32_t *d,
                       hipStream_t stream);

}  // namespace w4a8
