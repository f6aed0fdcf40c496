// Internal declarations shared by the HIP translation units of libw4a8 (not installed, not
// part of the C ABI).  Device helpers for the packed weight format live here so that the
// repacker and the two matmul kernels agree on it by construction.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace w4a8 {

constexpr int kPanelRows = 64;   // output channels per packed panel
constexpr int kChunkK = 32;      // k values per 16-byte chunk of one row
constexpr int kFmtSym = 0, kFmtAffine = 1, kFmtCodebook = 2, kFmtInt8 = 3, kFmtCQ2 = 4,
              kFmtCQ1 = 5, kFmtCQ3 = 6;

// What the kernels need from a w4a8_layout (plain values, passed by value to kernels).
struct Geom {
    int fmt, n, k, group, n_pad, meta_bytes;
    uint64_t off_codes, off_meta, off_codebook;
};

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

// ---- buffer loads
//
// A raw buffer descriptor (base, byte range) makes every load whose VGPR offset lies outside the
// range return zeros without touching memory.  The range check covers the VGPR offset and the
// instruction offset only, not the SGPR offset, so a load that may fall outside its buffer keeps
// its whole offset in the VGPR operand.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kRsrcCfg = 0x00020000u;
constexpr int kOOB = 0x7FFFFFF0;   // a VGPR offset past every range: the load returns zeros

// The descriptor is built from wave-uniform values (read from the first lane), so it lives in
// SGPRs: a descriptor the compiler places in VGPRs makes it loop over the lanes at every use.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(
        bytes > 0x7FFFFFF0ull ? 0x7FFFFFF0u : static_cast<uint32_t>(bytes));
    void *p = reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, 0, n, kRsrcCfg);
}
// Cache-policy operand of the buffer loads: bit 1 is the non-temporal (nt) hint on gfx950.
constexpr int kCachePolicyNT = 2;

__device__ __forceinline__ v4i ld128(rsrc_t r, int voff) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
// The same load with the non-temporal cache policy, for weight streams that one launch reads
// once (the one-row GEMVs): the lines are not kept in L2 for a reuse that never comes.  Measured
// on the 262144-row vocabulary head: 32.4 us against 35.3 us for the plain load.
__device__ __forceinline__ v4i ld128_stream(rsrc_t r, int voff) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kCachePolicyNT));
}
__device__ __forceinline__ v2i ld64(rsrc_t r, int voff) {
    return __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
}
__device__ __forceinline__ uint32_t ld32(rsrc_t r, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
}
__device__ __forceinline__ uint32_t ld16(rsrc_t r, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
}

// ---- 4-bit unpack helpers (packed chunk format: dword j, byte b holds the code of k = 4j+b in
// its low nibble and of k = 16+4j+b in its high nibble).

// Signed codes (SYM q, AFFINE u-8) as int8 bytes scaled by 16: the low nibbles moved to the top
// of each byte, and the high nibbles masked in place.  16*q is exact in int8 for q in [-8, 7].
__device__ __forceinline__ uint32_t lo_x16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t hi_x16(uint32_t w) { return w & 0xF0F0F0F0u; }

// Codebook lookup of four indices in a row's 16 int8 entries, held as dwords c0 (entries 0-3)
// .. c3 (entries 12-15).  v_perm picks bytes 0..7 of a dword pair, so one permute per half looks
// up the index's low three bits in entries 0-7 and in entries 8-15, and a third permute takes
// byte i of the first result or of the second (selector i or i + 4) by the index's bit 3.  All
// three are full-rate byte permutes; building a byte mask from bit 3 instead costs a multiply.
// `w` holds four indices as nibbles at bit offset `S` (0: low nibbles, 4: high nibbles).
template <int S>
__device__ __forceinline__ uint32_t cb_lookup(uint32_t w, uint4 cb) {
    const uint32_t sel = (w >> S) & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(cb.y, cb.x, sel);
    const uint32_t hi = __builtin_amdgcn_perm(cb.w, cb.z, sel);
    const uint32_t pick = ((w >> (S + 1)) & 0x04040404u) | 0x03020100u;
    return __builtin_amdgcn_perm(hi, lo, pick);
}
__device__ __forceinline__ uint32_t cb_lo(uint32_t w, uint4 cb) { return cb_lookup<0>(w, cb); }
__device__ __forceinline__ uint32_t cb_hi(uint32_t w, uint4 cb) { return cb_lookup<4>(w, cb); }

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// The 4-bit GEMM's int8 matrix products start each group's partial from this bit pattern
// instead of zero.  0x4B400000 is the float 1.5 * 2^23, whose ulp is 1, so for |D| < 2^22 the integer
// 0x4B400000 + D read as a float is exactly 1.5 * 2^23 + D, and one exact subtraction gives D as
// a float: the value an int-to-float conversion gives, for a cheaper instruction.  Every GEMM
// partial stays far inside that range: |code| <= 127 activations times weights of magnitude at
// most 128 (16 q and codebook entries) over at most 128 k give |D| <= 2,080,768.  (The int8-
// weight GEMM keeps the conversion: at its register bound the start value's 16 registers spill.)
constexpr int kPartialBias = 0x4B400000;
__device__ __forceinline__ v16i partial_start() {
    v16i z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = kPartialBias;
    return z;
}
__device__ __forceinline__ float partial_to_float(int biased) {
    return __builtin_bit_cast(float, biased) - 12582912.0f;
}

// ---- the activation prepass of one float4 quad
//
// Rotation (optional normalized Walsh-Hadamard transform of 128-wide blocks), per-group int8
// quantization and group sum, as defined in include/w4a8.h.  The calling wavefront holds
// consecutive quads of a row in consecutive lanes: the G/4 lanes of a group, and the 32 lanes of
// a 128-wide rotation block, are aligned runs of lanes that are either all active or all
// inactive (the cross-lane exchanges stay inside them).  Returns the four codes packed into a
// dword (first element in the low byte); scale and sum come back in every lane of the group.
// Bit-exactness: each value goes through the same fp32 operations as the definition (butterflies
// of span 1, 2 inside the lane and 4..64 across lanes 1..16 apart, each output one add or
// subtract of the same two operands, then one multiply by fp32(1/sqrt(128)); an IEEE-rounded
// divide by 127 for the scale; an IEEE-rounded divide then round-half-even for each code), with
// contraction off.
template <int G, bool ROT>
__device__ __forceinline__ int prep_quad(float4 v, int lane, float &scale, int &sum) {
#pragma clang fp contract(off)
    constexpr int kLanesPerGroup = G / 4;
    // 1/sqrt(128) = sqrt(2)/16 rounded to the nearest fp32: sqrt(2) rounds to 0x3FB504F3, and the
    // division by 16 only moves the exponent, giving 0x3DB504F3.
    constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;
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
    scale = amax / 127.0f;
    int q[4] = {0, 0, 0, 0};
    // Codes only where the scale is nonzero: amax / 127 also rounds to 0 for a group of tiny
    // subnormals (amax <= 63 * 2^-149), and then every code is 0, as for amax == 0.
    if (scale > 0.0f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float r = rintf(e[i] / scale);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            q[i] = static_cast<int>(r);
        }
    }
    sum = q[0] + q[1] + q[2] + q[3];
#pragma unroll
    for (int s = 1; s < kLanesPerGroup; s <<= 1) sum += __shfl_xor(sum, s, 64);
    return (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) | ((q[3] & 0xFF) << 24);
}

// ---- gated output of a [gate; up] linear: act(gate) * up
//
// Source: "cactus-compute/engine PR #750: Metal Support", the commit list (a gelu-gated
// feed-forward pair fused into one GEMV, sibling quantized GEMVs batched into one; gelu-erf and
// sigmoid activation codes).  The activations, in fp32 through the device math library:
// silu(v) = v / (1 + e^-v), the tanh approximation of gelu, and gelu with erf.
constexpr int kActSilu = 0, kActGeluTanh = 1, kActGeluErf = 2;
__device__ __forceinline__ float act_apply(int act, float v) {
    if (act == kActSilu) return v / (1.0f + expf(-v));
    if (act == kActGeluTanh)
        return 0.5f * v * (1.0f + tanhf(0.7978845608f * (v + 0.044715f * v * v * v)));
    return 0.5f * v * (1.0f + erff(v * 0.7071067812f));
}

// ---- launchers (each returns the hipGetLastError() of its launch)

hipError_t launch_pack(const Geom &g, const uint8_t *codes, const uint16_t *scales,
                       const uint16_t *bias, const int8_t *codebook, uint8_t *packed,
                       hipStream_t stream, bool row_scale = false);

hipError_t launch_prep(const float *x, int64_t m, int k, int group, int hadamard,
                       int8_t *xq, float *xs, int32_t *xsum, hipStream_t stream);

// y != nullptr: fp32 output; d != nullptr: int32 partials instead.
hipError_t launch_gemv(const Geom &g, const uint8_t *packed, const int8_t *xq, const float *xs,
                       const int32_t *xsum, float *y, int32_t *d, hipStream_t stream);

// The decode GEMV with the prepass of its one activation row fused in: every workgroup
// quantizes x into LDS; workgroup 0 also writes xq, xs, xsum.  k <= kFusedMaxK.  Each workgroup
// (one 64-row panel) repeats the quantization of its wavefronts' groups from L2, which costs less
// than a second launch up to a 262144-row vocabulary head without rotation (4096 panels,
// measured at k 1536: one kernel 35.9 us, prepass + GEMV 37.6 us).  With the 128-block rotation
// every workgroup also repeats the butterflies, and at 4096 panels the one kernel is slower
// (45.8 us against 39.4 + the prepass): there the bound stays 2048 panels, as for the
// fp16-activation path.  Beyond the bound the prepass runs on its own.
constexpr int kFusedMaxK = 16384;
constexpr int kFusedMaxPanels = 4096;
constexpr int kFusedMaxPanelsRot = 2048;
constexpr int kFusedMaxPanelsA16 = 2048;
inline int fused_max_panels(int hadamard) { return hadamard ? kFusedMaxPanelsRot : kFusedMaxPanels; }
constexpr int kFusedQuadsPerLane = 8;   // activation quads one lane of the fused GEMV quantizes
hipError_t launch_gemv_fused(const Geom &g, const uint8_t *packed, const float *x, int hadamard,
                             int8_t *xq, float *xs, int32_t *xsum, float *y, hipStream_t stream);

// Compute units of the current device (cached per device; 0 if the query fails).
int device_cus();
// Split-tile policy of the GEMMs: the number of tiles taken whole by one workgroup each; the rest
// (the tiles of a last, partial round over the CUs, when that round fills at most three quarters
// of them) go to four workgroups each, one k quarter per wavefront.  A CU's time follows how
// many tiles it holds, so such a round would otherwise cost nearly as much as a full one.
int whole_tiles(int tiles);
hipError_t launch_gemm(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                       const float *xs, const int32_t *xsum, float *y, int32_t *d,
                       hipStream_t stream);

// Gated variants: g describes the packed [gate; up] linear (g.n = 2F rows, F % 64 == 0, gate
// rows first); y is [m][F] = act(gate) * up, act one of kActSilu / kActGeluTanh / kActGeluErf.
hipError_t launch_gemv_glu(const Geom &g, int act, const uint8_t *packed, const int8_t *xq,
                           const float *xs, const int32_t *xsum, float *y, hipStream_t stream);
hipError_t launch_gemv_glu_fused(const Geom &g, int act, const uint8_t *packed, const float *x,
                                 int hadamard, int8_t *xq, float *xs, int32_t *xsum, float *y,
                                 hipStream_t stream);
// The greedy tail of one activation row: logits = cap * tanh(y / cap) (cap > 0) or y, stored to
// y; token / value = the smallest index of the largest logit and that logit.  Each GEMV
// workgroup stores the largest key (logit order, then smaller index) of its 64 rows to
// keys[panel]; a one-workgroup kernel after it on the stream reduces the n_pad / 64 keys.
struct Tail {
    float cap;
    unsigned long long *keys;
    int32_t *token;
    float *value;
};
hipError_t launch_gemv_argmax(const Geom &g, const uint8_t *packed, const int8_t *xq,
                              const float *xs, const int32_t *xsum, float *y, const Tail &tail,
                              hipStream_t stream);
// The same tail with the prepass fused into the GEMV (one row, within the fused GEMV's bounds):
// x fp32 [k] in, xq / xs / xsum written by workgroup 0, as launch_gemv_fused.
hipError_t launch_gemv_argmax_fused(const Geom &g, const uint8_t *packed, const float *x,
                                    int hadamard, int8_t *xq, float *xs, int32_t *xsum, float *y,
                                    const Tail &tail, hipStream_t stream);
// The fp16-activation path: the prepass (x fp32 [m][k] -> interleaved halves xh [m][k] and the
// fp32 group sums xsf [k/64][m]) and the linear on them (GEMV for m == 1, GEMM above), for the
// symmetric and affine formats with 64-wide groups.
hipError_t launch_prep_a16(const float *x, int64_t m, int k, uint16_t *xh, float *xsf,
                           hipStream_t stream);
hipError_t launch_linear_a16(const Geom &g, const uint8_t *packed, int m, const uint16_t *xh,
                             const float *xsf, float *y, hipStream_t stream);
// The one-row fp16-activation linear with its prepass fused in (k <= kFusedMaxK): every
// workgroup builds the row's halves and group sums in LDS, workgroup 0 also writes xh and xsf.
hipError_t launch_linear_a16_fused(const Geom &g, const uint8_t *packed, const float *x,
                                   uint16_t *xh, float *xsf, float *y, hipStream_t stream);

// Prefill attention over a packed int8 key/value cache (the packed layout is described in
// include/w4a8.h; offsets in bytes from the packed buffer).
struct AttnGeom {
    int nkvh, nkv, d, nblk;
    uint64_t off_kq, off_sk, off_pos, off_vt, off_sv, off_vsum;
};
int attn_splits(int nh, int nq, int nblk);
hipError_t launch_attn_pack(const AttnGeom &ag, const int8_t *k8, const float *ks,
                            const int8_t *v8, const float *vs, const int32_t *kvpos,
                            uint8_t *packed, hipStream_t stream);
hipError_t launch_attn(const AttnGeom &ag, const uint8_t *packed, const float *q, int nh, int nq,
                       int pos0, int window, int sink, float scale, int8_t *q8, float *sq,
                       float *o, float *m, float *l, float *work, hipStream_t stream);

// Int8 weights (format 3) and 2-, 1- and 3-bit codebook weights (formats 4, 5, 6): the codes
// (and the codebooks) of the packed layout, and the GEMV (m == 1) / GEMM of each.
hipError_t launch_pack_codes_w8(const Geom &g, const int8_t *w8, uint8_t *packed,
                                hipStream_t stream);
hipError_t launch_pack_cq2(const Geom &g, const uint8_t *codes, const int8_t *codebook,
                           uint8_t *packed, hipStream_t stream);
hipError_t launch_pack_bits(const Geom &g, const uint8_t *codes, const int8_t *codebook,
                            uint8_t *packed, hipStream_t stream);
hipError_t launch_w8(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                     const float *xs, const int32_t *xsum, float *y, hipStream_t stream);
// Their exact int32 partials d [m][n][k/group] from the same GEMV (m == 1) or GEMM code.
hipError_t launch_w8_partials(const Geom &g, const uint8_t *packed, int m, const int8_t *xq,
                              const int32_t *xsum, int32_t *d, hipStream_t stream);
// Their one-row GEMV with the prepass fused in (k <= kFusedMaxK): every workgroup quantizes x
// into LDS, workgroup 0 also writes xq, xs and xsum.  w8_gemv_workgroups is its grid size; past
// kFusedMaxW8Workgroups the separate prepass costs less than the repeats (at 2048 workgroups of
// a 262144-row head the fused int8 and 2-bit GEMVs measured 1-7% slower than prepass + GEMV).
struct FusedIO {
    const float *x;
    int8_t *xq;
    float *xs;
    int32_t *xsum;
};
constexpr int kFusedMaxW8Workgroups = 1024;
int w8_gemv_workgroups(const Geom &g);
hipError_t launch_w8_fused(const Geom &g, const uint8_t *packed, const float *x, int hadamard,
                           int8_t *xq, float *xs, int32_t *xsum, float *y, hipStream_t stream);

// The reduction of nkeys panel keys into token and value (one workgroup).
hipError_t launch_argmax_keys(const unsigned long long *keys, int nkeys, int32_t *token,
                              float *value, hipStream_t stream);

// The greedy tail's key of a logit v at row r: the logit's order in the high half (sign bit
// flipped for v >= 0, all bits for v < 0: unsigned order = float order), ~r in the low half (on
// equal logits the smaller row wins).  The largest key over a wavefront's lanes:
__device__ inline unsigned long long wave_max_key(unsigned long long key) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t lo = __shfl_xor(static_cast<uint32_t>(key), o, 64);
        const uint32_t hi = __shfl_xor(static_cast<uint32_t>(key >> 32), o, 64);
        const unsigned long long other = (static_cast<unsigned long long>(hi) << 32) | lo;
        key = other > key ? other : key;
    }
    return key;
}

hipError_t launch_gemm_glu(const Geom &g, int act, const uint8_t *packed, int m,
                           const int8_t *xq, const float *xs, const int32_t *xsum, float *y,
                           hipStream_t stream);

}  // namespace w4a8
