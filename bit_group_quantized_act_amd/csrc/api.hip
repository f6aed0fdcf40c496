// The C ABI of libw4a8 (declared in include/w4a8.h): host-side validation, the gfx950 device
// check, and the launches.  No entry point allocates memory or synchronizes.
#include "../../include/w4a8.h"
#include "w4a8_kernels.h"

#include <cmath>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

namespace {

thread_local char g_last_error[512] = "";

w4a8_status fail(w4a8_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

w4a8_status ok() {
    g_last_error[0] = '\0';
    return W4A8_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

w4a8_status check_device() {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
        (void)hipGetLastError();
        return fail(W4A8_ERR_DEVICE, "no HIP device is visible");
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(W4A8_ERR_DEVICE, "hipGetDevice failed");
    }
    if (dev >= kMaxDevices) return fail(W4A8_ERR_DEVICE, "device index %d is too large", dev);
    int state = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(W4A8_ERR_DEVICE, "hipGetDeviceProperties(%d) failed", dev);
        }
        state = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        g_arch_ok[dev].store(state, std::memory_order_relaxed);
        if (state == 2)
            return fail(W4A8_ERR_DEVICE, "device %d is %s, these kernels are built for gfx950",
                        dev, prop.gcnArchName);
    }
    if (state != 1) return fail(W4A8_ERR_DEVICE, "device %d is not gfx950", dev);
    return W4A8_OK;
}

w4a8_status check_layout(const w4a8_layout *L) {
    if (!L) return fail(W4A8_ERR_ARG, "layout is NULL");
    w4a8_layout ref;
    if (w4a8_packed_layout(L->format, L->n, L->k, L->group, &ref) != W4A8_OK)
        return W4A8_ERR_ARG;   // the message of w4a8_packed_layout stays in place
    if (memcmp(&ref, L, sizeof ref) != 0)
        return fail(W4A8_ERR_ARG, "layout was not produced by w4a8_packed_layout");
    return W4A8_OK;
}

w4a8::Geom geom_of(const w4a8_layout *L) {
    w4a8::Geom g;
    g.fmt = L->format;
    g.n = L->n;
    g.k = L->k;
    g.group = L->group;
    g.n_pad = L->n_pad;
    g.meta_bytes = L->meta_bytes;
    g.off_codes = L->off_codes;
    g.off_meta = L->off_meta;
    g.off_codebook = L->off_codebook;
    return g;
}

w4a8_status launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(W4A8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

#define W4A8_REQUIRE_PTR(p)                                                                    \
    do {                                                                                       \
        if (!(p)) return fail(W4A8_ERR_ARG, #p " is NULL");                                    \
        if (!aligned((p), 16)) return fail(W4A8_ERR_ARG, #p " is not 16-byte aligned");        \
    } while (0)

// Int8 and 1-, 2- and 3-bit codebook weights (byte-decoded) run through their own GEMV / GEMM.
bool byte_decoded(const w4a8_layout *L) {
    return L->format >= W4A8_INT8 && L->format <= W4A8_CQ3;
}

bool has_codebook(int32_t format) {
    return format == W4A8_CODEBOOK_I4 || format == W4A8_CQ2 || format == W4A8_CQ1 ||
           format == W4A8_CQ3;
}

// Entry points whose kernels read only the 4-bit formats.
w4a8_status reject_int8(const w4a8_layout *L, const char *what) {
    if (byte_decoded(L))
        return fail(W4A8_ERR_UNSUPPORTED, "%s takes the 4-bit formats, not format %d", what,
                    L->format);
    return W4A8_OK;
}

// Sizes the GEMM addresses with 32-bit offsets: the activation scales and sums of all rows
// (m * k/group dwords), the activation codes of the byte-decoded formats' GEMM, and the
// workgroup count.
w4a8_status check_gemm_size(const w4a8_layout *L, int32_t m) {
    // (the GEMM's copies run up to 16 groups past the last one)
    const int64_t scales = static_cast<int64_t>(m) * (L->k / L->group + 16) * 4;
    if (scales > 0x7FFFFFF0ll)
        return fail(W4A8_ERR_UNSUPPORTED, "m * k/group = %lld scales exceed 2 GiB",
                    static_cast<long long>(scales / 4));
    if (byte_decoded(L) && static_cast<int64_t>(m) * L->k > 0x7FFFFFF0ll)
        return fail(W4A8_ERR_UNSUPPORTED, "m * k = %lld activation codes exceed 2^31 - 16",
                    static_cast<long long>(static_cast<int64_t>(m) * L->k));
    const int64_t tiles = static_cast<int64_t>((m + 63) / 64) * ((L->n_pad + 127) / 128);
    if (tiles > 0x7FFFFFFFll)
        return fail(W4A8_ERR_UNSUPPORTED, "%lld GEMM tiles exceed the grid",
                    static_cast<long long>(tiles));
    return W4A8_OK;
}

w4a8_status check_activation_ptrs(const int8_t *xq, const float *xs, const int32_t *xsum) {
    W4A8_REQUIRE_PTR(xq);
    W4A8_REQUIRE_PTR(xs);
    W4A8_REQUIRE_PTR(xsum);
    return W4A8_OK;
}

// Checks shared by the greedy-tail entry points: the cap and the three tail buffers.
w4a8_status check_tail(const w4a8_layout *L, float softcap, const int32_t *token,
                       const float *value, const void *work, uint64_t work_bytes) {
    if (!(softcap >= 0.0f) || !std::isfinite(softcap))
        return fail(W4A8_ERR_ARG, "softcap %g is negative or not finite", softcap);
    if (!token) return fail(W4A8_ERR_ARG, "token is NULL");
    if (!value) return fail(W4A8_ERR_ARG, "value is NULL");
    if (!aligned(token, 4) || !aligned(value, 4))
        return fail(W4A8_ERR_ARG, "token / value are not 4-byte aligned");
    if (!work) return fail(W4A8_ERR_ARG, "work is NULL");
    if (!aligned(work, 8)) return fail(W4A8_ERR_ARG, "work is not 8-byte aligned");
    if (work_bytes < W4A8_ARGMAX_WORK_BYTES(L->n))
        return fail(W4A8_ERR_ARG, "work has %llu bytes, n = %d needs %llu",
                    static_cast<unsigned long long>(work_bytes), L->n,
                    static_cast<unsigned long long>(W4A8_ARGMAX_WORK_BYTES(L->n)));
    return W4A8_OK;
}

// Checks shared by the gated entry points (after check_layout): the [gate; up] split, the
// activation and the gate-to-up span that one descriptor addresses (offsets below 2^31).
w4a8_status check_glu(const w4a8_layout *L, int32_t m, const void *packed, int32_t act) {
    if (reject_int8(L, "the gated output") != W4A8_OK) return W4A8_ERR_UNSUPPORTED;
    if (m < 0) return fail(W4A8_ERR_ARG, "m = %d is negative", m);
    if (m > (1 << 20)) return fail(W4A8_ERR_UNSUPPORTED, "m = %d is above 2^20", m);
    if (!packed) return fail(W4A8_ERR_ARG, "packed is NULL");
    if (!aligned(packed, 256)) return fail(W4A8_ERR_ARG, "packed is not 256-byte aligned");
    if (L->n % (2 * W4A8_PANEL_ROWS) != 0)
        return fail(W4A8_ERR_ARG, "n = %d is not 2F with F a multiple of %d (gate, then up rows)",
                    L->n, W4A8_PANEL_ROWS);
    if (act < W4A8_ACT_SILU || act > W4A8_ACT_GELU_ERF)
        return fail(W4A8_ERR_ARG, "act = %d is not a w4a8_act", act);
    const uint64_t span_rows = static_cast<uint64_t>(L->n / 2 + W4A8_PANEL_ROWS);
    const uint64_t code_span = span_rows * static_cast<uint64_t>(L->k) / 2;
    const uint64_t meta_span = span_rows * ((static_cast<uint64_t>(L->k / L->group) + 3) / 4) * 4 *
                               static_cast<uint64_t>(L->format == W4A8_AFFINE_U4 ? 4 : 2);
    if (code_span > 0x7FFFFFF0ull || meta_span > 0x7FFFFFF0ull)
        return fail(W4A8_ERR_UNSUPPORTED, "the gate-to-up span (%llu code bytes) exceeds 2^31 - 16",
                    static_cast<unsigned long long>(code_span));
    return W4A8_OK;
}

}  // namespace

extern "C" {

w4a8_status w4a8_packed_layout(int32_t format, int32_t n, int32_t k, int32_t group,
                               w4a8_layout *L) {
    if (!L) return fail(W4A8_ERR_ARG, "layout is NULL");
    if (format < W4A8_SYM_I4 || format > W4A8_CQ3)
        return fail(W4A8_ERR_ARG, "format %d is not a w4a8_format", format);
    if (group != 64 && group != 128) return fail(W4A8_ERR_ARG, "group %d is not 64 or 128", group);
    if (n < 1 || n > (1 << 24)) return fail(W4A8_ERR_ARG, "n = %d is outside [1, 2^24]", n);
    if (k < group || k > (1 << 20) || k % group != 0)
        return fail(W4A8_ERR_ARG, "k = %d must be a multiple of group %d in [group, 2^20]", k,
                    group);
    memset(L, 0, sizeof *L);
    L->format = format;
    L->n = n;
    L->k = k;
    L->group = group;
    L->n_pad = static_cast<int32_t>(round_up(n, W4A8_PANEL_ROWS));
    L->meta_bytes = (format == W4A8_AFFINE_U4) ? 4 : 2;
    // bytes per 128 k of a row: 128 (int8), 64 (4-bit), 32 (CQ2), 16 (CQ1), 48 (CQ3; CQ1 and
    // CQ3 pad k up to a multiple of 128)
    const uint64_t chunks128 = static_cast<uint64_t>(k + 127) / 128;
    const uint64_t codes =
        format == W4A8_CQ1 ? L->n_pad * chunks128 * 16
        : format == W4A8_CQ3 ? L->n_pad * chunks128 * 48
        : static_cast<uint64_t>(L->n_pad) * k /
              (format == W4A8_INT8 ? 1 : format == W4A8_CQ2 ? 4 : 2);
    // metadata in blocks of 4 groups (the last block zero-padded)
    const uint64_t meta = static_cast<uint64_t>(L->n_pad) * ((k / group + 3) / 4) * 4 * L->meta_bytes;
    L->off_codes = 0;
    L->off_meta = round_up(codes, 256);
    uint64_t end = L->off_meta + round_up(meta, 256);
    if (has_codebook(format)) {
        L->off_codebook = end;
        const int per_row = format == W4A8_CODEBOOK_I4 ? 16 : format == W4A8_CQ3 ? 8 : 4;
        end += round_up(static_cast<uint64_t>(L->n_pad) * per_row, 256);
    }
    L->bytes = end;
    return ok();
}

namespace {
w4a8_status pack_checked(const w4a8_layout *L, const uint8_t *codes, const uint16_t *scales_f16,
                         const uint16_t *bias_f16, const int8_t *codebook, void *packed,
                         void *stream, bool row_scale) {
    w4a8_status s = check_layout(L);
    if (s != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(codes);
    W4A8_REQUIRE_PTR(scales_f16);
    if (!packed) return fail(W4A8_ERR_ARG, "packed is NULL");
    if (!aligned(packed, 256)) return fail(W4A8_ERR_ARG, "packed is not 256-byte aligned");
    if (L->format == W4A8_AFFINE_U4) {
        W4A8_REQUIRE_PTR(bias_f16);
    } else if (bias_f16) {
        return fail(W4A8_ERR_ARG, "bias_f16 is only used by the affine format; pass NULL");
    }
    if (has_codebook(L->format)) {
        W4A8_REQUIRE_PTR(codebook);
    } else if (codebook) {
        return fail(W4A8_ERR_ARG, "codebook is only used by the codebook format; pass NULL");
    }
    if ((s = check_device()) != W4A8_OK) return s;
    return launched(w4a8::launch_pack(geom_of(L), codes, scales_f16, bias_f16, codebook,
                                      static_cast<uint8_t *>(packed),
                                      static_cast<hipStream_t>(stream), row_scale),
                    "pack launch");
}
}  // namespace

w4a8_status w4a8_pack_weights(const w4a8_layout *L, const uint8_t *codes,
                              const uint16_t *scales_f16, const uint16_t *bias_f16,
                              const int8_t *codebook, void *packed, void *stream) {
    return pack_checked(L, codes, scales_f16, bias_f16, codebook, packed, stream, false);
}

w4a8_status w4a8_pack_weights_row_scale(const w4a8_layout *L, const uint8_t *codes,
                                        const uint16_t *row_scales_f16,
                                        const uint16_t *row_bias_f16, const int8_t *codebook,
                                        void *packed, void *stream) {
    return pack_checked(L, codes, row_scales_f16, row_bias_f16, codebook, packed, stream, true);
}

w4a8_status w4a8_prep(const float *x, int32_t m, int32_t k, int32_t group,
                      int32_t hadamard_block, int8_t *xq, float *xs, int32_t *xsum,
                      void *stream) {
    if (m < 0) return fail(W4A8_ERR_ARG, "m = %d is negative", m);
    if (group != 64 && group != 128) return fail(W4A8_ERR_ARG, "group %d is not 64 or 128", group);
    if (k < group || k > (1 << 20) || k % group != 0)
        return fail(W4A8_ERR_ARG, "k = %d must be a multiple of group %d in [group, 2^20]", k,
                    group);
    if (hadamard_block != 0 && hadamard_block != 128)
        return fail(W4A8_ERR_ARG, "hadamard_block %d is not 0 or 128", hadamard_block);
    if (hadamard_block == 128 && k % 128 != 0)
        return fail(W4A8_ERR_ARG, "k = %d is not a multiple of the rotation block 128", k);
    if (static_cast<int64_t>(m) * k > (int64_t{1} << 38))
        return fail(W4A8_ERR_UNSUPPORTED, "m * k = %lld is above 2^38",
                    static_cast<long long>(static_cast<int64_t>(m) * k));
    if (m == 0) return ok();   // nothing to do; the pointers may be NULL
    W4A8_REQUIRE_PTR(x);
    w4a8_status s = check_activation_ptrs(xq, xs, xsum);
    if (s != W4A8_OK) return s;
    if ((s = check_device()) != W4A8_OK) return s;
    return launched(w4a8::launch_prep(x, m, k, group, hadamard_block, xq, xs, xsum,
                                      static_cast<hipStream_t>(stream)),
                    "prep launch");
}

w4a8_status w4a8_gemv(const w4a8_layout *L, const void *packed, const int8_t *xq,
                      const float *xs, const int32_t *xsum, float *y, void *stream) {
    w4a8_status s = check_layout(L);
    if (s != W4A8_OK) return s;
    if (!packed) return fail(W4A8_ERR_ARG, "packed is NULL");
    if (!aligned(packed, 256)) return fail(W4A8_ERR_ARG, "packed is not 256-byte aligned");
    if ((s = check_activation_ptrs(xq, xs, xsum)) != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(y);
    if ((s = check_device()) != W4A8_OK) return s;
    if (byte_decoded(L))
        return launched(w4a8::launch_w8(geom_of(L), static_cast<const uint8_t *>(packed), 1, xq,
                                        xs, xsum, y, static_cast<hipStream_t>(stream)),
                        "int8-weight gemv launch");
    return launched(w4a8::launch_gemv(geom_of(L), static_cast<const uint8_t *>(packed), xq, xs,
                                      xsum, y, nullptr, static_cast<hipStream_t>(stream)),
                    "gemv launch");
}

w4a8_status w4a8_gemm(const w4a8_layout *L, const void *packed, int32_t m, const int8_t *xq,
                      const float *xs, const int32_t *xsum, float *y, void *stream) {
    w4a8_status s = check_layout(L);
    if (s != W4A8_OK) return s;
    if (m < 0) return fail(W4A8_ERR_ARG, "m = %d is negative", m);
    if (m > (1 << 20)) return fail(W4A8_ERR_UNSUPPORTED, "m = %d is above 2^20", m);
    if (!packed) return fail(W4A8_ERR_ARG, "packed is NULL");
    if (!aligned(packed, 256)) return fail(W4A8_ERR_ARG, "packed is not 256-byte aligned");
    if (m == 0) return ok();   // nothing to do; the activation and output pointers may be NULL
    if ((s = check_gemm_size(L, m)) != W4A8_OK) return s;
    if ((s = check_activation_ptrs(xq, xs, xsum)) != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(y);
    if ((s = check_device()) != W4A8_OK) return s;
    if (byte_decoded(L))
        return launched(w4a8::launch_w8(geom_of(L), static_cast<const uint8_t *>(packed), m, xq,
                                        xs, xsum, y, static_cast<hipStream_t>(stream)),
                        "int8-weight gemm launch");
    return launched(w4a8::launch_gemm(geom_of(L), static_cast<const uint8_t *>(packed), m, xq,
                                      xs, xsum, y, nullptr, static_cast<hipStream_t>(stream)),
                    "gemm launch");
}

w4a8_status w4a8_linear(const w4a8_layout *L, const void *packed, int32_t m, const float *x,
                        int32_t hadamard_block, int8_t *xq, float *xs, int32_t *xsum, float *y,
                        void *stream) {
    w4a8_status s = check_layout(L);
    if (s != W4A8_OK) return s;
    if (m < 0) return fail(W4A8_ERR_ARG, "m = %d is negative", m);
    if (m > (1 << 20)) return fail(W4A8_ERR_UNSUPPORTED, "m = %d is above 2^20", m);
    if (!packed) return fail(W4A8_ERR_ARG, "packed is NULL");
    if (!aligned(packed, 256)) return fail(W4A8_ERR_ARG, "packed is not 256-byte aligned");
    if (hadamard_block != 0 && hadamard_block != 128)
        return fail(W4A8_ERR_ARG, "hadamard_block %d is not 0 or 128", hadamard_block);
    if (hadamard_block == 128 && L->k % 128 != 0)
        return fail(W4A8_ERR_ARG, "k = %d is not a multiple of the rotation block 128", L->k);
    if (m == 0) return ok();
    if ((s = check_gemm_size(L, m)) != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(x);
    if ((s = check_activation_ptrs(xq, xs, xsum)) != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(y);
    if ((s = check_device()) != W4A8_OK) return s;
    const w4a8::Geom g = geom_of(L);
    const uint8_t *pk = static_cast<const uint8_t *>(packed);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!byte_decoded(L) && m == 1 && L->k <= w4a8::kFusedMaxK &&
        L->n_pad / W4A8_PANEL_ROWS <= w4a8::fused_max_panels(hadamard_block))
        return launched(w4a8::launch_gemv_fused(g, pk, x, hadamard_block, xq, xs, xsum, y, st),
                        "fused gemv launch");
    if (byte_decoded(L) && m == 1 && L->k <= w4a8::kFusedMaxK &&
        w4a8::w8_gemv_workgroups(g) <= w4a8::kFusedMaxW8Workgroups)
        return launched(w4a8::launch_w8_fused(g, pk, x, hadamard_block, xq, xs, xsum, y, st),
                        "fused int8-weight gemv launch");
    hipError_t e = w4a8::launch_prep(x, m, L->k, L->group, hadamard_block, xq, xs, xsum, st);
    if (e != hipSuccess) return launched(e, "prep launch");
    if (byte_decoded(L))
        return launched(w4a8::launch_w8(g, pk, m, xq, xs, xsum, y, st),
                        "int8-weight linear launch");
    if (m == 1)
        return launched(w4a8::launch_gemv(g, pk, xq, xs, xsum, y, nullptr, st), "gemv launch");
    return launched(w4a8::launch_gemm(g, pk, m, xq, xs, xsum, y, nullptr, st), "gemm launch");
}

w4a8_status w4a8_gemm_glu(const w4a8_layout *L, const void *packed, int32_t m, const int8_t *xq,
                          const float *xs, const int32_t *xsum, int32_t act, float *y,
                          void *stream) {
    w4a8_status s = check_layout(L);
    if (s != W4A8_OK) return s;
    if ((s = check_glu(L, m, packed, act)) != W4A8_OK) return s;
    if (m == 0) return ok();
    if ((s = check_gemm_size(L, m)) != W4A8_OK) return s;
    if ((s = check_activation_ptrs(xq, xs, xsum)) != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(y);
    if ((s = check_device()) != W4A8_OK) return s;
    const w4a8::Geom g = geom_of(L);
    const uint8_t *pk = static_cast<const uint8_t *>(packed);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (m == 1)
        return launched(w4a8::launch_gemv_glu(g, act, pk, xq, xs, xsum, y, st), "gated gemv launch");
    return launched(w4a8::launch_gemm_glu(g, act, pk, m, xq, xs, xsum, y, st), "gated gemm launch");
}

w4a8_status w4a8_linear_glu(const w4a8_layout *L, const void *packed, int32_t m, const float *x,
                            int32_t hadamard_block, int32_t act, int8_t *xq, float *xs,
                            int32_t *xsum, float *y, void *stream) {
    w4a8_status s = check_layout(L);
    if (s != W4A8_OK) return s;
    if ((s = check_glu(L, m, packed, act)) != W4A8_OK) return s;
    if (hadamard_block != 0 && hadamard_block != 128)
        return fail(W4A8_ERR_ARG, "hadamard_block %d is not 0 or 128", hadamard_block);
    if (hadamard_block == 128 && L->k % 128 != 0)
        return fail(W4A8_ERR_ARG, "k = %d is not a multiple of the rotation block 128", L->k);
    if (m == 0) return ok();
    if ((s = check_gemm_size(L, m)) != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(x);
    if ((s = check_activation_ptrs(xq, xs, xsum)) != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(y);
    if ((s = check_device()) != W4A8_OK) return s;
    const w4a8::Geom g = geom_of(L);
    const uint8_t *pk = static_cast<const uint8_t *>(packed);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (m == 1 && L->k <= w4a8::kFusedMaxK &&
        L->n_pad / W4A8_PANEL_ROWS <= w4a8::fused_max_panels(hadamard_block))
        return launched(w4a8::launch_gemv_glu_fused(g, act, pk, x, hadamard_block, xq, xs, xsum,
                                                    y, st),
                        "fused gated gemv launch");
    hipError_t e = w4a8::launch_prep(x, m, L->k, L->group, hadamard_block, xq, xs, xsum, st);
    if (e != hipSuccess) return launched(e, "prep launch");
    if (m == 1)
        return launched(w4a8::launch_gemv_glu(g, act, pk, xq, xs, xsum, y, st), "gated gemv launch");
    return launched(w4a8::launch_gemm_glu(g, act, pk, m, xq, xs, xsum, y, st), "gated gemm launch");
}

}  // extern "C"

namespace {
// Validation and launches of the one-row greedy tail on a given key buffer (the caller's work
// buffer, or the library's own static one for w4a8_lm_head_argmax_noalloc).
w4a8_status lm_head_argmax_checked(const w4a8_layout *L, const void *packed, const float *x,
                                   int32_t hadamard_block, float softcap, int8_t *xq, float *xs,
                                   int32_t *xsum, float *logits, int32_t *token, float *value,
                                   void *work, uint64_t work_bytes, void *stream) {
    w4a8_status s;
    if ((s = reject_int8(L, "the greedy tail")) != W4A8_OK) return s;
    if (!packed) return fail(W4A8_ERR_ARG, "packed is NULL");
    if (!aligned(packed, 256)) return fail(W4A8_ERR_ARG, "packed is not 256-byte aligned");
    if ((s = check_tail(L, softcap, token, value, work, work_bytes)) != W4A8_OK) return s;
    if (hadamard_block != 0 && hadamard_block != 128)
        return fail(W4A8_ERR_ARG, "hadamard_block %d is not 0 or 128", hadamard_block);
    if (hadamard_block == 128 && L->k % 128 != 0)
        return fail(W4A8_ERR_ARG, "k = %d is not a multiple of the rotation block 128", L->k);
    W4A8_REQUIRE_PTR(x);
    if ((s = check_activation_ptrs(xq, xs, xsum)) != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(logits);
    if ((s = check_device()) != W4A8_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const w4a8::Tail tail{softcap, static_cast<unsigned long long *>(work), token, value};
    const uint8_t *pk = static_cast<const uint8_t *>(packed);
    // within the fused GEMV's bounds the prepass runs inside the GEMV, as in w4a8_linear
    if (L->k <= w4a8::kFusedMaxK &&
        L->n_pad / W4A8_PANEL_ROWS <= w4a8::fused_max_panels(hadamard_block))
        return launched(w4a8::launch_gemv_argmax_fused(geom_of(L), pk, x, hadamard_block, xq, xs,
                                                       xsum, logits, tail, st),
                        "fused greedy tail gemv launch");
    hipError_t e = w4a8::launch_prep(x, 1, L->k, L->group, hadamard_block, xq, xs, xsum, st);
    if (e != hipSuccess) return launched(e, "prep launch");
    return launched(w4a8::launch_gemv_argmax(geom_of(L), pk, xq, xs, xsum, logits, tail, st),
                    "greedy tail gemv launch");
}

// ---- the key buffer of w4a8_lm_head_argmax_noalloc
//
// One 64-bit key per 64-row panel of the largest head the entry point takes.  Every GPU the
// library runs on holds its own copy until the process ends.  Host code never uses the array's
// name as an address (on the host it is only a stand-in for the symbol): the device address is
// looked up once per device with hipGetSymbolAddress, with that device current, and kept.
constexpr uint64_t kNoAllocKeyBytes = W4A8_ARGMAX_WORK_BYTES(W4A8_NOALLOC_MAX_N);
static __device__ __align__(256) unsigned long long scratch[kNoAllocKeyBytes / 8];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (nullptr: not yet)

w4a8_status scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(W4A8_ERR_DEVICE, "hipGetDevice failed");
    }
    if (dev >= kMaxDevices) return fail(W4A8_ERR_DEVICE, "device index %d is too large", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(W4A8_ERR_HIP, "hipGetSymbolAddress of the key buffer on device %d: %s",
                        dev, hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return W4A8_OK;
}
}  // namespace

extern "C" {

w4a8_status w4a8_lm_head_argmax(const w4a8_layout *L, const void *packed, const float *x,
                                int32_t hadamard_block, float softcap, int8_t *xq, float *xs,
                                int32_t *xsum, float *logits, int32_t *token, float *value,
                                void *work, uint64_t work_bytes, void *stream) {
    w4a8_status s = check_layout(L);
    if (s != W4A8_OK) return s;
    return lm_head_argmax_checked(L, packed, x, hadamard_block, softcap, xq, xs, xsum, logits,
                                  token, value, work, work_bytes, stream);
}

w4a8_status w4a8_lm_head_argmax_noalloc(const w4a8_layout *L, const void *packed,
                                        const float *x, int32_t hadamard_block, float softcap,
                                        int8_t *xq, float *xs, int32_t *xsum, float *logits,
                                        int32_t *token, float *value, void *stream) {
    w4a8_status s = check_layout(L);
    if (s != W4A8_OK) return s;
    if (L->n > W4A8_NOALLOC_MAX_N)
        return fail(W4A8_ERR_UNSUPPORTED,
                    "n = %d is above W4A8_NOALLOC_MAX_N = %d, the size of the library's own key "
                    "buffer (w4a8_lm_head_argmax takes a work buffer of any size)",
                    L->n, W4A8_NOALLOC_MAX_N);
    if ((s = check_device()) != W4A8_OK) return s;
    void *keys = nullptr;
    if ((s = scratch_of_current_device(&keys)) != W4A8_OK) return s;
    return lm_head_argmax_checked(L, packed, x, hadamard_block, softcap, xq, xs, xsum, logits,
                                  token, value, keys, kNoAllocKeyBytes, stream);
}

w4a8_status w4a8_gemv_argmax(const w4a8_layout *L, const void *packed, const int8_t *xq,
                             const float *xs, const int32_t *xsum, float softcap, float *logits,
                             int32_t *token, float *value, void *work, uint64_t work_bytes,
                             void *stream) {
    w4a8_status s = check_layout(L);
    if (s != W4A8_OK) return s;
    if ((s = reject_int8(L, "the greedy tail")) != W4A8_OK) return s;
    if (!packed) return fail(W4A8_ERR_ARG, "packed is NULL");
    if (!aligned(packed, 256)) return fail(W4A8_ERR_ARG, "packed is not 256-byte aligned");
    if ((s = check_tail(L, softcap, token, value, work, work_bytes)) != W4A8_OK) return s;
    if ((s = check_activation_ptrs(xq, xs, xsum)) != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(logits);
    if ((s = check_device()) != W4A8_OK) return s;
    const w4a8::Tail tail{softcap, static_cast<unsigned long long *>(work), token, value};
    return launched(w4a8::launch_gemv_argmax(geom_of(L), static_cast<const uint8_t *>(packed), xq,
                                             xs, xsum, logits, tail,
                                             static_cast<hipStream_t>(stream)),
                    "greedy tail gemv launch");
}

namespace {
// Arguments of the fp16-activation prepass (shared by the entry points that run it).
w4a8_status check_prep_a16(const float *x, int32_t m, int32_t k, int32_t group, uint16_t *xh,
                           float *xsf) {
    if (m < 0) return fail(W4A8_ERR_ARG, "m = %d is negative", m);
    if (group != 64)
        return fail(W4A8_ERR_ARG, "group %d: the fp16-activation path sums 64-wide groups",
                    group);
    if (k < 64 || k > (1 << 20) || k % 64 != 0)
        return fail(W4A8_ERR_ARG, "k = %d must be a multiple of 64 in [64, 2^20]", k);
    if (static_cast<int64_t>(m) * k * 2 > 0x7FFFFFF0ll)
        return fail(W4A8_ERR_UNSUPPORTED, "m * k = %lld halves exceed 2^31 - 16 bytes",
                    static_cast<long long>(static_cast<int64_t>(m) * k));
    if (m == 0) return W4A8_OK;
    W4A8_REQUIRE_PTR(x);
    W4A8_REQUIRE_PTR(xh);
    W4A8_REQUIRE_PTR(xsf);
    return W4A8_OK;
}

// The layout and output arguments of the fp16-activation linear.
w4a8_status check_linear_a16(const w4a8_layout *L, const void *packed, int32_t m, float *y) {
    w4a8_status s = check_layout(L);
    if (s != W4A8_OK) return s;
    if (L->format != W4A8_SYM_I4 && L->format != W4A8_AFFINE_U4)
        return fail(W4A8_ERR_UNSUPPORTED, "the fp16-activation path takes SYM or AFFINE weights");
    if (L->group != 64)
        return fail(W4A8_ERR_ARG, "group %d: the fp16-activation path sums 64-wide groups",
                    L->group);
    if (m < 0) return fail(W4A8_ERR_ARG, "m = %d is negative", m);
    if (m == 0) return W4A8_OK;
    if (!packed) return fail(W4A8_ERR_ARG, "packed is NULL");
    if (!aligned(packed, 256)) return fail(W4A8_ERR_ARG, "packed is not 256-byte aligned");
    W4A8_REQUIRE_PTR(y);
    return W4A8_OK;
}
}  // namespace

w4a8_status w4a8_prep_a16(const float *x, int32_t m, int32_t k, int32_t group, uint16_t *xh,
                          float *xsf, void *stream) {
    w4a8_status s = check_prep_a16(x, m, k, group, xh, xsf);
    if (s != W4A8_OK || m == 0) return s;
    if ((s = check_device()) != W4A8_OK) return s;
    return launched(w4a8::launch_prep_a16(x, m, k, xh, xsf, static_cast<hipStream_t>(stream)),
                    "fp16-activation prep launch");
}

w4a8_status w4a8_gemm_a16(const w4a8_layout *L, const void *packed, int32_t m,
                          const uint16_t *xh, const float *xsf, float *y, void *stream) {
    w4a8_status s = check_linear_a16(L, packed, m, y);
    if (s != W4A8_OK || m == 0) return s;
    if (static_cast<int64_t>(m) * L->k * 2 > 0x7FFFFFF0ll)
        return fail(W4A8_ERR_UNSUPPORTED, "m * k = %lld halves exceed 2^31 - 16 bytes",
                    static_cast<long long>(static_cast<int64_t>(m) * L->k));
    W4A8_REQUIRE_PTR(xh);
    W4A8_REQUIRE_PTR(xsf);
    if ((s = check_device()) != W4A8_OK) return s;
    return launched(w4a8::launch_linear_a16(geom_of(L), static_cast<const uint8_t *>(packed), m,
                                            xh, xsf, y, static_cast<hipStream_t>(stream)),
                    "fp16-activation linear launch");
}

w4a8_status w4a8_linear_a16(const w4a8_layout *L, const void *packed, int32_t m, const float *x,
                            uint16_t *xh, float *xsf, float *y, void *stream) {
    w4a8_status s = check_linear_a16(L, packed, m, y);
    if (s != W4A8_OK) return s;
    if ((s = check_prep_a16(x, m, L->k, L->group, xh, xsf)) != W4A8_OK || m == 0) return s;
    if ((s = check_device()) != W4A8_OK) return s;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (m == 1 && L->k <= w4a8::kFusedMaxK && L->n_pad / W4A8_PANEL_ROWS <= w4a8::kFusedMaxPanelsA16)
        return launched(w4a8::launch_linear_a16_fused(geom_of(L), static_cast<const uint8_t *>(packed),
                                                      x, xh, xsf, y, st),
                        "fused fp16-activation gemv launch");
    hipError_t e = w4a8::launch_prep_a16(x, m, L->k, xh, xsf, st);
    if (e != hipSuccess) return launched(e, "fp16-activation prep launch");
    return launched(w4a8::launch_linear_a16(geom_of(L), static_cast<const uint8_t *>(packed), m,
                                            xh, xsf, y, st),
                    "fp16-activation linear launch");
}

namespace {
w4a8_status check_attn_layout(const w4a8_attn_layout *AL) {
    if (!AL) return fail(W4A8_ERR_ARG, "attention layout is NULL");
    w4a8_attn_layout ref;
    if (w4a8_attn_layout_init(AL->nkvh, AL->nkv, AL->d, &ref) != W4A8_OK ||
        std::memcmp(&ref, AL, sizeof(ref)) != 0)
        return fail(W4A8_ERR_ARG, "attention layout was not filled by w4a8_attn_layout_init");
    return W4A8_OK;
}

w4a8::AttnGeom attn_geom_of(const w4a8_attn_layout *AL) {
    return w4a8::AttnGeom{AL->nkvh, AL->nkv, AL->d, AL->nblk, AL->off_kq, AL->off_sk,
                          AL->off_pos, AL->off_vt, AL->off_sv, AL->off_vsum};
}
}  // namespace

w4a8_status w4a8_attn_layout_init(int32_t nkvh, int32_t nkv, int32_t d, w4a8_attn_layout *AL) {
    if (!AL) return fail(W4A8_ERR_ARG, "AL is NULL");
    if (d != 64 && d != 128 && d != 256)
        return fail(W4A8_ERR_ARG, "head dimension %d is not 64, 128 or 256", d);
    if (nkvh < 1 || nkvh > 1024) return fail(W4A8_ERR_ARG, "nkvh = %d is outside [1, 1024]", nkvh);
    if (nkv < 1 || nkv > (1 << 24)) return fail(W4A8_ERR_ARG, "nkv = %d is outside [1, 2^24]", nkv);
    std::memset(AL, 0, sizeof(*AL));
    AL->nkvh = nkvh;
    AL->nkv = nkv;
    AL->d = d;
    AL->nblk = (nkv + 63) / 64;
    const uint64_t slots = static_cast<uint64_t>(nkvh) * AL->nblk * 64;
    uint64_t off = 0;
    AL->off_kq = off;   off = round_up(off + slots * d, 256);
    AL->off_sk = off;   off = round_up(off + slots * 4, 256);
    AL->off_pos = off;  off = round_up(off + slots * 4, 256);
    AL->off_vt = off;   off = round_up(off + slots * d, 256);
    AL->off_sv = off;   off = round_up(off + slots * (d / 32) * 4, 256);
    AL->off_vsum = off; off = round_up(off + static_cast<uint64_t>(nkvh) * AL->nblk * d * 4, 256);
    AL->bytes = off;
    return W4A8_OK;
}

w4a8_status w4a8_attn_pack_kv(const w4a8_attn_layout *AL, const int8_t *k8, const float *ks,
                              const int8_t *v8, const float *vs, const int32_t *kvpos,
                              void *packed, void *stream) {
    w4a8_status s = check_attn_layout(AL);
    if (s != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(k8);
    W4A8_REQUIRE_PTR(ks);
    W4A8_REQUIRE_PTR(v8);
    W4A8_REQUIRE_PTR(vs);
    W4A8_REQUIRE_PTR(kvpos);
    if (!packed) return fail(W4A8_ERR_ARG, "packed is NULL");
    if (!aligned(packed, 256)) return fail(W4A8_ERR_ARG, "packed is not 256-byte aligned");
    if ((s = check_device()) != W4A8_OK) return s;
    return launched(w4a8::launch_attn_pack(attn_geom_of(AL), k8, ks, v8, vs, kvpos,
                                           static_cast<uint8_t *>(packed),
                                           static_cast<hipStream_t>(stream)),
                    "attention cache pack launch");
}

uint64_t w4a8_attn_work_bytes(const w4a8_attn_layout *AL, int32_t nh, int32_t nq) {
    if (!AL || nh < 1 || nq < 1) return 0;
    const int splits = w4a8::attn_splits(nh, nq, AL->nblk);
    if (splits <= 1) return 0;
    return static_cast<uint64_t>(splits) * nh * nq * (AL->d + 2) * 4;
}

w4a8_status w4a8_attn_prefill(const w4a8_attn_layout *AL, const void *packed, const float *q,
                              int32_t nh, int32_t nq, int32_t pos0, int32_t window, int32_t sink,
                              float scale, int8_t *q8, float *sq, float *o, float *m, float *l,
                              void *work, uint64_t work_bytes, void *stream) {
    w4a8_status s = check_attn_layout(AL);
    if (s != W4A8_OK) return s;
    if (nh < 1 || nh % AL->nkvh != 0)
        return fail(W4A8_ERR_ARG, "nh = %d is not a positive multiple of nkvh = %d", nh, AL->nkvh);
    if (nq < 0 || pos0 < 0 || window < 0 || sink < 0)
        return fail(W4A8_ERR_ARG, "nq, pos0, window and sink must not be negative");
    if (!(scale > 0.0f) || !std::isfinite(scale))
        return fail(W4A8_ERR_ARG, "scale %g is not positive and finite", scale);
    if (static_cast<int64_t>(nh) * nq * AL->d > (int64_t{1} << 34))
        return fail(W4A8_ERR_UNSUPPORTED, "nh * nq * d is above 2^34");
    if (nq == 0) return W4A8_OK;
    if (!packed) return fail(W4A8_ERR_ARG, "packed is NULL");
    if (!aligned(packed, 256)) return fail(W4A8_ERR_ARG, "packed is not 256-byte aligned");
    W4A8_REQUIRE_PTR(q);
    W4A8_REQUIRE_PTR(q8);
    W4A8_REQUIRE_PTR(sq);
    W4A8_REQUIRE_PTR(o);
    W4A8_REQUIRE_PTR(m);
    W4A8_REQUIRE_PTR(l);
    const uint64_t need = w4a8_attn_work_bytes(AL, nh, nq);
    if (need > 0) {
        if (work_bytes < need)
            return fail(W4A8_ERR_ARG, "work has %llu bytes, %llu are needed",
                        static_cast<unsigned long long>(work_bytes),
                        static_cast<unsigned long long>(need));
        W4A8_REQUIRE_PTR(work);
    }
    if ((s = check_device()) != W4A8_OK) return s;
    return launched(w4a8::launch_attn(attn_geom_of(AL), static_cast<const uint8_t *>(packed), q,
                                      nh, nq, pos0, window, sink, scale, q8, sq, o, m, l,
                                      static_cast<float *>(work), static_cast<hipStream_t>(stream)),
                    "attention launch");
}

w4a8_status w4a8_debug_partials(const w4a8_layout *L, const void *packed, int32_t m,
                                const int8_t *xq, const int32_t *xsum, int32_t *d,
                                void *stream) {
    w4a8_status s = check_layout(L);
    if (s != W4A8_OK) return s;
    if (m < 1) return fail(W4A8_ERR_ARG, "m = %d must be at least 1", m);
    if (m > (1 << 20)) return fail(W4A8_ERR_UNSUPPORTED, "m = %d is above 2^20", m);
    if (!packed) return fail(W4A8_ERR_ARG, "packed is NULL");
    if (!aligned(packed, 256)) return fail(W4A8_ERR_ARG, "packed is not 256-byte aligned");
    if ((s = check_gemm_size(L, m)) != W4A8_OK) return s;
    W4A8_REQUIRE_PTR(xq);
    W4A8_REQUIRE_PTR(xsum);
    W4A8_REQUIRE_PTR(d);
    if ((s = check_device()) != W4A8_OK) return s;
    const w4a8::Geom g = geom_of(L);
    const uint8_t *pk = static_cast<const uint8_t *>(packed);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (byte_decoded(L))
        return launched(w4a8::launch_w8_partials(g, pk, m, xq, xsum, d, st),
                        "int8-weight partials launch");
    if (m == 1)
        return launched(w4a8::launch_gemv(g, pk, xq, nullptr, xsum, nullptr, d, st),
                        "gemv partials launch");
    return launched(w4a8::launch_gemm(g, pk, m, xq, nullptr, xsum, nullptr, d, st),
                    "gemm partials launch");
}

const char *w4a8_status_string(w4a8_status s) {
    switch (s) {
    case W4A8_OK: return "ok";
    case W4A8_ERR_ARG: return "invalid argument";
    case W4A8_ERR_UNSUPPORTED: return "unsupported";
    case W4A8_ERR_DEVICE: return "no gfx950 device";
    case W4A8_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *w4a8_last_error(void) { return g_last_error; }

}  // extern "C"
