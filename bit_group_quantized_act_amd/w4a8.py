"""Python binding of libw4a8 (the C ABI in include/w4a8.h) over torch device tensors.

Argument marshalling only: every step runs in the library's HIP kernels.  torch supplies device
memory (outputs are allocated with torch unless passed in) and the current HIP stream.  If
``libw4a8.so`` has not been built, loading raises: there is no other implementation to fall back
to.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a8.so")

SYM, AFFINE, CODEBOOK, INT8, CQ2, CQ1, CQ3 = 0, 1, 2, 3, 4, 5, 6
# k per byte of canonical codes, and codebook entries per row
_K_PER_BYTE = {INT8: 1, CQ2: 4, CQ1: 8, CQ3: 1}
_CB_ENTRIES = {CODEBOOK: 16, CQ2: 4, CQ1: 2, CQ3: 8}
PANEL_ROWS = 64
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "no gfx950 device", 4: "HIP error"}

# Every exported symbol of the C ABI (the header's declarations, in order).
EXPORTS = ("w4a8_packed_layout", "w4a8_pack_weights", "w4a8_pack_weights_row_scale",
           "w4a8_prep", "w4a8_gemv", "w4a8_gemm",
           "w4a8_linear", "w4a8_linear_glu", "w4a8_gemm_glu", "w4a8_lm_head_argmax",
           "w4a8_lm_head_argmax_noalloc",
           "w4a8_gemv_argmax", "w4a8_prep_a16", "w4a8_linear_a16", "w4a8_gemm_a16",
           "w4a8_attn_layout_init", "w4a8_attn_pack_kv", "w4a8_attn_work_bytes",
           "w4a8_attn_prefill", "w4a8_debug_partials", "w4a8_status_string", "w4a8_last_error")
_NOT_STATUS = ("w4a8_attn_work_bytes", "w4a8_status_string", "w4a8_last_error")
ACT_SILU, ACT_GELU_TANH, ACT_GELU_ERF = 0, 1, 2


class Layout(ctypes.Structure):
    """Mirror of w4a8_layout."""
    _fields_ = [("format", ctypes.c_int32), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("group", ctypes.c_int32), ("n_pad", ctypes.c_int32),
                ("meta_bytes", ctypes.c_int32), ("bytes", ctypes.c_uint64),
                ("off_codes", ctypes.c_uint64), ("off_meta", ctypes.c_uint64),
                ("off_codebook", ctypes.c_uint64)]

    def __repr__(self):
        return ("Layout(format=%d, n=%d, k=%d, group=%d, n_pad=%d, bytes=%d)"
                % (self.format, self.n, self.k, self.group, self.n_pad, self.bytes))


class W4A8Error(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load libw4a8.so (built in-tree by build.build()); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() or "
                          "python bit_group_quantized_act_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32 = ctypes.c_void_p, ctypes.c_int32
    LP = ctypes.POINTER(Layout)
    lib.w4a8_packed_layout.argtypes = [i32, i32, i32, i32, LP]
    lib.w4a8_pack_weights.argtypes = [LP, P, P, P, P, P, P]
    lib.w4a8_pack_weights_row_scale.argtypes = [LP, P, P, P, P, P, P]
    lib.w4a8_prep.argtypes = [P, i32, i32, i32, i32, P, P, P, P]
    lib.w4a8_gemv.argtypes = [LP, P, P, P, P, P, P]
    lib.w4a8_gemm.argtypes = [LP, P, i32, P, P, P, P, P]
    lib.w4a8_linear.argtypes = [LP, P, i32, P, i32, P, P, P, P, P]
    lib.w4a8_linear_glu.argtypes = [LP, P, i32, P, i32, i32, P, P, P, P, P]
    lib.w4a8_gemm_glu.argtypes = [LP, P, i32, P, P, P, i32, P, P]
    u64 = ctypes.c_uint64
    lib.w4a8_lm_head_argmax.argtypes = [LP, P, P, i32, ctypes.c_float, P, P, P, P, P, P, P, u64,
                                        P]
    lib.w4a8_lm_head_argmax_noalloc.argtypes = [LP, P, P, i32, ctypes.c_float, P, P, P, P, P,
                                                P, P]
    lib.w4a8_gemv_argmax.argtypes = [LP, P, P, P, P, ctypes.c_float, P, P, P, P, u64, P]
    lib.w4a8_prep_a16.argtypes = [P, i32, i32, i32, P, P, P]
    lib.w4a8_linear_a16.argtypes = [LP, P, i32, P, P, P, P, P]
    lib.w4a8_gemm_a16.argtypes = [LP, P, i32, P, P, P, P]
    AP = ctypes.POINTER(AttnLayout)
    lib.w4a8_attn_layout_init.argtypes = [i32, i32, i32, AP]
    lib.w4a8_attn_pack_kv.argtypes = [AP, P, P, P, P, P, P, P]
    lib.w4a8_attn_prefill.argtypes = [AP, P, P, i32, i32, i32, i32, i32, ctypes.c_float, P, P, P,
                                      P, P, P, u64, P]
    lib.w4a8_attn_work_bytes.argtypes = [AP, i32, i32]
    lib.w4a8_attn_work_bytes.restype = u64
    lib.w4a8_debug_partials.argtypes = [LP, P, i32, P, P, P, P]
    for f in EXPORTS:
        if f not in _NOT_STATUS:
            getattr(lib, f).restype = ctypes.c_int
    lib.w4a8_status_string.argtypes = [ctypes.c_int]
    lib.w4a8_status_string.restype = ctypes.c_char_p
    lib.w4a8_last_error.argtypes = []
    lib.w4a8_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        raise W4A8Error(rc, what, load().w4a8_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def packed_layout(fmt: int, n: int, k: int, group: int) -> Layout:
    L = Layout()
    _check(load().w4a8_packed_layout(fmt, n, k, group, ctypes.byref(L)), "w4a8_packed_layout")
    return L


def pack(codes: torch.Tensor, scales: torch.Tensor, fmt: int, group: int, bias=None,
         codebook=None, out: torch.Tensor | None = None):
    """Repack canonical device weights.  Returns (layout, packed uint8 tensor of layout.bytes).

    codes uint8 [n, k/2] (low nibble = even k), int8 [n, k] for INT8, uint8 [n, k/4] for CQ2,
    [n, k/8] for CQ1 (bit i of byte b = index of k = 8b + i), [n, k] for CQ3 (low 3 bits);
    scales float16 [n, k/group]; bias float16 [n, k/group] (affine); codebook int8 [n, 16]
    (codebook), [n, 4] (CQ2), [n, 2] (CQ1) or [n, 8] (CQ3).
    """
    n, kh = codes.shape
    k = kh * _K_PER_BYTE.get(fmt, 2)
    L = packed_layout(fmt, n, k, group)
    _dev(codes, torch.int8 if fmt == INT8 else torch.uint8, "codes")
    _dev(scales, torch.float16, "scales", (n, k // group))
    if bias is not None:
        _dev(bias, torch.float16, "bias", (n, k // group))
    if codebook is not None:
        _dev(codebook, torch.int8, "codebook", (n, _CB_ENTRIES.get(fmt, 16)))
    if out is None:
        out = torch.empty(L.bytes, dtype=torch.uint8, device=codes.device)
    _dev(out, torch.uint8, "packed", (L.bytes,))
    _check(load().w4a8_pack_weights(ctypes.byref(L), _ptr(codes), _ptr(scales), _ptr(bias),
                                    _ptr(codebook), _ptr(out), _stream(codes.device)),
           "w4a8_pack_weights")
    return L, out


def pack_row_scale(codes: torch.Tensor, row_scales: torch.Tensor, fmt: int, group: int,
                   row_bias=None, codebook=None, out: torch.Tensor | None = None):
    """Repack weights with one scale (affine: and one bias) per output row, float16 [n], seen as
    the scale of each of the row's k/group groups (w4a8_pack_weights_row_scale)."""
    n, kh = codes.shape
    L = packed_layout(fmt, n, kh * _K_PER_BYTE.get(fmt, 2), group)
    _dev(codes, torch.int8 if fmt == INT8 else torch.uint8, "codes")
    _dev(row_scales, torch.float16, "row_scales", (n,))
    if row_bias is not None:
        _dev(row_bias, torch.float16, "row_bias", (n,))
    if codebook is not None:
        _dev(codebook, torch.int8, "codebook", (n, _CB_ENTRIES.get(fmt, 16)))
    if out is None:
        out = torch.empty(L.bytes, dtype=torch.uint8, device=codes.device)
    _dev(out, torch.uint8, "packed", (L.bytes,))
    _check(load().w4a8_pack_weights_row_scale(ctypes.byref(L), _ptr(codes), _ptr(row_scales),
                                              _ptr(row_bias), _ptr(codebook), _ptr(out),
                                              _stream(codes.device)),
           "w4a8_pack_weights_row_scale")
    return L, out


def prep(x: torch.Tensor, group: int, hadamard_block: int = 0, out=None):
    """Activation prepass on fp32 [m, k] (or [k]).

    Returns (xq int8 [m, k], xs fp32 [k/group, m], xsum int32 [k/group, m]); the scales and sums
    are group-major.  For a 1-D x: (xq [k], xs [k/group], xsum [k/group]).
    """
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    _dev(x2, torch.float32, "x")
    m, k = x2.shape
    ng = k // group if group else 0
    if out is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
        xs = torch.empty((ng, m), dtype=torch.float32, device=x.device)
        xsum = torch.empty((ng, m), dtype=torch.int32, device=x.device)
    else:
        xq, xs, xsum = out
    _check(load().w4a8_prep(_ptr(x2), m, k, group, hadamard_block, _ptr(xq), _ptr(xs),
                            _ptr(xsum), _stream(x.device)), "w4a8_prep")
    if squeeze:
        return xq[0], xs.reshape(ng), xsum.reshape(ng)
    return xq, xs, xsum


def gemv(L: Layout, packed: torch.Tensor, xq, xs, xsum, out=None) -> torch.Tensor:
    """Decode GEMV: one activation row -> fp32 [n]."""
    y = out if out is not None else torch.empty(L.n, dtype=torch.float32, device=packed.device)
    _check(load().w4a8_gemv(ctypes.byref(L), _ptr(packed), _ptr(xq), _ptr(xs), _ptr(xsum),
                            _ptr(y), _stream(packed.device)), "w4a8_gemv")
    return y


def gemm(L: Layout, packed: torch.Tensor, xq, xs, xsum, out=None) -> torch.Tensor:
    """Prefill GEMM: m activation rows (xq int8 [m, k], xs / xsum [k/group, m]) -> fp32 [m, n]."""
    m = xq.shape[0]
    y = out if out is not None else torch.empty((m, L.n), dtype=torch.float32,
                                                device=packed.device)
    _check(load().w4a8_gemm(ctypes.byref(L), _ptr(packed), m, _ptr(xq), _ptr(xs), _ptr(xsum),
                            _ptr(y), _stream(packed.device)), "w4a8_gemm")
    return y


def debug_partials(L: Layout, packed: torch.Tensor, xq, xsum) -> torch.Tensor:
    """Exact int32 partials D [m, n, k/group] from the GEMV (m == 1) or GEMM (m > 1) kernels."""
    xq2 = xq.unsqueeze(0) if xq.dim() == 1 else xq
    m = xq2.shape[0]
    d = torch.empty((m, L.n, L.k // L.group), dtype=torch.int32, device=packed.device)
    _check(load().w4a8_debug_partials(ctypes.byref(L), _ptr(packed), m, _ptr(xq2), _ptr(xsum),
                                      _ptr(d), _stream(packed.device)), "w4a8_debug_partials")
    return d


def linear(L: Layout, packed: torch.Tensor, x: torch.Tensor, hadamard_block: int = 0, out=None,
           prep_out=None):
    """The whole layer (w4a8_linear): fp32 activations [m, k] or [k] -> fp32 output [m, n] or [n].

    One kernel for a single row (the GEMV quantizes the row itself), prepass + GEMM otherwise.
    prep_out = (xq, xs, xsum) receives the prepass outputs (allocated if None).  Returns y, or
    (y, (xq, xs, xsum)) when prep_out is given.
    """
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    _dev(x2, torch.float32, "x")
    m, k = x2.shape
    if k != L.k:
        raise ValueError(f"x has k = {k}, the layout {L.k}")
    ng = k // L.group
    if prep_out is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
        xs = torch.empty((ng, m), dtype=torch.float32, device=x.device)
        xsum = torch.empty((ng, m), dtype=torch.int32, device=x.device)
    else:
        xq, xs, xsum = prep_out
    y = out if out is not None else torch.empty((m, L.n), dtype=torch.float32, device=x.device)
    _check(load().w4a8_linear(ctypes.byref(L), _ptr(packed), m, _ptr(x2), hadamard_block,
                              _ptr(xq), _ptr(xs), _ptr(xsum), _ptr(y), _stream(x.device)),
           "w4a8_linear")
    y = y[0] if (squeeze and out is None) else y
    return (y, (xq, xs, xsum)) if prep_out is not None else y


def linear_glu(L: Layout, packed: torch.Tensor, x: torch.Tensor, act: int = ACT_SILU,
               hadamard_block: int = 0, out=None, prep_out=None):
    """Gated output of a [gate; up] linear (w4a8_linear_glu): fp32 activations [m, k] or [k]
    -> act(gate) * up, fp32 [m, n/2] or [n/2].  L.n must be 2F with F a multiple of 64 (gate
    rows first).  prep_out as for linear."""
    squeeze = x.dim() == 1
    x2 = x.unsqueeze(0) if squeeze else x
    _dev(x2, torch.float32, "x")
    m, k = x2.shape
    if k != L.k:
        raise ValueError(f"x has k = {k}, the layout {L.k}")
    ng = k // L.group
    if prep_out is None:
        xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
        xs = torch.empty((ng, m), dtype=torch.float32, device=x.device)
        xsum = torch.empty((ng, m), dtype=torch.int32, device=x.device)
    else:
        xq, xs, xsum = prep_out
    y = out if out is not None else torch.empty((m, L.n // 2), dtype=torch.float32,
                                                device=x.device)
    _check(load().w4a8_linear_glu(ctypes.byref(L), _ptr(packed), m, _ptr(x2), hadamard_block,
                                  act, _ptr(xq), _ptr(xs), _ptr(xsum), _ptr(y),
                                  _stream(x.device)), "w4a8_linear_glu")
    y = y[0] if (squeeze and out is None) else y
    return (y, (xq, xs, xsum)) if prep_out is not None else y


def gemm_glu(L: Layout, packed: torch.Tensor, xq: torch.Tensor, xs: torch.Tensor,
             xsum: torch.Tensor, act: int = ACT_SILU, out=None):
    """Gated output from prepared activations (w4a8_gemm_glu): xq [m, k] (or [k]), xs and xsum
    [k/group, m] -> act(gate) * up, fp32 [m, n/2] (or [n/2])."""
    squeeze = xq.dim() == 1
    q2 = xq.unsqueeze(0) if squeeze else xq
    m = q2.shape[0]
    y = out if out is not None else torch.empty((m, L.n // 2), dtype=torch.float32,
                                                device=xq.device)
    _check(load().w4a8_gemm_glu(ctypes.byref(L), _ptr(packed), m, _ptr(q2), _ptr(xs),
                                _ptr(xsum), act, _ptr(y), _stream(xq.device)), "w4a8_gemm_glu")
    return y[0] if (squeeze and out is None) else y


def argmax_work_bytes(n: int) -> int:
    """Bytes of the greedy tail's work buffer for an n-row head: one 64-bit key per 64 rows."""
    return (n + 63) // 64 * 8


def argmax_work(L: Layout, device) -> torch.Tensor:
    """A work buffer for lm_head_argmax / gemv_argmax on layout L (contents need no setting)."""
    return torch.empty(argmax_work_bytes(L.n) // 8, dtype=torch.int64, device=device)


def _work_bytes(work: torch.Tensor) -> int:
    return work.numel() * work.element_size()


NOALLOC_MAX_N = 1 << 20     # W4A8_NOALLOC_MAX_N


def lm_head_argmax_noalloc(L: Layout, packed: torch.Tensor, x: torch.Tensor, out,
                           prep_out, softcap: float = 0.0, hadamard_block: int = 0):
    """w4a8_lm_head_argmax_noalloc: the greedy tail with the library's own key buffer.  Every
    buffer is the caller's: out = (logits [n], token int32 [1], value fp32 [1]), prep_out =
    (xq [1, k], xs [k/group, 1], xsum [k/group, 1]); nothing is allocated here or in the
    library.  Returns out."""
    x1 = x.reshape(-1)
    _dev(x1, torch.float32, "x")
    if x1.numel() != L.k:
        raise ValueError(f"x has {x1.numel()} values, the layout k = {L.k}")
    xq, xs, xsum = prep_out
    logits, token, value = out
    _check(load().w4a8_lm_head_argmax_noalloc(ctypes.byref(L), _ptr(packed), _ptr(x1),
                                              hadamard_block, float(softcap), _ptr(xq), _ptr(xs),
                                              _ptr(xsum), _ptr(logits), _ptr(token), _ptr(value),
                                              _stream(x.device)),
           "w4a8_lm_head_argmax_noalloc")
    return out


def lm_head_argmax(L: Layout, packed: torch.Tensor, x: torch.Tensor, softcap: float = 0.0,
                   hadamard_block: int = 0, out=None, work=None, prep_out=None):
    """Greedy tail of a vocabulary head (w4a8_lm_head_argmax) for one row x [k]: returns
    (logits [n], token int32 [1], value fp32 [1]) as device tensors.  out = (logits, token,
    value) and work (argmax_work) may be given to avoid allocations."""
    x1 = x.reshape(-1)
    _dev(x1, torch.float32, "x")
    if x1.numel() != L.k:
        raise ValueError(f"x has {x1.numel()} values, the layout k = {L.k}")
    ng = L.k // L.group
    if prep_out is None:
        xq = torch.empty((1, L.k), dtype=torch.int8, device=x.device)
        xs = torch.empty((ng, 1), dtype=torch.float32, device=x.device)
        xsum = torch.empty((ng, 1), dtype=torch.int32, device=x.device)
    else:
        xq, xs, xsum = prep_out
    if out is None:
        out = (torch.empty(L.n, dtype=torch.float32, device=x.device),
               torch.empty(1, dtype=torch.int32, device=x.device),
               torch.empty(1, dtype=torch.float32, device=x.device))
    logits, token, value = out
    if work is None:
        work = argmax_work(L, x.device)
    _check(load().w4a8_lm_head_argmax(ctypes.byref(L), _ptr(packed), _ptr(x1), hadamard_block,
                                      float(softcap), _ptr(xq), _ptr(xs), _ptr(xsum),
                                      _ptr(logits), _ptr(token), _ptr(value), _ptr(work),
                                      _work_bytes(work), _stream(x.device)),
           "w4a8_lm_head_argmax")
    return logits, token, value


def gemv_argmax(L: Layout, packed: torch.Tensor, xq, xs, xsum, softcap: float = 0.0, out=None,
                work=None):
    """The GEMV + greedy tail of lm_head_argmax on prepared activations (w4a8_gemv_argmax).
    Returns (logits [n], token [1], value [1])."""
    if out is None:
        out = (torch.empty(L.n, dtype=torch.float32, device=packed.device),
               torch.empty(1, dtype=torch.int32, device=packed.device),
               torch.empty(1, dtype=torch.float32, device=packed.device))
    logits, token, value = out
    if work is None:
        work = argmax_work(L, packed.device)
    _check(load().w4a8_gemv_argmax(ctypes.byref(L), _ptr(packed), _ptr(xq), _ptr(xs),
                                   _ptr(xsum), float(softcap), _ptr(logits), _ptr(token),
                                   _ptr(value), _ptr(work), _work_bytes(work),
                                   _stream(packed.device)), "w4a8_gemv_argmax")
    return logits, token, value


def a16_buffers(m: int, k: int, device):
    """The fp16-activation prepass outputs: xh binary16 [m, k] (interleaved), xsf fp32 [k/64, m]."""
    return (torch.empty((m, k), dtype=torch.float16, device=device),
            torch.empty((k // 64, m), dtype=torch.float32, device=device))


def prep_a16(x: torch.Tensor, out=None):
    """fp16-activation prepass (w4a8_prep_a16) of x fp32 [m, k]: returns (xh, xsf)."""
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    _dev(x2, torch.float32, "x")
    m, k = x2.shape
    xh, xsf = out if out is not None else a16_buffers(m, k, x.device)
    _check(load().w4a8_prep_a16(_ptr(x2), m, k, 64, _ptr(xh), _ptr(xsf), _stream(x.device)),
           "w4a8_prep_a16")
    return xh, xsf


def linear_a16(L: Layout, packed: torch.Tensor, x: torch.Tensor, out=None, prep_out=None):
    """fp16-activation linear (w4a8_linear_a16): x fp32 [m, k] -> y fp32 [m, n]; with
    prep_out = (xh, xsf) also returns them."""
    x2 = x.unsqueeze(0) if x.dim() == 1 else x
    _dev(x2, torch.float32, "x")
    m = x2.shape[0]
    xh, xsf = prep_out if prep_out is not None else a16_buffers(m, L.k, x.device)
    y = out if out is not None else torch.empty((m, L.n), dtype=torch.float32, device=x.device)
    _check(load().w4a8_linear_a16(ctypes.byref(L), _ptr(packed), m, _ptr(x2), _ptr(xh),
                                  _ptr(xsf), _ptr(y), _stream(x.device)), "w4a8_linear_a16")
    return (y, (xh, xsf)) if prep_out is not None else y


def gemm_a16(L: Layout, packed: torch.Tensor, xh: torch.Tensor, xsf: torch.Tensor, out=None):
    """The fp16-activation GEMV / GEMM alone on prepared (xh, xsf) (w4a8_gemm_a16)."""
    m = xh.shape[0]
    y = out if out is not None else torch.empty((m, L.n), dtype=torch.float32,
                                                device=packed.device)
    _check(load().w4a8_gemm_a16(ctypes.byref(L), _ptr(packed), m, _ptr(xh), _ptr(xsf), _ptr(y),
                                _stream(packed.device)), "w4a8_gemm_a16")
    return y



class AttnLayout(ctypes.Structure):
    """w4a8_attn_layout: the packed int8 key/value cache of one attention layer."""
    _fields_ = [("nkvh", ctypes.c_int32), ("nkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("nblk", ctypes.c_int32), ("bytes", ctypes.c_uint64), ("off_kq", ctypes.c_uint64),
                ("off_sk", ctypes.c_uint64), ("off_pos", ctypes.c_uint64),
                ("off_vt", ctypes.c_uint64), ("off_sv", ctypes.c_uint64),
                ("off_vsum", ctypes.c_uint64)]


def attn_pack_kv(k8, ks, v8, vs, kvpos, out=None):
    """Pack a canonical int8 cache (k8 / v8 int8 [nkvh, nkv, d], ks / vs fp32 [nkvh, nkv, d/32],
    kvpos int32 [nkv], device tensors): returns (layout, packed uint8 tensor)."""
    nkvh, nkv, d = k8.shape
    AL = AttnLayout()
    _check(load().w4a8_attn_layout_init(nkvh, nkv, d, ctypes.byref(AL)), "w4a8_attn_layout_init")
    _dev(k8, torch.int8, "k8")
    _dev(v8, torch.int8, "v8", tuple(k8.shape))
    _dev(ks, torch.float32, "ks", (nkvh, nkv, d // 32))
    _dev(vs, torch.float32, "vs", (nkvh, nkv, d // 32))
    _dev(kvpos, torch.int32, "kvpos", (nkv,))
    if out is None:
        out = torch.empty(AL.bytes, dtype=torch.uint8, device=k8.device)
    _check(load().w4a8_attn_pack_kv(ctypes.byref(AL), _ptr(k8), _ptr(ks), _ptr(v8), _ptr(vs),
                                    _ptr(kvpos), _ptr(out), _stream(k8.device)),
           "w4a8_attn_pack_kv")
    return AL, out


def attn_prefill(AL: AttnLayout, packed, q, pos0: int, window: int = 0, sink: int = 0,
                 scale: float = 1.0, out=None, work=None):
    """Prefill attention of q fp32 [nh, nq, d] over the packed cache: returns (o unnormalized
    [nh, nq, d], m [nh, nq], l [nh, nq], q8 [nh, nq, d], sq [nh, nq])."""
    nh, nq, d = q.shape
    _dev(q, torch.float32, "q")
    dev = q.device
    if out is None:
        out = (torch.empty((nh, nq, d), dtype=torch.float32, device=dev),
               torch.empty((nh, nq), dtype=torch.float32, device=dev),
               torch.empty((nh, nq), dtype=torch.float32, device=dev),
               torch.empty((nh, nq, d), dtype=torch.int8, device=dev),
               torch.empty((nh, nq), dtype=torch.float32, device=dev))
    o, m, l, q8, sq = out
    need = load().w4a8_attn_work_bytes(ctypes.byref(AL), nh, nq)
    if work is None and need > 0:
        work = torch.empty(need // 4, dtype=torch.float32, device=dev)
    wb = 0 if work is None else work.numel() * work.element_size()
    _check(load().w4a8_attn_prefill(ctypes.byref(AL), _ptr(packed), _ptr(q), nh, nq, pos0, window,
                                    sink, float(scale), _ptr(q8), _ptr(sq), _ptr(o), _ptr(m),
                                    _ptr(l), _ptr(work), wb, _stream(dev)), "w4a8_attn_prefill")
    return o, m, l, q8, sq
