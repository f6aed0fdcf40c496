"""Host-side tests of the C ABI (no GPU needed): the library loads, exports every function the
header declares, computes packed layouts, and rejects invalid arguments before any device call.
"""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from bit_group_quantized_act_amd import w4a8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8.h")

ERR_ARG, ERR_UNSUPPORTED, ERR_DEVICE = 1, 2, 3


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="module")
def lib():
    return w4a8.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(w4a8_\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_binding_exports():
    assert tuple(_declared_functions()) == w4a8.EXPORTS


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", w4a8.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for s in range(5):
        assert lib.w4a8_status_string(s).decode() == w4a8.STATUS[s]
    assert lib.w4a8_status_string(99).decode() == "unknown status"


def test_layout_sizes():
    L = w4a8.packed_layout(w4a8.SYM, 16384, 2048, 64)
    assert (L.n_pad, L.meta_bytes) == (16384, 2)
    assert L.off_codes == 0 and L.off_meta == 16384 * 2048 // 2
    assert L.bytes == L.off_meta + 16384 * 32 * 2
    L = w4a8.packed_layout(w4a8.AFFINE, 34816, 5120, 64)
    assert L.meta_bytes == 4 and L.bytes == 34816 * 2560 + 34816 * 80 * 4
    L = w4a8.packed_layout(w4a8.CODEBOOK, 1000, 1536, 128)
    assert L.n_pad == 1024
    assert L.off_meta == 1024 * 768 and L.off_codebook == L.off_meta + 1024 * 12 * 2
    assert L.bytes == L.off_codebook + 1024 * 16
    for off in (L.off_meta, L.off_codebook, L.bytes):
        assert off % 256 == 0
    # metadata comes in blocks of 4 groups: 5 groups take 2 blocks (the last one padded)
    L = w4a8.packed_layout(w4a8.SYM, 64, 320, 64)
    assert L.off_meta == 64 * 160 and L.bytes == L.off_meta + 64 * 2 * 4 * 2


@pytest.mark.parametrize("args", [
    (7, 64, 64, 64), (-1, 64, 64, 64), (0, 64, 96, 64), (0, 64, 64, 32), (0, 0, 64, 64),
    (0, 64, 0, 64), (0, 64, 64 * 3, 128), (0, 1 << 25, 64, 64), (0, 64, (1 << 20) + 64, 64),
])
def test_layout_rejects(lib, args):
    L = w4a8.Layout()
    assert lib.w4a8_packed_layout(*args, ctypes.byref(L)) == ERR_ARG
    assert lib.w4a8_last_error().decode() != ""


def _fake(addr):
    # host-side validation never dereferences device pointers; these values are never launched
    return ctypes.c_void_p(addr)


def test_invalid_calls_are_rejected_on_the_host(lib):
    L = w4a8.packed_layout(w4a8.AFFINE, 128, 256, 64)
    LP = ctypes.byref(L)
    p, p16, p1 = _fake(1 << 20), _fake((1 << 20) + 16), _fake((1 << 20) + 1)
    # pack: missing bias (affine), misaligned packed, stray codebook, bad layout
    assert lib.w4a8_pack_weights(LP, p, p, None, None, p, None) == ERR_ARG
    assert lib.w4a8_pack_weights(LP, p, p, p, None, p16, None) == ERR_ARG
    assert lib.w4a8_pack_weights(LP, p, p, p, p, p, None) == ERR_ARG
    bad = w4a8.Layout.from_buffer_copy(L)
    bad.bytes += 1
    assert lib.w4a8_pack_weights(ctypes.byref(bad), p, p, p, None, p, None) == ERR_ARG
    assert "w4a8_packed_layout" in lib.w4a8_last_error().decode()
    assert lib.w4a8_pack_weights(None, p, p, p, None, p, None) == ERR_ARG
    # the row-scale view: the same checks
    assert lib.w4a8_pack_weights_row_scale(LP, p, p, None, None, p, None) == ERR_ARG
    assert lib.w4a8_pack_weights_row_scale(LP, p, p, p, None, p16, None) == ERR_ARG
    assert lib.w4a8_pack_weights_row_scale(LP, p, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_pack_weights_row_scale(LP, p, None, p, None, p, None) == ERR_ARG
    assert lib.w4a8_pack_weights_row_scale(None, p, p, p, None, p, None) == ERR_ARG
    # prep: m < 0, k % group, hadamard block, k % 128 with rotation, null and misaligned
    assert lib.w4a8_prep(p, -1, 256, 64, 0, p, p, p, None) == ERR_ARG
    assert lib.w4a8_prep(p, 2, 200, 64, 0, p, p, p, None) == ERR_ARG
    assert lib.w4a8_prep(p, 2, 256, 64, 64, p, p, p, None) == ERR_ARG
    assert lib.w4a8_prep(p, 2, 320, 64, 128, p, p, p, None) == ERR_ARG
    assert lib.w4a8_prep(p, 2, 256, 96, 0, p, p, p, None) == ERR_ARG
    assert lib.w4a8_prep(None, 2, 256, 64, 0, p, p, p, None) == ERR_ARG
    assert lib.w4a8_prep(p, 2, 256, 64, 0, p1, p, p, None) == ERR_ARG
    assert lib.w4a8_prep(p, 1 << 30, 1 << 20, 64, 0, p, p, p, None) == ERR_UNSUPPORTED
    # m == 0 is a no-op that needs no pointers and no device
    assert lib.w4a8_prep(None, 0, 256, 64, 0, None, None, None, None) == 0
    assert lib.w4a8_gemm(LP, p, 0, None, None, None, None, None) == 0
    # gemv / gemm / partials
    assert lib.w4a8_gemv(LP, None, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_gemv(LP, p16, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_gemv(LP, p, p, p, p, p1, None) == ERR_ARG
    assert lib.w4a8_gemm(LP, p, -3, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_gemm(LP, p, 4, p, None, p, p, None) == ERR_ARG
    assert lib.w4a8_debug_partials(LP, p, 0, p, p, p, None) == ERR_ARG
    assert lib.w4a8_debug_partials(LP, p, 2, p, p, None, None) == ERR_ARG
    # linear: m < 0, bad rotation block, k % 128 with rotation, missing x / xq / y, misaligned
    assert lib.w4a8_linear(LP, p, -1, p, 0, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_linear(LP, p, 1, p, 64, p, p, p, p, None) == ERR_ARG
    L320 = w4a8.packed_layout(w4a8.SYM, 64, 320, 64)
    assert lib.w4a8_linear(ctypes.byref(L320), p, 1, p, 128, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_linear(LP, p, 1, None, 0, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_linear(LP, p, 1, p, 0, None, p, p, p, None) == ERR_ARG
    assert lib.w4a8_linear(LP, p, 3, p, 0, p, p, p, None, None) == ERR_ARG
    assert lib.w4a8_linear(LP, p16, 1, p, 0, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_linear(LP, p, 1, p1, 0, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_linear(LP, p, 0, None, 0, None, None, None, None, None) == 0
    # linear_glu: n not 2F with F % 64 == 0, act out of range, bad rotation block, m < 0,
    # missing x / y, a gate-to-up span past 2^31 bytes; m == 0 is a no-op
    silu = w4a8.ACT_SILU
    L192 = w4a8.packed_layout(w4a8.SYM, 192, 256, 64)
    assert lib.w4a8_linear_glu(ctypes.byref(L192), p, 1, p, 0, silu, p, p, p, p, None) == ERR_ARG
    assert "gate" in lib.w4a8_last_error().decode()
    assert lib.w4a8_linear_glu(LP, p, 1, p, 0, 3, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_linear_glu(LP, p, 1, p, 0, -1, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_linear_glu(LP, p, 1, p, 64, silu, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_linear_glu(LP, p, -1, p, 0, silu, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_linear_glu(LP, p, 2, None, 0, silu, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_linear_glu(LP, p, 2, p, 0, silu, p, p, p, None, None) == ERR_ARG
    big = w4a8.packed_layout(w4a8.SYM, 262144, 32768, 64)
    assert lib.w4a8_linear_glu(ctypes.byref(big), p, 1, p, 0, silu, p, p, p, p,
                               None) == ERR_UNSUPPORTED
    assert lib.w4a8_linear_glu(LP, p, 0, None, 0, silu, None, None, None, None, None) == 0
    # gemm_glu: the same split / act / span checks, missing activations, m == 0 a no-op
    assert lib.w4a8_gemm_glu(ctypes.byref(L192), p, 2, p, p, p, silu, p, None) == ERR_ARG
    assert lib.w4a8_gemm_glu(LP, p, 2, p, p, p, 7, p, None) == ERR_ARG
    assert lib.w4a8_gemm_glu(LP, p, 2, None, p, p, silu, p, None) == ERR_ARG
    assert lib.w4a8_gemm_glu(LP, p, 2, p, p, p, silu, None, None) == ERR_ARG
    assert lib.w4a8_gemm_glu(LP, p16, 2, p, p, p, silu, p, None) == ERR_ARG
    assert lib.w4a8_gemm_glu(ctypes.byref(big), p, 2, p, p, p, silu, p, None) == ERR_UNSUPPORTED
    assert lib.w4a8_gemm_glu(LP, p, 0, None, None, None, silu, None, None) == 0
    # lm_head_argmax: softcap negative / not finite, missing token / value / work, misaligned
    # or too small work (n = 128: two 64-row panels, 16 bytes), bad rotation block
    f = ctypes.c_float
    wb = w4a8.argmax_work_bytes(L.n)
    assert wb == 16
    assert lib.w4a8_lm_head_argmax(LP, p, p, 0, f(-1.0), p, p, p, p, p, p, p, wb, None) == ERR_ARG
    assert lib.w4a8_lm_head_argmax(LP, p, p, 0, f(float("inf")), p, p, p, p, p, p, p, wb,
                                   None) == ERR_ARG
    assert lib.w4a8_lm_head_argmax(LP, p, p, 0, f(0.0), p, p, p, p, None, p, p, wb,
                                   None) == ERR_ARG
    assert lib.w4a8_lm_head_argmax(LP, p, p, 0, f(0.0), p, p, p, p, p, None, p, wb,
                                   None) == ERR_ARG
    assert lib.w4a8_lm_head_argmax(LP, p, p, 0, f(0.0), p, p, p, p, p, p, None, wb,
                                   None) == ERR_ARG
    assert lib.w4a8_lm_head_argmax(LP, p, p, 0, f(0.0), p, p, p, p, p, p, _fake((1 << 20) + 4),
                                   wb, None) == ERR_ARG
    assert lib.w4a8_lm_head_argmax(LP, p, p, 0, f(0.0), p, p, p, p, p, p, p, wb - 8,
                                   None) == ERR_ARG
    assert "work has 8 bytes" in lib.w4a8_last_error().decode()
    assert lib.w4a8_lm_head_argmax(LP, p, p, 64, f(0.0), p, p, p, p, p, p, p, wb, None) == ERR_ARG
    assert lib.w4a8_lm_head_argmax(LP, p, None, 0, f(30.0), p, p, p, p, p, p, p, wb,
                                   None) == ERR_ARG
    assert lib.w4a8_gemv_argmax(LP, p, p, p, p, f(-0.5), p, p, p, p, wb, None) == ERR_ARG
    assert lib.w4a8_gemv_argmax(LP, p, p, p, p, f(float("nan")), p, p, p, p, wb, None) == ERR_ARG
    assert lib.w4a8_gemv_argmax(LP, p, p, p, p, f(0.0), p, p, p, None, wb, None) == ERR_ARG
    assert lib.w4a8_gemv_argmax(LP, p, p, p, p, f(0.0), p, p, p, p, 0, None) == ERR_ARG
    assert lib.w4a8_gemv_argmax(LP, p, None, p, p, f(0.0), p, p, p, p, wb, None) == ERR_ARG
    assert lib.w4a8_gemv_argmax(LP, p, p, p, p, f(0.0), None, p, p, p, wb, None) == ERR_ARG
    assert lib.w4a8_gemv_argmax(LP, p1, p, p, p, f(0.0), p, p, p, p, wb, None) == ERR_ARG
    # fp16-activation path: group must be 64, k a multiple of 64, SYM / AFFINE only, sizes
    assert lib.w4a8_prep_a16(p, 2, 256, 128, p, p, None) == ERR_ARG
    assert lib.w4a8_prep_a16(p, 2, 200, 64, p, p, None) == ERR_ARG
    assert lib.w4a8_prep_a16(p, -1, 256, 64, p, p, None) == ERR_ARG
    assert lib.w4a8_prep_a16(None, 2, 256, 64, p, p, None) == ERR_ARG
    assert lib.w4a8_prep_a16(p, 2, 256, 64, p1, p, None) == ERR_ARG
    assert lib.w4a8_prep_a16(p, 1 << 20, 1 << 20, 64, p, p, None) == ERR_UNSUPPORTED
    assert lib.w4a8_prep_a16(None, 0, 256, 64, None, None, None) == 0
    assert lib.w4a8_linear_a16(LP, p, 2, p, p, p, None, None) == ERR_ARG          # y NULL
    assert lib.w4a8_linear_a16(LP, p16, 2, p, p, p, p, None) == ERR_ARG           # packed
    assert lib.w4a8_gemm_a16(LP, p, 2, None, p, p, None) == ERR_ARG
    assert lib.w4a8_gemm_a16(LP, p, -2, p, p, p, None) == ERR_ARG
    assert lib.w4a8_gemm_a16(LP, p, 0, None, None, None, None) == 0
    cbl = w4a8.packed_layout(w4a8.CODEBOOK, 128, 256, 64)
    assert lib.w4a8_linear_a16(ctypes.byref(cbl), p, 2, p, p, p, p, None) == ERR_UNSUPPORTED
    g128 = w4a8.packed_layout(w4a8.SYM, 128, 256, 128)
    assert lib.w4a8_gemm_a16(ctypes.byref(g128), p, 2, p, p, p, None) == ERR_ARG
    # int8 weights: one byte per weight in the layout; the 4-bit-only entry points refuse them
    L8 = w4a8.packed_layout(w4a8.INT8, 100, 256, 64)
    L4 = w4a8.packed_layout(w4a8.SYM, 100, 256, 64)
    assert L8.off_meta == 128 * 256 and L4.off_meta == 128 * 128 and L8.meta_bytes == 2
    L2 = w4a8.packed_layout(w4a8.CQ2, 100, 256, 64)
    assert L2.off_meta == 128 * 64 and L2.off_codebook > L2.off_meta and L2.bytes % 256 == 0
    assert lib.w4a8_pack_weights(ctypes.byref(L2), p, p, None, None, p, None) == ERR_ARG   # codebook
    assert lib.w4a8_debug_partials(ctypes.byref(L2), p, 0, p, p, p, None) == ERR_ARG   # m < 1
    # 1- and 3-bit codebooks: 16 / 48 bytes per 128 k of a row, k padded to a multiple of 128
    L1 = w4a8.packed_layout(w4a8.CQ1, 100, 192, 64)
    L3 = w4a8.packed_layout(w4a8.CQ3, 100, 192, 64)
    assert L1.off_meta == 128 * 2 * 16 and L3.off_meta == 128 * 2 * 48
    assert L1.bytes - L1.off_codebook == 512 and L3.bytes - L3.off_codebook == 1024
    assert lib.w4a8_pack_weights(ctypes.byref(L3), p, p, None, None, p, None) == ERR_ARG
    assert lib.w4a8_gemv_argmax(ctypes.byref(L1), p, p, p, p, f(0.0), p, p, p, p, 16,
                                None) == ERR_UNSUPPORTED
    assert lib.w4a8_packed_layout(7, 100, 256, 64, ctypes.byref(L1)) == ERR_ARG
    L8P = ctypes.byref(L8)
    assert lib.w4a8_gemm_glu(ctypes.byref(w4a8.packed_layout(w4a8.INT8, 128, 256, 64)), p, 2, p,
                             p, p, silu, p, None) == ERR_UNSUPPORTED
    assert lib.w4a8_gemv_argmax(L8P, p, p, p, p, f(0.0), p, p, p, p, 16, None) == ERR_UNSUPPORTED
    assert lib.w4a8_debug_partials(L8P, p, 2, p, p, None, None) == ERR_ARG     # no d
    assert lib.w4a8_gemm_a16(L8P, p, 2, p, p, p, None) == ERR_UNSUPPORTED
    assert lib.w4a8_gemm(ctypes.byref(w4a8.packed_layout(w4a8.INT8, 64, 1 << 20, 64)), p, 4096,
                         p, p, p, p, None) == ERR_UNSUPPORTED                # m * k above 2^31
    # attention: layout limits, a forged layout, heads, negative arguments, scale, work size
    AL = w4a8.AttnLayout()
    assert lib.w4a8_attn_layout_init(2, 100, 96, ctypes.byref(AL)) == ERR_ARG
    assert lib.w4a8_attn_layout_init(0, 100, 64, ctypes.byref(AL)) == ERR_ARG
    assert lib.w4a8_attn_layout_init(2, 0, 64, ctypes.byref(AL)) == ERR_ARG
    assert lib.w4a8_attn_layout_init(2, 1000, 256, ctypes.byref(AL)) == 0
    assert AL.nblk == 16 and AL.bytes % 256 == 0 and AL.off_vsum > AL.off_sv > AL.off_vt
    ALP = ctypes.byref(AL)
    forged = w4a8.AttnLayout.from_buffer_copy(AL)
    forged.off_vt += 256
    assert lib.w4a8_attn_pack_kv(ctypes.byref(forged), p, p, p, p, p, p, None) == ERR_ARG
    assert lib.w4a8_attn_pack_kv(ALP, p, p, p, p, None, p, None) == ERR_ARG
    assert lib.w4a8_attn_pack_kv(ALP, p, p, p, p, p, p16, None) == ERR_ARG
    f = ctypes.c_float
    wb = lib.w4a8_attn_work_bytes(ALP, 8, 256)
    assert wb > 0 and lib.w4a8_attn_work_bytes(ALP, 8, 0) == 0
    args = lambda **kw: [kw.get(k, v) for k, v in (
        ("AL", ALP), ("packed", p), ("q", p), ("nh", 8), ("nq", 256), ("pos0", 1000),
        ("window", 0), ("sink", 0), ("scale", f(0.0625)), ("q8", p), ("sq", p), ("o", p),
        ("m", p), ("l", p), ("work", p), ("wb", wb), ("stream", None))]
    assert lib.w4a8_attn_prefill(*args(nh=7)) == ERR_ARG                 # not a multiple of 2
    assert lib.w4a8_attn_prefill(*args(nq=-1)) == ERR_ARG
    assert lib.w4a8_attn_prefill(*args(window=-5)) == ERR_ARG
    assert lib.w4a8_attn_prefill(*args(scale=f(0.0))) == ERR_ARG
    assert lib.w4a8_attn_prefill(*args(scale=f(float("nan")))) == ERR_ARG
    assert lib.w4a8_attn_prefill(*args(wb=wb - 4)) == ERR_ARG
    assert lib.w4a8_attn_prefill(*args(o=None)) == ERR_ARG
    assert lib.w4a8_attn_prefill(*args(q=p1)) == ERR_ARG
    assert lib.w4a8_attn_prefill(*args(nq=0, q=None, o=None)) == 0

@pytest.mark.skipif(_gpu_visible(), reason="checks the no-device path; would launch on a GPU")
def test_valid_calls_without_a_device_report_device_error(lib):
    L = w4a8.packed_layout(w4a8.SYM, 128, 256, 64)
    p = _fake(1 << 20)
    assert lib.w4a8_gemv(ctypes.byref(L), p, p, p, p, p, None) == ERR_DEVICE
    assert lib.w4a8_pack_weights_row_scale(ctypes.byref(L), p, p, None, None, p,
                                           None) == ERR_DEVICE
    assert lib.w4a8_prep(p, 2, 256, 64, 0, p, p, p, None) == ERR_DEVICE
    assert lib.w4a8_linear(ctypes.byref(L), p, 1, p, 0, p, p, p, p, None) == ERR_DEVICE
    assert lib.w4a8_linear_glu(ctypes.byref(L), p, 2, p, 0, w4a8.ACT_GELU_TANH, p, p, p, p,
                               None) == ERR_DEVICE
    assert lib.w4a8_lm_head_argmax(ctypes.byref(L), p, p, 0, ctypes.c_float(30.0), p, p, p, p,
                                   p, p, p, 16, None) == ERR_DEVICE
    assert lib.w4a8_gemv_argmax(ctypes.byref(L), p, p, p, p, ctypes.c_float(0.0), p, p, p, p,
                                16, None) == ERR_DEVICE
    assert lib.w4a8_prep_a16(p, 2, 256, 64, p, p, None) == ERR_DEVICE
    AL = w4a8.AttnLayout()
    assert lib.w4a8_attn_layout_init(1, 64, 64, ctypes.byref(AL)) == 0
    assert lib.w4a8_attn_pack_kv(ctypes.byref(AL), p, p, p, p, p, p, None) == ERR_DEVICE
    assert lib.w4a8_linear_a16(ctypes.byref(L), p, 2, p, p, p, p, None) == ERR_DEVICE
    for fmt in (w4a8.INT8, w4a8.CQ2, w4a8.CQ1, w4a8.CQ3):     # the byte-decoded partials
        LB = w4a8.packed_layout(fmt, 128, 256, 64)
        assert lib.w4a8_debug_partials(ctypes.byref(LB), p, 3, p, p, p, None) == ERR_DEVICE
    assert lib.w4a8_last_error().decode() != ""


def test_build_rejects_gemm_scratch(tmp_path):
    """The build's guard: a GEMM kernel with a nonzero private segment (a spill) is an error."""
    from bit_group_quantized_act_amd import build
    asm = tmp_path / "k.s"
    asm.write_text(".amdhsa_kernel _ZN4w4a8_gemm_kernelILi0E\n  .amdhsa_private_segment_fixed_size 0\n"
                   ".end_amdhsa_kernel\n.amdhsa_kernel other_kernel\n"
                   "  .amdhsa_private_segment_fixed_size 64\n.end_amdhsa_kernel\n")
    build.check_no_scratch(str(asm), "gemm_kernel")          # only non-GEMM kernels spill: fine
    asm.write_text(".amdhsa_kernel _ZN4w4a8_gemm_kernelILi1E\n  .amdhsa_private_segment_fixed_size 48\n"
                   ".end_amdhsa_kernel\n")
    with pytest.raises(RuntimeError, match="scratch"):
        build.check_no_scratch(str(asm), "gemm_kernel")
