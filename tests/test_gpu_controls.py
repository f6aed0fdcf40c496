"""Planted controls on the GPU: each test feeds the HIP path one corrupted but valid input on the
device and shows that the parity checks of the other GPU tests turn red on it, after the same
run without the corruption has passed them.  The kernels run as always (every input stays in its
documented range); only the data is wrong.

Source: "TensorFold PR #3215", sections "Checks" and "Contract" (a control whose group sums are
left at zero must fail the parity check; controls are red as planted).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bit_group_quantized_act_amd import synth
from _util import check_y, oracle_layer, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _w4a8():
    from bit_group_quantized_act_amd import w4a8
    w4a8.load()
    return w4a8


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _pack(L):
    cfg = L["cfg"]
    return _w4a8().pack(to_dev(L["codes"]), to_dev(L["scales"]), cfg.fmt, cfg.group,
                        bias=to_dev(L["bias"]), codebook=to_dev(L["codebook"]))


def _matmul(lay, packed, m, xq, xs, xsum):
    w = _w4a8()
    y = w.gemv(lay, packed, xq[0], xs, xsum) if m == 1 else w.gemm(lay, packed, xq, xs, xsum)
    torch.cuda.synchronize()
    return y.cpu().numpy().reshape(m, lay.n)


@pytest.mark.parametrize("m", [1, 65], ids=["gemv", "gemm"])
def test_zeroed_group_sums_turn_the_affine_check_red(m):
    """The affine format needs xsum twice (the u - 8 code recovery and the bias term): with the
    sums left at zero both the output tolerance and the bit-exact partials must fail."""
    L = synth.make("C3a", full_range=True, m=m, n=320, k=640)
    cfg = L["cfg"]
    assert cfg.fmt == synth.FMT_AFFINE
    print(f"control zero xsum: m={m} n={cfg.n} k={cfg.k}", flush=True)
    w = _w4a8()
    lay, packed = _pack(L)
    xq, xs, xsum = w.prep(to_dev(L["x"]), cfg.group, cfg.hadamard)
    ref = oracle_layer(L)
    dref = oracle.partials(cfg.fmt, L["codes"], ref["xq"], cfg.group)
    check_y(_matmul(lay, packed, m, xq, xs, xsum), ref["y"], ref["t"], "unplanted")
    assert np.array_equal(w.debug_partials(lay, packed, xq, xsum).cpu().numpy(), dref)
    zero = torch.zeros_like(xsum)
    assert np.abs(ref["xsum"]).max() > 0                   # the planted change is a change
    with pytest.raises(AssertionError):
        check_y(_matmul(lay, packed, m, xq, xs, zero), ref["y"], ref["t"], "zeroed xsum")
    d0 = w.debug_partials(lay, packed, xq, zero).cpu().numpy()
    torch.cuda.synchronize()
    assert not np.array_equal(d0, dref)


def test_one_ulp_on_an_activation_scale_turns_the_prepass_check_red():
    """xs is compared bit for bit: one ulp on one group's scale must fail that compare, while
    the output moves by far less than the fp32 tolerance (which alone would not see it)."""
    L = synth.make("C3a", full_range=True, m=65, n=320, k=640)
    cfg = L["cfg"]
    print(f"control xs + 1 ulp: m={cfg.m} n={cfg.n} k={cfg.k}", flush=True)
    w = _w4a8()
    lay, packed = _pack(L)
    xq, xs, xsum = w.prep(to_dev(L["x"]), cfg.group, cfg.hadamard)
    ref = oracle_layer(L)
    got = xs.cpu().numpy().T.copy()
    assert np.array_equal(_bits(got), _bits(ref["xs"]))   # unplanted: the same bits
    bumped = xs.clone()
    bumped.view(torch.int32)[3, 17] += 1                   # group 3 of row 17, one ulp up
    got_b = bumped.cpu().numpy().T.copy()
    assert not np.array_equal(_bits(got_b), _bits(ref["xs"]))
    y = _matmul(lay, packed, cfg.m, xq, xs, xsum)
    y_b = _matmul(lay, packed, cfg.m, xq, bumped, xsum)
    assert not np.array_equal(_bits(y_b[17]), _bits(y[17]))   # the kernel reads the scale
    assert np.array_equal(_bits(np.delete(y_b, 17, 0)), _bits(np.delete(y, 17, 0)))
    check_y(y_b, ref["y"], ref["t"], "xs + 1 ulp")       # inside the output tolerance


@pytest.mark.parametrize("m", [1, 65], ids=["gemv", "gemm"])
def test_skipped_rotation_turns_the_rotated_check_red(m):
    """A C4 layer (128-block Walsh-Hadamard rotation of the activations) run without the
    rotation: the codes and the output must both fail against the rotated oracle."""
    L = synth.make("C4", full_range=True, m=m, n=320, k=768)
    cfg = L["cfg"]
    assert cfg.hadamard == 128
    print(f"control no rotation: m={m} n={cfg.n} k={cfg.k}", flush=True)
    w = _w4a8()
    lay, packed = _pack(L)
    x = to_dev(L["x"])
    ref = oracle_layer(L)
    xq, xs, xsum = w.prep(x, cfg.group, 128)
    assert np.array_equal(xq.cpu().numpy(), ref["xq"])
    check_y(_matmul(lay, packed, m, xq, xs, xsum), ref["y"], ref["t"], "unplanted")
    xq0, xs0, xsum0 = w.prep(x, cfg.group, 0)
    torch.cuda.synchronize()
    assert not np.array_equal(xq0.cpu().numpy(), ref["xq"])
    with pytest.raises(AssertionError):
        check_y(_matmul(lay, packed, m, xq0, xs0, xsum0), ref["y"], ref["t"], "no rotation")
