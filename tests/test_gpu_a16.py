"""GPU parity of the fp16-activation path (w4a8_prep_a16, w4a8_linear_a16, w4a8_gemm_a16)
against the oracle.

The prepass outputs are compared bit for bit: the halves (after undoing the documented
interleave) and the fp32 group sums, which the pages define by a fixed tree.  The output y must
meet the linear's bar: relative L2 error <= 1e-5 and |err| <= 1e-4 T per element, T the sum of
the magnitudes of the terms.  The GPU's products w_int * xh are exact in fp32 and its sums are
fp32, so the error is at most about (64 + K/64 + 3) * 2^-24 * T (8.8e-6 T at K = 5120)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bit_group_quantized_act_amd import synth
from _util import to_dev, check_y

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# element 8j + h of every 32-wide block holds input KORD[j][h] of the block
KORD = np.array([[4 * j, 4 * j + 2, 16 + 4 * j, 18 + 4 * j, 4 * j + 1, 4 * j + 3, 17 + 4 * j,
                  19 + 4 * j] for j in range(4)]).reshape(32)


def _w4a8():
    from bit_group_quantized_act_amd import w4a8
    w4a8.load()
    return w4a8


def natural_order(xh_inter: np.ndarray) -> np.ndarray:
    """Undo the interleave of the prepass's halves: [m, k] interleaved -> natural order."""
    m, k = xh_inter.shape
    blocks = xh_inter.reshape(m, k // 32, 32)
    out = np.empty_like(blocks)
    out[:, :, KORD] = blocks
    return out.reshape(m, k)


def _run(L, m_override=None):
    w = _w4a8()
    cfg = L["cfg"]
    lay, packed = w.pack(to_dev(L["codes"]), to_dev(L["scales"]), cfg.fmt, cfg.group,
                         bias=to_dev(L["bias"]), codebook=to_dev(L["codebook"]))
    x = to_dev(L["x"])
    bufs = w.a16_buffers(cfg.m, cfg.k, "cuda:0")
    y, (xh, xsf) = w.linear_a16(lay, packed, x, prep_out=bufs)
    torch.cuda.synchronize()
    return dict(y=y.cpu().numpy(), xh=natural_order(xh.cpu().numpy().view(np.uint16)),
                xsf=xsf.cpu().numpy().T.copy(), lay=lay, packed=packed, xh_dev=xh, xsf_dev=xsf)


def _oracle(L, cols=None):
    cfg = L["cfg"]
    xh, xsf = oracle.prep_a16(L["x"])
    sel = (lambda a: a) if cols is None else (lambda a: None if a is None else a[cols])
    y, t = oracle.linear_a16(cfg.fmt, sel(L["codes"]), sel(L["scales"]), xh, xsf, cfg.group,
                             bias_f16=sel(L["bias"]))
    return dict(y=y, t=t, xh=xh, xsf=xsf)


# one row (GEMV) and several (GEMM): ragged n (panel padding, a half-empty 128-channel tile),
# an odd group count (the last LDS stage holds one group), one group, ragged m tiles; GEMMs with
# k a multiple of 256 and fewer tiles than the CUs run every tile split over four workgroups
CASES = [
    ("C2a", dict(n=1000, k=2048)),
    ("C3a", dict(m=1, n=640, k=640)),
    ("C2a", dict(n=128, k=16384)),          # the fused prepass's largest row: 4 passes
    ("C3a", dict(m=1, n=100, k=8256)),      # 3 passes, the last one partly empty
    ("C1", dict(n=64, k=64)),
    ("C1", dict(n=320, k=1024, x_outliers=4)),
    ("C3a", dict(m=2, n=320, k=640)),
    ("C3a", dict(m=65, n=1000, k=192)),
    ("C3a", dict(m=130, n=384, k=1280)),
    ("C2a", dict(m=63, n=640, k=2048)),
    ("C5b", dict(m=64, n=1024, k=1536)),
    ("C3a", dict(m=3, n=64, k=64)),
    # more tiles than CUs: whole tiles and split tiles (one k quarter per wavefront) in one launch
    ("C3a", dict(m=64, n=34816, k=512)),
    # the largest k (2^20): one row past the fused bound (prepass + GEMV), and a one-tile GEMM
    # split over four workgroups
    ("C1", dict(n=64, k=1 << 20)),
    ("C3a", dict(m=2, n=64, k=1 << 20)),
]


@pytest.mark.parametrize("name,over", CASES,
                         ids=[f"{c}-{'-'.join(f'{k}{v}' for k, v in o.items())}"
                              for c, o in CASES])
def test_a16_parity(name, over):
    L = synth.make(name, full_range=True, **over)
    cfg = L["cfg"]
    print(f"a16 {name} {over} m={cfg.m} n={cfg.n} k={cfg.k} fmt={cfg.fmt}", flush=True)
    got = _run(L)
    ref = _oracle(L)
    assert np.array_equal(got["xh"], ref["xh"]), "halves differ"
    assert np.array_equal(got["xsf"].view(np.uint32), ref["xsf"].view(np.uint32)), \
        "group sums differ"
    check_y(got["y"], ref["y"], ref["t"], f"a16 {name} {over}")


def test_a16_gemm_on_prepared_activations_same_bits():
    w = _w4a8()
    for name, over in (("C3a", dict(m=65, n=1000, k=192)), ("C2a", dict(n=1000, k=2048))):
        L = synth.make(name, full_range=True, **over)
        got = _run(L)
        y2 = w.gemm_a16(got["lay"], got["packed"], got["xh_dev"], got["xsf_dev"])
        torch.cuda.synchronize()
        assert np.array_equal(got["y"].view(np.uint32),
                              y2.cpu().numpy().reshape(got["y"].shape).view(np.uint32))


def test_a16_group_sum_tree_on_the_gpu():
    # the hand-derived tree cases of the oracle's golden file, through the GPU prepass
    x = np.zeros((2, 128), np.float32)
    x[0, 0] = 16777216.0
    x[0, 8:64:8] = 1.0                     # c0 = 2^24, c1..c7 = 1: the tree gives 2^24 + 6
    x[1, 0] = 16777216.0
    x[1, 1:8] = 1.0                        # one octet: left to right gives 2^24
    x[:, 64:] = 1.0
    w = _w4a8()
    xh, xsf = w.prep_a16(to_dev(x))
    torch.cuda.synchronize()
    s = xsf.cpu().numpy()
    assert s[0, 0] == np.float32(16777222.0) and s[0, 1] == np.float32(16777216.0)
    assert np.all(s[1] == np.float32(64.0))


FULL = [("C3a", 384), ("C2a", None)]


@pytest.mark.parametrize("name,ncols", FULL, ids=[n for n, _ in FULL])
def test_a16_full_size_sampled(name, ncols, layer_cache):
    """The pages' 128-row gate_up prompt tile (C3a: 128 x 5120 x 34816, affine g64) on a seeded
    sample of output channels, and C2a's decode row whole."""
    key = name
    if key not in layer_cache:
        layer_cache[key] = synth.make(name)
    L = layer_cache[key]
    cfg = L["cfg"]
    print(f"a16 full {name}: m={cfg.m} n={cfg.n} k={cfg.k}", flush=True)
    got = _run(L)
    cols = None
    if ncols is not None:
        cols = np.sort(np.random.default_rng(23).choice(cfg.n, ncols, replace=False))
        cols[-1] = cfg.n - 1
    ref = _oracle(L, cols)
    assert np.array_equal(got["xh"], ref["xh"])
    assert np.array_equal(got["xsf"].view(np.uint32), ref["xsf"].view(np.uint32))
    yg = got["y"] if cols is None else got["y"][:, cols]
    check_y(yg, ref["y"], ref["t"], f"a16 full {name}")
