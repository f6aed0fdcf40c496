"""GPU parity of int8 weights (format 3, W8A8) and 2-, 1- and 3-bit codebook weights (formats 4, 5,
6: CQ2, CQ1, CQ3) through w4a8_linear / w4a8_gemv / w4a8_gemm against the oracle: the prepass
outputs and the int32 per-group partials (w4a8_debug_partials) bit-exact, y within the linear's
bar (relative L2 error <= 1e-5, |err| <= 1e-4 T per element)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bit_group_quantized_act_amd import synth
from _util import to_dev, check_y, oracle_layer

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _w4a8():
    from bit_group_quantized_act_amd import w4a8
    w4a8.load()
    return w4a8


def _run(L):
    w = _w4a8()
    cfg = L["cfg"]
    lay, packed = w.pack(to_dev(L["codes"]), to_dev(L["scales"]), cfg.fmt, cfg.group,
                         codebook=to_dev(L["codebook"]))
    ng = cfg.k // cfg.group
    po = (torch.empty((cfg.m, cfg.k), dtype=torch.int8, device="cuda:0"),
          torch.empty((ng, cfg.m), dtype=torch.float32, device="cuda:0"),
          torch.empty((ng, cfg.m), dtype=torch.int32, device="cuda:0"))
    y, (xq, xs, xsum) = w.linear(lay, packed, to_dev(L["x"]), cfg.hadamard, prep_out=po)
    torch.cuda.synchronize()
    return dict(y=y.cpu().numpy().reshape(cfg.m, cfg.n), xq=xq.cpu().numpy(),
                xs=xs.cpu().numpy().T.copy(), xsum=xsum.cpu().numpy().T.copy(), lay=lay,
                packed=packed, dev=(xq, xs, xsum))


# one row (GEMV) with both group widths and a rotated prepass; several rows (GEMM): ragged m and
# n (a half-empty 128-channel tile), an odd group count (a one-group last stage), one group; k
# an odd multiple of 64 (half of the bit-plane formats' last 128-k chunk is padding)
CASES = [
    ("C2a", dict(n=1000, k=2048)),
    ("C2a", dict(n=200, k=320)),
    ("C2a", dict(n=200, k=16384)),          # the fused prepass's largest row: 8 passes
    ("C4", dict(m=1, n=130, k=8320)),       # rotated, 5 passes, the last one partly empty
    ("C4", dict(m=1, n=320, k=1536)),
    ("C1", dict(n=64, k=64)),
    ("C3a", dict(m=65, n=1000, k=640)),
    ("C3a", dict(m=2, n=320, k=192)),
    ("C4", dict(m=130, n=384, k=1536)),
    ("C5b", dict(m=64, n=1024, k=1536)),
    ("C1", dict(m=3, n=64, k=64)),
    # more tiles than CUs: with the 64-group codebook formats the tiles of the last, partial
    # round run split over four workgroups (one k quarter per wavefront): 272 tiles (16 split,
    # four stages per quarter) and 516 (4 split, two stages per quarter, a 2-row last row block)
    ("C3a", dict(m=64, n=34816, k=512)),
    ("C3a", dict(m=130, n=22016, k=256)),
    ("C1", dict(m=2, n=64, k=1 << 20)),     # the largest k: one tile (split for the codebooks)
]


FORMATS = [synth.FMT_INT8, synth.FMT_CQ2, synth.FMT_CQ1, synth.FMT_CQ3]
FMT_IDS = ["int8", "cq2", "cq1", "cq3"]


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
@pytest.mark.parametrize("name,over", CASES,
                         ids=[f"{c}-{'-'.join(f'{k}{v}' for k, v in o.items())}"
                              for c, o in CASES])
def test_w8_parity(name, over, fmt):
    L = synth.make(name, full_range=True, fmt=fmt, **over)
    cfg = L["cfg"]
    print(f"fmt {fmt} {name} {over} m={cfg.m} n={cfg.n} k={cfg.k} g={cfg.group} "
          f"had={cfg.hadamard}",
          flush=True)
    got = _run(L)
    ref = oracle_layer(L)
    assert np.array_equal(got["xq"], ref["xq"])
    assert np.array_equal(got["xs"].view(np.uint32), ref["xs"].view(np.uint32))
    assert np.array_equal(got["xsum"], ref["xsum"])     # (written by the fused one-row kernel too)
    check_y(got["y"], ref["y"], ref["t"], f"w8 {name} {over}")
    # the int32 per-group dot products of the same GEMV / GEMM code, bit for bit
    w = _w4a8()
    xq, _, xsum = got["dev"]
    d = w.debug_partials(got["lay"], got["packed"], xq, xsum).cpu().numpy()
    dref = oracle.partials(cfg.fmt, L["codes"], ref["xq"], cfg.group, codebook=L["codebook"])
    assert np.array_equal(d, dref), f"partials differ at {np.argwhere(d != dref)[:5].tolist()}"


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_w8_gemv_gemm_entry_points_same_bits(fmt):
    # w4a8_gemv / w4a8_gemm on w4a8_linear's own prepass outputs run the same kernels
    w = _w4a8()
    for name, over in (("C2a", dict(n=1000, k=2048)), ("C3a", dict(m=65, n=1000, k=640))):
        L = synth.make(name, full_range=True, fmt=fmt, **over)
        got = _run(L)
        xq, xs, xsum = got["dev"]
        if L["cfg"].m == 1:
            y2 = w.gemv(got["lay"], got["packed"], xq[0], xs, xsum).cpu().numpy()[None, :]
        else:
            y2 = w.gemm(got["lay"], got["packed"], xq, xs, xsum).cpu().numpy()
        torch.cuda.synchronize()
        assert np.array_equal(got["y"].view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("fmt", FORMATS, ids=FMT_IDS)
def test_w8_full_size_prompt_tile(layer_cache, fmt):
    """C3a's 128 x 5120 x 34816 shape with int8 weights (Gaussian draws quantized per group) or
    1-, 2- or 3-bit codebook weights, on a seeded sample of output channels."""
    key = f"C3a-fmt{fmt}"
    if key not in layer_cache:
        layer_cache[key] = synth.make("C3a", fmt=fmt)
    L = layer_cache[key]
    cfg = L["cfg"]
    print(f"w8 full C3a: m={cfg.m} n={cfg.n} k={cfg.k}", flush=True)
    got = _run(L)
    cols = np.sort(np.random.default_rng(29).choice(cfg.n, 384, replace=False))
    cols[-1] = cfg.n - 1
    ref = oracle_layer(L, cols)
    check_y(got["y"][:, cols], ref["y"], ref["t"], "w8 full C3a")


def test_cq3_ignores_the_high_bits_of_its_codes():
    # the canonical 3-bit codes keep one index per byte; bits 3-7 are not part of it
    base = synth.make("C3a", full_range=True, fmt=synth.FMT_CQ3, m=3, n=200, k=320)
    noisy = dict(base)
    extra = np.random.default_rng(31).integers(0, 32, size=base["codes"].shape, dtype=np.uint8)
    noisy["codes"] = base["codes"] | (extra << 3)
    a, b = _run(base), _run(noisy)
    assert np.array_equal(a["y"].view(np.uint32), b["y"].view(np.uint32))
    ref = oracle_layer(noisy)
    check_y(b["y"], ref["y"], ref["t"], "cq3 high bits")


FULL_ROW = [(synth.FMT_INT8, 262144), (synth.FMT_CQ2, 262144), (synth.FMT_CQ1, 262080),
            (synth.FMT_CQ3, 262080)]


@pytest.mark.parametrize("fmt,n", FULL_ROW, ids=[f"{i}-n{n}" for i, (_, n) in
                                                  zip(FMT_IDS, FULL_ROW)])
def test_w8_full_size_decode_row(layer_cache, fmt, n):
    """C5a's one-row vocabulary shape (K = 1536): at this width several panels share a GEMV
    workgroup; n = 262080 (4095 panels) leaves the last workgroup partly empty.  A seeded sample
    of output channels and the last one."""
    key = f"C5a-fmt{fmt}-n{n}"
    if key not in layer_cache:
        layer_cache[key] = synth.make("C5a", full_range=True, fmt=fmt, n=n)
    L = layer_cache[key]
    cfg = L["cfg"]
    print(f"w8 full C5a: fmt={fmt} n={cfg.n} k={cfg.k}", flush=True)
    got = _run(L)
    cols = np.sort(np.random.default_rng(37).choice(cfg.n, 512, replace=False))
    cols[-1] = cfg.n - 1
    ref = oracle_layer(L, cols)
    check_y(got["y"][:, cols], ref["y"], ref["t"], "w8 full C5a")
