"""GPU parity of the gated output act(gate) * up (w4a8_linear_glu) against the oracle.

The packed linear is [gate; up] (n = 2F, gate rows first).  Acceptance, derived from the linear's
own bound (each fp32 linear output within 1e-4 of its term magnitude T): the oracle's bound term
tz = 1.2 |u| T_gate + |act(g)| T_up covers the propagated error (1.2 exceeds the slope of every
activation), and 1e-5 |z| the fp32 evaluation of the activation and the product, so per element
|z_gpu - z| <= 1e-4 tz + 1e-5 |z|; each factor contributes at most 1e-5 of relative L2 error, so
the relative L2 error of z is at most 2e-5.  The prepass outputs stay bit-exact."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bit_group_quantized_act_amd import synth
from _util import to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL_L2_MAX_GLU = 2e-5


def _w4a8():
    from bit_group_quantized_act_amd import w4a8
    w4a8.load()
    return w4a8


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def check_z(z_gpu, z_ref, tz, what=""):
    zg = np.asarray(z_gpu, dtype=np.float64).reshape(z_ref.shape)
    err = np.abs(zg - z_ref)
    nrm = np.linalg.norm(z_ref)
    rel = np.linalg.norm(zg - z_ref) / nrm if nrm > 0 else np.linalg.norm(zg - z_ref)
    bad = err > 1e-4 * tz + 1e-5 * np.abs(z_ref)
    assert rel <= REL_L2_MAX_GLU, f"{what}: relative L2 error {rel:.3e} > {REL_L2_MAX_GLU}"
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside the bound"


def _run_glu(L, act):
    w = _w4a8()
    cfg = L["cfg"]
    lay, packed = w.pack(to_dev(L["codes"]), to_dev(L["scales"]), cfg.fmt, cfg.group,
                         bias=to_dev(L["bias"]), codebook=to_dev(L["codebook"]))
    ng = cfg.k // cfg.group
    prep_out = (torch.empty((cfg.m, cfg.k), dtype=torch.int8, device="cuda:0"),
                torch.empty((ng, cfg.m), dtype=torch.float32, device="cuda:0"),
                torch.empty((ng, cfg.m), dtype=torch.int32, device="cuda:0"))
    z, (xq, xs, xsum) = w.linear_glu(lay, packed, to_dev(L["x"]), act, cfg.hadamard,
                                     prep_out=prep_out)
    torch.cuda.synchronize()
    return dict(z=z.cpu().numpy().reshape(cfg.m, cfg.n // 2), xq=xq.cpu().numpy(),
                xs=xs.cpu().numpy().T.copy(), xsum=xsum.cpu().numpy().T.copy())


def _oracle_glu(L, act, fcols=None):
    cfg = L["cfg"]
    f_n = cfg.n // 2
    xq, xs, xsum = oracle.prep(L["x"], cfg.group, cfg.hadamard)
    rows = None if fcols is None else np.concatenate([fcols, f_n + fcols])
    sel = (lambda a: a) if rows is None else (lambda a: None if a is None else a[rows])
    y, t = oracle.linear(cfg.fmt, sel(L["codes"]), sel(L["scales"]), xq, xs, xsum, cfg.group,
                         bias_f16=sel(L["bias"]), codebook=sel(L["codebook"]))
    z, tz = oracle.glu(act, y, t)
    return dict(z=z, tz=tz, xq=xq, xs=xs, xsum=xsum)


S, GT, GE = oracle.ACT_SILU, oracle.ACT_GELU_TANH, oracle.ACT_GELU_ERF
# one row: fused prepass + gated GEMV (rotation for C4; 2 activation quads per lane at k 4096);
# k 16448 exceeds the fused bound (prepass + gated GEMV); several rows: prepass + gated GEMM
GLU_CASES = [
    ("C1", dict(n=256), S),
    ("C2a", dict(n=640, k=4096), GT),
    ("C4", dict(m=1, n=384, k=1536), GE),
    ("C1", dict(n=640, k=1536), S),               # six metadata blocks: six wavefronts
    ("C3a", dict(m=1, n=1280, k=640), S),
    ("C1", dict(n=128, k=16448), GT),
    ("C3a", dict(m=65, n=1280, k=1280), S),
    ("C4", dict(m=200, n=384, k=1536), GT),
    ("C5b", dict(m=64, n=512, k=1536), GE),
    ("C1", dict(m=3, n=128, k=1024, group=128), S),
    # more tiles than CUs: whole gated tiles and split ones (gate and up halves of k) in one launch
    ("C3a", dict(m=64, n=34816, k=512), GE),
    ("C3a", dict(m=2, n=128, k=1 << 20), S),      # the largest k: one gated tile, split in two
]


@pytest.mark.parametrize("name,over,act", GLU_CASES,
                         ids=[f"{c}-{'-'.join(f'{k}{v}' for k, v in o.items())}-act{a}"
                              for c, o, a in GLU_CASES])
def test_glu_parity(name, over, act):
    L = synth.make(name, full_range=True, **over)
    cfg = L["cfg"]
    print(f"glu {name} {over} act={act} m={cfg.m} n={cfg.n} k={cfg.k} had={cfg.hadamard}",
          flush=True)
    got = _run_glu(L, act)
    ref = _oracle_glu(L, act)
    assert np.array_equal(got["xq"], ref["xq"]), "xq differs"
    assert np.array_equal(_bits(got["xs"]), _bits(ref["xs"])), "xs differs"
    assert np.array_equal(got["xsum"], ref["xsum"]), "xsum differs"
    check_z(got["z"], ref["z"], ref["tz"], f"glu {name} {over}")


@pytest.mark.parametrize("name,over,act", [("C2a", dict(n=640, k=4096), S),
                                            ("C4", dict(m=1, n=384, k=1536), GE),
                                            ("C3a", dict(m=65, n=1280, k=1280), GT)],
                         ids=["gemv-fused", "gemv-rot", "gemm"])
def test_glu_from_prepared_activations_same_bits(name, over, act):
    # w4a8_gemm_glu on w4a8_linear_glu's own prepass outputs: the same kernel arithmetic, so the
    # same bits (the decode row compares the fused kernel with prepass + gated GEMV)
    w = _w4a8()
    L = synth.make(name, full_range=True, **over)
    cfg = L["cfg"]
    lay, packed = w.pack(to_dev(L["codes"]), to_dev(L["scales"]), cfg.fmt, cfg.group,
                         bias=to_dev(L["bias"]), codebook=to_dev(L["codebook"]))
    z1, (xq, xs, xsum) = w.linear_glu(lay, packed, to_dev(L["x"]), act, cfg.hadamard,
                                      prep_out=tuple(torch.empty(s, dtype=d, device="cuda:0")
                                                     for s, d in (((cfg.m, cfg.k), torch.int8),
                                                                  ((cfg.k // cfg.group, cfg.m),
                                                                   torch.float32),
                                                                  ((cfg.k // cfg.group, cfg.m),
                                                                   torch.int32))))
    z2 = w.gemm_glu(lay, packed, xq, xs, xsum, act)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(z1.cpu().numpy().reshape(z2.shape)), _bits(z2.cpu().numpy()))


def test_glu_output_differs_from_the_other_activation():
    # the act argument reaches the kernel: silu and gelu outputs of one layer differ
    L = synth.make("C1", n=256, full_range=True)
    a = _run_glu(L, S)["z"]
    b = _run_glu(L, GT)["z"]
    assert not np.allclose(a, b, rtol=1e-3, atol=0)
    check_z(b, *[_oracle_glu(L, GT)[k] for k in ("z", "tz")], "gelu")


GLU_FULL = [("C2a", GT, None), ("C3a", S, 256)]


@pytest.mark.parametrize("name,act,ncols", GLU_FULL, ids=[f"{n}-act{a}" for n, a, _ in GLU_FULL])
def test_glu_full_size_sampled(name, act, ncols, layer_cache):
    """The benchmark's gated shapes: C2a's gate_up row (F = 8192) checked whole, C3a's 128 rows
    (F = 17408) on a seeded sample of output channels (the last included)."""
    if name not in layer_cache:
        layer_cache[name] = synth.make(name)
    L = layer_cache[name]
    cfg = L["cfg"]
    print(f"glu full {name}: m={cfg.m} n={cfg.n} k={cfg.k}", flush=True)
    got = _run_glu(L, act)
    f_n = cfg.n // 2
    fcols = None
    if ncols is not None:
        fcols = np.sort(np.random.default_rng(13).choice(f_n, ncols, replace=False))
        fcols[-1] = f_n - 1
    ref = _oracle_glu(L, act, fcols)
    assert np.array_equal(got["xq"], ref["xq"])
    assert np.array_equal(got["xsum"], ref["xsum"])
    zg = got["z"] if fcols is None else got["z"][:, fcols]
    check_z(zg, ref["z"], ref["tz"], name)
