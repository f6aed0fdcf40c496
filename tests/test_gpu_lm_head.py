"""GPU parity of the greedy tail of a vocabulary head (w4a8_lm_head_argmax) against the oracle.

Acceptance.  The cap c * tanh(y / c) has slope at most 1, so a logit inherits the linear's bound
(|err| <= 1e-4 T on y); 1e-5 |logit| covers the fp32 division, tanh and product.  The token is a
decision taken on the GPU's own fp32 logits: it must be the smallest index of their largest value
(bit-exact, checked on the host from the returned logits), `value` must be that logit's bits, and
the token must be a valid greedy choice for the oracle, whose logit it may trail by no more than
the two elements' error bounds."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bit_group_quantized_act_amd import synth
from _util import to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL_L2_MAX_LOGITS = 2e-5


def _w4a8():
    from bit_group_quantized_act_amd import w4a8
    w4a8.load()
    return w4a8


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _pack(L):
    w = _w4a8()
    cfg = L["cfg"]
    return w.pack(to_dev(L["codes"]), to_dev(L["scales"]), cfg.fmt, cfg.group,
                  bias=to_dev(L["bias"]), codebook=to_dev(L["codebook"]))


def _run(L, cap, x=None, work=None):
    w = _w4a8()
    cfg = L["cfg"]
    lay, packed = _pack(L)
    ng = cfg.k // cfg.group
    prep_out = (torch.empty((1, cfg.k), dtype=torch.int8, device="cuda:0"),
                torch.empty((ng, 1), dtype=torch.float32, device="cuda:0"),
                torch.empty((ng, 1), dtype=torch.int32, device="cuda:0"))
    xx = L["x"] if x is None else x
    logits, token, value = w.lm_head_argmax(lay, packed, to_dev(xx.reshape(-1)), cap,
                                            cfg.hadamard, work=work, prep_out=prep_out)
    torch.cuda.synchronize()
    return dict(logits=logits.cpu().numpy(), token=int(token.cpu().numpy()[0]),
                value=value.cpu().numpy()[0], xq=prep_out[0].cpu().numpy(),
                xs=prep_out[1].cpu().numpy().T.copy(), xsum=prep_out[2].cpu().numpy().T.copy())


def _oracle(L, cap, x=None, rows=None):
    cfg = L["cfg"]
    xx = L["x"] if x is None else x
    xq, xs, xsum = oracle.prep(xx.reshape(1, -1), cfg.group, cfg.hadamard)
    sel = (lambda a: a) if rows is None else (lambda a: None if a is None else a[rows])
    y, t = oracle.linear(cfg.fmt, sel(L["codes"]), sel(L["scales"]), xq, xs, xsum, cfg.group,
                         bias_f16=sel(L["bias"]), codebook=sel(L["codebook"]))
    logits, token, value = oracle.softcap_argmax(y[0], cap)
    return dict(logits=logits, t=t[0], token=token, value=value, xq=xq, xs=xs, xsum=xsum)


def _tol(ref):
    return 1e-4 * ref["t"] + 1e-5 * np.abs(ref["logits"])


def check_logits(got, ref, what=""):
    lg = np.asarray(got, dtype=np.float64)
    lr = ref["logits"]
    err = np.abs(lg - lr)
    nrm = np.linalg.norm(lr)
    rel = np.linalg.norm(lg - lr) / nrm if nrm > 0 else np.linalg.norm(lg - lr)
    bad = err > _tol(ref)
    assert rel <= REL_L2_MAX_LOGITS, f"{what}: relative L2 error {rel:.3e}"
    assert not bad.any(), f"{what}: {int(bad.sum())} logits outside the bound"


def check_token(got, ref, what=""):
    """The GPU's decision on its own logits (exact), and its validity for the oracle."""
    lg = got["logits"]
    t = got["token"]
    assert t == int(np.argmax(lg)), f"{what}: token {t}, first maximum at {int(np.argmax(lg))}"
    assert _bits(got["value"]) == _bits(lg[t]), f"{what}: value is not the token's logit"
    a = int(ref["token"])
    tol = _tol(ref)
    assert ref["logits"][t] >= ref["logits"][a] - (tol[t] + tol[a]), (
        f"{what}: token {t} trails the oracle's {a} by more than the error bounds")


def _check_all(L, cap, what):
    got = _run(L, cap)
    ref = _oracle(L, cap)
    assert np.array_equal(got["xq"], ref["xq"]), f"{what}: xq differs"
    assert np.array_equal(_bits(got["xs"]), _bits(ref["xs"])), f"{what}: xs differs"
    assert np.array_equal(got["xsum"], ref["xsum"]), f"{what}: xsum differs"
    check_logits(got["logits"], ref, what)
    check_token(got, ref, what)
    return got, ref


# the vocabulary head's shape scaled down (k 1536, g 64, symmetric), its ragged and rotated
# variants, the other two weight formats, and one wavefront-count switch (k 256: 4 waves)
CASES = [
    ("C5a", dict(n=4096), 0.0),
    ("C5a", dict(n=4096), 30.0),
    ("C5a", dict(n=1000), 30.0),
    ("C5a", dict(n=65), 0.0),
    ("C5a", dict(n=1), 30.0),
    ("C4", dict(m=1, n=2112, k=1536), 30.0),
    ("C3a", dict(m=1, n=1280, k=640), 15.0),
    ("C1", dict(n=300, k=256), 50.0),
    ("C1", dict(n=640, k=1024, group=128), 0.0),
    ("C1", dict(n=200, k=1 << 20), 30.0),        # the largest k: past the fused bound
]


@pytest.mark.parametrize("name,over,cap", CASES,
                         ids=[f"{c}-{'-'.join(f'{k}{v}' for k, v in o.items())}-cap{cap:g}"
                              for c, o, cap in CASES])
def test_lm_head_argmax_parity(name, over, cap):
    L = synth.make(name, full_range=True, **over)
    cfg = L["cfg"]
    print(f"lm_head {name} {over} cap={cap} n={cfg.n} k={cfg.k} fmt={cfg.fmt} "
          f"had={cfg.hadamard}", flush=True)
    _check_all(L, cap, f"{name} {over} cap {cap}")


def test_lm_head_uncapped_logits_are_the_gemv_output():
    # cap 0: the logits are the linear's output; the same GEMV arithmetic gives the same values
    w = _w4a8()
    L = synth.make("C5a", n=4096, full_range=True)
    got = _run(L, 0.0)
    lay, packed = _pack(L)
    xq, xs, xsum = w.prep(to_dev(L["x"]), L["cfg"].group, 0)
    y = w.gemv(lay, packed, xq, xs, xsum)
    torch.cuda.synchronize()
    assert np.array_equal(got["logits"], y.cpu().numpy())


def _dup_rows(L, src, dst):
    """Copy row src of the packed-by-row weights into each row of dst (all formats)."""
    for key in ("codes", "scales", "bias", "codebook"):
        a = L[key]
        if a is not None:
            a = a.copy()
            a[dst] = a[src]
            L[key] = a


def test_lm_head_ties_take_the_smallest_index():
    # the largest row copied to earlier and later rows, in other workgroups and in the ragged tail
    # (n = 1000): identical rows give identical logits, and the smallest index must win
    L = synth.make("C5a", n=1000, full_range=True)
    ref0 = _oracle(L, 30.0)
    lg = np.sort(ref0["logits"])
    a = int(ref0["token"])
    tol = _tol(ref0)
    assert lg[-1] - lg[-2] > 4 * tol.max(), "seeded case has a near tie"
    dst = sorted({a // 2, a // 2 + 1, 999, 998, (a + 500) % 1000} - {a})
    _dup_rows(L, a, dst)
    got = _run(L, 30.0)
    tied = [a] + dst
    vals = got["logits"][tied]
    assert np.all(_bits(vals) == _bits(vals[0])), "identical rows gave different logits"
    assert got["token"] == min(tied)
    check_token(got, _oracle(L, 30.0), "ties")


def test_lm_head_saturated_cap_ties():
    # a cap far below |y|: tanh rounds to 1 in fp32 on many rows, so many logits equal the cap;
    # the token must be the first of them
    L = synth.make("C5a", n=4096, full_range=True)
    y = _oracle(L, 0.0)["logits"]
    cap = float(np.percentile(np.abs(y), 50)) / 40.0
    got = _run(L, cap)
    ref = _oracle(L, cap)
    check_logits(got["logits"], ref, "saturated")
    check_token(got, ref, "saturated")
    assert int((got["logits"] == got["logits"][got["token"]]).sum()) > 100


def test_lm_head_all_negative_logits():
    # x >= 0 and every symmetric code negative: every logit is negative, so the key order of
    # negative floats decides the token
    L = synth.make("C5a", n=2048, full_range=True)
    r = np.random.default_rng(5)
    lo = r.integers(8, 16, size=L["codes"].shape, dtype=np.uint8)
    hi = r.integers(8, 16, size=L["codes"].shape, dtype=np.uint8)
    L["codes"] = (lo | (hi << 4)).astype(np.uint8)
    L["x"] = np.abs(L["x"])
    got, ref = _check_all(L, 30.0, "negative")
    assert (got["logits"] < 0).all()


def test_lm_head_zero_activation_gives_token_zero():
    L = synth.make("C5a", n=640, full_range=True)
    x = np.zeros_like(L["x"])
    got = _run(L, 30.0, x=x)
    assert not got["logits"].any()
    assert got["token"] == 0 and _bits(got["value"]) == 0


def test_lm_head_work_buffer_contents_do_not_matter():
    # a work buffer filled with ones, then reused by a second call on another activation: every
    # panel's key is written before the reduction reads it, so both tokens are right
    w = _w4a8()
    L = synth.make("C5a", n=2048, full_range=True)
    work = torch.full((w.argmax_work_bytes(2048) // 8,), -1, dtype=torch.int64, device="cuda:0")
    got = _run(L, 30.0, work=work)
    check_token(got, _oracle(L, 30.0), "first call")
    x2 = -L["x"]
    got2 = _run(L, 30.0, x=x2, work=work)
    ref2 = _oracle(L, 30.0, x=x2)
    check_logits(got2["logits"], ref2, "second call")
    check_token(got2, ref2, "second call")
    assert got2["token"] != got["token"]


def test_lm_head_full_vocabulary(layer_cache):
    """The 262144-entry vocabulary head (k 1536, g 64): the token checked against all the GPU's
    logits, and the logits against the oracle on a seeded sample plus the GPU's 64 largest (if
    every logit is within its bound, the token is a valid greedy choice for the oracle)."""
    if "C5a" not in layer_cache:
        layer_cache["C5a"] = synth.make("C5a")
    L = layer_cache["C5a"]
    cfg = L["cfg"]
    cap = 30.0
    print(f"lm_head full: n={cfg.n} k={cfg.k}", flush=True)
    got = _run(L, cap)
    lg = got["logits"]
    t = got["token"]
    assert t == int(np.argmax(lg)) and _bits(got["value"]) == _bits(lg[t])
    top = np.argsort(-lg.astype(np.float64), kind="stable")[:64]
    rows = np.unique(np.concatenate([np.random.default_rng(17).choice(cfg.n, 2048,
                                                                      replace=False), top,
                                     [cfg.n - 1]]))
    ref = _oracle(L, cap, rows=rows)
    check_logits(lg[rows], ref, "full vocabulary")


def test_gemv_argmax_on_prepared_activations_same_bits():
    # w4a8_gemv_argmax on lm_head_argmax's own prepass outputs: the same kernels, the same bits;
    # five calls in a row on one work buffer, alternating two activations
    w = _w4a8()
    L = synth.make("C5a", n=3000, full_range=True)
    cfg = L["cfg"]
    lay, packed = _pack(L)
    ng = cfg.k // cfg.group
    work = w.argmax_work(lay, "cuda:0")
    runs = []
    for sign in (1.0, -1.0):
        po = (torch.empty((1, cfg.k), dtype=torch.int8, device="cuda:0"),
              torch.empty((ng, 1), dtype=torch.float32, device="cuda:0"),
              torch.empty((ng, 1), dtype=torch.int32, device="cuda:0"))
        lg, tk, vl = w.lm_head_argmax(lay, packed, to_dev(sign * L["x"].reshape(-1)), 30.0,
                                      work=work, prep_out=po)
        torch.cuda.synchronize()
        runs.append((po, lg.cpu().numpy(), int(tk.cpu()[0]), vl.cpu().numpy()[0]))
    assert runs[0][2] != runs[1][2]
    for i in range(5):
        po, lg_ref, tk_ref, vl_ref = runs[i % 2]
        lg, tk, vl = w.gemv_argmax(lay, packed, po[0], po[1], po[2], 30.0, work=work)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(lg.cpu().numpy()), _bits(lg_ref)), f"call {i}: logits"
        assert int(tk.cpu()[0]) == tk_ref, f"call {i}: token"
        assert _bits(vl.cpu().numpy()[0]) == _bits(vl_ref), f"call {i}: value"


def _row_scaled(L):
    """L with one scale (and bias) per row: the first group's, written into every group."""
    ng = L["scales"].shape[1]
    L = dict(L)
    L["row_scales"] = np.ascontiguousarray(L["scales"][:, 0])
    L["scales"] = np.repeat(L["row_scales"][:, None], ng, axis=1)
    L["row_bias"] = None
    if L["bias"] is not None:
        L["row_bias"] = np.ascontiguousarray(L["bias"][:, 0])
        L["bias"] = np.repeat(L["row_bias"][:, None], ng, axis=1)
    return L


@pytest.mark.parametrize("name,over", [("C5o", dict(n=640)), ("C5a", dict(n=1000)),
                                       ("C3a", dict(m=1, n=320, k=640))],
                         ids=["codebook-g128", "sym-g64-ragged", "affine-g64"])
def test_row_scale_packing_is_the_replicated_layout(name, over):
    # the row-scale view writes the same packed bytes as w4a8_pack_weights given the row's value
    # in every group (so every kernel computes the view's formula)
    w = _w4a8()
    L = synth.make(name, full_range=True, **over)
    if "row_scales" not in L:
        L = _row_scaled(L)
    cfg = L["cfg"]
    _, ref = _pack(L)
    _, got = w.pack_row_scale(to_dev(L["codes"]), to_dev(L["row_scales"]), cfg.fmt, cfg.group,
                              row_bias=to_dev(L["row_bias"]), codebook=to_dev(L["codebook"]))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref.cpu().numpy())


def _run_row_scaled(L, cap):
    w = _w4a8()
    cfg = L["cfg"]
    lay, packed = w.pack_row_scale(to_dev(L["codes"]), to_dev(L["row_scales"]), cfg.fmt,
                                   cfg.group, row_bias=to_dev(L["row_bias"]),
                                   codebook=to_dev(L["codebook"]))
    logits, token, value = w.lm_head_argmax(lay, packed, to_dev(L["x"].reshape(-1)), cap,
                                            cfg.hadamard)
    torch.cuda.synchronize()
    return dict(logits=logits.cpu().numpy(), token=int(token.cpu().numpy()[0]),
                value=value.cpu().numpy()[0])


@pytest.mark.parametrize("n,cap", [(4000, 30.0), (4096, 0.0)], ids=["ragged-cap30", "cap0"])
def test_orthogonal_head_greedy_tail(n, cap):
    # the orthogonal head: rotated activations, codebook weights, one scale per row seen as
    # K/128 groups, packed by the row-scale view; the oracle takes the scale in every group
    L = synth.make("C5o", n=n, full_range=True)
    got = _run_row_scaled(L, cap)
    ref = _oracle(L, cap)
    check_logits(got["logits"], ref, f"orthogonal n {n}")
    check_token(got, ref, f"orthogonal n {n}")


def test_orthogonal_head_full_vocabulary(layer_cache):
    """The 262144-entry orthogonal head (k 1536, rotation, codebook, one scale per row): the token
    against all the GPU's logits, the logits against the oracle on a sample and the top 64."""
    if "C5o" not in layer_cache:
        layer_cache["C5o"] = synth.make("C5o")
    L = layer_cache["C5o"]
    cfg = L["cfg"]
    print(f"orthogonal head full: n={cfg.n} k={cfg.k}", flush=True)
    got = _run_row_scaled(L, 30.0)
    lg = got["logits"]
    t = got["token"]
    assert t == int(np.argmax(lg)) and _bits(got["value"]) == _bits(lg[t])
    top = np.argsort(-lg.astype(np.float64), kind="stable")[:64]
    rows = np.unique(np.concatenate([np.random.default_rng(19).choice(cfg.n, 2048,
                                                                      replace=False), top,
                                     [cfg.n - 1]]))
    check_logits(lg[rows], _oracle(L, 30.0, rows=rows), "orthogonal full vocabulary")
