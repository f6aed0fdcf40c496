"""GPU parity of the int8 prefill attention over a cached segment (w4a8_attn_pack_kv,
w4a8_attn_prefill) against the oracle's int8 method.

Bit-exact: the query codes and scales, and the requantized keys.  The running state: m within
2e-5 (1 + |m|) (fp32 logits against fp64), l within 1e-4 relative (fp32 exponentials summed),
and the normalized output O / l with relative L2 error <= 1e-4 over each case; per query row
<= 1e-3 for all but 0.1% of the rows and <= 4e-3 for every row.  Row bound: a code of the 8-bit
P can differ from the oracle's only where P' / sp lies within fp32 rounding of a half-integer,
and one such difference moves a row's output O / l by sp * v / l, at most 1/255 of the row's
largest P' against its value row; relative to the row (a weighted mean of value rows whose
largest weight is that slot's) this is at most about 1/255 = 3.9e-3, and it is that large only
in a row dominated by one slot, so almost every row stays far below 1e-3."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from bit_group_quantized_act_amd import synth
from _util import to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _w4a8():
    from bit_group_quantized_act_amd import w4a8
    w4a8.load()
    return w4a8


def _run(A):
    w = _w4a8()
    c = A["cfg"]
    AL, packed = w.attn_pack_kv(to_dev(A["k8"]), to_dev(A["ks"]), to_dev(A["v8"]),
                                to_dev(A["vs"]), to_dev(A["kvpos"]))
    o, m, l, q8, sq = w.attn_prefill(AL, packed, to_dev(A["q"]), A["pos0"], c.window, c.sink,
                                     A["scale"])
    torch.cuda.synchronize()
    pk = packed.cpu().numpy()
    npad = AL.nblk * 64
    kq = pk[AL.off_kq:AL.off_kq + c.nkvh * npad * c.d].view(np.int8).reshape(c.nkvh, npad, c.d)
    return dict(o=o.cpu().numpy(), m=m.cpu().numpy(), l=l.cpu().numpy(), q8=q8.cpu().numpy(),
                sq=sq.cpu().numpy(), kq=kq[:, :c.nkv])


def _oracle(A):
    c = A["cfg"]
    q8, sq = oracle.attn_quant_q(A["q"])
    kq, sk = oracle.attn_requant_k(A["k8"], A["ks"])
    o, m, l = oracle.attn_int8(q8, sq, kq, sk, A["v8"], A["vs"], A["kvpos"], A["pos0"],
                               c.window, c.sink, A["scale"])
    return dict(o=o, m=m, l=l, q8=q8, sq=sq, kq=kq)


def check_attn(got, ref, what):
    assert np.array_equal(got["q8"], ref["q8"]), f"{what}: query codes differ"
    assert np.array_equal(got["sq"].view(np.uint32), ref["sq"].view(np.uint32)), \
        f"{what}: query scales differ"
    assert np.array_equal(got["kq"], ref["kq"]), f"{what}: requantized keys differ"
    seen = np.isfinite(ref["m"])
    assert np.array_equal(np.isfinite(got["m"]), seen), f"{what}: visibility differs"
    assert np.all(got["l"][~seen] == 0) and not got["o"][~seen].any()
    assert np.all(np.abs(got["m"][seen] - ref["m"][seen]) <= 2e-5 * (1 + np.abs(ref["m"][seen])))
    np.testing.assert_allclose(got["l"][seen], ref["l"][seen], rtol=1e-4)
    if not seen.any():
        return 0.0, 0.0
    on = got["o"][seen] / got["l"][seen][:, None]
    rn = ref["o"][seen] / ref["l"][seen][:, None]
    row = np.linalg.norm(on - rn, axis=1) / np.maximum(np.linalg.norm(rn, axis=1), 1e-30)
    tot = np.linalg.norm(on - rn) / np.linalg.norm(rn)
    assert tot <= 1e-4, f"{what}: relative L2 error {tot:.3e}"
    assert row.max() <= 4e-3, f"{what}: worst row {row.max():.3e}"
    assert (row > 1e-3).sum() <= max(1, row.size // 1000), \
        f"{what}: {(row > 1e-3).sum()} of {row.size} rows above 1e-3"
    return tot, row.max()


# partial query tiles (nq % 32) and partial blocks (nkv % 64), every head dimension, key/value
# heads shared by several query heads, a rolled window ring with sinks, a window that hides the
# oldest blocks entirely (skipped), and queries that see no slot at all
CASES = [
    ("A1", dict(nh=2, nkvh=1, nq=40, nkv=150, d=64)),
    ("A2", dict(nh=4, nkvh=2, nq=33, nkv=200, d=128, window=70, sink=3, pos0=400)),
    ("A2", dict(nh=4, nkvh=1, nq=64, nkv=300, d=256, window=100, sink=0, rolled=False,
                pos0=300)),
    ("A1", dict(nh=3, nkvh=3, nq=7, nkv=64, d=256)),
    ("A2", dict(nh=2, nkvh=1, nq=20, nkv=90, d=64, window=5, sink=0, rolled=False, pos0=400)),
    # slot ranges longer than one staged chunk (1024 / head_dim blocks): several chunks per
    # workgroup, the last one partly past the cache
    ("A1", dict(nh=8, nkvh=2, nq=256, nkv=2100, d=256)),
    ("A2", dict(nh=16, nkvh=4, nq=128, nkv=3000, d=128, window=300, sink=2, pos0=3100)),
    ("A1", dict(nh=32, nkvh=8, nq=256, nkv=1200, d=64)),
]


@pytest.mark.parametrize("name,over", CASES,
                         ids=[f"{n}-{'-'.join(f'{k}{v}' for k, v in o.items())}"
                              for n, o in CASES])
def test_attn_parity(name, over):
    A = synth.make_attn(name, **over)
    c = A["cfg"]
    print(f"attn {name} {over}", flush=True)
    got = _run(A)
    ref = _oracle(A)
    if c.window == 5:
        assert not np.isfinite(ref["m"]).any()      # every query is past the cache's window
    check_attn(got, ref, f"attn {name} {over}")


def test_attn_empty_slots_and_rerun_same_bits():
    # slots holding no position are never seen; a second call gives the same bits
    A = synth.make_attn("A1", nh=2, nkvh=1, nq=32, nkv=128, d=128)
    pos = A["kvpos"].copy()
    pos[::3] = -1
    A = dict(A, kvpos=pos)
    got = _run(A)
    check_attn(got, _oracle(A), "empty slots")
    again = _run(A)
    assert np.array_equal(got["o"].view(np.uint32), again["o"].view(np.uint32))


def test_attn_p_value_scale_fold_golden_on_gpu():
    """The hand-derived case of tests/golden/attn_p_value_scale_fold.txt through the kernel:
    the value group's scale folded into P before its 8-bit quantization."""
    import os
    want = {}
    with open(os.path.join(os.path.dirname(__file__), "golden",
                           "attn_p_value_scale_fold.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                key, val = line.split()
                want[key] = float(val)
    w = _w4a8()
    k8 = np.zeros((1, 2, 64), np.int8)
    ks = np.ones((1, 2, 2), np.float32)
    v8 = np.empty((1, 2, 64), np.int8)
    v8[0, 0], v8[0, 1] = 51, -102
    vs = np.array([[[1.0, 0.25], [0.25, 1.0]]], np.float32)
    AL, packed = w.attn_pack_kv(to_dev(k8), to_dev(ks), to_dev(v8), to_dev(vs),
                                to_dev(np.array([0, 1], np.int32)))
    o, m, l, q8, sq = w.attn_prefill(AL, packed, to_dev(np.zeros((1, 1, 64), np.float32)), 5,
                                     0, 0, 0.125)
    torch.cuda.synchronize()
    o, m, l = o.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()
    assert m[0, 0] == want["m"] and l[0, 0] == want["l"]
    np.testing.assert_allclose(o[0, 0, :32], want["o_group0"], rtol=1e-6)
    np.testing.assert_allclose(o[0, 0, 32:], want["o_group1"], rtol=1e-6)


def test_attn_subnormal_query_rows():
    """Query rows of subnormals: a scale that underflows to 0 (all codes 0: uniform attention
    over the visible slots) and a subnormal scale 2^-149 whose largest code clamps at 127."""
    A = synth.make_attn("A1", nh=2, nkvh=1, nq=32, nkv=128, d=128)
    q = A["q"].copy()
    tiny = np.float32(2.0 ** -149)
    q[0, 3, :] = 0.0
    q[0, 3, :4] = [np.float32(j) * tiny for j in (5, -3, 2, 1)]        # scale -> 0
    q[1, 7, :] = 0.0
    q[1, 7, :3] = [np.float32(j) * tiny for j in (190, -95, 1)]        # scale 2^-149, clamp
    A = dict(A, q=q)
    got = _run(A)
    ref = _oracle(A)
    assert ref["sq"][0, 3] == 0 and not ref["q8"][0, 3].any()
    assert ref["sq"][1, 7].view(np.uint32) == 1 and ref["q8"][1, 7, 0] == 127
    check_attn(got, ref, "subnormal query rows")


@pytest.mark.parametrize("name", ["A1", "A2"])
def test_attn_full_size(name):
    """The Gemma-style layer: 8 query heads on 2 key/value heads, head_dim 256, 256 queries
    against 1024 cached slots (A2: a 512-wide window over a rolled ring with 4 sinks)."""
    A = synth.make_attn(name)
    print(f"attn full {name}", flush=True)
    got = _run(A)
    ref = _oracle(A)
    check_attn(got, ref, f"attn full {name}")
    # and the method's distance to plain attention on the dequantized cache stays at the
    # oracle's own level
    c = A["cfg"]
    exact = oracle.attn_exact(A["q"], A["k8"], A["ks"], A["v8"], A["vs"], A["kvpos"], A["pos0"],
                              c.window, c.sink, A["scale"])
    on = got["o"] / got["l"][..., None]
    rel = np.linalg.norm(on - exact, axis=-1) / np.linalg.norm(exact, axis=-1)
    assert rel.mean() < 1.5e-2 and rel.max() < 4e-2, (rel.mean(), rel.max())
