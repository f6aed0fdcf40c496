"""w4a8_lm_head_argmax_noalloc (the greedy tail with the library's own key buffer) against
w4a8_lm_head_argmax with a caller's work buffer: the same kernels, so the same bits.

Two calls in a row on one GPU, the second on a smaller head (fewer rows and a shorter k), so the
second call runs over keys left by the first; every output (prepass codes, scales and sums, the
logits, the token and its value) must equal the work-buffer entry point's bit for bit, and the
token must be the first maximum of the logits.  A head above the buffer's size is refused on the
host before any device work."""
from __future__ import annotations

import numpy as np
import pytest

from bit_group_quantized_act_amd import synth
from _util import to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _w4a8():
    from bit_group_quantized_act_amd import w4a8
    w4a8.load()
    return w4a8


def _bufs(cfg, n):
    ng = cfg.k // cfg.group
    prep = (torch.empty((1, cfg.k), dtype=torch.int8, device="cuda:0"),
            torch.empty((ng, 1), dtype=torch.float32, device="cuda:0"),
            torch.empty((ng, 1), dtype=torch.int32, device="cuda:0"))
    out = (torch.empty(n, dtype=torch.float32, device="cuda:0"),
           torch.empty(1, dtype=torch.int32, device="cuda:0"),
           torch.empty(1, dtype=torch.float32, device="cuda:0"))
    return prep, out


def _both(L, cap, plant_row=None):
    """Run the no-alloc entry point and the work-buffer one on the same head; numpy results."""
    w = _w4a8()
    cfg = L["cfg"]
    lay, packed = w.pack(to_dev(L["codes"]), to_dev(L["scales"]), cfg.fmt, cfg.group,
                         bias=to_dev(L["bias"]), codebook=to_dev(L["codebook"]))
    x = to_dev(L["x"].reshape(-1))
    res = []
    for noalloc in (True, False):
        prep, out = _bufs(cfg, cfg.n)
        if noalloc:
            w.lm_head_argmax_noalloc(lay, packed, x, out, prep, cap, cfg.hadamard)
        else:
            w.lm_head_argmax(lay, packed, x, cap, cfg.hadamard, out=out, prep_out=prep)
        torch.cuda.synchronize()
        res.append([t.cpu().numpy() for t in prep + out])
    return res


def _check_same(a, b, what):
    names = ("xq", "xs", "xsum", "logits", "token", "value")
    for name, u, v in zip(names, a, b):
        assert np.array_equal(np.ascontiguousarray(u).view(np.uint8),
                              np.ascontiguousarray(v).view(np.uint8)), f"{what}: {name} differs"
    logits, token, value = a[3], int(a[4][0]), a[5][0]
    assert token == int(np.argmax(logits)), f"{what}: token is not the first maximum"
    assert value.view(np.uint32) == logits[token].view(np.uint32)


def test_noalloc_matches_work_buffer_entry_point_twice():
    # first a 5000-row head whose largest logit is planted at row 4000 (its key stays in the
    # library's buffer), then a smaller head: 1000 rows and k 512, which must not see that key
    big = synth.make("C5a", full_range=True, n=5000, k=1536)
    codes = big["codes"].copy()
    nib = np.where(big["x"][0] >= 0, 7, 9).astype(np.uint8)   # q = 7 * sign(x): a dominant row
    codes[4000] = nib[0::2] | (nib[1::2] << 4)
    big = dict(big, codes=codes)
    a, b = _both(big, 0.0)
    _check_same(a, b, "first call, n = 5000")
    assert int(a[4][0]) == 4000
    small = synth.make("C1", full_range=True, n=1000, k=512)
    a, b = _both(small, 0.0)
    _check_same(a, b, "second call, n = 1000")
    assert int(a[4][0]) < 1000


def test_noalloc_rotated_codebook_head_and_ragged_rows():
    # a rotated codebook head (128-wide groups) with a ragged last panel, then a one-row head
    L = synth.make("C4", full_range=False, m=1, n=3001, k=768)
    a, b = _both(L, 15.0)
    _check_same(a, b, "rotated codebook head, n = 3001")
    L = synth.make("C1", full_range=True, n=1, k=256)
    a, b = _both(L, 0.0)
    _check_same(a, b, "n = 1")


def test_noalloc_refuses_a_head_above_its_buffer():
    w = _w4a8()
    lay = w.packed_layout(w.SYM, w.NOALLOC_MAX_N + 64, 128, 64)
    packed = torch.empty(256, dtype=torch.uint8, device="cuda:0")   # never read: refused first
    prep = (torch.empty((1, 128), dtype=torch.int8, device="cuda:0"),
            torch.empty((2, 1), dtype=torch.float32, device="cuda:0"),
            torch.empty((2, 1), dtype=torch.int32, device="cuda:0"))
    out = (torch.empty(16, dtype=torch.float32, device="cuda:0"),
           torch.empty(1, dtype=torch.int32, device="cuda:0"),
           torch.empty(1, dtype=torch.float32, device="cuda:0"))
    x = torch.zeros(128, dtype=torch.float32, device="cuda:0")
    with pytest.raises(w.W4A8Error) as ei:
        w.lm_head_argmax_noalloc(lay, packed, x, out, prep, 0.0, 0)
    assert ei.value.status == 2 and "W4A8_NOALLOC_MAX_N" in str(ei.value)
