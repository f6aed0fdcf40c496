"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: int8 codes xq, fp32 scales xs (compared as bit patterns), int32 group sums xsum and the
int32 per-group partials D.  Tolerance on the fp32 output y: relative L2 <= 1e-5 and per element
|err| <= 1e-4 * sum of the term magnitudes.  Shapes span several tiles plus ragged M and N tails;
full-size configs are checked on sampled output columns the oracle computes one by one.
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
    return w4a8


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


def _pack(L):
    cfg = L["cfg"]
    return _w4a8().pack(to_dev(L["codes"]), to_dev(L["scales"]), cfg.fmt, cfg.group,
                        bias=to_dev(L["bias"]), codebook=to_dev(L["codebook"]))


def _run(L, with_partials=True):
    """HIP prep + linear (+ partials) for a layer dict; returns numpy results."""
    w = _w4a8()
    cfg = L["cfg"]
    lay, packed = _pack(L)
    x = to_dev(L["x"])
    xq, xs, xsum = w.prep(x, cfg.group, cfg.hadamard)
    if cfg.m == 1:
        y = w.gemv(lay, packed, xq[0], xs, xsum)
    else:
        y = w.gemm(lay, packed, xq, xs, xsum)
    d = w.debug_partials(lay, packed, xq, xsum) if with_partials else None
    torch.cuda.synchronize()
    # the library keeps scales and sums group-major [k/group, m]; the oracle row-major [m, k/group]
    out = dict(xq=xq.cpu().numpy(), xs=xs.cpu().numpy().T.copy(), xsum=xsum.cpu().numpy().T.copy(),
               y=y.cpu().numpy().reshape(cfg.m, cfg.n))
    if d is not None:
        out["d"] = d.cpu().numpy()
    return out


# (config, overrides, full_range codes): every format and group, GEMV and GEMM, M tails
# {1, 2, 63, 65, 127, 130}, N tails {16, 1000, 2049}, several 64-row panels and 128-row M tiles.
# GEMMs with k a multiple of 256 (and of 512 for 128-groups) and fewer tiles than the CUs run
# every tile split over four workgroups; the others take whole tiles.
CASES = [
    ("C1", dict(), False),
    ("C1", dict(n=1000), True),
    ("C1", dict(n=16, k=256), True),
    ("C2b", dict(), False),
    ("C2b", dict(n=2049), True),
    ("C1", dict(group=128, k=1024, n=640), True),
    ("C3a", dict(m=1, n=1000, k=1024), True),
    ("C4", dict(m=1, n=320, k=768), False),
    ("C3a", dict(m=2, n=256, k=640), True),
    ("C3a", dict(m=65, n=1000, k=1280), True),
    ("C3a", dict(m=130, n=2049, k=512), True),
    ("C3a", dict(m=63, n=16, k=128), True),
    ("C1", dict(m=127, n=512, k=1024), True),
    ("C1", dict(m=128, n=384, k=768, group=128), True),
    ("C4", dict(m=200, n=448, k=1536), False),
    ("C4", dict(m=3, n=2049, k=512), False),
    ("C5b", dict(m=64, n=1000, k=1536), False),
    # taller activation blocks with 128-wide groups: several row tiles with a 1-row or a
    # 44-row last tile, ragged n, and 1024 rows in the sign-folded and affine formats
    ("C4", dict(m=256, n=96, k=384), False),
    ("C4", dict(m=300, n=1000, k=768), True),
    ("C1", dict(m=257, n=200, k=1024, group=128), True),
    ("C3a", dict(m=513, n=130, k=768, group=128), True),
    ("C3a", dict(m=1024, n=384, k=256, group=128), True),
    # more tiles than CUs: whole tiles and, for the last partial round, tiles split over four
    # workgroups (one k quarter per wavefront) in the same launch
    ("C3a", dict(m=64, n=34816, k=512), True),
    ("C4", dict(m=64, n=33000, k=512), False),
    # wide layers, few rows: 512 tiles (two whole rounds on 256 CUs), 516 tiles (a tail of four
    # split tiles, a last row block of 2 rows), 513 tiles (one split tile, a ragged channel tile)
    ("C5b", dict(m=3, n=65536, k=256), False),
    ("C3a", dict(m=130, n=22016, k=256), True),
    ("C4", dict(m=2, n=65600, k=512), False),
    # the largest k the ABI takes (2^20): one tile split over four workgroups, 1024 stages per
    # k quarter; and 2^19 with 128-groups over several whole tiles
    ("C1", dict(m=2, n=64, k=1 << 20), True),
    ("C3a", dict(m=5, n=200, k=1 << 19, group=128), True),
    # many rows: 128 row blocks of one channel tile, all split (512 workgroups)
    ("C3a", dict(m=8192, n=64, k=256), True),
]


@pytest.mark.parametrize("name,over,full", CASES,
                         ids=[f"{c}-{'-'.join(f'{k}{v}' for k, v in o.items())}-{'full' if f else 'w'}"
                              for c, o, f in CASES])
def test_parity_bitexact_and_tolerance(name, over, full):
    L = synth.make(name, full_range=full, **over)
    cfg = L["cfg"]
    print(f"case {name} {over} m={cfg.m} n={cfg.n} k={cfg.k} g={cfg.group} fmt={cfg.fmt}",
          flush=True)
    got = _run(L)
    ref = oracle_layer(L)
    assert np.array_equal(got["xq"], ref["xq"]), "xq differs"
    assert np.array_equal(_bits(got["xs"]), _bits(ref["xs"])), "xs differs"
    assert np.array_equal(got["xsum"], ref["xsum"]), "xsum differs"
    dref = oracle.partials(cfg.fmt, L["codes"], ref["xq"], cfg.group, codebook=L["codebook"])
    assert np.array_equal(got["d"], dref), \
        f"partials differ at {np.argwhere(got['d'] != dref)[:5].tolist()}"
    check_y(got["y"], ref["y"], ref["t"], f"{name} {over}")


def _run_linear(L):
    """The whole layer through w4a8_linear (fused prepass + GEMV for one row)."""
    w = _w4a8()
    cfg = L["cfg"]
    lay, packed = _pack(L)
    x = to_dev(L["x"])
    ng = cfg.k // cfg.group
    prep_out = (torch.empty((cfg.m, cfg.k), dtype=torch.int8, device="cuda:0"),
                torch.empty((ng, cfg.m), dtype=torch.float32, device="cuda:0"),
                torch.empty((ng, cfg.m), dtype=torch.int32, device="cuda:0"))
    y, (xq, xs, xsum) = w.linear(lay, packed, x, cfg.hadamard, prep_out=prep_out)
    torch.cuda.synchronize()
    return dict(xq=xq.cpu().numpy(), xs=xs.cpu().numpy().T.copy(), xsum=xsum.cpu().numpy().T.copy(),
                y=y.cpu().numpy().reshape(cfg.m, cfg.n))


# one-row cases take the fused kernel (rotation included for C4); the 16448-wide row exceeds the
# fused kernel's LDS bound, and 262145 outputs its panel bound, and take prepass + GEMV;
# multi-row cases take prepass + GEMM
LINEAR_CASES = [
    ("C1", dict(), False),
    ("C1", dict(n=1000), True),
    ("C2b", dict(n=2049), True),
    ("C1", dict(group=128, k=1024, n=640), True),
    ("C3a", dict(m=1, n=1000, k=1024), True),
    ("C3a", dict(m=1, n=200, k=640), True),
    ("C4", dict(m=1, n=320, k=768), False),
    ("C4", dict(m=1, n=130, k=1536), True),
    # fused at six metadata blocks (six wavefronts, one block each): 24 groups of 64, 22 groups
    # (a last block of two), 24 groups of 128 with rotation
    ("C1", dict(n=1000, k=1536), True),
    ("C3a", dict(m=1, n=600, k=1408), True),
    ("C4", dict(m=1, n=200, k=3072), True),
    ("C2a", dict(n=320, k=4096), True),           # fused, 2 activation quads per lane
    ("C4", dict(m=1, n=130, k=8192), True),        # fused with rotation, 4 quads per lane
    ("C1", dict(n=192, k=16384), True),            # fused at its k bound, 8 quads per lane
    ("C1", dict(n=64, k=16448), True),
    ("C1", dict(n=262144, k=128), False),          # fused at its row bound, 4096 panels
    ("C1", dict(n=262145, k=128), False),          # one row past it: prepass + GEMV
    ("C4", dict(m=1, n=131072, k=128), False),     # rotated: fused at its 2048-panel bound
    ("C4", dict(m=1, n=131073, k=128), False),     # one row past it: prepass + GEMV
    ("C3a", dict(m=65, n=1000, k=1280), True),
    ("C4", dict(m=200, n=448, k=1536), False),
    ("C1", dict(n=64, k=1 << 20), True),          # the largest k: prepass + GEMV, 4096 blocks
]


@pytest.mark.parametrize("name,over,full", LINEAR_CASES,
                         ids=[f"{c}-{'-'.join(f'{k}{v}' for k, v in o.items())}-{'full' if f else 'w'}"
                              for c, o, f in LINEAR_CASES])
def test_linear_bitexact_and_tolerance(name, over, full):
    L = synth.make(name, full_range=full, **over)
    cfg = L["cfg"]
    print(f"linear {name} {over} m={cfg.m} n={cfg.n} k={cfg.k} had={cfg.hadamard}", flush=True)
    got = _run_linear(L)
    ref = oracle_layer(L)
    assert np.array_equal(got["xq"], ref["xq"]), "xq differs"
    assert np.array_equal(_bits(got["xs"]), _bits(ref["xs"])), "xs differs"
    assert np.array_equal(got["xsum"], ref["xsum"]), "xsum differs"
    check_y(got["y"], ref["y"], ref["t"], f"linear {name} {over}")
    # the fused kernel runs the same arithmetic as prepass + GEMV: the same bits
    split = _run(L, with_partials=False)
    assert np.array_equal(_bits(got["y"]), _bits(split["y"])), "linear and prep+matmul differ"


def test_pack_round_trip_and_padding():
    """Decode the packed buffer on the host from the documented layout and recover the input."""
    for name, over in (("C3a", dict(m=1, n=100, k=640)), ("C4", dict(m=1, n=70, k=256)),
                       ("C1", dict(n=64, k=128))):
        L = synth.make(name, full_range=True, **over)
        cfg = L["cfg"]
        lay, packed = _pack(L)
        torch.cuda.synchronize()
        buf = packed.cpu().numpy()
        n, k, g = cfg.n, cfg.k, cfg.group
        npad, ng, kc = lay.n_pad, k // g, k // 32
        chunks = buf[lay.off_codes:lay.off_codes + npad * k // 2].reshape(npad // 64, kc, 64, 16)
        codes = np.zeros((npad, k), np.uint8)
        for j in range(4):
            for b in range(4):
                byte = chunks[:, :, :, 4 * j + b]                      # [panel, chunk, row]
                lo, hi = byte & 0xF, byte >> 4
                for kk, val in ((4 * j + b, lo), (16 + 4 * j + b, hi)):
                    codes.reshape(npad // 64, 64, kc, 32)[:, :, :, kk] = val.transpose(0, 2, 1)
        assert not codes[n:].any()                 # padding rows are zero nibbles
        if cfg.fmt == synth.FMT_AFFINE:
            codes ^= 8                             # affine stores u XOR 8
        assert np.array_equal(codes[:n], synth.unpack_nibbles(L["codes"])), name
        mb = lay.meta_bytes
        nblk = (ng + 3) // 4                       # metadata blocks of 4 groups
        meta = buf[lay.off_meta:lay.off_meta + npad * nblk * 4 * mb]
        meta = meta.view(np.uint32 if mb == 4 else np.uint16).reshape(npad // 64, nblk, 64, 4)
        meta = meta.transpose(0, 2, 1, 3).reshape(npad, nblk * 4)
        assert not meta[:, ng:].any()              # the padded entries of the last block
        meta = meta[:, :ng]
        sc = (meta & 0xFFFF).astype(np.uint16)
        assert np.array_equal(sc[:n], L["scales"].view(np.uint16)), name
        assert not sc[n:].any()
        if cfg.fmt == synth.FMT_AFFINE:
            assert np.array_equal((meta[:n] >> 16).astype(np.uint16), L["bias"].view(np.uint16))
        if cfg.fmt == synth.FMT_CODEBOOK:
            cb = buf[lay.off_codebook:lay.off_codebook + npad * 16].view(np.int8).reshape(npad, 16)
            assert np.array_equal(cb[:n], L["codebook"]) and not cb[n:].any()


def test_flipped_nibble_moves_one_column():
    L = synth.make("C1", full_range=True, n=256, k=512)
    base = _run(L, with_partials=False)["y"]
    codes = L["codes"].copy()
    codes[77, 100] ^= 0x10       # high nibble of byte 100 -> k = 201 of row 77
    L2 = dict(L, codes=codes)
    y2 = _run(L2, with_partials=False)["y"]
    diff = np.nonzero(base[0] != y2[0])[0]
    assert diff.tolist() == [77]


def _subnormal_groups(rows, k):
    """Rows whose 64-wide groups hold the subnormal golden cases (multiples j of 2^-149 whose
    scale rounds to 0, to 2^-149 with a clamped code, or to 3 * 2^-149), cycled over the
    groups; the rest of each group is zero."""
    cases = [[5, -3], [63, -63, 1], [64, -1, 6], [190, -95, 1], [381, -7, 3, 1, 2, -5]]
    x = np.zeros((rows, k), np.float32)
    tiny = np.float32(2.0 ** -149)
    for r in range(rows):
        for g in range(k // 64):
            vals = cases[(r * (k // 64) + g) % len(cases)]
            x[r, 64 * g:64 * g + len(vals)] = [np.float32(j) * tiny for j in vals]
    return x


def test_subnormal_groups_through_the_fused_gemv():
    """One decode row whose groups are subnormal golden cases, through the fused prepass + GEMV
    (with and without rotation) and through prepass + GEMV: codes, scales and sums bit-exact."""
    for name, over in (("C1", dict(n=192, k=640)), ("C4", dict(m=1, n=130, k=768))):
        L = synth.make(name, full_range=True, **over)
        cfg = L["cfg"]
        x = L["x"].copy()
        x[:, :320] = _subnormal_groups(1, 320)        # five subnormal groups, the rest normal
        L = dict(L, x=x)
        print(f"subnormal linear {name} {over} had={cfg.hadamard}", flush=True)
        got = _run_linear(L)
        ref = oracle_layer(L)
        if cfg.hadamard == 0:
            assert (ref["xs"][0, :5] == 0).sum() == 2 and (ref["xs"][0, :5] > 0).sum() == 3
            assert np.abs(ref["xq"][0, :320]).max() == 127
        assert np.array_equal(got["xq"], ref["xq"]), "xq differs"
        assert np.array_equal(_bits(got["xs"]), _bits(ref["xs"])), "xs differs"
        assert np.array_equal(got["xsum"], ref["xsum"]), "xsum differs"
        check_y(got["y"], ref["y"], ref["t"], f"subnormal linear {name}")
        split = _run(L, with_partials=False)
        assert np.array_equal(_bits(got["y"]), _bits(split["y"])), "linear and prep+matmul differ"


def test_prep_edge_cases():
    w = _w4a8()
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    x[0, :64] = 0.0                                    # all-zero group
    x[1, :] = 0.0                                      # all-zero row
    x[2, 64:128] = np.float32(127.0) * np.sign(rng.standard_normal(64)).astype(np.float32)
    x[2, 64] = 127.0                                   # amax 127 -> scale exactly 1
    x[2, 65:70] = [0.5, 1.5, 2.5, -0.5, -2.5]          # ties round to even
    x[3, :] = rng.standard_normal(256).astype(np.float32) * np.float32(1e-30)   # tiny values
    x[4, :] = rng.standard_normal(256).astype(np.float32) * np.float32(1e30)    # huge values
    # subnormal groups: scales that underflow to 0 (codes 0) and subnormal scales whose codes
    # clamp at 127 (the golden cases of the oracle's pins, one per 64-wide group)
    x = np.concatenate([x, _subnormal_groups(2, 256)])
    for group, had in ((64, 0), (128, 0), (64, 128), (128, 128)):
        xq, xs, xsum = w.prep(to_dev(x), group, had)
        torch.cuda.synchronize()
        oq, os_, osum = oracle.prep(x, group, had)
        assert np.array_equal(xq.cpu().numpy(), oq), (group, had)
        assert np.array_equal(_bits(xs.cpu().numpy().T), _bits(os_)), (group, had)
        assert np.array_equal(xsum.cpu().numpy().T, osum), (group, had)
    # m == 0 is a no-op
    e = torch.empty((0, 256), dtype=torch.float32, device="cuda:0")
    xq, xs, xsum = w.prep(e, 64)
    assert xq.shape == (0, 256)


def test_gemm_m0_is_noop():
    w = _w4a8()
    L = synth.make("C3a", full_range=True, m=2, n=64, k=128)
    lay, packed = _pack(L)
    z8 = torch.empty((0, 128), dtype=torch.int8, device="cuda:0")
    zf = torch.empty((2, 0), dtype=torch.float32, device="cuda:0")
    zi = torch.empty((2, 0), dtype=torch.int32, device="cuda:0")
    y = w.gemm(lay, packed, z8, zf, zi)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)


FULL = [("C2a", None), ("C5a", None), ("C3a", 384), ("C3b", 384), ("C4", 256), ("C5b", 256)]


@pytest.mark.parametrize("name,ncols", FULL, ids=[f for f, _ in FULL])
def test_full_size_sampled(name, ncols, layer_cache):
    """Full configs in the benchmark's launch configuration; the oracle checks every output of
    the GEMVs and a seeded sample of columns (all rows) of the GEMMs, plus the whole prepass."""
    if name not in layer_cache:
        layer_cache[name] = synth.make(name)
    L = layer_cache[name]
    cfg = L["cfg"]
    print(f"full {name}: m={cfg.m} n={cfg.n} k={cfg.k}", flush=True)
    got = _run(L, with_partials=False)
    lin = _run_linear(L)         # the benchmark's path (one fused kernel for a single row)
    assert np.array_equal(_bits(lin["y"]), _bits(got["y"])), "linear and prep+matmul differ"
    assert np.array_equal(lin["xq"], got["xq"]) and np.array_equal(lin["xsum"], got["xsum"])
    assert np.array_equal(_bits(lin["xs"]), _bits(got["xs"]))
    cols = None
    if ncols is not None:
        cols = np.sort(np.random.default_rng(11).choice(cfg.n, ncols, replace=False))
        cols[-1] = cfg.n - 1                               # include the last column
    ref = oracle_layer(L, cols)
    assert np.array_equal(got["xq"], ref["xq"])
    assert np.array_equal(_bits(got["xs"]), _bits(ref["xs"]))
    assert np.array_equal(got["xsum"], ref["xsum"])
    yg = got["y"] if cols is None else got["y"][:, cols]
    check_y(yg, ref["y"], ref["t"], name)
