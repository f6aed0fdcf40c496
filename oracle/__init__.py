"""CPU oracle of the W4A8 linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product path (the HIP library and its Python binding) never imports,
links or calls it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain C loops, built with ``-O2 -ffp-contract=off`` and no
fast-math); this module only builds that file with gcc, loads it with ctypes and marshals numpy
arrays.  See the header of ``oracle.c`` for what each step computes and which passage of the
pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FORMAT_SYM, FORMAT_AFFINE, FORMAT_CODEBOOK, FORMAT_INT8, FORMAT_CQ2, FORMAT_CQ1, FORMAT_CQ3 = \
    0, 1, 2, 3, 4, 5, 6

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc, OpenMP, strict IEEE fp32)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_wht_block.argtypes = [P, ctypes.c_int]
    lib.oracle_wht_block.restype = None
    lib.oracle_rotate.argtypes = [P, i64, i64, i32]
    lib.oracle_quantize.argtypes = [P, i64, i64, i32, P, P, P]
    lib.oracle_prep.argtypes = [P, i64, i64, i32, i32, P, P, P]
    lib.oracle_partials.argtypes = [i32, P, P, i64, i64, i32, P, i64, P]
    lib.oracle_linear.argtypes = [i32, P, P, P, P, i64, i64, i32, P, P, P, i64, P, P]
    lib.oracle_glu.argtypes = [i32, P, P, i64, i64, P, P]
    lib.oracle_softcap_argmax.argtypes = [P, i64, i64, ctypes.c_double, P, P, P]
    lib.oracle_float_to_half.argtypes = [ctypes.c_float]
    lib.oracle_float_to_half.restype = ctypes.c_uint16
    lib.oracle_prep_a16.argtypes = [P, i64, i64, P, P]
    lib.oracle_linear_a16.argtypes = [i32, P, P, P, P, i64, i64, i32, P, P, i64, P, P]
    lib.oracle_attn_requant_k.argtypes = [P, P, i64, i64, i32, P, P]
    lib.oracle_attn_int8.argtypes = [P, P, i64, i64, P, P, P, P, P, i64, i64, i64, i32, i64, i32,
                                     i32, ctypes.c_double, P, P, P]
    lib.oracle_attn_exact.argtypes = [P, i64, i64, P, P, P, P, P, i64, i64, i64, i32, i32, i64,
                                      i32, i32, ctypes.c_double, P]
    for f in ("oracle_rotate", "oracle_quantize", "oracle_prep", "oracle_partials",
              "oracle_linear", "oracle_glu", "oracle_softcap_argmax", "oracle_prep_a16",
              "oracle_linear_a16", "oracle_attn_requant_k", "oracle_attn_int8",
              "oracle_attn_exact", "oracle_num_threads"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc == 1:
        raise ValueError(f"{what}: invalid arguments")
    if rc == 2:
        raise OverflowError(f"{what}: an integer partial does not fit int32")
    if rc != 0:
        raise RuntimeError(f"{what}: status {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def half_to_double(h: int) -> float:
    return float(_load().oracle_half_to_double(int(h)))


def wht(x: np.ndarray, block: int = 128) -> np.ndarray:
    """Normalized Walsh-Hadamard transform of every `block`-wide block of each row (fp32)."""
    x = np.array(x, dtype=np.float32, order="C", copy=True)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    _check(_load().oracle_rotate(_ptr(x), m, k, block), "rotate")
    return x


def quantize(x: np.ndarray, group: int):
    """Per-row per-group int8 quantization: returns (xq int8 [m,k], xs f32 [m,k/g], xsum i32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    xq = np.empty((m, k), np.int8)
    xs = np.empty((m, k // group), np.float32)
    xsum = np.empty((m, k // group), np.int32)
    _check(_load().oracle_quantize(_ptr(x), m, k, group, _ptr(xq), _ptr(xs), _ptr(xsum)),
           "quantize")
    return xq, xs, xsum


def prep(x: np.ndarray, group: int, hadamard_block: int = 0):
    """The activation prepass: optional rotation, then quantize.  Returns (xq, xs, xsum)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    xq = np.empty((m, k), np.int8)
    xs = np.empty((m, k // group), np.float32)
    xsum = np.empty((m, k // group), np.int32)
    _check(_load().oracle_prep(_ptr(x), m, k, group, hadamard_block,
                               _ptr(xq), _ptr(xs), _ptr(xsum)), "prep")
    return xq, xs, xsum


def partials(fmt: int, codes: np.ndarray, xq: np.ndarray, group: int, codebook=None):
    """Integer per-group partials D [m, n, k/group] (int32)."""
    codes = np.ascontiguousarray(codes).view(np.uint8)      # int8 codes (format 3) as bytes
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    if xq.ndim == 1:
        xq = xq[None, :]
    n = codes.shape[0]
    m, k = xq.shape
    assert codes.shape[1] * {FORMAT_INT8: 1, FORMAT_CQ2: 4, FORMAT_CQ1: 8, FORMAT_CQ3: 1}.get(fmt, 2) == k
    cb = None if codebook is None else np.ascontiguousarray(codebook, dtype=np.int8)
    d = np.empty((m, n, k // group), np.int32)
    _check(_load().oracle_partials(fmt, _ptr(codes), _ptr(cb), n, k, group, _ptr(xq), m,
                                   _ptr(d)), "partials")
    return d


def linear(fmt: int, codes, scales_f16, xq, xs, xsum, group: int, bias_f16=None,
           codebook=None, with_terms: bool = True):
    """fp64 output y [m, n] (and the term magnitude T [m, n] if with_terms)."""
    codes = np.ascontiguousarray(codes).view(np.uint8)      # int8 codes (format 3) as bytes
    scales = np.ascontiguousarray(scales_f16, dtype=np.float16).view(np.uint16)
    bias = None if bias_f16 is None else \
        np.ascontiguousarray(bias_f16, dtype=np.float16).view(np.uint16)
    cb = None if codebook is None else np.ascontiguousarray(codebook, dtype=np.int8)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    xsum = np.ascontiguousarray(xsum, dtype=np.int32)
    if xq.ndim == 1:
        xq, xs, xsum = xq[None, :], xs[None, :], xsum[None, :]
    n = codes.shape[0]
    m, k = xq.shape
    y = np.empty((m, n), np.float64)
    t = np.empty((m, n), np.float64) if with_terms else None
    _check(_load().oracle_linear(fmt, _ptr(codes), _ptr(scales), _ptr(bias), _ptr(cb), n, k,
                                 group, _ptr(xq), _ptr(xs), _ptr(xsum), m, _ptr(y), _ptr(t)),
           "linear")
    return (y, t) if with_terms else y


ACT_SILU, ACT_GELU_TANH, ACT_GELU_ERF = 0, 1, 2


def glu(act: int, y: np.ndarray, t: np.ndarray = None):
    """Gated output of a [gate; up] linear: z [m, n/2] = act(y[:, :n/2]) * y[:, n/2:] in fp64,
    and its error-bound magnitude tz when the linear's term magnitudes t are given."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    if y.ndim == 1:
        y = y[None, :]
        t = None if t is None else np.ascontiguousarray(t, dtype=np.float64)[None, :]
    m, n = y.shape
    z = np.empty((m, n // 2), np.float64)
    tz = None
    if t is not None:
        t = np.ascontiguousarray(t, dtype=np.float64)
        tz = np.empty((m, n // 2), np.float64)
    _check(_load().oracle_glu(act, _ptr(y), _ptr(t), m, n, _ptr(z), _ptr(tz)), "glu")
    return (z, tz) if t is not None else z


def softcap_argmax(y: np.ndarray, cap: float = 0.0):
    """Greedy tail of a vocabulary head: (logits, token, value) per row of y [m, n] (or [n]);
    logits = cap * tanh(y / cap) for cap > 0 (y for cap == 0), token = the smallest index of
    the largest logit, all in fp64."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    one = y.ndim == 1
    if one:
        y = y[None, :]
    m, n = y.shape
    logits = np.empty_like(y)
    token = np.empty(m, np.int64)
    value = np.empty(m, np.float64)
    _check(_load().oracle_softcap_argmax(_ptr(y), m, n, float(cap), _ptr(logits), _ptr(token),
                                         _ptr(value)), "softcap_argmax")
    return (logits[0], int(token[0]), float(value[0])) if one else (logits, token, value)


def float_to_half(x) -> np.ndarray:
    """binary16 bit patterns (uint16) nearest to each fp32 value, ties to even (one call per
    value: meant for pins and small cases)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    f = _load().oracle_float_to_half
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def prep_a16(x):
    """fp16-activation prepass of x float32 [m, k] (k % 64 == 0): (xh uint16 binary16 bits
    [m, k] in natural order, S float32 [m, k/64] group sums by the fixed tree)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    m, k = x.shape
    xh = np.empty((m, k), np.uint16)
    xsf = np.empty((m, k // 64), np.float32)
    _check(_load().oracle_prep_a16(_ptr(x), m, k, _ptr(xh), _ptr(xsf)), "prep_a16")
    return xh, xsf


def linear_a16(fmt: int, codes, scales_f16, xh, xsf, group: int = 64, bias_f16=None,
               codebook=None, with_terms: bool = True):
    """fp64 output y [m, n] of the fp16-activation linear (and its term magnitude T)."""
    codes = np.ascontiguousarray(codes).view(np.uint8)      # int8 codes (format 3) as bytes
    scales = np.ascontiguousarray(scales_f16, dtype=np.float16).view(np.uint16)
    bias = None if bias_f16 is None else \
        np.ascontiguousarray(bias_f16, dtype=np.float16).view(np.uint16)
    cb = None if codebook is None else np.ascontiguousarray(codebook, dtype=np.int8)
    xh = np.ascontiguousarray(xh, dtype=np.uint16)
    xsf = np.ascontiguousarray(xsf, dtype=np.float32)
    if xh.ndim == 1:
        xh, xsf = xh[None, :], xsf[None, :]
    n = codes.shape[0]
    m, k = xh.shape
    y = np.empty((m, n), np.float64)
    t = np.empty((m, n), np.float64) if with_terms else None
    _check(_load().oracle_linear_a16(fmt, _ptr(codes), _ptr(scales), _ptr(bias), _ptr(cb), n, k,
                                     group, _ptr(xh), _ptr(xsf), m, _ptr(y), _ptr(t)),
           "linear_a16")
    return (y, t) if with_terms else y


# ---- prefill attention over the cached int8 segment

ATTN_GROUP = 32          # width of the cache's key and value scale groups (head_dim / 32 each)


def attn_requant_k(k8, ks, gk: int = ATTN_GROUP):
    """Keys to one flat scale per vector: (kq int8 [.., n, d], sk float32 [.., n])."""
    k8 = np.ascontiguousarray(k8, dtype=np.int8)
    ks = np.ascontiguousarray(ks, dtype=np.float32)
    d = k8.shape[-1]
    n = k8.size // d
    kq = np.empty_like(k8)
    sk = np.empty(k8.shape[:-1], np.float32)
    _check(_load().oracle_attn_requant_k(_ptr(k8), _ptr(ks), n, d, gk, _ptr(kq), _ptr(sk)),
           "attn_requant_k")
    return kq, sk


def attn_quant_q(q):
    """Queries to int8 with one flat scale per row: (q8 [.., d], sq [..])."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    d = q.shape[-1]
    q8, sq, _ = prep(q.reshape(-1, d), d, 0)
    return q8.reshape(q.shape), sq.reshape(q.shape[:-1])


def attn_int8(q8, sq, kq, sk, v8, vs, kvpos, pos0: int, window: int = 0, sink: int = 0,
              scale: float = 1.0, gv: int = ATTN_GROUP):
    """The int8 method: (o [nh, nq, d] unnormalized, m [nh, nq], l [nh, nq]) in fp64."""
    q8 = np.ascontiguousarray(q8, dtype=np.int8)
    nh, nq, d = q8.shape
    kq = np.ascontiguousarray(kq, dtype=np.int8)
    nkvh, nkv, _ = kq.shape
    args = [np.ascontiguousarray(a, dtype=t) for a, t in ((sq, np.float32), (sk, np.float32),
                                                           (v8, np.int8), (vs, np.float32),
                                                           (kvpos, np.int32))]
    o = np.empty((nh, nq, d), np.float64)
    m = np.empty((nh, nq), np.float64)
    l = np.empty((nh, nq), np.float64)
    _check(_load().oracle_attn_int8(_ptr(q8), _ptr(args[0]), nh, nq, _ptr(kq), _ptr(args[1]),
                                    _ptr(args[2]), _ptr(args[3]), _ptr(args[4]), nkvh, nkv, d,
                                    gv, pos0, window, sink, float(scale), _ptr(o), _ptr(m),
                                    _ptr(l)), "attn_int8")
    return o, m, l


def attn_exact(q, k8, ks, v8, vs, kvpos, pos0: int, window: int = 0, sink: int = 0,
               scale: float = 1.0, gk: int = ATTN_GROUP, gv: int = ATTN_GROUP):
    """Plain fp64 attention on unquantized q and the dequantized cache: out [nh, nq, d]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    nh, nq, d = q.shape
    k8 = np.ascontiguousarray(k8, dtype=np.int8)
    nkvh, nkv, _ = k8.shape
    ks, v8, vs, kvpos = (np.ascontiguousarray(a, dtype=t) for a, t in (
        (ks, np.float32), (v8, np.int8), (vs, np.float32), (kvpos, np.int32)))
    out = np.empty((nh, nq, d), np.float64)
    _check(_load().oracle_attn_exact(_ptr(q), nh, nq, _ptr(k8), _ptr(ks), _ptr(v8), _ptr(vs),
                                     _ptr(kvpos), nkvh, nkv, d, gk, gv, pos0, window, sink,
                                     float(scale), _ptr(out)), "attn_exact")
    return out
