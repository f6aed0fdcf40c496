"""Seeded synthetic inputs for the W4A8 linear layer (numpy only).

This module is shared by the tests, the benchmark and the smoke check.  It draws random
numbers and lays them out in the canonical input format; it contains none of the layer's own
arithmetic (no rotation, no activation quantization, no integer dot products, no rescale).
The weight codes it produces stand in for a quantized checkpoint: the offline weight quantizer
below (symmetric ``s = f16(max|w|/7)``, affine ``s = f16((max-min)/15), b = f16(min)``) only
turns Gaussian draws into plausible codes and scales.

Canonical formats (consumed by both the HIP library and the oracle):
  x          float32 [m, k]                   activations, row-major
  codes      uint8   [n, k/2]                 two 4-bit codes per byte, low nibble = even k
             sym:      two's-complement q in [-8, 7]
             affine:   unsigned u in [0, 15]
             codebook: index j in [0, 15] into the row's 16-entry int8 codebook
  scales     float16 [n, k/group]
  bias       float16 [n, k/group]            affine only
  codebook   int8    [n, 16]                 codebook only
  (int8 weights: codes int8 [n, k], one signed byte per weight, with the same fp16 scales)
  (2-bit codebook: codes uint8 [n, k/4], four indices per byte, low bits = first k; codebook
  int8 [n, 4]; 1-bit: codes uint8 [n, k/8], bit i of byte b = index of k = 8b + i, codebook
  [n, 2]; 3-bit: codes uint8 [n, k], one index 0..7 per byte, codebook [n, 8])

Shapes and distributions follow the workloads the pages measure: Gemma-style decode GEMVs
(K=2048, gate_up N=16384, o_proj N=2048), a 128-row prefill chunk of a 5120-wide model's fused
gate|up (N=34816) with 4-bit affine group-64 weights, a 128-block rotated codebook layer
(K=1536, N=6144), and a K=1536 x 262144 vocabulary head.  Seeds: every array has its own
stream, ``PCG64(SeedSequence([2026, cfg, variant, stream]))`` with streams 0 = X, 1 = outlier
channels, 2 = W, 3 = codebook entries, 4 = codebook indices, 5 = codebook scales.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
import numpy as np

FMT_SYM, FMT_AFFINE, FMT_CODEBOOK, FMT_INT8, FMT_CQ2, FMT_CQ1, FMT_CQ3 = 0, 1, 2, 3, 4, 5, 6
FORMAT_NAMES = {FMT_SYM: "sym", FMT_AFFINE: "affine", FMT_CODEBOOK: "codebook", FMT_INT8: "int8",
                FMT_CQ2: "cq2", FMT_CQ1: "cq1", FMT_CQ3: "cq3"}
CQ_BITS = {FMT_CQ1: 1, FMT_CQ2: 2, FMT_CQ3: 3}

_W_CHUNK_ROWS = 8192  # W is drawn in fixed row chunks so large heads stay within memory


@dataclass(frozen=True)
class LayerConfig:
    name: str
    m: int
    k: int
    n: int
    group: int
    fmt: int
    hadamard: int            # 0 or the rotation block width
    x_outliers: int          # number of outlier input channels
    x_outlier_scale: float
    w_sigma: float
    cfg_id: int              # seed component for X
    x_variant: int
    w_variant: int           # configs that share W share this and cfg_id
    note: str = ""
    extra: dict = field(default_factory=dict)


CONFIGS = {
    "C1": LayerConfig("C1", 1, 1024, 1024, 64, FMT_SYM, 0, 0, 1.0, 0.02, 1, 0, 0,
                      "tiny decode GEMV"),
    "C2a": LayerConfig("C2a", 1, 2048, 16384, 64, FMT_SYM, 0, 8, 20.0, 0.02, 2, 0, 0,
                       "decode GEMV, gate_up-shaped"),
    "C2b": LayerConfig("C2b", 1, 2048, 2048, 64, FMT_SYM, 0, 8, 20.0, 0.02, 2, 1, 1,
                       "decode GEMV, o_proj-shaped"),
    "C3a": LayerConfig("C3a", 128, 5120, 34816, 64, FMT_AFFINE, 0, 0, 1.0, 0.015, 3, 0, 0,
                       "prefill GEMM, fused gate|up, affine 4-bit"),
    "C3b": LayerConfig("C3b", 65, 5120, 34816, 64, FMT_AFFINE, 0, 0, 1.0, 0.015, 3, 1, 0,
                       "prefill GEMM, odd M"),
    "C4": LayerConfig("C4", 1024, 1536, 6144, 128, FMT_CODEBOOK, 128, 0, 1.0, 0.0, 4, 0, 0,
                      "rotated codebook GEMM"),
    "C5a": LayerConfig("C5a", 1, 1536, 262144, 64, FMT_SYM, 0, 15, 15.0, 0.02, 5, 0, 0,
                       "vocabulary head, decode GEMV"),
    "C5b": LayerConfig("C5b", 64, 1536, 262144, 64, FMT_SYM, 0, 15, 15.0, 0.02, 5, 1, 0,
                       "vocabulary head, chunked prefill"),
    "C5o": LayerConfig("C5o", 1, 1536, 262144, 128, FMT_CODEBOOK, 128, 15, 15.0, 0.0, 6, 0, 0,
                       "orthogonal vocabulary head: rotated codebook weights, one scale per "
                       "row seen as K/128 groups", extra={"row_scale": True}),
}


def rng(cfg_id: int, variant: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, cfg_id, variant,
                                                                       stream])))


def config(name: str, **overrides) -> LayerConfig:
    """A named config, optionally with shape overrides (m, k, n, ...) for small test cases."""
    return replace(CONFIGS[name], **overrides)


def pack_nibbles(c: np.ndarray) -> np.ndarray:
    """[n, k] codes in 0..15 -> [n, k/2] bytes, low nibble = even k."""
    c = np.asarray(c, dtype=np.uint8)
    return (c[:, 0::2] & 0x0F) | ((c[:, 1::2] & 0x0F) << 4)


def pack_crumbs(c: np.ndarray) -> np.ndarray:
    """[n, k] 2-bit indices in 0..3 -> [n, k/4] bytes, index of k = 4b + i in bits 2i, 2i+1."""
    c = np.asarray(c, dtype=np.uint8) & 3
    return c[:, 0::4] | (c[:, 1::4] << 2) | (c[:, 2::4] << 4) | (c[:, 3::4] << 6)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """[n, k/2] bytes -> [n, k] codes 0..15 (inverse of pack_nibbles)."""
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty((b.shape[0], b.shape[1] * 2), np.uint8)
    out[:, 0::2] = b & 0x0F
    out[:, 1::2] = b >> 4
    return out


def make_x(cfg: LayerConfig) -> np.ndarray:
    """float32 [m, k]: standard normal, with whole outlier columns scaled."""
    x = rng(cfg.cfg_id, cfg.x_variant, 0).standard_normal((cfg.m, cfg.k), dtype=np.float32)
    if cfg.x_outliers:
        cols = rng(cfg.cfg_id, cfg.x_variant, 1).choice(cfg.k, size=cfg.x_outliers,
                                                        replace=False)
        x[:, np.sort(cols)] *= np.float32(cfg.x_outlier_scale)
    return x


def _quantize_weights_sym(w: np.ndarray, group: int):
    n, k = w.shape
    wg = w.reshape(n, k // group, group)
    s16 = (np.abs(wg).max(axis=2) / np.float32(7.0)).astype(np.float16)
    s32 = s16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s32 > 0, np.rint(wg / np.where(s32 > 0, s32, 1)), 0)
    q = np.clip(q, -8, 7).astype(np.int8).reshape(n, k)
    return (q.astype(np.uint8) & 0x0F), s16, None


def _quantize_weights_affine(w: np.ndarray, group: int):
    n, k = w.shape
    wg = w.reshape(n, k // group, group)
    lo = wg.min(axis=2)
    hi = wg.max(axis=2)
    s16 = ((hi - lo) / np.float32(15.0)).astype(np.float16)
    b16 = lo.astype(np.float16)
    s32 = s16.astype(np.float32)[:, :, None]
    b32 = b16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(s32 > 0, np.rint((wg - b32) / np.where(s32 > 0, s32, 1)), 0)
    u = np.clip(u, 0, 15).astype(np.uint8).reshape(n, k)
    return u, s16, b16


def make_weights(cfg: LayerConfig, full_range: bool = False):
    """Canonical (codes [n,k/2] u8, scales [n,k/g] f16, bias f16|None, codebook i8|None)."""
    n, k, g = cfg.n, cfg.k, cfg.group
    ng = k // g
    if cfg.fmt in CQ_BITS:
        ne = 1 << CQ_BITS[cfg.fmt]
        cb = np.clip(np.rint(40.0 * rng(cfg.cfg_id, cfg.w_variant, 3).standard_normal((n, ne))),
                     -127, 127).astype(np.int8)
        idx = rng(cfg.cfg_id, cfg.w_variant, 4).integers(0, ne, size=(n, k), dtype=np.uint8)
        sc = (rng(cfg.cfg_id, cfg.w_variant, 5).uniform(0.5, 1.5, size=(n, ng))
              * 5e-4).astype(np.float16)
        codes = (pack_crumbs(idx) if cfg.fmt == FMT_CQ2 else
                 np.packbits(idx, axis=1, bitorder="little") if cfg.fmt == FMT_CQ1 else idx)
        return codes, sc, None, cb
    if cfg.fmt == FMT_CODEBOOK:
        cb = np.clip(np.rint(40.0 * rng(cfg.cfg_id, cfg.w_variant, 3).standard_normal((n, 16))),
                     -127, 127).astype(np.int8)
        idx = rng(cfg.cfg_id, cfg.w_variant, 4).integers(0, 16, size=(n, k), dtype=np.uint8)
        cols = 1 if cfg.extra.get("row_scale") else ng
        sc = (rng(cfg.cfg_id, cfg.w_variant, 5).uniform(0.5, 1.5, size=(n, cols))
              * 5e-4).astype(np.float16)
        return pack_nibbles(idx), np.repeat(sc, ng // cols, axis=1), None, cb
    r = rng(cfg.cfg_id, cfg.w_variant, 2)
    if cfg.fmt == FMT_INT8:
        if full_range:
            c = r.integers(-127, 128, size=(n, k), dtype=np.int8)
            sc = (r.uniform(0.5, 1.5, size=(n, ng)) * cfg.w_sigma / 40.0).astype(np.float16)
            return c, sc, None, None
        codes = np.empty((n, k), np.int8)
        scales = np.empty((n, ng), np.float16)
        for r0 in range(0, n, _W_CHUNK_ROWS):
            rows = min(_W_CHUNK_ROWS, n - r0)
            w = r.standard_normal((rows, k), dtype=np.float32) * np.float32(cfg.w_sigma)
            wg = w.reshape(rows, ng, g)
            s16 = (np.abs(wg).max(axis=2) / np.float32(127.0)).astype(np.float16)
            s32 = s16.astype(np.float32)[:, :, None]
            with np.errstate(divide="ignore", invalid="ignore"):
                q = np.where(s32 > 0, np.rint(wg / np.where(s32 > 0, s32, 1)), 0)
            codes[r0:r0 + rows] = np.clip(q, -127, 127).astype(np.int8).reshape(rows, k)
            scales[r0:r0 + rows] = s16
        return codes, scales, None, None
    if full_range:
        c = r.integers(0, 16, size=(n, k), dtype=np.uint8)
        sc = (r.uniform(0.5, 1.5, size=(n, ng)) * cfg.w_sigma / 3.0).astype(np.float16)
        bias = None
        if cfg.fmt == FMT_AFFINE:
            bias = (-7.5 * sc.astype(np.float32)
                    + r.normal(0, cfg.w_sigma / 10, size=(n, ng))).astype(np.float16)
        return pack_nibbles(c), sc, bias, None
    codes = np.empty((n, k // 2), np.uint8)
    scales = np.empty((n, ng), np.float16)
    bias = np.empty((n, ng), np.float16) if cfg.fmt == FMT_AFFINE else None
    quant = _quantize_weights_sym if cfg.fmt == FMT_SYM else _quantize_weights_affine
    for r0 in range(0, n, _W_CHUNK_ROWS):
        rows = min(_W_CHUNK_ROWS, n - r0)
        w = r.standard_normal((rows, k), dtype=np.float32) * np.float32(cfg.w_sigma)
        c, s, b = quant(w, g)
        codes[r0:r0 + rows] = pack_nibbles(c)
        scales[r0:r0 + rows] = s
        if bias is not None:
            bias[r0:r0 + rows] = b
    return codes, scales, bias, None


def make(name_or_cfg, full_range: bool = False, **overrides):
    """All inputs of one layer: dict(cfg, x, codes, scales, bias, codebook)."""
    cfg = name_or_cfg if isinstance(name_or_cfg, LayerConfig) else config(name_or_cfg,
                                                                          **overrides)
    codes, scales, bias, cb = make_weights(cfg, full_range=full_range)
    out = dict(cfg=cfg, x=make_x(cfg), codes=codes, scales=scales, bias=bias, codebook=cb)
    if cfg.extra.get("row_scale"):      # the per-row values (every group of a row holds them)
        out["row_scales"] = np.ascontiguousarray(scales[:, 0])
        out["row_bias"] = None if bias is None else np.ascontiguousarray(bias[:, 0])
    return out


def weight_bytes(cfg: LayerConfig) -> int:
    """Algorithmic weight bytes: nibbles + fp16 scales (+ fp16 bias) (+ int8 codebook); one
    scale (and bias) per row for a row-scaled head."""
    per_row = 1 if cfg.extra.get("row_scale") else cfg.k // cfg.group
    b = (cfg.n * cfg.k * CQ_BITS[cfg.fmt] // 8 if cfg.fmt in CQ_BITS else
         cfg.n * cfg.k // (1 if cfg.fmt == FMT_INT8 else 2)) + 2 * cfg.n * per_row
    if cfg.fmt == FMT_AFFINE:
        b += 2 * cfg.n * per_row
    if cfg.fmt == FMT_CODEBOOK:
        b += 16 * cfg.n
    if cfg.fmt in CQ_BITS:
        b += (1 << CQ_BITS[cfg.fmt]) * cfg.n
    return b


def algorithmic_bytes(cfg: LayerConfig, fused_prep: bool = False) -> int:
    """Bytes one linear call must move: weights + xq + xs + xsum + fp32 y; with the prepass fused
    into the same kernel (one activation row), also the fp32 row read."""
    ng = cfg.k // cfg.group
    b = weight_bytes(cfg) + cfg.m * cfg.k + 8 * cfg.m * ng + 4 * cfg.m * cfg.n
    if fused_prep:
        b += 4 * cfg.m * cfg.k
    return b


def int_ops(cfg: LayerConfig) -> int:
    return 2 * cfg.m * cfg.n * cfg.k


# ---- prefill attention over a cached int8 segment
#
# Gemma-style heads: head_dim 256, 8 query heads sharing 2 key/value heads, a 256-query prefill
# chunk against a 1024-slot cache (the pages' 1068-token prompt), scores scaled by 1/sqrt(256).
# The cache holds int8 keys and values with one fp32 scale per 32 of the head dimension (the
# cache writer's quantization, done here as input preparation: scale = max|v| / 127, codes
# rounded to nearest even).  A sliding-window layer keeps `sink` positions and a rolled ring of
# the most recent ones.  Streams: 0 = Q, 1 = K, 2 = V, 3 = ring rotation.

@dataclass(frozen=True)
class AttnConfig:
    name: str
    nh: int
    nkvh: int
    nq: int
    nkv: int
    d: int
    window: int          # 0: global layer
    sink: int            # slots exempt from the window
    rolled: bool         # the cache is a ring (slot order is not position order)
    cfg_id: int
    pos0: int = -1       # first query's position (-1: right after the cache)


ATTN_CONFIGS = {
    "A1": AttnConfig("A1", 8, 2, 256, 1024, 256, 0, 0, False, 11),
    "A2": AttnConfig("A2", 8, 2, 256, 1024, 256, 512, 4, True, 12, pos0=1500),
}


def attn_config(name: str, **overrides) -> AttnConfig:
    return replace(ATTN_CONFIGS[name], **overrides)


def _quantize_groups(v: np.ndarray, group: int):
    vg = v.reshape(*v.shape[:-1], v.shape[-1] // group, group)
    s = (np.abs(vg).max(axis=-1) / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s[..., None] > 0, np.rint(vg / np.where(s[..., None] > 0, s[..., None], 1)),
                     0)
    return np.clip(q, -127, 127).astype(np.int8).reshape(v.shape), s


def make_attn(name_or_cfg, **overrides):
    """Inputs of one attention call: dict(cfg, q fp32 [nh, nq, d], k8/v8 int8 [nkvh, nkv, d],
    ks/vs fp32 [nkvh, nkv, d/32], kvpos int32 [nkv], pos0, scale)."""
    cfg = name_or_cfg if isinstance(name_or_cfg, AttnConfig) else attn_config(name_or_cfg,
                                                                              **overrides)
    q = rng(cfg.cfg_id, 0, 0).standard_normal((cfg.nh, cfg.nq, cfg.d), dtype=np.float32)
    kf = rng(cfg.cfg_id, 0, 1).standard_normal((cfg.nkvh, cfg.nkv, cfg.d), dtype=np.float32)
    vf = rng(cfg.cfg_id, 0, 2).standard_normal((cfg.nkvh, cfg.nkv, cfg.d), dtype=np.float32)
    k8, ks = _quantize_groups(kf, 32)
    v8, vs = _quantize_groups(vf, 32)
    pos0 = cfg.pos0 if cfg.pos0 >= 0 else cfg.nkv
    if cfg.rolled:
        ring = cfg.nkv - cfg.sink
        recent = np.arange(pos0 - ring, pos0, dtype=np.int64)
        shift = int(rng(cfg.cfg_id, 0, 3).integers(0, ring))
        kvpos = np.concatenate([np.arange(cfg.sink), np.roll(recent, shift)]).astype(np.int32)
    else:
        kvpos = np.arange(cfg.nkv, dtype=np.int32)
    return dict(cfg=cfg, q=q, k8=k8, ks=ks, v8=v8, vs=vs, kvpos=kvpos, pos0=pos0,
                scale=1.0 / np.sqrt(cfg.d))
