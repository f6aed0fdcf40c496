"""Shared helpers of the GPU parity tests: device transfer, the oracle side of a layer, and the
acceptance check on fp32 outputs (relative L2 error <= 1e-5 and, per element,
|err| <= 1e-4 * sum of the magnitudes of the terms)."""
from __future__ import annotations

import numpy as np

import oracle

REL_L2_MAX = 1e-5
TERM_FRAC_MAX = 1e-4


def to_dev(a, device="cuda:0"):
    import torch
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def check_y(y_gpu, y_ref, terms, what=""):
    """Acceptance of an fp32 output against the fp64 oracle output and its term magnitudes."""
    yg = np.asarray(y_gpu, dtype=np.float64).reshape(y_ref.shape)
    err = np.abs(yg - y_ref)
    nrm = np.linalg.norm(y_ref)
    rel = np.linalg.norm(yg - y_ref) / nrm if nrm > 0 else np.linalg.norm(yg - y_ref)
    bad = err > TERM_FRAC_MAX * terms
    assert rel <= REL_L2_MAX, f"{what}: relative L2 error {rel:.3e} > {REL_L2_MAX}"
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements exceed 1e-4*T, worst "
                           f"{float((err / np.maximum(terms, 1e-300)).max()):.3e}")
    return rel


def oracle_layer(L, cols=None):
    """Oracle prep and output for a generated layer dict, optionally on a subset of columns."""
    cfg = L["cfg"]
    xq, xs, xsum = oracle.prep(L["x"], cfg.group, cfg.hadamard)
    sel = (lambda a: a) if cols is None else (lambda a: None if a is None else a[cols])
    y, t = oracle.linear(cfg.fmt, sel(L["codes"]), sel(L["scales"]), xq, xs, xsum, cfg.group,
                         bias_f16=sel(L["bias"]), codebook=sel(L["codebook"]))
    return dict(xq=xq, xs=xs, xsum=xsum, y=y, t=t)
