"""TV soft labels c* = 1 - 1/2 ||p_d - p_t||_1, fp64 oracle (test infrastructure only).

[P3] "DSpark Speculative Decoding", section "Confidence-Scheduled Verification": the
confidence head is supervised with c*_k = 1 - 1/2 ||p_d - p_t||_1. [P1] section
"硬件感知与置信度自适应调度机制" calls it the analytic acceptance rate obtained from the total
variation distance between the draft and target distributions. It equals
sum_v min(p_d(v), p_t(v)), the probability that the acceptance test keeps a token drawn
from p_d; both forms are computed and must agree.

Positions are k = 1..len[b]; later entries are NaN. A row whose logits are all -inf is
taken as the zero vector.
"""
from __future__ import annotations

import numpy as np

from .numerics import softmax_row


def tv_row_pair(ld_row, lt_row) -> float:
    V = np.asarray(ld_row).shape[0]
    sd = softmax_row(ld_row)
    st = softmax_row(lt_row)
    pd = sd[0] if sd is not None else np.zeros(V)
    pt = st[0] if st is not None else np.zeros(V)
    c_min = np.minimum(pd, pt).sum()
    c_l1 = 1.0 - 0.5 * np.abs(pd - pt).sum()
    if sd is not None and st is not None and abs(c_min - c_l1) > 1e-12:
        raise AssertionError(f"sum-min and L1 forms disagree: {c_min} vs {c_l1}")
    return float(c_min)


def tv_labels(Ld, Lt, t_off=None, length=None, requests=None):
    """c* [B][gamma] float64 for Ld [B][gamma][V] against flattened target rows Lt."""
    Ld = np.asarray(Ld)
    B, G, V = Ld.shape
    out = np.full((B, G), np.nan)
    todo = range(B) if requests is None else requests
    for b in todo:
        ell = G if length is None else int(length[b])
        off = b * (G + 1) if t_off is None else int(t_off[b])
        for k in range(ell):
            out[b, k] = tv_row_pair(Ld[b, k], Lt[off + k])
    return out
