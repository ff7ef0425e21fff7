"""Comparison rules shared by the GPU parity tests (host side, numpy).

Tolerances (the stated parity bar of the DSA hot path): indices bit-exact when the indexer
inputs are exactly representable small integers with power-of-two weights; on float inputs a
top-k set mismatch is allowed only for keys whose exact score lies within 1e-5 (relative) of
the row's k-th score; attention output, dq and dkv within 2e-2 max-abs of the fp64 oracle;
LSE within 1e-3.
"""

from __future__ import annotations

import numpy as np

import oracle

ATOL_OUT = 2e-2
ATOL_LSE = 1e-3
NEAR_TIE_REL = 1e-5


def check_topk_structure(idx: np.ndarray, ln: np.ndarray, rows: np.ndarray, start: np.ndarray,
                         K: int):
    """Exact structure of every given row: len = min(K, L), ascending, unique, causal, -1 tail."""
    for r, t in enumerate(rows):
        L = t - start[r] + 1
        n = min(K, L)
        assert ln[r] == n, f"row {t}: len {ln[r]} != {n}"
        row = idx[r]
        assert (row[n:] == -1).all(), f"row {t}: -1 suffix broken"
        v = row[:n]
        assert (np.diff(v) > 0).all(), f"row {t}: not strictly ascending"
        assert v.min() >= start[r] and v.max() <= t, f"row {t}: non-causal index"


def check_topk_near_tie(q_rows, k_idx, w_rows, gpu_idx: np.ndarray, ora_idx: np.ndarray,
                        kth: np.ndarray, rows: np.ndarray):
    """Set equality up to near-ties; returns the number of mismatching keys.

    q_rows [n,H,D] / w_rows [n,H] hold the inputs of the n checked query rows (global row
    numbers ``rows``); gpu_idx, ora_idx and kth are per checked row."""
    q_rows = oracle._u16(q_rows)
    k_idx = oracle._u16(k_idx)
    w_rows = np.ascontiguousarray(oracle._np(w_rows, np.float32))
    mism = 0
    for r, t in enumerate(rows):
        g = set(gpu_idx[r][gpu_idx[r] >= 0].tolist())
        o = set(ora_idx[r][ora_idx[r] >= 0].tolist())
        diff = g ^ o
        if not diff:
            continue
        tau = kth[r]
        for s in diff:
            score = oracle.indexer_score_rows(q_rows[r], k_idx, w_rows[r], int(s))
            assert abs(score - tau) <= NEAR_TIE_REL * abs(tau), (
                f"row {t} key {s}: score {score} vs k-th {tau} is not a near tie")
        mism += len(diff)
    return mism


def check_topk_structure_device(idx, ln, seq_start, K: int):
    """check_topk_structure over every row at once, with torch ops on the tensors' device."""
    import torch
    T = idx.shape[0]
    t = torch.arange(T, device=idx.device, dtype=torch.int64)
    L = t - seq_start.to(torch.int64) + 1
    n = torch.clamp(L, max=K)
    bad = (ln.to(torch.int64) != n).nonzero()
    assert bad.numel() == 0, f"len wrong at rows {bad[:8].flatten().tolist()}"
    pos = torch.arange(K, device=idx.device, dtype=torch.int64)
    valid = pos[None, :] < n[:, None]
    iv = idx.to(torch.int64)
    assert bool(((iv == -1) | valid).all()), "-1 suffix broken"
    lo_ok = (iv >= seq_start.to(torch.int64)[:, None]) & (iv <= t[:, None])
    assert bool((lo_ok | ~valid).all()), "non-causal index"
    if K > 1:
        asc = (iv[:, 1:] > iv[:, :-1]) | ~valid[:, 1:]
        assert bool(asc.all()), "prefix not strictly ascending"


def max_abs(a, b) -> float:
    """Largest |a - b|.  Equal infinities (an empty row's LSE) count as zero error; a NaN on
    either side that the other side does not share, or unequal infinities, make it inf, so
    that assert_close fails on them."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    a, b = np.broadcast_arrays(a, b)
    if a.size == 0:
        return 0.0
    na, nb = np.isnan(a), np.isnan(b)
    if (na != nb).any():
        return float("inf")
    same = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))) | (na & nb)
    with np.errstate(invalid="ignore"):
        d = np.where(same, 0.0, np.abs(a - b))
    return float(d.max())


def assert_close(name, gpu, ref, atol):
    err = max_abs(gpu, ref)
    assert np.isfinite(err) and err <= atol, f"{name}: max-abs error {err:.3e} > {atol:.1e}"
    return err
