"""GPU parity of the k-pool indexer (pools of keys scored by one pooled indexer key each, the
best pools expanded to their keys, then the query's incomplete tail pool) against the oracle.

Every input comes from dsa_inputs (seeded); expected values come from oracle/ only.
"""

import numpy as np
import pytest
import torch

import dsa_inputs as gen
import oracle
from tests import checks

pytestmark = pytest.mark.gpu

dev = "cuda"


def _dsa():
    import sparse_attention_12_amd as dsa
    return dsa


def _np(t):
    return t.detach().to("cpu").numpy()


def _run(inp, K_pools):
    dsa = _dsa()
    md = dsa.prepare_kpool_metadata(inp["cu_seqlens"].to(dev).to(torch.int32), inp["pool"],
                                    K_pools)
    idx, ln = dsa.kpool_indexer_topk(inp["q_idx"].to(dev), inp["k_pool"].to(dev),
                                     inp["w"].to(dev), md, K_pools)
    torch.cuda.synchronize()
    return idx, ln, md


def _row_coords(cu, pool):
    """Per row: first key of its sequence, first pool row of its sequence, complete pools seen."""
    cu = np.asarray(cu, np.int64)
    T = int(cu[-1])
    ks = np.zeros(T, np.int64)
    cp = np.zeros(T, np.int64)
    P = np.zeros(T, np.int64)
    c = 0
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        ks[s0:s1] = s0
        cp[s0:s1] = c
        P[s0:s1] = (np.arange(s0, s1) - s0 + 1) // pool
        c += (s1 - s0) // pool
    return ks, cp, P


def _check_structure(idx, ln, rows, ks, P, pool, K_pools):
    """Exact layout of each given row: n = min(K_pools, P) whole pools in ascending order, then
    the tail pool's keys, then -1; returns the selected pools (sequence-relative) per row."""
    out = []
    for r, t in enumerate(rows):
        n = min(K_pools, int(P[r]))
        tail = int(t - ks[r] + 1 - P[r] * pool)
        assert 0 <= tail < pool
        assert ln[r] == n * pool + tail, f"row {t}: len {ln[r]} != {n * pool + tail}"
        row = idx[r].astype(np.int64)
        assert (row[n * pool + tail:] == -1).all(), f"row {t}: -1 suffix broken"
        sel = row[:n * pool].reshape(n, pool) - ks[r]
        first = sel[:, 0]
        assert (first % pool == 0).all(), f"row {t}: a pool does not start on a pool boundary"
        assert (sel == first[:, None] + np.arange(pool)[None, :]).all(), f"row {t}: pool split"
        assert (np.diff(first) > 0).all(), f"row {t}: pools not strictly ascending"
        assert n == 0 or (first[-1] // pool) < P[r], f"row {t}: pool beyond the row"
        np.testing.assert_array_equal(row[n * pool:n * pool + tail],
                                      ks[r] + P[r] * pool + np.arange(tail),
                                      err_msg=f"row {t}: tail pool")
        out.append(first // pool)
    return out


@pytest.mark.parametrize("cu,pool,K_pools,H,D", [
    ([0, 3, 4, 1000, 1001, 2600], 4, 64, 64, 128),
    ([0, 1500, 1502, 3100], 3, 200, 64, 128),
    ([0, 900, 2000], 4, 100, 8, 64),
    ([0, 5, 2200], 16, 7, 33, 128),
])
def test_kpool_integer_inputs_bit_exact(cu, pool, K_pools, H, D):
    """Small integers with power-of-two weights: every pool score is exact, so the selection,
    ties to the lower pool included, must match the oracle bit for bit on every row."""
    inp = gen.kpool_indexer_inputs(1, cu_seqlens=cu, pool=pool, heads=H, dim=D, int_inputs=True)
    idx, ln, md = _run(inp, K_pools)
    assert md.total_key_tokens == inp["k_pool"].shape[0]
    ridx, rln = oracle.kpool_indexer(inp["q_idx"], inp["k_pool"], inp["w"], inp["cu_seqlens"],
                                     pool, K_pools)
    np.testing.assert_array_equal(_np(ln), rln)
    np.testing.assert_array_equal(_np(idx), ridx)


@pytest.mark.parametrize("cu,pool,K_pools", [([0, 4000], 4, 512), ([0, 37, 2100, 2103], 4, 128),
                                             ([0, 3000], 4, 1)])
def test_kpool_float_inputs_near_tie(cu, pool, K_pools):
    """N(0,1) inputs: exact layout on every row; against the oracle on sampled rows, a pool may
    differ only when its exact score is a near tie with the row's K_pools-th best."""
    inp = gen.kpool_indexer_inputs(3, cu_seqlens=cu, pool=pool)
    idx, ln, _ = _run(inp, K_pools)
    idx, ln = _np(idx), _np(ln)
    T = cu[-1]
    ks, cp, P = _row_coords(cu, pool)
    rows = np.arange(T)
    _check_structure(idx, ln, rows, ks, P, pool, K_pools)
    samp = np.unique(np.concatenate([np.arange(max(0, T - 8), T),
                                     np.linspace(0, T - 1, 24).astype(np.int64)]))
    for t in samp:
        ridx, rln, kth = oracle.kpool_indexer(inp["q_idx"], inp["k_pool"], inp["w"],
                                              inp["cu_seqlens"], pool, K_pools,
                                              rows=(int(t), int(t) + 1))
        assert rln[0] == ln[t]
        mine = _check_structure(idx[t:t + 1], ln[t:t + 1], [t], ks[t:t + 1], P[t:t + 1], pool,
                                K_pools)[0] + cp[t]
        ref = _check_structure(ridx, rln, [t], ks[t:t + 1], P[t:t + 1], pool, K_pools)[0] + cp[t]
        checks.check_topk_near_tie(inp["q_idx"][t:t + 1], inp["k_pool"], inp["w"][t:t + 1],
                                   mine[None, :], ref[None, :], kth, np.array([t]))


def test_kpool_unit_pool_equals_token_indexer():
    """pool = 1: one indexer key per key and no tail, so the k-pool path is the token-level
    indexer; integer inputs, compared with the oracle's token-level top-k."""
    cu = [0, 700, 2900]
    K = 256
    inp = gen.kpool_indexer_inputs(1, cu_seqlens=cu, pool=1, int_inputs=True)
    idx, ln, _ = _run(inp, K)
    ridx, rln, _ = oracle.indexer_topk(inp["q_idx"], inp["k_pool"], inp["w"], inp["cu_seqlens"],
                                       K)
    np.testing.assert_array_equal(_np(ln), rln)
    np.testing.assert_array_equal(_np(idx), ridx)


def test_kpool_metadata_rejected_by_token_indexer_and_mismatch():
    dsa = _dsa()
    inp = gen.kpool_indexer_inputs(1, cu_seqlens=[0, 300], pool=4, int_inputs=True)
    md = dsa.prepare_kpool_metadata(inp["cu_seqlens"].to(dev), 4, 16)
    q, kp, w = inp["q_idx"].to(dev), inp["k_pool"].to(dev), inp["w"].to(dev)
    with pytest.raises(ValueError, match="k-pool metadata"):
        dsa.indexer_topk(q, kp, w, md, 16)
    with pytest.raises((RuntimeError, ValueError)):
        dsa.kpool_indexer_topk(q, kp, w, md, 32)
    tmd = dsa.prepare_thd_metadata(inp["cu_seqlens"].to(dev), 16)
    with pytest.raises((RuntimeError, ValueError)):
        dsa.kpool_indexer_topk(q, kp, w, tmd, 16)
    with pytest.raises(ValueError, match="pool=0"):
        dsa.prepare_kpool_metadata(inp["cu_seqlens"].to(dev), 0, 16)
    # a row that sees no complete pool and a sequence shorter than one pool
    inp = gen.kpool_indexer_inputs(1, cu_seqlens=[0, 2, 3, 9], pool=4, int_inputs=True)
    idx, ln, _ = _run(inp, 4)
    ridx, rln = oracle.kpool_indexer(inp["q_idx"], inp["k_pool"], inp["w"], inp["cu_seqlens"],
                                     4, 4)
    np.testing.assert_array_equal(_np(ln), rln)
    np.testing.assert_array_equal(_np(idx), ridx)


def test_kpool_full_size_T65536():
    """One causal sequence of 65536 tokens, pools of 4, the 512 best pools (width 2051), 64
    indexer heads of 128: exact layout of every row on the device, oracle on sampled rows."""
    T, pool, K_pools = 65536, 4, 512
    cu = [0, T]
    inp = gen.kpool_indexer_inputs(4, pool=pool)
    assert inp["k_pool"].shape == (T // pool, 128)
    idx_d, ln_d, _ = _run(inp, K_pools)
    W = K_pools * pool + pool - 1
    assert idx_d.shape == (T, W)
    # device-side layout of every row
    t = torch.arange(T, device=dev, dtype=torch.int64)
    P = (t + 1) // pool
    n = torch.clamp(P, max=K_pools)
    tail = t + 1 - P * pool
    assert bool((ln_d.to(torch.int64) == n * pool + tail).all())
    j = torch.arange(W, device=dev, dtype=torch.int64)[None, :]
    iv = idx_d.to(torch.int64)
    sel = j < (n * pool)[:, None]
    tl = (j >= (n * pool)[:, None]) & (j < (n * pool + tail)[:, None])
    assert bool(((iv == -1) | sel | tl).all()), "-1 suffix broken"
    assert bool(((iv % pool == j % pool) | ~sel).all()), "pool split"
    assert bool(((iv < (P * pool)[:, None]) | ~sel).all()), "pool beyond the row"
    exp_tail = (P * pool)[:, None] + (j - (n * pool)[:, None])
    assert bool(((iv == exp_tail) | ~tl).all()), "tail pool"
    asc = (iv[:, 1:] > iv[:, :-1]) | ~(sel[:, 1:] | tl[:, 1:])
    assert bool(asc.all()), "not strictly ascending"
    idx, ln = _np(idx_d), _np(ln_d)
    del idx_d, ln_d
    ks, cp, Pn = _row_coords(cu, pool)
    samp = np.unique(np.concatenate([[0, 3, 2046, 2047, 2048, 2049, 2050, 2051, 2052, 4099],
                                     np.arange(T - 4, T),
                                     np.linspace(2100, T - 5, 10).astype(np.int64)]))
    for s in samp:
        ridx, rln, kth = oracle.kpool_indexer(inp["q_idx"], inp["k_pool"], inp["w"],
                                              inp["cu_seqlens"], pool, K_pools,
                                              rows=(int(s), int(s) + 1))
        assert rln[0] == ln[s]
        mine = _check_structure(idx[s:s + 1], ln[s:s + 1], [s], ks[s:s + 1], Pn[s:s + 1], pool,
                                K_pools)[0] + cp[s]
        ref = _check_structure(ridx, rln, [s], ks[s:s + 1], Pn[s:s + 1], pool, K_pools)[0] + cp[s]
        checks.check_topk_near_tie(inp["q_idx"][s:s + 1], inp["k_pool"], inp["w"][s:s + 1],
                                   mine[None, :], ref[None, :], kth, np.array([s]))
