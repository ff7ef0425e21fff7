"""GPU parity of the indexer on scores with a trend along each sequence.

The indexer's compactions may raise a row's threshold speculatively, from the keys seen so far;
a row whose later keys score lower than that sample suggests ends with fewer than K keys above
its threshold and is recomputed by the second launch.  Falling scores force that path on every
long row, rising ones the opposite (many compactions, no recompute).  Integer inputs make every
score exact, so the indices must match the oracle bit for bit; for falling scores the answer
is also known in closed form (the first K keys of the row: ties go to the lower position).

Every input comes from dsa_inputs (seeded); expected values come from oracle/ only.
"""

import numpy as np
import pytest
import torch

import dsa_inputs as gen
import oracle

pytestmark = pytest.mark.gpu

dev = "cuda"


def _dsa():
    import sparse_attention_12_amd as dsa
    return dsa


def _run(inp, K, times=None):
    """The indexer on inp; with `times` (a dict), the durations of its two launches (ms)."""
    dsa = _dsa()
    md = dsa.prepare_thd_metadata(inp["cu_seqlens"].to(dev), K)
    args = (inp["q_idx"].to(dev), inp["k_idx"].to(dev), inp["w"].to(dev))
    torch.cuda.synchronize()
    timer = None
    if times is not None:
        from bench import KernelTimer
        timer = KernelTimer(dsa.lib(), 8)
        timer.arm()
    try:
        idx, ln = dsa.indexer_topk(*args, md, K)
        torch.cuda.synchronize()
    finally:
        if timer is not None:
            timer.disarm()
    if timer is not None:
        times.update({n: sum(v) for n, v in timer.totals().items()})
    return idx.cpu().numpy(), ln.cpu().numpy()


def _sample_rows(cu, n=6):
    rows = []
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        rows += list(np.unique(np.linspace(s0, s1 - 1, n).astype(np.int64)))
    return rows


# block: keys per score level; a speculative threshold then lands inside a level below the
# K-th key's, and every key of that level is kept, so K must not be a sum of whole levels that
# the threshold reaches (with 512 and levels of 256 the kept levels make exactly K)
@pytest.mark.parametrize("cu,K,block", [([0, 16384], 2048, 256),
                                        ([0, 3000, 12000, 12001, 20000], 2048, 256),
                                        ([0, 9000], 512, 64)])
def test_falling_scores_first_keys(cu, K, block):
    inp = gen.indexer_trend_inputs(cu, "falling", block=block)
    times = {}
    idx, ln = _run(inp, K, times)
    # the rows long enough to speculate failed and were recomputed: the second launch did real
    # work (with scores like a uniform sample it takes a hundredth of the first)
    assert times["indexer_topk_redo"] > 0.2 * times["indexer_topk"], times
    T = cu[-1]
    start = np.zeros(T, np.int64)
    for b in range(len(cu) - 1):
        start[cu[b]:cu[b + 1]] = cu[b]
    L = np.arange(T) - start + 1
    n = np.minimum(L, K)
    np.testing.assert_array_equal(ln, n)
    j = np.arange(K)[None, :]
    exp = np.where(j < n[:, None], start[:, None] + j, -1)
    np.testing.assert_array_equal(idx, exp)
    for t in _sample_rows(cu, 3):
        ridx, rln, _ = oracle.indexer_topk(inp["q_idx"], inp["k_idx"], inp["w"],
                                           inp["cu_seqlens"], K, rows=(int(t), int(t) + 1))
        np.testing.assert_array_equal(idx[t:t + 1], ridx)
        np.testing.assert_array_equal(ln[t:t + 1], rln)


@pytest.mark.parametrize("heads,dim", [(16, 128), (64, 64), (24, 64)])
def test_falling_scores_other_shapes(heads, dim):
    """The kernel instances for up to 32 heads (one 32-row MFMA tile) and for 64-wide indexer
    keys take the same speculation and second launch: closed form on every row."""
    cu, K = [0, 12000], 1024
    inp = gen.indexer_trend_inputs(cu, "falling", heads=heads, dim=dim, block=128)
    times = {}
    idx, ln = _run(inp, K, times)
    assert times["indexer_topk_redo"] > 0.2 * times["indexer_topk"], times
    n = np.minimum(np.arange(cu[-1]) + 1, K)
    j = np.arange(K)[None, :]
    np.testing.assert_array_equal(ln, n)
    np.testing.assert_array_equal(idx, np.where(j < n[:, None], j, -1))


@pytest.mark.parametrize("cu,K", [([0, 16384], 2048), ([0, 5000, 11000], 1024)])
def test_rising_scores_against_oracle(cu, K):
    inp = gen.indexer_trend_inputs(cu, "rising")
    times = {}
    idx, ln = _run(inp, K, times)
    assert times["indexer_topk_redo"] < 0.1 * times["indexer_topk"], times
    for t in _sample_rows(cu, 8):
        ridx, rln, _ = oracle.indexer_topk(inp["q_idx"], inp["k_idx"], inp["w"],
                                           inp["cu_seqlens"], K, rows=(int(t), int(t) + 1))
        np.testing.assert_array_equal(idx[t:t + 1], ridx, err_msg=f"row {t}")
        np.testing.assert_array_equal(ln[t:t + 1], rln)


def test_kpool_falling_pool_scores_first_pools():
    """The k-pool indexer (the same kernel over pooled keys, rows in key coordinates) with pool
    scores falling along the sequence: every row that sees enough pools to speculate is
    recomputed, and keeps its first K_pools pools, then its tail pool (closed form), equal to
    the oracle on sampled rows."""
    dsa = _dsa()
    T, pool, K_pools = 40000, 4, 512
    cu = [0, T]
    n_pools = T // pool
    kin = gen.indexer_trend_inputs([0, n_pools], "falling", heads=8, block=64)
    qin = gen.indexer_trend_inputs(cu, "falling", heads=8)
    q, kp, w = qin["q_idx"], kin["k_idx"], qin["w"]
    md = dsa.prepare_kpool_metadata(torch.tensor(cu, dtype=torch.int32, device=dev), pool, K_pools)
    from bench import KernelTimer
    timer = KernelTimer(dsa.lib(), 8)
    timer.arm()
    try:
        idx_d, ln_d = dsa.kpool_indexer_topk(q.to(dev), kp.to(dev), w.to(dev), md, K_pools)
        torch.cuda.synchronize()
    finally:
        timer.disarm()
    times = {n: sum(v) for n, v in timer.totals().items()}
    assert times["indexer_topk_redo"] > 0.2 * times["indexer_topk"], times
    idx, ln = idx_d.cpu().numpy(), ln_d.cpu().numpy()
    t = np.arange(T)
    P = (t + 1) // pool
    n = np.minimum(P, K_pools)
    tail = t + 1 - P * pool
    np.testing.assert_array_equal(ln, n * pool + tail)
    W = K_pools * pool + pool - 1
    j = np.arange(W)[None, :]
    exp = np.where(j < (n * pool)[:, None], j,
                   np.where(j < (n * pool + tail)[:, None],
                            (P * pool)[:, None] + j - (n * pool)[:, None], -1))
    np.testing.assert_array_equal(idx, exp)
    for r in [0, 2051, 2052, 15000, T - 1]:
        ridx, rln, _ = oracle.kpool_indexer(q, kp, w, torch.tensor(cu, dtype=torch.int32), pool,
                                            K_pools, rows=(r, r + 1))
        np.testing.assert_array_equal(idx[r:r + 1], ridx)
        np.testing.assert_array_equal(ln[r:r + 1], rln)


def test_mixed_batch_recomputes_only_failed_groups():
    """A falling-score sequence packed with a random one: rows of both kinds in one launch,
    the second launch recomputing the failed groups among them; both sequences are checked
    (closed form for the first, the oracle with the near-tie rule on sampled rows of the
    second)."""
    from tests import checks
    L0, L1, K = 16384, 12288, 2048
    a = gen.indexer_trend_inputs([0, L0], "falling")
    b = gen.indexer_inputs(3, cu_seqlens=[0, L1])
    inp = dict(q_idx=torch.cat([a["q_idx"], b["q_idx"]]).contiguous(),
               k_idx=torch.cat([a["k_idx"], b["k_idx"]]).contiguous(),
               w=torch.cat([a["w"], b["w"]]).contiguous(),
               cu_seqlens=torch.tensor([0, L0, L0 + L1], dtype=torch.int32))
    times = {}
    idx, ln = _run(inp, K, times)
    assert times["indexer_topk_redo"] > 0.1 * times["indexer_topk"], times
    L = np.arange(L0) + 1
    n = np.minimum(L, K)
    j = np.arange(K)[None, :]
    np.testing.assert_array_equal(ln[:L0], n)
    np.testing.assert_array_equal(idx[:L0], np.where(j < n[:, None], j, -1))
    rows = np.unique(np.concatenate([np.linspace(L0, L0 + L1 - 1, 12).astype(np.int64),
                                     [L0 + K - 1, L0 + K, L0 + L1 - 1]]))
    for t in rows:
        ridx, rln, kth = oracle.indexer_topk(inp["q_idx"], inp["k_idx"], inp["w"],
                                             inp["cu_seqlens"], K, rows=(int(t), int(t) + 1))
        assert ln[t] == rln[0]
        checks.check_topk_near_tie(inp["q_idx"][t:t + 1], inp["k_idx"], inp["w"][t:t + 1],
                                   idx[t:t + 1], ridx, kth, np.array([t]))


def test_local_rows_falling_scores_two_ranks():
    """Local query rows in global padded coordinates (two ranks' zig-zag chunks, padding rows
    and one masked row) with falling scores: the second launch recomputes the long rows through
    the local-row metadata; every real row keeps the first K keys of its sequence in padded
    storage, padding and masked rows are empty."""
    dsa = _dsa()
    cu, cu_pad, K = [0, 14000], [0, 14336], 1024
    T, Tk = cu[-1], cu_pad[-1]
    inp = gen.indexer_trend_inputs(cu, "falling", block=128)
    kp = torch.zeros((Tk, inp["k_idx"].shape[1]), dtype=torch.bfloat16)
    kp[:T] = inp["k_idx"]                       # one sequence from 0: coordinates equal rows
    kp[T:] = 7.0                                # padding rows: junk that must never be picked
    chunks = np.array_split(np.arange(T), 4)
    ranks = [np.concatenate([chunks[0], chunks[3]]), np.concatenate([chunks[1], chunks[2]])]
    for r, rows in enumerate(ranks):
        qi = np.concatenate([rows, [14100, 14335]]).astype(np.int32)    # two padding positions
        qr = torch.cat([inp["q_idx"][rows], inp["q_idx"][:2]]).contiguous()
        wr = torch.cat([inp["w"][rows], inp["w"][:2]]).contiguous()
        mask = np.zeros(qi.size, bool)
        mask[len(rows) // 2] = True
        md = dsa.prepare_local_metadata(torch.tensor(cu, dtype=torch.int32, device=dev), Tk, K,
                                        cu_seqlens_padded=torch.tensor(cu_pad, dtype=torch.int32,
                                                                       device=dev),
                                        query_indices=torch.from_numpy(qi).to(dev),
                                        padding_mask=torch.from_numpy(mask).to(dev))
        from bench import KernelTimer
        timer = KernelTimer(dsa.lib(), 8)
        timer.arm()
        try:
            idx_d, ln_d = dsa.indexer_topk(qr.to(dev), kp.to(dev), wr.to(dev), md, K)
            torch.cuda.synchronize()
        finally:
            timer.disarm()
        times = {n: sum(v) for n, v in timer.totals().items()}
        assert times["indexer_topk_redo"] > 0.1 * times["indexer_topk"], times
        idx, ln = idx_d.cpu().numpy(), ln_d.cpu().numpy()
        n = np.minimum(qi.astype(np.int64) + 1, K)
        n[len(rows):] = 0
        n[len(rows) // 2] = 0
        j = np.arange(K)[None, :]
        np.testing.assert_array_equal(ln, n, err_msg=f"rank {r} lengths")
        np.testing.assert_array_equal(idx, np.where(j < n[:, None], j, -1),
                                      err_msg=f"rank {r} indices")
