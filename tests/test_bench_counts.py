"""The bench's algorithmic work counts (the numerators of every achieved rate and roofline
fraction) against brute-force sums over the rows of each workload."""

import numpy as np

import bench
import dsa_inputs as gen
import oracle


def _rows(cfg):
    """Causal length of every row of the workload."""
    cu = np.array(cfg.cu_seqlens, np.int64)
    return np.concatenate([np.arange(1, b - a + 1) for a, b in zip(cu[:-1], cu[1:])])


def test_token_workload_counts_match_brute_force():
    cfg = gen.workload(3)
    K, H, Dqk, Dv, Hi, Di = cfg.topk, cfg.heads, cfg.d_qk, cfg.d_v, cfg.idx_heads, cfg.idx_dim
    L = _rows(cfg)
    valid = int(np.minimum(L, K).sum())
    md = oracle.thd_metadata(cfg.cu_seqlens, cfg.T, K)
    assert int(md["topk_length"].astype(np.int64).sum()) == valid == 59_248_128
    c = bench.workload_counts(dict(total_valid=valid), cfg, Hi, Di, K, H, Dqk, Dv)
    # rows with L > K score every causal key; the others keep their prefix unscored
    assert c["idx_pairs"] == int(L[L > K].sum())
    assert c["idx_flops"] == c["idx_pairs"] * 2 * Hi * Di
    # forward: S = q.k over D_qk and P.V over D_v per (head, valid slot)
    assert c["fwd_flops"] == valid * H * (2 * Dqk + 2 * Dv)
    # backward: S and dP recomputed, dq = dZ.k, dk = dZ^T.q (D_qk), dv = P^T.dO (D_v)
    assert c["bwd_flops"] == valid * H * (2 * Dqk + 2 * Dv + 2 * Dqk + 2 * Dqk + 2 * Dv)


def test_kpool_pairs_match_brute_force():
    for cu, pool, kp in ([0, 65536], 4, 512), ([0, 37, 2100, 2103], 4, 128), ([0, 999], 3, 7):
        brute = 0
        for a, b in zip(cu[:-1], cu[1:]):
            for pos in range(b - a):
                P = (pos + 1) // pool  # complete pools the row sees
                if P > kp:
                    brute += P
        assert bench.kpool_pairs(cu, pool, kp) == brute
