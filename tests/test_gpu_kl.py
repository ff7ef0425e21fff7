"""GPU parity of the indexer KL training path (score recompute -> loss and indexer gradients),
through the C ABI, against the CPU oracle.

Tolerances (no figure on the pages; derived from the arithmetic of the kernels):
  target   |err| <= 1e-4 max|target|: probabilities from fp32 logits (relative error of a few
           1e-6 at |z| of tens) and the forward's fp32 lse, renormalised in fp32;
  loss     |err| <= 1e-4 (1 + |loss|): fp32 scores (bf16 products, fp32 sums) and fp32 logs;
  dq_idx   |err| <= 4e-3 max|dq_idx| + 1e-7: bf16 output (2^-9 relative), G = dI w as a bf16
           pair (about 2^-17);
  dw       |err| <= 1e-3 max|dw| + 1e-7: fp32 sums;
  dk_idx   |err| <= 1e-3 max|dk_idx| + 1e-7: per (query, slot) contributions staged as 16-bit
           block floating point (2^-15 of the block maximum each), summed in fp32.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from tests import checks

pytestmark = pytest.mark.gpu

dev = "cuda"
DI = 128


def _dsa():
    import sparse_attention_12_amd as dsa
    return dsa


def _np(t):
    return t.detach().to("cpu").numpy()


def _inputs(T, H, Dqk, K, n_valid, Hi, seed, minus_one_frac=0.0, Tkv=None):
    Tkv = Tkv or T
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn((T, H, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    kv = (torch.randn((Tkv, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    q_idx = torch.randn((T, Hi, DI), generator=g).to(torch.bfloat16)
    k_idx = torch.randn((Tkv, DI), generator=g).to(torch.bfloat16)
    w = torch.randn((T, Hi), generator=g) / 8
    r = np.random.default_rng(seed)
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        hi = t + 1 if Tkv == T else Tkv
        n = min(n_valid, hi)
        sel = np.sort(r.choice(hi, size=n, replace=False))
        if minus_one_frac > 0:
            pos = np.flatnonzero(r.random(K) >= minus_one_frac)[:n]
            idx[t, pos] = sel[:pos.size]
        else:
            idx[t, :n] = sel
    return q, kv, q_idx, k_idx, w, idx


def _check(name, got, ref, rel, abs_=1e-7):
    got = np.asarray(got, np.float64)
    bar = rel * float(np.abs(ref).max()) + abs_
    err = checks.max_abs(got, ref)
    assert err <= bar, f"{name}: max-abs error {err:.3e} > {bar:.3e}"
    return err


def _run(q, kv, q_idx, k_idx, w, idx, lens, scale, grad, sink=None, workspace_rows=0,
         chunks=None):
    dsa = _dsa()
    qd, kvd = q.to(dev), kv.to(dev)
    idd = torch.from_numpy(idx).to(dev)
    lnd = None if lens is None else torch.from_numpy(lens).to(dev)
    skd = None if sink is None else torch.tensor(sink, dtype=torch.float32, device=dev)
    out, lse = dsa.sparse_mla_fwd(qd, kvd, idd, scale, lnd, sink=skd)
    target = dsa.indexer_kl_target(qd, kvd, idd, lse, scale, lnd)
    ws = None
    if workspace_rows:
        ws = torch.empty(dsa.indexer_kl_bwd_workspace_bytes(q.shape[0], kv.shape[0], idx.shape[1],
                                                           workspace_rows),
                         dtype=torch.uint8, device=dev)
    qi, ki, wd = q_idx.to(dev), k_idx.to(dev), w.to(dev)
    if chunks is None:
        loss, dq_idx, dw, dk_idx = dsa.indexer_kl_bwd(qi, ki, wd, idd, target, grad, lnd,
                                                      workspace=ws)
    else:
        dk_idx = torch.zeros((kv.shape[0], DI), dtype=torch.float32, device=dev)
        parts = []
        for r0 in range(0, q.shape[0], chunks):
            r1 = min(q.shape[0], r0 + chunks)
            parts.append(dsa.indexer_kl_bwd(qi[r0:r1], ki, wd[r0:r1], idd[r0:r1],
                                            target[r0:r1], grad,
                                            None if lnd is None else lnd[r0:r1], dk_idx=dk_idx,
                                            accumulate=True))
        loss = torch.cat([p[0] for p in parts])
        dq_idx = torch.cat([p[1] for p in parts])
        dw = torch.cat([p[2] for p in parts])
    torch.cuda.synchronize()
    return dict(target=_np(target), loss=_np(loss), dq_idx=_np(dq_idx.float()), dw=_np(dw),
                dk_idx=_np(dk_idx))


def _compare(gpu, ref):
    e = {"target": _check("target", gpu["target"], ref["target"], 1e-4),
         "dq_idx": _check("dq_idx", gpu["dq_idx"], ref["dq_idx"], 4e-3),
         "dw": _check("dw", gpu["dw"], ref["dw"], 1e-3),
         "dk_idx": _check("dk_idx", gpu["dk_idx"], ref["dk_idx"], 1e-3)}
    lerr = np.abs(gpu["loss"] - ref["loss"]) / (1 + np.abs(ref["loss"]))
    assert not np.isnan(gpu["loss"]).any() and lerr.max() <= 1e-4, f"loss {lerr.max():.3e}"
    e["loss"] = float(lerr.max())
    print({k: f"{v:.2e}" for k, v in e.items()}, flush=True)


@pytest.mark.parametrize("T,H,Dqk,K,n_valid,Hi", [(200, 64, 576, 128, 77, 64),
                                                  (130, 8, 512, 75, 70, 16),
                                                  (96, 16, 576, 64, 64, 8),
                                                  (64, 64, 576, 2051, 2051, 40)])
def test_kl_matches_oracle(T, H, Dqk, K, n_valid, Hi):
    q, kv, q_idx, k_idx, w, idx = _inputs(T, H, Dqk, K, n_valid, Hi, seed=T + H + Hi)
    scale = 1.0 / math.sqrt(Dqk)
    gpu = _run(q, kv, q_idx, k_idx, w, idx, None, scale, grad=0.5)
    ref = oracle.indexer_kl(q, kv, idx, None, scale, q_idx, k_idx, w, g=0.5)
    _compare(gpu, ref)


def test_kl_prefix_lengths_scattered_minus_one_and_sink():
    T, H, Dqk, K, Hi = 150, 64, 576, 100, 64
    q, kv, q_idx, k_idx, w, idx = _inputs(T, H, Dqk, K, 60, Hi, seed=21, minus_one_frac=0.3)
    scale = 1.0 / math.sqrt(Dqk)
    sink = np.linspace(-2.0, 2.0, H)
    gpu = _run(q, kv, q_idx, k_idx, w, idx, None, scale, grad=1.0, sink=sink)
    ref = oracle.indexer_kl(q, kv, idx, None, scale, q_idx, k_idx, w, g=1.0, sink=sink)
    _compare(gpu, ref)
    # prefix lengths: only the first len[t] slots are read (garbage after them)
    lens = np.minimum(np.arange(T) + 1, 37).astype(np.int32)
    idx2 = np.where(np.arange(K)[None, :] < lens[:, None],
                    np.minimum(np.arange(K)[None, :], np.arange(T)[:, None]), 7).astype(np.int32)
    gpu = _run(q, kv, q_idx, k_idx, w, idx2, lens, scale, grad=1.0)
    ref = oracle.indexer_kl(q, kv, idx2, lens, scale, q_idx, k_idx, w, g=1.0)
    _compare(gpu, ref)


def test_kl_local_queries_passes_and_chunks():
    """Query rows against a larger key set (T_q != T_kv); a workspace of 7 rows per pass and
    query chunks with accumulated key gradients give the one-pass result."""
    T, Tkv, H, Dqk, K, Hi = 90, 300, 16, 576, 64, 32
    q, kv, q_idx, k_idx, w, idx = _inputs(T, H, Dqk, K, 64, Hi, seed=33, Tkv=Tkv)
    scale = 1.0 / math.sqrt(Dqk)
    one = _run(q, kv, q_idx, k_idx, w, idx, None, scale, grad=2.0)
    ref = oracle.indexer_kl(q, kv, idx, None, scale, q_idx, k_idx, w, g=2.0)
    _compare(one, ref)
    many = _run(q, kv, q_idx, k_idx, w, idx, None, scale, grad=2.0, workspace_rows=7)
    chunked = _run(q, kv, q_idx, k_idx, w, idx, None, scale, grad=2.0, chunks=40)
    for other in (many, chunked):
        for k in ("loss", "dq_idx", "dw", "target"):
            np.testing.assert_array_equal(other[k], one[k])
        scale_ref = np.abs(one["dk_idx"]).max()
        assert np.abs(other["dk_idx"] - one["dk_idx"]).max() <= 1e-5 * scale_ref + 1e-7


def test_kl_empty_and_single_slot_rows():
    T, H, Dqk, K, Hi = 40, 16, 512, 16, 8
    q, kv, q_idx, k_idx, w, idx = _inputs(T, H, Dqk, K, 16, Hi, seed=5)
    idx[3] = -1          # no valid slot
    idx[4, :] = -1
    idx[4, 5] = 2        # one valid slot
    scale = 1.0 / math.sqrt(Dqk)
    gpu = _run(q, kv, q_idx, k_idx, w, idx, None, scale, grad=1.0)
    ref = oracle.indexer_kl(q, kv, idx, None, scale, q_idx, k_idx, w, g=1.0)
    _compare(gpu, ref)
    assert gpu["loss"][3] == 0.0 and not gpu["target"][3].any() and not gpu["dq_idx"][3].any()
    assert gpu["target"][4, 5] == 1.0 and abs(gpu["loss"][4]) <= 1e-6


@pytest.mark.parametrize("T,H,Dqk,K,n_valid,passes", [(200, 64, 576, 128, 77, 1),
                                                       (130, 8, 512, 75, 70, 3)])
def test_fused_target_from_the_attention_backward(T, H, Dqk, K, n_valid, passes):
    """dsa_sparse_mla_bwd_kl_target: dq and dkv as the plain backward, and the KL target within
    the target tolerance of the oracle (its P is staged in fp16: about 2^-12 per term)."""
    dsa = _dsa()
    q, kv, q_idx, k_idx, w, idx = _inputs(T, H, Dqk, K, n_valid, 8, seed=T + 3)
    idx[5] = -1  # a row without a valid slot
    scale = 1.0 / math.sqrt(Dqk)
    qd, kvd, idd = q.to(dev), kv.to(dev), torch.from_numpy(idx).to(dev)
    dout = torch.randn((T, H, 512), generator=torch.Generator().manual_seed(T)).to(
        torch.bfloat16).to(dev)
    out, lse = dsa.sparse_mla_fwd(qd, kvd, idd, scale)
    ws = torch.empty(dsa.bwd_workspace_bytes(T, T, H, Dqk, K, rows_per_pass=-(-T // passes)),
                     dtype=torch.uint8, device=dev)
    dq0, dkv0 = dsa.sparse_mla_bwd(qd, kvd, idd, out, lse, dout, scale, workspace=ws)
    tgt = torch.full((T, K), 5.0, dtype=torch.float32, device=dev)  # overwritten everywhere
    dq1, dkv1 = dsa.sparse_mla_bwd(qd, kvd, idd, out, lse, dout, scale, workspace=ws,
                                   kl_target=tgt)
    torch.cuda.synchronize()
    assert torch.equal(dq0, dq1)
    assert (dkv0 - dkv1).abs().max().item() <= 1e-5 * dkv0.abs().max().item() + 1e-6
    ref = oracle.indexer_kl(q, kv, idx, None, scale, q_idx, k_idx, w)
    e = _check("fused target", _np(tgt), ref["target"], 1e-4)
    assert not _np(tgt)[5].any()
    print(f"fused target {e:.2e}", flush=True)
