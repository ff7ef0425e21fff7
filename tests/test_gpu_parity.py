"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, small and ragged sizes.

Every input comes from dsa_inputs (seeded); expected values come from oracle/ only.
"""

import math

import numpy as np
import pytest
import torch

import dsa_inputs as gen
import oracle
from tests import checks, pins

pytestmark = pytest.mark.gpu

dev = "cuda"


def _dsa():
    import sparse_attention_12_amd as dsa
    return dsa


def _np(t):
    return t.detach().to("cpu").numpy()


# ----------------------------------------------------------------------------------------
# metadata
# ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("cu", [[0, 1024, 4096, 16384, 32768], [0, 0, 5, 5, 9, 300, 301],
                                [0, 7], [0, 2049, 2050, 6000]])
def test_metadata_matches_oracle(cu):
    dsa = _dsa()
    T = cu[-1]
    K = 2048
    md = dsa.prepare_thd_metadata(torch.tensor(cu, dtype=torch.int32, device=dev), K)
    torch.cuda.synchronize()
    ref = oracle.thd_metadata(np.array(cu, np.int32), T, K)
    np.testing.assert_array_equal(_np(md.seq_start), ref["seq_start"])
    np.testing.assert_array_equal(_np(md.causal_len), ref["causal_len"])
    np.testing.assert_array_equal(_np(md.topk_length), ref["topk_length"])
    assert md.max_seqlen == ref["max_seqlen"]
    assert md.total_pairs == int(ref["causal_len"].astype(np.int64).sum())
    assert md.total_valid == int(ref["topk_length"].astype(np.int64).sum())
    order = _np(md.row_order)
    assert sorted(order.tolist()) == list(range(T))
    L = ref["causal_len"][order]
    assert (np.diff(L) <= 0).all()
    groups = _np(md.groups)
    lens = np.diff(cu)
    assert md.n_groups == int(((lens + 3) // 4).sum())
    # every row is covered by exactly one group of <= 4 consecutive rows
    covered = np.zeros(T, np.int32)
    for last in groups:
        s = ref["seq_start"][last]
        covered[max(s, last - 3): last + 1] += 1
    assert (covered == 1).all()
    costs = ref["causal_len"][groups]
    assert (np.diff(costs) <= 0).all()


def test_metadata_rejects_bad_offsets():
    dsa = _dsa()
    with pytest.raises(ValueError):
        dsa.prepare_thd_metadata(torch.tensor([0, 5, 3], dtype=torch.int32, device=dev))
    with pytest.raises(ValueError):
        dsa.prepare_thd_metadata(torch.tensor([1, 5], dtype=torch.int32, device=dev))


# ----------------------------------------------------------------------------------------
# indexer
# ----------------------------------------------------------------------------------------

def _run_indexer(inp, K):
    dsa = _dsa()
    md = dsa.prepare_thd_metadata(inp["cu_seqlens"].to(dev).to(torch.int32), K)
    idx, ln = dsa.indexer_topk(inp["q_idx"].to(dev), inp["k_idx"].to(dev), inp["w"].to(dev),
                               md, K)
    torch.cuda.synchronize()
    return _np(idx), _np(ln)


def test_indexer_integer_inputs_bit_exact():
    """Tiny workload (T=256, 4 heads x 64, integers in [-4,4], weights in {0.5,1,2}, k=64)."""
    w = gen.workload(1)
    inp = gen.indexer_inputs(1)
    idx, ln = _run_indexer(inp, w.topk)
    ridx, rln, _ = oracle.indexer_topk(inp["q_idx"], inp["k_idx"], inp["w"], inp["cu_seqlens"],
                                       w.topk)
    np.testing.assert_array_equal(ln, rln)
    np.testing.assert_array_equal(idx, ridx)


@pytest.mark.parametrize("cu,K,H,D", [([0, 700], 64, 64, 128), ([0, 100, 1000, 1300], 256, 64, 128),
                                      ([0, 3000], 2048, 64, 128), ([0, 5000], 1000, 40, 64),
                                      ([0, 4200], 1, 8, 128)])
def test_indexer_float_inputs_near_tie(cu, K, H, D):
    inp = gen.indexer_inputs(2, cu_seqlens=cu)
    inp = dict(inp, q_idx=inp["q_idx"][:, :H].contiguous(), w=inp["w"][:, :H].contiguous())
    if D != inp["k_idx"].shape[1]:
        inp = dict(inp, q_idx=inp["q_idx"][..., :D].contiguous(),
                   k_idx=inp["k_idx"][:, :D].contiguous())
    idx, ln = _run_indexer(inp, K)
    T = cu[-1]
    rows = np.arange(T)
    start = oracle.thd_metadata(np.array(cu, np.int32), T, K)["seq_start"]
    checks.check_topk_structure(idx, ln, rows, start, K)
    # oracle on a sample: the longest rows and a spread of others
    samp = np.unique(np.concatenate([np.arange(max(0, T - 12), T),
                                     np.linspace(0, T - 1, 24).astype(np.int64)]))
    for t in samp:
        ridx, rln, kth = oracle.indexer_topk(inp["q_idx"], inp["k_idx"], inp["w"],
                                             inp["cu_seqlens"], K, rows=(int(t), int(t) + 1))
        assert rln[0] == ln[t]
        checks.check_topk_near_tie(inp["q_idx"][t:t + 1], inp["k_idx"], inp["w"][t:t + 1],
                                   idx[t:t + 1], ridx, kth, np.array([t]))


@pytest.mark.parametrize("H,D", [(64, 128), (1, 128), (32, 64), (33, 128)])
def test_indexer_integer_inputs_thd_long_rows_bit_exact(H, D):
    """Integer inputs over long rows (many compaction rounds) and several sequences: exact; at
    the head counts and key widths where the kernel instances change."""
    cu = [0, 70, 2500, 2501, 9000]
    g = torch.Generator().manual_seed(77)
    T, K = cu[-1], 512
    q = torch.randint(-4, 5, (T, H, D), generator=g).to(torch.bfloat16)
    k = torch.randint(-4, 5, (T, D), generator=g).to(torch.bfloat16)
    w = torch.tensor([0.5, 1.0, 2.0, 0.25])[torch.randint(0, 4, (T, H), generator=g)]
    inp = dict(q_idx=q, k_idx=k, w=w, cu_seqlens=torch.tensor(cu, dtype=torch.int32))
    idx, ln = _run_indexer(inp, K)
    rows = (0, 10, 69, 70, 71, 600, 2499, 2500, 2501, 2600, 5000, 8997, 8998, 8999)
    for t in rows:
        ridx, rln, _ = oracle.indexer_topk(q, k, w, inp["cu_seqlens"], K, rows=(t, t + 1))
        assert rln[0] == ln[t], t
        np.testing.assert_array_equal(idx[t], ridx[0], err_msg=f"row {t}")


# ----------------------------------------------------------------------------------------
# sparse MLA forward / backward
# ----------------------------------------------------------------------------------------

def _random_indices(T, Tkv, K, n_valid, seed, minus_one_frac=0.0, causal=True):
    g = np.random.default_rng(seed)
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        hi = (t + 1) if causal else Tkv
        n = min(n_valid, hi)
        sel = np.sort(g.choice(hi, size=n, replace=False))
        idx[t, :n] = sel
        if minus_one_frac > 0:
            pos = g.random(K) < minus_one_frac
            row = idx[t].copy()
            idx[t] = -1
            keep = row[row >= 0]
            slots = np.flatnonzero(~pos)[: keep.size]
            idx[t, slots] = keep[: slots.size]
    return idx


def _fwd_bwd_case(T, H, Dqk, K, n_valid, seed, minus_one_frac=0.0, use_len=False,
                  check_bwd=True, Tkv=None):
    dsa = _dsa()
    Tkv = Tkv or T
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn((T, H, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    kv = (torch.randn((Tkv, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    idx = _random_indices(T, Tkv, K, n_valid, seed, minus_one_frac, causal=Tkv == T)
    lens = None
    if use_len:
        lens = (idx >= 0).sum(1).astype(np.int32)
        # canonical prefix: move valid entries to the front, garbage after the prefix
        idx = np.where(np.arange(K)[None, :] < lens[:, None], np.sort(np.where(idx >= 0, idx,
                       np.iinfo(np.int32).max), axis=1), 12345 % Tkv).astype(np.int32)
    scale = 1.0 / math.sqrt(Dqk)
    idx_t = torch.from_numpy(idx)
    len_t = None if lens is None else torch.from_numpy(lens)
    out, lse = dsa.sparse_mla_fwd(q.to(dev), kv.to(dev), idx_t.to(dev), scale,
                                  None if len_t is None else len_t.to(dev))
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_mla_fwd(q, kv, idx, lens, scale, 512)
    checks.assert_close("out", _np(out.float()), ro, checks.ATOL_OUT)
    checks.assert_close("lse", _np(lse), rl, checks.ATOL_LSE)
    if not check_bwd:
        return
    dq, dkv = dsa.sparse_mla_bwd(q.to(dev), kv.to(dev), idx_t.to(dev), out, lse, dout.to(dev),
                                 scale, None if len_t is None else len_t.to(dev))
    torch.cuda.synchronize()
    rdq, rdkv = oracle.sparse_mla_bwd(q, kv, idx, lens, dout, scale)
    checks.assert_close("dq", _np(dq.float()), rdq, checks.ATOL_OUT)
    checks.assert_close("dkv", _np(dkv), rdkv, checks.ATOL_OUT)


@pytest.mark.parametrize("T,H,Dqk,K,n_valid", [(96, 16, 576, 64, 64), (200, 64, 576, 128, 77),
                                               (130, 8, 512, 75, 70), (64, 20, 576, 40, 33),
                                               (50, 64, 512, 2051, 2051),
                                               # head counts at the kernels' boundaries
                                               (70, 1, 576, 40, 40), (70, 32, 512, 64, 50),
                                               (70, 33, 576, 64, 64), (70, 48, 576, 96, 90)])
def test_fwd_bwd_matches_oracle(T, H, Dqk, K, n_valid):
    _fwd_bwd_case(T, H, Dqk, K, n_valid, seed=T * 7 + H)


def test_fwd_bwd_minus_one_slots_scattered():
    _fwd_bwd_case(120, 64, 576, 96, 50, seed=3, minus_one_frac=0.3)


def test_fwd_bwd_topk_length_prefix():
    _fwd_bwd_case(150, 16, 576, 100, 60, seed=4, use_len=True)


def test_fwd_bwd_query_rows_differ_from_key_rows():
    """Local queries against a larger gathered key set (T_q != T_kv)."""
    _fwd_bwd_case(40, 64, 576, 64, 64, seed=5, Tkv=333)


@pytest.mark.parametrize("H", [64, 40])
def test_fwd_rows_with_late_dominant_logits(H):
    """Rows whose first 32 slots are all masked, or whose later logits exceed every logit of
    the first 32 slots by far (one-hot softmax) or by about 2^20 (large unnormalised weights):
    the forward's fast path for 33..64 heads scales each head by a reference taken from the
    first chunk and must hand such rows to the exact path."""
    dsa = _dsa()
    T, Tkv, K, D = 24, 200, 96, 576
    g = torch.Generator().manual_seed(21)
    q = (torch.randn((T, H, D), generator=g) * 0.5)
    kv = (torch.randn((Tkv, D), generator=g) * 0.5)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    idx = np.stack([np.sort(np.random.default_rng(t).choice(Tkv - 2, K, replace=False))
                    for t in range(T)]).astype(np.int32)
    idx[0, :32] = -1                      # chunk 0 fully masked
    idx[1, :40] = -1                      # chunk 0 masked, chunk 1 partly
    for t, row, mag in ((2, Tkv - 1, 2.0), (3, Tkv - 2, 0.6), (4, Tkv - 1, 2.0)):
        q[t] = 1.0
        idx[t, 70] = row                  # slot in the third chunk
        idx[t, (idx[t] == row) & (np.arange(K) != 70)] = -1
        kv[row] = mag
    for t in (2, 3, 4):
        kv[idx[t, :32][idx[t, :32] >= 0]] *= 0.02
    q, kv = q.to(torch.bfloat16), kv.to(torch.bfloat16)
    scale = 1.0 / 24.0
    idx_t = torch.from_numpy(idx).to(dev)
    out, lse = dsa.sparse_mla_fwd(q.to(dev), kv.to(dev), idx_t, scale)
    dq, dkv = dsa.sparse_mla_bwd(q.to(dev), kv.to(dev), idx_t, out, lse, dout.to(dev), scale)
    torch.cuda.synchronize()
    assert not torch.isnan(lse).any()
    ro, rl = oracle.sparse_mla_fwd(q, kv, idx, None, scale, 512)
    checks.assert_close("out", _np(out.float()), ro, checks.ATOL_OUT)
    checks.assert_close("lse", _np(lse), rl, checks.ATOL_LSE)
    rdq, rdkv = oracle.sparse_mla_bwd(q, kv, idx, None, dout, scale)
    checks.assert_close("dq", _np(dq.float()), rdq, checks.ATOL_OUT)
    checks.assert_close("dkv", _np(dkv), rdkv, checks.ATOL_OUT)


@pytest.mark.parametrize("rows_per_pass", [17, 1])
def test_bwd_passes_over_two_staging_buffers(rows_per_pass):
    """A workspace that holds only a few query rows: the backward runs in passes over two
    staging buffers, each pass's key-gradient reduction on the library's helper stream while
    the next pass computes.  dq must equal the one-pass result exactly (rows are independent),
    dkv up to summation order, and both must match the oracle."""
    dsa = _dsa()
    T, H, D, K = 150, 64, 576, 96
    g = torch.Generator().manual_seed(31)
    q = (torch.randn((T, H, D), generator=g) * 0.5).to(torch.bfloat16)
    kv = (torch.randn((T, D), generator=g) * 0.5).to(torch.bfloat16)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    idx = _random_indices(T, T, K, 80, seed=32, minus_one_frac=0.1)
    scale = 1.0 / math.sqrt(D)
    qd, kvd, dd, idx_t = q.to(dev), kv.to(dev), dout.to(dev), torch.from_numpy(idx).to(dev)
    out, lse = dsa.sparse_mla_fwd(qd, kvd, idx_t, scale)
    dq1, dkv1 = dsa.sparse_mla_bwd(qd, kvd, idx_t, out, lse, dd, scale)
    ws = torch.empty(dsa.bwd_workspace_bytes(T, T, H, D, K, rows_per_pass), dtype=torch.uint8,
                     device=dev)
    assert ws.numel() < dsa.bwd_workspace_bytes(T, T, H, D, K, 0)
    dq2, dkv2 = dsa.sparse_mla_bwd(qd, kvd, idx_t, out, lse, dd, scale, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq2)
    assert (dkv1 - dkv2).abs().max().item() <= 1e-4
    rdq, rdkv = oracle.sparse_mla_bwd(q, kv, idx, None, dout, scale)
    checks.assert_close("dq", _np(dq2.float()), rdq, checks.ATOL_OUT)
    checks.assert_close("dkv", _np(dkv2), rdkv, checks.ATOL_OUT)


def test_fwd_bwd_wide_dynamic_range():
    """Rows of q, dO and the latent rows scaled by powers of two over several octaves: the
    backward's per-row fp16 operand scales (largest |q| and |dO| of the row, largest |kv|) and
    the 16-bit block staging must keep every row's relative accuracy.  Each tensor is compared
    row by row against the oracle, relative to that row's largest magnitude (the absolute bar
    of the other tests assumes unit-scale values)."""
    dsa = _dsa()
    T, H, Dqk, K = 300, 64, 576, 128
    g = torch.Generator().manual_seed(4242)
    qs = torch.pow(2.0, torch.randint(-5, 4, (T, 1, 1), generator=g).float())
    ds = torch.pow(2.0, torch.randint(-6, 7, (T, 1, 1), generator=g).float())
    ks = torch.pow(2.0, torch.randint(-3, 3, (T, 1), generator=g).float())
    q = (torch.randn((T, H, Dqk), generator=g) * 0.5 * qs).to(torch.bfloat16)
    kv = (torch.randn((T, Dqk), generator=g) * 0.5 * ks).to(torch.bfloat16)
    dout = (torch.randn((T, H, 512), generator=g) * ds).to(torch.bfloat16)
    idx = _random_indices(T, T, K, K, 4242)
    scale = 1.0 / math.sqrt(Dqk)
    idx_t = torch.from_numpy(idx).to(dev)
    out, lse = dsa.sparse_mla_fwd(q.to(dev), kv.to(dev), idx_t, scale)
    dq, dkv = dsa.sparse_mla_bwd(q.to(dev), kv.to(dev), idx_t, out, lse, dout.to(dev), scale)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_mla_fwd(q, kv, idx, None, scale, 512)
    rdq, rdkv = oracle.sparse_mla_bwd(q, kv, idx, None, dout, scale)
    checks.assert_close("lse", _np(lse), rl, checks.ATOL_LSE)

    def rel_rows(name, got, ref, tol, floor):
        """Row error within tol of the row's largest |ref|, or of `floor` (the size of one
        term of the row before cancellation) where the row cancels to about zero."""
        got = got.reshape(got.shape[0], -1).astype(np.float64)
        ref = ref.reshape(ref.shape[0], -1).astype(np.float64)
        assert np.isfinite(got).all(), f"{name}: non-finite values"
        err = np.abs(got - ref).max(1)
        lim = tol * np.maximum(np.abs(ref).max(1), floor)
        zero = lim == 0.0                      # rows that no slot touches: exactly zero
        assert (err[zero] == 0.0).all(), f"{name}: nonzero values in rows that must be zero"
        worst = float((err[~zero] / lim[~zero]).max()) * tol if (~zero).any() else 0.0
        print(f"{name}: worst row error {worst:.3e} of its scale")
        assert (err[~zero] <= lim[~zero]).all(), f"{name}: worst row error {worst:.3e} of its scale"

    # dq of (t, h) cancels to about zero where the softmax is peaked; there its error is set by
    # Delta = dO . O formed from the bf16 output (each term rounded by up to 2^-9 of itself),
    # which enters dq as scale * dDelta * sum_j P_j kv_j: the floor below is 4 times that bound
    kf = oracle._np(kv.float(), np.float64)
    of = _np(out.float()).astype(np.float64)
    dfl = oracle._np(dout.float(), np.float64)
    d_delta = 2.0 ** -9 * np.abs(dfl * of).sum(-1)                       # [T, H]
    dq_floor = 4.0 * scale * d_delta * np.abs(kf).max() / 1e-2
    rel_rows("out", _np(out.float()), ro, 1e-2, 0.0)
    rel_rows("dq", _np(dq.float()).reshape(T * H, -1), rdq.reshape(T * H, -1), 1e-2,
             dq_floor.reshape(-1))
    rel_rows("dkv", _np(dkv), rdkv, 2e-2, 0.0)


def test_tiny_workload_end_to_end():
    """Tiny workload: indexer (bit-exact) -> forward -> backward vs the oracle."""
    dsa = _dsa()
    w = gen.workload(1)
    ii = gen.indexer_inputs(1)
    ai = gen.attention_inputs(1)
    md = dsa.prepare_thd_metadata(ii["cu_seqlens"].to(dev), w.topk)
    idx, ln = dsa.indexer_topk(ii["q_idx"].to(dev), ii["k_idx"].to(dev), ii["w"].to(dev), md,
                               w.topk)
    out, lse = dsa.sparse_mla_fwd(ai["q"].to(dev), ai["kv"].to(dev), idx, ai["scale"], ln)
    dq, dkv = dsa.sparse_mla_bwd(ai["q"].to(dev), ai["kv"].to(dev), idx, out, lse,
                                 ai["dout"].to(dev), ai["scale"], ln)
    torch.cuda.synchronize()
    ridx, rln, _ = oracle.indexer_topk(ii["q_idx"], ii["k_idx"], ii["w"], ii["cu_seqlens"],
                                       w.topk)
    np.testing.assert_array_equal(_np(idx), ridx)
    ro, rl = oracle.sparse_mla_fwd(ai["q"], ai["kv"], ridx, rln, ai["scale"], 512)
    checks.assert_close("out", _np(out.float()), ro, checks.ATOL_OUT)
    checks.assert_close("lse", _np(lse), rl, checks.ATOL_LSE)
    rdq, rdkv = oracle.sparse_mla_bwd(ai["q"], ai["kv"], ridx, rln, ai["dout"], ai["scale"])
    checks.assert_close("dq", _np(dq.float()), rdq, checks.ATOL_OUT)
    checks.assert_close("dkv", _np(dkv), rdkv, checks.ATOL_OUT)


def test_empty_rows_and_single_slot_rows():
    dsa = _dsa()
    T, H, D = 6, 16, 576
    g = torch.Generator().manual_seed(9)
    q = (torch.randn((T, H, D), generator=g) * 0.5).to(torch.bfloat16)
    kv = (torch.randn((T, D), generator=g) * 0.5).to(torch.bfloat16)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    idx = np.full((T, 5), -1, np.int32)
    idx[1, 3] = 0
    idx[3, 0] = 2
    idx[4, :2] = [1, 4]
    out, lse = dsa.sparse_mla_fwd(q.to(dev), kv.to(dev), torch.from_numpy(idx).to(dev), 0.04)
    dq, dkv = dsa.sparse_mla_bwd(q.to(dev), kv.to(dev), torch.from_numpy(idx).to(dev), out, lse,
                                 dout.to(dev), 0.04)
    torch.cuda.synchronize()
    o, l = _np(out.float()), _np(lse)
    for t in (0, 2, 5):
        assert (o[t] == 0).all() and np.isneginf(l[t]).all() and (_np(dq[t].float()) == 0).all()
    # single valid slot: out equals the value row (bf16 exact)
    np.testing.assert_array_equal(o[1], np.broadcast_to(_np(kv[0, :512].float()), o[1].shape))
    ro, rl = oracle.sparse_mla_fwd(q, kv, idx, None, 0.04, 512)
    checks.assert_close("lse", l, rl, checks.ATOL_LSE)
    rdq, rdkv = oracle.sparse_mla_bwd(q, kv, idx, None, dout, 0.04)
    checks.assert_close("dq", _np(dq.float()), rdq, checks.ATOL_OUT)
    checks.assert_close("dkv", _np(dkv), rdkv, checks.ATOL_OUT)


def test_chunked_equals_one_shot():
    """SkyRL PR 2423: query chunks are independent; key gradients summed over chunks
    (accumulate flag) equal the one-shot key gradients up to summation order."""
    dsa = _dsa()
    T = 700
    ai = gen.attention_inputs(4, cu_seqlens=[0, T])
    idx = gen.kpool_indices(T, topk=131, tail=3).to(dev)
    q, kv, dout = ai["q"].to(dev), ai["kv"].to(dev), ai["dout"].to(dev)
    out, lse = dsa.sparse_mla_fwd(q, kv, idx, ai["scale"])
    dq, dkv = dsa.sparse_mla_bwd(q, kv, idx, out, lse, dout, ai["scale"])
    dkv_c = torch.zeros_like(dkv)
    for r0, r1 in [(0, 256), (256, 512), (512, 700)]:
        oc, lc = dsa.sparse_mla_fwd(q[r0:r1], kv, idx[r0:r1].contiguous(), ai["scale"])
        assert torch.equal(oc, out[r0:r1]) and torch.equal(lc, lse[r0:r1])
        dqc, _ = dsa.sparse_mla_bwd(q[r0:r1], kv, idx[r0:r1].contiguous(), oc, lc,
                                    dout[r0:r1].contiguous(), ai["scale"], dkv=dkv_c,
                                    accumulate=True)
        assert torch.equal(dqc, dq[r0:r1])
    torch.cuda.synchronize()
    assert (dkv_c - dkv).abs().max().item() <= 1e-3


def test_debug_index_check_rejects_out_of_range():
    dsa = _dsa()
    T, H, D = 8, 16, 576
    q = torch.zeros((T, H, D), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((T, D), dtype=torch.bfloat16, device=dev)
    idx = torch.zeros((T, 4), dtype=torch.int32, device=dev)
    out, lse = dsa.sparse_mla_fwd(q, kv, idx, 0.1)
    bad = idx.clone()
    bad[3, 2] = T  # out of range: only caught by the debug check, before any kernel reads it
    with pytest.raises(ValueError, match="out of range"):
        dsa.sparse_mla_bwd(q, kv, bad, out, lse, torch.zeros_like(out), 0.1,
                           check_indices=True)


# ----------------------------------------------------------------------------------------
# attention sink (one zero-valued logit per head in the softmax denominator)
# ----------------------------------------------------------------------------------------

def _sink_values(H, seed):
    g = np.random.default_rng(seed)
    s = (g.standard_normal(H) * 2.0).astype(np.float32)
    s[0] = 8.0                # dominates every row of head 0
    if H > 2:
        s[1] = -np.inf        # no sink for head 1
    return s


def _dsink_bound(ro, rl, dout, sink):
    """Bound on |dsink_gpu - dsink_oracle| from the arithmetic: the kernels form
    Delta = dO . out' from the bf16 output (rounded to nearest, then rescaled and rounded once
    more: relative error below 2^-8 per element), weighted by the sink probability; plus fp32
    accumulation slack."""
    p_sink = np.exp(np.where(np.isneginf(sink), -np.inf, sink)[None, :] - rl)
    p_sink = np.where(np.isfinite(p_sink), p_sink, 0.0)
    mag = (np.abs(pins.bf16_to_f64(dout)) * np.abs(ro)).sum(-1)          # [T, H]
    return (p_sink * mag).sum(0) * 2.0 ** -7 + 1e-3


@pytest.mark.parametrize("T,H,Dqk,K,n_valid", [(96, 16, 576, 64, 64), (200, 64, 576, 128, 77),
                                               (130, 8, 512, 75, 70)])
def test_sink_fwd_bwd_matches_oracle(T, H, Dqk, K, n_valid):
    dsa = _dsa()
    g = torch.Generator().manual_seed(T + 11 * H)
    q = (torch.randn((T, H, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    kv = (torch.randn((T, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    idx = _random_indices(T, T, K, n_valid, seed=T + H, minus_one_frac=0.1)
    sink = _sink_values(H, seed=H)
    scale = 1.0 / math.sqrt(Dqk)
    sk = torch.from_numpy(sink).to(dev)
    idx_t = torch.from_numpy(idx).to(dev)
    out, lse = dsa.sparse_mla_fwd(q.to(dev), kv.to(dev), idx_t, scale, sink=sk)
    dq, dkv, dsink = dsa.sparse_mla_bwd(q.to(dev), kv.to(dev), idx_t, out, lse, dout.to(dev),
                                        scale, sink=sk)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_mla_fwd(q, kv, idx, None, scale, 512, sink=sink)
    checks.assert_close("out", _np(out.float()), ro, checks.ATOL_OUT)
    checks.assert_close("lse", _np(lse), rl, checks.ATOL_LSE)
    rdq, rdkv, rds = oracle.sparse_mla_bwd(q, kv, idx, None, dout, scale, sink=sink)
    checks.assert_close("dq", _np(dq.float()), rdq, checks.ATOL_OUT)
    checks.assert_close("dkv", _np(dkv), rdkv, checks.ATOL_OUT)
    err = np.abs(_np(dsink).astype(np.float64) - rds)
    bound = _dsink_bound(ro, rl, dout, sink)
    assert (err <= bound).all(), f"dsink error {err.max():.3e} above its bound {bound.min():.3e}"
    assert rds[1] == 0.0 and _np(dsink)[1] == 0.0   # the -inf sink has no gradient


def test_sink_empty_rows_minus_inf_sink_and_chunks():
    """Empty rows: out' = 0, lse' = sink, dq = 0.  sink = -inf everywhere equals no sink
    bitwise.  Query chunks with accumulate sum dsink (and dkv) like the one-shot call."""
    dsa = _dsa()
    T, H, D, K = 300, 64, 576, 96
    g = torch.Generator().manual_seed(21)
    q = (torch.randn((T, H, D), generator=g) * 0.5).to(torch.bfloat16).to(dev)
    kv = (torch.randn((T, D), generator=g) * 0.5).to(torch.bfloat16).to(dev)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16).to(dev)
    idx = _random_indices(T, T, K, 80, seed=22)
    idx[[0, 7, 150]] = -1                                  # three empty rows
    idx_t = torch.from_numpy(idx).to(dev)
    sink = torch.from_numpy(_sink_values(H, seed=5)).to(dev)
    out, lse = dsa.sparse_mla_fwd(q, kv, idx_t, 0.04, sink=sink)
    dq, dkv, dsink = dsa.sparse_mla_bwd(q, kv, idx_t, out, lse, dout, 0.04, sink=sink)
    torch.cuda.synchronize()
    for t in (0, 7, 150):
        assert not out[t].any() and not dq[t].any()
        assert torch.equal(lse[t], sink)
    o0, l0 = dsa.sparse_mla_fwd(q, kv, idx_t, 0.04)
    om, lm = dsa.sparse_mla_fwd(q, kv, idx_t, 0.04, sink=torch.full((H,), -math.inf, device=dev))
    torch.cuda.synchronize()
    assert torch.equal(om, o0) and torch.equal(lm, l0)
    dkv_c = torch.zeros_like(dkv)
    ds_c = torch.zeros_like(dsink)
    for r0, r1 in [(0, 128), (128, 300)]:
        oc, lc = dsa.sparse_mla_fwd(q[r0:r1], kv, idx_t[r0:r1], 0.04, sink=sink)
        assert torch.equal(oc, out[r0:r1]) and torch.equal(lc, lse[r0:r1])
        dqc, _, _ = dsa.sparse_mla_bwd(q[r0:r1], kv, idx_t[r0:r1], oc, lc, dout[r0:r1], 0.04,
                                       dkv=dkv_c, accumulate=True, sink=sink, dsink=ds_c)
        assert torch.equal(dqc, dq[r0:r1])
    torch.cuda.synchronize()
    assert (dkv_c - dkv).abs().max().item() <= 1e-5 * dkv.abs().max().item() + 1e-4
    assert (ds_c - dsink).abs().max().item() <= 1e-5 * dsink.abs().max().item() + 1e-4


# ----------------------------------------------------------------------------------------
# local query rows against gathered global keys (padded-storage coordinates)
# ----------------------------------------------------------------------------------------

def test_local_indexer_padded_storage_two_ranks_bit_exact():
    """Two ranks each own zig-zag chunks of the real tokens (global padded coordinates), plus a
    few padding coordinates and one masked row; integer inputs make every top-k set unique, so
    each rank's indices equal the oracle's exactly.  Rows reach 2000 keys (many tiles and
    compaction rounds) and groups are cut at chunk and sequence boundaries."""
    dsa = _dsa()
    cu, cu_pad, K, H, D = [0, 700, 1900, 2450], [0, 768, 2000, 2560], 300, 64, 128
    T, Tk = cu[-1], cu_pad[-1]
    g = torch.Generator().manual_seed(31)
    qf = torch.randint(-4, 5, (T, H, D), generator=g).to(torch.bfloat16)
    wf = torch.tensor([0.5, 1.0, 2.0, 0.25])[torch.randint(0, 4, (T, H), generator=g)]
    kc = torch.randint(-4, 5, (T, D), generator=g).to(torch.bfloat16)
    kp = torch.randint(-4, 5, (Tk, D), generator=g).to(torch.bfloat16)   # padding rows: junk
    seq = np.searchsorted(np.array(cu), np.arange(T), side="right") - 1
    coord = (np.arange(T) + np.array(cu_pad)[seq] - np.array(cu)[seq]).astype(np.int32)
    kp[torch.from_numpy(coord).long()] = kc
    chunks = np.array_split(np.arange(T), 8)
    ranks = [np.concatenate([chunks[0], chunks[3], chunks[4], chunks[7]]),
             np.concatenate([chunks[1], chunks[2], chunks[5], chunks[6]])]
    extra_coord = np.array([705, 720, 1999, 2555], np.int32)          # padding positions
    for r, rows in enumerate(ranks):
        qi = np.concatenate([coord[rows], extra_coord]).astype(np.int32)
        qr = torch.cat([qf[rows], qf[:4]])
        wr = torch.cat([wf[rows], wf[:4]])
        mask = np.zeros(qi.size, bool)
        mask[len(rows) // 2] = True                                     # one masked real row
        md = dsa.prepare_local_metadata(torch.tensor(cu, dtype=torch.int32, device=dev), Tk, K,
                                        cu_seqlens_padded=torch.tensor(cu_pad, dtype=torch.int32,
                                                                       device=dev),
                                        query_indices=torch.from_numpy(qi).to(dev),
                                        padding_mask=torch.from_numpy(mask).to(dev))
        idx, ln = dsa.indexer_topk(qr.to(dev).contiguous(), kp.to(dev), wr.to(dev).contiguous(),
                                   md, K)
        torch.cuda.synchronize()
        ridx, rln = oracle.indexer_topk_local(qr.contiguous(), kp, wr.contiguous(), cu, K,
                                              cu_seqlens_padded=cu_pad, query_indices=qi,
                                              padding_mask=mask)
        np.testing.assert_array_equal(_np(ln), rln, err_msg=f"rank {r} lengths")
        np.testing.assert_array_equal(_np(idx), ridx, err_msg=f"rank {r} indices")
        assert (rln[-4:] == 0).all() and rln[len(rows) // 2] == 0
        # metadata of a real row: its sequence start in padded storage and its causal length
        i = 0
        b = seq[rows[i]]
        assert int(md.seq_start[i]) == cu_pad[b]
        assert int(md.causal_len[i]) == rows[i] - cu[b] + 1


def test_local_indexer_unordered_rows_duplicates_and_errors():
    """Local rows in any order (groups of one row where neighbours are not consecutive keys),
    a coordinate listed twice, and float inputs: every row equals the oracle up to near ties.
    Coordinates outside the padded storage and offsets that are not ordered are rejected."""
    dsa = _dsa()
    cu, cu_pad, K, H, D = [0, 300, 1200], [0, 320, 1300], 128, 64, 128
    T, Tk = cu[-1], cu_pad[-1]
    inp = gen.indexer_inputs(2, cu_seqlens=cu)
    kc = inp["k_idx"]
    g = torch.Generator().manual_seed(12)
    kp = torch.randn((Tk, D), generator=g).to(torch.bfloat16)
    seq = np.searchsorted(np.array(cu), np.arange(T), side="right") - 1
    coord = (np.arange(T) + np.array(cu_pad)[seq] - np.array(cu)[seq]).astype(np.int32)
    kp[torch.from_numpy(coord).long()] = kc
    perm = np.random.default_rng(5).permutation(T)[:400]
    rows = np.concatenate([perm, perm[:1]])                     # the first row twice
    qi = coord[rows]
    qr = inp["q_idx"][torch.from_numpy(rows).long()].contiguous()
    wr = inp["w"][torch.from_numpy(rows).long()].contiguous()
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    cp_d = torch.tensor(cu_pad, dtype=torch.int32, device=dev)
    md = dsa.prepare_local_metadata(cu_d, Tk, K, cu_seqlens_padded=cp_d,
                                    query_indices=torch.from_numpy(qi).to(dev))
    idx, ln = dsa.indexer_topk(qr.to(dev), kp.to(dev), wr.to(dev), md, K)
    torch.cuda.synchronize()
    gi, gl = _np(idx), _np(ln)
    assert np.array_equal(gi[0], gi[-1]) and gl[0] == gl[-1]
    # oracle on the compact layout (local row i is compact row rows[i]), mapped to padded
    shift = (np.array(cu_pad)[seq] - np.array(cu)[seq])[rows]
    for i in range(0, len(rows), 37):
        t = int(rows[i])
        ridx, rln, kth = oracle.indexer_topk(inp["q_idx"], inp["k_idx"], inp["w"], cu, K,
                                             rows=(t, t + 1))
        assert rln[0] == gl[i]
        ridx_p = np.where(ridx >= 0, ridx + shift[i], -1)
        # compare in compact coordinates (the near-tie check scores against the compact keys)
        gi_c = np.where(gi[i:i + 1] >= 0, gi[i:i + 1] - shift[i], -1)
        checks.check_topk_near_tie(inp["q_idx"][t:t + 1], inp["k_idx"], inp["w"][t:t + 1],
                                   gi_c, ridx, kth, np.array([t]))
        assert ((gi[i] >= 0) == (ridx_p[0] >= 0)).all()
    with pytest.raises(ValueError, match="outside"):
        dsa.prepare_local_metadata(cu_d, Tk, K, cu_seqlens_padded=cp_d,
                                   query_indices=torch.tensor([5, Tk + 3], dtype=torch.int32,
                                                              device=dev))
    with pytest.raises(ValueError, match="shorter"):
        dsa.prepare_local_metadata(cu_d, Tk, K, cu_seqlens_padded=torch.tensor(
            [0, 200, 1300], dtype=torch.int32, device=dev))
