"""Pins of the CPU oracle against what the pages and the mathematics fix.

CPU only.  Each test checks oracle/ against something other than itself:
hand-derived worked examples (tests/golden), brute force over the full score
matrix, closed forms, a library routine (torch SDPA + autograd in float64),
central finite differences, and the invariances the pages state (-1 slots are
masked, zero-padding q/k from 512 to 576 channels is exact, -1 padding of the
top-k width is exact, query chunks are independent and their key gradients
sum).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import dsa_inputs as gen
import oracle
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(a):
    return torch.tensor(a, dtype=torch.float32).to(torch.bfloat16)


# ----------------------------------------------------------------------------
# metadata
# ----------------------------------------------------------------------------

def test_metadata_thd_cfg3():
    w = gen.workload(3)
    md = oracle.thd_metadata(np.array(w.cu_seqlens, np.int32), w.T, 2048)
    cu = w.cu_seqlens
    assert md["max_seqlen"] == 16384
    assert md["all_rows_nonempty"]
    for b in range(4):
        for t in (cu[b], cu[b] + 1, cu[b + 1] - 1):
            assert md["seq_start"][t] == cu[b]
            assert md["causal_len"][t] == t - cu[b] + 1
            assert md["topk_length"][t] == min(2048, t - cu[b] + 1)
    # sum of causal lengths = sum of triangular numbers of the sequence lengths
    lens = np.diff(cu)
    assert md["causal_len"].astype(np.int64).sum() == int((lens * (lens + 1) // 2).sum())


@pytest.mark.parametrize("cu", [[1, 4], [0, 3, 2, 4], [0, 2, 5]])
def test_metadata_rejects_bad_offsets(cu):
    with pytest.raises(ValueError):
        oracle.thd_metadata(np.array(cu, np.int32), 4, 8)


# ----------------------------------------------------------------------------
# indexer
# ----------------------------------------------------------------------------

def test_indexer_golden():
    g = json.load(open(os.path.join(GOLDEN, "indexer_tiny.json")))
    q, k = _bf16(g["q"]), _bf16(g["k"])
    w = torch.tensor(g["w"], dtype=torch.float32)
    cu = np.array(g["cu_seqlens"], np.int32)
    idx, ln, _ = oracle.indexer_topk(q, k, w, cu, g["K"])
    assert idx.tolist() == g["expect_idx"]
    assert ln.tolist() == g["expect_len"]
    for t, row in g["expect_scores"].items():
        for s, v in row.items():
            assert oracle.indexer_score(q, k, w, int(t), int(s)) == v


@pytest.mark.parametrize("int_inputs", [True, False])
@pytest.mark.parametrize("cu,K,H,D", [([0, 97], 16, 4, 64), ([0, 40, 41, 130], 24, 8, 32),
                                      ([0, 64, 200], 64, 4, 16)])
def test_indexer_matches_brute_force(int_inputs, cu, K, H, D):
    T = cu[-1]
    g = torch.Generator().manual_seed(1234 + T + K)
    if int_inputs:
        q = torch.randint(-4, 5, (T, H, D), generator=g).to(torch.bfloat16)
        k = torch.randint(-4, 5, (T, D), generator=g).to(torch.bfloat16)
        w = torch.tensor([0.5, 1.0, 2.0])[torch.randint(0, 3, (T, H), generator=g)]
    else:
        q = torch.randn((T, H, D), generator=g).to(torch.bfloat16)
        k = torch.randn((T, D), generator=g).to(torch.bfloat16)
        w = torch.randn((T, H), generator=g) / 8
    cua = np.array(cu, np.int32)
    idx, ln, kth = oracle.indexer_topk(q, k, w, cua, K)
    scores = pins.brute_indexer_scores(q, k, w, cua)
    bidx, bln = pins.brute_topk(scores, K)
    np.testing.assert_array_equal(idx, bidx)
    np.testing.assert_array_equal(ln, bln)
    # threshold = n-th best score of the row
    for t in range(T):
        row = np.sort(scores[t][np.isfinite(scores[t])])[::-1]
        assert kth[t] == pytest.approx(row[ln[t] - 1], rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("int_inputs", [True, False])
def test_indexer_rows_with_offset_matches_brute_force(int_inputs):
    """indexer_topk_rows sees only the q / w of rows [r0, r1) (r0 inside a sequence, as the
    full-size GPU checks call it): its indices, lengths and k-th scores must equal brute force
    over the whole batch, and indexer_topk over the same rows."""
    cu = [0, 40, 41, 130, 200]
    T, K, H, D = cu[-1], 24, 8, 32
    g = torch.Generator().manual_seed(4321 + int(int_inputs))
    if int_inputs:
        q = torch.randint(-4, 5, (T, H, D), generator=g).to(torch.bfloat16)
        k = torch.randint(-4, 5, (T, D), generator=g).to(torch.bfloat16)
        w = torch.tensor([0.5, 1.0, 2.0])[torch.randint(0, 3, (T, H), generator=g)]
    else:
        q = torch.randn((T, H, D), generator=g).to(torch.bfloat16)
        k = torch.randn((T, D), generator=g).to(torch.bfloat16)
        w = torch.randn((T, H), generator=g) / 8
    cua = np.array(cu, np.int32)
    scores = pins.brute_indexer_scores(q, k, w, cua)
    bidx, bln = pins.brute_topk(scores, K)
    for r0, r1 in [(57, 90), (41, 42), (150, 200), (0, 5), (39, 45)]:
        idx, ln, kth = oracle.indexer_topk_rows(q[r0:r1].contiguous(), k, w[r0:r1].contiguous(),
                                                cua, K, r0)
        np.testing.assert_array_equal(idx, bidx[r0:r1])
        np.testing.assert_array_equal(ln, bln[r0:r1])
        for i, t in enumerate(range(r0, r1)):
            row = np.sort(scores[t][np.isfinite(scores[t])])[::-1]
            assert kth[i] == pytest.approx(row[ln[i] - 1], rel=1e-12, abs=1e-12)
        a_idx, a_ln, a_kth = oracle.indexer_topk(q, k, w, cua, K, rows=(r0, r1))
        np.testing.assert_array_equal(idx, a_idx)
        np.testing.assert_array_equal(ln, a_ln)
        np.testing.assert_array_equal(kth, a_kth)


def test_indexer_short_rows_closed_form():
    """Rows with at most K causal keys return exactly their whole prefix."""
    w_ = gen.workload(1)
    inp = gen.indexer_inputs(1)
    idx, ln, _ = oracle.indexer_topk(inp["q_idx"], inp["k_idx"], inp["w"],
                                     inp["cu_seqlens"], w_.topk, rows=(0, 80))
    for t in range(80):
        n = min(64, t + 1)
        assert ln[t] == n
        if t + 1 <= 64:
            assert idx[t, :t + 1].tolist() == list(range(t + 1))
            assert (idx[t, t + 1:] == -1).all()


def test_indexer_head_permutation_invariance():
    inp = gen.indexer_inputs(1)
    perm = torch.randperm(4, generator=torch.Generator().manual_seed(7))
    a = oracle.indexer_topk(inp["q_idx"], inp["k_idx"], inp["w"], inp["cu_seqlens"], 64,
                            rows=(100, 160))
    b = oracle.indexer_topk(inp["q_idx"][:, perm].contiguous(), inp["k_idx"],
                            inp["w"][:, perm].contiguous(), inp["cu_seqlens"], 64,
                            rows=(100, 160))
    np.testing.assert_array_equal(a[0], b[0])


def test_indexer_structure_float_thd():
    cu = [0, 50, 300, 330]
    inp = gen.indexer_inputs(3, cu_seqlens=cu)
    K = 96
    idx, ln, _ = oracle.indexer_topk(inp["q_idx"][:, :8].contiguous(), inp["k_idx"][:, :32]
                                     .contiguous(), inp["w"][:, :8].contiguous(),
                                     inp["cu_seqlens"], K)
    start = pins.segment_of(np.array(cu), cu[-1])
    for t in range(cu[-1]):
        n = ln[t]
        assert n == min(K, t - start[t] + 1)
        row = idx[t]
        assert (row[n:] == -1).all()
        v = row[:n]
        assert (np.diff(v) > 0).all()
        assert v.min() >= start[t] and v.max() <= t


# ----------------------------------------------------------------------------
# sparse MLA forward
# ----------------------------------------------------------------------------

def test_attention_golden():
    g = json.load(open(os.path.join(GOLDEN, "attention_tiny.json")))
    q, kv, dout = _bf16(g["q"]), _bf16(g["kv"]), _bf16(g["dout"])
    idx = np.array(g["idx"], np.int32)
    out, lse = oracle.sparse_mla_fwd(q, kv, idx, None, g["scale"], g["d_v"])
    np.testing.assert_allclose(out, g["expect_out"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, g["expect_lse"], rtol=0, atol=1e-15)
    dq, dkv = oracle.sparse_mla_bwd(q, kv, idx, None, dout, g["scale"])
    np.testing.assert_allclose(dq, g["expect_dq"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dkv, g["expect_dkv"], rtol=0, atol=1e-15)


def _all_causal_indices(cu, K):
    T = cu[-1]
    start = pins.segment_of(np.array(cu), T)
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        L = t - start[t] + 1
        assert L <= K
        idx[t, :L] = np.arange(start[t], t + 1)
    return idx


@pytest.mark.parametrize("cu,H,Dqk,Dv", [([0, 48], 4, 576, 512), ([0, 20, 33, 64], 3, 64, 48),
                                         ([0, 40], 2, 512, 512)])
def test_fwd_bwd_equals_dense_when_k_covers_causal(cu, H, Dqk, Dv):
    """Sparse over every causal key == dense block-causal attention (SDPA, autograd)."""
    T = cu[-1]
    g = torch.Generator().manual_seed(99 + T)
    q = (torch.randn((T, H, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    kv = (torch.randn((T, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    dout = torch.randn((T, H, Dv), generator=g).to(torch.bfloat16)
    scale = 1 / math.sqrt(Dqk)
    K = max(np.diff(cu)) + 3          # extra -1 slots on every row
    idx = _all_causal_indices(cu, K)
    out, lse = oracle.sparse_mla_fwd(q, kv, idx, None, scale, Dv)
    ref = pins.dense_attention(q, kv, cu, scale, Dv, dout=dout)
    np.testing.assert_allclose(out, ref["out"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, ref["lse"], rtol=1e-12, atol=1e-12)
    dq, dkv = oracle.sparse_mla_bwd(q, kv, idx, None, dout, scale)
    np.testing.assert_allclose(dq, ref["dq"], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dkv, ref["dkv"], rtol=1e-10, atol=1e-11)


def test_fwd_single_slot_closed_form():
    """First token of a sequence: O = kv[s, :Dv] and LSE = scale * q.kv[s]."""
    inp = gen.attention_inputs(1, cu_seqlens=[0, 8])
    q, kv = inp["q"], inp["kv"]
    idx = np.full((8, 5), -1, np.int32)
    idx[:, 2] = np.arange(8)[::-1]          # one valid slot per row, in the middle
    out, lse = oracle.sparse_mla_fwd(q, kv, idx, None, inp["scale"], 512)
    qd, kvd = pins.bf16_to_f64(q), pins.bf16_to_f64(kv)
    for t in range(8):
        s = 7 - t
        np.testing.assert_array_equal(out[t], np.broadcast_to(kvd[s, :512], out[t].shape))
        np.testing.assert_allclose(lse[t], inp["scale"] * qd[t] @ kvd[s], rtol=1e-13, atol=1e-14)


def _rand_indices(T, Tkv, n_valid, K, g):
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        idx[t, :n_valid] = g.choice(Tkv, size=n_valid, replace=False)
    return idx


def test_fwd_minus_one_slots_and_order_invariance():
    rng = np.random.default_rng(5)
    inp = gen.attention_inputs(1, cu_seqlens=[0, 64], heads=4)
    q, kv = inp["q"], inp["kv"]
    idx = _rand_indices(64, 64, 20, 20, rng)
    base_o, base_l = oracle.sparse_mla_fwd(q, kv, idx, None, inp["scale"], 512)
    # scatter -1 slots among the valid ones and permute the valid ones
    wide = np.full((64, 37), -1, np.int32)
    for t in range(64):
        pos = np.sort(rng.choice(37, size=20, replace=False))
        wide[t, pos] = rng.permutation(idx[t])
    o2, l2 = oracle.sparse_mla_fwd(q, kv, wide, None, inp["scale"], 512)
    np.testing.assert_allclose(o2, base_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, base_l, rtol=1e-13, atol=1e-13)
    # topk_length: only the prefix is read, garbage after it is ignored
    garbage = idx.copy()
    garbage = np.concatenate([garbage, rng.integers(0, 64, (64, 9)).astype(np.int32)], axis=1)
    lens = np.full(64, 20, np.int32)
    o3, l3 = oracle.sparse_mla_fwd(q, kv, garbage, lens, inp["scale"], 512)
    np.testing.assert_array_equal(o3, base_o)
    np.testing.assert_array_equal(l3, base_l)


def test_empty_row_and_bad_index():
    inp = gen.attention_inputs(1, cu_seqlens=[0, 4], heads=2)
    idx = np.full((4, 3), -1, np.int32)
    idx[1, 0] = 0
    out, lse = oracle.sparse_mla_fwd(inp["q"], inp["kv"], idx, None, inp["scale"], 512)
    assert np.isneginf(lse[0]).all() and (out[0] == 0).all()
    dq, dkv = oracle.sparse_mla_bwd(inp["q"], inp["kv"], idx, None, inp["dout"], inp["scale"])
    assert (dq[0] == 0).all() and (dq[2] == 0).all()
    assert (dkv[1:] == 0).all()
    idx[2, 1] = 4                      # out of range
    with pytest.raises(ValueError):
        oracle.sparse_mla_fwd(inp["q"], inp["kv"], idx, None, inp["scale"], 512)


def test_nope_zero_padding_and_topk_padding_are_exact():
    """SkyRL PR 2388 'Change': q/k zero-padded 512->576 and -1 padding of the top-k width."""
    T = 48
    inp = gen.attention_inputs(4, cu_seqlens=[0, T])
    q, kv, dout = inp["q"], inp["kv"], inp["dout"]
    K = 2051 if T > 2051 else 11
    idx = gen.kpool_indices(T, topk=K, tail=3)
    o, l = oracle.sparse_mla_fwd(q, kv, idx, None, inp["scale"], 512)
    qp = torch.cat([q, torch.zeros(T, q.shape[1], 64, dtype=q.dtype)], dim=2)
    kvp = torch.cat([kv, torch.zeros(T, 64, dtype=kv.dtype)], dim=1)
    pad = (-K) % 64
    idxp = torch.cat([idx, torch.full((T, pad), -1, dtype=torch.int32)], dim=1)
    op, lp = oracle.sparse_mla_fwd(qp, kvp, idxp, None, inp["scale"], 512)
    np.testing.assert_array_equal(op, o)
    np.testing.assert_array_equal(lp, l)
    dq, dkv = oracle.sparse_mla_bwd(q, kv, idx, None, dout, inp["scale"])
    dqp, dkvp = oracle.sparse_mla_bwd(qp, kvp, idxp, None, dout, inp["scale"])
    np.testing.assert_array_equal(dqp[..., :512], dq)
    np.testing.assert_array_equal(dkvp[:, :512], dkv)
    assert (dqp[..., 512:] == 0).all() and (dkvp[:, 512:] == 0).all()


def test_query_chunks_are_independent_and_key_grads_sum():
    """SkyRL PR 2423 'Summary': chunked == one-shot; key grads of the chunks sum."""
    T = 70
    inp = gen.attention_inputs(4, cu_seqlens=[0, T])
    idx = gen.kpool_indices(T, topk=19, tail=3)
    q, kv, dout, sc = inp["q"], inp["kv"], inp["dout"], inp["scale"]
    o, l = oracle.sparse_mla_fwd(q, kv, idx, None, sc, 512)
    dq, dkv = oracle.sparse_mla_bwd(q, kv, idx, None, dout, sc)
    dkv_c = np.zeros_like(dkv)
    for r0, r1 in [(0, 32), (32, 64), (64, 70)]:
        oc, lc = oracle.sparse_mla_fwd(q, kv, idx, None, sc, 512, rows=(r0, r1))
        np.testing.assert_array_equal(oc, o[r0:r1])
        np.testing.assert_array_equal(lc, l[r0:r1])
        dqc, dkv_c = oracle.sparse_mla_bwd(q, kv, idx, None, dout, sc, rows=(r0, r1), dkv=dkv_c)
        np.testing.assert_array_equal(dqc, dq[r0:r1])
    np.testing.assert_allclose(dkv_c, dkv, rtol=1e-12, atol=1e-13)


def test_bwd_central_finite_differences():
    """d/dx of L = sum(dout * out) by central differences with Richardson extrapolation.

    Inputs sit on a 1/8 grid in (-2, 2) so that x +- 2^-6 and x +- 2^-7 are exact
    bfloat16 values; the oracle forward is evaluated at the perturbed inputs."""
    rng = np.random.default_rng(11)
    T, H, Dqk, Dv, K = 10, 2, 8, 4, 6
    q = torch.tensor(rng.integers(-15, 16, (T, H, Dqk)) / 8.0).to(torch.bfloat16)
    kv = torch.tensor(rng.integers(-15, 16, (T, Dqk)) / 8.0).to(torch.bfloat16)
    dout = torch.tensor(rng.integers(-15, 16, (T, H, Dv)) / 8.0).to(torch.bfloat16)
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        n = min(t + 1, 4)
        idx[t, rng.choice(K, n, replace=False)] = rng.choice(t + 1, n, replace=False)
    sc = 0.5
    dq, dkv = oracle.sparse_mla_bwd(q, kv, idx, None, dout, sc)
    d64 = pins.bf16_to_f64(dout)

    def loss(qx, kvx):
        o, _ = oracle.sparse_mla_fwd(qx, kvx, idx, None, sc, Dv)
        return float((o * d64).sum())

    def fd(which, pos):
        vals = []
        for h in (2.0 ** -6, 2.0 ** -7):
            res = []
            for sgn in (1, -1):
                qx, kvx = q.clone(), kv.clone()
                tgt = qx if which == "q" else kvx
                tgt[pos] = (tgt[pos].float() + sgn * h).to(torch.bfloat16)
                assert float(tgt[pos]) == float((q if which == "q" else kv)[pos]) + sgn * h
                res.append(loss(qx, kvx))
            vals.append((res[0] - res[1]) / (2 * h))
        return (4 * vals[1] - vals[0]) / 3

    for pos in [(3, 1, 2), (9, 0, 7), (5, 1, 0)]:
        assert fd("q", pos) == pytest.approx(dq[pos], rel=1e-5, abs=1e-7)
    for pos in [(0, 0), (2, 3), (4, 6), (7, 1)]:
        assert fd("kv", pos) == pytest.approx(dkv[pos], rel=1e-5, abs=1e-7)


def test_bwd_logit_shift_gradient_vanishes():
    """sum_j dZ_j = 0: shifting every logit of a row by the same amount changes nothing,
    so the gradient along q[t,h] parallel to a direction that shifts all keys equally is 0.
    With a constant extra channel c in every key, dL/dq[t,h,c] = scale*c*sum_j dZ_j = 0."""
    T, H, D = 12, 3, 16
    g = torch.Generator().manual_seed(3)
    q = torch.randn((T, H, D), generator=g).to(torch.bfloat16)
    kv = torch.randn((T, D), generator=g).to(torch.bfloat16)
    kv[:, D - 1] = 1.0                                  # constant key channel
    dout = torch.randn((T, H, 8), generator=g).to(torch.bfloat16)
    idx = np.array([[s if s <= t else -1 for s in range(T)] for t in range(T)], np.int32)
    dq, _ = oracle.sparse_mla_bwd(q, kv, idx, None, dout, 0.25)
    np.testing.assert_allclose(dq[..., D - 1], 0.0, atol=1e-14)


def test_kpool_generator_structure():
    T, K = 40, 11
    idx = gen.kpool_indices(T, topk=K, tail=3).numpy()
    for t in range(T):
        row = idx[t]
        if t + 1 <= K:
            assert row[:t + 1].tolist() == list(range(t + 1)) and (row[t + 1:] == -1).all()
        else:
            assert row[-3:].tolist() == [t - 2, t - 1, t]
            head = row[:-3]
            assert (np.diff(head) > 0).all() and head.max() <= t - 3 and head.min() >= 0


# ---- attention sink: one zero-valued logit per head in the softmax denominator ([API]
# _pad_attention_heads pads a sink [H] with the heads; the arithmetic is the reading taken)

@pytest.mark.parametrize("cu,H,Dqk,Dv", [([0, 40], 4, 576, 512), ([0, 20, 33, 64], 3, 64, 48)])
def test_sink_equals_dense_with_a_zero_valued_extra_key(cu, H, Dqk, Dv):
    """Sink == dense block-causal attention over one more key (zero key and value vectors,
    logit lifted to sink[h] by an additive mask): out, lse, dq, dkv and dsink (autograd)."""
    T = cu[-1]
    g = torch.Generator().manual_seed(7 + T)
    q = (torch.randn((T, H, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    kv = (torch.randn((T, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    dout = torch.randn((T, H, Dv), generator=g).to(torch.bfloat16)
    sink = torch.randn(H, generator=g).numpy().astype(np.float64)
    sink[0] = 6.0                     # a sink that dominates most rows
    scale = 1 / math.sqrt(Dqk)
    idx = _all_causal_indices(cu, max(np.diff(cu)) + 2)
    out, lse = oracle.sparse_mla_fwd(q, kv, idx, None, scale, Dv, sink=sink)
    ref = pins.dense_attention_sink(q, kv, cu, scale, Dv, sink, dout=dout)
    np.testing.assert_allclose(out, ref["out"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, ref["lse"], rtol=1e-12, atol=1e-12)
    dq, dkv, dsink = oracle.sparse_mla_bwd(q, kv, idx, None, dout, scale, sink=sink)
    np.testing.assert_allclose(dq, ref["dq"], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dkv, ref["dkv"], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dsink, ref["dsink"], rtol=1e-10, atol=1e-11)


def test_sink_single_slot_closed_form_and_identities():
    """One valid slot: out = kv[s] e^z / (e^z + e^sink), lse = logaddexp(z, sink).  Any row:
    lse' = logaddexp(lse, sink) and out' = out exp(lse - lse') against the sink-free result;
    sink = -inf is exactly no sink; an empty row gives lse = sink, out = 0 and no gradient."""
    inp = gen.attention_inputs(1, cu_seqlens=[0, 8])
    q, kv, dout, scale = inp["q"], inp["kv"], inp["dout"], inp["scale"]
    H = q.shape[1]
    sink = np.linspace(-3.0, 3.0, H)
    idx = np.full((8, 4), -1, np.int32)
    idx[:, 1] = np.arange(8)[::-1]
    out, lse = oracle.sparse_mla_fwd(q, kv, idx, None, scale, 512, sink=sink)
    qd, kvd = pins.bf16_to_f64(q), pins.bf16_to_f64(kv)
    for t in range(8):
        s = 7 - t
        z = scale * qd[t] @ kvd[s]                                      # [H]
        np.testing.assert_allclose(lse[t], np.logaddexp(z, sink), rtol=1e-13, atol=1e-13)
        w = 1.0 / (1.0 + np.exp(sink - z))
        np.testing.assert_allclose(out[t], w[:, None] * kvd[s, :512][None], rtol=1e-12,
                                   atol=1e-13)
    # identities on a row set with several slots
    g = np.random.default_rng(3)
    idx2 = np.full((8, 9), -1, np.int32)
    for t in range(8):
        idx2[t, :t + 1] = g.permutation(t + 1)
    o0, l0 = oracle.sparse_mla_fwd(q, kv, idx2, None, scale, 512)
    o1, l1 = oracle.sparse_mla_fwd(q, kv, idx2, None, scale, 512, sink=sink)
    np.testing.assert_allclose(l1, np.logaddexp(l0, sink[None]), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o1, o0 * np.exp(l0 - l1)[..., None], rtol=1e-12, atol=1e-13)
    om, lm = oracle.sparse_mla_fwd(q, kv, idx2, None, scale, 512, sink=np.full(H, -np.inf))
    np.testing.assert_array_equal(om, o0)
    np.testing.assert_array_equal(lm, l0)
    # empty rows
    empty = np.full((8, 3), -1, np.int32)
    oe, le = oracle.sparse_mla_fwd(q, kv, empty, None, scale, 512, sink=sink)
    assert not oe.any()
    np.testing.assert_array_equal(le, np.broadcast_to(sink, le.shape))
    dq, dkv, dsink = oracle.sparse_mla_bwd(q, kv, empty, None, dout, scale, sink=sink)
    assert not dq.any() and not dkv.any() and not dsink.any()


# ---- local query rows against gathered global keys in padded-storage coordinates ([API]
# prepare_cudnn_dsa_packed_metadata: query_indices, cu_seqlens_padded, padding_mask)

def _padded_layout(cu, cu_pad, k_compact, D, g):
    """k in padded storage: sequence b's real keys at cu_pad[b] + j, random padding rows."""
    k = torch.randn((cu_pad[-1], D), generator=g).to(torch.bfloat16)
    for b in range(len(cu) - 1):
        n = cu[b + 1] - cu[b]
        k[cu_pad[b]:cu_pad[b] + n] = k_compact[cu[b]:cu[b + 1]]
    return k


def test_local_indexer_identity_padding_and_cp_split():
    """Identity coordinates equal the compact oracle; a padded layout gives the compact result
    with positions mapped to padded storage; two ranks' query subsets together give the full
    result; rows in the padding (by position or by the mask) get len 0 and -1."""
    cu, cu_pad, K, H, D = [0, 5, 30, 71], [0, 8, 40, 84], 9, 4, 64
    T = cu[-1]
    inp = gen.indexer_inputs(1, cu_seqlens=cu)
    q, k, w = inp["q_idx"][:, :H], inp["k_idx"], inp["w"][:, :H].contiguous()
    ref_i, ref_l, _ = oracle.indexer_topk(q.contiguous(), k, w, cu, K)
    idx, ln = oracle.indexer_topk_local(q.contiguous(), k, w, cu, K)
    np.testing.assert_array_equal(idx, ref_i)
    np.testing.assert_array_equal(ln, ref_l)
    # padded storage: every real token as a local query, coordinates cu_pad[b] + j
    g = torch.Generator().manual_seed(4)
    kp = _padded_layout(cu, cu_pad, k, D, g)
    seq = np.searchsorted(np.array(cu), np.arange(T), side="right") - 1
    shift = (np.array(cu_pad)[seq] - np.array(cu)[seq]).astype(np.int32)
    coord = (np.arange(T) + shift).astype(np.int32)
    idx_p, ln_p = oracle.indexer_topk_local(q.contiguous(), kp, w, cu, K, cu_seqlens_padded=cu_pad,
                                            query_indices=coord)
    expect = np.where(ref_i >= 0, ref_i + shift[:, None], -1)
    np.testing.assert_array_equal(idx_p, expect)
    np.testing.assert_array_equal(ln_p, ref_l)
    # two ranks with zig-zag chunks of the local rows
    chunks = np.array_split(np.arange(T), 4)
    ranks = [np.concatenate([chunks[0], chunks[3]]), np.concatenate([chunks[1], chunks[2]])]
    for rows in ranks:
        i_r, l_r = oracle.indexer_topk_local(q[rows].contiguous(), kp, w[rows].contiguous(), cu,
                                             K, cu_seqlens_padded=cu_pad,
                                             query_indices=coord[rows])
        np.testing.assert_array_equal(i_r, expect[rows])
        np.testing.assert_array_equal(l_r, ref_l[rows])
    # padding rows: coordinates beyond a sequence's real length, and masked rows
    pad_coord = np.array([5, 7, 35, 39, 82, 12], np.int32)   # the last one is real (seq 1)
    qr = q[:6].contiguous()
    wr = w[:6].contiguous()
    mask = np.array([0, 0, 0, 0, 0, 1], np.uint8)
    i_p, l_p = oracle.indexer_topk_local(qr, kp, wr, cu, K, cu_seqlens_padded=cu_pad,
                                         query_indices=pad_coord, padding_mask=mask)
    assert (i_p == -1).all() and (l_p == 0).all()
    i_u, l_u = oracle.indexer_topk_local(qr, kp, wr, cu, K, cu_seqlens_padded=cu_pad,
                                         query_indices=pad_coord)
    assert (l_u[:5] == 0).all() and l_u[5] == 5 and (i_u[5, :5] == np.arange(8, 13)).all()


# ----------------------------------------------------------------------------
# indexer KL loss (training path)
# ----------------------------------------------------------------------------

def _kl_case(T, H, Dqk, K, Hi, Di, n_valid, seed, cu=None):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn((T, H, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    kv = (torch.randn((T, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    q_idx = torch.randn((T, Hi, Di), generator=g).to(torch.bfloat16)
    k_idx = torch.randn((T, Di), generator=g).to(torch.bfloat16)
    w = torch.randn((T, Hi), generator=g) / 8
    cu = cu or [0, T]
    start = pins.segment_of(np.array(cu), T)
    r = np.random.default_rng(seed)
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        L = t - start[t] + 1
        n = min(n_valid, L)
        idx[t, :n] = np.sort(start[t] + r.choice(L, size=n, replace=False))
    return q, kv, idx, q_idx, k_idx, w


@pytest.mark.parametrize("sink", [False, True])
def test_indexer_kl_matches_dense_autograd(sink):
    """Loss, target and gradients equal a dense fp64 route through torch autograd: attention
    probabilities restricted to the selected keys, their head sum renormalised, the indexer's
    log-softmax over the same keys, KL(target || indexer) with the target detached."""
    T, H, Dqk, K, Hi, Di = 48, 4, 64, 24, 8, 32
    cu = [0, 17, 48]
    q, kv, idx, q_idx, k_idx, w = _kl_case(T, H, Dqk, K, Hi, Di, 20, seed=11 + int(sink), cu=cu)
    scale = 0.2
    sk = np.array([0.3, -1.0, 2.0, -0.5]) if sink else None
    ora = oracle.indexer_kl(q, kv, idx, None, scale, q_idx, k_idx, w, g=1.0, sink=sk)
    # dense route
    qd, kvd = pins.bf16_to_f64(q), pins.bf16_to_f64(kv)
    qi = torch.tensor(pins.bf16_to_f64(q_idx), requires_grad=True)
    ki = torch.tensor(pins.bf16_to_f64(k_idx), requires_grad=True)
    wd = torch.tensor(w.numpy().astype(np.float64), requires_grad=True)
    mask = torch.zeros((T, T), dtype=torch.bool)
    for t in range(T):
        sel = idx[t][idx[t] >= 0]
        mask[t, torch.from_numpy(sel.astype(np.int64))] = True
    z = scale * torch.einsum("thd,sd->ths", torch.from_numpy(qd), torch.from_numpy(kvd))
    z = z.masked_fill(~mask[:, None, :], -math.inf)
    if sink:
        zs = torch.cat([z, torch.from_numpy(sk)[None, :, None].expand(T, H, 1)], dim=-1)
        P = torch.exp(z - torch.logsumexp(zs, dim=-1, keepdim=True))
    else:
        P = torch.softmax(z, dim=-1)
    pt = P.sum(1)
    pt = pt / pt.sum(-1, keepdim=True)
    dots = torch.einsum("thd,sd->ths", qi, ki)
    I = torch.einsum("th,ths->ts", wd, torch.relu(dots))
    logu = torch.log_softmax(I.masked_fill(~mask, -math.inf), dim=-1)
    terms = torch.where(mask & (pt > 0), pt * (torch.log(pt) - logu), torch.zeros_like(pt))
    loss_t = terms.sum(-1)
    loss_t.sum().backward()
    np.testing.assert_allclose(ora["loss"], loss_t.detach().numpy(), rtol=1e-10, atol=1e-12)
    tgt = np.zeros((T, K))
    for t in range(T):
        for j in range(K):
            if idx[t, j] >= 0:
                tgt[t, j] = pt[t, idx[t, j]].item()
    np.testing.assert_allclose(ora["target"], tgt, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(ora["dw"], wd.grad.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(ora["dq_idx"], qi.grad.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(ora["dk_idx"], ki.grad.numpy(), rtol=1e-9, atol=1e-12)
    assert (ora["loss"] >= -1e-15).all()


def test_indexer_kl_head_weight_finite_differences():
    """dw against central differences of the loss in the fp32 head weights (the loss is smooth
    in w: the ReLU acts on q_idx . k_idx only), with exactly representable steps."""
    T, H, Dqk, K, Hi, Di = 20, 2, 32, 16, 4, 16
    q, kv, idx, q_idx, k_idx, w = _kl_case(T, H, Dqk, K, Hi, Di, 12, seed=5)
    w = torch.round(w * 1024) / 1024
    scale = 0.3
    base = oracle.indexer_kl(q, kv, idx, None, scale, q_idx, k_idx, w, g=1.0)
    eps = 2.0 ** -12
    for t, h in [(3, 0), (9, 2), (15, 1), (19, 3)]:
        wp, wm = w.clone(), w.clone()
        wp[t, h] += eps
        wm[t, h] -= eps
        lp = oracle.indexer_kl(q, kv, idx, None, scale, q_idx, k_idx, wp, rows=(t, t + 1))
        lm = oracle.indexer_kl(q, kv, idx, None, scale, q_idx, k_idx, wm, rows=(t, t + 1))
        fd = (lp["loss"][0] - lm["loss"][0]) / (2 * eps)
        assert fd == pytest.approx(base["dw"][t, h], rel=1e-5, abs=1e-9)


def test_indexer_kl_closed_forms():
    """q_idx = 0: every indexer score is 0, the indexer distribution is uniform over the n valid
    slots, loss = sum p log p + log n, and no gradient reaches q_idx, k_idx or w (the ReLU's
    argument is 0 everywhere).  A row with one valid slot has loss 0."""
    T, H, Dqk, K, Hi, Di = 24, 4, 64, 10, 4, 32
    q, kv, idx, q_idx, k_idx, w = _kl_case(T, H, Dqk, K, Hi, Di, 10, seed=7)
    zero = torch.zeros_like(q_idx)
    r = oracle.indexer_kl(q, kv, idx, None, 0.25, zero, k_idx, w, g=1.0)
    for t in range(T):
        n = int((idx[t] >= 0).sum())
        p = r["target"][t][idx[t] >= 0]
        assert p.sum() == pytest.approx(1.0, abs=1e-14)
        expect = float((p[p > 0] * np.log(p[p > 0])).sum() + math.log(n))
        assert r["loss"][t] == pytest.approx(expect, abs=1e-13)
    assert not r["dq_idx"].any() and not r["dw"].any() and not r["dk_idx"].any()
    r1 = oracle.indexer_kl(q, kv, idx, None, 0.25, q_idx, k_idx, w, g=1.0)
    assert r1["loss"][0] == 0.0 and not r1["dq_idx"][0].any() and not r1["dw"][0].any()


def test_indexer_kl_chunks_and_head_permutation():
    """Query chunks give the same rows and key gradients that sum to the one-shot result;
    permuting indexer heads together with their weights permutes dq_idx and dw only."""
    T, H, Dqk, K, Hi, Di = 40, 4, 64, 16, 8, 32
    q, kv, idx, q_idx, k_idx, w = _kl_case(T, H, Dqk, K, Hi, Di, 14, seed=9)
    full = oracle.indexer_kl(q, kv, idx, None, 0.2, q_idx, k_idx, w, g=0.5)
    a = oracle.indexer_kl(q, kv, idx, None, 0.2, q_idx, k_idx, w, g=0.5, rows=(0, 13))
    b = oracle.indexer_kl(q, kv, idx, None, 0.2, q_idx, k_idx, w, g=0.5, rows=(13, T),
                          dk_idx=a["dk_idx"].copy())
    np.testing.assert_array_equal(np.concatenate([a["loss"], b["loss"]]), full["loss"])
    np.testing.assert_array_equal(np.concatenate([a["dq_idx"], b["dq_idx"]]), full["dq_idx"])
    np.testing.assert_allclose(b["dk_idx"], full["dk_idx"], rtol=1e-13, atol=1e-15)
    perm = torch.randperm(Hi, generator=torch.Generator().manual_seed(3))
    p = oracle.indexer_kl(q, kv, idx, None, 0.2, q_idx[:, perm].contiguous(), k_idx,
                          w[:, perm].contiguous(), g=0.5)
    np.testing.assert_allclose(p["loss"], full["loss"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(p["dq_idx"], full["dq_idx"][:, perm.numpy()], rtol=1e-12,
                               atol=1e-15)
    np.testing.assert_allclose(p["dw"], full["dw"][:, perm.numpy()], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(p["dk_idx"], full["dk_idx"], rtol=1e-11, atol=1e-14)


# ----------------------------------------------------------------------------
# k-pool indexer
# ----------------------------------------------------------------------------

def _kpool_case(cu, pool, H, D, int_inputs, seed):
    T = cu[-1]
    n_pools = sum((cu[b + 1] - cu[b]) // pool for b in range(len(cu) - 1))
    g = torch.Generator().manual_seed(seed)
    if int_inputs:
        q = torch.randint(-4, 5, (T, H, D), generator=g).to(torch.bfloat16)
        kp = torch.randint(-4, 5, (n_pools, D), generator=g).to(torch.bfloat16)
        w = torch.tensor([0.5, 1.0, 2.0])[torch.randint(0, 3, (T, H), generator=g)]
    else:
        q = torch.randn((T, H, D), generator=g).to(torch.bfloat16)
        kp = torch.randn((n_pools, D), generator=g).to(torch.bfloat16)
        w = torch.randn((T, H), generator=g) / 8
    return q, kp, w


def _kpool_brute(q, kp, w, cu, pool, K_pools):
    """Pool scores by einsum, ranking by (score desc, pool asc), expansion to keys and the
    incomplete tail pool, written from the reading with numpy."""
    qd, kd = pins.bf16_to_f64(q), pins.bf16_to_f64(kp)
    wd = w.numpy().astype(np.float64)
    T = cu[-1]
    W = K_pools * pool + pool - 1
    idx = np.full((T, W), -1, np.int32)
    ln = np.zeros(T, np.int32)
    cp = 0
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        npool = (s1 - s0) // pool
        scores = np.einsum("th,thp->tp", wd[s0:s1],
                           np.maximum(np.einsum("thd,pd->thp", qd[s0:s1], kd[cp:cp + npool]), 0))
        for t in range(s0, s1):
            P = (t - s0 + 1) // pool
            sc = scores[t - s0, :P]
            order = np.lexsort((np.arange(P), -sc))[:min(K_pools, P)]
            keys = [s0 + i * pool + r for i in np.sort(order) for r in range(pool)]
            keys += list(range(s0 + P * pool, t + 1))
            idx[t, :len(keys)] = keys
            ln[t] = len(keys)
        cp += npool
    return idx, ln


@pytest.mark.parametrize("int_inputs", [True, False])
@pytest.mark.parametrize("cu,pool,K_pools", [([0, 97], 4, 8), ([0, 40, 41, 130, 203], 4, 5),
                                             ([0, 64, 150], 3, 7)])
def test_kpool_indexer_matches_brute_force(int_inputs, cu, pool, K_pools):
    q, kp, w = _kpool_case(cu, pool, 4, 32, int_inputs, seed=cu[-1] + pool + K_pools)
    idx, ln = oracle.kpool_indexer(q, kp, w, np.array(cu, np.int32), pool, K_pools)
    bidx, bln = _kpool_brute(q, kp, w, cu, pool, K_pools)
    np.testing.assert_array_equal(idx, bidx)
    np.testing.assert_array_equal(ln, bln)
    # structure: ascending, causal, len = pool min(K_pools, P) + tail
    start = pins.segment_of(np.array(cu), cu[-1])
    for t in range(cu[-1]):
        pos = t - start[t]
        P = (pos + 1) // pool
        assert ln[t] == pool * min(K_pools, P) + (pos + 1 - pool * P)
        v = idx[t, :ln[t]]
        assert (np.diff(v) > 0).all() and (v >= start[t]).all() and (v <= t).all()
        if P <= K_pools:  # every complete pool and the tail: the whole causal prefix
            assert v.tolist() == list(range(start[t], t + 1))
    # a row range (as the full-size GPU checks call it) and its k-th pool scores
    r0, r1 = cu[-1] // 3, cu[-1]
    ridx, rln, kth = oracle.kpool_indexer(q, kp, w, np.array(cu, np.int32), pool, K_pools,
                                          rows=(r0, r1))
    np.testing.assert_array_equal(ridx, bidx[r0:r1])
    np.testing.assert_array_equal(rln, bln[r0:r1])
    qd, kd = pins.bf16_to_f64(q), pins.bf16_to_f64(kp)
    cps = np.concatenate([[0], np.cumsum(np.diff(cu) // pool)])
    for t in range(r0, r1):
        b = int(np.searchsorted(cu, t, side="right") - 1)
        P = (t - cu[b] + 1) // pool
        if P == 0:
            assert kth[t - r0] == 0.0
            continue
        sc = (w.numpy()[t][:, None].astype(np.float64) *
              np.maximum(qd[t] @ kd[cps[b]:cps[b] + P].T, 0)).sum(0)
        assert kth[t - r0] == pytest.approx(np.sort(sc)[::-1][min(K_pools, P) - 1], rel=1e-12,
                                            abs=1e-12)


def test_kpool_indexer_with_unit_pools_is_the_token_indexer():
    """pool = 1 with the token keys as pool keys: the token-level indexer's result."""
    cu = [0, 50, 131]
    q, k, w = _kpool_case(cu, 1, 4, 32, False, seed=77)
    idx, ln = oracle.kpool_indexer(q, k, w, np.array(cu, np.int32), 1, 24)
    ridx, rln, _ = oracle.indexer_topk(q, k, w, np.array(cu, np.int32), 24)
    np.testing.assert_array_equal(idx, ridx)
    np.testing.assert_array_equal(ln, rln)
