"""The allocation-free backward (dsa_sparse_mla_bwd_noalloc, called through the C ABI) against
the workspace backward (dsa_sparse_mla_bwd) and the oracle: two calls in a row, the first large
enough to need many passes over the fixed scratch, the second smaller.

dq is bitwise reproducible and must be identical; dkv is reproducible up to summation order
and must agree within the chunked-execution tolerance; both must meet the oracle's bar where
the oracle is run."""

import ctypes as C
import math

import numpy as np
import pytest
import torch

import oracle
from tests import checks

pytestmark = pytest.mark.gpu

dev = "cuda"


def _dsa():
    import sparse_attention_12_amd as dsa
    return dsa


def _inputs(T, H, Dqk, K, n_valid, seed):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn((T, H, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    kv = (torch.randn((T, Dqk), generator=g) * 0.5).to(torch.bfloat16)
    dout = torch.randn((T, H, 512), generator=g).to(torch.bfloat16)
    r = np.random.default_rng(seed)
    idx = np.full((T, K), -1, np.int32)
    for t in range(T):
        n = min(n_valid, t + 1)
        idx[t, :n] = np.sort(r.choice(t + 1, size=n, replace=False))
    lens = (idx >= 0).sum(1).astype(np.int32)
    return q, kv, dout, idx, lens


def _call_noalloc(dsa, q, kv, idx, ln, out, lse, dout, scale, dq, dkv):
    L = dsa.lib()
    T, H, Dqk = q.shape
    rc = L.dsa_sparse_mla_bwd_noalloc(
        q.data_ptr(), kv.data_ptr(), idx.data_ptr(), ln.data_ptr(), out.data_ptr(),
        lse.data_ptr(), dout.data_ptr(), T, kv.shape[0], H, Dqk, 512, idx.shape[1],
        C.c_float(scale), dq.data_ptr(), dkv.data_ptr(), 0,
        C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, L.dsa_last_error().decode()


@pytest.mark.parametrize("calls", [[(3000, 64, 576, 2048, 1500, True), (97, 16, 512, 40, 33, False)]])
def test_noalloc_backward_matches_workspace_backward(calls):
    dsa = _dsa()
    per_call = {}
    for T, H, Dqk, K, n_valid, big in calls:
        print(f"noalloc call T={T} H={H} D_qk={Dqk} K={K}", flush=True)
        q, kv, dout, idx, lens = _inputs(T, H, Dqk, K, n_valid, seed=T + H)
        scale = 1.0 / math.sqrt(Dqk)
        qd, kvd, dd = q.to(dev), kv.to(dev), dout.to(dev)
        idd, lnd = torch.from_numpy(idx).to(dev), torch.from_numpy(lens).to(dev)
        out, lse = dsa.sparse_mla_fwd(qd, kvd, idd, scale, lnd)
        dq_ref, dkv_ref = dsa.sparse_mla_bwd(qd, kvd, idd, out, lse, dd, scale, lnd)
        # outputs pre-filled with garbage: the entry point must overwrite dq and dkv
        dq = torch.full_like(dq_ref, 7.0)
        dkv = torch.full_like(dkv_ref, -3.0)
        _call_noalloc(dsa, qd, kvd, idd, lnd, out, lse, dd, scale, dq, dkv)
        torch.cuda.synchronize()
        assert torch.equal(dq, dq_ref), "dq differs from the workspace backward"
        diff = (dkv - dkv_ref).abs().max().item()
        ref_max = dkv_ref.abs().max().item()
        assert diff <= 1e-5 * ref_max + 1e-4, f"dkv differs by {diff} (max {ref_max})"
        if big:
            # the scratch holds far fewer than T rows: the call ran in many passes
            per_row = K * (2 * Dqk + 20)
            assert T * per_row > L_scratch(dsa), "case must need several passes"
        else:
            rdq, rdkv = oracle.sparse_mla_bwd(q, kv, idx, lens, dout, scale)
            checks.assert_close("noalloc dq", dq.float().cpu().numpy(), rdq, checks.ATOL_OUT)
            checks.assert_close("noalloc dkv", dkv.cpu().numpy(), rdkv, checks.ATOL_OUT)
        per_call[T] = diff
        print(f"  dkv vs workspace backward {diff:.2e}", flush=True)


def L_scratch(dsa):
    return dsa.lib().dsa_sparse_mla_bwd_noalloc_scratch_bytes()
