"""CPU oracle for the DSA hot path -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and the CPU-baseline leg of
bench.py may import this package.  The product library never does, and the
oracle never imports the product: the two share nothing except the seeded
input generators in dsa_inputs.py.

Thin ctypes/numpy wrappers around oracle/dsa_oracle.c (fp64 definitions of
the THD metadata, indexer top-k, sparse MLA forward and backward, and the
indexer's KL training loss with its gradients).  bf16
tensors are passed as their uint16 bit patterns.  See dsa_oracle.c for the
page passages each function follows.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        L = C.CDLL(path)
        i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
        u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        L.oracle_thd_metadata.argtypes = [i32p, C.c_int32, C.c_int64, C.c_int32, i32p, i32p, i32p,
                                          C.POINTER(C.c_int32), C.POINTER(C.c_int32)]
        L.oracle_thd_metadata.restype = C.c_int
        L.oracle_indexer_score.argtypes = [u16p, u16p, f32p, C.c_int32, C.c_int32, C.c_int64,
                                           C.c_int64]
        L.oracle_indexer_score.restype = C.c_double
        L.oracle_indexer_topk.argtypes = [u16p, u16p, f32p, i32p, C.c_int32, C.c_int64, C.c_int32,
                                          C.c_int32, C.c_int32, C.c_int64, C.c_int64, i32p, i32p,
                                          C.c_void_p]
        L.oracle_indexer_topk.restype = C.c_int
        L.oracle_indexer_topk_rows.argtypes = [u16p, u16p, f32p, i32p, C.c_int32, C.c_int64,
                                               C.c_int32, C.c_int32, C.c_int32, C.c_int64,
                                               C.c_int64, C.c_int64, i32p, i32p, C.c_void_p]
        L.oracle_indexer_topk_rows.restype = C.c_int
        L.oracle_indexer_topk_local.argtypes = [u16p, u16p, f32p, i32p, C.c_void_p, C.c_void_p,
                                                C.c_void_p, C.c_int32, C.c_int64, C.c_int64,
                                                C.c_int32, C.c_int32, C.c_int32, i32p, i32p]
        L.oracle_indexer_topk_local.restype = C.c_int
        L.oracle_sparse_mla_fwd.argtypes = [u16p, u16p, i32p, C.c_void_p, C.c_int64, C.c_int64,
                                            C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_double,
                                            C.c_void_p, C.c_int64, C.c_int64, f64p, f64p]
        L.oracle_sparse_mla_fwd.restype = C.c_int
        L.oracle_sparse_mla_bwd.argtypes = [u16p, u16p, i32p, C.c_void_p, u16p, C.c_int64,
                                            C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                            C.c_double, C.c_void_p, C.c_int64, C.c_int64, f64p,
                                            f64p, C.c_void_p]
        L.oracle_sparse_mla_bwd.restype = C.c_int
        L.oracle_indexer_kl.argtypes = [u16p, u16p, i32p, C.c_void_p, C.c_int64, C.c_int64,
                                        C.c_int32, C.c_int32, C.c_int32, C.c_double, C.c_void_p,
                                        u16p, u16p, f32p, C.c_int32, C.c_int32, C.c_double,
                                        C.c_int64, C.c_int64, f64p, f64p, f64p, f64p, f64p]
        L.oracle_indexer_kl.restype = C.c_int
        L.oracle_kpool_indexer.argtypes = [u16p, u16p, f32p, i32p, C.c_int32, C.c_int64,
                                           C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                           C.c_int64, C.c_int64, i32p, i32p, C.c_void_p]
        L.oracle_kpool_indexer.restype = C.c_int
        _lib = L
    return _lib


def _u16(x):
    """Accept a torch bf16 tensor or a uint16 numpy array of bf16 bits."""
    if hasattr(x, "dtype") and str(x.dtype) == "torch.bfloat16":
        import torch  # noqa: F401
        x = x.detach().to("cpu").contiguous().view(__import__("torch").int16).numpy()
    x = np.ascontiguousarray(x)
    return x.view(np.uint16)


def _np(x, dtype):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").numpy()
    return np.ascontiguousarray(x, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its inputs (code {rc})")


def thd_metadata(cu_seqlens, T: int, K: int):
    cu = _np(cu_seqlens, np.int32)
    B = cu.shape[0] - 1
    ss = np.zeros(T, np.int32)
    cl = np.zeros(T, np.int32)
    tl = np.zeros(T, np.int32)
    mx = C.c_int32(0)
    ne = C.c_int32(0)
    _check(lib().oracle_thd_metadata(cu, B, T, K, ss, cl, tl, C.byref(mx), C.byref(ne)),
           "thd_metadata")
    return dict(seq_start=ss, causal_len=cl, topk_length=tl, max_seqlen=mx.value,
                all_rows_nonempty=bool(ne.value))


def indexer_score(q_idx, k_idx, w, t: int, s: int) -> float:
    q = _u16(q_idx)
    k = _u16(k_idx)
    wt = _np(w, np.float32)
    T, H, D = q.shape
    return lib().oracle_indexer_score(q.reshape(-1), k.reshape(-1), wt.reshape(-1), H, D, t, s)


def indexer_topk(q_idx, k_idx, w, cu_seqlens, K: int, rows=None):
    """Top-k for rows [r0, r1) (default all): (idx [n,K] int32, len [n] int32, kth [n] f64)."""
    q = _u16(q_idx)
    k = _u16(k_idx)
    wt = _np(w, np.float32)
    cu = _np(cu_seqlens, np.int32)
    T, H, D = q.shape
    r0, r1 = (0, T) if rows is None else rows
    n = r1 - r0
    idx = np.zeros((n, K), np.int32)
    ln = np.zeros(n, np.int32)
    kth = np.zeros(n, np.float64)
    _check(lib().oracle_indexer_topk(q.reshape(-1), k.reshape(-1), wt.reshape(-1), cu,
                                     cu.shape[0] - 1, T, H, D, K, r0, r1, idx, ln,
                                     kth.ctypes.data), "indexer_topk")
    return idx, ln, kth


def indexer_topk_rows(q_rows, k_idx, w_rows, cu_seqlens, K: int, row_begin: int):
    """Top-k of rows [row_begin, row_begin + len(q_rows)) given only those rows' q and w."""
    q = _u16(q_rows)
    k = _u16(k_idx)
    wt = _np(w_rows, np.float32)
    cu = _np(cu_seqlens, np.int32)
    n, H, D = q.shape
    T = k.shape[0]
    idx = np.zeros((n, K), np.int32)
    ln = np.zeros(n, np.int32)
    kth = np.zeros(n, np.float64)
    _check(lib().oracle_indexer_topk_rows(q.reshape(-1), k.reshape(-1), wt.reshape(-1), cu,
                                          cu.shape[0] - 1, T, H, D, K, row_begin, row_begin + n,
                                          row_begin, idx, ln, kth.ctypes.data),
           "indexer_topk_rows")
    return idx, ln, kth


def indexer_topk_local(q_idx, k_idx, w, cu_seqlens, K: int, cu_seqlens_padded=None,
                       query_indices=None, padding_mask=None):
    """Local query rows (q_idx / w [T_q,...]) against gathered global keys (k_idx [T_k,D]) in
    padded-storage coordinates.  Returns (idx int32 [T_q,K] global padded coordinates,
    len int32 [T_q]); padding rows get len 0 and -1."""
    qa = _u16(q_idx)
    ka = _u16(k_idx)
    wa = _np(w, np.float32)
    cu = _np(cu_seqlens, np.int32)
    cp, cpp = _opt_i32(cu_seqlens_padded)
    qi, qip = _opt_i32(query_indices)
    pm = pmp = None
    if padding_mask is not None:
        pm = np.ascontiguousarray(np.asarray(
            padding_mask.cpu().numpy() if hasattr(padding_mask, "cpu") else padding_mask,
            dtype=np.uint8))
        pmp = pm.ctypes.data
    Tq, H, D = qa.shape
    Tk = ka.shape[0]
    idx = np.zeros((Tq, K), np.int32)
    ln = np.zeros(Tq, np.int32)
    _check(lib().oracle_indexer_topk_local(qa.reshape(-1), ka.reshape(-1), wa.reshape(-1), cu,
                                           cpp, qip, pmp, cu.size - 1, Tq, Tk, H, D, K, idx, ln),
           "indexer_topk_local")
    del cp, qi, pm
    return idx, ln


def indexer_score_rows(q_row, k_idx, w_row, s: int) -> float:
    """Score of one query row (q_row [H,D], w_row [H]) against key s."""
    q = _u16(q_row)
    k = _u16(k_idx)
    wt = _np(w_row, np.float32)
    H, D = q.shape
    return lib().oracle_indexer_score(q.reshape(-1), k.reshape(-1), wt.reshape(-1), H, D, 0, s)


def _opt_i32(x):
    if x is None:
        return None, None
    a = _np(x, np.int32)
    return a, a.ctypes.data


def _opt_sink(sink, H):
    """Per-head sink logits as a double array [H] (exact widening), or None."""
    if sink is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(
        sink.detach().cpu().numpy() if hasattr(sink, "detach") else sink, np.float64).reshape(-1))
    if a.shape[0] != H:
        raise ValueError("sink must hold one logit per head")
    return a, a.ctypes.data


def sparse_mla_fwd(q, kv, idx, topk_length, scale: float, d_v: int, rows=None, sink=None):
    """Returns (out [n,H,Dv] f64, lse [n,H] f64) for query rows [r0, r1); `sink` [H] adds one
    zero-valued logit per head to the softmax denominator."""
    qa = _u16(q)
    kva = _u16(kv).reshape(kv.shape[0], -1)
    ia = _np(idx, np.int32).reshape(qa.shape[0], -1)
    tl, tlp = _opt_i32(topk_length)
    Tq, H, Dqk = qa.shape
    Tkv = kva.shape[0]
    K = ia.shape[1]
    r0, r1 = (0, Tq) if rows is None else rows
    sk, skp = _opt_sink(sink, H)
    out = np.zeros((r1 - r0, H, d_v), np.float64)
    lse = np.zeros((r1 - r0, H), np.float64)
    _check(lib().oracle_sparse_mla_fwd(qa.reshape(-1), kva.reshape(-1), ia.reshape(-1), tlp, Tq,
                                       Tkv, H, Dqk, d_v, K, float(scale), skp, r0, r1, out, lse),
           "sparse_mla_fwd")
    del tl, sk
    return out, lse


def sparse_mla_bwd(q, kv, idx, topk_length, dout, scale: float, rows=None, dkv=None, sink=None):
    """Returns (dq [n,H,Dqk] f64, dkv [T_kv,Dqk] f64) for query rows [r0, r1), and with a
    `sink` [H] also dsink [H] f64 (the sink logits' gradient summed over those rows).

    dkv accumulates the contributions of the given rows only (pass ``dkv`` to
    keep accumulating into an existing buffer)."""
    qa = _u16(q)
    kva = _u16(kv).reshape(kv.shape[0], -1)
    ia = _np(idx, np.int32).reshape(qa.shape[0], -1)
    da = _u16(dout)
    tl, tlp = _opt_i32(topk_length)
    Tq, H, Dqk = qa.shape
    Tkv = kva.shape[0]
    K = ia.shape[1]
    Dv = da.shape[2]
    r0, r1 = (0, Tq) if rows is None else rows
    dq = np.zeros((r1 - r0, H, Dqk), np.float64)
    if dkv is None:
        dkv = np.zeros((Tkv, Dqk), np.float64)
    sk, skp = _opt_sink(sink, H)
    dsink = np.zeros(H, np.float64) if sink is not None else None
    _check(lib().oracle_sparse_mla_bwd(qa.reshape(-1), kva.reshape(-1), ia.reshape(-1), tlp,
                                       da.reshape(-1), Tq, Tkv, H, Dqk, Dv, K, float(scale), skp,
                                       r0, r1, dq, dkv,
                                       None if dsink is None else dsink.ctypes.data),
           "sparse_mla_bwd")
    del tl, sk
    if sink is None:
        return dq, dkv
    return dq, dkv, dsink


def indexer_kl(q, kv, idx, topk_length, scale: float, q_idx, k_idx, w, g: float = 1.0,
               rows=None, sink=None, dk_idx=None):
    """Indexer KL loss and its gradients for query rows [r0, r1): a dict with target
    [n,K], loss [n], dq_idx [n,Hi,Di], dw [n,Hi] (row-relative) and dk_idx [T_kv,Di]
    (accumulated over the given rows; pass ``dk_idx`` to keep accumulating)."""
    qa = _u16(q)
    kva = _u16(kv).reshape(kv.shape[0], -1)
    ia = _np(idx, np.int32).reshape(qa.shape[0], -1)
    tl, tlp = _opt_i32(topk_length)
    qi = _u16(q_idx)
    ki = _u16(k_idx).reshape(k_idx.shape[0], -1)
    wa = _np(w, np.float32)
    Tq, H, Dqk = qa.shape
    Tkv = kva.shape[0]
    K = ia.shape[1]
    Hi, Di = qi.shape[1], qi.shape[2]
    if ki.shape[0] != Tkv or ki.shape[1] != Di or qi.shape[0] != Tq or wa.shape != (Tq, Hi):
        raise ValueError("indexer_kl: k_idx must have the rows of kv, q_idx / w the rows of q")
    r0, r1 = (0, Tq) if rows is None else rows
    n = r1 - r0
    sk, skp = _opt_sink(sink, H)
    target = np.zeros((n, K), np.float64)
    loss = np.zeros(n, np.float64)
    dq_idx = np.zeros((n, Hi, Di), np.float64)
    dw = np.zeros((n, Hi), np.float64)
    if dk_idx is None:
        dk_idx = np.zeros((Tkv, Di), np.float64)
    _check(lib().oracle_indexer_kl(qa.reshape(-1), kva.reshape(-1), ia.reshape(-1), tlp, Tq,
                                   Tkv, H, Dqk, K, float(scale), skp, qi.reshape(-1),
                                   ki.reshape(-1), wa.reshape(-1), Hi, Di, float(g), r0, r1,
                                   target, loss, dq_idx, dw, dk_idx), "indexer_kl")
    del tl, sk
    return dict(target=target, loss=loss, dq_idx=dq_idx, dw=dw, dk_idx=dk_idx)


def kpool_indexer(q_idx, k_pool, w, cu_seqlens, pool: int, K_pools: int, rows=None):
    """k-pool top-k of rows [r0, r1) (default all): (idx int32 [n, K_pools*pool + pool - 1],
    len int32 [n], kth f64 [n] the n-th best pool score); k_pool holds one key per complete
    pool of each sequence, in sequence order."""
    q = _u16(q_idx)
    k = _u16(k_pool)
    wt = _np(w, np.float32)
    cu = _np(cu_seqlens, np.int32)
    T, H, D = q.shape
    n_pools = int(sum((int(cu[b + 1]) - int(cu[b])) // pool for b in range(cu.shape[0] - 1)))
    if k.shape[0] != n_pools:
        raise ValueError(f"kpool_indexer: k_pool must hold {n_pools} rows (one per complete pool)")
    W = K_pools * pool + pool - 1
    r0, r1 = (0, T) if rows is None else rows
    idx = np.zeros((r1 - r0, W), np.int32)
    ln = np.zeros(r1 - r0, np.int32)
    kth = np.zeros(r1 - r0, np.float64)
    _check(lib().oracle_kpool_indexer(q.reshape(-1), k.reshape(-1), wt.reshape(-1), cu,
                                      cu.shape[0] - 1, T, H, D, pool, K_pools, r0, r1, idx, ln,
                                      kth.ctypes.data), "kpool_indexer")
    if rows is None:
        return idx, ln
    return idx, ln, kth
