"""Independent references that pin the oracle (CPU, float64).

These are written from the definitions with whole-matrix library routines
(numpy einsum / lexsort, torch's scaled_dot_product_attention and autograd),
so they share no code path with oracle/dsa_oracle.c.
"""

from __future__ import annotations

import numpy as np
import torch


def bf16_to_f64(x) -> np.ndarray:
    """bf16 tensor or uint16 bit array -> float64 numpy (exact widening)."""
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def segment_of(cu: np.ndarray, T: int) -> np.ndarray:
    """Sequence start of every token (written with searchsorted, not loops)."""
    cu = np.asarray(cu, dtype=np.int64)
    b = np.searchsorted(cu, np.arange(T), side="right") - 1
    return cu[b]


def brute_indexer_scores(q_idx, k_idx, w, cu) -> np.ndarray:
    """Full [T, T] score matrix; entries outside each row's causal keys are -inf."""
    q = bf16_to_f64(q_idx)
    k = bf16_to_f64(k_idx)
    wt = np.asarray(w.detach().cpu().numpy() if isinstance(w, torch.Tensor) else w, np.float64)
    dots = np.einsum("thd,sd->ths", q, k)
    scores = np.einsum("th,ths->ts", wt, np.maximum(dots, 0.0))
    T = q.shape[0]
    start = segment_of(cu, T)
    s = np.arange(T)
    ok = (s[None, :] >= start[:, None]) & (s[None, :] <= np.arange(T)[:, None])
    return np.where(ok, scores, -np.inf)


def brute_topk(scores: np.ndarray, K: int):
    """Top-K of each row by (score desc, position asc), ascending, -1 padded."""
    T = scores.shape[0]
    idx = np.full((T, K), -1, np.int32)
    ln = np.zeros(T, np.int32)
    pos = np.arange(scores.shape[1])
    for t in range(T):
        row = scores[t]
        valid = np.isfinite(row)
        order = np.lexsort((pos[valid], -row[valid]))  # last key is primary
        chosen = np.sort(pos[valid][order][:K])
        idx[t, :chosen.size] = chosen
        ln[t] = chosen.size
    return idx, ln


def dense_attention(q, kv, cu, scale: float, d_v: int, dout=None):
    """Dense block-causal attention in float64 via torch SDPA (and autograd).

    q [T,H,Dqk] bf16, kv [T,Dqk] bf16 (keys = kv, values = kv[:, :d_v]).
    Returns out [T,H,Dv], lse [T,H] and, if dout is given, dq and dkv."""
    qd = q.detach().to(torch.float64).clone().requires_grad_(dout is not None)
    kvd = kv.detach().to(torch.float64).clone().requires_grad_(dout is not None)
    T, H, D = qd.shape
    start = torch.as_tensor(segment_of(np.asarray(cu), T))
    t = torch.arange(T)
    mask = (t[None, :] >= start[:, None]) & (t[None, :] <= t[:, None])
    qh = qd.permute(1, 0, 2).unsqueeze(0)                      # [1,H,T,D]
    kh = kvd.unsqueeze(0).unsqueeze(0).expand(1, H, T, D)       # shared by all heads
    vh = kvd[:, :d_v].unsqueeze(0).unsqueeze(0).expand(1, H, T, d_v)
    out = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask,
                                                           scale=scale)
    out = out.squeeze(0).permute(1, 0, 2)                       # [T,H,Dv]
    logits = torch.einsum("thd,sd->hts", qd.detach(), kvd.detach()) * scale
    lse = torch.logsumexp(logits.masked_fill(~mask[None], float("-inf")), dim=-1).T
    res = dict(out=out.detach().numpy(), lse=lse.numpy())
    if dout is not None:
        out.backward(dout.detach().to(torch.float64))
        res["dq"] = qd.grad.numpy()
        res["dkv"] = kvd.grad.numpy()
    return res


def dense_attention_sink(q, kv, cu, scale: float, d_v: int, sink, dout=None):
    """Dense block-causal attention with a per-head sink, in float64 via torch SDPA.

    The sink is realised as one extra key whose key and value vectors are zero, so its logit
    scale * q . 0 = 0 is lifted to sink[h] by an additive mask, and it adds nothing to the
    output.  Returns out, lse and, if dout is given, dq, dkv and dsink (autograd)."""
    grad = dout is not None
    qd = q.detach().to(torch.float64).clone().requires_grad_(grad)
    kvd = kv.detach().to(torch.float64).clone().requires_grad_(grad)
    sk = torch.as_tensor(np.asarray(sink, np.float64)).clone().requires_grad_(grad)
    T, H, D = qd.shape
    start = torch.as_tensor(segment_of(np.asarray(cu), T))
    t = torch.arange(T)
    causal = (t[None, :] >= start[:, None]) & (t[None, :] <= t[:, None])
    zero_t = torch.zeros((T, T), dtype=torch.float64)
    real = zero_t.masked_fill(~causal, float("-inf"))                  # [T, T]
    bias = torch.cat([real.unsqueeze(0).expand(H, T, T),
                      sk[:, None, None].expand(H, T, 1)], dim=2)       # [H, T, T+1]
    keys = torch.cat([kvd, torch.zeros((1, D), dtype=torch.float64)], dim=0)
    vals = torch.cat([kvd[:, :d_v], torch.zeros((1, d_v), dtype=torch.float64)], dim=0)
    qh = qd.permute(1, 0, 2).unsqueeze(0)
    kh = keys.unsqueeze(0).unsqueeze(0).expand(1, H, T + 1, D)
    vh = vals.unsqueeze(0).unsqueeze(0).expand(1, H, T + 1, d_v)
    out = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=bias.unsqueeze(0),
                                                           scale=scale)
    out = out.squeeze(0).permute(1, 0, 2)
    logits = torch.einsum("thd,sd->hts", qd.detach(), keys.detach()) * scale + bias.detach()
    lse = torch.logsumexp(logits, dim=-1).T
    res = dict(out=out.detach().numpy(), lse=lse.numpy())
    if grad:
        out.backward(dout.detach().to(torch.float64))
        res["dq"] = qd.grad.numpy()
        res["dkv"] = kvd.grad.numpy()
        res["dsink"] = sk.grad.numpy()
    return res
