"""Seeded synthetic inputs for the DSA indexer and absorbed sparse MLA.

This module only draws random tensors; it holds none of the method's
arithmetic (no scores, no selection, no softmax).  Both the CPU oracle and the
HIP path consume exactly the tensors it returns, so the two sides always see
identical bits.

Shapes and value distributions follow the five workloads of the DSA hot path:

  1  tiny single sequence, T=256: integer-valued indexer inputs (exact in fp32),
     H=16 attention over 576-wide latent rows;
  2  one 8192-token sequence with the DeepSeek-V3.2 / GLM-5.2 indexer shape
     (64 heads x 128), top-k 2048, forward only;
  3  packed THD batch of 32768 tokens in four sequences (1024, 3072, 12288,
     16384), forward and backward;
  4  GLM-5.3-Flash NoPE shard: T=65536, H=8, q/k width 512, top-k width 2051;
     its indices come from the k-pool indexer (64 heads x 128 over pools of 4
     keys, the 512 best pools plus the tail pool), or for attention-only cases
     from a random causal subset plus the three most recent tokens;
  5  IndexShare block: T=131072, indexer once, four attention layers.

The indexer shape (64 heads of width 128, k=2048) is the one the Megatron
flags list on the NVIDIA GLM-5.2 cuDNN DSA page ("How DSA works"); the latent
width 576 = 512 + 64 and the value width 512 come from the NeMo AutoModel
cudnn_dsa API reference (`cudnn_sparse_attention`, argument q); the NoPE width
512 and the 2048 + 3 = 2051 top-k width come from SkyRL PR 2388 ("Why").

Every tensor is drawn in float32 from one torch.Generator per workload and
rounded to bfloat16 with round-to-nearest-even.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

SEED_BASE = 0xD5A0


@dataclass(frozen=True)
class Workload:
    name: str
    cu_seqlens: tuple
    # indexer (None when the workload feeds synthetic indices to attention)
    idx_heads: int | None
    idx_dim: int | None
    topk: int
    idx_int_inputs: bool
    # attention
    heads: int
    d_qk: int
    d_v: int
    attn_std: float
    backward: bool
    layers: int = 1
    kpool_tail: int = 0          # >0: synthetic k-pool indices (random subset + tail)
    pool: int = 0                # >0: the indexer selects pools of this many keys (k-pool)
    notes: str = field(default="")

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)


WORKLOADS = {
    1: Workload("tiny-T256", (0, 256), 4, 64, 64, True, 16, 576, 512, 1.0, True),
    2: Workload("v32-T8192", (0, 8192), 64, 128, 2048, False, 64, 576, 512, 0.5, False),
    3: Workload("thd-T32768", (0, 1024, 4096, 16384, 32768), 64, 128, 2048, False,
                64, 576, 512, 0.5, True),
    4: Workload("nope-kpool-T65536", (0, 65536), 64, 128, 2051, False, 8, 512, 512, 0.5,
                True, kpool_tail=3, pool=4),
    5: Workload("indexshare-T131072", (0, 131072), 64, 128, 2048, False, 64, 576, 512, 0.5,
                True, layers=4),
}


def workload(cfg: int, cu_seqlens=None) -> Workload:
    """Return workload ``cfg``; ``cu_seqlens`` overrides the packing (reduced sizes)."""
    w = WORKLOADS[cfg]
    if cu_seqlens is None:
        return w
    return Workload(**{**w.__dict__, "cu_seqlens": tuple(int(x) for x in cu_seqlens)})


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def cu_seqlens_tensor(w: Workload, device="cpu") -> torch.Tensor:
    return torch.tensor(w.cu_seqlens, dtype=torch.int32, device=device)


def indexer_inputs(cfg: int, cu_seqlens=None, device="cpu", seed=None):
    """Indexer query [T,Hi,Di] bf16, key [T,Di] bf16, weights [T,Hi] fp32.

    Workload 1 draws integers uniform in [-4, 4] for q and k and weights from
    {0.5, 1, 2}; the others draw q, k ~ N(0,1) and weights ~ N(0,1)/8.  The
    weights are handed over as already scaled (the caller owns any
    1/sqrt(heads) and 1/sqrt(dim) factors).
    """
    w = workload(cfg, cu_seqlens)
    assert w.idx_heads is not None and w.pool == 0, "workload has no token-level indexer"
    T, Hi, Di = w.T, w.idx_heads, w.idx_dim
    g = _gen((seed if seed is not None else SEED_BASE + cfg), device)
    if w.idx_int_inputs:
        q = torch.randint(-4, 5, (T, Hi, Di), generator=g, device=device).to(torch.bfloat16)
        k = torch.randint(-4, 5, (T, Di), generator=g, device=device).to(torch.bfloat16)
        choice = torch.randint(0, 3, (T, Hi), generator=g, device=device)
        wt = torch.tensor([0.5, 1.0, 2.0], device=device)[choice].to(torch.float32)
    else:
        q = torch.randn((T, Hi, Di), generator=g, device=device).to(torch.bfloat16)
        k = torch.randn((T, Di), generator=g, device=device).to(torch.bfloat16)
        wt = (torch.randn((T, Hi), generator=g, device=device) / 8.0).to(torch.float32)
    return dict(q_idx=q.contiguous(), k_idx=k.contiguous(), w=wt.contiguous(),
                cu_seqlens=cu_seqlens_tensor(w, device), topk=w.topk)


def indexer_trend_inputs(cu_seqlens, trend: str, heads=64, dim=128, block=256, device="cpu",
                         seed=None):
    """Integer indexer inputs whose scores follow a trend along each sequence.

    Key s at offset p = s - start of its sequence is c(p) * v, with v a fixed vector of 1s and
    2s and c(p) = max(1, 64 - p // block) ("falling") or min(64, 1 + p // block) ("rising");
    every query row has entries in [0, 2] with a 1 in its first column and weights from
    {0.5, 1, 2}, all positive, so a row's scores are c(p) times a positive row constant (exact
    in fp32).  Falling scores put a row's largest keys at its start, unlike a uniform sample;
    rising ones at its end.  Shapes as indexer_inputs; cu_seqlens is a list of offsets."""
    assert trend in ("falling", "rising")
    cu = [int(x) for x in cu_seqlens]
    T = cu[-1]
    g = _gen(seed if seed is not None else SEED_BASE + 0x500, device)
    v = torch.randint(1, 3, (dim,), generator=g, device=device).to(torch.float32)
    p = torch.zeros(T, dtype=torch.int64, device=device)
    for b in range(len(cu) - 1):
        p[cu[b]:cu[b + 1]] = torch.arange(cu[b + 1] - cu[b], device=device)
    if trend == "falling":
        c = torch.clamp(64 - p // block, min=1)
    else:
        c = torch.clamp(1 + p // block, max=64)
    k = (c.to(torch.float32)[:, None] * v[None, :]).to(torch.bfloat16)
    q = torch.randint(0, 3, (T, heads, dim), generator=g, device=device)
    q[:, :, 0] = 1
    choice = torch.randint(0, 3, (T, heads), generator=g, device=device)
    wt = torch.tensor([0.5, 1.0, 2.0], device=device)[choice].to(torch.float32)
    return dict(q_idx=q.to(torch.bfloat16).contiguous(), k_idx=k.contiguous(),
                w=wt.contiguous(), cu_seqlens=torch.tensor(cu, dtype=torch.int32, device=device))


def kpool_indexer_inputs(cfg: int, cu_seqlens=None, device="cpu", seed=None, pool=None,
                         heads=64, dim=128, int_inputs=False):
    """k-pool indexer query [T,Hi,Di] bf16, one pooled indexer key per complete pool of each
    sequence [T_pool,Di] bf16 (T_pool = sum of floor(length / pool)), weights [T,Hi] fp32.
    Float inputs: q, k ~ N(0,1), weights ~ N(0,1)/8; integer inputs as workload 1."""
    w = workload(cfg, cu_seqlens)
    T = w.T
    if pool is None:
        pool = w.pool if w.pool > 0 else 4
    n_pools = sum((w.cu_seqlens[b + 1] - w.cu_seqlens[b]) // pool
                  for b in range(len(w.cu_seqlens) - 1))
    g = _gen((seed if seed is not None else SEED_BASE + cfg + 0x300), device)
    if int_inputs:
        q = torch.randint(-4, 5, (T, heads, dim), generator=g, device=device).to(torch.bfloat16)
        k = torch.randint(-4, 5, (n_pools, dim), generator=g, device=device).to(torch.bfloat16)
        choice = torch.randint(0, 3, (T, heads), generator=g, device=device)
        wt = torch.tensor([0.5, 1.0, 2.0], device=device)[choice].to(torch.float32)
    else:
        q = torch.randn((T, heads, dim), generator=g, device=device).to(torch.bfloat16)
        k = torch.randn((n_pools, dim), generator=g, device=device).to(torch.bfloat16)
        wt = (torch.randn((T, heads), generator=g, device=device) / 8.0).to(torch.float32)
    return dict(q_idx=q.contiguous(), k_pool=k.contiguous(), w=wt.contiguous(),
                cu_seqlens=cu_seqlens_tensor(w, device), pool=pool)


def attention_inputs(cfg: int, cu_seqlens=None, device="cpu", layer=0, seed=None,
                     heads=None, d_qk=None):
    """Absorbed query [T,H,Dqk], latent rows [T,Dqk], output grad [T,H,Dv] (bf16)."""
    w = workload(cfg, cu_seqlens)
    T = w.T
    H = heads if heads is not None else w.heads
    Dqk = d_qk if d_qk is not None else w.d_qk
    base = seed if seed is not None else SEED_BASE + cfg + 0x100
    g = _gen(base + 16 * layer, device)
    q = (torch.randn((T, H, Dqk), generator=g, device=device) * w.attn_std).to(torch.bfloat16)
    kv = (torch.randn((T, Dqk), generator=g, device=device) * w.attn_std).to(torch.bfloat16)
    dout = torch.randn((T, H, w.d_v), generator=g, device=device).to(torch.bfloat16)
    return dict(q=q.contiguous(), kv=kv.contiguous(), dout=dout.contiguous(),
                scale=1.0 / math.sqrt(Dqk), d_v=w.d_v)


def sink_logits(H: int, device="cpu", seed=None) -> torch.Tensor:
    """Per-head attention-sink logits fp32 [H] ~ N(0,1) * 2 (the pages give no distribution;
    this spread lets the sink dominate some heads and vanish in others)."""
    g = _gen(seed if seed is not None else SEED_BASE + 0x200 + H, device)
    return (torch.randn((H,), generator=g, device=device) * 2.0).to(torch.float32).contiguous()


def kpool_indices(T: int, topk: int = 2051, tail: int = 3, device="cpu", seed=None,
                  row_block: int = 256) -> torch.Tensor:
    """Synthetic k-pool selection for a single causal sequence, int32 [T, topk].

    Row t with t+1 > topk: (topk - tail) distinct positions drawn uniformly
    without replacement from [0, t - tail], sorted ascending, followed by the
    ``tail`` most recent positions t-tail+1 .. t.  Rows with t+1 <= topk hold
    0..t followed by -1.  This mirrors the GLM-5.3-Flash k-pool width (2048
    selected plus the query's incomplete tail pool of 3).
    """
    g = _gen(seed if seed is not None else SEED_BASE + 0x404, device)
    out = torch.full((T, topk), -1, dtype=torch.int32, device=device)
    ar = torch.arange(topk, device=device, dtype=torch.int32)
    short = min(T, topk)
    # rows whose whole causal prefix fits
    rows = torch.arange(short, device=device, dtype=torch.int32)
    out[:short] = torch.where(ar[None, :] <= rows[:, None], ar[None, :].expand(short, topk),
                              torch.full_like(out[:short], -1))
    nsel = topk - tail
    for r0 in range(short, T, row_block):
        r1 = min(T, r0 + row_block)
        t = torch.arange(r0, r1, device=device)
        pool = r1 - tail                     # max candidate count (positions 0..t-tail)
        keys = torch.rand((r1 - r0, pool), generator=g, device=device)
        pos = torch.arange(pool, device=device)
        keys = torch.where(pos[None, :] <= (t - tail)[:, None], keys, torch.full_like(keys, -1.0))
        sel = torch.topk(keys, nsel, dim=1).indices.sort(dim=1).values.to(torch.int32)
        out[r0:r1, :nsel] = sel
        out[r0:r1, nsel:] = (t[:, None] - tail + 1 + torch.arange(tail, device=device)[None, :]
                             ).to(torch.int32)
    return out


def bf16_bits(x: torch.Tensor):
    """bfloat16 tensor -> numpy uint16 array of its bit patterns (host copy)."""
    return x.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
