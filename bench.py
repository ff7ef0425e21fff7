"""Benchmark of the DSA hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input: THD metadata,
lightning indexer + top-k, sparse MLA forward, sparse MLA backward (delta, dq, dkv).

Default workload: the packed THD batch of 32768 tokens (sequences of 1024, 3072, 12288 and
16384 tokens), indexer 64 heads x 128 with k = 2048, attention H = 64 over 576-wide latent
rows (values = first 512 channels).  Inputs are generated on the GPU before timing and stay
resident in HBM.

Prints one JSON line.  `value` is hot-path tokens per second (query tokens through indexer,
forward and backward per second); `components` breaks it down per stage with algorithmic
TFLOP/s and the fraction of the bf16 dense MFMA peak; `roofline` describes the kernel with the
largest share of the step time, timed with HIP events recorded by the library around each of
its kernel launches; `cpu_baseline` times the CPU oracle on a bounded row sample.
`ms_per_step` is the wall-clock mean over the timed steps, `median_ms_per_step` the median of
per-step HIP events, and `cold_ms_per_step` one more step after 1 GiB has been written to
evict the inputs from L2 and the 256 MB last-level cache (not part of `value`).
`gather_ceiling` is the rate at which the GPU gathers uniformly random rows of the step's
latent table through LDS the way the attention kernels do, with nothing else to do (measured
after the timed steps); `components.*.gather_vs_ceiling` sets the forward's and backward's
gather rates against it.
"""

from __future__ import annotations

import argparse
import ctypes as C
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense bf16 MFMA peak (2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0
METRIC = "sparse-MLA fwd/bwd TFLOP/s + indexer top-k tokens/s at T=32K,k=2048; % roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, choices=[2, 3, 4, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget of the oracle sample")
    ap.add_argument("--bwd-passes", type=int, default=0,
                    help="query-row passes of the backward (several passes overlap a pass's "
                         "key-gradient reduction with the next pass's compute); 0: the fewest "
                         "whose workspace fits in 60%% of the free device memory")
    ap.add_argument("--layers", type=int, default=0,
                    help="attention layers per step sharing one indexer pass (IndexShare); 0: "
                         "the workload's own count (4 for the 131072-token block, else 1)")
    ap.add_argument("--cp", type=int, default=1, metavar="N",
                    help="time one GPU's share under N-way context parallelism: the query rows "
                         "of rank 0 (zig-zag: chunks 0 and 2N-1 of every sequence split in 2N) "
                         "against all keys, through the local-query metadata")
    ap.add_argument("--sink", action="store_true",
                    help="run the step with a per-head attention sink (sink forward epilogue and "
                         "sink gradient kernels added)")
    ap.add_argument("--indexer-loss", action="store_true",
                    help="add the indexer's KL training loss to the step: the score recompute "
                         "of the attention target and the indexer backward (coefficient 0.001 "
                         "over the rows)")
    ap.add_argument("--synthetic-indices", action="store_true",
                    help="k-pool workload: feed the attention seeded random causal indices "
                         "instead of running the k-pool indexer in the step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="after the timed steps, copy a device buffer of BYTES bytes once with "
                         "an elementwise kernel (x * 1): a plain copy of known size, which "
                         "scales the HBM byte counters of a profiler run")
    return ap.parse_args()


# Source files whose kernels each timed kernel runs (a counter summary is used only while
# their contents are unchanged).
KERNEL_SOURCES = {
    "indexer_topk": ["indexer_topk.hip", "tile.h", "dsa_common.h"],
    "sparse_mla_fwd": ["sparse_mla_fwd.hip", "tile.h", "dsa_common.h"],
    "sparse_mla_bwd_rows": ["sparse_mla_bwd.hip", "tile.h", "dsa_common.h", "dsa_internal.h"],
    "sparse_mla_bwd_reduce": ["sparse_mla_bwd.hip", "dsa_common.h", "dsa_internal.h"],
}


def source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sparse_attention_12_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` (fetched + written) from the committed counter summary
    profiles/<kernel>_<workload>_traffic.md, or None when there is none or it was taken on
    other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != source_digest(kernel):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measured_mfma(kernel: str, workload: str):
    """Counter-based MFMA figures of `kernel` from the committed summary
    profiles/<kernel>_<workload>_mfma.md (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE,
    SQ_INSTS_VALU_MFMA_MOPS_*, SQ_INSTS_VALU / SQ_INSTS_MFMA), or None when there is none or
    it was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_mfma.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.startswith("- "):
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != source_digest(kernel):
        return None
    try:
        return {"mfma_busy": float(fields["mfma_busy"]),
                "mfma_flops_executed": float(fields["mfma_flops_executed"]),
                "valu_per_mfma": float(fields["valu_per_mfma"])}
    except (KeyError, ValueError):
        return None


class KernelTimer:
    """Arms dsa_record_kernel_events with a pool of HIP events (created through the HIP
    runtime that torch already loaded)."""

    def __init__(self, dsa_lib, n_slots: int):
        self.hip = C.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.lib = dsa_lib

        class Slot(C.Structure):
            _fields_ = [("start", C.c_void_p), ("stop", C.c_void_p), ("name", C.c_char_p)]

        self.slots = (Slot * n_slots)()
        for s in self.slots:
            a, b = C.c_void_p(), C.c_void_p()
            assert self.hip.hipEventCreate(C.byref(a)) == 0
            assert self.hip.hipEventCreate(C.byref(b)) == 0
            s.start, s.stop = a, b
        self.n = n_slots
        self.used = C.c_int(0)
        self.lib.dsa_record_kernel_events.argtypes = [C.c_void_p, C.c_int, C.POINTER(C.c_int)]

    def arm(self):
        assert self.lib.dsa_record_kernel_events(C.byref(self.slots), self.n,
                                                 C.byref(self.used)) == 0

    def disarm(self):
        self.lib.dsa_record_kernel_events(None, 0, None)

    def totals(self):
        """{kernel name: [durations in ms]} for the recorded launches (after a sync)."""
        out = {}
        for i in range(self.used.value):
            s = self.slots[i]
            ms = C.c_float(0)
            assert self.hip.hipEventElapsedTime(C.byref(ms), s.start, s.stop) == 0
            out.setdefault(s.name.decode(), []).append(ms.value)
        return out


def ms_step_events(step_ev):
    """Mean step time from the per-step events."""
    n = len(step_ev) - 1
    return sum(step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(n)) / n


def kpool_pairs(cu_seqlens, pool, K_pools):
    """Pool scores of a k-pool indexer pass: every complete pool a row sees, for the rows that
    see more than K_pools of them (the others keep all their pools without scoring)."""
    import numpy as np
    pairs = 0
    for L in np.diff(np.array(cu_seqlens, np.int64)):
        P = (np.arange(L) + 1) // pool
        pairs += int(P[P > K_pools].sum())
    return pairs


def workload_counts(md_host, cfg, H_i, D_i, K, H, Dqk, Dv, kpool=None):
    """Algorithmic work of one step (see the module docstring of the pass)."""
    import numpy as np
    cu = np.array(cfg.cu_seqlens, np.int64)
    lens = np.diff(cu)
    # indexer: rows with L > K need every causal score; rows with L <= K are decided
    # without scoring (they keep their whole prefix)
    idx_pairs = 0
    if cfg.pool > 0:
        idx_pairs = kpool_pairs(cfg.cu_seqlens, cfg.pool, (K - cfg.pool + 1) // cfg.pool)
    else:
        for L in lens:
            if L > K:
                idx_pairs += (L * (L + 1) // 2) - (K * (K + 1) // 2)
    valid = md_host["total_valid"] if kpool is None else kpool
    return dict(
        idx_pairs=int(idx_pairs),
        idx_flops=float(idx_pairs) * 2 * H_i * D_i,
        valid=int(valid),
        fwd_flops=float(valid) * 2 * H * (Dqk + Dv),
        bwd_flops=float(valid) * 2 * H * (3 * Dqk + 2 * Dv),
        bwd_dq_flops=float(valid) * 2 * H * (2 * Dqk + Dv),
        bwd_dkv_flops=float(valid) * 2 * H * (Dqk + Dv),
    )


def cpu_baseline(inputs, counts, T, K, budget_s, pool=0, kl=False, sink=None, local_rows=None):
    """Time the oracle (as it stands) on a bounded sample of the same workload: the longest
    rows of the last sequence, sized from a small calibration run so that the stages take
    about budget_s seconds together; per-stage flop rates extrapolate to the whole step (with
    `kl`, the indexer's KL loss and backward as a fourth stage, extrapolated per valid slot).
    With `local_rows` (one GPU's query rows under context parallelism, global coordinates)
    the sample is the last local rows, which lie at the end of the last sequence, and the
    indexer leg is the oracle's local-query indexer."""
    import numpy as np

    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    q_idx = inputs["q_idx"].cpu()
    k_idx = (inputs["k_pool"] if pool else inputs["k_idx"]).cpu()
    w = inputs["w"].cpu()
    cu = inputs["cu_seqlens"].cpu()
    start = int(cu[-2])
    if local_rows is not None:
        gl = local_rows.cpu().numpy().astype(np.int64)
        last = len(gl) - 1  # rows are local: the sample is the last local rows
        n_tail = int((gl >= start).sum())  # local rows in the last sequence (they end the list)
        assert (gl[len(gl) - n_tail:] >= start).all()
    else:
        last = int(cu[-1]) - 1
    Hi, Di = q_idx.shape[1], q_idx.shape[2]
    q_all, idx_all, ln_all, do_all = inputs["q"], inputs["idx"], inputs["len"], inputs["dout"]
    kv = inputs["kv"].cpu()
    H, Dqk = q_all.shape[1], q_all.shape[2]
    per_stage = budget_s / (4.0 if kl else 3.0)
    max_rows = n_tail if local_rows is not None else last - start + 1

    def indexer(n):
        r0 = last - n + 1
        t0 = time.perf_counter()
        if local_rows is not None:
            rows_g = gl[r0:last + 1]
            oracle.indexer_topk_local(q_idx[r0:last + 1], k_idx, w[r0:last + 1], cu, K,
                                      query_indices=rows_g.astype(np.int32))
            return time.perf_counter() - t0, float((rows_g - start + 1).sum()) * 2.0 * Hi * Di
        if pool:
            oracle.kpool_indexer(q_idx, k_idx, w, cu, pool, (K - pool + 1) // pool,
                                 rows=(r0, last + 1))
        else:
            oracle.indexer_topk(q_idx, k_idx, w, cu, K, rows=(r0, last + 1))
        dt = time.perf_counter() - t0
        if pool:
            keys = sum((t - start + 1) // pool for t in range(r0, last + 1))
        else:
            keys = sum(t - start + 1 for t in range(r0, last + 1))
        return dt, keys * 2.0 * Hi * Di

    def attention(n, backward):
        sl = slice(last - n + 1, last + 1)
        q, idx, ln, dout = (x[sl].cpu() for x in (q_all, idx_all, ln_all, do_all))
        nvalid = int(ln.sum())
        t0 = time.perf_counter()
        if backward:
            oracle.sparse_mla_bwd(q, kv, idx, ln, dout, inputs["scale"], sink=sink)
        else:
            oracle.sparse_mla_fwd(q, kv, idx, ln, inputs["scale"], 512, sink=sink)
        dt = time.perf_counter() - t0
        per = (3 * Dqk + 2 * 512) if backward else (Dqk + 512)
        return dt, nvalid * 2.0 * H * per, nvalid

    def kl_loss(n):
        # target (the attention probabilities, recomputed), loss and the indexer backward
        r0 = last - n + 1
        nvalid = int(ln_all[r0:last + 1].sum())
        t0 = time.perf_counter()
        oracle.indexer_kl(q_all.cpu(), kv, idx_all.cpu(), ln_all.cpu(), inputs["scale"], q_idx,
                          k_idx, w, g=1.0, rows=(r0, last + 1))
        return time.perf_counter() - t0, nvalid

    def sized(run, n0):
        dt = run(n0)[0]  # calibration (also warms the library and caches)
        n = int(min(max_rows, max(n0, n0 * per_stage / max(dt, 1e-3))))
        return n, run(n)

    n_i, (t_idx, f_idx) = sized(indexer, max(1, threads // 2))
    n_f, (t_fwd, f_fwd, v_f) = sized(lambda n: attention(n, False), threads)
    n_b, (t_bwd, f_bwd, v_b) = sized(lambda n: attention(n, True), threads)
    idx_rate, fwd_rate, bwd_rate = f_idx / t_idx, f_fwd / t_fwd, f_bwd / t_bwd
    kl_slot_s = None
    if kl:
        n_k, (t_kl, v_kl) = sized(kl_loss, threads)
        kl_slot_s = t_kl / max(v_kl, 1)  # seconds per valid slot

    def step_seconds(ri, rf, rb, kls=None):
        return (counts["idx_flops"] / ri + counts["fwd_flops"] / rf + counts["bwd_flops"] / rb
                + (kls * counts["valid"] if kls else 0.0))

    full_s = step_seconds(idx_rate, fwd_rate, bwd_rate, kl_slot_s)
    # the same oracle on one thread (OpenMP's thread count set through libgomp for the calls
    # below), on samples an eighth of the size
    single = None
    try:
        gomp = C.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        try:
            t1i, f1i = indexer(max(1, n_i // 8))
            t1f, f1f, _ = attention(max(1, n_f // 8), False)
            t1b, f1b, _ = attention(max(1, n_b // 8), True)
            t1k, v1k = kl_loss(max(1, n_k // 8)) if kl else (0.0, 1)
        finally:
            gomp.omp_set_num_threads(threads)
        r1 = (f1i / t1i, f1f / t1f, f1b / t1b)
        single = {"value": T / step_seconds(*r1, t1k / max(v1k, 1) if kl else None),
                  "indexer_tflops": r1[0] / 1e12,
                  "fwd_tflops": r1[1] / 1e12, "bwd_tflops": r1[2] / 1e12,
                  "seconds": t1i + t1f + t1b + t1k}
    except OSError:
        pass
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": T / full_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "cpu_model": cpu_model,
        "sample": ((f"fp64 oracle on the last of this GPU's {max_rows} local rows of the last "
                    f"sequence: " if local_rows is not None else
                    f"fp64 oracle on the last rows of the {max_rows}-token sequence: ")
                   + f"{'k-pool ' if pool else ''}indexer "
                   f"top-k of {n_i} rows ({t_idx:.1f}s), forward of {n_f} rows / {v_f} valid "
                   f"slots ({t_fwd:.1f}s), backward of {n_b} rows / {v_b} valid slots "
                   f"({t_bwd:.1f}s)"
                   + (f", indexer KL loss and backward of {n_k} rows / {v_kl} valid slots "
                      f"({t_kl:.1f}s, extrapolated per valid slot)" if kl else "")
                   + "; per-stage flop rates extrapolated to the whole step; "
                   "single_thread: the same on one thread, samples of an eighth"),
        "indexer_tflops": idx_rate / 1e12, "fwd_tflops": fwd_rate / 1e12,
        "bwd_tflops": bwd_rate / 1e12, "single_thread": single,
        "indexer_loss_us_per_row": (kl_slot_s * counts["valid"] / T * 1e6) if kl else None,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by query rows; see the design notes)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import dsa_inputs as gen
    import sparse_attention_12_amd as dsa

    dev = "cuda"
    cfg = gen.workload(args.config)
    T, K = cfg.T, cfg.topk
    torch.manual_seed(0)
    cu = gen.cu_seqlens_tensor(cfg, dev)
    has_indexer = cfg.idx_heads is not None
    # the k-pool indexer: pools of cfg.pool keys, the K_pools best plus the tail pool (width K)
    kpool = cfg.pool > 0 and not args.synthetic_indices
    has_indexer = has_indexer and not args.synthetic_indices
    K_pools = (K - cfg.pool + 1) // cfg.pool if cfg.pool > 0 else 0
    inputs = dict(cu_seqlens=cu, scale=cfg.scale)
    if kpool:
        inputs.update(gen.kpool_indexer_inputs(args.config, device=dev, heads=cfg.idx_heads,
                                               dim=cfg.idx_dim))
    elif has_indexer:
        inputs.update(gen.indexer_inputs(args.config, device=dev))
    att = gen.attention_inputs(args.config, device=dev)
    n_layers = args.layers if args.layers > 0 else cfg.layers
    # every further layer has its own q, latent rows and output gradient (drawn per layer)
    extra_layers = [gen.attention_inputs(args.config, device=dev, layer=l)
                    for l in range(1, n_layers)]
    T_keys = T
    local_rows = None
    if args.cp > 1:
        if not has_indexer or kpool:
            raise SystemExit("--cp needs a workload with an indexer stage")
        # rank 0's rows under zig-zag context parallelism
        parts = []
        for b in range(len(cfg.cu_seqlens) - 1):
            ch = np.array_split(np.arange(cfg.cu_seqlens[b], cfg.cu_seqlens[b + 1]), 2 * args.cp)
            parts += [ch[0], ch[-1]]
        local_rows = torch.from_numpy(np.concatenate(parts).astype(np.int32)).to(dev)
        sel = local_rows.long()
        inputs.update(q_idx=inputs["q_idx"][sel].contiguous(), w=inputs["w"][sel].contiguous())
        att = dict(att, q=att["q"][sel].contiguous(), dout=att["dout"][sel].contiguous())
        extra_layers = [dict(a, q=a["q"][sel].contiguous(), dout=a["dout"][sel].contiguous())
                        for a in extra_layers]
        T = local_rows.numel()
    inputs.update(q=att["q"], kv=att["kv"], dout=att["dout"])
    H, Dqk, Dv = cfg.heads, cfg.d_qk, cfg.d_v
    idx_buf = torch.empty((T, K), dtype=torch.int32, device=dev)
    len_buf = torch.empty((T,), dtype=torch.int32, device=dev)
    out_buf = torch.empty((T, H, Dv), dtype=torch.bfloat16, device=dev)
    lse_buf = torch.empty((T, H), dtype=torch.float32, device=dev)
    dq_buf = torch.empty_like(att["q"])
    dkv_buf = torch.empty((T_keys, Dqk), dtype=torch.float32, device=dev)
    # backward workspace for --bwd-passes passes over the query rows
    if args.bwd_passes <= 0:
        free = torch.cuda.mem_get_info()[0]
        args.bwd_passes = 1
        while (args.bwd_passes < T and dsa.bwd_workspace_bytes(
                T, T_keys, H, Dqk, K, rows_per_pass=-(-T // args.bwd_passes)) > 0.6 * free):
            args.bwd_passes *= 2
    rows_per_pass = -(-T // max(1, args.bwd_passes))
    ws = torch.empty(dsa.bwd_workspace_bytes(T, T_keys, H, Dqk, K, rows_per_pass=rows_per_pass),
                     dtype=torch.uint8, device=dev)
    sink = gen.sink_logits(H, device=dev) if args.sink else None
    dsink_buf = torch.empty((H,), dtype=torch.float32, device=dev) if args.sink else None
    kpool_valid = None
    if not has_indexer and cfg.pool > 0:
        kp = gen.kpool_indices(T, topk=K, tail=cfg.kpool_tail, device=dev)
        idx_buf.copy_(kp)
        len_buf.copy_((kp >= 0).sum(1).to(torch.int32))
        kpool_valid = int(len_buf.sum().item())
        del kp

    kl = args.indexer_loss
    if kl and (not has_indexer or kpool):
        raise SystemExit("--indexer-loss needs a workload with an indexer stage")
    if kl and args.sink:
        raise SystemExit("--indexer-loss and --sink are measured separately")
    if kl:
        tgt_buf = torch.empty((T, K), dtype=torch.float32, device=dev)
        dk_idx_buf = torch.empty((T_keys, cfg.idx_dim), dtype=torch.float32, device=dev)
        kl_ws = torch.empty(dsa.indexer_kl_bwd_workspace_bytes(T, T_keys, K), dtype=torch.uint8,
                            device=dev)
        kl_grad = 0.001 / T
    bwd_events = []  # (start, stop) around each backward call while timing
    kl_events = []   # (start, stop) around the indexer loss while timing

    def step():
        if kpool:
            md = dsa.prepare_kpool_metadata(cu, cfg.pool, K_pools)
            dsa.kpool_indexer_topk(inputs["q_idx"], inputs["k_pool"], inputs["w"], md, K_pools,
                                   idx=idx_buf, length=len_buf)
        elif local_rows is None:
            # the metadata's top-k width is an indexer width (at most 2048); synthetic k-pool
            # indices (width 2051) carry their own lengths
            md = dsa.prepare_thd_metadata(cu, min(K, dsa.MAX_INDEXER_TOPK), T=T)
        else:
            md = dsa.prepare_local_metadata(cu, T_keys, K, query_indices=local_rows)
        if has_indexer and not kpool:
            dsa.indexer_topk(inputs["q_idx"], inputs["k_idx"], inputs["w"], md, K, idx=idx_buf,
                             length=len_buf)
        for li, a in enumerate([att] + extra_layers):  # the layers reuse the indexer's indices
            dsa.sparse_mla_fwd(a["q"], a["kv"], idx_buf, cfg.scale, len_buf, out=out_buf,
                               lse=lse_buf, sink=sink)
            if timing:
                ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                ev[0].record()
            # with the indexer loss, the first layer's backward also writes the loss's target
            # (the fused KL-score path: the head sums of the probabilities it recomputes)
            dsa.sparse_mla_bwd(a["q"], a["kv"], idx_buf, out_buf, lse_buf, a["dout"],
                               cfg.scale, len_buf, dkv=dkv_buf, dq=dq_buf, workspace=ws,
                               sink=sink, dsink=dsink_buf,
                               kl_target=tgt_buf if kl and li == 0 else None)
            if timing:
                ev[1].record()
                bwd_events.append(ev)
            if kl and li == 0:
                # the indexer's KL loss and its backward against the first layer's attention
                if timing:
                    kev = (torch.cuda.Event(enable_timing=True),
                           torch.cuda.Event(enable_timing=True))
                    kev[0].record()
                dsa.indexer_kl_bwd(inputs["q_idx"], inputs["k_idx"], inputs["w"], idx_buf,
                                   tgt_buf, kl_grad, len_buf, dk_idx=dk_idx_buf,
                                   workspace=kl_ws)
                if timing:
                    kev[1].record()
                    kl_events.append(kev)
        return md

    timing = False
    for _ in range(args.warmup):
        md = step()
    torch.cuda.synchronize()
    md_host = dict(total_valid=md.total_valid)
    if kpool:
        kpool_valid = int(len_buf.sum().item())  # key slots the attention reads
    counts = workload_counts(md_host, cfg, cfg.idx_heads if has_indexer else 0,
                             cfg.idx_dim if has_indexer else 0, K, H, Dqk, Dv, kpool_valid)
    if local_rows is not None:
        # scored pairs of the local rows: every causal key of a row with L > K
        L_rows = md.causal_len.to(torch.int64)
        pairs = int(L_rows[L_rows > K].sum().item())
        counts.update(idx_pairs=pairs,
                      idx_flops=float(pairs) * 2 * cfg.idx_heads * cfg.idx_dim)

    timer = KernelTimer(dsa.lib(), 64 * args.steps * n_layers * max(1, args.bwd_passes))
    timing = True
    timer.arm()
    torch.cuda.synchronize()
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    step_ev[0].record()
    for i in range(args.steps):
        step()
        step_ev[i + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timer.disarm()
    per_kernel = timer.totals()
    step_ms = sorted(step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(args.steps))
    median_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else \
        0.5 * (step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    # one cold step: 1 GiB written first evicts the inputs from L2 and the 256 MB MALL
    timing = False
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    flush.fill_(1.0)
    cold_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    cold_ev[0].record()
    step()
    cold_ev[1].record()
    torch.cuda.synchronize()
    cold_ms = cold_ev[0].elapsed_time(cold_ev[1])
    del flush
    # gather ceiling: uniformly random rows of the step's latent table (up to 2^23 of them),
    # streamed through LDS as the attention kernels gather them and used for nothing else
    # (dsa_gather_probe); the median of three runs
    n_g = max(1 << 20, min(counts["valid"], 1 << 23)) // 2048 * 2048
    g_rows = torch.randint(0, T_keys, (n_g,), device=dev, dtype=torch.int32,
                           generator=torch.Generator(device=dev).manual_seed(0x6A7E))
    dsa.gather_probe(att["kv"], g_rows)
    g_ms = []
    for _ in range(3):
        gev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        gev[0].record()
        dsa.gather_probe(att["kv"], g_rows)
        gev[1].record()
        torch.cuda.synchronize()
        g_ms.append(gev[0].elapsed_time(gev[1]))
    g_ms = sorted(g_ms)[1]
    gather_ceiling = {"gbs": n_g * Dqk * 2 / g_ms / 1e6, "ms": g_ms, "rows": n_g,
                      "row_bytes": Dqk * 2, "table_mb": T_keys * Dqk * 2 / 1e6,
                      "frac_hbm_peak": n_g * Dqk * 2 / g_ms / 1e6 / PEAK_HBM_GBS}
    del g_rows

    ms_step = elapsed * 1e3 / args.steps
    value = T * args.steps / elapsed

    def avg(name):
        v = per_kernel.get(name, [])
        return sum(v) / len(v) if v else float("nan")

    def avg_or_zero(name):
        v = per_kernel.get(name, [])
        return sum(v) / len(v) if v else 0.0

    # each kernel's second launch (rows whose speculative threshold or fixed softmax reference
    # failed are recomputed there) belongs to its stage
    t_idx = avg("indexer_topk") + avg_or_zero("indexer_topk_redo")
    if kpool:  # the expansion of the selected pools to their keys belongs to the indexer
        t_idx += avg("kpool_expand")
    t_fwd = avg("sparse_mla_fwd") + avg_or_zero("sparse_mla_fwd_redo")
    # the backward's own wall time (its passes overlap on two streams, so kernel times overlap)
    t_bwd = sum(a.elapsed_time(b) for a, b in bwd_events) / len(bwd_events)
    # latent rows gathered per valid slot: once in the forward, twice in the backward (its dq
    # and key-gradient phases); these bytes mostly come from L2 and the last-level cache
    row_bytes = counts["valid"] * Dqk * 2
    comp = {
        "fwd": {"ms": t_fwd, "tflops": counts["fwd_flops"] / t_fwd / 1e9,
                "frac_mfma_peak": counts["fwd_flops"] / t_fwd / 1e9 / PEAK_BF16_TFLOPS,
                "gather_gbs": row_bytes / t_fwd / 1e6},
        "bwd": {"ms": t_bwd, "tflops": counts["bwd_flops"] / t_bwd / 1e9,
                "frac_mfma_peak": counts["bwd_flops"] / t_bwd / 1e9 / PEAK_BF16_TFLOPS,
                "gather_gbs": 2 * row_bytes / t_bwd / 1e6},
    }
    for c in ("fwd", "bwd"):
        comp[c]["gather_vs_ceiling"] = comp[c]["gather_gbs"] / gather_ceiling["gbs"]
    if has_indexer:
        comp["indexer"] = {"ms": t_idx, "tokens_per_s": T / (t_idx * 1e-3),
                           "tflops": counts["idx_flops"] / t_idx / 1e9,
                           "frac_mfma_peak": counts["idx_flops"] / t_idx / 1e9 / PEAK_BF16_TFLOPS}
    if kl:
        # MFMA work per valid slot of the indexer backward: the dot products in both passes,
        # dq_idx and the key-gradient contributions (4 x 2 H_i D_i); the target comes out of
        # the attention backward (its extra time is inside the backward's)
        kl_flops = counts["valid"] * 8.0 * cfg.idx_heads * cfg.idx_dim
        t_kl = sum(a.elapsed_time(b) for a, b in kl_events) / len(kl_events)
        comp["indexer_loss"] = {"ms": t_kl, "share_of_step": t_kl / ms_step_events(step_ev),
                                "target": "fused into the attention backward",
                                "bwd_rows_ms": avg("indexer_kl_bwd"),
                                "tflops": kl_flops / t_kl / 1e9,
                                "frac_mfma_peak": kl_flops / t_kl / 1e9 / PEAK_BF16_TFLOPS}
    if args.sink:
        # HBM-streaming kernels: the epilogue reads and writes out [T,H,Dv] bf16 and lse; the
        # gradient kernel reads out, dout and lse
        for name, nbytes in (("sink_fwd", T * H * (4 * Dv + 8)), ("sink_bwd", T * H * (4 * Dv + 4))):
            ms = avg(name)
            comp[name] = {"ms": ms, "gbs": nbytes / ms / 1e6,
                          "frac_hbm_peak": nbytes / ms / 1e6 / PEAK_HBM_GBS}
    kernels = {n: {"avg_ms": sum(v) / len(v), "launches": len(v)} for n, v in per_kernel.items()}
    # counter-based MFMA utilisation beside the algorithmic fractions (committed summaries)
    for comp_name, kern in (("indexer", "indexer_topk"), ("fwd", "sparse_mla_fwd"),
                            ("bwd", "sparse_mla_bwd_rows")):
        if comp_name in comp:
            comp[comp_name]["counters"] = measured_mfma(kern, cfg.name)

    # algorithmic work per launch of each hot kernel: MFMA flops, or HBM bytes for the
    # reduction of the staged key-gradient contributions (a staged row of 2 bytes per channel
    # and 16 exponent bytes, and the 4-byte pair id, read once per valid pair; dkv read and
    # written)
    passes = max(1, len(per_kernel.get("sparse_mla_bwd_rows", [])) // args.steps)
    work = {"indexer_topk": ("mfma", counts["idx_flops"]),
            "sparse_mla_fwd": ("mfma", counts["fwd_flops"]),
            "sparse_mla_bwd_rows": ("mfma", counts["bwd_flops"] / passes),
            "sparse_mla_bwd_reduce": ("hbm", (counts["valid"] * (Dqk * 2 + 20) / passes
                                              + 2 * T_keys * Dqk * 4))}
    dom = max((n for n in work if n in per_kernel), key=lambda n: sum(per_kernel[n]))
    bound, amount = work[dom]
    if bound == "mfma":
        achieved, peak, unit = amount / avg(dom) / 1e9, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = amount / avg(dom) / 1e6, PEAK_HBM_GBS, "GB/s"
    roofline = {"kernel": dom, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": measured_traffic(dom, cfg.name)}
    if args.copy_calibration:
        # an elementwise kernel that reads and writes BYTES each (copy_ would use the DMA path)
        a = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del a, b

    res = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "median_ms_per_step": median_ms,
        "cold_ms_per_step": cold_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": T, "cu_seqlens": list(cfg.cu_seqlens),
                   "indexer": ((f"{cfg.idx_heads}x{cfg.idx_dim}"
                                + (f", pools of {cfg.pool}, {K_pools} best + tail pool"
                                   if kpool else "")) if has_indexer else None),
                   "topk": K, "heads": H, "d_qk": Dqk, "d_v": Dv, "bwd_passes": args.bwd_passes,
                   "attention_sink": bool(args.sink), "attention_layers": n_layers,
                   "indexer_loss": bool(kl),
                   "context_parallel": ({"ranks": args.cp, "rank": 0, "local_tokens": T,
                                         "key_tokens": T_keys} if args.cp > 1 else None),
                   "parallelism": "none"},
        "components": comp, "kernels": kernels, "roofline": roofline,
        "gather_ceiling": gather_ceiling,
    }
    if not args.no_cpu_baseline:
        inputs.update(idx=idx_buf, len=len_buf)
        try:
            res["cpu_baseline"] = cpu_baseline(inputs, counts, T, K, args.cpu_seconds,
                                               pool=cfg.pool if kpool else 0, kl=kl,
                                               sink=sink.cpu() if sink is not None else None,
                                               local_rows=local_rows)
        except Exception as e:  # the GPU figure stands on its own
            res["cpu_baseline"] = {"error": repr(e)}
    print(json.dumps(res))


if __name__ == "__main__":
    main()
