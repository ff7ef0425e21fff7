"""Python binding of libdsa (DeepSeek Sparse Attention hot path on MI355X / gfx950).

Argument marshalling only: every step of the indexer, the top-k selection and the sparse MLA
forward / backward runs in the HIP kernels of lib/libdsa.so, called through its C ABI
(include/dsa.h).  PyTorch supplies device memory and the current stream.  There is no
fallback: if the library is missing or the device is not gfx950 the calls raise.

Errors map onto the exception classes of the NeMo AutoModel cudnn_dsa wrappers
(cudnn_indexer_topk / cudnn_sparse_attention "Raises"): RuntimeError for an unavailable
device or library, TypeError for wrong dtypes, ValueError for shapes, sizes and values.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libdsa.so")

DSA_OK = 0
DSA_ERR_INVALID_VALUE = 1
DSA_ERR_UNSUPPORTED = 2
DSA_ERR_WORKSPACE = 3
DSA_ERR_HIP = 4
DSA_BWD_ACCUMULATE_DKV = 0x1
DSA_DEBUG_CHECK_INDICES = 0x100
MAX_INDEXER_TOPK = 2048


class _Metadata(C.Structure):
    _fields_ = [("seq_start", C.c_void_p), ("causal_len", C.c_void_p),
                ("topk_length", C.c_void_p), ("row_order", C.c_void_p), ("groups", C.c_void_p),
                ("T", C.c_int64), ("B", C.c_int32), ("K", C.c_int32), ("max_seqlen", C.c_int32),
                ("all_rows_nonempty", C.c_int32), ("total_pairs", C.c_int64),
                ("total_valid", C.c_int64), ("n_groups", C.c_int32), ("gpos", C.c_void_p),
                ("group_first", C.c_void_p), ("total_key_tokens", C.c_int64),
                ("key_start", C.c_void_p), ("pool", C.c_int32)]


_lib = None


def lib():
    """Load libdsa.so (raises RuntimeError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libdsa.so not found at {LIB_PATH}; build it with "
                               "`python -m sparse_attention_12_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, u32, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_float, C.c_size_t
        L.dsa_last_error.restype = C.c_char_p
        L.dsa_last_error.argtypes = []
        L.dsa_device_supported.restype = C.c_int
        L.dsa_device_supported.argtypes = [C.c_int]
        L.dsa_thd_metadata_workspace_size.restype = sz
        L.dsa_thd_metadata_workspace_size.argtypes = [i64]
        L.dsa_prepare_thd_metadata.restype = C.c_int
        L.dsa_prepare_thd_metadata.argtypes = [vp, i32, i64, i32, vp, sz, C.POINTER(_Metadata), vp]
        L.dsa_local_metadata_workspace_size.restype = sz
        L.dsa_local_metadata_workspace_size.argtypes = [i64]
        L.dsa_prepare_local_metadata.restype = C.c_int
        L.dsa_prepare_local_metadata.argtypes = [vp, vp, vp, vp, i32, i64, i64, i32, vp, sz,
                                                 C.POINTER(_Metadata), vp]
        L.dsa_kpool_metadata_workspace_size.restype = sz
        L.dsa_kpool_metadata_workspace_size.argtypes = [i64]
        L.dsa_prepare_kpool_metadata.restype = C.c_int
        L.dsa_prepare_kpool_metadata.argtypes = [vp, i32, i64, i32, i32, vp, sz,
                                                 C.POINTER(_Metadata), vp]
        L.dsa_kpool_indexer_topk_workspace_size.restype = sz
        L.dsa_kpool_indexer_topk_workspace_size.argtypes = [i64, i32]
        L.dsa_kpool_indexer_topk.restype = C.c_int
        L.dsa_kpool_indexer_topk.argtypes = [vp, vp, vp, C.POINTER(_Metadata), i32, i32, i32, vp,
                                             vp, vp, sz, vp]
        L.dsa_indexer_topk_workspace_size.restype = sz
        L.dsa_indexer_topk_workspace_size.argtypes = [i64, i32, i32, i32]
        L.dsa_indexer_topk.restype = C.c_int
        L.dsa_indexer_topk.argtypes = [vp, vp, vp, C.POINTER(_Metadata), i32, i32, i32, vp, vp, vp,
                                       sz, vp]
        L.dsa_sparse_mla_fwd.restype = C.c_int
        L.dsa_sparse_mla_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, f32, vp, vp,
                                         vp]
        L.dsa_sparse_mla_bwd_workspace_size.restype = sz
        L.dsa_sparse_mla_bwd_workspace_size.argtypes = [i64, i64, i32, i32, i32, i64]
        L.dsa_sparse_mla_bwd.restype = C.c_int
        L.dsa_sparse_mla_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, i32,
                                         f32, vp, vp, u32, vp, sz, vp]
        L.dsa_sparse_mla_fwd_sink.restype = C.c_int
        L.dsa_sparse_mla_fwd_sink.argtypes = [vp, vp, vp, vp, i64, i64, i32, i32, i32, i32, f32,
                                              vp, vp, vp, vp]
        L.dsa_sparse_mla_bwd_sink.restype = C.c_int
        L.dsa_sparse_mla_bwd_sink.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32,
                                              i32, f32, vp, vp, vp, vp, u32, vp, sz, vp]
        L.dsa_indexer_kl_target.restype = C.c_int
        L.dsa_indexer_kl_target.argtypes = [vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, f32, vp,
                                             vp]
        L.dsa_sparse_mla_bwd_kl_target.restype = C.c_int
        L.dsa_sparse_mla_bwd_kl_target.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32,
                                                    i32, i32, f32, vp, vp, vp, u32, vp, sz, vp]
        L.dsa_indexer_kl_bwd_workspace_size.restype = sz
        L.dsa_indexer_kl_bwd_workspace_size.argtypes = [i64, i64, i32, i64]
        L.dsa_indexer_kl_bwd.restype = C.c_int
        L.dsa_indexer_kl_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, f32, vp,
                                         vp, vp, vp, u32, vp, sz, vp]
        L.dsa_sparse_mla_bwd_noalloc_scratch_bytes.argtypes = []
        L.dsa_sparse_mla_bwd_noalloc_scratch_bytes.restype = sz
        L.dsa_sparse_mla_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32,
                                                 i32, i32, f32, vp, vp, u32, vp]
        L.dsa_sparse_mla_bwd_noalloc.restype = C.c_int
        L.dsa_record_kernel_events.restype = C.c_int
        L.dsa_record_kernel_events.argtypes = [vp, C.c_int, C.POINTER(C.c_int)]
        L.dsa_gather_probe_groups.restype = i64
        L.dsa_gather_probe_groups.argtypes = [i64]
        L.dsa_gather_probe.restype = C.c_int
        L.dsa_gather_probe.argtypes = [vp, i64, i32, vp, i64, vp, vp]
        _lib = L
    return _lib


def _raise(code: int, what: str):
    msg = lib().dsa_last_error().decode(errors="replace")
    text = f"{what}: {msg}" if msg else what
    if code in (DSA_ERR_INVALID_VALUE, DSA_ERR_WORKSPACE):
        raise ValueError(text)
    raise RuntimeError(text)


def _call(fn, what, *args):
    rc = fn(*args)
    if rc != DSA_OK:
        _raise(rc, what)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _require(op: str, *tensors):
    for t in tensors:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{op}: expected torch.Tensor, got {type(t).__name__}")
        if not t.is_cuda:
            raise RuntimeError(f"{op}: tensors must live on a GPU device")
        if not t.is_contiguous():
            raise ValueError(f"{op}: tensors must be contiguous")
    dev = tensors[0].device
    if any(t is not None and t.device != dev for t in tensors):
        raise ValueError(f"{op}: all tensors must be on one device")
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    if not lib().dsa_device_supported(idx):
        raise RuntimeError(f"{op}: device {idx} is not an AMD gfx950 GPU")


def _dtype(op, name, t, dt):
    if t is not None and t.dtype != dt:
        raise TypeError(f"{op}: {name} must be {dt}, got {t.dtype}")


def is_available() -> bool:
    """True when libdsa.so loads and the current device is gfx950."""
    try:
        return torch.cuda.is_available() and bool(lib().dsa_device_supported(
            torch.cuda.current_device()))
    except (RuntimeError, OSError):
        return False


class ThdMetadata:
    """Packed-THD metadata (device arrays live in `workspace`; reusable across layers)."""

    def __init__(self, struct: _Metadata, workspace: torch.Tensor, cu_seqlens: torch.Tensor):
        self._s = struct
        self.workspace = workspace
        self.cu_seqlens = cu_seqlens

    def _view(self, ptr_name: str, n: int) -> torch.Tensor:
        off = getattr(self._s, ptr_name) - self.workspace.data_ptr()
        assert off % 4 == 0
        return self.workspace.view(torch.int32)[off // 4: off // 4 + n]

    @property
    def T(self):
        return self._s.T

    @property
    def total_key_tokens(self):
        return self._s.total_key_tokens

    @property
    def seq_start(self):
        return self._view("seq_start", self._s.T)

    @property
    def causal_len(self):
        return self._view("causal_len", self._s.T)

    @property
    def topk_length(self):
        return self._view("topk_length", self._s.T)

    @property
    def row_order(self):
        return self._view("row_order", self._s.T)

    @property
    def groups(self):
        return self._view("groups", self._s.n_groups)

    def __getattr__(self, name):
        if name in ("B", "K", "max_seqlen", "all_rows_nonempty", "total_pairs", "total_valid",
                    "n_groups"):
            return getattr(self._s, name)
        raise AttributeError(name)


def prepare_thd_metadata(cu_seqlens: torch.Tensor, K: int = MAX_INDEXER_TOPK,
                         T: int | None = None) -> ThdMetadata:
    """dsa_prepare_thd_metadata: cu_seqlens int32 [B+1] on the GPU (one host synchronisation).

    T (total tokens) is read from cu_seqlens when not given; the library checks it."""
    op = "prepare_thd_metadata"
    _require(op, cu_seqlens)
    _dtype(op, "cu_seqlens", cu_seqlens, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError(f"{op}: cu_seqlens must be 1-D with at least 2 entries")
    if T is None:
        T = int(cu_seqlens[-1].item())
    ws_bytes = lib().dsa_thd_metadata_workspace_size(T)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=cu_seqlens.device)
    md = _Metadata()
    _call(lib().dsa_prepare_thd_metadata, op, cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, T,
          int(K), ws.data_ptr(), ws_bytes, C.byref(md), _stream())
    return ThdMetadata(md, ws, cu_seqlens)


def prepare_local_metadata(cu_seqlens: torch.Tensor, total_key_tokens: int,
                           K: int = MAX_INDEXER_TOPK, cu_seqlens_padded=None, query_indices=None,
                           padding_mask=None) -> ThdMetadata:
    """dsa_prepare_local_metadata: local query rows (global padded-storage coordinates in
    `query_indices`, int32 [T_q]; padding rows flagged in `padding_mask`, bool [T_q]) against
    gathered global keys of `total_key_tokens` rows laid out by `cu_seqlens_padded`."""
    op = "prepare_local_metadata"
    _require(op, cu_seqlens, cu_seqlens_padded, query_indices, padding_mask)
    _dtype(op, "cu_seqlens", cu_seqlens, torch.int32)
    _dtype(op, "cu_seqlens_padded", cu_seqlens_padded, torch.int32)
    _dtype(op, "query_indices", query_indices, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError(f"{op}: cu_seqlens must be 1-D with at least 2 entries")
    B = cu_seqlens.numel() - 1
    if cu_seqlens_padded is not None and cu_seqlens_padded.shape != cu_seqlens.shape:
        raise ValueError(f"{op}: cu_seqlens_padded must match cu_seqlens")
    if query_indices is not None:
        T_q = query_indices.numel()
    else:
        T_q = int((cu_seqlens_padded if cu_seqlens_padded is not None else cu_seqlens)[-1].item())
    pm = None
    if padding_mask is not None:
        if padding_mask.dtype != torch.bool or padding_mask.shape != (T_q,):
            raise ValueError(f"{op}: padding_mask must be bool [T_q]")
        pm = padding_mask.to(torch.uint8)
    ws_bytes = lib().dsa_local_metadata_workspace_size(T_q)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=cu_seqlens.device)
    md = _Metadata()
    _call(lib().dsa_prepare_local_metadata, op, cu_seqlens.data_ptr(), _ptr(cu_seqlens_padded),
          _ptr(query_indices), _ptr(pm), B, T_q, int(total_key_tokens), int(K), ws.data_ptr(),
          ws_bytes, C.byref(md), _stream())
    return ThdMetadata(md, ws, cu_seqlens)


def indexer_topk(q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor,
                 meta: ThdMetadata, K: int = MAX_INDEXER_TOPK, idx=None, length=None):
    """dsa_indexer_topk -> (idx int32 [T,K] ascending with -1 suffix, len int32 [T])."""
    op = "indexer_topk"
    _require(op, q_idx, k_idx, w)
    _dtype(op, "q_idx", q_idx, torch.bfloat16)
    _dtype(op, "k_idx", k_idx, torch.bfloat16)
    _dtype(op, "w", w, torch.float32)
    if q_idx.dim() != 3 or k_idx.dim() != 2 or w.dim() != 2:
        raise ValueError(f"{op}: expected q_idx [T,H,D], k_idx [T,D], w [T,H]")
    T, H, D = q_idx.shape
    Tk = meta.total_key_tokens
    if k_idx.shape != (Tk, D) or w.shape != (T, H) or T != meta.T:
        raise ValueError(f"{op}: shapes {tuple(q_idx.shape)}, {tuple(k_idx.shape)}, "
                         f"{tuple(w.shape)} do not match T={meta.T} query rows and "
                         f"{Tk} key rows")
    if not isinstance(K, int) or isinstance(K, bool):
        raise TypeError(f"{op}: K must be an int")
    if idx is None:
        idx = torch.empty((T, K), dtype=torch.int32, device=q_idx.device)
    if length is None:
        length = torch.empty((T,), dtype=torch.int32, device=q_idx.device)
    _require(op, idx, length)
    if idx.shape != (T, K) or length.shape != (T,):
        raise ValueError(f"{op}: output shapes do not match")
    ws_bytes = lib().dsa_indexer_topk_workspace_size(T, H, D, K)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q_idx.device)
    _call(lib().dsa_indexer_topk, op, q_idx.data_ptr(), k_idx.data_ptr(), w.data_ptr(),
          C.byref(meta._s), H, D, K, idx.data_ptr(), length.data_ptr(), ws.data_ptr(), ws_bytes,
          _stream())
    return idx, length


def prepare_kpool_metadata(cu_seqlens: torch.Tensor, pool: int = 4,
                           K_pools: int = 512) -> ThdMetadata:
    """dsa_prepare_kpool_metadata: k-pool rows of a packed batch (pools of `pool` keys from each
    sequence start, one indexer key per complete pool); meta.total_key_tokens is the number
    of pool keys the indexer reads."""
    op = "prepare_kpool_metadata"
    _require(op, cu_seqlens)
    _dtype(op, "cu_seqlens", cu_seqlens, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError(f"{op}: cu_seqlens must be 1-D with at least 2 entries")
    B = cu_seqlens.numel() - 1
    T = int(cu_seqlens[-1].item())
    ws_bytes = lib().dsa_kpool_metadata_workspace_size(T)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=cu_seqlens.device)
    md = _Metadata()
    _call(lib().dsa_prepare_kpool_metadata, op, cu_seqlens.data_ptr(), B, T, int(pool),
          int(K_pools), ws.data_ptr(), ws_bytes, C.byref(md), _stream())
    return ThdMetadata(md, ws, cu_seqlens)


def kpool_indexer_topk(q_idx: torch.Tensor, k_pool: torch.Tensor, w: torch.Tensor,
                       meta: ThdMetadata, K_pools: int = 512, idx=None, length=None):
    """dsa_kpool_indexer_topk -> (idx int32 [T, K_pools*pool + pool - 1] ascending key
    positions with a -1 suffix, len int32 [T])."""
    op = "kpool_indexer_topk"
    _require(op, q_idx, k_pool, w)
    _dtype(op, "q_idx", q_idx, torch.bfloat16)
    _dtype(op, "k_pool", k_pool, torch.bfloat16)
    _dtype(op, "w", w, torch.float32)
    if q_idx.dim() != 3 or k_pool.dim() != 2 or w.dim() != 2:
        raise ValueError(f"{op}: expected q_idx [T,H,D], k_pool [T_pool,D], w [T,H]")
    T, H, D = q_idx.shape
    pool = meta._s.pool
    if pool < 1:
        raise ValueError(f"{op}: metadata is not from prepare_kpool_metadata")
    if k_pool.shape != (meta.total_key_tokens, D) or w.shape != (T, H) or T != meta.T:
        raise ValueError(f"{op}: shapes do not match the metadata (T={meta.T}, "
                         f"{meta.total_key_tokens} pools)")
    W = K_pools * pool + pool - 1
    if idx is None:
        idx = torch.empty((T, W), dtype=torch.int32, device=q_idx.device)
    if length is None:
        length = torch.empty((T,), dtype=torch.int32, device=q_idx.device)
    _require(op, idx, length)
    if idx.shape != (T, W) or length.shape != (T,):
        raise ValueError(f"{op}: output shapes do not match")
    ws_bytes = lib().dsa_kpool_indexer_topk_workspace_size(T, int(K_pools))
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q_idx.device)
    _call(lib().dsa_kpool_indexer_topk, op, q_idx.data_ptr(), k_pool.data_ptr(), w.data_ptr(),
          C.byref(meta._s), H, D, int(K_pools), idx.data_ptr(), length.data_ptr(),
          ws.data_ptr(), ws_bytes, _stream())
    return idx, length


def _attn_shapes(op, q, kv, idx, topk_length):
    _dtype(op, "q", q, torch.bfloat16)
    _dtype(op, "kv", kv, torch.bfloat16)
    _dtype(op, "topk_indices", idx, torch.int32)
    _dtype(op, "topk_length", topk_length, torch.int32)
    if q.dim() != 3:
        raise ValueError(f"{op}: q must be [T_q, H, D_qk]")
    Tq, H, Dqk = q.shape
    if kv.dim() == 3 and kv.shape[1] == 1:
        kv = kv.view(kv.shape[0], kv.shape[2])
    if kv.dim() != 2 or kv.shape[1] != Dqk:
        raise ValueError(f"{op}: kv must be [T_kv, {Dqk}] or [T_kv, 1, {Dqk}]")
    if idx.dim() == 3 and idx.shape[1] == 1:
        idx = idx.view(idx.shape[0], idx.shape[2])
    if idx.dim() != 2 or idx.shape[0] != Tq:
        raise ValueError(f"{op}: topk_indices must be [T_q, K] or [T_q, 1, K]")
    if topk_length is not None and topk_length.shape != (Tq,):
        raise ValueError(f"{op}: topk_length must be [T_q]")
    return kv, idx, Tq, H, Dqk, kv.shape[0], idx.shape[1]


def _sink_arg(op, sink, H):
    _require(op, sink)
    _dtype(op, "sink", sink, torch.float32)
    if sink.shape != (H,):
        raise ValueError(f"{op}: sink must be [H] = [{H}] fp32")
    return sink


def sparse_mla_fwd(q: torch.Tensor, kv: torch.Tensor, topk_indices: torch.Tensor,
                   softmax_scale: float, topk_length: torch.Tensor | None = None,
                   d_v: int = 512, out=None, lse=None, sink=None):
    """dsa_sparse_mla_fwd -> (out bf16 [T_q,H,512], lse fp32 [T_q,H]); with `sink` (fp32 [H],
    one zero-valued logit per head) dsa_sparse_mla_fwd_sink."""
    op = "sparse_mla_fwd"
    _require(op, q, kv, topk_indices, topk_length)
    kv, idx, Tq, H, Dqk, Tkv, K = _attn_shapes(op, q, kv, topk_indices, topk_length)
    if out is None:
        out = torch.empty((Tq, H, d_v), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((Tq, H), dtype=torch.float32, device=q.device)
    _require(op, out, lse)
    if sink is None:
        _call(lib().dsa_sparse_mla_fwd, op, q.data_ptr(), kv.data_ptr(), idx.data_ptr(),
              _ptr(topk_length), Tq, Tkv, H, Dqk, d_v, K, float(softmax_scale), out.data_ptr(),
              lse.data_ptr(), _stream())
    else:
        _sink_arg(op, sink, H)
        _call(lib().dsa_sparse_mla_fwd_sink, op, q.data_ptr(), kv.data_ptr(), idx.data_ptr(),
              _ptr(topk_length), Tq, Tkv, H, Dqk, d_v, K, float(softmax_scale), sink.data_ptr(),
              out.data_ptr(), lse.data_ptr(), _stream())
    return out, lse


# staged key-gradient contributions per backward pass when the caller brings no workspace
DEFAULT_BWD_STAGE_BYTES = 16 << 30


def bwd_workspace_bytes(T_q: int, T_kv: int, H: int, D_qk: int, K: int,
                        rows_per_pass: int | None = None) -> int:
    """Workspace bytes of dsa_sparse_mla_bwd for passes of `rows_per_pass` query rows
    (0: all rows in one pass; None: as many rows as DEFAULT_BWD_STAGE_BYTES of staging hold).
    Several passes use two staging buffers (a pass's reduction overlaps the next pass)."""
    if rows_per_pass is None:
        per_row = K * (2 * D_qk + 16)
        rows_per_pass = (T_q if T_q * per_row <= DEFAULT_BWD_STAGE_BYTES
                         else max(1, DEFAULT_BWD_STAGE_BYTES // (2 * per_row)))
    return lib().dsa_sparse_mla_bwd_workspace_size(T_q, T_kv, H, D_qk, K, rows_per_pass)


def sparse_mla_bwd(q, kv, topk_indices, out, lse, dout, softmax_scale: float,
                   topk_length=None, dkv=None, accumulate: bool = False, dq=None,
                   check_indices: bool = False, workspace=None, sink=None, dsink=None,
                   kl_target=None):
    """dsa_sparse_mla_bwd -> (dq bf16 [T_q,H,D_qk], dkv fp32 [T_kv,D_qk]).

    With accumulate=True the gradients of the latent rows are added into `dkv`
    (query-chunked execution); otherwise dkv is overwritten.  `workspace` (uint8 device
    tensor) sets how many query rows a pass stages (see bwd_workspace_bytes); by default one
    the workspace is sized to the call: one pass over every query row when its staging (about
    T_q * K * (2 * D_qk + 20) bytes) fits DEFAULT_BWD_STAGE_BYTES, else passes over two
    buffers that share that cap (allocated through torch's caching allocator, so repeated
    calls of one shape reuse the memory).  With `sink` (fp32 [H]; out / lse then come from
    the sink forward) this is dsa_sparse_mla_bwd_sink and returns (dq, dkv, dsink fp32 [H]);
    accumulate=True adds into `dsink` too.  With `kl_target` (fp32 [T_q, K]) this is
    dsa_sparse_mla_bwd_kl_target, which also writes the indexer KL loss's target."""
    op = "sparse_mla_bwd"
    _require(op, q, kv, topk_indices, out, lse, dout, topk_length, dkv)
    kv2, idx, Tq, H, Dqk, Tkv, K = _attn_shapes(op, q, kv, topk_indices, topk_length)
    _dtype(op, "out", out, torch.bfloat16)
    _dtype(op, "dout", dout, torch.bfloat16)
    _dtype(op, "lse", lse, torch.float32)
    _dtype(op, "dkv", dkv, torch.float32)
    d_v = out.shape[-1]
    if out.shape != (Tq, H, d_v) or dout.shape != out.shape or lse.shape != (Tq, H):
        raise ValueError(f"{op}: out/dout must be [T_q,H,D_v] and lse [T_q,H]")
    if dkv is None:
        if accumulate:
            raise ValueError(f"{op}: accumulate=True needs a dkv buffer")
        dkv = torch.empty((Tkv, Dqk), dtype=torch.float32, device=q.device)
    if dkv.numel() != Tkv * Dqk:
        raise ValueError(f"{op}: dkv must hold [T_kv, D_qk] fp32")
    if dq is None:
        dq = torch.empty_like(q)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_bytes(Tq, Tkv, H, Dqk, K), 1),
                                dtype=torch.uint8, device=q.device)
    flags = (DSA_BWD_ACCUMULATE_DKV if accumulate else 0) | (
        DSA_DEBUG_CHECK_INDICES if check_indices else 0)
    if kl_target is not None:
        if sink is not None:
            raise ValueError(f"{op}: kl_target with a sink is not supported in one call")
        _require(op, q, kl_target)
        _dtype(op, "kl_target", kl_target, torch.float32)
        if kl_target.shape != (Tq, K):
            raise ValueError(f"{op}: kl_target must be [T_q, K] fp32")
        _call(lib().dsa_sparse_mla_bwd_kl_target, op, q.data_ptr(), kv2.data_ptr(),
              idx.data_ptr(), _ptr(topk_length), out.data_ptr(), lse.data_ptr(),
              dout.data_ptr(), Tq, Tkv, H, Dqk, d_v, K, float(softmax_scale), dq.data_ptr(),
              dkv.data_ptr(), kl_target.data_ptr(), flags, workspace.data_ptr(),
              workspace.numel(), _stream())
        return dq, dkv
    if sink is None:
        _call(lib().dsa_sparse_mla_bwd, op, q.data_ptr(), kv2.data_ptr(), idx.data_ptr(),
              _ptr(topk_length), out.data_ptr(), lse.data_ptr(), dout.data_ptr(), Tq, Tkv, H, Dqk,
              d_v, K, float(softmax_scale), dq.data_ptr(), dkv.data_ptr(), flags,
              workspace.data_ptr(), workspace.numel(), _stream())
        return dq, dkv
    _sink_arg(op, sink, H)
    if dsink is None:
        if accumulate:
            raise ValueError(f"{op}: accumulate=True needs a dsink buffer")
        dsink = torch.empty((H,), dtype=torch.float32, device=q.device)
    _require(op, dsink)
    _dtype(op, "dsink", dsink, torch.float32)
    if dsink.shape != (H,):
        raise ValueError(f"{op}: dsink must be [H] fp32")
    _call(lib().dsa_sparse_mla_bwd_sink, op, q.data_ptr(), kv2.data_ptr(), idx.data_ptr(),
          _ptr(topk_length), out.data_ptr(), lse.data_ptr(), dout.data_ptr(), Tq, Tkv, H, Dqk,
          d_v, K, float(softmax_scale), sink.data_ptr(), dq.data_ptr(), dkv.data_ptr(),
          dsink.data_ptr(), flags, workspace.data_ptr(), workspace.numel(), _stream())
    return dq, dkv, dsink


def sparse_mla_bwd_noalloc(q, kv, topk_indices, out, lse, dout, softmax_scale: float, dq, dkv,
                           topk_length=None, accumulate: bool = False):
    """dsa_sparse_mla_bwd_noalloc: the backward without a workspace (the library's fixed
    per-GPU scratch), for callers that cannot allocate.  dq (bf16 [T_q,H,D_qk]) and dkv (fp32
    [T_kv,D_qk]) are caller-provided outputs; nothing is allocated.  Calls that overlap in time
    on one GPU share that scratch and race."""
    op = "sparse_mla_bwd_noalloc"
    _require(op, q, kv, topk_indices, out, lse, dout, topk_length, dkv, dq)
    kv2, idx, Tq, H, Dqk, Tkv, K = _attn_shapes(op, q, kv, topk_indices, topk_length)
    _dtype(op, "out", out, torch.bfloat16)
    _dtype(op, "dout", dout, torch.bfloat16)
    _dtype(op, "lse", lse, torch.float32)
    _dtype(op, "dkv", dkv, torch.float32)
    _dtype(op, "dq", dq, torch.bfloat16)
    d_v = out.shape[-1]
    if out.shape != (Tq, H, d_v) or dout.shape != out.shape or lse.shape != (Tq, H):
        raise ValueError(f"{op}: out/dout must be [T_q,H,D_v] and lse [T_q,H]")
    if dkv.numel() != Tkv * Dqk or dq.shape != q.shape:
        raise ValueError(f"{op}: dq must match q and dkv hold [T_kv, D_qk] fp32")
    flags = DSA_BWD_ACCUMULATE_DKV if accumulate else 0
    _call(lib().dsa_sparse_mla_bwd_noalloc, op, q.data_ptr(), kv2.data_ptr(), idx.data_ptr(),
          _ptr(topk_length), out.data_ptr(), lse.data_ptr(), dout.data_ptr(), Tq, Tkv, H, Dqk,
          d_v, K, float(softmax_scale), dq.data_ptr(), dkv.data_ptr(), flags, _stream())
    return dq, dkv


def indexer_kl_target(q, kv, topk_indices, lse, softmax_scale: float, topk_length=None,
                      target=None):
    """dsa_indexer_kl_target -> target fp32 [T_q, K]: the head-summed attention probabilities of
    every valid slot, renormalised per row (the KL loss's target; no gradient)."""
    op = "indexer_kl_target"
    _require(op, q, kv, topk_indices, lse, topk_length, target)
    kv2, idx, Tq, H, Dqk, Tkv, K = _attn_shapes(op, q, kv, topk_indices, topk_length)
    _dtype(op, "lse", lse, torch.float32)
    if lse.shape != (Tq, H):
        raise ValueError(f"{op}: lse must be [T_q, H]")
    if target is None:
        target = torch.empty((Tq, K), dtype=torch.float32, device=q.device)
    _dtype(op, "target", target, torch.float32)
    if target.shape != (Tq, K):
        raise ValueError(f"{op}: target must be [T_q, K] fp32")
    _call(lib().dsa_indexer_kl_target, op, q.data_ptr(), kv2.data_ptr(), idx.data_ptr(),
          _ptr(topk_length), lse.data_ptr(), Tq, Tkv, H, Dqk, K, float(softmax_scale),
          target.data_ptr(), _stream())
    return target


def indexer_kl_bwd_workspace_bytes(T_q: int, T_kv: int, K: int,
                                   rows_per_pass: int = 0) -> int:
    return lib().dsa_indexer_kl_bwd_workspace_size(T_q, T_kv, K, rows_per_pass)


def indexer_kl_bwd(q_idx, k_idx, w, topk_indices, target, grad: float = 1.0, topk_length=None,
                   dk_idx=None, accumulate: bool = False, workspace=None):
    """dsa_indexer_kl_bwd -> (loss fp32 [T_q], dq_idx bf16 [T_q,H_i,128], dw fp32 [T_q,H_i],
    dk_idx fp32 [T_kv,128]); `grad` is the gradient of the caller's loss with respect to
    sum_t loss[t] (for example the coefficient 0.001 divided by the number of rows)."""
    op = "indexer_kl_bwd"
    _require(op, q_idx, k_idx, w, topk_indices, target, topk_length, dk_idx)
    _dtype(op, "q_idx", q_idx, torch.bfloat16)
    _dtype(op, "k_idx", k_idx, torch.bfloat16)
    _dtype(op, "w", w, torch.float32)
    _dtype(op, "topk_indices", topk_indices, torch.int32)
    _dtype(op, "target", target, torch.float32)
    _dtype(op, "topk_length", topk_length, torch.int32)
    _dtype(op, "dk_idx", dk_idx, torch.float32)
    if q_idx.dim() != 3 or k_idx.dim() != 2:
        raise ValueError(f"{op}: q_idx must be [T_q,H_i,D_i] and k_idx [T_kv,D_i]")
    Tq, Hi, Di = q_idx.shape
    Tkv = k_idx.shape[0]
    idx = topk_indices.reshape(Tq, -1)
    K = idx.shape[1]
    if k_idx.shape[1] != Di or w.shape != (Tq, Hi) or target.shape != (Tq, K):
        raise ValueError(f"{op}: shapes of k_idx, w or target do not match q_idx / topk_indices")
    if dk_idx is None:
        if accumulate:
            raise ValueError(f"{op}: accumulate=True needs a dk_idx buffer")
        dk_idx = torch.empty((Tkv, Di), dtype=torch.float32, device=q_idx.device)
    loss = torch.empty((Tq,), dtype=torch.float32, device=q_idx.device)
    dq_idx = torch.empty_like(q_idx)
    dw = torch.empty_like(w)
    if workspace is None:
        workspace = torch.empty(max(indexer_kl_bwd_workspace_bytes(Tq, Tkv, K), 1),
                                dtype=torch.uint8, device=q_idx.device)
    _call(lib().dsa_indexer_kl_bwd, op, q_idx.data_ptr(), k_idx.data_ptr(), w.data_ptr(),
          idx.data_ptr(), _ptr(topk_length), target.data_ptr(), Tq, Tkv, Hi, Di, K,
          float(grad), loss.data_ptr(), dq_idx.data_ptr(), dw.data_ptr(), dk_idx.data_ptr(),
          DSA_BWD_ACCUMULATE_DKV if accumulate else 0, workspace.data_ptr(), workspace.numel(),
          _stream())
    return loss, dq_idx, dw, dk_idx


def gather_probe(table: torch.Tensor, rows: torch.Tensor, sink=None):
    """dsa_gather_probe: streams table[rows] (bf16 [T_kv, 512 or 576], rows int32 [n]) through
    LDS as the attention kernels gather latent rows, and returns one checksum word per work
    group of 2048 listed rows (int32 [dsa_gather_probe_groups(n)], the uint32 bits)."""
    op = "gather_probe"
    _require(op, table, rows, sink)
    _dtype(op, "table", table, torch.bfloat16)
    _dtype(op, "rows", rows, torch.int32)
    if table.dim() != 2 or rows.dim() != 1:
        raise ValueError(f"{op}: table must be [T_kv, width] and rows [n]")
    n = rows.shape[0]
    g = lib().dsa_gather_probe_groups(n)
    if sink is None:
        sink = torch.empty((max(g, 1),), dtype=torch.int32, device=table.device)
    _dtype(op, "sink", sink, torch.int32)
    if sink.numel() < g:
        raise ValueError(f"{op}: sink holds {sink.numel()} words, {g} needed")
    _call(lib().dsa_gather_probe, op, table.data_ptr(), table.shape[0], table.shape[1],
          rows.data_ptr(), n, sink.data_ptr(), _stream())
    return sink[:g]
