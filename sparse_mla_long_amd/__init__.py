"""Python binding of the MI355X sparse-MLA prefill library (libmla_sparse.so).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in include/mla_sparse.h. torch tensors provide the
device memory and the current HIP stream; nothing here computes any part of
the method, and there is no CPU fallback -- if the library is missing, the
import of its symbols fails loudly.

Calls (same names as the C ABI, without the ``mla_`` prefix):
  indexer_score(batch, q_idx, k_idx, w, ...)   -> scores [total_q, ld] fp32
  indexer_score_fp8(batch, q_idx, q_scale, k_idx, k_scale, w, ...)
                                               -> scores from E4M3 codes with scales
  kv_decode_ds656(kv)                          -> bf16 rows from 656-byte latent rows
  topk_select(batch, scores, k, ...)           -> indices [total_q, k] int32
  indexer_topk(batch, q_idx, k_idx, w, k, ...) -> indices, without the score matrix
  indexer_topk_fp8(batch, q_idx, q_scale, k_idx, k_scale, w, k, ...)
  sparse_prefill(batch, q, kv, ...)            -> (out [total_q, H, 512] bf16, lse [total_q, H] fp32)
      (n_split=S: the split-KV call, mla_sparse_prefill_split; with
      noalloc=True, mla_sparse_prefill_split_noalloc)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla_sparse.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_HIP = 0, 1, 2, 3
MLA_KV_BF16, MLA_KV_FP8_E4M3 = 0, 1
QK_DIM, V_DIM = 576, 512


class MlaBatch(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_q", ctypes.c_int32),
                ("total_kv", ctypes.c_int32), ("max_kv_len", ctypes.c_int32),
                ("cu_seqlens_q_host", ctypes.c_void_p), ("cu_seqlens_kv_host", ctypes.c_void_p),
                ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_kv", ctypes.c_void_p),
                ("q_pos", ctypes.c_void_p)]


EXPORTS = ("mla_indexer_score", "mla_indexer_score_fp8", "mla_topk_select", "mla_sparse_prefill",
           "mla_sparse_prefill_split", "mla_sparse_prefill_split_workspace_size",
           "mla_sparse_prefill_split_noalloc", "mla_topk_workspace_size", "mla_indexer_topk",
           "mla_indexer_topk_fp8", "mla_kv_decode_ds656",
           "mla_merge_attention", "mla_status_string", "mla_last_error", "mla_abi_version")

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmla_sparse.so and declare its signatures. Raises if it is missing."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("HIP library %s is not built; run __graft_entry__.build()" % path)
    L = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    BP = ctypes.POINTER(MlaBatch)
    L.mla_indexer_score.argtypes = [BP, P, P, P, I32, I32, P, I64, P]
    L.mla_indexer_score_fp8.argtypes = [BP, P, P, P, P, P, I32, I32, P, I64, P]
    L.mla_topk_select.argtypes = [BP, P, I64, I32, P, P]
    L.mla_kv_decode_ds656.argtypes = [P, I64, I64, P, P]
    L.mla_topk_workspace_size.argtypes = [BP, I32]
    L.mla_topk_workspace_size.restype = ctypes.c_size_t
    L.mla_indexer_topk.argtypes = [BP, P, P, P, I32, I32, I32, P, P, ctypes.c_size_t, P]
    L.mla_indexer_topk_fp8.argtypes = [BP, P, P, P, P, P, I32, I32, I32, P, P, ctypes.c_size_t, P]
    L.mla_sparse_prefill.argtypes = [BP, P, P, P, ctypes.c_int, I64, I64, P, I32, I32,
                                     ctypes.c_float, P, P, P]
    L.mla_sparse_prefill_split.argtypes = [BP, P, P, P, ctypes.c_int, I64, I64, P, I32, I32,
                                           ctypes.c_float, I32, P, ctypes.c_size_t, P, P, P]
    L.mla_sparse_prefill_split_noalloc.argtypes = [BP, P, P, P, ctypes.c_int, I64, I64, P, I32,
                                                   I32, ctypes.c_float, I32, P, P, P]
    L.mla_sparse_prefill_split_workspace_size.argtypes = [I32, I32, I32]
    L.mla_sparse_prefill_split_workspace_size.restype = ctypes.c_size_t
    L.mla_merge_attention.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(ctypes.c_void_p),
                                      I32, I32, I32, P, P, P]
    for f in ("mla_indexer_score", "mla_indexer_score_fp8", "mla_topk_select", "mla_indexer_topk",
              "mla_indexer_topk_fp8", "mla_kv_decode_ds656", "mla_sparse_prefill",
              "mla_sparse_prefill_split", "mla_sparse_prefill_split_noalloc", "mla_merge_attention"):
        getattr(L, f).restype = ctypes.c_int
    L.mla_status_string.argtypes = [ctypes.c_int]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_last_error.argtypes = []
    L.mla_last_error.restype = ctypes.c_char_p
    L.mla_abi_version.argtypes = []
    L.mla_abi_version.restype = ctypes.c_int32
    if path == LIB_PATH:
        _lib = L
    return L


class MlaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__("%s (%s)" % (load_library().mla_status_string(status).decode(), detail))


def _check(status: int):
    if status != MLA_OK:
        raise MlaError(status, load_library().mla_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, dtype, device, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


class Batch:
    """Ragged batch: sequence b owns queries [cu_q[b], cu_q[b+1]) and KV rows
    [cu_kv[b], cu_kv[b+1]); q_pos[i] is query i's absolute position."""

    def __init__(self, cu_seqlens_q: Sequence[int], cu_seqlens_kv: Sequence[int],
                 q_pos, device="cuda"):
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.cu_q_host = np.ascontiguousarray(np.asarray(cu_seqlens_q), dtype=np.int32)
        self.cu_kv_host = np.ascontiguousarray(np.asarray(cu_seqlens_kv), dtype=np.int32)
        self.cu_q = torch.from_numpy(self.cu_q_host).to(self.device)
        self.cu_kv = torch.from_numpy(self.cu_kv_host).to(self.device)
        if isinstance(q_pos, torch.Tensor):
            self.q_pos = q_pos.to(device=self.device, dtype=torch.int32).contiguous()
        else:
            self.q_pos = torch.from_numpy(np.asarray(q_pos, dtype=np.int32)).to(self.device)
        lens = np.diff(self.cu_kv_host)
        self.num_seqs = len(self.cu_q_host) - 1
        self.total_q = int(self.cu_q_host[-1]) if self.num_seqs >= 0 else 0
        self.total_kv = int(self.cu_kv_host[-1]) if self.num_seqs >= 0 else 0
        self.max_kv_len = int(lens.max()) if len(lens) else 0
        self._c = MlaBatch(self.num_seqs, self.total_q, self.total_kv, self.max_kv_len,
                           self.cu_q_host.ctypes.data, self.cu_kv_host.ctypes.data,
                           self.cu_q.data_ptr(), self.cu_kv.data_ptr(), self.q_pos.data_ptr())

    @classmethod
    def from_inputs(cls, inp: dict, device=None):
        dev = device or inp["q"].device
        return cls(inp["cu_seqlens_q_host"], inp["cu_seqlens_kv_host"], inp["q_pos"], dev)

    @property
    def c(self):
        return ctypes.byref(self._c)


def indexer_score(batch: Batch, q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor,
                  scores: Optional[torch.Tensor] = None, ld: Optional[int] = None) -> torch.Tensor:
    """mla_indexer_score. Returns scores [total_q, ld] fp32 (entries j > q_pos[i]
    are left as they were)."""
    dev = batch.device
    n_heads, head_dim = q_idx.shape[1], q_idx.shape[2]
    _need(q_idx, "q_idx", torch.bfloat16, dev, (batch.total_q, n_heads, head_dim))
    _need(k_idx, "k_idx", torch.bfloat16, dev, (batch.total_kv, head_dim))
    _need(w, "w", torch.float32, dev, (batch.total_q, n_heads))
    if scores is None:
        ld = ld or max(batch.max_kv_len, 1)
        scores = torch.empty((batch.total_q, ld), dtype=torch.float32, device=dev)
    else:
        _need(scores, "scores", torch.float32, dev)
        ld = scores.shape[1]
    _check(load_library().mla_indexer_score(batch.c, _ptr(q_idx), _ptr(k_idx), _ptr(w), n_heads,
                                            head_dim, _ptr(scores), ld, _stream(q_idx)))
    return scores


def indexer_score_fp8(batch: Batch, q_idx: torch.Tensor, q_scale: torch.Tensor,
                      k_idx: torch.Tensor, k_scale: torch.Tensor, w: torch.Tensor,
                      scores: Optional[torch.Tensor] = None, ld: Optional[int] = None) -> torch.Tensor:
    """mla_indexer_score_fp8: q_idx [total_q, H, D] and k_idx [total_kv, D] are
    uint8 E4M3 codes, q_scale [total_q, H] and k_scale [total_kv] fp32 (>= 0).
    Returns scores [total_q, ld] fp32 (entries j > q_pos[i] are left as they were)."""
    dev = batch.device
    n_heads, head_dim = q_idx.shape[1], q_idx.shape[2]
    _need(q_idx, "q_idx", torch.uint8, dev, (batch.total_q, n_heads, head_dim))
    _need(q_scale, "q_scale", torch.float32, dev, (batch.total_q, n_heads))
    _need(k_idx, "k_idx", torch.uint8, dev, (batch.total_kv, head_dim))
    _need(k_scale, "k_scale", torch.float32, dev, (batch.total_kv,))
    _need(w, "w", torch.float32, dev, (batch.total_q, n_heads))
    if scores is None:
        ld = ld or max(batch.max_kv_len, 1)
        scores = torch.empty((batch.total_q, ld), dtype=torch.float32, device=dev)
    else:
        _need(scores, "scores", torch.float32, dev)
        ld = scores.shape[1]
    _check(load_library().mla_indexer_score_fp8(batch.c, _ptr(q_idx), _ptr(q_scale), _ptr(k_idx),
                                                _ptr(k_scale), _ptr(w), n_heads, head_dim,
                                                _ptr(scores), ld, _stream(q_idx)))
    return scores


def topk_select(batch: Batch, scores: torch.Tensor, k: int,
                indices: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mla_topk_select. Returns indices [total_q, k] int32 (ascending, -1 padded)."""
    dev = batch.device
    _need(scores, "scores", torch.float32, dev)
    if scores.dim() != 2 or scores.shape[0] != batch.total_q:
        raise ValueError("scores must be [total_q, ld]")
    if indices is None:
        indices = torch.empty((batch.total_q, k), dtype=torch.int32, device=dev)
    else:
        _need(indices, "indices", torch.int32, dev, (batch.total_q, k))
    _check(load_library().mla_topk_select(batch.c, _ptr(scores), scores.shape[1], int(k),
                                          _ptr(indices), _stream(scores)))
    return indices


DS656_ROW = 656


def kv_decode_ds656(kv: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mla_kv_decode_ds656: 656-byte latent rows (uint8 [n, 656], or a
    row-strided uint8 view of wider rows) -> bf16 [n, 576]."""
    if kv.dtype != torch.uint8 or kv.dim() != 2 or kv.shape[1] < DS656_ROW or kv.stride(1) != 1:
        raise ValueError("kv must be uint8 [n, >= 656] with contiguous rows")
    n = kv.shape[0]
    if out is None:
        out = torch.empty((n, QK_DIM), dtype=torch.bfloat16, device=kv.device)
    else:
        _need(out, "out", torch.bfloat16, kv.device, (n, QK_DIM))
    _check(load_library().mla_kv_decode_ds656(_ptr(kv), int(kv.stride(0)), int(n), _ptr(out),
                                              _stream(kv)))
    return out


def topk_workspace(batch: Batch, k: int) -> torch.Tensor:
    """A workspace for indexer_topk / indexer_topk_fp8 (mla_topk_workspace_size bytes)."""
    need = load_library().mla_topk_workspace_size(batch.c, int(k))
    return torch.empty((max(need, 1),), dtype=torch.uint8, device=batch.device)


def indexer_topk(batch: Batch, q_idx: torch.Tensor, k_idx: torch.Tensor, w: torch.Tensor, k: int,
                 indices: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mla_indexer_topk: the indexer and top-k in one pass, no score matrix.
    Returns indices [total_q, k] int32 (ascending, -1 padded)."""
    dev = batch.device
    n_heads, head_dim = q_idx.shape[1], q_idx.shape[2]
    _need(q_idx, "q_idx", torch.bfloat16, dev, (batch.total_q, n_heads, head_dim))
    _need(k_idx, "k_idx", torch.bfloat16, dev, (batch.total_kv, head_dim))
    _need(w, "w", torch.float32, dev, (batch.total_q, n_heads))
    indices = _indices_out(batch, k, indices)
    workspace = topk_workspace(batch, k) if workspace is None else workspace
    _need(workspace, "workspace", torch.uint8, dev)
    _check(load_library().mla_indexer_topk(batch.c, _ptr(q_idx), _ptr(k_idx), _ptr(w), n_heads,
                                           head_dim, int(k), _ptr(indices), _ptr(workspace),
                                           workspace.numel(), _stream(q_idx)))
    return indices


def indexer_topk_fp8(batch: Batch, q_idx: torch.Tensor, q_scale: torch.Tensor,
                     k_idx: torch.Tensor, k_scale: torch.Tensor, w: torch.Tensor, k: int,
                     indices: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mla_indexer_topk_fp8: indexer_score_fp8's scores and top-k in one pass."""
    dev = batch.device
    n_heads, head_dim = q_idx.shape[1], q_idx.shape[2]
    _need(q_idx, "q_idx", torch.uint8, dev, (batch.total_q, n_heads, head_dim))
    _need(q_scale, "q_scale", torch.float32, dev, (batch.total_q, n_heads))
    _need(k_idx, "k_idx", torch.uint8, dev, (batch.total_kv, head_dim))
    _need(k_scale, "k_scale", torch.float32, dev, (batch.total_kv,))
    _need(w, "w", torch.float32, dev, (batch.total_q, n_heads))
    indices = _indices_out(batch, k, indices)
    workspace = topk_workspace(batch, k) if workspace is None else workspace
    _need(workspace, "workspace", torch.uint8, dev)
    _check(load_library().mla_indexer_topk_fp8(batch.c, _ptr(q_idx), _ptr(q_scale), _ptr(k_idx),
                                               _ptr(k_scale), _ptr(w), n_heads, head_dim, int(k),
                                               _ptr(indices), _ptr(workspace), workspace.numel(),
                                               _stream(q_idx)))
    return indices


def _indices_out(batch: Batch, k: int, indices: Optional[torch.Tensor]) -> torch.Tensor:
    if indices is None:
        return torch.empty((batch.total_q, k), dtype=torch.int32, device=batch.device)
    _need(indices, "indices", torch.int32, batch.device, (batch.total_q, k))
    return indices


def sparse_prefill(batch: Batch, q: torch.Tensor, kv: torch.Tensor,
                   kv_scale: Optional[torch.Tensor] = None,
                   indices: Optional[torch.Tensor] = None, sm_scale: float = 192 ** -0.5,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   kv_row_stride: Optional[int] = None, kv_scale_stride: int = 4,
                   n_split: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                   noalloc: bool = False):
    """mla_sparse_prefill. kv is [total_kv, 576] bf16, or uint8 E4M3 codes with
    kv_scale [total_kv] fp32 (or a strided view given by the byte strides).
    indices [total_q, k] int32 or None for dense causal attention.
    n_split (1..16): mla_sparse_prefill_split, every query's keys in n_split
    parts merged by their LSE; workspace (uint8, device) is allocated here
    when not given. noalloc (with n_split): mla_sparse_prefill_split_noalloc,
    the parts in the library's own scratch array (no workspace).
    Returns (out [total_q, H, 512] bf16, lse [total_q, H] fp32)."""
    dev = batch.device
    H = q.shape[1]
    _need(q, "q", torch.bfloat16, dev, (batch.total_q, H, QK_DIM))
    if kv.dtype == torch.bfloat16:
        dtype = MLA_KV_BF16
    elif kv.dtype in (torch.uint8, torch.float8_e4m3fn):
        dtype = MLA_KV_FP8_E4M3
    else:
        raise TypeError("kv must be bf16 or uint8/float8_e4m3fn codes")
    if kv.device != dev:
        raise ValueError("kv must be on %s" % dev)
    if kv_row_stride is None:
        _need(kv, "kv", kv.dtype, dev, (batch.total_kv, QK_DIM))
        kv_row_stride = kv.stride(0) * kv.element_size()
    if dtype == MLA_KV_FP8_E4M3:
        if kv_scale is None or kv_scale.dtype != torch.float32 or kv_scale.device != dev:
            raise TypeError("FP8 kv needs kv_scale: fp32 on %s" % dev)
    k = 0
    if indices is not None:
        _need(indices, "indices", torch.int32, dev)
        if indices.dim() != 2 or indices.shape[0] != batch.total_q:
            raise ValueError("indices must be [total_q, k]")
        k = indices.shape[1]
    if out is None:
        out = torch.empty((batch.total_q, H, V_DIM), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, dev, (batch.total_q, H, V_DIM))
    if lse is None:
        lse = torch.empty((batch.total_q, H), dtype=torch.float32, device=dev)
    else:
        _need(lse, "lse", torch.float32, dev, (batch.total_q, H))
    scale = _ptr(kv_scale) if dtype == MLA_KV_FP8_E4M3 else None
    if n_split is None:
        _check(load_library().mla_sparse_prefill(
            batch.c, _ptr(q), _ptr(kv), scale, dtype, int(kv_row_stride), int(kv_scale_stride),
            _ptr(indices), int(k), H, float(sm_scale), _ptr(out), _ptr(lse), _stream(q)))
        return out, lse
    L = load_library()
    if noalloc:
        _check(L.mla_sparse_prefill_split_noalloc(
            batch.c, _ptr(q), _ptr(kv), scale, dtype, int(kv_row_stride), int(kv_scale_stride),
            _ptr(indices), int(k), H, float(sm_scale), int(n_split), _ptr(out), _ptr(lse),
            _stream(q)))
        return out, lse
    need = L.mla_sparse_prefill_split_workspace_size(batch.total_q, H, int(n_split))
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, dev)
    _check(L.mla_sparse_prefill_split(
        batch.c, _ptr(q), _ptr(kv), scale, dtype, int(kv_row_stride), int(kv_scale_stride),
        _ptr(indices), int(k), H, float(sm_scale), int(n_split), _ptr(workspace),
        workspace.numel(), _ptr(out), _ptr(lse), _stream(q)))
    return out, lse


def merge_attention(o_parts: Sequence[torch.Tensor], lse_parts: Sequence[torch.Tensor],
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """mla_merge_attention: attention over the union of disjoint key sets from
    the parts' results. o_parts: tensors [total_q, H, 512] bf16; lse_parts:
    [total_q, H] fp32 (all on one device). Returns (out, lse) like sparse_prefill."""
    n = len(o_parts)
    if n != len(lse_parts) or n < 1:
        raise ValueError("need as many lse parts as o parts (at least one)")
    o0 = o_parts[0]
    if o0.dim() != 3 or o0.shape[2] != V_DIM:
        raise ValueError("o parts must be [total_q, H, 512]")
    total_q, H = o0.shape[0], o0.shape[1]
    dev = o0.device
    for o, l in zip(o_parts, lse_parts):
        _need(o, "o part", torch.bfloat16, dev, (total_q, H, V_DIM))
        _need(l, "lse part", torch.float32, dev, (total_q, H))
    if out is None:
        out = torch.empty((total_q, H, V_DIM), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, dev, (total_q, H, V_DIM))
    if lse is None:
        lse = torch.empty((total_q, H), dtype=torch.float32, device=dev)
    else:
        _need(lse, "lse", torch.float32, dev, (total_q, H))
    optrs = (ctypes.c_void_p * n)(*[o.data_ptr() for o in o_parts])
    lptrs = (ctypes.c_void_p * n)(*[l.data_ptr() for l in lse_parts])
    _check(load_library().mla_merge_attention(optrs, lptrs, n, int(total_q), int(H), _ptr(out),
                                              _ptr(lse), _stream(o0)))
    return out, lse


def prefill(batch: Batch, inp: dict, topk: int, sm_scale: float, dense: bool = False,
            scores: Optional[torch.Tensor] = None, fused: bool = False):
    """The whole path for one layer: indexer -> top-k -> sparse attention
    (or dense causal attention when ``dense``; with ``fused``, indexer and
    top-k in one pass). Returns (out, lse, indices)."""
    if dense:
        out, lse = sparse_prefill(batch, inp["q"], inp["kv"], inp.get("kv_scale"), None,
                                  sm_scale)
        return out, lse, None
    if fused:
        if inp.get("k_idx_scale") is not None:
            idx = indexer_topk_fp8(batch, inp["q_idx"], inp["q_idx_scale"], inp["k_idx"],
                                   inp["k_idx_scale"], inp["w"], topk)
        else:
            idx = indexer_topk(batch, inp["q_idx"], inp["k_idx"], inp["w"], topk)
        out, lse = sparse_prefill(batch, inp["q"], inp["kv"], inp.get("kv_scale"), idx, sm_scale)
        return out, lse, idx
    if inp.get("k_idx_scale") is not None:
        sc = indexer_score_fp8(batch, inp["q_idx"], inp["q_idx_scale"], inp["k_idx"],
                               inp["k_idx_scale"], inp["w"], scores=scores)
    else:
        sc = indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"], scores=scores)
    idx = topk_select(batch, sc, topk)
    out, lse = sparse_prefill(batch, inp["q"], inp["kv"], inp.get("kv_scale"), idx, sm_scale)
    return out, lse, idx
