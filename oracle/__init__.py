"""fp64 CPU oracle for GLM-style sparse MLA prefill -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package. The HIP library never does, and the oracle uses
nothing from it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over query rows);
this file compiles it with gcc, loads it with ctypes and adds the ragged-batch
bookkeeping (slicing each query's own sequence out of the packed tensors) and
the explicit, non-absorbed MLA form used to check the absorbed one.

Parity status of each function (what pins it, besides itself) is stated in
the pin tests; every function here has at least one pin.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

FMT_BF16, FMT_E4M3, FMT_F64, FMT_DS656 = 0, 1, 2, 3
DS656_ROW = 656
QK_DIM, V_DIM = 576, 512


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, OpenMP)."""
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
                    "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            L = ctypes.CDLL(_LIB_PATH)
            P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
            L.oracle_num_threads.argtypes = []
            L.oracle_num_threads.restype = ctypes.c_int
            L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
            L.oracle_bf16_decode.restype = D
            L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
            L.oracle_e4m3_decode.restype = D
            L.oracle_indexer.argtypes = [I64, I64, I64, I64, P, P, P, P, P, I64]
            L.oracle_indexer.restype = None
            L.oracle_indexer_e4m3.argtypes = [I64, I64, I64, I64, P, P, P, P, P, P, P, I64]
            L.oracle_indexer_e4m3.restype = None
            L.oracle_topk.argtypes = [I64, P, I64, P, I32, P]
            L.oracle_topk.restype = None
            L.oracle_attention.argtypes = [I64, I64, I64, ctypes.c_int, P, ctypes.c_int, P, P,
                                           P, I32, P, D, P, P]
            L.oracle_attention.restype = None
            _lib = L
    return _lib


# ---------------------------------------------------------------- helpers --
def as_numpy(x) -> Optional[np.ndarray]:
    """torch tensor (any device) or numpy array -> contiguous host numpy array.
    bf16 tensors come back as their raw uint16 bit patterns."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16)
            if x.dtype == torch.float8_e4m3fn:
                return x.view(torch.uint8).numpy()
            return x.numpy()
    except ImportError:
        pass
    return np.ascontiguousarray(x)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops run on."""
    return int(lib().oracle_num_threads())


def bf16_decode(h: int) -> float:
    return lib().oracle_bf16_decode(int(h))


def e4m3_decode(c: int) -> float:
    return lib().oracle_e4m3_decode(int(c))


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Vector form of the bf16 decoder (bits to the top half of an fp32)."""
    a = np.asarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------- single sequence --
def indexer_seq(q_idx_bits: np.ndarray, k_idx_bits: np.ndarray, w: np.ndarray,
                q_pos: np.ndarray) -> np.ndarray:
    """Scores of n queries of one sequence: [n, L] fp32, NaN where j > q_pos[i].
    q_idx_bits [n, H_I, D_I] uint16 (bf16), k_idx_bits [L, D_I] uint16, w [n, H_I] fp32."""
    q_idx_bits = np.ascontiguousarray(q_idx_bits, dtype=np.uint16)
    k_idx_bits = np.ascontiguousarray(k_idx_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    n, h, d = q_idx_bits.shape
    L = k_idx_bits.shape[0]
    assert k_idx_bits.shape[1] == d and w.shape == (n, h)
    assert n == 0 or int(q_pos.max()) < L
    scores = np.full((n, L), np.nan, dtype=np.float32)
    if n:
        lib().oracle_indexer(n, h, d, L, _ptr(q_idx_bits), _ptr(k_idx_bits), _ptr(w),
                             _ptr(q_pos), _ptr(scores), L)
    return scores


def indexer_seq_fp8(q_codes: np.ndarray, q_scale: np.ndarray, k_codes: np.ndarray,
                    k_scale: np.ndarray, w: np.ndarray, q_pos: np.ndarray) -> np.ndarray:
    """Scores from FP8 indexer inputs: q_codes [n, H_I, D_I] and k_codes [L, D_I]
    uint8 E4M3, q_scale [n, H_I] and k_scale [L] fp32, w [n, H_I] fp32.
    [n, L] fp32, NaN where j > q_pos[i]."""
    q_codes = np.ascontiguousarray(q_codes, dtype=np.uint8)
    k_codes = np.ascontiguousarray(k_codes, dtype=np.uint8)
    q_scale = np.ascontiguousarray(q_scale, dtype=np.float32)
    k_scale = np.ascontiguousarray(k_scale, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    n, h, d = q_codes.shape
    L = k_codes.shape[0]
    assert k_codes.shape[1] == d and w.shape == (n, h) and q_scale.shape == (n, h)
    assert k_scale.shape == (L,)
    assert n == 0 or int(q_pos.max()) < L
    scores = np.full((n, L), np.nan, dtype=np.float32)
    if n:
        lib().oracle_indexer_e4m3(n, h, d, L, _ptr(q_codes), _ptr(q_scale), _ptr(k_codes),
                                  _ptr(k_scale), _ptr(w), _ptr(q_pos), _ptr(scores), L)
    return scores


def topk_seq(scores: np.ndarray, q_pos: np.ndarray, k: int) -> np.ndarray:
    """scores [n, ld] fp32 (row i valid for j <= q_pos[i]) -> [n, k] int32,
    ascending local indices padded with -1."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    n, ld = scores.shape
    assert n == 0 or int(q_pos.max()) < ld
    out = np.empty((n, k), dtype=np.int32)
    if n:
        lib().oracle_topk(n, _ptr(scores), ld, _ptr(q_pos), int(k), _ptr(out))
    return out


def attention_seq(q, kv, q_pos, sm_scale: float, kv_scale=None, indices=None,
                  q_fmt: int = FMT_BF16, kv_fmt: int = FMT_BF16):
    """Absorbed MLA attention of n queries of one sequence.
    q [n, H, 576] (uint16 bf16 bits, or float64 with q_fmt=FMT_F64);
    kv [L, 576] (uint16 bf16 bits, uint8 e4m3 codes + kv_scale [L], or float64),
    or [L, 656] uint8 656-byte rows (kv_fmt=FMT_DS656: 512 E4M3 latent codes,
    four fp32 scales of 128 values each, 64 bf16 rope values);
    indices [n, k] int32 or None (all earlier tokens).
    Returns (out [n, H, 512] float64, lse [n, H] float64)."""
    dt = {FMT_BF16: np.uint16, FMT_E4M3: np.uint8, FMT_F64: np.float64, FMT_DS656: np.uint8}
    q = np.ascontiguousarray(q, dtype=dt[q_fmt])
    kv = np.ascontiguousarray(kv, dtype=dt[kv_fmt])
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int32)
    n, H, dq = q.shape
    L = kv.shape[0]
    assert dq == QK_DIM and kv.shape[1] == (DS656_ROW if kv_fmt == FMT_DS656 else QK_DIM)
    if kv_fmt == FMT_E4M3:
        kv_scale = np.ascontiguousarray(kv_scale, dtype=np.float32)
        assert kv_scale.shape == (L,)
    else:
        kv_scale = None
    k = 0
    if indices is not None:
        indices = np.ascontiguousarray(indices, dtype=np.int32)
        assert indices.shape[0] == n
        k = indices.shape[1]
    out = np.zeros((n, H, V_DIM), dtype=np.float64)
    lse = np.zeros((n, H), dtype=np.float64)
    if n:
        lib().oracle_attention(n, H, L, q_fmt, _ptr(q), kv_fmt, _ptr(kv), _ptr(kv_scale),
                               _ptr(indices), k, _ptr(q_pos), float(sm_scale), _ptr(out),
                               _ptr(lse))
    return out, lse


def merge_lse(o_parts, lse_parts):
    """Attention over the union of disjoint key sets, from the results of each
    set (spke.com GLM-5.3 PCP/DCP article, section "DCP": partial attention
    results combine through their log-sum-exp). o_parts [n_parts, ..., 512],
    lse_parts [n_parts, ...] (natural log, -inf for an empty set). In float64:
    lse = ln sum_r exp(lse_r), out = sum_r exp(lse_r - lse) o_r; every part
    empty gives out = 0, lse = -inf. Returns (out, lse)."""
    o = np.asarray(o_parts, dtype=np.float64)
    l = np.asarray(lse_parts, dtype=np.float64)
    m = l.max(axis=0)
    any_set = np.isfinite(m)
    ref = np.where(any_set, m, 0.0)
    w = np.exp(l - ref)                                  # an empty part weighs 0
    tot = np.where(any_set, w.sum(axis=0), 1.0)
    lse = np.where(any_set, ref + np.log(tot), -np.inf)
    out = np.where(any_set[..., None], (w[..., None] * o).sum(axis=0) / tot[..., None], 0.0)
    return out, lse


# ------------------------------------------------------------ ragged batch --
def _seq_of_rows(cu_q: np.ndarray, rows: np.ndarray) -> np.ndarray:
    return np.searchsorted(cu_q, rows, side="right") - 1


def _take_rows(x, rows: np.ndarray) -> np.ndarray:
    """Rows of a (possibly device-resident) tensor, copied to host numpy."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return as_numpy(x[torch.as_tensor(rows, dtype=torch.long, device=x.device)])
    except ImportError:
        pass
    return np.asarray(x)[rows]


def indexer_rows(batch: dict, rows: Sequence[int]):
    """Oracle scores for selected global query rows of a packed batch (FP8
    indexer inputs when the batch holds "k_idx_scale" and "q_idx_scale").
    Returns a list of fp32 arrays, row r of length q_pos[r] + 1."""
    rows = np.asarray(rows, dtype=np.int64)
    cu_q, cu_kv = batch["cu_seqlens_q_host"], batch["cu_seqlens_kv_host"]
    q_pos = np.asarray(batch["q_pos_host"])
    fp8 = batch.get("k_idx_scale") is not None
    kI = as_numpy(batch["k_idx"])
    qI, w = _take_rows(batch["q_idx"], rows), _take_rows(batch["w"], rows)
    if fp8:
        qs, ks = _take_rows(batch["q_idx_scale"], rows), as_numpy(batch["k_idx_scale"])
    seq = _seq_of_rows(cu_q, rows)
    result = [None] * len(rows)
    for b in np.unique(seq):
        sel = np.nonzero(seq == b)[0]
        r = rows[sel]
        ka, kb = cu_kv[b], cu_kv[b + 1]
        if fp8:
            sc = indexer_seq_fp8(qI[sel], qs[sel], kI[ka:kb], ks[ka:kb], w[sel], q_pos[r])
        else:
            sc = indexer_seq(qI[sel], kI[ka:kb], w[sel], q_pos[r])
        for t, s in zip(sel, sc):
            result[t] = s[: q_pos[rows[t]] + 1].copy()
    return result


def topk_rows(score_rows, q_pos_rows: Sequence[int], k: int) -> np.ndarray:
    """Top-k of given score rows (row t has q_pos_rows[t] + 1 valid entries)."""
    q_pos_rows = np.asarray(q_pos_rows, dtype=np.int32)
    n = len(score_rows)
    width = int(q_pos_rows.max()) + 1 if n else 1
    S = np.full((n, width), np.nan, dtype=np.float32)
    for t, s in enumerate(score_rows):
        S[t, : len(s)] = s
    return topk_seq(S, q_pos_rows, k)


def attention_rows(batch: dict, rows: Sequence[int], indices=None, sm_scale=None):
    """Oracle attention for selected global query rows of a packed batch.
    indices: [len(rows), k] local indices for those rows, or None (dense)."""
    rows = np.asarray(rows, dtype=np.int64)
    cu_q, cu_kv = batch["cu_seqlens_q_host"], batch["cu_seqlens_kv_host"]
    q_pos = np.asarray(batch["q_pos_host"])
    if sm_scale is None:
        sm_scale = batch["workload"].sm_scale
    q = _take_rows(batch["q"], rows)
    kv = as_numpy(batch["kv"])
    fp8 = batch["kv_dtype"] == "fp8"
    ds656 = batch["kv_dtype"] == "ds656"
    scale = as_numpy(batch["kv_scale"]) if fp8 else None
    seq = _seq_of_rows(cu_q, rows)
    H = q.shape[1]
    out = np.zeros((len(rows), H, V_DIM))
    lse = np.zeros((len(rows), H))
    for b in np.unique(seq):
        sel = np.nonzero(seq == b)[0]
        r = rows[sel]
        lo, hi = cu_kv[b], cu_kv[b + 1]
        o, l = attention_seq(q[sel], kv[lo:hi], q_pos[r], sm_scale,
                             kv_scale=None if scale is None else scale[lo:hi],
                             indices=None if indices is None else np.asarray(indices)[sel],
                             kv_fmt=FMT_E4M3 if fp8 else FMT_DS656 if ds656 else FMT_BF16)
        out[sel], lse[sel] = o, l
    return out, lse


# ------------------------------------------------ explicit (non-absorbed) --
def explicit_mla(qn: np.ndarray, qr: np.ndarray, c: np.ndarray, r: np.ndarray,
                 W_UK: np.ndarray, W_UV: np.ndarray, q_pos: np.ndarray, sm_scale: float):
    """MLA with per-head K/V up-projection (the form the absorbed kernel avoids).

    Per token j: latent c_j (512) and shared rope key r_j (64). Per head h:
    k_j^h = [W_UK[h] c_j ; r_j] (128 + 64 dims), v_j^h = W_UV[h] c_j (128 dims).
    Query q^h = [qn^h ; qr^h]. O^h = softmax_j(sm_scale q^h . k_j^h) v^h over
    j <= q_pos. Returns the per-head value outputs [n, H, 128] and the LSE [n, H].
    (DeepSeek-style MLA: one latent vector per token shared by every head --
    mibrahim.dev post, "System architecture".)"""
    n, H, _ = qn.shape
    out = np.zeros((n, H, W_UV.shape[1]))
    lse = np.zeros((n, H))
    for i in range(n):
        p = int(q_pos[i])
        for h in range(H):
            kn = c[: p + 1] @ W_UK[h].T            # [p+1, 128]
            v = c[: p + 1] @ W_UV[h].T             # [p+1, 128]
            z = sm_scale * (kn @ qn[i, h] + r[: p + 1] @ qr[i, h])
            m = z.max()
            L = m + np.log(np.exp(z - m).sum())
            out[i, h] = np.exp(z - L) @ v
            lse[i, h] = L
    return out, lse
