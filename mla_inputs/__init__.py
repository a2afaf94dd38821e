"""Seeded synthetic inputs for GLM-style sparse MLA prefill.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only *draws* inputs: it holds none of the method's arithmetic
(no indexer score, no selection, no attention). What it does besides drawing
random numbers is input preparation that the pages place before the method:

* rounding fp32 draws to bf16 (round-to-nearest-even, via torch's cast);
* storing the latent KV in FP8 E4M3 with one fp32 scale per token
  (GLM-5.3 serves its KV cache in FP8 -- mibrahim.dev B300 post, "System
  architecture"; spke.com PCP/DCP article, footnote 1), the scale being the
  row's absolute maximum over 448 (the largest finite E4M3 value);
* describing a ragged batch (cu_seqlens and per-query absolute positions),
  including one rank's share of the load-balanced 16-chunk context-parallel
  split (spke.com article, section "PCP: teile die Token, nicht die Koepfe")
  and prefix-resume suffixes behind 256-token cached chunks (mibrahim.dev
  post, "KV hand-off and caching").

Every tensor is drawn from its own ``torch.Generator`` seeded from
``(workload seed, tensor id)``, so a tensor does not depend on the device or
on which other tensors were drawn.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

D_LATENT = 512          # latent ("nope") part of a KV row, also the PV width
D_ROPE = 64             # rotary part of a KV row
D_QK = D_LATENT + D_ROPE
E4M3_MAX = 448.0

# tensor ids used to derive per-tensor seeds
T_Q, T_KV, T_QI, T_KI, T_W = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic prefill workload.

    kv_lens[b] is L_b, the number of latent-KV rows of sequence b; q_pos_ranges
    lists, per sequence, half-open ranges of absolute positions whose queries
    are computed (concatenated in order).
    """
    name: str
    kv_lens: tuple
    q_pos_ranges: tuple          # per sequence: tuple of (start, stop)
    n_heads: int
    idx_heads: int
    idx_dim: int
    topk: int
    kv_dtype: str                # "bf16" or "fp8"
    dense: bool = False          # indexer bypassed, attention over all earlier tokens
    seed: int = 0
    sm_scale: float = 1.0 / math.sqrt(192.0)

    @property
    def num_seqs(self) -> int:
        return len(self.kv_lens)

    def q_counts(self) -> List[int]:
        return [sum(b - a for a, b in r) for r in self.q_pos_ranges]

    @property
    def total_q(self) -> int:
        return sum(self.q_counts())

    @property
    def total_kv(self) -> int:
        return sum(self.kv_lens)

    @property
    def max_kv_len(self) -> int:
        return max(self.kv_lens) if self.kv_lens else 0

    def cu_seqlens_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.q_counts())]).astype(np.int32)

    def cu_seqlens_kv(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.kv_lens)]).astype(np.int32)

    def q_pos(self) -> np.ndarray:
        parts = [np.arange(a, b, dtype=np.int32) for r in self.q_pos_ranges for a, b in r]
        return np.concatenate(parts) if parts else np.zeros(0, np.int32)

    def q_seq(self) -> np.ndarray:
        """Sequence id of every query row."""
        return np.repeat(np.arange(self.num_seqs, dtype=np.int32), self.q_counts())

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def cp_share_ranges(seq_len: int, n_ranks: int, rank: int) -> tuple:
    """Query positions of one rank under the load-balanced 2N-chunk split.

    The prompt is cut into 2N equal chunks; rank r computes chunk r from the
    front and chunk 2N-1-r from the back, so every rank gets the same mix of
    cheap (early) and expensive (late) causal rows.
    """
    n_chunks = 2 * n_ranks
    assert seq_len % n_chunks == 0
    c = seq_len // n_chunks
    a, b = rank, n_chunks - 1 - rank
    return ((a * c, (a + 1) * c), (b * c, (b + 1) * c))


def _resume(cached: Sequence[int], new: Sequence[int]):
    kv = tuple(c + n for c, n in zip(cached, new))
    q = tuple(((c, c + n),) for c, n in zip(cached, new))
    return kv, q


_RAGGED_KV, _RAGGED_Q = _resume([8960, 32512, 65280, 196608], [512, 2048, 4096, 6144])

# The workloads: tiny (oracle on every row), dense 16k, sparse 32k, one
# rank's context-parallel share of a 131,072-token prompt, a ragged
# prefix-resume batch, and a 64-token resume behind a 32k prefix.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", (1024,), (((0, 1024),),), n_heads=8, idx_heads=4, idx_dim=64,
                     topk=256, kv_dtype="bf16", seed=0),
    "dense16k": Workload("dense16k", (16384,), (((0, 16384),),), n_heads=64, idx_heads=64,
                         idx_dim=128, topk=16384, kv_dtype="bf16", dense=True, seed=1),
    "sparse32k": Workload("sparse32k", (32768,), (((0, 32768),),), n_heads=64, idx_heads=64,
                          idx_dim=128, topk=2048, kv_dtype="fp8", seed=2),
    "cp131k": Workload("cp131k", (131072,), (cp_share_ranges(131072, 8, 0),), n_heads=64,
                       idx_heads=64, idx_dim=128, topk=2048, kv_dtype="fp8", seed=3),
    "ragged": Workload("ragged", _RAGGED_KV, _RAGGED_Q, n_heads=64, idx_heads=64, idx_dim=128,
                       topk=2048, kv_dtype="fp8", seed=4),
    # a short new chunk behind a long cached prefix: fewer queries than the
    # GPU has compute units (the split-KV case)
    "resume64": Workload("resume64", *_resume([32704], [64]), n_heads=64, idx_heads=64,
                         idx_dim=128, topk=2048, kv_dtype="fp8", seed=5),
}


def _gen(seed: int, tensor_id: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * (seed + 1) + 7919 * tensor_id)
    return g


def normal_bf16(shape, seed: int, tensor_id: int, device="cpu", chunk_rows: int = 4096):
    """N(0,1) drawn in fp32, rounded to bf16 (RNE). Drawn in row chunks to
    bound the fp32 temporary; the chunking is part of the stream definition."""
    g = _gen(seed, tensor_id, device)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(shape[0], -1)
    for r in range(0, shape[0], chunk_rows):
        n = min(chunk_rows, shape[0] - r)
        flat[r:r + n] = torch.randn((n, flat.shape[1]), generator=g, device=device,
                                    dtype=torch.float32).to(torch.bfloat16)
    return out


def uniform_f32(shape, seed: int, tensor_id: int, device="cpu"):
    g = _gen(seed, tensor_id, device)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32)


def quantize_e4m3_rows(x: torch.Tensor):
    """Per-row FP8 E4M3 (OCP e4m3fn) with an fp32 scale: sigma = amax/448
    (1 for an all-zero row), codes = RNE-saturating(x / sigma).
    Returns (codes uint8 [N, D], sigma fp32 [N])."""
    x = x.float()
    amax = x.abs().amax(dim=1)
    sigma = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / sigma[:, None]).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), sigma.contiguous()


def fp8_kv(n_rows: int, seed: int, device="cpu", chunk_rows: int = 8192):
    """Latent KV rows: N(0,1) in fp32, stored as E4M3 codes plus one scale per row."""
    g = _gen(seed, T_KV, device)
    codes = torch.empty((n_rows, D_QK), dtype=torch.uint8, device=device)
    sigma = torch.empty((n_rows,), dtype=torch.float32, device=device)
    for r in range(0, n_rows, chunk_rows):
        n = min(chunk_rows, n_rows - r)
        x = torch.randn((n, D_QK), generator=g, device=device, dtype=torch.float32)
        codes[r:r + n], sigma[r:r + n] = quantize_e4m3_rows(x)
    return codes, sigma


DS656_ROW = 656         # 512 E4M3 latent codes + 4 fp32 scales + 64 bf16 rope values


def pack_ds656_rows(x: torch.Tensor) -> torch.Tensor:
    """656-byte latent rows (a reading of FlashMLA's fp8_ds_mla row, which the
    spke.com PCP/DCP article's footnote 1 names at 656 bytes per token) from
    fp32 rows x [N, 576]: bytes 0..511 the E4M3 codes of the latent values,
    each 128-value tile quantised with its own scale amax/448 (1 for an
    all-zero tile, RNE, saturating); bytes 512..527 the four fp32 scales;
    bytes 528..655 the 64 rope values rounded to bf16. uint8 [N, 656]."""
    x = x.float()
    n = x.shape[0]
    lat = x[:, :D_LATENT].reshape(n, 4, 128)
    amax = lat.abs().amax(dim=2)
    sigma = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    codes = (lat / sigma[:, :, None]).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    rows = torch.empty((n, DS656_ROW), dtype=torch.uint8, device=x.device)
    rows[:, :D_LATENT] = codes.view(torch.uint8).reshape(n, D_LATENT)
    rows[:, D_LATENT:D_LATENT + 16] = sigma.contiguous().view(torch.uint8).reshape(n, 16)
    rows[:, D_LATENT + 16:] = x[:, D_LATENT:].to(torch.bfloat16).contiguous().view(torch.uint8)
    return rows


def ds656_kv(n_rows: int, seed: int, device="cpu", chunk_rows: int = 8192) -> torch.Tensor:
    """Latent KV rows: N(0,1) in fp32 (the same draw as fp8_kv and the bf16
    rows), stored as 656-byte rows (pack_ds656_rows)."""
    g = _gen(seed, T_KV, device)
    rows = torch.empty((n_rows, DS656_ROW), dtype=torch.uint8, device=device)
    for r in range(0, n_rows, chunk_rows):
        n = min(chunk_rows, n_rows - r)
        rows[r:r + n] = pack_ds656_rows(torch.randn((n, D_QK), generator=g, device=device,
                                                    dtype=torch.float32))
    return rows


def quantize_e4m3_chunked(x: torch.Tensor, chunk_rows: int = 1 << 16):
    """quantize_e4m3_rows over the rows of x viewed as [-1, x.shape[-1]], in
    chunks (bounds the fp32 temporary). Returns (codes like x as uint8,
    scales of shape x.shape[:-1])."""
    flat = x.reshape(-1, x.shape[-1])
    codes = torch.empty(flat.shape, dtype=torch.uint8, device=x.device)
    sigma = torch.empty((flat.shape[0],), dtype=torch.float32, device=x.device)
    for r in range(0, flat.shape[0], chunk_rows):
        codes[r:r + chunk_rows], sigma[r:r + chunk_rows] = quantize_e4m3_rows(flat[r:r + chunk_rows])
    return codes.view(x.shape), sigma.view(x.shape[:-1])


def make_inputs(wl: Workload, device="cpu", kv_dtype: Optional[str] = None,
                with_indexer: Optional[bool] = None, idx_dtype: str = "bf16") -> dict:
    """All tensors of one workload on ``device``.

    q   [total_q, H, 576] bf16    absorbed query (512 latent + 64 rope)
    kv  [total_kv, 576]   bf16, or uint8 E4M3 codes with kv_scale [total_kv] fp32,
                          or ("ds656") uint8 656-byte rows [total_kv, 656]
    q_idx [total_q, H_I, D_I] bf16, k_idx [total_kv, D_I] bf16, w [total_q, H_I] fp32
    (idx_dtype "fp8": q_idx and k_idx are the E4M3 codes of those same draws,
    one scale per (query, head) row in q_idx_scale [total_q, H_I] and per key
    in k_idx_scale [total_kv])
    plus the batch description (int32 cu_seqlens_q/kv, q_pos) on ``device``
    and on the host (numpy).
    """
    kv_dtype = kv_dtype or wl.kv_dtype
    if with_indexer is None:
        with_indexer = not wl.dense
    s = wl.seed
    out = {
        "workload": wl,
        "kv_dtype": kv_dtype,
        "cu_seqlens_q_host": wl.cu_seqlens_q(),
        "cu_seqlens_kv_host": wl.cu_seqlens_kv(),
        "q_pos_host": wl.q_pos(),
    }
    out["cu_seqlens_q"] = torch.from_numpy(out["cu_seqlens_q_host"]).to(device)
    out["cu_seqlens_kv"] = torch.from_numpy(out["cu_seqlens_kv_host"]).to(device)
    out["q_pos"] = torch.from_numpy(out["q_pos_host"]).to(device)
    out["q"] = normal_bf16((wl.total_q, wl.n_heads, D_QK), s, T_Q, device)
    if kv_dtype == "bf16":
        out["kv"] = normal_bf16((wl.total_kv, D_QK), s, T_KV, device)
        out["kv_scale"] = None
    elif kv_dtype == "fp8":
        out["kv"], out["kv_scale"] = fp8_kv(wl.total_kv, s, device)
    elif kv_dtype == "ds656":
        out["kv"] = ds656_kv(wl.total_kv, s, device)
        out["kv_scale"] = None
    else:
        raise ValueError(kv_dtype)
    if with_indexer:
        out["q_idx"] = normal_bf16((wl.total_q, wl.idx_heads, wl.idx_dim), s, T_QI, device)
        out["k_idx"] = normal_bf16((wl.total_kv, wl.idx_dim), s, T_KI, device)
        out["w"] = uniform_f32((wl.total_q, wl.idx_heads), s, T_W, device)
        if idx_dtype == "fp8":
            out["q_idx"], out["q_idx_scale"] = quantize_e4m3_chunked(out["q_idx"])
            out["k_idx"], out["k_idx_scale"] = quantize_e4m3_chunked(out["k_idx"])
        elif idx_dtype != "bf16":
            raise ValueError(idx_dtype)
    out["idx_dtype"] = idx_dtype
    return out


def sample_rows(wl: Workload, n: int = 512, seed: int = 12345, per_seq: int = 64) -> np.ndarray:
    """Query rows checked at full size. Forced: the first and last 4 queries
    of every contiguous run of positions (a context-parallel share has two
    runs, its two chunks) and the queries at p in {k-2, k-1, k, k+1} (the
    keep-all boundary). Then seeded uniform picks: at least min(per_seq, n_b)
    rows of every sequence b, and up to n rows in all. Sorted, unique."""
    q_pos = wl.q_pos()
    cu = wl.cu_seqlens_q()
    rng = np.random.default_rng(seed)
    picks = set()
    for b in range(wl.num_seqs):
        a, e = int(cu[b]), int(cu[b + 1])
        if e == a:
            continue
        seg = q_pos[a:e]
        breaks = (np.nonzero(np.diff(seg) != 1)[0] + 1).tolist()
        for s0, s1 in zip([0] + breaks, breaks + [e - a]):
            picks.update(range(a + s0, a + min(s0 + 4, s1)))
            picks.update(range(a + max(s0, s1 - 4), a + s1))
        for p in (wl.topk - 2, wl.topk - 1, wl.topk, wl.topk + 1):
            hit = np.nonzero(seg == p)[0]
            if hit.size:
                picks.add(a + int(hit[0]))
        want = min(per_seq, e - a)
        while sum(1 for r in picks if a <= r < e) < want:
            picks.add(int(rng.integers(a, e)))
    total = wl.total_q
    while len(picks) < min(n, total):
        picks.add(int(rng.integers(0, total)))
    return np.array(sorted(picks), dtype=np.int64)
