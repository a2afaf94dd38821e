#!/usr/bin/env python3
"""Placeholder; replaced by the full benchmark below once the HIP path exists."""
from __future__ import annotations

import numpy as np

D_QK, D_V = 576, 512


# ------------------------------------------------------------- accounting --
# Algorithmic work only: causal pairs and selected pairs, never padded tiles.
def attn_flop_per_pair(n_heads: int) -> int:
    """FLOP per (query, attended key): every head does QK over 576 dims and PV
    over 512 (spke.com article, footnote 1: 2,176 FLOP per row and head)."""
    return 2 * (D_QK + D_V) * n_heads


def indexer_flop_per_pair(idx_heads: int, idx_dim: int) -> int:
    """MFMA FLOP per (query, earlier key) of the indexer GEMM."""
    return 2 * idx_heads * idx_dim


def sparse_query_bytes(n_heads: int, topk: int, row_bytes: int = 660) -> int:
    """Bytes one sparse-MLA query moves: topk gathered rows (KV row + 4-byte
    index) plus, per head, its bf16 query (576) and output (512)."""
    return topk * row_bytes + n_heads * 2 * (D_QK + D_V)


def kv_bytes_per_token(mla_layers=78, mla_row=656, idx_layers=21, idx_key=132, mtp=788) -> int:
    return mla_layers * mla_row + idx_layers * idx_key + mtp


def pair_counts(wl) -> dict:
    """Causal (query, key) pairs and selected pairs of a workload."""
    p = wl.q_pos().astype(np.int64)
    causal = int((p + 1).sum())
    selected = causal if wl.dense else int(np.minimum(p + 1, wl.topk).sum())
    return {"causal": causal, "selected": selected}


def workload_flops(wl) -> dict:
    pc = pair_counts(wl)
    f_idx = 0 if wl.dense else pc["causal"] * indexer_flop_per_pair(wl.idx_heads, wl.idx_dim)
    f_attn = pc["selected"] * attn_flop_per_pair(wl.n_heads)
    return {"indexer": f_idx, "attention": f_attn, **pc}


if __name__ == "__main__":
    raise SystemExit("benchmark not built yet")
