"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call
(so the failure paths are exercised here with fake device pointers that are
never dereferenced)."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_mla_long_amd as sm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_sparse.h")
FAKE = 0x10000          # 16-byte aligned, never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sm.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return sm.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[a-z_ ]+\*?\s*(mla_[a-z_]+)\(", text, flags=re.M)))


def test_header_declares_the_path(lib):
    names = declared_functions()
    assert {"mla_indexer_score", "mla_topk_select", "mla_sparse_prefill"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_exports_match_the_header():
    if not os.path.exists(sm.LIB_PATH):
        pytest.skip("library not built")
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", sm.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (mla_[a-z_]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_version_and_status_strings(lib):
    assert lib.mla_abi_version() == 1
    for s in range(4):
        assert lib.mla_status_string(s)
    assert b"unknown" in lib.mla_status_string(99)


def make_batch(cu_q=(0, 4), cu_kv=(0, 10), max_kv=None, total_q=None, total_kv=None, num=None):
    cq = np.asarray(cu_q, np.int32)
    ck = np.asarray(cu_kv, np.int32)
    keep = (cq, ck)
    b = sm.MlaBatch(len(cq) - 1 if num is None else num,
                    int(cq[-1]) if total_q is None else total_q,
                    int(ck[-1]) if total_kv is None else total_kv,
                    int(np.diff(ck).max()) if max_kv is None else max_kv,
                    cq.ctypes.data, ck.ctypes.data, FAKE, FAKE, FAKE)
    return b, keep


def idx_call(lib, b, q=FAKE, k=FAKE, w=FAKE, H=64, D=128, s=FAKE, ld=None):
    ld = b.max_kv_len if ld is None else ld
    return lib.mla_indexer_score(ctypes.byref(b), q, k, w, H, D, s, ld, None)


def idx8_call(lib, b, q=FAKE, qs=FAKE, k=FAKE, ks=FAKE, w=FAKE, H=64, D=128, s=FAKE, ld=None):
    ld = b.max_kv_len if ld is None else ld
    return lib.mla_indexer_score_fp8(ctypes.byref(b), q, qs, k, ks, w, H, D, s, ld, None)


def topk_call(lib, b, s=FAKE, ld=None, k=8, out=FAKE):
    ld = b.max_kv_len if ld is None else ld
    return lib.mla_topk_select(ctypes.byref(b), s, ld, k, out, None)


def attn_call(lib, b, q=FAKE, kv=FAKE, sc=FAKE, dtype=1, stride=576, sstride=4, idx=FAKE, k=8,
              H=64, scale=0.07, out=FAKE, lse=FAKE):
    return lib.mla_sparse_prefill(ctypes.byref(b), q, kv, sc, dtype, stride, sstride, idx, k, H,
                                  scale, out, lse, None)


INVALID, UNSUPPORTED = sm.MLA_ERR_INVALID_ARG, sm.MLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(cu_q=(1, 4)), INVALID),                      # does not start at 0
    (dict(cu_q=(0, 5, 4), cu_kv=(0, 5, 10)), INVALID),  # decreasing
    (dict(total_q=3), INVALID),                        # totals mismatch
    (dict(total_kv=11), INVALID),
    (dict(max_kv=9), INVALID),                         # max_kv_len wrong
    (dict(cu_q=(0, 2, 4), cu_kv=(0, 10, 10)), INVALID),  # queries without KV
    (dict(num=0), INVALID),
])
def test_bad_batches_rejected_by_every_call(lib, kw, code):
    b, keep = make_batch(**kw)
    assert idx_call(lib, b) == code
    assert lib.mla_last_error()
    assert idx8_call(lib, b) == code
    assert topk_call(lib, b) == code
    assert attn_call(lib, b) == code


def test_null_batch(lib):
    assert lib.mla_indexer_score(None, FAKE, FAKE, FAKE, 64, 128, FAKE, 10, None) == INVALID
    assert b"NULL" in lib.mla_last_error()


def test_indexer_argument_checks(lib):
    b, keep = make_batch()
    assert idx_call(lib, b, H=0) == INVALID
    assert idx_call(lib, b, H=65) == UNSUPPORTED
    assert idx_call(lib, b, D=96) == UNSUPPORTED
    assert idx_call(lib, b, ld=9) == INVALID
    assert idx_call(lib, b, q=None) == INVALID
    assert idx_call(lib, b, q=FAKE + 8) == INVALID            # misaligned bf16 rows
    assert idx_call(lib, b, s=FAKE + 2) == INVALID


def test_indexer_fp8_argument_checks(lib):
    b, keep = make_batch()
    assert idx8_call(lib, b, H=0) == INVALID
    assert idx8_call(lib, b, H=65) == UNSUPPORTED
    assert idx8_call(lib, b, D=96) == UNSUPPORTED
    assert idx8_call(lib, b, ld=9) == INVALID
    assert idx8_call(lib, b, qs=None) == INVALID
    assert b"scale" in lib.mla_last_error()
    assert idx8_call(lib, b, ks=None) == INVALID
    assert idx8_call(lib, b, k=None) == INVALID
    assert idx8_call(lib, b, q=FAKE + 8) == INVALID           # misaligned code rows
    assert idx8_call(lib, b, ks=FAKE + 2) == INVALID          # misaligned scales
    assert idx8_call(lib, b, qs=FAKE + 1) == INVALID
    empty, keep2 = make_batch(cu_q=(0, 0), cu_kv=(0, 10))
    assert idx8_call(lib, empty, q=None, qs=None, k=None, ks=None, w=None, s=None) == sm.MLA_OK


def test_topk_argument_checks(lib):
    b, keep = make_batch()
    assert topk_call(lib, b, k=0) == INVALID
    assert topk_call(lib, b, k=4097) == UNSUPPORTED
    assert topk_call(lib, b, ld=5) == INVALID
    long_rows, keep2 = make_batch(cu_q=(0, 4), cu_kv=(0, 524289))
    assert topk_call(lib, long_rows) == UNSUPPORTED             # row bitmaps would overflow LDS
    assert topk_call(lib, b, out=None) == INVALID


def test_attention_argument_checks(lib):
    b, keep = make_batch()
    assert attn_call(lib, b, dtype=7) == INVALID
    assert attn_call(lib, b, stride=584) == INVALID           # not a multiple of 16
    assert attn_call(lib, b, stride=560) == INVALID           # shorter than an fp8 row
    assert attn_call(lib, b, dtype=0, stride=1136) == INVALID  # shorter than a bf16 row
    assert attn_call(lib, b, sstride=2) == INVALID
    assert attn_call(lib, b, sc=None) == INVALID              # fp8 needs scales
    assert attn_call(lib, b, scale=0.0) == INVALID
    assert attn_call(lib, b, scale=float("nan")) == INVALID
    assert attn_call(lib, b, k=0) == INVALID
    assert attn_call(lib, b, H=12) == UNSUPPORTED
    assert attn_call(lib, b, k=70000) == UNSUPPORTED
    assert attn_call(lib, b, q=FAKE + 4) == INVALID
    assert attn_call(lib, b, lse=None) == INVALID
    assert attn_call(lib, b, out=FAKE + 2) == INVALID        # 16-byte output stores
    big, keep2 = make_batch(cu_q=(0, 4), cu_kv=(0, 8_000_000))
    assert attn_call(lib, big) == UNSUPPORTED                  # 8M rows x 576 B >= 4 GiB
    assert attn_call(lib, big, stride=512 + 64) == UNSUPPORTED
    mid, keep3 = make_batch(cu_q=(0, 4), cu_kv=(0, 5_000_000))   # rows: 2.9 GB, fits
    assert attn_call(lib, mid, sstride=1024) == UNSUPPORTED       # scales: 5.1 GB >= 4 GiB


def split_call(lib, b, n_split=2, ws=FAKE * 16, ws_bytes=None, k=8, idx=FAKE, **kw):
    if ws_bytes is None:
        ws_bytes = lib.mla_sparse_prefill_split_workspace_size(b.total_q, kw.get("H", 64), n_split)
    return lib.mla_sparse_prefill_split(ctypes.byref(b), kw.get("q", FAKE), kw.get("kv", FAKE),
                                        kw.get("sc", FAKE), kw.get("dtype", 1), 576, 4, idx, k,
                                        kw.get("H", 64), 0.07, n_split, ws, ws_bytes,
                                        kw.get("out", FAKE), kw.get("lse", FAKE), None)


def test_split_attention_argument_checks(lib):
    """mla_sparse_prefill_split: the attention checks, plus the split count and
    the workspace, all on the host before any HIP call."""
    b, keep = make_batch()
    size = lib.mla_sparse_prefill_split_workspace_size
    # 4 queries x 64 heads x 2 parts: bf16 outputs (256-byte rounded), then fp32 LSEs
    assert size(4, 64, 2) == 2 * 4 * 64 * 1024 + 2 * 4 * 64 * 4
    assert size(3, 8, 3) == (3 * 3 * 8 * 1024 + 255) // 256 * 256 + 3 * 3 * 8 * 4
    assert size(4, 64, 1) == 0 and size(0, 64, 4) == 0
    assert split_call(lib, b, n_split=-1) == INVALID
    assert split_call(lib, b, n_split=17) == UNSUPPORTED
    assert split_call(lib, b, n_split=9, k=8) == INVALID       # a part without a list entry
    assert split_call(lib, b, ws=None) == INVALID
    assert split_call(lib, b, ws=FAKE * 16 + 16) == INVALID    # not 256-byte aligned
    assert split_call(lib, b, ws_bytes=size(4, 64, 2) - 1) == INVALID
    assert b"workspace" in lib.mla_last_error()
    assert split_call(lib, b, dtype=7) == INVALID              # the attention checks apply
    assert split_call(lib, b, H=12) == UNSUPPORTED
    assert split_call(lib, b, out=None) == INVALID
    bad, keep2 = make_batch(total_q=3)
    assert split_call(lib, bad) == INVALID
    empty, keep3 = make_batch(cu_q=(0, 0), cu_kv=(0, 10))
    assert split_call(lib, empty, ws=None, out=None, lse=None) == sm.MLA_OK


def test_split_noalloc_argument_checks(lib):
    """mla_sparse_prefill_split_noalloc: the split checks, and parts larger
    than the library's scratch array rejected, all before any HIP call."""
    def call(b, n_split=2, k=8, H=64, out=FAKE):
        return lib.mla_sparse_prefill_split_noalloc(ctypes.byref(b), FAKE, FAKE, FAKE, 1, 576, 4,
                                                    FAKE, k, H, 0.07, n_split, out, FAKE, None)
    b, keep = make_batch()
    assert call(b, n_split=-1) == INVALID
    assert call(b, n_split=17) == UNSUPPORTED
    assert call(b, n_split=9, k=8) == INVALID                 # a part without a list entry
    assert call(b, H=12) == UNSUPPORTED                        # the attention checks apply
    assert call(b, out=None) == INVALID
    # 257 queries x 64 heads in 2 parts need 33.8 MB: above the 16.06 MiB array
    big, keep2 = make_batch(cu_q=(0, 257), cu_kv=(0, 300))
    assert call(big, n_split=2) == UNSUPPORTED
    assert b"MLA_SPLIT_SCRATCH_BYTES" in lib.mla_last_error()
    # 256 virtual queries of 64 heads fit exactly
    assert lib.mla_sparse_prefill_split_workspace_size(64, 64, 4) == 16 * 1024 * 1024 + 64 * 1024
    empty, keep3 = make_batch(cu_q=(0, 0), cu_kv=(0, 10))
    assert call(empty, out=None) == sm.MLA_OK


def fused_call(lib, b, k=8, ws=FAKE * 16, ws_bytes=None, idx=FAKE, fp8=False, H=64, D=128):
    if ws_bytes is None:
        ws_bytes = lib.mla_topk_workspace_size(ctypes.byref(b), k)
    if fp8:
        return lib.mla_indexer_topk_fp8(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, FAKE, H, D, k, idx,
                                        ws, ws_bytes, None)
    return lib.mla_indexer_topk(ctypes.byref(b), FAKE, FAKE, FAKE, H, D, k, idx, ws, ws_bytes, None)


@pytest.mark.parametrize("fp8", [False, True])
def test_indexer_topk_argument_checks(lib, fp8):
    """mla_indexer_topk(_fp8) and mla_topk_workspace_size: k, the indices, the
    workspace and the indexer's own checks, all on the host before any HIP call."""
    b, keep = make_batch()
    size = lib.mla_topk_workspace_size
    # 4 queries, one key part (no device: one CU, so no key split): lists of
    # cand_capacity(8) = 320 (key, j) entries, then the 4 list lengths
    assert size(ctypes.byref(b), 8) == (4 * 320 * 8 + 255) // 256 * 256 + 4 * 4
    assert size(ctypes.byref(b), 2048) == 4 * 6400 * 8 + 4 * 4
    assert size(ctypes.byref(b), 0) == 0 and size(None, 8) == 0
    bad, keep2 = make_batch(total_q=3)
    assert size(ctypes.byref(bad), 8) == 0
    assert fused_call(lib, b, fp8=fp8, k=0) == INVALID
    assert fused_call(lib, b, fp8=fp8, k=-3, ws_bytes=1 << 20) == INVALID
    assert fused_call(lib, b, fp8=fp8, k=4097, ws_bytes=1 << 30) == UNSUPPORTED
    assert fused_call(lib, b, fp8=fp8, ws=None) == INVALID
    assert fused_call(lib, b, fp8=fp8, ws=FAKE * 16 + 16) == INVALID       # not 256-byte aligned
    assert fused_call(lib, b, fp8=fp8, ws_bytes=size(ctypes.byref(b), 8) - 1) == INVALID
    assert b"mla_topk_workspace_size" in lib.mla_last_error()
    assert fused_call(lib, b, fp8=fp8, idx=None) == INVALID
    assert fused_call(lib, b, fp8=fp8, idx=FAKE + 2) == INVALID            # misaligned indices
    assert fused_call(lib, b, fp8=fp8, H=65) == UNSUPPORTED                 # the indexer's checks
    assert fused_call(lib, b, fp8=fp8, D=96) == UNSUPPORTED
    assert fused_call(lib, bad, fp8=fp8, ws_bytes=1 << 20) == INVALID
    empty, keep3 = make_batch(cu_q=(0, 0), cu_kv=(0, 10))
    assert fused_call(lib, empty, fp8=fp8, ws=None, idx=None) == sm.MLA_OK


def test_kv_decode_ds656_argument_checks(lib):
    """mla_kv_decode_ds656 validates on the host before any HIP call."""
    call = lib.mla_kv_decode_ds656
    assert call(FAKE, 656, -1, FAKE, None) == INVALID
    assert call(FAKE, 640, 4, FAKE, None) == INVALID            # shorter than a row
    assert call(FAKE, 664, 4, FAKE, None) == INVALID            # not a multiple of 16
    assert call(None, 656, 4, FAKE, None) == INVALID
    assert call(FAKE, 656, 4, None, None) == INVALID
    assert call(FAKE + 8, 656, 4, FAKE, None) == INVALID        # misaligned
    assert call(FAKE, 656, 4, FAKE + 8, None) == INVALID
    assert call(None, 656, 0, None, None) == sm.MLA_OK          # nothing to do


def test_merge_argument_checks(lib):
    """mla_merge_attention validates on the host before any HIP call."""
    import ctypes
    def call(n=2, total_q=4, H=8, o=(FAKE, FAKE), l=(FAKE, FAKE), out=FAKE, lse=FAKE):
        optr = (ctypes.c_void_p * max(len(o), 1))(*o) if o is not None else None
        lptr = (ctypes.c_void_p * max(len(l), 1))(*l) if l is not None else None
        return lib.mla_merge_attention(optr, lptr, n, total_q, H, out, lse, None)
    assert call(n=0) == INVALID
    assert call(n=17, o=(FAKE,) * 17, l=(FAKE,) * 17) == UNSUPPORTED
    assert call(total_q=-1) == INVALID
    assert call(H=0) == INVALID
    assert call(o=None) == INVALID
    assert call(o=(FAKE, None)) == INVALID
    assert call(l=(FAKE + 2, FAKE)) == INVALID              # misaligned LSE part
    assert call(o=(FAKE + 8, FAKE)) == INVALID              # 16-byte part loads
    assert call(out=None) == INVALID
    assert call(out=FAKE + 4) == INVALID
    assert call(total_q=0, out=None, lse=None) == sm.MLA_OK  # nothing to merge, nothing enqueued


def test_empty_batch_enqueues_nothing(lib):
    """total_q == 0 returns OK without any HIP call (so it works with no GPU)."""
    b, keep = make_batch(cu_q=(0, 0), cu_kv=(0, 10))
    assert idx_call(lib, b, q=None, k=None, w=None, s=None) == sm.MLA_OK
    assert topk_call(lib, b, s=None, out=None) == sm.MLA_OK
    assert attn_call(lib, b, q=None, kv=None, sc=None, out=None, lse=None) == sm.MLA_OK
    assert lib.mla_last_error() == b""


def test_binding_refuses_wrong_dtypes_before_the_library():
    import torch
    b = sm.Batch.__new__(sm.Batch)
    b.device = torch.device("cpu")
    b.total_q, b.total_kv, b.max_kv_len = 4, 10, 10
    with pytest.raises(TypeError):
        sm.indexer_score(b, torch.zeros(4, 64, 128), torch.zeros(10, 128, dtype=torch.bfloat16),
                         torch.zeros(4, 64))
