"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Staged so errors do not compound (the comparison procedure of the method):
  * indexer scores vs the oracle's, |g - r| <= 1e-3 |r| + 1e-4 (fp32 sums of
    exact bf16 products); bit-exact on small-integer inputs; FP8 indexer
    inputs add 2^-14 of the sum of absolute terms (the E4M3 MFMA's summation);
  * top-k bit-exact: the oracle's selection run on the GPU's own score rows;
  * attention on the GPU's own index lists: out within |g - r| <= tol + tol |r|
    (tol = 2e-2 for bf16 KV, 6e-2 for FP8 KV), LSE within 1e-3 + 1e-4 |r|
    (fp32 arithmetic; a query missing one 32-key block of 2,048 fails it);
  * the set overlap when each side uses its own scores is reported, and at
    full size gated (mean and worst row).
The tiny workload is checked on every row; the full-size workloads run the
whole path in the launch configuration the benchmark times and are checked
on sampled rows.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import mla_inputs
import oracle
import tolerances as tl

pytestmark = pytest.mark.gpu

TOL = tl.OUT_TOL
LSE_ATOL, LSE_RTOL = tl.LSE_ATOL, tl.LSE_RTOL
assert_close = tl.assert_close


@pytest.fixture(scope="module")
def sm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_long_amd as sm
    sm.load_library()
    return sm


def say(*a):
    print(*a, flush=True)


def to_gpu(inp):
    out = dict(inp)
    for k, v in inp.items():
        if isinstance(v, torch.Tensor):
            out[k] = v.cuda()
    return out


# The E4M3 MFMA does not sum its 64 products like IEEE fp32: its error is a
# fraction of the magnitude of the terms, not of the result (measured up to
# 2^-16.4 of sum |terms| on these inputs; FP8 matrix units are known to keep
# a limited number of accumulation bits). FP8 indexer scores therefore get an
# absolute allowance of 2^-14 of M_ij = sum_h w_ih sum_d |q_ihd k_jd| (decoded
# and scaled), on top of the indexer tolerance; M_ij is the oracle's score of
# the sign-cleared codes, where every dot product is non-negative.
FP8_SUM_REL = 2.0 ** -14


def fp8_score_magnitude(inp, rows):
    mag_inp = dict(inp)
    mag_inp["q_idx"] = inp["q_idx"] & 0x7f
    mag_inp["k_idx"] = inp["k_idx"] & 0x7f
    return oracle.indexer_rows(mag_inp, rows)


def run_path(sm, batch, inp):
    """indexer (bf16 or FP8 inputs) -> top-k -> sparse attention on the GPU
    (656-byte rows: decoded to bf16 rows first, then attended)."""
    wl = inp["workload"]
    if inp.get("k_idx_scale") is not None:
        scores = sm.indexer_score_fp8(batch, inp["q_idx"], inp["q_idx_scale"], inp["k_idx"],
                                      inp["k_idx_scale"], inp["w"])
    else:
        scores = sm.indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"])
    idx = sm.topk_select(batch, scores, wl.topk)
    kv = sm.kv_decode_ds656(inp["kv"]) if inp["kv_dtype"] == "ds656" else inp["kv"]
    out, lse = sm.sparse_prefill(batch, inp["q"], kv, inp["kv_scale"], idx, wl.sm_scale)
    return out, lse, idx, scores


# End-to-end selection overlap |S_oracle & S_gpu| / |S_oracle| when each side
# picks from its own scores (mean over rows, worst row). Near-ties between the
# fp64 scores and the GPU's fp32 (bf16 inputs) or E4M3-MFMA (FP8 inputs) sums
# can swap members at the k-th place, so this is a gate on the rate of such
# swaps, not a bit-exact check (top-k itself is bit-exact on equal scores).
OVERLAP_GATE = {"bf16": (0.999, 0.98), "fp8": (0.999, 0.99)}


def check_path(sm, inp, rows, label, check_indexer=True, gate_overlap=False):
    """Run indexer -> top-k -> attention on the GPU for the whole batch and
    check the given rows against the oracle, stage by stage."""
    wl = inp["workload"]
    batch = sm.Batch.from_inputs(inp)
    say("[%s] GPU path: %d queries, %d KV rows, H=%d, k=%d, kv=%s, indexer=%s" %
        (label, wl.total_q, wl.total_kv, wl.n_heads, wl.topk, inp["kv_dtype"],
         inp.get("idx_dtype", "bf16")))
    out, lse, idx, scores = run_path(sm, batch, inp)
    torch.cuda.synchronize()
    q_pos = inp["q_pos_host"]
    rows = np.asarray(rows)
    rt = torch.as_tensor(rows, device="cuda")
    g_scores = [scores[int(r), : q_pos[r] + 1].cpu().numpy() for r in rows]
    g_idx = idx[rt].cpu().numpy()
    if check_indexer:
        say("[%s] oracle indexer on %d rows" % (label, len(rows)))
        r_scores = oracle.indexer_rows(inp, rows)
        fp8 = inp.get("k_idx_scale") is not None
        if fp8:
            mag = fp8_score_magnitude(inp, rows)
        for t, r in enumerate(rows):
            atol = 1e-4 + FP8_SUM_REL * mag[t] if fp8 else 1e-4
            assert_close("%s indexer row %d" % (label, r), g_scores[t], r_scores[t], atol, 1e-3)
    say("[%s] oracle top-k on the GPU's scores" % label)
    r_idx = oracle.topk_rows(g_scores, q_pos[rows], wl.topk)
    mism = np.nonzero((r_idx != g_idx).any(axis=1))[0]
    assert len(mism) == 0, "%s top-k differs on rows %s" % (label, rows[mism][:8])
    say("[%s] oracle attention on the GPU's index lists" % label)
    r_out, r_lse = oracle.attention_rows(inp, rows, g_idx)
    tl.assert_attention(label, inp["kv_dtype"], out[rt].float().cpu().numpy(),
                        lse[rt].cpu().numpy(), r_out, r_lse, say)
    if check_indexer:
        own = oracle.topk_rows(r_scores, q_pos[rows], wl.topk)
        ov = tl.set_overlap(own, g_idx)
        say("[%s] end-to-end top-k set overlap (own scores each side): mean %.5f, worst row "
            "%.4f, over %d rows" % (label, ov.mean(), ov.min(), len(rows)))
        if gate_overlap:
            mean_min, row_min = OVERLAP_GATE[inp.get("idx_dtype", "bf16")]
            assert ov.mean() >= mean_min and ov.min() >= row_min, (label, ov.mean(), ov.min())
    return scores, idx, out, lse


# ------------------------------------------------------------------ tiny --
@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_tiny_all_rows(sm, kv_dtype):
    wl = mla_inputs.WORKLOADS["tiny"]
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu", kv_dtype=kv_dtype))
    scores, idx, out, lse = check_path(sm, inp, np.arange(wl.total_q), "tiny-" + kv_dtype)
    # end-to-end overlap with the oracle's own selection (reported)
    rows = np.arange(0, wl.total_q, 37)
    ref_idx = oracle.topk_rows(oracle.indexer_rows(inp, rows), inp["q_pos_host"][rows], wl.topk)
    g = idx[torch.as_tensor(rows, device="cuda")].cpu().numpy()
    ov = np.mean([len(set(a) & set(b)) / len(set(a)) for a, b in zip(ref_idx, g)])
    say("tiny end-to-end top-k set overlap (own scores each side): %.4f" % ov)
    assert ov > 0.99


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("n_heads", [8, 16, 32, 64])
def test_dense_attention_small(sm, n_heads, kv_dtype):
    wl = mla_inputs.Workload("dense-small", (300, 77), (((0, 300),), ((0, 77),)), n_heads=n_heads,
                             idx_heads=4, idx_dim=64, topk=512, kv_dtype=kv_dtype, dense=True, seed=21)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu"))
    batch = sm.Batch.from_inputs(inp)
    out, lse = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], None, wl.sm_scale)
    torch.cuda.synchronize()
    rows = np.arange(wl.total_q)
    r_out, r_lse = oracle.attention_rows(inp, rows, None)
    tl.assert_attention("dense-H%d-%s" % (n_heads, kv_dtype), kv_dtype, out.float().cpu().numpy(),
                        lse.cpu().numpy(), r_out, r_lse, say)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("n_heads", [8, 16, 32])
def test_sparse_path_head_counts(sm, n_heads, kv_dtype):
    """The whole path at the head counts below 64 the attention supports,
    every row: a ragged batch with an empty sequence, a CP-style gap, a
    one-token sequence and rows shorter than k (heads past n_heads in a
    32-head group are masked off in the kernels)."""
    wl = mla_inputs.Workload("heads", (300, 0, 1000, 1, 130),
                             (((0, 300),), (), ((0, 70), (930, 1000)), ((0, 1),), ((64, 130),)),
                             n_heads=n_heads, idx_heads=16, idx_dim=64, topk=96,
                             kv_dtype=kv_dtype, seed=90 + n_heads)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu"))
    check_path(sm, inp, np.arange(wl.total_q), "heads-H%d-%s" % (n_heads, kv_dtype))


def test_dense_equals_sparse_with_full_lists(sm):
    """With every earlier token listed, the sparse path equals the dense one."""
    wl = mla_inputs.Workload("full", (200,), (((0, 200),),), n_heads=64, idx_heads=4, idx_dim=64,
                             topk=256, kv_dtype="fp8", seed=22)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu"))
    batch = sm.Batch.from_inputs(inp)
    full = torch.arange(256, device="cuda", dtype=torch.int32)[None].repeat(200, 1)
    full = torch.where(full <= inp["q_pos"][:, None], full, torch.full_like(full, -1))
    o1, l1 = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], full, wl.sm_scale)
    o2, l2 = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], None, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("kv_dtype,listed", [("bf16", False), ("bf16", True), ("fp8", False),
                                             ("fp8", True)])
def test_wide_logit_range(sm, kv_dtype, listed):
    """Logits spread over hundreds of units (q scaled by 40): block maxima
    climb far above the first block's, across several chunks of the entry
    table, with the keys listed in a shuffled order."""
    L, L2 = 6000, 3000
    wl = mla_inputs.Workload("wide", (L,), (((L - 12, L),),), n_heads=64, idx_heads=4,
                             idx_dim=64, topk=L, kv_dtype=kv_dtype, dense=not listed, seed=25)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu"))
    inp["q"] = (inp["q"].float() * 40).to(torch.bfloat16)
    batch = sm.Batch.from_inputs(inp)
    idx = None
    if listed:
        g = torch.Generator().manual_seed(5)
        idx = torch.stack([torch.randperm(L, generator=g) for _ in range(wl.total_q)]).int().cuda()
        idx = torch.where(idx <= inp["q_pos"][:, None], idx, torch.full_like(idx, -1))
    out, lse = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale)
    torch.cuda.synchronize()
    rows = np.arange(wl.total_q)
    r_out, r_lse = oracle.attention_rows(inp, rows, None if idx is None else idx.cpu().numpy())
    tol = TOL[kv_dtype]
    assert_close("wide out", out.float().cpu().numpy(), r_out, tol, tol)
    assert_close("wide lse", lse.cpu().numpy(), r_lse, LSE_ATOL, LSE_RTOL)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("lead", [70, 2100])
def test_masked_leading_entries(sm, kv_dtype, lead):
    """Index lists whose first `lead` entries are all masked (-1, or keys past
    the query's position): the query's first step (70: more than one 64-key
    FP8 step) or its whole first 2,048-entry chunk (2,100) holds no valid key,
    so the kernels start the query with no reference max and must redo it
    once valid keys appear. One row is masked throughout (O = 0, LSE = -inf).
    Every row against the oracle on the same lists."""
    inp = _few_queries(kv_dtype, 70 + lead)
    wl = inp["workload"]
    batch = sm.Batch.from_inputs(inp)
    q_pos = inp["q_pos_host"]
    g = np.random.default_rng(71 + lead)
    n_valid = 300
    lists = np.full((wl.total_q, lead + n_valid), -1, np.int32)
    for i, p in enumerate(q_pos):
        past = p + 1 + g.integers(0, 50, lead)          # keys after the query's position
        lists[i, :lead] = np.where(g.random(lead) < 0.5, -1, past)
        m = min(p + 1, n_valid)
        lists[i, lead:lead + m] = g.permutation(p + 1)[:m]
    lists[wl.total_q // 2] = -1
    idx = torch.from_numpy(lists).cuda()
    out, lse = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale)
    torch.cuda.synchronize()
    rows = np.arange(wl.total_q)
    r_out, r_lse = oracle.attention_rows(inp, rows, lists)
    assert np.isneginf(r_lse[wl.total_q // 2]).all()
    tol = TOL[kv_dtype]
    assert_close("masked-lead out", out.float().cpu().numpy(), r_out, tol, tol)
    assert_close("masked-lead lse", lse.cpu().numpy(), r_lse, LSE_ATOL, LSE_RTOL)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("n_split", [1, 3])
def test_masked_trailing_entries(sm, kv_dtype, n_split):
    """Index lists of 4,200 entries whose valid keys stop early, the rest
    masked (-1, or keys past the query's position): the valid prefix ends on
    a 32- or 64-key step boundary, one entry after it, or in the first
    2,048-entry chunk (later chunks and split parts then hold no valid key);
    one row keeps a lone valid entry at 4,000 after a masked gap. Every row
    against the oracle, and bit-identical to the same lists cut to 2,600
    entries (trailing masked entries contribute nothing)."""
    inp = _few_queries(kv_dtype, 90 + n_split)
    wl = inp["workload"]
    batch = sm.Batch.from_inputs(inp)
    q_pos = inp["q_pos_host"]
    g = np.random.default_rng(91 + n_split)
    n_list = 4200
    ends = [64, 65, 128, 2048, 2049, 31, 1, 0, 2600]
    lists = np.full((wl.total_q, n_list), -1, np.int32)
    for i, p in enumerate(q_pos):
        m = min(ends[i % len(ends)], p + 1)
        lists[i, :m] = g.permutation(p + 1)[:m]
        tail = np.arange(m, n_list)
        past = g.random(len(tail)) < 0.3                 # keys after the position
        lists[i, tail[past]] = p + 1 + g.integers(0, 40, int(past.sum()))
    lone = wl.total_q - 1
    lists[lone] = -1
    lists[lone, 4000] = q_pos[lone] // 2
    kw = {} if n_split == 1 else {"n_split": n_split}
    idx = torch.from_numpy(lists).cuda()
    out, lse = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale, **kw)
    torch.cuda.synchronize()
    rows = np.arange(wl.total_q)
    r_out, r_lse = oracle.attention_rows(inp, rows, lists)
    tl.assert_attention("masked-tail split%d" % n_split, kv_dtype, out.float().cpu().numpy(),
                        lse.cpu().numpy(), r_out, r_lse, say)
    if n_split == 1:
        cut = idx[:, :2600].contiguous()
        keep = np.ones(wl.total_q, bool)
        keep[lone] = False
        o2, l2 = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], cut, wl.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(o2[torch.from_numpy(keep).cuda()], out[torch.from_numpy(keep).cuda()])
        assert torch.equal(l2[torch.from_numpy(keep).cuda()], lse[torch.from_numpy(keep).cuda()])


def _random_batch(seed):
    """A seeded random ragged batch: 1-4 sequences of 1..3,000 KV rows, each
    with one or two runs of query positions (a CP-style gap when two)."""
    g = np.random.default_rng(seed)
    n_seq = int(g.integers(1, 5))
    kv_lens, ranges = [], []
    for _ in range(n_seq):
        L = int(g.integers(1, 3001))
        kv_lens.append(L)
        a = int(g.integers(0, L))
        b = int(min(L, a + g.integers(1, 40)))
        r = [(a, b)]
        if L - b > 2 and g.random() < 0.5:           # a second run after a gap
            c = int(g.integers(b + 1, L))
            r.append((c, int(min(L, c + g.integers(1, 20)))))
        ranges.append(tuple(r))
    return tuple(kv_lens), tuple(ranges), g


@pytest.mark.parametrize("seed", range(16))
def test_attention_random_batches(sm, seed):
    """Seeded random ragged batches, head counts, k, KV types, list shapes
    (the GPU's own top-k lists, or shuffled lists with masked entries mixed
    in) and split counts: every row of every case against the oracle."""
    kv_lens, ranges, g = _random_batch(1000 + seed)
    n_heads = int(g.choice([8, 16, 32, 64]))
    kv_dtype = ["bf16", "fp8"][seed % 2]
    k = int(g.choice([1, 17, 256, 2048]))
    wl = mla_inputs.Workload("rand%d" % seed, kv_lens, ranges, n_heads=n_heads, idx_heads=4,
                             idx_dim=64, topk=k, kv_dtype=kv_dtype, seed=2000 + seed)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu"))
    batch = sm.Batch.from_inputs(inp)
    q_pos = inp["q_pos_host"]
    if seed % 4 < 2:                                 # the GPU's own selection
        sc = sm.indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"])
        idx = sm.topk_select(batch, sc, k)
        lists = idx.cpu().numpy()
    else:                                            # shuffled lists, masked entries mixed in
        lists = np.full((wl.total_q, k), -1, np.int32)
        for i, p in enumerate(q_pos):
            m = min(p + 1, k)
            sel = g.permutation(p + 1)[:m].astype(np.int32)
            junk = g.random(m) < 0.2                 # some entries past the position
            sel[junk] = p + 1 + g.integers(0, 30, int(junk.sum()))
            lists[i, :m] = sel
            lists[i] = lists[i][g.permutation(k)]
        idx = torch.from_numpy(lists).cuda()
    n_split = int(g.choice([1, 1, 2, 3]))
    n_split = min(n_split, k)
    say("[rand%d] %d seqs, %d queries, H=%d, k=%d, kv=%s, split=%d" %
        (seed, len(kv_lens), wl.total_q, n_heads, k, kv_dtype, n_split))
    kw = {} if n_split == 1 else {"n_split": n_split}
    out, lse = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale, **kw)
    torch.cuda.synchronize()
    rows = np.arange(wl.total_q)
    r_out, r_lse = oracle.attention_rows(inp, rows, lists)
    tl.assert_attention("rand%d" % seed, kv_dtype, out.float().cpu().numpy(), lse.cpu().numpy(),
                        r_out, r_lse, say)


# --------------------------------------------------------------- indexer --
@pytest.mark.parametrize("H,D", [(64, 128), (4, 64), (33, 128)])
def test_indexer_small_integers_bit_exact(sm, H, D):
    """Small-integer inputs make every product and partial sum an exact fp32
    integer, so any summation order gives the oracle's value exactly."""
    g = torch.Generator().manual_seed(H + D)
    L, nq = 333, 333
    q = torch.randint(-8, 9, (nq, H, D), generator=g).to(torch.bfloat16)
    k = torch.randint(-8, 9, (L, D), generator=g).to(torch.bfloat16)
    w = torch.randint(0, 5, (nq, H), generator=g).float()
    inp = {"q_idx": q, "k_idx": k, "w": w, "cu_seqlens_q_host": np.array([0, nq], np.int32),
           "cu_seqlens_kv_host": np.array([0, L], np.int32),
           "q_pos_host": np.arange(nq, dtype=np.int32)}
    batch = sm.Batch([0, nq], [0, L], np.arange(nq), "cuda")
    sc = sm.indexer_score(batch, q.cuda(), k.cuda(), w.cuda())
    torch.cuda.synchronize()
    ref = oracle.indexer_rows(inp, np.arange(nq))
    for i in range(nq):
        assert np.array_equal(sc[i, : i + 1].cpu().numpy(), ref[i]), i


@pytest.mark.parametrize("H,D", [(64, 128), (4, 64), (33, 128)])
def test_indexer_fp8_small_integers_bit_exact(sm, H, D):
    """FP8 indexer on integer codes (|x| <= 8 is exact in E4M3) with
    power-of-two scales per (query, head) and per key: every product, partial
    sum and scaling is exact in fp32, so the scores equal the oracle's
    exactly. Unequal scales pin which row each scale belongs to."""
    g = torch.Generator().manual_seed(7 * H + D)
    L, nq = 333, 333
    q = torch.randint(-8, 9, (nq, H, D), generator=g).float().to(torch.float8_e4m3fn).view(torch.uint8)
    k = torch.randint(-8, 9, (L, D), generator=g).float().to(torch.float8_e4m3fn).view(torch.uint8)
    qs = torch.ldexp(torch.ones(nq, H), torch.randint(-3, 4, (nq, H), generator=g))
    ks = torch.ldexp(torch.ones(L), torch.randint(-3, 4, (L,), generator=g))
    w = torch.randint(0, 5, (nq, H), generator=g).float()
    inp = {"q_idx": q, "k_idx": k, "q_idx_scale": qs, "k_idx_scale": ks, "w": w,
           "cu_seqlens_q_host": np.array([0, nq], np.int32),
           "cu_seqlens_kv_host": np.array([0, L], np.int32),
           "q_pos_host": np.arange(nq, dtype=np.int32)}
    batch = sm.Batch([0, nq], [0, L], np.arange(nq), "cuda")
    sc = sm.indexer_score_fp8(batch, q.cuda(), qs.cuda(), k.cuda(), ks.cuda(), w.cuda())
    torch.cuda.synchronize()
    ref = oracle.indexer_rows(inp, np.arange(nq))
    for i in range(nq):
        assert np.array_equal(sc[i, : i + 1].cpu().numpy(), ref[i]), i


@pytest.mark.parametrize("idx_heads,idx_dim", [(4, 64), (64, 128), (48, 128)])
def test_indexer_fp8_path_all_rows(sm, idx_heads, idx_dim):
    """FP8 indexer inputs through the whole path, every row: scores within
    the indexer tolerance, top-k bit-exact on those scores, attention on the
    GPU's lists. Ragged: an empty sequence, a CP-style gap in the positions,
    a one-token sequence, rows shorter than k and partial key tiles."""
    wl = mla_inputs.Workload("fp8-indexer", (300, 0, 1000, 1, 130),
                             (((0, 300),), (), ((0, 70), (930, 1000)), ((0, 1),), ((64, 130),)),
                             n_heads=64, idx_heads=idx_heads, idx_dim=idx_dim, topk=96,
                             kv_dtype="fp8", seed=29)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu", idx_dtype="fp8"))
    check_path(sm, inp, np.arange(wl.total_q), "fp8-indexer-%dx%d" % (idx_heads, idx_dim))


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("n_queries", [24, 5000])
def test_indexer_writes_only_causal_entries(sm, fp8, n_queries):
    """The score buffer outside j <= q_pos[i] (later keys, and the padding up
    to ld_scores beyond the longest sequence) keeps what the caller put there,
    bit for bit: with few queries (the key split over many workgroups) and
    with many (626 blocks of eight queries, no split), for both input types."""
    L, L2 = 6000, 3000
    na = n_queries // 2                      # the last na tokens of the first sequence,
    nb = n_queries - na                      # the last nb of the second
    wl = mla_inputs.Workload("causal-only", (L, L2), (((L - na, L),), ((L2 - nb, L2),)),
                             n_heads=64, idx_heads=64, idx_dim=128, topk=96, kv_dtype="fp8", seed=70)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu", idx_dtype="fp8" if fp8 else "bf16"))
    batch = sm.Batch.from_inputs(inp)
    ld = L + 77
    sentinel = torch.full((wl.total_q, ld), float("nan"), device="cuda")
    sentinel.view(torch.int32)[:] = 0x7fc0beef
    scores = sentinel.clone()
    if fp8:
        sm.indexer_score_fp8(batch, inp["q_idx"], inp["q_idx_scale"], inp["k_idx"], inp["k_idx_scale"],
                             inp["w"], scores=scores)
    else:
        sm.indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"], scores=scores)
    torch.cuda.synchronize()
    bits = scores.view(torch.int32).cpu().numpy()
    q_pos = inp["q_pos_host"]
    col = np.arange(ld)[None, :]
    written = col <= q_pos[:, None]
    assert (bits[~written] == 0x7fc0beef).all()
    assert not (bits[written] == 0x7fc0beef).any()
    rows = np.array([0, wl.total_q // 2, wl.total_q - 1])
    ref = oracle.indexer_rows(inp, rows)
    mag = fp8_score_magnitude(inp, rows) if fp8 else None
    for t, r in enumerate(rows):
        atol = 1e-4 + FP8_SUM_REL * mag[t] if fp8 else 1e-4
        assert_close("causal-only row %d" % r, scores[int(r), : q_pos[r] + 1].cpu().numpy(), ref[t], atol, 1e-3)


# ----------------------------------------------------------------- top-k --
@pytest.mark.parametrize("kind", ["all_equal", "relu_zeros", "small_int", "signed_zero", "normal",
                                  "coarse", "sample_low", "sample_high", "short_bin_ties",
                                  "short_bin_few_ties"])
def test_topk_ties_bit_exact(sm, kind):
    """Selection bit-exact against the oracle's on score rows built to reach
    each path of the kernel: one key value (no radix level), a threshold bin
    too large for the candidate list (an extra pass: 12 of the 20 rows of
    "normal"), a few dozen candidates resolved by ranking (positive scores on
    a 1/256 or 1/1,024 grid: every row; up to 28 or 9 keys tie with the k-th
    and in most rows only some of them are kept), and sampled or periodic
    structure."""
    g = torch.Generator().manual_seed(3)
    n, L, k = 24, 70000, 2048
    pos = torch.tensor([0, 1, 2046, 2047, 2048, 2049, 5000, 32767, 32768, 32769, 40000, 69999] +
                       torch.randint(0, L, (12,), generator=g).tolist(), dtype=torch.int32)
    if kind == "all_equal":
        s = torch.full((n, L), 7.5)
    elif kind == "relu_zeros":
        s = torch.relu(torch.randn(n, L, generator=g))
    elif kind == "small_int":
        s = torch.randint(0, 6, (n, L), generator=g).float()
    elif kind == "signed_zero":
        s = torch.where(torch.rand(n, L, generator=g) < 0.5, -0.0, 0.0)
        s[:, ::97] = 1.0
    elif kind == "coarse":                 # many exact ties inside the threshold bin
        s = torch.round(torch.randn(n, L, generator=g) * 4) * 2.5
    elif kind in ("short_bin_ties", "short_bin_few_ties"):
        q = 256.0 if kind == "short_bin_ties" else 1024.0
        s = torch.round((torch.randn(n, L, generator=g) + 8) * q) / q
    elif kind in ("sample_low", "sample_high"):
        # periodic structure: one 128-byte line in 16 holds the row's lowest
        # (or highest) scores, far from the rest
        lines = (torch.arange(L) % 512) < 32
        s = torch.randn(n, L, generator=g) + (100.0 if kind == "sample_low" else 0.0)
        s[:, lines] = torch.randn(n, int(lines.sum()), generator=g) + (0.0 if kind == "sample_low" else 1e4)
    else:
        s = torch.randn(n, L, generator=g) * 100
    batch = sm.Batch([0, n], [0, L], pos, "cuda")
    idx = sm.topk_select(batch, s.cuda(), k)
    torch.cuda.synchronize()
    ref = oracle.topk_seq(s.numpy(), pos.numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("k", [1, 4096])
@pytest.mark.parametrize("kind", ["normal", "coarse"])
def test_topk_limits_bit_exact(sm, k, kind):
    """The largest k (4,096) and k = 1, on rows up to the longest the kernel
    takes (524,288 keys), around the keep-all boundary and at p = 0."""
    g = torch.Generator().manual_seed(11 + k)
    L = 524288
    pos = torch.tensor([0, k - 2, k - 1, k, k + 1, 100000, L - 2, L - 1], dtype=torch.int32).clamp(min=0)
    n = len(pos)
    s = torch.randn(n, L, generator=g) * 100
    if kind == "coarse":
        s = torch.round(s / 25) * 25
    batch = sm.Batch([0, n], [0, L], pos, "cuda")
    idx = sm.topk_select(batch, s.cuda(), k)
    torch.cuda.synchronize()
    ref = oracle.topk_seq(s.numpy(), pos.numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ref)


# ------------------------------------------------------ ragged and layout --
def test_ragged_small_batch_all_rows(sm):
    """Empty sequence, gaps in the positions (a CP-style share), rows shorter
    than k, a one-token sequence and a ragged tail."""
    wl = mla_inputs.Workload("ragged-small", (300, 0, 1000, 1, 130),
                             (((0, 300),), (), ((0, 70), (930, 1000)), ((0, 1),), ((64, 130),)),
                             n_heads=64, idx_heads=64, idx_dim=128, topk=96, kv_dtype="fp8", seed=23)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu"))
    check_path(sm, inp, np.arange(wl.total_q), "ragged-small")


def test_inline_scale_row_layout(sm):
    """sigma stored inline at the tail of a 640-byte row (byte strides) gives
    the same result as separate arrays."""
    wl = mla_inputs.Workload("inline", (500,), (((0, 500),),), n_heads=64, idx_heads=4,
                             idx_dim=64, topk=128, kv_dtype="fp8", seed=24)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu"))
    batch = sm.Batch.from_inputs(inp)
    sc = sm.indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"])
    idx = sm.topk_select(batch, sc, wl.topk)
    o1, l1 = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale)
    packed = torch.zeros((wl.total_kv, 640), dtype=torch.uint8, device="cuda")
    packed[:, :576] = inp["kv"]
    packed[:, 576:580] = inp["kv_scale"].view(torch.uint8).view(-1, 4)
    o2, l2 = sm.sparse_prefill(batch, inp["q"], packed, packed[:, 576:].view(torch.float32)[:, 0],
                               idx, wl.sm_scale, kv_row_stride=640, kv_scale_stride=640)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------- full-size workloads --
FULL = [("sparse32k", "fp8", "bf16"), ("sparse32k", "bf16", "bf16"), ("dense16k", "bf16", "bf16"),
        ("cp131k", "fp8", "bf16"), ("ragged", "fp8", "bf16"), ("sparse32k", "fp8", "fp8"),
        ("ragged", "fp8", "fp8"), ("sparse32k", "ds656", "bf16")]


@pytest.mark.parametrize("name,kv_dtype,idx_dtype", FULL)
def test_full_size_sampled_rows(sm, name, kv_dtype, idx_dtype):
    wl = mla_inputs.WORKLOADS[name]
    n_rows = int(os.environ.get("MLA_PARITY_ROWS", "512"))
    rows = mla_inputs.sample_rows(wl, n_rows)
    say("[%s/%s/indexer %s] generating inputs on the GPU" % (name, kv_dtype, idx_dtype))
    inp = mla_inputs.make_inputs(wl, "cuda", kv_dtype=kv_dtype, idx_dtype=idx_dtype)
    if wl.dense:
        batch = sm.Batch.from_inputs(inp)
        out, lse = sm.sparse_prefill(batch, inp["q"], inp["kv"], None, None, wl.sm_scale)
        torch.cuda.synchronize()
        say("[%s] oracle dense attention on %d rows" % (name, len(rows)))
        r_out, r_lse = oracle.attention_rows(inp, rows, None)
        rt = torch.as_tensor(rows, device="cuda")
        tl.assert_attention("dense16k", "bf16", out[rt].float().cpu().numpy(),
                            lse[rt].cpu().numpy(), r_out, r_lse, say)
    else:
        check_path(sm, inp, rows, "%s-%s-idx%s" % (name, kv_dtype, idx_dtype), gate_overlap=True)
    del inp
    torch.cuda.empty_cache()


# ------------------------------------------------------- split-KV attention --
def _few_queries(kv_dtype, seed, k=96):
    """Few queries (fewer than the CUs) over long rows: ragged, with a CP-style
    gap and rows shorter than k."""
    wl = mla_inputs.Workload("split", (700, 1, 2500), (((0, 6), (690, 700)), ((0, 1),),
                                                      ((0, 2), (2480, 2500))),
                             n_heads=64, idx_heads=4, idx_dim=64, topk=k, kv_dtype=kv_dtype, seed=seed)
    return to_gpu(mla_inputs.make_inputs(wl, "cpu"))


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("n_split", [0, 2, 3, 7, 16])
def test_split_kv_listed_keys(sm, kv_dtype, n_split):
    """mla_sparse_prefill_split over the GPU's own index lists: every row
    against the oracle on the same lists (parts are rounded to bf16 before the
    merge; the attention tolerance covers it), and against the unsplit call.
    n_split 0: the count chosen from the CU count (here CUs / 39 queries)."""
    inp = _few_queries(kv_dtype, 40 + n_split)
    wl = inp["workload"]
    batch = sm.Batch.from_inputs(inp)
    sc = sm.indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"])
    idx = sm.topk_select(batch, sc, wl.topk)
    o1, l1 = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale)
    o2, l2 = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale,
                               n_split=n_split)
    torch.cuda.synchronize()
    rows = np.arange(wl.total_q)
    r_out, r_lse = oracle.attention_rows(inp, rows, idx.cpu().numpy())
    tol = TOL[kv_dtype]
    assert_close("split%d out" % n_split, o2.float().cpu().numpy(), r_out, tol, tol)
    assert_close("split%d lse" % n_split, l2.cpu().numpy(), r_lse, LSE_ATOL, LSE_RTOL)
    assert_close("split%d vs unsplit" % n_split, o2.float().cpu().numpy(),
                 o1.float().cpu().numpy(), 1e-2, 1e-2)
    np.testing.assert_allclose(l2.cpu().numpy(), l1.cpu().numpy(), rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_split_kv_dense_with_empty_parts(sm, kv_dtype):
    """Dense split: key ranges of 0..p_i, so rows with p_i + 1 < n_split have
    empty parts (out 0, lse -inf before the merge); every row vs the oracle."""
    inp = _few_queries(kv_dtype, 50)
    wl = inp["workload"]
    batch = sm.Batch.from_inputs(inp)
    out, lse = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], None, wl.sm_scale,
                                 n_split=5)
    torch.cuda.synchronize()
    assert (inp["q_pos_host"] + 1 < 5).any()
    rows = np.arange(wl.total_q)
    r_out, r_lse = oracle.attention_rows(inp, rows, None)
    tol = TOL[kv_dtype]
    assert_close("dense split out", out.float().cpu().numpy(), r_out, tol, tol)
    assert_close("dense split lse", lse.cpu().numpy(), r_lse, LSE_ATOL, LSE_RTOL)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_split_kv_long_lists_and_single_entry_parts(sm, kv_dtype):
    """Lists longer than one 2,048-entry chunk (k = 4,500, parts of 1,500 and
    of 2,250 keys), and n_split = k (one entry per part), against the oracle."""
    inp = _few_queries(kv_dtype, 60)
    wl = inp["workload"]
    batch = sm.Batch.from_inputs(inp)
    q_pos = inp["q_pos_host"]
    g = np.random.default_rng(61)
    lists = np.full((wl.total_q, 4500), -1, np.int32)
    for i, p in enumerate(q_pos):            # every earlier key, shuffled, -1 padded
        lists[i, : p + 1] = g.permutation(p + 1)
    idx = torch.from_numpy(lists).cuda()
    rows = np.arange(wl.total_q)
    r_out, r_lse = oracle.attention_rows(inp, rows, lists)
    tol = TOL[kv_dtype]
    for n_split in (2, 3):
        out, lse = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale,
                                     n_split=n_split)
        torch.cuda.synchronize()
        assert_close("long split%d out" % n_split, out.float().cpu().numpy(), r_out, tol, tol)
        assert_close("long split%d lse" % n_split, lse.cpu().numpy(), r_lse, LSE_ATOL, LSE_RTOL)
    few = idx[:, :5].contiguous()
    out, lse = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], few, wl.sm_scale,
                                 n_split=5)
    torch.cuda.synchronize()
    r_out, r_lse = oracle.attention_rows(inp, rows, lists[:, :5])
    assert_close("k=n_split out", out.float().cpu().numpy(), r_out, tol, tol)
    assert_close("k=n_split lse", lse.cpu().numpy(), r_lse, LSE_ATOL, LSE_RTOL)


def test_split_kv_tail_of_32k(sm):
    """The last 64 queries of the 32k workload (top-2,048 lists, FP8 KV):
    fewer queries than CUs, the case split-KV is for. Split 4 vs unsplit on
    every row, and sampled rows vs the oracle."""
    wl = mla_inputs.WORKLOADS["sparse32k"]
    tail = mla_inputs.Workload("tail64", (32768,), (((32704, 32768),),), n_heads=64, idx_heads=64,
                               idx_dim=128, topk=2048, kv_dtype="fp8", seed=wl.seed)
    inp = mla_inputs.make_inputs(tail, "cuda")
    batch = sm.Batch.from_inputs(inp)
    sc = sm.indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"])
    idx = sm.topk_select(batch, sc, tail.topk)
    o1, l1 = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, tail.sm_scale)
    o4, l4 = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, tail.sm_scale,
                               n_split=4)
    torch.cuda.synchronize()
    assert_close("tail split4 vs unsplit", o4.float().cpu().numpy(), o1.float().cpu().numpy(),
                 1e-2, 1e-2)
    np.testing.assert_allclose(l4.cpu().numpy(), l1.cpu().numpy(), rtol=1e-5, atol=1e-5)
    rows = np.array([0, 17, 40, 63])
    r_out, r_lse = oracle.attention_rows(inp, rows, idx[torch.as_tensor(rows).cuda()].cpu().numpy())
    assert_close("tail split4 out", o4[torch.as_tensor(rows).cuda()].float().cpu().numpy(), r_out,
                 6e-2, 6e-2)
    assert_close("tail split4 lse", l4[torch.as_tensor(rows).cuda()].cpu().numpy(), r_lse, LSE_ATOL, LSE_RTOL)


def test_resume64_key_split_indexer_and_auto_split(sm):
    """64 new tokens behind a 32,704-token prefix: eight query blocks, so the
    indexer splits each block's keys over many workgroups, and attention runs
    with the automatic split. The whole path on every row, both ways round."""
    wl = mla_inputs.WORKLOADS["resume64"]
    inp = mla_inputs.make_inputs(wl, "cuda")
    batch = sm.Batch.from_inputs(inp)
    sc = sm.indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"])
    idx = sm.topk_select(batch, sc, wl.topk)
    out, lse = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale,
                                 n_split=0)
    torch.cuda.synchronize()
    rows = np.arange(wl.total_q)
    q_pos = inp["q_pos_host"]
    r_scores = oracle.indexer_rows(inp, rows)
    g_scores = [sc[int(r), : q_pos[r] + 1].cpu().numpy() for r in rows]
    for r in rows:
        assert_close("resume64 indexer row %d" % r, g_scores[r], r_scores[r], 1e-4, 1e-3)
    r_idx = oracle.topk_rows(g_scores, q_pos[rows], wl.topk)
    assert np.array_equal(r_idx, idx.cpu().numpy())
    r_out, r_lse = oracle.attention_rows(inp, rows, idx.cpu().numpy())
    assert_close("resume64 out", out.float().cpu().numpy(), r_out, 6e-2, 6e-2)
    assert_close("resume64 lse", lse.cpu().numpy(), r_lse, LSE_ATOL, LSE_RTOL)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("dense", [False, True])
@pytest.mark.parametrize("n_split", [None, 4])
def test_attention_writes_stay_in_bounds(sm, kv_dtype, dense, n_split):
    """Guard rows after out and lse, and guard bytes after the split
    workspace, keep their sentinel: no write lands outside the buffers."""
    inp = _few_queries(kv_dtype, 80)
    wl = inp["workload"]
    batch = sm.Batch.from_inputs(inp)
    H, nq, G = wl.n_heads, wl.total_q, 5
    idx = None
    if not dense:
        sc = sm.indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"])
        idx = sm.topk_select(batch, sc, wl.topk)
    out_all = torch.full((nq + G, H, 512), -7.0, dtype=torch.bfloat16, device="cuda")
    lse_all = torch.full((nq + G, H), -7.0, dtype=torch.float32, device="cuda")
    ws = None
    need = 0
    if n_split:
        need = sm.load_library().mla_sparse_prefill_split_workspace_size(nq, H, n_split)
        ws = torch.full((need + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale,
                      out=out_all[:nq], lse=lse_all[:nq], n_split=n_split,
                      workspace=ws[:need] if n_split else None)
    torch.cuda.synchronize()
    assert (out_all[nq:].float() == -7.0).all() and (lse_all[nq:] == -7.0).all()
    assert not (lse_all[:nq] == -7.0).any()
    if n_split:
        assert (ws[need:] == 0xA5).all()
    r_out, r_lse = oracle.attention_rows(inp, np.arange(nq), None if dense else idx.cpu().numpy())
    tol = TOL[kv_dtype]
    assert_close("bounds out", out_all[:nq].float().cpu().numpy(), r_out, tol, tol)
    assert_close("bounds lse", lse_all[:nq].cpu().numpy(), r_lse, LSE_ATOL, LSE_RTOL)


# ------------------------------------------------- LSE merge and key shards --
def test_merge_random_parts(sm):
    """mla_merge_attention against oracle.merge_lse on the same bf16 parts:
    random outputs and LSEs, some parts empty (-inf), some rows with every
    part empty."""
    g = torch.Generator().manual_seed(11)
    n_parts, total_q, H = 5, 300, 16
    o = [(torch.randn(total_q, H, 512, generator=g) * 3).to(torch.bfloat16) for _ in range(n_parts)]
    l = [torch.randn(total_q, H, generator=g) * 20 for _ in range(n_parts)]
    for r in range(n_parts):                     # empty parts here and there
        l[r][torch.rand(total_q, H, generator=g) < 0.3] = -math.inf
    for r in range(n_parts):                     # rows 0..9: every part empty
        l[r][:10] = -math.inf
        o[r][:10] = 0
    out, lse = sm.merge_attention([t.cuda() for t in o], [t.cuda() for t in l])
    torch.cuda.synchronize()
    r_out, r_lse = oracle.merge_lse([t.float().numpy() for t in o], [t.numpy() for t in l])
    # fp32 weights and sums, out rounded once to bf16
    assert_close("merge out", out.float().cpu().numpy(), r_out, 2e-2, 1e-2)
    assert_close("merge lse", lse.cpu().numpy(), r_lse, 1e-5, 1e-6)
    assert (out[:10] == 0).all().item() and torch.isneginf(lse[:10]).all().item()


def test_topk_and_merge_writes_stay_in_bounds(sm):
    """Guard rows after the top-k index array and after the merge outputs keep
    their sentinel; the written rows are the oracle's."""
    g = torch.Generator().manual_seed(12)
    n, L, k, G = 40, 9000, 512, 3
    pos = torch.randint(0, L, (n,), generator=g, dtype=torch.int32)
    pos[:4] = torch.tensor([0, k - 1, k, L - 1], dtype=torch.int32)
    s = torch.randn(n, L, generator=g)
    batch = sm.Batch([0, n], [0, L], pos, "cuda")
    idx_all = torch.full((n + G, k), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    sm.topk_select(batch, s.cuda(), k, indices=idx_all[:n])
    torch.cuda.synchronize()
    assert (idx_all[n:] == 0x5A5A5A5A).all()
    assert np.array_equal(idx_all[:n].cpu().numpy(), oracle.topk_seq(s.numpy(), pos.numpy(), k))

    total_q, H, P = 33, 8, 3
    o = [(torch.randn(total_q, H, 512, generator=g)).to(torch.bfloat16).cuda() for _ in range(P)]
    l = [(torch.randn(total_q, H, generator=g) * 5).cuda() for _ in range(P)]
    out_all = torch.full((total_q + G, H, 512), -7.0, dtype=torch.bfloat16, device="cuda")
    lse_all = torch.full((total_q + G, H), -7.0, dtype=torch.float32, device="cuda")
    sm.merge_attention(o, l, out=out_all[:total_q], lse=lse_all[:total_q])
    torch.cuda.synchronize()
    assert (out_all[total_q:].float() == -7.0).all() and (lse_all[total_q:] == -7.0).all()
    r_out, r_lse = oracle.merge_lse([t.float().cpu().numpy() for t in o], [t.cpu().numpy() for t in l])
    assert_close("merge bounds out", out_all[:total_q].float().cpu().numpy(), r_out, 2e-2, 1e-2)
    assert_close("merge bounds lse", lse_all[:total_q].cpu().numpy(), r_lse, 1e-5, 1e-6)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_dcp_key_shards_merge_to_full(sm, kv_dtype):
    """DCP-style attention on one GPU: the tiny batch's KV rows dealt round-
    robin to 8 shards (row j on shard j mod 8), attention of every query over
    each shard's part of its top-k list, then mla_merge_attention. The merge
    must match the unsharded GPU result and the oracle."""
    wl = mla_inputs.WORKLOADS["tiny"]
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu", kv_dtype=kv_dtype))
    batch = sm.Batch.from_inputs(inp)
    scores = sm.indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"])
    idx = sm.topk_select(batch, scores, wl.topk)
    full_o, full_l = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale)
    n_shards, L, k = 8, wl.total_kv, wl.topk
    idx_h = idx.cpu().numpy()
    parts_o, parts_l = [], []
    for r in range(n_shards):
        rows = np.arange(r, L, n_shards)
        sel = np.where((idx_h >= 0) & (idx_h % n_shards == r), idx_h // n_shards, -1)
        loc = np.full_like(idx_h, -1)                    # shard-local lists, ascending, -1 padded
        for i in range(idx_h.shape[0]):
            v = np.sort(sel[i][sel[i] >= 0])
            loc[i, : len(v)] = v
        Lr = len(rows)
        sb = sm.Batch([0, wl.total_q], [0, Lr], torch.full((wl.total_q,), Lr - 1, dtype=torch.int32), "cuda")
        rt = torch.as_tensor(rows, device="cuda")
        kv_r = inp["kv"][rt].contiguous()
        sc_r = inp["kv_scale"][rt].contiguous() if inp["kv_scale"] is not None else None
        o_r, l_r = sm.sparse_prefill(sb, inp["q"], kv_r, sc_r, torch.as_tensor(loc, device="cuda"),
                                     wl.sm_scale)
        parts_o.append(o_r)
        parts_l.append(l_r)
    m_o, m_l = sm.merge_attention(parts_o, parts_l)
    torch.cuda.synchronize()
    tol = TOL[kv_dtype]
    assert_close("dcp out vs unsharded", m_o.float().cpu().numpy(), full_o.float().cpu().numpy(), 2e-2, 2e-2)
    assert_close("dcp lse vs unsharded", m_l.cpu().numpy(), full_l.cpu().numpy(), LSE_ATOL, LSE_RTOL)
    rows = np.arange(0, wl.total_q, 7)
    r_out, r_lse = oracle.attention_rows(inp, rows, idx_h[rows])
    rt = torch.as_tensor(rows, device="cuda")
    assert_close("dcp out vs oracle", m_o[rt].float().cpu().numpy(), r_out, tol, tol)
    assert_close("dcp lse vs oracle", m_l[rt].cpu().numpy(), r_lse, LSE_ATOL, LSE_RTOL)


# ---------------------------------------------- fused indexer + top-k --
def _fused_vs_unfused(sm, inp, label, oracle_rows=None):
    """mla_indexer_topk(_fp8) against mla_topk_select on mla_indexer_score(_fp8)'s
    scores for the same inputs: equal on every row, bit for bit (the fused
    kernel computes the same scores with the same instructions and applies
    the same selection rule). On oracle_rows, also the oracle's selection on
    those GPU scores."""
    wl = inp["workload"]
    k = wl.topk
    batch = sm.Batch.from_inputs(inp)
    if inp.get("k_idx_scale") is not None:
        args = (batch, inp["q_idx"], inp["q_idx_scale"], inp["k_idx"], inp["k_idx_scale"], inp["w"])
        sc = sm.indexer_score_fp8(*args)
        fused = sm.indexer_topk_fp8(*args, k)
    else:
        args = (batch, inp["q_idx"], inp["k_idx"], inp["w"])
        sc = sm.indexer_score(*args)
        fused = sm.indexer_topk(*args, k)
    ref = sm.topk_select(batch, sc, k)
    torch.cuda.synchronize()
    bad = (fused != ref).any(dim=1).nonzero().flatten()
    assert bad.numel() == 0, "%s: fused top-k differs on %d rows, first %s" % (
        label, bad.numel(), bad[:8].tolist())
    say("[%s] fused indexer + top-k equals the unfused path on all %d rows" % (label, wl.total_q))
    if oracle_rows is not None:
        q_pos = inp["q_pos_host"]
        rows = np.asarray(oracle_rows)
        g_scores = [sc[int(r), : q_pos[r] + 1].cpu().numpy() for r in rows]
        r_idx = oracle.topk_rows(g_scores, q_pos[rows], k)
        got = fused[torch.as_tensor(rows, device="cuda")].cpu().numpy()
        assert np.array_equal(r_idx, got), label
        say("[%s] fused indices equal the oracle's selection on the GPU scores of %d rows" %
            (label, len(rows)))
    return fused, sc


@pytest.mark.parametrize("idx_dtype", ["bf16", "fp8"])
def test_fused_topk_tiny_and_ragged_all_rows(sm, idx_dtype):
    """Tiny (k = 256 on 1,024 keys) and a ragged batch (an empty sequence, a
    CP-style gap, a one-token sequence, rows shorter than k, k = 96): every
    row against the unfused path and the oracle."""
    wl = mla_inputs.WORKLOADS["tiny"]
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu", idx_dtype=idx_dtype))
    _fused_vs_unfused(sm, inp, "fused-tiny-" + idx_dtype, np.arange(wl.total_q))
    wl = mla_inputs.Workload("fused-ragged", (300, 0, 1000, 1, 130),
                             (((0, 300),), (), ((0, 70), (930, 1000)), ((0, 1),), ((64, 130),)),
                             n_heads=8, idx_heads=64, idx_dim=128, topk=96, kv_dtype="fp8", seed=101)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu", idx_dtype=idx_dtype))
    _fused_vs_unfused(sm, inp, "fused-ragged-" + idx_dtype, np.arange(wl.total_q))


@pytest.mark.parametrize("seed", range(8))
def test_path_random_batches(sm, seed):
    """Seeded random ragged batches through the whole path: the indexer (bf16
    or FP8 inputs; 4, 33 or 64 heads of 64 or 128 dims) against the oracle on
    every row, top-k bit-exact against the oracle's selection on the GPU's
    scores, attention (FP8 or bf16 rows) on every row, and the fused indexer +
    top-k equal to the unfused pair, bit for bit."""
    kv_lens, ranges, g = _random_batch(3000 + seed)
    idx_heads = int(g.choice([4, 33, 64]))
    idx_dim = int(g.choice([64, 128]))
    k = int(g.choice([1, 17, 256, 2048]))
    n_heads = int(g.choice([8, 16, 32, 64]))
    kv_dtype = ["fp8", "bf16"][seed % 2]
    idx_dtype = ["bf16", "fp8"][(seed // 2) % 2]
    wl = mla_inputs.Workload("path%d" % seed, kv_lens, ranges, n_heads=n_heads, idx_heads=idx_heads,
                             idx_dim=idx_dim, topk=k, kv_dtype=kv_dtype, seed=4000 + seed)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu", idx_dtype=idx_dtype))
    say("[path%d] %d seqs, %d queries, indexer %dx%d %s, k=%d, H=%d, kv=%s" %
        (seed, len(kv_lens), wl.total_q, idx_heads, idx_dim, idx_dtype, k, n_heads, kv_dtype))
    check_path(sm, inp, np.arange(wl.total_q), "path%d" % seed)
    _fused_vs_unfused(sm, inp, "path%d-fused" % seed)


def _indexer_only(nq, L, H, D, k, q, kI, w, q_lo):
    """A one-sequence batch of nq queries at positions q_lo .. q_lo + nq - 1."""
    wl = mla_inputs.Workload("fused-custom", (L,), (((q_lo, q_lo + nq),),), n_heads=8,
                             idx_heads=H, idx_dim=D, topk=k, kv_dtype="bf16", seed=0)
    return {"workload": wl, "q_idx": q.cuda(), "k_idx": kI.cuda(), "w": w.cuda(),
            "cu_seqlens_q_host": wl.cu_seqlens_q(), "cu_seqlens_kv_host": wl.cu_seqlens_kv(),
            "q_pos_host": wl.q_pos(), "q_pos": torch.from_numpy(wl.q_pos()).cuda(),
            "q": torch.empty((nq, 1, 576), dtype=torch.bfloat16, device="cuda")}


@pytest.mark.parametrize("kind", ["small_int", "all_zero", "rising", "falling"])
def test_fused_topk_ties_and_order(sm, kind):
    """Score patterns that stress the candidate list: small-integer inputs
    (many exact ties), all scores zero (every key ties: the first k win),
    scores rising with j in steps of 24 equal keys (every key beats the
    threshold, so the list is compacted every few tiles, ties at each
    compaction), and falling (nothing is appended after the first k)."""
    g = torch.Generator().manual_seed(17)
    nq, L, H, D, k = 64, 9000, 4, 64, 200
    w = torch.randint(0, 3, (nq, H), generator=g).float()
    if kind == "small_int":
        q = torch.randint(-3, 4, (nq, H, D), generator=g).to(torch.bfloat16)
        kI = torch.randint(-3, 4, (L, D), generator=g).to(torch.bfloat16)
    elif kind == "all_zero":
        q = torch.zeros((nq, H, D), dtype=torch.bfloat16)
        kI = torch.randint(-3, 4, (L, D), generator=g).to(torch.bfloat16)
    else:
        q = torch.ones((nq, H, D), dtype=torch.bfloat16)
        ramp = torch.arange(L) // 24 if kind == "rising" else (L - 1 - torch.arange(L)) // 24
        kI = ramp[:, None].expand(L, D).to(torch.bfloat16)      # integers <= 374: exact in bf16
        w = torch.ones((nq, H))
    inp = _indexer_only(nq, L, H, D, k, q, kI, w, L - nq)
    _fused_vs_unfused(sm, inp, "fused-" + kind, np.arange(nq))


@pytest.mark.parametrize("k", [1, 4096])
def test_fused_topk_k_limits(sm, k):
    """k = 1 and the largest k (4,096) on rows of up to 20,000 keys, rows
    around the keep-all boundary and p = 0."""
    g = torch.Generator().manual_seed(k)
    L, H, D = 20000, 8, 64
    pos = np.array(sorted({0, max(k - 2, 0), max(k - 1, 0), k, k + 1, 9999, L - 2, L - 1}))
    nq = len(pos)
    q = torch.randn((nq, H, D), generator=g).to(torch.bfloat16)
    kI = torch.randn((L, D), generator=g).to(torch.bfloat16)
    w = torch.rand((nq, H), generator=g)
    batch = sm.Batch([0, nq], [0, L], pos, "cuda")
    sc = sm.indexer_score(batch, q.cuda(), kI.cuda(), w.cuda())
    fused = sm.indexer_topk(batch, q.cuda(), kI.cuda(), w.cuda(), k)
    ref = sm.topk_select(batch, sc, k)
    torch.cuda.synchronize()
    assert torch.equal(fused, ref)
    g_scores = [sc[i, : pos[i] + 1].cpu().numpy() for i in range(nq)]
    assert np.array_equal(oracle.topk_rows(g_scores, pos, k), fused.cpu().numpy())


@pytest.mark.parametrize("idx_dtype", ["bf16", "fp8"])
def test_fused_topk_key_split_merge(sm, idx_dtype):
    """Few queries behind long prefixes (fewer eight-query blocks than twice
    the CUs): every block's keys are split over many workgroups, each keeps
    its own candidate list, and the merge kernel selects over their
    concatenation. Every row against the unfused path and the oracle."""
    wl = mla_inputs.Workload("fused-split", (30000, 5000), (((29970, 30000),), ((0, 3), (4990, 5000))),
                             n_heads=8, idx_heads=64, idx_dim=128, topk=2048, kv_dtype="fp8", seed=103)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu", idx_dtype=idx_dtype))
    batch = sm.Batch.from_inputs(inp)
    need = sm.load_library().mla_topk_workspace_size(batch.c, wl.topk)
    assert need > wl.total_q * 4352 * 8                 # more than one list per query: split
    _fused_vs_unfused(sm, inp, "fused-split-" + idx_dtype, np.arange(wl.total_q))


FUSED_FULL = [("sparse32k", "bf16"), ("cp131k", "bf16"), ("ragged", "bf16"), ("sparse32k", "fp8"),
              ("ragged", "fp8"), ("resume64", "bf16")]


@pytest.mark.parametrize("name,idx_dtype", FUSED_FULL)
def test_fused_topk_full_size(sm, name, idx_dtype):
    """The benchmark workloads: fused indices equal the unfused path's on
    every row, and the oracle's selection on the GPU's scores on 64 sampled
    rows (chunk edges, keep-all boundary, seeded picks)."""
    wl = mla_inputs.WORKLOADS[name]
    say("[fused %s/%s] generating inputs on the GPU" % (name, idx_dtype))
    inp = mla_inputs.make_inputs(wl, "cuda", idx_dtype=idx_dtype)
    rows = mla_inputs.sample_rows(wl, 64, per_seq=8)
    _fused_vs_unfused(sm, inp, "fused-%s-%s" % (name, idx_dtype), rows)
    del inp
    torch.cuda.empty_cache()


# ------------------------------------------------------ 656-byte latent rows --
def test_ds656_decode_bit_exact(sm):
    """mla_kv_decode_ds656 against torch's own float8 decode, fp32 multiply
    and bf16 cast (each rounding to nearest even) on rows with tiles of very
    different ranges, an all-zero tile, and a 672-byte row stride."""
    g = torch.Generator().manual_seed(31)
    n = 3001
    x = torch.randn((n, 576), generator=g)
    x[:, 128:256] *= 300.0
    x[:, 384:512] *= 1e-3
    x[7, :128] = 0.0
    rows = mla_inputs.pack_ds656_rows(x)
    wide = torch.zeros((n, 672), dtype=torch.uint8)
    wide[:, :656] = rows
    got = sm.kv_decode_ds656(wide.cuda()[:, :656])
    codes = rows[:, :512].contiguous().view(torch.float8_e4m3fn).float().reshape(n, 4, 128)
    scales = rows[:, 512:528].contiguous().view(torch.float32)
    latent = (codes * scales[:, :, None]).reshape(n, 512).to(torch.bfloat16)
    rope = rows[:, 528:656].contiguous().view(torch.bfloat16)
    ref = torch.cat([latent, rope], dim=1)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu().view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("name", ["tiny", "ragged-small"])
def test_ds656_path_all_rows(sm, name):
    """The whole path on 656-byte rows (indexer -> top-k -> decode -> bf16
    attention), every row against the oracle's exact decode of the same
    bytes, at the 656-byte row gates."""
    if name == "tiny":
        wl = mla_inputs.WORKLOADS["tiny"].scaled(n_heads=64)
    else:
        wl = mla_inputs.Workload("ds656-ragged", (300, 0, 1000, 1, 130),
                                 (((0, 300),), (), ((0, 70), (930, 1000)), ((0, 1),), ((64, 130),)),
                                 n_heads=64, idx_heads=64, idx_dim=128, topk=96, kv_dtype="ds656",
                                 seed=33)
    inp = to_gpu(mla_inputs.make_inputs(wl, "cpu", kv_dtype="ds656"))
    check_path(sm, inp, np.arange(wl.total_q), "ds656-" + name)
