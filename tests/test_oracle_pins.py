"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test fixes part of what the oracle computes with an independent fact:
an explicit (non-absorbed) MLA form, torch's float64 scaled-dot-product
attention, brute-force sorting, integer closed forms, torch's own bf16/fp8
casts, the log-sum-exp merge rule, and the arithmetic the spke.com article
prints in its footnotes. The sizes are tiny so the suite runs in seconds.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import FMT_BF16, FMT_DS656, FMT_E4M3, FMT_F64
import mla_inputs
import bench

SM = 1.0 / math.sqrt(192.0)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- formats --
def test_e4m3_decoder_matches_torch_for_all_codes():
    """OCP E4M3 (e4m3fn) decode of all 256 codes equals torch's float8_e4m3fn."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([oracle.e4m3_decode(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2                      # 0x7f and 0xff
    assert np.array_equal(ref[~nan], got[~nan])
    assert got[0x7e] == 448.0 and got[0x01] == 2.0 ** -9


def test_e4m3_roundtrip_and_error_bound():
    """quantize(decode(c)) == c for every finite code; RNE relative error of
    normals <= 2^-4 (3 mantissa bits)."""
    codes = np.array([c for c in range(256) if c not in (0x7f, 0xff)], dtype=np.uint8)
    vals = torch.tensor([oracle.e4m3_decode(c) for c in codes], dtype=torch.float32)
    back = vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # +0 and -0 both decode to a zero that re-encodes to its own sign
    assert np.array_equal(back, codes)
    x = torch.randn(4096, 576, generator=torch.Generator().manual_seed(5))
    c, s = mla_inputs.quantize_e4m3_rows(x)
    dec = np.vectorize(oracle.e4m3_decode)(c.numpy()[:64]) * s.numpy()[:64, None]
    xx = x.numpy()[:64].astype(np.float64)
    normal = np.abs(xx / s.numpy()[:64, None]) >= 2.0 ** -6
    rel = np.abs(dec - xx)[normal] / np.abs(xx)[normal]
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)
    assert (c.numpy() & 0x7f).max() <= 0x7e   # saturating: no NaN codes


def test_bf16_decoder_matches_torch():
    bits = np.random.default_rng(0).integers(0, 2 ** 16, 5000).astype(np.uint16)
    bits = bits[(bits & 0x7f80) != 0x7f80]     # drop inf/nan
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_decode(b) for b in bits[:500]])
    assert np.array_equal(ref[:500], got)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), ref)


# ----------------------------------------------------------------- indexer --
def _int_indexer_case(rng, n, H, D, L, lo=-8, hi=8, wmax=4):
    q = rng.integers(lo, hi + 1, (n, H, D))
    k = rng.integers(lo, hi + 1, (L, D))
    w = rng.integers(0, wmax + 1, (n, H))
    p = rng.integers(0, L, n)
    return q, k, w, p


def _int_indexer_expected(q, k, w, p):
    """Brute force in Python integers: sum_h w * max(0, q.k)."""
    out = []
    for i in range(q.shape[0]):
        row = []
        for j in range(int(p[i]) + 1):
            s = 0
            for h in range(q.shape[1]):
                dot = int(np.dot(q[i, h].astype(object), k[j].astype(object)))
                s += int(w[i, h]) * max(0, dot)
            row.append(s)
        out.append(row)
    return out


@pytest.mark.parametrize("H,D", [(1, 16), (4, 64), (3, 128)])
def test_indexer_integer_closed_form(H, D):
    """Small-integer inputs keep every product and partial sum an exact
    integer, so the score equals a Python-integer brute force exactly. Distinct
    integer weights per (query, head) pin the weight indexing; mixed-sign dots
    pin ReLU per head before weighting."""
    rng = np.random.default_rng(H * 1000 + D)
    q, k, w, p = _int_indexer_case(rng, 6, H, D, 40)
    got = oracle.indexer_seq(bf16_bits(q), bf16_bits(k), w.astype(np.float32), p)
    exp = _int_indexer_expected(q, k, w, p)
    for i in range(6):
        assert np.array_equal(got[i, : p[i] + 1], np.array(exp[i], dtype=np.float32))
        assert np.isnan(got[i, p[i] + 1:]).all()        # causal: later keys untouched


def test_indexer_single_head_is_relu_dot():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((5, 1, 64)).astype(np.float32)
    k = rng.standard_normal((30, 64)).astype(np.float32)
    qb, kb = bf16_bits(q), bf16_bits(k)
    got = oracle.indexer_seq(qb, kb, np.ones((5, 1), np.float32), np.full(5, 29))
    qd, kd = oracle.bf16_bits_to_f64(qb)[:, 0], oracle.bf16_bits_to_f64(kb)
    ref = np.maximum(qd @ kd.T, 0.0).astype(np.float32)   # numpy matmul: independent path
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-6)
    assert (got == 0).any() and (got > 0).any()


# ------------------------------------------------------------ FP8 indexer --
def _e4m3_codes(x: np.ndarray) -> np.ndarray:
    """torch's float32 -> float8_e4m3fn cast (RNE), as raw codes."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3(codes: np.ndarray) -> np.ndarray:
    """torch's float8_e4m3fn decode (a library decoder, not the oracle's)."""
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).double().numpy()


@pytest.mark.parametrize("H,D", [(4, 64), (3, 128)])
def test_indexer_fp8_power_of_two_scales_equal_bf16_path(H, D):
    """An E4M3 code times a power of two is exact in bf16, so with
    power-of-two scales the FP8 indexer must equal the (pinned) bf16 indexer
    on the bf16 encodings of the decoded, scaled values -- bit for bit, since
    both sum the same fp64 terms in the same order. Scales differ per
    (query, head) and per key, which pins the row each scale belongs to."""
    rng = np.random.default_rng(31 + H)
    n, L = 7, 45
    qc = _e4m3_codes(rng.standard_normal((n, H, D)) * 20)
    kc = _e4m3_codes(rng.standard_normal((L, D)) * 20)
    qs = np.ldexp(1.0, rng.integers(-6, 4, (n, H))).astype(np.float32)
    ks = np.ldexp(1.0, rng.integers(-6, 4, L)).astype(np.float32)
    w = rng.uniform(0, 1, (n, H)).astype(np.float32)
    p = rng.integers(0, L, n).astype(np.int32)
    got = oracle.indexer_seq_fp8(qc, qs, kc, ks, w, p)
    qv = _torch_e4m3(qc) * qs[:, :, None]
    kv = _torch_e4m3(kc) * ks[:, None]
    qb, kb = bf16_bits(qv), bf16_bits(kv)
    assert np.array_equal(oracle.bf16_bits_to_f64(qb), qv)      # the encodings are exact
    assert np.array_equal(oracle.bf16_bits_to_f64(kb), kv)
    ref = oracle.indexer_seq(qb, kb, w, p)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert (got[~np.isnan(got)] > 0).any() and (got[~np.isnan(got)] == 0).any()


def test_indexer_fp8_general_scales_brute_force():
    """Arbitrary positive scales: the FP8 indexer equals a numpy evaluation of
    sum_h w * max(0, (sq qc) . (sk kc)) on torch-decoded codes; scaling every
    key scale by c > 0 scales every score by c (the scale multiplies, once)."""
    rng = np.random.default_rng(77)
    n, H, D, L = 5, 4, 64, 33
    qc = _e4m3_codes(rng.standard_normal((n, H, D)) * 50)
    kc = _e4m3_codes(rng.standard_normal((L, D)) * 50)
    qs = rng.uniform(0.01, 3.0, (n, H)).astype(np.float32)
    ks = rng.uniform(0.01, 3.0, L).astype(np.float32)
    w = rng.uniform(0, 1, (n, H)).astype(np.float32)
    p = np.full(n, L - 1, np.int32)
    got = oracle.indexer_seq_fp8(qc, qs, kc, ks, w, p)
    qv = _torch_e4m3(qc) * qs.astype(np.float64)[:, :, None]
    kv = _torch_e4m3(kc) * ks.astype(np.float64)[:, None]
    dots = np.einsum("ihd,jd->ihj", qv, kv)
    ref = np.einsum("ih,ihj->ij", w.astype(np.float64), np.maximum(dots, 0.0))
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-9)
    c = np.float32(0.375)
    got_c = oracle.indexer_seq_fp8(qc, qs, kc, ks * c, w, p)
    np.testing.assert_allclose(got_c, got * np.float64(c), rtol=1e-6)


# -------------------------------------------------------------------- top-k --
def _brute_topk(s, p, k):
    cand = list(range(p + 1))
    if p + 1 <= k:
        keep = cand
    else:
        keep = sorted(sorted(cand, key=lambda j: (-float(s[j]), j))[:k])
    return keep + [-1] * (k - len(keep))


@pytest.mark.parametrize("kind", ["normal", "all_equal", "relu_zeros", "small_int", "signed_zero"])
def test_topk_matches_brute_force(kind):
    rng = np.random.default_rng(["normal", "all_equal", "relu_zeros", "small_int",
                                 "signed_zero"].index(kind))
    L, n = 97, 40
    if kind == "normal":
        s = rng.standard_normal((n, L)).astype(np.float32)
    elif kind == "all_equal":
        s = np.full((n, L), 3.25, np.float32)
    elif kind == "relu_zeros":
        s = np.maximum(rng.standard_normal((n, L)), 0).astype(np.float32)
    elif kind == "small_int":
        s = rng.integers(0, 4, (n, L)).astype(np.float32)
    else:
        s = np.where(rng.random((n, L)) < 0.5, np.float32(-0.0), np.float32(0.0))
        s[:, ::7] = 1.0
    p = rng.integers(0, L, n)
    for k in (1, 5, 16):
        got = oracle.topk_seq(s, p, k)
        for i in range(n):
            assert list(got[i]) == _brute_topk(s[i], int(p[i]), k), (kind, k, i)
    # k at the keep-all boundary: p, p+1, p+2
    for i in range(n):
        for k in (int(p[i]), int(p[i]) + 1, int(p[i]) + 2):
            if k < 1:
                continue
            got = oracle.topk_seq(s[i:i + 1], p[i:i + 1], k)[0]
            assert list(got) == _brute_topk(s[i], int(p[i]), k)


# ---------------------------------------------------------------- attention --
def _rand_seq(rng, n_heads, L, fmt="f64"):
    q = rng.standard_normal((L, n_heads, 576))
    kv = rng.standard_normal((L, 576))
    return q, kv


def test_dense_attention_matches_torch_sdpa():
    """Dense MQA attention equals torch SDPA (float64, CPU): K = the 576-dim
    latent row shared by all heads, V = its first 512 dims, causal mask j <= p."""
    rng = np.random.default_rng(1)
    L, H = 48, 3
    q, kv = _rand_seq(rng, H, L)
    p = np.arange(L)
    out, lse = oracle.attention_seq(q, kv, p, SM, q_fmt=FMT_F64, kv_fmt=FMT_F64)
    Q = torch.from_numpy(q).permute(1, 0, 2)                  # [H, L, 576]
    K = torch.from_numpy(kv)[None].expand(H, L, 576)
    V = torch.from_numpy(kv[:, :512])[None].expand(H, L, 512)
    mask = torch.from_numpy(np.arange(L)[None, :] <= p[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=SM)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_absorbed_equals_explicit_mla():
    """Absorbed form (one 576-dim latent row for all heads) equals per-head K/V
    up-projection: Q = [W_UK^T qn ; qr], O = W_UV . O_latent."""
    rng = np.random.default_rng(2)
    L, H = 20, 4
    c = rng.standard_normal((L, 512))
    r = rng.standard_normal((L, 64))
    W_UK = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    W_UV = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    qn = rng.standard_normal((L, H, 128))
    qr = rng.standard_normal((L, H, 64))
    p = np.arange(L)
    ref_o, ref_lse = oracle.explicit_mla(qn, qr, c, r, W_UK, W_UV, p, SM)
    Q = np.concatenate([np.einsum("hdc,ihd->ihc", W_UK, qn), qr], axis=2)
    KV = np.concatenate([c, r], axis=1)
    o_lat, lse = oracle.attention_seq(Q, KV, p, SM, q_fmt=FMT_F64, kv_fmt=FMT_F64)
    o = np.einsum("hdc,ihc->ihd", W_UV, o_lat)
    np.testing.assert_allclose(o, ref_o, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-9, atol=1e-12)


def test_keep_all_topk_makes_sparse_equal_dense_exactly():
    rng = np.random.default_rng(3)
    L, H = 64, 2
    q, kv = _rand_seq(rng, H, L)
    p = np.arange(L)
    scores = rng.standard_normal((L, L)).astype(np.float32)
    idx = oracle.topk_seq(scores, p, L)
    a = oracle.attention_seq(q, kv, p, SM, indices=idx, q_fmt=FMT_F64, kv_fmt=FMT_F64)
    b = oracle.attention_seq(q, kv, p, SM, q_fmt=FMT_F64, kv_fmt=FMT_F64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_weights_sum_to_one_and_lse_merge():
    """(a) rows with one shared latent part u and random rope parts give
    O = (sum_j p_j) u, so O / u == 1; (b) splitting the selected set into two
    halves, or into eight round-robin shards, and merging the parts with
    oracle.merge_lse reproduces the full result."""
    rng = np.random.default_rng(4)
    L, H = 40, 2
    q, kv = _rand_seq(rng, H, L)
    p = np.arange(L)
    kv1 = kv.copy()
    u = rng.uniform(1, 2, 512)
    kv1[:, :512] = u
    o, _ = oracle.attention_seq(q, kv1, p, SM, q_fmt=FMT_F64, kv_fmt=FMT_F64)
    np.testing.assert_allclose(o / u, 1.0, rtol=1e-12)

    full_o, full_l = oracle.attention_seq(q, kv, p, SM, q_fmt=FMT_F64, kv_fmt=FMT_F64)
    even = np.full((L, L), -1, np.int32)
    odd = np.full((L, L), -1, np.int32)
    for i in range(L):
        e = list(range(0, i + 1, 2))
        o_ = list(range(1, i + 1, 2))
        even[i, : len(e)] = e
        odd[i, : len(o_)] = o_
    oa, la = oracle.attention_seq(q, kv, p, SM, indices=even, q_fmt=FMT_F64, kv_fmt=FMT_F64)
    ob, lb = oracle.attention_seq(q, kv, p, SM, indices=odd, q_fmt=FMT_F64, kv_fmt=FMT_F64)
    assert np.isneginf(lb[0]).all() and (ob[0] == 0).all()     # empty half: O = 0, LSE = -inf
    om, Lm = oracle.merge_lse([oa, ob], [la, lb])
    np.testing.assert_allclose(Lm, full_l, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(om, full_o, rtol=1e-10, atol=1e-13)
    # eight round-robin key shards (row j on shard j mod 8), most rows with
    # some empty shards, merge back to the full result too
    parts = []
    for r in range(8):
        ind = np.full((L, L), -1, np.int32)
        for i in range(L):
            sel = list(range(r, i + 1, 8))
            ind[i, : len(sel)] = sel
        parts.append(oracle.attention_seq(q, kv, p, SM, indices=ind, q_fmt=FMT_F64, kv_fmt=FMT_F64))
    om8, Lm8 = oracle.merge_lse([o_ for o_, _ in parts], [l_ for _, l_ in parts])
    np.testing.assert_allclose(Lm8, full_l, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(om8, full_o, rtol=1e-10, atol=1e-13)
    # every part empty: O = 0, LSE = -inf
    oz, lz = oracle.merge_lse([ob[:1], ob[:1]], [lb[:1], lb[:1]])
    assert (oz == 0).all() and np.isneginf(lz).all()


def test_closed_forms_first_row_and_identical_rows():
    """p = 0: O = K_0[:512], LSE = z_0. All rows equal: O = that row and
    LSE = z + ln|S|. Integer data make z exact: z = sm_scale * integer dot."""
    rng = np.random.default_rng(5)
    L, H = 16, 3
    q = rng.integers(-3, 4, (L, H, 576)).astype(np.float64)
    kv = rng.integers(-3, 4, (L, 576)).astype(np.float64)
    o, lse = oracle.attention_seq(q, kv, np.zeros(L, int), SM, q_fmt=FMT_F64, kv_fmt=FMT_F64)
    for i in range(L):
        for h in range(H):
            z0 = SM * int(np.dot(q[i, h].astype(np.int64), kv[0].astype(np.int64)))
            assert o[i, h].tolist() == kv[0, :512].tolist()
            assert abs(lse[i, h] - z0) <= 1e-12 * max(1.0, abs(z0))
    same = np.repeat(kv[3:4], L, axis=0)
    p = np.arange(L)
    o, lse = oracle.attention_seq(q, same, p, SM, q_fmt=FMT_F64, kv_fmt=FMT_F64)
    for i in range(L):
        for h in range(H):
            z = SM * int(np.dot(q[i, h].astype(np.int64), kv[3].astype(np.int64)))
            np.testing.assert_allclose(o[i, h], kv[3, :512], rtol=1e-12)
            assert abs(lse[i, h] - (z + math.log(i + 1))) <= 1e-11 * max(1.0, abs(z))


def test_fp8_rows_decode_with_scale():
    """An FP8 row is decode(code) * sigma: attention on (codes, sigma) equals
    attention on the explicitly decoded float64 rows."""
    rng = np.random.default_rng(6)
    L, H = 24, 2
    q = bf16_bits(rng.standard_normal((L, H, 576)))
    x = torch.from_numpy(rng.standard_normal((L, 576)).astype(np.float32))
    codes, sigma = mla_inputs.quantize_e4m3_rows(x)
    dec = torch.from_numpy(codes.numpy()).view(torch.float8_e4m3fn).double().numpy() * \
        sigma.numpy().astype(np.float64)[:, None]
    p = np.arange(L)
    a = oracle.attention_seq(q, codes.numpy(), p, SM, kv_scale=sigma.numpy(), kv_fmt=FMT_E4M3)
    b = oracle.attention_seq(q, dec, p, SM, kv_fmt=FMT_F64)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-14, atol=1e-15)


def test_fp8_quantisation_gap_exceeds_the_fp8_tolerance():
    """The oracle's FP8-KV output against its unquantised (bf16) KV output on
    the same fp32 draw: the gap is input quantisation (E4M3 keeps about 2^-4
    of each value), larger for queries that average few rows. Its maximum is
    above the FP8 attention tolerance (6e-2), so the GPU must be, and is,
    compared with the oracle on the same FP8 bytes: a path that read the
    wrong KV form would fail the comparison. (A scratch draw of this shape:
    mean 0.010, max 0.21.)"""
    rng = np.random.default_rng(41)
    L, H = 256, 8
    q = bf16_bits(rng.standard_normal((L, H, 576)))
    x = torch.from_numpy(rng.standard_normal((L, 576)).astype(np.float32))
    codes, sigma = mla_inputs.quantize_e4m3_rows(x)
    p = np.arange(L)
    o8, l8 = oracle.attention_seq(q, codes.numpy(), p, SM, kv_scale=sigma.numpy(), kv_fmt=FMT_E4M3)
    ob, lb = oracle.attention_seq(q, bf16_bits(x.numpy()), p, SM, kv_fmt=FMT_BF16)
    gap = np.abs(o8.astype(np.float64) - ob.astype(np.float64))
    assert 1e-3 < gap.mean() < 3e-2
    assert gap.max() > 6e-2
    assert gap[L // 2:].mean() < gap[:8].mean()                           # averaging shrinks it
    assert np.abs(l8 - lb).max() < 0.25                                   # the LSE moves less


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8", "ds656"])
def test_attention_gates_reject_a_dropped_key_block(kv_dtype):
    """The attention parity gates catch a kernel that skips keys: 16 queries x
    64 heads near position 4,095 attend to 2,048 random earlier keys; the same
    attention with one 32-key block of each list left out (entries 1,024 ..
    1,055) misses the LSE gate on most (query, head) pairs. Its output moves
    far less, so the O gate alone would catch it only now and then."""
    import tolerances as tl
    rng = np.random.default_rng(77)
    L, H, n, k = 4096, 64, 16, 2048
    q = bf16_bits(rng.standard_normal((n, H, 576)))
    x = rng.standard_normal((L, 576)).astype(np.float32)
    if kv_dtype == "fp8":
        codes, sigma = mla_inputs.quantize_e4m3_rows(torch.from_numpy(x))
        kv, kv_scale, fmt = codes.numpy(), sigma.numpy(), FMT_E4M3
    elif kv_dtype == "ds656":
        kv, kv_scale, fmt = mla_inputs.pack_ds656_rows(torch.from_numpy(x)).numpy(), None, FMT_DS656
    else:
        kv, kv_scale, fmt = bf16_bits(x), None, FMT_BF16
    p = np.arange(L - n, L)
    idx = np.stack([np.sort(rng.choice(pi + 1, k, replace=False)) for pi in p]).astype(np.int32)
    dropped = idx.copy()
    dropped[:, 1024:1056] = -1
    o, l = oracle.attention_seq(q, kv, p, SM, kv_scale=kv_scale, indices=idx, kv_fmt=fmt)
    od, ld = oracle.attention_seq(q, kv, p, SM, kv_scale=kv_scale, indices=dropped, kv_fmt=fmt)
    lse_bad = tl.outside(ld, l, *tl.LSE_TOL[kv_dtype])
    tol = tl.OUT_TOL[kv_dtype]
    out_bad = tl.outside(od, o, tol, tol)
    shift = np.abs(ld - l)
    assert 0.01 < shift.mean() < 0.03                     # about 32/2048 of the mass
    assert lse_bad.mean() > (0.1 if kv_dtype == "ds656" else 0.6), lse_bad.mean()
    assert out_bad.mean() < 0.1                           # the O gate alone is much weaker
    # the undropped lists pass both gates against themselves rounded like
    # the kernel's outputs (bf16 O, fp32 LSE)
    o_b = torch.from_numpy(o).to(torch.bfloat16).double().numpy()
    assert not tl.outside(o_b, o, tol, tol).any()
    assert not tl.outside(l.astype(np.float32), l, *tl.LSE_TOL[kv_dtype]).any()


def _torch_decode_ds656(rows: np.ndarray) -> np.ndarray:
    """656-byte rows decoded with torch's own float8 / float32 / bf16 views of
    the bytes (not the oracle's decoders): [N, 576] float64."""
    t = torch.from_numpy(np.ascontiguousarray(rows))
    n = t.shape[0]
    codes = t[:, :512].contiguous().view(torch.float8_e4m3fn).double().reshape(n, 4, 128)
    scales = t[:, 512:528].contiguous().view(torch.float32).double()
    rope = t[:, 528:656].contiguous().view(torch.bfloat16).double()
    return torch.cat([(codes * scales[:, :, None]).reshape(n, 512), rope], dim=1).numpy()


def test_ds656_rows_decode_with_tile_scales():
    """A 656-byte row decodes as code * (the scale of its 128-value tile) for
    the latent values and bf16 for the rope: attention on the rows equals
    attention on the rows decoded independently through torch's views."""
    rng = np.random.default_rng(61)
    L, H = 40, 3
    x = rng.standard_normal((L, 576)).astype(np.float32)
    x[:, 128:256] *= 30.0                                  # tiles of very different ranges
    x[:, 384:512] *= 0.01
    x[5, :128] = 0.0                                       # an all-zero tile: scale 1
    rows = mla_inputs.pack_ds656_rows(torch.from_numpy(x)).numpy()
    assert rows.shape == (L, 656)
    q = bf16_bits(rng.standard_normal((L, H, 576)))
    p = np.arange(L)
    a = oracle.attention_seq(q, rows, p, SM, kv_fmt=FMT_DS656)
    b = oracle.attention_seq(q, _torch_decode_ds656(rows), p, SM, kv_fmt=FMT_F64)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-14, atol=1e-15)
    # each tile's relative quantisation error stays within E4M3's 2^-4
    dec = _torch_decode_ds656(rows)
    big = np.abs(x[:, :512]) > 0.05 * np.abs(x[:, :512]).max(axis=1, keepdims=True)
    assert (np.abs(dec[:, :512] - x[:, :512])[big] <= 2.0 ** -4 * np.abs(x[:, :512])[big]).all()


def test_ds656_closed_form_row():
    """A hand-built row: every latent code 0x38 (1.0), tile scales 1, 2, 0.25
    and 8, every rope value bf16 0.5 (0x3f00). A query at position 0 attends
    to that one row: O is its 512 latent values exactly, and the LSE is the
    logit sm_scale * q . K, exact for small-integer queries."""
    row = np.zeros(656, np.uint8)
    row[:512] = 0x38
    row[512:528] = np.array([1.0, 2.0, 0.25, 8.0], np.float32).view(np.uint8)
    row[528:656] = np.full(64, 0x3f00, np.uint16).view(np.uint8)
    K = np.concatenate([np.full(128, 1.0), np.full(128, 2.0), np.full(128, 0.25),
                        np.full(128, 8.0), np.full(64, 0.5)])
    q = np.random.default_rng(62).integers(-3, 4, (1, 2, 576)).astype(np.float64)
    o, lse = oracle.attention_seq(q, row[None], np.zeros(1, np.int32), SM, q_fmt=FMT_F64,
                                  kv_fmt=FMT_DS656)
    for h in range(2):
        assert o[0, h].tolist() == K[:512].tolist()
        assert lse[0, h] == pytest.approx(SM * float(q[0, h] @ K), rel=1e-15)


def test_ds656_gate_covers_the_bf16_decode():
    """The 656-byte path's LSE gate (2e-2 + 1e-4 |r|) is derived from its
    arithmetic: rows decoded to bf16, bf16(code * scale). Attention on those
    bf16-rounded rows against the exact rows, 8 heads, every position of a
    1,024-token causal sequence: the LSE moves by under 40 % of the gate
    (7.8e-3 at most on this draw, about 3 standard deviations of the logit
    error), and the outputs stay within a quarter of the FP8-KV output
    tolerance."""
    import tolerances as tl
    rng = np.random.default_rng(63)
    L, H = 1024, 8
    x = torch.from_numpy(rng.standard_normal((L, 576)).astype(np.float32))
    exact = _torch_decode_ds656(mla_inputs.pack_ds656_rows(x).numpy())
    rounded = torch.from_numpy(exact).to(torch.bfloat16).double().numpy()
    q = bf16_bits(rng.standard_normal((L, H, 576)))
    p = np.arange(L)
    o1, l1 = oracle.attention_seq(q, exact, p, SM, kv_fmt=FMT_F64)
    o2, l2 = oracle.attention_seq(q, rounded, p, SM, kv_fmt=FMT_F64)
    atol, rtol = tl.LSE_TOL["ds656"]
    assert (np.abs(l2 - l1) <= 0.4 * (atol + rtol * np.abs(l1))).all()
    assert np.abs(l2 - l1).max() > tl.LSE_ATOL           # the fp32 gate would not hold here
    assert np.abs(o2 - o1).max() < 0.25 * tl.OUT_TOL["ds656"]


# ----------------------------------------------------- batch-level invariants --
def _small_batch(kv_lens, q_ranges, H=2, HI=2, DI=16, k=8, kv_dtype="bf16", seed=9):
    wl = mla_inputs.Workload("t", tuple(kv_lens), tuple(tuple(r) for r in q_ranges), n_heads=H,
                             idx_heads=HI, idx_dim=DI, topk=k, kv_dtype=kv_dtype, seed=seed)
    return mla_inputs.make_inputs(wl, "cpu")


def _run_path(batch, rows):
    """indexer -> top-k -> attention for the given rows, all in the oracle."""
    wl = batch["workload"]
    sc = oracle.indexer_rows(batch, rows)
    idx = oracle.topk_rows(sc, batch["q_pos_host"][rows], wl.topk)
    return idx, oracle.attention_rows(batch, rows, idx)


def test_cp_16_chunk_split_reassembles_and_balances():
    """Rank r of 8 computes chunks r and 15-r of a 16-chunk prompt (true
    positions) against the full KV; scattered back, the 8 shares equal the
    unsplit run exactly, and every rank has the same number of causal pairs."""
    L = 256
    full = _small_batch([L], [[(0, L)]])
    all_rows = np.arange(L)
    idx_full, (o_full, l_full) = _run_path(full, all_rows)
    o = np.zeros_like(o_full)
    l = np.zeros_like(l_full)
    pairs = []
    for r in range(8):
        ranges = mla_inputs.cp_share_ranges(L, 8, r)
        share = _small_batch([L], [ranges])
        # same tensors as the full run, restricted to this rank's queries
        pos = share["q_pos_host"]
        for key in ("q", "q_idx", "w"):
            share[key] = full[key][torch.from_numpy(pos.astype(np.int64))]
        share["kv"], share["k_idx"] = full["kv"], full["k_idx"]
        idx_r, (o_r, l_r) = _run_path(share, np.arange(len(pos)))
        o[pos], l[pos] = o_r, l_r
        assert np.array_equal(idx_r, idx_full[pos])
        pairs.append(int((pos + 1).sum()))
    assert np.array_equal(o, o_full) and np.array_equal(l, l_full)
    assert len(set(pairs)) == 1


def test_prefix_resume_equals_tail_of_full_prefill():
    L, cached = 96, 64
    full = _small_batch([L], [[(0, L)]])
    resume = _small_batch([L], [[(cached, L)]])
    tail = torch.arange(cached, L)
    for key in ("q", "q_idx", "w"):
        resume[key] = full[key][tail]
    resume["kv"], resume["k_idx"] = full["kv"], full["k_idx"]
    i_full, (o_full, l_full) = _run_path(full, np.arange(L))
    i_res, (o_res, l_res) = _run_path(resume, np.arange(L - cached))
    assert np.array_equal(i_res, i_full[cached:])
    assert np.array_equal(o_res, o_full[cached:]) and np.array_equal(l_res, l_full[cached:])


def test_ragged_batch_equals_concatenated_sequences():
    lens = [40, 0, 77, 13]
    ranges = [[(0, 40)], [], [(20, 77)], [(0, 5), (10, 13)]]
    batch = _small_batch(lens, ranges, kv_dtype="fp8")
    rows = np.arange(batch["workload"].total_q)
    idx_b, (o_b, l_b) = _run_path(batch, rows)
    cu_q, cu_kv = batch["cu_seqlens_q_host"], batch["cu_seqlens_kv_host"]
    for b in range(len(lens)):
        r = np.arange(cu_q[b], cu_q[b + 1])
        if not len(r):
            continue
        one = _small_batch([lens[b]], [ranges[b]], kv_dtype="fp8")
        for key in ("q", "q_idx", "w"):
            one[key] = batch[key][torch.from_numpy(r)]
        sl = slice(int(cu_kv[b]), int(cu_kv[b + 1]))
        one["kv"], one["kv_scale"], one["k_idx"] = batch["kv"][sl], batch["kv_scale"][sl], \
            batch["k_idx"][sl]
        i1, (o1, l1) = _run_path(one, np.arange(len(r)))
        assert np.array_equal(i1, idx_b[r])
        assert np.array_equal(o1, o_b[r]) and np.array_equal(l1, l_b[r])


def test_planted_needle_is_selected_and_dominates():
    """A key whose indexer key aligns with every query's indexer heads must be
    in every later query's top-k (a synthetic stand-in for a needle prompt)."""
    L, H = 128, 2
    batch = _small_batch([L], [[(0, L)]], H=H, HI=2, DI=16, k=8)
    needle = 37
    qI = batch["q_idx"].float()
    kI = batch["k_idx"].float()
    kI[needle] = 4.0 * torch.sign(qI.mean(dim=(0, 1)))
    batch["k_idx"] = kI.to(torch.bfloat16)
    batch["q_idx"] = (qI.abs() * torch.sign(qI.mean(dim=(0, 1)))).to(torch.bfloat16)
    rows = np.arange(needle, L)
    sc = oracle.indexer_rows(batch, rows)
    idx = oracle.topk_rows(sc, batch["q_pos_host"][rows], 8)
    assert all(needle in set(r) for r in idx)


# -------------------------------------------------- the pages' own arithmetic --
def test_footnote_arithmetic_golden():
    g = json.load(open(os.path.join(GOLDEN, "footnote_arithmetic.json")))
    f1 = g["footnote_1"]
    assert bench.attn_flop_per_pair(1) == f1["flop_per_row_head"]
    assert 2 * (f1["qk_dims"] + f1["pv_dims"]) == f1["flop_per_row_head"]
    assert 2 * (f1["qk_dims"] + f1["pv_dims"]) == f1["qo_bytes_per_head"]
    assert round(f1["topk"] * f1["row_bytes"] / 1e6, 2) == f1["row_bytes_per_query_MB"]
    for h in (8, 64):
        ref = f1["heads_%d" % h]
        flop = bench.attn_flop_per_pair(h) * f1["topk"]
        byt = bench.sparse_query_bytes(h, f1["topk"], f1["row_bytes"])
        # printed to 3 significant figures: 285 and 35.7 MFLOP
        assert abs(flop / 1e6 - ref["MFLOP"]) <= 0.005 * ref["MFLOP"]
        assert round(byt / 1e6, 2) == ref["MB"]
        assert round(flop / byt) == ref["flop_per_byte"]
    assert bench.attn_flop_per_pair(64) * 2048 == 285_212_672
    assert bench.attn_flop_per_pair(8) * 2048 == 35_651_584
    f3 = g["footnote_3"]
    per_tok = bench.kv_bytes_per_token(f3["mla_layers"], f3["mla_row_bytes"], f3["indexer_layers"],
                                       f3["indexer_key_bytes"], f3["mtp_bytes"])
    assert per_tok == f3["total_bytes_per_token"]
    assert round(per_tok * f3["tokens"] / 2 ** 30, 1) == f3["total_GiB"]
    assert round(per_tok * f3["tokens"] / 2 ** 30 / 8, 1) == f3["per_gpu_GiB_8way"]
    # a 256-token cache chunk of 78 FP8 MLA layers is the ~12.4 MB the B300 post quotes
    assert round(78 * 656 * 256 / 2 ** 20, 1) == 12.5


def test_workload_shapes_match_their_descriptions():
    W = mla_inputs.WORKLOADS
    assert W["cp131k"].q_pos_ranges == (((0, 8192), (122880, 131072)),)
    rg = W["ragged"]
    assert list(rg.cu_seqlens_kv()) == [0, 9472, 44032, 113408, 316160]
    assert list(rg.cu_seqlens_q()) == [0, 512, 2560, 6656, 12800]
    assert all(c % 256 == 0 for c in (8960, 32512, 65280, 196608))
    f = bench.workload_flops(W["sparse32k"])
    assert f["causal"] == 32768 * 32769 // 2
    assert abs(f["indexer"] / 1e12 - 8.80) < 0.01 and abs(f["attention"] / 1e12 - 9.05) < 0.01
    assert abs(bench.workload_flops(W["dense16k"])["attention"] / 1e12 - 18.69) < 0.01
