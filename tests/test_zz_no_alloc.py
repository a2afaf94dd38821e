"""mla_sparse_prefill_split_noalloc: the split-KV call with its parts in the
library's own per-GPU scratch array instead of a caller workspace (for callers
that cannot allocate). Its output must equal the workspace form's bit for bit
(same kernels, same parts), call after call, with the array reused."""
import numpy as np
import pytest
import torch

import mla_inputs
import oracle
import tolerances as tl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_long_amd as sm
    sm.load_library()
    return sm


def _tail_of_32k():
    """The last 64 queries of the 32k workload, FP8 KV, top-2,048 lists."""
    wl = mla_inputs.WORKLOADS["sparse32k"]
    tail = mla_inputs.Workload("tail64", (32768,), (((32704, 32768),),), n_heads=64, idx_heads=64,
                               idx_dim=128, topk=2048, kv_dtype="fp8", seed=wl.seed)
    return mla_inputs.make_inputs(tail, "cuda")


def _few_queries(kv_dtype, seed):
    wl = mla_inputs.Workload("split", (700, 1, 2500), (((0, 6), (690, 700)), ((0, 1),),
                                                      ((0, 2), (2480, 2500))),
                             n_heads=64, idx_heads=4, idx_dim=64, topk=96, kv_dtype=kv_dtype, seed=seed)
    inp = mla_inputs.make_inputs(wl, "cpu")
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _lists(sm, inp):
    batch = sm.Batch.from_inputs(inp)
    sc = sm.indexer_score(batch, inp["q_idx"], inp["k_idx"], inp["w"])
    return batch, sm.topk_select(batch, sc, inp["workload"].topk)


def _both(sm, inp, batch, idx, n_split):
    wl = inp["workload"]
    o1, l1 = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale,
                               n_split=n_split)
    o2, l2 = sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale,
                               n_split=n_split, noalloc=True)
    torch.cuda.synchronize()
    return o1, l1, o2, l2


def test_noalloc_split_equals_workspace_split(sm):
    """Two calls in a row, the second on a smaller batch: (1) 64 queries x 64
    heads in 4 parts, which fills the scratch array exactly; (2) 39 queries in
    3 parts, bf16 KV, dense. Each equals the workspace form bit for bit, and
    the first matches the oracle on sampled rows."""
    L = sm.load_library()
    inp = _tail_of_32k()
    batch, idx = _lists(sm, inp)
    assert L.mla_sparse_prefill_split_workspace_size(64, 64, 4) == 16 * 1024 * 1024 + 64 * 1024
    o1, l1, o2, l2 = _both(sm, inp, batch, idx, 4)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    rows = np.array([0, 31, 63])
    rt = torch.as_tensor(rows, device="cuda")
    r_out, r_lse = oracle.attention_rows(inp, rows, idx[rt].cpu().numpy())
    tl.assert_attention("noalloc tail64", "fp8", o2[rt].float().cpu().numpy(),
                        l2[rt].cpu().numpy(), r_out, r_lse)

    small = _few_queries("bf16", 91)
    sb = sm.Batch.from_inputs(small)
    wl = small["workload"]
    o1, l1 = sm.sparse_prefill(sb, small["q"], small["kv"], None, None, wl.sm_scale, n_split=3)
    o2, l2 = sm.sparse_prefill(sb, small["q"], small["kv"], None, None, wl.sm_scale, n_split=3,
                               noalloc=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    r_out, r_lse = oracle.attention_rows(small, np.arange(wl.total_q), None)
    tl.assert_attention("noalloc few", "bf16", o2.float().cpu().numpy(), l2.cpu().numpy(),
                        r_out, r_lse)


def test_noalloc_split_rejects_parts_beyond_the_array(sm):
    """Parts that need more than MLA_SPLIT_SCRATCH_BYTES: MLA_ERR_UNSUPPORTED,
    nothing enqueued (the outputs keep their sentinel); a later fitting call on
    the same batch still works. n_split = 1 needs no array at all."""
    inp = _tail_of_32k()
    batch, idx = _lists(sm, inp)
    wl = inp["workload"]
    out = torch.full((64, 64, 512), -3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((64, 64), -3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(sm.MlaError) as e:
        sm.sparse_prefill(batch, inp["q"], inp["kv"], inp["kv_scale"], idx, wl.sm_scale,
                          out=out, lse=lse, n_split=5, noalloc=True)
    assert e.value.status == sm.MLA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (out.float() == -3.0).all() and (lse == -3.0).all()
    o1, l1, o2, l2 = _both(sm, inp, batch, idx, 2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o1, l1, o2, l2 = _both(sm, inp, batch, idx, 1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
