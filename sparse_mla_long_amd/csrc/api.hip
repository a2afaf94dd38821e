// C ABI of the sparse-MLA prefill library: host-side validation and launch.
//
// Every check runs on the host before the first HIP call, so a rejected call
// enqueues nothing and touches no device. Device data (q_pos, indices) is
// trusted; kernels clamp positions into their sequence so a bad q_pos cannot
// read outside the sequence's rows.
#include <algorithm>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string>

#include "kernels.h"
#include "mla_sparse.h"

namespace {

thread_local std::string g_last_error;

mla_status_t fail(mla_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
mla_status_t fail(mla_status_t s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

mla_status_t ok() {
    g_last_error.clear();
    return MLA_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Validates the batch description; on success fills the device view.
mla_status_t check_batch(const mla_batch_t *b, mla::BatchDev *dev) {
    if (!b) return fail(MLA_ERR_INVALID_ARG, "batch is NULL");
    if (b->num_seqs < 1) return fail(MLA_ERR_INVALID_ARG, "num_seqs must be >= 1 (got %d)", b->num_seqs);
    if (b->total_q < 0 || b->total_kv < 0 || b->max_kv_len < 0)
        return fail(MLA_ERR_INVALID_ARG, "negative total_q / total_kv / max_kv_len");
    if (!b->cu_seqlens_q_host || !b->cu_seqlens_kv_host)
        return fail(MLA_ERR_INVALID_ARG, "host cu_seqlens are NULL");
    const int32_t *cq = b->cu_seqlens_q_host, *ck = b->cu_seqlens_kv_host;
    if (cq[0] != 0 || ck[0] != 0) return fail(MLA_ERR_INVALID_ARG, "cu_seqlens must start at 0");
    int32_t max_len = 0;
    for (int32_t s = 0; s < b->num_seqs; ++s) {
        if (cq[s + 1] < cq[s] || ck[s + 1] < ck[s])
            return fail(MLA_ERR_INVALID_ARG, "cu_seqlens decrease at sequence %d", s);
        const int32_t nq = cq[s + 1] - cq[s], nk = ck[s + 1] - ck[s];
        if (nq > 0 && nk == 0)
            return fail(MLA_ERR_INVALID_ARG, "sequence %d has queries but no KV rows", s);
        if (nk > max_len) max_len = nk;
    }
    if (cq[b->num_seqs] != b->total_q || ck[b->num_seqs] != b->total_kv)
        return fail(MLA_ERR_INVALID_ARG, "cu_seqlens end at (%d, %d), totals are (%d, %d)",
                    cq[b->num_seqs], ck[b->num_seqs], b->total_q, b->total_kv);
    if (b->max_kv_len != max_len)
        return fail(MLA_ERR_INVALID_ARG, "max_kv_len is %d, longest sequence has %d rows",
                    b->max_kv_len, max_len);
    if (b->total_q > 0 && (!b->cu_seqlens_q || !b->cu_seqlens_kv || !b->q_pos))
        return fail(MLA_ERR_INVALID_ARG, "device cu_seqlens / q_pos are NULL");
    dev->cu_q = b->cu_seqlens_q;
    dev->cu_kv = b->cu_seqlens_kv;
    dev->q_pos = b->q_pos;
    dev->num_seqs = b->num_seqs;
    dev->total_q = b->total_q;
    return MLA_OK;
}

mla_status_t hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Library-owned workspace of mla_sparse_prefill_split_noalloc (the parts'
// outputs and LSEs between its two launches). Every GPU the library runs on
// holds its own copy until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: host code uses only the device
// address taken once per device with hipGetSymbolAddress below.
static __device__ __align__(256) uint8_t scratch[MLA_SPLIT_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};   // device address of `scratch` per device, once taken

// Device address of the current device's `scratch`, looked up on the first
// call on that device (with it current) and kept.
mla_status_t scratch_of_current_device(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MLA_ERR_UNSUPPORTED, "device %d: the scratch table holds %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MLA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *ptr = g_scratch_dev[dev];
    return MLA_OK;
}

}  // namespace

extern "C" {

namespace {
// Eight-query indexer blocks of a (validated) batch.
int64_t indexer_blocks(const mla_batch_t *batch) {
    int64_t blocks = 0;
    for (int32_t s = 0; s < batch->num_seqs; ++s) {
        const int32_t nq = batch->cu_seqlens_q_host[s + 1] - batch->cu_seqlens_q_host[s];
        blocks += (nq + mla::kIdxQueriesPerBlock - 1) / mla::kIdxQueriesPerBlock;
    }
    return blocks;
}

// Few query blocks (a short chunk behind a long prefix): split every block's
// keys over several workgroups, about two per CU in all, down to one key tile
// each. Each score is still computed once.
int32_t indexer_key_split(const mla_batch_t *batch, int64_t blocks) {
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        n_cu = 1;
    int64_t split = 1;
    if (blocks > 0 && blocks < 2 * (int64_t)n_cu) {
        split = (2 * (int64_t)n_cu + blocks - 1) / blocks;
        split = std::min<int64_t>(split, ((int64_t)batch->max_kv_len + mla::kIdxKeyTile - 1) / mla::kIdxKeyTile);
        split = std::max<int64_t>(split, 1);
    }
    return (int32_t)split;
}

// Workspace of the fused indexer + top-k: candidate lists of
// cand_capacity(k) (key, j) entries per (query, key part), then the lists'
// lengths.
size_t cand_list_bytes(int64_t total_q, int64_t parts, int64_t k) {
    return ((size_t)(total_q * parts * mla::cand_capacity(k)) * 8 + 255) / 256 * 256;
}
size_t topk_ws_bytes(int64_t total_q, int64_t parts, int64_t k) {
    return cand_list_bytes(total_q, parts, k) + (size_t)(total_q * parts) * 4;
}

// Shared checks and launch of the indexer entry points (scales are NULL for
// bf16). topk > 0: the fused form, which writes indices instead of scores
// and keeps its candidate lists in the workspace.
mla_status_t indexer(const mla_batch_t *batch, const void *q_idx, const float *q_scale,
                     const void *k_idx, const float *k_scale, const float *w, int32_t n_heads,
                     int32_t head_dim, float *scores, int64_t ld_scores, bool fp8, void *stream,
                     int32_t topk = 0, int32_t *indices = nullptr, void *workspace = nullptr,
                     size_t workspace_bytes = 0) {
    mla::IndexerArgs a{};
    mla_status_t st = check_batch(batch, &a.batch);
    if (st != MLA_OK) return st;
    const bool fused = topk != 0;
    if (n_heads < 1) return fail(MLA_ERR_INVALID_ARG, "n_heads must be >= 1 (got %d)", n_heads);
    if (head_dim < 1) return fail(MLA_ERR_INVALID_ARG, "head_dim must be >= 1 (got %d)", head_dim);
    if (fused && topk < 1) return fail(MLA_ERR_INVALID_ARG, "k must be >= 1 (got %d)", topk);
    if (n_heads > 64) return fail(MLA_ERR_UNSUPPORTED, "indexer n_heads %d > 64", n_heads);
    if (head_dim != 64 && head_dim != 128)
        return fail(MLA_ERR_UNSUPPORTED, "indexer head_dim %d not in {64, 128}", head_dim);
    if (fused && topk > 4096) return fail(MLA_ERR_UNSUPPORTED, "k %d > 4096", topk);
    if (!fused && ld_scores < batch->max_kv_len)
        return fail(MLA_ERR_INVALID_ARG, "ld_scores %lld < max_kv_len %d", (long long)ld_scores,
                    batch->max_kv_len);
    if (batch->total_q == 0) return ok();
    if (!q_idx || !k_idx || !w || (fused ? !indices : !scores))
        return fail(MLA_ERR_INVALID_ARG, "q_idx / k_idx / w / %s is NULL", fused ? "indices" : "scores");
    if (fp8 && (!q_scale || !k_scale))
        return fail(MLA_ERR_INVALID_ARG, "q_scale / k_scale is NULL");
    if (!aligned(q_idx, 16) || !aligned(k_idx, 16))
        return fail(MLA_ERR_INVALID_ARG, "q_idx and k_idx must be 16-byte aligned");
    if (!aligned(w, 4) || (fused ? !aligned(indices, 4) : !aligned(scores, 4)))
        return fail(MLA_ERR_INVALID_ARG, "w and %s must be 4-byte aligned", fused ? "indices" : "scores");
    if (fp8 && (!aligned(q_scale, 4) || !aligned(k_scale, 4)))
        return fail(MLA_ERR_INVALID_ARG, "q_scale and k_scale must be 4-byte aligned");
    const int64_t blocks = indexer_blocks(batch);
    const int32_t split = indexer_key_split(batch, blocks);
    if (fused) {
        const size_t need = topk_ws_bytes(batch->total_q, split, topk);
        if (!workspace) return fail(MLA_ERR_INVALID_ARG, "workspace is NULL");
        if (!aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
        if (workspace_bytes < need)
            return fail(MLA_ERR_INVALID_ARG, "workspace_bytes %zu < %zu (mla_topk_workspace_size)",
                        workspace_bytes, need);
        a.topk = topk;
        a.cand = (uint2 *)workspace;
        a.cand_cap = (int32_t)mla::cand_capacity(topk);
        a.cand_n = (int32_t *)((uint8_t *)workspace + cand_list_bytes(batch->total_q, split, topk));
    }
    a.q_idx = q_idx;
    a.k_idx = k_idx;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.w = w;
    a.scores = scores;
    a.ld = ld_scores;
    a.n_heads = n_heads;
    a.head_dim = head_dim;
    a.key_split = split;
    a.n_blocks = (int32_t)(blocks * split);
    a.fp8 = fp8;
    st = hip_status(mla::launch_indexer(a, (hipStream_t)stream), "indexer launch");
    if (st != MLA_OK || !fused) return st;
    mla::CandSelectArgs m{};
    m.batch = a.batch;
    m.cand = a.cand;
    m.cand_n = a.cand_n;
    m.cand_cap = a.cand_cap;
    m.n_parts = split;
    m.topk = topk;
    m.indices = indices;
    return hip_status(mla::launch_cand_select(m, (hipStream_t)stream), "top-k select launch");
}
}  // namespace

size_t mla_topk_workspace_size(const mla_batch_t *batch, int32_t k) {
    mla::BatchDev dev{};
    if (k < 1 || check_batch(batch, &dev) != MLA_OK || batch->total_q == 0) return 0;
    return topk_ws_bytes(batch->total_q, indexer_key_split(batch, indexer_blocks(batch)), k);
}

mla_status_t mla_indexer_topk(const mla_batch_t *batch, const void *q_idx, const void *k_idx,
                              const float *w, int32_t n_heads, int32_t head_dim, int32_t k,
                              int32_t *indices, void *workspace, size_t workspace_bytes,
                              void *stream) {
    if (k == 0) return fail(MLA_ERR_INVALID_ARG, "k must be >= 1 (got 0)");
    return indexer(batch, q_idx, nullptr, k_idx, nullptr, w, n_heads, head_dim, nullptr, 0, false,
                   stream, k, indices, workspace, workspace_bytes);
}

mla_status_t mla_indexer_topk_fp8(const mla_batch_t *batch, const void *q_idx, const float *q_scale,
                                  const void *k_idx, const float *k_scale, const float *w,
                                  int32_t n_heads, int32_t head_dim, int32_t k, int32_t *indices,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    if (k == 0) return fail(MLA_ERR_INVALID_ARG, "k must be >= 1 (got 0)");
    return indexer(batch, q_idx, q_scale, k_idx, k_scale, w, n_heads, head_dim, nullptr, 0, true,
                   stream, k, indices, workspace, workspace_bytes);
}

mla_status_t mla_indexer_score(const mla_batch_t *batch, const void *q_idx, const void *k_idx,
                               const float *w, int32_t n_heads, int32_t head_dim, float *scores,
                               int64_t ld_scores, void *stream) {
    return indexer(batch, q_idx, nullptr, k_idx, nullptr, w, n_heads, head_dim, scores, ld_scores,
                   false, stream);
}

mla_status_t mla_indexer_score_fp8(const mla_batch_t *batch, const void *q_idx, const float *q_scale,
                                   const void *k_idx, const float *k_scale, const float *w,
                                   int32_t n_heads, int32_t head_dim, float *scores,
                                   int64_t ld_scores, void *stream) {
    return indexer(batch, q_idx, q_scale, k_idx, k_scale, w, n_heads, head_dim, scores, ld_scores,
                   true, stream);
}

mla_status_t mla_topk_select(const mla_batch_t *batch, const float *scores, int64_t ld_scores,
                             int32_t k, int32_t *indices, void *stream) {
    mla::TopkArgs a{};
    mla_status_t st = check_batch(batch, &a.batch);
    if (st != MLA_OK) return st;
    if (k < 1) return fail(MLA_ERR_INVALID_ARG, "k must be >= 1 (got %d)", k);
    if (k > 4096) return fail(MLA_ERR_UNSUPPORTED, "k %d > 4096", k);
    if (ld_scores < batch->max_kv_len)
        return fail(MLA_ERR_INVALID_ARG, "ld_scores %lld < max_kv_len %d", (long long)ld_scores,
                    batch->max_kv_len);
    if (batch->max_kv_len > mla::kTopkMaxRow)
        return fail(MLA_ERR_UNSUPPORTED, "max_kv_len %d > %d (top-k row bitmaps live in LDS)",
                    batch->max_kv_len, mla::kTopkMaxRow);
    if (batch->total_q == 0) return ok();
    if (!scores || !indices) return fail(MLA_ERR_INVALID_ARG, "scores / indices is NULL");
    if (!aligned(scores, 4) || !aligned(indices, 4))
        return fail(MLA_ERR_INVALID_ARG, "scores and indices must be 4-byte aligned");
    a.scores = scores;
    a.ld = ld_scores;
    a.indices = indices;
    a.k = k;
    a.max_row = batch->max_kv_len;
    return hip_status(mla::launch_topk(a, batch->cu_seqlens_q_host, batch->cu_seqlens_kv_host,
                                      (hipStream_t)stream),
                      "top-k launch");
}

namespace {
// Checks shared by the attention entry points; fills everything of `a` but the
// outputs and the split. *none: valid, but there is no query (nothing to run).
mla_status_t attention_args(const mla_batch_t *batch, const void *q, const void *kv,
                            const float *kv_scale, mla_kv_dtype_t kv_dtype, int64_t kv_row_stride,
                            int64_t kv_scale_stride, const int32_t *indices, int32_t k,
                            int32_t n_heads, float sm_scale, void *out, float *lse,
                            mla::AttnArgs *a, bool *fp8_out, bool *none) {
    *none = false;
    mla_status_t st = check_batch(batch, &a->batch);
    if (st != MLA_OK) return st;
    if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
        return fail(MLA_ERR_INVALID_ARG, "unknown kv_dtype %d", (int)kv_dtype);
    const bool fp8 = kv_dtype == MLA_KV_FP8_E4M3;
    const int64_t row_bytes = fp8 ? MLA_QK_DIM : 2 * MLA_QK_DIM;
    if (kv_row_stride < row_bytes || kv_row_stride % 16 != 0)
        return fail(MLA_ERR_INVALID_ARG, "kv_row_stride %lld must be >= %lld and a multiple of 16",
                    (long long)kv_row_stride, (long long)row_bytes);
    if (fp8 && (kv_scale_stride < 4 || kv_scale_stride % 4 != 0))
        return fail(MLA_ERR_INVALID_ARG, "kv_scale_stride %lld must be a positive multiple of 4",
                    (long long)kv_scale_stride);
    if (!(sm_scale > 0.f) || !(sm_scale < 1e30f))
        return fail(MLA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
    if (indices && k < 1) return fail(MLA_ERR_INVALID_ARG, "k must be >= 1 with indices (got %d)", k);
    if (n_heads != 8 && n_heads != 16 && n_heads != 32 && n_heads != 64)
        return fail(MLA_ERR_UNSUPPORTED, "n_heads %d not in {8, 16, 32, 64}", n_heads);
    if (indices && k > 65536) return fail(MLA_ERR_UNSUPPORTED, "k %d > 65536", k);
    if ((int64_t)batch->max_kv_len * kv_row_stride > (int64_t)UINT32_MAX)
        return fail(MLA_ERR_UNSUPPORTED, "a sequence's KV rows span %lld bytes (>= 4 GiB)",
                    (long long)batch->max_kv_len * kv_row_stride);
    if (fp8 && (int64_t)batch->max_kv_len * kv_scale_stride > (int64_t)UINT32_MAX)
        return fail(MLA_ERR_UNSUPPORTED, "a sequence's KV scales span %lld bytes (>= 4 GiB)",
                    (long long)batch->max_kv_len * kv_scale_stride);
    if (batch->total_q == 0) {
        *none = true;
        return ok();
    }
    if (!q || !kv || !out || !lse || (fp8 && !kv_scale))
        return fail(MLA_ERR_INVALID_ARG, "q / kv / out / lse%s is NULL", fp8 ? " / kv_scale" : "");
    if (!aligned(q, 16) || !aligned(kv, 16))
        return fail(MLA_ERR_INVALID_ARG, "q and kv must be 16-byte aligned");
    if (!aligned(out, 16) || !aligned(lse, 4) || (fp8 && !aligned(kv_scale, 4)) ||
        (indices && !aligned(indices, 4)))
        return fail(MLA_ERR_INVALID_ARG, "out / lse / kv_scale / indices misaligned");
    a->q = (const __bf16 *)q;
    a->kv = (const uint8_t *)kv;
    a->kv_scale = (const uint8_t *)kv_scale;
    a->kv_stride = kv_row_stride;
    a->scale_stride = kv_scale_stride;
    a->indices = indices;
    a->k = indices ? k : 0;
    a->idx_ld = indices ? k : 0;
    a->n_heads = n_heads;
    a->scale_log2 = sm_scale * 1.4426950408889634f;
    *fp8_out = fp8;
    return ok();
}

// Workspace of a split-KV call: the parts' outputs, then their LSEs.
size_t split_o_bytes(int64_t total_q, int64_t n_heads, int64_t n_split) {
    return ((size_t)(n_split * total_q * n_heads * MLA_V_DIM * 2) + 255) / 256 * 256;
}

// n_split == 0: as many parts as fill the current device's compute units once
// (CUs / total_q), 1..16, and at most k when a list is given.
int32_t auto_split(int64_t total_q, int32_t k_or_0) {
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
        n_cu = 1;
    int64_t s = total_q > 0 ? n_cu / total_q : 1;
    s = std::max<int64_t>(1, std::min<int64_t>(s, mla::kMergeMaxParts));
    if (k_or_0 > 0) s = std::min<int64_t>(s, k_or_0);
    return (int32_t)s;
}
}  // namespace

mla_status_t mla_sparse_prefill(const mla_batch_t *batch, const void *q, const void *kv,
                                const float *kv_scale, mla_kv_dtype_t kv_dtype,
                                int64_t kv_row_stride, int64_t kv_scale_stride,
                                const int32_t *indices, int32_t k, int32_t n_heads,
                                float sm_scale, void *out, float *lse, void *stream) {
    mla::AttnArgs a{};
    bool fp8 = false, none = false;
    mla_status_t st = attention_args(batch, q, kv, kv_scale, kv_dtype, kv_row_stride, kv_scale_stride,
                                     indices, k, n_heads, sm_scale, out, lse, &a, &fp8, &none);
    if (st != MLA_OK || none) return st;
    a.n_split = 1;
    a.out = (__bf16 *)out;
    a.lse = lse;
    return hip_status(mla::launch_attention(a, fp8, (hipStream_t)stream), "attention launch");
}

size_t mla_sparse_prefill_split_workspace_size(int32_t total_q, int32_t n_heads, int32_t n_split) {
    if (n_split == 0) n_split = auto_split(total_q, 0);
    if (total_q <= 0 || n_heads <= 0 || n_split <= 1) return 0;
    return split_o_bytes(total_q, n_heads, n_split) + (size_t)n_split * total_q * n_heads * 4;
}

namespace {
// The split-KV call with the caller's workspace, or (library_scratch) with
// the current device's `scratch` array.
mla_status_t split_impl(const mla_batch_t *batch, const void *q, const void *kv,
                        const float *kv_scale, mla_kv_dtype_t kv_dtype, int64_t kv_row_stride,
                        int64_t kv_scale_stride, const int32_t *indices, int32_t k,
                        int32_t n_heads, float sm_scale, int32_t n_split, void *workspace,
                        size_t workspace_bytes, bool library_scratch, void *out, float *lse,
                        void *stream) {
    if (n_split < 0) return fail(MLA_ERR_INVALID_ARG, "n_split must be >= 0 (got %d)", n_split);
    if (n_split == 0 && batch && batch->total_q > 0) n_split = auto_split(batch->total_q, indices ? k : 0);
    if (n_split == 0) n_split = 1;
    if (n_split > mla::kMergeMaxParts)
        return fail(MLA_ERR_UNSUPPORTED, "n_split %d > %d", n_split, mla::kMergeMaxParts);
    if (indices && n_split > k)
        return fail(MLA_ERR_INVALID_ARG, "n_split %d > k %d: every part needs a list entry", n_split, k);
    mla::AttnArgs a{};
    bool fp8 = false, none = false;
    mla_status_t st = attention_args(batch, q, kv, kv_scale, kv_dtype, kv_row_stride, kv_scale_stride,
                                     indices, k, n_heads, sm_scale, out, lse, &a, &fp8, &none);
    if (st != MLA_OK || none) return st;
    if (n_split == 1) {
        a.n_split = 1;
        a.out = (__bf16 *)out;
        a.lse = lse;
        return hip_status(mla::launch_attention(a, fp8, (hipStream_t)stream), "attention launch");
    }
    const int64_t total_q = batch->total_q;
    if (total_q * n_split > (int64_t)INT32_MAX)
        return fail(MLA_ERR_UNSUPPORTED, "total_q * n_split = %lld exceeds int32",
                    (long long)(total_q * n_split));
    const size_t need = mla_sparse_prefill_split_workspace_size((int32_t)total_q, n_heads, n_split);
    if (library_scratch) {
        if (need > (size_t)MLA_SPLIT_SCRATCH_BYTES)
            return fail(MLA_ERR_UNSUPPORTED,
                        "the %d parts of %lld queries x %d heads need %zu bytes; the library's "
                        "scratch array holds %zu (MLA_SPLIT_SCRATCH_BYTES)",
                        n_split, (long long)total_q, n_heads, need, (size_t)MLA_SPLIT_SCRATCH_BYTES);
        st = scratch_of_current_device(&workspace);
        if (st != MLA_OK) return st;
        workspace_bytes = MLA_SPLIT_SCRATCH_BYTES;
    }
    if (!workspace) return fail(MLA_ERR_INVALID_ARG, "workspace is NULL");
    if (!aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (workspace_bytes < need)
        return fail(MLA_ERR_INVALID_ARG, "workspace_bytes %zu < %zu", workspace_bytes, need);
    uint8_t *ws = (uint8_t *)workspace;
    const int64_t rows = total_q * n_heads;                 // (query, head) rows per part
    a.n_split = n_split;
    a.out = (__bf16 *)ws;
    a.lse = (float *)(ws + split_o_bytes(total_q, n_heads, n_split));
    st = hip_status(mla::launch_attention(a, fp8, (hipStream_t)stream), "attention launch");
    if (st != MLA_OK) return st;
    mla::MergeArgs m{};
    for (int32_t r = 0; r < n_split; ++r) {
        m.o[r] = a.out + r * rows * MLA_V_DIM;
        m.lse[r] = a.lse + r * rows;
    }
    m.n_parts = n_split;
    m.rows = rows;
    m.out = (__bf16 *)out;
    m.lse_out = lse;
    return hip_status(mla::launch_merge(m, (hipStream_t)stream), "merge launch");
}
}  // namespace

mla_status_t mla_sparse_prefill_split(const mla_batch_t *batch, const void *q, const void *kv,
                                      const float *kv_scale, mla_kv_dtype_t kv_dtype,
                                      int64_t kv_row_stride, int64_t kv_scale_stride,
                                      const int32_t *indices, int32_t k, int32_t n_heads,
                                      float sm_scale, int32_t n_split, void *workspace,
                                      size_t workspace_bytes, void *out, float *lse, void *stream) {
    return split_impl(batch, q, kv, kv_scale, kv_dtype, kv_row_stride, kv_scale_stride, indices, k,
                      n_heads, sm_scale, n_split, workspace, workspace_bytes, false, out, lse, stream);
}

mla_status_t mla_sparse_prefill_split_noalloc(const mla_batch_t *batch, const void *q,
                                              const void *kv, const float *kv_scale,
                                              mla_kv_dtype_t kv_dtype, int64_t kv_row_stride,
                                              int64_t kv_scale_stride, const int32_t *indices,
                                              int32_t k, int32_t n_heads, float sm_scale,
                                              int32_t n_split, void *out, float *lse, void *stream) {
    return split_impl(batch, q, kv, kv_scale, kv_dtype, kv_row_stride, kv_scale_stride, indices, k,
                      n_heads, sm_scale, n_split, nullptr, 0, true, out, lse, stream);
}

mla_status_t mla_merge_attention(const void *const *o_parts, const float *const *lse_parts,
                                 int32_t n_parts, int32_t total_q, int32_t n_heads, void *out,
                                 float *lse, void *stream) {
    if (n_parts < 1) return fail(MLA_ERR_INVALID_ARG, "n_parts must be >= 1 (got %d)", n_parts);
    if (n_parts > mla::kMergeMaxParts)
        return fail(MLA_ERR_UNSUPPORTED, "n_parts %d > %d", n_parts, mla::kMergeMaxParts);
    if (total_q < 0 || n_heads < 1)
        return fail(MLA_ERR_INVALID_ARG, "total_q must be >= 0 and n_heads >= 1 (got %d, %d)", total_q, n_heads);
    if (!o_parts || !lse_parts) return fail(MLA_ERR_INVALID_ARG, "o_parts / lse_parts is NULL");
    if (total_q == 0) return ok();
    if (!out || !lse) return fail(MLA_ERR_INVALID_ARG, "out / lse is NULL");
    if (!aligned(out, 16) || !aligned(lse, 4)) return fail(MLA_ERR_INVALID_ARG, "out / lse misaligned");
    mla::MergeArgs a{};
    for (int32_t r = 0; r < n_parts; ++r) {
        if (!o_parts[r] || !lse_parts[r])
            return fail(MLA_ERR_INVALID_ARG, "part %d: o / lse pointer is NULL", r);
        if (!aligned(o_parts[r], 16) || !aligned(lse_parts[r], 4))
            return fail(MLA_ERR_INVALID_ARG, "part %d: o / lse pointer misaligned", r);
        a.o[r] = (const __bf16 *)o_parts[r];
        a.lse[r] = lse_parts[r];
    }
    a.n_parts = n_parts;
    a.rows = (int64_t)total_q * n_heads;
    a.out = (__bf16 *)out;
    a.lse_out = lse;
    return hip_status(mla::launch_merge(a, (hipStream_t)stream), "merge launch");
}

mla_status_t mla_kv_decode_ds656(const void *kv_ds656, int64_t row_stride, int64_t n_rows,
                                 void *kv_bf16, void *stream) {
    if (n_rows < 0) return fail(MLA_ERR_INVALID_ARG, "n_rows must be >= 0 (got %lld)", (long long)n_rows);
    if (row_stride < MLA_DS656_ROW_BYTES || row_stride % 16 != 0)
        return fail(MLA_ERR_INVALID_ARG, "row_stride %lld must be >= %d and a multiple of 16",
                    (long long)row_stride, MLA_DS656_ROW_BYTES);
    if (n_rows == 0) return ok();
    if (!kv_ds656 || !kv_bf16) return fail(MLA_ERR_INVALID_ARG, "kv_ds656 / kv_bf16 is NULL");
    if (!aligned(kv_ds656, 16) || !aligned(kv_bf16, 16))
        return fail(MLA_ERR_INVALID_ARG, "kv_ds656 and kv_bf16 must be 16-byte aligned");
    if (n_rows > (int64_t)INT32_MAX * 8)
        return fail(MLA_ERR_UNSUPPORTED, "n_rows %lld too large", (long long)n_rows);
    mla::Ds656Args a{(const uint8_t *)kv_ds656, row_stride, n_rows, (uint8_t *)kv_bf16};
    return hip_status(mla::launch_ds656_decode(a, (hipStream_t)stream), "row decode launch");
}

const char *mla_status_string(mla_status_t s) {
    switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument, nothing enqueued";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: shape not supported, nothing enqueued";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: a HIP call or kernel launch failed";
    }
    return "unknown mla_status_t";
}

const char *mla_last_error(void) { return g_last_error.c_str(); }

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

}  // extern "C"
