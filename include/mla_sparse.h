/*
 * mla_sparse.h -- C ABI of an MI355X (gfx950) library for GLM-style causal
 * prefill attention over a multi-head latent attention (MLA) KV cache.
 *
 * The path has three calls, run in this order for one attention layer, and a
 * fourth that merges attention results computed over parts of the keys:
 *
 *   mla_indexer_score   the indexer scores every earlier token of each query
 *                       (spke.com GLM-5.3 PCP/DCP article, section "Warum nicht
 *                       TP oder DP?": it scores every earlier token to pick the
 *                       2,048 that sparse MLA attends to; its cost grows with
 *                       the square of the prompt length, section "PCP").
 *                       mla_indexer_score_fp8 is the same score from FP8
 *                       queries and keys with a scale each (footnote 3 stores
 *                       an indexer key as 128 FP8 values plus a 4-byte scale).
 *   mla_topk_select     keeps the k best-scoring earlier tokens per query.
 *   mla_indexer_topk    both in one pass, without the score matrix (and
 *                       mla_indexer_topk_fp8 from FP8 indexer inputs).
 *   mla_sparse_prefill  absorbed (MQA-form) MLA attention over the kept tokens:
 *                       one 576-value latent row per token (512 latent + 64
 *                       rope) serves every head, QK over 576 dims and PV over
 *                       the first 512 (same article, footnote 1), with the
 *                       log-sum-exp of every (query, head) as a second output
 *                       (the mergeable quantity of its section "DCP").
 *   mla_merge_attention combines attention results over disjoint key sets
 *                       (key shards, or splits of one query's keys) through
 *                       their log-sum-exp.
 *   mla_sparse_prefill_split  split-KV attention: each query's keys in up to
 *                       16 parts run as separate work items, then merged.
 *   mla_kv_decode_ds656 decodes 656-byte latent rows (E4M3 with four tile
 *                       scales, bf16 rope) to the bf16 rows attention reads.
 *
 * Batches are packed: sequence b owns query rows [cu_q[b], cu_q[b+1]) and
 * latent-KV rows [cu_kv[b], cu_kv[b+1]); every query carries its true
 * absolute position p_i = q_pos[i] inside its sequence, 0 <= p_i < L_b. One
 * call therefore covers whole prompts, one GPU's context-parallel share (the
 * queries of chunks r and 2N-1-r of a 2N-chunk prompt against the full
 * gathered KV -- article, section "PCP") or new suffix tokens resuming behind
 * a cached prefix. A query attends to the keys j <= p_i of its own sequence
 * (its own token included).
 *
 * Conventions shared by every call:
 *  - Pointers marked "device" must point to GPU memory of the current HIP
 *    device; "host" pointers to CPU memory read during the call only.
 *  - The caller owns every buffer. The library allocates no memory and keeps
 *    no pointer after a call returns. Its only global state is the scratch
 *    array of mla_sparse_prefill_split_noalloc (one per GPU, with its device
 *    address taken once per device under a lock); every other call is safe
 *    from several host threads.
 *  - Calls validate their arguments on the host, enqueue kernels on `stream`
 *    (a hipStream_t; NULL means the null stream) and return without waiting.
 *    Outputs are valid once the stream has reached that point; inputs must
 *    stay alive until then.
 *  - Return codes: MLA_OK; MLA_ERR_INVALID_ARG (nothing was enqueued: a null
 *    required pointer, a bad scalar, host cu_seqlens that are not monotone or
 *    do not end at the totals, a misaligned pointer or stride);
 *    MLA_ERR_UNSUPPORTED (a valid shape this build has no kernel for; nothing
 *    enqueued); MLA_ERR_HIP (a HIP call or launch failed). mla_last_error()
 *    gives a human-readable reason for the last failure on this thread.
 *  - q_pos[i] < L_b is a caller contract on device data; it is not checked
 *    (checking would need a device synchronisation).
 *  - bf16 is IEEE bfloat16; fp8 is OCP E4M3 (e4m3fn: bias 7, max 448, no inf).
 */
#ifndef MLA_SPARSE_H
#define MLA_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 1
#define MLA_QK_DIM 576 /* absorbed query / latent KV row width: 512 latent + 64 rope */
#define MLA_V_DIM 512  /* output width per head: the latent part of the row */

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1,
    MLA_ERR_UNSUPPORTED = 2,
    MLA_ERR_HIP = 3
} mla_status_t;

typedef enum { MLA_KV_BF16 = 0, MLA_KV_FP8_E4M3 = 1 } mla_kv_dtype_t;

/* Ragged batch description. The host copies of cu_seqlens are validated and
 * used to size the launches; the device copies must hold the same values. */
typedef struct {
    int32_t num_seqs;               /* B >= 1                                         */
    int32_t total_q;                /* cu_seqlens_q[B]  (>= 0)                          */
    int32_t total_kv;               /* cu_seqlens_kv[B] (>= 0)                          */
    int32_t max_kv_len;             /* max_b L_b                                       */
    const int32_t *cu_seqlens_q_host;  /* host   [B+1], cu[0] = 0, non-decreasing       */
    const int32_t *cu_seqlens_kv_host; /* host   [B+1], cu[0] = 0, non-decreasing       */
    const int32_t *cu_seqlens_q;       /* device [B+1], same values                     */
    const int32_t *cu_seqlens_kv;      /* device [B+1], same values                     */
    const int32_t *q_pos;              /* device [total_q], 0 <= q_pos[i] < L_b(i)      */
} mla_batch_t;

/* Indexer scores (spke.com article, section "Warum nicht TP oder DP?"; one
 * indexer key per token shared by all indexer heads, footnote 3). For every
 * query i and every key j <= q_pos[i] of its sequence:
 *
 *     scores[i * ld_scores + j] = sum_h w[i, h] * max(0, sum_d q_idx[i, h, d] * k_idx[j, d])
 *
 * with fp32 accumulation of exact bf16 x bf16 products. Entries j > q_pos[i]
 * are not written.
 *   q_idx   device [total_q, n_heads, head_dim] bf16, 16-byte aligned
 *   k_idx   device [total_kv, head_dim] bf16 (row = cu_seqlens_kv[b] + j), 16-byte aligned
 *   w       device [total_q, n_heads] fp32
 *   scores  device [total_q, ld_scores] fp32; ld_scores >= max_kv_len
 * Supported: 1 <= n_heads <= 64, head_dim in {64, 128}. */
mla_status_t mla_indexer_score(const mla_batch_t *batch, const void *q_idx, const void *k_idx,
                               const float *w, int32_t n_heads, int32_t head_dim, float *scores,
                               int64_t ld_scores, void *stream);

/* Indexer scores from FP8 queries and keys (spke.com article, footnote 3: an
 * indexer key is kept as 128 FP8 values plus a 4-byte scale per token). With
 * decoded E4M3 codes qc, kc and the scales sq, sk:
 *
 *     scores[i * ld_scores + j] =
 *         sum_h w[i, h] * max(0, sum_d (sq[i, h] * qc[i, h, d]) * (sk[j] * kc[j, d]))
 *
 * for every key j <= q_pos[i]; entries j > q_pos[i] are not written. The
 * code products are exact and accumulate in fp32; the scales are applied to
 * the finished dot products (ReLU commutes with a non-negative factor).
 *   q_idx    device [total_q, n_heads, head_dim] E4M3 codes (1 byte each), 16-byte aligned
 *   q_scale  device [total_q, n_heads] fp32, finite and >= 0, 4-byte aligned
 *   k_idx    device [total_kv, head_dim] E4M3 codes (row = cu_seqlens_kv[b] + j), 16-byte aligned
 *   k_scale  device [total_kv] fp32, finite and >= 0, 4-byte aligned
 *   w, scores, ld_scores, n_heads, head_dim: as mla_indexer_score.
 * A negative or non-finite scale gives undefined scores (not checked: device
 * data), and so are scores from NaN codes (0x7f, 0xff). */
mla_status_t mla_indexer_score_fp8(const mla_batch_t *batch, const void *q_idx, const float *q_scale,
                                   const void *k_idx, const float *k_scale, const float *w,
                                   int32_t n_heads, int32_t head_dim, float *scores,
                                   int64_t ld_scores, void *stream);

/* Top-k selection over the indexer scores of each query (same section: keep
 * the 2,048 best earlier tokens). For query i with n_i = q_pos[i] + 1 scored
 * keys: if n_i <= k, every key 0..n_i-1 is kept; otherwise the k largest
 * scores are kept, equal scores going to the smaller j (-0.0 equals +0.0).
 * indices[i, 0:k] lists the kept local key indices in ascending order and is
 * padded with -1. Scores must not be NaN.
 *   scores  device [total_q, ld_scores] fp32 (row i read for j <= q_pos[i])
 *   indices device [total_q, k] int32
 * Supported: 1 <= k <= 4096; max_kv_len <= 524288 (MLA_ERR_UNSUPPORTED otherwise). */
mla_status_t mla_topk_select(const mla_batch_t *batch, const float *scores, int64_t ld_scores,
                             int32_t k, int32_t *indices, void *stream);

/* Bytes of workspace mla_indexer_topk and mla_indexer_topk_fp8 need for this
 * batch and k (0 for an invalid batch, k < 1 or no query). It depends on the
 * current device's compute-unit count, which sets how the keys of a small
 * batch are split over workgroups: query it with the device the call will
 * run on current. About total_q * (3k + 256) * 8 bytes when the batch has at
 * least two eight-query blocks per compute unit. */
size_t mla_topk_workspace_size(const mla_batch_t *batch, int32_t k);

/* Indexer and top-k in one pass, without the score matrix (spke.com article,
 * section "PCP": the indexer's cost, and its score matrix, grow with the
 * square of the prompt length; section "Warum nicht TP oder DP?": it keeps
 * the 2,048 best earlier tokens). indices[i, 0:k] is exactly what
 * mla_topk_select gives on the scores mla_indexer_score computes for the same
 * inputs: the same kernels compute every score with the same instructions in
 * the same order, and the selection rule (k largest, equal scores to the
 * smaller j, -0 equal to +0, all keys when q_pos[i] + 1 <= k, ascending,
 * -1 padded) is applied exactly, to a candidate list that provably holds the
 * top k. Scores must not be NaN.
 *   q_idx, k_idx, w, n_heads, head_dim: as mla_indexer_score
 *   k          1..4096
 *   indices    device [total_q, k] int32, 4-byte aligned
 *   workspace  device, 256-byte aligned, at least mla_topk_workspace_size(batch, k)
 *              bytes, owned by the caller; holds each query's candidate list
 *              of (score key, index) pairs; two calls in flight on different
 *              streams must not share it
 * Errors as mla_indexer_score (ld_scores aside), plus MLA_ERR_INVALID_ARG for
 * k < 1, a NULL indices or workspace, a misaligned or too small workspace,
 * and MLA_ERR_UNSUPPORTED for k > 4096. Nothing is enqueued then. */
mla_status_t mla_indexer_topk(const mla_batch_t *batch, const void *q_idx, const void *k_idx,
                              const float *w, int32_t n_heads, int32_t head_dim, int32_t k,
                              int32_t *indices, void *workspace, size_t workspace_bytes,
                              void *stream);

/* mla_indexer_topk from FP8 indexer inputs: the scores of
 * mla_indexer_score_fp8 (same arguments q_idx, q_scale, k_idx, k_scale), then
 * the same exact selection. */
mla_status_t mla_indexer_topk_fp8(const mla_batch_t *batch, const void *q_idx, const float *q_scale,
                                  const void *k_idx, const float *k_scale, const float *w,
                                  int32_t n_heads, int32_t head_dim, int32_t k, int32_t *indices,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* Absorbed MLA attention over selected latent rows (spke.com article,
 * footnote 1 and section "PCP": one latent row read per selected key serves
 * all heads; QK over 576 dims, PV over 512; dense path of section
 * "Ausprobieren" when indices == NULL). For query i, head h and the set S_i of
 * its selected keys (entries of indices[i, :] with 0 <= j <= q_pos[i];
 * others are skipped; with indices == NULL, S_i = {0..q_pos[i]}):
 *
 *     K_j     = decode(kv row cu_seqlens_kv[b] + j)   (bf16, or e4m3 * kv_scale)
 *     z_j     = sm_scale * sum_{d<576} q[i, h, d] * K_j[d]
 *     lse[i,h]= ln sum_{j in S_i} exp(z_j)
 *     out[i,h,c] = sum_{j in S_i} exp(z_j - lse[i,h]) * K_j[c],   c < 512
 *
 * An empty S_i gives out = 0 and lse = -inf. Duplicate entries in a row of
 * indices are a caller error (the key would be counted twice).
 *   q        device [total_q, n_heads, 576] bf16, 16-byte aligned
 *   kv       device, row r at byte offset r * kv_row_stride: 576 bf16 or 576 e4m3 codes;
 *            16-byte aligned, kv_row_stride a multiple of 16 and >= the row size
 *   kv_scale device fp32, scale of row r at byte offset r * kv_scale_stride (a
 *            multiple of 4); required for MLA_KV_FP8_E4M3, ignored for bf16
 *   indices  device [total_q, k] int32 local key indices, or NULL (dense causal)
 *   out      device [total_q, n_heads, 512] bf16 (round to nearest even), 16-byte aligned
 *   lse      device [total_q, n_heads] fp32, natural log (sm_scale included)
 * Supported: n_heads in {8, 16, 32, 64}; 1 <= k <= 65536 when indices != NULL;
 * max_kv_len * kv_row_stride < 4 GiB and, for FP8, max_kv_len * kv_scale_stride
 * < 4 GiB (the rows and scales of one sequence are addressed with 32-bit
 * offsets); MLA_ERR_UNSUPPORTED otherwise. */
mla_status_t mla_sparse_prefill(const mla_batch_t *batch, const void *q, const void *kv,
                                const float *kv_scale, mla_kv_dtype_t kv_dtype,
                                int64_t kv_row_stride, int64_t kv_scale_stride,
                                const int32_t *indices, int32_t k, int32_t n_heads,
                                float sm_scale, void *out, float *lse, void *stream);

/* Split-KV form of mla_sparse_prefill: the same out and lse, computed with
 * every query's keys cut into n_split parts that run as separate work items,
 * so a batch with fewer queries than the GPU has compute units still fills
 * it. The parts' (out, lse) pairs are combined by the log-sum-exp merge of
 * the spke.com article, section "DCP" (as mla_merge_attention).
 * Parts are contiguous and differ in size by at most one: entries
 * [floor(p k / n_split), floor((p+1) k / n_split)) of each index row, or,
 * with indices == NULL, keys [floor(p n / n_split), floor((p+1) n / n_split))
 * of the n = q_pos[i] + 1 causal keys (a part may then be empty).
 * Arguments as mla_sparse_prefill, plus:
 *   n_split    1..16; <= k when indices != NULL. 1 runs mla_sparse_prefill.
 *              0 chooses min(16, max(1, CUs of the current device / total_q)),
 *              and at most k: one round of work items over the GPU.
 *   workspace  device, 256-byte aligned, at least
 *              mla_sparse_prefill_split_workspace_size(total_q, n_heads, n_split)
 *              bytes (n_split 0: the size for the automatic choice with no k
 *              limit, which covers every k), owned by the caller; it holds the
 *              parts' bf16 outputs and fp32 LSEs between the two launches
 *              (unused when the split is 1).
 * The parts' outputs are rounded to bf16 before the merge, so results differ
 * from mla_sparse_prefill by about one more bf16 rounding. Two calls in flight
 * on different streams must not share a workspace.
 * Errors, besides those of mla_sparse_prefill: MLA_ERR_INVALID_ARG for
 * n_split < 0, n_split > k with indices, or (when the split is above 1) a
 * NULL, misaligned or too small workspace; MLA_ERR_UNSUPPORTED for
 * n_split > 16 or total_q * n_split above INT32_MAX. Nothing is enqueued then. */
size_t mla_sparse_prefill_split_workspace_size(int32_t total_q, int32_t n_heads, int32_t n_split);
mla_status_t mla_sparse_prefill_split(const mla_batch_t *batch, const void *q, const void *kv,
                                      const float *kv_scale, mla_kv_dtype_t kv_dtype,
                                      int64_t kv_row_stride, int64_t kv_scale_stride,
                                      const int32_t *indices, int32_t k, int32_t n_heads,
                                      float sm_scale, int32_t n_split, void *workspace,
                                      size_t workspace_bytes, void *out, float *lse, void *stream);

/* Bytes of the library's own scratch array behind
 * mla_sparse_prefill_split_noalloc: the parts of up to 256 virtual queries
 * (query x part) of 64 heads, i.e. every automatic split (n_split = 0 gives
 * total_q * n_split <= 256 on a 256-CU GPU). 16 MiB + 64 KiB per GPU. */
#define MLA_SPLIT_SCRATCH_BYTES (16u * 1024u * 1024u + 64u * 1024u)

/* mla_sparse_prefill_split without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The parts' outputs and LSEs live in
 * a device array the library owns (MLA_SPLIT_SCRATCH_BYTES on every GPU it
 * runs on, held until the process ends; its address is looked up once per
 * device, on the first call with that device current). The call allocates
 * nothing and calls no allocating routine. Arguments, results and errors as
 * mla_sparse_prefill_split, plus MLA_ERR_UNSUPPORTED (nothing enqueued) when
 * mla_sparse_prefill_split_workspace_size(total_q, n_heads, n_split) exceeds
 * MLA_SPLIT_SCRATCH_BYTES. Nothing in the array needs to start at zero (every
 * part's rows are written before the merge reads them). All calls on one GPU
 * share its array and it keeps the last call's contents: calls whose work
 * overlaps on one GPU (other streams, other host threads) race on it and must
 * be serialised by the caller. */
mla_status_t mla_sparse_prefill_split_noalloc(const mla_batch_t *batch, const void *q,
                                              const void *kv, const float *kv_scale,
                                              mla_kv_dtype_t kv_dtype, int64_t kv_row_stride,
                                              int64_t kv_scale_stride, const int32_t *indices,
                                              int32_t k, int32_t n_heads, float sm_scale,
                                              int32_t n_split, void *out, float *lse, void *stream);

/* The 656-byte latent row (spke.com article, footnote 1: 656 bytes of FP8 KV
 * per token, in FlashMLA's fp8_ds_mla format; this library reads it as):
 *   bytes   0..511  E4M3 codes of the 512 latent values
 *   bytes 512..527  four little-endian fp32 scales; scale t covers latent
 *                   values 128t .. 128t+127
 *   bytes 528..655  the 64 rope values, bf16
 * Latent value d is e4m3(code d) * scale[d / 128]; rope value r is bf16. */
#define MLA_DS656_ROW_BYTES 656

/* Decodes n_rows 656-byte rows into the 576 bf16 values of a latent row that
 * mla_sparse_prefill reads with MLA_KV_BF16: latent value d becomes
 * bf16(fp32(e4m3(code) * scale)) (each rounding to nearest even), the rope
 * values are copied. Attention over 656-byte rows is this call followed by
 * the attention call on its output; decoding the product to bf16 before the
 * contraction is what the fp8_ds_mla decoder does (up to 2^-9 of each latent
 * value).
 *   kv_ds656   device, row r at byte offset r * row_stride, 16-byte aligned
 *   row_stride bytes between rows: >= 656 and a multiple of 16
 *   kv_bf16    device [n_rows, 576] bf16, 16-byte aligned, owned by the caller
 * Errors: MLA_ERR_INVALID_ARG (nothing enqueued) for n_rows < 0, a bad
 * stride, a NULL or misaligned pointer. Codes 0x7f / 0xff (NaN) decode to
 * NaN. */
mla_status_t mla_kv_decode_ds656(const void *kv_ds656, int64_t row_stride, int64_t n_rows,
                                 void *kv_bf16, void *stream);

/* Merge of attention results over disjoint key sets by their log-sum-exp
 * (spke.com article, section "DCP": every GPU attends over its share of the
 * KV and the partial results combine through the LSE; the same merge makes
 * split-KV attention on one GPU). For every query i and head h, with parts
 * r = 0 .. n_parts-1 computed by mla_sparse_prefill over key sets that
 * partition the wanted set:
 *
 *     lse[i,h]   = ln sum_r exp(lse_r[i,h])
 *     out[i,h,c] = sum_r exp(lse_r[i,h] - lse[i,h]) * out_r[i,h,c],   c < 512
 *
 * which is attention over the union of the sets. A part with lse_r = -inf (an
 * empty set) contributes nothing; if every part is empty, out = 0 and
 * lse = -inf. The merge works in fp32 and rounds out to bf16 (nearest even).
 *   o_parts   host array of n_parts device pointers, each [total_q, n_heads, 512] bf16, 16-byte aligned
 *   lse_parts host array of n_parts device pointers, each [total_q, n_heads] fp32
 *   out       device [total_q, n_heads, 512] bf16, 16-byte aligned
 *   lse       device [total_q, n_heads] fp32
 * out and lse must not overlap any part. Supported: 1 <= n_parts <= 16
 * (MLA_ERR_UNSUPPORTED above). */
mla_status_t mla_merge_attention(const void *const *o_parts, const float *const *lse_parts,
                                 int32_t n_parts, int32_t total_q, int32_t n_heads, void *out,
                                 float *lse, void *stream);

/* Static description of a status code. */
const char *mla_status_string(mla_status_t status);

/* Reason for the last non-OK status returned on the calling thread ("" if none). */
const char *mla_last_error(void);

/* MLA_ABI_VERSION of the built library. */
int32_t mla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MLA_SPARSE_H */
