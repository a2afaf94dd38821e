// Launch interfaces of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct BatchDev {
    const int32_t *cu_q;
    const int32_t *cu_kv;
    const int32_t *q_pos;
    int32_t num_seqs;
    int32_t total_q;
};

struct IndexerArgs {
    BatchDev batch;
    const void *q_idx;     // [total_q, n_heads, head_dim] bf16, or E4M3 codes
    const void *k_idx;     // [total_kv, head_dim] bf16, or E4M3 codes
    const float *q_scale;  // E4M3: [total_q, n_heads] fp32, >= 0
    const float *k_scale;  // E4M3: [total_kv] fp32, >= 0
    const float *w;        // [total_q, n_heads]
    float *scores;         // [total_q, ld]
    int64_t ld;
    int32_t n_heads;
    int32_t head_dim;
    int32_t key_split;     // workgroups per query block, each over a contiguous range of key tiles
    int32_t n_blocks;      // key_split * sum over sequences of ceil(n_q(b) / queries per block)
    bool fp8;              // E4M3 queries and keys with scales
    // Fused top-k (topk > 0): no scores are written. Each (query, key part)
    // keeps a candidate list of (order key, j) entries in ascending j that
    // holds every key able to reach the query's top k; cand_select_kernel
    // then selects the top k over the parts' lists.
    int32_t topk;
    uint2 *cand;           // [total_q * key_split, cand_cap]
    int32_t cand_cap;      // entries per list (>= 3 topk + kIdxKeyTile)
    int32_t *cand_n;       // [total_q * key_split] final list lengths
};
constexpr int kIdxQueriesPerBlock = 8;
constexpr int kIdxKeyTile = 256;          // keys per indexer LDS tile
// Candidate list entries for top-k k: a compaction leaves at most about 2k
// (k, or more when ties crowd its threshold bin), so there is room for k or
// more appends plus one key tile before the next. 3k measured faster than 2k
// (more compactions) and 4k (longer lists for the final select).
constexpr int64_t cand_capacity(int64_t k) { return (3 * k + kIdxKeyTile + 63) / 64 * 64; }

// Exact top-k selection over the key parts' candidate lists of each query.
struct CandSelectArgs {
    BatchDev batch;
    const uint2 *cand;
    const int32_t *cand_n;
    int32_t cand_cap;
    int32_t n_parts;
    int32_t topk;
    int32_t *indices;
};
struct TopkArgs {
    BatchDev batch;
    const float *scores;
    int64_t ld;
    int32_t *indices;      // [total_q, k]
    int32_t k;
    int32_t max_row;       // max_kv_len: longest possible score row
    int32_t q_begin, q_end;  // this launch's query rows (set by launch_topk)
};

struct AttnArgs {
    BatchDev batch;
    const __bf16 *q;            // [total_q, n_heads, 576]
    const uint8_t *kv;          // row r at kv + r * kv_stride
    const uint8_t *kv_scale;    // fp32 scale of row r at kv_scale + r * scale_stride
    int64_t kv_stride;
    int64_t scale_stride;
    const int32_t *indices;     // [total_q, idx_ld], first k entries used; or null (dense causal)
    int32_t k;
    int32_t idx_ld;             // entries between index rows
    int32_t n_heads;
    float scale_log2;           // sm_scale * log2(e)
    // Split-KV: every query's keys (list entries, or causal keys when dense)
    // are cut into n_split contiguous parts, each run as its own virtual
    // query; part p of query i writes output row p * total_q + i. 1: no split.
    int32_t n_split;
    __bf16 *out;                // [n_split * total_q, n_heads, 512]
    float *lse;                 // [n_split * total_q, n_heads]
};

// LSE merge of attention parts over disjoint key sets
constexpr int kMergeMaxParts = 16;
constexpr int kMergeDim = 512;              // output dims per (query, head) row
struct MergeArgs {
    const __bf16 *o[kMergeMaxParts];        // part r: [rows, 512]
    const float *lse[kMergeMaxParts];       // part r: [rows]
    int32_t n_parts;
    int64_t rows;                           // total_q * n_heads
    __bf16 *out;                            // [rows, 512]
    float *lse_out;                         // [rows]
};

// Decode of 656-byte latent rows (512 E4M3 codes, four fp32 tile scales, 64
// bf16 rope values) to bf16 rows of 576 values.
struct Ds656Args {
    const uint8_t *in;     // row r at in + r * in_stride
    int64_t in_stride;
    int64_t n_rows;
    uint8_t *out;          // [n_rows, 576] bf16
};
hipError_t launch_ds656_decode(const Ds656Args &a, hipStream_t s);

hipError_t launch_indexer(const IndexerArgs &a, hipStream_t s);
// cu_q_host / cu_kv_host: the batch's host cu_seqlens (the launch shape per sequence)
hipError_t launch_topk(const TopkArgs &a, const int32_t *cu_q_host, const int32_t *cu_kv_host,
                       hipStream_t s);
hipError_t launch_cand_select(const CandSelectArgs &a, hipStream_t s);
constexpr int32_t kTopkMaxRow = 1 << 19;   // longest score row top-k takes (its bitmaps sit in LDS)
hipError_t launch_attention(const AttnArgs &a, bool fp8, hipStream_t s);
// FP8 (E4M3) latent rows (launch_attention dispatches to it)
hipError_t launch_attention_fp8_f8(const AttnArgs &a, hipStream_t s);
hipError_t launch_merge(const MergeArgs &a, hipStream_t s);

}  // namespace mla
