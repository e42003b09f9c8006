// launch.h — host-side launchers implemented next to their kernels (internal to libcsa).
// Each returns 0 on success, -2 when the shape/dtype has no kernel.  Arguments were
// validated by the C-ABI layer (api.cpp) before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

int launch_compress(const void* Ca, const void* Za, const float* Ba, const void* Cb, const void* Zb, const float* Bb,
                    int64_t batch, int64_t n, int m, int c, int in_t, void* out, int out_t, hipStream_t stream);

// One decode step of CSA compression: the state holds the raw tokens of blocks block-1 and
// block ([batch, 2m, c] each stream; [batch, m, c] when block == 0); writes entry `block` to
// row `block` of the cache [batch, cache_rows, c].
int launch_compress_step(const void* Ca, const void* Za, const float* Ba, const void* Cb, const void* Zb,
                         const float* Bb, int64_t batch, int64_t block, int m, int c, int in_t, void* cache,
                         int64_t cache_rows, int out_t, hipStream_t stream);

// The state and cache of one decode-step compression (as launch_compress_step takes them).
struct StepStreams {
    const void* Ca;
    const void* Za;
    const float* Ba;
    const void* Cb;
    const void* Zb;
    const float* Bb;
    int c;
    void* cache;
    int64_t cache_rows;
    int out_t;
};

// Two decode-step compressions with the same batch, block, m and input dtype (a CSA layer's KV
// entry and index-key entry): one launch when m == 4, else two launch_compress_step launches.
// The results are those of the two separate calls, bit for bit.
int launch_compress_step_pair(const StepStreams& s0, const StepStreams& s1, int64_t batch, int64_t block, int m,
                              int in_t, hipStream_t stream);

// Indexer scores for every (query, entry) pair into `scores` ([batch*T, ld] fp32, ld >= N).
// write_invisible: also write -inf for entries the query may not see (else they are skipped).
// chunk_mm (optional, [batch*T, index_chunks(...)] pairs): min / max of each chunk of visible
// scores, written by the decode-shaped MFMA kernel (chunks without visible entries hold
// +inf / -inf); *n_chunk_mm receives the chunk count, 0 when the kernel used writes none.
// zero / zero_words (optional): the decode-shaped kernel also zeroes zero_words uint32 per row
// at zero + row * zero_words (the selection's per-row histogram and counters).
// gmax / G / gld (optional, decode-shaped kernel only): the maximum of every group of G
// consecutive visible scores of a row at gmax + row * gld + s / G (G from topk_group).
int launch_index_scores(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0,
                        int64_t N, int H_I, int c_I, int m, int qk_t, float* scores, int64_t ld, bool write_invisible,
                        float* chunk_mm, int* n_chunk_mm, uint32_t* zero, int zero_words, float* gmax, int G,
                        int64_t gld, hipStream_t stream);

// Number of (min, max) pairs per row the indexer writes into chunk_mm for these sizes (0: none).
int index_chunks(int64_t batch, int64_t T, int64_t N, int H_I, int c_I, int qk_t);
// Upper bound of index_chunks(...) over every batch, T, shape and dtype for N entries.
int64_t max_index_chunks(int64_t N);

// Workspace bytes needed by launch_topk beyond the score rows.
size_t topk_extra_workspace(int64_t rows, int64_t N, int k);

// Per-row top-k over the visible prefix of each score row.  chunk_mm / n_chunk_mm: optional
// per-chunk (min, max) of the row's visible scores from the indexer (NULL / 0: not available).
// extra_ws: topk_extra_workspace(...) bytes.  With chunk_mm, few rows and long rows, the
// multi-workgroup path runs; it expects the region topk_zero_region(...) to hold zeros for the
// topk_zero_words(...) words of each row (the decode indexer clears it).
// gmax / G / gld: group maxima from the indexer (NULL / 0: not available); with them the
// group-bounded selection runs.
int launch_topk(const float* scores, int64_t ld, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
                int32_t* idx, float* sel, const float* chunk_mm, int n_chunk_mm, const float* gmax, int G,
                int64_t gld, void* extra_ws, hipStream_t stream);
// Group size of the group-bounded selection for rows of up to nv_max visible entries (0: the
// selection cannot use group maxima for these sizes).  At most 8192 groups per row.
int topk_group(int64_t nv_max, int k);
constexpr int64_t kTopkMaxGroups = 8192;
int topk_zero_words(int64_t rows, int64_t nv_max);
uint32_t* topk_zero_region(void* extra_ws, int64_t rows, int64_t N);

// Partial RoPE, in place on x [batch, T, H, c]: the last d channels of row (b, t) turn by the
// position pos0 + t * pos_step (inverse: by its negative).
int launch_rope(void* x, int64_t batch, int64_t T, int H, int c, int d, int64_t pos0, int64_t pos_step, float base,
                bool inverse, int t, hipStream_t stream);

// Sliding-window branch of the sparse attention: raw (uncompressed) KV rows kv [batch, W, c]
// at absolute positions win_pos0 + j; query t (position q_pos0 + t) also attends to the rows
// whose position lies in [p - n_win + 1, p].  n_win = 0: no window.
struct SwaArgs {
    const void* kv;
    int64_t W, win_pos0, q_pos0;
    int n_win;
};

// Device workspace bytes launch_sparse_mqa needs (0: none) for the key-range partials.
// `sink` (both MQA launchers): per-head sink logits [H] in natural-log units, or nullptr.
size_t sparse_mqa_workspace(int64_t batch, int64_t T, int H, int c, int k, int t);

int launch_sparse_mqa(const void* q, const void* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N, int H,
                      int c, int k, float scale, int t, void* out, void* ws, const float* sink, const SwaArgs& swa,
                      hipStream_t stream);

// Dense causal MQA over the visible entries (ratio r) and, with swa.n_win > 0, the query's
// window rows (swa.q_pos0 must equal q_pos0).
int launch_dense_mqa(const void* q, const void* kv, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int H, int c,
                     int ratio, float scale, int t, void* out, const float* sink, const SwaArgs& swa,
                     hipStream_t stream);

// HCA compression as a decode step: the state holds the raw tokens of block `block`
// ([batch, m', c] per stream); writes entry `block` to row `block` of the cache.
int launch_hca_compress_step(const void* C, const void* Z, const float* B, int64_t batch, int64_t block, int m_prime,
                             int c, int in_t, void* cache, int64_t cache_rows, int out_t, hipStream_t stream);

}  // namespace csa
