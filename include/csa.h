/*
 * csa.h — C ABI of libcsa: the CSA / HCA attention hot path on AMD Instinct MI355X (gfx950).
 *
 * Method sources (web pages on the DeepSeek-V4 report):
 *   [N] "DeepSeek-V4: 迈向高效百万级上下文智能" (notes.kuangjux.top): §1.1 step 1 (token-level
 *       compression, eq. C_i^Comp), §1.1 step 2 (lightning indexer eq. I_{t,s}, top-k,
 *       shared-KV MQA), §1.2 (HCA: ratio m' = 128, no overlap, dense attention).
 *   [M] mlpod.com summary of "DeepSeek-V4: Towards Highly Efficient Million-Token Context
 *       Intelligence": §2.3.1 (CSA), §2.3.2 (HCA, shared-KV MQA).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA memory), owned by the
 *     caller, dense row-major with the shapes given, 16-byte aligned.  The library keeps no
 *     reference to them after the call returns.
 *   - `batch` independent sequences of equal length.  Query i of every sequence sits at the
 *     absolute position q_pos0 + i.
 *   - Causal visibility: compressed entry s (ratio r) may be used by a query at absolute
 *     position p iff r*(s+1)-1 <= p, i.e. once every raw token of the entry is at or before
 *     the query.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream).  The
 *     library never allocates device memory, never synchronises, and holds no mutable global
 *     state other than the fixed scratch of csa_index_topk_noalloc, so calls on different
 *     streams may overlap freely (calls of csa_index_topk_noalloc on one GPU excepted).
 *   - A tensor with zero elements may be passed as NULL (calls with an empty output return
 *     CSA_OK after the size and dtype checks and launch nothing).
 *   - Return value: CSA_OK or a negative csa_status.  All argument checks run on the host
 *     before anything is launched; an invalid call launches nothing and writes nothing.
 *     CSA_ERR_HIP reports a launch failure (hipGetLastError); faults inside a kernel surface
 *     at the caller's next synchronisation.
 *   - Raw tokens past the last full window (n mod ratio) are not compressed: they belong to
 *     the caller's state cache.
 *   - fp8 means OCP FP8 e4m3fn (max 448, no infinities), one byte per value, scale 1.
 */
#ifndef LIBCSA_CSA_H
#define LIBCSA_CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * CSA_MXFP4 (indexer q / keys only; [N] §2.4: the indexer's QK activations are stored,
 * loaded and multiplied in MXFP4): the OCP Microscaling Formats v1.0 MXFP4 — blocks of 32
 * consecutive values of a row share one E8M0 scale (2^(s-127), s = 255 is NaN), each value
 * is E2M1.  A tensor of R rows of c values (c % 32 == 0) is one buffer: all rows' element
 * bytes first, c/2 per row with value 2i in the low nibble of byte i and 2i+1 in the high
 * nibble, then all rows' scales, c/32 bytes per row (R * (c/2 + c/32) bytes in all).
 */
/*
 * CSA_KV_FP8_BF16 (KV entries of csa_sparse_mqa only; [N] §1.3 and [M] §2.3.4: the KV cache
 * keeps its RoPE dimensions in bf16 and the others in fp8; [N] §1.3 and [M] §2.3.3 item 2:
 * RoPE covers the last 64 dimensions): a row of c values is c - 64 fp8 bytes (dimensions
 * 0 .. c-65), then 64 bf16 values (dimensions c-64 .. c-1): c + 64 bytes per row.
 */
typedef enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8_E4M3 = 2, CSA_MXFP4 = 3, CSA_KV_FP8_BF16 = 4 } csa_dtype;

typedef enum {
    CSA_OK = 0,
    CSA_ERR_INVALID_ARG = -1,  /* null pointer, negative or inconsistent size */
    CSA_ERR_UNSUPPORTED = -2,  /* valid but not implemented: dtype combination or shape limit */
    CSA_ERR_WORKSPACE = -3,    /* workspace pointer null or smaller than the required size */
    CSA_ERR_HIP = -4,          /* the HIP runtime reported an error at launch */
    CSA_ERR_TOO_LARGE = -5     /* csa_index_topk_noalloc: the call needs more than its fixed scratch */
} csa_status;

/* A hipStream_t passed through the C ABI. */
typedef void* csa_stream_t;

/* Shape limits (CSA_ERR_UNSUPPORTED beyond them). */
#define CSA_MAX_RATIO 1024      /* m, m' */
#define CSA_MAX_WIDTH 1024      /* c, c_I: must be a multiple of 8 */
#define CSA_MAX_TOPK 2048       /* k */
#define CSA_MAX_HEADS 256       /* H, H_I */

/*
 * csa_compress — overlapped softmax-weighted compression ([N] §1.1 step 1, eq. C_i^Comp;
 * [M] §2.3.1).  For entry i < N = floor(n/m) and channel d, one softmax per channel taken
 * jointly over the 2m scores
 *     Za[j,d] + Ba[j-mi, d]      for j in [mi, m(i+1))        (window i of stream a)
 *     Zb[j,d] + Bb[j-m(i-1), d]  for j in [m(i-1), mi)        (window i-1 of stream b)
 * weights the matching Ca / Cb values:  out[i,d] = sum_j S_j * C_j.  Entry 0 has no previous
 * window; its weights come from window 0 of stream a alone.
 *   Ca, Cb, Za, Zb : [batch, n, c], dtype in_t (CSA_F32 or CSA_BF16)
 *   Ba, Bb         : [m, c] float32 learned position biases
 *   out            : [batch, floor(n/m), c], dtype out_t (CSA_F32, CSA_BF16 or CSA_FP8_E4M3;
 *                    bf16 and fp8 are rounded to nearest even from the fp32 result, fp8
 *                    saturating at +-448: e.g. fp8 indexer keys)
 * Used for both the KV entries (width c) and the indexer keys (width c_I).
 * Limits: 1 <= m <= CSA_MAX_RATIO, c % 8 == 0, c <= CSA_MAX_WIDTH.  n < m is valid and
 * writes nothing.
 */
int csa_compress(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                 const float* Bb, int64_t batch, int64_t n, int m, int c, csa_dtype in_t, void* out,
                 csa_dtype out_t, csa_stream_t stream);

/*
 * hca_compress — non-overlapping compression for HCA ([N] §1.2 table: m' = 128, no
 * overlap; [M] §2.3.2).  out[i,d] = sum over j in [m'i, m'(i+1)) of softmax_j(Z[j,d] +
 * B[j-m'i, d]) * C[j,d].
 *   C, Z : [batch, n, c], dtype in_t;  B : [m', c] float32;  out : [batch, floor(n/m'), c].
 * Limits as csa_compress.
 */
int hca_compress(const void* C, const void* Z, const float* B, int64_t batch, int64_t n, int m_prime,
                 int c, csa_dtype in_t, void* out, csa_dtype out_t, csa_stream_t stream);

/*
 * csa_index_topk_workspace_size — bytes of device workspace csa_index_topk needs for these
 * sizes (the fp32 score rows plus selection state).  Returns 0 for invalid sizes.
 */
size_t csa_index_topk_workspace_size(int64_t batch, int64_t T, int64_t N, int H_I, int k);

/*
 * csa_index_topk — lightning indexer + per-query top-k ([N] §1.1 step 2, eq. I_{t,s};
 * [M] §2.3.1).  For every query t and visible entry s:
 *     I[t,s] = sum_{h < H_I} w[t,h] * ReLU(qI[t,h,:] . kI[s,:])      (fp32 accumulation,
 *     ReLU(x) = x > 0 ? x : +0), no scale factor.
 * Then keeps the min(k, |visible|) entries with the highest score, ties broken toward the
 * LOWER entry index, and writes them in ASCENDING entry order, padded with -1.
 *   qI : [batch, T, H_I, c_I], kI : [batch, N, c_I], both dtype qk_t (F32, BF16, FP8_E4M3,
 *        or MXFP4 in the layout described at csa_dtype: rows of c_I values, batch*T*H_I
 *        rows in qI and batch*N rows in kI)
 *   w  : [batch, T, H_I] float32
 *   idx        : [batch, T, k] int32 out
 *   sel_scores : [batch, T, k] float32 out, or NULL: the score of each selected entry
 *                (-inf at pads)
 *   workspace  : device scratch of at least csa_index_topk_workspace_size(...) bytes,
 *                16-byte aligned; contents on entry are ignored.
 *   m          : CSA compression ratio (for the visibility rule).
 * Limits: c_I % 8 == 0, c_I <= CSA_MAX_WIDTH, 1 <= H_I <= CSA_MAX_HEADS, 1 <= k <=
 * CSA_MAX_TOPK, N < 2^31.  MXFP4 runs on the matrix-core decode kernel only: T < 4,
 * c_I = 128, H_I = 32 or 64 (else CSA_ERR_UNSUPPORTED); its scales must not be 255 (NaN).
 */
int csa_index_topk(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0,
                   int64_t N, int H_I, int c_I, int m, int k, csa_dtype qk_t, int32_t* idx, float* sel_scores,
                   void* workspace, size_t ws_bytes, csa_stream_t stream);

/*
 * csa_index_topk_noalloc — csa_index_topk for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, arguments and results, without a workspace argument.  Its scratch is a
 * fixed array of CSA_NOALLOC_SCRATCH_BYTES in the library's device code, one copy per GPU,
 * held from the first call on that GPU until the process ends; its address is looked up on
 * the first call on each device (hipGetSymbolAddress, no allocation).  The call runs on the
 * CURRENT device (hipSetDevice), which must be the device of `stream` and of every pointer.
 * No call allocates, frees or synchronises.
 * Every call on a GPU uses that GPU's one scratch array: calls that may overlap on one GPU
 * (on different streams, or from several host threads) RACE and must be serialised by the
 * caller, e.g. by issuing them on one stream.  Nothing is assumed about the array's contents
 * on entry (it keeps the previous call's data).
 * Returns CSA_ERR_TOO_LARGE when csa_index_topk_workspace_size(batch, T, N, H_I, k) exceeds
 * CSA_NOALLOC_SCRATCH_BYTES (about 32 query rows of up to 224,000 entries, or 8 rows of up to
 * 976,000: decode batches of 32 sequences at a 128K-token context and of 8 at a 1M-token
 * context fit; the 8192 query rows of an 8K-token prefill do not),
 * CSA_ERR_HIP when the device or the scratch address cannot be obtained; otherwise as
 * csa_index_topk (argument checks first: an invalid call makes no HIP call at all).
 */
#define CSA_NOALLOC_SCRATCH_BYTES (32u << 20)
int csa_index_topk_noalloc(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0,
                           int64_t N, int H_I, int c_I, int m, int k, csa_dtype qk_t, int32_t* idx, float* sel_scores,
                           csa_stream_t stream);

/*
 * csa_index_scores — the indexer scores alone, as a dense [batch, T, N] float32 matrix
 * (invisible pairs = -inf).  Same arguments and formula as csa_index_topk; meant for
 * parity checks and for callers with their own selection.
 */
int csa_index_scores(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0,
                     int64_t N, int H_I, int c_I, int m, csa_dtype qk_t, float* scores, csa_stream_t stream);

/*
 * csa_topk_workspace_size / csa_topk — the selection step of csa_index_topk alone, over
 * caller-provided fp32 score rows (for callers that produce scores with csa_index_scores
 * or their own kernel).  Same rule as csa_index_topk: per row, among the entries s < nv
 * visible to the query (m(s+1)-1 <= q_pos0 + t), keep the min(k, nv) highest scores, ties
 * toward the lower index, written in ascending index order and padded with -1.
 *   scores : [batch*T rows] fp32, row r starting at scores + r*ld (ld >= N, ld % 4 == 0);
 *            only the first nv entries of each row are read
 *   idx, sel_scores, workspace : as csa_index_topk (sel_scores may be NULL)
 * Limits: 1 <= k <= CSA_MAX_TOPK, N < 2^31.
 */
size_t csa_topk_workspace_size(int64_t batch, int64_t T, int64_t N, int k);
int csa_topk(const float* scores, int64_t ld, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
             int32_t* idx, float* sel_scores, void* workspace, size_t ws_bytes, csa_stream_t stream);

/*
 * csa_sparse_mqa — shared-KV multi-query attention over the selected entries ([N] §1.1
 * step 2, last paragraph; [M] §2.3.2): all H heads of query t attend to the same entries
 * idx[t,:], each entry serving as both key and value:
 *     out[t,h,:] = sum_{s in idx[t]} softmax_s(scale * q[t,h,:] . kv[s,:]) * kv[s,:]
 * (fp32 logits, softmax and accumulation).  Ids outside [0, N) — the -1 pads — are
 * skipped; a query with no valid id gets a zero output.  Ids must be distinct.
 *   q   : [batch, T, H, c]  dtype t (CSA_F32 or CSA_BF16; CSA_BF16 when t = CSA_KV_FP8_BF16)
 *   kv  : [batch, N, c]     dtype t (CSA_KV_FP8_BF16: [batch, N, c + 64] bytes, the mixed rows)
 *   idx : [batch, T, k]     int32
 *   out : [batch, T, H, c]  dtype t (CSA_BF16 when t = CSA_KV_FP8_BF16)
 *   workspace : device scratch of at least csa_sparse_mqa_workspace_size(...) bytes (may be
 *               NULL when that size is 0), 16-byte aligned; holds per-key-range partial
 *               results when a query's keys are split over several workgroups.
 * Limits: c % 8 == 0, c <= CSA_MAX_WIDTH, 1 <= H <= CSA_MAX_HEADS, 1 <= k <= CSA_MAX_TOPK.
 * CSA_KV_FP8_BF16 (c >= 64): decode shapes (c == 512, H % 64 == 0, batch * T * H / 64 <=
 * 256, k <= 1024, no window) run on the matrix cores; every other shape, the window branch
 * and hca_dense_mqa take a vector-ALU kernel (any shape; the prefill and HCA matrix-core
 * paths are compute-bound, where fp8 rows would save no time).  The fp8 values are used
 * exactly; logits, softmax and accumulation stay fp32.
 */
size_t csa_sparse_mqa_workspace_size(int64_t batch, int64_t T, int H, int c, int k, csa_dtype t);
int csa_sparse_mqa(const void* q, const void* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N, int H,
                   int c, int k, float scale, csa_dtype t, void* out, void* workspace, size_t ws_bytes,
                   csa_stream_t stream);

/*
 * hca_dense_mqa — dense causal shared-KV MQA over every visible HCA entry ([M] §2.3.2; [N]
 * §1.2: no selection): for the query at position p, the entries s with m'(s+1)-1 <= p.
 *   q : [batch, T, H, c], kv : [batch, N, c], out : [batch, T, H, c], all dtype t (or
 *   t = CSA_KV_FP8_BF16: kv in the mixed rows of csa_sparse_mqa, q and out bf16).
 * A query that sees no entry gets a zero output.  Limits as csa_sparse_mqa.
 */
int hca_dense_mqa(const void* q, const void* kv, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int H,
                  int c, int m_prime, float scale, csa_dtype t, void* out, csa_stream_t stream);

/*
 * csa_sparse_mqa_sink / hca_dense_mqa_sink — the same attention with an attention sink ([N]
 * §1.3 and [M] §2.3.3 item 4): head h has a learned logit sink[h] (natural-log units, like
 * scale * q . kv) that joins the softmax denominator,
 *     weight_s = exp(z_s) / (sum_r exp(z_r) + exp(sink[h])),
 * so a head may give part of its attention to nothing.  A query with no entry still gets a
 * zero output.  sink: device fp32 [H], 4-byte aligned, or NULL (the plain entry point's
 * result).  Other arguments, dtypes and limits as csa_sparse_mqa / hca_dense_mqa.
 */
int csa_sparse_mqa_sink(const void* q, const void* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N,
                        int H, int c, int k, float scale, const float* sink, csa_dtype t, void* out, void* workspace,
                        size_t ws_bytes, csa_stream_t stream);
int hca_dense_mqa_sink(const void* q, const void* kv, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int H,
                       int c, int m_prime, float scale, const float* sink, csa_dtype t, void* out,
                       csa_stream_t stream);

/*
 * csa_rope — partial rotary position embedding ([N] §1.3 and [M] §2.3.3 item 2: RoPE on the
 * last 64 channels of queries and KV entries; the core attention output gets the rotation of
 * the negative query position, so it reflects the query-to-entry distance), in place:
 *   x : [batch, T, H, c], dtype t (CSA_F32 or CSA_BF16); H = 1 for KV entries.
 * Row (b, t) has position p = pos0 + t * pos_step.  Channel pair (c - d + 2i, c - d + 2i + 1),
 * i < d/2, turns by the angle p * base^(-2i/d) (RoFormer's pairing), or by its negative when
 * inverse != 0 (the output side):  (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).
 * Angles, sines and cosines in double, the products in double, rounded once to dtype t.
 * Limits: d even, 2 <= d <= min(c, 128), c % 8 == 0, c <= CSA_MAX_WIDTH, 1 <= H <=
 * CSA_MAX_HEADS, base > 1.
 */
int csa_rope(void* x, int64_t batch, int64_t T, int H, int c, int d, int64_t pos0, int64_t pos_step, float base,
             int inverse, csa_dtype t, csa_stream_t stream);

/*
 * csa_sparse_mqa_swa — csa_sparse_mqa (with optional sink) plus the sliding-window branch ([N]
 * §1.3 and [M] §2.3.3 item 3: next to the compressed attention, each query also attends to the
 * most recent n_win uncompressed KV tokens, n_win = 128 on the pages): the query at absolute
 * position p = q_pos0 + t attends, in one softmax, to its selected entries idx[t,:] and to the
 * raw rows win_kv[j] whose position win_pos0 + j lies in [p - n_win + 1, p].
 *   win_kv : [batch, W, c] raw KV rows of each sequence (bf16 / fp32 as q; bf16 with
 *            CSA_KV_FP8_BF16 entries), rows at absolute positions win_pos0 .. win_pos0 + W - 1
 *            (a decode step passes its window state; a prefill chunk its own raw KV).  May be
 *            NULL when n_win == 0 or W == 0.
 *   workspace : at least csa_sparse_mqa_workspace_size(batch, T, H, c, k + n_win, t) bytes.
 * Limits: as csa_sparse_mqa; 0 <= n_win <= 1024; N + W < 2^31.
 */
int csa_sparse_mqa_swa(const void* q, const void* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N,
                       int H, int c, int k, float scale, const float* sink, const void* win_kv, int64_t W,
                       int64_t win_pos0, int64_t q_pos0, int n_win, csa_dtype t, void* out, void* workspace,
                       size_t ws_bytes, csa_stream_t stream);

/*
 * csa_compress_step — CSA compression as a decode step ([N] §1.1 step 1; [M] "state cache":
 * the tokens of a block that is not complete yet, and the previous block's, stay uncompressed
 * in a per-request state until the block fills): once block `block` (tokens m*block ..
 * m*block + m - 1) is complete, computes compressed entry `block` exactly as csa_compress
 * would for the whole sequence, and writes it to row `block` of the caller's cache.
 *   Ca, Za, Cb, Zb : the state, [batch, 2m, c] each (the raw tokens of blocks block-1 and
 *                    block, in token order); [batch, m, c] (block `block` only) when block == 0.
 *   Ba, Bb         : [m, c] fp32 position biases.
 *   cache          : [batch, cache_rows, c] dtype out_t; only row `block` of each sequence is
 *                    written.  0 <= block < cache_rows.
 * Dtypes and limits as csa_compress.
 */
int csa_compress_step(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                      const float* Bb, int64_t batch, int64_t block, int m, int c, csa_dtype in_t, void* cache,
                      int64_t cache_rows, csa_dtype out_t, csa_stream_t stream);

/*
 * hca_dense_mqa_swa — hca_dense_mqa (with optional sink) plus the sliding-window branch ([N]
 * §1.3: the window of the most recent n_win uncompressed tokens is given to HCA as well as to
 * CSA; [M] §2.3.3 item 3): the query at absolute position p = q_pos0 + t attends, in one
 * softmax, to every HCA entry it may see (m'(s+1)-1 <= p) and to the raw rows win_kv[j] whose
 * position win_pos0 + j lies in [p - n_win + 1, p].  A raw row whose tokens an entry also
 * covers is still attended to as its own key (the two branches are a plain union).
 *   win_kv : [batch, W, c] raw KV rows (dtype t), rows at absolute positions win_pos0 ..
 *            win_pos0 + W - 1.  May be NULL when n_win == 0 or W == 0.
 * Limits: as hca_dense_mqa; 0 <= n_win <= 1024; N + W < 2^31.
 */
int hca_dense_mqa_swa(const void* q, const void* kv, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int H,
                      int c, int m_prime, float scale, const float* sink, const void* win_kv, int64_t W,
                      int64_t win_pos0, int n_win, csa_dtype t, void* out, csa_stream_t stream);

/*
 * hca_compress_step — HCA compression as a decode step ([N] §1.2: m' = 128, no overlap; [M]
 * "state cache": the raw tokens of a block that is not complete yet stay in a per-request
 * state until the block fills): once block `block` (tokens m'*block .. m'*block + m' - 1) is
 * complete, computes HCA entry `block` exactly as hca_compress would for the whole sequence and
 * writes it to row `block` of the caller's cache.
 *   C, Z  : the state, [batch, m', c] each: the raw tokens of block `block`, in token order
 *   B     : [m', c] fp32 position biases
 *   cache : [batch, cache_rows, c] dtype out_t; only row `block` of each sequence is written.
 *           0 <= block < cache_rows.
 * Dtypes and limits as hca_compress.
 */
int hca_compress_step(const void* C, const void* Z, const float* B, int64_t batch, int64_t block, int m_prime, int c,
                      csa_dtype in_t, void* cache, int64_t cache_rows, csa_dtype out_t, csa_stream_t stream);

/*
 * csa_compress_step_kv_index — the decode-step compression of one CSA layer ([N] §1.1 step 1:
 * the KV entries and the indexer's keys are compressed from the same tokens by the same
 * overlapped softmax pooling, each stream with its own weights; [M] "state cache"): once block
 * `block` is complete, its KV entry and its index-key entry, each exactly as csa_compress_step
 * computes it (the same bits), written to row `block` of the two caches.  One kernel launch
 * when m == 4 (the pages' CSA ratio), else two.
 *   Ca, Cb, Za, Zb, Ba, Bb     : the KV state [batch, 2m, c] ([batch, m, c] when block == 0) and
 *                                [m, c] fp32 biases, as csa_compress_step
 *   kv_cache                   : [batch, kv_rows, c] dtype kv_t
 *   ICa, ICb, IZa, IZb, IBa, IBb : the index-key state [batch, 2m, c_I] (or [batch, m, c_I]) and
 *                                [m, c_I] fp32 biases
 *   ki_cache                   : [batch, ki_rows, c_I] dtype ki_t
 *   in_t                       : dtype of both states (CSA_F32 or CSA_BF16)
 * Limits: as csa_compress_step for each stream; block < kv_rows and block < ki_rows.  Errors
 * are reported before anything is launched.
 */
int csa_compress_step_kv_index(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                               const float* Bb, int c, void* kv_cache, int64_t kv_rows, csa_dtype kv_t,
                               const void* ICa, const void* ICb, const void* IZa, const void* IZb, const float* IBa,
                               const float* IBb, int c_I, void* ki_cache, int64_t ki_rows, csa_dtype ki_t,
                               int64_t batch, int64_t block, int m, csa_dtype in_t, csa_stream_t stream);

/* Human-readable name of a csa_status value (static storage). */
const char* csa_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int csa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBCSA_CSA_H */
