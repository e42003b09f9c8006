// api.cpp — the C ABI of libcsa (declared in include/csa.h): host-side argument checks, then
// dispatch to the kernel launchers.  Nothing here allocates, synchronises or keeps state.
// Every check runs before the first HIP call, so an invalid call never touches the device.
#include <math.h>

#include <atomic>
#include <mutex>

#include "../../include/csa.h"
#include "launch.h"

// Scratch of csa_index_topk_noalloc: one copy per GPU the library runs on, kept until the
// process ends.  On the host this name is only a stand-in symbol, never a device address:
// host code uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kVersion = 100;   // 0.1.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool width_ok(int c) { return c > 0 && c % 8 == 0 && c <= CSA_MAX_WIDTH; }

bool io_dtype(csa_dtype t) { return t == CSA_F32 || t == CSA_BF16; }

// compressed entries may also be stored as fp8 (e.g. indexer keys)
bool compress_out_dtype(csa_dtype t) { return io_dtype(t) || t == CSA_FP8_E4M3; }

int finish(int rc) {
    if (rc == -2) return CSA_ERR_UNSUPPORTED;
    if (rc != 0) return CSA_ERR_INVALID_ARG;
    return hipGetLastError() == hipSuccess ? CSA_OK : CSA_ERR_HIP;
}

// Row stride (floats) of the score workspace: N rounded up to 4 so rows stay 16-byte aligned.
int64_t score_ld(int64_t N) { return (N + 3) & ~int64_t(3); }

constexpr size_t kWsAlign = 256;
size_t round_up(size_t x) { return (x + kWsAlign - 1) & ~(kWsAlign - 1); }

int check_indexer(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0, int64_t N,
                  int H_I, int c_I, int m, csa_dtype qk_t) {
    if (batch < 0 || T < 0 || N < 0 || q_pos0 < 0) return CSA_ERR_INVALID_ARG;
    if (m < 1 || H_I < 1 || c_I < 1) return CSA_ERR_INVALID_ARG;
    if (qk_t != CSA_F32 && qk_t != CSA_BF16 && qk_t != CSA_FP8_E4M3 && qk_t != CSA_MXFP4) return CSA_ERR_UNSUPPORTED;
    if (!width_ok(c_I) || H_I > CSA_MAX_HEADS || m > CSA_MAX_RATIO) return CSA_ERR_UNSUPPORTED;
    // MXFP4: the matrix-core decode kernel only (c_I = 128: four scale blocks per row)
    if (qk_t == CSA_MXFP4 && (T >= 4 || c_I != 128 || (H_I != 32 && H_I != 64))) return CSA_ERR_UNSUPPORTED;
    if (N >= (int64_t(1) << 31)) return CSA_ERR_UNSUPPORTED;
    if (batch * T == 0) return CSA_OK;   // nothing to compute: pointers may be NULL
    if (!qI || !w || (N > 0 && !kI)) return CSA_ERR_INVALID_ARG;
    if (!aligned16(qI) || !aligned16(kI) || !aligned16(w)) return CSA_ERR_INVALID_ARG;
    return CSA_OK;
}

int check_mqa(const void* q, const void* kv, void* out, int64_t batch, int64_t T, int64_t N, int H, int c, float scale,
              csa_dtype t) {
    if (batch < 0 || T < 0 || N < 0 || H < 1 || c < 1) return CSA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return CSA_ERR_INVALID_ARG;
    if (!io_dtype(t)) return CSA_ERR_UNSUPPORTED;
    if (!width_ok(c) || H > CSA_MAX_HEADS) return CSA_ERR_UNSUPPORTED;
    if (batch * T == 0) return CSA_OK;   // nothing to compute: pointers may be NULL
    if (!q || (N > 0 && !kv) || !out) return CSA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(out)) return CSA_ERR_INVALID_ARG;
    return CSA_OK;
}

}  // namespace

extern "C" {

const char* csa_status_string(int status) {
    switch (status) {
        case CSA_OK: return "CSA_OK";
        case CSA_ERR_INVALID_ARG: return "CSA_ERR_INVALID_ARG: null pointer, misalignment or inconsistent size";
        case CSA_ERR_UNSUPPORTED: return "CSA_ERR_UNSUPPORTED: dtype or shape outside the implemented limits";
        case CSA_ERR_WORKSPACE: return "CSA_ERR_WORKSPACE: workspace missing or too small";
        case CSA_ERR_HIP: return "CSA_ERR_HIP: the HIP runtime reported a launch error";
        case CSA_ERR_TOO_LARGE:
            return "CSA_ERR_TOO_LARGE: the call needs more scratch than the allocation-free entry point holds";
        default: return "unknown csa_status";
    }
}

int csa_version(void) { return kVersion; }

int csa_compress(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba, const float* Bb,
                 int64_t batch, int64_t n, int m, int c, csa_dtype in_t, void* out, csa_dtype out_t,
                 csa_stream_t stream) {
    if (batch < 0 || n < 0 || m < 1 || c < 1) return CSA_ERR_INVALID_ARG;
    if (!io_dtype(in_t) || !compress_out_dtype(out_t)) return CSA_ERR_UNSUPPORTED;
    if (!width_ok(c) || m > CSA_MAX_RATIO) return CSA_ERR_UNSUPPORTED;
    if (batch == 0 || n / m == 0) return CSA_OK;   // empty output: pointers may be NULL
    if (!Ca || !Cb || !Za || !Zb || !Ba || !Bb || !out) return CSA_ERR_INVALID_ARG;
    if (!aligned16(Ca) || !aligned16(Cb) || !aligned16(Za) || !aligned16(Zb) || !aligned16(Ba) || !aligned16(Bb) ||
        !aligned16(out))
        return CSA_ERR_INVALID_ARG;
    return finish(csa::launch_compress(Ca, Za, Ba, Cb, Zb, Bb, batch, n, m, c, in_t, out, out_t,
                                       static_cast<hipStream_t>(stream)));
}

namespace {
// the checks of csa_compress_step for one stream (CSA_OK: valid)
int step_stream_status(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                       const float* Bb, int64_t batch, int64_t block, int m, int c, csa_dtype in_t, const void* cache,
                       int64_t cache_rows, csa_dtype out_t) {
    if (batch < 0 || block < 0 || m < 1 || c < 1 || cache_rows <= block) return CSA_ERR_INVALID_ARG;
    if (!io_dtype(in_t) || !compress_out_dtype(out_t)) return CSA_ERR_UNSUPPORTED;
    if (!width_ok(c) || m > CSA_MAX_RATIO) return CSA_ERR_UNSUPPORTED;
    if (batch == 0) return CSA_OK;
    if (!Ca || !Za || !Ba || !cache || (block > 0 && (!Cb || !Zb || !Bb))) return CSA_ERR_INVALID_ARG;
    if (!aligned16(Ca) || !aligned16(Za) || !aligned16(Ba) || !aligned16(cache) ||
        (block > 0 && (!aligned16(Cb) || !aligned16(Zb) || !aligned16(Bb))))
        return CSA_ERR_INVALID_ARG;
    return CSA_OK;
}
}  // namespace

int csa_compress_step(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                      const float* Bb, int64_t batch, int64_t block, int m, int c, csa_dtype in_t, void* cache,
                      int64_t cache_rows, csa_dtype out_t, csa_stream_t stream) {
    const int rc = step_stream_status(Ca, Cb, Za, Zb, Ba, Bb, batch, block, m, c, in_t, cache, cache_rows, out_t);
    if (rc != CSA_OK || batch == 0) return rc;
    return finish(csa::launch_compress_step(Ca, Za, Ba, block > 0 ? Cb : Ca, block > 0 ? Zb : Za, block > 0 ? Bb : Ba,
                                            batch, block, m, c, in_t, cache, cache_rows, out_t,
                                            static_cast<hipStream_t>(stream)));
}

int csa_compress_step_kv_index(const void* Ca, const void* Cb, const void* Za, const void* Zb, const float* Ba,
                               const float* Bb, int c, void* kv_cache, int64_t kv_rows, csa_dtype kv_t,
                               const void* ICa, const void* ICb, const void* IZa, const void* IZb, const float* IBa,
                               const float* IBb, int c_I, void* ki_cache, int64_t ki_rows, csa_dtype ki_t,
                               int64_t batch, int64_t block, int m, csa_dtype in_t, csa_stream_t stream) {
    int rc = step_stream_status(Ca, Cb, Za, Zb, Ba, Bb, batch, block, m, c, in_t, kv_cache, kv_rows, kv_t);
    if (rc != CSA_OK) return rc;
    rc = step_stream_status(ICa, ICb, IZa, IZb, IBa, IBb, batch, block, m, c_I, in_t, ki_cache, ki_rows, ki_t);
    if (rc != CSA_OK) return rc;
    if (batch == 0) return CSA_OK;
    // (block 0: the one-block state stands in for the missing previous block, which is masked)
    const csa::StepStreams kv{Ca, Za, Ba, block > 0 ? Cb : Ca, block > 0 ? Zb : Za, block > 0 ? Bb : Ba,
                              c, kv_cache, kv_rows, kv_t};
    const csa::StepStreams ki{ICa, IZa, IBa, block > 0 ? ICb : ICa, block > 0 ? IZb : IZa, block > 0 ? IBb : IBa,
                              c_I, ki_cache, ki_rows, ki_t};
    return finish(csa::launch_compress_step_pair(kv, ki, batch, block, m, in_t, static_cast<hipStream_t>(stream)));
}

int hca_compress(const void* C, const void* Z, const float* B, int64_t batch, int64_t n, int m_prime, int c,
                 csa_dtype in_t, void* out, csa_dtype out_t, csa_stream_t stream) {
    if (batch < 0 || n < 0 || m_prime < 1 || c < 1) return CSA_ERR_INVALID_ARG;
    if (!io_dtype(in_t) || !compress_out_dtype(out_t)) return CSA_ERR_UNSUPPORTED;
    if (!width_ok(c) || m_prime > CSA_MAX_RATIO) return CSA_ERR_UNSUPPORTED;
    if (batch == 0 || n / m_prime == 0) return CSA_OK;   // empty output: pointers may be NULL
    if (!C || !Z || !B || !out) return CSA_ERR_INVALID_ARG;
    if (!aligned16(C) || !aligned16(Z) || !aligned16(B) || !aligned16(out)) return CSA_ERR_INVALID_ARG;
    return finish(csa::launch_compress(C, Z, B, nullptr, nullptr, nullptr, batch, n, m_prime, c, in_t, out, out_t,
                                       static_cast<hipStream_t>(stream)));
}

// Workspace of csa_index_topk: the fp32 score rows, then room for the indexer's per-chunk
// (min, max) pairs, then whatever the selection needs.  The chunk region is sized for the
// largest chunk count any shape/dtype could use (csa::max_index_chunks).
size_t chunk_region(int64_t rows, int64_t N) {
    return round_up((size_t)rows * (size_t)csa::max_index_chunks(N) * 2 * sizeof(float));
}

// Group maxima for the group-bounded selection (decode-shaped calls, T < 4): at most
// csa::kTopkMaxGroups per row.
size_t group_region(int64_t rows, int64_t T, int64_t N, int k) {
    if (T >= 4 || N <= k) return 0;
    return round_up((size_t)rows * (size_t)csa::kTopkMaxGroups * sizeof(float));
}

size_t csa_index_topk_workspace_size(int64_t batch, int64_t T, int64_t N, int H_I, int k) {
    if (batch < 0 || T < 0 || N < 0 || H_I < 1 || k < 1) return 0;
    const int64_t rows = batch * T;
    const size_t scores = round_up((size_t)rows * (size_t)score_ld(N) * sizeof(float));
    return scores + chunk_region(rows, N) + round_up(csa::topk_extra_workspace(rows, N, k)) +
           group_region(rows, T, N, k) + kWsAlign;
}

// The argument checks of csa_index_topk other than the workspace's.
int check_index_topk(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0,
                     int64_t N, int H_I, int c_I, int m, int k, csa_dtype qk_t, const int32_t* idx,
                     const float* sel_scores) {
    int rc = check_indexer(qI, w, kI, batch, T, q_pos0, N, H_I, c_I, m, qk_t);
    if (rc != CSA_OK) return rc;
    if (k < 1) return CSA_ERR_INVALID_ARG;
    if (k > CSA_MAX_TOPK) return CSA_ERR_UNSUPPORTED;
    if (batch == 0 || T == 0) return CSA_OK;
    if (!idx) return CSA_ERR_INVALID_ARG;
    if (sel_scores && !aligned16(sel_scores)) return CSA_ERR_INVALID_ARG;
    return CSA_OK;
}

int csa_index_topk(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0, int64_t N,
                   int H_I, int c_I, int m, int k, csa_dtype qk_t, int32_t* idx, float* sel_scores, void* workspace,
                   size_t ws_bytes, csa_stream_t stream) {
    int rc = check_index_topk(qI, w, kI, batch, T, q_pos0, N, H_I, c_I, m, k, qk_t, idx, sel_scores);
    if (rc != CSA_OK || batch == 0 || T == 0) return rc;
    const size_t need = csa_index_topk_workspace_size(batch, T, N, H_I, k);
    if (!workspace || ws_bytes < need || !aligned16(workspace)) return CSA_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t ld = score_ld(N);
    float* scores = static_cast<float*>(workspace);
    const int64_t rows = batch * T;
    float* chunk_mm = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                               round_up((size_t)rows * (size_t)ld * sizeof(float)));
    void* extra = reinterpret_cast<char*>(chunk_mm) + chunk_region(rows, N);
    int64_t nv_max = (q_pos0 + T) / m;
    if (nv_max > N) nv_max = N;
    // the decode-shaped indexer clears the selection's per-row counters when it will use them
    const int n_chunks = csa::index_chunks(batch, T, N, H_I, c_I, qk_t);
    if (n_chunks > csa::max_index_chunks(N)) return CSA_ERR_UNSUPPORTED;   // would overrun the chunk region
    // the decode-shaped indexer (n_chunks > 0) also writes group maxima when the selection can
    // use them; otherwise it clears the multi-workgroup selection's per-row counters if needed
    const int G = n_chunks > 0 && group_region(rows, T, N, k) > 0 ? csa::topk_group(nv_max, k) : 0;
    // (rows of group maxima start 16-byte aligned: a multiple of 4, <= kTopkMaxGroups)
    const int64_t gld = G > 0 ? ((nv_max + G - 1) / G + 3) & ~int64_t(3) : 0;
    float* gmax = G > 0 ? reinterpret_cast<float*>(static_cast<char*>(extra) +
                                                   round_up(csa::topk_extra_workspace(rows, N, k)))
                        : nullptr;
    // (the per-row counters of the multi-workgroup selections: with or without group maxima)
    const int zero_words = n_chunks > 0 ? csa::topk_zero_words(rows, nv_max) : 0;
    uint32_t* zero = zero_words > 0 ? csa::topk_zero_region(extra, rows, N) : nullptr;
    int n_chunk_mm = 0;
    rc = csa::launch_index_scores(qI, w, kI, batch, T, q_pos0, N, H_I, c_I, m, qk_t, scores, ld, false, chunk_mm,
                                  &n_chunk_mm, zero, zero_words, gmax, G, gld, st);
    if (rc != 0) return finish(rc);
    return finish(csa::launch_topk(scores, ld, batch, T, q_pos0, N, m, k, idx, sel_scores,
                                   n_chunk_mm > 0 ? chunk_mm : nullptr, n_chunk_mm, gmax, G, gld,
                                   zero_words > 0 ? extra : nullptr, st));
}

// ---- allocation-free variant: the workspace is this device's copy of `scratch`
namespace {
constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`, looked up once per device.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return CSA_ERR_HIP;
    }
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
                (void)hipGetLastError();
                return CSA_ERR_HIP;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return CSA_OK;
}
}  // namespace

int csa_index_topk_noalloc(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0,
                           int64_t N, int H_I, int c_I, int m, int k, csa_dtype qk_t, int32_t* idx, float* sel_scores,
                           csa_stream_t stream) {
    int rc = check_index_topk(qI, w, kI, batch, T, q_pos0, N, H_I, c_I, m, k, qk_t, idx, sel_scores);
    if (rc != CSA_OK || batch == 0 || T == 0) return rc;
    if (csa_index_topk_workspace_size(batch, T, N, H_I, k) > CSA_NOALLOC_SCRATCH_BYTES) return CSA_ERR_TOO_LARGE;
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != CSA_OK) return rc;
    return csa_index_topk(qI, w, kI, batch, T, q_pos0, N, H_I, c_I, m, k, qk_t, idx, sel_scores, ws,
                          CSA_NOALLOC_SCRATCH_BYTES, stream);
}

int csa_index_scores(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0, int64_t N,
                     int H_I, int c_I, int m, csa_dtype qk_t, float* scores, csa_stream_t stream) {
    int rc = check_indexer(qI, w, kI, batch, T, q_pos0, N, H_I, c_I, m, qk_t);
    if (rc != CSA_OK) return rc;
    if (batch == 0 || T == 0 || N == 0) return CSA_OK;
    if (!scores) return CSA_ERR_INVALID_ARG;
    return finish(csa::launch_index_scores(qI, w, kI, batch, T, q_pos0, N, H_I, c_I, m, qk_t, scores, N, true, nullptr,
                                           nullptr, nullptr, 0, nullptr, 0, 0, static_cast<hipStream_t>(stream)));
}

size_t csa_topk_workspace_size(int64_t batch, int64_t T, int64_t N, int k) {
    if (batch < 0 || T < 0 || N < 0 || k < 1) return 0;
    return round_up(csa::topk_extra_workspace(batch * T, N, k)) + kWsAlign;
}

int csa_topk(const float* scores, int64_t ld, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
             int32_t* idx, float* sel_scores, void* workspace, size_t ws_bytes, csa_stream_t stream) {
    if (batch < 0 || T < 0 || N < 0 || q_pos0 < 0 || m < 1 || k < 1 || ld < N || ld % 4 != 0)
        return CSA_ERR_INVALID_ARG;
    if (k > CSA_MAX_TOPK || m > CSA_MAX_RATIO || N >= (int64_t(1) << 31)) return CSA_ERR_UNSUPPORTED;
    if (batch == 0 || T == 0) return CSA_OK;
    if (!idx || (N > 0 && !scores) || !aligned16(scores)) return CSA_ERR_INVALID_ARG;
    if (sel_scores && !aligned16(sel_scores)) return CSA_ERR_INVALID_ARG;
    if (!workspace || ws_bytes < csa_topk_workspace_size(batch, T, N, k) || !aligned16(workspace))
        return CSA_ERR_WORKSPACE;
    return finish(csa::launch_topk(scores, ld, batch, T, q_pos0, N, m, k, idx, sel_scores, nullptr, 0, nullptr, 0, 0,
                                   nullptr, static_cast<hipStream_t>(stream)));
}

size_t csa_sparse_mqa_workspace_size(int64_t batch, int64_t T, int H, int c, int k, csa_dtype t) {
    if (batch < 0 || T < 0 || H < 1 || c < 1 || k < 1) return 0;
    return csa::sparse_mqa_workspace(batch, T, H, c, k, t);
}

int csa_sparse_mqa(const void* q, const void* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N, int H, int c,
                   int k, float scale, csa_dtype t, void* out, void* workspace, size_t ws_bytes, csa_stream_t stream) {
    return csa_sparse_mqa_sink(q, kv, idx, batch, T, N, H, c, k, scale, nullptr, t, out, workspace, ws_bytes, stream);
}

int csa_sparse_mqa_sink(const void* q, const void* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N, int H,
                        int c, int k, float scale, const float* sink, csa_dtype t, void* out, void* workspace,
                        size_t ws_bytes, csa_stream_t stream) {
    return csa_sparse_mqa_swa(q, kv, idx, batch, T, N, H, c, k, scale, sink, nullptr, 0, 0, 0, 0, t, out, workspace,
                              ws_bytes, stream);
}

int csa_sparse_mqa_swa(const void* q, const void* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N, int H,
                       int c, int k, float scale, const float* sink, const void* win_kv, int64_t W, int64_t win_pos0,
                       int64_t q_pos0, int n_win, csa_dtype t, void* out, void* workspace, size_t ws_bytes,
                       csa_stream_t stream) {
    if (sink && (reinterpret_cast<uintptr_t>(sink) & 3u)) return CSA_ERR_INVALID_ARG;
    if (n_win < 0 || W < 0 || win_pos0 < 0 || q_pos0 < 0) return CSA_ERR_INVALID_ARG;
    if (n_win > 1024) return CSA_ERR_UNSUPPORTED;
    if (n_win > 0 && W > 0 && (!win_kv || !aligned16(win_kv))) return CSA_ERR_INVALID_ARG;
    if (N + W >= (int64_t(1) << 31)) return CSA_ERR_UNSUPPORTED;   // one 32-bit id space
    const bool mixed = t == CSA_KV_FP8_BF16;   // q and out are bf16 then
    int rc = check_mqa(q, kv, out, batch, T, N, H, c, scale, mixed ? CSA_BF16 : t);
    if (rc != CSA_OK) return rc;
    if (k < 1) return CSA_ERR_INVALID_ARG;
    if (k > CSA_MAX_TOPK) return CSA_ERR_UNSUPPORTED;
    if (mixed && c < 64) return CSA_ERR_UNSUPPORTED;   // the last 64 channels are the bf16 part
    if (batch == 0 || T == 0) return CSA_OK;
    if (!idx) return CSA_ERR_INVALID_ARG;
    const size_t need = csa_sparse_mqa_workspace_size(batch, T, H, c, k + n_win, t);
    if (need > 0 && (!workspace || ws_bytes < need || !aligned16(workspace))) return CSA_ERR_WORKSPACE;
    const csa::SwaArgs swa{n_win > 0 ? win_kv : nullptr, n_win > 0 ? W : 0, win_pos0, q_pos0, n_win};
    return finish(csa::launch_sparse_mqa(q, kv, idx, batch, T, N, H, c, k, scale, t, out, workspace, sink, swa,
                                         static_cast<hipStream_t>(stream)));
}

int csa_rope(void* x, int64_t batch, int64_t T, int H, int c, int d, int64_t pos0, int64_t pos_step, float base,
             int inverse, csa_dtype t, csa_stream_t stream) {
    if (batch < 0 || T < 0 || H < 1 || c < 1 || d < 2 || d % 2 != 0 || d > c) return CSA_ERR_INVALID_ARG;
    if (!(base > 1.f) || !isfinite(base)) return CSA_ERR_INVALID_ARG;
    if (!io_dtype(t)) return CSA_ERR_UNSUPPORTED;
    if (!width_ok(c) || H > CSA_MAX_HEADS || d > 128) return CSA_ERR_UNSUPPORTED;
    if (batch * T == 0) return CSA_OK;
    if (!x || !aligned16(x)) return CSA_ERR_INVALID_ARG;
    return finish(csa::launch_rope(x, batch, T, H, c, d, pos0, pos_step, base, inverse != 0, t,
                                   static_cast<hipStream_t>(stream)));
}

int hca_dense_mqa(const void* q, const void* kv, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int H, int c,
                  int m_prime, float scale, csa_dtype t, void* out, csa_stream_t stream) {
    return hca_dense_mqa_sink(q, kv, batch, T, q_pos0, N, H, c, m_prime, scale, nullptr, t, out, stream);
}

int hca_dense_mqa_sink(const void* q, const void* kv, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int H, int c,
                       int m_prime, float scale, const float* sink, csa_dtype t, void* out, csa_stream_t stream) {
    return hca_dense_mqa_swa(q, kv, batch, T, q_pos0, N, H, c, m_prime, scale, sink, nullptr, 0, 0, 0, t, out, stream);
}

int hca_dense_mqa_swa(const void* q, const void* kv, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int H, int c,
                      int m_prime, float scale, const float* sink, const void* win_kv, int64_t W, int64_t win_pos0,
                      int n_win, csa_dtype t, void* out, csa_stream_t stream) {
    if (sink && (reinterpret_cast<uintptr_t>(sink) & 3u)) return CSA_ERR_INVALID_ARG;
    if (n_win < 0 || W < 0 || win_pos0 < 0) return CSA_ERR_INVALID_ARG;
    if (n_win > 1024) return CSA_ERR_UNSUPPORTED;
    if (n_win > 0 && W > 0 && (!win_kv || !aligned16(win_kv))) return CSA_ERR_INVALID_ARG;
    if (N + W >= (int64_t(1) << 31)) return CSA_ERR_UNSUPPORTED;   // one 32-bit id space
    const bool mixed = t == CSA_KV_FP8_BF16;   // q, out and window rows are bf16 then
    if (mixed && c < 64) return CSA_ERR_UNSUPPORTED;
    int rc = check_mqa(q, kv, out, batch, T, N, H, c, scale, mixed ? CSA_BF16 : t);
    if (rc != CSA_OK) return rc;
    if (m_prime < 1 || q_pos0 < 0) return CSA_ERR_INVALID_ARG;
    if (m_prime > CSA_MAX_RATIO) return CSA_ERR_UNSUPPORTED;
    if (batch == 0 || T == 0) return CSA_OK;
    const csa::SwaArgs swa{n_win > 0 ? win_kv : nullptr, n_win > 0 ? W : 0, win_pos0, q_pos0, n_win};
    return finish(csa::launch_dense_mqa(q, kv, batch, T, q_pos0, N, H, c, m_prime, scale, t, out, sink, swa,
                                        static_cast<hipStream_t>(stream)));
}

int hca_compress_step(const void* C, const void* Z, const float* B, int64_t batch, int64_t block, int m_prime, int c,
                      csa_dtype in_t, void* cache, int64_t cache_rows, csa_dtype out_t, csa_stream_t stream) {
    if (batch < 0 || block < 0 || m_prime < 1 || c < 1 || cache_rows <= block) return CSA_ERR_INVALID_ARG;
    if (!io_dtype(in_t) || !compress_out_dtype(out_t)) return CSA_ERR_UNSUPPORTED;
    if (!width_ok(c) || m_prime > CSA_MAX_RATIO) return CSA_ERR_UNSUPPORTED;
    if (batch == 0) return CSA_OK;
    if (!C || !Z || !B || !cache) return CSA_ERR_INVALID_ARG;
    if (!aligned16(C) || !aligned16(Z) || !aligned16(B) || !aligned16(cache)) return CSA_ERR_INVALID_ARG;
    return finish(csa::launch_hca_compress_step(C, Z, B, batch, block, m_prime, c, in_t, cache, cache_rows, out_t,
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"
