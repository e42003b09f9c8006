// topk.hip — per-query top-k block selection over fp32 indexer scores
// ("DeepSeek-V4: 迈向高效百万级上下文智能", §1.1 step 2: keep the k best compressed blocks per
// query; mlpod.com DeepSeek-V4 summary §2.3.1).
//
// Selection rule: among the visible entries s < nv of a row, keep the min(k, nv) largest
// scores; equal scores are ordered by LOWER index first; the kept ids are written in
// ascending order and padded with -1 (pad scores -inf).  Scores compare as fp32 values
// (+0 == -0) through an order-preserving uint32 key.
//
// One workgroup of 1024 threads per row:
//   A  min / max of the row                          (one read of the row)
//   B  2048-bin histogram, bins LINEAR in value       (one read; spreads the atomics,
//      unlike a radix digit of the float bit pattern, where almost all scores share the
//      top byte and every atomic hits one bin)
//   C  the bin b* holding the k-th largest value; its members are gathered to LDS and the
//      exact k-th (value desc, index asc) is found by ranking (one read)
//      — if b* holds more than kCap members (heavy ties), an exact 8-bit radix select on
//      the order keys restricted to b* runs instead (four reads).
//   D  ordered compaction: keep s iff key > K* or (key == K* and it is among the first
//      `need_eq` such s), written at its prefix-sum position (one read).
#include "device_common.h"
#include "launch.h"

namespace csa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 2048;
constexpr int kCap = 4096;

struct TopkShared {
    uint32_t hist[kBins];
    float cval[kCap];
    int32_t cidx[kCap];
    float red_lo[kWaves], red_hi[kWaves];
    uint32_t wsum[kWaves];
    uint32_t wsum2[kWaves];
    float lo, inv;
    int bstar;
    uint32_t need;        // how many of bin b* to take
    uint32_t ncand;
    uint32_t kstar;       // order key of the k-th element
    uint32_t need_eq;     // how many entries with key == kstar to take (lowest indices)
    uint32_t prefix, pmask;
};

__device__ __forceinline__ int bin_of(float v, float lo, float inv) {
    float x = (v - lo) * inv;
    x = fminf(fmaxf(x, 0.f), (float)(kBins - 1));
    return (int)x;
}

// Inclusive prefix within the block of a per-thread count; returns exclusive prefix and
// writes the block total to *total.  Uses `buf` (kWaves entries).
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* buf, uint32_t* total) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    uint32_t inc = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        uint32_t y = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += y;
    }
    if (lane == kWave - 1) buf[wid] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int i = 0; i < kWaves; ++i) {
        const uint32_t v = buf[i];
        before += (i < wid) ? v : 0u;
        all += v;
    }
    __syncthreads();
    *total = all;
    return before + inc - x;
}

__global__ void __launch_bounds__(kThreads)
topk_row_kernel(const float* __restrict__ scores, int64_t ld, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
                int32_t* __restrict__ idx, float* __restrict__ sel) {
    __shared__ TopkShared sh;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    const int64_t row = blockIdx.x;
    const int64_t t = row % T;
    const int64_t nv = visible_entries(q_pos0 + t, m, N);
    const float* sc = scores + row * ld;
    int32_t* oi = idx + row * k;
    float* os = sel ? sel + row * k : nullptr;

    if (nv <= k) {   // everything visible is kept
        for (int r = tid; r < k; r += kThreads) {
            oi[r] = r < nv ? r : -1;
            if (os) os[r] = r < nv ? sc[r] : -INFINITY;
        }
        return;
    }

    // ---- A: min / max
    float lo = INFINITY, hi = -INFINITY;
    for (int64_t s = tid; s < nv; s += kThreads) {
        const float v = sc[s];
        lo = fminf(lo, v);
        hi = fmaxf(hi, v);
    }
    lo = -wave_max(-lo);
    hi = wave_max(hi);
    if (lane == 0) { sh.red_lo[wid] = lo; sh.red_hi[wid] = hi; }
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
    __syncthreads();
    if (tid == 0) {
        float l = sh.red_lo[0], h = sh.red_hi[0];
        for (int i = 1; i < kWaves; ++i) { l = fminf(l, sh.red_lo[i]); h = fmaxf(h, sh.red_hi[i]); }
        float inv = (float)kBins / (h - l);
        if (!(h > l) || !isfinite(inv)) inv = 0.f;
        sh.lo = l;
        sh.inv = inv;
        sh.ncand = 0u;
        sh.bstar = 0;              // always overwritten below (the bin counts sum to nv > k)
        sh.need = (uint32_t)k;
    }
    __syncthreads();
    lo = sh.lo;
    const float inv = sh.inv;

    // ---- B: histogram
    for (int64_t s = tid; s < nv; s += kThreads) atomicAdd(&sh.hist[bin_of(sc[s], lo, inv)], 1u);
    __syncthreads();

    // find b*: bins scanned from the top; wave 0 does it, 32 bins per lane
    if (wid == 0) {
        const int per = kBins / kWave;          // 32
        const int top = kBins - 1 - lane * per;  // lane 0 owns the highest bins
        uint32_t mine = 0;
        for (int j = 0; j < per; ++j) mine += sh.hist[top - j];
        uint32_t inc = mine;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            uint32_t y = __shfl_up(inc, off, kWave);
            if (lane >= off) inc += y;
        }
        const uint32_t before = inc - mine;
        if (before < (uint32_t)k && inc >= (uint32_t)k) {   // exactly one lane
            uint32_t acc = before;
            for (int j = 0; j < per; ++j) {
                const uint32_t h = sh.hist[top - j];
                if (acc + h >= (uint32_t)k) {
                    sh.bstar = top - j;
                    sh.need = (uint32_t)k - acc;
                    break;
                }
                acc += h;
            }
        }
    }
    __syncthreads();
    const int bstar = sh.bstar;
    const uint32_t need = sh.need;
    const uint32_t cnt_star = sh.hist[bstar];

    if (cnt_star <= (uint32_t)kCap) {
        // ---- C: gather bin b* and rank its members
        for (int64_t s = tid; s < nv; s += kThreads) {
            const float v = sc[s];
            if (bin_of(v, lo, inv) == bstar) {
                const uint32_t p = atomicAdd(&sh.ncand, 1u);
                if (p < (uint32_t)kCap) {   // always true: b* holds cnt_star <= kCap members
                    sh.cval[p] = v;
                    sh.cidx[p] = (int32_t)s;
                }
            }
        }
        __syncthreads();
        const uint32_t nc = min(sh.ncand, (uint32_t)kCap);
        for (uint32_t i = tid; i < nc; i += kThreads) {
            const uint32_t ki = order_key(sh.cval[i]);
            const int32_t si = sh.cidx[i];
            uint32_t rank = 0;
            for (uint32_t j = 0; j < nc; ++j) {
                const uint32_t kj = order_key(sh.cval[j]);
                rank += (kj > ki || (kj == ki && sh.cidx[j] < si)) ? 1u : 0u;
            }
            if (rank == need - 1) sh.kstar = ki;
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t gt = 0;
            for (uint32_t j = 0; j < nc; ++j) gt += order_key(sh.cval[j]) > sh.kstar ? 1u : 0u;
            sh.need_eq = need - gt;
        }
        __syncthreads();
    } else {
        // ---- C': exact radix select (8-bit digits of the order key) restricted to bin b*
        if (tid == 0) { sh.prefix = 0u; sh.pmask = 0u; sh.need_eq = need; }
        __syncthreads();
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kThreads) sh.hist[i] = 0u;
            __syncthreads();
            const uint32_t prefix = sh.prefix, pmask = sh.pmask;
            for (int64_t s = tid; s < nv; s += kThreads) {
                const float v = sc[s];
                if (bin_of(v, lo, inv) != bstar) continue;
                const uint32_t key = order_key(v);
                if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                uint32_t remaining = sh.need_eq, acc = 0;
                for (int d = 255; d >= 0; --d) {
                    const uint32_t h = sh.hist[d];
                    if (acc + h >= remaining) {
                        sh.prefix = prefix | ((uint32_t)d << shift);
                        sh.pmask = pmask | (255u << shift);
                        sh.need_eq = remaining - acc;
                        break;
                    }
                    acc += h;
                }
            }
            __syncthreads();
        }
        if (tid == 0) sh.kstar = sh.prefix;
        __syncthreads();
    }

    // ---- D: ordered compaction
    const uint32_t kstar = sh.kstar, need_eq = sh.need_eq;
    uint32_t taken = 0, eq_seen = 0;
    for (int64_t base = 0; base < nv; base += kThreads) {
        const int64_t s = base + tid;
        float v = 0.f;
        uint32_t key = 0u;
        if (s < nv) { v = sc[s]; key = order_key(v); }
        const uint32_t is_eq = (s < nv && key == kstar) ? 1u : 0u;
        uint32_t eq_total;
        const uint32_t eq_rank = eq_seen + block_exclusive_scan(is_eq, sh.wsum, &eq_total);
        const uint32_t take = (s < nv && (key > kstar || (is_eq && eq_rank < need_eq))) ? 1u : 0u;
        uint32_t take_total;
        const uint32_t pos = taken + block_exclusive_scan(take, sh.wsum2, &take_total);
        if (take && pos < (uint32_t)k) {
            oi[pos] = (int32_t)s;
            if (os) os[pos] = v;
        }
        taken += take_total;
        eq_seen += eq_total;
        if (taken >= (uint32_t)k) break;   // uniform across the block
    }
    for (int64_t r = (int64_t)taken + tid; r < k; r += kThreads) {   // defensive: unreachable when nv > k
        oi[r] = -1;
        if (os) os[r] = -INFINITY;
    }
}

}  // namespace

size_t topk_extra_workspace(int64_t rows, int64_t N, int k) {
    (void)rows;
    (void)N;
    (void)k;
    return 0;
}

int launch_topk(const float* scores, int64_t ld, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
                int32_t* idx, float* sel, void* extra_ws, hipStream_t stream) {
    (void)extra_ws;
    const int64_t rows = batch * T;
    if (rows == 0) return 0;
    if (rows > 0x7fffffffLL) return -2;
    hipLaunchKernelGGL(topk_row_kernel, dim3((unsigned)rows), dim3(kThreads), 0, stream, scores, ld, T, q_pos0, N, m, k,
                       idx, sel);
    return 0;
}

}  // namespace csa
