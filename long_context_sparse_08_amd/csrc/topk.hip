// topk.hip — per-query top-k block selection over fp32 indexer scores
// ("DeepSeek-V4: 迈向高效百万级上下文智能", §1.1 step 2: keep the k best compressed blocks per
// query; mlpod.com DeepSeek-V4 summary §2.3.1).
//
// Selection rule: among the visible entries s < nv of a row, keep the min(k, nv) largest
// scores; equal scores are ordered by LOWER index first; the kept ids are written in
// ascending order and padded with -1 (pad scores -inf).  Scores compare as fp32 values
// (+0 == -0) through an order-preserving uint32 key.
//
// One workgroup of 1024 threads per row.  Rows of up to 32768 visible entries are staged
// in LDS once (128 KB of the 160 KB a gfx950 CU has); longer rows are read from global
// memory in every pass.
//   A  min / max of the row (fused into the LDS staging pass)
//   B  2048-bin histogram with bins LINEAR in value: spreads the LDS atomics (a radix digit
//      of the float bit pattern would put nearly every score of a row in one bin)
//   C  the bin b* that holds the k-th largest value; its members are gathered and the exact
//      k-th element in (value desc, index asc) order is found by ranking them.  If b*
//      holds more than kCap members (heavy ties), an exact 8-bit radix select on the order
//      keys restricted to b* runs instead.
//   D  ordered compaction: keep s iff key > K*, or key == K* and s is among the first
//      need_eq such indices.  Each wave compacts a contiguous segment with ballots; a
//      16-entry scan of the per-wave counts gives each segment its output offset.
#include "device_common.h"
#include "launch.h"

namespace csa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 2048;
constexpr int kCap = 1024;
constexpr int kRowLds = 32768;   // floats of a row staged in LDS

struct TopkShared {
    uint32_t hist[kBins];
    float cval[kCap];
    int32_t cidx[kCap];
    float red_lo[kWaves], red_hi[kWaves];
    uint32_t wgt[kWaves], weq[kWaves];
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

template <bool IN_LDS>
__global__ void __launch_bounds__(kThreads)
topk_row_kernel(const float* __restrict__ scores, int64_t ld, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
                int32_t* __restrict__ idx, float* __restrict__ sel) {
    __shared__ TopkShared sh;
    __shared__ float rowbuf[IN_LDS ? kRowLds : 1];
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
    auto val = [&](int64_t s) -> float {
        if constexpr (IN_LDS) return rowbuf[s];
        else return sc[s];
    };

    // ---- A: min / max (and LDS staging)
    float lo = INFINITY, hi = -INFINITY;
    if constexpr (IN_LDS) {
        const int64_t n4 = nv >> 2;
        const float4* s4 = reinterpret_cast<const float4*>(sc);
        float4* d4 = reinterpret_cast<float4*>(rowbuf);
        for (int64_t i = tid; i < n4; i += kThreads) {
            const float4 v = s4[i];
            d4[i] = v;
            lo = fminf(lo, fminf(fminf(v.x, v.y), fminf(v.z, v.w)));
            hi = fmaxf(hi, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
        }
        for (int64_t s = 4 * n4 + tid; s < nv; s += kThreads) {
            const float v = sc[s];
            rowbuf[s] = v;
            lo = fminf(lo, v);
            hi = fmaxf(hi, v);
        }
    } else {
        for (int64_t s = tid; s < nv; s += kThreads) {
            const float v = sc[s];
            lo = fminf(lo, v);
            hi = fmaxf(hi, v);
        }
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
    for (int64_t s = tid; s < nv; s += kThreads) atomicAdd(&sh.hist[bin_of(val(s), lo, inv)], 1u);
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
            const float v = val(s);
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
        if (wid == 0) {
            uint32_t gt = 0;
            for (uint32_t j = lane; j < nc; j += kWave) gt += order_key(sh.cval[j]) > sh.kstar ? 1u : 0u;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) gt += __shfl_xor(gt, off, kWave);
            if (lane == 0) sh.need_eq = need - gt;
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
                const float v = val(s);
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

    // ---- D: ordered compaction, one contiguous segment per wave
    const uint32_t kstar = sh.kstar, need_eq = sh.need_eq;
    const int64_t seg = ((nv + (int64_t)kWaves * kWave - 1) / ((int64_t)kWaves * kWave)) * kWave;
    const int64_t s_begin = (int64_t)wid * seg;
    const int64_t s_end = min(nv, s_begin + seg);
    const unsigned long long lt = (1ull << lane) - 1ull;
    uint32_t c_gt = 0, c_eq = 0;
    for (int64_t s0 = s_begin; s0 < s_end; s0 += kWave) {
        const int64_t s = s0 + lane;
        const bool ok = s < s_end;
        const uint32_t key = ok ? order_key(val(s)) : 0u;
        c_gt += __popcll(__ballot(ok && key > kstar));
        c_eq += __popcll(__ballot(ok && key == kstar));
    }
    if (lane == 0) { sh.wgt[wid] = c_gt; sh.weq[wid] = c_eq; }
    __syncthreads();
    uint32_t gt_before = 0, eq_before = 0;
    for (int v = 0; v < wid; ++v) { gt_before += sh.wgt[v]; eq_before += sh.weq[v]; }
    uint32_t run_eq = eq_before;
    uint32_t run_take = gt_before + min(eq_before, need_eq);
    for (int64_t s0 = s_begin; s0 < s_end; s0 += kWave) {
        const int64_t s = s0 + lane;
        const bool ok = s < s_end;
        const float v = ok ? val(s) : 0.f;
        const uint32_t key = ok ? order_key(v) : 0u;
        const bool is_gt = ok && key > kstar;
        const bool is_eq = ok && key == kstar;
        const unsigned long long meq = __ballot(is_eq);
        const uint32_t eq_rank = run_eq + __popcll(meq & lt);
        const bool take = is_gt || (is_eq && eq_rank < need_eq);
        const unsigned long long mt = __ballot(take);
        const uint32_t pos = run_take + __popcll(mt & lt);
        if (take && pos < (uint32_t)k) {
            oi[pos] = (int32_t)s;
            if (os) os[pos] = v;
        }
        run_eq += __popcll(meq);
        run_take += __popcll(mt);
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
    // the longest visible row is that of the last query
    int64_t nv_max = (q_pos0 + T) / m;
    if (nv_max > N) nv_max = N;
    if (nv_max <= kRowLds)
        hipLaunchKernelGGL((topk_row_kernel<true>), dim3((unsigned)rows), dim3(kThreads), 0, stream, scores, ld, T,
                           q_pos0, N, m, k, idx, sel);
    else
        hipLaunchKernelGGL((topk_row_kernel<false>), dim3((unsigned)rows), dim3(kThreads), 0, stream, scores, ld, T,
                           q_pos0, N, m, k, idx, sel);
    return 0;
}

}  // namespace csa
