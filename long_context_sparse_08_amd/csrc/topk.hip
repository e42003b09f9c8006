// topk.hip — per-query top-k block selection over fp32 indexer scores
// ("DeepSeek-V4: 迈向高效百万级上下文智能", §1.1 step 2: keep the k best compressed blocks per
// query; mlpod.com DeepSeek-V4 summary §2.3.1).
//
// Selection rule: among the visible entries s < nv of a row, keep the min(k, nv) largest
// scores; equal scores are ordered by LOWER index first; the kept ids are written in
// ascending order and padded with -1 (pad scores -inf).  Scores compare as fp32 values
// (+0 == -0) through an order-preserving uint32 key.
//
// topk_row_kernel (rows longer than 262144 visible entries), one workgroup of 1024 threads
// per row.  Rows of up to 32768 visible entries are staged
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
#include <type_traits>

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


// ============================================================================ bitmap kernel
// topk_bitmap: the same selection with two changes that cut the per-element work.
//  * The row range (min / max) can come from per-chunk min / max the decode indexer writes
//    next to the scores, so no pass is spent on it.
//  * After b* is known, one pass marks every entry of a bin above b* in an LDS bitmap (all of
//    them are kept) and gathers b*'s members; the members that are kept are marked after
//    ranking.  The ordered output is then read off the bitmap: each thread owns a run of
//    32-bit words, one block scan of their popcounts gives its output offset.
// Rows up to kBmMaxRow = 262144 visible entries (a 32 KB bitmap); rows up to kRowLds are
// staged in LDS first.
constexpr int kBmMaxRow = 262144;
constexpr int kShortRow = 4096;      // rows up to this use 256-thread workgroups
constexpr int kShortThreads = 256;
constexpr int kBmWordsGlb = kBmMaxRow / 32;

// Exclusive prefix sum of x over the workgroup's NW waves (every thread active) and the
// total; two barriers, buf holds NW words.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* buf, uint32_t* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t inc = wave_incl_scan(x);
    if (lane == kWave - 1) buf[wid] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int i = 0; i < NW; ++i) {
        const uint32_t v = buf[i];
        before += (i < wid) ? v : 0u;
        all += v;
    }
    __syncthreads();
    *total = all;
    return before + inc - x;
}

template <int NB>
__device__ __forceinline__ int bin_of_n(float v, float lo, float inv) {
    float x = (v - lo) * inv;
    x = fminf(fmaxf(x, 0.f), (float)(NB - 1));
    return (int)x;
}

// NT threads per row, rows up to ROWL entries staged in LDS (IN_LDS), NB linear bins.
template <bool IN_LDS, int NT, int ROWL, int NB>
__global__ void __launch_bounds__(NT)
topk_bitmap(const float* __restrict__ scores, int64_t ld, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
            const float* __restrict__ mm, int nmm, int32_t* __restrict__ idx, float* __restrict__ sel) {
    constexpr int NW = NT / kWave;
    constexpr int kWords = IN_LDS ? ROWL / 32 : kBmWordsGlb;
    __shared__ float rowbuf[IN_LDS ? ROWL : 1];
    __shared__ uint32_t bits[kWords];
    __shared__ uint32_t hist[NB];
    __shared__ float cval[kCap];
    __shared__ int32_t cidx[kCap];
    __shared__ float red_lo[NW], red_hi[NW];
    __shared__ uint32_t scan_buf[NW];
    __shared__ float s_lo, s_inv;
    __shared__ int s_bstar;
    __shared__ uint32_t s_need, s_ncand, s_need_eq, s_prefix, s_pmask;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: scalar registers
    const int64_t row = blockIdx.x;
    const int64_t nv = visible_entries(q_pos0 + row % T, m, N);
    const float* sc = scores + row * ld;
    int32_t* oi = idx + row * k;
    float* os = sel ? sel + row * k : nullptr;
    if (nv <= k) {
        for (int r = tid; r < k; r += NT) {
            oi[r] = r < nv ? r : -1;
            if (os) os[r] = r < nv ? sc[r] : -INFINITY;
        }
        return;
    }
    auto val = [&](int64_t s) -> float {
        if constexpr (IN_LDS) return rowbuf[s];
        else return sc[s];
    };
    const int64_t nwords = (nv + 31) >> 5;

    // ---- row range, LDS staging, histogram.  With the indexer's per-chunk (min, max) the
    // range is known first and the histogram is built from the staging registers (one pass).
    float lo = INFINITY, hi = -INFINITY;
    const bool have_mm = mm != nullptr;
    auto publish_range = [&]() {
        lo = -wave_max(-lo);
        hi = wave_max(hi);
        if (lane == 0) { red_lo[wid] = lo; red_hi[wid] = hi; }
        for (int i = tid; i < NB; i += NT) hist[i] = 0u;
        for (int64_t i = tid; i < nwords; i += NT) bits[i] = 0u;
        __syncthreads();
        if (tid == 0) {
            float l = red_lo[0], h = red_hi[0];
            for (int i = 1; i < NW; ++i) { l = fminf(l, red_lo[i]); h = fmaxf(h, red_hi[i]); }
            float inv = (float)NB / (h - l);
            if (!(h > l) || !isfinite(inv)) inv = 0.f;
            s_lo = l;
            s_inv = inv;
            s_ncand = 0u;
            s_bstar = 0;   // always overwritten: the bin counts sum to nv > k
            s_need = (uint32_t)k;
        }
        __syncthreads();
        lo = s_lo;
    };
    auto range_from_mm = [&]() {
        const float* r = mm + row * (int64_t)nmm * 2;
        for (int i = tid; i < nmm; i += NT) {
            lo = fminf(lo, r[2 * i]);
            hi = fmaxf(hi, r[2 * i + 1]);
        }
        publish_range();
    };
    if constexpr (IN_LDS) {
        // one pass: the row's loads are issued first (their latency overlaps the range
        // reduction), then the values go to LDS and into the histogram (or the min / max)
        constexpr int kF4 = ROWL / (4 * NT);   // float4 per thread
        static_assert(ROWL == 4 * kF4 * NT, "a staged row is kF4 float4 per thread");
        const int64_t n4 = nv >> 2;
        const float4* s4 = reinterpret_cast<const float4*>(sc);
        float4* d4 = reinterpret_cast<float4*>(rowbuf);
        float4 v[kF4];
#pragma unroll
        for (int u = 0; u < kF4; ++u) {
            const int64_t i = tid + (int64_t)u * NT;
            v[u] = i < n4 ? s4[i] : make_float4(INFINITY, INFINITY, -INFINITY, -INFINITY);
        }
        const int64_t st = 4 * n4 + tid;   // the last nv % 4 entries, one per thread
        const float vt = st < nv ? sc[st] : 0.f;
        if (have_mm) range_from_mm();
        const float hlo = have_mm ? s_lo : 0.f, hinv = have_mm ? s_inv : 0.f;
#pragma unroll
        for (int u = 0; u < kF4; ++u) {
            const int64_t i = tid + (int64_t)u * NT;
            if (i >= n4) continue;
            d4[i] = v[u];
            if (have_mm) {
                atomicAdd(&hist[bin_of_n<NB>(v[u].x, hlo, hinv)], 1u);
                atomicAdd(&hist[bin_of_n<NB>(v[u].y, hlo, hinv)], 1u);
                atomicAdd(&hist[bin_of_n<NB>(v[u].z, hlo, hinv)], 1u);
                atomicAdd(&hist[bin_of_n<NB>(v[u].w, hlo, hinv)], 1u);
            } else {
                lo = fminf(lo, fminf(fminf(v[u].x, v[u].y), fminf(v[u].z, v[u].w)));
                hi = fmaxf(hi, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)));
            }
        }
        if (st < nv) {
            rowbuf[st] = vt;
            if (have_mm) atomicAdd(&hist[bin_of_n<NB>(vt, hlo, hinv)], 1u);
            else { lo = fminf(lo, vt); hi = fmaxf(hi, vt); }
        }
    } else {
        if (have_mm) range_from_mm();
        else {
            for (int64_t s = tid; s < nv; s += NT) {
                const float v = sc[s];
                lo = fminf(lo, v);
                hi = fmaxf(hi, v);
            }
        }
    }
    if (!have_mm) {
        __syncthreads();   // staging done before the range is published (hist is reset there)
        publish_range();
    }
    const float inv = s_inv;

    // ---- histogram (unless built while staging)
    if (!(IN_LDS && have_mm)) {
        if constexpr (IN_LDS) {
            for (int64_t s = tid; s < nv; s += NT) atomicAdd(&hist[bin_of_n<NB>(rowbuf[s], lo, inv)], 1u);
        } else {
            for (int64_t s0 = tid; s0 < nv; s0 += 8 * NT) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t s = s0 + (int64_t)u * NT;
                    v[u] = s < nv ? sc[s] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (s0 + (int64_t)u * NT < nv) atomicAdd(&hist[bin_of_n<NB>(v[u], lo, inv)], 1u);
            }
        }
    }
    __syncthreads();
    {   // b*: a block scan over the bins from the top, two per thread
        static_assert(NB == 2 * NT, "two bins per thread");
        const int top = NB - 1 - 2 * tid;
        const uint32_t h0 = hist[top], h1 = hist[top - 1];
        uint32_t total;
        const uint32_t before = block_excl_scan<NW>(h0 + h1, scan_buf, &total);
        if (before < (uint32_t)k && before + h0 + h1 >= (uint32_t)k) {   // exactly one thread
            if (before + h0 >= (uint32_t)k) {
                s_bstar = top;
                s_need = (uint32_t)k - before;
            } else {
                s_bstar = top - 1;
                s_need = (uint32_t)k - before - h0;
            }
        }
    }
    __syncthreads();
    const int bstar = s_bstar;
    const uint32_t need = s_need;
    const bool fits = hist[bstar] <= (uint32_t)kCap;

    // ---- mark bins above b*, gather b*'s members
    auto mark = [&](int64_t s, float v) {
        const int bn = bin_of_n<NB>(v, lo, inv);
        if (bn > bstar) {
            atomicOr(&bits[s >> 5], 1u << (s & 31));
        } else if (bn == bstar && fits) {
            const uint32_t p = atomicAdd(&s_ncand, 1u);
            if (p < (uint32_t)kCap) { cval[p] = v; cidx[p] = (int32_t)s; }
        }
    };
    if constexpr (IN_LDS) {
        // chunks of 64 entries, one per wave step: a ballot gives the chunk's two bitmap words
        // (every word is written, no atomics); b*'s members are appended one wave at a time
        const int nvi = (int)nv;   // <= ROWL
        const int nchunk = (nvi + kWave - 1) / kWave;
        const unsigned long long below = (1ull << lane) - 1ull;
        // bin(v) > b* and bin(v) == b* straight from x = (v - lo) * inv, the expression the
        // histogram's bins come from: bin(v) = trunc(clamp(x, 0, NB-1)), so bin(v) > b* iff
        // x >= b*+1 (none when b* is the top bin), and bin(v) >= b* iff x >= b* (all when
        // b* = 0: values below lo, -inf and NaN land in bin 0)
        const float thr_gt = bstar < NB - 1 ? (float)(bstar + 1) : INFINITY;
        const float thr_ge = bstar > 0 ? (float)bstar : -INFINITY;
        // A wave takes 8 chunks per round (chunk c0 + u*NW).  Lane 2u / 2u+1 collects the two
        // bitmap words of chunk u, so the words are stored once per round (no per-chunk
        // exec-mask changes: the scalar unit, shared by the CU's 16 waves, bounds this loop).
        const bool ge_all = bstar == 0;
        // Lane masks come straight from compares (one VALU op each into a scalar register
        // pair); the chunk's tail and the b* test combine on the scalar unit.
        auto round = [&](int c0) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)   // clamped reads: always in the row; masked below
                v[u] = rowbuf[min((c0 + u * NW) * kWave + lane, nvi - 1)];
            uint32_t wv = 0u;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int c = c0 + u * NW;
                const int nin = nvi - c * kWave;   // entries of this chunk in the row (uniform)
                const unsigned long long okm = nin >= kWave ? ~0ull : nin > 0 ? (1ull << nin) - 1ull : 0ull;
                const float x = (v[u] - lo) * inv;
                const unsigned long long gtm = __ballot(x >= thr_gt);
                const unsigned long long mk = gtm & okm;
                wv = lane == 2 * u ? (uint32_t)mk : lane == 2 * u + 1 ? (uint32_t)(mk >> 32) : wv;
                if (fits) {
                    const unsigned long long gem = ge_all ? ~0ull : __ballot(x >= thr_ge);
                    const unsigned long long me = gem & ~gtm & okm;
                    if (me) {
                        const bool eq = (me >> lane) & 1ull;
                        uint32_t base = 0;
                        if (lane == 0) base = atomicAdd(&s_ncand, (uint32_t)__popcll(me));
                        base = __shfl(base, 0, kWave);
                        const uint32_t p = base + (uint32_t)__popcll(me & below);
                        if (eq && p < (uint32_t)kCap) {
                            cval[p] = v[u];
                            cidx[p] = c * kWave + lane;
                        }
                    }
                }
            }
            const int cw = c0 + (lane >> 1) * NW;
            if (lane < 16 && cw < nchunk) bits[2 * cw + (lane & 1)] = wv;
        };
        for (int c0 = wid; c0 < nchunk; c0 += 8 * NW) round(c0);
    } else {
        for (int64_t s0 = tid; s0 < nv; s0 += 8 * NT) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t s = s0 + (int64_t)u * NT;
                v[u] = s < nv ? sc[s] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + (int64_t)u * NT < nv) mark(s0 + (int64_t)u * NT, v[u]);
        }
    }
    __syncthreads();

    if (fits && s_ncand <= (uint32_t)kWave) {
        // rank b*'s members by (value desc, index asc) within one wave: lane i holds member i,
        // the others' keys are read with readlane (no LDS round trips); keep ranks < need
        const uint32_t nc = s_ncand;
        if (wid == 0) {
            const bool have = (uint32_t)lane < nc;
            const uint32_t ki = have ? order_key(cval[lane]) : 0u;
            const int32_t si = have ? cidx[lane] : 0;
            uint32_t rank = 0;
            for (uint32_t j = 0; j < nc; ++j) {
                const uint32_t kj = __builtin_amdgcn_readlane(ki, j);
                const int32_t sj = __builtin_amdgcn_readlane(si, j);
                rank += (kj > ki || (kj == ki && sj < si)) ? 1u : 0u;
            }
            if (have && rank < need) atomicOr(&bits[si >> 5], 1u << (si & 31));
        }
    } else if (fits) {
        // rank b*'s members by (value desc, index asc); keep ranks < need
        const uint32_t nc = min(s_ncand, (uint32_t)kCap);
        for (uint32_t i = tid; i < nc; i += NT) {
            const uint32_t ki = order_key(cval[i]);
            const int32_t si = cidx[i];
            uint32_t rank = 0;
            for (uint32_t j = 0; j < nc; ++j) {
                const uint32_t kj = order_key(cval[j]);
                rank += (kj > ki || (kj == ki && cidx[j] < si)) ? 1u : 0u;
            }
            if (rank < need) atomicOr(&bits[si >> 5], 1u << (si & 31));
        }
    } else {
        // heavy ties in b*: exact 8-bit radix select of the need-th largest order key in b*
        if (tid == 0) { s_prefix = 0u; s_pmask = 0u; s_need_eq = need; }
        __syncthreads();
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += NT) hist[i] = 0u;
            __syncthreads();
            const uint32_t prefix = s_prefix, pmask = s_pmask;
            for (int64_t s = tid; s < nv; s += NT) {
                const float v = val(s);
                if (bin_of_n<NB>(v, lo, inv) != bstar) continue;
                const uint32_t key = order_key(v);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                uint32_t remaining = s_need_eq, acc = 0;
                for (int d = 255; d >= 0; --d) {
                    const uint32_t hh = hist[d];
                    if (acc + hh >= remaining) {
                        s_prefix = prefix | ((uint32_t)d << shift);
                        s_pmask = pmask | (255u << shift);
                        s_need_eq = remaining - acc;
                        break;
                    }
                    acc += hh;
                }
            }
            __syncthreads();
        }
        const uint32_t kstar = s_prefix, need_eq = s_need_eq;
        // keys above K* in b* are kept; of the keys equal to K*, the need_eq lowest indices
        const int64_t seg = ((nv + (int64_t)NW * kWave - 1) / ((int64_t)NW * kWave)) * kWave;
        const int64_t a = (int64_t)wid * seg, e = min(nv, a + seg);
        const unsigned long long lt = (1ull << lane) - 1ull;
        uint32_t c_eq = 0;
        for (int64_t b0 = a; b0 < e; b0 += kWave) {
            const int64_t s = b0 + lane;
            const bool ok = s < e;
            const float v = ok ? val(s) : 0.f;
            const bool inb = ok && bin_of_n<NB>(v, lo, inv) == bstar;
            const uint32_t key = order_key(v);
            if (inb && key > kstar) atomicOr(&bits[s >> 5], 1u << (s & 31));
            c_eq += __popcll(__ballot(inb && key == kstar));
        }
        if (lane == 0) scan_buf[wid] = c_eq;
        __syncthreads();
        uint32_t run = 0;
        for (int v = 0; v < wid; ++v) run += scan_buf[v];
        for (int64_t b0 = a; b0 < e; b0 += kWave) {
            const int64_t s = b0 + lane;
            const bool ok = s < e;
            const float v = ok ? val(s) : 0.f;
            const bool is_eq = ok && bin_of_n<NB>(v, lo, inv) == bstar && order_key(v) == kstar;
            const unsigned long long meq = __ballot(is_eq);
            if (is_eq && run + __popcll(meq & lt) < need_eq) atomicOr(&bits[s >> 5], 1u << (s & 31));
            run += __popcll(meq);
        }
    }
    __syncthreads();

    // ---- ordered extraction: each thread owns a run of bitmap words
    const int64_t per = (nwords + NT - 1) / NT;
    const int64_t w0 = (int64_t)tid * per, w1 = min(nwords, w0 + per);
    uint32_t cnt = 0;
    for (int64_t w = w0; w < w1; ++w) cnt += __popc(bits[w]);
    uint32_t total;
    uint32_t pos = block_excl_scan<NW>(cnt, scan_buf, &total);
    for (int64_t w = w0; w < w1; ++w) {
        uint32_t word = bits[w];
        while (word) {
            const int b = __ffs(word) - 1;
            word &= word - 1;
            const int64_t s = (w << 5) + b;
            if (pos < (uint32_t)k) {
                oi[pos] = (int32_t)s;
                if (os) os[pos] = val(s);
            }
            ++pos;
        }
    }
}


// ============================================================================ multi-workgroup
// Few long rows (decode: 8-32 rows of 32K-262K scores): the row is cut into slices of
// kSlice entries and three kernels share the work.  Needs the indexer's per-chunk (min, max)
// (the row range) and a per-row region the indexer zeroes (histogram + counters).
//   tkm_hist   (row x slice)  slice histogram in LDS, added into the row histogram
//   tkm_mark   (row x slice)  every slice finds b* from the row histogram; writes its words of
//                             the row keep-bitmap (bins above b*) and appends b*'s members
//   tkm_select (row)          ranks b*'s members, sets the bits of the kept ones, reads the
//                             ordered output off the bitmap
// If b* has more members than kMCap (heavy ties), tkm_select finds the cut with an exact
// radix select over the row instead.
constexpr int kSlice = 4096;
constexpr int kMCap = 8192;
constexpr int kZeroWords = kBins + 8;   // per row: histogram + counters, zeroed by the indexer
constexpr int kSliceThreads = 256;

struct MultiWs {
    uint32_t* zero;    // [rows][kZeroWords]: hist[kBins], then counter[0] = b* member count
    float* cval;       // [rows][kMCap]
    int32_t* cidx;     // [rows][kMCap]
    uint32_t* bits;    // [rows][words]
    int64_t words;     // bitmap words per row
};

__host__ inline size_t multi_bytes(int64_t rows, int64_t N, MultiWs* L, void* base) {
    const int64_t words = (N + 63) / 64 * 2;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) & ~size_t(255); return o; };
    const size_t o_zero = take((size_t)rows * kZeroWords * 4);
    const size_t o_cval = take((size_t)rows * kMCap * 4);
    const size_t o_cidx = take((size_t)rows * kMCap * 4);
    const size_t o_bits = take((size_t)rows * words * 4);
    if (L && base) {
        uint8_t* b = static_cast<uint8_t*>(base);
        L->zero = reinterpret_cast<uint32_t*>(b + o_zero);
        L->cval = reinterpret_cast<float*>(b + o_cval);
        L->cidx = reinterpret_cast<int32_t*>(b + o_cidx);
        L->bits = reinterpret_cast<uint32_t*>(b + o_bits);
        L->words = words;
    }
    return off;
}

__device__ __forceinline__ void row_range_mm(const float* mm, int nmm, float& lo, float& inv) {
    float l = INFINITY, h = -INFINITY;
    for (int i = 0; i < nmm; ++i) {
        l = fminf(l, mm[2 * i]);
        h = fmaxf(h, mm[2 * i + 1]);
    }
    float iv = (float)kBins / (h - l);
    if (!(h > l) || !isfinite(iv)) iv = 0.f;
    lo = l;
    inv = iv;
}

__global__ void __launch_bounds__(kSliceThreads)
tkm_hist(const float* __restrict__ scores, int64_t ld, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
         const float* __restrict__ mm, int nmm, int P, MultiWs L) {
    __shared__ uint32_t h[kBins];
    __shared__ float s_lo, s_inv;
    const int64_t row = blockIdx.x / P;
    const int p = (int)(blockIdx.x % P);
    const int64_t nv = visible_entries(q_pos0 + row % T, m, N);
    if (nv <= k) return;
    const int64_t s0 = (int64_t)p * kSlice, s1 = min(nv, s0 + kSlice);
    if (s0 >= s1) return;
    for (int i = threadIdx.x; i < kBins; i += kSliceThreads) h[i] = 0u;
    if (threadIdx.x == 0) {
        float lo, inv;
        row_range_mm(mm + row * (int64_t)nmm * 2, nmm, lo, inv);
        s_lo = lo;
        s_inv = inv;
    }
    __syncthreads();
    const float lo = s_lo, inv = s_inv;
    const float* sc = scores + row * ld;
    // 16 entries per thread, loads issued before use
    float v[kSlice / kSliceThreads];
#pragma unroll
    for (int u = 0; u < kSlice / kSliceThreads; ++u) {
        const int64_t s = s0 + threadIdx.x + (int64_t)u * kSliceThreads;
        v[u] = s < s1 ? sc[s] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kSlice / kSliceThreads; ++u)
        if (s0 + threadIdx.x + (int64_t)u * kSliceThreads < s1) atomicAdd(&h[bin_of(v[u], lo, inv)], 1u);
    __syncthreads();
    uint32_t* hg = L.zero + row * kZeroWords;
    for (int i = threadIdx.x; i < kBins; i += kSliceThreads)
        if (h[i]) atomicAdd(&hg[i], h[i]);
}

// b* and need from the row histogram (all threads of the block get them)
__device__ __forceinline__ void find_bstar(const uint32_t* hg, int k, uint32_t* sh_hist, uint32_t* scan, int& bstar,
                                           uint32_t& need, int nthreads) {
    // suffix sums over bins from the top: thread t owns kBins/nthreads consecutive bins
    const int per = kBins / nthreads;
    const int tid = threadIdx.x;
    const int top = kBins - 1 - tid * per;
    uint32_t mine = 0;
    for (int j = 0; j < per; ++j) {
        const uint32_t c = hg[top - j];
        sh_hist[top - j] = c;
        mine += c;
    }
    // inclusive scan of `mine` over threads (thread 0 = highest bins)
    const int lane = tid & 63, wid = tid >> 6;
    uint32_t inc = mine;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += y;
    }
    if (lane == kWave - 1) scan[wid] = inc;
    __syncthreads();
    uint32_t before_w = 0;
    for (int w = 0; w < wid; ++w) before_w += scan[w];
    const uint32_t before = before_w + inc - mine;
    if (before < (uint32_t)k && before + mine >= (uint32_t)k) {
        uint32_t acc = before;
        for (int j = 0; j < per; ++j) {
            const uint32_t c = sh_hist[top - j];
            if (acc + c >= (uint32_t)k) {
                scan[nthreads / kWave] = (uint32_t)(top - j);
                scan[nthreads / kWave + 1] = (uint32_t)k - acc;
                break;
            }
            acc += c;
        }
    }
    __syncthreads();
    bstar = (int)scan[nthreads / kWave];
    need = scan[nthreads / kWave + 1];
}

__global__ void __launch_bounds__(kSliceThreads)
tkm_mark(const float* __restrict__ scores, int64_t ld, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
         const float* __restrict__ mm, int nmm, int P, MultiWs L) {
    __shared__ uint32_t sh_hist[kBins];
    __shared__ uint32_t scan[kSliceThreads / kWave + 2];
    __shared__ float s_lo, s_inv;
    const int64_t row = blockIdx.x / P;
    const int p = (int)(blockIdx.x % P);
    const int64_t nv = visible_entries(q_pos0 + row % T, m, N);
    if (nv <= k) return;
    const int64_t s0 = (int64_t)p * kSlice, s1 = min(nv, s0 + kSlice);
    if (s0 >= s1) return;
    if (threadIdx.x == 0) {
        float lo, inv;
        row_range_mm(mm + row * (int64_t)nmm * 2, nmm, lo, inv);
        s_lo = lo;
        s_inv = inv;
        scan[kSliceThreads / kWave] = 0;
        scan[kSliceThreads / kWave + 1] = (uint32_t)k;
    }
    int bstar;
    uint32_t need;
    uint32_t* hg = L.zero + row * kZeroWords;
    __syncthreads();
    find_bstar(hg, k, sh_hist, scan, bstar, need, kSliceThreads);
    const float lo = s_lo, inv = s_inv;
    const float* sc = scores + row * ld;
    uint32_t* bits = L.bits + row * L.words;
    uint32_t* ccount = hg + kBins;
    float* cval = L.cval + row * kMCap;
    int32_t* cidx = L.cidx + row * kMCap;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    // each wave takes 64-entry runs: one ballot gives two bitmap words
    for (int64_t b0 = s0 + (int64_t)wid * kWave; b0 < s1; b0 += kSliceThreads) {
        const int64_t s = b0 + lane;
        const bool ok = s < s1;
        const float v = ok ? sc[s] : 0.f;
        const int bn = ok ? bin_of(v, lo, inv) : -1;
        const unsigned long long above = __ballot(bn > bstar);
        if (bn == bstar) {
            const uint32_t pos = atomicAdd(ccount, 1u);
            if (pos < (uint32_t)kMCap) { cval[pos] = v; cidx[pos] = (int32_t)s; }
        }
        if (lane == 0) {
            bits[b0 >> 5] = (uint32_t)above;
            bits[(b0 >> 5) + 1] = (uint32_t)(above >> 32);
        }
    }
}

__global__ void __launch_bounds__(kThreads)
tkm_select(const float* __restrict__ scores, int64_t ld, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
           const float* __restrict__ mm, int nmm, MultiWs L, int32_t* __restrict__ idx, float* __restrict__ sel) {
    __shared__ uint32_t sh_hist[kBins];
    __shared__ uint32_t scan[kThreads / kWave + 2];
    __shared__ float cv[kCap];
    __shared__ int32_t ci[kCap];
    __shared__ uint32_t s_prefix, s_pmask, s_rem;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t row = blockIdx.x;
    const int64_t nv = visible_entries(q_pos0 + row % T, m, N);
    const float* sc = scores + row * ld;
    int32_t* oi = idx + row * k;
    float* os = sel ? sel + row * k : nullptr;
    if (nv <= k) {
        for (int r = tid; r < k; r += kThreads) {
            oi[r] = r < nv ? r : -1;
            if (os) os[r] = r < nv ? sc[r] : -INFINITY;
        }
        return;
    }
    uint32_t* hg = L.zero + row * kZeroWords;
    uint32_t* bits = L.bits + row * L.words;
    if (tid == 0) { scan[kThreads / kWave] = 0; scan[kThreads / kWave + 1] = (uint32_t)k; }
    __syncthreads();
    int bstar;
    uint32_t need;
    find_bstar(hg, k, sh_hist, scan, bstar, need, kThreads);
    const uint32_t ncand = hg[kBins];
    if (ncand <= (uint32_t)kCap) {
        const float* cval = L.cval + row * kMCap;
        const int32_t* cidx = L.cidx + row * kMCap;
        for (uint32_t i = tid; i < ncand; i += kThreads) { cv[i] = cval[i]; ci[i] = cidx[i]; }
        __syncthreads();
        for (uint32_t i = tid; i < ncand; i += kThreads) {
            const uint32_t ki = order_key(cv[i]);
            const int32_t si = ci[i];
            uint32_t rank = 0;
            for (uint32_t j = 0; j < ncand; ++j) {
                const uint32_t kj = order_key(cv[j]);
                rank += (kj > ki || (kj == ki && ci[j] < si)) ? 1u : 0u;
            }
            if (rank < need) atomicOr(&bits[si >> 5], 1u << (si & 31));
        }
    } else {
        // heavy ties in b*: exact radix select of the need-th largest order key among b*'s
        // members, over the row in global memory
        float lo, inv;
        row_range_mm(mm + row * (int64_t)nmm * 2, nmm, lo, inv);
        if (tid == 0) { s_prefix = 0u; s_pmask = 0u; s_rem = need; }
        __syncthreads();
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kThreads) sh_hist[i] = 0u;
            __syncthreads();
            const uint32_t prefix = s_prefix, pmask = s_pmask;
            for (int64_t s = tid; s < nv; s += kThreads) {
                const float v = sc[s];
                if (bin_of(v, lo, inv) != bstar) continue;
                const uint32_t key = order_key(v);
                if ((key & pmask) == prefix) atomicAdd(&sh_hist[(key >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                uint32_t remaining = s_rem, acc = 0;
                for (int d = 255; d >= 0; --d) {
                    const uint32_t hh = sh_hist[d];
                    if (acc + hh >= remaining) {
                        s_prefix = prefix | ((uint32_t)d << shift);
                        s_pmask = pmask | (255u << shift);
                        s_rem = remaining - acc;
                        break;
                    }
                    acc += hh;
                }
            }
            __syncthreads();
        }
        const uint32_t kstar = s_prefix, need_eq = s_rem;
        // members above K* are kept; of those equal to K*, the need_eq lowest indices
        const int64_t seg = ((nv + (int64_t)kWaves * kWave - 1) / ((int64_t)kWaves * kWave)) * kWave;
        const int64_t a = (int64_t)wid * seg, e = min(nv, a + seg);
        const unsigned long long lt = (1ull << lane) - 1ull;
        uint32_t c_eq = 0;
        for (int64_t b0 = a; b0 < e; b0 += kWave) {
            const int64_t s = b0 + lane;
            const bool ok = s < e;
            const float v = ok ? sc[s] : 0.f;
            const bool inb = ok && bin_of(v, lo, inv) == bstar;
            const uint32_t key = order_key(v);
            if (inb && key > kstar) atomicOr(&bits[s >> 5], 1u << (s & 31));
            c_eq += __popcll(__ballot(inb && key == kstar));
        }
        if (lane == 0) scan[wid] = c_eq;
        __syncthreads();
        uint32_t run = 0;
        for (int v = 0; v < wid; ++v) run += scan[v];
        for (int64_t b0 = a; b0 < e; b0 += kWave) {
            const int64_t s = b0 + lane;
            const bool ok = s < e;
            const float v = ok ? sc[s] : 0.f;
            const bool is_eq = ok && bin_of(v, lo, inv) == bstar && order_key(v) == kstar;
            const unsigned long long meq = __ballot(is_eq);
            if (is_eq && run + __popcll(meq & lt) < need_eq) atomicOr(&bits[s >> 5], 1u << (s & 31));
            run += __popcll(meq);
        }
    }
    __threadfence();   // the bit updates above are device-memory atomics: make them visible
    __syncthreads();
    // ordered extraction: each thread owns a run of bitmap words
    const int64_t nwords = (nv + 31) >> 5;
    const int64_t per = (nwords + kThreads - 1) / kThreads;
    const int64_t w0 = (int64_t)tid * per, w1 = min(nwords, w0 + per);
    uint32_t cnt = 0;
    for (int64_t w = w0; w < w1; ++w) {
        uint32_t word = bits[w];
        if (w == nwords - 1 && (nv & 31)) word &= (1u << (nv & 31)) - 1u;
        cnt += __popc(word);
    }
    uint32_t total;
    uint32_t pos = block_excl_scan<kWaves>(cnt, scan, &total);
    for (int64_t w = w0; w < w1; ++w) {
        uint32_t word = bits[w];
        if (w == nwords - 1 && (nv & 31)) word &= (1u << (nv & 31)) - 1u;
        while (word) {
            const int b = __ffs(word) - 1;
            word &= word - 1;
            const int64_t s = (w << 5) + b;
            if (pos < (uint32_t)k) {
                oi[pos] = (int32_t)s;
                if (os) os[pos] = sc[s];
            }
            ++pos;
        }
    }
}

// ============================================================================ group-bounded
// Decode rows too long for LDS staging (32769 to 262144 visible entries, few queries).  The
// indexer also writes the maximum of every group of G consecutive scores of a row (G a power
// of two up to 32, chosen so that a row has several times k groups).  With the group maxima
// put into 2048 bins linear in value, let b* be the highest bin that has at least k group
// maxima in it and above.  Those k groups hold k distinct entries in bins >= b*, so the k-th
// largest score is in a bin >= b* (binning is monotonic), and so is every entry of the row's
// top k, whose group's maximum is then in a bin >= b* as well.  One workgroup per row:
//   1  the group maxima into LDS, their range, the bin histogram and b*
//   2  candidates: the entries in bins >= b* of the groups whose maximum is in a bin >= b*
//      (about k of them for scores without heavy ties), loaded with 16-byte reads
//   3  K* = the exact k-th largest candidate key (radix select from the highest bit where the
//      candidates differ), and how many candidates equal to K* belong to the top k (need_eq);
//      every entry equal to K* is a candidate
//   4  bitmaps over the row: kept (key > K*) and ties (key == K*); the first need_eq ties in
//      index order join the kept ones, and each kept candidate goes to its rank in index order
// More than kGCap candidates (heavy ties) or too few groups: steps 3-4 run over the whole row,
// read from global memory.
constexpr int kGThreads = 1024;
constexpr int kGWaves = kGThreads / kWave;
constexpr int kGMaxGroups = 8192;    // group maxima per row, staged in LDS
static_assert(kGMaxGroups == kTopkMaxGroups, "group region size");
constexpr int kGMaxRow = 262144;     // visible entries per row: bitmaps of 32 KB
constexpr int kGCap = 4096;          // candidates per row
constexpr int kGMaxG = 32;           // groups never cross the indexer's 32-entry blocks

constexpr int kGBins = 2048;         // linear bins over the group maxima

constexpr int kGMaxSlices = 32;      // group slices of the longest row (two-launch select)

struct GroupShared {
    uint32_t a[kGMaxRow / 32];   // group maxima (fp32 bits), then the tie bitmap, then word offsets
    uint32_t b[kGMaxRow / 32];   // indices of the selected groups, then the kept bitmap
    uint32_t ckey[kGCap];
    int32_t cidx[kGCap];
    uint32_t hist[256];
    uint32_t ghist[kGBins];
    float flo, fhi;
    int bstar;
    uint32_t scan[kGWaves + 2];
    uint32_t red_lo[kGWaves], red_hi[kGWaves];
    uint32_t ctl[3];   // radix select state
    uint32_t ngroups, ncand;
    uint32_t neq;      // entries with key == K* (all of them are taken when need_eq equals it)
    // two-launch select: slice p's chunk of the candidate list (start, count) and the
    // candidates of the slices before it
    uint32_t rbase[kGMaxSlices], rcnt[kGMaxSlices], rpre[kGMaxSlices];
};
static_assert(kGMaxRow / 32 >= kGMaxGroups, "group keys share the tie bitmap");

// Block-wide min and max of the per-thread values lo / hi (every thread gets both).
__device__ __forceinline__ void block_minmax(uint32_t& lo, uint32_t& hi, GroupShared& sh) {
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, kWave));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, kWave));
    }
    if (lane == 0) {
        sh.red_lo[wid] = lo;
        sh.red_hi[wid] = hi;
    }
    __syncthreads();
    lo = sh.red_lo[0];
    hi = sh.red_hi[0];
#pragma unroll
    for (int w = 1; w < kGWaves; ++w) {
        lo = min(lo, sh.red_lo[w]);
        hi = max(hi, sh.red_hi[w]);
    }
    __syncthreads();   // read by all before the next use
}

// Exact k-th largest (k >= 1) of the keys the workgroup's NT threads visit (visit(f) calls
// f(key) for every key the calling thread holds; at least k keys in all, all within [kmin,
// kmax]): the bits above the highest bit where kmin and kmax differ are common to every key;
// the rest is resolved in passes over 8-bit digits from the top, each narrowing to the keys
// that share the digits found so far.  (Starting at the first varying bit spreads the
// histogram: scores of similar size share their sign and exponent bits.)
// hist: 256 words of LDS, ctl: 3 (prefix, mask, remaining).  Returns K*; *need_eq receives
// how many keys equal to K* belong to the k largest.
template <int NT, class V>
__device__ __forceinline__ uint32_t radix_kth(V visit, uint32_t k, uint32_t kmin, uint32_t kmax, uint32_t* hist, uint32_t* ctl,
                              uint32_t* need_eq) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const uint32_t diff = kmin ^ kmax;
    int hb = diff == 0u ? 0 : 32 - __clz(diff);   // bits [0, hb) vary
    const uint32_t low = hb == 32 ? ~0u : (1u << hb) - 1u;
    if (tid == 0) {
        ctl[0] = kmin & ~low;
        ctl[1] = ~low;
        ctl[2] = k;
    }
    while (hb > 0) {
        const int wd = hb < 8 ? hb : 8, shift = hb - wd;
        const uint32_t dmask = (1u << wd) - 1u;
        for (int i = tid; i < 256; i += NT) hist[i] = 0u;
        __syncthreads();   // also publishes the previous pass's prefix
        const uint32_t prefix = ctl[0], pmask = ctl[1];
        visit([&](uint32_t key) {
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
        });
        __syncthreads();
        if (tid < kWave) {
            // lane l holds digits 255-4l .. 252-4l (descending); inclusive scan from the top
            uint32_t c[4], mine = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = hist[255 - 4 * lane - j];
                mine += c[j];
            }
            const uint32_t inc = wave_incl_scan(mine);
            const uint32_t rem = ctl[2], before = inc - mine;
            if (before < rem && inc >= rem) {   // exactly one lane
                uint32_t acc = before;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (acc + c[j] >= rem) {
                        ctl[0] = prefix | ((uint32_t)(255 - 4 * lane - j) << shift);
                        ctl[1] = pmask | (dmask << shift);
                        ctl[2] = rem - acc;
                        break;
                    }
                    acc += c[j];
                }
            }
        }
        __syncthreads();   // the search is done before the histogram is cleared again
        hb = shift;
    }
    __syncthreads();
    const uint32_t kth = ctl[0], rem = ctl[2];
    __syncthreads();   // every thread has read them before a later call rewrites them
    *need_eq = rem;
    return kth;
}

// inverse of order_key (-0 comes back as +0)
__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Appends the lanes with `take` to a list: one LDS atomic per wave; returns this lane's slot.
__device__ __forceinline__ uint32_t wave_append(bool take, uint32_t* counter) {
    const unsigned long long m = __ballot(take);
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t base = 0;
    if (lane == 0 && m != 0ull) base = atomicAdd(counter, (uint32_t)__popcll(m));
    base = __builtin_amdgcn_readlane(base, 0);
    return base + (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
}

// the first n set bits of w (n < popcount(w))
__device__ __forceinline__ uint32_t first_bits(uint32_t w, uint32_t n) {
    uint32_t r = 0u;
    for (; n > 0; --n) {
        r |= w & (0u - w);
        w &= w - 1u;
    }
    return r;
}

// MODE 0: the whole row in one workgroup, as above.  Long rows of a few queries spread the
// candidate step over the chip in two launches:
// MODE 1 (grid rows x P): workgroup (row, p) finds b* as in step 1 (every workgroup of a row
//   from the same maxima: the same b*) and appends the candidates of groups p*kSliceGroups ..
//   (p+1)*kSliceGroups - 1 to the row's list (value, index) in global memory as one chunk in
//   index order, its place taken by one atomic per workgroup on the row's counter (cleared by
//   the indexer at the start of the call), and records the chunk (start, count);
// MODE 2 (grid rows): the exact cut over that list (radix select), then the chunks copied in
//   slice order, which is index order, and the output placed by one block scan (more than
//   kGCap candidates: steps 3-4 over the whole row).
constexpr int kSliceGroups = 256;
static_assert(kGMaxGroups / kSliceGroups <= kGMaxSlices, "a record per slice");

template <int MODE>
__global__ void __launch_bounds__(kGThreads)
topk_groups(const float* __restrict__ scores, int64_t ld, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
            const float* __restrict__ gmax, int64_t gld, int G, int32_t* __restrict__ idx, float* __restrict__ sel,
            int64_t rows, int P, uint32_t* __restrict__ ccount, int ccount_ld, float* __restrict__ cval,
            int32_t* __restrict__ cidx) {
    __shared__ GroupShared sh;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: scalar registers
    // MODE 1: the slices of row r run on XCD r % 8 (workgroups are dealt round-robin over the
    // 8 XCDs), where the indexer wrote the row's scores and maxima and where the selecting
    // workgroup of the row runs: their loads and the candidates they write stay in that L2
    const int64_t row = MODE == 1 ? (int64_t)(blockIdx.x / 8 / P) * 8 + blockIdx.x % 8 : (int64_t)blockIdx.x;
    const int slice = MODE == 1 ? (int)(blockIdx.x / 8 % P) : 0;
    if (MODE == 1 && row >= rows) return;   // (rows padded to whole XCD rounds)
    const int64_t nv = visible_entries(q_pos0 + row % T, m, N);
    const float* sc = scores + row * ld;
    int32_t* oi = idx + row * k;
    float* os = sel ? sel + row * k : nullptr;
    if (MODE == 1 && nv <= k) return;
    if (nv <= k) {
        for (int r = tid; r < k; r += kGThreads) {
            oi[r] = r < nv ? r : -1;
            if (os) os[r] = r < nv ? sc[r] : -INFINITY;
        }
        return;
    }
    // (the launcher sends rows of at most kGMaxRow entries and at most kGMaxGroups groups)
    const int64_t ng = (nv + G - 1) / G;
    bool full = ng <= k;
    if (MODE == 1 && full) return;
    uint32_t kstar = 0u, need_eq = 0u;
    int64_t ncand = 0;
    if (MODE == 2 && !full) {
        // the candidates the slices appended: keys and indices into LDS, their range.  The
        // list's first kGCap slots are loaded together with its length (one memory round trip
        // instead of two; slots past the length hold stale values and are dropped)
        constexpr int kCPer = kGCap / kGThreads;
        float cv[kCPer];
        int32_t ci[kCPer];
#pragma unroll
        for (int u = 0; u < kCPer; ++u) {
            cv[u] = cval[row * kMCap + tid + u * kGThreads];
            ci[u] = cidx[row * kMCap + tid + u * kGThreads];
        }
        // slice `tid`'s chunk record (zero for a slice without candidates)
        const uint32_t rb = tid < P ? ccount[row * ccount_ld + 1 + 2 * tid] : 0u;
        const uint32_t rc = tid < P ? ccount[row * ccount_ld + 2 + 2 * tid] : 0u;
        ncand = ccount[row * ccount_ld];
        if (ncand > kGCap || ncand < k) {
            full = true;   // heavy ties at b* (the second cannot happen)
        } else {
            uint32_t lo = ~0u, hi = 0u;
#pragma unroll
            for (int u = 0; u < kCPer; ++u) {
                const int i2 = tid + u * kGThreads;
                if (i2 < ncand) {
                    const uint32_t key = order_key(cv[u]);
                    sh.ckey[i2] = key;
                    sh.cidx[i2] = ci[u];
                    lo = min(lo, key);
                    hi = max(hi, key);
                }
            }
            if (wid == 0) {   // the chunks' places in index order (P <= 64: one wave)
                const uint32_t c = lane < P ? rc : 0u;
                const uint32_t inc = wave_incl_scan(c);
                if (lane < P) {
                    sh.rbase[lane] = rb;
                    sh.rcnt[lane] = c;
                    sh.rpre[lane] = inc - c;
                }
            }
            block_minmax(lo, hi, sh);   // (its barrier also publishes the candidates and chunks)
            kstar = radix_kth<kGThreads>(
                [&](auto f) {
                    for (int64_t i2 = tid; i2 < ncand; i2 += kGThreads) f(sh.ckey[i2]);
                },
                (uint32_t)k, lo, hi, sh.hist, sh.ctl, &need_eq);
            // The candidates in index order: each slice appended its own in index order, and
            // slices follow each other in the row, so chunk p goes to slots rpre[p] .. of a / b
            // (threads 32p .. 32p + 31 copy chunk p).  No row bitmap is needed then.
            {
                const int p = tid >> 5, j = tid & 31;
                if (p < P) {
                    const uint32_t s0 = sh.rbase[p], d0 = sh.rpre[p], n = sh.rcnt[p];
                    for (uint32_t u = (uint32_t)j; u < n; u += 32u) {
                        sh.a[d0 + u] = sh.ckey[s0 + u];
                        sh.b[d0 + u] = (uint32_t)sh.cidx[s0 + u];
                    }
                }
            }
            __syncthreads();
            // Ordered output: thread t holds candidates 4t .. 4t+3 (index order); one block scan
            // of (ties << 16 | greater) counts gives the kept entries before it: every entry
            // with key > K*, and of the ties (key == K*) the first need_eq in index order.
            constexpr int kOPer = kGCap / kGThreads;
            uint32_t gt = 0u, eqm = 0u;
#pragma unroll
            for (int u = 0; u < kOPer; ++u) {
                const int64_t i = (int64_t)kOPer * tid + u;
                if (i < ncand) {
                    const uint32_t key = sh.a[i];
                    gt |= (key > kstar ? 1u : 0u) << u;
                    eqm |= (key == kstar ? 1u : 0u) << u;
                }
            }
            uint32_t tot;
            const uint32_t pre =
                block_excl_scan<kGWaves>(((uint32_t)__popc(eqm) << 16) | (uint32_t)__popc(gt), sh.scan, &tot);
            const uint32_t tb = pre >> 16, gb = pre & 0xffffu;
            uint32_t takeq = 0u;
            if (tb < need_eq) {
                const uint32_t room = need_eq - tb;
                takeq = (uint32_t)__popc(eqm) <= room ? eqm : first_bits(eqm, room);
            }
            const uint32_t keep = gt | takeq;
            uint32_t slot = gb + min(tb, need_eq);
#pragma unroll
            for (int u = 0; u < kOPer; ++u) {
                if ((keep >> u) & 1u) {
                    const int64_t i = (int64_t)kOPer * tid + u;
                    if (slot < (uint32_t)k) {
                        oi[slot] = (int32_t)sh.b[i];
                        if (os) os[slot] = key_value(sh.a[i]);
                    }
                    ++slot;
                }
            }
            return;
        }
    }
    if (MODE != 2 && !full) {
        // group maxima into LDS (all loads in flight together) and their range
        const float* gm = gmax + row * gld;
        float* gv = reinterpret_cast<float*>(sh.a);
        constexpr int kPer = kGMaxGroups / kGThreads;
        float v[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int64_t j = tid + (int64_t)u * kGThreads;
            v[u] = j < ng ? gm[j] : -INFINITY;
        }
        float flo = INFINITY, fhi = -INFINITY;
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int64_t j = tid + (int64_t)u * kGThreads;
            if (j < ng) {
                gv[j] = v[u];
                flo = fminf(flo, v[u]);
                fhi = fmaxf(fhi, v[u]);
            }
        }
        for (int i2 = tid; i2 < kGBins; i2 += kGThreads) sh.ghist[i2] = 0u;
        if (tid == 0) {
            sh.ngroups = 0u;
            sh.ncand = 0u;
        }
        uint32_t klo = order_key(flo), khi = order_key(fhi);
        block_minmax(klo, khi, sh);   // its barriers also publish the maxima and the cleared bins
        flo = key_value(klo);
        fhi = key_value(khi);
        float inv = (float)kGBins / (fhi - flo);
        if (!(fhi > flo) || !isfinite(inv)) inv = 0.f;
        // b*: the highest linear bin with at least k group maxima in it and above.  Every
        // group in a bin >= b* has an entry in a bin >= b*, so the row's top k are among the
        // entries in bins >= b* of those groups.
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int64_t j = tid + (int64_t)u * kGThreads;
            if (j < ng) atomicAdd(&sh.ghist[bin_of_n<kGBins>(v[u], flo, inv)], 1u);
        }
        __syncthreads();
        {
            static_assert(kGBins == 2 * kGThreads, "two bins per thread");
            const int top = kGBins - 1 - 2 * tid;
            const uint32_t h0 = sh.ghist[top], h1 = sh.ghist[top - 1];
            uint32_t total;
            const uint32_t before = block_excl_scan<kGWaves>(h0 + h1, sh.scan, &total);
            if (before < (uint32_t)k && before + h0 + h1 >= (uint32_t)k) sh.bstar = before + h0 >= (uint32_t)k ? top : top - 1;
        }
        __syncthreads();
        const int bstar = sh.bstar;
        auto in_b = [&](int64_t e, float x) { return e < nv && bin_of_n<kGBins>(x, flo, inv) >= bstar; };
        if constexpr (MODE == 1) {
            // this slice's groups whose maximum is in a bin >= b*: their entries in bins >= b*
            // (G >= 4: 16-byte pieces, 1 << lq per group, kSP consecutive ones per thread, all
            // loads in flight together); placed by one block scan (so the slice's chunk of the
            // list is in index order) and one atomic per workgroup on the row's count
            constexpr int kSP = kSliceGroups * (kGMaxG / 4) / kGThreads;
            const int lq = __builtin_ctz((unsigned)G) - 2;
            const int64_t j0 = (int64_t)slice * kSliceGroups, j1 = min(ng, j0 + kSliceGroups);
            const int npieces = j1 > j0 ? (int)((j1 - j0) << lq) : 0;
            int64_t e0[kSP];
            float xs[4 * kSP];
#pragma unroll
            for (int u = 0; u < kSP; ++u) {
                const int q = kSP * tid + u;
                const int64_t j = j0 + (q >> lq);
                e0[u] = (q < npieces && bin_of_n<kGBins>(gv[j], flo, inv) >= bstar)
                            ? (j << (lq + 2)) + ((int64_t)(q & ((1 << lq) - 1)) << 2) : -1;
                if (e0[u] >= nv) e0[u] = -1;   // wholly past the row (see step 2 of MODE 0)
                const float4 x4 = e0[u] >= 0 ? *reinterpret_cast<const float4*>(sc + e0[u]) : make_float4(0.f, 0.f, 0.f, 0.f);
                xs[4 * u] = x4.x;
                xs[4 * u + 1] = x4.y;
                xs[4 * u + 2] = x4.z;
                xs[4 * u + 3] = x4.w;
            }
            uint32_t mask = 0u;
#pragma unroll
            for (int u = 0; u < kSP; ++u)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (e0[u] >= 0 && in_b(e0[u] + c, xs[4 * u + c])) mask |= 1u << (4 * u + c);
            uint32_t total;
            const uint32_t pre = block_excl_scan<kGWaves>((uint32_t)__popc(mask), sh.scan, &total);
            if (total == 0u) return;
            if (tid == 0) {
                const uint32_t at0 = atomicAdd(&ccount[row * ccount_ld], total);
                sh.ngroups = at0;
                // this slice's chunk of the list (its candidates in index order): start, count
                ccount[row * ccount_ld + 1 + 2 * slice] = at0;
                ccount[row * ccount_ld + 2 + 2 * slice] = total;
            }
            __syncthreads();
            uint32_t at = sh.ngroups + pre;
#pragma unroll
            for (int u = 0; u < kSP; ++u)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if ((mask >> (4 * u + c)) & 1u) {
                        if (at < (uint32_t)kMCap) {
                            cval[row * kMCap + at] = xs[4 * u + c];
                            cidx[row * kMCap + at] = (int32_t)(e0[u] + c);
                        }
                        ++at;
                    }
                }
            return;
        }
        // the selected groups in index order: thread t takes groups kPer*t .. kPer*t + kPer-1,
        // one block scan of the per-thread counts places them (no atomics on one counter)
        {
            uint32_t tk = 0u, cnt = 0u;
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const int64_t j = (int64_t)kPer * tid + u;
                if (j < ng && bin_of_n<kGBins>(gv[j], flo, inv) >= bstar) {
                    tk |= 1u << u;
                    ++cnt;
                }
            }
            uint32_t total;
            uint32_t p = block_excl_scan<kGWaves>(cnt, sh.scan, &total);
#pragma unroll
            for (int u = 0; u < kPer; ++u)
                if ((tk >> u) & 1u) sh.b[p++] = (uint32_t)(kPer * tid + u);
            if (tid == 0) sh.ngroups = total;
        }
        __syncthreads();
        const int64_t nsel = sh.ngroups;
        // candidates: their entries in bins >= b*, loaded 8 at a time per thread (16-byte loads
        // for groups of 4 or more); a thread's takes form a bit mask, and one wave-wide scan of
        // the per-lane counts places them
        uint32_t lo = ~0u, hi = 0u;
        // (NX values per thread, PER consecutive entries from each ebase; static indexing keeps
        // the arrays in registers)
        auto append = [&](uint32_t mask, const int64_t* ebase, const float* xs, auto nx_tag, auto per_tag) {
            constexpr int NX = decltype(nx_tag)::value, PER = decltype(per_tag)::value;
            const uint32_t c = __popc(mask);
            const uint32_t inc = wave_incl_scan(c);
            uint32_t base = 0;
            if (lane == kWave - 1 && inc) base = atomicAdd(&sh.ncand, inc);
            base = __builtin_amdgcn_readlane(base, kWave - 1) + inc - c;
#pragma unroll
            for (int bit = 0; bit < NX; ++bit) {
                if ((mask >> bit) & 1u) {
                    const int64_t e = ebase[bit / PER] + bit % PER;
                    const uint32_t key = order_key(xs[bit]);
                    lo = min(lo, key);
                    hi = max(hi, key);
                    if (base < (uint32_t)kGCap) {
                        sh.ckey[base] = key;
                        sh.cidx[base] = (int32_t)e;
                    }
                    ++base;
                }
            }
        };
        if (G >= 4) {
            const int lq = __builtin_ctz((unsigned)G) - 2;   // 16-byte pieces per group: 1 << lq
            const int64_t nq = nsel << lq;
            // kCPer pieces per thread, every load of a round in flight together: the ~k selected
            // groups of a k = 1024 selection take one round (8 pieces per thread took two)
            constexpr int kCPer = 12, kCHalf = kCPer / 2;
            for (int64_t q0 = 0; q0 < nq; q0 += kCPer * kGThreads) {
                float xs[4 * kCPer];
                int64_t e0[kCPer];
#pragma unroll
                for (int u = 0; u < kCPer; ++u) {
                    const int64_t q = q0 + tid + (int64_t)u * kGThreads;
                    e0[u] = q < nq ? ((int64_t)sh.b[q >> lq] << (lq + 2)) + ((q & ((1 << lq) - 1)) << 2) : -1;
                    if (e0[u] >= nv) e0[u] = -1;   // wholly past the row (a piece that starts below
                                                   // nv <= N ends inside the row's ld >= N, ld % 4 == 0)
                    const float4 x4 = e0[u] >= 0 ? *reinterpret_cast<const float4*>(sc + e0[u]) : make_float4(0.f, 0.f, 0.f, 0.f);
                    xs[4 * u] = x4.x;
                    xs[4 * u + 1] = x4.y;
                    xs[4 * u + 2] = x4.z;
                    xs[4 * u + 3] = x4.w;
                }
                // appended in two halves (a thread's takes of a half fit one 32-bit mask)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    uint32_t mask = 0u;
#pragma unroll
                    for (int u = 0; u < kCHalf; ++u)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int uu = kCHalf * hf + u;
                            if (e0[uu] >= 0 && in_b(e0[uu] + c, xs[4 * uu + c])) mask |= 1u << (4 * u + c);
                        }
                    append(mask, e0 + kCHalf * hf, xs + 4 * kCHalf * hf, std::integral_constant<int, 4 * kCHalf>{},
                           std::integral_constant<int, 4>{});
                }
            }
        } else {
            const int lg = __builtin_ctz((unsigned)G);
            const int64_t ne = nsel << lg;
            for (int64_t i0 = 0; i0 < ne; i0 += 8 * kGThreads) {
                float xs[8];
                int64_t e[8];
                uint32_t mask = 0u;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t i2 = i0 + tid + (int64_t)u * kGThreads;
                    e[u] = i2 < ne ? ((int64_t)sh.b[i2 >> lg] << lg) + (i2 & (G - 1)) : -1;
                    xs[u] = e[u] >= 0 && e[u] < nv ? sc[e[u]] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (e[u] >= 0 && in_b(e[u], xs[u])) mask |= 1u << u;
                append(mask, e, xs, std::integral_constant<int, 8>{}, std::integral_constant<int, 1>{});
            }
        }
        block_minmax(lo, hi, sh);   // (its barrier also publishes the candidates)
        ncand = sh.ncand;
        if (ncand > kGCap || ncand < k) full = true;   // heavy ties at b* (the second cannot happen)
        else
            kstar = radix_kth<kGThreads>(
                [&](auto f) {
                    for (int64_t i2 = tid; i2 < ncand; i2 += kGThreads) f(sh.ckey[i2]);
                },
                (uint32_t)k, lo, hi, sh.hist, sh.ctl, &need_eq);
    }
    if (full) {
        uint32_t lo = ~0u, hi = 0u;
        for (int64_t e = tid; e < nv; e += kGThreads) {
            const uint32_t key = order_key(sc[e]);
            lo = min(lo, key);
            hi = max(hi, key);
        }
        block_minmax(lo, hi, sh);
        kstar = radix_kth<kGThreads>(
            [&](auto f) {
                for (int64_t e = tid; e < nv; e += kGThreads) f(order_key(sc[e]));
            },
            (uint32_t)k, lo, hi, sh.hist, sh.ctl, &need_eq);
    }

    // bitmaps: kept (key > K*) in b, ties (key == K*) in a
    const int64_t nwords = (nv + 31) >> 5;
    for (int64_t w = tid; w < nwords; w += kGThreads) {
        sh.a[w] = 0u;
        sh.b[w] = 0u;
    }
    if (tid == 0) sh.neq = 0u;
    __syncthreads();
    if (!full) {
        uint32_t neq = 0u;
        for (int64_t i = tid; i < ncand; i += kGThreads) {
            const uint32_t key = sh.ckey[i];
            const int32_t e = sh.cidx[i];
            if (key > kstar) {
                atomicOr(&sh.b[e >> 5], 1u << (e & 31));
            } else if (key == kstar) {
                atomicOr(&sh.a[e >> 5], 1u << (e & 31));
                ++neq;
            }
        }
        if (neq != 0u) atomicAdd(&sh.neq, neq);
    } else {
        // one ballot per 64 entries gives two words of each bitmap
        for (int64_t b0 = (int64_t)wid * kWave; b0 < nv; b0 += kGThreads) {
            const int64_t e = b0 + lane;
            const bool ok = e < nv;
            const uint32_t key = ok ? order_key(sc[e]) : 0u;
            const unsigned long long gt = __ballot(ok && key > kstar);
            const unsigned long long eq = __ballot(ok && key == kstar);
            if (lane == 0) {
                if (eq != 0ull) atomicAdd(&sh.neq, (uint32_t)__popcll(eq));
                sh.b[b0 >> 5] = (uint32_t)gt;
                sh.a[b0 >> 5] = (uint32_t)eq;
                if ((b0 >> 5) + 1 < nwords) {
                    sh.b[(b0 >> 5) + 1] = (uint32_t)(gt >> 32);
                    sh.a[(b0 >> 5) + 1] = (uint32_t)(eq >> 32);
                }
            }
        }
    }
    __syncthreads();

    // ordered extraction.  Wave v owns words [v*R, v*R + R) (R a multiple of 64) and lane l of
    // its round j takes word v*R + 64*j + l, so that every LDS access of a round is one
    // contiguous run (threads that own runs of consecutive words hit the same banks 16 times
    // over: 4.5 us of scans at a 1M context).  A word's prefix in index order is the earlier
    // waves' total, the wave's earlier rounds' totals and the earlier lanes' counts in its round.
    constexpr int kXR = kGMaxRow / 32 / kGThreads;   // rounds at most
    const int64_t R = ((nwords + kGWaves - 1) / kGWaves + kWave - 1) / kWave * kWave;
    const int nr = (int)(R / kWave);
    auto word_at = [&](int j) { return (int64_t)wid * R + (int64_t)kWave * j + lane; };
    // pre[j]: the sum of c over the words before word_at(j) (c is 0 past the row)
    auto prefix = [&](const uint32_t (&c)[kXR], uint32_t (&pre)[kXR]) {
        uint32_t run = 0u;
#pragma unroll
        for (int j = 0; j < kXR; ++j) {
            if (j < nr) {
                const uint32_t inc = wave_incl_scan(c[j]);
                pre[j] = run + inc - c[j];
                run += __builtin_amdgcn_readlane(inc, kWave - 1);
            }
        }
        uint32_t total;
        const uint32_t wb = block_excl_scan<kGWaves>(lane == 0 ? run : 0u, sh.scan, &total);
        const uint32_t base = __builtin_amdgcn_readlane(wb, 0);
#pragma unroll
        for (int j = 0; j < kXR; ++j) pre[j] += base;
    };
    uint32_t eq[kXR], kw[kXR], cnt[kXR], pre[kXR];
#pragma unroll
    for (int j = 0; j < kXR; ++j) {
        const int64_t w = word_at(j);
        const bool in = j < nr && w < nwords;
        eq[j] = in ? sh.a[w] : 0u;
        kw[j] = in ? sh.b[w] : 0u;
        cnt[j] = __popc(eq[j]);
    }
    if (sh.neq == need_eq) {   // every entry equal to K* is taken (block-uniform)
#pragma unroll
        for (int j = 0; j < kXR; ++j) {
            kw[j] |= eq[j];
            cnt[j] = __popc(kw[j]);
        }
    } else {
        prefix(cnt, pre);   // the ties before each word decide how many of its own it keeps
#pragma unroll
        for (int j = 0; j < kXR; ++j) {
            const uint32_t taken = pre[j];
            uint32_t eqw = eq[j];
            if (taken >= need_eq) eqw = 0u;
            else if (taken + __popc(eqw) > need_eq) eqw = first_bits(eqw, need_eq - taken);
            kw[j] |= eqw;
            cnt[j] = __popc(kw[j]);
        }
    }
    prefix(cnt, pre);   // kept entries before each word
    if (!full) {
        // every kept entry is a candidate: its slot is the kept count before its word plus
        // the kept bits below it in the word; its score comes back from its key
#pragma unroll
        for (int j = 0; j < kXR; ++j) {
            const int64_t w = word_at(j);
            if (j < nr && w < nwords) {
                sh.b[w] = kw[j];
                sh.a[w] = pre[j];
            }
        }
        __syncthreads();
        for (int64_t i2 = tid; i2 < ncand; i2 += kGThreads) {
            const int32_t e = sh.cidx[i2];
            const uint32_t word = sh.b[e >> 5], bit = 1u << (e & 31);
            if (word & bit) {
                const uint32_t slot = sh.a[e >> 5] + __popc(word & (bit - 1u));
                oi[slot] = e;
                if (os) os[slot] = key_value(sh.ckey[i2]);
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < kXR; ++j) {
        uint32_t word = kw[j], pos = pre[j];
        const int64_t w = word_at(j);
        while (word) {
            const int bit = __ffs(word) - 1;
            word &= word - 1;
            const int64_t e = (w << 5) + bit;
            if (pos < (uint32_t)k) {
                oi[pos] = (int32_t)e;
                if (os) os[pos] = sc[e];
            }
            ++pos;
        }
    }
}

// ============================================================================ register-staged
// Decode rows of up to 32768 visible entries with at least 8k of them (few queries, long
// rows): one 1024-thread workgroup per row keeps the row in registers (float4 j of the row in
// thread j % 1024, eight per thread, loaded coalesced; the nv % 4 last entries one per
// thread).  Each float4 is a group of 4 entries.
//   1  the group maxima, their range, a 2048-bin histogram linear in value of them (8 LDS
//      atomics per thread instead of 32) and b1: the highest bin with at least k group maxima
//      in it and above.  Those k groups hold k distinct entries in bins >= b1 and binning is
//      monotonic, so the k-th largest entry and every entry of the top k (ties included) lie
//      in bins >= b1: these are the candidates, about k of them.
//   2  the groups whose maximum is in a bin >= b1 (about k) are copied to an LDS list, one
//      wave ballot per float4; their entries in bins >= b1 become the candidates (value,
//      index), counted at once into a second linear histogram over the candidates' range
//   3  candidates above the bin b2 that holds the k-th largest are kept; b2's few members
//      are ranked inside one wave (value desc, index asc) and the first need2 kept
//   4  kept entries set their bit in a row bitmap; a block scan of the word popcounts gives
//      each kept candidate its output slot (ids ascending)
// The bin that holds the k-th largest count is found by one wave (32 bins per lane, one wave
// scan) while the others wait at the next barrier.  More than kRGCap selected groups or kRCap
// candidates (heavy ties) take an exact radix select over the row's keys, more than 64
// members of b2 one over those members; ties at the cut are then resolved in index order
// through a tie bitmap.
constexpr int kRThreads = 1024;
constexpr int kRWaves = kRThreads / kWave;
constexpr int kRRow = 32768;                     // visible entries per row, at most
constexpr int kRF4 = kRRow / (4 * kRThreads);    // float4 per thread
constexpr int kRBins = 2048;
constexpr int kRGCap = 4096;                     // selected groups
constexpr int kRCap = 4096;                      // candidates
constexpr int kRWords = kRRow / 32;
static_assert(kRWords == kRThreads, "one bitmap word per thread");
static_assert(kRBins == 32 * kWave, "32 bins per lane of the searching wave");
static_assert(kRGCap % kRThreads == 0, "whole rounds over the group list");

struct RegShared {
    float4 gval[kRGCap];         // selected groups: values and float4 index
    uint16_t gidx[kRGCap];
    uint2 cand[kRCap];           // candidates: (value bits, index)
    uint32_t kept[kRWords];
    uint32_t ties[kRWords];
    uint32_t wpos[kRWords];      // kept entries before each word
    uint32_t hist[kRBins];       // group maxima; later the radix select's digits
    uint32_t hist2[kRBins];      // candidates
    uint2 mem[kWave];            // members of b2
    float red_lo[kRWaves], red_hi[kRWaves];
    uint32_t ured_lo[kRWaves], ured_hi[kRWaves];
    uint32_t scan[kRWaves];
    uint32_t ctl[3];
    int b1, b2;
    uint32_t need2, ngsel, ncand, nmem;
};

// block-wide min / max of order keys (every thread gets both)
__device__ __forceinline__ void block_minmax_keys(uint32_t& lo, uint32_t& hi, RegShared& sh) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, kWave));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, kWave));
    }
    if (lane == 0) {
        sh.ured_lo[wid] = lo;
        sh.ured_hi[wid] = hi;
    }
    __syncthreads();
    lo = sh.ured_lo[0];
    hi = sh.ured_hi[0];
#pragma unroll
    for (int w = 1; w < kRWaves; ++w) {
        lo = min(lo, sh.ured_lo[w]);
        hi = max(hi, sh.ured_hi[w]);
    }
    __syncthreads();
}

// One wave: the bin of kRBins that holds the k-th largest of the counted values, searched from
// the top; *b receives it and *need how many of its members belong to the k largest (nothing
// is written when the counts sum to less than k).  Lane l sums the l-th chunk of 32 bins from
// the top (16-byte reads rotated by l / 2 so that 16 lanes hit 16 different bank groups), a
// wave scan finds the chunk, then the chunk's bins one per lane and a second scan the bin.
__device__ __forceinline__ void wave_kth_bin(const uint32_t* hist, uint32_t k, int* b, uint32_t* need) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint4* h4 = reinterpret_cast<const uint4*>(hist + kRBins - 32 * (lane + 1));
    uint32_t sum = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint4 x = h4[(q + (lane >> 1)) & 7];
        sum += x.x + x.y + x.z + x.w;
    }
    const uint32_t inc = wave_incl_scan(sum);
    const unsigned long long hit = __ballot(inc - sum < k && inc >= k);   // at most one lane
    if (hit == 0ull) return;
    const int L = __builtin_ctzll(hit);
    const uint32_t before = __builtin_amdgcn_readlane(inc - sum, L);
    const int bin = kRBins - 32 * L - 1 - lane;   // lanes 0-31: the chunk's bins, top down
    const uint32_t h = lane < 32 ? hist[bin] : 0u;
    const uint32_t inc2 = before + wave_incl_scan(h);
    if (lane < 32 && inc2 - h < k && inc2 >= k) {   // exactly one lane
        *b = bin;
        if (need) *need = k - (inc2 - h);
    }
}

__global__ void __launch_bounds__(kRThreads)
topk_regs(const float* __restrict__ scores, int64_t ld, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
          int32_t* __restrict__ idx, float* __restrict__ sel) {
    __shared__ RegShared sh;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: scalar registers
    const int64_t row = blockIdx.x;
    const int64_t nv = visible_entries(q_pos0 + row % T, m, N);
    const float* sc = scores + row * ld;
    int32_t* oi = idx + row * k;
    float* os = sel ? sel + row * k : nullptr;
    if (nv <= k) {
        for (int r = tid; r < k; r += kRThreads) {
            oi[r] = r < nv ? r : -1;
            if (os) os[r] = r < nv ? sc[r] : -INFINITY;
        }
        return;
    }
    // (the launcher sends rows of at most kRRow visible entries)
    const int nvi = (int)nv, n4 = nvi >> 2;
    const float4* s4 = reinterpret_cast<const float4*>(sc);
    float4 v[kRF4];
#pragma unroll
    for (int u = 0; u < kRF4; ++u) {
        const int j = tid + u * kRThreads;
        v[u] = j < n4 ? s4[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int et = 4 * n4 + tid;   // the last nv % 4 entries, one per thread
    const bool has_t = et < nvi;
    const float vt = has_t ? sc[et] : 0.f;
    auto valid = [&](int u) { return tid + u * kRThreads < n4; };

    // LDS state cleared while the loads are in flight
    sh.kept[tid] = 0u;
    sh.ties[tid] = 0u;
    sh.hist[tid] = 0u;
    sh.hist[tid + kRThreads] = 0u;
    sh.hist2[tid] = 0u;
    sh.hist2[tid + kRThreads] = 0u;
    if (tid == 0) {
        sh.ngsel = 0u;
        sh.ncand = 0u;
        sh.nmem = 0u;
        sh.b1 = 0;   // stays 0 when the groups number fewer than k: every entry is a candidate
        sh.b2 = 0;
        sh.need2 = 0u;
    }

    // ---- 1: group maxima, their range, histogram, b1
    float gm[kRF4];
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int u = 0; u < kRF4; ++u) {
        gm[u] = fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w));
        if (valid(u)) {
            lo = fminf(lo, gm[u]);
            hi = fmaxf(hi, gm[u]);
        }
    }
    if (has_t) {
        lo = fminf(lo, vt);
        hi = fmaxf(hi, vt);
    }
    lo = wave_ext<false>(lo);
    hi = wave_ext<true>(hi);
    if (lane == 0) {
        sh.red_lo[wid] = lo;
        sh.red_hi[wid] = hi;
    }
    __syncthreads();
    lo = sh.red_lo[0];
    hi = sh.red_hi[0];
#pragma unroll
    for (int w = 1; w < kRWaves; ++w) {
        lo = fminf(lo, sh.red_lo[w]);
        hi = fmaxf(hi, sh.red_hi[w]);
    }
    float inv = (float)kRBins / (hi - lo);
    if (!(hi > lo) || !isfinite(inv)) inv = 0.f;
    int gb[kRF4];   // the groups' bins (-1: no group)
#pragma unroll
    for (int u = 0; u < kRF4; ++u) {
        gb[u] = valid(u) ? bin_of_n<kRBins>(gm[u], lo, inv) : -1;
        if (gb[u] >= 0) atomicAdd(&sh.hist[gb[u]], 1u);
    }
    if (has_t) atomicAdd(&sh.hist[bin_of_n<kRBins>(vt, lo, inv)], 1u);
    __syncthreads();
    if (wid == 0) wave_kth_bin(sh.hist, (uint32_t)k, &sh.b1, nullptr);
    __syncthreads();
    const int b1 = sh.b1;

    // ---- 2: an entry is in a bin >= b1 iff (v - lo) * inv >= b1 (the expression the bins come
    // from, before clamping; every entry when b1 = 0).  First the groups whose maximum is:
    const float thr = (float)b1;
    auto is_cand = [&](float x) { return b1 == 0 || (x - lo) * inv >= thr; };
    {
        // (a group is selected iff its bin is >= b1: the same test on its maximum)
        unsigned long long sm[kRF4];
        uint32_t wtot = 0u;
#pragma unroll
        for (int u = 0; u < kRF4; ++u) {
            sm[u] = __ballot(gb[u] >= b1);
            wtot += (uint32_t)__popcll(sm[u]);
        }
        uint32_t gbase = 0u;
        if (lane == 0 && wtot != 0u) gbase = atomicAdd(&sh.ngsel, wtot);
        gbase = __builtin_amdgcn_readlane(gbase, 0);
        if (gbase + wtot <= (uint32_t)kRGCap) {   // (else the row takes the radix select)
#pragma unroll
            for (int u = 0; u < kRF4; ++u) {
                if (gb[u] >= b1) {
                    const uint32_t slot = gbase + __builtin_amdgcn_mbcnt_hi((uint32_t)(sm[u] >> 32),
                                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)sm[u], 0u));
                    sh.gval[slot] = v[u];
                    sh.gidx[slot] = (uint16_t)(tid + u * kRThreads);
                }
                gbase += (uint32_t)__popcll(sm[u]);
            }
        }
    }
    __syncthreads();
    const uint32_t ngsel = sh.ngsel;
    // the candidates' histogram: over [about the lower edge of b1, hi] (b1 > 0: inv > 0)
    const float lo2 = b1 > 0 ? lo + thr / inv : lo;
    float inv2 = (float)kRBins / (hi - lo2);
    if (!(hi > lo2) || !isfinite(inv2)) inv2 = 0.f;
    bool row_select = ngsel > (uint32_t)kRGCap;   // heavy ties (block-uniform)
    if (!row_select) {
        // the selected groups' entries in bins >= b1 (and the tail's), appended with one
        // atomic per wave and counted into the second histogram
        for (uint32_t i0 = 0; i0 == 0 || i0 < ngsel; i0 += kRThreads) {   // (the tail: round 0)
            const uint32_t i = i0 + tid;
            const bool ok = i < ngsel;
            const float4 x = ok ? sh.gval[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            const int e0 = ok ? 4 * (int)sh.gidx[i] : 0;
            const bool tl = i0 == 0 && has_t && is_cand(vt);
            const uint32_t cm = (ok && is_cand(x.x) ? 1u : 0u) | (ok && is_cand(x.y) ? 2u : 0u) |
                                (ok && is_cand(x.z) ? 4u : 0u) | (ok && is_cand(x.w) ? 8u : 0u) | (tl ? 16u : 0u);
            const uint32_t cnt = (uint32_t)__popc(cm);
            const uint32_t inc = wave_incl_scan(cnt);
            uint32_t base = 0u;
            if (lane == kWave - 1 && inc != 0u) base = atomicAdd(&sh.ncand, inc);
            base = __builtin_amdgcn_readlane(base, kWave - 1) + inc - cnt;
            auto put = [&](float xv, int e) {
                if (base < (uint32_t)kRCap) sh.cand[base] = make_uint2(__float_as_uint(xv), (uint32_t)e);
                ++base;
                atomicAdd(&sh.hist2[bin_of_n<kRBins>(xv, lo2, inv2)], 1u);
            };
            if (cm & 1u) put(x.x, e0);
            if (cm & 2u) put(x.y, e0 + 1);
            if (cm & 4u) put(x.z, e0 + 2);
            if (cm & 8u) put(x.w, e0 + 3);
            if (cm & 16u) put(vt, et);
        }
        __syncthreads();
        row_select = sh.ncand > (uint32_t)kRCap;
    }
    const uint32_t ncand = sh.ncand;   // >= k: the candidates hold the top k

    // ---- 3: the cut.  Entries set in `kept` are taken; of the entries set in `ties` (equal to
    // the k-th key K*) the first need_eq in index order are taken too.
    bool with_ties = false;
    uint32_t need_eq = 0u;
    if (!row_select) {
        if (wid == 0) wave_kth_bin(sh.hist2, (uint32_t)k, &sh.b2, &sh.need2);
        __syncthreads();
        const int b2 = sh.b2;
        const uint32_t need2 = sh.need2;
        // candidates above b2 are kept; b2's members are listed (every lane of a wave runs the
        // same trip count: the list append is wave-wide)
        for (uint32_t i0 = 0; i0 < ncand; i0 += kRThreads) {
            const uint32_t i = i0 + tid;
            const bool ok = i < ncand;
            const uint2 c = ok ? sh.cand[i] : make_uint2(0u, 0u);
            const int bn = ok ? bin_of_n<kRBins>(__uint_as_float(c.x), lo2, inv2) : -1;
            if (bn > b2) atomicOr(&sh.kept[c.y >> 5], 1u << (c.y & 31));
            const bool mb = bn == b2;
            const uint32_t p = wave_append(mb, &sh.nmem);
            if (mb && p < (uint32_t)kWave) sh.mem[p] = c;
        }
        __syncthreads();
        const uint32_t nmem = sh.nmem;
        if (nmem <= (uint32_t)kWave) {
            // lane i holds member i; the others' keys come by readlane (no LDS round trips)
            if (wid == 0) {
                const bool have = (uint32_t)lane < nmem;
                const uint2 c = have ? sh.mem[lane] : make_uint2(0u, 0u);
                const uint32_t ki = order_key(__uint_as_float(c.x));
                uint32_t rank = 0u;
                for (uint32_t j = 0; j < nmem; ++j) {
                    const uint32_t kj = __builtin_amdgcn_readlane(ki, j);
                    const uint32_t sj = __builtin_amdgcn_readlane(c.y, j);
                    rank += (kj > ki || (kj == ki && sj < c.y)) ? 1u : 0u;
                }
                if (have && rank < need2) atomicOr(&sh.kept[c.y >> 5], 1u << (c.y & 31));
            }
        } else {
            // many members (ties): K* among them by radix select
            auto visit = [&](auto f) {
                for (uint32_t i = tid; i < ncand; i += kRThreads) {
                    const float x = __uint_as_float(sh.cand[i].x);
                    if (bin_of_n<kRBins>(x, lo2, inv2) == b2) f(order_key(x));
                }
            };
            uint32_t klo = ~0u, khi = 0u;
            visit([&](uint32_t key) {
                klo = min(klo, key);
                khi = max(khi, key);
            });
            block_minmax_keys(klo, khi, sh);
            const uint32_t kstar = radix_kth<kRThreads>(visit, need2, klo, khi, sh.hist, sh.ctl, &need_eq);
            for (uint32_t i = tid; i < ncand; i += kRThreads) {
                const uint2 c = sh.cand[i];
                const float x = __uint_as_float(c.x);
                if (bin_of_n<kRBins>(x, lo2, inv2) != b2) continue;
                const uint32_t key = order_key(x);
                if (key > kstar) atomicOr(&sh.kept[c.y >> 5], 1u << (c.y & 31));
                else if (key == kstar) atomicOr(&sh.ties[c.y >> 5], 1u << (c.y & 31));
            }
            with_ties = true;
        }
    } else {
        // heavy ties: K* over the whole row (keys from the registers)
        auto visit = [&](auto f) {
#pragma unroll
            for (int u = 0; u < kRF4; ++u) {
                if (!valid(u)) continue;
                f(order_key(v[u].x));
                f(order_key(v[u].y));
                f(order_key(v[u].z));
                f(order_key(v[u].w));
            }
            if (has_t) f(order_key(vt));
        };
        uint32_t klo = ~0u, khi = 0u;
        visit([&](uint32_t key) {
            klo = min(klo, key);
            khi = max(khi, key);
        });
        block_minmax_keys(klo, khi, sh);
        const uint32_t kstar = radix_kth<kRThreads>(visit, (uint32_t)k, klo, khi, sh.hist, sh.ctl, &need_eq);
        // float4 j holds entries 4j .. 4j+3: bits 4 (j % 8) .. of word j / 8
#pragma unroll
        for (int u = 0; u < kRF4; ++u) {
            if (!valid(u)) continue;
            const int j = tid + u * kRThreads;
            const float xs[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            uint32_t kn = 0u, tn = 0u;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t key = order_key(xs[c]);
                kn |= (key > kstar ? 1u : 0u) << c;
                tn |= (key == kstar ? 1u : 0u) << c;
            }
            if (kn) atomicOr(&sh.kept[j >> 3], kn << (4 * (j & 7)));
            if (tn) atomicOr(&sh.ties[j >> 3], tn << (4 * (j & 7)));
        }
        if (has_t) {
            const uint32_t key = order_key(vt);
            if (key > kstar) atomicOr(&sh.kept[et >> 5], 1u << (et & 31));
            else if (key == kstar) atomicOr(&sh.ties[et >> 5], 1u << (et & 31));
        }
        with_ties = true;
    }
    __syncthreads();

    // ---- 4: ordered output, thread w owns bitmap word w
    const int nwords = (nvi + 31) >> 5;
    uint32_t kw = tid < nwords ? sh.kept[tid] : 0u;
    uint32_t total;
    if (with_ties) {
        const uint32_t tw = tid < nwords ? sh.ties[tid] : 0u;
        const uint32_t taken = block_excl_scan<kRWaves>((uint32_t)__popc(tw), sh.scan, &total);
        uint32_t eqw = tw;
        if (taken >= need_eq) eqw = 0u;
        else if (taken + (uint32_t)__popc(tw) > need_eq) eqw = first_bits(tw, need_eq - taken);
        kw |= eqw;
    }
    const uint32_t pos = block_excl_scan<kRWaves>((uint32_t)__popc(kw), sh.scan, &total);
    if (!row_select) {
        // every kept entry is a candidate: its slot is the kept count before its word plus the
        // kept bits below it in the word
        if (tid < nwords) {
            sh.kept[tid] = kw;
            sh.wpos[tid] = pos;
        }
        __syncthreads();
        for (uint32_t i = tid; i < ncand; i += kRThreads) {
            const uint2 c = sh.cand[i];
            const uint32_t word = sh.kept[c.y >> 5], bit = 1u << (c.y & 31);
            if (word & bit) {
                const uint32_t slot = sh.wpos[c.y >> 5] + (uint32_t)__popc(word & (bit - 1u));
                if (slot < (uint32_t)k) {
                    oi[slot] = (int32_t)c.y;
                    if (os) os[slot] = __uint_as_float(c.x);
                }
            }
        }
    } else {
        uint32_t p = pos, word = kw;
        while (word) {
            const int b = __ffs(word) - 1;
            word &= word - 1u;
            const int e = 32 * tid + b;
            if (p < (uint32_t)k) {
                oi[p] = e;
                if (os) os[p] = sc[e];
            }
            ++p;
        }
    }
}

// Short rows (prefill: at most 2048 visible entries), one wave per row and four rows per
// workgroup, with no workgroup barrier: the wave holds its row in registers (entry 64 i + lane
// in value i of the lane, 32 per lane, loaded coalesced), finds the row's range with two wave
// reductions, counts a 256-bin histogram LINEAR in value in its own LDS, and takes the bin b*
// that holds the k-th largest value (bins are monotone in value, so every entry of a higher
// bin is kept and none of a lower one).  The order keys of b*'s members go to a list in the
// wave's LDS; the exact k-th key K* among them and the number of entries equal to it to take
// come from an 8-bit radix select over that list (four passes over the same histogram).  The
// output goes out in index order with one ballot per 64 entries: entry e is kept iff its bin
// is above b*, or it is in b* with key > K*, or key == K* and it is among the first need_eq
// such entries.  (The rows are short and many: the kernel is bound by instruction issue, so
// each value's bin is kept in a register and key work is skipped wherever no lane of the wave
// holds a member of b*.)
constexpr int kWvRow = 2048;                 // longest row served
constexpr int kWvPer = kWvRow / kWave;       // values per lane (32)
constexpr int kWvRows = 4;                   // rows (waves) per workgroup
constexpr int kWvBins = 256;

// the wave's LDS operations so far are complete, and the compiler moves none across this point
// (a wave's histogram and list are only ever touched by that wave)
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    asm volatile("" ::: "memory");
}

// one wave: the bin of `hist` (kWvBins counts) that holds the need-th largest counted value,
// searched from the top, and how many of its members that leaves to take (need >= 1, and the
// counts sum to at least need)
__device__ __forceinline__ void wave_top_bin(const uint32_t* hist, uint32_t need, int* bin, uint32_t* left) {
    const int lane = threadIdx.x & (kWave - 1);
    // lane l: bins 255 - 4l (x.w) down to 252 - 4l (x.x)
    const uint4 x = *reinterpret_cast<const uint4*>(hist + kWvBins - 4 - 4 * lane);
    const uint32_t sum = x.x + x.y + x.z + x.w;
    const uint32_t inc = wave_incl_scan(sum);
    const unsigned long long hit = __ballot(inc - sum < need && inc >= need);   // exactly one lane
    const int L = __builtin_ctzll(hit);
    uint32_t cum = inc - sum;
    int b;
    if (cum + x.w >= need) {
        b = kWvBins - 1 - 4 * lane;
    } else if ((cum += x.w) + x.z >= need) {
        b = kWvBins - 2 - 4 * lane;
    } else if ((cum += x.z) + x.y >= need) {
        b = kWvBins - 3 - 4 * lane;
    } else {
        cum += x.y;
        b = kWvBins - 4 - 4 * lane;
    }
    *bin = __builtin_amdgcn_readlane(b, L);
    *left = need - __builtin_amdgcn_readlane(cum, L);
}

struct WaveTopkShared {
    uint32_t hist[kWvRows][kWvBins];
    uint32_t mem[kWvRows][kWvRow];   // order keys of b*'s members
};

__global__ void __launch_bounds__(kWvRows * kWave)
topk_wave(const float* __restrict__ scores, int64_t ld, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
          int64_t rows, int32_t* __restrict__ idx, float* __restrict__ sel) {
    __shared__ __attribute__((aligned(16))) WaveTopkShared sh;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row = (int64_t)blockIdx.x * kWvRows + wid;
    if (row >= rows) return;   // a whole wave; the kernel has no workgroup barrier
    uint32_t* hist = sh.hist[wid];
    uint32_t* mem = sh.mem[wid];
    const int64_t nv = visible_entries(q_pos0 + row % T, m, N);
    const float* sc = scores + row * ld;
    int32_t* oi = idx + row * k;
    float* os = sel ? sel + row * k : nullptr;
    if (nv <= k) {
        for (int r = lane; r < k; r += kWave) {
            oi[r] = r < nv ? r : -1;
            if (os) os[r] = r < nv ? sc[r] : -INFINITY;
        }
        return;
    }
    // (the launcher sends rows of at most kWvRow visible entries)
    const int nvi = (int)nv;
    // the row's visible entries; loads past them read 0
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sc), (short)0,
                                                                        (int)(4 * nvi), 0x00020000);
    float v[kWvPer];
#pragma unroll
    for (int i = 0; i < kWvPer; ++i)
        v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4u * lane, 4u * kWave * i, 0));
    // value i of this lane is an entry iff i < nmine
    const int nmine = (nvi - lane + kWave - 1) / kWave;

    // range (entries only) and linear bins (inv = 0: one bin, the radix select does all the work)
    float lo = v[0], hi = v[0];   // entry `lane`; lanes past a row of fewer than 64 take entry 0's
    if (lane >= nvi) lo = hi = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v[0])));
#pragma unroll
    for (int i = 1; i < kWvPer; ++i)
        if (i < nmine) {
            lo = fminf(lo, v[i]);
            hi = fmaxf(hi, v[i]);
        }
    lo = wave_ext<false>(lo);
    hi = wave_ext<true>(hi);
    float inv = (float)kWvBins / (hi - lo);
    if (!(hi > lo) || !isfinite(inv)) inv = 0.f;
    *reinterpret_cast<uint4*>(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
    int bn[kWvPer];   // bin of value i (-1: not an entry)
#pragma unroll
    for (int i = 0; i < kWvPer; ++i) {
        bn[i] = i < nmine ? bin_of_n<kWvBins>(v[i], lo, inv) : -1;
        if (i < nmine) atomicAdd(&hist[bn[i]], 1u);
    }
    int bstar;
    uint32_t need;   // members of b* to take (1 .. its count)
    wave_lds_sync();
    wave_top_bin(hist, (uint32_t)k, &bstar, &need);

    // b*'s members' keys to the list
    const unsigned long long below = (1ull << lane) - 1ull;   // lanes before this one
    uint32_t nmem = 0u;
#pragma unroll
    for (int i = 0; i < kWvPer; ++i) {
        const bool mb = bn[i] == bstar;
        const unsigned long long mm = __ballot(mb);
        if (mm != 0ull) {   // wave-uniform
            if (mb) mem[nmem + (uint32_t)__popcll(mm & below)] = order_key(v[i]);
            nmem += (uint32_t)__popcll(mm);
        }
    }

    // K* among the members: 8 bits of the key per pass, from the top
    uint32_t prefix = 0u;
#pragma unroll 1
    for (int p = 0; p < 4; ++p) {
        const int shift = 24 - 8 * p;
        const uint32_t hmask = p == 0 ? 0u : ~0u << (shift + 8);
        wave_lds_sync();
        *reinterpret_cast<uint4*>(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
        for (uint32_t j = lane; j < nmem; j += kWave) {
            const uint32_t key = mem[j];
            if ((key & hmask) == prefix) atomicAdd(&hist[(key >> shift) & (kWvBins - 1)], 1u);
        }
        int d;
        wave_lds_sync();
        wave_top_bin(hist, need, &d, &need);
        prefix |= (uint32_t)d << shift;
    }
    const uint32_t kstar = prefix, need_eq = need;   // take the first need_eq entries with key K*

    // ordered output
    uint32_t base = 0u, eq_seen = 0u;
#pragma unroll
    for (int i = 0; i < kWvPer; ++i) {
        bool take = bn[i] > bstar;
        const bool mb = bn[i] == bstar;
        if (__ballot(mb) != 0ull) {   // wave-uniform: some lane holds a member of b*
            const uint32_t key = order_key(v[i]);
            const bool eq = mb && key == kstar;
            const unsigned long long em = __ballot(eq);
            take = take || (mb && key > kstar) || (eq && eq_seen + (uint32_t)__popcll(em & below) < need_eq);
            eq_seen += (uint32_t)__popcll(em);
        }
        const unsigned long long tm = __ballot(take);
        if (take) {
            const uint32_t slot = base + (uint32_t)__popcll(tm & below);
            oi[slot] = kWave * i + lane;
            if (os) os[slot] = v[i];
        }
        base += (uint32_t)__popcll(tm);
    }
}

// Group size for the group-bounded selection (0: not used): a power of two up to kGMaxG with
// at most kGMaxGroups groups in the longest row, and preferably at least 4k of them.
// Rows that fit the LDS staging of the one-workgroup bitmap selection are faster there.
int group_size(int64_t nv_max, int k) {
    if (nv_max > kGMaxRow || nv_max <= k || nv_max <= kRowLds) return 0;
    int g = 1;
    while ((nv_max + g - 1) / g > kGMaxGroups) g *= 2;
    while (g < kGMaxG && nv_max / (2 * g) >= 4 * (int64_t)k) g *= 2;
    if (g > kGMaxG || (nv_max + g - 1) / g <= k) return 0;
    return g;
}

// rows that fit the LDS staging are faster in one workgroup (no inter-kernel round trips)
bool multi_rows(int64_t rows, int64_t nv_max) { return rows < 256 && nv_max > kRowLds; }

}  // namespace

size_t topk_extra_workspace(int64_t rows, int64_t N, int k) {
    (void)k;
    if (!multi_rows(rows, N)) return 0;
    return multi_bytes(rows, N, nullptr, nullptr);
}

int topk_zero_words(int64_t rows, int64_t nv_max) { return multi_rows(rows, nv_max) ? kZeroWords : 0; }

int topk_group(int64_t nv_max, int k) { return group_size(nv_max, k); }

int launch_topk(const float* scores, int64_t ld, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int m, int k,
                int32_t* idx, float* sel, const float* chunk_mm, int n_chunk_mm, const float* gmax, int G,
                int64_t gld, void* extra_ws, hipStream_t stream) {
    const int64_t rows = batch * T;
    if (rows == 0) return 0;
    if (rows > 0x7fffffffLL) return -2;
    // the longest visible row is that of the last query
    int64_t nv_max = (q_pos0 + T) / m;
    if (nv_max > N) nv_max = N;
    if (gmax != nullptr && G > 0) {   // the indexer wrote the group maxima (G = topk_group)
        if (extra_ws != nullptr && G >= 4 && multi_rows(rows, nv_max)) {
            // few long rows: the candidates of each row found by (row, group slice) workgroups
            // over the chip, then one workgroup per row selects from them (the indexer cleared
            // the rows' candidate counters)
            MultiWs L;
            multi_bytes(rows, N, &L, extra_ws);
            const int P = (int)(((nv_max + G - 1) / G + kSliceGroups - 1) / kSliceGroups);
            // (each row's zeroed region: word 0 the list length, words 1 + 2p, 2 + 2p slice p's chunk)
            static_assert(1 + 2 * kGMaxSlices <= kZeroWords, "the chunk records fit the row's zeroed words");
            hipLaunchKernelGGL(topk_groups<1>, dim3((unsigned)((rows + 7) / 8 * 8 * P)), dim3(kGThreads), 0, stream, scores, ld, T,
                               q_pos0, N, m, k, gmax, gld, G, idx, sel, rows, P, L.zero, kZeroWords, L.cval, L.cidx);
            hipLaunchKernelGGL(topk_groups<2>, dim3((unsigned)rows), dim3(kGThreads), 0, stream, scores, ld, T, q_pos0,
                               N, m, k, gmax, gld, G, idx, sel, rows, P, L.zero, kZeroWords, L.cval, L.cidx);
            return 0;
        }
        hipLaunchKernelGGL(topk_groups<0>, dim3((unsigned)rows), dim3(kGThreads), 0, stream, scores, ld, T, q_pos0, N,
                           m, k, gmax, gld, G, idx, sel, rows, 1, nullptr, 0, nullptr, nullptr);
        return 0;
    }
    if (chunk_mm != nullptr && extra_ws != nullptr && multi_rows(rows, nv_max)) {
        // the indexer zeroed the per-row histogram / counter region (topk_zero_words)
        MultiWs L;
        multi_bytes(rows, N, &L, extra_ws);
        const int P = (int)((nv_max + kSlice - 1) / kSlice);
        const dim3 grid((unsigned)(rows * P));
        hipLaunchKernelGGL(tkm_hist, grid, dim3(kSliceThreads), 0, stream, scores, ld, T, q_pos0, N, m, k, chunk_mm,
                           n_chunk_mm, P, L);
        hipLaunchKernelGGL(tkm_mark, grid, dim3(kSliceThreads), 0, stream, scores, ld, T, q_pos0, N, m, k, chunk_mm,
                           n_chunk_mm, P, L);
        hipLaunchKernelGGL(tkm_select, dim3((unsigned)rows), dim3(kThreads), 0, stream, scores, ld, T, q_pos0, N, m, k,
                           chunk_mm, n_chunk_mm, L, idx, sel);
        return 0;
    }
    const dim3 grid((unsigned)rows), block(kThreads);
    // the shortest visible row is that of each sequence's first query
    int64_t nv_min = (q_pos0 + 1) / m;
    if (nv_min > N) nv_min = N;
    if (rows < 256 && nv_max > kShortRow && nv_max <= kRRow && nv_min >= 8 * (int64_t)k) {
        hipLaunchKernelGGL(topk_regs, grid, dim3(kRThreads), 0, stream, scores, ld, T, q_pos0, N, m, k, idx, sel);
        return 0;
    }
    if (nv_max <= kWvRow) {   // prefill rows of up to 2048 entries: one wave per row
        hipLaunchKernelGGL(topk_wave, dim3((unsigned)((rows + kWvRows - 1) / kWvRows)), dim3(kWvRows * kWave), 0,
                           stream, scores, ld, T, q_pos0, N, m, k, rows, idx, sel);
        return 0;
    }
    if (nv_max <= kShortRow)   // short rows (prefill): small workgroups, several rows per CU
        hipLaunchKernelGGL((topk_bitmap<true, kShortThreads, kShortRow, 2 * kShortThreads>), grid, dim3(kShortThreads),
                           0, stream, scores, ld, T, q_pos0, N, m, k, chunk_mm, n_chunk_mm, idx, sel);
    else if (nv_max <= kRowLds)
        hipLaunchKernelGGL((topk_bitmap<true, kThreads, kRowLds, kBins>), grid, block, 0, stream, scores, ld, T, q_pos0,
                           N, m, k, chunk_mm, n_chunk_mm, idx, sel);
    else if (nv_max <= kBmMaxRow)
        hipLaunchKernelGGL((topk_bitmap<false, kThreads, kRowLds, kBins>), grid, block, 0, stream, scores, ld, T,
                           q_pos0, N, m, k, chunk_mm, n_chunk_mm, idx, sel);
    else
        hipLaunchKernelGGL((topk_row_kernel<false>), grid, block, 0, stream, scores, ld, T, q_pos0, N, m, k, idx, sel);
    return 0;
}

uint32_t* topk_zero_region(void* extra_ws, int64_t rows, int64_t N) {
    MultiWs L;
    multi_bytes(rows, N, &L, extra_ws);
    return L.zero;
}

}  // namespace csa
