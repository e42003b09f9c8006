// mqa.hip — shared-KV multi-query attention over compressed entries.
//
// Operation ("DeepSeek-V4: 迈向高效百万级上下文智能", §1.1 step 2 last paragraph; mlpod.com
// DeepSeek-V4 summary §2.3.2): every query head attends to one shared set of compressed
// entries, each entry serving as key and value:
//     out[t,h,:] = sum_s softmax_s(scale * q[t,h,:] . kv[s,:]) kv[s,:]
// over s in idx[t] (CSA, sparse) or over every visible HCA entry (dense, causal).
//
// mqa_generic: one wave per (query, head), lanes across channels, online softmax over the
// entries four at a time, fp32 throughout.  Works for any c % 8 == 0 up to 1024.  The MFMA
// kernels for the large shapes are further down.
#include "device_common.h"
#include "launch.h"

namespace csa {

namespace {

constexpr int kGenWaves = 4;
constexpr int kKeyBatch = 4;

template <int DT, int CPL, bool DENSE>
__global__ void __launch_bounds__(kGenWaves * kWave)
mqa_generic(const void* __restrict__ q, const void* __restrict__ kv, const int32_t* __restrict__ idx, int64_t T,
            int64_t N, int H, int c, int k, float scale, int64_t q_pos0, int ratio, void* __restrict__ out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int h = blockIdx.y * kGenWaves + threadIdx.x / kWave;
    const int64_t row = blockIdx.x;  // b*T + t
    if (h >= H) return;
    const int64_t b = row / T, t = row - b * T;
    const float sl2 = scale * kLog2e;

    float qv[CPL], acc[CPL];
    const int64_t qbase = (row * H + h) * c;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int d = lane + kWave * j;
        qv[j] = d < c ? load1<DT>(q, qbase + d) : 0.f;
        acc[j] = 0.f;
    }
    float mx = -INFINITY, den = 0.f;

    const int64_t count = DENSE ? visible_entries(q_pos0 + t, ratio, N) : (int64_t)k;
    const int32_t* ids = DENSE ? nullptr : idx + row * k;
    const int64_t kvbase = b * N * c;

    for (int64_t r0 = 0; r0 < count; r0 += kKeyBatch) {
        int64_t sidx[kKeyBatch];
        bool ok[kKeyBatch];
#pragma unroll
        for (int u = 0; u < kKeyBatch; ++u) {
            const int64_t r = r0 + u;
            int64_t s = -1;
            if (r < count) s = DENSE ? r : (int64_t)ids[r];
            ok[u] = s >= 0 && s < N;
            sidx[u] = ok[u] ? s : 0;
        }
        float kvv[kKeyBatch][CPL], part[kKeyBatch];
#pragma unroll
        for (int u = 0; u < kKeyBatch; ++u) {
            part[u] = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int d = lane + kWave * j;
                kvv[u][j] = (ok[u] && d < c) ? load1<DT>(kv, kvbase + sidx[u] * c + d) : 0.f;
                part[u] = fmaf(qv[j], kvv[u][j], part[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kKeyBatch; ++u) part[u] = wave_sum(part[u]);
#pragma unroll
        for (int u = 0; u < kKeyBatch; ++u) {
            if (!ok[u]) continue;   // uniform across the wave
            const float l = part[u] * sl2;
            const float nm = fmaxf(mx, l);
            const float a = exp2f(mx - nm);
            const float p = exp2f(l - nm);
            den = fmaf(den, a, p);
#pragma unroll
            for (int j = 0; j < CPL; ++j) acc[j] = fmaf(acc[j], a, p * kvv[u][j]);
            mx = nm;
        }
    }
    const float rden = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int d = lane + kWave * j;
        if (d < c) store1<DT>(out, qbase + d, acc[j] * rden);
    }
}

template <int DT, bool DENSE>
int launch_generic(const void* q, const void* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N, int H, int c,
                   int k, float scale, int64_t q_pos0, int ratio, void* out, hipStream_t stream) {
    const int64_t rows = batch * T;
    if (rows > 0x7fffffffLL) return -2;
    const int cpl = (c + kWave - 1) / kWave;
    const dim3 grid((unsigned)rows, (unsigned)((H + kGenWaves - 1) / kGenWaves));
#define CSA_LAUNCH_CPL(C)                                                                                          \
    if (cpl <= C) {                                                                                                \
        hipLaunchKernelGGL((mqa_generic<DT, C, DENSE>), grid, dim3(kGenWaves * kWave), 0, stream, q, kv, idx, T, N, H, \
                           c, k, scale, q_pos0, ratio, out);                                                       \
        return 0;                                                                                                  \
    }
    CSA_LAUNCH_CPL(1)
    CSA_LAUNCH_CPL(2)
    CSA_LAUNCH_CPL(4)
    CSA_LAUNCH_CPL(8)
    CSA_LAUNCH_CPL(16)
#undef CSA_LAUNCH_CPL
    return -2;
}

}  // namespace

int launch_sparse_mqa(const void* q, const void* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N, int H,
                      int c, int k, float scale, int t, void* out, hipStream_t stream) {
    if (batch == 0 || T == 0) return 0;
    if (t == DT_F32) return launch_generic<DT_F32, false>(q, kv, idx, batch, T, N, H, c, k, scale, 0, 1, out, stream);
    if (t == DT_BF16) return launch_generic<DT_BF16, false>(q, kv, idx, batch, T, N, H, c, k, scale, 0, 1, out, stream);
    return -2;
}

int launch_dense_mqa(const void* q, const void* kv, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int H, int c,
                     int ratio, float scale, int t, void* out, hipStream_t stream) {
    if (batch == 0 || T == 0) return 0;
    if (t == DT_F32)
        return launch_generic<DT_F32, true>(q, kv, nullptr, batch, T, N, H, c, 0, scale, q_pos0, ratio, out, stream);
    if (t == DT_BF16)
        return launch_generic<DT_BF16, true>(q, kv, nullptr, batch, T, N, H, c, 0, scale, q_pos0, ratio, out, stream);
    return -2;
}

}  // namespace csa
