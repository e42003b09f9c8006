// indexer.hip — lightning-indexer scores  I[t,s] = sum_h w[t,h] * ReLU(qI[t,h,:] . kI[s,:])
// for every causally visible compressed entry s ("DeepSeek-V4: 迈向高效百万级上下文智能",
// §1.1 step 2, eq. I_{t,s}; mlpod.com DeepSeek-V4 summary §2.3.1: scores only against blocks
// before the query).  fp32 accumulation, ReLU(x) = max(x, +0), no scale factor.
//
// Kernels:
//   index_scores_generic  any dtype / head count: VALU dot products, q of one query in LDS.
//   (the MFMA kernels for the large prefill and decode shapes live further down)
#include "device_common.h"
#include "launch.h"

namespace csa {

namespace {

constexpr int kGenThreads = 256;
constexpr int kGenHeadGroup = 16;
constexpr int kGenMaxLds = 65536;  // bytes of LDS for q (H_I * c_I floats) and w (H_I floats)

template <int DT>
__global__ void __launch_bounds__(kGenThreads)
index_scores_generic(const void* __restrict__ qI, const float* __restrict__ w, const void* __restrict__ kI, int64_t T,
                     int64_t q_pos0, int64_t N, int H_I, int c_I, int m, float* __restrict__ scores, int64_t ld,
                     int write_invisible) {
    extern __shared__ float smem[];
    float* qs = smem;                 // [H_I][c_I]
    float* ws = smem + H_I * c_I;     // [H_I]
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;   // b*T + t
    const int64_t b = row / T, t = row - b * T;
    const int64_t nv = visible_entries(q_pos0 + t, m, N);
    const int64_t qbase = row * H_I * c_I;
    for (int i = tid; i < H_I * c_I; i += kGenThreads) qs[i] = load1<DT>(qI, qbase + i);
    for (int i = tid; i < H_I; i += kGenThreads) ws[i] = w[row * H_I + i];
    __syncthreads();
    float* out = scores + row * ld;
    for (int64_t tile = blockIdx.y; tile * kGenThreads < N; tile += gridDim.y) {
        const int64_t s = tile * kGenThreads + tid;
        if (s >= N) continue;
        if (s >= nv) {
            if (write_invisible) out[s] = -INFINITY;
            continue;
        }
        const int64_t kbase = (b * N + s) * c_I;
        float total = 0.f;
        for (int h0 = 0; h0 < H_I; h0 += kGenHeadGroup) {
            const int hn = min(kGenHeadGroup, H_I - h0);
            float dot[kGenHeadGroup];
#pragma unroll
            for (int hh = 0; hh < kGenHeadGroup; ++hh) dot[hh] = 0.f;
            for (int d = 0; d < c_I; d += 8) {
                float kv[8];
                load8<DT>(kI, kbase + d, kv);
#pragma unroll
                for (int hh = 0; hh < kGenHeadGroup; ++hh) {
                    if (hh < hn) {
                        const float* qp = qs + (h0 + hh) * c_I + d;
#pragma unroll
                        for (int e = 0; e < 8; ++e) dot[hh] = fmaf(qp[e], kv[e], dot[hh]);
                    }
                }
            }
#pragma unroll
            for (int hh = 0; hh < kGenHeadGroup; ++hh)
                if (hh < hn) total = fmaf(ws[h0 + hh], fmaxf(dot[hh], 0.f), total);
        }
        out[s] = total;
    }
}

template <int DT>
int launch_generic(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0, int64_t N,
                   int H_I, int c_I, int m, float* scores, int64_t ld, bool write_invisible, hipStream_t stream) {
    if (((int64_t)H_I * c_I + H_I) * (int64_t)sizeof(float) > kGenMaxLds) return -2;
    const int64_t rows = batch * T;
    if (rows > 0x7fffffffLL) return -2;
    const int64_t tiles = (N + kGenThreads - 1) / kGenThreads;
    const unsigned gy = (unsigned)(tiles < 65535 ? tiles : 65535);
    const size_t lds = ((size_t)H_I * c_I + H_I) * sizeof(float);
    hipLaunchKernelGGL((index_scores_generic<DT>), dim3((unsigned)rows, gy), dim3(kGenThreads), lds, stream, qI, w, kI, T,
                       q_pos0, N, H_I, c_I, m, scores, ld, write_invisible ? 1 : 0);
    return 0;
}

}  // namespace

int launch_index_scores(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0,
                        int64_t N, int H_I, int c_I, int m, int qk_t, float* scores, int64_t ld, bool write_invisible,
                        hipStream_t stream) {
    if (batch == 0 || T == 0 || N == 0) return 0;
    switch (qk_t) {
        case DT_F32:
            return launch_generic<DT_F32>(qI, w, kI, batch, T, q_pos0, N, H_I, c_I, m, scores, ld, write_invisible,
                                          stream);
        case DT_BF16:
            return launch_generic<DT_BF16>(qI, w, kI, batch, T, q_pos0, N, H_I, c_I, m, scores, ld, write_invisible,
                                           stream);
        case DT_FP8:
            return launch_generic<DT_FP8>(qI, w, kI, batch, T, q_pos0, N, H_I, c_I, m, scores, ld, write_invisible,
                                          stream);
    }
    return -2;
}

}  // namespace csa
