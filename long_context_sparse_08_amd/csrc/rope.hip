// rope.hip — partial rotary position embedding on the last channels of q / KV rows and its
// inverse on the attention output.
//
// Sources: "DeepSeek-V4: 迈向高效百万级上下文智能" (notes.kuangjux.top) §1.3 and the mlpod.com
// summary §2.3.3 item 2 (RoPE on the last 64 channels of queries and KV entries; the attention
// output gets the rotation of the negative query position, so it carries the query-to-entry
// distance).  The rotation itself follows RoFormer (Su et al. 2021): channel pair
// (2i, 2i+1) of the rotated part turns by position * base^(-2i/d).
//
// A thread takes one (row, pair, group of kRopeHeads heads): every lane works (d/2 = 32 pairs
// fill half a wave), and the rotation of a pair, which is the same for all heads of a row, is
// computed once per group.  Consecutive lanes take consecutive pairs of a row (contiguous
// channels), and the group's heads are independent loads in flight together.  The angle and
// its sine and cosine are taken in double: positions reach 2^20 and more, where a float angle
// would be off by a sizeable fraction of a radian.  The work is a few bytes per channel:
// HBM-bound.
#include "device_common.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeHeads = 8;

template <int DT>
__global__ void __launch_bounds__(kRopeThreads)
rope_kernel(void* __restrict__ x, int64_t rows, int64_t T, int H, int c, int d, int64_t pos0, int64_t pos_step,
            double log2_base, double sign) {
    const int half = d / 2;
    const int HG = (H + kRopeHeads - 1) / kRopeHeads;
    const int64_t f = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
    if (f >= rows * HG * half) return;
    const int p = (int)(f % half);
    const int64_t rest = f / half;
    const int hg = (int)(rest % HG);
    const int64_t row = rest / HG;
    const double pos = (double)(pos0 + (row % T) * pos_step);
    const double ang = sign * pos * exp2(-log2_base * (double)(2 * p) / (double)d);
    double sn, cs;
    sincos(ang, &sn, &cs);
    const int h0 = hg * kRopeHeads;
    float va[kRopeHeads], vb[kRopeHeads];
#pragma unroll
    for (int j = 0; j < kRopeHeads; ++j) {
        if (h0 + j >= H) break;
        const int64_t i0 = (row * H + h0 + j) * c + (c - d) + 2 * p;
        if constexpr (DT == DT_F32) {
            const float2 v = *reinterpret_cast<const float2*>(static_cast<const float*>(x) + i0);
            va[j] = v.x;
            vb[j] = v.y;
        } else {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(x) + i0);
            va[j] = bf16_to_f32(w & 0xffffu);
            vb[j] = bf16_to_f32(w >> 16);
        }
    }
#pragma unroll
    for (int j = 0; j < kRopeHeads; ++j) {
        if (h0 + j >= H) break;
        const int64_t i0 = (row * H + h0 + j) * c + (c - d) + 2 * p;
        const float ra = (float)((double)va[j] * cs - (double)vb[j] * sn);
        const float rb = (float)((double)va[j] * sn + (double)vb[j] * cs);
        if constexpr (DT == DT_F32) {
            *reinterpret_cast<float2*>(static_cast<float*>(x) + i0) = make_float2(ra, rb);
        } else {
            *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(x) + i0) =
                f32_to_bf16_rne(ra) | (f32_to_bf16_rne(rb) << 16);
        }
    }
}

}  // namespace

int launch_rope(void* x, int64_t batch, int64_t T, int H, int c, int d, int64_t pos0, int64_t pos_step, float base,
                bool inverse, int t, hipStream_t stream) {
    const int64_t threads = batch * T * ((H + kRopeHeads - 1) / kRopeHeads) * (d / 2);
    if (threads == 0) return 0;
    const int64_t grid = (threads + kRopeThreads - 1) / kRopeThreads;
    if (grid > 0x7fffffffLL) return -2;
    const double lb = log2((double)base), sg = inverse ? -1.0 : 1.0;
    if (t == DT_F32)
        hipLaunchKernelGGL(rope_kernel<DT_F32>, dim3((unsigned)grid), dim3(kRopeThreads), 0, stream, x, batch * T, T,
                           H, c, d, pos0, pos_step, lb, sg);
    else if (t == DT_BF16)
        hipLaunchKernelGGL(rope_kernel<DT_BF16>, dim3((unsigned)grid), dim3(kRopeThreads), 0, stream, x, batch * T,
                           T, H, c, d, pos0, pos_step, lb, sg);
    else
        return -2;
    return 0;
}

}  // namespace csa
