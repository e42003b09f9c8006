// rope.hip — partial rotary position embedding on the last channels of q / KV rows and its
// inverse on the attention output.
//
// Sources: "DeepSeek-V4: 迈向高效百万级上下文智能" (notes.kuangjux.top) §1.3 and the mlpod.com
// summary §2.3.3 item 2 (RoPE on the last 64 channels of queries and KV entries; the attention
// output gets the rotation of the negative query position, so it carries the query-to-entry
// distance).  The rotation itself follows RoFormer (Su et al. 2021): channel pair
// (2i, 2i+1) of the rotated part turns by position * base^(-2i/d).
//
// One wave per (row, head); lane i owns pair i (d/2 <= 64 pairs).  The angle and its sine and
// cosine are taken in double: positions reach 2^20 and more, where a float angle would be off
// by a sizeable fraction of a radian.  The work is a few bytes per channel: HBM-bound.
#include "device_common.h"
#include "launch.h"

namespace csa {
namespace {

constexpr int kRopeWaves = 4;

template <int DT>
__global__ void __launch_bounds__(kRopeWaves * kWave)
rope_kernel(void* __restrict__ x, int64_t rows, int64_t T, int H, int c, int d, int64_t pos0, int64_t pos_step,
            double log2_base, double sign) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t unit = (int64_t)blockIdx.x * kRopeWaves + (threadIdx.x >> 6);   // (row, head)
    if (unit >= rows * H || 2 * lane >= d) return;
    const int64_t row = unit / H;
    const double pos = (double)(pos0 + (row % T) * pos_step);
    const double ang = sign * pos * exp2(-log2_base * (double)(2 * lane) / (double)d);
    double sn, cs;
    sincos(ang, &sn, &cs);
    const int64_t i0 = unit * c + (c - d) + 2 * lane;
    float a, b;
    if constexpr (DT == DT_F32) {
        float* p = static_cast<float*>(x);
        a = p[i0];
        b = p[i0 + 1];
    } else {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(x) + i0);
        a = bf16_to_f32(w & 0xffffu);
        b = bf16_to_f32(w >> 16);
    }
    const float ra = (float)((double)a * cs - (double)b * sn);
    const float rb = (float)((double)a * sn + (double)b * cs);
    if constexpr (DT == DT_F32) {
        float* p = static_cast<float*>(x);
        p[i0] = ra;
        p[i0 + 1] = rb;
    } else {
        *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(x) + i0) = f32_to_bf16_rne(ra) | (f32_to_bf16_rne(rb) << 16);
    }
}

}  // namespace

int launch_rope(void* x, int64_t batch, int64_t T, int H, int c, int d, int64_t pos0, int64_t pos_step, float base,
                bool inverse, int t, hipStream_t stream) {
    const int64_t units = batch * T * H;
    if (units == 0) return 0;
    const int64_t grid = (units + kRopeWaves - 1) / kRopeWaves;
    if (grid > 0x7fffffffLL) return -2;
    const double lb = log2((double)base), sg = inverse ? -1.0 : 1.0;
    if (t == DT_F32)
        hipLaunchKernelGGL(rope_kernel<DT_F32>, dim3((unsigned)grid), dim3(kRopeWaves * kWave), 0, stream, x,
                           batch * T, T, H, c, d, pos0, pos_step, lb, sg);
    else if (t == DT_BF16)
        hipLaunchKernelGGL(rope_kernel<DT_BF16>, dim3((unsigned)grid), dim3(kRopeWaves * kWave), 0, stream, x,
                           batch * T, T, H, c, d, pos0, pos_step, lb, sg);
    else
        return -2;
    return 0;
}

}  // namespace csa
