// compress.hip — softmax-weighted token compression for CSA (overlapped windows) and HCA
// (disjoint windows).
//
// Operation ("DeepSeek-V4: 迈向高效百万级上下文智能", §1.1 step 1, eq. C_i^Comp, and §1.2
// table; mlpod.com DeepSeek-V4 summary §2.3.1-§2.3.2): entry i, channel d is the softmax-
// weighted sum of the raw values over its window(s); the per-channel softmax runs over
// score = Z + position bias.  CSA: window i of stream a plus window i-1 of stream b, one
// joint softmax (entry 0: window 0 of stream a only).  HCA: window i of its single stream.
//
// Design (HBM-bound, ~1 flop per byte): each thread owns 8 consecutive channels (one
// 16-byte bf16 load or two fp32 float4 loads per token and stream), so a wave reads whole
// rows coalesced.  The softmax is computed online over chunks of 4 tokens (one rescale per
// chunk, so ~1.25 exp per element).  Long HCA windows are split across the rows of a block
// and merged through LDS so that enough loads are in flight per CU.
#include "device_common.h"
#include "launch.h"

namespace csa {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4;

struct CompressArgs {
    const void* Ca;
    const void* Za;
    const float* Ba;
    const void* Cb;   // null: no overlapped window (HCA)
    const void* Zb;
    const float* Bb;
    int64_t batch, n, N;
    int m, c;
    void* out;
    // entries first .. N-1 of each sequence are computed; entry i of sequence b goes to output
    // row b * out_ld + out_off + (i - first)
    int64_t first, out_ld, out_off;
};

template <int DTI, int DTO>
__global__ void __launch_bounds__(kThreads) compress_kernel(CompressArgs a, int G, int split, int epb) {
    __shared__ float sm[3][kThreads][8];
    const int tid = threadIdx.x;
    const int row = tid / G, g = tid - row * G;
    const int e_local = row / split, part = row - e_local * split;
    const int64_t ent = (int64_t)blockIdx.x * epb + e_local;
    const int64_t per_seq = a.N - a.first;
    const bool active = (g < G) && (row < epb * split) && (ent < a.batch * per_seq);
    const bool overlap = a.Cb != nullptr;

    float mx[8], sum[8], acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { mx[e] = -INFINITY; sum[e] = 0.f; acc[e] = 0.f; }

    int64_t b = 0, i = 0;
    if (active) {
        b = ent / per_seq;
        i = a.first + (ent - b * per_seq);
        const int m = a.m;
        const int W = overlap ? 2 * m : m;        // window positions u: [0,m) stream a, [m,2m) stream b
        const int per = (W + split - 1) / split;
        const int u0 = part * per;
        const int u1 = min(W, u0 + per);
        const int64_t seq = b * a.n;
        for (int u = u0; u < u1; u += kChunk) {
            float z[kChunk][8], cv[kChunk][8];
#pragma unroll
            for (int q = 0; q < kChunk; ++q) {
                const int uu = u + q;
                const bool is_a = uu < m;
                const bool ok = uu < u1 && (is_a || i > 0);
                if (ok) {
                    const int off = is_a ? uu : uu - m;                  // offset inside its window
                    const int64_t tok = is_a ? m * i + off : m * (i - 1) + off;
                    const int64_t el = (seq + tok) * a.c + 8 * g;
                    load8<DTI>(is_a ? a.Za : a.Zb, el, z[q]);
                    load8<DTI>(is_a ? a.Ca : a.Cb, el, cv[q]);
                    const float4* bp = reinterpret_cast<const float4*>((is_a ? a.Ba : a.Bb) + (int64_t)off * a.c + 8 * g);
                    const float4 b0 = bp[0], b1 = bp[1];
                    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) z[q][e] = (z[q][e] + bb[e]) * kLog2e;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) { z[q][e] = -INFINITY; cv[q][e] = 0.f; }
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float cm = z[0][e];
#pragma unroll
                for (int q = 1; q < kChunk; ++q) cm = fmaxf(cm, z[q][e]);
                const float nm = fmaxf(mx[e], cm);
                if (nm == -INFINITY) continue;
                const float r = exp2f(mx[e] - nm);
                float s = sum[e] * r, ac = acc[e] * r;
#pragma unroll
                for (int q = 0; q < kChunk; ++q) {
                    const float p = exp2f(z[q][e] - nm);
                    s += p;
                    ac = fmaf(p, cv[q][e], ac);
                }
                sum[e] = s;
                acc[e] = ac;
                mx[e] = nm;
            }
        }
    }

    if (split > 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { sm[0][tid][e] = mx[e]; sm[1][tid][e] = sum[e]; sm[2][tid][e] = acc[e]; }
        __syncthreads();
        if (active && part == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float M = mx[e];
                for (int p = 1; p < split; ++p) M = fmaxf(M, sm[0][tid + p * G][e]);
                float s = 0.f, ac = 0.f;
                for (int p = 0; p < split; ++p) {
                    const int t2 = tid + p * G;
                    const float r = exp2f(sm[0][t2][e] - M);
                    s = fmaf(sm[1][t2][e], r, s);
                    ac = fmaf(sm[2][t2][e], r, ac);
                }
                sum[e] = s;
                acc[e] = ac;
            }
        }
    }
    if (active && part == 0) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = acc[e] / sum[e];
        store8<DTO>(a.out, (b * a.out_ld + a.out_off + (i - a.first)) * a.c + 8 * g, o);
    }
}

template <int DTI, int DTO>
int launch(const CompressArgs& a, hipStream_t stream) {
    const int G = a.c / 8;                     // threads per entry row
    const int rows = kThreads / G;
    const int W = a.Cb ? 2 * a.m : a.m;
    int split = 1;
    // split long windows across rows (>= 8 tokens per part) to keep more loads in flight
    while (split * 2 <= rows && W / (split * 2) >= 8) split *= 2;
    const int epb = rows / split;
    const int64_t entries = a.batch * (a.N - a.first);
    const int64_t blocks = (entries + epb - 1) / epb;
    if (blocks > 0x7fffffffLL) return -2;
    hipLaunchKernelGGL((compress_kernel<DTI, DTO>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, G, split,
                       epb);
    return 0;
}

int launch_any(const CompressArgs& a, int in_t, int out_t, hipStream_t stream);

}  // namespace

int launch_compress(const void* Ca, const void* Za, const float* Ba, const void* Cb, const void* Zb, const float* Bb,
                    int64_t batch, int64_t n, int m, int c, int in_t, void* out, int out_t, hipStream_t stream) {
    CompressArgs a{Ca, Za, Ba, Cb, Zb, Bb, batch, n, n / m, m, c, out, 0, n / m, 0};
    if (a.N == 0 || batch == 0) return 0;
    return launch_any(a, in_t, out_t, stream);
}

int launch_compress_step(const void* Ca, const void* Za, const float* Ba, const void* Cb, const void* Zb,
                         const float* Bb, int64_t batch, int64_t block, int m, int c, int in_t, void* cache,
                         int64_t cache_rows, int out_t, hipStream_t stream) {
    // the state holds the raw tokens of blocks block-1 and block (only block 0 when block == 0):
    // entry `block` is the last entry of that 2m- (or m-) token sequence
    const int64_t ns = block > 0 ? 2 * (int64_t)m : m;
    CompressArgs a{Ca, Za, Ba, Cb, Zb, Bb, batch, ns, ns / m, m, c, cache, ns / m - 1, cache_rows, block};
    if (batch == 0) return 0;
    return launch_any(a, in_t, out_t, stream);
}

namespace {
int launch_any(const CompressArgs& a, int in_t, int out_t, hipStream_t stream) {
    if (in_t == DT_F32 && out_t == DT_F32) return launch<DT_F32, DT_F32>(a, stream);
    if (in_t == DT_F32 && out_t == DT_BF16) return launch<DT_F32, DT_BF16>(a, stream);
    if (in_t == DT_BF16 && out_t == DT_F32) return launch<DT_BF16, DT_F32>(a, stream);
    if (in_t == DT_BF16 && out_t == DT_BF16) return launch<DT_BF16, DT_BF16>(a, stream);
    return -2;
}
}  // namespace

}  // namespace csa
