// compress.hip — softmax-weighted token compression for CSA (overlapped windows) and HCA
// (disjoint windows).
//
// Operation ("DeepSeek-V4: 迈向高效百万级上下文智能", §1.1 step 1, eq. C_i^Comp, and §1.2
// table; mlpod.com DeepSeek-V4 summary §2.3.1-§2.3.2): entry i, channel d is the softmax-
// weighted sum of the raw values over its window(s); the per-channel softmax runs over
// score = Z + position bias.  CSA: window i of stream a plus window i-1 of stream b, one
// joint softmax (entry 0: window 0 of stream a only).  HCA: window i of its single stream.
//
// exp2 is the hardware instruction (v_exp_f32, 1 ulp): the library exp2f's extra range
// handling only changes terms below 2^-126 of the window maximum, and its instruction count cost
// ~7 % of a 1M-token compression (0.895 -> 0.837 ms) and ~1 us of a decode step's.
//
// Design (HBM-bound, ~1 flop per byte): each thread owns 8 consecutive channels (one
// 16-byte bf16 load or two fp32 float4 loads per token and stream), so a wave reads whole
// rows coalesced.  The softmax is computed online over chunks of CH tokens (one rescale per
// chunk).  The loads in flight per CU set the speed, so registers (occupancy) matter more than
// the rescale count: CSA windows (2m = 8 tokens at m = 4) take CH = 2 (94 registers, five waves
// per SIMD: 0.89 ms for a 1M-token sequence, against 0.92 ms with CH = 4 at 128 registers, 1.23
// ms with CH = 8 and 0.99 ms with CH = 1); the long HCA windows CH = 4 (~1.25 exp per element),
// split across the rows of a block and merged through LDS so that enough loads are in flight
// per CU.
#include "device_common.h"
#include "launch.h"

namespace csa {

namespace {

constexpr int kThreads = 256;

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

// PRE > 0 (CSA with m = PRE / 2, split == 1): the window's PRE positions are loaded first, in
// straight-line code with every load in flight at once (entry 0's missing b-window reads block
// 0's rows, which exist, and is masked), then the same chunked online softmax
// runs from registers: the same arithmetic in the same order as PRE == 0, so the results are
// identical bit for bit.  For launches of a few entries (a decode step), where nothing hides a
// memory round trip per position (32 entries: 5.1 us against 6.2 without the preload).
// The entries of workgroup `wg` (epb per workgroup, split threads-rows per entry); sm is the
// workgroup's merge area (used when split > 1).
template <int DTI, int DTO, int CH, int PRE>
__device__ __forceinline__ void compress_entries(const CompressArgs& a, int G, int split, int epb, int64_t wg,
                                                 float (&sm)[3][kThreads][8]) {
    const int tid = threadIdx.x;
    const int row = tid / G, g = tid - row * G;
    const int e_local = row / split, part = row - e_local * split;
    const int64_t ent = wg * epb + e_local;
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
        float zp[PRE > 0 ? PRE : 1][8], cp[PRE > 0 ? PRE : 1][8];
        if constexpr (PRE > 0) {
            // positions 0..M-1: stream a, block i; M..2M-1: stream b, block i-1 (for i == 0 the
            // rows of block 0, masked below); every address is formed without a branch
            constexpr int M = PRE / 2;
            const int64_t ra = (seq + (int64_t)M * i) * a.c + 8 * g;
            const int64_t rb = (seq + (int64_t)M * (i > 0 ? i - 1 : 0)) * a.c + 8 * g;
#pragma unroll
            for (int q = 0; q < M; ++q) {
                load8<DTI>(a.Za, ra + (int64_t)q * a.c, zp[q]);
                load8<DTI>(a.Ca, ra + (int64_t)q * a.c, cp[q]);
                load8<DTI>(a.Zb, rb + (int64_t)q * a.c, zp[M + q]);
                load8<DTI>(a.Cb, rb + (int64_t)q * a.c, cp[M + q]);
            }
            float bb[PRE][8];
#pragma unroll
            for (int q = 0; q < PRE; ++q) {
                const float4* bp = reinterpret_cast<const float4*>((q < M ? a.Ba : a.Bb) + (int64_t)(q % M) * a.c + 8 * g);
                const float4 b0 = bp[0], b1 = bp[1];
                bb[q][0] = b0.x; bb[q][1] = b0.y; bb[q][2] = b0.z; bb[q][3] = b0.w;
                bb[q][4] = b1.x; bb[q][5] = b1.y; bb[q][6] = b1.z; bb[q][7] = b1.w;
            }
            const bool okb = i > 0;
#pragma unroll
            for (int q = 0; q < PRE; ++q)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool ok = q < M || okb;
                    zp[q][e] = ok ? (zp[q][e] + bb[q][e]) * kLog2e : -INFINITY;
                    cp[q][e] = ok ? cp[q][e] : 0.f;
                }
        }
        // one chunk of the online softmax (the same arithmetic on both paths)
        auto chunk = [&](const float (&z)[CH][8], const float (&cv)[CH][8]) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float cm = z[0][e];
#pragma unroll
                for (int q = 1; q < CH; ++q) cm = fmaxf(cm, z[q][e]);
                const float nm = fmaxf(mx[e], cm);
                if (nm == -INFINITY) continue;
                const float r = __builtin_amdgcn_exp2f(mx[e] - nm);
                float s = sum[e] * r, ac = acc[e] * r;
#pragma unroll
                for (int q = 0; q < CH; ++q) {
                    const float p = __builtin_amdgcn_exp2f(z[q][e] - nm);
                    s += p;
                    ac = fmaf(p, cv[q][e], ac);
                }
                sum[e] = s;
                acc[e] = ac;
                mx[e] = nm;
            }
        };
        if constexpr (PRE > 0) {
#pragma unroll
            for (int u = 0; u < PRE; u += CH) {
                float z[CH][8], cv[CH][8];
#pragma unroll
                for (int q = 0; q < CH; ++q)
#pragma unroll
                    for (int e = 0; e < 8; ++e) { z[q][e] = zp[u + q][e]; cv[q][e] = cp[u + q][e]; }
                chunk(z, cv);
            }
        } else {
            for (int u = u0; u < u1; u += CH) {
                float z[CH][8], cv[CH][8];
#pragma unroll
                for (int q = 0; q < CH; ++q) {
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
                chunk(z, cv);
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
                    const float r = __builtin_amdgcn_exp2f(sm[0][t2][e] - M);
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

template <int DTI, int DTO, int CH, int PRE>
__global__ void __launch_bounds__(kThreads) compress_kernel(CompressArgs a, int G, int split, int epb) {
    __shared__ float sm[3][kThreads][8];
    compress_entries<DTI, DTO, CH, PRE>(a, G, split, epb, blockIdx.x, sm);
}

// Two decode-step compressions of m = 4 in one launch (a CSA layer's KV entry and index-key
// entry): workgroups 0 .. wgs0-1 compute a0's entries, the rest a1's, each as the one-wave
// decode-step launch of compress_kernel would (the same arithmetic, so the same bits).
template <int DTI, int DTO0, int DTO1>
__global__ void __launch_bounds__(kThreads) compress_pair_kernel(CompressArgs a0, int G0, int epw0, int64_t wgs0,
                                                                 CompressArgs a1, int G1, int epw1) {
    __shared__ float sm[3][kThreads][8];
    if ((int64_t)blockIdx.x < wgs0) compress_entries<DTI, DTO0, 2, 8>(a0, G0, 1, epw0, blockIdx.x, sm);
    else compress_entries<DTI, DTO1, 2, 8>(a1, G1, 1, epw1, blockIdx.x - wgs0, sm);
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
    if (split == 1 && a.Cb != nullptr && a.m == 4 && entries < 2048) {
        // a few CSA entries (a decode step): one-wave workgroups (whole entries each) spread the
        // loads over as many CUs as possible (32 entries of c = 512: 32 CUs instead of 8)
        const int nt = (G + kWave - 1) / kWave * kWave;
        const int epw = nt / G;
        hipLaunchKernelGGL((compress_kernel<DTI, DTO, 2, 8>), dim3((unsigned)((entries + epw - 1) / epw)), dim3(nt), 0,
                           stream, a, G, 1, epw);
    } else if (split == 1 && W <= 8)   // short (CSA) windows
        hipLaunchKernelGGL((compress_kernel<DTI, DTO, 2, 0>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a,
                           G, split, epb);
    else
        hipLaunchKernelGGL((compress_kernel<DTI, DTO, 4, 0>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, a,
                           G, split, epb);
    return 0;
}

int launch_any(const CompressArgs& a, int in_t, int out_t, hipStream_t stream);

// the arguments of a decode step: the state holds the raw tokens of blocks block-1 and block
// (only block 0 when block == 0), so entry `block` is the last entry of that 2m- (or m-) token
// sequence
CompressArgs step_args(const void* Ca, const void* Za, const float* Ba, const void* Cb, const void* Zb,
                       const float* Bb, int64_t batch, int64_t block, int m, int c, void* cache, int64_t cache_rows) {
    const int64_t ns = block > 0 ? 2 * (int64_t)m : m;
    return CompressArgs{Ca, Za, Ba, Cb, Zb, Bb, batch, ns, ns / m, m, c, cache, ns / m - 1, cache_rows, block};
}

template <int DTI, int DTO0, int DTO1>
int launch_pair(const CompressArgs& a0, const CompressArgs& a1, hipStream_t stream) {
    const int G0 = a0.c / 8, G1 = a1.c / 8;
    const int nt = max((G0 + kWave - 1) / kWave, (G1 + kWave - 1) / kWave) * kWave;   // <= kThreads
    const int epw0 = nt / G0, epw1 = nt / G1;
    const int64_t w0 = (a0.batch * (a0.N - a0.first) + epw0 - 1) / epw0;
    const int64_t w1 = (a1.batch * (a1.N - a1.first) + epw1 - 1) / epw1;
    if (w0 + w1 > 0x7fffffffLL) return -2;
    hipLaunchKernelGGL((compress_pair_kernel<DTI, DTO0, DTO1>), dim3((unsigned)(w0 + w1)), dim3(nt), 0, stream, a0, G0,
                       epw0, w0, a1, G1, epw1);
    return 0;
}

template <int DTI, int DTO0>
int launch_pair_out1(const CompressArgs& a0, const CompressArgs& a1, int out1, hipStream_t stream) {
    if (out1 == DT_F32) return launch_pair<DTI, DTO0, DT_F32>(a0, a1, stream);
    if (out1 == DT_BF16) return launch_pair<DTI, DTO0, DT_BF16>(a0, a1, stream);
    if (out1 == DT_FP8) return launch_pair<DTI, DTO0, DT_FP8>(a0, a1, stream);
    return -2;
}

template <int DTI>
int launch_pair_out0(const CompressArgs& a0, const CompressArgs& a1, int out0, int out1, hipStream_t stream) {
    if (out0 == DT_F32) return launch_pair_out1<DTI, DT_F32>(a0, a1, out1, stream);
    if (out0 == DT_BF16) return launch_pair_out1<DTI, DT_BF16>(a0, a1, out1, stream);
    if (out0 == DT_FP8) return launch_pair_out1<DTI, DT_FP8>(a0, a1, out1, stream);
    return -2;
}

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
    if (batch == 0) return 0;
    return launch_any(step_args(Ca, Za, Ba, Cb, Zb, Bb, batch, block, m, c, cache, cache_rows), in_t, out_t, stream);
}

int launch_compress_step_pair(const StepStreams& s0, const StepStreams& s1, int64_t batch, int64_t block, int m,
                              int in_t, hipStream_t stream) {
    if (batch == 0) return 0;
    const CompressArgs a0 = step_args(s0.Ca, s0.Za, s0.Ba, s0.Cb, s0.Zb, s0.Bb, batch, block, m, s0.c, s0.cache,
                                      s0.cache_rows);
    const CompressArgs a1 = step_args(s1.Ca, s1.Za, s1.Ba, s1.Cb, s1.Zb, s1.Bb, batch, block, m, s1.c, s1.cache,
                                      s1.cache_rows);
    if (m != 4) {   // (the one-launch kernel is the m = 4 window kernel)
        const int r = launch_any(a0, in_t, s0.out_t, stream);
        return r != 0 ? r : launch_any(a1, in_t, s1.out_t, stream);
    }
    if (in_t == DT_F32) return launch_pair_out0<DT_F32>(a0, a1, s0.out_t, s1.out_t, stream);
    if (in_t == DT_BF16) return launch_pair_out0<DT_BF16>(a0, a1, s0.out_t, s1.out_t, stream);
    return -2;
}

int launch_hca_compress_step(const void* C, const void* Z, const float* B, int64_t batch, int64_t block, int m_prime,
                             int c, int in_t, void* cache, int64_t cache_rows, int out_t, hipStream_t stream) {
    // the state is the m' raw tokens of block `block`: entry `block` is its only entry
    CompressArgs a{C, Z, B, nullptr, nullptr, nullptr, batch, m_prime, 1, m_prime, c, cache, 0, cache_rows, block};
    if (batch == 0) return 0;
    return launch_any(a, in_t, out_t, stream);
}

namespace {
int launch_any(const CompressArgs& a, int in_t, int out_t, hipStream_t stream) {
    if (in_t == DT_F32 && out_t == DT_F32) return launch<DT_F32, DT_F32>(a, stream);
    if (in_t == DT_F32 && out_t == DT_BF16) return launch<DT_F32, DT_BF16>(a, stream);
    if (in_t == DT_BF16 && out_t == DT_F32) return launch<DT_BF16, DT_F32>(a, stream);
    if (in_t == DT_BF16 && out_t == DT_BF16) return launch<DT_BF16, DT_BF16>(a, stream);
    if (in_t == DT_F32 && out_t == DT_FP8) return launch<DT_F32, DT_FP8>(a, stream);
    if (in_t == DT_BF16 && out_t == DT_FP8) return launch<DT_BF16, DT_FP8>(a, stream);
    return -2;
}
}  // namespace

}  // namespace csa
