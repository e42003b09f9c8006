// indexer.hip — lightning-indexer scores  I[t,s] = sum_h w[t,h] * ReLU(qI[t,h,:] . kI[s,:])
// for every causally visible compressed entry s ("DeepSeek-V4: 迈向高效百万级上下文智能",
// §1.1 step 2, eq. I_{t,s}; mlpod.com DeepSeek-V4 summary §2.3.1: scores only against blocks
// before the query).  fp32 accumulation, ReLU(x) = max(x, +0), no scale factor.
//
// Kernels:
//   index_scores_mfma     c_I = 128, H_I in {32, 64}, bf16 or fp8: matrix cores (below).
//   index_scores_generic  any other dtype / shape: VALU dot products, q of one query in LDS.
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


// ============================================================================ MFMA kernel
// Scores for c_I = 128 and H_I = 32 * MB heads with v_mfma_f32_32x32x16 (bf16 or fp8 e4m3).
// Heads sit on the MFMA M dimension and 32 entries on N, so one 32x32 accumulator holds 32
// heads x 32 entries and the ReLU * w head-sum runs in-lane over a lane's 16 heads plus one
// cross-lane add (lane l and l^32 hold the two halves of an entry's heads).
//
// Operand layout: lane l takes entry (or head) l%32 and the contiguous half g = l/32 of the
// 128-wide key (64 bytes fp8, 128 bytes bf16), read as 16-byte loads.  MFMA step j (K = 16)
// feeds elements [8j, 8j+8) of that half.  q and k use the same (g, j) -> channel map, so the
// dot product is over the right pairs whatever order the unit sums its K slots in.
//
// Accumulator layout (32x32, f32): lane l holds column n = l%32 and rows
// m = 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
//
// TOK = 1 (decode): the 4 waves of a workgroup take interleaved 32-entry blocks of one query.
// TOK = 4 (prefill): wave w takes query t0 + w; all four read the same key blocks (L1 hits).
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kMfmaCI = 128;

template <int DT>
struct IdxOps;

typedef int i32x8 __attribute__((ext_vector_type(8)));

template <>
struct IdxOps<DT_FP8> {
    static constexpr int kLoads = 4;      // 16-byte loads per half row (64 fp8)
    static constexpr int kEsz = 1;
    struct Frag { uint4 v[kLoads]; };
    // gfx950 v_mfma_scale_f32_32x32x64_f8f6f4 with both operands e4m3 (format 0) and unit
    // block scales (E8M0 exponent 127 = 2^0): each lane feeds 32 of its 64 bytes per step.
    static __device__ __forceinline__ f32x16 mma(const Frag& a, const Frag& b, f32x16 acc) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const i32x8 av = {(int)a.v[2 * j].x, (int)a.v[2 * j].y, (int)a.v[2 * j].z, (int)a.v[2 * j].w,
                              (int)a.v[2 * j + 1].x, (int)a.v[2 * j + 1].y, (int)a.v[2 * j + 1].z,
                              (int)a.v[2 * j + 1].w};
            const i32x8 bv = {(int)b.v[2 * j].x, (int)b.v[2 * j].y, (int)b.v[2 * j].z, (int)b.v[2 * j].w,
                              (int)b.v[2 * j + 1].x, (int)b.v[2 * j + 1].y, (int)b.v[2 * j + 1].z,
                              (int)b.v[2 * j + 1].w};
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
        }
        return acc;
    }
};

// MXFP4 (OCP MX: E2M1 values, one E8M0 scale per 32 consecutive values of a row): the same
// instruction with both operands in format 4 (E2M1, 16 bytes = 32 values per lane) and the
// block scales as its per-lane scale operands.  A lane's half row g (values 64g .. 64g+63)
// feeds 32 values to each of the two steps j, which are scale blocks 2g + j; the loader
// shifts the row's 4 scale bytes so that byte j is block 2g + j (the step selects byte j).
template <>
struct IdxOps<DT_MXFP4> {
    static constexpr int kLoads = 2;      // 16-byte loads per half row (64 E2M1 values)
    struct Frag {
        uint4 v[kLoads];
        uint32_t s;                       // the two scale bytes of this half row, bytes 0 and 1
    };
    static __device__ __forceinline__ f32x16 mma(const Frag& a, const Frag& b, f32x16 acc) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const i32x8 av = {(int)a.v[j].x, (int)a.v[j].y, (int)a.v[j].z, (int)a.v[j].w, 0, 0, 0, 0};
            const i32x8 bv = {(int)b.v[j].x, (int)b.v[j].y, (int)b.v[j].z, (int)b.v[j].w, 0, 0, 0, 0};
            acc = j == 0 ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, 0, (int)a.s, 0, (int)b.s)
                         : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 4, 4, 1, (int)a.s, 1, (int)b.s);
        }
        return acc;
    }
};

template <>
struct IdxOps<DT_BF16> {
    static constexpr int kLoads = 8;      // 16-byte loads per half row (64 bf16)
    static constexpr int kEsz = 2;
    struct Frag { uint4 v[kLoads]; };
    static __device__ __forceinline__ f32x16 mma(const Frag& a, const Frag& b, f32x16 acc) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const bf16x8 av = __builtin_bit_cast(bf16x8, a.v[i]);
            const bf16x8 bv = __builtin_bit_cast(bf16x8, b.v[i]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
        }
        return acc;
    }
};

// Half row g of `row` of a [rows_total, 128] operand (rows_total: MXFP4's scales follow the
// element bytes of all rows)
template <int DT>
__device__ __forceinline__ void load_half_row(const void* __restrict__ base, int64_t row, int g,
                                              typename IdxOps<DT>::Frag& f, int64_t rows_total) {
    using O = IdxOps<DT>;
    const uint8_t* b = static_cast<const uint8_t*>(base);
    if constexpr (DT == DT_MXFP4) {
        const uint4* p = reinterpret_cast<const uint4*>(b + row * (kMfmaCI / 2) + g * (kMfmaCI / 4));
#pragma unroll
        for (int i = 0; i < O::kLoads; ++i) f.v[i] = p[i];
        const uint32_t sw = *reinterpret_cast<const uint32_t*>(b + rows_total * (kMfmaCI / 2) + row * (kMfmaCI / 32));
        f.s = sw >> (16 * g);
    } else {
        (void)rows_total;
        const uint4* p = reinterpret_cast<const uint4*>(b + (row * kMfmaCI + g * (kMfmaCI / 2)) * O::kEsz);
#pragma unroll
        for (int i = 0; i < O::kLoads; ++i) f.v[i] = p[i];
    }
}

// Outputs of the decode-shaped kernel for the selection (each optional): per-chunk (min, max)
// of the visible scores, a per-row region to clear, and the maximum of every group of
// `group` consecutive visible scores at gmax + row * gld + s / group.
struct DecodeOut {
    float* chunk_mm;
    uint32_t* zero;
    int zero_words;
    float* gmax;
    int group;
    int64_t gld;
};

// x of the lane that the DPP control CTRL names (all rows and banks enabled)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int DT, int MB, int TOK>
__global__ void __launch_bounds__(256)
index_scores_mfma(const void* __restrict__ qI, const float* __restrict__ w, const void* __restrict__ kI, int64_t batch,
                  int64_t T, int64_t q_pos0, int64_t N, int m, float* __restrict__ scores, int64_t ld,
                  int write_invisible, int chunks, int cb, DecodeOut dec) {
    using O = IdxOps<DT>;
    constexpr int H = 32 * MB;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int g = lane >> 5, n = lane & 31;
    const int64_t groups = (T + TOK - 1) / TOK;
    // XCD-aware order: workgroups are dealt round-robin over the 8 XCDs, so unit u runs on XCD
    // u % 8; every chunk of row group bg goes to XCD bg % 8, whose L2 then holds the whole
    // score row for the selection that reads it next
    const int64_t unit = blockIdx.x;
    const int64_t slot = unit / 8;
    const int chunk = (int)(slot % chunks);
    const int64_t bg = (slot / chunks) * 8 + unit % 8;
    const int64_t b = bg / groups, tg = bg - b * groups;
    const int64_t t = TOK == 1 ? tg : tg * TOK + wid;
    if (b >= batch || t >= T) return;
    const int64_t row = b * T + t;
    const int64_t nv = visible_entries(q_pos0 + t, m, N);
    const int64_t nblk_all = (N + 31) / 32;
    if (TOK == 1 && dec.zero != nullptr && chunk == 0)   // clear the selection's per-row counters
        for (int i = threadIdx.x; i < dec.zero_words; i += 256) dec.zero[row * dec.zero_words + i] = 0u;

    // per-wave block list
    const int64_t blk0 = (int64_t)chunk * cb;
    const int64_t blk1 = min(blk0 + cb, nblk_all);
    const int first = TOK == 1 ? wid : 0;
    const int step = TOK == 1 ? 4 : 1;
    float* out = scores + row * ld;

    // q of this token (A operands) and the w of the heads this lane's accumulator rows hold
    typename O::Frag qa[MB];
    float wv[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        load_half_row<DT>(qI, row * H + 32 * mb + n, g, qa[mb], batch * T * H);
        // accumulator row r of this lane is head 8*(r/4) + 4*g + r%4: four runs of 4 heads
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 w4 = *reinterpret_cast<const float4*>(w + row * H + 32 * mb + 8 * q4 + 4 * g);
            wv[mb][4 * q4 + 0] = w4.x;
            wv[mb][4 * q4 + 1] = w4.y;
            wv[mb][4 * q4 + 2] = w4.z;
            wv[mb][4 * q4 + 3] = w4.w;
        }
    }

    const int64_t kbase = b * N;
    float smin = INFINITY, smax = -INFINITY;   // over this wave's visible scores (TOK == 1)

    // this wave's blocks: blk0 + first + i*step for i < nb_all (those inside the chunk); the
    // first nb of them hold visible entries (visibility is a prefix of the row)
    const int64_t span = blk1 - (blk0 + first);
    const int nb_all = span > 0 ? (int)((span + step - 1) / step) : 0;
    const int64_t nvis_blk = (nv + 31) / 32;   // blocks with at least one visible entry
    int nb = 0;
    if (blk0 + first < nvis_blk) nb = (int)min((int64_t)nb_all, (nvis_blk - (blk0 + first) + step - 1) / step);
    if (write_invisible && g == 0) {
        for (int i = nb; i < nb_all; ++i) {
            const int64_t s = (blk0 + first + (int64_t)i * step) * 32 + n;
            if (s < N) out[s] = -INFINITY;
        }
    }
    // three fragment buffers in a ring (the block computed + two in flight); loads are issued
    // unconditionally, clamped to this wave's last visible block, so the waits stay static
    auto load_blk = [&](typename O::Frag& f, int i) {
        const int64_t bb = blk0 + first + (int64_t)min(i, nb - 1) * step;
        load_half_row<DT>(kI, kbase + min(bb * 32 + n, N - 1), g, f, batch * N);
    };
    auto compute_blk = [&](const typename O::Frag& cur, int i) {
        const int64_t s = (blk0 + first + (int64_t)i * step) * 32 + n;
        float contrib = 0.f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x16 acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            acc = O::mma(qa[mb], cur, acc);
#pragma unroll
            for (int r = 0; r < 16; ++r) contrib = fmaf(wv[mb][r], fmaxf(acc[r], 0.f), contrib);
        }
        contrib += __shfl_xor(contrib, 32, kWave);
        if (g == 0 && s < N) {
            if (s < nv) out[s] = contrib;
            else if (write_invisible) out[s] = -INFINITY;
        }
        if (s < nv) {
            smin = fminf(smin, contrib);
            smax = fmaxf(smax, contrib);
        }
        if (TOK == 1 && dec.gmax != nullptr) {
            // maximum of each group of G consecutive visible scores (lanes n of one group)
            float v = s < nv ? contrib : -INFINITY;
            const int G = dec.group;
            if (G >= 2) v = fmaxf(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]: lane ^ 1
            if (G >= 4) v = fmaxf(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]: lane ^ 2
            if (G >= 8) v = fmaxf(v, dpp_f<0x141>(v));   // row_half_mirror: the other quad of 8
            if (G >= 16) v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror: the other half of 16
            if (G >= 32) {                               // lanes l and l ^ 16
                const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
                v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
            }
            if (g == 0 && (n & (G - 1)) == 0 && s < nv) dec.gmax[row * dec.gld + s / G] = v;
        }
    };
    if (nb > 0) {
        typename O::Frag f0, f1, f2;
        load_blk(f0, 0);
        load_blk(f1, 1);
        for (int i = 0; i < nb; i += 3) {
            load_blk(f2, i + 2);
            compute_blk(f0, i);
            if (i + 1 >= nb) break;
            load_blk(f0, i + 3);
            compute_blk(f1, i + 1);
            if (i + 2 >= nb) break;
            load_blk(f1, i + 4);
            compute_blk(f2, i + 2);
        }
    }
    if constexpr (TOK == 1) {
        if (dec.chunk_mm != nullptr) {   // (min, max) of the chunk's visible scores for the selection
            __shared__ float red[2][4];
            smin = -wave_max(-smin);
            smax = wave_max(smax);
            if (lane == 0) { red[0][wid] = smin; red[1][wid] = smax; }
            __syncthreads();
            if (threadIdx.x == 0) {
                float* o = dec.chunk_mm + (row * chunks + chunk) * 2;
                o[0] = fminf(fminf(red[0][0], red[0][1]), fminf(red[0][2], red[0][3]));
                o[1] = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
            }
        }
    }
}

// Prefill shape (many queries): a workgroup of 8 waves takes 8 consecutive queries (wave w:
// query t0 + w) and a chunk of 32-entry key blocks.  Each key block is read from global memory
// once per workgroup, coalesced (one 16-byte load per lane covers 1 KB of consecutive rows),
// three blocks ahead into registers, and written to LDS rows padded by 16 bytes, from where
// every wave reads its MFMA operand without bank conflicts (each 16-lane phase of a read then
// touches 16 distinct 4-bank groups).  The ReLU / w sum of a 32-head tile runs under the
// matrix work of the next tile.  Visibility grows with the query, so the
// group walks the blocks its last query sees and each wave masks its own tail.
constexpr int kPfWaves = 8;
constexpr int kPfPad = 16;

template <int DT, int MB>
__global__ void __launch_bounds__(kPfWaves * kWave, 1)
index_scores_prefill(const void* __restrict__ qI, const float* __restrict__ w, const void* __restrict__ kI,
                     int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int m, float* __restrict__ scores, int64_t ld,
                     int write_invisible, int chunks, int cb) {
    using O = IdxOps<DT>;
    constexpr int H = 32 * MB;
    constexpr int kRowB = kMfmaCI * O::kEsz;          // bytes per key row: 256 (bf16) / 128 (fp8)
    constexpr int kPitch = kRowB + kPfPad;
    constexpr int kLanesPerRow = kRowB / 16;
    constexpr int kRowsPerLoad = kWave / kLanesPerRow;  // rows one wave-wide 16-byte load covers
    constexpr int kLoadWaves = 32 / kRowsPerLoad;       // waves that stage a block (8 / 4)
    static_assert(kLoadWaves <= kPfWaves, "staging waves");
    __shared__ __attribute__((aligned(16))) uint8_t stg[2][32 * kPitch];
    __shared__ __attribute__((aligned(16))) uint8_t qst[kPfWaves][H * kRowB];
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, n = lane & 31;
    const int64_t groups = (T + kPfWaves - 1) / kPfWaves;
    // later query groups see more blocks: dealing the workgroups longest first (the hardware
    // hands them out in blockIdx order) keeps the triangle's short ones for the end
    const int64_t unit = (int64_t)gridDim.x - 1 - blockIdx.x;
    const int chunk = (int)(unit % chunks);
    const int64_t bg = unit / chunks;
    const int64_t b = bg / groups, tg = bg - b * groups;
    if (b >= batch) return;
    const int64_t t0 = tg * kPfWaves;
    const int64_t t = t0 + wid;
    const bool tok = t < T;
    const int64_t tq = tok ? t : T - 1;   // waves past T run on the last query and store nothing
    const int64_t row = b * T + tq;
    const int64_t nv = tok ? visible_entries(q_pos0 + t, m, N) : 0;
    const int64_t nv_last = visible_entries(q_pos0 + min(t0 + kPfWaves - 1, T - 1), m, N);
    const int64_t nblk_all = (N + 31) / 32;
    const int64_t blk0 = (int64_t)chunk * cb;
    const int64_t blk1 = min(blk0 + cb, nblk_all);
    float* out = scores + row * ld;
    const int64_t bend = min(blk1, (nv_last + 31) / 32);
    const int nb = bend > blk0 ? (int)(bend - blk0) : 0;   // the same for the whole workgroup
    auto invisible = [&]() {   // -inf where the entry is not visible to this wave's query
        if (write_invisible && tok)
            for (int64_t s = max(nv, blk0 * 32) + lane; s < min(blk1 * 32, N); s += kWave) out[s] = -INFINITY;
    };
    if (nb == 0) {
        invisible();
        return;
    }

    // this wave's q (H rows of kRowB bytes) goes through the wave's own LDS region: loaded with
    // wave-wide 16-byte loads that each cover 1 KB of consecutive bytes, then read back in the
    // MFMA operand order (after the first barrier).  Loading the operand order straight from
    // global memory makes each wave-wide load touch 64 cache lines, which the CU's address unit
    // takes one line at a time.  16-byte chunk c of row r sits at chunk position c ^ s(r), so
    // that the 16 lanes of a read phase (rows n .. n+15, one chunk) hit distinct banks.
    auto qpos = [](int r, int c) {
        return r * kRowB + ((c ^ (kRowB == 256 ? (r & 15) : ((r >> 1) & 7))) << 4);
    };
    {
        constexpr int kQLoads = H * kRowB / 1024;
        const uint8_t* qb = static_cast<const uint8_t*>(qI) + row * (int64_t)H * kRowB;
        uint4 qv[kQLoads];
#pragma unroll
        for (int r = 0; r < kQLoads; ++r) qv[r] = *reinterpret_cast<const uint4*>(qb + 1024 * r + 16 * lane);
#pragma unroll
        for (int r = 0; r < kQLoads; ++r) {
            const int o = 1024 * r + 16 * lane;
            *reinterpret_cast<uint4*>(&qst[wid][qpos(o / kRowB, (o % kRowB) >> 4)]) = qv[r];
        }
    }
    // the w of the heads this wave's accumulator rows hold
    typename O::Frag qa[MB];
    float wv[MB][16];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 w4 = *reinterpret_cast<const float4*>(w + row * H + 32 * mb + 8 * q4 + 4 * g);
            wv[mb][4 * q4 + 0] = w4.x;
            wv[mb][4 * q4 + 1] = w4.y;
            wv[mb][4 * q4 + 2] = w4.z;
            wv[mb][4 * q4 + 3] = w4.w;
        }
    }

    const bool loader = wid < kLoadWaves;
    const int srow = kRowsPerLoad * wid + lane / kLanesPerRow;   // row of the block this lane stages
    const int scol = 16 * (lane % kLanesPerRow);
    const uint8_t* kb = static_cast<const uint8_t*>(kI) + b * N * (int64_t)kRowB;
    auto gload = [&](int i) {   // block blk0 + min(i, nb-1); rows past N repeat the last row (never scored)
        const int64_t e = min((blk0 + min(i, nb - 1)) * 32 + srow, N - 1);
        return *reinterpret_cast<const uint4*>(kb + e * kRowB + scol);
    };
    // The ReLU / w head sum of each 32-head tile runs under the next tile's matrix work: with
    // 64 heads, step i issues block i's tile 0, then the sum of block i-1's tile 1 (and block
    // i-1's store), then block i's tile 1, then the sum of block i's tile 0; with 32 heads,
    // block i's tile, then block i-1's sum.  Two accumulators alternate.
    auto operand = [&](int i, typename O::Frag& kf) {   // entry n, channel half g, from buffer i & 1
        const uint8_t* st = &stg[i & 1][0] + n * kPitch + g * (kRowB / 2);
#pragma unroll
        for (int j = 0; j < O::kLoads; ++j) kf.v[j] = *reinterpret_cast<const uint4*>(st + 16 * j);
    };
    auto tile = [&](const typename O::Frag& kf, int mb, f32x16& acc) {
        acc = f32x16{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        acc = O::mma(qa[mb], kf, acc);
    };
    auto head_sum = [&](int mb, const f32x16& acc, float contrib) {
#pragma unroll
        for (int r = 0; r < 16; ++r) contrib = fmaf(wv[mb][r], fmaxf(acc[r], 0.f), contrib);
        return contrib;
    };
    auto finish = [&](int i, float contrib) {
        // lanes l and l^32 hold the two halves of entry n's heads
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(contrib), __float_as_uint(contrib), false,
                                                         false);
        contrib = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        const int64_t s = (blk0 + i) * 32 + n;
        if (g == 0 && tok && s < nv) out[s] = contrib;
    };
    // block i is computed from buffer i & 1; during step i the block i+1 goes from registers
    // to the other buffer (read by everyone in step i-1, closed by its barrier) and block i+3
    // is requested into the registers block i-1 used
    uint4 ra = {}, rb = {}, rc = {}, rd = {};
    if (loader) {
        ra = gload(0);
        rb = gload(1);
        rc = gload(2);
        *reinterpret_cast<uint4*>(&stg[0][srow * kPitch + scol]) = ra;
    }
    // the -inf stores go out after the loads: vector memory operations complete in order, so
    // stores issued first would hold up the first block's staging
    invisible();
    __syncthreads();
    // q operands: entry row 32 mb + n, channel half g (chunks g * kLoads .. g * kLoads + kLoads - 1)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < O::kLoads; ++j)
            qa[mb].v[j] = *reinterpret_cast<const uint4*>(&qst[wid][qpos(32 * mb + n, g * O::kLoads + j)]);
    f32x16 acc0, acc1;
    float part = 0.f;   // 64 heads: block i's tile-0 sum, carried into step i+1
    // x: the accumulator step i writes first; y: the one holding the previous tile
    auto step = [&](int i, const uint4& next, uint4& fetch, f32x16& x, f32x16& y) {
        if (loader) {
            fetch = gload(i + 3);
            if (i + 1 < nb) *reinterpret_cast<uint4*>(&stg[(i + 1) & 1][srow * kPitch + scol]) = next;
        }
        typename O::Frag kf;
        operand(i, kf);
        tile(kf, 0, x);
        if constexpr (MB == 2) {
            if (i > 0) finish(i - 1, head_sum(1, y, part));
            tile(kf, 1, y);
            part = head_sum(0, x, 0.f);
        } else {
            if (i > 0) finish(i - 1, head_sum(0, y, 0.f));
        }
        __syncthreads();
    };
    auto last = [&](int i, f32x16& x, f32x16& y) {   // the sums step i left
        if constexpr (MB == 2) finish(i, head_sum(1, y, part));
        else finish(i, head_sum(0, x, 0.f));
    };
    // with 64 heads tile 0 always goes to acc0; with 32, the blocks alternate
    f32x16& x1 = MB == 2 ? acc0 : acc1;
    f32x16& y1 = MB == 2 ? acc1 : acc0;
    for (int i = 0; i < nb; i += 4) {
        step(i, rb, rd, acc0, acc1);
        if (i + 1 >= nb) { last(i, acc0, acc1); break; }
        step(i + 1, rc, ra, x1, y1);
        if (i + 2 >= nb) { last(i + 1, x1, y1); break; }
        step(i + 2, rd, rb, acc0, acc1);
        if (i + 3 >= nb) { last(i + 2, acc0, acc1); break; }
        step(i + 3, ra, rc, x1, y1);
        if (i + 4 >= nb) { last(i + 3, x1, y1); break; }
    }
}

bool mfma_shape(int H_I, int c_I, int qk_t) {
    return c_I == kMfmaCI && (H_I == 32 || H_I == 64) && (qk_t == DT_FP8 || qk_t == DT_BF16 || qk_t == DT_MXFP4);
}

// Decode: 32-entry blocks per workgroup chunk (a multiple of 4, at least 4) for total_blk
// blocks over all rows.  The grid is sized to be resident at once (no partly filled second
// round): up to 32768 blocks one workgroup of 4 waves per CU, each streaming a long chunk (its
// start, the q / w loads and the first block loads, is paid once per CU); more, three per CU,
// for more loads in flight.  MXFP4 blocks are half the bytes: twice the workgroups keep as many
// bytes in flight.  (Measured at 32 rows of 32768 entries: fp8 22.7 us at one workgroup per CU
// vs 24.4 at three; MXFP4 13.7 at two vs 15.9 at one.  At 8 rows of 262144 fp8 entries: 43.7
// us at three vs 47.2 at one.)
int decode_chunk_blocks(int64_t total_blk, int qk_t) {
    const int per_cu = min(3, (total_blk <= 32768 ? 1 : 3) * (qk_t == DT_MXFP4 ? 2 : 1));
    const int64_t target = (int64_t)per_cu * 256;
    const int cb = (int)(((total_blk + target - 1) / target + 3) / 4 * 4);
    return cb < 4 ? 4 : cb;
}

template <int DT, int MB>
int launch_mfma(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0, int64_t N,
                int m, float* scores, int64_t ld, bool write_invisible, DecodeOut dec, int* n_chunk_mm,
                hipStream_t stream) {
    const int64_t nblk = (N + 31) / 32;
    if (T >= 4) {
        if constexpr (DT == DT_MXFP4) return -2;   // (decode shapes only)
        else {
        // prefill: 8 queries per workgroup share each staged key block.  Long chunks amortise
        // the workgroup's q loads (128 KB); rows are cut into chunks only as far as needed to
        // keep ~1024 workgroups (four rounds of one per CU)
        const int64_t groups = batch * ((T + kPfWaves - 1) / kPfWaves);
        const int64_t want = (1024 + groups - 1) / groups;
        int cb = (int)(((nblk + want - 1) / want + 3) / 4 * 4);
        if (cb < 4) cb = 4;
        const int chunks = (int)((nblk + cb - 1) / cb);
        const int64_t grid = groups * chunks;
        if (grid > 0x7fffffffLL) return -2;
        hipLaunchKernelGGL((index_scores_prefill<DT, MB>), dim3((unsigned)grid), dim3(kPfWaves * kWave), 0, stream, qI,
                           w, kI, batch, T, q_pos0, N, m, scores, ld, write_invisible ? 1 : 0, chunks, cb);
        if (n_chunk_mm) *n_chunk_mm = 0;
        }
    } else {
        const int cb = decode_chunk_blocks(batch * T * nblk, DT);
        const int chunks = (int)((nblk + cb - 1) / cb);
        const int64_t grid = (batch * T + 7) / 8 * 8 * chunks;   // row groups padded to whole XCD rounds
        if (grid > 0x7fffffffLL) return -2;
        hipLaunchKernelGGL((index_scores_mfma<DT, MB, 1>), dim3((unsigned)grid), dim3(256), 0, stream, qI, w, kI, batch,
                           T, q_pos0, N, m, scores, ld, write_invisible ? 1 : 0, chunks, cb, dec);
        if (n_chunk_mm) *n_chunk_mm = dec.chunk_mm ? chunks : 0;
    }
    return 0;
}

}  // namespace

// a decode chunk holds at least 4 key blocks of 32 entries
int64_t max_index_chunks(int64_t N) { return (N + 127) / 128; }

int index_chunks(int64_t batch, int64_t T, int64_t N, int H_I, int c_I, int qk_t) {
    if (!mfma_shape(H_I, c_I, qk_t) || T >= 4 || N == 0) return 0;
    const int64_t nblk = (N + 31) / 32;
    const int cb = decode_chunk_blocks(batch * T * nblk, qk_t);
    return (int)((nblk + cb - 1) / cb);
}

int launch_index_scores(const void* qI, const float* w, const void* kI, int64_t batch, int64_t T, int64_t q_pos0,
                        int64_t N, int H_I, int c_I, int m, int qk_t, float* scores, int64_t ld, bool write_invisible,
                        float* chunk_mm, int* n_chunk_mm, uint32_t* zero, int zero_words, float* gmax, int G,
                        int64_t gld, hipStream_t stream) {
    if (n_chunk_mm) *n_chunk_mm = 0;
    if (batch == 0 || T == 0 || N == 0) return 0;
    if (gmax != nullptr && (G < 1 || G > 32 || (G & (G - 1)) != 0)) return -2;
    const DecodeOut dec{chunk_mm, zero, zero_words, gmax, gmax ? G : 0, gld};
    if (mfma_shape(H_I, c_I, qk_t)) {
        if (qk_t == DT_MXFP4)
            return H_I == 64 ? launch_mfma<DT_MXFP4, 2>(qI, w, kI, batch, T, q_pos0, N, m, scores, ld, write_invisible,
                                                        dec, n_chunk_mm, stream)
                             : launch_mfma<DT_MXFP4, 1>(qI, w, kI, batch, T, q_pos0, N, m, scores, ld, write_invisible,
                                                        dec, n_chunk_mm, stream);
        if (qk_t == DT_FP8)
            return H_I == 64 ? launch_mfma<DT_FP8, 2>(qI, w, kI, batch, T, q_pos0, N, m, scores, ld, write_invisible,
                                                      dec, n_chunk_mm, stream)
                             : launch_mfma<DT_FP8, 1>(qI, w, kI, batch, T, q_pos0, N, m, scores, ld, write_invisible,
                                                      dec, n_chunk_mm, stream);
        return H_I == 64 ? launch_mfma<DT_BF16, 2>(qI, w, kI, batch, T, q_pos0, N, m, scores, ld, write_invisible,
                                                   dec, n_chunk_mm, stream)
                         : launch_mfma<DT_BF16, 1>(qI, w, kI, batch, T, q_pos0, N, m, scores, ld, write_invisible,
                                                   dec, n_chunk_mm, stream);
    }
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
