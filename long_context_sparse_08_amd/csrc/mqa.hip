// mqa.hip — shared-KV multi-query attention over compressed entries.
//
// Operation ("DeepSeek-V4: 迈向高效百万级上下文智能", §1.1 step 2 last paragraph; mlpod.com
// DeepSeek-V4 summary §2.3.2): every query head attends to one shared set of compressed
// entries, each entry serving as key and value:
//     out[t,h,:] = sum_s softmax_s(scale * q[t,h,:] . kv[s,:]) kv[s,:]
// over s in idx[t] (CSA, sparse) or over every visible HCA entry (dense, causal).
//
// mqa_generic: one wave per (query, head), lanes across channels, online softmax over the
// entries four at a time, fp32 throughout.  Works for any c % 8 == 0 up to 1024.
// mqa_sparse_mfma: bf16, c = 512, H % 64 == 0 on matrix cores (further down).
#include "device_common.h"
#include "launch.h"

#define CSA_MAX_TOPK_DEV 2048

namespace csa {

namespace {

constexpr int kGenWaves = 4;
constexpr int kKeyBatch = 4;

// Attention sink ([N] §1.3 and [M] §2.3.3 item 4: a learned per-head logit z' joins the
// softmax denominator as exp(z')): its term against the reference maximum m (log2 units) of
// a head's accumulated weights.  None without sink logits or before any entry was seen (the
// output is zero then anyway).
__device__ __forceinline__ float sink_term(const float* sink, int64_t head, float m) {
    return (sink != nullptr && m != -INFINITY) ? exp2f(sink[head] * kLog2e - m) : 0.f;
}

// Window slot j < n_win of the query at position p ([N] §1.3 and [M] §2.3.3 item 3: a
// sliding-window branch over the most recent n_win uncompressed tokens joins the compressed
// entries): the raw token at position p - n_win + 1 + j, id n_ent + its row in the window
// buffer, or -1 when that position is before 0 or outside the given raw rows.
__device__ __forceinline__ int window_key(int64_t p, const SwaArgs& w, int j, int n_ent) {
    const int64_t pw = p - w.n_win + 1 + j;
    return (pw >= 0 && pw >= w.win_pos0 && pw < w.win_pos0 + w.W) ? n_ent + (int)(pw - w.win_pos0) : -1;
}

// Key i of a sparse row's list: i < k is the selected entry idx[row, i] (its id, or -1 if
// outside [0, N)); k <= i < k + n_win is window slot i - k.
__device__ __forceinline__ int list_key(const int32_t* __restrict__ idx, int64_t row, int k, int n_ent, int64_t p,
                                        const SwaArgs& w, int i) {
    if (i < k) {
        const int s = idx[row * k + i];
        return (uint32_t)s < (uint32_t)n_ent ? s : -1;
    }
    return window_key(p, w, i - k, n_ent);
}

// Channel d of KV entry s of sequence b.  MIX: entries in the mixed storage (c - 64 e4m3 bytes,
// then 64 bf16 values; c + 64 bytes per row), decoded exactly; else dtype DT like q.
template <int DT, bool MIX>
__device__ __forceinline__ float kv_elem(const void* __restrict__ kv, int64_t b, int64_t N, int c, int64_t s, int d) {
    if constexpr (MIX) {
        const uint8_t* row = static_cast<const uint8_t*>(kv) + (b * N + s) * (int64_t)(c + 64);
        const int nf = c - 64;
        return d < nf ? e4m3_to_f32(row[d]) : bf16_to_f32(reinterpret_cast<const uint16_t*>(row + nf)[d - nf]);
    } else {
        return load1<DT>(kv, (b * N + s) * c + d);
    }
}

template <int DT, int CPL, bool DENSE, bool MIX = false>
__global__ void __launch_bounds__(kGenWaves * kWave)
mqa_generic(const void* __restrict__ q, const void* __restrict__ kv, const int32_t* __restrict__ idx, int64_t T,
            int64_t N, int H, int c, int k, float scale, int64_t q_pos0, int ratio, void* __restrict__ out,
            const float* __restrict__ sink, SwaArgs swa) {
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

    // dense: the visible entries 0 .. nvis-1, then the window slots (if any)
    const int64_t nvis = DENSE ? visible_entries(q_pos0 + t, ratio, N) : 0;
    const int64_t count = DENSE ? nvis + swa.n_win : (int64_t)k + swa.n_win;

    for (int64_t r0 = 0; r0 < count; r0 += kKeyBatch) {
        int64_t sidx[kKeyBatch];
        bool ok[kKeyBatch];
#pragma unroll
        for (int u = 0; u < kKeyBatch; ++u) {
            const int64_t r = r0 + u;
            int64_t s = -1;
            if (r < count)
                s = !DENSE ? (int64_t)list_key(idx, row, k, (int)N, swa.q_pos0 + t, swa, (int)r)
                    : r < nvis ? r
                               : (int64_t)window_key(q_pos0 + t, swa, (int)(r - nvis), (int)N);
            ok[u] = s >= 0;
            sidx[u] = ok[u] ? s : 0;
        }
        float kvv[kKeyBatch][CPL], part[kKeyBatch];
#pragma unroll
        for (int u = 0; u < kKeyBatch; ++u) {
            part[u] = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int d = lane + kWave * j;
                kvv[u][j] = !(ok[u] && d < c) ? 0.f
                            : sidx[u] < N ? kv_elem<DT, MIX>(kv, b, N, c, sidx[u], d)
                                          : load1<DT>(swa.kv, (b * swa.W + sidx[u] - N) * c + d);
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
    const float dtot = den + sink_term(sink, h, mx);
    const float rden = dtot > 0.f ? 1.f / dtot : 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int d = lane + kWave * j;
        if (d < c) store1<DT>(out, qbase + d, acc[j] * rden);
    }
}

template <int DT, bool DENSE, bool MIX = false>
int launch_generic(const void* q, const void* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N, int H, int c,
                   int k, float scale, int64_t q_pos0, int ratio, void* out, const float* sink, const SwaArgs& swa,
                   hipStream_t stream) {
    const int64_t rows = batch * T;
    if (rows > 0x7fffffffLL) return -2;
    const int cpl = (c + kWave - 1) / kWave;
    const dim3 grid((unsigned)rows, (unsigned)((H + kGenWaves - 1) / kGenWaves));
#define CSA_LAUNCH_CPL(C)                                                                                          \
    if (cpl <= C) {                                                                                                \
        hipLaunchKernelGGL((mqa_generic<DT, C, DENSE, MIX>), grid, dim3(kGenWaves * kWave), 0, stream, q, kv, idx, T, N, H, \
                           c, k, scale, q_pos0, ratio, out, sink, swa);                                            \
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


// ============================================================================ MFMA kernel
// Sparse MQA for bf16, c = 512, H % 64 == 0 (the workload shapes), on v_mfma_f32_16x16x32_bf16.
//
// Workgroup = (query row, 64 heads, one contiguous range of key slots).  Its 4 waves own 16
// heads each and walk the same 32-key blocks: the selected KV rows of a block are gathered
// straight from global memory into LDS (buffer_load_dwordx4 ... lds: one 1 KB row per
// instruction, no registers), so later blocks load while block j computes.  The buffer form,
// not global_load_lds: the compiler counts a global (flat-encoded) load to LDS as pending on
// both memory counters, and would then wait for every LDS read in flight (lgkmcnt(0)) before
// using any one of them, which defeats the operand prefetch below.
//
//   S^T = KV_blk . Q^T   M = 16 keys, N = 16 heads, K = c.  A = KV rows from LDS (16-byte
//                        reads), B = this wave's q, held in registers for the whole kernel.
//   online softmax       per head (accumulator column), exp2 domain, fp32.
//   O^T += V^T . P^T     M = 16 columns of c, N = 16 heads, K = 32 keys.  B = P straight from
//                        the S^T accumulators (bf16), A = V^T read with the gfx950 transpose
//                        LDS read (ds_read_b64_tr_b16: 4 consecutive keys of one column).
//
// K and V are the same rows (shared-KV MQA), so one staged block serves both products.  Key
// slot <-> MFMA K index: the S^T accumulator gives lane group g the keys {4g..4g+3} of each
// 16-key half; P^T uses them as K slots (g, e) = key 4g+e (e < 4) or 16+4g+(e-4), and the
// V^T operand is read with exactly that map.
//
// Accumulator layout (16x16 f32): lane l holds column n = l%16, rows 4*(l/16) + i, i = 0..3.
// With several key ranges per row (few rows, e.g. decode), each workgroup writes its partial
// normalised by its own softmax sum (bf16) with its (running max, running sum) in fp32, and
// mqa_combine merges them.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kMC = 512;                       // head dim handled by the MFMA kernel
// entries of one sequence's KV one buffer resource can address (32-bit byte offsets)
constexpr int64_t kMMaxEntries = ((int64_t(1) << 32) - 1) / (2 * kMC);
constexpr int kMHeadsWG = 64;                  // heads per workgroup
constexpr int kMBlk = 32;                      // keys per staged block
// LDS bytes per staged row: swizzled 1 KB rows (see swz) or, where the registers for the
// swizzled addresses are not available, plain rows padded by 32 bytes (a bank spread that
// leaves the plain reads of the scores with two-way conflicts)
template <bool SWZ> constexpr int kMPitch = SWZ ? kMC * 2 : kMC * 2 + 32;
template <bool SWZ> constexpr int kMBuf = kMBlk * kMPitch<SWZ>;   // bytes per staged block
constexpr int kMLoadsPerBlk = kMBlk / 4;       // rows each of the 4 waves stages per block (8)

// A staged row keeps its 16-byte chunk c (8 channels) at chunk position c ^ swz(r), r the
// row's index in its block.  The 64 banks of 4 bytes see the 16 rows a 16-lane group of
// plain reads touches (same chunk, rows 0-15) in 16 different 4-bank groups, and the 8 rows
// of a half-wave of transposing reads (two chunks each, rows 0-7 or 8-15) in 16 groups too:
// neither access pattern has a bank conflict, where an unswizzled layout (or a padded row
// pitch) gives at least one of them a two-way conflict.
__device__ __forceinline__ int swz(int r) {   // chunk swizzle of row r (0..15 per half block)
    r &= 15;
    return ((2 * r) & 15) | (r >> 3);
}

// s_waitcnt with vmcnt = n (0..63), expcnt and lgkmcnt left at their maximum (no wait)
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// two floats to bf16 (round to nearest even, v_cvt_pk_bf16_f32), a in the low half
// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// global loads (the next block's gather stays in flight).  The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt and expcnt at their maximum
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// max / sum of x over lanes l and l^32 (l^16): gfx950's lane swaps return the pair
// {x[l], x[l^32]} ({x[l], x[l^16]}) in the two results, on the VALU instead of through LDS
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// DENSE: the key list of the query at position p is 0 .. nv-1 with nv the number of HCA
// entries it may see (ratio*(s+1)-1 <= p); `k` is then unused.
//
// Workgroup = 4 waves over the workgroup's 64 heads and key range, ~80 KB of LDS, so two
// workgroups share a CU (one wave of each per SIMD).  Their barriers are independent, so the
// phases of the two drift apart and one workgroup's softmax and barrier waits overlap the
// other's matrix-core work.  The scores and their softmax are split by heads (wave w: heads
// 16w..16w+15) and the P.KV product by output columns (wave w: columns 128w..128w+127 for all
// 64 heads).  The P.KV operand is the transposed KV block, read from LDS with transposing
// reads that run at about half the rate of plain ones; split by columns, each transposed
// fragment feeds four head tiles instead of one.  The waves swap their bf16 probability
// tiles (1 KB each) and rescale factors through LDS once per block.
//
// Two staging buffers of one 32-key block each: while one block is computed the next one
// loads; the co-resident workgroup covers the rest of the gather latency.  (Launches of at
// most one workgroup per CU, such as decode, take mqa_sparse_ws below.)
constexpr int kMWaves = 4;
constexpr int kMHT = kMHeadsWG / 16;      // 16-head tiles per workgroup (4)
constexpr int kMColW = kMC / kMHT;        // output columns per wave (128)
constexpr int kMColBlkW = kMColW / 16;    // 16-column blocks per wave (8)
constexpr int kMIdsLds = 1024;            // key ids staged per workgroup (longer ranges are split)
constexpr int kMFillWGs = 256;            // workgroups a key split aims for

template <bool DENSE, bool WIN>   // WIN: the row lists hold window tokens (a second KV buffer)
__global__ void __launch_bounds__(kMWaves * kWave, 2)   // two workgroups per CU
mqa_sparse_mfma(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx,
                int64_t rows, int64_t T, int64_t N, int H, int k, int ks_count, int keys_per_split, float sl2,
                int64_t q_pos0, int ratio, uint16_t* __restrict__ out, uint16_t* __restrict__ part,
                float* __restrict__ part_ml, const float* __restrict__ sink, SwaArgs swa) {
    // one array per pipeline parity: the DMA into one and the reads of the other are then
    // provably disjoint, so no wait for the in-flight gather is forced before the current
    // block's LDS reads
    // (plain padded rows: at two workgroups per CU the registers for swizzled addresses are
    // not available)
    constexpr int kPitch = kMPitch<false>, kBuf = kMBuf<false>;
    __shared__ __attribute__((aligned(16))) uint8_t stage_a[kBuf];
    __shared__ __attribute__((aligned(16))) uint8_t stage_b[kBuf];
    __shared__ int32_t ids[DENSE ? 1 : kMIdsLds];
    __shared__ uint32_t vmask[DENSE ? 1 : kMIdsLds / 32];
    // [0]: probability tiles in the B-operand lane layout; [1][tile][head].x: rescale factor.
    // One array, so both are stored through the same lane address (no extra register).
    __shared__ uint4 xp[2][kMHT][kWave];
    __shared__ __attribute__((aligned(16))) int xflag[kMHT];   // tile rescaled in the current block
    __shared__ float xm[kMHT][16], xl[kMHT][16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int tw = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: kept in scalar registers
    const int g = lane >> 4, n16 = lane & 15;
    const int HG = H / kMHeadsWG;
    // XCD-aware order: consecutive units of a row go to one XCD (workgroups are dealt
    // round-robin over the 8 XCDs), so they share that XCD's L2 for the row's KV.  Sparse rows
    // are dealt last row first: early queries of a prefill see fewer than k entries (less
    // work), which then fills the end (the grid is a multiple of 8, so x % 8 keeps a row on
    // one XCD).
    const int64_t x = DENSE ? (int64_t)blockIdx.x : (int64_t)gridDim.x - 1 - blockIdx.x;
    const int64_t per_row = (int64_t)HG * ks_count;
    const int64_t slot = x / 8, xcd = x % 8;
    const int64_t row = (slot / per_row) * 8 + xcd;
    const int64_t rem = slot % per_row;
    const int hg = (int)(rem / ks_count), ks = (int)(rem % ks_count);
    if (row >= rows) return;
    const int64_t b = row / T;
    // dense: the visible entries 0 .. nvis-1, then (WIN) the window slots
    const int64_t nvis = DENSE ? visible_entries(q_pos0 + row % T, ratio, N) : 0;
    const int64_t klen = DENSE ? nvis + (WIN ? swa.n_win : 0) : (int64_t)k + swa.n_win;
    const int key0 = ks * keys_per_split;
    const int nkeys = (int)max((int64_t)0, min(klen, (int64_t)key0 + keys_per_split) - key0);
    const int h0 = hg * kMHeadsWG;
    const int n_ent = (int)N;   // entry ids are 32-bit (the C ABI rejects N >= 2^31)
    // dense window slot j: its id (>= n_ent), or -1
    auto dense_window = [&](int j) { return window_key(q_pos0 + row % T, swa, j, n_ent); };
    // entry gathered for slot i of this range: slots past the range and invalid ids load
    // entry 0, which the validity mask of the block keeps out of the softmax
    auto key_id = [&](int i) -> int {
        if (i >= nkeys) return 0;
        if constexpr (DENSE) {
            const int j = key0 + i;
            if (!WIN || j < nvis) return j;
            const int w = dense_window(j - (int)nvis);
            return w < 0 ? 0 : w;
        } else {
            return ids[i];
        }
    };

    // key ids first, then q: q's loads overlap the id round trip and the first gather
    constexpr int kIdsPerThread = DENSE ? 1 : kMIdsLds / (kMWaves * kWave);
    int idv[kIdsPerThread];
    if constexpr (!DENSE) {
#pragma unroll
        for (int u = 0; u < kIdsPerThread; ++u) {
            const int i = tid + u * kMWaves * kWave;
            idv[u] = i < nkeys ? list_key(idx, row, k, n_ent, swa.q_pos0 + row % T, swa, key0 + i) : -1;
        }
    }
    // this wave's q (head tile tw) as the B operand of S^T: head n16, channels 32*s + 8*g .. +8
    bf16x8_t qb[kMC / 32];
    const uint16_t* qrow = q + ((row * H) + h0 + 16 * tw + n16) * (int64_t)kMC + 8 * g;
#pragma unroll
    for (int s = 0; s < kMC / 32; ++s) qb[s] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * s);
    if constexpr (!DENSE) {
        // ids in LDS with invalid ones (negative padding, or >= N) replaced by 0, and a bit
        // per slot (word j: the 32 slots of block j) that tells the valid ones
#pragma unroll
        for (int u = 0; u < kIdsPerThread; ++u) {
            const int i = tid + u * kMWaves * kWave;
            const bool ok = i < nkeys && idv[u] >= 0;
            if (i < nkeys) ids[i] = ok ? idv[u] : 0;
            const unsigned long long bits = __ballot(ok);
            if (lane == 0) {
                const int w = (u * kMWaves * kWave + kWave * tw) / 32;
                vmask[w] = (uint32_t)bits;
                vmask[w + 1] = (uint32_t)(bits >> 32);
            }
        }
        __syncthreads();
    }

    // O^T of this wave: columns 128*tw + 16*cb + 4*g + i, head 16*ht + n16
    f32x4 acc[kMHT][kMColBlkW];
#pragma unroll
    for (int ht = 0; ht < kMHT; ++ht)
#pragma unroll
        for (int cb = 0; cb < kMColBlkW; ++cb) acc[ht][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;   // head 16*tw + n16

    int nblk = (nkeys + kMBlk - 1) / kMBlk;
    if constexpr (!DENSE) {
        // a query that sees fewer than k entries has its tail padded with -1: blocks past the
        // last valid key would leave the softmax state as it is, so the walk stops there
        while (nblk > 0 && vmask[nblk - 1] == 0u) --nblk;
        nblk = __builtin_amdgcn_readfirstlane(nblk);
    }
    const uint8_t* kvbytes = reinterpret_cast<const uint8_t*>(kv + b * N * (int64_t)kMC);
    // this sequence's KV rows (N <= kMMaxEntries, checked at launch); loads past them read 0
    const __amdgpu_buffer_rsrc_t kvres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kvbytes), (short)0, (int)(uint32_t)(N * 2 * kMC), 0x00020000);
    // the sequence's raw window rows (bf16, 1 KB each; none without a window)
    const __amdgpu_buffer_rsrc_t winres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(swa.kv != nullptr ? static_cast<const void*>(static_cast<const uint8_t*>(swa.kv) +
                                                                       b * swa.W * (int64_t)(2 * kMC))
                                            : static_cast<const void*>(kvbytes)),
        (short)0, swa.kv != nullptr ? (int)(uint32_t)(swa.W * 2 * kMC) : 0, 0x00020000);
    const uint32_t lane_off = 16u * lane;
    auto gather = [&](int blk, uint8_t* dst) {   // block `blk` of the range into `dst`
        // (the key ids one by one: at two workgroups per CU the kernel is at its register limit)
#pragma unroll
        for (int r8 = 0; r8 < kMLoadsPerBlk; ++r8) {
            const int r = kMLoadsPerBlk * tw + r8;
            // one 1 KB row per instruction: the row is wave-uniform (scalar base, lane offset)
            const int sidx = __builtin_amdgcn_readfirstlane(key_id(blk * kMBlk + r));
            const bool wr = WIN && sidx >= n_ent;   // a window row (wave-uniform)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr ? winres : kvres, (lds_void_ptr)(dst + r * kPitch), 16,
                                                     lane_off, (uint32_t)(wr ? sidx - n_ent : sidx) * (2 * kMC), 0, 0);
        }
    };
    auto compute = [&](int blk, const uint8_t* st) {
        // validity of the 32 keys of this block (bit r), shifted to this lane's key group
        uint32_t vg;
        if constexpr (DENSE && WIN) {
            // bit r: slot blk*32 + r is a visible entry or a window row (a ballot of lanes 0-31)
            const int i = blk * kMBlk + (lane & 31), j = key0 + i;
            const bool ok = i < nkeys && (j < nvis || dense_window(j - (int)nvis) >= 0);
            vg = (uint32_t)__ballot(ok) >> (4 * g);
        } else if constexpr (DENSE) {
            const int nv = nkeys - blk * kMBlk;   // >= 1
            vg = (nv >= 32 ? ~0u : (1u << nv) - 1u) >> (4 * g);
        } else {
            vg = vmask[blk] >> (4 * g);
        }

        // S^T for the two 16-key halves (two independent accumulation chains); the A operands
        // are read kSD steps ahead of their use so LDS latency overlaps the matrix work
        constexpr int kSD = DENSE ? 4 : 3;   // the sparse kernel is at its register limit
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        // chunk 4s + g of rows n16 and 16 + n16
        const uint8_t* arow = st + n16 * kPitch + 16 * g;
        auto lda = [&](int s, int h) {
            return *reinterpret_cast<const bf16x8_t*>(arow + 16 * kPitch * h + 64 * s);
        };
        bf16x8_t ra[kSD][2];
#pragma unroll
        for (int j = 0; j < kSD; ++j) {
            ra[j][0] = lda(j, 0);
            ra[j][1] = lda(j, 1);
        }
#pragma unroll
        for (int s = 0; s < kMC / 32; ++s) {
            sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[s % kSD][0], qb[s], sacc[0], 0, 0, 0);
            sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[s % kSD][1], qb[s], sacc[1], 0, 0, 0);
            if (s + kSD < kMC / 32) {
                ra[s % kSD][0] = lda(s + kSD, 0);
                ra[s % kSD][1] = lda(s + kSD, 1);
            }
        }

        // V^T operands of this wave's columns: transpose reads of keys {4g..4g+3} and
        // {16+4g..}; the first kVD column blocks are requested before the softmax
        constexpr int kVD = 3;
        // columns 128 tw + 16 cb + 4 (n16 & 3) .. +4 of rows 4g + (n16 >> 2) and 16 + that
        const int vr = 4 * g + (n16 >> 2);
        const uint8_t* vbase = st + vr * kPitch + 8 * (n16 & 3) + 2 * kMColW * tw;
        auto ldv = [&](int cb) {
            typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
            const uint8_t* va_ = vbase + 32 * cb;
            const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)va_);
            const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(va_ + 16 * kPitch));
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            const i16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            return __builtin_bit_cast(bf16x8_t, va);
        };
        bf16x8_t rv[kVD];
#pragma unroll
        for (int j = 0; j < kVD; ++j) rv[j] = ldv(j);

        // online softmax for head 16*tw + n16 (values of lane: keys 16*hb + 4g + i)
        float p[8];
        float bmax = -INFINITY;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = ((vg >> (16 * hb + i)) & 1u) ? sacc[hb][i] * sl2 : -INFINITY;
                p[4 * hb + i] = v;
                bmax = fmaxf(bmax, v);
            }
        bmax = max_xor32(max_xor16(bmax));
        // Lazy rescale: the reference max moves (and acc / l are rescaled) only when a logit
        // exceeds it by more than 2^8 in the exp2 domain; otherwise p <= 256, exact enough in
        // bf16 / fp32.  Decided for the whole wave (a lane whose max did not grow gets 1).
        const bool resc = __any(bmax > m_run + 8.f);
        if (resc) {
            const float m_new = fmaxf(m_run, bmax);
            const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);   // 0 at the first valid block
            l_run *= alpha;
            m_run = m_new;
            if (g == 0) xp[1][tw][lane].x = __float_as_uint(alpha);   // lane == n16 here
        }
        // while nothing valid has been seen m_run is -inf and every p is exp2(-inf) = 0
        const float m_ref = m_run == -INFINITY ? 0.f : m_run;
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = __builtin_amdgcn_exp2f(p[e] - m_ref);   // argument <= 8: no range reduction needed
            psum += p[e];
        }
        l_run += psum;
        uint4 pw;
        pw.x = pack_bf16x2(p[0], p[1]);
        pw.y = pack_bf16x2(p[2], p[3]);
        pw.z = pack_bf16x2(p[4], p[5]);
        pw.w = pack_bf16x2(p[6], p[7]);
        xp[0][tw][lane] = pw;
        if (lane == 0) xflag[tw] = resc ? 1 : 0;
        lds_barrier();   // the four probability tiles and rescale factors are published

        bf16x8_t pb[kMHT];
#pragma unroll
        for (int ht = 0; ht < kMHT; ++ht) pb[ht] = __builtin_bit_cast(bf16x8_t, xp[0][ht][lane]);
        const int4 fl = *reinterpret_cast<const int4*>(xflag);
        const int flags[kMHT] = {fl.x, fl.y, fl.z, fl.w};
#pragma unroll
        for (int ht = 0; ht < kMHT; ++ht) {
            if (__builtin_amdgcn_readfirstlane(flags[ht])) {
                const float a = __uint_as_float(xp[1][ht][n16].x);
#pragma unroll
                for (int cb = 0; cb < kMColBlkW; ++cb) acc[ht][cb] = acc[ht][cb] * a;
            }
        }

        // O^T += V^T P^T over this wave's columns, each V^T operand shared by the four head tiles
#pragma unroll
        for (int cb = 0; cb < kMColBlkW; ++cb) {
            const bf16x8_t vb = rv[cb % kVD];
            if (cb + kVD < kMColBlkW) rv[cb % kVD] = ldv(cb + kVD);
#pragma unroll
            for (int ht = 0; ht < kMHT; ++ht)
                acc[ht][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pb[ht], acc[ht][cb], 0, 0, 0);
        }
    };
    {
        if (nblk > 0) gather(0, stage_a);   // the loop's first wait also covers q
        for (int blk = 0; blk < nblk; blk += 2) {
            wait_vmcnt<0>();
            __syncthreads();   // block blk is staged in A; every wave is done with B
            if (blk + 1 < nblk) gather(blk + 1, stage_b);
            compute(blk, stage_a);
            if (blk + 1 >= nblk) break;
            wait_vmcnt<0>();
            __syncthreads();   // block blk+1 is staged in B; every wave is done with A
            if (blk + 2 < nblk) gather(blk + 2, stage_a);
            compute(blk + 1, stage_b);
        }
    }

    // sum of the softmax denominators over the four lane groups that share a head
    l_run = sum_xor32(sum_xor16(l_run));
    if (g == 0) {
        xm[tw][n16] = m_run;
        // a complete row's denominator takes the sink here; key-range partials leave it to the merge
        xl[tw][n16] = l_run + (part == nullptr ? sink_term(sink, h0 + 16 * tw + n16, m_run) : 0.f);
    }
    __syncthreads();   // every wave is past its last block: the staging buffers are free
    // Normalised bf16 rows go through LDS (heads 0-31 in A, 32-63 in B, one row per head) so
    // that each store below writes one head's whole 1 KB row instead of 32-byte pieces of 16.
#pragma unroll
    for (int ht = 0; ht < kMHT; ++ht) {
        const float l = xl[ht][n16];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        // columns 128 tw + 16 cb + 4g .. +4 of head row 16 (ht & 1) + n16
        const int eofs = (16 * (ht & 1) + n16) * kPitch + 256 * tw + 8 * g;
        uint8_t* sbuf = ht < 2 ? stage_a : stage_b;
#pragma unroll
        for (int cb = 0; cb < kMColBlkW; ++cb) {
            uint2 w2;
            w2.x = pack_bf16x2(acc[ht][cb][0] * inv, acc[ht][cb][1] * inv);
            w2.y = pack_bf16x2(acc[ht][cb][2] * inv, acc[ht][cb][3] * inv);
            *reinterpret_cast<uint2*>(sbuf + eofs + 32 * cb) = w2;
        }
    }
    __syncthreads();
    // the (row, 64 heads) slab of the output, or of this key range's partials
    uint16_t* dst = out + (row * H + h0) * (int64_t)kMC;
    if constexpr (!DENSE)
        if (part != nullptr) dst = part + ((row * ks_count + ks) * H + h0) * (int64_t)kMC;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int r = 8 * tw + j;
        const uint4 va = *reinterpret_cast<const uint4*>(stage_a + r * kPitch + 16 * lane);
        const uint4 vb = *reinterpret_cast<const uint4*>(stage_b + r * kPitch + 16 * lane);
        *reinterpret_cast<uint4*>(dst + (int64_t)r * kMC + 8 * lane) = va;
        *reinterpret_cast<uint4*>(dst + (int64_t)(32 + r) * kMC + 8 * lane) = vb;
    }
    if constexpr (!DENSE) {
        if (part != nullptr && g == 0) {
            const int64_t prow = (row * ks_count + ks) * H + h0 + 16 * tw + n16;
            part_ml[2 * prow] = m_run;
            part_ml[2 * prow + 1] = l_run;
        }
    }
}

// Warp-specialised sparse MQA for launches of at most one workgroup per CU (decode).  With one
// 4-wave workgroup per CU each SIMD runs a single wave, which idles the matrix core through
// every LDS wait, softmax and barrier (a phase trace gave ~3600 cycles per 32-key block for
// ~1100 cycles of MFMA issue).  Here a workgroup has 8 waves, two per SIMD, in two roles:
//   waves 0-3 (score waves, 16 heads each): gather the key blocks, S^T = KV.Q^T, the online
//     softmax, and publish block j's bf16 P tiles and rescale factors (parity j % 2)
//   waves 4-7 (value waves, 128 output columns each over the 64 heads): rescale and add
//     V^T.P^T of block j-1 while the score waves work on block j
// One workgroup barrier per block; four staging buffers hold blocks j-1 (value waves), j
// (score waves), and j+1, j+2 (loading), in swizzled 1 KB rows (see swz).
//
// MIX: KV rows in the mixed format (448 fp8 channels, then the 64 RoPE channels in bf16; 576
// bytes).  The gathers land unconverted in three raw buffers (blocks j, j+1, j+2).  A score
// wave's 8 rows fill a 5 KB region of a raw buffer: 8 x 576 bytes back to back, then 512
// bytes of padding, written by five 1 KB LDS-DMA loads in which lane i fetches the 16 bytes
// that belong at region byte 1024 j + 16 i (the padding's lanes fetch entry 0); no lane is
// masked off.  Row n keeps its 16-byte chunk c at chunk position (c + (n % 16) / 4) mod 36,
// so the 16 rows a 16-lane group reads (same chunk) fall in 16 different 4-bank groups.  A
// score wave reads 16 bytes per lane per two score steps (16 fp8 channels), converts them to
// bf16 in registers, and writes the converted channels of its quarter (128 of them) of every
// row into a swizzled 1 KB-row buffer (parity j % 2), from which the value waves take block
// j in the next step, unchanged.  For the score products the 32 channels of step s < 14 are
// 64 (s/2) + 16 g + 8 (s%2) + 0..7 for lane group g (q is loaded in the same order).
constexpr int kWsWaves = 8;
constexpr int kMixRowB = kMC + 64;       // bytes of a mixed row (36 chunks)
constexpr int kMixRegion = 5 * 1024;     // one score wave's 8 rows in a raw buffer
constexpr int kMixGathers = 5;           // LDS-DMA loads per score wave and block

// byte offset of chunk c (0..35) of row n (0..31) in a raw buffer
__device__ __forceinline__ int mix_pos(int n, int c) {
    int pc = c + ((n & 15) >> 2);
    if (pc >= 36) pc -= 36;
    return (n >> 3) * kMixRegion + (n & 7) * kMixRowB + 16 * pc;
}

// 8 fp8 e4m3 values (bytes of w0, then of w1) -> 8 bf16 (exact)
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
    const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false);
    const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true);
    const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false);
    const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <bool MIX, bool WIN>   // WIN: the row lists hold window tokens (a second KV buffer)
__global__ void __launch_bounds__(kWsWaves * kWave, 1)
mqa_sparse_ws(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kvb, const int32_t* __restrict__ idx,
              int64_t rows, int64_t T, int64_t N, int H, int k, int ks_count, int keys_per_split, float sl2,
              uint16_t* __restrict__ out, uint16_t* __restrict__ part, float* __restrict__ part_ml,
              const float* __restrict__ sink, SwaArgs swa) {
    constexpr int kPitch = kMPitch<true>, kBuf = kMBuf<true>;
    constexpr int kRawBuf = kMHT * kMixRegion;
    constexpr int kRowB = MIX ? kMixRowB : 2 * kMC;   // bytes of one KV row in memory
    // bf16: a-d are the four staging buffers; MIX: c-e hold raw gathered blocks, a-b the
    // converted blocks the value waves read
    __shared__ __attribute__((aligned(16))) uint8_t stage_a[kBuf];
    __shared__ __attribute__((aligned(16))) uint8_t stage_b[kBuf];
    __shared__ __attribute__((aligned(16))) uint8_t stage_c[MIX ? kRawBuf : kBuf];
    __shared__ __attribute__((aligned(16))) uint8_t stage_d[MIX ? kRawBuf : kBuf];
    __shared__ __attribute__((aligned(16))) uint8_t stage_e[MIX ? kRawBuf : 16];
    __shared__ int32_t ids[kMIdsLds];
    __shared__ uint32_t vmask[kMIdsLds / 32];
    __shared__ uint4 xpp[2][kMHT][kWave];     // P tiles of block j (B-operand lane layout), parity j % 2
    __shared__ float xalpha[2][kMHT][16];     // rescale factor of each head at block j
    __shared__ __attribute__((aligned(16))) int xflag[2][kMHT];   // head tile rescaled at block j
    __shared__ float xm[kMHT][16], xl[kMHT][16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool score = wid < kMHT;             // the role is wave-uniform
    const int tw = wid & (kMHT - 1);           // head tile (score) / column group (value)
    const int g = lane >> 4, n16 = lane & 15;
    const int HG = H / kMHeadsWG;
    // XCD-aware order: consecutive units of a row go to one XCD (workgroups are dealt
    // round-robin over the 8 XCDs), so they share that XCD's L2 for the row's KV.
    const int64_t x = blockIdx.x;
    const int64_t per_row = (int64_t)HG * ks_count;
    const int64_t slot = x / 8, xcd = x % 8;
    const int64_t row = (slot / per_row) * 8 + xcd;
    const int64_t rem = slot % per_row;
    const int hg = (int)(rem / ks_count), ks = (int)(rem % ks_count);
    if (row >= rows) return;
    const int64_t b = row / T;
    const int key0 = ks * keys_per_split;
    const int nkeys = (int)max((int64_t)0, min((int64_t)k + swa.n_win, (int64_t)key0 + keys_per_split) - key0);
    const int h0 = hg * kMHeadsWG;
    const int n_ent = (int)N;
    auto key_id = [&](int i) -> int { return i < nkeys ? ids[i] : 0; };

    // key ids (sanitised, with a validity bit per slot)
    constexpr int kIdsPerThread = kMIdsLds / (kWsWaves * kWave);
    int idv[kIdsPerThread];
#pragma unroll
    for (int u = 0; u < kIdsPerThread; ++u) {
        const int i = tid + u * kWsWaves * kWave;
        idv[u] = i < nkeys ? list_key(idx, row, k, n_ent, swa.q_pos0 + row % T, swa, key0 + i) : -1;
    }
#pragma unroll
    for (int u = 0; u < kIdsPerThread; ++u) {
        const int i = tid + u * kWsWaves * kWave;
        const bool ok = i < nkeys && idv[u] >= 0;
        if (i < nkeys) ids[i] = ok ? idv[u] : 0;
        const unsigned long long bits = __ballot(ok);
        if (lane == 0) {
            const int w = (u * kWsWaves * kWave + kWave * wid) / 32;
            vmask[w] = (uint32_t)bits;
            vmask[w + 1] = (uint32_t)(bits >> 32);
        }
    }
    __syncthreads();

    const int nblk = (nkeys + kMBlk - 1) / kMBlk;
    const uint8_t* kvbytes = kvb + b * N * (int64_t)kRowB;
    // this sequence's KV rows (N * kRowB < 2^32, checked at launch); loads past them read 0
    const __amdgpu_buffer_rsrc_t kvres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kvbytes), (short)0, (int)(uint32_t)(N * kRowB), 0x00020000);
    // the sequence's raw window rows (bf16, 1 KB each; none without a window)
    const __amdgpu_buffer_rsrc_t winres = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(swa.kv != nullptr ? static_cast<const void*>(static_cast<const uint8_t*>(swa.kv) +
                                                                       b * swa.W * (int64_t)(2 * kMC))
                                            : static_cast<const void*>(kvbytes)),
        (short)0, swa.kv != nullptr ? (int)(uint32_t)(swa.W * 2 * kMC) : 0, 0x00020000);

    // Each role keeps its state inside its own branch (the barriers of the two branches pair
    // up one to one), so the score waves' q and the value waves' accumulators never share
    // registers' live ranges.
    if (score) {
        float m_run = -INFINITY, l_run = 0.f;   // head 16*tw + n16
        // this wave's q (head tile tw) as the B operand of S^T: head n16, channels 32*s + 8*g .. +8
        bf16x8_t qb[kMC / 32];
        const uint16_t* qrow = q + ((row * H) + h0 + 16 * tw + n16) * (int64_t)kMC;
#pragma unroll
        for (int s = 0; s < kMC / 32; ++s) {
            const int ch = MIX && s < 14 ? 64 * (s >> 1) + 16 * g + 8 * (s & 1) : 32 * s + 8 * g;
            qb[s] = *reinterpret_cast<const bf16x8_t*>(qrow + ch);
        }
        // block `blk` into `dst`: this wave's 8 rows, ids in one LDS round trip; blocks past the
        // range load entry 0 (a gather is issued every step: one wait count fits every step)
        auto gather_ids = [&](int blk) {   // lane j: the id of this wave's row j of block blk
            return lane < kMLoadsPerBlk ? key_id(blk * kMBlk + kMLoadsPerBlk * tw + lane) : 0;
        };
        auto gather_row = [&](int myid, int r8, uint8_t* dst) {
            const int r = kMLoadsPerBlk * tw + r8;
            const int sidx = __builtin_amdgcn_readlane(myid, r8);
            const bool wr = WIN && sidx >= n_ent;   // a window row (wave-uniform)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wr ? winres : kvres, (lds_void_ptr)(dst + r * kPitch), 16,
                                                     16u * (lane ^ swz(r)), (uint32_t)(wr ? sidx - n_ent : sidx) * kRowB,
                                                     0, 0);
        };
        // MIX: load j (0..4) of this wave's region of block blk; `myid` as from gather_ids
        auto gather_mix = [&](int myid, int j, uint8_t* dst) {
            const int pbyte = 1024 * j + 16 * lane;   // byte of this wave's region
            const int r8 = pbyte / kMixRowB;          // 8: padding
            const int n = kMLoadsPerBlk * tw + (r8 < 8 ? r8 : 7);
            const int id = __builtin_amdgcn_ds_bpermute(4 * (r8 < 8 ? r8 : 7), myid);
            int c = (pbyte - kMixRowB * r8) / 16 - ((n & 15) >> 2);
            if (c < 0) c += 36;
            const uint32_t src = r8 < 8 ? (uint32_t)id * kMixRowB + 16u * c : 0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kvres, (lds_void_ptr)(dst + tw * kMixRegion + 1024 * j), 16, src,
                                                     0, 0, 0);
        };
        auto gather = [&](int blk, uint8_t* dst) {
            const int myid = gather_ids(blk);
            if constexpr (MIX) {
#pragma unroll
                for (int j = 0; j < kMixGathers; ++j) gather_mix(myid, j, dst);
            } else {
#pragma unroll
                for (int r8 = 0; r8 < kMLoadsPerBlk; ++r8) gather_row(myid, r8, dst);
            }
        };
        // gather loads per block and wave: a step waits until only the newest block's are out
        constexpr int kGathers = MIX ? kMixGathers : kMLoadsPerBlk;
        int aoff[4];
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) aoff[b4] = 16 * ((4 * b4 + g) ^ swz(n16));
        // scores, softmax and P of block blk (parity par) from `st`
        // (the gather of a later block into `nxt` is issued row by row between the matrix
        // instructions: its address work and the memory pipeline's intake then overlap them)
        static_assert(kMC / 32 == 2 * kMLoadsPerBlk, "one gathered row every second step of the scores");
        auto s_phase = [&](int blk, const uint8_t* st, int par, int gblk, uint8_t* nxt,
                           uint8_t* vdst) __attribute__((always_inline)) {
            const int gid = gather_ids(gblk);
            const uint32_t vg = vmask[blk] >> (4 * g);
            f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
          if constexpr (MIX) {
            // every operand byte of the block first: 7 fp8 pairs (chunk 4p + g) and the two bf16
            // steps (chunk 28 + 4e + g), rows n16 and n16 + 16
            uint4 rq[7][2], rb[2][2];
#pragma unroll
            for (int pp = 0; pp < 7; ++pp)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    rq[pp][h] = *reinterpret_cast<const uint4*>(st + mix_pos(n16 + 16 * h, 4 * pp + g));
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    rb[e][h] = *reinterpret_cast<const uint4*>(st + mix_pos(n16 + 16 * h, 28 + 4 * e + g));
#pragma unroll
            for (int s = 0; s < kMC / 32; ++s) {
                bf16x8_t av[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (s < 14) {
                        const uint4 r4 = rq[s >> 1][h];
                        av[h] = (s & 1) ? fp8x8_to_bf16(r4.z, r4.w) : fp8x8_to_bf16(r4.x, r4.y);
                    } else {
                        av[h] = __builtin_bit_cast(bf16x8_t, rb[s - 14][h]);
                    }
                }
                sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[0], qb[s], sacc[0], 0, 0, 0);
                sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[1], qb[s], sacc[1], 0, 0, 0);
                if ((s >> 2) == tw) {   // this wave's quarter of the channels, for the value waves
                    const int ch = s < 14 ? 8 * (s >> 1) + 2 * g + (s & 1) : 4 * s + g;   // 16-byte chunk
                    const int vo = n16 * kPitch + 256 * (ch >> 4) + 16 * ((ch & 15) ^ swz(n16));
                    *reinterpret_cast<bf16x8_t*>(vdst + vo) = av[0];
                    *reinterpret_cast<bf16x8_t*>(vdst + vo + 16 * kPitch) = av[1];
                }
                if (s % 3 == 0 && s / 3 < kMixGathers) gather_mix(gid, s / 3, nxt);   // steps 0, 3, 6, 9, 12
            }
          } else {
            constexpr int kSD = 8;
            const uint8_t* arow = st + n16 * kPitch;
            auto lda = [&](int s, int h) {
                return *reinterpret_cast<const bf16x8_t*>(arow + 16 * kPitch * h + 256 * (s >> 2) + aoff[s & 3]);
            };
            bf16x8_t ra[kSD][2];
#pragma unroll
            for (int j = 0; j < kSD; ++j) {
                ra[j][0] = lda(j, 0);
                ra[j][1] = lda(j, 1);
            }
#pragma unroll
            for (int s = 0; s < kMC / 32; ++s) {
                sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[s % kSD][0], qb[s], sacc[0], 0, 0, 0);
                sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ra[s % kSD][1], qb[s], sacc[1], 0, 0, 0);
                if (s + kSD < kMC / 32) {
                    ra[s % kSD][0] = lda(s + kSD, 0);
                    ra[s % kSD][1] = lda(s + kSD, 1);
                }
                if ((s & 1) == 0) gather_row(gid, s >> 1, nxt);
            }
          }
            // online softmax for head 16*tw + n16 (values of lane: keys 16*hb + 4g + i)
            float p[8];
            float bmax = -INFINITY;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = ((vg >> (16 * hb + i)) & 1u) ? sacc[hb][i] * sl2 : -INFINITY;
                    p[4 * hb + i] = v;
                    bmax = fmaxf(bmax, v);
                }
            bmax = max_xor32(max_xor16(bmax));
            // lazy rescale (see mqa_sparse_mfma): the reference max moves only when a logit
            // exceeds it by more than 2^8, decided for the whole wave
            const bool resc = __any(bmax > m_run + 8.f);
            if (resc) {
                const float m_new = fmaxf(m_run, bmax);
                const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
                m_run = m_new;
                if (g == 0) xalpha[par][tw][n16] = alpha;
            }
            const float m_ref = m_run == -INFINITY ? 0.f : m_run;
            float psum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = __builtin_amdgcn_exp2f(p[e] - m_ref);
                psum += p[e];
            }
            l_run += psum;
            uint4 pw;
            pw.x = pack_bf16x2(p[0], p[1]);
            pw.y = pack_bf16x2(p[2], p[3]);
            pw.z = pack_bf16x2(p[4], p[5]);
            pw.w = pack_bf16x2(p[6], p[7]);
            xpp[par][tw][lane] = pw;
            if (lane == 0) xflag[par][tw] = resc ? 1 : 0;
        };
        // the buffer block i is gathered into (bf16: four in turn; MIX: the three raw ones)
        auto gbuf = [&](int i) -> uint8_t* {
            if constexpr (MIX) {
                const int r = i % 3;
                return r == 0 ? stage_c : r == 1 ? stage_d : stage_e;
            } else {
                const int r = i & 3;
                return r == 0 ? stage_a : r == 1 ? stage_b : r == 2 ? stage_c : stage_d;
            }
        };
        // MIX: the converted copy of block i (parity i % 2)
        auto vbuf = [&](int i) -> uint8_t* { return (i & 1) ? stage_b : stage_a; };
        // blocks 0 and 1 in flight; block 0 staged before the first barrier
        gather(0, gbuf(0));
        gather(1, gbuf(1));
        wait_vmcnt<kGathers>();
        // step j < nblk: barrier j, gather block j+2 into the buffer block j-2 used (its
        // scores, then its values, are done by now), scores of block j, then wait until block
        // j+1 is staged; every step issues the same loads (no data-dependent branch inside)
        auto step = [&](int j) __attribute__((always_inline)) {
            lds_barrier();
            s_phase(j, gbuf(j), j & 1, j + 2, gbuf(j + 2), vbuf(j));
            wait_vmcnt<kGathers>();
        };
        // The first 8 blocks (all of them in decode splits) run as nested straight-line steps:
        // where control flow merges (a loop back-edge, the join after an early exit) the
        // compiler no longer knows which buffer each in-flight gather writes, and would wait
        // for every gather (the one of block j+2 too) before the next block's first read.
        // (the block numbers are constants here, so every buffer choice folds away)
        if (nblk > 0) {
            step(0);
            if (nblk > 1) {
                step(1);
                if (nblk > 2) {
                    step(2);
                    if (nblk > 3) {
                        step(3);
                        if (nblk > 4) {
                            step(4);
                            if (nblk > 5) {
                                step(5);
                                if (nblk > 6) {
                                    step(6);
                                    if (nblk > 7) {
                                        step(7);
                                        // past 8 blocks: bf16 unrolled by the four buffers; MIX
                                        // chooses its buffers at run time
                                        for (int j = 8; j < nblk; j += 4) {
                                            step(j);
                                            if (j + 1 >= nblk) break;
                                            step(j + 1);
                                            if (j + 2 >= nblk) break;
                                            step(j + 2);
                                            if (j + 3 >= nblk) break;
                                            step(j + 3);
                                        }
                                    }
                                }
                            }
                        }
                    }
                }
            }
        }
        lds_barrier();     // barrier nblk: the value waves take the last block
        wait_vmcnt<0>();   // the loads past the last block, before the buffers are reused
        l_run = sum_xor32(sum_xor16(l_run));
        if (g == 0) {
            xm[tw][n16] = m_run;
            // a complete row's denominator takes the sink here; key-range partials leave it to the merge
            xl[tw][n16] = l_run + (part == nullptr ? sink_term(sink, h0 + 16 * tw + n16, m_run) : 0.f);
            if (part != nullptr) {
                const int64_t prow = (row * ks_count + ks) * H + h0 + 16 * tw + n16;
                part_ml[2 * prow] = m_run;
                part_ml[2 * prow + 1] = l_run;
            }
        }
        __syncthreads();   // pairs with the value waves' barrier after their last block
        __syncthreads();   // pairs with the value waves' barrier after the staging
    } else {
        f32x4 acc[kMHT][kMColBlkW];   // columns 128*tw + 16*cb + 4*g + i, head 16*ht + n16
#pragma unroll
        for (int ht = 0; ht < kMHT; ++ht)
#pragma unroll
            for (int cb = 0; cb < kMColBlkW; ++cb) acc[ht][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // P.V of block blk (parity par) from `st`
        auto pv_phase = [&](const uint8_t* st, int par) {
            bf16x8_t pb[kMHT];
#pragma unroll
            for (int ht = 0; ht < kMHT; ++ht) pb[ht] = __builtin_bit_cast(bf16x8_t, xpp[par][ht][lane]);
            const int4 fl = *reinterpret_cast<const int4*>(xflag[par]);
            const int flags[kMHT] = {fl.x, fl.y, fl.z, fl.w};
#pragma unroll
            for (int ht = 0; ht < kMHT; ++ht) {
                if (__builtin_amdgcn_readfirstlane(flags[ht])) {
                    const float a = xalpha[par][ht][n16];
#pragma unroll
                    for (int cb = 0; cb < kMColBlkW; ++cb) acc[ht][cb] = acc[ht][cb] * a;
                }
            }
            constexpr int kVD = 4;
            const int vr = 4 * g + (n16 >> 2), vs = swz(vr);
            const int vofs = vr * kPitch + 256 * tw + 32 * (vs >> 1) + 16 * (((n16 & 3) >> 1) ^ (vs & 1)) + 8 * (n16 & 1);
            // the buffer's LDS address as a wave-uniform value the compiler does not fold into
            // per-buffer address registers (the value waves issue no loads into LDS, so nothing
            // needs to tell the buffers apart here)
            typedef __attribute__((address_space(3))) uint8_t lds_u8;
            uint32_t sbase = (uint32_t)(uintptr_t)(const lds_u8*)st;
            asm("" : "+s"(sbase));   // opaque: kept in a scalar register, not folded per buffer
            auto ldv = [&](int cb) {
                typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
                const uint32_t va_ = sbase + (uint32_t)(vofs ^ (32 * cb));
                const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)va_);
                const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)(va_ + 16 * kPitch));
                typedef short i16x8 __attribute__((ext_vector_type(8)));
                const i16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                return __builtin_bit_cast(bf16x8_t, va);
            };
            bf16x8_t rv[kVD];
#pragma unroll
            for (int j = 0; j < kVD; ++j) rv[j] = ldv(j);
#pragma unroll
            for (int cb = 0; cb < kMColBlkW; ++cb) {
                const bf16x8_t vb = rv[cb % kVD];
                if (cb + kVD < kMColBlkW) rv[cb % kVD] = ldv(cb + kVD);
#pragma unroll
                for (int ht = 0; ht < kMHT; ++ht)
                    acc[ht][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pb[ht], acc[ht][cb], 0, 0, 0);
            }
        };
        // barrier 0, then step j = 1..nblk: barrier j, P.V of block j-1 (buffer (j-1) % 4,
        // parity (j-1) % 2)
        lds_barrier();
        auto step = [&](int j, const uint8_t* prev) {
            lds_barrier();
            pv_phase(prev, (j - 1) & 1);
        };
        // (not unrolled: with four copies of the step and their early exits the compiler
        // copies the accumulators between steps and runs out of registers)
        for (int j = 1; j <= nblk; ++j) {
            if constexpr (MIX) {
                step(j, ((j - 1) & 1) ? stage_b : stage_a);
            } else {
                const int sl = (j - 1) & 3;
                step(j, sl == 0 ? stage_a : sl == 1 ? stage_b : sl == 2 ? stage_c : stage_d);
            }
        }
        __syncthreads();   // every block done, the (m, l) pairs published, no load in flight
        // normalised bf16 rows through LDS (heads 0-31 in A, 32-63 in B, swizzled as the
        // staged keys are); then every wave writes whole 1 KB head rows
#pragma unroll
        for (int ht = 0; ht < kMHT; ++ht) {
            const float l = xl[ht][n16];
            const float inv = l > 0.f ? 1.f / l : 0.f;
            const int sw = swz(n16);
            const int eofs = (16 * (ht & 1) + n16) * kPitch + 256 * tw + 32 * (sw >> 1) + 16 * ((g >> 1) ^ (sw & 1)) + 8 * (g & 1);
            uint8_t* sbuf = ht < 2 ? stage_a : stage_b;
#pragma unroll
            for (int cb = 0; cb < kMColBlkW; ++cb) {
                uint2 w2;
                w2.x = pack_bf16x2(acc[ht][cb][0] * inv, acc[ht][cb][1] * inv);
                w2.y = pack_bf16x2(acc[ht][cb][2] * inv, acc[ht][cb][3] * inv);
                *reinterpret_cast<uint2*>(sbuf + (eofs ^ (32 * cb))) = w2;
            }
        }
        __syncthreads();
    }
    uint16_t* dst = part != nullptr ? part + ((row * ks_count + ks) * H + h0) * (int64_t)kMC
                                    : out + (row * H + h0) * (int64_t)kMC;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int hr = 8 * wid + j;   // head row 0..63: rows 0-31 of A, then of B
        const int r = hr & 31;
        const uint8_t* sb = hr < 32 ? stage_a : stage_b;
        const int c = lane ^ swz(r);
        const uint4 v = *reinterpret_cast<const uint4*>(sb + r * kPitch + 16 * lane);
        *reinterpret_cast<uint4*>(dst + (int64_t)hr * kMC + 8 * c) = v;
    }
}

// Merge the key-range partials of one (row, head).  Partial j holds o_j = acc_j / l_j:
// out = sum_j w_j o_j / sum_j w_j with w_j = l_j 2^(m_j - M), M = max_j m_j (log2 domain).
// Ranges are taken CG at a time with every load of a group in flight together (CG = 4 for
// up to four ranges, as in decode: one round trip, no duplicate loads; else 8); a later group
// with a larger max rescales what is already summed.  One wave per (row, head), four per
// workgroup.
constexpr int kCombWaves = 4;

template <int CG>
__global__ void __launch_bounds__(kCombWaves * kWave)
mqa_combine(const uint16_t* __restrict__ part, const float* __restrict__ part_ml, int64_t rows, int H, int ks_count,
            uint16_t* __restrict__ out, const float* __restrict__ sink) {
    constexpr int kCombGroup = CG;
    // XCD-aware order (as the attention kernel's): row r on XCD r % 8, whose L2 holds the
    // row's partials; H / kCombWaves workgroups per row (H % 64 == 0 on this path)
    const int64_t per_row = H / kCombWaves, x = blockIdx.x, slot = x / 8;
    const int64_t row = (slot / per_row) * 8 + x % 8;
    const int64_t head = (slot % per_row) * kCombWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const int64_t prow0 = row * ks_count * H + head;   // partial row of range j: prow0 + j * H
    float M = -INFINITY, L = 0.f;
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < ks_count; j0 += kCombGroup) {
        uint4 pv[kCombGroup];
        float mj[kCombGroup], lj[kCombGroup];
#pragma unroll
        for (int u = 0; u < kCombGroup; ++u) {
            const bool have = j0 + u < ks_count;
            const int64_t prow = prow0 + (int64_t)min(j0 + u, ks_count - 1) * H;
            pv[u] = *reinterpret_cast<const uint4*>(part + prow * kMC + 8 * lane);
            mj[u] = have ? part_ml[2 * prow] : -INFINITY;
            lj[u] = part_ml[2 * prow + 1];
        }
        float Mg = M;
#pragma unroll
        for (int u = 0; u < kCombGroup; ++u) Mg = fmaxf(Mg, mj[u]);
        if (Mg == -INFINITY) continue;   // nothing visible so far
        const float a = M == -INFINITY ? 0.f : exp2f(M - Mg);   // rescale of the sum so far
        L *= a;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= a;
        M = Mg;
#pragma unroll
        for (int u = 0; u < kCombGroup; ++u) {
            const float w = mj[u] == -INFINITY ? 0.f : lj[u] * exp2f(mj[u] - M);
            L += w;
            const uint32_t pw[4] = {pv[u].x, pv[u].y, pv[u].z, pv[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[2 * e] = fmaf(bf16_to_f32(pw[e] & 0xffffu), w, o[2 * e]);
                o[2 * e + 1] = fmaf(bf16_to_f32(pw[e] >> 16), w, o[2 * e + 1]);
            }
        }
    }
    L += sink_term(sink, head, M);
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= inv;
    store8<DT_BF16>(out, (row * H + head) * kMC + 8 * lane, o);
}

// Key ranges per row: each range's key ids fit the LDS list; then, while the chip (two
// workgroups per CU) is not filled, halve the ranges down to 4 blocks each.
int mqa_splits(int64_t rows, int H, int k) {
    const int64_t wgs = rows * (H / kMHeadsWG);
    int ks = 1;
    while ((k + ks - 1) / ks > kMIdsLds) ks *= 2;
    while (wgs * ks < kMFillWGs && (k + ks * 2 - 1) / (ks * 2) >= 4 * kMBlk) ks *= 2;
    return ks;
}

}  // namespace

size_t sparse_mqa_workspace(int64_t batch, int64_t T, int H, int c, int k, int t) {
    if ((t != DT_BF16 && t != DT_KV_FP8_BF16) || c != kMC || H % kMHeadsWG != 0) return 0;
    const int64_t rows = batch * T;
    const int ks = mqa_splits(rows, H, k);
    if (ks == 1) return 0;
    return (size_t)rows * ks * H * (kMC * sizeof(uint16_t) + 2 * sizeof(float)) + 256;
}

int launch_sparse_mqa(const void* q, const void* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N, int H,
                      int c, int k, float scale, int t, void* out, void* ws, const float* sink, const SwaArgs& swa,
                      hipStream_t stream) {
    if (batch == 0 || T == 0) return 0;
    const int kt = k + swa.n_win;   // keys per row's list: the selected entries, then the window
    if (t == DT_KV_FP8_BF16) {
        // mixed-precision KV rows: the warp-specialised kernel for decode shapes without a
        // window, the generic kernel (bf16 q and window rows) for every other shape
        const int64_t rows = batch * T;
        if (swa.n_win > 0 || c != kMC || H % kMHeadsWG != 0 || N < 1 || N > 0xffffffffLL / (kMC + 64) ||
            k > kMIdsLds || rows * (H / kMHeadsWG) > kMFillWGs)
            return launch_generic<DT_BF16, false, true>(q, kv, idx, batch, T, N, H, c, k, scale, 0, 1, out, sink, swa,
                                                        stream);
        const int ks = mqa_splits(rows, H, k);
        const int kps = ((k + ks - 1) / ks + kMBlk - 1) / kMBlk * kMBlk;
        const int64_t units = ((rows + 7) / 8) * 8 * (H / kMHeadsWG) * ks;
        uint16_t* part = nullptr;
        float* part_ml = nullptr;
        if (ks > 1) {
            part = static_cast<uint16_t*>(ws);
            part_ml = reinterpret_cast<float*>(part + rows * ks * H * (int64_t)kMC);
        }
        hipLaunchKernelGGL((mqa_sparse_ws<true, false>), dim3((unsigned)units), dim3(kWsWaves * kWave), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(kv), idx, rows, T, N, H, k, ks,
                           kps, scale * kLog2e, static_cast<uint16_t*>(out), part, part_ml, sink, swa);
        if (ks > 1) {
            const dim3 cgrid((unsigned)((rows + 7) / 8 * 8 * (H / kCombWaves))), cblock(kCombWaves * kWave);
            if (ks <= 4)
                hipLaunchKernelGGL(mqa_combine<4>, cgrid, cblock, 0, stream, part, part_ml, rows, H, ks,
                                   static_cast<uint16_t*>(out), sink);
            else
                hipLaunchKernelGGL(mqa_combine<8>, cgrid, cblock, 0, stream, part, part_ml, rows, H, ks,
                                   static_cast<uint16_t*>(out), sink);
        }
        return 0;
    }
    if (t == DT_BF16 && c == kMC && H % kMHeadsWG == 0 && N > 0 && N <= kMMaxEntries && swa.W <= kMMaxEntries) {
        const int64_t rows = batch * T;
        const int ks = mqa_splits(rows, H, kt);
        const int kps = ((kt + ks - 1) / ks + kMBlk - 1) / kMBlk * kMBlk;
        const int64_t units = ((rows + 7) / 8) * 8 * (H / kMHeadsWG) * ks;
        if (units > 0x7fffffffLL) return -2;
        uint16_t* part = nullptr;
        float* part_ml = nullptr;
        if (ks > 1) {
            part = static_cast<uint16_t*>(ws);
            part_ml = reinterpret_cast<float*>(part + rows * ks * H * (int64_t)kMC);
        }
        const float sl2 = scale * kLog2e;
        if (units <= kMFillWGs)   // at most one workgroup per CU: two waves per SIMD in two roles
            hipLaunchKernelGGL((swa.n_win > 0 ? mqa_sparse_ws<false, true> : mqa_sparse_ws<false, false>),
                               dim3((unsigned)units), dim3(kWsWaves * kWave), 0, stream,
                               static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(kv), idx, rows, T, N, H,
                               k, ks, kps, sl2, static_cast<uint16_t*>(out), part, part_ml, sink, swa);
        else
            hipLaunchKernelGGL((swa.n_win > 0 ? mqa_sparse_mfma<false, true> : mqa_sparse_mfma<false, false>),
                               dim3((unsigned)units), dim3(kMWaves * kWave), 0, stream,
                               static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kv), idx, rows, T, N, H,
                               k, ks, kps, sl2, (int64_t)0, 1, static_cast<uint16_t*>(out), part, part_ml, sink, swa);
        if (ks > 1) {
            const dim3 cgrid((unsigned)((rows + 7) / 8 * 8 * (H / kCombWaves))), cblock(kCombWaves * kWave);
            if (ks <= 4)
                hipLaunchKernelGGL(mqa_combine<4>, cgrid, cblock, 0, stream, part, part_ml, rows, H, ks,
                                   static_cast<uint16_t*>(out), sink);
            else
                hipLaunchKernelGGL(mqa_combine<8>, cgrid, cblock, 0, stream, part, part_ml, rows, H, ks,
                                   static_cast<uint16_t*>(out), sink);
        }
        return 0;
    }
    if (t == DT_F32) return launch_generic<DT_F32, false>(q, kv, idx, batch, T, N, H, c, k, scale, 0, 1, out, sink, swa, stream);
    if (t == DT_BF16) return launch_generic<DT_BF16, false>(q, kv, idx, batch, T, N, H, c, k, scale, 0, 1, out, sink, swa, stream);
    return -2;
}

int launch_dense_mqa(const void* q, const void* kv, int64_t batch, int64_t T, int64_t q_pos0, int64_t N, int H, int c,
                     int ratio, float scale, int t, void* out, const float* sink, const SwaArgs& swa,
                     hipStream_t stream) {
    if (batch == 0 || T == 0) return 0;
    if (t == DT_BF16 && c == kMC && H % kMHeadsWG == 0 && N <= kMMaxEntries && swa.W <= kMMaxEntries) {
        // one workgroup per (query, 64 heads) walks every visible entry (and its window rows):
        // no key split, no partials (used for query chunks, which supply rows * H / 64 >= 256
        // workgroups)
        const int64_t rows = batch * T;
        const int64_t units = ((rows + 7) / 8) * 8 * (H / kMHeadsWG);
        if (units > 0x7fffffffLL) return -2;
        hipLaunchKernelGGL((swa.n_win > 0 ? mqa_sparse_mfma<true, true> : mqa_sparse_mfma<true, false>),
                           dim3((unsigned)units), dim3(kMWaves * kWave), 0, stream, static_cast<const uint16_t*>(q),
                           static_cast<const uint16_t*>(kv), nullptr, rows, T, N, H, 0, 1, 0x7fffffff, scale * kLog2e,
                           q_pos0, ratio, static_cast<uint16_t*>(out), nullptr, nullptr, sink, swa);
        return 0;
    }
    if (t == DT_KV_FP8_BF16)   // mixed-precision entries (bf16 q, output and window rows)
        return launch_generic<DT_BF16, true, true>(q, kv, nullptr, batch, T, N, H, c, 0, scale, q_pos0, ratio, out,
                                                   sink, swa, stream);
    if (t == DT_F32)
        return launch_generic<DT_F32, true>(q, kv, nullptr, batch, T, N, H, c, 0, scale, q_pos0, ratio, out, sink, swa,
                                            stream);
    if (t == DT_BF16)
        return launch_generic<DT_BF16, true>(q, kv, nullptr, batch, T, N, H, c, 0, scale, q_pos0, ratio, out, sink, swa,
                                             stream);
    return -2;
}

}  // namespace csa
