/*
 * csa_oracle.c — CPU oracle for the CSA / HCA attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Plain, slow, double-precision loops that state what the
 * path computes, so that the GPU kernels can be checked against them.  Only the tests,
 * the smoke check and the benchmark's CPU-baseline leg may load this library; the
 * product path never calls it.  It shares no source with the HIP kernels.
 *
 * Sources (web pages on the DeepSeek-V4 report):
 *   [N]  "DeepSeek-V4: 迈向高效百万级上下文智能", notes.kuangjux.top:
 *        §1.1 step 1 (token-level compression, eq. C_i^Comp), §1.1 step 2 (lightning
 *        indexer, eq. I_{t,s}; top-k; shared-KV MQA), §1.2 (HCA comparison table).
 *   [M]  mlpod.com summary of "DeepSeek-V4: Towards Highly Efficient Million-Token
 *        Context Intelligence": §2.3.1 (CSA compression with softmax normalisation and
 *        Hadamard product; index keys made by the same compression; indexer scores only
 *        against earlier blocks; top-k), §2.3.2 (HCA: larger ratio, no selection, dense
 *        attention; shared-KV MQA).
 *
 * Readings where the pages leave a step open (each one is listed with its reason in the
 * design notes):
 *   R1  the compression weights S^a, S^b come from ONE softmax per channel taken jointly
 *       over the 2m scores of window i (stream a) and window i-1 (stream b);
 *   R2  the learned position bias is a [m, c] table indexed by offset inside the window;
 *   R3  block 0 has no previous window: its b-terms are absent (not zero-padded);
 *   R4  n not a multiple of the ratio: floor(n/ratio) entries, the tail is left alone;
 *   R5  causal visibility: entry s is usable by the query at absolute position p iff
 *       ratio*(s+1)-1 <= p;
 *   R6  ReLU(x) = x if x > 0 else +0.0; the indexer has no scale factor;
 *   R7  top-k keeps the min(k, |visible|) best entries by (score desc, index asc), emits
 *       them in ascending index order and pads with -1 (scores of pads: -inf);
 *   R8  MQA logits are scale * q.kv with the scale given by the caller (1/sqrt(c) in the
 *       workloads); every compressed entry is both key and value; with nothing selected
 *       the output is 0.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared, no fast-math.  OpenMP only splits independent
 * output rows across threads; the arithmetic inside a row is sequential.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8_E4M3 = 2 };

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ storage formats */

/* bf16: the upper 16 bits of an IEEE binary32. */
static double decode_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities,
 * S.1111.111 is NaN; subnormals are mant * 2^-9. */
static double decode_e4m3(uint8_t b) {
    int sign = b >> 7, e = (b >> 3) & 15, mant = b & 7;
    double v;
    if (e == 15 && mant == 7) return NAN;
    if (e == 0) v = ldexp((double)mant, -9);
    else v = ldexp((double)(8 + mant), e - 10);
    return sign ? -v : v;
}

/* MXFP4 ([N] §2.4: the indexer's QK path runs in MXFP4; format: OCP Microscaling Formats
 * v1.0 — blocks of 32 elements, E2M1 elements, one E8M0 scale per block).
 * E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal
 * (mant * 2^-1), otherwise (1 + mant/2) * 2^(e-1).  E8M0: 2^(s-127), s = 255 is NaN. */
static double decode_e2m1(unsigned nib) {
    unsigned e = (nib >> 1) & 3u, mant = nib & 1u;
    double v = e == 0 ? 0.5 * mant : ldexp(1.0 + 0.5 * mant, (int)e - 1);
    return (nib & 8u) ? -v : v;
}

/* Storage of `rows` rows of c values: rows * c/2 element bytes (value 2i in the low nibble
 * of byte i of its row, 2i+1 in the high nibble), then rows * c/32 scale bytes. */
int oracle_decode_mxfp4(const uint8_t* buf, int64_t rows, int c, double* dst) {
    int64_t r;
    int j;
    if (c % 32 != 0) return -1;
    for (r = 0; r < rows; ++r) {
        const uint8_t* el = buf + r * (c / 2);
        const uint8_t* sc = buf + rows * (c / 2) + r * (c / 32);
        for (j = 0; j < c; ++j) {
            unsigned byte = el[j / 2];
            unsigned nib = (j % 2 == 0) ? (byte & 15u) : (byte >> 4);
            unsigned s = sc[j / 32];
            dst[r * c + j] = s == 255u ? NAN : decode_e2m1(nib) * ldexp(1.0, (int)s - 127);
        }
    }
    return 0;
}

/* Mixed-precision KV rows ([N] §1.3 and [M] §2.3.4: the RoPE dimensions of a KV entry are
 * kept in bf16, the others in fp8; [N] §1.3 and [M] §2.3.3 item 2: RoPE covers the last 64
 * dimensions).  A row of c values is c - 64 OCP e4m3fn bytes (dimensions 0 .. c-65), then
 * 64 bf16 values (dimensions c-64 .. c-1, little-endian): c + 64 bytes in all. */
int oracle_decode_kv_fp8_bf16(const uint8_t* buf, int64_t rows, int c, double* dst) {
    int64_t r;
    int j;
    if (c < 64) return -1;
    for (r = 0; r < rows; ++r) {
        const uint8_t* row = buf + r * (int64_t)(c + 64);
        for (j = 0; j < c - 64; ++j) dst[r * c + j] = decode_e4m3(row[j]);
        for (j = 0; j < 64; ++j) {
            const uint8_t* p = row + (c - 64) + 2 * j;
            dst[r * c + (c - 64) + j] = decode_bf16((uint16_t)(p[0] | (p[1] << 8)));
        }
    }
    return 0;
}

/* Partial RoPE ([N] §1.3 and [M] §2.3.3 item 2: the last d channels of q and KV rows; the
 * attention output turns by the negative query position).  Rotation as defined by RoFormer
 * (Su et al. 2021): channel pair (c-d+2i, c-d+2i+1) of the row at position p turns by
 * p * base^(-2i/d); `inverse` negates the angle.  In place on x [batch, T, H, c]; row (b, t)
 * sits at position pos0 + t * pos_step. */
void oracle_rope(double* x, int64_t batch, int64_t T, int H, int c, int d, int64_t pos0, int64_t pos_step,
                 double base, int inverse) {
    int64_t r;
    for (r = 0; r < batch * T * H; ++r) {
        const double p = (double)(pos0 + ((r / H) % T) * pos_step);
        int i;
        for (i = 0; i < d / 2; ++i) {
            double* v = x + r * c + (c - d) + 2 * i;
            const double a = (inverse ? -p : p) * pow(base, -2.0 * i / d);
            const double x0 = v[0], x1 = v[1];
            v[0] = x0 * cos(a) - x1 * sin(a);
            v[1] = x0 * sin(a) + x1 * cos(a);
        }
    }
}

/* Decode `count` stored values of type `dtype` into doubles (exact). */
int oracle_decode(const void* src, int dtype, int64_t count, double* dst) {
    int64_t i;
    if (dtype == OR_F32) {
        const float* s = (const float*)src;
        for (i = 0; i < count; ++i) dst[i] = (double)s[i];
    } else if (dtype == OR_BF16) {
        const uint16_t* s = (const uint16_t*)src;
        for (i = 0; i < count; ++i) dst[i] = decode_bf16(s[i]);
    } else if (dtype == OR_FP8_E4M3) {
        const uint8_t* s = (const uint8_t*)src;
        for (i = 0; i < count; ++i) dst[i] = decode_e4m3(s[i]);
    } else {
        return -1;
    }
    return 0;
}

/* Round a double to the nearest bf16 value, ties to even (the quantum of the 8-bit
 * significand, or 2^-133 below the normal range). */
static double round_bf16(double x) {
    int e;
    double q;
    if (x == 0.0 || !isfinite(x)) return x;
    frexp(x, &e);                 /* x = f * 2^e, 0.5 <= |f| < 1 */
    q = ldexp(1.0, (e - 8 > -133) ? e - 8 : -133);
    return nearbyint(x / q) * q;  /* default rounding mode: to nearest, ties to even */
}

/* Round a finite double to the nearest OCP e4m3fn value, ties to even, saturating at +-448:
 * the grid's quantum at |x| is 2^(floor(log2|x|) - 3) for normal values (exponent >= -6) and
 * 2^-9 for subnormals (R12: unit scale). */
static double round_e4m3(double x) {
    int e;
    double a = fabs(x), q;
    if (a == 0.0 || !isfinite(x)) return x;
    if (a > 448.0) a = 448.0;
    frexp(a, &e);                 /* a = f * 2^e, 0.5 <= f < 1: floor(log2 a) = e - 1 */
    q = ldexp(1.0, ((e - 1 > -6) ? e - 1 : -6) - 3);
    return copysign(nearbyint(a / q) * q, x);
}

static double round_to(double x, int dtype) {
    if (dtype == OR_F32) return (double)(float)x;
    if (dtype == OR_BF16) return round_bf16(x);
    if (dtype == OR_FP8_E4M3) return round_e4m3(x);
    return x;                     /* -1: keep double */
}

/* Round `count` doubles in place to storage type `dtype` (values stay doubles). */
int oracle_round(double* x, int dtype, int64_t count) {
    int64_t i;
    if (dtype != OR_F32 && dtype != OR_BF16 && dtype != OR_FP8_E4M3) return -1;
    for (i = 0; i < count; ++i) x[i] = round_to(x[i], dtype);
    return 0;
}

/* ------------------------------------------------------------------ compression */

/*
 * CSA compression ([N] §1.1 step 1, eq. C_i^Comp; [M] §2.3.1):
 *   C_i^Comp = sum_{j=mi}^{m(i+1)-1} S^a_j (.) C^a_j + sum_{j=m(i-1)}^{mi-1} S^b_j (.) C^b_j
 * with, per channel d (R1, R2), the weights
 *   S^a_j = exp(Za[j]+Ba[j-mi]) / D,  S^b_j = exp(Zb[j]+Bb[j-m(i-1)]) / D,
 *   D = sum over both windows of exp(score).
 * Block 0 has no b window (R3).  Max-subtraction only guards exp against overflow.
 * Layouts: C*, Z* [batch, n, c]; B* [m, c]; out [batch, n/m, c].
 */
void oracle_csa_compress(const double* Ca, const double* Cb, const double* Za, const double* Zb,
                         const double* Ba, const double* Bb, int64_t batch, int64_t n, int m, int c,
                         int out_dtype, double* out) {
    int64_t N = n / m;
    int64_t bi;
#pragma omp parallel for schedule(dynamic, 16)
    for (bi = 0; bi < batch * N; ++bi) {
        int64_t b = bi / N, i = bi % N;
        const int64_t base = b * n * c;
        int d;
        for (d = 0; d < c; ++d) {
            double mu = -INFINITY, num = 0.0, den = 0.0;
            int64_t j;
            for (j = m * i; j < m * (i + 1); ++j) {
                double s = Za[base + j * c + d] + Ba[(j - m * i) * c + d];
                if (s > mu) mu = s;
            }
            if (i >= 1) {
                for (j = m * (i - 1); j < m * i; ++j) {
                    double s = Zb[base + j * c + d] + Bb[(j - m * (i - 1)) * c + d];
                    if (s > mu) mu = s;
                }
            }
            for (j = m * i; j < m * (i + 1); ++j) {
                double e = exp(Za[base + j * c + d] + Ba[(j - m * i) * c + d] - mu);
                num += e * Ca[base + j * c + d];
                den += e;
            }
            if (i >= 1) {
                for (j = m * (i - 1); j < m * i; ++j) {
                    double e = exp(Zb[base + j * c + d] + Bb[(j - m * (i - 1)) * c + d] - mu);
                    num += e * Cb[base + j * c + d];
                    den += e;
                }
            }
            out[(b * N + i) * c + d] = round_to(num / den, out_dtype);
        }
    }
}

/*
 * HCA compression ([N] §1.2 table: ratio m' = 128, no overlap; [M] §2.3.2): entry i is
 * the softmax-weighted sum of the m' tokens of window i alone:
 *   out[i,d] = sum_{j=m'i}^{m'(i+1)-1} exp(Z[j,d]+B[j-m'i,d]) C[j,d] / sum exp(...).
 * Layouts: C, Z [batch, n, c]; B [m', c]; out [batch, n/m', c].
 */
void oracle_hca_compress(const double* C, const double* Z, const double* B, int64_t batch, int64_t n,
                         int mp, int c, int out_dtype, double* out) {
    int64_t N = n / mp;
    int64_t bi;
#pragma omp parallel for schedule(dynamic, 4)
    for (bi = 0; bi < batch * N; ++bi) {
        int64_t b = bi / N, i = bi % N;
        const int64_t base = b * n * c;
        int d;
        for (d = 0; d < c; ++d) {
            double mu = -INFINITY, num = 0.0, den = 0.0;
            int64_t j;
            for (j = mp * i; j < mp * (i + 1); ++j) {
                double s = Z[base + j * c + d] + B[(j - mp * i) * c + d];
                if (s > mu) mu = s;
            }
            for (j = mp * i; j < mp * (i + 1); ++j) {
                double e = exp(Z[base + j * c + d] + B[(j - mp * i) * c + d] - mu);
                num += e * C[base + j * c + d];
                den += e;
            }
            out[(b * N + i) * c + d] = round_to(num / den, out_dtype);
        }
    }
}

/* ------------------------------------------------------------------ indexer */

static int visible(int64_t s, int ratio, int64_t pos) { return ratio * (s + 1) - 1 <= pos; }  /* R5 */

/*
 * Lightning-indexer scores ([N] §1.1 step 2, eq. I_{t,s}; [M] §2.3.1):
 *   I[t,s] = sum_{h=1}^{H_I} w[t,h] * ReLU(q^I[t,h,:] . K^I[s,:])   for visible s,
 * -inf for entries the query may not see (R5, R6).
 * Layouts: qI [batch, T, H_I, c_I]; w [batch, T, H_I]; kI [batch, N, c_I];
 * qpos [T] absolute positions; scores [batch, T, N].
 */
void oracle_index_scores(const double* qI, const double* w, const double* kI, int64_t batch, int64_t T,
                         const int64_t* qpos, int64_t N, int H_I, int c_I, int m, double* scores) {
    int64_t bt;
#pragma omp parallel for schedule(dynamic, 1)
    for (bt = 0; bt < batch * T; ++bt) {
        int64_t b = bt / T, t = bt % T, s;
        for (s = 0; s < N; ++s) {
            double acc = 0.0;
            int h;
            if (!visible(s, m, qpos[t])) {
                scores[bt * N + s] = -INFINITY;
                continue;
            }
            for (h = 0; h < H_I; ++h) {
                double dot = 0.0;
                int d;
                for (d = 0; d < c_I; ++d) dot += qI[(bt * H_I + h) * c_I + d] * kI[(b * N + s) * c_I + d];
                acc += w[bt * H_I + h] * (dot > 0.0 ? dot : 0.0);
            }
            scores[bt * N + s] = acc;
        }
    }
}

typedef struct { double score; int64_t s; } scored;

static int by_score_desc_index_asc(const void* pa, const void* pb) {
    const scored* a = (const scored*)pa;
    const scored* b = (const scored*)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->s < b->s) ? -1 : (a->s > b->s);
}

static int by_index(const void* pa, const void* pb) {
    const scored* a = (const scored*)pa;
    const scored* b = (const scored*)pb;
    return (a->s < b->s) ? -1 : (a->s > b->s);
}

/*
 * Per-query top-k block selection ([N] §1.1 step 2; [M] §2.3.1), reading R7: full sort
 * of the visible entries by (score desc, index asc), keep the first min(k, |V|), emit
 * in ascending index order, pad with -1 / -inf.
 * Layouts: scores [batch, T, N]; idx [batch, T, k]; sel [batch, T, k] (may be NULL).
 */
void oracle_topk(const double* scores, int64_t batch, int64_t T, const int64_t* qpos, int64_t N, int m,
                 int k, int32_t* idx, double* sel) {
    int64_t bt;
#pragma omp parallel for schedule(dynamic, 1)
    for (bt = 0; bt < batch * T; ++bt) {
        int64_t t = bt % T, s, nv = 0, keep, r;
        scored* v = (scored*)malloc((size_t)(N > 0 ? N : 1) * sizeof(scored));
        for (s = 0; s < N; ++s) {
            if (visible(s, m, qpos[t])) {
                v[nv].score = scores[bt * N + s];
                v[nv].s = s;
                ++nv;
            }
        }
        qsort(v, (size_t)nv, sizeof(scored), by_score_desc_index_asc);
        keep = nv < k ? nv : k;
        qsort(v, (size_t)keep, sizeof(scored), by_index);
        for (r = 0; r < k; ++r) {
            idx[bt * k + r] = r < keep ? (int32_t)v[r].s : -1;
            if (sel) sel[bt * k + r] = r < keep ? v[r].score : -INFINITY;
        }
        free(v);
    }
}

/* ------------------------------------------------------------------ attention */

/* One query head attending to the entries listed in `ids` (shared-KV MQA, R8):
 * l_s = scale * q . kv_s, p = softmax(l), o = sum_s p_s kv_s. */
/* Softmax attention of one head over the entries `ids`.  With a sink logit z' ([N] §1.3 and
 * [M] §2.3.3 item 4, attention sink: the softmax denominator gains exp(z'), so a head may give
 * part of its weight to nothing) the weights are exp(z_s) / (sum_r exp(z_r) + exp(z')); `sink`
 * NULL means no sink.  Nothing selected: a zero output either way. */
static void attend(const double* q, const double* kv, const int64_t* ids, int64_t nsel, int c,
                   double scale, const double* sink, double* logit, double* o) {
    int64_t r;
    int d;
    double mx = -INFINITY, den = 0.0;
    for (d = 0; d < c; ++d) o[d] = 0.0;
    if (nsel == 0) return;
    for (r = 0; r < nsel; ++r) {
        double dot = 0.0;
        for (d = 0; d < c; ++d) dot += q[d] * kv[ids[r] * c + d];
        logit[r] = scale * dot;
        if (logit[r] > mx) mx = logit[r];
    }
    if (sink && *sink > mx) mx = *sink;
    for (r = 0; r < nsel; ++r) {
        double p = exp(logit[r] - mx);
        den += p;
        for (d = 0; d < c; ++d) o[d] += p * kv[ids[r] * c + d];
    }
    if (sink) den += exp(*sink - mx);
    for (d = 0; d < c; ++d) o[d] /= den;
}

/*
 * Sparse shared-KV MQA over the selected entries ([N] §1.1 step 2, last paragraph;
 * [M] §2.3.2 "shared-KV MQA"): every one of the H query heads attends to the same
 * selected compressed entries, each serving as key and value.  Ids outside [0, N)
 * (the -1 pads) are skipped.
 * Layouts: q [batch, T, H, c]; kv [batch, N, c]; idx [batch, T, k]; out [batch, T, H, c].
 */
void oracle_sparse_mqa(const double* q, const double* kv, const int32_t* idx, int64_t batch, int64_t T,
                       int64_t N, int H, int c, int k, double scale, const double* sink, double* out) {
    int64_t bt;
#pragma omp parallel for schedule(dynamic, 1)
    for (bt = 0; bt < batch * T; ++bt) {
        int64_t b = bt / T, nsel = 0;
        int r, h;
        int64_t* ids = (int64_t*)malloc((size_t)(k > 0 ? k : 1) * sizeof(int64_t));
        double* logit = (double*)malloc((size_t)(k > 0 ? k : 1) * sizeof(double));
        for (r = 0; r < k; ++r) {
            int32_t s = idx[bt * k + r];
            if (s >= 0 && s < N) ids[nsel++] = s;
        }
        for (h = 0; h < H; ++h)
            attend(q + (bt * H + h) * (int64_t)c, kv + b * N * c, ids, nsel, c, scale, sink ? sink + h : NULL,
                   logit, out + (bt * H + h) * (int64_t)c);
        free(ids);
        free(logit);
    }
}

/*
 * HCA dense MQA ([M] §2.3.2; [N] §1.2: no selection): every head of the query at
 * position p attends to every HCA entry s with m'(s+1)-1 <= p (R5).
 * Layouts: q [batch, T, H, c]; kv [batch, N, c]; qpos [T]; out [batch, T, H, c].
 */
void oracle_hca_dense_mqa(const double* q, const double* kv, int64_t batch, int64_t T, const int64_t* qpos,
                          int64_t N, int H, int c, int mp, double scale, const double* sink, double* out) {
    int64_t bt;
#pragma omp parallel for schedule(dynamic, 1)
    for (bt = 0; bt < batch * T; ++bt) {
        int64_t b = bt / T, t = bt % T, s, nsel = 0;
        int h;
        int64_t* ids = (int64_t*)malloc((size_t)(N > 0 ? N : 1) * sizeof(int64_t));
        double* logit = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
        for (s = 0; s < N; ++s)
            if (visible(s, mp, qpos[t])) ids[nsel++] = s;
        for (h = 0; h < H; ++h)
            attend(q + (bt * H + h) * (int64_t)c, kv + b * N * c, ids, nsel, c, scale, sink ? sink + h : NULL,
                   logit, out + (bt * H + h) * (int64_t)c);
        free(ids);
        free(logit);
    }
}
