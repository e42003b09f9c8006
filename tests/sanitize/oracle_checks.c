/* oracle_checks.c — drives every function of the C oracle on small inputs held in buffers of
 * exactly the sizes the functions are documented to touch, for an AddressSanitizer /
 * UndefinedBehaviorSanitizer build (tests/test_sanitizers.py compiles it with the oracle and
 * -fsanitize=address,undefined; any out-of-bounds access or undefined operation aborts).
 * A few results are checked too (weights summing to 1, the top-k rule on a tiny row). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_decode(const void* src, int dtype, int64_t count, double* dst);
int oracle_decode_mxfp4(const uint8_t* buf, int64_t rows, int c, double* dst);
int oracle_decode_kv_fp8_bf16(const uint8_t* buf, int64_t rows, int c, double* dst);
void oracle_rope(double* x, int64_t batch, int64_t T, int H, int c, int d, int64_t pos0, int64_t pos_step,
                 double base, int inverse);
int oracle_round(double* x, int dtype, int64_t count);
void oracle_csa_compress(const double* Ca, const double* Cb, const double* Za, const double* Zb, const double* Ba,
                         const double* Bb, int64_t batch, int64_t n, int m, int c, int out_dtype, double* out);
void oracle_hca_compress(const double* C, const double* Z, const double* B, int64_t batch, int64_t n, int mp, int c,
                         int out_dtype, double* out);
void oracle_index_scores(const double* qI, const double* w, const double* kI, int64_t batch, int64_t T,
                         const int64_t* qpos, int64_t N, int H_I, int c_I, int m, double* out);
void oracle_topk(const double* scores, int64_t batch, int64_t T, const int64_t* qpos, int64_t N, int m, int k,
                 int32_t* idx, double* sel);
void oracle_sparse_mqa(const double* q, const double* kv, const int32_t* idx, int64_t batch, int64_t T, int64_t N,
                       int H, int c, int k, double scale, const double* sink, double* out);
void oracle_hca_dense_mqa(const double* q, const double* kv, int64_t batch, int64_t T, const int64_t* qpos,
                          int64_t N, int H, int c, int mp, double scale, const double* sink, double* out);

static int fails = 0;
#define CHECK(cond)                                                       \
    do {                                                                  \
        if (!(cond)) {                                                    \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);        \
            ++fails;                                                      \
        }                                                                 \
    } while (0)

static uint64_t s_state = 88172645463325252ull;
static double rnd(void) {   /* xorshift64, uniform in [-1, 1) */
    s_state ^= s_state << 13;
    s_state ^= s_state >> 7;
    s_state ^= s_state << 17;
    return (double)(s_state >> 11) / 4503599627370496.0 - 1.0;
}
static double* vec(int64_t n) {
    double* p = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (int64_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}

int main(void) {
    /* storage decoders */
    {
        uint8_t b[256];
        double d[256];
        for (int i = 0; i < 256; ++i) b[i] = (uint8_t)i;
        CHECK(oracle_decode(b, 2, 256, d) == 0);
        CHECK(d[0x38] == 1.0 && isnan(d[0x7f]));
        uint16_t h[4] = {0x3f80, 0xbf80, 0x0000, 0x7f80};
        CHECK(oracle_decode(h, 1, 4, d) == 0 && d[0] == 1.0 && d[1] == -1.0 && isinf(d[3]));
        const int rows = 3, c = 64;
        uint8_t* mx = (uint8_t*)malloc((size_t)rows * (c / 2 + c / 32));
        for (int i = 0; i < rows * (c / 2 + c / 32); ++i) mx[i] = (uint8_t)(i * 37 + 11);
        for (int i = rows * c / 2; i < rows * (c / 2 + c / 32); ++i) mx[i] = 127;   /* scales 2^0 */
        double* out = vec(rows * c);
        CHECK(oracle_decode_mxfp4(mx, rows, c, out) == 0);
        free(mx);
        free(out);
        uint8_t* kv = (uint8_t*)malloc((size_t)rows * (128 + 64));
        for (int i = 0; i < rows * (128 + 64); ++i) kv[i] = (uint8_t)(i * 13);
        double* kd = vec(rows * 128);
        CHECK(oracle_decode_kv_fp8_bf16(kv, rows, 128, kd) == 0);
        free(kv);
        free(kd);
    }
    /* rounding */
    {
        double x[5] = {1.0 / 3.0, -500.0, 1e-9, 3.5, -0.0};
        CHECK(oracle_round(x, 2, 5) == 0 && x[1] == -448.0 && x[3] == 3.5);
        CHECK(oracle_round(x, 1, 5) == 0);
        CHECK(oracle_round(x, 7, 5) != 0);
    }
    /* compression: C = 1 gives 1 (weights sum to 1), ratio 1 and a ragged tail included */
    for (int m = 1; m <= 5; m += 2) {
        const int64_t batch = 2, n = 4 * m + 3;
        const int c = 8;
        double *Ca = vec(batch * n * c), *Cb = vec(batch * n * c), *Za = vec(batch * n * c), *Zb = vec(batch * n * c);
        double *Ba = vec(m * c), *Bb = vec(m * c);
        double* out = vec(batch * (n / m) * c);
        for (int64_t i = 0; i < batch * n * c; ++i) Ca[i] = Cb[i] = 1.0;
        oracle_csa_compress(Ca, Cb, Za, Zb, Ba, Bb, batch, n, m, c, -1, out);
        for (int64_t i = 0; i < batch * (n / m) * c; ++i) CHECK(fabs(out[i] - 1.0) < 1e-12);
        oracle_hca_compress(Ca, Za, Ba, batch, n, m, c, 1, out);
        for (int64_t i = 0; i < batch * (n / m) * c; ++i) CHECK(out[i] == 1.0);
        free(Ca); free(Cb); free(Za); free(Zb); free(Ba); free(Bb); free(out);
    }
    /* indexer, top-k, attention: queries before, at and after the visibility edges */
    {
        const int64_t batch = 2, T = 5, N = 9;
        const int H_I = 3, c_I = 8, H = 2, c = 16, m = 2, k = 4;
        int64_t qpos[5] = {0, 1, 2, 7, 40};
        double *qI = vec(batch * T * H_I * c_I), *w = vec(batch * T * H_I), *kI = vec(batch * N * c_I);
        double* sc = vec(batch * T * N);
        oracle_index_scores(qI, w, kI, batch, T, qpos, N, H_I, c_I, m, sc);
        CHECK(isinf(sc[0]) && sc[0] < 0);             /* position 0 sees nothing */
        int32_t* idx = (int32_t*)malloc((size_t)batch * T * k * sizeof(int32_t));
        double* sel = vec(batch * T * k);
        oracle_topk(sc, batch, T, qpos, N, m, k, idx, sel);
        CHECK(idx[0] == -1);
        for (int64_t r = 0; r < batch * T; ++r)
            for (int j = 1; j < k; ++j) CHECK(idx[r * k + j] == -1 || idx[r * k + j] > idx[r * k + j - 1]);
        /* ties: all-equal scores keep the lowest indices */
        double* flat = vec(N);
        for (int i = 0; i < N; ++i) flat[i] = 2.0;
        int64_t p1 = 100;
        int32_t ti[4];
        double ts[4];
        oracle_topk(flat, 1, 1, &p1, N, m, 4, ti, ts);
        CHECK(ti[0] == 0 && ti[1] == 1 && ti[2] == 2 && ti[3] == 3);
        double *q = vec(batch * T * H * c), *kv = vec(batch * N * c), *out = vec(batch * T * H * c), *sink = vec(H);
        idx[3] = 1000;   /* an id past the entries is skipped */
        oracle_sparse_mqa(q, kv, idx, batch, T, N, H, c, k, 0.25, NULL, out);
        oracle_sparse_mqa(q, kv, idx, batch, T, N, H, c, k, 0.25, sink, out);
        oracle_hca_dense_mqa(q, kv, batch, T, qpos, N, H, c, m, 0.25, sink, out);
        oracle_hca_dense_mqa(q, kv, batch, T, qpos, N, H, c, m, 0.25, NULL, out);
        for (int i = 0; i < H * c; ++i) CHECK(out[i] == 0.0);   /* query 0 sees nothing */
        oracle_rope(q, batch, T, H, c, 8, 1 << 20, 1, 10000.0, 0);
        oracle_rope(q, batch, T, H, c, 8, 1 << 20, 1, 10000.0, 1);
        free(qI); free(w); free(kI); free(sc); free(idx); free(sel); free(flat);
        free(q); free(kv); free(out); free(sink);
    }
    printf("oracle checks: %d failures\n", fails);
    return fails != 0;
}
