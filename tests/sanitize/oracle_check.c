/*
 * The CPU oracle (oracle/oracle.c) built with -fsanitize=address,undefined and run over random
 * small shapes (ragged K, salient subsets, every group width, ternary layers, a short fit): no
 * out-of-bounds access or undefined behaviour, and the oracle's two routes agree (the
 * dequantize-and-multiply definition and the table route; the ternary definition and its two
 * half-scale bases). Prints "ok" and exits 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_set_threads(int n);
void oracle_gemv(const uint32_t* bits, const float* alpha_r, const float* alpha_c, int nb, int64_t N, int64_t K,
                 const int32_t* idx, int64_t s, const uint32_t* bits_s, const float* alpha_r_s,
                 const float* alpha_c_s, int ns, const double* x, int batch, double* y);
void oracle_gemv_gs(const uint32_t* bits, const float* alpha_rg, int64_t gcols, int gsize, const float* alpha_c,
                    int nb, int64_t N, int64_t K, const int32_t* idx, int64_t s, const uint32_t* bits_s,
                    const float* alpha_r_s, const float* alpha_c_s, int ns, const double* x, int batch, double* y);
void oracle_patterns(const uint32_t* bits, int nb, int64_t N, int64_t K, int g, uint16_t* out);
void oracle_lut_tables(const double* x, int batch, const float* alpha_c, int nb, int64_t K, int g, double* out);
void oracle_lut_gemv(const uint32_t* bits, const float* alpha_r, const float* alpha_c, int nb, int64_t N, int64_t K,
                     const int32_t* idx, int64_t s, const uint32_t* bits_s, const float* alpha_r_s,
                     const float* alpha_c_s, int ns, const double* x, int batch, int g, double* y);
void oracle_ternary_gemv(const int8_t* w, const float* scale, int64_t N, int64_t K, const double* x, int batch,
                         double* y);
void oracle_ternary_encode(const int8_t* w, int64_t N, int64_t K, int zero_first_plus, uint32_t* out);
void oracle_fit(const float* w, int64_t N, int64_t K, int nb, int iters, uint32_t* bits, double* alpha_r,
                double* alpha_c, double* residual);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) { /* splitmix64 */
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static int64_t rnd(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }
static double unif(void) { return (double)(next() >> 11) / 9007199254740992.0; }
static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

static int fails = 0;
static void check(int ok, const char* what, int64_t a, int64_t b) {
    if (!ok && fails++ < 20) fprintf(stderr, "FAIL %s (%lld, %lld)\n", what, (long long)a, (long long)b);
}

static int close_to(double a, double b, double scale) { return fabs(a - b) <= 1e-9 * (scale > 1.0 ? scale : 1.0); }

int main(void) {
    oracle_set_threads(2);
    for (int it = 0; it < 120; ++it) {
        const int nb = (int)rnd(1, 3), batch = (int)rnd(1, 3);
        const int64_t N = rnd(1, 40), K = rnd(1, 300);
        const int64_t kw = (K + 31) / 32;
        const int64_t s = rnd(0, K < 40 ? K : 40);
        const int ns = s ? (int)rnd(1, 3) : 0;
        const int64_t sw = (s + 31) / 32;
        uint32_t* bits = xmalloc(sizeof(uint32_t) * (size_t)(nb * N * kw));
        for (int64_t i = 0; i < nb * N * kw; ++i) bits[i] = (uint32_t)next(); /* garbage past K too */
        float* ar = xmalloc(sizeof(float) * (size_t)(nb * N));
        float* ac = xmalloc(sizeof(float) * (size_t)(nb * K));
        for (int64_t i = 0; i < nb * N; ++i) ar[i] = (float)(0.1 + unif());
        for (int64_t i = 0; i < nb * K; ++i) ac[i] = (float)(0.1 + unif());
        int32_t* idx = xmalloc(sizeof(int32_t) * (size_t)s);
        { /* s distinct ascending columns */
            int64_t q = 0;
            for (int64_t j = 0; j < K && q < s; ++j)
                if ((int64_t)(next() % (uint64_t)(K - j)) < s - q) idx[q++] = (int32_t)j;
        }
        uint32_t* bits_s = xmalloc(sizeof(uint32_t) * (size_t)(ns * N * sw));
        for (int64_t i = 0; i < ns * N * sw; ++i) bits_s[i] = (uint32_t)next();
        float* ars = xmalloc(sizeof(float) * (size_t)(ns * N));
        float* acs = xmalloc(sizeof(float) * (size_t)(ns * s));
        for (int64_t i = 0; i < ns * N; ++i) ars[i] = (float)(0.1 + unif());
        for (int64_t i = 0; i < ns * s; ++i) acs[i] = (float)(0.1 + unif());
        double* x = xmalloc(sizeof(double) * (size_t)(batch * K));
        for (int64_t i = 0; i < batch * K; ++i) x[i] = unif() * 2.0 - 1.0;
        double* y0 = xmalloc(sizeof(double) * (size_t)(batch * N));
        double* y1 = xmalloc(sizeof(double) * (size_t)(batch * N));
        oracle_gemv(bits, ar, ac, nb, N, K, idx, s, bits_s, ars, acs, ns, x, batch, y0);
        double scale = 0.0;
        for (int64_t i = 0; i < batch * N; ++i) scale = fabs(y0[i]) > scale ? fabs(y0[i]) : scale;
        const int gs[2] = {4, 8};
        for (int gi = 0; gi < 2; ++gi) {
            oracle_lut_gemv(bits, ar, ac, nb, N, K, idx, s, bits_s, ars, acs, ns, x, batch, gs[gi], y1);
            for (int64_t i = 0; i < batch * N; ++i) check(close_to(y0[i], y1[i], scale), "table route", it, i);
            const int64_t ng = (K + gs[gi] - 1) / gs[gi];
            uint16_t* pat = xmalloc(sizeof(uint16_t) * (size_t)(nb * N * ng));
            oracle_patterns(bits, nb, N, K, gs[gi], pat);
            for (int64_t i = 0; i < nb * N * ng; ++i) check(pat[i] < (1u << gs[gi]), "pattern range", it, i);
            free(pat);
            double* T = xmalloc(sizeof(double) * (size_t)(batch * nb * ng * (1 << gs[gi])));
            oracle_lut_tables(x, batch, ac, nb, K, gs[gi], T);
            /* complementary patterns negate: T[p] = -T[~p] */
            const int np = 1 << gs[gi];
            for (int64_t t = 0; t < batch * nb * ng; ++t)
                for (int p = 0; p < np; ++p)
                    check(close_to(T[t * np + p], -T[t * np + (np - 1 - p)], 1.0), "table symmetry", it, p);
            free(T);
        }
        /* group scales equal along the row reduce to the per-row scale */
        {
            const int gsize = 128;
            const int64_t gcols = (K + gsize - 1) / gsize + 1;
            float* arg = xmalloc(sizeof(float) * (size_t)(nb * N * gcols));
            for (int k = 0; k < nb; ++k)
                for (int64_t r = 0; r < N; ++r)
                    for (int64_t c = 0; c < gcols; ++c) arg[(k * N + r) * gcols + c] = ar[k * N + r];
            oracle_gemv_gs(bits, arg, gcols, gsize, ac, nb, N, K, idx, s, bits_s, ars, acs, ns, x, batch, y1);
            for (int64_t i = 0; i < batch * N; ++i) check(close_to(y0[i], y1[i], scale), "group scales", it, i);
            free(arg);
        }
        /* ternary: the definition against two half-scale bases through the table route */
        {
            int8_t* w = xmalloc((size_t)(N * K));
            for (int64_t i = 0; i < N * K; ++i) w[i] = (int8_t)((int)(next() % 3) - 1);
            float* sc = xmalloc(sizeof(float) * (size_t)N);
            for (int64_t r = 0; r < N; ++r) sc[r] = (float)(0.01 + 0.1 * unif());
            uint32_t* tb = xmalloc(sizeof(uint32_t) * (size_t)(2 * N * kw));
            oracle_ternary_encode(w, N, K, (int)(it & 1), tb);
            float* tar = xmalloc(sizeof(float) * (size_t)(2 * N));
            float* tac = xmalloc(sizeof(float) * (size_t)(2 * K));
            for (int64_t r = 0; r < N; ++r) tar[r] = tar[N + r] = 0.5f * sc[r];
            for (int64_t j = 0; j < 2 * K; ++j) tac[j] = 1.0f;
            oracle_ternary_gemv(w, sc, N, K, x, batch, y0);
            oracle_lut_gemv(tb, tar, tac, 2, N, K, NULL, 0, NULL, NULL, NULL, 0, x, batch, 8, y1);
            double ts = 0.0;
            for (int64_t i = 0; i < batch * N; ++i) ts = fabs(y0[i]) > ts ? fabs(y0[i]) : ts;
            for (int64_t i = 0; i < batch * N; ++i) check(close_to(y0[i], y1[i], ts), "ternary", it, i);
            free(w); free(sc); free(tb); free(tar); free(tac);
        }
        /* a short fit: the residual never grows with the bases */
        if (it % 4 == 0) {
            const int fnb = (int)rnd(1, 3);
            float* w = xmalloc(sizeof(float) * (size_t)(N * K));
            double norm0 = 0.0;
            for (int64_t i = 0; i < N * K; ++i) w[i] = (float)(unif() * 2.0 - 1.0), norm0 += (double)w[i] * w[i];
            uint32_t* fb = xmalloc(sizeof(uint32_t) * (size_t)(fnb * N * kw));
            double* far = xmalloc(sizeof(double) * (size_t)(fnb * N));
            double* fac = xmalloc(sizeof(double) * (size_t)(fnb * K));
            double* res = xmalloc(sizeof(double) * (size_t)(N * K));
            oracle_fit(w, N, K, fnb, (int)rnd(0, 3), fb, far, fac, res);
            double norm1 = 0.0;
            for (int64_t i = 0; i < N * K; ++i) norm1 += res[i] * res[i];
            check(norm1 <= norm0 * (1.0 + 1e-12), "fit residual", it, 0);
            free(w); free(fb); free(far); free(fac); free(res);
        }
        free(bits); free(ar); free(ac); free(idx); free(bits_s); free(ars); free(acs); free(x); free(y0); free(y1);
    }
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("ok\n");
    return 0;
}
