/*
 * CPU oracle for the matrix-vector product against decoupled row-column binary bases.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load this library. The GPU library never calls it, links it or shares code with it.
 *
 * Source: "FluxBin: Flexible LUT-based Ultra-low-bit LLM Inference by Algorithm-Kernel
 * Synergy" (gist.science/ko/paper/2608.15602), technical summary:
 *   - "1. Algorithm innovation", decoupled row-column binary decomposition: each base is
 *     W_hat^(k) = (alpha_r^(k) alpha_c^(k)^T) (.) B^(k) with B^(k) in {-1,+1}, and the dense
 *     weight is approximated by the sum of the bases.
 *   - same section, hybrid bases: a global approximation over the whole matrix plus a
 *     salient-refinement branch on selected columns; the final weight is their sum.
 *   - "2. Kernel innovation", LUT-BSF and the execution flow: the column scale is folded into
 *     precomputed partial-sum tables, pattern indices are read from the packed bits, the
 *     partial sums are fetched and the row scale is applied during the reduction.
 *
 * Every function here works in fp64. fp32 and fp16 inputs convert to fp64 exactly, and the
 * product alpha_r * alpha_c of two fp32 values is exact in fp64.
 *
 * Bit convention (the page does not fix one; this reading is used throughout):
 *   bit value 1 means +1 and 0 means -1; column j of a row lives in word j/32 at bit j%32
 *   (least significant bit first). Rows of base k are stored [k][row][ceil(K/32) words].
 *   Bits at columns >= K in the last word of a row are ignored.
 *
 * Pins: tests/test_oracle.py checks these functions against brute-force sign enumeration,
 * closed forms, integer matvecs done by numpy, invariants of the decomposition and a
 * hand-worked fixture.
 */
#include <stdint.h>
#include <stdlib.h>
#include <math.h>
#include <string.h>
#include <omp.h>

static int64_t words_per_row(int64_t K) { return (K + 31) / 32; }

/* Sign of column j of one canonical row: +1.0 when the bit is set, -1.0 otherwise. */
static double sign_at(const uint32_t* row, int64_t j) {
    return ((row[j / 32] >> (j % 32)) & 1u) ? 1.0 : -1.0;
}

/* Bit j of one canonical row, with columns >= K reading as 0. */
static unsigned bit_at(const uint32_t* row, int64_t K, int64_t j) {
    if (j >= K) return 0u;
    return (row[j / 32] >> (j % 32)) & 1u;
}

void oracle_set_threads(int n) {
    if (n > 0) omp_set_num_threads(n);
}

int oracle_max_threads(void) { return omp_get_max_threads(); }

/*
 * Dequantize-and-multiply: the plain definition.
 *
 * W_hat[r][j] = sum_{k<nb} alpha_r[k][r] * alpha_c[k][j] * B^(k)[r][j]
 *             + sum over salient positions q<s with idx[q] == j of
 *               sum_{k<ns} alpha_r_s[k][r] * alpha_c_s[k][q] * B_s^(k)[r][q]
 * y[b][r]     = sum_{j<K} W_hat[r][j] * x[b][j]
 *
 * bits:      [nb][N][ceil(K/32)]      canonical words of the main bases
 * alpha_r:   [nb][N], alpha_c: [nb][K]
 * idx:       [s] salient column indices (any order, each in [0,K)); s may be 0
 * bits_s:    [ns][N][ceil(s/32)]      canonical words of the refinement bases
 * alpha_r_s: [ns][N], alpha_c_s: [ns][s]
 * x:         [batch][K]               activations, already in fp64
 * y:         [batch][N]               output, overwritten
 *
 * One row of W_hat is built at a time, so memory stays O(K) per thread.
 */
void oracle_gemv(const uint32_t* bits, const float* alpha_r, const float* alpha_c, int nb,
                 int64_t N, int64_t K,
                 const int32_t* idx, int64_t s, const uint32_t* bits_s,
                 const float* alpha_r_s, const float* alpha_c_s, int ns,
                 const double* x, int batch, double* y) {
    const int64_t kw = words_per_row(K);
    const int64_t sw = words_per_row(s);
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < N; ++r) {
            for (int64_t j = 0; j < K; ++j) w[j] = 0.0;
            /* global bases over every column */
            for (int k = 0; k < nb; ++k) {
                const uint32_t* row = bits + ((int64_t)k * N + r) * kw;
                const double ar = (double)alpha_r[(int64_t)k * N + r];
                for (int64_t j = 0; j < K; ++j)
                    w[j] += ar * (double)alpha_c[(int64_t)k * K + j] * sign_at(row, j);
            }
            /* salient refinement, added on top at the salient columns */
            for (int k = 0; k < ns && s > 0; ++k) {
                const uint32_t* row = bits_s + ((int64_t)k * N + r) * sw;
                const double ar = (double)alpha_r_s[(int64_t)k * N + r];
                for (int64_t q = 0; q < s; ++q)
                    w[idx[q]] += ar * (double)alpha_c_s[(int64_t)k * s + q] * sign_at(row, q);
            }
            for (int b = 0; b < batch; ++b) {
                const double* xb = x + (int64_t)b * K;
                double acc = 0.0;
                for (int64_t j = 0; j < K; ++j) acc += w[j] * xb[j];
                y[(int64_t)b * N + r] = acc;
            }
        }
        free(w);
    }
}


/*
 * Group-scale variant of the same definition: the row scale of a main base varies along the
 * row, one value per block of gsize columns (the technical summary's "Experimental results"
 * name a "2b-s16-g128" setting; read as 2 bases, 16-bit scales, 128-column groups):
 *
 * W_hat[r][j] = sum_{k<nb} alpha_rg[k][r][j / gsize] * alpha_c[k][j] * B^(k)[r][j]
 *             + the salient refinement exactly as in oracle_gemv
 * y[b][r]     = sum_{j<K} W_hat[r][j] * x[b][j]
 *
 * alpha_rg: [nb][N][gcols], gcols >= ceil(K / gsize) (entries past that are not read).
 * Other arguments as oracle_gemv.
 */
void oracle_gemv_gs(const uint32_t* bits, const float* alpha_rg, int64_t gcols, int gsize,
                    const float* alpha_c, int nb, int64_t N, int64_t K,
                    const int32_t* idx, int64_t s, const uint32_t* bits_s,
                    const float* alpha_r_s, const float* alpha_c_s, int ns,
                    const double* x, int batch, double* y) {
    const int64_t kw = words_per_row(K);
    const int64_t sw = words_per_row(s);
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(static)
        for (int64_t r = 0; r < N; ++r) {
            for (int64_t j = 0; j < K; ++j) w[j] = 0.0;
            for (int k = 0; k < nb; ++k) {
                const uint32_t* row = bits + ((int64_t)k * N + r) * kw;
                const float* ar = alpha_rg + ((int64_t)k * N + r) * gcols;
                for (int64_t j = 0; j < K; ++j)
                    w[j] += (double)ar[j / gsize] * (double)alpha_c[(int64_t)k * K + j] * sign_at(row, j);
            }
            for (int k = 0; k < ns && s > 0; ++k) {
                const uint32_t* row = bits_s + ((int64_t)k * N + r) * sw;
                const double ar = (double)alpha_r_s[(int64_t)k * N + r];
                for (int64_t q = 0; q < s; ++q)
                    w[idx[q]] += ar * (double)alpha_c_s[(int64_t)k * s + q] * sign_at(row, q);
            }
            for (int b = 0; b < batch; ++b) {
                const double* xb = x + (int64_t)b * K;
                double acc = 0.0;
                for (int64_t j = 0; j < K; ++j) acc += w[j] * xb[j];
                y[(int64_t)b * N + r] = acc;
            }
        }
        free(w);
    }
}

/*
 * Pattern indices: for base k, row r and group gi (columns gi*g .. gi*g+g-1), the g-bit
 * number whose bit i is the sign bit of column gi*g+i. Columns >= K read as 0.
 * out: [nb][N][ceil(K/g)]
 */
void oracle_patterns(const uint32_t* bits, int nb, int64_t N, int64_t K, int g, uint16_t* out) {
    const int64_t kw = words_per_row(K);
    const int64_t ng = (K + g - 1) / g;
#pragma omp parallel for schedule(static)
    for (int64_t kr = 0; kr < (int64_t)nb * N; ++kr) {
        const uint32_t* row = bits + kr * kw;
        for (int64_t gi = 0; gi < ng; ++gi) {
            unsigned p = 0;
            for (int i = 0; i < g; ++i) p |= bit_at(row, K, gi * g + i) << i;
            out[kr * ng + gi] = (uint16_t)p;
        }
    }
}

/*
 * LUT-BSF tables, fp64: with v = alpha_c^(k) (.) x_b (v = 0 past column K),
 * T[b][k][gi][p] = sum_{i<g} (2*bit_i(p) - 1) * v[gi*g + i],  p in [0, 2^g).
 * out: [batch][nb][ceil(K/g)][2^g]
 */
void oracle_lut_tables(const double* x, int batch, const float* alpha_c, int nb, int64_t K, int g,
                       double* out) {
    const int64_t ng = (K + g - 1) / g;
    const int64_t np = (int64_t)1 << g;
#pragma omp parallel for schedule(static)
    for (int64_t bkg = 0; bkg < (int64_t)batch * nb * ng; ++bkg) {
        const int64_t gi = bkg % ng;
        const int64_t k = (bkg / ng) % nb;
        const int64_t b = bkg / ng / nb;
        double v[16];
        for (int i = 0; i < g; ++i) {
            const int64_t j = gi * g + i;
            v[i] = j < K ? (double)alpha_c[k * K + j] * x[b * K + j] : 0.0;
        }
        for (int64_t p = 0; p < np; ++p) {
            double t = 0.0;
            for (int i = 0; i < g; ++i) t += ((p >> i) & 1) ? v[i] : -v[i];
            out[bkg * np + p] = t;
        }
    }
}

/*
 * The same product evaluated the way the kernel section describes, in fp64: build the
 * partial-sum tables with alpha_c folded in, read each row's pattern indices, sum the table
 * entries and scale by alpha_r. The refinement branch does the same over a virtual matrix
 * whose column q holds the salient column idx[q] (activations gathered by idx, scales
 * alpha_c_s), which is the virtual columnar mapping. Used to check that the table route
 * reaches the dequantized result.
 * Arguments as oracle_gemv, plus g (1..12).
 */
static void lut_branch(const uint32_t* bits, const float* alpha_r, const double* v_all /*[batch][nb][Kc]*/,
                       int nb, int64_t N, int64_t Kc, int g, int batch, double* y) {
    const int64_t kw = words_per_row(Kc);
    const int64_t ng = (Kc + g - 1) / g;
    const int64_t np = (int64_t)1 << g;
    double* T = (double*)malloc(sizeof(double) * (size_t)(batch * nb * ng * np + 1));
    for (int64_t bkg = 0; bkg < (int64_t)batch * nb * ng; ++bkg) {
        const int64_t gi = bkg % ng;
        const int64_t bk = bkg / ng;
        for (int64_t p = 0; p < np; ++p) {
            double t = 0.0;
            for (int i = 0; i < g; ++i) {
                const int64_t j = gi * g + i;
                const double vi = j < Kc ? v_all[bk * Kc + j] : 0.0;
                t += ((p >> i) & 1) ? vi : -vi;
            }
            T[bkg * np + p] = t;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; ++r) {
        for (int b = 0; b < batch; ++b) {
            double acc = 0.0;
            for (int k = 0; k < nb; ++k) {
                const uint32_t* row = bits + ((int64_t)k * N + r) * kw;
                const double* Tk = T + (((int64_t)b * nb + k) * ng) * np;
                double sk = 0.0;
                for (int64_t gi = 0; gi < ng; ++gi) {
                    unsigned p = 0;
                    for (int i = 0; i < g; ++i) p |= bit_at(row, Kc, gi * g + i) << i;
                    sk += Tk[gi * np + p];
                }
                acc += (double)alpha_r[(int64_t)k * N + r] * sk;
            }
            y[(int64_t)b * N + r] += acc;
        }
    }
    free(T);
}

void oracle_lut_gemv(const uint32_t* bits, const float* alpha_r, const float* alpha_c, int nb,
                     int64_t N, int64_t K,
                     const int32_t* idx, int64_t s, const uint32_t* bits_s,
                     const float* alpha_r_s, const float* alpha_c_s, int ns,
                     const double* x, int batch, int g, double* y) {
    for (int64_t i = 0; i < (int64_t)batch * N; ++i) y[i] = 0.0;
    double* v = (double*)calloc((size_t)(batch * nb * K + 1), sizeof(double));
    for (int b = 0; b < batch; ++b)
        for (int k = 0; k < nb; ++k)
            for (int64_t j = 0; j < K; ++j)
                v[((int64_t)b * nb + k) * K + j] = (double)alpha_c[(int64_t)k * K + j] * x[(int64_t)b * K + j];
    lut_branch(bits, alpha_r, v, nb, N, K, g, batch, y);
    free(v);
    if (s > 0 && ns > 0) {
        double* vs = (double*)calloc((size_t)(batch * ns * s) + 1, sizeof(double));
        for (int b = 0; b < batch; ++b)
            for (int k = 0; k < ns; ++k)
                for (int64_t q = 0; q < s; ++q)
                    vs[((int64_t)b * ns + k) * s + q] =
                        (double)alpha_c_s[(int64_t)k * s + q] * x[(int64_t)b * K + idx[q]];
        lut_branch(bits_s, alpha_r_s, vs, ns, N, s, g, batch, y);
        free(vs);
    }
}

/*
 * Ternary linear layer, by its definition: y[b][r] = scale[r] * sum_j w[r][j] * x[b][j],
 * w in {-1, 0, +1} stored as int8 [N][K].
 */
void oracle_ternary_gemv(const int8_t* w, const float* scale, int64_t N, int64_t K,
                         const double* x, int batch, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; ++r) {
        for (int b = 0; b < batch; ++b) {
            double acc = 0.0;
            for (int64_t j = 0; j < K; ++j) acc += (double)w[r * K + j] * x[(int64_t)b * K + j];
            y[(int64_t)b * N + r] = (double)scale[r] * acc;
        }
    }
}

/*
 * Ternary weights as two binary bases at half scale: w = (B1 + B2) / 2 with
 * B1 = +1 where w > 0, -1 where w < 0; B2 likewise; and for w == 0 one base is +1 and the
 * other -1. zero_first_plus selects which: 1 gives (B1, B2) = (+1, -1), 0 gives (-1, +1).
 * out: canonical words [2][N][ceil(K/32)], fully overwritten (unused high bits zero).
 */
void oracle_ternary_encode(const int8_t* w, int64_t N, int64_t K, int zero_first_plus, uint32_t* out) {
    const int64_t kw = words_per_row(K);
    memset(out, 0, sizeof(uint32_t) * (size_t)(2 * N * kw));
    for (int64_t r = 0; r < N; ++r) {
        for (int64_t j = 0; j < K; ++j) {
            const int8_t v = w[r * K + j];
            unsigned b1, b2;
            if (v > 0) { b1 = 1; b2 = 1; }
            else if (v < 0) { b1 = 0; b2 = 0; }
            else { b1 = zero_first_plus ? 1u : 0u; b2 = zero_first_plus ? 0u : 1u; }
            out[(0 * N + r) * kw + j / 32] |= b1 << (j % 32);
            out[(1 * N + r) * kw + j / 32] |= b2 << (j % 32);
        }
    }
}

/*
 * Offline fit of the decomposition from a dense matrix: residual binarization with
 * alternating least squares for the two scale vectors. The page ("1. Algorithm innovation")
 * gives only the form W ~ sum_k (alpha_r^(k) alpha_c^(k)^T) (.) B^(k); the steps below are
 * the plainest fit of that form, written out:
 *
 *   R = W
 *   for each base k:
 *     B = sign(R)  (+1 where R >= 0), so that R (.) B = |R| =: A
 *     alpha_r[r] = mean_j A[r][j], alpha_c = 1                      (per-row binarization)
 *     repeat iters times (each half step is the exact least-squares solution of
 *     min ||A - alpha_r alpha_c^T||_F for one vector with the other fixed):
 *       alpha_c[j] = sum_r A[r][j] alpha_r[r] / sum_r alpha_r[r]^2   (0 if the sum is 0)
 *       alpha_r[r] = sum_j A[r][j] alpha_c[j] / sum_j alpha_c[j]^2   (0 if the sum is 0)
 *     R = R - (alpha_r alpha_c^T) (.) B
 *
 * w [N][K] (fp32 values), bits [nb][N][ceil(K/32)] canonical (columns >= K zero),
 * alpha_r [nb][N], alpha_c [nb][K], residual [N][K] (the final R). All arithmetic fp64.
 */
void oracle_fit(const float* w, int64_t N, int64_t K, int nb, int iters, uint32_t* bits,
                double* alpha_r, double* alpha_c, double* residual) {
    const int64_t kw = words_per_row(K);
    double* R = residual;
    for (int64_t i = 0; i < N * K; ++i) R[i] = (double)w[i];
    memset(bits, 0, sizeof(uint32_t) * (size_t)(nb * N * kw));
    for (int k = 0; k < nb; ++k) {
        uint32_t* bk = bits + (int64_t)k * N * kw;
        double* ar = alpha_r + (int64_t)k * N;
        double* ac = alpha_c + (int64_t)k * K;
        for (int64_t r = 0; r < N; ++r) {
            double s = 0.0;
            for (int64_t j = 0; j < K; ++j) {
                const double v = R[r * K + j];
                if (v >= 0.0) bk[r * kw + j / 32] |= 1u << (j % 32);
                s += fabs(v);
            }
            ar[r] = s / (double)K;
        }
        for (int64_t j = 0; j < K; ++j) ac[j] = 1.0;
        for (int it = 0; it < iters; ++it) {
            double sr = 0.0;
            for (int64_t r = 0; r < N; ++r) sr += ar[r] * ar[r];
            for (int64_t j = 0; j < K; ++j) ac[j] = 0.0;
            for (int64_t r = 0; r < N; ++r)
                for (int64_t j = 0; j < K; ++j) ac[j] += fabs(R[r * K + j]) * ar[r];
            for (int64_t j = 0; j < K; ++j) ac[j] = sr > 0.0 ? ac[j] / sr : 0.0;
            double sc = 0.0;
            for (int64_t j = 0; j < K; ++j) sc += ac[j] * ac[j];
#pragma omp parallel for schedule(static)
            for (int64_t r = 0; r < N; ++r) {
                double s = 0.0;
                for (int64_t j = 0; j < K; ++j) s += fabs(R[r * K + j]) * ac[j];
                ar[r] = sc > 0.0 ? s / sc : 0.0;
            }
        }
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < N; ++r)
            for (int64_t j = 0; j < K; ++j) {
                const double b = ((bk[r * kw + j / 32] >> (j % 32)) & 1u) ? 1.0 : -1.0;
                R[r * K + j] -= ar[r] * ac[j] * b;
            }
    }
}
