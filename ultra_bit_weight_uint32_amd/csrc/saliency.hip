// Hessian-guided salient-column search (load time, before the GEMV path).
//
// "FluxBin" technical summary, "1. Algorithm innovation", saliency search: weight
// sensitivities are approximated through the inverse Hessian in the Optimal Brain
// Quantization framework, and the columns with the highest scores form the salient mask.
// Reading taken here (the page gives no formula): H = 2 X^T X from calibration activations X
// [T][K]; H_d = H + lambda I with lambda = damp * mean(diag H) (1 when that mean is 0);
// d_j = [H_d^-1]_jj; score_j = sum_r W[r][j]^2 / d_j^2; the s highest scores (ties: lower index)
// are the salient columns, returned ascending.
//
// Kernels:
//   k_gram         H = scale X^T X on the matrix cores (v_mfma_f32_32x32x16_f16): the one
//                  dense contraction of the method. One workgroup per 128 x 128 tile of the
//                  upper triangle (mirrored), X double-buffered through LDS 32 rows per stage.
//   k_damp         lambda from the diagonal, added to it.
//   k_chol_diag    Cholesky of one 64 x 64 diagonal block in one wave (a row per lane), and
//                  the inverse of that factor (kept for the panel and for the inverse's diagonal).
//   k_chol_panel   L_ik = A_ik L_kk^-T for the block rows below.
//   k_chol_update  A_ij -= L_ik L_jk^T for the trailing lower blocks.
//   k_trsm_row / k_trsm_update   the solve L Z = I right-looking by block rows (every step one
//                  launch of independent 64 x 64 block products); k_colnorm then sums the
//                  squares of Z's columns: d_j = ||L^-1 e_j||^2.
//   k_score_part / k_score_finish   column sums of W^2 in row chunks, then score = sum / d^2.
//   k_rank         rank of every score (count of larger scores, equal ones at lower indices),
//                  in 16 partial counts per score over slices of the scores.
//   k_rank_finish  adds the partial counts: one flag per column, rank < s.
//   k_select       the flagged columns, ascending, by one prefix scan.
// Everything after the Gram matrix is fp32 vector arithmetic in a fixed order.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "ubw_internal.h"

namespace ubw {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kGT = 128;  // H tile per workgroup
constexpr int kGS = 32;   // rows of X per stage
constexpr int kGP = 8;    // LDS row padding (halves): 80-byte rows keep 16-byte reads aligned

// Upper-triangle tile p (tiles (ti, tj) with ti <= tj, row-major) of an nt x nt tile grid.
__device__ __forceinline__ void upper_tile(int p, int nt, int& ti, int& tj) {
    int r = 0, rem = p;
    while (rem >= nt - r) {
        rem -= nt - r;
        ++r;
    }
    ti = r;
    tj = r + rem;
}

// One workgroup per tile (ti <= tj) of H = scale X^T X (H is symmetric: the tile is written at
// (ti, tj) and mirrored at (tj, ti)). Four waves, each a 64 x 64 quarter as 2 x 2 tiles of
// v_mfma_f32_32x32x16_f16. X streams through LDS 32 rows per stage, two buffers: the next
// stage's loads are issued before this stage's matrix instructions. Each thread loads 4 rows x
// 2 columns per task (4-byte loads, consecutive threads on consecutive column pairs) and stores
// them transposed as two 8-byte LDS writes, [column][row], so that a lane's 8 consecutive rows
// (its k values) are one 16-byte LDS read. k is summed over, so any assignment of rows to
// (lane half, element) that is the same for both operands gives X^T X.
// pairs: K even and X 4-byte aligned, so every column pair is one aligned 4-byte load.
__global__ __launch_bounds__(256) void k_gram(const __half* __restrict__ X, int T, int K, int pairs, float scale,
                                              float* __restrict__ H) {
    __shared__ __align__(16) _Float16 sA[2][kGT][kGS + kGP];
    __shared__ __align__(16) _Float16 sB[2][kGT][kGS + kGP];
    const int nt = (K + kGT - 1) / kGT;
    int ti, tj;
    upper_tile(blockIdx.x, nt, ti, tj);
    const int i0 = ti * kGT, j0 = tj * kGT;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    const uint16_t* Xu = reinterpret_cast<const uint16_t*>(X);
    // load tasks: task q = tid + 256 e (e = 0, 1): rows 4 (q / 64) .. +3, columns 2 (q % 64), +1
    uint32_t ra[2][4], rb[2][4];
    auto load = [&](int t0) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int q = tid + 256 * e;
            const int tr = 4 * (q >> 6), c = 2 * (q & 63);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = t0 + tr + u;
                const int64_t off = (int64_t)t * K;
                uint32_t va = 0, vb = 0;
                const int ia = i0 + c, jb = j0 + c;
                if (t < T && pairs) {  // c even, K even: a pair starting below K ends below K
                    if (ia < K) va = *reinterpret_cast<const uint32_t*>(Xu + off + ia);
                    if (jb < K) vb = *reinterpret_cast<const uint32_t*>(Xu + off + jb);
                } else if (t < T) {
                    if (ia + 1 < K) va = (uint32_t)Xu[off + ia] | ((uint32_t)Xu[off + ia + 1] << 16);
                    else if (ia < K) va = Xu[off + ia];
                    if (jb + 1 < K) vb = (uint32_t)Xu[off + jb] | ((uint32_t)Xu[off + jb + 1] << 16);
                    else if (jb < K) vb = Xu[off + jb];
                }
                ra[e][u] = va;
                rb[e][u] = vb;
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int q = tid + 256 * e;
            const int tr = 4 * (q >> 6), c = 2 * (q & 63);
            // column c: low halves of rows tr..tr+3; column c + 1: high halves
            auto lo2 = [](uint32_t p, uint32_t q) { return (p & 0xFFFFu) | (q << 16); };
            auto hi2 = [](uint32_t p, uint32_t q) { return (p >> 16) | (q & 0xFFFF0000u); };
            const uint2 a0 = make_uint2(lo2(ra[e][0], ra[e][1]), lo2(ra[e][2], ra[e][3]));
            const uint2 a1 = make_uint2(hi2(ra[e][0], ra[e][1]), hi2(ra[e][2], ra[e][3]));
            const uint2 b0 = make_uint2(lo2(rb[e][0], rb[e][1]), lo2(rb[e][2], rb[e][3]));
            const uint2 b1 = make_uint2(hi2(rb[e][0], rb[e][1]), hi2(rb[e][2], rb[e][3]));
            *reinterpret_cast<uint2*>(&sA[buf][c][tr]) = a0;
            *reinterpret_cast<uint2*>(&sA[buf][c + 1][tr]) = a1;
            *reinterpret_cast<uint2*>(&sB[buf][c][tr]) = b0;
            *reinterpret_cast<uint2*>(&sB[buf][c + 1][tr]) = b1;
        }
    };
    float16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
    load(0);
    store(0);
    __syncthreads();
    int buf = 0;
    for (int t0 = 0; t0 < T; t0 += kGS) {
        const bool more = t0 + kGS < T;
        if (more) load(t0 + kGS);  // in flight during this stage's matrix instructions
#pragma unroll
        for (int kk = 0; kk < kGS; kk += 16) {
            half8_t a[2], b[2];
            const int ko = kk + 8 * (lane >> 5);
#pragma unroll
            for (int m = 0; m < 2; ++m)
                a[m] = *reinterpret_cast<const half8_t*>(&sA[buf][wm * 64 + m * 32 + (lane & 31)][ko]);
#pragma unroll
            for (int n = 0; n < 2; ++n)
                b[n] = *reinterpret_cast<const half8_t*>(&sB[buf][wn * 64 + n * 32 + (lane & 31)][ko]);
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m], b[n], acc[m][n], 0, 0, 0);
        }
        if (more) store(buf ^ 1);  // the other buffer: last read before the previous barrier
        __syncthreads();
        buf ^= 1;
    }
    // result element (row 8 (v / 4) + 4 (lane / 32) + v % 4, column lane % 32) of each 32 x 32 tile
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int i = i0 + wm * 64 + m * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int j = j0 + wn * 64 + n * 32 + (lane & 31);
                if (i < K && j < K) {
                    const float h = scale * acc[m][n][v];
                    H[(int64_t)i * K + j] = h;
                    if (ti != tj) H[(int64_t)j * K + i] = h;
                }
            }
}

// Sum over a 256-thread workgroup; every thread gets the total.
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// misc[0] = lambda, misc[1] = error code (0 none, 1 a pivot was not positive, 2 the selection
// did not find exactly s columns).
__global__ __launch_bounds__(256) void k_damp(float* H, int K, float damp, float* misc) {
    __shared__ float red[4];
    float s = 0.f;
    for (int j = threadIdx.x; j < K; j += 256) s += H[(int64_t)j * K + j];
    s = block_sum256(s, red);
    float lam = damp * (s / (float)K);
    if (!(lam > 0.f)) lam = 1.f;
    for (int j = threadIdx.x; j < K; j += 256) H[(int64_t)j * K + j] += lam;
    if (threadIdx.x == 0) {
        misc[0] = lam;
        misc[1] = 0.f;
    }
}

constexpr int kCB = 64;  // Cholesky block

// Cholesky of diagonal block kb, written back, and its inverse to Linv[kb]. Rows/columns past K
// act as an identity block. One wave and no cross-wave barrier: lane r holds row r of the block
// in registers. The factorization is right-looking on the unscaled Schur complement S: step c
// publishes column c through LDS (the same wave reads it back, in order) and every lane
// subtracts (S[r][c] / S[c][c]) S[q][c] from S[r][q], q > c, which leaves column c untouched; the
// pivots' roots scale the columns at the end (the wave reads its own LDS writes in order, so
// the steps need no barrier). The inverse Z = L^-1 is one forward substitution
// per column, lane j computing column j from the rows of L broadcast from LDS. (A 1024-thread
// version with 16 waves, a barrier per step and the inverse solved by rows took 49 us per block;
// the search at K = 4096 runs 64 of them one after another: 7.40 ms, 6.52 ms with this kernel
// using a barrier per step and one chain per substitution sum.)
constexpr int kDiagThreads = 64;

__global__ __launch_bounds__(kDiagThreads) void k_chol_diag(float* A, int K, int kb, float* Linv, float* misc) {
    __shared__ float T[kCB][kCB + 1];  // the block (rows loaded coalesced), then L
    __shared__ float colv[2][kCB];     // column c of S at step c (two buffers: one barrier per step)
    __shared__ float rcp[kCB];         // 1 / L[c][c]
    const int r = threadIdx.x;
    const int o = kb * kCB;
    const int n = K - o < kCB ? K - o : kCB;
    for (int rr = 0; rr < kCB; ++rr)  // coalesced: lane r reads column r of row rr
        T[rr][r] = (rr < n && r < n) ? A[(int64_t)(o + rr) * K + o + r] : (rr == r ? 1.f : 0.f);
    __syncthreads();
    float a[kCB];
#pragma unroll
    for (int q = 0; q < kCB; ++q) a[q] = T[r][q];
    float piv = 1.f;  // this lane's pivot S[r][r] at step r
#pragma unroll
    for (int c = 0; c < kCB; ++c) {
        colv[c & 1][r] = a[c];
        // one wave: its LDS operations complete in order, so the reads below see every lane's
        // write without a barrier (this only keeps the compiler from moving them across)
        __builtin_amdgcn_wave_barrier();
        float p = colv[c & 1][c];
        if (r == c) piv = p;
        if (!(p > 0.f)) p = 1e-30f;  // not positive definite in fp32: flagged below
        const float m = a[c] / p;
#pragma unroll
        for (int q = c + 1; q < kCB; ++q) a[q] = fmaf(-m, colv[c & 1][q], a[q]);
    }
    if (!(piv > 0.f)) misc[1] = 1.f;  // keep going with a tiny pivot
    const float root = sqrtf(piv > 0.f ? piv : 1e-30f);
    rcp[r] = 1.f / root;
    __syncthreads();
    // L: row r is S[r][c] / root_c below the diagonal, root_r on it, 0 above
#pragma unroll
    for (int c = 0; c < kCB; ++c) T[r][c] = c < r ? a[c] * rcp[c] : (c == r ? root : 0.f);
    __syncthreads();
    for (int rr = 0; rr < kCB; ++rr)  // coalesced write-back of the lower triangle
        if (rr < n && r < n && r <= rr) A[(int64_t)(o + rr) * K + o + r] = T[rr][r];
    // Z = L^-1, column j = r: z_i = (delta_ij - sum_{k<i} L[i][k] z_k) / L[i][i]
    float z[kCB];
#pragma unroll
    for (int i = 0; i < kCB; ++i) {
        float t[4] = {i == r ? 1.f : 0.f, 0.f, 0.f, 0.f};  // four chains of the sum
#pragma unroll
        for (int k = 0; k < i; ++k) t[k & 3] = fmaf(-T[i][k], z[k], t[k & 3]);
        z[i] = ((t[0] + t[1]) + (t[2] + t[3])) * rcp[i];
    }
#pragma unroll
    for (int i = 0; i < kCB; ++i) Linv[(int64_t)kb * kCB * kCB + i * kCB + r] = z[i];  // 0 above the diagonal
}

// Block rows i = kb + 1 + blockIdx.x: L_ik = A_ik Linv_kk^T.
__global__ __launch_bounds__(256) void k_chol_panel(float* A, int K, int kb, const float* Linv) {
    __shared__ float S[kCB][kCB + 1];  // A_ik
    __shared__ float V[kCB][kCB + 1];  // Linv_kk
    const int tid = threadIdx.x;
    const int ib = kb + 1 + blockIdx.x;
    const int ro = ib * kCB, co = kb * kCB;
    const int nr = K - ro < kCB ? K - ro : kCB;
    for (int e = tid; e < kCB * kCB; e += 256) {
        const int r = e / kCB, c = e % kCB;
        S[r][c] = (r < nr) ? A[(int64_t)(ro + r) * K + co + c] : 0.f;  // co + c < K: block kb is full
        V[r][c] = Linv[(int64_t)kb * kCB * kCB + e];
    }
    __syncthreads();
    // thread: rows r = 4 (tid / 16) .. +3, columns c = tid % 16 + 16 q
    const int r0 = 4 * (tid >> 4), c0 = tid & 15;
    float out[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) out[a][b] = 0.f;
    for (int m = 0; m < kCB; ++m) {
        float s[4], v[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) s[a] = S[r0 + a][m];
#pragma unroll
        for (int b = 0; b < 4; ++b) v[b] = V[c0 + 16 * b][m];  // Linv[c][m]: (Linv^T)[m][c]
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) out[a][b] += s[a] * v[b];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (r0 + a < nr) A[(int64_t)(ro + r0 + a) * K + co + c0 + 16 * b] = out[a][b];
}

// Trailing update: block pair number blockIdx.x over the lower triangle of the blocks after
// kb (i >= j), A_ij -= L_ik L_jk^T.
__global__ __launch_bounds__(256) void k_chol_update(float* A, int K, int kb) {
    __shared__ float P[kCB][kCB + 1];  // L_ik
    __shared__ float Q[kCB][kCB + 1];  // L_jk
    const int tid = threadIdx.x;
    // pair index -> (ii, jj) with 0 <= jj <= ii (row-major over the lower triangle)
    const int64_t p = blockIdx.x;
    int ii = (int)((sqrt(8.0 * (double)p + 1.0) - 1.0) / 2.0);
    while ((int64_t)(ii + 1) * (ii + 2) / 2 <= p) ++ii;
    while ((int64_t)ii * (ii + 1) / 2 > p) --ii;
    const int jj = (int)(p - (int64_t)ii * (ii + 1) / 2);
    const int ib = kb + 1 + ii, jb = kb + 1 + jj;
    const int ro = ib * kCB, jo = jb * kCB, co = kb * kCB;
    const int nr = K - ro < kCB ? K - ro : kCB;
    const int nc = K - jo < kCB ? K - jo : kCB;
    for (int e = tid; e < kCB * kCB; e += 256) {
        const int r = e / kCB, c = e % kCB;
        P[r][c] = (r < nr) ? A[(int64_t)(ro + r) * K + co + c] : 0.f;
        Q[r][c] = (r < nc) ? A[(int64_t)(jo + r) * K + co + c] : 0.f;
    }
    __syncthreads();
    const int r0 = 4 * (tid >> 4), c0 = tid & 15;
    float out[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) out[a][b] = 0.f;
    for (int m = 0; m < kCB; ++m) {
        float s[4], v[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) s[a] = P[r0 + a][m];
#pragma unroll
        for (int b = 0; b < 4; ++b) v[b] = Q[c0 + 16 * b][m];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) out[a][b] += s[a] * v[b];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int r = r0 + a, c = c0 + 16 * b;
            if (r < nr && c < nc) A[(int64_t)(ro + r) * K + jo + c] -= out[a][b];
        }
}

// The triangular solve L Z = I for the inverse's diagonal d_j = sum_i Z[i][j]^2, right-looking
// by block rows so that each step is one launch of independent 64 x 64 block products:
//   step r: Z_rc = Linv_r B_rc for c <= r (B_rr = I: Z_rr = Linv_r), then
//           B_ic -= L_ir Z_rc for every i > r, c <= r.
// B and Z share the scratch blocks (lower block triangle, block (i, c) at z_offset(c) + (i - c)
// blocks), zero-filled first. Rows and columns past K: zero rows of L, identity padding of Linv.
__host__ __device__ inline int64_t z_offset(int64_t c, int64_t K) {
    const int64_t Kp = (K + kCB - 1) / kCB * kCB;
    return (int64_t)kCB * (c * Kp - (int64_t)kCB * c * (c - 1) / 2);
}
__device__ __forceinline__ float* z_block(float* Zs, int i, int c, int K) {
    return Zs + z_offset(c, K) + (int64_t)(i - c) * kCB * kCB;
}

__global__ __launch_bounds__(256) void k_zero(float* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// 64 x 64 x 64 product in LDS by 256 threads (4 x 4 outputs each): out[r][c] = sum_q P[r][q] Q[q][c].
__device__ __forceinline__ void block_mm(float (*P)[kCB + 1], float (*Q)[kCB + 1], float out[4][4]) {
    const int tid = threadIdx.x;
    const int r0 = 4 * (tid >> 4), c0 = tid & 15;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) out[a][b] = 0.f;
    for (int q = 0; q < kCB; ++q) {
        float p[4], v[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) p[a] = P[r0 + a][q];
#pragma unroll
        for (int b = 0; b < 4; ++b) v[b] = Q[q][c0 + 16 * b];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) out[a][b] += p[a] * v[b];
    }
}

// Step r, part 1: workgroup c (0..r) forms Z_rc = Linv_r B_rc (Z_rr = Linv_r).
__global__ __launch_bounds__(256) void k_trsm_row(const float* Linv, float* Zs, int K, int r) {
    __shared__ float P[kCB][kCB + 1];
    __shared__ float Q[kCB][kCB + 1];
    const int tid = threadIdx.x;
    const int c = blockIdx.x;
    float* Z = z_block(Zs, r, c, K);
    const float* Li = Linv + (int64_t)r * kCB * kCB;
    if (c == r) {
        for (int e = tid; e < kCB * kCB; e += 256) Z[e] = Li[e];
        return;
    }
    for (int e = tid; e < kCB * kCB; e += 256) {
        P[e / kCB][e % kCB] = Li[e];
        Q[e / kCB][e % kCB] = Z[e];
    }
    __syncthreads();
    float out[4][4];
    block_mm(P, Q, out);
    const int r0 = 4 * (tid >> 4), c0 = tid & 15;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) Z[(r0 + a) * kCB + c0 + 16 * b] = out[a][b];
}

// Step r, part 2: workgroup (i - r - 1, c) for i > r, c <= r: B_ic -= L_ir Z_rc.
__global__ __launch_bounds__(256) void k_trsm_update(const float* A, float* Zs, int K, int r) {
    __shared__ float P[kCB][kCB + 1];
    __shared__ float Q[kCB][kCB + 1];
    const int tid = threadIdx.x;
    const int i = r + 1 + blockIdx.x, c = blockIdx.y;
    const int ro = i * kCB, co = r * kCB;  // L_ir: rows of block i, columns of block r (full)
    const int nr = K - ro < kCB ? K - ro : kCB;
    const float* Zr = z_block(Zs, r, c, K);
    for (int e = tid; e < kCB * kCB; e += 256) {
        const int rr = e / kCB, cc = e % kCB;
        P[rr][cc] = rr < nr ? A[(int64_t)(ro + rr) * K + co + cc] : 0.f;
        Q[rr][cc] = Zr[e];
    }
    __syncthreads();
    float out[4][4];
    block_mm(P, Q, out);
    float* B = z_block(Zs, i, c, K);
    const int r0 = 4 * (tid >> 4), c0 = tid & 15;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) B[(r0 + a) * kCB + c0 + 16 * b] -= out[a][b];
}

constexpr int kSplit = 16;  // partial sums per column in the norm and rank passes

// Partial column norms: workgroup (c, g) sums the squares of column block c of Z over the block
// rows i = c + g, c + g + kSplit, ... into aux[g][j].
__global__ __launch_bounds__(256) void k_colnorm(const float* Zs, int K, float* aux) {
    __shared__ float part[4][kCB];
    const int tid = threadIdx.x;
    const int c = blockIdx.x, g = blockIdx.y;
    const int nblk = (K + kCB - 1) / kCB;
    const int col = tid & 63, rg = tid >> 6;  // 4 row groups of 16 rows
    float s = 0.f;
    for (int i = c + g; i < nblk; i += kSplit) {
        const float* Z = Zs + z_offset(c, K) + (int64_t)(i - c) * kCB * kCB;
        const int nr = K - i * kCB < kCB ? K - i * kCB : kCB;
        for (int rr = rg * 16; rr < rg * 16 + 16; ++rr)
            if (rr < nr) {
                const float v = Z[rr * kCB + col];
                s += v * v;
            }
    }
    part[rg][col] = s;
    __syncthreads();
    if (tid < kCB) {
        const int j = c * kCB + tid;
        if (j < K) aux[(int64_t)g * K + j] = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]);
    }
}

__global__ __launch_bounds__(256) void k_colnorm_finish(const float* aux, int K, float* d) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= K) return;
    float s = 0.f;
    for (int g = 0; g < kSplit; ++g) s += aux[(int64_t)g * K + j];
    d[j] = s;
}

// score: column sums of W^2 over row chunks, then score_j = sum / d_j^2.
constexpr int kSChunk = 64;
__global__ __launch_bounds__(256) void k_score_part(const float* W, int N, int K, float* part) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    const int c = blockIdx.y;
    const int r0 = c * kSChunk, r1 = r0 + kSChunk < N ? r0 + kSChunk : N;
    if (j >= K) return;
    float s = 0.f;
    for (int r = r0; r < r1; ++r) {
        const float v = W[(int64_t)r * K + j];
        s += v * v;
    }
    part[(int64_t)c * K + j] = s;
}

__global__ __launch_bounds__(256) void k_score_finish(const float* part, int chunks, int K, const float* d,
                                                      float* score) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= K) return;
    // four independent sums so the loads of the partials overlap, added in a fixed order
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    int c = 0;
    for (; c + 3 < chunks; c += 4) {
        s0 += part[(int64_t)c * K + j];
        s1 += part[(int64_t)(c + 1) * K + j];
        s2 += part[(int64_t)(c + 2) * K + j];
        s3 += part[(int64_t)(c + 3) * K + j];
    }
    for (; c < chunks; ++c) s0 += part[(int64_t)c * K + j];
    const float s = (s0 + s1) + (s2 + s3);
    score[j] = s / (d[j] * d[j]);
}

// Partial ranks: workgroup (bx, g) counts, for its 256 scores j, the i in slice g of [0, K) with
// score_i > score_j, or equal with i < j; the rank of j is the sum over the kSplit slices.
__global__ __launch_bounds__(256) void k_rank(const float* score, int K, int* cnt) {
    __shared__ float tile[256];
    const int j = blockIdx.x * 256 + threadIdx.x;
    const int g = blockIdx.y;
    const int per = (K + kSplit - 1) / kSplit;
    const int b0 = g * per, b1 = b0 + per < K ? b0 + per : K;
    const float v = j < K ? score[j] : 0.f;
    int rank = 0;
    for (int t0 = b0; t0 < b1; t0 += 256) {
        __syncthreads();
        tile[threadIdx.x] = t0 + (int)threadIdx.x < b1 ? score[t0 + threadIdx.x] : 0.f;
        __syncthreads();
        const int n = b1 - t0 < 256 ? b1 - t0 : 256;
        for (int q = 0; q < n; ++q) {
            const float u = tile[q];
            rank += (u > v || (u == v && t0 + q < j)) ? 1 : 0;
        }
    }
    if (j < K) cnt[(int64_t)g * K + j] = rank;
}

// One workgroup of 1024 threads: idx = the selected columns in ascending order (at most s of
// them: ranks are distinct for any scores that compare, so exactly s are selected; NaN scores,
// which compare with nothing, can break that, and then misc[1] is set to 2).
// sel[j] = rank_j < s, the rank being the sum of the kSplit partial counts (in place: rk[j]
// holds the flag afterwards).
__global__ __launch_bounds__(256) void k_rank_finish(int* rk, int K, int s) {
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= K) return;
    int r = 0;
    for (int g = 0; g < kSplit; ++g) r += rk[(int64_t)g * K + j];
    rk[j] = r < s ? 1 : 0;
}

__global__ __launch_bounds__(1024) void k_select(const int* sel, int K, int s, int32_t* idx, float* misc) {
    __shared__ int cnt[1024];
    const int tid = threadIdx.x;
    const int per = (K + 1023) / 1024;
    const int b = tid * per, e = b + per < K ? b + per : K;
    auto selected = [&](int j) { return sel[j]; };
    int c = 0;
    for (int j = b; j < e; ++j) c += selected(j);
    cnt[tid] = c;
    __syncthreads();
    // exclusive scan over the 1024 counts (Hillis-Steele on a copy)
    for (int off = 1; off < 1024; off <<= 1) {
        const int v = tid >= off ? cnt[tid - off] : 0;
        __syncthreads();
        cnt[tid] += v;
        __syncthreads();
    }
    int pos = cnt[tid] - c;
    for (int j = b; j < e; ++j)
        if (selected(j) && pos < s) idx[pos++] = j;
    if (tid == 1023 && cnt[1023] != s) misc[1] = 2.f;
}

}  // namespace

hipError_t launch_gram(const void* x, int T, int K, float scale, float* H, hipStream_t s) {
    const int64_t nt = (K + kGT - 1) / kGT;
    const int pairs = (K % 2 == 0 && (reinterpret_cast<uintptr_t>(x) & 3u) == 0) ? 1 : 0;
    hipLaunchKernelGGL(k_gram, dim3((unsigned)(nt * (nt + 1) / 2)), dim3(256), 0, s, (const __half*)x, T, K, pairs,
                       scale, H);
    return hipGetLastError();
}

int64_t saliency_workspace_floats(int64_t N, int64_t K) {
    const int64_t nblk = ceil_div(K, kCB);
    const int64_t chunks = ceil_div(N, kSChunk);
    return 16 + nblk * kCB * kCB + z_offset(nblk, K) + chunks * K + kSplit * K;
}

hipError_t launch_saliency(float* H, int K, float damp, const float* W, int N, int s, float* d, float* score,
                           int32_t* idx, float* ws, hipStream_t st) {
    const int nblk = (K + kCB - 1) / kCB;
    const int chunks = (N + kSChunk - 1) / kSChunk;
    float* misc = ws;
    float* Linv = ws + 16;
    float* Z = Linv + (int64_t)nblk * kCB * kCB;
    float* part = Z + z_offset(nblk, K);
    float* aux = part + (int64_t)chunks * K;  // kSplit x K: norm partials, then rank partials
    int* rk = reinterpret_cast<int*>(aux);
    hipLaunchKernelGGL(k_damp, dim3(1), dim3(256), 0, st, H, K, damp, misc);
    for (int kb = 0; kb < nblk; ++kb) {
        hipLaunchKernelGGL(k_chol_diag, dim3(1), dim3(kDiagThreads), 0, st, H, K, kb, Linv, misc);
        const int m = nblk - kb - 1;
        if (m > 0) {
            hipLaunchKernelGGL(k_chol_panel, dim3(m), dim3(256), 0, st, H, K, kb, Linv);
            hipLaunchKernelGGL(k_chol_update, dim3((unsigned)((int64_t)m * (m + 1) / 2)), dim3(256), 0, st, H, K, kb);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t zn = z_offset(nblk, K);
    hipLaunchKernelGGL(k_zero, dim3((unsigned)((zn + 255) / 256)), dim3(256), 0, st, Z, zn);
    for (int r = 0; r < nblk; ++r) {
        hipLaunchKernelGGL(k_trsm_row, dim3(r + 1), dim3(256), 0, st, Linv, Z, K, r);
        if (r + 1 < nblk)
            hipLaunchKernelGGL(k_trsm_update, dim3(nblk - r - 1, r + 1), dim3(256), 0, st, H, Z, K, r);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_colnorm, dim3(nblk, kSplit), dim3(256), 0, st, Z, K, aux);
    hipLaunchKernelGGL(k_colnorm_finish, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, aux, K, d);
    const unsigned cb = (unsigned)((K + 255) / 256);
    hipLaunchKernelGGL(k_score_part, dim3(cb, chunks), dim3(256), 0, st, W, N, K, part);
    hipLaunchKernelGGL(k_score_finish, dim3(cb), dim3(256), 0, st, part, chunks, K, d, score);
    hipLaunchKernelGGL(k_rank, dim3(cb, kSplit), dim3(256), 0, st, score, K, rk);
    hipLaunchKernelGGL(k_rank_finish, dim3(cb), dim3(256), 0, st, rk, K, s);
    hipLaunchKernelGGL(k_select, dim3(1), dim3(1024), 0, st, rk, K, s, idx, misc);
    return hipGetLastError();
}

}  // namespace ubw
