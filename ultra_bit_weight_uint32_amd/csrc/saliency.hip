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
//   k_gram         H = scale X^T X on the matrix cores (v_mfma_f32_32x32x8f16): the one dense
//                  contraction of the method. 128 x 128 tiles of H per workgroup, 32 rows of X
//                  per step staged through LDS transposed so that each lane's 4 consecutive
//                  k values are one 8-byte LDS read.
//   k_damp         lambda from the diagonal, added to it.
//   k_chol_diag    Cholesky of one 64 x 64 diagonal block in LDS, and the inverse of that
//                  factor (kept for the panel and for the inverse's diagonal).
//   k_chol_panel   L_ik = A_ik L_kk^-T for the block rows below.
//   k_chol_update  A_ij -= L_ik L_jk^T for the trailing lower blocks.
//   k_inv_diag     one workgroup per 64-column block k solves L Z = E_k (rows >= 64 k) block
//                  row by block row and sums the squares of Z's columns: d_j = ||L^-1 e_j||^2.
//   k_score_part / k_score_finish   column sums of W^2 in row chunks, then score = sum / d^2.
//   k_rank         rank of every score (count of larger scores, equal ones at lower indices).
//   k_select       the columns of rank < s, ascending, by one prefix scan.
// Everything after the Gram matrix is fp32 vector arithmetic in a fixed order.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "ubw_internal.h"

namespace ubw {

namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr int kGT = 128;  // H tile per workgroup
constexpr int kGS = 32;   // rows of X per step
constexpr int kGP = 8;    // LDS row padding (halves)

__global__ __launch_bounds__(256) void k_gram(const __half* __restrict__ X, int T, int K, float scale,
                                              float* __restrict__ H) {
    __shared__ __align__(16) _Float16 sA[kGT][kGS + kGP];  // X[t0 + t][i0 + i] at [i][t]
    __shared__ __align__(16) _Float16 sB[kGT][kGS + kGP];  // X[t0 + t][j0 + j] at [j][t]
    const int i0 = blockIdx.y * kGT, j0 = blockIdx.x * kGT;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wm = wv >> 1, wn = wv & 1;  // this wave's 64 x 64 quarter of the tile
    const _Float16* Xh = reinterpret_cast<const _Float16*>(X);
    float16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;
    for (int t0 = 0; t0 < T; t0 += kGS) {
        for (int e = tid; e < kGS * kGT; e += 256) {
            const int t = e / kGT, c = e % kGT;
            const bool tv = t0 + t < T;
            const int64_t rowoff = (int64_t)(t0 + t) * K;
            sA[c][t] = (tv && i0 + c < K) ? Xh[rowoff + i0 + c] : (_Float16)0;
            sB[c][t] = (tv && j0 + c < K) ? Xh[rowoff + j0 + c] : (_Float16)0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kGS; kk += 8) {
            half4_t a[2], b[2];
            const int ko = kk + 4 * (lane >> 5);
#pragma unroll
            for (int m = 0; m < 2; ++m)
                a[m] = *reinterpret_cast<const half4_t*>(&sA[wm * 64 + m * 32 + (lane & 31)][ko]);
#pragma unroll
            for (int n = 0; n < 2; ++n)
                b[n] = *reinterpret_cast<const half4_t*>(&sB[wn * 64 + n * 32 + (lane & 31)][ko]);
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x8f16(a[m], b[n], acc[m][n], 0, 0, 0);
        }
        __syncthreads();
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
                if (i < K && j < K) H[(int64_t)i * K + j] = scale * acc[m][n][v];
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

// Cholesky of diagonal block kb (lower, in LDS), written back, and its inverse to Linv[kb].
// Rows/columns past K act as an identity block.
__global__ __launch_bounds__(256) void k_chol_diag(float* A, int K, int kb, float* Linv, float* misc) {
    __shared__ float L[kCB][kCB + 1];
    __shared__ float Z[kCB][kCB + 1];
    const int tid = threadIdx.x;
    const int o = kb * kCB;
    const int n = K - o < kCB ? K - o : kCB;
    for (int e = tid; e < kCB * kCB; e += 256) {
        const int r = e / kCB, c = e % kCB;
        L[r][c] = (r < n && c < n) ? A[(int64_t)(o + r) * K + o + c] : (r == c ? 1.f : 0.f);
    }
    __syncthreads();
    for (int c = 0; c < kCB; ++c) {
        float p = L[c][c];
        if (!(p > 0.f)) {  // not positive definite in fp32: flag it, keep going with a tiny pivot
            if (tid == 0) misc[1] = 1.f;
            p = 1e-30f;
        }
        const float piv = sqrtf(p);
        __syncthreads();
        for (int r = c + 1 + tid; r < kCB; r += 256) L[r][c] /= piv;
        __syncthreads();
        if (tid == 0) L[c][c] = piv;
        // trailing update of the lower triangle: L[r][q] -= L[r][c] L[q][c], c < q <= r
        const int m = kCB - c - 1;
        for (int e = tid; e < m * m; e += 256) {
            const int r = c + 1 + e / m, q = c + 1 + e % m;
            if (q <= r) L[r][q] -= L[r][c] * L[q][c];
        }
        __syncthreads();
    }
    // inverse of the lower factor: column c by forward substitution (one thread per column)
    if (tid < kCB) {
        const int c = tid;
        for (int r = 0; r < kCB; ++r) {
            float v = (r == c) ? 1.f : 0.f;
            if (r < c) {
                Z[r][c] = 0.f;
                continue;
            }
            for (int q = c; q < r; ++q) v -= L[r][q] * Z[q][c];
            Z[r][c] = v / L[r][r];
        }
    }
    __syncthreads();
    for (int e = tid; e < kCB * kCB; e += 256) {
        const int r = e / kCB, c = e % kCB;
        if (r < n && c < n && c <= r) A[(int64_t)(o + r) * K + o + c] = L[r][c];
        Linv[(int64_t)kb * kCB * kCB + e] = Z[r][c];
    }
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

// Offset (floats) of block column k's Z in the scratch: whole 64 x 64 blocks for the block
// rows k .. nblk - 1 (K padded to whole blocks).
__host__ __device__ inline int64_t z_offset(int64_t k, int64_t K) {
    const int64_t Kp = (K + kCB - 1) / kCB * kCB;
    return (int64_t)kCB * (k * Kp - (int64_t)kCB * k * (k - 1) / 2);
}

// Block column k = blockIdx.x: Z_i = Linv_i (delta_ik I - sum_{k <= m < i} L_im Z_m) for the
// block rows i >= k, then d_j = sum over those rows of Z[.][j]^2 for the 64 columns of block k.
__global__ __launch_bounds__(256) void k_inv_diag(const float* A, int K, const float* Linv, float* Zs, float* d) {
    __shared__ float S[kCB][kCB + 1];
    __shared__ float M[kCB][kCB + 1];
    const int tid = threadIdx.x;
    const int kb = blockIdx.x;
    const int nblk = (K + kCB - 1) / kCB;
    float* Z = Zs + z_offset(kb, K);  // Z_i at rows (i - kb) * 64 .. , 64 columns, row-major
    const int r0 = 4 * (tid >> 4), c0 = tid & 15;
    float dsum[4] = {0.f, 0.f, 0.f, 0.f};  // columns c0 + 16 b, rows r0 .. r0 + 3 of every block
    for (int ib = kb; ib < nblk; ++ib) {
        const int ro = ib * kCB;
        const int nr = K - ro < kCB ? K - ro : kCB;
        float acc[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = (ib == kb && r0 + a == c0 + 16 * b) ? 1.f : 0.f;
        for (int mb = kb; mb < ib; ++mb) {
            const int mo = mb * kCB;
            __syncthreads();
            for (int e = tid; e < kCB * kCB; e += 256) {
                const int r = e / kCB, c = e % kCB;
                S[r][c] = (r < nr) ? A[(int64_t)(ro + r) * K + mo + c] : 0.f;  // L_im (block mb is full)
                M[r][c] = Z[(int64_t)(mb - kb) * kCB * kCB + e];                 // Z_m
            }
            __syncthreads();
            for (int q = 0; q < kCB; ++q) {
                float s[4], z[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) s[a] = S[r0 + a][q];
#pragma unroll
                for (int b = 0; b < 4; ++b) z[b] = M[q][c0 + 16 * b];
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b) acc[a][b] -= s[a] * z[b];
            }
        }
        // Z_i = Linv_i acc: stage acc in S, Linv_i in M
        __syncthreads();
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) S[r0 + a][c0 + 16 * b] = acc[a][b];
        for (int e = tid; e < kCB * kCB; e += 256) M[e / kCB][e % kCB] = Linv[(int64_t)ib * kCB * kCB + e];
        __syncthreads();
        float z[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) z[a][b] = 0.f;
        for (int q = 0; q < kCB; ++q) {
            float l[4], s[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) l[a] = M[r0 + a][q];
#pragma unroll
            for (int b = 0; b < 4; ++b) s[b] = S[q][c0 + 16 * b];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) z[a][b] += l[a] * s[b];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float v = (r0 + a < nr) ? z[a][b] : 0.f;  // rows past K: identity padding
                Z[(int64_t)(ib - kb) * kCB * kCB + (r0 + a) * kCB + c0 + 16 * b] = v;
                dsum[b] += v * v;
            }
    }
    // sum dsum over the 16 row groups of threads sharing a column
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 4; ++b) S[tid >> 4][c0 + 16 * b] = dsum[b];
    __syncthreads();
    if (tid < kCB) {
        float t = 0.f;
        for (int g = 0; g < 16; ++g) t += S[g][tid];
        const int j = kb * kCB + tid;
        if (j < K) d[j] = t;
    }
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
    float s = 0.f;
    for (int c = 0; c < chunks; ++c) s += part[(int64_t)c * K + j];
    score[j] = s / (d[j] * d[j]);
}

// rank[j] = #{i : score_i > score_j} + #{i < j : score_i == score_j}; sel[j] = rank < s.
__global__ __launch_bounds__(256) void k_rank(const float* score, int K, int s, int* sel) {
    __shared__ float tile[256];
    const int j = blockIdx.x * 256 + threadIdx.x;
    const float v = j < K ? score[j] : 0.f;
    int rank = 0;
    for (int t0 = 0; t0 < K; t0 += 256) {
        __syncthreads();
        tile[threadIdx.x] = t0 + (int)threadIdx.x < K ? score[t0 + threadIdx.x] : 0.f;
        __syncthreads();
        const int n = K - t0 < 256 ? K - t0 : 256;
        for (int q = 0; q < n; ++q) {
            const float u = tile[q];
            rank += (u > v || (u == v && t0 + q < j)) ? 1 : 0;
        }
    }
    if (j < K) sel[j] = rank < s ? 1 : 0;
}

// One workgroup of 1024 threads: idx = the selected columns in ascending order (at most s of
// them: ranks are distinct for any scores that compare, so exactly s are selected; NaN scores,
// which compare with nothing, can break that, and then misc[1] is set to 2).
__global__ __launch_bounds__(1024) void k_select(const int* sel, int K, int s, int32_t* idx, float* misc) {
    __shared__ int cnt[1024];
    const int tid = threadIdx.x;
    const int per = (K + 1023) / 1024;
    const int b = tid * per, e = b + per < K ? b + per : K;
    int c = 0;
    for (int j = b; j < e; ++j) c += sel[j];
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
        if (sel[j] && pos < s) idx[pos++] = j;
    if (tid == 1023 && cnt[1023] != s) misc[1] = 2.f;
}

}  // namespace

hipError_t launch_gram(const void* x, int T, int K, float scale, float* H, hipStream_t s) {
    const unsigned g = (unsigned)((K + kGT - 1) / kGT);
    hipLaunchKernelGGL(k_gram, dim3(g, g), dim3(256), 0, s, (const __half*)x, T, K, scale, H);
    return hipGetLastError();
}

int64_t saliency_workspace_floats(int64_t N, int64_t K) {
    const int64_t nblk = ceil_div(K, kCB);
    const int64_t chunks = ceil_div(N, kSChunk);
    return 16 + nblk * kCB * kCB + z_offset(nblk, K) + chunks * K + K;
}

hipError_t launch_saliency(float* H, int K, float damp, const float* W, int N, int s, float* d, float* score,
                           int32_t* idx, float* ws, hipStream_t st) {
    const int nblk = (K + kCB - 1) / kCB;
    const int chunks = (N + kSChunk - 1) / kSChunk;
    float* misc = ws;
    float* Linv = ws + 16;
    float* Z = Linv + (int64_t)nblk * kCB * kCB;
    float* part = Z + z_offset(nblk, K);
    int* sel = reinterpret_cast<int*>(part + (int64_t)chunks * K);
    hipLaunchKernelGGL(k_damp, dim3(1), dim3(256), 0, st, H, K, damp, misc);
    for (int kb = 0; kb < nblk; ++kb) {
        hipLaunchKernelGGL(k_chol_diag, dim3(1), dim3(256), 0, st, H, K, kb, Linv, misc);
        const int m = nblk - kb - 1;
        if (m > 0) {
            hipLaunchKernelGGL(k_chol_panel, dim3(m), dim3(256), 0, st, H, K, kb, Linv);
            hipLaunchKernelGGL(k_chol_update, dim3((unsigned)((int64_t)m * (m + 1) / 2)), dim3(256), 0, st, H, K, kb);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_inv_diag, dim3(nblk), dim3(256), 0, st, H, K, Linv, Z, d);
    const unsigned cb = (unsigned)((K + 255) / 256);
    hipLaunchKernelGGL(k_score_part, dim3(cb, chunks), dim3(256), 0, st, W, N, K, part);
    hipLaunchKernelGGL(k_score_finish, dim3(cb), dim3(256), 0, st, part, chunks, K, d, score);
    hipLaunchKernelGGL(k_rank, dim3(cb), dim3(256), 0, st, score, K, s, sel);
    hipLaunchKernelGGL(k_select, dim3(1), dim3(1024), 0, st, sel, K, s, idx, misc);
    return hipGetLastError();
}

}  // namespace ubw
