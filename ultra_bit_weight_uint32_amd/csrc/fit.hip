// Offline fit of the decoupled row-column decomposition from a dense matrix (load time, before
// the GEMV path): residual sign binarization with alternating least squares for the two scale
// vectors of each base.
//
// "FluxBin" technical summary, "1. Algorithm innovation": each base is
// (alpha_r alpha_c^T) (.) B with B in {-1,+1}, and W is approximated by the sum of the bases.
// The page gives the form, not the fit; the fit here is the plainest one:
//   R = W; per base: B = sign(R) (+1 where R >= 0), A = |R| = R (.) B;
//   alpha_r = row means of A, alpha_c = 1; then `iters` rounds of
//   alpha_c = A^T alpha_r / |alpha_r|^2, alpha_r = A alpha_c / |alpha_c|^2
//   (each the exact least-squares solution for one vector with the other fixed);
//   R -= (alpha_r alpha_c^T) (.) B.
//
// Every pass streams R once (HBM-bound): a row pass (one workgroup per row) that applies the
// previous base's update, writes the new signs as canonical bits (one wave ballot per 64
// columns) and the row means; a column pass in row chunks writing partial column sums, a small
// pass that finishes them into alpha_c; a row pass for alpha_r. Sums are in fp32 in a fixed
// order (no atomics), so the fit is deterministic.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ubw_internal.h"

namespace ubw {

namespace {

constexpr int kFitThreads = 256;

__device__ __forceinline__ float load_w(const float* w, int64_t i) { return w[i]; }
__device__ __forceinline__ float load_w(const __half* w, int64_t i) { return __half2float(w[i]); }

// Sum over the workgroup (256 threads = 4 waves); every thread gets the total.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    const int wv = threadIdx.x >> 6;
    __syncthreads();  // red may still be read from a previous call
    if ((threadIdx.x & 63) == 0) red[wv] = v;
    __syncthreads();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

enum { kRowsFirst = 0, kRowsNext = 1, kRowsFinal = 2 };

// One workgroup per row r.
//   kRowsFirst: R = W.                                      Then signs + row mean.
//   kRowsNext:  R -= ar_prev[r] ac_prev[j] sign(R).         Then signs + row mean.
//   kRowsFinal: R -= ar_prev[r] ac_prev[j] sign(R).         Nothing else.
// Signs go to bits [N][kw] (canonical: column j at word j / 32, bit j % 32; bits >= K zero),
// the row mean of |R| to ar_out[r].
template <typename WT>
__global__ __launch_bounds__(kFitThreads) void k_fit_rows(const WT* w, float* R, int N, int K, int kw, int mode,
                                                          const float* ar_prev, const float* ac_prev,
                                                          uint32_t* bits, float* ar_out) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int64_t row = (int64_t)r * K;
    const float a = mode == kRowsFirst ? 0.f : ar_prev[r];
    float s = 0.f;
    for (int j0 = 0; j0 < K; j0 += kFitThreads) {
        const int j = j0 + tid;
        const bool valid = j < K;
        float v = 0.f;
        if (valid) {
            if (mode == kRowsFirst) {
                v = load_w(w, row + j);
            } else {
                v = R[row + j];
                v -= a * ac_prev[j] * (v >= 0.f ? 1.f : -1.f);
            }
            R[row + j] = v;
            s += fabsf(v);
        }
        if (mode != kRowsFinal) {
            const uint64_t m = __ballot(valid && v >= 0.f);
            const int c0 = j0 + 64 * wv;  // first column of this wave
            if (lane == 0 && c0 < K) bits[(int64_t)r * kw + c0 / 32] = (uint32_t)m;
            if (lane == 32 && c0 + 32 < K) bits[(int64_t)r * kw + c0 / 32 + 1] = (uint32_t)(m >> 32);
        }
    }
    if (mode == kRowsFinal) return;
    s = block_sum(s, red);
    if (tid == 0) ar_out[r] = s / (float)K;
}

// Partial column sums over a chunk of kFitChunk rows: part[c][j] = sum_r |R[r][j]| ar[r];
// the first column block also writes sq[c] = sum_r ar[r]^2 over the chunk.
constexpr int kFitChunk = 64;
__global__ __launch_bounds__(kFitThreads) void k_fit_colsum(const float* R, int N, int K, const float* ar,
                                                            float* part, float* sq) {
    __shared__ float red[4];
    const int j = blockIdx.x * kFitThreads + threadIdx.x;
    const int c = blockIdx.y;
    const int r0 = c * kFitChunk;
    const int r1 = r0 + kFitChunk < N ? r0 + kFitChunk : N;
    float acc = 0.f;
    if (j < K) {
        for (int r = r0; r < r1; ++r) acc += fabsf(R[(int64_t)r * K + j]) * ar[r];
        part[(int64_t)c * K + j] = acc;
    }
    if (blockIdx.x == 0) {
        const int r = r0 + (int)threadIdx.x;
        const float q = (threadIdx.x < kFitChunk && r < r1) ? ar[r] * ar[r] : 0.f;
        const float t = block_sum(q, red);
        if (threadIdx.x == 0) sq[c] = t;
    }
}

// alpha_c[j] = sum_c part[c][j] / sum_c sq[c] (0 when the denominator is 0); each workgroup
// also writes sqc[b] = sum of alpha_c^2 over its kFinCols columns. A workgroup takes 64
// columns (one per lane); its 4 waves split the chunks, each with 4 independent sums so that
// the loads overlap, and the wave sums are added in a fixed order.
constexpr int kFinCols = 64;
__global__ __launch_bounds__(kFitThreads) void k_fit_colfinish(const float* part, const float* sq, int chunks,
                                                               int K, float* ac, float* sqc) {
    __shared__ float red[4];
    __shared__ float colp[4][kFinCols];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int j = blockIdx.x * kFinCols + lane;
    float d = 0.f;
    for (int c = threadIdx.x; c < chunks; c += kFitThreads) d += sq[c];
    const float den = block_sum(d, red);
    float n0 = 0.f, n1 = 0.f, n2 = 0.f, n3 = 0.f;
    if (j < K) {
        int c = wv;
        for (; c + 12 < chunks; c += 16) {
            n0 += part[(int64_t)c * K + j];
            n1 += part[(int64_t)(c + 4) * K + j];
            n2 += part[(int64_t)(c + 8) * K + j];
            n3 += part[(int64_t)(c + 12) * K + j];
        }
        for (; c < chunks; c += 4) n0 += part[(int64_t)c * K + j];
    }
    colp[wv][lane] = (n0 + n1) + (n2 + n3);
    __syncthreads();
    float v = 0.f;
    if (wv == 0 && j < K) {
        const float num = (colp[0][lane] + colp[1][lane]) + (colp[2][lane] + colp[3][lane]);
        v = den > 0.f ? num / den : 0.f;
        ac[j] = v;
    }
    const float t = block_sum(v * v, red);
    if (threadIdx.x == 0) sqc[blockIdx.x] = t;
}

// alpha_r[r] = sum_j |R[r][j]| ac[j] / sum_b sqc[b] (0 when the denominator is 0); the
// denominator's partials are read by all threads at once and added in the same tree order
// in every workgroup.
__global__ __launch_bounds__(kFitThreads) void k_fit_rowals(const float* R, int K, const float* ac,
                                                            const float* sqc, int cblocks, float* ar) {
    __shared__ float red[4];
    const int r = blockIdx.x;
    const int64_t row = (int64_t)r * K;
    float s = 0.f;
    for (int j = threadIdx.x; j < K; j += kFitThreads) s += fabsf(R[row + j]) * ac[j];
    s = block_sum(s, red);
    float dp = 0.f;
    for (int b = threadIdx.x; b < cblocks; b += kFitThreads) dp += sqc[b];
    const float den = block_sum(dp, red);
    if (threadIdx.x == 0) ar[r] = den > 0.f ? s / den : 0.f;
}

__global__ void k_fit_ones(float* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 1.f;
}

template <typename WT>
hipError_t fit_t(const WT* w, int N, int K, int nb, int iters, uint32_t* bits, float* alpha_r, float* alpha_c,
                 float* R, float* ws, hipStream_t s) {
    const int kw = (K + 31) / 32;
    const int chunks = (N + kFitChunk - 1) / kFitChunk;
    const int cblocks = (K + kFitThreads - 1) / kFitThreads;
    const int fblocks = (K + kFinCols - 1) / kFinCols;
    float* part = ws;
    float* sq = part + (int64_t)chunks * K;
    float* sqc = sq + chunks;
    for (int k = 0; k < nb; ++k) {
        float* ar = alpha_r + (int64_t)k * N;
        float* ac = alpha_c + (int64_t)k * K;
        const float* arp = k ? alpha_r + (int64_t)(k - 1) * N : nullptr;
        const float* acp = k ? alpha_c + (int64_t)(k - 1) * K : nullptr;
        hipLaunchKernelGGL(k_fit_rows<WT>, dim3(N), dim3(kFitThreads), 0, s, w, R, N, K, kw,
                           k ? (int)kRowsNext : (int)kRowsFirst, arp, acp, bits + (int64_t)k * N * kw, ar);
        hipLaunchKernelGGL(k_fit_ones, dim3(cblocks), dim3(kFitThreads), 0, s, ac, K);
        for (int it = 0; it < iters; ++it) {
            hipLaunchKernelGGL(k_fit_colsum, dim3(cblocks, chunks), dim3(kFitThreads), 0, s, R, N, K, ar, part, sq);
            hipLaunchKernelGGL(k_fit_colfinish, dim3(fblocks), dim3(kFitThreads), 0, s, part, sq, chunks, K, ac, sqc);
            hipLaunchKernelGGL(k_fit_rowals, dim3(N), dim3(kFitThreads), 0, s, R, K, ac, sqc, fblocks, ar);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_fit_rows<WT>, dim3(N), dim3(kFitThreads), 0, s, w, R, N, K, kw, (int)kRowsFinal,
                       alpha_r + (int64_t)(nb - 1) * N, alpha_c + (int64_t)(nb - 1) * K, bits, alpha_r);
    return hipGetLastError();
}

}  // namespace

int64_t fit_workspace_floats(int64_t N, int64_t K) {
    const int64_t chunks = ceil_div(N, kFitChunk);
    return chunks * K + chunks + ceil_div(K, kFinCols);
}

hipError_t launch_fit(const void* w, int w_dtype, int N, int K, int nb, int iters, uint32_t* bits, float* alpha_r,
                      float* alpha_c, float* residual, float* ws, hipStream_t s) {
    if (w_dtype == UBW_F16)
        return fit_t((const __half*)w, N, K, nb, iters, bits, alpha_r, alpha_c, residual, ws, s);
    return fit_t((const float*)w, N, K, nb, iters, bits, alpha_r, alpha_c, residual, ws, s);
}

}  // namespace ubw
