// HIP kernels for gfx950: packing, ternary encoding, LUT-BSF table build, pattern
// extraction and the table-lookup GEMV over decoupled row-column binary bases.
//
// Method: FluxBin (gist.science/ko/paper/2608.15602), technical summary, "2. Kernel
// innovation": tables with alpha_c folded in (LUT-BSF), virtual columnar mapping for the
// salient columns (VCM), and the execution flow stream packed uint32 -> extract pattern
// indices with bit operations -> fetch precomputed partial sums -> apply alpha_r.
//
// gfx950 mapping (the page's kernel targets another GPU; only its dataflow is kept):
//   - one workgroup of 256 threads owns 256-row tiles x 256-column slices; each lane owns one
//     row of a tile and walks the slice's 32 groups of 8 columns;
//   - a group table has 256 fp32 entries, all in one LDS bank (entry p of the table in
//     column x lives at byte 256 p + 4 x), duplicated in column x + 32;
//   - lane with l = lane mod 32 reads column l + t at step t, so each half-wave touches 32
//     distinct banks per lookup (the LDS serves a wave64 access as two 32-lane halves over
//     32 banks);
//   - the lookup address is one v_perm_b32 of the weight byte with the lane's column offset;
//     a v_alignbyte_b32 per 4 lookups supplies the lane's rotated byte order;
//   - no MFMA: the work is a memory-bound table-lookup reduction.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "../../include/ubw.h"
#include "ubw_internal.h"

namespace ubw {

typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) const char lds_cchar;

// ---------------------------------------------------------------------------------------
// Small helpers shared by several kernels.

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__half v) { return __half2float(v); }

// Rotation of the lane that owns tile row rho: word rotation a and byte rotation c.
__device__ __forceinline__ int rot_words(int rho) { return (rho & 31) >> 2; }
__device__ __forceinline__ int rot_bytes(int rho) { return rho & 3; }

// Address (or, with lanec = 0, 256 * pattern) of the step t = 4 i + jj lookup: byte jj of the
// aligned word A is the pattern, placed in byte 1; bytes 0 and 2 come from lanec.
template <int JJ>
__device__ __forceinline__ uint32_t perm_addr(uint32_t A, uint32_t lanec) {
    return __builtin_amdgcn_perm(A, lanec, 0x0C020400u | ((uint32_t)JJ << 8));
}

// The four patterns of steps 4i .. 4i+3 start at byte c of the slot pair (W[i], W[i+1]).
__device__ __forceinline__ uint32_t aligned_pair(uint32_t lo, uint32_t hi, uint32_t c) {
    return __builtin_amdgcn_alignbyte(hi, lo, c);
}

// LUT-BSF entries T[p0 .. p0+31] of one group of 8 columns with scaled activations v[0..7]
// (p0 a multiple of 32): T[p] = sum_i (2 bit_i(p) - 1) v[i], built as Lo[p & 15] + Hi[p >> 4]
// with Lo/Hi the 4-column half tables. Lo is built by doubling from the all-minus entry.
__device__ __forceinline__ void lut8_block(const float v[8], int p0, float T[32]) {
    const float u0 = v[0] + v[0], u1 = v[1] + v[1], u2 = v[2] + v[2], u3 = v[3] + v[3];
    float lo[16];
    lo[0] = -((v[0] + v[1]) + (v[2] + v[3]));
    lo[1] = lo[0] + u0;
    lo[2] = lo[0] + u1;
    lo[3] = lo[1] + u1;
#pragma unroll
    for (int q = 0; q < 4; ++q) lo[4 + q] = lo[q] + u2;
#pragma unroll
    for (int q = 0; q < 8; ++q) lo[8 + q] = lo[q] + u3;
    const int q0 = p0 >> 4;  // even
    const float s5 = (q0 & 2) ? v[5] : -v[5];
    const float s6 = (q0 & 4) ? v[6] : -v[6];
    const float s7 = (q0 & 8) ? v[7] : -v[7];
    const float hi0 = (s5 - v[4]) + (s6 + s7);
    const float hi1 = hi0 + (v[4] + v[4]);
#pragma unroll
    for (int pp = 0; pp < 32; ++pp) T[pp] = lo[pp & 15] + (pp < 16 ? hi0 : hi1);
}

// 4-column group table (g = 4): T[p] = sum_{i<4} (2 bit_i(p) - 1) v[i], p < 16.
__device__ __forceinline__ void lut4_table(const float v[4], float T[16]) {
    const float u0 = v[0] + v[0], u1 = v[1] + v[1], u2 = v[2] + v[2], u3 = v[3] + v[3];
    T[0] = -((v[0] + v[1]) + (v[2] + v[3]));
    T[1] = T[0] + u0;
    T[2] = T[0] + u1;
    T[3] = T[1] + u1;
#pragma unroll
    for (int q = 0; q < 4; ++q) T[4 + q] = T[q] + u2;
#pragma unroll
    for (int q = 0; q < 8; ++q) T[8 + q] = T[q] + u3;
}

// Sum over the 32 groups of one row's slice: the lane's 8 slots hold words (s + a) mod 8;
// step t reads the table in LDS column l + t at the pattern of group (t + l) mod 32.
__device__ __forceinline__ float lookup_row(lds_cchar* tb, const uint4& w0, const uint4& w1,
                                            uint32_t lanec, uint32_t c) {
    const uint32_t W[9] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w, w0.x};
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t A = aligned_pair(W[i], W[i + 1], c);
        s0 += *(const lds_f32*)(tb + perm_addr<0>(A, lanec) + 4 * (4 * i + 0));
        s1 += *(const lds_f32*)(tb + perm_addr<1>(A, lanec) + 4 * (4 * i + 1));
        s2 += *(const lds_f32*)(tb + perm_addr<2>(A, lanec) + 4 * (4 * i + 2));
        s3 += *(const lds_f32*)(tb + perm_addr<3>(A, lanec) + 4 * (4 * i + 3));
    }
    return (s0 + s1) + (s2 + s3);
}

// ---------------------------------------------------------------------------------------
// Zero fill (used before K-split atomics when the caller asks for y = result).

__global__ void k_fill_zero(float* __restrict__ y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] = 0.f;
}

// ---------------------------------------------------------------------------------------
// Packing. One thread per output word; the inverse of the tile layout described in
// ubw_internal.h.

struct PackPos {
    int k, row, wcol;  // base, matrix row, canonical word column
};

__device__ __forceinline__ PackPos pack_pos(int64_t o, int nb, int KT) {
    const int e = (int)(o & 3);
    const int rho = (int)((o >> 2) & 255);
    const int q = (int)((o >> 10) & 1);
    const int64_t rest = o >> 11;
    const int k = (int)(rest % nb);
    const int64_t tile = rest / nb;
    const int ks = (int)(tile % KT);
    const int rt = (int)(tile / KT);
    const int s = 4 * q + e;
    const int wi = (s + rot_words(rho)) & 7;
    return PackPos{k, rt * kTileRows + rho, ks * kSliceWords + wi};
}

__global__ void k_pack_canon(const uint32_t* __restrict__ src, int nb, int N, int K, int KT,
                             int64_t total, uint32_t* __restrict__ dst) {
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= total) return;
    const PackPos p = pack_pos(o, nb, KT);
    const int kw = (K + 31) >> 5;
    uint32_t val = 0;
    if (p.row < N && p.wcol < kw) {
        val = src[((int64_t)p.k * N + p.row) * kw + p.wcol];
        const int rem = K - p.wcol * 32;
        if (rem < 32) val &= (1u << rem) - 1u;
    }
    dst[o] = val;
}

__global__ void k_pack_int8(const int8_t* __restrict__ src, int nb, int N, int K, int KT, int64_t total,
                            uint32_t* __restrict__ dst) {
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= total) return;
    const PackPos p = pack_pos(o, nb, KT);
    uint32_t val = 0;
    if (p.row < N) {
        const int8_t* r = src + ((int64_t)p.k * N + p.row) * K;
        for (int b = 0; b < 32; ++b) {
            const int col = p.wcol * 32 + b;
            if (col < K && r[col] > 0) val |= 1u << b;
        }
    }
    dst[o] = val;
}

// Ternary weights as two half-scale bases: base 0 bit = (w >= 0), base 1 bit = (w > 0), so
// w = +1 -> (+1,+1), w = -1 -> (-1,-1), w = 0 -> (+1,-1).
__global__ void k_ternary_bits(const int8_t* __restrict__ w, int N, int K, int KT, int64_t total,
                               uint32_t* __restrict__ dst) {
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= total) return;
    const PackPos p = pack_pos(o, 2, KT);
    uint32_t val = 0;
    if (p.row < N) {
        const int8_t* r = w + (int64_t)p.row * K;
        for (int b = 0; b < 32; ++b) {
            const int col = p.wcol * 32 + b;
            if (col < K) {
                const int8_t v = r[col];
                if (p.k == 0 ? (v >= 0) : (v > 0)) val |= 1u << b;
            }
        }
    }
    dst[o] = val;
}

__global__ void k_ternary_scales(const float* __restrict__ scale, int N, int K, float* __restrict__ alpha_r,
                                 float* __restrict__ alpha_c) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < N) {
        const float h = 0.5f * scale[i];
        alpha_r[i] = h;
        alpha_r[N + i] = h;
    }
    if (i < K) {
        alpha_c[i] = 1.f;
        alpha_c[K + i] = 1.f;
    }
}

// ---------------------------------------------------------------------------------------
// LUT-BSF tables into memory: one thread per (batch row, base, group).

template <typename XT>
__global__ void k_build_lut(const XT* __restrict__ x, int batch, const float* __restrict__ alpha_c, int nb, int K,
                            int g, float* __restrict__ lut) {
    const int ng = (K + g - 1) / g;
    const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (id >= (int64_t)batch * nb * ng) return;
    const int gi = (int)(id % ng);
    const int k = (int)((id / ng) % nb);
    const int b = (int)(id / ng / nb);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int col = gi * g + i;
        v[i] = (i < g && col < K) ? alpha_c[(int64_t)k * K + col] * to_f32(x[(int64_t)b * K + col]) : 0.f;
    }
    float* out = lut + id * ((int64_t)1 << g);
    if (g == 8) {
        for (int p0 = 0; p0 < 256; p0 += 32) {
            float T[32];
            lut8_block(v, p0, T);
#pragma unroll
            for (int pp = 0; pp < 32; ++pp) out[p0 + pp] = T[pp];
        }
    } else {
        float T[16];
        lut4_table(v, T);
#pragma unroll
        for (int p = 0; p < 16; ++p) out[p] = T[p];
    }
}

// ---------------------------------------------------------------------------------------
// Pattern extraction (test export): one thread per (base, tile row, tile, slice), reading the
// slots exactly as the GEMV does.

__global__ void k_extract8(const uint32_t* __restrict__ packed, int nb, int N, int K, int NT, int KT,
                           uint16_t* __restrict__ out) {
    const int rho = threadIdx.x;
    const int64_t blk = blockIdx.x;  // ((rt * KT + ks) * nb + k)
    const int k = (int)(blk % nb);
    const int ks = (int)((blk / nb) % KT);
    const int rt = (int)(blk / nb / KT);
    const int row = rt * kTileRows + rho;
    if (rt >= NT || row >= N) return;
    const uint4* tp = reinterpret_cast<const uint4*>(packed + blk * kTileWords);
    const uint4 w0 = tp[rho], w1 = tp[kTileRows + rho];
    const uint32_t W[9] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w, w0.x};
    const uint32_t c = rot_bytes(rho);
    const int l = rho & 31;
    const int ng = (K + 7) / 8;
    uint16_t* o = out + ((int64_t)k * N + row) * ng;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t A = aligned_pair(W[i], W[i + 1], c);
        const uint32_t pat[4] = {perm_addr<0>(A, 0u) >> 8, perm_addr<1>(A, 0u) >> 8, perm_addr<2>(A, 0u) >> 8,
                                 perm_addr<3>(A, 0u) >> 8};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int gi = ks * 32 + ((4 * i + jj + l) & 31);
            if (gi < ng) o[gi] = (uint16_t)pat[jj];
        }
    }
}

__global__ void k_extract4(const uint32_t* __restrict__ packed, int nb, int N, int K, int NT, int KT,
                           uint16_t* __restrict__ out) {
    const int rho = threadIdx.x;
    const int64_t blk = blockIdx.x;
    const int k = (int)(blk % nb);
    const int ks = (int)((blk / nb) % KT);
    const int rt = (int)(blk / nb / KT);
    const int row = rt * kTileRows + rho;
    if (rt >= NT || row >= N) return;
    const uint4* tp = reinterpret_cast<const uint4*>(packed + blk * kTileWords);
    const uint4 w0 = tp[rho], w1 = tp[kTileRows + rho];
    const uint32_t S[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    const int a = rot_words(rho);
    const int ng = (K + 3) / 4;
    uint16_t* o = out + ((int64_t)k * N + row) * ng;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int wi = (s + a) & 7;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int gi = ks * 64 + wi * 8 + n;
            if (gi < ng) o[gi] = (uint16_t)((S[s] >> (4 * n)) & 15u);
        }
    }
}

// ---------------------------------------------------------------------------------------
// The GEMV (g = 8). Grid: one workgroup per (group of RPL row tiles, group of column slices).
// Per work unit (slice ks, base k) every lane holds its rows' 8 words; the next unit's words,
// scales and activations are requested before the current unit is processed. Per activation
// row b: build the 32 tables of the slice in LDS, barrier, look up every owned row,
// accumulate alpha_r^(k)[row] * sum into the lane's accumulator, barrier.

template <typename XT, bool VCM, int RPL, int BMAX>
struct UnitRegs {
    uint4 w[RPL][2];
    float ar[RPL];
    float ac;
    XT xv[BMAX];
};

template <typename XT, bool VCM, int RPL, int BMAX>
__device__ __forceinline__ void load_unit(UnitRegs<XT, VCM, RPL, BMAX>& R, const GemvArgs& a, int ks, int k,
                                          int rt0, int NT, int KT, int tid) {
    const int col = ks * kSliceCols + tid;
    const bool cvalid = col < a.Kv;
    int xcol = col;
    if (VCM) xcol = cvalid ? a.idx[col] : 0;  // requested first: the gather below waits on it
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int rt = rt0 + j;
        if (rt < NT) {
            const uint4* tp =
                reinterpret_cast<const uint4*>(a.packed + ((int64_t)(rt * KT + ks) * a.nb + k) * kTileWords);
            R.w[j][0] = tp[tid];
            R.w[j][1] = tp[kTileRows + tid];
        } else {
            R.w[j][0] = make_uint4(0, 0, 0, 0);
            R.w[j][1] = make_uint4(0, 0, 0, 0);
        }
        const int row = rt * kTileRows + tid;
        R.ar[j] = (rt < NT && row < a.N) ? a.alpha_r[(int64_t)k * a.N + row] : 0.f;
    }
    R.ac = cvalid ? a.alpha_c[(int64_t)k * a.Kv + col] : 0.f;
    const XT* xp = reinterpret_cast<const XT*>(a.x);
#pragma unroll
    for (int b = 0; b < BMAX; ++b) R.xv[b] = (b < a.batch && cvalid) ? xp[(int64_t)b * a.ldx + xcol] : XT(0.f);
}

template <typename XT, bool VCM, int RPL, int BMAX>
__global__ __launch_bounds__(256, 2) void k_lut_gemv8(GemvArgs a, int NT, int KT, int n_kgroups) {
    __shared__ __align__(16) float s_tab[256 * 64];  // 256 rows x 64 columns of fp32 = 64 KiB
    __shared__ __align__(16) float s_vbuf[BMAX * 256];  // scaled activations of the slice
    lds_f32* tab = (lds_f32*)s_tab;
    lds_f32* vbuf = (lds_f32*)s_vbuf;
    lds_cchar* tb = (lds_cchar*)s_tab;

    const int tid = threadIdx.x;
    const int L = tid & 63, wv = tid >> 6;
    const int l = L & 31, h = L >> 5;
    const uint32_t c = (uint32_t)rot_bytes(tid);
    const uint32_t lanec = 4u * (uint32_t)l;
    const int p0 = 32 * (2 * wv + h);         // table rows this lane writes

    const int kg = blockIdx.x % n_kgroups;
    const int rg = blockIdx.x / n_kgroups;
    const int rt0 = rg * RPL;
    const int ks0 = kg * a.slices_per_group;
    const int ks1 = min(ks0 + a.slices_per_group, KT);
    const int nunits = (ks1 - ks0) * a.nb;

    float acc[RPL][BMAX];
#pragma unroll
    for (int j = 0; j < RPL; ++j)
#pragma unroll
        for (int b = 0; b < BMAX; ++b) acc[j][b] = 0.f;

    UnitRegs<XT, VCM, RPL, BMAX> cur, nxt;
    if (nunits > 0) load_unit(cur, a, ks0, 0, rt0, NT, KT, tid);
    for (int u = 0; u < nunits; ++u) {
        if (u + 1 < nunits) {
            const int un = u + 1;
            load_unit(nxt, a, ks0 + un / a.nb, un % a.nb, rt0, NT, KT, tid);
        }
        // scaled activations of this slice: v = alpha_c * x (LUT-BSF folds alpha_c here)
#pragma unroll
        for (int b = 0; b < BMAX; ++b)
            if (b < a.batch) vbuf[b * 256 + tid] = cur.ac * to_f32(cur.xv[b]);
        __syncthreads();
        for (int b = 0; b < a.batch; ++b) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = vbuf[b * 256 + 8 * l + i];
            float T[32];
            lut8_block(v, p0, T);
#pragma unroll
            for (int pp = 0; pp < 32; ++pp) {
                tab[(p0 + pp) * 64 + l] = T[pp];
                tab[(p0 + pp) * 64 + l + 32] = T[pp];
            }
            __syncthreads();
            float S[RPL];
#pragma unroll
            for (int j = 0; j < RPL; ++j) S[j] = cur.ar[j] * lookup_row(tb, cur.w[j][0], cur.w[j][1], lanec, c);
#pragma unroll
            for (int bb = 0; bb < BMAX; ++bb)
                if (bb == b) {
#pragma unroll
                    for (int j = 0; j < RPL; ++j) acc[j][bb] += S[j];
                }
            __syncthreads();
        }
        if (u + 1 < nunits) cur = nxt;
    }

    const bool atomic = n_kgroups > 1;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int rt = rt0 + j;
        const int row = rt * kTileRows + tid;
        if (rt >= NT || row >= a.N) continue;
#pragma unroll
        for (int b = 0; b < BMAX; ++b) {
            if (b >= a.batch) break;
            float* dst = a.y + (int64_t)b * a.N + row;
            if (atomic) atomicAdd(dst, acc[j][b]);
            else if (a.accumulate) *dst += acc[j][b];
            else *dst = acc[j][b];
        }
    }
}

// ---------------------------------------------------------------------------------------
// Streaming read with the GEMV's access shape (measurement helper).

__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ p, int64_t n16, uint32_t* out) {
    const int64_t base = (int64_t)blockIdx.x * 512 + threadIdx.x;
    uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
    if (base < n16) a = p[base];
    if (base + 256 < n16) b = p[base + 256];
    uint32_t v = a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    // fold across the wave so the loads cannot be dropped, then one store per workgroup
    for (int off = 32; off > 0; off >>= 1) v ^= __shfl_xor(v, off);
    if (threadIdx.x == 0) out[blockIdx.x] = v;
}

// ---------------------------------------------------------------------------------------
// Launchers.

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)ceil_div(n16, 512)), dim3(256), 0, s, (const uint4*)buf, n16,
                       out);
    return hipGetLastError();
}

static inline unsigned grid_for(int64_t n, int block) { return (unsigned)((n + block - 1) / block); }

hipError_t launch_fill_zero(float* y, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(n, 256)), dim3(256), 0, s, y, n);
    return hipGetLastError();
}

hipError_t launch_pack(const void* src, int src_fmt, int nb, int N, int K, uint32_t* dst, hipStream_t s) {
    const int NT = (int)ceil_div(N, kTileRows), KT = (int)ceil_div(K, kSliceCols);
    const int64_t total = (int64_t)nb * NT * KT * kTileWords;
    if (src_fmt == UBW_SRC_CANON_BITS)
        hipLaunchKernelGGL(k_pack_canon, dim3(grid_for(total, 256)), dim3(256), 0, s, (const uint32_t*)src, nb, N,
                           K, KT, total, dst);
    else
        hipLaunchKernelGGL(k_pack_int8, dim3(grid_for(total, 256)), dim3(256), 0, s, (const int8_t*)src, nb, N, K,
                           KT, total, dst);
    return hipGetLastError();
}

hipError_t launch_ternary(const int8_t* w, const float* scale, int N, int K, uint32_t* packed, float* alpha_r,
                          float* alpha_c, hipStream_t s) {
    const int NT = (int)ceil_div(N, kTileRows), KT = (int)ceil_div(K, kSliceCols);
    const int64_t total = (int64_t)2 * NT * KT * kTileWords;
    hipLaunchKernelGGL(k_ternary_bits, dim3(grid_for(total, 256)), dim3(256), 0, s, w, N, K, KT, total, packed);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_ternary_scales, dim3(grid_for(N > K ? N : K, 256)), dim3(256), 0, s, scale, N, K, alpha_r,
                       alpha_c);
    return hipGetLastError();
}

hipError_t launch_build_lut(const void* x, int x_dtype, int batch, const float* alpha_c, int nb, int K, int g,
                            float* lut, hipStream_t s) {
    const int64_t n = (int64_t)batch * nb * ((K + g - 1) / g);
    if (x_dtype == UBW_F16)
        hipLaunchKernelGGL(k_build_lut<__half>, dim3(grid_for(n, 128)), dim3(128), 0, s, (const __half*)x, batch,
                           alpha_c, nb, K, g, lut);
    else
        hipLaunchKernelGGL(k_build_lut<float>, dim3(grid_for(n, 128)), dim3(128), 0, s, (const float*)x, batch,
                           alpha_c, nb, K, g, lut);
    return hipGetLastError();
}

hipError_t launch_extract(const uint32_t* packed, int nb, int N, int K, int g, uint16_t* out, hipStream_t s) {
    const int NT = (int)ceil_div(N, kTileRows), KT = (int)ceil_div(K, kSliceCols);
    const unsigned blocks = (unsigned)((int64_t)nb * NT * KT);
    if (g == 8)
        hipLaunchKernelGGL(k_extract8, dim3(blocks), dim3(kTileRows), 0, s, packed, nb, N, K, NT, KT, out);
    else
        hipLaunchKernelGGL(k_extract4, dim3(blocks), dim3(kTileRows), 0, s, packed, nb, N, K, NT, KT, out);
    return hipGetLastError();
}

template <typename XT, bool VCM, int RPL, int BMAX>
static hipError_t launch_gemv8_t(const GemvArgs& a, hipStream_t s) {
    const int NT = (int)ceil_div(a.N, kTileRows), KT = (int)ceil_div(a.Kv, kSliceCols);
    const int n_kgroups = (int)ceil_div(KT, a.slices_per_group);
    const int n_rgroups = (int)ceil_div(NT, RPL);
    hipLaunchKernelGGL((k_lut_gemv8<XT, VCM, RPL, BMAX>), dim3((unsigned)((int64_t)n_rgroups * n_kgroups)),
                       dim3(kThreads), 0, s, a, NT, KT, n_kgroups);
    return hipGetLastError();
}

// Instances: (row tiles per workgroup, batch bound) pairs whose registers fit without spills;
// max_rows_per_group() below is the host-side rule that keeps requests inside this set.
template <typename XT, bool VCM>
static hipError_t launch_gemv8_r(const GemvArgs& a, hipStream_t s) {
    if (a.batch <= 1) {
        if (a.rows_per_group >= 4) return launch_gemv8_t<XT, VCM, 4, 1>(a, s);
        if (a.rows_per_group >= 2) return launch_gemv8_t<XT, VCM, 2, 1>(a, s);
        return launch_gemv8_t<XT, VCM, 1, 1>(a, s);
    }
    if (a.batch <= 2) {
        if (a.rows_per_group >= 2) return launch_gemv8_t<XT, VCM, 2, 2>(a, s);
        return launch_gemv8_t<XT, VCM, 1, 2>(a, s);
    }
    if (a.batch <= 4) return launch_gemv8_t<XT, VCM, 1, 4>(a, s);
    if (a.batch <= 8) return launch_gemv8_t<XT, VCM, 1, 8>(a, s);
    return launch_gemv8_t<XT, VCM, 1, 16>(a, s);
}

int max_rows_per_group(int batch) { return batch <= 1 ? 4 : (batch <= 2 ? 2 : 1); }

hipError_t launch_gemv8(const GemvArgs& a, hipStream_t s) {
    const bool vcm = a.idx != nullptr;
    if (a.x_dtype == UBW_F16)
        return vcm ? launch_gemv8_r<__half, true>(a, s) : launch_gemv8_r<__half, false>(a, s);
    return vcm ? launch_gemv8_r<float, true>(a, s) : launch_gemv8_r<float, false>(a, s);
}

}  // namespace ubw
