// HIP kernels for gfx950: packing, ternary encoding, LUT-BSF table build, pattern
// extraction and the table-lookup GEMV over decoupled row-column binary bases.
//
// Method: FluxBin (gist.science/ko/paper/2608.15602), technical summary, "2. Kernel
// innovation": tables with alpha_c folded in (LUT-BSF), virtual columnar mapping for the
// salient columns (VCM), and the execution flow stream packed uint32 -> extract pattern
// indices with bit operations -> fetch precomputed partial sums -> apply alpha_r.
//
// gfx950 mapping (the page's kernel targets another GPU; only its dataflow is kept):
//   - a workgroup of 256 threads owns 256-row tiles x 256-column slices; each lane owns one row
//     of a tile and walks the slice's 32 groups of 8 columns, for two bases at a time;
//   - a group table has 256 fp32 entries, all in one LDS bank: entry p of group x of base
//     k (k = 0, 1 within the pair) lives at byte 256 p + 128 k + 4 x, so the two bases' tables
//     of a slice fill one 64 KiB block and every table sits in bank x;
//   - the lane with l = lane mod 32 reads group (l + t) mod 32 at step t, so each half-wave
//     touches 32 distinct banks per lookup (the LDS serves a wave64 access as two 32-lane
//     halves over 32 banks);
//   - the lookup address is one v_perm_b32 that puts the weight byte (the pattern) in byte 1
//     and the lane's column offset for that step in byte 0; a v_alignbyte_b32 per 4 lookups
//     supplies the lane's rotated byte order;
//   - slices of one row are combined with fp32 atomics; when the caller asks for y = result the
//     first workgroup to arrive at a row group zeroes those rows and the others wait for its
//     flag before adding (atomics only, no fences), so one launch does the whole step;
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

// Per-lane column offsets of the 32 steps, four per register: byte jj of lc[i] is
// 4 * ((l + 4 i + jj) mod 32), the byte offset of the group the lane reads at step 4 i + jj.
__device__ __forceinline__ void lane_columns(int l, uint32_t lc[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) v |= (uint32_t)(4 * ((l + 4 * i + jj) & 31)) << (8 * jj);
        lc[i] = v;
    }
}

// Address of the step 4 i + jj lookup: byte 0 = the lane's column offset for that step (byte
// jj of lc), byte 1 = the pattern (byte jj of the aligned word A), bytes 2-3 zero. So the
// result is 256 * pattern + 4 * group.
template <int JJ>
__device__ __forceinline__ uint32_t perm_addr(uint32_t A, uint32_t lc) {
    return __builtin_amdgcn_perm(A, lc, 0x0C0C0000u | ((4u + JJ) << 8) | (uint32_t)JJ);
}

// The four patterns of steps 4i .. 4i+3 start at byte c of the slot pair (W[i], W[i+1]).
__device__ __forceinline__ uint32_t aligned_pair(uint32_t lo, uint32_t hi, uint32_t c) {
    return __builtin_amdgcn_alignbyte(hi, lo, c);
}

// LUT-BSF for one group of 8 columns with scaled activations v[0..7]:
// T[p] = sum_i (2 bit_i(p) - 1) v[i] = lo[p & 15] + hi(p >> 4), where lo and hi are the
// 4-column half tables. This returns lo[0..15] (built by doubling from the all-minus entry)
// and, for a block of 32 entries starting at p0 (a multiple of 32), hi(p0 / 16) and
// hi(p0 / 16 + 1).
__device__ __forceinline__ void lut8_parts(const float v[8], int p0, float lo[16], float& hi0, float& hi1) {
    const float u0 = v[0] + v[0], u1 = v[1] + v[1], u2 = v[2] + v[2], u3 = v[3] + v[3];
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
    hi0 = (s5 - v[4]) + (s6 + s7);
    hi1 = hi0 + (v[4] + v[4]);
}

__device__ __forceinline__ float lut8_entry(const float lo[16], float hi0, float hi1, int pp) {
    return lo[pp & 15] + (pp < 16 ? hi0 : hi1);
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

// Sum over the 32 groups of one row's slice for one base: the lane's 8 slots hold words
// (s + a) mod 8; step t reads the table of group (t + l) mod 32 at that group's pattern.
// tb points at the base's half of the table block.
__device__ __forceinline__ float lookup_row(lds_cchar* tb, const uint4& w0, const uint4& w1, const uint32_t lc[8],
                                            uint32_t c) {
    const uint32_t W[9] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w, w0.x};
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t A = aligned_pair(W[i], W[i + 1], c);
        s0 += *(const lds_f32*)(tb + perm_addr<0>(A, lc[i]));
        s1 += *(const lds_f32*)(tb + perm_addr<1>(A, lc[i]));
        s2 += *(const lds_f32*)(tb + perm_addr<2>(A, lc[i]));
        s3 += *(const lds_f32*)(tb + perm_addr<3>(A, lc[i]));
    }
    return (s0 + s1) + (s2 + s3);
}

// ---------------------------------------------------------------------------------------
// Zero fill (used before K-split atomics when the caller asks for y = result and passes no
// workspace).

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
// LUT-BSF tables into memory: one thread per (batch row, base, group), same arithmetic as the
// tables the GEMV builds in LDS.

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
            float lo[16], hi0, hi1;
            lut8_parts(v, p0, lo, hi0, hi1);
#pragma unroll
            for (int pp = 0; pp < 32; ++pp) out[p0 + pp] = lut8_entry(lo, hi0, hi1, pp);
        }
    } else {
        float T[16];
        lut4_table(v, T);
#pragma unroll
        for (int p = 0; p < 16; ++p) out[p] = T[p];
    }
}

// ---------------------------------------------------------------------------------------
// Pattern extraction (test export): one thread per (base, tile row, tile, slice). The g = 8
// path reads the slots and forms the lookup addresses exactly as the GEMV does, then takes
// the pattern from byte 1 and the group from byte 0 of each address.

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
    uint32_t lc[8];
    lane_columns(rho & 31, lc);
    const int ng = (K + 7) / 8;
    uint16_t* o = out + ((int64_t)k * N + row) * ng;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t A = aligned_pair(W[i], W[i + 1], c);
        const uint32_t ad[4] = {perm_addr<0>(A, lc[i]), perm_addr<1>(A, lc[i]), perm_addr<2>(A, lc[i]),
                                perm_addr<3>(A, lc[i])};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int gi = ks * 32 + (int)((ad[jj] & 0xFFu) >> 2);
            if (gi < ng) o[gi] = (uint16_t)(ad[jj] >> 8);
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
// The GEMV step (g = 8).
//
// Grid: C workgroups of 512 threads per row group (RPL tiles of 256 rows), one per
// (segment, group of column slices); C = sum over segments of ceil(KT / slices_per_group).
// A workgroup's work is a list of items (slice, base) of its slices; a unit is two
// consecutive items, one per half of every wave: lane l of half h in wave w owns tile row
// 32 w + l for item h. Per unit and activation row b: stage v = alpha_c * x for both items,
// build each item's 32 tables (half h writes LDS columns 32 h .. 32 h + 31), barrier, look
// up every owned row, accumulate alpha_r * sum, barrier. The two halves of a row (different
// items) are added with a cross-lane swap at the end. Weights, scales and activations of
// the next units are in flight while a unit is processed (three register slots).

enum { kModeStore = 0, kModeAdd = 1, kModeAtomic = 2, kModeFirst = 3 };
constexpr int kSpinLimit = 1 << 20;
constexpr int kStepThreads = 512;

struct StepParams {
    StepArgs a;
    int NT;
    int C;            // workgroups per row group
    int KT[2];        // slices per segment
    int nkg[2];       // slice groups per segment
    int mode;
};

template <typename XT, int RPL, int BMAX>
struct Unit {
    uint4 w[RPL][2];   // this lane's item: its rows' 8 words (two 16-byte halves of the slice)
    float ar[RPL];     // alpha_r of the item's base at the lane's rows
    float ac;          // staging: alpha_c of the staged item's base at the staged column
    XT xv[BMAX];       // staging: activations at the staged column
};

// Item `it` (slice ks0 + it / nb, base it % nb) of the workgroup's list, or none.
struct Item {
    int ks, k;
    bool valid;
};

__device__ __forceinline__ Item item_of(int it, int nitems, int ks0, int nb) {
    Item r;
    r.valid = it < nitems;
    const int q = r.valid ? it : 0;
    r.ks = ks0 + q / nb;
    r.k = q - (q / nb) * nb;
    return r;
}

template <typename XT, int RPL, int BMAX>
__device__ __forceinline__ void load_unit(Unit<XT, RPL, BMAX>& U, const Segment& sg, const StepArgs& a, int KT,
                                          int NT, int u, int nitems, int ks0, int rt0, int h, int rho, int tid) {
    // staging role: thread tid stages column (tid mod 256) of item 2u + tid / 256
    const Item st = item_of(2 * u + (tid >> 8), nitems, ks0, sg.nb);
    const int col = st.ks * kSliceCols + (tid & 255);
    const bool cvalid = st.valid && col < sg.Kv;
    int xcol = col;
    if (sg.idx) xcol = cvalid ? sg.idx[col] : 0;  // requested first: the gather below waits on it
    // lookup role: item 2u + h for tile row rho
    const Item lk = item_of(2 * u + h, nitems, ks0, sg.nb);
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int rt = rt0 + j;
        U.w[j][0] = U.w[j][1] = make_uint4(0, 0, 0, 0);
        if (lk.valid && rt < NT) {
            const uint4* tp =
                reinterpret_cast<const uint4*>(sg.packed + ((int64_t)(rt * KT + lk.ks) * sg.nb + lk.k) * kTileWords);
            U.w[j][0] = tp[rho];
            U.w[j][1] = tp[kTileRows + rho];
        }
        const int row = rt * kTileRows + rho;
        U.ar[j] = (lk.valid && rt < NT && row < a.N) ? sg.alpha_r[(int64_t)lk.k * a.N + row] : 0.f;
    }
    U.ac = cvalid ? sg.alpha_c[(int64_t)st.k * sg.Kv + col] : 0.f;
    const XT* xp = reinterpret_cast<const XT*>(a.x);
#pragma unroll
    for (int b = 0; b < BMAX; ++b) U.xv[b] = (b < a.batch && cvalid) ? xp[(int64_t)b * a.ldx + xcol] : XT(0.f);
}

template <typename XT, int RPL, int BMAX>
__global__ __launch_bounds__(kStepThreads, (BMAX <= 4 ? 2 : 1)) void k_gemv8(StepParams P) {
    // Batches above 2 keep their per-row accumulators in thread-private LDS slots (registers
    // indexed by a runtime batch index would go to scratch).
    constexpr bool kAccLds = BMAX > 2;
    __shared__ __align__(16) float s_tab[256 * 64];       // one unit's 64 tables: 64 KiB
    __shared__ __align__(16) float s_v[BMAX * 2 * 256];   // scaled activations [b][item][column]
    __shared__ __align__(16) float s_acc[kAccLds ? RPL * BMAX * kStepThreads : 1];
    lds_f32* tab = (lds_f32*)s_tab;
    lds_f32* sv = (lds_f32*)s_v;
    lds_f32* sacc = (lds_f32*)s_acc;
    lds_cchar* tb = (lds_cchar*)s_tab;
    const StepArgs& a = P.a;

    const int tid = threadIdx.x;
    const int wv = tid >> 6, L = tid & 63;
    const int h = L >> 5, l = L & 31;
    const int rho = 32 * wv + l;                  // tile row of this lane
    const uint32_t c = (uint32_t)rot_bytes(rho);
    const int p0 = 32 * wv;                       // table entries this lane builds
    uint32_t lc[8];
    lane_columns(l, lc);
#pragma unroll
    for (int i = 0; i < 8; ++i) lc[i] += 0x80808080u * (uint32_t)h;  // half h's tables: +128 bytes

    const int rg = blockIdx.x / P.C;
    const int kslot = blockIdx.x - rg * P.C;
    const int si = kslot < P.nkg[0] ? 0 : 1;
    const int kg = si ? kslot - P.nkg[0] : kslot;
    const Segment sg = a.seg[si];
    const int KT = P.KT[si];
    const int rt0 = rg * RPL;
    const int ks0 = kg * sg.slices_per_group;
    const int ks1 = min(ks0 + sg.slices_per_group, KT);
    const int nitems = (ks1 - ks0) * sg.nb;
    const int nunits = (nitems + 1) >> 1;

    // The first units' weights, scales and activations are requested before anything waits.
    Unit<XT, RPL, BMAX> cur, n1, n2;
    if (nunits > 0) load_unit(cur, sg, a, KT, P.NT, 0, nitems, ks0, rt0, h, rho, tid);
    if (nunits > 1) load_unit(n1, sg, a, KT, P.NT, 1, nitems, ks0, rt0, h, rho, tid);
    if (nunits > 2) load_unit(n2, sg, a, KT, P.NT, 2, nitems, ks0, rt0, h, rho, tid);

    // y = result with several contributors per row (kModeFirst): the row group's workgroup for
    // the first column-slice group (kslot 0) zeroes the rows and raises the row group's flag;
    // every other contributor reads the flag before its atomics. The arrival counter only
    // supplies the call's generation, so nobody waits on it early. Per row group, 256 bytes
    // of workspace: word 0 = (generation << 8) | arrivals, word 32 = flag (separate lines).
    const bool zeroer = P.mode == kModeFirst && kslot == 0;
    uint32_t* cnt = a.ws + kWsHeaderWords + kWsRowGroupWords * rg;
    uint32_t* flag = cnt + kWsFlagOffset;
    uint32_t arrived = 0;  // thread 0: the counter's value before this workgroup's arrival
    if (P.mode == kModeFirst && tid == 0) arrived = atomicAdd(cnt, 1u);
    if (zeroer) {
        float sink = 0.f;
        if (tid < kTileRows) {
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                const int row = (rt0 + j) * kTileRows + tid;
                if (rt0 + j >= P.NT || row >= a.N) continue;
                for (int b = 0; b < a.batch; ++b)
                    sink += __hip_atomic_exchange(a.y + (int64_t)b * a.N + row, 0.f, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        // depend on every returned value (so each exchange has been performed before the
        // barrier); the store itself is harmless scratch in an unused workspace word
        if (sink == 1.5e38f) a.ws[1] = 1u;
        __syncthreads();
        if (tid == 0)
            __hip_atomic_exchange(flag, ((arrived >> 8) + 1) & 0xFFFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    uint32_t seen = 0;

    float acc[RPL][kAccLds ? 1 : BMAX];
#pragma unroll
    for (int j = 0; j < RPL; ++j)
#pragma unroll
        for (int b = 0; b < (kAccLds ? 1 : BMAX); ++b) acc[j][b] = 0.f;
    if (kAccLds) {
#pragma unroll
        for (int i = 0; i < RPL * BMAX; ++i) sacc[i * kStepThreads + tid] = 0.f;  // own slots only
    }

    // One activation row of one unit: build the tables, barrier, look up, accumulate, barrier.
    auto row_pass = [&](const Unit<XT, RPL, BMAX>& U, int u, int b, bool mine, float S[RPL]) {
        if (mine) {
            float v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = sv[b * 512 + 256 * h + 8 * l + i];
            float lo[16], hi0, hi1;
            lut8_parts(v, p0, lo, hi0, hi1);
#pragma unroll
            for (int pp = 0; pp < 32; ++pp) tab[(p0 + pp) * 64 + 32 * h + l] = lut8_entry(lo, hi0, hi1, pp);
        }
        __syncthreads();
        // look at the zeroer's flag while the last lookups run; used after the loop
        if (P.mode == kModeFirst && !zeroer && tid == 0 && u + 1 == nunits && b == 0)
            seen = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int j = 0; j < RPL; ++j) S[j] = mine ? U.ar[j] * lookup_row(tb, U.w[j][0], U.w[j][1], lc, c) : 0.f;
    };
    // One unit: stage v for both items, then every activation row.
    auto process = [&](const Unit<XT, RPL, BMAX>& U, int u) {
        const bool mine = 2 * u + h < nitems;  // this half has an item in this unit
        // scaled activations of both items: v = alpha_c * x (LUT-BSF folds alpha_c here)
#pragma unroll
        for (int b = 0; b < BMAX; ++b)
            if (b < a.batch) sv[b * 512 + tid] = U.ac * to_f32(U.xv[b]);
        __syncthreads();
        if constexpr (!kAccLds) {
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
                if (b < a.batch) {
                    float S[RPL];
                    row_pass(U, u, b, mine, S);
#pragma unroll
                    for (int j = 0; j < RPL; ++j) acc[j][kAccLds ? 0 : b] += S[j];
                    __syncthreads();
                }
            }
        } else {
            for (int b = 0; b < a.batch; ++b) {
                float S[RPL];
                row_pass(U, u, b, mine, S);
#pragma unroll
                for (int j = 0; j < RPL; ++j) sacc[(j * BMAX + b) * kStepThreads + tid] += S[j];
                __syncthreads();
            }
        }
    };
    // Three register slots, each reloaded in place three units ahead (no copies between
    // slots, which would wait on loads still in flight).
    for (int u = 0; u < nunits; u += 3) {
        process(cur, u);
        if (u + 3 < nunits) load_unit(cur, sg, a, KT, P.NT, u + 3, nitems, ks0, rt0, h, rho, tid);
        if (u + 1 < nunits) {
            process(n1, u + 1);
            if (u + 4 < nunits) load_unit(n1, sg, a, KT, P.NT, u + 4, nitems, ks0, rt0, h, rho, tid);
        }
        if (u + 2 < nunits) {
            process(n2, u + 2);
            if (u + 5 < nunits) load_unit(n2, sg, a, KT, P.NT, u + 5, nitems, ks0, rt0, h, rho, tid);
        }
    }

    if (P.mode == kModeFirst && tid == 0 && (arrived & 0xFFu) + 1 == (uint32_t)P.C)
        atomicAdd(cnt, 0x100u - (uint32_t)P.C);  // last to arrive: arrivals back to 0, next generation
    if (P.mode == kModeFirst && !zeroer) {
        if (tid == 0) {
            const uint32_t want = ((arrived >> 8) + 1) & 0xFFFFFFu;
            int n = 0;
            while (seen != want) {
                __builtin_amdgcn_s_sleep(2);
                seen = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (++n > kSpinLimit) {  // cannot happen while the zeroer runs; never hang
                    atomicOr(a.ws, 1u);
                    break;
                }
            }
        }
        __syncthreads();
    }

    // The two halves of every row hold different items' sums: add them across lanes l, l + 32,
    // then the first half writes.
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int rt = rt0 + j;
        const int row = rt * kTileRows + rho;
        const bool rv = rt < P.NT && row < a.N;
#pragma unroll
        for (int b = 0; b < BMAX; ++b) {
            if (b >= a.batch) continue;
            const float part = kAccLds ? sacc[(j * BMAX + b) * kStepThreads + tid] : acc[j][kAccLds ? 0 : b];
            const uint32_t pv = __float_as_uint(part);
            const auto sw = __builtin_amdgcn_permlane32_swap(pv, pv, false, false);
            const float total = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            if (h == 0 && rv) {
                float* dst = a.y + (int64_t)b * a.N + row;
                if (P.mode == kModeStore) *dst = total;
                else if (P.mode == kModeAdd) *dst += total;
                else atomicAdd(dst, total);
            }
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

static inline unsigned grid_for(int64_t n, int block) { return (unsigned)((n + block - 1) / block); }

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)ceil_div(n16, 512)), dim3(256), 0, s, (const uint4*)buf, n16,
                       out);
    return hipGetLastError();
}

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

// Workgroups of this instance that the device can hold at once (occupancy x CUs), cached.
template <typename XT, int RPL, int BMAX>
static int64_t resident_capacity() {
    static int64_t cap = -1;  // benign race: every thread computes the same value
    if (cap < 0) {
        int dev = 0, cus = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gemv8<XT, RPL, BMAX>, kStepThreads, 0) !=
                hipSuccess)
            return 0;
        cap = (int64_t)cus * per_cu;
    }
    return cap;
}

template <typename XT, int RPL, int BMAX>
static hipError_t launch_step_t(StepParams P, int n_rgroups, hipStream_t s) {
    const int64_t grid = (int64_t)n_rgroups * P.C;
    if (P.mode == kModeFirst && grid > resident_capacity<XT, RPL, BMAX>()) {
        // Waiting on another workgroup is safe only when the whole grid is resident at once;
        // otherwise zero y with a separate launch and let every workgroup add.
        hipError_t e = launch_fill_zero(P.a.y, (int64_t)P.a.batch * P.a.N, s);
        if (e != hipSuccess) return e;
        P.mode = kModeAtomic;
    }
    hipLaunchKernelGGL((k_gemv8<XT, RPL, BMAX>), dim3((unsigned)grid), dim3(kStepThreads), 0, s, P);
    return hipGetLastError();
}

// Instances: (row tiles per workgroup, batch bound) pairs whose registers fit without spills;
// max_rows_per_group() is the host-side rule that keeps requests inside this set.
template <typename XT>
static hipError_t launch_step_x(const StepParams& P, int n_rgroups, int rpl, hipStream_t s) {
    const int batch = P.a.batch;
    if (batch <= 1) {
        if (rpl >= 2) return launch_step_t<XT, 2, 1>(P, n_rgroups, s);
        return launch_step_t<XT, 1, 1>(P, n_rgroups, s);
    }
    if (batch <= 2) {
        if (rpl >= 2) return launch_step_t<XT, 2, 2>(P, n_rgroups, s);
        return launch_step_t<XT, 1, 2>(P, n_rgroups, s);
    }
    if (batch <= 4) return launch_step_t<XT, 1, 4>(P, n_rgroups, s);
    if (batch <= 8) return launch_step_t<XT, 1, 8>(P, n_rgroups, s);
    return launch_step_t<XT, 1, 16>(P, n_rgroups, s);
}

int max_rows_per_group(int batch) { return batch <= 2 ? 2 : 1; }

hipError_t launch_step(const StepArgs& a, hipStream_t s) {
    StepParams P{};
    P.a = a;
    P.NT = (int)ceil_div(a.N, kTileRows);
    P.C = 0;
    for (int i = 0; i < 2; ++i) {
        if (i < a.nseg) {
            P.KT[i] = (int)ceil_div(a.seg[i].Kv, kSliceCols);
            P.nkg[i] = (int)ceil_div(P.KT[i], a.seg[i].slices_per_group);
        } else {
            P.KT[i] = 0;
            P.nkg[i] = 0;
        }
        P.C += P.nkg[i];
    }
    const int rpl = a.rows_per_group;
    const int n_rgroups = (int)ceil_div(P.NT, rpl);
    if (a.accumulate) {
        P.mode = P.C > 1 ? kModeAtomic : kModeAdd;
    } else if (P.C == 1) {
        P.mode = kModeStore;
    } else if (a.ws != nullptr && P.C <= 255) {
        P.mode = kModeFirst;
    } else {
        hipError_t e = launch_fill_zero(a.y, (int64_t)a.batch * a.N, s);
        if (e != hipSuccess) return e;
        P.mode = kModeAtomic;
    }
    if (a.x_dtype == UBW_F16) return launch_step_x<__half>(P, n_rgroups, rpl, s);
    return launch_step_x<float>(P, n_rgroups, rpl, s);
}

}  // namespace ubw
