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
// The GEMV step (g = 8): a persistent, stream-K style kernel.
//
// Work list: for each row group rg (RPL tiles of 256 rows), the units of each segment in
// order. A segment's items are (slice, base) pairs, slice-major; a unit is two consecutive
// items, one per half of every wave: lane l of half h in wave w owns tile row 32 w + l for
// item h. The list holds U = NRG * Urg units; workgroup g of G takes units
// [g U / G, (g + 1) U / G), keeps per-row partial sums across consecutive units of one row
// group and adds them into y with fp32 atomics when its range leaves that row group.
// Per unit and activation row b: stage v = alpha_c * x for both items, build each item's 32
// tables (half h writes LDS columns 32 h .. 32 h + 31), barrier, look up every owned row,
// accumulate alpha_r * sum, barrier. The two halves of a row (different items) are added with
// a cross-lane swap when flushing. The weights, scales and activations of the next units are
// in flight while a unit is processed (three register slots, reloaded in place).
//
// y = result in one launch (kModeFirst): at its start workgroup g zeroes the rows of every
// row group rg with rg mod G == g and raises that row group's flag; a workgroup reads the flag
// of a row group before adding into it. Zeroing depends on nothing and the grid never exceeds
// what the device holds at once, so every wait ends. Per row group, 256 bytes of workspace:
// word 0 = (generation << 12) | arrivals, word 32 = flag.

enum { kModeStore = 0, kModeAdd = 1, kModeAtomic = 2, kModeFirst = 3 };
constexpr int kSpinLimit = 1 << 20;
constexpr int kStepThreads = 512;
constexpr uint32_t kArrBits = 12;
constexpr uint32_t kArrMask = (1u << kArrBits) - 1u;
constexpr uint32_t kGenMask = (1u << (32 - kArrBits)) - 1u;

struct StepParams {
    StepArgs a;
    int NT;
    int NRG;          // row groups
    int KT[2];        // slices per segment
    int US[2];        // units per row group per segment
    int Urg;          // units per row group
    int U;            // units in the whole list (U * G < 2^32, checked on the host)
    int G;            // workgroups
    int mode;
};

template <typename XT, int RPL, int BMAX>
struct Unit {
    uint4 w[RPL][2];   // this lane's item: its rows' 8 words (two 16-byte halves of the slice)
    float ar[RPL];     // alpha_r of the item's base at the lane's rows
    float ac;          // staging: alpha_c of the staged item's base at the staged column
    XT xv[BMAX];       // staging: activations at the staged column
};

// Where unit x of the list lives.
struct UnitPos {
    int rg;     // row group
    int si;     // segment
    int pair;   // unit within the segment's units of this row group
};

// (row group, unit within the row group) of a cursor walking the list.
struct Cursor {
    int rg, q;
};

__device__ __forceinline__ void advance(Cursor& cu, int Urg) {
    if (++cu.q == Urg) {
        cu.q = 0;
        ++cu.rg;
    }
}

__device__ __forceinline__ UnitPos unit_pos(const StepParams& P, Cursor cu) {
    UnitPos r;
    r.rg = cu.rg;
    r.si = cu.q < P.US[0] ? 0 : 1;
    r.pair = r.si ? cu.q - P.US[0] : cu.q;
    return r;
}

template <typename XT, int RPL, int BMAX>
__device__ __forceinline__ void load_unit(Unit<XT, RPL, BMAX>& U, const StepParams& P, Cursor cu, int h, int rho,
                                          int tid) {
    const StepArgs& a = P.a;
    const UnitPos up = unit_pos(P, cu);
    const Segment& sg = a.seg[up.si];
    const int KT = P.KT[up.si];
    const int nitems = KT * sg.nb;
    const int rt0 = up.rg * RPL;
    // staging role: thread tid stages column (tid mod 256) of item 2 pair + tid / 256
    const int its = 2 * up.pair + (tid >> 8);
    const bool sval = its < nitems;
    const int sks = sval ? its / sg.nb : 0, sk = sval ? its - sks * sg.nb : 0;
    const int col = sks * kSliceCols + (tid & 255);
    const bool cvalid = sval && col < sg.Kv;
    int xcol = col;
    if (sg.idx) xcol = cvalid ? sg.idx[col] : 0;  // requested first: the gather below waits on it
    // lookup role: item 2 pair + h for tile row rho
    const int itl = 2 * up.pair + h;
    const bool lval = itl < nitems;
    const int lks = lval ? itl / sg.nb : 0, lk = lval ? itl - lks * sg.nb : 0;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int rt = rt0 + j;
        U.w[j][0] = U.w[j][1] = make_uint4(0, 0, 0, 0);
        if (lval && rt < P.NT) {
            const uint4* tp =
                reinterpret_cast<const uint4*>(sg.packed + ((int64_t)(rt * KT + lks) * sg.nb + lk) * kTileWords);
            U.w[j][0] = tp[rho];
            U.w[j][1] = tp[kTileRows + rho];
        }
        const int row = rt * kTileRows + rho;
        U.ar[j] = (lval && rt < P.NT && row < a.N) ? sg.alpha_r[(int64_t)lk * a.N + row] : 0.f;
    }
    U.ac = cvalid ? sg.alpha_c[(int64_t)sk * sg.Kv + col] : 0.f;
    const XT* xp = reinterpret_cast<const XT*>(a.x);
#pragma unroll
    for (int b = 0; b < BMAX; ++b) U.xv[b] = (b < a.batch && cvalid) ? xp[(int64_t)b * a.ldx + xcol] : XT(0.f);
}

// First unit of workgroup g's range, and the workgroup whose range holds unit x (the largest g
// with start(g) <= x). 32-bit: the host guarantees U * G < 2^32.
__device__ __forceinline__ uint32_t range_start(const StepParams& P, uint32_t g) {
    return g * (uint32_t)P.U / (uint32_t)P.G;
}
__device__ __forceinline__ int owner_of(const StepParams& P, uint32_t x) {
    return (int)(((x + 1) * (uint32_t)P.G - 1) / (uint32_t)P.U);
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

    const int g = blockIdx.x;
    const int x0 = (int)range_start(P, g);
    const int x1 = (int)range_start(P, g + 1);
    Cursor lcur{x0 / P.Urg, x0 % P.Urg};  // next unit to load
    Cursor pcur = lcur;                     // next unit to process

    // The first units' weights, scales and activations are requested before anything waits.
    Unit<XT, RPL, BMAX> s0, s1, s2;
    if (x0 < x1) { load_unit(s0, P, lcur, h, rho, tid); advance(lcur, P.Urg); }
    if (x0 + 1 < x1) { load_unit(s1, P, lcur, h, rho, tid); advance(lcur, P.Urg); }
    if (x0 + 2 < x1) { load_unit(s2, P, lcur, h, rho, tid); advance(lcur, P.Urg); }

    const bool first_mode = P.mode == kModeFirst;
    if (first_mode) {
        // zero the rows of the row groups this workgroup owns and raise their flags
        for (int rg = g; rg < P.NRG; rg += P.G) {
            uint32_t* cnt = a.ws + kWsHeaderWords + kWsRowGroupWords * rg;
            float sink = 0.f;
            uint32_t gen = 0;
            if (tid == 0) gen = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> kArrBits;
            if (tid < kTileRows) {
#pragma unroll
                for (int j = 0; j < RPL; ++j) {
                    const int rt = rg * RPL + j;
                    const int row = rt * kTileRows + tid;
                    if (rt >= P.NT || row >= a.N) continue;
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
                __hip_atomic_exchange(cnt + kWsFlagOffset, (gen + 1) & kGenMask, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        }
    }

    float acc[RPL][kAccLds ? 1 : BMAX];
    auto clear_acc = [&]() {
#pragma unroll
        for (int j = 0; j < RPL; ++j)
#pragma unroll
            for (int b = 0; b < (kAccLds ? 1 : BMAX); ++b) acc[j][b] = 0.f;
        if (kAccLds) {
#pragma unroll
            for (int i = 0; i < RPL * BMAX; ++i) sacc[i * kStepThreads + tid] = 0.f;  // own slots only
        }
    };
    clear_acc();

    // Row-group bookkeeping (thread 0): arrival counter value and the flag as last read.
    int cur_rg = -1;
    uint32_t arrived = 0, seen = 0;

    // Add this workgroup's partial sums of row group rg into y.
    auto flush = [&](int rg) {
        uint32_t* cnt = a.ws + kWsHeaderWords + kWsRowGroupWords * rg;
        if (first_mode) {
            if (tid == 0) {
                const uint32_t want = ((arrived >> kArrBits) + 1) & kGenMask;
                int n = 0;
                while (seen != want) {
                    __builtin_amdgcn_s_sleep(2);
                    seen = __hip_atomic_load(cnt + kWsFlagOffset, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (++n > kSpinLimit) {  // cannot happen while the owner runs; never hang
                        atomicOr(a.ws, 1u);
                        break;
                    }
                }
                // contributors of rg: the workgroups whose ranges meet rg's units
                const int cg = owner_of(P, (uint32_t)(rg + 1) * P.Urg - 1) - owner_of(P, (uint32_t)rg * P.Urg) + 1;
                if ((arrived & kArrMask) + 1 == (uint32_t)cg)  // last to arrive: arrivals 0, next generation
                    atomicAdd(cnt, (1u << kArrBits) - (uint32_t)cg);
            }
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            const int rt = rg * RPL + j;
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
    };

    // One activation row of one unit: build the tables, barrier, look up.
    auto row_pass = [&](const Unit<XT, RPL, BMAX>& U, bool mine, bool poll, int rg, int b, float S[RPL]) {
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
        // look at the row group's flag while the last lookups before a flush run
        if (poll && tid == 0 && b == 0)
            seen = __hip_atomic_load(a.ws + kWsHeaderWords + kWsRowGroupWords * rg + kWsFlagOffset, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int j = 0; j < RPL; ++j) S[j] = mine ? U.ar[j] * lookup_row(tb, U.w[j][0], U.w[j][1], lc, c) : 0.f;
    };

    // One unit of the list (the one at pcur, which it then advances).
    auto process = [&](const Unit<XT, RPL, BMAX>& U, int x) {
        const UnitPos up = unit_pos(P, pcur);
        if (up.rg != cur_rg) {  // entering a row group: arrive on its counter
            cur_rg = up.rg;
            if (first_mode && tid == 0)
                arrived = atomicAdd(a.ws + kWsHeaderWords + kWsRowGroupWords * up.rg, 1u);
        }
        const int nitems = P.KT[up.si] * a.seg[up.si].nb;
        const bool mine = 2 * up.pair + h < nitems;  // this half has an item in this unit
        const bool last_of_rg = x + 1 == x1 || pcur.q + 1 == P.Urg;
        advance(pcur, P.Urg);
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
                    row_pass(U, mine, first_mode && last_of_rg, up.rg, b, S);
#pragma unroll
                    for (int j = 0; j < RPL; ++j) acc[j][kAccLds ? 0 : b] += S[j];
                    __syncthreads();
                }
            }
        } else {
            for (int b = 0; b < a.batch; ++b) {
                float S[RPL];
                row_pass(U, mine, first_mode && last_of_rg, up.rg, b, S);
#pragma unroll
                for (int j = 0; j < RPL; ++j) sacc[(j * BMAX + b) * kStepThreads + tid] += S[j];
                __syncthreads();
            }
        }
        if (last_of_rg) {
            flush(up.rg);
            clear_acc();
        }
    };

    // Three register slots, each reloaded in place three units ahead (no copies between
    // slots, which would wait on loads still in flight).
    for (int x = x0; x < x1; x += 3) {
        process(s0, x);
        if (x + 3 < x1) { load_unit(s0, P, lcur, h, rho, tid); advance(lcur, P.Urg); }
        if (x + 1 < x1) {
            process(s1, x + 1);
            if (x + 4 < x1) { load_unit(s1, P, lcur, h, rho, tid); advance(lcur, P.Urg); }
        }
        if (x + 2 < x1) {
            process(s2, x + 2);
            if (x + 5 < x1) { load_unit(s2, P, lcur, h, rho, tid); advance(lcur, P.Urg); }
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

static inline bool a_ws_missing(const StepParams& P) { return P.a.ws == nullptr; }

template <typename XT, int RPL, int BMAX>
static hipError_t launch_step_t(StepParams P, hipStream_t s) {
    const int64_t cap = resident_capacity<XT, RPL, BMAX>();
    if (cap <= 0) return hipErrorInvalidConfiguration;
    // Never more workgroups than the device holds at once: the flag waits rely on it.
    int64_t G = P.a.workgroups > 0 ? P.a.workgroups : cap;
    G = G < cap ? G : cap;
    G = G < P.U ? G : P.U;
    P.G = (int)G;
    if ((uint64_t)P.U * (uint64_t)P.G >= (1ull << 32)) return hipErrorInvalidValue;  // 32-bit range math
    if (P.mode == kModeFirst && P.G == P.NRG) {
        P.mode = kModeStore;  // every workgroup holds exactly one whole row group: plain stores
    }
    // the arrival field counts contributors of a row group: at most Urg + 1 workgroups
    if (P.mode == kModeFirst && (a_ws_missing(P) || P.Urg + 1 > (int)kArrMask)) {
        hipError_t e = launch_fill_zero(P.a.y, (int64_t)P.a.batch * P.a.N, s);
        if (e != hipSuccess) return e;
        P.mode = kModeAtomic;
    }
    if (P.mode == kModeAdd && P.G != P.NRG) P.mode = kModeAtomic;
    hipLaunchKernelGGL((k_gemv8<XT, RPL, BMAX>), dim3((unsigned)P.G), dim3(kStepThreads), 0, s, P);
    return hipGetLastError();
}

// Instances: (row tiles per workgroup, batch bound) pairs whose registers fit without spills;
// max_rows_per_group() is the host-side rule that keeps requests inside this set.
template <typename XT>
static hipError_t launch_step_x(const StepParams& P, int rpl, hipStream_t s) {
    const int batch = P.a.batch;
    if (batch <= 1) {
        if (rpl >= 4) return launch_step_t<XT, 4, 1>(P, s);
        if (rpl >= 2) return launch_step_t<XT, 2, 1>(P, s);
        return launch_step_t<XT, 1, 1>(P, s);
    }
    if (batch <= 2) {
        if (rpl >= 2) return launch_step_t<XT, 2, 2>(P, s);
        return launch_step_t<XT, 1, 2>(P, s);
    }
    if (batch <= 4) return launch_step_t<XT, 1, 4>(P, s);
    if (batch <= 8) return launch_step_t<XT, 1, 8>(P, s);
    return launch_step_t<XT, 1, 16>(P, s);
}

int max_rows_per_group(int batch) { return batch <= 1 ? 4 : (batch <= 2 ? 2 : 1); }

hipError_t launch_step(const StepArgs& a, hipStream_t s) {
    StepParams P{};
    P.a = a;
    const int rpl = a.rows_per_group;
    P.NT = (int)ceil_div(a.N, kTileRows);
    P.NRG = (int)ceil_div(P.NT, rpl);
    P.Urg = 0;
    for (int i = 0; i < 2; ++i) {
        if (i < a.nseg) {
            P.KT[i] = (int)ceil_div(a.seg[i].Kv, kSliceCols);
            P.US[i] = (int)ceil_div((int64_t)P.KT[i] * a.seg[i].nb, 2);
        } else {
            P.KT[i] = 0;
            P.US[i] = 0;
        }
        P.Urg += P.US[i];
    }
    if ((int64_t)P.NRG * P.Urg > INT32_MAX / 1024) return hipErrorInvalidValue;
    P.U = P.NRG * P.Urg;
    P.mode = a.accumulate ? kModeAdd : kModeFirst;
    if (a.x_dtype == UBW_F16) return launch_step_x<__half>(P, rpl, s);
    return launch_step_x<float>(P, rpl, s);
}

}  // namespace ubw
