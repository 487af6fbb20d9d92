// HIP kernels for gfx950: packing, ternary encoding, LUT-BSF table build, pattern
// extraction and the table-lookup GEMV over decoupled row-column binary bases.
//
// Method: FluxBin (gist.science/ko/paper/2608.15602), technical summary, "2. Kernel
// innovation": tables with alpha_c folded in (LUT-BSF), virtual columnar mapping for the
// salient columns (VCM), and the execution flow stream packed uint32 -> extract pattern
// indices with bit operations -> fetch precomputed partial sums -> apply alpha_r.
//
// gfx950 mapping (the page's kernel targets another GPU; only its dataflow is kept):
//   - a workgroup of 512 threads works through a contiguous range of units (stream-K); a unit is
//     one or more 256-row tiles x two (256-column slice, base) items, one per half of each wave,
//     each lane owning one row of the tile;
//   - a group table has 256 fp32 entries, all in one LDS bank: entry p of group x of item h
//     lives at byte 256 p + 128 h + 4 x, so a unit's 64 tables fill one 64 KiB block and every
//     table sits in bank x;
//   - the lane with l = lane mod 32 reads group t ^ l at step t, and the packer stores each row's
//     words and bytes in the matching XOR order, so each half-wave touches 32 distinct banks per
//     lookup and the pattern byte sits where the lookup reads it;
//   - the lookup address is one v_perm_b32 that puts the weight byte (the pattern) in byte 1
//     and the lane's column offset for that step in byte 0;
//   - slices of one row are combined with fp32 atomics; when the caller asks for y = result, the
//     rows of each row group are initialized once per launch (by a zeroing workgroup with a lower
//     ID on the same XCD, or by the first workgroup to arrive) and the others wait for its flag
//     before adding (atomics only, no fences), so one launch does the whole step;
//   - no MFMA in this file: the work is a memory-bound table-lookup reduction (larger batches
//     go to the matrix-core kernel in mfma.hip).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <type_traits>

#include "../../include/ubw.h"
#include "ubw_internal.h"

namespace ubw {

typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) const char lds_cchar;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// Element i of an activation block held in LDS, as fp32.
template <typename XT>
__device__ __forceinline__ float lds_x(lds_cchar* base, uint32_t i);
template <>
__device__ __forceinline__ float lds_x<float>(lds_cchar* base, uint32_t i) {
    return *(const __attribute__((address_space(3))) float*)(base + 4 * i);
}
template <>
__device__ __forceinline__ float lds_x<__half>(lds_cchar* base, uint32_t i) {
    const unsigned short v = *(const __attribute__((address_space(3))) unsigned short*)(base + 2 * i);
    return __half2float(__builtin_bit_cast(__half, v));
}

// ---------------------------------------------------------------------------------------
// Small helpers shared by several kernels.

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__half v) { return __half2float(v); }

// Order of the lane that owns tile row rho: slot s holds word s ^ a, byte jj of a slot holds
// byte jj ^ c of that word.
__device__ __forceinline__ int xor_words(int rho) { return (rho & 31) >> 2; }
__device__ __forceinline__ int xor_bytes(int rho) { return rho & 3; }

// Bytes of a canonical word in the order of the row that owns it: byte jj = byte jj ^ c.
__device__ __forceinline__ uint32_t bytes_for_row(uint32_t v, int c) {
    const uint32_t sel = 0x03020100u ^ (0x01010101u * (uint32_t)c);
    return __builtin_amdgcn_perm(0u, v, sel);
}

// Per-lane column offsets of the 32 steps, four per register: byte jj of lc[i] is
// 4 * ((4 i + jj) ^ l), the byte offset of the group the lane reads at step 4 i + jj.
__device__ __forceinline__ void lane_columns(int l, uint32_t lc[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t v = 0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) v |= (uint32_t)(4 * ((4 * i + jj) ^ l)) << (8 * jj);
        lc[i] = v;
    }
}

// Address of the step 4 i + jj lookup: byte 0 = the lane's column offset for that step (byte
// jj of lc), byte 1 = the pattern (byte jj of slot i), bytes 2-3 zero. So the result is
// 256 * pattern + 4 * group.
template <int JJ>
__device__ __forceinline__ uint32_t perm_addr(uint32_t A, uint32_t lc) {
    return __builtin_amdgcn_perm(A, lc, 0x0C0C0000u | ((4u + JJ) << 8) | (uint32_t)JJ);
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

__device__ __forceinline__ float half_bits_to_f32(uint32_t h) {
    return __half2float(__ushort_as_half((unsigned short)h));
}

// Two slots' lookups (8 table reads) added into s[0..3]: all 8 addresses, then all 8 reads, then
// the adds, written in that order. Where the kernel's scalar registers run over their budget
// the compiler's scheduler keeps a region in source order; in this order 8 reads are in flight
// at once even then (read-add pairs one at a time would each wait out the LDS latency).
__device__ __forceinline__ void lookup_pair(lds_cchar* tb, uint32_t wa, uint32_t wb, uint32_t la, uint32_t lb,
                                            float s[4]) {
    const uint32_t ad[8] = {perm_addr<0>(wa, la), perm_addr<1>(wa, la), perm_addr<2>(wa, la), perm_addr<3>(wa, la),
                            perm_addr<0>(wb, lb), perm_addr<1>(wb, lb), perm_addr<2>(wb, lb), perm_addr<3>(wb, lb)};
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = *(const lds_f32*)(tb + ad[e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e & 3] += t[e];
}

// Sums over the 32 groups of one row's slice for one base: step t = 4 i + jj reads the table
// of group t ^ l at the pattern in byte jj of slot i. lo gets steps 0..15 (groups of the
// 128-column half (l >> 4) of the slice), hi steps 16..31 (the other half).
// tb points at the base's half of the table block.
__device__ __forceinline__ void lookup_halves(lds_cchar* tb, const uint4& w0, const uint4& w1, const uint32_t lc[8],
                                              float& lo, float& hi) {
    const uint32_t W[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float s[2][4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        s[half][0] = s[half][1] = s[half][2] = s[half][3] = 0.f;
#pragma unroll
        for (int i = 4 * half; i < 4 * half + 4; i += 2) lookup_pair(tb, W[i], W[i + 1], lc[i], lc[i + 1], s[half]);
    }
    lo = (s[0][0] + s[0][1]) + (s[0][2] + s[0][3]);
    hi = (s[1][0] + s[1][1]) + (s[1][2] + s[1][3]);
}

// The whole slice: one sum over the 32 groups.
__device__ __forceinline__ float lookup_row(lds_cchar* tb, const uint4& w0, const uint4& w1, const uint32_t lc[8]) {
    const uint32_t W[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; i += 2) lookup_pair(tb, W[i], W[i + 1], lc[i], lc[i + 1], s);
    return (s[0] + s[1]) + (s[2] + s[3]);
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
    int c;             // byte order of the row (bytes_for_row)
};

__device__ __forceinline__ PackPos pack_pos(int64_t o, int nb, int KT) {
    const int e = (int)(o & 3);
    const int rho = (int)((o >> 2) & 255);
    const int q = (int)((o >> 10) & 1);
    // o < 2^39 (the host caps the packed size at INT_MAX * 256 words): the tile index fits 32 bits
    const uint32_t rest = (uint32_t)(o >> 11);
    const int k = (int)(rest % (uint32_t)nb);
    const uint32_t tile = rest / (uint32_t)nb;
    const int ks = (int)(tile % (uint32_t)KT);
    const int rt = (int)(tile / (uint32_t)KT);
    const int s = 4 * q + e;
    const int wi = s ^ xor_words(rho);
    return PackPos{k, rt * kTileRows + rho, ks * kSliceWords + wi, xor_bytes(rho)};
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
    dst[o] = bytes_for_row(val, p.c);
}

// Bits of 32 int8 values of a row (columns c0 .. c0 + 31; columns >= K read as bit 0): bit b is
// v > 0 (ge = false) or v >= 0 (ge = true). Whole, aligned 32-byte runs are read as two 16-byte
// loads (four threads cover 128 contiguous bytes of a row), ragged ones byte by byte.
__device__ __forceinline__ uint32_t int8_bits(const int8_t* r, int c0, int K, bool ge) {
    uint32_t val = 0;
    if (c0 + 32 <= K && (reinterpret_cast<uintptr_t>(r + c0) & 15u) == 0) {
        const uint4 a = *reinterpret_cast<const uint4*>(r + c0);
        const uint4 b = *reinterpret_cast<const uint4*>(r + c0 + 16);
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int8_t v = (int8_t)(w[i >> 2] >> (8 * (i & 3)));
            if (ge ? v >= 0 : v > 0) val |= 1u << i;
        }
        return val;
    }
    for (int i = 0; i < 32; ++i) {
        const int col = c0 + i;
        if (col < K) {
            const int8_t v = r[col];
            if (ge ? v >= 0 : v > 0) val |= 1u << i;
        }
    }
    return val;
}

__global__ void k_pack_int8(const int8_t* __restrict__ src, int nb, int N, int K, int KT, int64_t total,
                            uint32_t* __restrict__ dst) {
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= total) return;
    const PackPos p = pack_pos(o, nb, KT);
    uint32_t val = 0;
    if (p.row < N) val = int8_bits(src + ((int64_t)p.k * N + p.row) * K, p.wcol * 32, K, false);
    dst[o] = bytes_for_row(val, p.c);
}

// Ternary weights as two half-scale bases: base 0 bit = (w >= 0), base 1 bit = (w > 0), so
// w = +1 -> (+1,+1), w = -1 -> (-1,-1), w = 0 -> (+1,-1).
__global__ void k_ternary_bits(const int8_t* __restrict__ w, int N, int K, int KT, int64_t total,
                               uint32_t* __restrict__ dst) {
    // one thread per base-0 word; the base-1 word at the same position is in the next tile
    // (tiles of one slice are [base][...] adjacent), and both come from the same 32 bytes
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t o = ((t >> 11) << 12) | (t & 2047);  // tile pair t / 2048, word t % 2048 of base 0
    if (o >= total) return;
    const PackPos p = pack_pos(o, 2, KT);
    uint32_t v0 = 0, v1 = 0;
    if (p.row < N) {
        const int8_t* r = w + (int64_t)p.row * K;
        v0 = int8_bits(r, p.wcol * 32, K, true);
        v1 = int8_bits(r, p.wcol * 32, K, false);
    }
    dst[o] = bytes_for_row(v0, p.c);
    dst[o + kTileWords] = bytes_for_row(v1, p.c);
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
    const uint32_t W[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    uint32_t lc[8];
    lane_columns(rho & 31, lc);
    const int ng = (K + 7) / 8;
    uint16_t* o = out + ((int64_t)k * N + row) * ng;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t A = W[i];
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
    const int a = xor_words(rho), c = xor_bytes(rho);
    const int ng = (K + 3) / 4;
    uint16_t* o = out + ((int64_t)k * N + row) * ng;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int wi = s ^ a;
#pragma unroll
        for (int n = 0; n < 8; ++n) {  // nibble n of the word: nibble n & 1 of stored byte (n >> 1) ^ c
            const int gi = ks * 64 + wi * 8 + n;
            if (gi < ng) o[gi] = (uint16_t)((S[s] >> (8 * ((n >> 1) ^ c) + 4 * (n & 1))) & 15u);
        }
    }
}

// ---------------------------------------------------------------------------------------
// The GEMV step (g = 8): a persistent, stream-K style kernel.
//
// Work list: the units of segment 0 (the main bases) row group by row group, then those of
// segment 1 (the salient refinement, if any) row group by row group. For each row group (RPL
// tiles of 256 rows) a segment's items are its (slice, base) pairs, slice-major; a unit is two
// consecutive items, one per half of every wave: lane l of half h in wave w owns tile row
// 32 w + l for item h. Workgroup g of G takes units [g U / G, (g + 1) U / G): at most one run
// of main units and one run of refinement units, each processed by its own loop, so that every
// unit of a loop reads its activations the same way. Per-row partial sums stay in registers
// across consecutive units of one row group and go into y with fp32 atomics when the run leaves
// that row group.
// Per unit and activation row b: stage v = alpha_c * x for both items, build each item's 32
// tables (half h writes LDS columns 32 h .. 32 h + 31), barrier, look up every owned row,
// accumulate alpha_r * sum, barrier. The two halves of a row (different items) are added with a
// cross-lane swap when flushing. The next unit's data are in flight while a unit is processed
// (two register slots, reloaded in place).
//
// y = result in one launch (kModeFirst, with a workspace). Per row group, 256 bytes of
// workspace: word 0 counts arrivals, (generation << 12) | units announced in this launch, and
// word 32 (the flag) counts the launches that initialized the row group's rows of y; between
// launches both hold the same count. A workgroup announces its units of a row group with one
// atomic add when it starts on them, and adds into y only after it has seen the flag raised for
// this launch (one past the generation its add returned), unless it initialized the rows
// itself; the participant whose add brings the arrivals to the row group's total resets the
// field and advances the generation. Two ways to initialize (zero) the rows:
//  * XCD-local mode (8 or more row groups and workgroups): the dispatcher deals a launch's
//    workgroups out to the eight XCDs in turn (workgroup g runs on XCD g mod 8) and allocates
//    each XCD's share in ID order. Row group rg is worked on only by workgroups on XCD rg mod 8,
//    and zeroed by workgroup rg, which has no units, runs on that XCD and has a lower ID than
//    every workgroup that adds into it: whenever one of those waits, workgroup rg has been
//    allocated, and it zeroes the rows with device-scope atomic stores, waits until they are
//    acknowledged and raises the flag without waiting for anything else. No zeroing waits for
//    an atomic's answer first.
//  * First-arriver mode (otherwise, e.g. grouped launches): the value the add returns says
//    whether the workgroup arrived first, and the first arriver initializes the rows. A
//    candidate (an arriver without units, or a run that starts among the row group's first
//    units) makes its add before its loads and looks at the answer right away: if first, wave 0
//    zeroes the rows, waits for the stores and raises the flag. Any other workgroup looks at
//    the answer only at its flush and, if it did arrive first, writes its own partial sums there
//    with atomic stores (every row of the row group) and then raises the flag. The first arriver is
//    running (it made the add) and raises the flag without waiting for any other workgroup;
//    every waiter arrived after it.
// Either way nothing depends on how many workgroups the device holds at once, so launches on
// other streams (with their own workspaces) cannot stall the protocol. A bounded spin still
// guards each wait: if it ever ran out, the workgroup would set bit 0 of workspace word 0 and
// add nothing.

enum { kModeStore = 0, kModeAtomic = 2, kModeFirst = 3 };
constexpr int kSpinLimit = 1 << 20;
constexpr int kStepThreads = 512;
constexpr uint32_t kArrBits = 12;
constexpr uint32_t kArrMask = (1u << kArrBits) - 1u;
constexpr uint32_t kGenMask = (1u << (32 - kArrBits)) - 1u;

// Division by a divisor fixed for the launch (plan.h).
using plan::FastDiv;
using plan::div_by;
using plan::fast_div;

struct StepParams {
    StepArgs a;
    int NT;
    int NRG;          // row groups
    int KT[2];        // slices per segment
    int US[2];        // units per row group per segment
    int Urg;          // units per row group, both segments
    int U;            // units in the whole list (< 2^31)
    int G;            // workgroups: Zn arrivers without units (IDs 0 .. Zn - 1), then Gu with units
    int Gu;           // workgroups with units
    int Zn;           // arrivers without units, one per row group (0 or NRG)
    int Arr;          // arrivals that complete a row group: Urg, plus 1 when Zn > 0
    int mode;
    int xmode;        // 1: XCD-local row groups with static zeroing (see step_body), 0: first arriver
    FastDiv dUS[2];   // division by US[si]
    FastDiv dNb[2];   // division by seg[si].nb
};

// XL: the refinement segment gathers x through LDS (the whole activation block, at most
// kXlBytes, is loaded with the unit and the gather reads it there), so its units wait for one
// memory round trip instead of two (idx, then x at idx).
constexpr uint32_t kXlBytes = 16 * kStepThreads;
template <typename XT, int RPL, int BMAX, bool XL>
struct Unit {
    uint4 w[RPL][2];   // this lane's item: its rows' 8 words (two 16-byte halves of the slice)
    float ar[RPL];     // alpha_r of the item's base at the lane's rows (with group scales: the two
                       // fp16 scales of the item's slice at those rows, low half first)
    float ac;          // staging: alpha_c of the staged item's base at the staged column
    XT xv[BMAX];       // staging: activations of the staged column (0 for rows >= batch)
    uint4 xb;          // XL: this thread's 16 bytes of the activation block
    uint32_t xc;       // idx of the staged column (XL: read at staging; otherwise at the gather, one
                       // unit later, so nothing waits for it at the load)
    uint32_t xp;       // idx of the column before it (for the ascending-order check)
    uint32_t xf;       // without XL: bit 0 the staged column is valid, bit 1 it is not column 0
};

// A unit within its segment's part of the list: row group, unit within the row group, and the
// slice and base of the unit's first item (item 2 q), kept incrementally so that walking the
// list needs no division.
struct Cursor {
    int rg, q, ks, k;
};

__device__ __forceinline__ Cursor cursor_at(uint32_t u, int US, FastDiv dUS, int nb, FastDiv dNb) {
    Cursor cu;
    cu.rg = (int)div_by(u, dUS);
    cu.q = (int)(u - (uint32_t)cu.rg * (uint32_t)US);
    cu.ks = (int)div_by(2u * (uint32_t)cu.q, dNb);
    cu.k = 2 * cu.q - cu.ks * nb;
    return cu;
}

__device__ __forceinline__ void advance(Cursor& cu, int US, int nb) {
    if (++cu.q == US) {
        cu.q = 0;
        cu.ks = 0;
        cu.k = 0;
        ++cu.rg;
        return;
    }
    cu.k += 2;  // two items on; nb may be 1
    if (cu.k >= nb) { cu.k -= nb; ++cu.ks; }
    if (cu.k >= nb) { cu.k -= nb; ++cu.ks; }
}

// Slice and base of item 2 q + d (d = 0 or 1) of the cursor's unit.
__device__ __forceinline__ void item_of(const Cursor& cu, int d, int nb, int& ks, int& k) {
    k = cu.k + d;
    ks = cu.ks;
    if (k >= nb) { k -= nb; ++ks; }
}

// Raw buffer access: a load whose offset lies at or beyond the descriptor's size returns 0 and
// touches no memory. Every buffer the step reads is below 2 GiB (checked on the host), so
// kOob is out of range for all of them, and a descriptor of size 0 turns all its loads off.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;
// Descriptor fields must sit in scalar registers. Every caller passes values that are uniform
// over the workgroup, but some are computed on the vector unit (divisions, 64-bit products), where
// the compiler cannot prove it and would wrap each load in a loop over distinct descriptors;
// readfirstlane states the uniformity.
__device__ __forceinline__ Rsrc make_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* base = (void*)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ float buf_f32(Rsrc r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint4 buf_u128(Rsrc r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void buf_x(Rsrc r, uint32_t off, float& v) { v = buf_f32(r, off); }
__device__ __forceinline__ void buf_x(Rsrc r, uint32_t off, __half& v) {
    v = __builtin_bit_cast(__half, __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
}

// Requests one unit of segment SI (1: the columns go through idx). Every load is issued on every
// path, out-of-range items, rows and columns reading 0 through the buffer bounds, so the
// compiler's waits stay exact: a unit waits for its own data only, never for the units requested
// after it. Order: alpha_c and x first (for idx segments: idx, alpha_c and, with XL, the whole
// activation block), so the tables can be built while the weights are still arriving; then the
// weights and alpha_r; for idx segments without XL the gather of x follows later (gather_unit),
// once idx is in. A unit past the run (!valid) issues the
// same loads through empty descriptors: they read nothing. (Branching around them instead
// makes the compiler merge two register assignments with copies that wait for everything.)
// Per-lane constants of the loads, computed once: a unit's offsets are then a scalar (uniform)
// part plus one of these, so each unit costs a handful of vector instructions.
struct LaneC {
    uint32_t sd;      // staged item within the unit (tid / 256): uniform over a wave
    uint32_t colL;    // staged column within the slice (tid mod 256)
    uint32_t hsel;    // lookup item within the unit (half of the wave)
    uint32_t wl;      // byte offset of this lane's row in its item's tile, item 2 q + h relative to 2 q
    uint32_t rho;     // tile row
    int rgo, rgs;     // row group rgo + rgs * rg for a cursor's rg (this workgroup's row groups)
};

template <int SI, bool XL, bool GS, typename XT, int RPL, int BMAX>
__device__ __forceinline__ void load_unit(Unit<XT, RPL, BMAX, XL>& U, const StepParams& P, Cursor cu, bool valid,
                                          const LaneC& lcn, int tid) {
    const StepArgs& a = P.a;
    const Segment& sg = a.seg[SI];
    const int nitems = P.KT[SI] * sg.nb;
    const uint32_t xs = sizeof(XT);
    const uint32_t ldx = (uint32_t)a.ldx;
    const Rsrc r_x = make_rsrc(a.x, valid ? (uint32_t)a.batch * ldx * xs : 0u);
    // the unit's two items (slice, base): item 2 q and item 2 q + 1
    int ks1, k1;
    item_of(cu, 1, sg.nb, ks1, k1);
    // staging role: column (tid mod 256) of item 2 q + tid / 256 (scalar per wave)
    const int sks = lcn.sd ? ks1 : cu.ks, sk = lcn.sd ? k1 : cu.k;
    const bool its_ok = 2 * cu.q + (int)lcn.sd < nitems;
    const uint32_t colBase = (uint32_t)sks * kSliceCols;
    const bool cvalid = its_ok && colBase + lcn.colL < (uint32_t)sg.Kv;
    // idx of the staged column and of the one before it (for the checks), loaded straight into
    // the unit (a copy of a value still in flight would wait for it) and checked where they are
    // used: at staging with XL, otherwise at the gather (gather_unit)
    const uint32_t col = colBase + lcn.colL;
    if constexpr (SI == 1) {
        const Rsrc r_idx = make_rsrc(sg.idx, valid ? (uint32_t)sg.Kv * 4u : 0u);
        const int ioff = (int)(cvalid ? col * 4u : kOob);
        const int poff = (int)(cvalid && col > 0 ? col * 4u - 4u : kOob);
        U.xc = __builtin_amdgcn_raw_buffer_load_b32(r_idx, ioff, 0, 0);
        U.xp = __builtin_amdgcn_raw_buffer_load_b32(r_idx, poff, 0, 0);
        if constexpr (!XL) U.xf = (valid && cvalid ? 1u : 0u) | (col > 0 ? 2u : 0u);
    }
    const uint32_t acBase = ((uint32_t)sk * (uint32_t)sg.Kv + colBase) * 4u;
    U.ac = buf_f32(make_rsrc(sg.alpha_c, valid ? (uint32_t)sg.nb * (uint32_t)sg.Kv * 4u : 0u),
                   cvalid ? acBase + lcn.colL * 4u : kOob);
    if constexpr (SI == 0) {
#pragma unroll
        for (int b = 0; b < BMAX; ++b)
            buf_x(r_x, cvalid ? ((uint32_t)b * ldx + colBase) * xs + lcn.colL * xs : kOob, U.xv[b]);
    } else if constexpr (XL) {
        U.xb = buf_u128(r_x, 16u * (uint32_t)tid);  // before the weights, like x in the main segment
    }
    // lookup role: item 2 q + h for tile row rho
    const bool lval = 2 * cu.q + (int)lcn.hsel < nitems;
    const uint32_t slab = (uint32_t)nitems * kTileWords * 4u;  // one row tile: all slices and bases
    const uint32_t woff = lval ? (uint32_t)cu.q * (2u * kTileWords * 4u) + lcn.wl : kOob;
    // alpha_r: one fp32 per row, or (group scales) the two fp16 scales of the item's slice,
    // stored [nb][KT][N][2] so that consecutive rows (lanes) read consecutive 4-byte words
    constexpr bool gsc = SI == 0 && GS;
    const uint32_t kh = lcn.hsel ? (uint32_t)k1 : (uint32_t)cu.k;
    const uint32_t arRow = gsc ? kh * (uint32_t)P.KT[0] + (uint32_t)(lcn.hsel ? ks1 : cu.ks) : kh;
    const uint32_t arBase = arRow * (uint32_t)a.N * 4u;
    const Rsrc r_ar =
        make_rsrc(sg.alpha_r, valid ? (uint32_t)sg.nb * (gsc ? (uint32_t)P.KT[0] : 1u) * (uint32_t)a.N * 4u : 0u);
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
        const int rt = (lcn.rgo + lcn.rgs * cu.rg) * RPL + j;
        const Rsrc r_w = make_rsrc(sg.packed + (int64_t)rt * nitems * kTileWords, valid && rt < P.NT ? slab : 0u);
        U.w[j][0] = buf_u128(r_w, woff);
        U.w[j][1] = buf_u128(r_w, lval ? woff + kTileRows * 16u : kOob);
        const uint32_t row = (uint32_t)rt * kTileRows + lcn.rho;
        U.ar[j] = buf_f32(r_ar, lval && row < (uint32_t)a.N ? arBase + row * 4u : kOob);
    }
}

// The refinement's activations without XL: x at the staged column's index, loaded once idx has
// arrived. It is issued while the unit before is processed (after that unit's staging), so no
// load waits for idx: a gather issued with the unit's own loads waited for idx at once, one
// memory round trip per refinement unit. VCM: the index must lie in [0, K) and exceed the one
// before it (ascending, distinct); either fault sets bit 1 of workspace word 0, and a column
// outside [0, K) reads nothing (x = 0, so it contributes nothing; one out of order still adds
// x[idx]).
template <typename XT, int RPL, int BMAX, bool XL>
__device__ __forceinline__ void gather_unit(Unit<XT, RPL, BMAX, XL>& U, const StepParams& P) {
    static_assert(!XL, "with XL the gather reads the activation block in LDS at staging");
    const StepArgs& a = P.a;
    const uint32_t ldx = (uint32_t)a.ldx;
    const uint32_t xs = sizeof(XT);
    const bool cvalid = (U.xf & 1u) != 0;
    const bool bad = cvalid && (U.xc >= ldx || ((U.xf & 2u) != 0 && (int)U.xp >= (int)U.xc));
    if (bad && a.ws != nullptr) atomicOr(a.ws, kWsErrIndex);
    const bool use = cvalid && U.xc < ldx;
    const Rsrc r_x = make_rsrc(a.x, (uint32_t)a.batch * ldx * xs);
#pragma unroll
    for (int b = 0; b < BMAX; ++b) buf_x(r_x, use ? ((uint32_t)b * ldx + U.xc) * xs : kOob, U.xv[b]);
}

// The body of a step: workgroup g of the P.G that work on the GEMV described by P.
template <typename XT, int RPL, int BMAX, bool XL, bool GS>
__device__ __forceinline__ void step_body(const StepParams& P, int g) {
    // Per-row partial sums live in registers, one per (row tile, activation row): the batch
    // loops below are unrolled over BMAX (at most kBatchChunk) with a runtime bound, so every
    // index is a constant.
    static_assert(BMAX <= kBatchChunk, "larger batches run as chunks");
    __shared__ __align__(16) float s_tab[256 * 64];       // one unit's 64 tables: 64 KiB
    __shared__ __align__(16) float s_v[BMAX * 2 * 256];   // scaled activations [b][item][column]
    lds_f32* tab = (lds_f32*)s_tab;
    lds_f32* sv = (lds_f32*)s_v;
    lds_cchar* tb = (lds_cchar*)s_tab;
    const StepArgs& a = P.a;
    // The parameter block spans four 64-byte lines of the scalar cache, and every fetch of a
    // missing line costs a full trip to where the runtime keeps kernel arguments. Asking for one
    // word of each line here puts all four fetches in one batch instead of letting them
    // trickle in as first used (one wait instead of several).
    static_assert(sizeof(StepParams) <= 256, "parameter block grew: touch its new lines");
    static_assert(offsetof(StepParams, dNb) >= 192, "one touched word per 64-byte line");
    asm volatile("" ::"s"(P.a.seg[0].nb), "s"(P.a.N), "s"(P.NRG), "s"(P.dNb[1].sh));

    const int tid = threadIdx.x;
    const int wv = tid >> 6, L = tid & 63;
    const int h = L >> 5, l = L & 31;
    const int rho = 32 * wv + l;                  // tile row of this lane
    const bool l_hi = (l & 16) != 0;              // its first 16 lookup steps are the slice's upper half
    const int p0 = 32 * wv;                       // table entries this lane builds
    uint32_t lc[8];
    lane_columns(l, lc);
    LaneC lcn;
    lcn.sd = (uint32_t)__builtin_amdgcn_readfirstlane(tid >> 8);
    lcn.colL = (uint32_t)(tid & 255);
    lcn.hsel = (uint32_t)h;
    lcn.wl = (uint32_t)h * (kTileWords * 4u) + 16u * (uint32_t)rho;
    lcn.rho = (uint32_t)rho;
#pragma unroll
    for (int i = 0; i < 8; ++i) lc[i] += 0x80808080u * (uint32_t)h;  // half h's tables: +128 bytes

    // y = result protocol (kModeFirst; see the comment above kModeStore)
    const bool first_mode = P.mode == kModeFirst;
    auto rg_word = [&](int grg) { return a.ws + kWsHeaderWords + kWsRowGroupWords * grg; };
    __shared__ uint32_t s_fm;  // flush mode from thread 0: bit 0 add nothing, bit 1 initialize y
    // The flag of row group grg: the count of launches that initialized its rows.
    auto read_flag = [&](int grg) -> uint32_t {
        return __hip_atomic_load(rg_word(grg) + kWsFlagOffset, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // Wait until every memory operation this wave issued has completed (for stores: been
    // acknowledged); vmcnt(0), the other counters left alone.
    auto wait_stores = []() { __builtin_amdgcn_s_waitcnt(0x0F70); };
    auto raise_flag = [&](int grg) {
        __hip_atomic_fetch_add(rg_word(grg) + kWsFlagOffset, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // Wave 0 of a row group's zeroing workgroup: y = 0 on every row of row group grg (all
    // activation rows) with device-scope atomic stores, wait until all have been acknowledged
    // (each has then been performed where the adds are), raise the flag. (Exchanges, which must
    // read each cold line first, took ~6.5 us under a full device's loads.)
    auto zero_rows = [&](int grg) {
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            const int rt = grg * RPL + j;
#pragma unroll
            for (int q = 0; q < kTileRows / 64; ++q) {
                const int row = rt * kTileRows + 64 * q + L;
                const bool rv = rt < P.NT && row < a.N;
#pragma unroll
                for (int b = 0; b < BMAX; ++b)
                    if (rv && b < a.batch)
                        __hip_atomic_store(a.y + (int64_t)b * a.N + row, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        wait_stores();
        if (L == 0) raise_flag(grg);
    };

    // The first Zn workgroups have no units. XCD-local mode: workgroup g < NRG zeroes row group g
    // at once and raises its flag (it runs on XCD g mod 8, with every workgroup that adds into row
    // group g, and has a lower ID than all of them). First-arriver mode: it announces one arrival
    // at row group g, zeroes its rows if first, and completes the row group if last.
    if (g < P.Zn) {
        if (wv == 0 && g < P.NRG) {
            if (P.xmode) {
                zero_rows(g);
            } else {
                uint32_t arr = 0;
                if (L == 0) arr = atomicAdd(rg_word(g), 1u);
                arr = __builtin_amdgcn_readfirstlane(arr);
                if ((arr & kArrMask) == 0) zero_rows(g);
                if (L == 0 && (arr & kArrMask) + 1u == (uint32_t)P.Arr)
                    atomicAdd(rg_word(g), (1u << kArrBits) - (uint32_t)P.Arr);
            }
        }
        return;
    }

    // The row groups this workgroup works on and its range of units. XCD-local mode: workgroup g
    // runs on XCD g mod 8 (the dispatcher deals a launch's workgroups out to the eight XCDs in
    // turn) and works only on the row groups rg = g mod 8, g mod 8 + 8, ..., as rank g / 8 of that
    // XCD's workgroups, over a unit list of those row groups alone; otherwise on every row group
    // as rank g - Zn. Either way the list holds the main units row group by row group, then the
    // refinement units, and rank r takes an equal contiguous range (the first ones one unit more).
    // A cursor's rg counts the listed row groups; it is row group rgo + rgs * rg of the matrix.
    const plan::WgRange wr = plan::wg_range(g, P.Zn, P.Gu, P.NRG, P.Urg, P.xmode != 0);
    lcn.rgo = wr.rgo;
    lcn.rgs = wr.rgs;
    const int NRGx = wr.NRGx;
    auto grg = [&](int rg) { return lcn.rgo + lcn.rgs * rg; };
    const uint32_t Qx = (uint32_t)NRGx * (uint32_t)P.Urg / (uint32_t)wr.Gx;
    const uint32_t x0 = wr.x0, x1 = wr.x1;
    const uint32_t Um = (uint32_t)NRGx * (uint32_t)P.US[0];  // units of segment 0 in the list

    float acc[RPL][BMAX];
    auto clear_acc = [&]() {
#pragma unroll
        for (int j = 0; j < RPL; ++j)
#pragma unroll
            for (int b = 0; b < BMAX; ++b) acc[j][b] = 0.f;
    };
    clear_acc();

    // Row-group bookkeeping (thread 0, except `zeroed`, which wave 0 sets): the arrival counter's
    // value returned on entry, the units this workgroup adds to it, the flag as read on entry and,
    // if that read did not find it raised, as read again before the last lookups of the run (kept
    // apart so that a flush after a successful first read does not wait for the loads issued after
    // it), and whether this workgroup has zeroed the row group's rows (first-arriver mode).
    uint32_t arrived = 0, units_in = 0, seen = 0, seen_late = 0;
    bool late = false, zeroed = false;
    auto want = [&]() { return ((arrived >> kArrBits) + 1) & kGenMask; };
    // whether this workgroup adds into row group rg without waiting for its flag (it initializes it)
    auto no_wait = [&](int) { return !P.xmode && (arrived & kArrMask) == 0; };
    // Entering row group rg with n of its units to process: add n to its arrival field and take a
    // first look at its flag.
    auto enter = [&](int rg, uint32_t n) {
        zeroed = false;
        if (first_mode && tid == 0) {
            units_in = n;
            arrived = atomicAdd(rg_word(grg(rg)), n);
            seen = read_flag(grg(rg));
        }
    };
    // First-arriver mode, after an entry at the start of a run (its add the oldest memory
    // operation of the run): if this workgroup arrived first, wave 0 zeroes the rows now.
    auto zero_if_first = [&](int rg) {
        if (first_mode && wv == 0) {
            const uint32_t arr = __builtin_amdgcn_readfirstlane(arrived);
            if ((arr & kArrMask) == 0) {
                zero_rows(grg(rg));
                zeroed = true;
            }
        }
    };

    // Add this workgroup's partial sums of row group rg into y.
    auto flush = [&](int rg) {
        uint32_t fm = 0;
        const int gr = grg(rg);
        if (first_mode) {
            if (tid == 0) {
                uint32_t m = 0;
                if (no_wait(rg)) {
                    if (!P.xmode && !zeroed) m = 2;  // arrived first mid-run: initialize y with these sums
                } else {
                    const uint32_t wnt = want();
                    uint32_t cur = seen;
                    if (late) {
                        asm volatile("");  // keeps this a branch: only this path waits for seen_late
                        cur = seen_late;
                    }
                    int n = 0;
                    while ((cur & kGenMask) != wnt) {
                        if (++n > kSpinLimit) {  // the zeroer raises it; never hang regardless
                            atomicOr(a.ws, kWsErrWait);
                            m = 1;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                        cur = read_flag(gr);
                    }
                }
                late = false;
                const uint32_t total = (uint32_t)P.Arr;
                if ((arrived & kArrMask) + units_in == total)  // completes it: arrivals 0, next generation
                    atomicAdd(rg_word(gr), (1u << kArrBits) - total);
                s_fm = m;
            }
            __syncthreads();
            fm = __builtin_amdgcn_readfirstlane(s_fm);  // uniform: the branches below are scalar
        }
        if (fm & 1u) return;  // a wait gave up: add nothing (workspace word 0 says so)
        // The row sums (the two halves of each row added across the wave) go out in one of three
        // ways, each a loop of its own, so that no path carries another's waits (a value returned
        // by an atomic that could reach the other paths made every flush wait for all loads in
        // flight, the units requested ahead).
        auto put = [&](auto out) {
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                const int rt = gr * RPL + j;
                const int row = rt * kTileRows + rho;
                const bool rv = rt < P.NT && row < a.N;
#pragma unroll
                for (int b = 0; b < BMAX; ++b) {
                    if (b >= a.batch) continue;
                    const uint32_t pv = __float_as_uint(acc[j][b]);
                    const auto sw = __builtin_amdgcn_permlane32_swap(pv, pv, false, false);
                    const float total = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
                    if (h == 0 && rv) out(a.y + (int64_t)b * a.N + row, total);
                }
            }
        };
        if (fm & 2u) {  // every row of the row group written with atomic stores, then the flag raised
            put([](float* dst, float v) { __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); });
            wait_stores();  // all of them acknowledged
            __syncthreads();
            if (tid == 0) raise_flag(gr);
        } else if (P.mode == kModeStore) {
            put([](float* dst, float v) { *dst = v; });
        } else {
            put([](float* dst, float v) { atomicAdd(dst, v); });
        }
    };

    // One activation row of one unit: build the tables, barrier, look up.
    auto row_pass = [&](const Unit<XT, RPL, BMAX, XL>& U, bool mine, bool last, int rg, int b, auto gs_c,
                        float S[RPL]) {
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
        // before the lookups that end a row group, look at its flag again if the look on entry
        // did not find it raised (the read then overlaps the lookups)
        if (first_mode && last && tid == 0 && b == 0 && !no_wait(rg) && (seen & kGenMask) != want()) {
            seen_late = read_flag(grg(rg));
            late = true;
        }
        if constexpr (decltype(gs_c)::value) {
            // group scales: the first 16 steps of a lane cover the 128-column half (l >> 4) of the
            // slice, the last 16 the other half
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                float lo, hi;
                lookup_halves(tb, U.w[j][0], U.w[j][1], lc, lo, hi);
                const uint32_t pr = __float_as_uint(U.ar[j]);
                const float a0 = half_bits_to_f32(pr & 0xFFFFu), a1 = half_bits_to_f32(pr >> 16);
                // a half past column K sums to exactly 0 and its scale (padding) is not read
                const float pa = lo != 0.f ? (l_hi ? a1 : a0) * lo : 0.f;
                const float pb = hi != 0.f ? (l_hi ? a0 : a1) * hi : 0.f;
                S[j] = mine ? pa + pb : 0.f;
            }
        } else {
#pragma unroll
            for (int j = 0; j < RPL; ++j) S[j] = mine ? U.ar[j] * lookup_row(tb, U.w[j][0], U.w[j][1], lc) : 0.f;
        }
    };

    // One unit: stage, then one table build + lookup pass per activation row; flush if it is
    // the last unit of its row group in this run.
    auto process = [&](const Unit<XT, RPL, BMAX, XL>& U, int nitems, Cursor cu, bool last, auto si_c,
                       auto&& after_stage) {
        constexpr int SI = decltype(si_c)::value;
        const bool mine = 2 * cu.q + h < nitems;  // this half has an item in this unit
        // scaled activations of both items: v = alpha_c * x (LUT-BSF folds alpha_c here)
        if constexpr (SI == 1 && XL) {
            // VCM: the staged column's index must lie in [0, K) and exceed the one before it
            // (ascending, distinct); either fault sets bit 1 of workspace word 0, and a column
            // outside [0, K) contributes nothing (one out of order still adds x[idx])
            const uint32_t ldx = (uint32_t)a.ldx;
            int sks, sk;
            item_of(cu, (int)lcn.sd, a.seg[1].nb, sks, sk);
            const uint32_t col = (uint32_t)sks * kSliceCols + lcn.colL;
            const bool cvalid = 2 * cu.q + (int)lcn.sd < nitems && col < (uint32_t)a.seg[1].Kv;
            const bool bad = cvalid && (U.xc >= ldx || (col > 0 && (int)U.xp >= (int)U.xc));
            if (bad && a.ws != nullptr) atomicOr(a.ws, kWsErrIndex);
            const bool use = cvalid && U.xc < ldx;
            // the activation block into the table area (free until the build below), then the
            // gather through idx from there
            lds_u32x4* blk = (lds_u32x4*)(tab + 4 * tid);
            *blk = u32x4{U.xb.x, U.xb.y, U.xb.z, U.xb.w};
            __syncthreads();
            const uint32_t xc = use ? U.xc : 0u;
#pragma unroll
            for (int b = 0; b < BMAX; ++b)
                if (b < a.batch) sv[b * 512 + tid] = use ? U.ac * lds_x<XT>(tb, (uint32_t)b * ldx + xc) : 0.f;
        } else {
#pragma unroll
            for (int b = 0; b < BMAX; ++b)
                if (b < a.batch) sv[b * 512 + tid] = U.ac * to_f32(U.xv[b]);
        }
        after_stage();
        __syncthreads();
#pragma unroll
        for (int b = 0; b < BMAX; ++b) {
            if (b < a.batch) {
                float S[RPL];
                row_pass(U, mine, last, cu.rg, b, std::integral_constant<bool, SI == 0 && GS>{}, S);
#pragma unroll
                for (int j = 0; j < RPL; ++j) acc[j][b] += S[j];
                __syncthreads();
            }
        }
        if (last) {
            flush(cu.rg);
            clear_acc();
        }
    };

    // The run of segment SI's units in [x0, x1). Two register slots, each reloaded in place two
    // units ahead (no copies between slots, which would wait on loads still in flight);
    // loads past the run are issued with valid = false and read nothing, so every path issues
    // the same loads. The run's first arrival is made before its loads, so that a first arriver
    // learns it (and zeroes) without waiting for them.
    auto run = [&](auto si_c) {
        constexpr int SI = decltype(si_c)::value;
        const uint32_t base = SI ? Um : 0u;
        const uint32_t lo = SI ? (x0 > Um ? x0 : Um) : x0;
        const uint32_t hi = SI ? x1 : (x1 < Um ? x1 : Um);
        if (lo >= hi) return;
        const int US = P.US[SI];
        const int nb = a.seg[SI].nb;
        const int nitems = P.KT[SI] * nb;
        Cursor lcur = cursor_at(lo - base, US, P.dUS[SI], nb, P.dNb[SI]);
        Cursor pcur = lcur;
        // units of the run in the row group entered at unit x with cursor cu
        auto run_units = [&](uint32_t x, const Cursor& cu) {
            const uint32_t left = (uint32_t)(US - cu.q);
            return hi - x < left ? hi - x : left;
        };
        // Two register slots: a unit's loads are issued while the unit before it is processed.
        // (A third slot, loads two units ahead, lost everywhere it was measured, cold: the 4096 x
        // 4096 step 6.95 -> 6.28 us and main only 6.06 -> 5.53 us with two, 11008 x 4096 with
        // refinement 8.9 -> 8.1 us, the 70B gate 30.6 -> 28.8 us, 8192 x 8192 13.8 -> 12.4 us.
        // At launch every workgroup requests its slots' units at once; per-workgroup timestamps
        // on the 70B gate had the later-dispatched half of the workgroups waiting behind that
        // burst, and the third slot's registers cost the instances their scheduling room.)
        Unit<XT, RPL, BMAX, XL> s0, s1;
        // The candidate zeroer of the row group this run starts in is a run that starts among the
        // row group's first Q + 1 units of this segment (none when arrivers without units go
        // first): it announces its arrival before its loads and looks at the answer as soon as
        // it returns. Every other workgroup announces after its first unit's loads (so that the
        // candidate's add usually comes first) and looks only at its flush, by when the answer
        // is long back; if it did arrive first after all, it initializes the rows there.
        const bool cand = first_mode && !P.xmode && P.Zn == 0 && (uint32_t)pcur.q <= Qx;
        if (cand) enter(pcur.rg, run_units(lo, pcur));
        load_unit<SI, XL, GS>(s0, P, lcur, true, lcn, tid);
        advance(lcur, US, nb);
        if (!cand) enter(pcur.rg, run_units(lo, pcur));
        load_unit<SI, XL, GS>(s1, P, lcur, lo + 1 < hi, lcn, tid);
        advance(lcur, US, nb);
        if (cand) zero_if_first(pcur.rg);
        // The refinement without XL gathers a unit's activations once its idx is in: the first
        // unit's here, every later one's after the staging of the unit before it.
        constexpr bool deferred = SI == 1 && !XL;
        auto gather = [&](Unit<XT, RPL, BMAX, XL>& V) {
            if constexpr (deferred) gather_unit(V, P);
        };
        gather(s0);
        auto step = [&](const Unit<XT, RPL, BMAX, XL>& U, uint32_t x, Unit<XT, RPL, BMAX, XL>& next) {
            const bool last = x + 1 == hi || pcur.q + 1 == US;
            process(U, nitems, pcur, last, si_c, [&]() { gather(next); });
            advance(pcur, US, nb);
            if (last && x + 1 < hi) enter(pcur.rg, run_units(x + 1, pcur));
        };
        // Wave priority from the units this workgroup has left, in the instances with two or
        // more row tiles per unit (the large matrices, two workgroups per CU with several units
        // each): of two workgroups sharing a CU the one behind gets issue priority, so that both
        // stay busy to the end (with equal priorities the older one's waves issue first and the
        // younger finishes alone: 70B gate + up grouped 48.2 -> 44.6 us, the 70B gate at 4 rows
        // 64.0 -> 60.0 us). The one-row-tile instances keep the default priority (on the 4096 x
        // 4096 step it cost 0.1 us).
        auto set_prio = [&](uint32_t x) {
            if constexpr (RPL >= 2) {
                const uint32_t rem = x1 - x;
                if (rem >= 6) __builtin_amdgcn_s_setprio(3);
                else if (rem >= 4) __builtin_amdgcn_s_setprio(2);
                else if (rem >= 2) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
            }
        };
        for (uint32_t x = lo; x < hi; x += 2) {
            set_prio(x);
            step(s0, x, s1);
            load_unit<SI, XL, GS>(s0, P, lcur, x + 2 < hi, lcn, tid);
            advance(lcur, US, nb);
            if (x + 1 < hi) set_prio(x + 1);
            if (x + 1 < hi) step(s1, x + 1, s0);
            load_unit<SI, XL, GS>(s1, P, lcur, x + 3 < hi, lcn, tid);
            advance(lcur, US, nb);
        }
    };
    run(std::integral_constant<int, 0>{});
    if (P.US[1] > 0) run(std::integral_constant<int, 1>{});
}


// Occupancy: the second argument is a minimum of waves per SIMD (2 lets the compiler use up to
// 256 VGPRs); two workgroups per CU need at most 128, which the instances with one or two row
// tiles and batch up to 4 stay within on their own, except two row tiles at four activation rows
// (per-row scales), which sits at the edge and is held to four waves per SIMD explicitly. (Asking for 4 waves per
// SIMD everywhere makes the compiler issue the table lookups in smaller batches, which costs
// more than it gains.)
template <int RPL, int BMAX, bool GS>
constexpr int kMinWaves = (RPL == 2 && BMAX == 4 && !GS) ? 4 : 2;
template <typename XT, int RPL, int BMAX, bool XL, bool GS>
__global__ __launch_bounds__(kStepThreads, (kMinWaves<RPL, BMAX, GS>)) void k_gemv8(StepParams P) {
    step_body<XT, RPL, BMAX, XL, GS>(P, (int)blockIdx.x);
}

// Several GEMVs sharing x in one launch: GEMV i gets workgroups [start[i], start[i + 1]) and
// runs the same body on them.
struct GroupParams {
    int count;
    int start[kMaxGroup + 1];
    StepParams p[kMaxGroup];
};

template <typename XT, int RPL, int BMAX, bool XL>
__global__ __launch_bounds__(kStepThreads, (kMinWaves<RPL, BMAX, false>)) void k_gemv8_group(GroupParams GP) {
    const int b = (int)blockIdx.x;
    int i = 0;
    while (i + 1 < GP.count && b >= GP.start[i + 1]) ++i;
    step_body<XT, RPL, BMAX, XL, false>(GP.p[i], b - GP.start[i]);
}

// ---------------------------------------------------------------------------------------
// The GEMV workspace of ubw_lut_gemv_refined_noalloc, for callers that cannot allocate: one
// static array per device, zero when the code object is loaded and kept consistent by every
// call (the counters of at most kScratchRowGroups row groups; header word 0 the error word).
// Host code reaches it only through the device address that scratch_address() looks up once per
// device.
static __device__ __align__(256) uint32_t scratch[kScratchWords];

hipError_t scratch_address(uint32_t** out) {
    static std::atomic<uint32_t*> addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    uint32_t* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {  // first call on this device (which is current): look the array up
        e = hipGetSymbolAddress(reinterpret_cast<void**>(&p), HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
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
    hipLaunchKernelGGL(k_ternary_bits, dim3(grid_for(total / 2, 256)), dim3(256), 0, s, w, N, K, KT, total, packed);
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

// Workgroups of a kernel instance that the current device can hold at once (occupancy x CUs),
// cached per device (thread-safe: each entry is written once with the value every thread
// computes; devices numbered kMaxDevices or above are queried on every call).
template <typename Kernel>
static int64_t capacity_of(Kernel k, std::atomic<int64_t>* cache) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const bool cached = dev >= 0 && dev < kMaxDevices;
    if (cached) {
        const int64_t c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, kStepThreads, 0) != hipSuccess)
        return 0;
    const int64_t c = (int64_t)cus * per_cu;
    if (cached) cache[dev].store(c, std::memory_order_relaxed);
    return c;
}
template <typename XT, int RPL, int BMAX, bool XL, bool GS>
static int64_t resident_capacity() {
    static std::atomic<int64_t> cap[kMaxDevices];
    return capacity_of(k_gemv8<XT, RPL, BMAX, XL, GS>, cap);
}
template <typename XT, int RPL, int BMAX, bool XL>
static int64_t resident_capacity_group() {
    static std::atomic<int64_t> cap[kMaxDevices];
    return capacity_of(k_gemv8_group<XT, RPL, BMAX, XL>, cap);
}

using plan::default_workgroups;

// Split of P's units over Gu workgroups and the final output mode; zero-fills y first when the
// single-launch protocol cannot be used (no workspace, or too many arrivals per row group for
// the counter's field).
// The single-launch protocol runs in XCD-local mode (static zeroing by NRG workgroups without
// units at the lowest IDs; see step_body) when allowed, every one of the eight XCDs gets
// workgroups and the same number of row groups (Gu >= 8, NRG a multiple of 8), and the zeroing
// workgroups fit on the device beside the others (Gu + NRG <= cap). Otherwise it runs in
// first-arriver mode. (Measured cold with salient refinement, y = result: with workgroups beyond
// the device's capacity the last ones start only when zeroers end, 70B gate 31.4 us vs 30.4 us
// first-arriver; with 43 row groups, six on three XCDs and five on the others, 11008 x 4096 at
// 4 rows 20.0 us vs 16.5 us; 4096 x 4096, all resident and balanced: 6.9 us vs 7.05 us.)
// In first-arriver mode,
// where with equal ranges (R = 0) and room on the device
// (Gu + NRG <= cap) NRG arrivers without units go first (lowest IDs), one per row group: they
// usually arrive first and zero, so no workgroup with units waits for the zeroing's round trip
// (measured on 4096 x 4096, 256 units, with such workgroups as zeroing owners: 5.84 -> 5.36 us).
// With R > 0 such workgroups would crowd the CUs of the longer ranges (4096 x 4096 with 5%
// salient columns, 272 units: 6.12 us without, 6.29 us with).
constexpr int kXcds = 8;  // XCDs of an MI355X; workgroup g runs on XCD g mod 8

static hipError_t finish_params(StepParams& P, int64_t Gu, int64_t cap, bool allow_xcd, hipStream_t s) {
    P.Gu = (int)Gu;
    P.Zn = 0;
    P.xmode = 0;
    const int64_t R = P.U % Gu;
    // every workgroup holds exactly one whole row group (one segment only: a refinement
    // segment's units of a row group sit in another part of the list): plain stores
    const bool whole_rows = P.Gu == P.NRG && P.US[1] == 0;
    if (P.mode == kModeFirst && whole_rows) P.mode = kModeStore;
    // the arrival field counts a row group's arrivals (Urg, plus one) and must not overflow into
    // the generation
    if (P.mode == kModeFirst && (P.a.ws == nullptr || P.Urg + 1 > (int)kArrMask)) {
        hipError_t e = launch_fill_zero(P.a.y, (int64_t)P.a.batch * P.a.N, s);
        if (e != hipSuccess) return e;
        P.mode = kModeAtomic;
    }
    if (P.mode == kModeFirst && allow_xcd && Gu >= kXcds && P.NRG >= kXcds && P.NRG % kXcds == 0 &&
        Gu + P.NRG <= cap) {
        P.xmode = 1;
        P.Zn = (int)ceil_div(P.NRG, kXcds) * kXcds;  // keeps unit workgroup g - Zn on the XCD of g
    } else if (P.mode == kModeFirst && R == 0 && Gu + P.NRG <= cap) {
        P.Zn = P.NRG;
    }
    P.Arr = P.Urg + (P.Zn > 0 && !P.xmode ? 1 : 0);
    P.G = P.Zn + P.Gu;
    return hipSuccess;
}

template <typename XT, int RPL, int BMAX, bool XL, bool GS>
static hipError_t launch_step_t(StepParams P, hipStream_t s) {
    const int64_t cap = resident_capacity<XT, RPL, BMAX, XL, GS>();
    if (cap <= 0) return hipErrorInvalidConfiguration;
    // Persistent workgroups: by default no more than the device holds at once (an explicit
    // geometry may ask for more; the flag waits do not depend on it).
    int64_t G = P.a.workgroups > 0 ? P.a.workgroups : default_workgroups(P.U, cap, P.a.batch);
    G = G < P.U ? G : P.U;
    hipError_t e = finish_params(P, G, cap, true, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemv8<XT, RPL, BMAX, XL, GS>), dim3((unsigned)P.G), dim3(kStepThreads), 0, s, P);
    return hipGetLastError();
}

// Grouped launch: the workgroups the device holds at once (at most the total units) are shared
// out in proportion to each GEMV's units, at least one each. (One per CU, as default_workgroups
// picks for single launches, measured slower here: 70B q+k+v at batch 1 14.4 -> 17.0 us.)
template <typename XT, int RPL, int BMAX, bool XL>
static hipError_t launch_group_t(GroupParams GP, hipStream_t s) {
    const int64_t cap = resident_capacity_group<XT, RPL, BMAX, XL>();
    if (cap < GP.count) return hipErrorInvalidConfiguration;
    int64_t Ut = 0;
    for (int i = 0; i < GP.count; ++i) Ut += GP.p[i].U;
    const int64_t Gt = Ut < cap ? Ut : cap;
    int64_t Gi[kMaxGroup], sum = 0;
    for (int i = 0; i < GP.count; ++i) {
        Gi[i] = Gt * GP.p[i].U / Ut;
        Gi[i] = Gi[i] < 1 ? 1 : (Gi[i] > GP.p[i].U ? GP.p[i].U : Gi[i]);
        sum += Gi[i];
    }
    while (sum > Gt) {  // the minimum of one each can overshoot: take from the largest share
        int j = 0;
        for (int i = 1; i < GP.count; ++i) j = Gi[i] > Gi[j] ? i : j;
        --Gi[j];
        --sum;
    }
    for (int i = 0; i < GP.count && sum < Gt; ++i) {  // hand out what rounding left over
        const int64_t add = Gt - sum < GP.p[i].U - Gi[i] ? Gt - sum : GP.p[i].U - Gi[i];
        Gi[i] += add;
        sum += add;
    }
    GP.start[0] = 0;
    for (int i = 0; i < GP.count; ++i) {
        hipError_t e = finish_params(GP.p[i], Gi[i], 0, false, s);
        if (e != hipSuccess) return e;
        GP.start[i + 1] = GP.start[i] + (int)Gi[i];
    }
    hipLaunchKernelGGL((k_gemv8_group<XT, RPL, BMAX, XL>), dim3((unsigned)GP.start[GP.count]), dim3(kStepThreads), 0,
                       s, GP);
    return hipGetLastError();
}

// Instances: (row tiles per workgroup, batch bound, refinement gather through LDS) choices whose
// registers fit without spills; max_rows_per_group() is the host-side rule that keeps requests
// inside this set. f(XT, RPL, BMAX, XL) is called with the chosen instance's parameters.
template <typename XT, typename F>
static hipError_t dispatch_instance(int batch, int rpl, bool xl, F f) {
    using std::integral_constant;
    if (batch <= 1) {
        if (xl) {
            if (rpl >= 4) return f(XT{}, integral_constant<int, 4>{}, integral_constant<int, 1>{}, std::true_type{});
            if (rpl >= 2) return f(XT{}, integral_constant<int, 2>{}, integral_constant<int, 1>{}, std::true_type{});
            return f(XT{}, integral_constant<int, 1>{}, integral_constant<int, 1>{}, std::true_type{});
        }
        if (rpl >= 4) return f(XT{}, integral_constant<int, 4>{}, integral_constant<int, 1>{}, std::false_type{});
        if (rpl >= 2) return f(XT{}, integral_constant<int, 2>{}, integral_constant<int, 1>{}, std::false_type{});
        return f(XT{}, integral_constant<int, 1>{}, integral_constant<int, 1>{}, std::false_type{});
    }
    if (batch <= 2) {
        if (rpl >= 2) return f(XT{}, integral_constant<int, 2>{}, integral_constant<int, 2>{}, std::false_type{});
        return f(XT{}, integral_constant<int, 1>{}, integral_constant<int, 2>{}, std::false_type{});
    }
    if (batch <= kBatchChunk) {
        if (rpl >= 2) return f(XT{}, integral_constant<int, 2>{}, integral_constant<int, 4>{}, std::false_type{});
        return f(XT{}, integral_constant<int, 1>{}, integral_constant<int, 4>{}, std::false_type{});
    }
    return hipErrorInvalidValue;  // larger batches run as chunks of kBatchChunk rows
}

// The gather of a refinement segment goes through LDS when the activation block fits (in whole,
// aligned 16-byte pieces, so that no load straddles the end of x).
static bool gather_in_lds(const StepArgs& a) {
    const uint64_t xbytes = (uint64_t)a.batch * (uint64_t)a.ldx * (a.x_dtype == UBW_F16 ? 2u : 4u);
    return xbytes <= kXlBytes && xbytes % 16 == 0 && (reinterpret_cast<uintptr_t>(a.x) & 15u) == 0;
}

// Batches above kBatchChunk rows run as consecutive launches of at most kBatchChunk activation
// rows each (the weights are read once per chunk). Per activation row a launch builds and
// searches its tables again, so a chunk costs the same per row as one launch of the whole
// batch would; what chunking keeps is the 4-row instance's footprint (80 KiB of LDS, two
// workgroups per CU), which measured twice as fast per row as 8- or 16-row instances holding
// one workgroup per CU.
static StepArgs batch_chunk(const StepArgs& a, int r0) {
    StepArgs c = a;
    const int64_t xs = a.x_dtype == UBW_F16 ? 2 : 4;
    c.x = static_cast<const char*>(a.x) + (int64_t)r0 * a.ldx * xs;
    c.y = a.y + (int64_t)r0 * a.N;
    c.batch = a.batch - r0 < kBatchChunk ? a.batch - r0 : kBatchChunk;
    return c;
}

int max_rows_per_group(int batch) { return batch <= 1 ? 4 : 2; }

// The step reads every buffer through 32-bit buffer offsets below 2^31 (kOob is out of range).
bool step_buffers_fit(const StepArgs& a) {
    const int64_t lim = (int64_t)1 << 31;
    const int64_t xs = a.x_dtype == UBW_F16 ? 2 : 4;
    if ((int64_t)a.batch * a.ldx * xs >= lim) return false;
    for (int i = 0; i < a.nseg; ++i) {
        const Segment& sg = a.seg[i];
        const int64_t KT = ceil_div(sg.Kv, kSliceCols);
        const int64_t arows = (i == 0 && a.gs) ? KT : 1;  // alpha_r: [nb][N] fp32 or [nb][KT][N][2] fp16
        if ((int64_t)sg.nb * arows * a.N * 4 >= lim || (int64_t)sg.nb * sg.Kv * 4 >= lim) return false;
        if ((int64_t)sg.Kv * 4 >= lim || KT * sg.nb * kTileWords * 4 >= lim) return false;
    }
    return true;
}

// Everything of a GEMV's parameters except its workgroup split and final mode.
static hipError_t make_params(const StepArgs& a, StepParams& P) {
    P = StepParams{};
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
    for (int i = 0; i < 2; ++i) {
        P.dUS[i] = fast_div(P.US[i] > 0 ? (uint32_t)P.US[i] : 1u);
        P.dNb[i] = fast_div(i < a.nseg && a.seg[i].nb > 0 ? (uint32_t)a.seg[i].nb : 1u);
    }
    if (!step_buffers_fit(a)) return hipErrorInvalidValue;
    // the kernel gathers through idx in seg[1] only
    if (a.seg[0].idx != nullptr || (a.nseg == 2 && a.seg[1].idx == nullptr)) return hipErrorInvalidValue;
    if (P.Urg == 0) return hipErrorInvalidValue;
    P.U = P.NRG * P.Urg;
    P.mode = a.accumulate ? kModeAtomic : kModeFirst;
    return hipSuccess;
}

static hipError_t launch_step_rows(const StepArgs& a, hipStream_t s) {
    StepParams P;
    hipError_t e = make_params(a, P);
    if (e != hipSuccess) return e;
    const bool xl = P.US[1] > 0 && gather_in_lds(a);
    // group scales are a separate set of instances: the per-row kernels carry no code for them
    auto go = [&](auto xt, auto rpl_c, auto bmax_c, auto xl_c) {
        return launch_step_t<decltype(xt), decltype(rpl_c)::value, decltype(bmax_c)::value, decltype(xl_c)::value,
                             false>(P, s);
    };
    auto go_gs = [&](auto xt, auto rpl_c, auto bmax_c, auto xl_c) {
        return launch_step_t<decltype(xt), decltype(rpl_c)::value, decltype(bmax_c)::value, decltype(xl_c)::value,
                             true>(P, s);
    };
    if (a.gs) {
        if (a.x_dtype == UBW_F16) return dispatch_instance<__half>(a.batch, a.rows_per_group, xl, go_gs);
        return dispatch_instance<float>(a.batch, a.rows_per_group, xl, go_gs);
    }
    if (a.x_dtype == UBW_F16) return dispatch_instance<__half>(a.batch, a.rows_per_group, xl, go);
    return dispatch_instance<float>(a.batch, a.rows_per_group, xl, go);
}

static bool use_mfma(const StepArgs& a) {
    if (a.tables_only || !mfma_step_supported(a)) return false;
    int64_t bits = 0;
    for (int i = 0; i < a.nseg; ++i) bits += (int64_t)a.seg[i].nb * a.N * a.seg[i].Kv;
    return plan::prefer_mfma(bits / 8, a.batch);
}

hipError_t launch_step(const StepArgs& a, hipStream_t s) {
    if (use_mfma(a)) return launch_step_mfma(a, s);
    if (a.batch <= kBatchChunk) return launch_step_rows(a, s);
    for (int r0 = 0; r0 < a.batch; r0 += kBatchChunk) {
        hipError_t e = launch_step_rows(batch_chunk(a, r0), s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

static hipError_t launch_step_group_rows(const StepArgs* a, int count, hipStream_t s) {
    if (count < 1 || count > kMaxGroup) return hipErrorInvalidValue;
    GroupParams GP{};
    GP.count = count;
    bool any_refine = false, lds_ok = true;
    for (int i = 0; i < count; ++i) {
        if (a[i].gs || a[i].x != a[0].x || a[i].batch != a[0].batch || a[i].x_dtype != a[0].x_dtype ||
            a[i].ldx != a[0].ldx || a[i].rows_per_group != a[0].rows_per_group)
            return hipErrorInvalidValue;
        hipError_t e = make_params(a[i], GP.p[i]);
        if (e != hipSuccess) return e;
        any_refine = any_refine || GP.p[i].US[1] > 0;
        lds_ok = lds_ok && gather_in_lds(a[i]);
    }
    const bool xl = any_refine && lds_ok;
    auto go = [&](auto xt, auto rpl_c, auto bmax_c, auto xl_c) {
        return launch_group_t<decltype(xt), decltype(rpl_c)::value, decltype(bmax_c)::value, decltype(xl_c)::value>(GP, s);
    };
    if (a[0].x_dtype == UBW_F16) return dispatch_instance<__half>(a[0].batch, a[0].rows_per_group, xl, go);
    return dispatch_instance<float>(a[0].batch, a[0].rows_per_group, xl, go);
}

// Several GEMVs that share x, batch, dtype and rows_per_group, in one launch (on the tables, or
// on the matrix cores when every GEMV of the group goes there).
hipError_t launch_step_group(const StepArgs* a, int count, hipStream_t s) {
    if (count < 1 || count > kMaxGroup) return hipErrorInvalidValue;
    bool all_mfma = true;
    for (int i = 0; i < count; ++i) all_mfma = all_mfma && use_mfma(a[i]);
    if (all_mfma) return launch_step_mfma_group(a, count, s);
    if (a[0].batch <= kBatchChunk) return launch_step_group_rows(a, count, s);
    for (int r0 = 0; r0 < a[0].batch; r0 += kBatchChunk) {
        StepArgs c[kMaxGroup];
        for (int i = 0; i < count; ++i) c[i] = batch_chunk(a[i], r0);
        hipError_t e = launch_step_group_rows(c, count, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace ubw
