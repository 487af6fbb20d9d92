// The GEMV step at group width 4 with whole rows per workgroup (g = 4).
//
// FluxBin (gist.science/ko/paper/2608.15602), technical summary, "2. Kernel innovation": the
// tables with alpha_c folded in (LUT-BSF), the salient columns mapped onto a dense virtual matrix
// (VCM), and the execution flow uint32 weights -> pattern indices by bit operations -> partial
// sums -> alpha_r. The same dataflow as the tile kernel, with 4-column groups: a table has 16
// entries, T[p] = sum_{i<4} (2 bit_i(p) - 1) v_i, so the tables of a whole row fit in LDS (16
// bytes per column and base: 128 KiB for 4096 columns and two bases). A workgroup then owns 16
// complete rows, builds every table of the row once and writes each output with a plain store:
// no partial sums cross workgroups, so there is no zeroing, no flag and no atomic, and y = result
// and y += result are the same single launch.
//
// Workgroup = 512 threads = 16 half-waves; half-wave h owns row 16 w + h. A row's (base, column)
// space is cut into 32 chunks, one per lane of the half-wave, each inside one base (32 / nb chunks
// per base, C = 32 CW columns each, the columns padded with zero weight bits and zero v up to
// 32 / nb chunks): lane c looks up the C / 4 groups of its chunk and the half-wave adds the 32
// lanes' alpha_r-scaled sums. The refinement segment (ns bases over the s salient columns, padded
// to its tiles' 256 columns) is cut the same way into 32 chunks of Cs columns.
// Table of group i of chunk c: its 16 entries at words (e G + i) * 32 + c of the segment's table
// area (G = groups per chunk), i.e. every table of chunk c sits in LDS bank c: at each lookup step
// the 32 lanes of a half-wave read 32 different banks whatever their patterns are.
// Lookup: entry e = nibble of the lane's canonical word, address = e * 128 G + 4 c (one
// v_mad_u32_u24) + 128 i (the instruction's constant offset); 3 VALU + 1 LDS read per 4 columns.
// The packed words arrive in the tile layout (slot s of row rho holds canonical word s ^ a with
// bytes permuted by c, a = (rho & 31) >> 2, c = rho & 3): each lane undoes that once per slice
// (three conditional swaps of word halves and one byte permute per word).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "ubw_internal.h"

namespace ubw {

namespace {

constexpr int kR4Threads = 512;
constexpr int kR4Rows = 16;                  // rows per workgroup: one per half-wave
constexpr uint32_t kR4LdsBytes = 159744;     // 156 KiB of the CU's 160 KiB
constexpr uint32_t kR4Oob = 0x80000000u;     // beyond every buffer (all below 2 GiB)

struct R4Seg {
    const uint32_t* packed;  // tile layout, nb bases x Kv columns
    const float* alpha_r;    // [nb][N]
    const float* alpha_c;    // [nb][Kv]
    const int32_t* idx;      // refinement: [Kv] activation column of each virtual column
    int nb;                  // 0: the segment is empty
    int Kv;                  // columns (K, or s)
    int KT;                  // 256-column tiles along the columns
    int cpb;                 // chunks per base (32 / nb)
    int lcpb;                // log2(cpb)
    int C;                   // columns per chunk (a multiple of 4)
    int G;                   // groups per chunk (C / 4)
    uint32_t tab;            // byte offset of the segment's tables in LDS
};

struct R4Params {
    R4Seg seg[2];            // main (no idx), refinement (idx)
    const void* x;
    int64_t ldx;             // K
    int batch;
    float* y;                // [batch][N]
    int N, NT;
    int accumulate;
    uint32_t* err;           // workspace word 0 for index errors, or nullptr
    uint32_t xs_off;         // byte offset of the fp32 staging of x in LDS
    uint32_t K4;             // K rounded up to a multiple of 4
    uint32_t xsh;            // staging: column c at float c + 4 (c >> xsh): 4 padding floats after every
                             // 4 main chunks of columns, so that the 8 lanes of an LDS pass of the
                             // main build (8 chunk quadruples, 4 chunks apart) read different banks
    int xvec;                // 1: 16-byte aligned x rows (16-byte loads), 0: one element per load
};

typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc rsrc4(const void* p, uint32_t bytes) {
    const uint64_t a = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void* base = (void*)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ uint32_t ld32(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0); }
__device__ __forceinline__ uint2 ld64(Rsrc r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint4 ld128(Rsrc r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Activations: 16-byte vectors (8 fp16 or 4 fp32 columns) staged as fp32, or one element at a
// time where rows are not 16-byte aligned.
template <typename XT> constexpr uint32_t kVecCols = 16u / (uint32_t)sizeof(XT);
__device__ __forceinline__ float h2f(uint32_t h) { return __half2float(__ushort_as_half((unsigned short)h)); }
template <typename XT> __device__ __forceinline__ void stage_vec(float* xs, uint32_t c0, uint32_t sh, const uint4& v);
template <> __device__ __forceinline__ void stage_vec<__half>(float* xs, uint32_t c0, uint32_t sh, const uint4& v) {
    *reinterpret_cast<float4*>(&xs[plan::r4_xpos(c0, sh)]) = make_float4(h2f(v.x & 0xFFFFu), h2f(v.x >> 16), h2f(v.y & 0xFFFFu), h2f(v.y >> 16));
    *reinterpret_cast<float4*>(&xs[plan::r4_xpos(c0 + 4u, sh)]) =
        make_float4(h2f(v.z & 0xFFFFu), h2f(v.z >> 16), h2f(v.w & 0xFFFFu), h2f(v.w >> 16));
}
template <> __device__ __forceinline__ void stage_vec<float>(float* xs, uint32_t c0, uint32_t sh, const uint4& v) {
    *reinterpret_cast<float4*>(&xs[plan::r4_xpos(c0, sh)]) =
        make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
template <typename XT> __device__ __forceinline__ float x_at(Rsrc r, uint32_t off);
template <> __device__ __forceinline__ float x_at<__half>(Rsrc r, uint32_t off) {
    return h2f(__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
}
template <> __device__ __forceinline__ float x_at<float>(Rsrc r, uint32_t off) { return __uint_as_float(ld32(r, off)); }

// The 16-entry table of 4 scaled activations, built by doubling from the all-minus entry.
__device__ __forceinline__ void lut4(const float v[4], float T[16]) {
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


// Base of lane c's chunk (32 / nb chunks per base), 0 for an empty segment.
__device__ __forceinline__ int k0_of(int c, const R4Seg& sg) { return sg.nb > 0 ? c >> sg.lcpb : 0; }

// Word offset (bytes) of row r's slice ks of base k in a segment's tile layout, first half.
__device__ __forceinline__ uint32_t slice_off(const R4Seg& sg, int r, int ks, int k) {
    const int rt = r >> 8, rho = r & 255;
    return ((uint32_t)((rt * sg.KT + ks) * sg.nb + k) * (uint32_t)kTileWords + 4u * (uint32_t)rho) * 4u;
}

// 16-byte activation vectors prefetched per thread and row: 1024 vectors, 8192 fp16 columns
// (more than any K whose tables fit) or 4096 fp32 ones (the staging reads the rest, if any).
constexpr int kXPre = 2;

// CW: canonical words per main chunk (C = 32 CW columns), 1, 2, 4 or 8; AV: main K a multiple
// of 4 and alpha_c 16-byte aligned (one load per group of 4 scales).
template <typename XT, int CW, bool AV>
__global__ __launch_bounds__(kR4Threads, 1) void k_rows4(const R4Params P) {
    __shared__ __align__(16) unsigned char s_lds[kR4LdsBytes];
    const int tid = threadIdx.x;
    const int hw = tid >> 5, lane = tid & 31;
    const int row = (int)blockIdx.x * kR4Rows + hw;
    const R4Seg& S0 = P.seg[0];
    const R4Seg& S1 = P.seg[1];
    float* xs = reinterpret_cast<float*>(s_lds + P.xs_off);
    // a = bits 2..4 of the row: the same for the wave's two rows (16 w + 2 k, 16 w + 2 k + 1)
    const int a = (int)__builtin_amdgcn_readfirstlane((uint32_t)(row & 31) >> 2);
    const uint32_t unperm = 0x03020100u ^ (0x01010101u * (uint32_t)(row & 3));

    // ---- loads, in the order they are needed: the first activation row (staging), alpha_c and
    // the refinement's indices and scales (table builds), alpha_r and the weights (lookups); a
    // wait for one of them leaves the later ones in flight
    const uint32_t ldx = (uint32_t)P.ldx;
    const uint32_t xrow = ldx * (uint32_t)sizeof(XT);             // bytes per activation row
    const uint32_t nvx = P.xvec ? ldx / kVecCols<XT> : 0u;         // 16-byte vectors per row
    const Rsrc rx = rsrc4(P.x, (uint32_t)P.batch * xrow);
    uint4 xv[kXPre];
    auto prefetch = [&](int b) {
#pragma unroll
        for (int i = 0; i < kXPre; ++i) {
            const uint32_t v = (uint32_t)(tid + kR4Threads * i);
            if ((uint32_t)(kR4Threads * i) < nvx) xv[i] = ld128(rx, v < nvx ? (uint32_t)b * xrow + 16u * v : kR4Oob);
        }
    };
    // x[b] into the staging as fp32, from the prefetched vectors (and loads for the rest, if any)
    auto stage = [&](int b) {
        if (P.xvec) {
#pragma unroll
            for (int i = 0; i < kXPre; ++i) {
                const uint32_t v = (uint32_t)(tid + kR4Threads * i);
                if (v < nvx) stage_vec<XT>(xs, kVecCols<XT> * v, P.xsh, xv[i]);
            }
            for (uint32_t v = (uint32_t)tid + kR4Threads * kXPre; v < nvx; v += kR4Threads)
                stage_vec<XT>(xs, kVecCols<XT> * v, P.xsh, ld128(rx, (uint32_t)b * xrow + 16u * v));
        } else {
            for (uint32_t i = (uint32_t)tid; i < ldx; i += kR4Threads)
                xs[plan::r4_xpos(i, P.xsh)] = x_at<XT>(rx, (uint32_t)b * xrow + (uint32_t)sizeof(XT) * i);
        }
    };

    // ---- loads, in the order they are needed: x (staging; first, so that every wave has it in
    // flight before the address arithmetic), alpha_c and the refinement's indices and scales
    // (table builds), alpha_r and the weights (lookups); a wait for one of them leaves the later
    // ones in flight. (Offsets use 24-bit multiplies: a 32 x 32 multiply-add may be compiled to a
    // 64-bit one whose unused high input is any register, possibly one a load is still to write,
    // which forces an early wait.)
    prefetch(0);

    // main build role: thread t < 8 G0 builds the tables of group gi = t / 8 of chunks 4 qd ..
    // 4 qd + 3, qd = t % 8: the 8 lanes of each LDS pass write 8 different bank quadruples. Per
    // chunk: alpha_c of the group's 4 columns and the LDS address of their staged x (the zero pad
    // for columns >= K, whose alpha_c reads as 0 too)
    const int gi = tid >> 3, qd = tid & 7;
    const bool mb = S0.nb > 0 && gi < S0.G;
    const uint32_t xpad = P.xs_off + 4u * plan::r4_xpos(P.K4, P.xsh);
    uint4 acm[4];
    uint32_t xa[4];
    {
        const Rsrc r = rsrc4(S0.alpha_c, (uint32_t)S0.nb * (uint32_t)S0.Kv * 4u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t cb = (uint32_t)(4 * qd + j), kb = cb >> S0.lcpb;
            const uint32_t col = __umul24(cb & (uint32_t)(S0.cpb - 1), (uint32_t)S0.C) + 4u * (uint32_t)gi;
            const bool in = mb && col < (uint32_t)S0.Kv;
            const uint32_t o = (__umul24(kb, (uint32_t)S0.Kv) + col) * 4u;
            if constexpr (AV) {  // K a multiple of 4 and alpha_c 16-byte aligned: one load per group
                acm[j] = ld128(r, in ? o : kR4Oob);
            } else {
                acm[j].x = ld32(r, in ? o : kR4Oob);
                acm[j].y = ld32(r, in && col + 1u < (uint32_t)S0.Kv ? o + 4u : kR4Oob);
                acm[j].z = ld32(r, in && col + 2u < (uint32_t)S0.Kv ? o + 8u : kR4Oob);
                acm[j].w = ld32(r, in && col + 3u < (uint32_t)S0.Kv ? o + 12u : kR4Oob);
            }
            xa[j] = in ? P.xs_off + 4u * plan::r4_xpos(col, P.xsh) : xpad;
        }
    }
    // refinement build role: one table per thread, on the last waves: thread 511 - t, t < 32 G1,
    // builds the table of group gj = t / 32 of chunk ce = t % 32 from its 4 virtual columns (their
    // idx, the idx before the first for the order check, and alpha_c_s)
    const int tr = kR4Threads - 1 - tid;
    const int ce = tr & 31, gj = tr >> 5;
    const bool rb = S1.nb > 0 && gj < S1.G;
    uint32_t ix[4] = {0u, 0u, 0u, 0u}, acs[4] = {0u, 0u, 0u, 0u}, ixp = 0u;
    const uint32_t q0 = __umul24((uint32_t)ce & (uint32_t)(S1.cpb - 1), (uint32_t)S1.C) + 4u * (uint32_t)gj;
    if (rb) {  // the last waves only (the others skip this)
        const Rsrc ri = rsrc4(S1.idx, (uint32_t)S1.Kv * 4u);
        const Rsrc ra = rsrc4(S1.alpha_c, (uint32_t)S1.nb * (uint32_t)S1.Kv * 4u);
        const uint32_t sb = __umul24((uint32_t)ce >> S1.lcpb, (uint32_t)S1.Kv);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t q = q0 + (uint32_t)t;
            ix[t] = ld32(ri, q < (uint32_t)S1.Kv ? 4u * q : kR4Oob);
            acs[t] = ld32(ra, q < (uint32_t)S1.Kv ? 4u * (sb + q) : kR4Oob);
        }
        ixp = ld32(ri, q0 > 0u && q0 <= (uint32_t)S1.Kv ? 4u * (q0 - 1u) : kR4Oob);
    }
    // alpha_r of the lane's chunks
    const uint32_t aro0 =
        S0.nb > 0 && row < P.N ? (__umul24((uint32_t)k0_of(lane, S0), (uint32_t)P.N) + (uint32_t)row) * 4u : kR4Oob;
    const uint32_t aro1 =
        S1.nb > 0 && row < P.N ? (__umul24((uint32_t)k0_of(lane, S1), (uint32_t)P.N) + (uint32_t)row) * 4u : kR4Oob;
    const float ar0 = __uint_as_float(ld32(rsrc4(S0.alpha_r, (uint32_t)S0.nb * (uint32_t)P.N * 4u), aro0));
    const float ar1 = __uint_as_float(ld32(rsrc4(S1.alpha_r, (uint32_t)S1.nb * (uint32_t)P.N * 4u), aro1));
    // main chunk: base k0, columns [cib0 C, cib0 C + C), canonical words [w0, w0 + CW) of the row.
    // The lane loads the stored slots that hold them (canonical word w of a slice is slot w ^ a):
    // MW = min(CW, 8) words per slice, element m of a slice's load holding the chunk's word m ^ am
    // of that slice, am = a & (MW - 1). Bytes stay in stored order (undone at the lookups).
    constexpr int MW = CW < 8 ? CW : 8;
    constexpr int NS = CW / MW;
    const int am = a & (MW - 1);
    uint32_t wm[CW];
    {
        const Rsrc r = rsrc4(S0.packed, (uint32_t)S0.nb * (uint32_t)P.NT * (uint32_t)S0.KT * kTileWords * 4u);
        const int k0 = k0_of(lane, S0);
        const int w0 = (S0.nb > 0 ? lane & (S0.cpb - 1) : 0) * CW;  // first canonical word of the chunk
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            const int ks = (w0 >> 3) + j;
            const bool ok = S0.nb > 0 && row < P.N && ks < S0.KT;
            const uint32_t o = ok ? slice_off(S0, row, ks, k0) : 0u;
            if constexpr (MW == 8) {  // both 16-byte halves of the slice
                const uint4 h0 = ld128(r, ok ? o : kR4Oob);
                const uint4 h1 = ld128(r, ok ? o + (uint32_t)kTileRows * 16u : kR4Oob);
                wm[8 * j + 0] = h0.x; wm[8 * j + 1] = h0.y; wm[8 * j + 2] = h0.z; wm[8 * j + 3] = h0.w;
                wm[8 * j + 4] = h1.x; wm[8 * j + 5] = h1.y; wm[8 * j + 6] = h1.z; wm[8 * j + 7] = h1.w;
            } else {  // the MW slots of the chunk's words: an aligned run inside one half
                const int slot = ((w0 & 7) ^ a) & ~(MW - 1);
                const uint32_t oo =
                    ok ? o + (uint32_t)(slot >> 2) * (uint32_t)kTileRows * 16u + 4u * (uint32_t)(slot & 3) : kR4Oob;
                if constexpr (MW == 4) {
                    const uint4 h = ld128(r, oo);
                    wm[0] = h.x; wm[1] = h.y; wm[2] = h.z; wm[3] = h.w;
                } else if constexpr (MW == 2) {
                    const uint2 h = ld64(r, oo);
                    wm[0] = h.x; wm[1] = h.y;
                } else {
                    wm[0] = ld32(r, oo);
                }
            }
        }
    }
    // refinement chunk: base k1, virtual columns [c1, c1 + Cs) inside canonical word wi of slice
    // ks (Cs <= 32 and divides 32): one stored slot, wi ^ a
    const int c1 = (S1.nb > 0 ? lane & (S1.cpb - 1) : 0) * S1.C;  // first virtual column of the chunk
    uint32_t Wr0;
    {
        const int ks = c1 >> 8, slot = ((c1 & 255) >> 5) ^ a;
        const bool ok = S1.nb > 0 && row < P.N && ks < S1.KT;
        Wr0 = ld32(rsrc4(S1.packed, (uint32_t)S1.nb * (uint32_t)P.NT * (uint32_t)S1.KT * kTileWords * 4u),
                   ok ? slice_off(S1, row, ks, k0_of(lane, S1)) + (uint32_t)(slot >> 2) * (uint32_t)kTileRows * 16u +
                            4u * (uint32_t)(slot & 3)
                      : kR4Oob);
    }

    // ---- index checks (the weights stay in flight): an index outside [0, K) or not above the one
    // before it is reported; a column outside [0, K) reads the zero pad with alpha_c_s = 0 (it
    // adds nothing; one out of order still adds x[idx]), and so do the padding columns
    uint32_t ia[4] = {xpad, xpad, xpad, xpad};  // LDS addresses of the table's 4 staged activations
    if (rb) {
        bool bad_idx = false;
        uint32_t prev = ixp;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t q = q0 + (uint32_t)t;
            const uint32_t xi = ix[t];
            const bool live = q < (uint32_t)S1.Kv;
            const bool bad = live && (xi >= ldx || (q > 0u && (int)prev >= (int)xi));
            bad_idx = bad_idx || bad;
            const bool use = live && xi < ldx;
            ia[t] = use ? P.xs_off + 4u * plan::r4_xpos(xi, P.xsh) : xpad;
            acs[t] = use ? acs[t] : 0u;
            prev = xi;
        }
        if (bad_idx && P.err != nullptr) atomicOr(P.err, kWsErrIndex);
    }
    // the zero pad: every position after column K - 1 (ordered by the first barrier below)
    {
        const uint32_t zlo = plan::r4_xpos(ldx - 1u, P.xsh) + 1u, zhi = plan::r4_xpos(P.K4, P.xsh) + 4u;
        if ((uint32_t)tid < zhi - zlo) xs[zlo + (uint32_t)tid] = 0.f;
    }

    // row 0 staged before the loop (its wait leaves the weights in flight); row b + 1 is staged
    // after row b's lookups, from vectors loaded during row b's build
    stage(0);
    if (P.batch > 1) prefetch(1);
    for (int b = 0; b < P.batch; ++b) {
        __syncthreads();  // x[b] staged; every lookup of row b - 1 done
        // ---- build: main tables (v = alpha_c x)
        if (mb) {
            float T[4][16];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 xv4 = *reinterpret_cast<const float4*>(s_lds + xa[j]);
                const float v[4] = {__uint_as_float(acm[j].x) * xv4.x, __uint_as_float(acm[j].y) * xv4.y,
                                    __uint_as_float(acm[j].z) * xv4.z, __uint_as_float(acm[j].w) * xv4.w};
                lut4(v, T[j]);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e)
                *reinterpret_cast<float4*>(s_lds + S0.tab + 4u * ((uint32_t)(e * S0.G + gi) * 32u + 4u * (uint32_t)qd)) =
                    make_float4(T[0][e], T[1][e], T[2][e], T[3][e]);
        }
        // ---- build: refinement tables (v = alpha_c_s x[idx]), one per thread
        if (rb) {
            float v[4], T[16];
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = __uint_as_float(acs[t]) * *reinterpret_cast<const float*>(s_lds + ia[t]);
            lut4(v, T);
#pragma unroll
            for (int e = 0; e < 16; ++e)
                *reinterpret_cast<float*>(s_lds + S1.tab + 4u * ((uint32_t)(e * S1.G + gj) * 32u + (uint32_t)ce)) = T[e];
        }
        __syncthreads();
        // ---- lookups: main chunk (G0 = 8 CW groups), then the refinement chunk (G1 groups).
        // (The weights are marked as changing here: otherwise their table addresses, the same in
        // every row, are computed once before the loop, which waits for the weights before the
        // first table build and holds 8 CW more registers.)
#pragma unroll
        for (int i = 0; i < CW; ++i) asm volatile("" : "+v"(wm[i]));
        uint32_t Wr = Wr0;
        asm volatile("" : "+v"(Wr));
        float sm[4] = {0.f, 0.f, 0.f, 0.f};
        if (S0.nb > 0) {
            const uint32_t lb = S0.tab + 4u * (uint32_t)lane;
            const uint32_t es = 128u * (uint32_t)S0.G;
#pragma unroll
            for (int j = 0; j < NS; ++j) {
#pragma unroll
                for (int m = 0; m < MW; ++m) {
                    // element m holds the chunk's word MW j + (m ^ am): groups 8 (MW j + (m ^ am)) + n
                    const uint32_t wv = __builtin_amdgcn_perm(0u, wm[MW * j + m], unperm);
                    const uint32_t bm = lb + 1024u * (uint32_t)(MW * j + (m ^ am));
#pragma unroll
                    for (int n = 0; n < 8; ++n) {
                        const uint32_t e = __builtin_amdgcn_ubfe(wv, 4 * n, 4);
                        sm[n & 3] += *reinterpret_cast<const float*>(s_lds + (__umul24(e, es) + bm) + 128u * (uint32_t)n);
                    }
                }
            }
        }
        float sr = 0.f;
        if (S1.nb > 0) {
            const uint32_t lb = S1.tab + 4u * (uint32_t)lane;
            const uint32_t es = 128u * (uint32_t)S1.G;
            uint32_t w = __builtin_amdgcn_perm(0u, Wr, unperm) >> (uint32_t)(c1 & 31);  // first nibble at bit 0
            for (int i = 0; i < S1.G; ++i) {  // G1 <= 8: one word
                const uint32_t e = w & 15u;
                w >>= 4;
                sr += *reinterpret_cast<const float*>(s_lds + (__umul24(e, es) + lb) + 128u * (uint32_t)i);
            }
        }
        float val = ar0 * ((sm[0] + sm[1]) + (sm[2] + sm[3])) + ar1 * sr;
        // ---- the row's 32 lanes
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) val += __shfl_xor(val, off, 32);
        if (lane == 0 && row < P.N) {
            float* dst = P.y + (int64_t)b * P.N + row;
            *dst = P.accumulate ? *dst + val : val;
        }
        if (b + 1 < P.batch) {  // every build of row b is done: the staging is free
            stage(b + 1);
            if (b + 2 < P.batch) prefetch(b + 2);
        }
    }
}

// A segment's chunking (plan.h) with its buffers; false when it cannot be cut that way.
bool chunk_segment(const Segment& sg, int cw_main, bool refinement, R4Seg& out) {
    out = R4Seg{};
    out.packed = sg.packed;
    out.alpha_r = static_cast<const float*>(sg.alpha_r);
    out.alpha_c = sg.alpha_c;
    out.idx = sg.idx;
    out.nb = sg.nb;
    out.Kv = sg.Kv;
    const plan::R4Chunk c = plan::r4_chunk(sg.nb, sg.Kv, refinement, cw_main);
    out.KT = c.KT;
    out.cpb = c.cpb;
    out.lcpb = c.lcpb;
    out.C = c.C;
    out.G = c.G;
    return c.ok;
}

}  // namespace

bool rows4_supported(const StepArgs& a) {
    if (a.gs || a.batch < 1 || a.batch > UBW_MAX_BATCH || !step_buffers_fit(a)) return false;
    const Segment empty{};
    const Segment& m = a.nseg >= 1 ? a.seg[0] : empty;
    const Segment& r = a.nseg >= 2 ? a.seg[1] : empty;
    if (m.nb == 0 && r.nb == 0) return false;
    const int cw = m.nb > 0 ? plan::r4_main_chunk_words(m.nb, m.Kv) : 1;
    if (cw > 8) return false;
    const plan::R4Chunk c0 = plan::r4_chunk(m.nb, m.Kv, false, cw), c1 = plan::r4_chunk(r.nb, r.Kv, true, cw);
    return c0.ok && c1.ok && plan::r4_lds_bytes(c0, c1, a.ldx) <= (int64_t)kR4LdsBytes;
}

hipError_t launch_rows4(const StepArgs& a, hipStream_t s) {
    if (!rows4_supported(a)) return hipErrorInvalidValue;
    R4Params P{};
    const Segment empty{};
    const int cw = a.seg[0].nb > 0 && a.nseg >= 1 ? plan::r4_main_chunk_words(a.seg[0].nb, a.seg[0].Kv) : 1;
    chunk_segment(a.nseg >= 1 ? a.seg[0] : empty, cw, false, P.seg[0]);
    chunk_segment(a.nseg >= 2 ? a.seg[1] : empty, cw, true, P.seg[1]);
    uint32_t off = 0;
    if (P.seg[0].nb) { P.seg[0].tab = off; off += 512u * (uint32_t)P.seg[0].C; }
    if (P.seg[1].nb) { P.seg[1].tab = off; off += 512u * (uint32_t)P.seg[1].C; }
    P.xs_off = off;
    P.K4 = (uint32_t)(ceil_div(a.ldx, 4) * 4);
    P.xsh = plan::r4_staging_shift(P.seg[0].C);
    const int64_t xsz = a.x_dtype == UBW_F16 ? 2 : 4;
    P.xvec = (a.ldx * xsz) % 16 == 0 && (reinterpret_cast<uintptr_t>(a.x) & 15u) == 0;
    const bool av = P.seg[0].Kv % 4 == 0 && (reinterpret_cast<uintptr_t>(P.seg[0].alpha_c) & 15u) == 0;
    P.x = a.x;
    P.ldx = a.ldx;
    P.batch = a.batch;
    P.y = a.y;
    P.N = a.N;
    P.NT = (int)ceil_div(a.N, kTileRows);
    P.accumulate = a.accumulate;
    P.err = a.ws;
    const dim3 grid((unsigned)ceil_div(a.N, kR4Rows));
    auto go = [&](auto xt, auto avc) -> hipError_t {
        using XT = decltype(xt);
        constexpr bool AV = decltype(avc)::value;
        switch (cw) {
            case 1: hipLaunchKernelGGL((k_rows4<XT, 1, AV>), grid, dim3(kR4Threads), 0, s, P); break;
            case 2: hipLaunchKernelGGL((k_rows4<XT, 2, AV>), grid, dim3(kR4Threads), 0, s, P); break;
            case 4: hipLaunchKernelGGL((k_rows4<XT, 4, AV>), grid, dim3(kR4Threads), 0, s, P); break;
            default: hipLaunchKernelGGL((k_rows4<XT, 8, AV>), grid, dim3(kR4Threads), 0, s, P); break;
        }
        return hipGetLastError();
    };
    if (a.x_dtype == UBW_F16)
        return av ? go(__half{}, std::true_type{}) : go(__half{}, std::false_type{});
    return av ? go(float{}, std::true_type{}) : go(float{}, std::false_type{});
}

}  // namespace ubw
