// The GEMV step for several activation rows at once on the matrix cores.
//
// FluxBin (gist.science/ko/paper/2608.15602), technical summary, "1. Algorithm innovation" and
// "2. Kernel innovation": each base is
// (alpha_r alpha_c^T) (.) B with B in {-1,+1}, so y_b = sum_k alpha_r^(k) (.) (B^(k) v_b^(k)) with
// v_b^(k) = alpha_c^(k) (.) x_b. The page's table lookup replaces the multiply-adds of one
// activation row; with several rows the tables must be built and searched once per row, while
// B^(k) V^(k) (V = the rows' v side by side) is a dense contraction whose cost does not grow with
// the rows up to the matrix instruction's width. Here the sign bits are expanded to fp16 +-1
// (exact) and multiplied on v_mfma_f32_16x16x32_f16 against V split into fp16 high and low
// parts, accumulating in fp32. Each activation row of a staged slice is scaled by a power of two
// 2^e (exact) that puts its largest |v| in [2^14, 2^15), so no value overflows fp16; the MFMA
// result of the slice is scaled back before it is added to the running sums. Precision of the
// split, per element (hi = v rounded toward zero to fp16, lo = the exact fp32 remainder v - hi
// rounded the same way): |v - hi - lo| < 2^-20 |v| + 2^-24 2^e <= 2^-20 |v| + 2^-38 m, where m
// is the largest |v| of the activation row in the slice (the 2^-24 term covers fp16's
// subnormal spacing). The tables use v itself in fp32 (2^-24 |v|), so the two paths agree to
// that bound per element plus their different fp32 summation orders. Main bases and the salient
// refinement (columns gathered through idx) go through the same loop.
//
// GEMVs that share x run in one launch: grid x covers their row tiles one GEMV after the other
// (so the small k and v projections fill the CUs next to q), grid y the column chunks, each GEMV
// with its own count (its workgroups beyond it exit at once).
// Workgroup (row tile rt, chunk kc): 256 threads, 4 waves, wave w owns tile rows 64 w .. +63 as
// four 16-row blocks. For each base and each 256-column slice of the chunk:
//   * the packed words of the wave's rows are loaded once (the tile layout: row rho's 8 words as
//     two 16-byte halves, slot s holding canonical word s ^ ((rho & 31) >> 2) with bytes permuted
//     by rho & 3): lane (g = lane / 16, r16) loads slots 2 g and 2 g + 1 of its row, and the four
//     lanes of a row trade bytes with two cross-lane swaps until each holds the canonical byte g
//     of every word of its row,
//   * v = alpha_c * x for the slice's 256 columns and up to 16 activation rows goes to LDS as
//     fp16 hi and lo (each thread a row's 8 column pairs 32 i + 2 cg, so that the 16 threads
//     of a row read consecutive columns),
//   * per 32-column step t: A = the 16 rows' 8 sign bits of columns 32 t + 8 g .. + 7, expanded
//     nibble by nibble through a 16-entry table to 8 halves; B = v hi (then lo) of the same
//     columns; two MFMAs
//     (at 8 activation rows or fewer, one: hi of row b is column b, lo column 8 + b).
// The k order inside an operand only has to be the same for A and B (k is summed over): lane
// group g holds columns 8 g .. 8 g + 7 of the step in both. Each lane holds D[4 g + j][lane
// mod 16] of each 16-row block (row 4 g + j, activation row lane mod 16); per slice it scales
// that back by the row's power of two and by alpha_r of the slice's base into one running sum
// per (row, activation row), which goes into y at the end (atomics when the columns are split
// over several workgroups). The staging area is double-buffered, so one barrier per slice
// suffices and a wave done with a slice's matrix work stages the next. Each slice's loads are
// issued when it is staged, and alpha_r of the slot's base sits in LDS: holding the next slice's
// operands or the 16 scales in registers would leave room for two or three waves per SIMD, and
// four (127 VGPRs, 40 KiB of LDS per workgroup) hide more of the LDS and memory latency (70B
// gate at 16 rows: 131 us at two, 113 us at three, 107 us at four).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>

#include "ubw_internal.h"

namespace ubw {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kMmThreads = 256;
constexpr int kMmBatch = 16;     // activation rows per launch (the MFMA's N)
constexpr int kMmSlots = 6;      // main + refinement bases per launch
constexpr int kMmMinSlices = 3;  // slices per workgroup before the columns are split further
constexpr int kBStride = 132;    // dwords per activation row of a staged slice (128 + 4: no bank conflicts)

struct MmSeg {
    const uint32_t* packed;
    const float* alpha_r;  // [nb][N]
    const float* alpha_c;  // [nb][Kv]
    const int32_t* idx;    // [Kv] or nullptr
    int nb, Kv, KT;
};

// One GEMV of a launch.
struct MmParams {
    MmSeg seg[2];
    float* y;
    int N, NT;
    int ST;      // slices over both segments (seg[0].KT + seg[1].KT)
    int KC;      // column chunks (grid y at most this GEMV's KC; workgroups beyond it exit)
    int atomic;  // 1: add into y with atomics, 0: store
    uint32_t* err;  // the GEMV's workspace (word 0: bit 1 set for a salient index out of range or
                    // out of order), or nullptr
};

// GEMVs sharing x in one launch: grid x covers their row tiles one GEMV after the other.
struct MmGroup {
    MmParams p[kMaxGroup];
    int tile0[kMaxGroup + 1];  // first grid x of GEMV i; tile0[count] = grid x
    int count;
    int batch;
    const void* x;
    int64_t ldx;
};


// Raw buffer loads: an offset at or beyond the descriptor's size returns 0 and touches no
// memory, so loads that are not wanted are issued with a size-0 descriptor instead of being
// branched around (a branch would make the compiler wait for each load inside it).
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc rsrc(const void* p, uint32_t bytes) {
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
__device__ __forceinline__ uint32_t ldx_raw(Rsrc r, uint32_t i, float*) { return ld32(r, 4u * i); }
__device__ __forceinline__ uint32_t ldx_raw(Rsrc r, uint32_t i, __half*) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)(2u * i), 0, 0);
}
// An element index whose byte offset lies beyond every activation buffer (below 2 GiB): the
// buffer load returns 0 for it.
__device__ __forceinline__ uint32_t x_oob(float*) { return 0x3FFFFFFFu; }
__device__ __forceinline__ uint32_t x_oob(__half*) { return 0x7FFFFFFFu; }
__device__ __forceinline__ float x_from_raw(uint32_t v, float*) { return __uint_as_float(v); }
__device__ __forceinline__ float x_from_raw(uint32_t v, __half*) { return __half2float(__ushort_as_half((unsigned short)v)); }


// kPack (at most 8 activation rows): v hi of row b is the MFMA's column b and v lo its column
// 8 + b, so one MFMA per step instead of two; the two columns' sums are added at the end.
template <typename XT, bool kPack>
// four waves per SIMD: see the header
__global__ __launch_bounds__(kMmThreads, 4) void k_pm1_mfma(const MmGroup G) {
    // nibble -> 4 halves of +-1: 16 entries of 8 bytes, one dword per bank, so any pattern of
    // lookups is conflict-free (lanes that read the same entry get it broadcast). (A 256-entry
    // byte table of 16-byte entries, one read per byte, spread its lookups over 8 bank groups:
    // 1.47e7 bank-conflict cycles on the 70B gate at 16 rows, 24 us per CU of a 104 us launch.)
    __shared__ __align__(16) uint32_t s_lut[16 * 2];
    // staged v (hi, lo) and row scales (row b holds v * 2^-e[b]), two buffers: a slice is staged
    // into one while the other is still read by the previous slice's matrix work
    __shared__ __align__(16) uint32_t s_v[2][2][kMmBatch * kBStride];
    __shared__ int s_e[2][kMmBatch];
    __shared__ float s_ar[2][kTileRows];  // alpha_r of the slot's base at the tile's rows
    int gi = 0;  // this workgroup's GEMV (uniform)
    while (gi + 1 < G.count && (int)blockIdx.x >= G.tile0[gi + 1]) ++gi;
    const MmParams& P = G.p[gi];
    if ((int)blockIdx.y >= P.KC) return;  // the whole workgroup: no barrier is left waiting
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, g = lane >> 4;
    const int rt = (int)blockIdx.x - G.tile0[gi];
    const int s0 = (int)((int64_t)blockIdx.y * P.ST / P.KC);
    const int s1 = (int)((int64_t)(blockIdx.y + 1) * P.ST / P.KC);
    const XT* x = static_cast<const XT*>(G.x);
    const int batch = G.batch;
    const int64_t ldx = G.ldx;

    if (tid < 32) {  // expansion table: entry n, half i = +1 (0x3C00) if bit i of n is set, else -1 (0xBC00)
        const int n = tid >> 1, q = tid & 1;
        const uint32_t lo = (n >> (2 * q)) & 1 ? 0x3C00u : 0xBC00u;
        const uint32_t hi = (n >> (2 * q + 1)) & 1 ? 0x3C00u : 0xBC00u;
        s_lut[tid] = lo | (hi << 16);
    }

    // Per 16-row block m of this wave: the lane's row is rho = 64 w + 16 m + r16, whose slots are
    // permuted by a = ((rho & 31) >> 2) = 4 (m & 1) + (r16 >> 2) and bytes by c = r16 & 3: slot q
    // holds word q ^ a, and canonical byte g of each word sits at byte g ^ c. Lane (g, r16) loads
    // slots 2 g and 2 g + 1 of its row and needs byte g ^ c of all eight; the four lanes of a row
    // (16 apart) trade those bytes in two cross-lane swaps. Byte selectors, fixed per lane:
    const uint32_t cc = (uint32_t)(r16 & 3);
    const uint32_t alo = (uint32_t)(r16 >> 2);  // low two bits of a (the same for every m)
    auto pair_sel = [](uint32_t b0, uint32_t b1) { return b0 | ((4u + b0) << 8) | (b1 << 16) | ((4u + b1) << 24); };
    // the 2 bytes (one per loaded slot) each lane group needs: groups 0, 1 and groups 2, 3
    const uint32_t sel_lo = pair_sel(cc, cc ^ 1u), sel_hi = pair_sel(cc ^ 2u, cc ^ 3u);
    // after the swaps a lane holds byte g ^ c of slots {0, 1, 4, 5} in one dword and {2, 3, 6, 7}
    // in the other; position of slot s in that 8-byte pair: nibble s of 0x76325410. The dword of
    // words 4 h .. 4 h + 3 (h = 0, 1) takes at byte j word 4 h + j, i.e. slot (4 h + j) ^ a.
    uint32_t selc[2][2];
#pragma unroll
    for (int pm = 0; pm < 2; ++pm)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            uint32_t sel = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t slot = ((uint32_t)j ^ alo) + 4u * (uint32_t)(hh ^ pm);
                sel |= ((0x76325410u >> (4u * slot)) & 0xFu) << (8 * j);
            }
            selc[pm][hh] = sel;
        }

    // running sums of y for the lane's 16 (row, activation row) pairs: D[4 g + j][r16] of block m
    float acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = 0.f;

    const MmSeg S0 = P.seg[0], S1 = P.seg[1];
    const int nb0 = S0.nb, nbt = S0.nb + S1.nb;
    // staging role: activation row b, the 8 column pairs 32 i + 2 cg (+1), i < 8: at each step
    // the 16 threads of a row read 32 consecutive columns (coalesced)
    const int b = tid >> 4, cg = tid & 15;
    const bool brow = b < batch;
    int buf = 0, arb = 0;
    // Grouped launches: wave priority from the (base, slice) steps this workgroup has left, so
    // that of the workgroups sharing a CU the ones behind issue first.
    const bool balance = G.count > 1;
    int left = 0;
#pragma unroll
    for (int slot = 0; slot < kMmSlots; ++slot) {
        if (slot >= nbt) break;
        const int lo = slot >= nb0 ? (s0 > S0.KT ? s0 - S0.KT : 0) : s0;
        const int hi = slot >= nb0 ? s1 - S0.KT : (s1 < S0.KT ? s1 : S0.KT);
        left += hi > lo ? hi - lo : 0;
    }
#pragma unroll
    for (int slot = 0; slot < kMmSlots; ++slot) {
        if (slot >= nbt) break;
        const int si = slot < nb0 ? 0 : 1;
        const int k = si ? slot - nb0 : slot;
        const MmSeg sg = si ? S1 : S0;
        const int lo = si ? (s0 > S0.KT ? s0 - S0.KT : 0) : s0;
        const int hi = si ? s1 - S0.KT : (s1 < S0.KT ? s1 : S0.KT);
        if (lo >= hi) continue;
        const int nitems = sg.KT * sg.nb;
        const float* acr = sg.alpha_c + (int64_t)k * sg.Kv;
        // alpha_r of this base at the tile's 256 rows, in LDS (two buffers by the slot's parity: a
        // slower wave may still read the previous slot's; every slot with slices passes barriers
        // before its buffer is written again)
        {
            const int row = rt * kTileRows + tid;
            s_ar[arb][tid] = sg.alpha_r[(int64_t)k * P.N + (row < P.N ? row : P.N - 1)];
        }
        // Loads of one slice: the wave's packed rows, alpha_c and (main segment) x or
        // (refinement) idx of the staged columns. Every load is issued (clamped to a valid address,
        // the value dropped later) before any is used.
        uint2 pq[4];  // per 16-row block: slots 2 g and 2 g + 1 of the lane's row
        uint32_t xi[16], xw[16], aw[16];  // idx (refinement), raw x bits (main), alpha_c bits
        const Rsrc r_ac = rsrc(acr, (uint32_t)sg.Kv * 4u);
        // this row tile's slab of the segment (all slices and bases): below 2 GiB (checked)
        const Rsrc r_w = rsrc(sg.packed + (int64_t)rt * nitems * kTileWords, (uint32_t)nitems * kTileWords * 4u);
        const Rsrc r_xg = rsrc(x, si ? (uint32_t)batch * (uint32_t)ldx * (uint32_t)sizeof(XT) : 0u);
        const Rsrc r_idx = rsrc(S1.idx, si ? (uint32_t)sg.Kv * 4u : 0u);
        // descriptors are uniform over the wave: x as a whole, the row in the offset
        const Rsrc r_xd = rsrc(x, si ? 0u : (uint32_t)batch * (uint32_t)ldx * (uint32_t)sizeof(XT));
        const uint32_t xrow = (uint32_t)(brow ? b : 0) * (uint32_t)ldx;
        auto issue = [&](int ks) {
            // the item's 8 KiB within this row tile's slab (32-bit offsets)
            const uint32_t ib = ((uint32_t)ks * (uint32_t)sg.nb + (uint32_t)k) * (kTileWords * 4u);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const uint32_t rho = (uint32_t)(64 * w + 16 * m + r16);
                // slots 0..3 of a row are its first 16-byte half, slots 4..7 the second
                pq[m] = ld64(r_w, ib + 16u * ((g >> 1) ? kTileRows + rho : rho) + 8u * (uint32_t)(g & 1));
            }
            // per-lane base offsets and a constant per element (the load's immediate offset);
            // columns past Kv read 0 from alpha_c and idx (out of the descriptors' range) and
            // are dropped at staging
            const uint32_t col0 = (uint32_t)(ks * kSliceCols + 2 * cg);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t d = 32u * (uint32_t)(i >> 1) + (uint32_t)(i & 1);
                aw[i] = ld32(r_ac, 4u * col0 + 4u * d);
                xi[i] = ld32(r_idx, 4u * col0 + 4u * d);
                xw[i] = ldx_raw(r_xd, xrow + col0 + d, (XT*)nullptr);
            }
        };
        for (int ks = lo; ks < hi; ++ks) {
            if (balance) {
                if (left >= 9) __builtin_amdgcn_s_setprio(3);
                else if (left >= 6) __builtin_amdgcn_s_setprio(2);
                else if (left >= 3) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
                --left;
            }
            issue(ks);
            // stage v = alpha_c * x of this slice, each activation row scaled by 2^-e
            {
                float xv[16];
                if (si) {  // the gather through idx (the loads wait here, where they are used anyway)
                    // VCM: an index outside [0, K) reads beyond the buffer (0: its column adds
                    // nothing); a padding column past s has idx 0 (read out of idx's range) and
                    // alpha_c 0. The indices are checked and reported once per launch, at the end.
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const uint32_t off = xi[i] < (uint64_t)ldx ? xrow + xi[i] : x_oob((XT*)nullptr);
                        xv[i] = x_from_raw(ldx_raw(r_xg, off, (XT*)nullptr), (XT*)nullptr);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 16; ++i) xv[i] = x_from_raw(xw[i], (XT*)nullptr);
                }
                const int col0 = ks * kSliceCols + 2 * cg;
                float v[16];
                float mx = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int col = col0 + 32 * (i >> 1) + (i & 1);
                    v[i] = brow && col < sg.Kv ? __uint_as_float(aw[i]) * xv[i] : 0.f;
                    mx = fmaxf(mx, fabsf(v[i]));
                }
                // the 16 threads of row b are 16 consecutive lanes
#pragma unroll
                for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
                int eb = 0;
                if (mx > 0.f) {
                    int E;
                    frexpf(mx, &E);  // mx in [2^(E-1), 2^E)
                    eb = E - 15;
                }
                if (cg == 0) s_e[buf][b] = eb;
                uint32_t hv[8], lv[8];
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    // hi = v rounded toward zero to fp16 (a pair per instruction), lo = the
                    // remainder (exact in fp32) rounded the same way: |v - hi - lo| < 2^-20 |v|
                    const float v0 = ldexpf(v[i], -eb), v1 = ldexpf(v[i + 1], -eb);
                    const auto hp = __builtin_amdgcn_cvt_pkrtz(v0, v1);
                    const auto lp = __builtin_amdgcn_cvt_pkrtz(v0 - (float)hp[0], v1 - (float)hp[1]);
                    hv[i / 2] = __builtin_bit_cast(uint32_t, hp);
                    lv[i / 2] = __builtin_bit_cast(uint32_t, lp);
                }
                // the pair of columns 32 i + 2 cg (+1) is dword 16 i + cg of the row
                if (kPack) {
                    if (b < 8) {
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            s_v[buf][0][b * kBStride + 16 * i + cg] = hv[i];
                            s_v[buf][0][(b + 8) * kBStride + 16 * i + cg] = lv[i];
                        }
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        s_v[buf][0][b * kBStride + 16 * i + cg] = hv[i];
                        s_v[buf][1][b * kBStride + 16 * i + cg] = lv[i];
                    }
                }
            }
            // canonical byte g of words 0..7 of each row, in word order: two dwords per block
            uint32_t cb[4][2];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // per loaded slot, the byte of each lane group: groups 0, 1 in Plo, 2, 3 in Phi
                const uint32_t Plo = __builtin_amdgcn_perm(pq[m].y, pq[m].x, sel_lo);
                const uint32_t Phi = __builtin_amdgcn_perm(pq[m].y, pq[m].x, sel_hi);
                // lanes l and l ^ 32 (groups g, g ^ 2): the upper half's Plo and the lower half's
                // Phi change places; then each lane holds the bytes of groups g & 2 (low 16 bits)
                // and (g & 2) + 1 from source groups g & 1 (first) and (g & 1) + 2 (second)
                const auto s1 = __builtin_amdgcn_permlane32_swap(Plo, Phi, false, false);
                const uint32_t A = __builtin_amdgcn_perm(s1[1], s1[0], 0x05040100u);  // for group g & 2
                const uint32_t B = __builtin_amdgcn_perm(s1[1], s1[0], 0x07060302u);  // for group (g & 2) + 1
                // lanes l and l ^ 16 (groups g, g ^ 1): the odd group's A and the even group's B
                // change places; then the first dword holds slots {0, 1, 4, 5}, the second {2, 3, 6, 7}
                const auto s2 = __builtin_amdgcn_permlane16_swap(A, B, false, false);
                cb[m][0] = __builtin_amdgcn_perm(s2[1], s2[0], selc[m & 1][0]);
                cb[m][1] = __builtin_amdgcn_perm(s2[1], s2[0], selc[m & 1][1]);
            }
            __syncthreads();
            float4_t c[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) c[m] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint4 bh = *reinterpret_cast<const uint4*>(&s_v[buf][0][r16 * kBStride + 16 * t + 4 * g]);
                const half8_t Bh = __builtin_bit_cast(half8_t, bh);
                half8_t Bl;
                if (!kPack) {
                    const uint4 bl = *reinterpret_cast<const uint4*>(&s_v[buf][1][r16 * kBStride + 16 * t + 4 * g]);
                    Bl = __builtin_bit_cast(half8_t, bl);
                }
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const uint32_t e = cb[m][t >> 2] >> (8 * (t & 3));
                    const uint2 a0 = *reinterpret_cast<const uint2*>(&s_lut[2 * (e & 15u)]);
                    const uint2 a1 = *reinterpret_cast<const uint2*>(&s_lut[2 * ((e >> 4) & 15u)]);
                    const half8_t A = __builtin_bit_cast(half8_t, make_uint4(a0.x, a0.y, a1.x, a1.y));
                    c[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bh, c[m], 0, 0, 0);
                    if (!kPack) c[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bl, c[m], 0, 0, 0);
                }
            }
            // D's column is activation row r16 (kPack: r16 mod 8): undo that row's staging scale,
            // apply alpha_r
            const int ec = s_e[buf][kPack ? (r16 & 7) : r16];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[m][j] += s_ar[arb][64 * w + 16 * m + 4 * g + j] * ldexpf(c[m][j], ec);
            // The next slice is staged into the other buffer: its last readers (the slice before
            // this one) have all passed this slice's barrier.
            buf ^= 1;
        }
        arb ^= 1;
    }

    // VCM index check, once per GEMV (its first row tile and column chunk), after the matrix work:
    // an index outside [0, K) or not above the one before it sets bit 1 of workspace word 0
    if (rt == 0 && blockIdx.y == 0 && S1.nb > 0 && P.err != nullptr) {
        const Rsrc r_i = rsrc(S1.idx, (uint32_t)S1.Kv * 4u);
        bool bad = false;
        for (int q = tid; q < S1.Kv; q += kMmThreads) {
            const uint32_t v = ld32(r_i, 4u * (uint32_t)q), pv = ld32(r_i, q > 0 ? 4u * (uint32_t)(q - 1) : 0u);
            bad = bad || v >= (uint64_t)ldx || (q > 0 && (int)pv >= (int)v);
        }
        if (bad) atomicOr(P.err, kWsErrIndex);
    }

    // y[b][row] (+)= the running sums (kPack: lane r16 < 8 adds the lo sums of lane r16 + 8)
    if (kPack) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[m][j] += __shfl_xor(acc[m][j], 8);
    }
    if (r16 >= batch) return;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = rt * kTileRows + 64 * w + 16 * m + 4 * g + j;
            if (row >= P.N) continue;
            float* dst = P.y + (int64_t)r16 * P.N + row;
            if (P.atomic) atomicAdd(dst, acc[m][j]);
            else *dst = acc[m][j];
        }
    }
}

// y = 0 for the GEMVs of a launch whose column chunks all add with atomics: one launch for all.
struct MmZero {
    float* y[kMaxGroup];
    int64_t end[kMaxGroup];  // outputs to clear in buffers 0 .. i together
    int count;
};

__global__ void k_mm_zero(const MmZero Z) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int j = 0;
    while (j < Z.count && i >= Z.end[j]) ++j;
    if (j == Z.count) return;
    Z.y[j][i - (j ? Z.end[j - 1] : 0)] = 0.f;
}

}  // namespace

// Workgroups of the instance the current device holds at once (CUs x occupancy) and its CU
// count, cached per device (thread-safe: each entry is written once with the value every thread
// computes; devices numbered kMaxDevices or above are queried on every call).
struct MmCapacity {
    int64_t cap, cus;
};
template <typename XT>
static MmCapacity mm_capacity() {
    static std::atomic<int64_t> cache[kMaxDevices];  // cus << 32 | workgroups per CU
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MmCapacity{0, 0};
    const bool cached = dev >= 0 && dev < kMaxDevices;
    int64_t v = cached ? cache[dev].load(std::memory_order_relaxed) : 0;
    if (v <= 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_pm1_mfma<XT, false>, kMmThreads, 0) != hipSuccess)
            return MmCapacity{0, 0};
        v = ((int64_t)cus << 32) | (per_cu > 0 ? per_cu : 1);
        if (cached) cache[dev].store(v, std::memory_order_relaxed);
    }
    const int64_t cus = v >> 32;
    return MmCapacity{cus * (v & 0xFFFFFFFF), cus};
}

bool mfma_step_supported(const StepArgs& a) {
    if (a.gs || a.batch < 1 || a.batch > kMmBatch || !step_buffers_fit(a)) return false;
    const int nbt = a.seg[0].nb + (a.nseg > 1 ? a.seg[1].nb : 0);
    return nbt >= 1 && nbt <= kMmSlots;
}

hipError_t launch_step_mfma_group(const StepArgs* a, int count, hipStream_t s) {
    if (count < 1 || count > kMaxGroup) return hipErrorInvalidValue;
    MmGroup G{};
    G.count = count;
    G.batch = a[0].batch;
    G.x = a[0].x;
    G.ldx = a[0].ldx;
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) {
        if (!mfma_step_supported(a[i]) || a[i].x != a[0].x || a[i].batch != a[0].batch ||
            a[i].x_dtype != a[0].x_dtype || a[i].ldx != a[0].ldx)
            return hipErrorInvalidValue;
        if (a[i].nseg > 1 && a[i].seg[1].idx == nullptr) return hipErrorInvalidValue;
        MmParams& P = G.p[i];
        for (int j = 0; j < 2; ++j) {
            if (j < a[i].nseg) {
                const Segment& sg = a[i].seg[j];
                P.seg[j] = MmSeg{sg.packed, static_cast<const float*>(sg.alpha_r), sg.alpha_c, sg.idx, sg.nb, sg.Kv,
                                 (int)ceil_div(sg.Kv, kSliceCols)};
            } else {
                P.seg[j] = MmSeg{nullptr, nullptr, nullptr, nullptr, 0, 0, 0};
            }
        }
        P.y = a[i].y;
        P.err = a[i].ws;
        P.N = a[i].N;
        P.NT = (int)ceil_div(a[i].N, kTileRows);
        P.ST = P.seg[0].KT + P.seg[1].KT;
        if (P.ST < 1) return hipErrorInvalidValue;
        G.tile0[i] = (int)tiles;
        tiles += P.NT;
    }
    if (tiles > INT32_MAX) return hipErrorInvalidValue;
    G.tile0[count] = (int)tiles;
    // At most as many workgroups as the device holds at once, split over whole
    // slices. Each workgroup of a split chunk adds 16 x 256 partial sums to y with atomics and
    // loads its own tile setup, so a chunk takes at least kMmMinSlices slices unless that would
    // leave CUs idle (8192 x 8192 at 16 rows: 76 us at about one slice per chunk, 59 us at two,
    // 52 us at three). The GEMVs of a group share those workgroups: each gets the same number of
    // workgroups per row tile (or fewer, when it has fewer slices).
    const MmCapacity mc = a[0].x_dtype == UBW_F16 ? mm_capacity<__half>() : mm_capacity<float>();
    if (mc.cap <= 0) return hipErrorInvalidConfiguration;
    int64_t kc_grid = 1;
    MmZero Z{};
    for (int i = 0; i < count; ++i) {
        MmParams& P = G.p[i];
        int64_t kc = mc.cap / tiles;
        const int64_t kc_fill = ceil_div(mc.cus, tiles);
        const int64_t kc_min_slices = ceil_div((int64_t)P.ST, (int64_t)kMmMinSlices);
        const int64_t kc_want = kc_fill > kc_min_slices ? kc_fill : kc_min_slices;
        kc = kc > kc_want ? kc_want : kc;
        kc = kc < 1 ? 1 : (kc > P.ST ? P.ST : kc);
        kc = kc > 65535 ? 65535 : kc;
        P.KC = (int)kc;
        kc_grid = kc > kc_grid ? kc : kc_grid;
        P.atomic = (a[i].accumulate || P.KC > 1) ? 1 : 0;
        if (!a[i].accumulate && P.KC > 1) {
            Z.y[Z.count] = a[i].y;
            Z.end[Z.count] = (Z.count ? Z.end[Z.count - 1] : 0) + (int64_t)a[i].batch * a[i].N;
            ++Z.count;
        }
    }
    if (Z.count > 0) {
        const int64_t n = Z.end[Z.count - 1];
        if (ceil_div(n, 256) > INT32_MAX) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_mm_zero, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, Z);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)tiles, (unsigned)kc_grid);
    const bool pack = G.batch <= 8;
    if (a[0].x_dtype == UBW_F16) {
        if (pack) hipLaunchKernelGGL((k_pm1_mfma<__half, true>), grid, dim3(kMmThreads), 0, s, G);
        else hipLaunchKernelGGL((k_pm1_mfma<__half, false>), grid, dim3(kMmThreads), 0, s, G);
    } else {
        if (pack) hipLaunchKernelGGL((k_pm1_mfma<float, true>), grid, dim3(kMmThreads), 0, s, G);
        else hipLaunchKernelGGL((k_pm1_mfma<float, false>), grid, dim3(kMmThreads), 0, s, G);
    }
    return hipGetLastError();
}

hipError_t launch_step_mfma(const StepArgs& a, hipStream_t s) { return launch_step_mfma_group(&a, 1, s); }

}  // namespace ubw
