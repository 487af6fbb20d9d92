// Launch planning and argument checks of the GEMV calls: plain integer arithmetic with no HIP
// dependency, shared by the host code, the kernels (the functions marked UBW_HD) and a host
// test program built with address and undefined-behaviour sanitizers.
#pragma once
#include <stdint.h>

#include "../../include/ubw.h"

#if defined(__HIPCC__) || defined(__HIP__)
#define UBW_HD __host__ __device__
#else
#define UBW_HD
#endif

namespace ubw {
namespace plan {

constexpr int kTileRows = 256;   // rows of a packed tile
constexpr int kSliceCols = 256;  // columns of a packed tile (a slice of one row: 8 words)
constexpr int kTileWords = kTileRows * 8;

UBW_HD inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- division by a divisor fixed for the launch: q = (n * m) >> sh for 0 <= n < 2^31, with
// sh = 31 + ceil(log2 d) and m = ceil(2^sh / d); for 1 <= d < 2^31 the rounding error
// n (m d - 2^sh) / (d 2^sh) stays below 1 / d, so the quotient is exact.
struct FastDiv {
    uint32_t m, sh;
};
UBW_HD inline FastDiv fast_div(uint32_t d) {
    uint32_t l = 0;
    while (l < 31 && (1u << l) < d) ++l;
    const uint64_t p = 1ull << (31 + l);
    return FastDiv{(uint32_t)((p + d - 1) / d), 31 + l};
}
UBW_HD inline uint32_t div_by(uint32_t n, FastDiv f) { return (uint32_t)(((uint64_t)n * f.m) >> f.sh); }

// ---- the part of the unit list a workgroup works on. The list holds, row group by row group,
// the Urg units of each; workgroup g >= Zn (the Zn lowest IDs only zero rows) takes rank
// g - Zn of an equal contiguous split (the first ranks one unit more). XCD-local mode: workgroup
// g runs on XCD g mod 8 and works only on row groups rgo + 8 i (rgo = g mod 8), as rank
// (g - Zn) / 8 of that XCD's Gx workgroups over a list of those NRGx row groups; list row group
// i is matrix row group rgo + rgs i.
struct WgRange {
    int rgo, rgs, rank, Gx, NRGx;
    uint32_t x0, x1;  // units [x0, x1) of the workgroup's list
};
UBW_HD inline WgRange wg_range(int g, int Zn, int Gu, int NRG, int Urg, bool xmode) {
    WgRange w;
    if (xmode) {  // Zn is a multiple of 8: unit workgroup g - Zn is on the XCD of g
        w.rgo = g & 7;
        w.rgs = 8;
        w.rank = (g - Zn) >> 3;
        w.Gx = (Gu - w.rgo + 7) >> 3;
        w.NRGx = (NRG - w.rgo + 7) >> 3;
    } else {
        w.rgo = 0;
        w.rgs = 1;
        w.rank = g - Zn;
        w.Gx = Gu;
        w.NRGx = NRG;
    }
    const uint32_t Ux = (uint32_t)w.NRGx * (uint32_t)Urg;
    const uint32_t Qx = Ux / (uint32_t)w.Gx, Rx = Ux - Qx * (uint32_t)w.Gx;
    const uint32_t r = (uint32_t)w.rank;
    w.x0 = r * Qx + (r < Rx ? r : Rx);
    w.x1 = w.x0 + Qx + (r < Rx ? 1u : 0u);
    return w;
}

// Workgroups with units for U units when the device holds cap at once (two per CU): one per
// CU at batch 1 when the units fit in two per CU. A second workgroup on a CU runs behind the
// first (the CU issues the older waves' instructions first), so with one unit each the doubled
// CUs finish last; one workgroup per CU taking two units where needed ends sooner (measured,
// batch 1, K = 4096: 272 units 6.36 -> 6.24 us, 384 units 6.53 -> 6.44, 512 units
// 7.16 -> 6.61). With more units, or a larger batch, two workgroups per CU hide more latency.
inline int64_t default_workgroups(int64_t U, int64_t cap, int batch) {
    const int64_t cus = cap / 2;
    if (batch == 1 && U > cus && U <= cap) return cus;
    return cap;
}

// ---- which path a GEMV of b activation rows takes: the one predicted to be faster. Each path's
// time is linear in the weight bytes W (MB, main + refinement bases) and in the rows, with
// coefficients fitted (least squares on relative error) to cold timings of both paths on seven
// shapes (4096 x 4096 to 28672 x 8192 and 8192 x 28672, 2-3 bases, 5% salient columns in 2
// bases, fp16 x, y = result) at 1-16 rows. Tables: one launch of r <= 4 rows, a batch as
// consecutive launches of 4. Matrix cores: one launch of any b <= 16. Within 25% of every
// measurement; the faster path chosen in 76 of 77 cases (the miss: 8192 x 8192 at 6 rows,
// 0.86 us).
struct PathCost {
    double c0, c1, w0, w1;  // c0 + c1 (r - 1) + W (w0 + w1 (r - 1)) us
};
constexpr PathCost kTablesCost{5.10722, 0.92463, 0.21975, 0.12134};
constexpr PathCost kMfmaCost{17.20606, 0.34310, 0.60430, 0.02099};
inline double path_us(const PathCost& c, double W, int r) {
    return c.c0 + c.c1 * (r - 1) + W * (c.w0 + c.w1 * (r - 1));
}
inline double tables_us(double W, int b) {
    double t = 0.0;
    for (; b > 0; b -= 4) t += path_us(kTablesCost, W, b < 4 ? b : 4);
    return t;
}
inline double mfma_us(double W, int b) { return path_us(kMfmaCost, W, b); }
// weight_bytes: packed bytes of every base of the GEMV (main and refinement)
inline bool prefer_mfma(int64_t weight_bytes, int b) {
    const double W = (double)weight_bytes * 1e-6;
    return mfma_us(W, b) < tables_us(W, b);
}

// ---- group width 4: 32 chunks per row (32 / nb per base), C columns each.
struct R4Chunk {
    bool ok;
    int KT;    // 256-column tiles along the segment's columns
    int cpb;   // chunks per base
    int lcpb;  // log2(cpb)
    int C;     // columns per chunk (a multiple of 4)
    int G;     // 4-column groups per chunk
};
// Words per main chunk for K columns and nb bases: the smallest power of two >= nb K / 1024.
inline int r4_main_chunk_words(int nb, int64_t K) {
    const int64_t need = cdiv((int64_t)nb * K, 1024);
    int cw = 1;
    while (cw < need && cw < (1 << 20)) cw *= 2;
    return cw;
}
// The main segment (refinement = false) takes C = 32 cw columns per chunk; the refinement's
// virtual columns are padded to its tiles and cut into 32 chunks of Cs = nb KT 8 columns, at most
// one word (Cs <= 32, a divisor of 32).
inline R4Chunk r4_chunk(int nb, int64_t Kv, bool refinement, int cw_main) {
    R4Chunk c{};
    if (nb == 0) {
        c.ok = true;
        return c;
    }
    if (nb != 1 && nb != 2 && nb != 4) return c;
    c.KT = (int)cdiv(Kv, kSliceCols);
    c.cpb = 32 / nb;
    c.lcpb = nb == 1 ? 5 : nb == 2 ? 4 : 3;
    if (!refinement) {
        if (cw_main < 1 || cw_main > 8) return c;
        c.C = 32 * cw_main;
    } else {
        const int64_t cs = (int64_t)nb * c.KT * kSliceCols / 32;
        if (cs > 32 || cs % 4 != 0 || 32 % cs != 0) return c;
        c.C = (int)cs;
    }
    c.G = c.C / 4;
    c.ok = (int64_t)c.cpb * c.C >= Kv;
    return c;
}
// Staging of the activation row as fp32: column j at float j + 4 (j >> sh), 4 padding floats after
// every 4 C main columns (C a power of two), none without a main segment; the padded K4 columns
// (K rounded up to 4) and 4 zeros.
UBW_HD inline uint32_t r4_xpos(uint32_t j, uint32_t sh) { return j + 4u * (j >> sh); }
inline uint32_t r4_staging_shift(int C) {
    if (C <= 0) return 31;
    uint32_t sh = 0;
    while ((1 << sh) < 4 * C) ++sh;
    return sh;
}
inline int64_t r4_staging_floats(int64_t K, int C) {
    const int64_t K4 = cdiv(K, 4) * 4;
    return K4 + 4 * (K4 >> r4_staging_shift(C)) + 4;
}
// LDS bytes of a group-width-4 launch: 16 entries x 4 bytes per 4-column group of each of the 32
// chunks of both segments (512 C bytes a segment), then the staging.
inline int64_t r4_lds_bytes(const R4Chunk& m, const R4Chunk& r, int64_t K) {
    return 512ll * (m.C) + 512ll * (r.C) + 4ll * r4_staging_floats(K, m.C);
}

// ---- argument checks of the C ABI (every one on the host, before anything is enqueued)
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool fits_int(int64_t v) { return v >= 1 && v <= (int64_t)0x3FFFFFFF; }
inline int64_t packed_words(int nb, int64_t N, int64_t K) {
    return (int64_t)nb * cdiv(N, kTileRows) * cdiv(K, kSliceCols) * kTileWords;
}
inline int check_gemv_common(const void* packed, const void* ar, const void* ac, int nb, int64_t N, int64_t Kv,
                             const void* x, int x_dtype, int batch, const void* y) {
    if (!packed || !ar || !ac || !x || !y) return UBW_EINVAL;
    if (nb < 1 || nb > 64 || !fits_int(N) || !fits_int(Kv)) return UBW_EINVAL;
    if (batch < 1 || batch > UBW_MAX_BATCH) return UBW_EINVAL;
    if (x_dtype != UBW_F16 && x_dtype != UBW_F32) return UBW_EUNSUPPORTED;
    if (!aligned16(packed)) return UBW_EALIGN;
    return UBW_OK;
}
// Words of a GEMV workspace at group width 8: a 16-word header (word 0: errors), then 64 words
// per 256-row group (arrival counter at word 0, zeroing flag at word 32).
constexpr int kWsHeaderWords = 16;
constexpr int kWsRowGroupWords = 64;
inline int64_t workspace_words(int64_t N) { return kWsHeaderWords + kWsRowGroupWords * cdiv(N, kTileRows); }
// NULL with 0 bytes means "none"; otherwise 16-byte aligned and large enough: the row-group
// counters of N rows at g = 8, the header alone at g = 4.
inline int check_workspace(const void* ws, uint64_t ws_bytes, int64_t N, int g) {
    if (ws == nullptr) return ws_bytes == 0 ? UBW_OK : UBW_EINVAL;
    if (!aligned16(ws)) return UBW_EALIGN;
    const int64_t need = g == 4 ? kWsHeaderWords : workspace_words(N);
    if (ws_bytes < (uint64_t)need * 4u) return UBW_ESIZE;
    return UBW_OK;
}

}  // namespace plan
}  // namespace ubw
