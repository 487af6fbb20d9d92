// Host checks of the GEMV launch planning and argument validation (ultra_bit_weight_uint32_amd/
// csrc/plan.h), built with -fsanitize=address,undefined: every function over random and edge
// shapes, each result compared with a plain recomputation. Prints "ok" and exits 0 on success.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "../../ultra_bit_weight_uint32_amd/csrc/plan.h"

using namespace ubw::plan;

static int fails = 0;
#define CHECK(c, ...)                                                       \
    do {                                                                    \
        if (!(c)) {                                                         \
            if (fails++ < 20) {                                             \
                std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);   \
                std::fprintf(stderr, __VA_ARGS__);                          \
                std::fprintf(stderr, "\n");                                 \
            }                                                               \
        }                                                                   \
    } while (0)

static uint64_t rnd(std::mt19937_64& rng, uint64_t lo, uint64_t hi) {  // uniform in [lo, hi]
    return lo + rng() % (hi - lo + 1);
}

// q = n / d exactly for every divisor 1 <= d < 2^31 and numerator n < 2^31
static void check_fast_div(std::mt19937_64& rng) {
    std::vector<uint32_t> ds = {1, 2, 3, 5, 7, 8, 9, 255, 256, 257, 65535, 65536, 65537, (1u << 24) - 1, 1u << 24,
                                (1u << 30) + 1, (1u << 31) - 1};
    for (int i = 0; i < 3000; ++i) ds.push_back((uint32_t)rnd(rng, 1, (1u << 31) - 1));
    for (int i = 0; i < 500; ++i) ds.push_back((uint32_t)rnd(rng, 1, 200));
    for (uint32_t d : ds) {
        const FastDiv f = fast_div(d);
        std::vector<uint64_t> ns = {0, 1, d - 1ull, d, d + 1ull, 2ull * d - 1, 2ull * d, (1ull << 31) - 1};
        for (uint64_t k = (1ull << 31) / d; k > 0 && ns.size() < 12; k /= 2) ns.push_back(k * d - 1);
        for (int i = 0; i < 64; ++i) ns.push_back(rnd(rng, 0, (1ull << 31) - 1));
        for (uint64_t n : ns) {
            if (n >= (1ull << 31)) continue;
            const uint32_t q = div_by((uint32_t)n, f);
            CHECK(q == (uint32_t)(n / d), "fast_div: %llu / %u gave %u", (unsigned long long)n, d, q);
        }
    }
}

// Every (row group, unit) of the list is taken by exactly one workgroup, ranges are contiguous
// and equal to one unit, and in XCD-local mode workgroup g works on row groups of XCD g mod 8.
static void check_wg_range(std::mt19937_64& rng) {
    for (int it = 0; it < 4000; ++it) {
        const int NRG = (int)rnd(rng, 1, it < 2000 ? 40 : 400);
        const int Urg = (int)rnd(rng, 1, it < 2000 ? 20 : 120);
        const int64_t U = (int64_t)NRG * Urg;
        const int Gu = (int)rnd(rng, 1, (uint64_t)(U < 1200 ? U : 1200));
        const bool xmode = Gu >= 8 && NRG >= 8 && (rng() & 1);
        const int Zn = xmode ? (int)(cdiv(NRG, 8) * 8) : ((rng() & 1) ? NRG : 0);
        std::vector<uint8_t> seen((size_t)U, 0);
        std::vector<int> sizes;
        int64_t prev_end[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        bool prev_set[8] = {false, false, false, false, false, false, false, false};
        for (int g = Zn; g < Zn + Gu; ++g) {
            const WgRange w = wg_range(g, Zn, Gu, NRG, Urg, xmode);
            CHECK(w.Gx >= 1 && w.rank >= 0 && w.rank < w.Gx, "rank %d of %d", w.rank, w.Gx);
            CHECK(w.x0 <= w.x1 && (int64_t)w.x1 <= (int64_t)w.NRGx * Urg, "range [%u, %u) of %d", w.x0, w.x1,
                  w.NRGx * Urg);
            if (xmode) {
                CHECK(w.rgo == g % 8 && w.rgs == 8, "xcd row groups of %d: %d + 8 i", g, w.rgo);
                CHECK(w.rgo + 8 * (w.NRGx - 1) < NRG && w.rgo + 8 * w.NRGx >= NRG, "xcd list of %d", g);
            } else {
                CHECK(w.rgo == 0 && w.rgs == 1 && w.NRGx == NRG && w.Gx == Gu, "plain list");
            }
            const int lane = xmode ? w.rgo : 0;  // ranks of one list are consecutive
            if (prev_set[lane]) CHECK(w.x0 == (uint32_t)prev_end[lane], "gap before rank %d", w.rank);
            else CHECK(w.x0 == 0, "first range starts at %u", w.x0);
            prev_set[lane] = true;
            prev_end[lane] = w.x1;
            sizes.push_back((int)(w.x1 - w.x0));
            for (uint32_t u = w.x0; u < w.x1; ++u) {
                const int rg = w.rgo + w.rgs * (int)(u / (uint32_t)Urg);
                const int q = (int)(u % (uint32_t)Urg);
                CHECK(rg < NRG, "row group %d of %d", rg, NRG);
                if (rg < NRG) seen[(size_t)rg * Urg + q]++;
            }
        }
        for (int64_t i = 0; i < U; ++i) CHECK(seen[(size_t)i] == 1, "unit %lld taken %d times", (long long)i, seen[(size_t)i]);
        if (!xmode && !sizes.empty()) {
            int mn = sizes[0], mx = sizes[0];
            for (int v : sizes) mn = v < mn ? v : mn, mx = v > mx ? v : mx;
            CHECK(mx - mn <= 1, "unequal split %d..%d", mn, mx);
        }
    }
}

// Path choice: the tables up to 4 rows (one launch) at any size, the matrix cores from 9 rows on,
// the crossover between them falling as the matrix grows (never back to the tables with more
// weights or more rows), and the measured crossovers of the fitted shapes.
static void check_path_choice(std::mt19937_64& rng) {
    for (int it = 0; it < 20000; ++it) {
        const int64_t wb = (int64_t)rnd(rng, 1, (uint64_t)1 << (it % 2 ? 24 : 34));
        for (int b = 1; b <= 16; ++b) {
            const bool m = prefer_mfma(wb, b);
            if (b <= 4) CHECK(!m, "matrix cores at %d rows, %lld bytes", b, (long long)wb);
            if (b >= 9) CHECK(m, "tables at %d rows, %lld bytes", b, (long long)wb);
            if (m && b < 16) CHECK(prefer_mfma(wb, b + 1), "back to the tables at %d rows", b + 1);
            if (m) CHECK(prefer_mfma(wb * 2, b), "back to the tables at %lld bytes", (long long)wb * 2);
        }
    }
    struct Case {
        int64_t bytes;
        int tables_up_to;  // the largest batch that stays on the tables
    } cases[] = {{91019264, 4}, {91017216, 4}, {26005504, 5}, {11836352, 7}, {11835392, 7}, {4404224, 8},
                 {3250688, 8}};
    for (const Case& c : cases)
        for (int b = 1; b <= 16; ++b)
            CHECK(prefer_mfma(c.bytes, b) == (b > c.tables_up_to), "%lld bytes at %d rows", (long long)c.bytes, b);
}

static void check_default_workgroups(std::mt19937_64& rng) {
    for (int it = 0; it < 20000; ++it) {
        const int64_t cap = 2 * (int64_t)rnd(rng, 1, 1024);
        const int64_t U = (int64_t)rnd(rng, 1, 1u << 20);
        const int batch = (int)rnd(rng, 1, 16);
        const int64_t G = default_workgroups(U, cap, batch);
        CHECK(G >= 1 && G <= cap, "workgroups %lld of %lld", (long long)G, (long long)cap);
    }
}

// Group width 4: chunks cover every column inside one base, tables and staging stay inside the
// LDS bytes the host reserves, every staged column has its own float and a float4 never
// straddles a padding gap.
static void check_rows4(std::mt19937_64& rng) {
    for (int it = 0; it < 20000; ++it) {
        const int nb = (int)rnd(rng, 0, 5), ns = (int)rnd(rng, 0, 5);
        const int64_t K = (int64_t)rnd(rng, 1, it % 3 == 0 ? 200 : 12000);
        const int64_t s = ns ? (int64_t)rnd(rng, 1, 1300) : 0;
        const int cw = nb > 0 ? r4_main_chunk_words(nb, K) : 1;
        CHECK(cw >= 1 && (cw & (cw - 1)) == 0 && (nb == 0 || ((int64_t)cw * 1024 >= (int64_t)nb * K &&
                                                                 (cw == 1 || (int64_t)cw * 512 < (int64_t)nb * K))),
              "chunk words %d for nb %d K %lld", cw, nb, (long long)K);
        const R4Chunk m = r4_chunk(nb, K, false, cw), r = r4_chunk(ns, s, true, cw);
        for (const auto& pr : {std::make_pair(m, K), std::make_pair(r, s)}) {
            const R4Chunk& c = pr.first;
            if (!c.ok || c.cpb == 0) continue;
            CHECK(c.C % 4 == 0 && c.G * 4 == c.C && (1 << c.lcpb) == c.cpb, "chunk shape C %d cpb %d", c.C, c.cpb);
            CHECK((int64_t)c.cpb * c.C >= pr.second, "chunks cover %lld columns", (long long)pr.second);
            CHECK(c.cpb * (32 / c.cpb) == 32, "32 chunks");
        }
        if (r.ok && r.cpb) CHECK(r.C <= 32 && 32 % r.C == 0, "refinement chunk of %d columns", r.C);
        if (!m.ok || !r.ok || cw > 8) continue;
        const uint32_t sh = r4_staging_shift(m.C);
        const int64_t floats = r4_staging_floats(K, m.C);
        const int64_t K4 = cdiv(K, 4) * 4;
        uint32_t last = 0;
        for (int64_t j = 0; j < K4; ++j) {
            const uint32_t p = r4_xpos((uint32_t)j, sh);
            CHECK(j == 0 || p > last, "staging positions increase");
            CHECK((int64_t)p < floats - 4, "column %lld at %u of %lld floats", (long long)j, p, (long long)floats);
            if (j % 4 == 0) CHECK(r4_xpos((uint32_t)j + 3, sh) == p + 3, "float4 straddles a gap at %lld", (long long)j);
            last = p;
        }
        CHECK((int64_t)r4_xpos((uint32_t)K4, sh) + 4 <= floats, "zero pad inside the staging");
        // the largest table word a lookup reads: entry 15, last group, last chunk
        for (const R4Chunk& c : {m, r}) {
            if (!c.cpb) continue;
            const int64_t maxw = (15ll * c.G + c.G - 1) * 32 + 31;
            CHECK(maxw * 4 + 4 <= 512ll * c.C, "table of %d bytes read at word %lld", 512 * c.C, (long long)maxw);
        }
        CHECK(r4_lds_bytes(m, r, K) == 512ll * m.C + 512ll * r.C + 4 * floats, "lds bytes");
    }
}

// The C-ABI checks never misbehave on hostile arguments and give the documented codes.
static void check_validation(std::mt19937_64& rng) {
    const void* ok = reinterpret_cast<const void*>(uintptr_t(0x10000));
    const void* mis = reinterpret_cast<const void*>(uintptr_t(0x10004));
    const int64_t edges[] = {INT64_MIN, -1, 0, 1, 255, 256, 257, 0x3FFFFFFF, 0x40000000, INT32_MAX, INT64_MAX};
    for (int it = 0; it < 50000; ++it) {
        const void* p[5];
        for (auto& q : p) {
            const int r = (int)(rng() % 8);
            q = r == 0 ? nullptr : r == 1 ? mis : ok;
        }
        const int nb = (int)rnd(rng, 0, 80) - 5;
        const int64_t N = (rng() & 3) ? (int64_t)rnd(rng, 0, 1u << 20) : edges[rng() % 11];
        const int64_t K = (rng() & 3) ? (int64_t)rnd(rng, 0, 1u << 20) : edges[rng() % 11];
        const int batch = (int)rnd(rng, 0, 20) - 2;
        const int xdt = (int)rnd(rng, 0, 4) - 1;
        const int st = check_gemv_common(p[0], p[1], p[2], nb, N, K, p[3], xdt, batch, p[4]);
        const bool any_null = !p[0] || !p[1] || !p[2] || !p[3] || !p[4];
        const bool bad_size = nb < 1 || nb > 64 || N < 1 || N > 0x3FFFFFFF || K < 1 || K > 0x3FFFFFFF ||
                              batch < 1 || batch > UBW_MAX_BATCH;
        int want = UBW_OK;
        if (any_null || bad_size) want = UBW_EINVAL;
        else if (xdt != UBW_F16 && xdt != UBW_F32) want = UBW_EUNSUPPORTED;
        else if (p[0] == mis) want = UBW_EALIGN;
        CHECK(st == want, "check_gemv_common gave %d, want %d", st, want);
        if (nb >= 1 && nb <= 64 && N >= 1 && N <= 0x3FFFFFFF && K >= 1 && K <= 0x3FFFFFFF) {
            const int64_t w = packed_words(nb, N, K);
            CHECK(w == (int64_t)nb * cdiv(N, 256) * cdiv(K, 256) * 2048, "packed words");
            const uint64_t wsb = rng() % (1u << 22);
            const int g = (rng() & 1) ? 4 : 8;
            const void* ws = (rng() & 3) == 0 ? nullptr : (rng() & 3) == 0 ? mis : ok;
            const int wst = check_workspace(ws, ws ? wsb : (rng() & 1 ? 0 : wsb), N, g);
            CHECK(wst == UBW_OK || wst == UBW_EINVAL || wst == UBW_EALIGN || wst == UBW_ESIZE, "workspace code %d", wst);
            if (ws == ok) {
                const uint64_t need = 4ull * (uint64_t)(g == 4 ? 16 : 16 + 64 * cdiv(N, 256));
                CHECK((wst == UBW_OK) == (wsb >= need), "workspace size %llu vs %llu", (unsigned long long)wsb,
                      (unsigned long long)need);
            }
        }
    }
}

int main() {
    std::mt19937_64 rng(20260805);
    check_fast_div(rng);
    check_wg_range(rng);
    check_path_choice(rng);
    check_default_workgroups(rng);
    check_rows4(rng);
    check_validation(rng);
    if (fails) {
        std::fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
