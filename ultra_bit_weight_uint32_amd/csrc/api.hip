// C ABI of libubw.so: argument validation, launch-geometry choice and dispatch.
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <climits>

#include "../../include/ubw.h"
#include "ubw_internal.h"

using namespace ubw;

namespace {

constexpr int kVersion = 8;
constexpr int kMaxFitIters = 10000;

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
using plan::aligned16;
using plan::fits_int;
inline int hip_status(hipError_t e) { return e == hipSuccess ? UBW_OK : UBW_EHIP; }

int64_t packed_words_of(int nb, int64_t N, int64_t K) { return plan::packed_words(nb, N, K); }

// Rows per unit: 2 row tiles when the list still holds at least 768 units (enough to keep every
// workgroup busy; the tables, built once per unit and activation row, then serve 512 rows),
// else 1. Measured on the configs' shapes: 2 tiles win on the 70B gate/up/down (26.6 vs 28.9 us
// at batch 1, 62 vs 81 us at batch 4) and on the grouped q/k/v (1000 units: 14.3 vs 16.2 us),
// tie on 8192 x 8192 alone (800 units) and lose on 4096 x 4096 (128 units: 6.9 vs 5.9 us);
// 4 tiles (one workgroup per CU: 166+ VGPRs) never won, and stay reachable through the
// geometry export.
int choose_rows(int64_t NT, int64_t units_per_tile_row_group, int batch) {
    if (2 <= max_rows_per_group(batch) && ceil_div(NT, 2) * units_per_tile_row_group >= 768) return 2;
    return 1;
}

int64_t units_of(int64_t Kv, int nb) { return ceil_div(ceil_div(Kv, kSliceCols) * nb, 2); }

int validate_gemv_common(const void* packed, const void* ar, const float* ac, int nb, int64_t N, int64_t Kv,
                         const void* x, int x_dtype, int batch, const float* y) {
    return plan::check_gemv_common(packed, ar, ac, nb, N, Kv, x, x_dtype, batch, y);
}

// Workspace check at group width g (plan.h): NULL with 0 bytes means "none" (the y = result mode
// then zero-fills y with a separate launch at g = 8).
int check_workspace_g(void* ws, size_t ws_bytes, int64_t N, int g, uint32_t** out) {
    *out = nullptr;
    const int st = plan::check_workspace(ws, ws_bytes, N, g);
    if (st == UBW_OK) *out = static_cast<uint32_t*>(ws);
    return st;
}
int check_workspace(void* ws, size_t ws_bytes, int64_t N, uint32_t** out) { return check_workspace_g(ws, ws_bytes, N, 8, out); }

Segment make_segment(const uint32_t* packed, const void* ar, const float* ac, const int32_t* idx, int nb,
                     int64_t Kv) {
    Segment g{};
    g.packed = packed;
    g.alpha_r = ar;
    g.alpha_c = ac;
    g.idx = idx;
    g.nb = nb;
    g.Kv = (int)Kv;
    return g;
}

StepArgs make_step(int64_t N, const void* x, int x_dtype, int64_t K, int batch, float* y, int accumulate,
                   uint32_t* ws) {
    StepArgs a{};
    a.N = (int)N;
    a.x = x;
    a.x_dtype = x_dtype;
    a.ldx = K;
    a.batch = batch;
    a.y = y;
    a.accumulate = accumulate ? 1 : 0;
    a.ws = ws;
    a.rows_per_group = 1;
    a.workgroups = 0;
    return a;
}

// Launches a step. The main segment goes in seg[0] (no idx) and a refinement segment in
// seg[1] (with idx); a refinement-only step leaves seg[0] empty.
int run_step(StepArgs& a, void* stream) {
    if (!step_buffers_fit(a)) return UBW_EUNSUPPORTED;
    return hip_status(launch_step(a, as_stream(stream)));
}

// A step at group width g (4 or 8, checked by the caller). Shapes whose group-4 tables do not
// fit one workgroup's LDS are refused at g = 4 (UBW_EUNSUPPORTED): the caller chooses g, so
// nothing silently switches width.
int run_step_g(StepArgs& a, int g, void* stream) {
    if (g != 4) return run_step(a, stream);
    if (!rows4_supported(a)) return UBW_EUNSUPPORTED;
    return hip_status(launch_rows4(a, as_stream(stream)));
}

}  // namespace

extern "C" {

const char* ubw_status_str(int status) {
    switch (status) {
        case UBW_OK: return "UBW_OK";
        case UBW_EINVAL: return "UBW_EINVAL: invalid argument (null pointer or size out of range)";
        case UBW_EUNSUPPORTED: return "UBW_EUNSUPPORTED: unsupported group width, dtype or format";
        case UBW_EALIGN: return "UBW_EALIGN: pointer not 16-byte aligned";
        case UBW_ERANGE: return "UBW_ERANGE: index out of range or not ascending";
        case UBW_EHIP: return "UBW_EHIP: HIP runtime error";
        case UBW_ESIZE: return "UBW_ESIZE: buffer too small";
        case UBW_EWAIT: return "UBW_EWAIT: a workgroup gave up waiting for a row group's zeroing (outputs not written)";
        default: return "unknown ubw status";
    }
}

int ubw_version(void) { return kVersion; }

int ubw_packed_words(int nb, int64_t N, int64_t K, int g, int64_t* out_words) {
    if (!out_words || nb < 1 || nb > 64 || !fits_int(N) || !fits_int(K)) return UBW_EINVAL;
    if (g != 8 && g != 4) return UBW_EUNSUPPORTED;
    *out_words = packed_words_of(nb, N, K);
    return UBW_OK;
}

int ubw_pack_bases(const void* src, int src_fmt, int nb, int64_t N, int64_t K, int g, uint32_t* dst,
                   void* stream) {
    if (!src || !dst || nb < 1 || nb > 64 || !fits_int(N) || !fits_int(K)) return UBW_EINVAL;
    if (g != 8 && g != 4) return UBW_EUNSUPPORTED;
    if (src_fmt != UBW_SRC_CANON_BITS && src_fmt != UBW_SRC_INT8_SIGNS) return UBW_EUNSUPPORTED;
    if (!aligned16(dst)) return UBW_EALIGN;
    if (packed_words_of(nb, N, K) > (int64_t)INT_MAX * 256) return UBW_ERANGE;
    return hip_status(launch_pack(src, src_fmt, nb, (int)N, (int)K, dst, as_stream(stream)));
}

int ubw_ternary_encode(const int8_t* w, const float* scale, int64_t N, int64_t K, int g, uint32_t* packed,
                       float* alpha_r, float* alpha_c, void* stream) {
    if (!w || !scale || !packed || !alpha_r || !alpha_c || !fits_int(N) || !fits_int(K)) return UBW_EINVAL;
    if (g != 8 && g != 4) return UBW_EUNSUPPORTED;
    if (!aligned16(packed)) return UBW_EALIGN;
    if (packed_words_of(2, N, K) > (int64_t)INT_MAX * 256) return UBW_ERANGE;
    return hip_status(launch_ternary(w, scale, (int)N, (int)K, packed, alpha_r, alpha_c, as_stream(stream)));
}

int ubw_build_lut(const void* x, int x_dtype, int batch, const float* alpha_c, int nb, int64_t K, int g,
                  float* lut, void* stream) {
    if (!x || !alpha_c || !lut || nb < 1 || nb > 64 || !fits_int(K)) return UBW_EINVAL;
    if (batch < 1 || batch > UBW_MAX_BATCH) return UBW_EINVAL;
    if (g != 8 && g != 4) return UBW_EUNSUPPORTED;
    if (x_dtype != UBW_F16 && x_dtype != UBW_F32) return UBW_EUNSUPPORTED;
    return hip_status(launch_build_lut(x, x_dtype, batch, alpha_c, nb, (int)K, g, lut, as_stream(stream)));
}

int ubw_lut_gemv_workspace_bytes(int nb, int64_t N, int64_t K, int g, int batch, size_t* out) {
    if (!out || nb < 1 || !fits_int(N) || !fits_int(K) || batch < 1 || batch > UBW_MAX_BATCH) return UBW_EINVAL;
    if (g != 8 && g != 4) return UBW_EUNSUPPORTED;
    *out = g == 4 ? (size_t)kWsHeaderWords * 4 : (size_t)step_workspace_words(N) * 4;
    return UBW_OK;
}

int ubw_workspace_bytes(int nb, int64_t N, int64_t K, int g, int batch, size_t* out) {
    return ubw_lut_gemv_workspace_bytes(nb, N, K, g, batch, out);
}

int ubw_workspace_check(void* workspace, int clear, void* stream, uint32_t* out_word) {
    if (!out_word) return UBW_EINVAL;
    if (!workspace) {  // the static workspace of ubw_lut_gemv_refined_noalloc on the current device
        uint32_t* p = nullptr;
        if (scratch_address(&p) != hipSuccess) return UBW_EHIP;
        workspace = p;
    }
    if (!aligned16(workspace)) return UBW_EALIGN;
    hipStream_t st = as_stream(stream);
    uint32_t word = 0;
    if (hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return UBW_EHIP;
    *out_word = word;
    if (clear && word != 0) {
        const uint32_t zero = 0;
        if (hipMemcpyAsync(workspace, &zero, sizeof(zero), hipMemcpyHostToDevice, st) != hipSuccess ||
            hipStreamSynchronize(st) != hipSuccess)
            return UBW_EHIP;
    }
    if (word & kWsErrWait) return UBW_EWAIT;
    if (word & kWsErrIndex) return UBW_ERANGE;
    return UBW_OK;
}

int ubw_lut_gemv(const uint32_t* packed, const float* alpha_r, const float* alpha_c, int nb, int64_t N,
                 int64_t K, int g, const void* x, int x_dtype, int batch, float* y, int accumulate,
                 void* workspace, size_t ws_bytes, void* stream) {
    int st = validate_gemv_common(packed, alpha_r, alpha_c, nb, N, K, x, x_dtype, batch, y);
    if (st != UBW_OK) return st;
    if (g != 8 && g != 4) return UBW_EUNSUPPORTED;
    uint32_t* ws = nullptr;
    if ((st = check_workspace_g(workspace, ws_bytes, N, g, &ws)) != UBW_OK) return st;
    StepArgs a = make_step(N, x, x_dtype, K, batch, y, accumulate, ws);
    a.nseg = 1;
    a.seg[0] = make_segment(packed, alpha_r, alpha_c, nullptr, nb, K);
    a.rows_per_group = choose_rows(ceil_div(N, kTileRows), units_of(K, nb), batch);
    return run_step_g(a, g, stream);
}

int ubw_vcm_gather_refine(const int32_t* idx, int64_t s, const uint32_t* packed_s, const float* alpha_r_s,
                          const float* alpha_c_s, int ns, int64_t N, int64_t K, int g, const void* x,
                          int x_dtype, int batch, float* y, void* workspace, size_t ws_bytes, void* stream) {
    if (!idx) return UBW_EINVAL;
    int st = validate_gemv_common(packed_s, alpha_r_s, alpha_c_s, ns, N, s, x, x_dtype, batch, y);
    if (st != UBW_OK) return st;
    if (!fits_int(K)) return UBW_EINVAL;
    if (g != 8 && g != 4) return UBW_EUNSUPPORTED;
    uint32_t* ws = nullptr;
    if ((st = check_workspace_g(workspace, ws_bytes, N, g, &ws)) != UBW_OK) return st;
    StepArgs a = make_step(N, x, x_dtype, K, batch, y, 1, ws);
    a.nseg = 2;
    a.seg[1] = make_segment(packed_s, alpha_r_s, alpha_c_s, idx, ns, s);
    a.rows_per_group = choose_rows(ceil_div(N, kTileRows), units_of(s, ns), batch);
    return run_step_g(a, g, stream);
}

int ubw_lut_gemv_refined(const uint32_t* packed, const float* alpha_r, const float* alpha_c, int nb,
                         const int32_t* idx, int64_t s, const uint32_t* packed_s, const float* alpha_r_s,
                         const float* alpha_c_s, int ns, int64_t N, int64_t K, int g, const void* x, int x_dtype,
                         int batch, float* y, int accumulate, void* workspace, size_t ws_bytes, void* stream) {
    int st = validate_gemv_common(packed, alpha_r, alpha_c, nb, N, K, x, x_dtype, batch, y);
    if (st != UBW_OK) return st;
    if (!idx) return UBW_EINVAL;
    if ((st = validate_gemv_common(packed_s, alpha_r_s, alpha_c_s, ns, N, s, x, x_dtype, batch, y)) != UBW_OK)
        return st;
    if (g != 8 && g != 4) return UBW_EUNSUPPORTED;
    uint32_t* ws = nullptr;
    if ((st = check_workspace_g(workspace, ws_bytes, N, g, &ws)) != UBW_OK) return st;
    StepArgs a = make_step(N, x, x_dtype, K, batch, y, accumulate, ws);
    a.nseg = 2;
    a.seg[0] = make_segment(packed, alpha_r, alpha_c, nullptr, nb, K);
    a.seg[1] = make_segment(packed_s, alpha_r_s, alpha_c_s, idx, ns, s);
    a.rows_per_group = choose_rows(ceil_div(N, kTileRows), units_of(K, nb) + units_of(s, ns), batch);
    return run_step_g(a, g, stream);
}

int ubw_lut_gemv_refined_noalloc(const uint32_t* packed, const float* alpha_r, const float* alpha_c, int nb,
                                 const int32_t* idx, int64_t s, const uint32_t* packed_s, const float* alpha_r_s,
                                 const float* alpha_c_s, int ns, int64_t N, int64_t K, int g, const void* x,
                                 int x_dtype, int batch, float* y, int accumulate, void* stream) {
    // every check that needs no device first, so that rejected calls touch nothing
    int st = validate_gemv_common(packed, alpha_r, alpha_c, nb, N, K, x, x_dtype, batch, y);
    if (st != UBW_OK) return st;
    if (!idx) return UBW_EINVAL;
    if ((st = validate_gemv_common(packed_s, alpha_r_s, alpha_c_s, ns, N, s, x, x_dtype, batch, y)) != UBW_OK)
        return st;
    if (g != 8 && g != 4) return UBW_EUNSUPPORTED;
    if (g == 8 && N > kScratchMaxRows) return UBW_ERANGE;  // g = 4 uses the header only
    if (g == 4) {
        StepArgs a = make_step(N, x, x_dtype, K, batch, y, accumulate, nullptr);
        a.nseg = 2;
        a.seg[0] = make_segment(packed, alpha_r, alpha_c, nullptr, nb, K);
        a.seg[1] = make_segment(packed_s, alpha_r_s, alpha_c_s, idx, ns, s);
        if (!rows4_supported(a)) return UBW_EUNSUPPORTED;
    }
    uint32_t* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return UBW_EHIP;
    return ubw_lut_gemv_refined(packed, alpha_r, alpha_c, nb, idx, s, packed_s, alpha_r_s, alpha_c_s, ns, N, K, g, x,
                                x_dtype, batch, y, accumulate, ws, (size_t)kScratchWords * 4, stream);
}

int ubw_lut_gemv_gs(const uint32_t* packed, const uint16_t* alpha_rg, const float* alpha_c, int nb, int gsize,
                    const int32_t* idx, int64_t s, const uint32_t* packed_s, const float* alpha_r_s,
                    const float* alpha_c_s, int ns, int64_t N, int64_t K, int g, const void* x, int x_dtype,
                    int batch, float* y, int accumulate, void* workspace, size_t ws_bytes, void* stream) {
    int st = validate_gemv_common(packed, alpha_rg, alpha_c, nb, N, K, x, x_dtype, batch, y);
    if (st != UBW_OK) return st;
    if (idx && (st = validate_gemv_common(packed_s, alpha_r_s, alpha_c_s, ns, N, s, x, x_dtype, batch, y)) != UBW_OK)
        return st;
    if (g != 8 || gsize != UBW_GROUP_COLS) return UBW_EUNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(alpha_rg) & 3u) != 0) return UBW_EALIGN;
    uint32_t* ws = nullptr;
    if ((st = check_workspace(workspace, ws_bytes, N, &ws)) != UBW_OK) return st;
    StepArgs a = make_step(N, x, x_dtype, K, batch, y, accumulate, ws);
    a.gs = 1;
    a.nseg = 1;
    a.seg[0] = make_segment(packed, alpha_rg, alpha_c, nullptr, nb, K);
    int64_t units = units_of(K, nb);
    if (idx) {
        a.nseg = 2;
        a.seg[1] = make_segment(packed_s, alpha_r_s, alpha_c_s, idx, ns, s);
        units += units_of(s, ns);
    }
    a.rows_per_group = choose_rows(ceil_div(N, kTileRows), units, batch);
    return run_step(a, stream);
}

int ubw_lut_gemv_multi(const ubw_gemv_desc* descs, int count, int64_t K, int g, const void* x, int x_dtype,
                       int batch, int accumulate, void* stream) {
    if (!descs || count < 1 || count > UBW_MAX_GROUP || !fits_int(K)) return UBW_EINVAL;
    if (g != 8) return UBW_EUNSUPPORTED;
    StepArgs args[UBW_MAX_GROUP];
    int64_t units = 0, NTmax = 0;
    for (int i = 0; i < count; ++i) {
        const ubw_gemv_desc& d = descs[i];
        int st = validate_gemv_common(d.packed, d.alpha_r, d.alpha_c, d.nb, d.N, K, x, x_dtype, batch, d.y);
        if (st != UBW_OK) return st;
        if (d.idx && (st = validate_gemv_common(d.packed_s, d.alpha_r_s, d.alpha_c_s, d.ns, d.N, d.s, x, x_dtype,
                                                batch, d.y)) != UBW_OK)
            return st;
        uint32_t* ws = nullptr;
        if ((st = check_workspace(d.workspace, d.ws_bytes, d.N, &ws)) != UBW_OK) return st;
        for (int j = 0; j < i; ++j)  // one output and one workspace per GEMV
            if (descs[j].y == d.y || (ws && descs[j].workspace == d.workspace)) return UBW_EINVAL;
        StepArgs a = make_step(d.N, x, x_dtype, K, batch, d.y, accumulate, ws);
        a.seg[0] = make_segment(d.packed, d.alpha_r, d.alpha_c, nullptr, d.nb, K);
        a.nseg = 1;
        int64_t u = units_of(K, d.nb);
        if (d.idx) {
            a.nseg = 2;
            a.seg[1] = make_segment(d.packed_s, d.alpha_r_s, d.alpha_c_s, d.idx, d.ns, d.s);
            u += units_of(d.s, d.ns);
        }
        if (!step_buffers_fit(a)) return UBW_EUNSUPPORTED;
        args[i] = a;
        units += ceil_div(d.N, kTileRows) * u;
        NTmax = ceil_div(d.N, kTileRows) > NTmax ? ceil_div(d.N, kTileRows) : NTmax;
    }
    // one row-tile count for all: as for a single GEMV, over the group's total units per tile row
    const int rpl = choose_rows(NTmax, (units + NTmax - 1) / NTmax, batch);
    for (int i = 0; i < count; ++i) args[i].rows_per_group = rpl;
    return hip_status(launch_step_group(args, count, as_stream(stream)));
}

int ubw_fit_workspace_bytes(int64_t N, int64_t K, size_t* out) {
    if (!out || !fits_int(N) || !fits_int(K)) return UBW_EINVAL;
    *out = (size_t)fit_workspace_floats(N, K) * 4;
    return UBW_OK;
}

int ubw_fit_bases(const void* w, int w_dtype, int64_t N, int64_t K, int nb, int iters, uint32_t* bits,
                  float* alpha_r, float* alpha_c, float* residual, void* workspace, size_t ws_bytes, void* stream) {
    if (!w || !bits || !alpha_r || !alpha_c || !residual || !workspace) return UBW_EINVAL;
    if (!fits_int(N) || !fits_int(K) || nb < 1 || nb > 64 || iters < 0 || iters > kMaxFitIters) return UBW_EINVAL;
    if (w_dtype != UBW_F16 && w_dtype != UBW_F32) return UBW_EUNSUPPORTED;
    if (ceil_div(N, 64) > 65535) return UBW_ERANGE;  // column-sum grid height
    if ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(bits) | reinterpret_cast<uintptr_t>(alpha_r) |
         reinterpret_cast<uintptr_t>(alpha_c) | reinterpret_cast<uintptr_t>(residual) |
         reinterpret_cast<uintptr_t>(workspace)) & 3u)
        return UBW_EALIGN;
    if (ws_bytes < (size_t)fit_workspace_floats(N, K) * 4) return UBW_ESIZE;
    return hip_status(launch_fit(w, w_dtype, (int)N, (int)K, nb, iters, bits, alpha_r, alpha_c, residual,
                                 (float*)workspace, as_stream(stream)));
}

int ubw_gram(const void* x, int x_dtype, int64_t T, int64_t K, float scale, float* H, void* stream) {
    if (!x || !H || !fits_int(T) || !fits_int(K)) return UBW_EINVAL;
    if (x_dtype != UBW_F16) return UBW_EUNSUPPORTED;
    if (ceil_div(K, 128) > 65535) return UBW_ERANGE;
    if ((reinterpret_cast<uintptr_t>(x) & 1u) || (reinterpret_cast<uintptr_t>(H) & 3u)) return UBW_EALIGN;
    return hip_status(launch_gram(x, (int)T, (int)K, scale, H, as_stream(stream)));
}

int ubw_saliency_workspace_bytes(int64_t N, int64_t K, size_t* out) {
    if (!out || !fits_int(N) || !fits_int(K)) return UBW_EINVAL;
    *out = (size_t)saliency_workspace_floats(N, K) * 4;
    return UBW_OK;
}

int ubw_hessian_saliency(float* H, int64_t K, float damp, const float* W, int64_t N, int64_t s, float* d,
                         float* score, int32_t* idx, void* workspace, size_t ws_bytes, void* stream) {
    if (!H || !W || !d || !score || !idx || !workspace) return UBW_EINVAL;
    if (!fits_int(K) || !fits_int(N) || s < 1 || s > K) return UBW_EINVAL;
    if (!(damp >= 0.f) || !(damp < 1e30f)) return UBW_EINVAL;
    if (ceil_div(N, 64) > 65535) return UBW_ERANGE;
    if ((reinterpret_cast<uintptr_t>(H) | reinterpret_cast<uintptr_t>(W) | reinterpret_cast<uintptr_t>(d) |
         reinterpret_cast<uintptr_t>(score) | reinterpret_cast<uintptr_t>(idx) |
         reinterpret_cast<uintptr_t>(workspace)) & 3u)
        return UBW_EALIGN;
    if (ws_bytes < (size_t)saliency_workspace_floats(N, K) * 4) return UBW_ESIZE;
    return hip_status(launch_saliency(H, (int)K, damp, W, (int)N, (int)s, d, score, idx, (float*)workspace,
                                      as_stream(stream)));
}

int ubw_check_indices(const int32_t* idx_host, int64_t s, int64_t K) {
    if (!idx_host || s < 1 || K < 1) return UBW_EINVAL;
    for (int64_t q = 0; q < s; ++q) {
        if (idx_host[q] < 0 || idx_host[q] >= K) return UBW_ERANGE;
        if (q > 0 && idx_host[q] <= idx_host[q - 1]) return UBW_ERANGE;
    }
    return UBW_OK;
}

int ubw_extract_patterns(const uint32_t* packed, int nb, int64_t N, int64_t K, int g, uint16_t* out,
                         void* stream) {
    if (!packed || !out || nb < 1 || nb > 64 || !fits_int(N) || !fits_int(K)) return UBW_EINVAL;
    if (g != 8 && g != 4) return UBW_EUNSUPPORTED;
    if (!aligned16(packed)) return UBW_EALIGN;
    return hip_status(launch_extract(packed, nb, (int)N, (int)K, g, out, as_stream(stream)));
}

int ubw_lut_gemv_geometry(const uint32_t* packed, const void* alpha_r, const float* alpha_c, int nb, int64_t N,
                          int64_t Kv, const int32_t* idx, int64_t K, const void* x, int x_dtype, int batch,
                          float* y, int accumulate, int mode, int rows_per_group, int workgroups,
                          void* workspace, size_t ws_bytes, void* stream) {
    int st = validate_gemv_common(packed, alpha_r, alpha_c, nb, N, Kv, x, x_dtype, batch, y);
    if (st != UBW_OK) return st;
    if (mode < 0 || mode > 2) return UBW_ERANGE;
    const bool vcm = mode == 1;
    if (mode == 2 && (reinterpret_cast<uintptr_t>(alpha_r) & 3u) != 0) return UBW_EALIGN;
    if (rows_per_group != 1 && rows_per_group != 2 && rows_per_group != 4) return UBW_ERANGE;
    if (rows_per_group > max_rows_per_group(batch)) return UBW_ERANGE;
    if (workgroups < 0) return UBW_ERANGE;
    if (vcm && (!idx || !fits_int(K))) return UBW_EINVAL;
    uint32_t* ws = nullptr;
    if ((st = check_workspace(workspace, ws_bytes, N, &ws)) != UBW_OK) return st;
    StepArgs a = make_step(N, x, x_dtype, vcm ? K : Kv, batch, y, accumulate, ws);
    a.gs = mode == 2 ? 1 : 0;
    if (vcm) {
        a.nseg = 2;
        a.seg[1] = make_segment(packed, alpha_r, alpha_c, idx, nb, Kv);
    } else {
        a.nseg = 1;
        a.seg[0] = make_segment(packed, alpha_r, alpha_c, nullptr, nb, Kv);
    }
    a.rows_per_group = rows_per_group;
    a.workgroups = workgroups;
    a.tables_only = 1;
    return run_step(a, stream);
}

int ubw_bench_stream_read(const void* buf, int64_t bytes, uint32_t* out, void* stream) {
    if (!buf || !out || bytes < 16 || (bytes & 15) != 0) return UBW_EINVAL;
    if (!aligned16(buf)) return UBW_EALIGN;
    return hip_status(launch_stream_read(buf, bytes, out, as_stream(stream)));
}

}  // extern "C"
