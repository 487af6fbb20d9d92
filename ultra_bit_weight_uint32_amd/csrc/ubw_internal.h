// Internal declarations shared by the host API (api.hip) and the kernels (kernels.hip).
//
// Packed tile layout
// ------------------
// A base of an N x K sign matrix is cut into tiles of 256 rows x 256 columns (8 uint32 words
// per row). Tile (rt, ks) of base k starts at word ((rt * KT + ks) * nb + k) * 2048, where
// NT = ceil(N / 256) and KT = ceil(K / 256). Inside a tile the words are stored
// [q in 0..1][rho in 0..255][e in 0..3]: row rho's slot s = 4q + e, so one 16-byte vector per
// row and half-tile, and consecutive rows (= consecutive lanes of a wave) read consecutive
// vectors.
//
// Slot s of row rho holds word s ^ a of the row's 256-column slice, with its bytes permuted:
// byte jj of the slot is byte jj ^ c of the word, where l = rho mod 32 = 4 a + c. Byte jj of
// slot i is then the pattern of column group (4 i + jj) ^ l, so the lane that owns row rho
// visits the 32 groups of the slice in the order t ^ l for t = 0..31: the 32 lanes of each
// half-wave look up 32 different tables at every step (each table sits in a single LDS bank,
// which makes every lookup instruction bank-conflict free), and steps 0..15 cover one
// 128-column half of the slice, steps 16..31 the other.
// Rows >= N and columns >= K are stored as zero bits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ubw.h"
#include "plan.h"

namespace ubw {

constexpr int kTileRows = 256;
constexpr int kSliceWords = 8;
constexpr int kSliceCols = 256;
constexpr int kTileWords = kTileRows * kSliceWords;  // 2048 words = 8 KiB per base per tile
constexpr int kThreads = 256;
constexpr int kMaxGroup = UBW_MAX_GROUP;  // GEMVs per grouped launch
constexpr int kBatchChunk = 4;          // activation rows per launch (larger batches: several)
constexpr int kMaxDevices = 64;         // devices whose launch capacities are cached

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One matrix of a GEMV step: the main bases over all K columns, or the salient refinement
// bases over the s virtual columns that idx maps onto activation columns.
struct Segment {
    const uint32_t* packed;
    const void* alpha_r;    // [nb][N] fp32; with StepArgs::gs, fp16 [nb][N][2 * ceil(Kv / 256)]
    const float* alpha_c;   // [nb][Kv]
    const int32_t* idx;     // [Kv] virtual column -> activation column, or nullptr (identity)
    int nb;
    int Kv;                 // columns of this matrix: K, or s
};

// One launch: up to two segments accumulated into the same y. seg[0] is the main matrix
// (idx == nullptr, may be empty: nb = Kv = 0), seg[1] the refinement (idx != nullptr).
struct StepArgs {
    Segment seg[2];
    int nseg;               // 1 (seg[0] only) or 2
    int N;
    const void* x;          // [batch][ldx]
    int x_dtype;            // UBW_F32 / UBW_F16
    int gs;                 // 1: seg[0] has one fp16 row scale per 128 columns (see Segment)
    int64_t ldx;            // activation row length K
    int batch;
    float* y;               // [batch][N]
    int accumulate;         // 0: y = result, 1: y += result
    uint32_t* ws;           // zero-initialised counters (single-launch y = result), or nullptr
    int rows_per_group;     // row tiles per unit: 1, 2 or 4 (<= max_rows_per_group(batch))
    int workgroups;         // persistent workgroups to launch, 0 = as many as fit at once
    int tables_only;        // 1: the table kernels at every batch (explicit geometry)
};

// Workspace of the GEMV calls: a 16-word header, then 64 words (256 bytes) per row group (at
// most one per 256-row tile) for the single-launch y = result mode: the arrival counter at word
// 0 and the zeroing flag at word 32, on separate cache lines. Header word 0 collects errors the
// kernels find: kWsErrWait (a wait for a row group's zeroing gave up; that workgroup added
// nothing) and kWsErrIndex (a salient index outside [0, K) or not above the one before it).
constexpr uint32_t kWsErrWait = 1u;
constexpr uint32_t kWsErrIndex = 2u;
constexpr int kWsHeaderWords = plan::kWsHeaderWords;
constexpr int kWsRowGroupWords = plan::kWsRowGroupWords;
constexpr int kWsFlagOffset = 32;
inline int64_t step_workspace_words(int64_t N) { return plan::workspace_words(N); }

// The static workspace of ubw_lut_gemv_refined_noalloc: the counters of up to 256 row groups
// (N <= 65536 rows), 65,600 bytes per device; scratch_address() gives this device's copy.
constexpr int kScratchRowGroups = 256;
constexpr int64_t kScratchMaxRows = (int64_t)kScratchRowGroups * kTileRows;
constexpr int kScratchWords = kWsHeaderWords + kWsRowGroupWords * kScratchRowGroups;
hipError_t scratch_address(uint32_t** out);

hipError_t launch_fill_zero(float* y, int64_t n, hipStream_t s);
hipError_t launch_pack(const void* src, int src_fmt, int nb, int N, int K, uint32_t* dst, hipStream_t s);
hipError_t launch_ternary(const int8_t* w, const float* scale, int N, int K, uint32_t* packed,
                          float* alpha_r, float* alpha_c, hipStream_t s);
hipError_t launch_build_lut(const void* x, int x_dtype, int batch, const float* alpha_c, int nb, int K,
                            int g, float* lut, hipStream_t s);
hipError_t launch_extract(const uint32_t* packed, int nb, int N, int K, int g, uint16_t* out, hipStream_t s);
// A step: on the matrix cores when that path is predicted to be faster (plan::prefer_mfma)
// and supported, unless a.tables_only; otherwise through the tables.
hipError_t launch_step(const StepArgs& a, hipStream_t s);
// Several steps sharing x (same x, batch, dtype, rows_per_group) in one launch.
hipError_t launch_step_group(const StepArgs* a, int count, hipStream_t s);
// Steps of several activation rows on the matrix cores (mfma.hip): up to 16 rows per launch,
// at most six bases (main + refinement), per-row alpha_r only. Their cost hardly depends on the
// rows while the tables' grows with every activation row; plan::prefer_mfma compares the two.
bool mfma_step_supported(const StepArgs& a);
hipError_t launch_step_mfma(const StepArgs& a, hipStream_t s);
// Several GEMVs sharing x (same x, batch, dtype, ldx) in one matrix-core launch.
hipError_t launch_step_mfma_group(const StepArgs* a, int count, hipStream_t s);
// Whether every buffer of a step is small enough for the kernel's 32-bit buffer offsets.
bool step_buffers_fit(const StepArgs& a);
// Group width 4 (rows4.hip): 16 whole rows per workgroup with all of a row's tables in LDS, one
// plain store per output. Needs main and refinement with 1, 2 or 4 bases, a refinement of at
// whose ns x tiles is 1, 2 or 4 (32 chunks of 8, 16 or 32 columns), and the
// tables + fp32 activations within 156 KiB of LDS (2 bases: K <= 4096 with a refinement of at
// most 256 columns in 2 bases or 512 in 1); a.ws only takes error bits.
bool rows4_supported(const StepArgs& a);
hipError_t launch_rows4(const StepArgs& a, hipStream_t s);

// Hessian-guided saliency (saliency.hip).
hipError_t launch_gram(const void* x, int T, int K, float scale, float* H, hipStream_t s);
int64_t saliency_workspace_floats(int64_t N, int64_t K);
hipError_t launch_saliency(float* H, int K, float damp, const float* W, int N, int s, float* d, float* score,
                           int32_t* idx, float* ws, hipStream_t st);

// Offline fit (fit.hip): scratch floats for partial sums, and the launch sequence.
int64_t fit_workspace_floats(int64_t N, int64_t K);
hipError_t launch_fit(const void* w, int w_dtype, int N, int K, int nb, int iters, uint32_t* bits, float* alpha_r,
                      float* alpha_c, float* residual, float* ws, hipStream_t s);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s);
// Largest rows_per_group the GEMV instances support for this batch (4 for batch 1, else 1).
int max_rows_per_group(int batch);

}  // namespace ubw
