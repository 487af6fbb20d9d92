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
// Slot s of row rho holds word (s + a) mod 8 of the row's 256-column slice, where
// a = (rho mod 32) / 4. That rotation, together with a byte rotation by c = rho mod 4, makes
// the lane that owns row rho visit the 32 column groups of the slice in the order
// (t + rho mod 32) mod 32 for t = 0..31, so that the 32 lanes of each half-wave look up 32
// different tables at every step; the tables are laid out so that each one sits in a single
// LDS bank, which makes every lookup instruction bank-conflict free.
// Rows >= N and columns >= K are stored as zero bits.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ubw {

constexpr int kTileRows = 256;
constexpr int kSliceWords = 8;
constexpr int kSliceCols = 256;
constexpr int kTileWords = kTileRows * kSliceWords;  // 2048 words = 8 KiB per base per tile
constexpr int kThreads = 256;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct GemvArgs {
    const uint32_t* packed;
    const float* alpha_r;   // [nb][N]
    const float* alpha_c;   // [nb][Kv]
    int nb;
    int N;
    int Kv;                 // columns of the (virtual) matrix: K, or s for the refinement
    const void* x;          // [batch][ldx]
    int x_dtype;            // UBW_F32 / UBW_F16
    int64_t ldx;            // activation row length K
    const int32_t* idx;     // salient columns (refinement only), else nullptr
    int batch;
    float* y;               // [batch][N]
    int accumulate;         // 0: y = result, 1: y += result
    int rows_per_group;     // 1, 2, 4 row tiles per workgroup
    int slices_per_group;   // >= 1 column slices per workgroup
};

hipError_t launch_fill_zero(float* y, int64_t n, hipStream_t s);
hipError_t launch_pack(const void* src, int src_fmt, int nb, int N, int K, uint32_t* dst, hipStream_t s);
hipError_t launch_ternary(const int8_t* w, const float* scale, int N, int K, uint32_t* packed,
                          float* alpha_r, float* alpha_c, hipStream_t s);
hipError_t launch_build_lut(const void* x, int x_dtype, int batch, const float* alpha_c, int nb, int K,
                            int g, float* lut, hipStream_t s);
hipError_t launch_extract(const uint32_t* packed, int nb, int N, int K, int g, uint16_t* out, hipStream_t s);
hipError_t launch_gemv8(const GemvArgs& a, hipStream_t s);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* out, hipStream_t s);
// Largest rows_per_group the GEMV instances support for this batch (1, 2 or 4).
int max_rows_per_group(int batch);

}  // namespace ubw
