/*
 * ubw.h — C ABI of libubw.so: matrix-vector products against decoupled row-column binary
 * bases, evaluated by table lookup on AMD MI355X (gfx950).
 *
 * Method: "FluxBin: Flexible LUT-based Ultra-low-bit LLM Inference by Algorithm-Kernel
 * Synergy" (gist.science/ko/paper/2608.15602), technical summary.
 *   - "1. Algorithm innovation": each base is W_hat^(k) = (alpha_r^(k) alpha_c^(k)^T) (.) B^(k)
 *     with B^(k) in {-1,+1}^{N x K}; the weight is the sum of the global bases plus a
 *     salient-refinement branch on selected columns.
 *   - "2. Kernel innovation": LUT-BSF folds alpha_c into the partial-sum tables when they are
 *     built; VCM maps the sparse salient columns onto a dense virtual matrix by gathering
 *     activations and scales; the kernel streams packed uint32 words, extracts pattern
 *     indices with bit operations, fetches partial sums and applies alpha_r in the reduction.
 * So y[b][r] = sum_k alpha_r^(k)[r] * sum_j B^(k)[r][j] * alpha_c^(k)[j] * x[b][j]
 *            + the same over the salient columns with the refinement bases.
 *
 * Conventions shared by every call
 *   - Sign bits: bit 1 means +1, bit 0 means -1.
 *   - Canonical bit format (input of ubw_pack_bases): uint32 words [nb][N][ceil(K/32)], column
 *     j of a row at word j/32, bit j%32 (least significant first). Bits at columns >= K are
 *     ignored.
 *   - Packed format (output of ubw_pack_bases, input of the GEMV calls): an opaque GPU tile
 *     layout of ubw_packed_words() uint32 words. Tiles of 256 rows x 256 columns per base;
 *     padding rows and columns are zero. Only this library reads it.
 *   - Group width g: the number of columns one pattern index covers (tables of 2^g entries).
 *     Every call takes g = 4 or 8 (ubw_lut_gemv_multi and ubw_lut_gemv_gs: 8 only). At g = 8
 *     the GEMV splits K over workgroups; at g = 4 a workgroup owns whole rows (the 16-entry
 *     tables of a full row fit in its LDS), for the shapes listed at ubw_lut_gemv.
 *   - Scalars: alpha_r [nb][N] and alpha_c [nb][K] fp32, row-major; y [batch][N] fp32.
 *   - Activations x [batch][K], fp16 (UBW_F16) or fp32 (UBW_F32), row-major.
 *   - Pointers are device pointers unless a comment says otherwise. The caller allocates
 *     and owns every buffer; the library allocates nothing. Its process-wide state is a
 *     per-device cache of how many workgroups of each kernel a device holds at once (filled
 *     on first use, thread-safe) and the static device array that
 *     ubw_lut_gemv_refined_noalloc uses as its workspace (one per device, loaded with the
 *     library).
 *   - stream is a hipStream_t (NULL = the default stream). Every call only enqueues work on
 *     it and returns; results are ready when the stream is synchronized.
 *   - Return value: UBW_OK (0) or a negative ubw_status. Arguments are validated on the host
 *     before anything is enqueued, so a failing call leaves every buffer untouched. Faults
 *     inside kernels surface at the next stream synchronization.
 *   - Outputs must not alias inputs.
 */
#ifndef UBW_H
#define UBW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    UBW_OK = 0,
    UBW_EINVAL = -1,        /* null pointer, non-positive size, batch out of range */
    UBW_EUNSUPPORTED = -2,  /* g or dtype or source format not supported */
    UBW_EALIGN = -3,        /* packed / x / workspace pointer not 16-byte aligned */
    UBW_ERANGE = -4,        /* a size or index out of its allowed range */
    UBW_EHIP = -5,          /* the HIP runtime rejected a launch */
    UBW_ESIZE = -6,         /* a caller buffer is smaller than required */
    UBW_EWAIT = -7          /* (ubw_workspace_check) a workgroup gave up waiting and wrote nothing */
} ubw_status;

enum { UBW_F32 = 0, UBW_F16 = 1 };                       /* activation dtypes */
enum { UBW_SRC_CANON_BITS = 0, UBW_SRC_INT8_SIGNS = 1 };  /* ubw_pack_bases sources */

/* Largest batch one GEMV call accepts. At group width 8 a batch runs in one launch on the
 * matrix cores when that is predicted to be faster than the tables (a cost model of both paths in
 * the weight bytes and the rows: from 5 to 9 rows on, depending on the matrix size) and the call
 * has per-row scales and at most six bases (main + refinement): the
 * sign bits are expanded to fp16 +-1 and v = alpha_c * x is split into fp16 high and low parts
 * (round toward zero each), so that per element |v - hi - lo| < 2^-20 |v| + 2^-38 m, m the
 * largest |v| of that activation row within the 256-column slice, against the tables' fp32 v
 * (2^-24 |v|); accumulation is fp32 in both. Otherwise batches above 4 rows run through the
 * tables as consecutive launches of 4 rows on the call's stream. */
#define UBW_MAX_BATCH 16
/* columns per row scale in ubw_lut_gemv_gs */
#define UBW_GROUP_COLS 128
/* most GEMVs one ubw_lut_gemv_multi call takes */
#define UBW_MAX_GROUP 8

/* Human-readable name of a status code (static string, never NULL). */
const char* ubw_status_str(int status);

/* Library ABI version (increments when a signature or the packed layout changes). */
int ubw_version(void);

/*
 * Size in uint32 words of the packed layout of nb bases of an N x K matrix (padding
 * included). Host-only, enqueues nothing. *out_words is a host pointer.
 */
int ubw_packed_words(int nb, int64_t N, int64_t K, int g, int64_t* out_words);

/*
 * Pack sign bases into the GPU tile layout (load time; not on the per-token path).
 * Section "2. Kernel innovation", execution flow: the kernel streams compressed uint32
 * weights. The layout puts each 256-row x 256-column tile of a base in one contiguous
 * block whose 16-byte vectors are read by consecutive lanes, so the GEMV's weight stream
 * is a sequence of fully coalesced 1 KiB wave reads.
 *   src      UBW_SRC_CANON_BITS: uint32 [nb][N][ceil(K/32)] canonical words;
 *            UBW_SRC_INT8_SIGNS: int8 [nb][N][K], value > 0 means +1, otherwise -1.
 *   dst      uint32 [ubw_packed_words(nb, N, K, g)], fully overwritten.
 * Errors: UBW_EINVAL (null, nb < 1, N < 1, K < 1), UBW_EUNSUPPORTED (src_fmt, g),
 *         UBW_EALIGN (dst not 16-byte aligned), UBW_EHIP.
 */
int ubw_pack_bases(const void* src, int src_fmt, int nb, int64_t N, int64_t K, int g,
                   uint32_t* dst, void* stream);

/*
 * Encode ternary weights w in {-1, 0, +1} as two binary bases at half scale:
 * w = (B1 + B2) / 2, with B1 = B2 = sign(w) where w != 0 and (B1, B2) = (+1, -1) where
 * w == 0; both bases get alpha_r = scale / 2 and alpha_c = 1. (FlashLM v6 page: 81% of the
 * model's parameters are ternary; the two-base encoding lets the binary-basis GEMV run them.)
 *   w        int8 [N][K] (values outside {-1,0,1} are read by sign)
 *   scale    fp32 [N] per-row scale of the ternary layer
 *   packed   uint32 [ubw_packed_words(2, N, K, g)] output
 *   alpha_r  fp32 [2][N] output;  alpha_c  fp32 [2][K] output
 * Errors: UBW_EINVAL, UBW_EUNSUPPORTED (g), UBW_EALIGN (packed), UBW_ERANGE (more than
 *         INT_MAX * 256 packed words), UBW_EHIP.
 */
int ubw_ternary_encode(const int8_t* w, const float* scale, int64_t N, int64_t K, int g,
                       uint32_t* packed, float* alpha_r, float* alpha_c, void* stream);

/*
 * LUT-BSF tables written to memory (the GEMV builds the same tables in LDS with the same
 * device code; this call exists so the tables can be checked).
 * Section "2. Kernel innovation", LUT-BSF: v = alpha_c^(k) (.) x_b rounded to fp32; for the
 * group of columns gi*g .. gi*g+g-1 (v = 0 past column K),
 * lut[b][k][gi][p] = sum_{i<g} (2*bit_i(p) - 1) * v[gi*g + i],  p in [0, 2^g).
 *   x        [batch][K] fp16 or fp32;  alpha_c fp32 [nb][K]
 *   lut      fp32 [batch][nb][ceil(K/g)][2^g] output
 * Errors: UBW_EINVAL (null, sizes, batch < 1), UBW_EUNSUPPORTED (g, dtype), UBW_EHIP.
 */
int ubw_build_lut(const void* x, int x_dtype, int batch, const float* alpha_c, int nb,
                  int64_t K, int g, float* lut, void* stream);

/*
 * Workspace bytes the GEMV calls use for this shape (64 + 256 * ceil(N / 256)). *out is a
 * host pointer. ubw_workspace_bytes is the same call under its earlier name.
 * A workspace lets a call that overwrites y (accumulate = 0) run as ONE launch: the kernel's
 * persistent workgroups combine partial sums with fp32 atomics; per row group of 256 (or 512)
 * rows, the first workgroup to announce its arrival in the workspace zeroes those rows (or
 * writes its own sums there) and then raises the row group's flag, and every other workgroup
 * adds into the rows only after it has seen the flag. The first arriver never waits for another
 * workgroup before raising the flag, so every call completes whatever else runs on the device.
 * Without a workspace (NULL, 0 bytes) the library zero-fills y with a separate launch first.
 * Rules: zero-fill the workspace once after allocating it (the kernels leave it consistent
 * after every call, whatever the shape); a workspace serves calls on one stream at a time
 * (calls that may run concurrently need separate workspaces).
 * Word 0 of the workspace collects errors found on the device (read it with
 * ubw_workspace_check): bit 0 (UBW_EWAIT) a wait gave up and that workgroup added nothing
 * (a safety net; the protocol above makes it unreachable), bit 1 (UBW_ERANGE) a salient index
 * outside [0, K) or not above the index before it. Calls with a workspace set these bits and
 * never clear them. At g = 4 (whole rows per workgroup, no cross-workgroup sums) only the
 * 16-word header is used: *out = 64.
 * Errors: UBW_EINVAL (null, sizes, batch), UBW_EUNSUPPORTED (g not 4 or 8).
 */
int ubw_lut_gemv_workspace_bytes(int nb, int64_t N, int64_t K, int g, int batch, size_t* out);
int ubw_workspace_bytes(int nb, int64_t N, int64_t K, int g, int batch, size_t* out);

/*
 * Reads (and with clear != 0 then zeroes) word 0 of a GEMV workspace, or with workspace == NULL
 * of the static workspace of ubw_lut_gemv_refined_noalloc on the current device: waits for
 * `stream` to finish, so it is not for use inside graph capture. *out_word (host) gets the word.
 * Returns UBW_OK (no error recorded), UBW_EWAIT (bit 0 set: some outputs were not written),
 * UBW_ERANGE (bit 1 set, bit 0 clear: a salient index was out of range or out of order; see
 * ubw_vcm_gather_refine), or UBW_EINVAL / UBW_EALIGN / UBW_EHIP for the call.
 */
int ubw_workspace_check(void* workspace, int clear, void* stream, uint32_t* out_word);

/*
 * Main GEMV: y (= or +=) sum_k alpha_r^(k) (.) (B^(k) (alpha_c^(k) (.) x)), for every
 * activation row, with tables of g columns (LUT-BSF; section "2. Kernel innovation").
 *   g = 8: tables of 256 entries per 8 columns, built per 256-column slice in LDS; pattern
 *          indices are read from the packed words with byte-permute operations and alpha_r is
 *          applied to each row's partial sum; slices of one row are combined with fp32 atomics,
 *          so the summation order (not the result beyond rounding) varies between runs.
 *   g = 4: tables of 16 entries per 4 columns for the whole row in LDS (16 bytes per column and
 *          base); a workgroup owns 16 complete rows and writes each output once with a plain
 *          store (fixed summation order, no workspace needed). The tables and the fp32 copy of
 *          x must fit 156 KiB: main nb in {1, 2, 4} with nb * K <= 8192 (nb = 1: K up to ~6000),
 *          refinement ns in {1, 2, 4} with ns * ceil(s / 256) in {1, 2, 4}; other shapes are
 *          UBW_EUNSUPPORTED (never switched to g = 8).
 *   Both widths read the same packed layout.
 *   packed       from ubw_pack_bases(nb, N, K, g)
 *   accumulate   0: y = result; 1: y += result
 *   workspace    ubw_workspace_bytes() bytes, or NULL with ws_bytes == 0 (see there)
 * Errors: UBW_EINVAL (null, nb < 1, N < 1, K < 1, batch not in [1, UBW_MAX_BATCH], workspace
 *         NULL with ws_bytes != 0), UBW_EUNSUPPORTED (g not 4 or 8, a g = 4 shape that does
 *         not fit, dtype, or an operand of 2 GiB or more: the kernels address each operand
 *         with 32-bit offsets), UBW_EALIGN (packed or workspace), UBW_ESIZE (ws_bytes too
 *         small), UBW_EHIP.
 */
int ubw_lut_gemv(const uint32_t* packed, const float* alpha_r, const float* alpha_c, int nb,
                 int64_t N, int64_t K, int g, const void* x, int x_dtype, int batch,
                 float* y, int accumulate, void* workspace, size_t ws_bytes, void* stream);

/*
 * Salient refinement by virtual columnar mapping, accumulated into y.
 * Section "2. Kernel innovation", VCM: the s salient columns idx[0..s) are mapped onto a
 * dense virtual N x s matrix; its activations x[b][idx[q]] and scales alpha_c_s[k][q] are
 * gathered while the tables are built, and the same LUT-GEMV runs over it:
 * y[b][r] += sum_{k<ns} alpha_r_s[k][r] * sum_{q<s} B_s^(k)[r][q] * alpha_c_s[k][q] * x[b][idx[q]].
 *   idx          int32 [s], strictly ascending, each in [0, K)
 *   packed_s     from ubw_pack_bases(ns, N, s, g) of the refinement bases [ns][N][s]
 *   alpha_r_s    fp32 [ns][N];  alpha_c_s fp32 [ns][s]
 *   K            columns of x (the activation row length)
 * The kernels check idx on the device: a position q whose idx[q] lies outside [0, K), or is not
 * above idx[q - 1], sets bit 1 of the workspace's word 0 (UBW_ERANGE from ubw_workspace_check).
 * A position outside [0, K) reads nothing and contributes nothing; one out of order still adds
 * its term of the sum above (which is defined for any order). Without a workspace nothing
 * records the fault; ubw_check_indices checks a host copy of idx.
 * Errors: as ubw_lut_gemv; s < 1 is UBW_EINVAL.
 */
int ubw_vcm_gather_refine(const int32_t* idx, int64_t s, const uint32_t* packed_s,
                          const float* alpha_r_s, const float* alpha_c_s, int ns, int64_t N,
                          int64_t K, int g, const void* x, int x_dtype, int batch, float* y,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * The whole step in ONE launch: main bases plus salient refinement (ubw_lut_gemv followed by
 * ubw_vcm_gather_refine on the same x and y, with the same results up to fp32 summation
 * order). Section "2. Kernel innovation", VCM: the mapping exists so that the refinement runs
 * in the same unified kernel as the global bases; here the refinement's workgroups are part
 * of the main grid. Arguments as the two calls; accumulate and workspace as ubw_lut_gemv.
 */
int ubw_lut_gemv_refined(const uint32_t* packed, const float* alpha_r, const float* alpha_c, int nb,
                         const int32_t* idx, int64_t s, const uint32_t* packed_s,
                         const float* alpha_r_s, const float* alpha_c_s, int ns, int64_t N,
                         int64_t K, int g, const void* x, int x_dtype, int batch, float* y,
                         int accumulate, void* workspace, size_t ws_bytes, void* stream);

/*
 * ubw_lut_gemv_refined for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid it. The workspace
 * is a static array inside the library, one per device (65,600 bytes, held until the process
 * ends), so y = result stays one launch and the call allocates nothing. Arguments and results as
 * ubw_lut_gemv_refined, without workspace and ws_bytes.
 *   N            at most 65536 rows at g = 8 (UBW_ERANGE above); g = 4 uses only the array's
 *                error word and takes any N
 * The first call on a device looks up the array's device address (hipGetSymbolAddress, with that
 * device current), so make it before any graph capture. All calls on one device share the one
 * array: calls that may overlap on a GPU (other streams, other threads) race and must not be
 * issued. Its error word is read (and cleared) with ubw_workspace_check(NULL, ...).
 * Errors: as ubw_lut_gemv_refined, plus UBW_ERANGE (N), UBW_EHIP (the address lookup failed).
 */
int ubw_lut_gemv_refined_noalloc(const uint32_t* packed, const float* alpha_r, const float* alpha_c,
                                 int nb, const int32_t* idx, int64_t s, const uint32_t* packed_s,
                                 const float* alpha_r_s, const float* alpha_c_s, int ns, int64_t N,
                                 int64_t K, int g, const void* x, int x_dtype, int batch, float* y,
                                 int accumulate, void* stream);

/*
 * Group-scale variant: the row scale of the main bases varies along the row, one value per
 * 128-column block. The technical summary's "Experimental results" (accuracy) names a
 * "2b-s16-g128" setting without defining its fields; read here as 2 bases, 16-bit scales,
 * groups of 128 columns:
 * y[b][r] (+)= sum_{k<nb} sum_j alpha_rg[k][r][j / 128] * B^(k)[r][j] * alpha_c^(k)[j] * x[b][j]
 *              + the refinement of ubw_lut_gemv_refined when idx != NULL (its row scales stay
 *              one fp32 per row; with idx == NULL the refinement arguments are ignored).
 *   alpha_rg     fp16 [nb][ceil(K / 256)][N][2]: element [k][t][r][h] is the scale of base k,
 *                row r, columns 256 t + 128 h ... 256 t + 128 h + 127 (block 2 t + h), so that
 *                the rows of one 256-column slice are contiguous. A block wholly past column K
 *                (h = 1 of the last slice when K mod 256 is in 1..128) is padding and never used
 *                (any value, NaN included). 4-byte aligned.
 *   gsize        must be UBW_GROUP_COLS
 * Everything else as ubw_lut_gemv_refined (main bases, alpha_c, x, y, accumulate, workspace).
 * Errors: as ubw_lut_gemv_refined; gsize other than 128 is UBW_EUNSUPPORTED, an alpha_rg not
 *         4-byte aligned UBW_EALIGN.
 */
int ubw_lut_gemv_gs(const uint32_t* packed, const uint16_t* alpha_rg, const float* alpha_c, int nb,
                    int gsize, const int32_t* idx, int64_t s, const uint32_t* packed_s,
                    const float* alpha_r_s, const float* alpha_c_s, int ns, int64_t N, int64_t K,
                    int g, const void* x, int x_dtype, int batch, float* y, int accumulate,
                    void* workspace, size_t ws_bytes, void* stream);

/*
 * One GEMV of a grouped call: its own bases, scales, optional refinement, output and workspace.
 * All pointers are device pointers except as noted; the struct array itself is host memory.
 */
typedef struct ubw_gemv_desc {
    const uint32_t* packed;     /* main bases from ubw_pack_bases(nb, N, K, g=8) */
    const float* alpha_r;       /* [nb][N] */
    const float* alpha_c;       /* [nb][K] */
    int nb;
    const int32_t* idx;         /* [s] salient columns, or NULL: no refinement (the next five ignored) */
    int64_t s;
    const uint32_t* packed_s;   /* from ubw_pack_bases(ns, N, s, g=8) */
    const float* alpha_r_s;     /* [ns][N] */
    const float* alpha_c_s;     /* [ns][s] */
    int ns;
    int64_t N;
    float* y;                   /* [batch][N] */
    void* workspace;            /* ubw_workspace_bytes(nb, N, K, 8, batch) bytes, or NULL (see there) */
    size_t ws_bytes;
} ubw_gemv_desc;

/*
 * Several steps that read the same activations (e.g. the q, k, v projections, or gate and up)
 * in ONE launch: for each desc, what ubw_lut_gemv_refined (idx != NULL) or ubw_lut_gemv
 * (idx == NULL) computes. The device's workgroups are shared out in proportion to each GEMV's
 * work (on the matrix cores, when every GEMV of the call goes there, one grid covers all their
 * row tiles, each GEMV with its own column split); each GEMV's outputs and workspace are its
 * own. The GEMVs of a call must not write
 * overlapping outputs. Section "2. Kernel innovation" (unified kernel execution) carried over
 * to GEMVs that share x.
 *   descs        HOST array of count descriptors, 1 <= count <= UBW_MAX_GROUP
 *   K, g, x, x_dtype, batch, accumulate   shared by all, as ubw_lut_gemv (g = 8 only)
 * Errors: UBW_EINVAL (count out of range, null descs, or any desc invalid as in the single
 *         calls), UBW_EUNSUPPORTED (g != 8), otherwise as ubw_lut_gemv.
 */
int ubw_lut_gemv_multi(const ubw_gemv_desc* descs, int count, int64_t K, int g, const void* x,
                       int x_dtype, int batch, int accumulate, void* stream);

/*
 * Offline fit of the decomposition from a dense matrix (load time; its output feeds
 * ubw_pack_bases with UBW_SRC_CANON_BITS). Section "1. Algorithm innovation" gives the form
 * W ~ sum_k (alpha_r^(k) alpha_c^(k)^T) (.) B^(k), B in {-1,+1}, but not how it is fitted; the
 * fit here is residual binarization with alternating least squares:
 *   R = W; for k < nb: B^(k) = sign(R) (+1 where R >= 0); A = |R|;
 *   alpha_r = row means of A, alpha_c = 1; then `iters` rounds of
 *   alpha_c = A^T alpha_r / ||alpha_r||^2 and alpha_r = A alpha_c / ||alpha_c||^2 (each the
 *   least-squares optimum for one vector given the other; 0 where the norm is 0);
 *   R = R - (alpha_r alpha_c^T) (.) B^(k).
 * The error ||R|| never increases from one base, or one round, to the next.
 *   w          [N][K] fp32 (UBW_F32) or fp16 (UBW_F16), row-major
 *   nb         bases, 1..64; iters: ALS rounds per base, 0..10000 (0 = per-row binarization)
 *   bits       OUT canonical signs [nb][N][ceil(K/32)] uint32 (column j: word j/32, bit j%32;
 *              bits past column K are 0)
 *   alpha_r    OUT fp32 [nb][N];  alpha_c OUT fp32 [nb][K]
 *   residual   OUT fp32 [N][K]: W minus the fitted bases. It may be the same buffer as w when w
 *              is fp32 (the fit then overwrites W).
 *   workspace  ubw_fit_workspace_bytes(N, K) bytes of scratch (partial sums), caller-owned
 * All sums are fp32 in a fixed order (no atomics): the result is deterministic.
 * Errors: UBW_EINVAL (null, sizes, nb, iters), UBW_EUNSUPPORTED (w_dtype), UBW_EALIGN (a pointer
 *         not 4-byte aligned), UBW_ERANGE (N above 4,194,240), UBW_ESIZE (workspace), UBW_EHIP.
 */
int ubw_fit_workspace_bytes(int64_t N, int64_t K, size_t* out);
int ubw_fit_bases(const void* w, int w_dtype, int64_t N, int64_t K, int nb, int iters, uint32_t* bits,
                  float* alpha_r, float* alpha_c, float* residual, void* workspace, size_t ws_bytes,
                  void* stream);

/*
 * Gram matrix of calibration activations on the matrix cores: H = scale * X^T X, the proxy
 * Hessian 2 X^T X of a linear layer's squared output error when scale = 2 (input to
 * ubw_hessian_saliency).
 *   x   fp16 [T][K] (UBW_F16 only), row-major;  H  OUT fp32 [K][K], both triangles written
 * Errors: UBW_EINVAL (null, T or K < 1), UBW_EUNSUPPORTED (x_dtype), UBW_ERANGE (K above
 *         8,388,480), UBW_EALIGN (x not 2-, H not 4-byte aligned), UBW_EHIP.
 */
int ubw_gram(const void* x, int x_dtype, int64_t T, int64_t K, float scale, float* H, void* stream);

/*
 * Hessian-guided salient-column search. Section "1. Algorithm innovation", saliency search:
 * weight sensitivities come from the inverse Hessian (Optimal Brain Quantization) and the
 * highest-scoring columns form the salient mask. The page gives no formula; read as
 *   H_d = H + lambda I, lambda = damp * mean(diag H) (1 when that mean is not positive)
 *   d_j = [H_d^-1]_jj,  score_j = sum_r W[r][j]^2 / d_j^2
 *   idx = the s columns with the highest scores (equal scores: lower index first), ascending
 * computed by a blocked fp32 Cholesky of H_d and a blocked triangular solve for diag(H_d^-1).
 *   H          IN symmetric [K][K] fp32 (e.g. from ubw_gram); OUT its lower triangle holds the
 *              Cholesky factor of H_d (the upper triangle is left partly updated)
 *   W          fp32 [N][K], the layer's dense weights
 *   d, score   OUT fp32 [K];  idx OUT int32 [s], 1 <= s <= K
 *   workspace  ubw_saliency_workspace_bytes(N, K) bytes (about 2 K^2 + N K / 16 + 64 K bytes:
 *              the factor's block inverses and the triangular solve's blocks), caller-owned.
 *              On return its float 0 holds lambda and float 1 an error code: 0 none, 1 a
 *              pivot was not positive (H_d not positive definite in fp32), 2 the selection
 *              did not find exactly s columns (NaN scores).
 * Errors: UBW_EINVAL (null, sizes, s, damp negative or not finite), UBW_ERANGE (N above
 *         4,194,240), UBW_EALIGN (a pointer not 4-byte aligned), UBW_ESIZE, UBW_EHIP.
 */
int ubw_saliency_workspace_bytes(int64_t N, int64_t K, size_t* out);
int ubw_hessian_saliency(float* H, int64_t K, float damp, const float* W, int64_t N, int64_t s,
                         float* d, float* score, int32_t* idx, void* workspace, size_t ws_bytes,
                         void* stream);

/*
 * Host-side check of a salient index list: every idx[q] in [0, K) and strictly ascending (the
 * rule the kernels check on the device). idx is a HOST pointer. Returns UBW_OK or UBW_ERANGE
 * (UBW_EINVAL for null / s < 1).
 */
int ubw_check_indices(const int32_t* idx_host, int64_t s, int64_t K);

/*
 * Test export: pattern indices as the GEMV's bit extraction sees them, written in canonical
 * order out[k][r][gi] (uint16), gi < ceil(K/g); columns >= K read as 0.
 * Errors: UBW_EINVAL, UBW_EUNSUPPORTED (g not 4 or 8), UBW_EALIGN (packed), UBW_EHIP.
 */
int ubw_extract_patterns(const uint32_t* packed, int nb, int64_t N, int64_t K, int g,
                         uint16_t* out, void* stream);

/*
 * Test and tuning export: ubw_lut_gemv (mode = 0), ubw_vcm_gather_refine (mode = 1) or the
 * main bases of ubw_lut_gemv_gs (mode = 2: alpha_r is then its fp16 alpha_rg) with an
 * explicit launch geometry, always through the tables (at every batch). The kernel walks a list
 * of units (a unit: rows_per_group tiles of 256 rows x two (256-column slice, base) items) split
 * into equal contiguous ranges over `workgroups` persistent workgroups (0 = the default: as many
 * as the device holds at once, or one per CU at batch 1 when the units fit in two per CU; larger
 * values are capped to the number of units only, so a launch may hold more workgroups than the
 * device runs at once). With a workspace and equal ranges, the launch may add one workgroup per
 * row group that takes part in the zeroing only. rows_per_group is 1, 2 or 4 for batch 1 and 1 or 2 above
 * (UBW_ERANGE otherwise). Results equal the default geometry's up to fp32 summation
 * order. For modes 0 and 2, idx is ignored and Kv = K; for mode 1, Kv = s. workspace as
 * ubw_lut_gemv. A mode outside 0..2 is UBW_ERANGE.
 */
int ubw_lut_gemv_geometry(const uint32_t* packed, const void* alpha_r, const float* alpha_c,
                          int nb, int64_t N, int64_t Kv, const int32_t* idx, int64_t K,
                          const void* x, int x_dtype, int batch, float* y, int accumulate,
                          int mode, int rows_per_group, int workgroups, void* workspace,
                          size_t ws_bytes, void* stream);

/*
 * Measurement helper (no part of the product computation): reads `bytes` bytes of `buf` with
 * the GEMV's access shape (16-byte loads, consecutive lanes on consecutive vectors, one
 * workgroup per 8 KiB, every load issued before any is consumed) and writes one word per
 * workgroup to out[ceil(bytes / 8192)] that depends on the data. Benchmarks time it at the
 * size of a GEMV's weight stream to show the ceiling of a single read of that size.
 * Errors: UBW_EINVAL (null, bytes < 16 or not a multiple of 16), UBW_EALIGN, UBW_EHIP.
 */
int ubw_bench_stream_read(const void* buf, int64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* UBW_H */
