"""CPU oracle: a plain, slow fp64 evaluation of the binary-basis matrix-vector product.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never imports, links or calls it, and
the two share no code: the only thing both sides consume is the seeded input generator in
``workloads/``, which holds none of the method's arithmetic.

What it computes follows "FluxBin: Flexible LUT-based Ultra-low-bit LLM Inference by
Algorithm-Kernel Synergy" (gist.science/ko/paper/2608.15602), technical summary, section
"1. Algorithm innovation" (the decomposition W_hat^(k) = (alpha_r^(k) alpha_c^(k)^T) (.) B^(k)
and the hybrid global + salient-refinement bases) and section "2. Kernel innovation" (LUT-BSF
tables and the execution flow). The arithmetic lives in ``oracle.c``; this module only
marshals numpy arrays through ctypes.

Canonical bit format (used by every function): uint32 words [bases][rows][ceil(K/32)], column
j of a row at word j//32, bit j%32; bit 1 means +1 and bit 0 means -1.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIBPATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIBPATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.oracle_gemv.argtypes = [P, P, P, I, I64, I64, P, I64, P, P, P, I, P, I, P]
    lib.oracle_gemv.restype = None
    lib.oracle_gemv_gs.argtypes = [P, P, I64, I, P, I, I64, I64, P, I64, P, P, P, I, P, I, P]
    lib.oracle_gemv_gs.restype = None
    lib.oracle_fit.argtypes = [P, I64, I64, I, I, P, P, P, P]
    lib.oracle_fit.restype = None
    lib.oracle_lut_gemv.argtypes = [P, P, P, I, I64, I64, P, I64, P, P, P, I, P, I, I, P]
    lib.oracle_lut_gemv.restype = None
    lib.oracle_patterns.argtypes = [P, I, I64, I64, I, P]
    lib.oracle_patterns.restype = None
    lib.oracle_lut_tables.argtypes = [P, I, P, I, I64, I, P]
    lib.oracle_lut_tables.restype = None
    lib.oracle_ternary_gemv.argtypes = [P, P, I64, I64, P, I, P]
    lib.oracle_ternary_gemv.restype = None
    lib.oracle_ternary_encode.argtypes = [P, I64, I64, I, P]
    lib.oracle_ternary_encode.restype = None
    lib.oracle_set_threads.argtypes = [I]
    lib.oracle_set_threads.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = I
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _x64(x):
    """Activations as a contiguous [batch, K] float64 array (fp16/fp32 convert exactly)."""
    x = np.asarray(x)
    if x.ndim == 1:
        x = x[None, :]
    return np.ascontiguousarray(x.astype(np.float64))


def words_per_row(k: int) -> int:
    return (int(k) + 31) // 32


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _refine_args(idx, bits_s, alpha_r_s, alpha_c_s, n_rows):
    if idx is None or len(idx) == 0:
        return None, 0, None, None, None, 0
    idx = _c(idx, np.int32)
    bits_s = _c(bits_s, np.uint32)
    alpha_r_s = _c(alpha_r_s, np.float32)
    alpha_c_s = _c(alpha_c_s, np.float32)
    ns = alpha_r_s.shape[0]
    s = idx.shape[0]
    assert bits_s.shape == (ns, n_rows, words_per_row(s)), bits_s.shape
    assert alpha_c_s.shape == (ns, s)
    return idx, s, bits_s, alpha_r_s, alpha_c_s, ns


def gemv(bits, alpha_r, alpha_c, x, idx=None, bits_s=None, alpha_r_s=None, alpha_c_s=None):
    """y[b, r] = sum_j W_hat[r, j] x[b, j] by dequantizing W_hat row by row in fp64.

    bits [nb, N, ceil(K/32)] uint32, alpha_r [nb, N], alpha_c [nb, K], x [batch, K] or [K].
    Optional salient refinement: idx [s] int32 columns, bits_s [ns, N, ceil(s/32)],
    alpha_r_s [ns, N], alpha_c_s [ns, s]. Returns float64 [batch, N].
    """
    bits = _c(bits, np.uint32)
    alpha_r = _c(alpha_r, np.float32)
    alpha_c = _c(alpha_c, np.float32)
    nb, n, _ = bits.shape
    k = alpha_c.shape[1]
    assert bits.shape[2] == words_per_row(k) and alpha_r.shape == (nb, n) and alpha_c.shape == (nb, k)
    x = _x64(x)
    assert x.shape[1] == k
    batch = x.shape[0]
    idx, s, bits_s, alpha_r_s, alpha_c_s, ns = _refine_args(idx, bits_s, alpha_r_s, alpha_c_s, n)
    if s:
        assert idx.min() >= 0 and idx.max() < k
    y = np.empty((batch, n), dtype=np.float64)
    _load().oracle_gemv(_ptr(bits), _ptr(alpha_r), _ptr(alpha_c), nb, n, k,
                        _ptr(idx), s, _ptr(bits_s), _ptr(alpha_r_s), _ptr(alpha_c_s), ns,
                        _ptr(x), batch, _ptr(y))
    return y


def gemv_gs(bits, alpha_rg, alpha_c, x, gsize=128, idx=None, bits_s=None, alpha_r_s=None, alpha_c_s=None):
    """Group-scale variant of gemv: alpha_rg [nb, N, G] (G >= ceil(K / gsize)) holds one row
    scale per block of gsize columns; fp16 scales are passed as their exact fp32 values.
    Returns float64 [batch, N]."""
    bits = _c(bits, np.uint32)
    alpha_rg = _c(np.asarray(alpha_rg).astype(np.float32), np.float32)
    alpha_c = _c(alpha_c, np.float32)
    nb, n, _ = bits.shape
    k = alpha_c.shape[1]
    gcols = alpha_rg.shape[2]
    assert bits.shape[2] == words_per_row(k) and alpha_c.shape == (nb, k)
    assert alpha_rg.shape[:2] == (nb, n) and gcols >= -(-k // gsize)
    x = _x64(x)
    assert x.shape[1] == k
    batch = x.shape[0]
    idx, s, bits_s, alpha_r_s, alpha_c_s, ns = _refine_args(idx, bits_s, alpha_r_s, alpha_c_s, n)
    if s:
        assert idx.min() >= 0 and idx.max() < k
    y = np.empty((batch, n), dtype=np.float64)
    _load().oracle_gemv_gs(_ptr(bits), _ptr(alpha_rg), gcols, int(gsize), _ptr(alpha_c), nb, n, k,
                           _ptr(idx), s, _ptr(bits_s), _ptr(alpha_r_s), _ptr(alpha_c_s), ns,
                           _ptr(x), batch, _ptr(y))
    return y


def lut_gemv(bits, alpha_r, alpha_c, x, g=8, idx=None, bits_s=None, alpha_r_s=None, alpha_c_s=None):
    """The same product by the table route (fp64): LUT-BSF tables, pattern lookups, alpha_r."""
    bits = _c(bits, np.uint32)
    alpha_r = _c(alpha_r, np.float32)
    alpha_c = _c(alpha_c, np.float32)
    nb, n, _ = bits.shape
    k = alpha_c.shape[1]
    assert bits.shape[2] == words_per_row(k)
    assert 1 <= g <= 12
    x = _x64(x)
    batch = x.shape[0]
    idx, s, bits_s, alpha_r_s, alpha_c_s, ns = _refine_args(idx, bits_s, alpha_r_s, alpha_c_s, n)
    y = np.empty((batch, n), dtype=np.float64)
    _load().oracle_lut_gemv(_ptr(bits), _ptr(alpha_r), _ptr(alpha_c), nb, n, k,
                            _ptr(idx), s, _ptr(bits_s), _ptr(alpha_r_s), _ptr(alpha_c_s), ns,
                            _ptr(x), batch, int(g), _ptr(y))
    return y


def patterns(bits, k, g=8):
    """Pattern indices [nb, N, ceil(K/g)] (uint16) from canonical bits; columns >= K read 0."""
    bits = _c(bits, np.uint32)
    nb, n, _ = bits.shape
    assert bits.shape[2] == words_per_row(k)
    ng = (k + g - 1) // g
    out = np.empty((nb, n, ng), dtype=np.uint16)
    _load().oracle_patterns(_ptr(bits), nb, n, int(k), int(g), _ptr(out))
    return out


def lut_tables(x, alpha_c, g=8):
    """fp64 LUT-BSF tables [batch, nb, ceil(K/g), 2**g] with alpha_c folded in."""
    alpha_c = _c(alpha_c, np.float32)
    nb, k = alpha_c.shape
    x = _x64(x)
    batch = x.shape[0]
    ng = (k + g - 1) // g
    out = np.empty((batch, nb, ng, 1 << g), dtype=np.float64)
    _load().oracle_lut_tables(_ptr(x), batch, _ptr(alpha_c), nb, k, int(g), _ptr(out))
    return out


def ternary_gemv(w, scale, x):
    """Ternary layer by definition: y[b, r] = scale[r] * sum_j w[r, j] x[b, j]."""
    w = _c(w, np.int8)
    scale = _c(scale, np.float32)
    n, k = w.shape
    x = _x64(x)
    batch = x.shape[0]
    y = np.empty((batch, n), dtype=np.float64)
    _load().oracle_ternary_gemv(_ptr(w), _ptr(scale), n, k, _ptr(x), batch, _ptr(y))
    return y


def ternary_encode(w, zero_first_plus=True):
    """Two canonical bases [2, N, ceil(K/32)] with w = (B1 + B2) / 2."""
    w = _c(w, np.int8)
    n, k = w.shape
    out = np.empty((2, n, words_per_row(k)), dtype=np.uint32)
    _load().oracle_ternary_encode(_ptr(w), n, k, 1 if zero_first_plus else 0, _ptr(out))
    return out


def fit(w, nb, iters):
    """Offline fit of nb bases to a dense w [N, K] (fp32 values): residual sign binarization
    with `iters` alternating least-squares rounds for (alpha_r, alpha_c) per base. Returns
    (bits [nb, N, ceil(K/32)] uint32, alpha_r [nb, N], alpha_c [nb, K], residual [N, K]), the
    scales and residual in float64."""
    w = _c(np.asarray(w).astype(np.float32), np.float32)
    n, k = w.shape
    bits = np.empty((nb, n, words_per_row(k)), dtype=np.uint32)
    ar = np.empty((nb, n), dtype=np.float64)
    ac = np.empty((nb, k), dtype=np.float64)
    res = np.empty((n, k), dtype=np.float64)
    _load().oracle_fit(_ptr(w), n, k, int(nb), int(iters), _ptr(bits), _ptr(ar), _ptr(ac), _ptr(res))
    return bits, ar, ac, res


def hessian(x):
    """H = 2 X^T X for calibration activations x [T, K] (the OBQ proxy Hessian of a linear
    layer's squared output error), fp64."""
    x = np.asarray(x).astype(np.float64)
    return 2.0 * (x.T @ x)


def saliency(h, w, s, damp=0.01):
    """Hessian-guided salient-column search ("1. Algorithm innovation", saliency search: OBQ
    sensitivities through the inverse Hessian; the columns with the highest scores form the
    mask). Reading: H_d = H + lambda I with lambda = damp * mean(diag H) (1 when that is 0);
    d_j = [H_d^-1]_jj; the OBQ error of removing weight w_rj is w_rj^2 / d_j, and its
    second-order sensitivity score is w_rj^2 / d_j^2, summed over the rows of a column:
    score_j = sum_r w_rj^2 / d_j^2. The s columns with the largest scores (ties: lower index
    first) are returned ascending. Returns (d, score, idx)."""
    h = np.array(h, dtype=np.float64)
    k = h.shape[0]
    lam = damp * float(np.mean(np.diag(h)))
    if lam == 0.0:
        lam = 1.0
    h[np.diag_indices(k)] += lam
    d = np.diag(np.linalg.inv(h)).copy()
    score = (np.asarray(w, dtype=np.float64) ** 2).sum(axis=0) / (d * d)
    order = np.lexsort((np.arange(k), -score))
    idx = np.sort(order[:s]).astype(np.int32)
    return d, score, idx
