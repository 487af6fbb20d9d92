"""Table-lookup GEMV over decoupled row-column binary bases for AMD MI355X (gfx950).

Thin ctypes binding over ``libubw.so`` (C ABI declared in ``include/ubw.h``). Every step of the
computation runs in the library's HIP kernels; this module only checks tensor devices, dtypes
and shapes, allocates outputs with PyTorch, and passes device pointers and the current HIP
stream. There is no CPU fallback: if the library is missing or the tensors are not on a GPU,
calls raise.

Method: FluxBin (gist.science/ko/paper/2608.15602), technical summary — "1. Algorithm
innovation" (W_hat^(k) = (alpha_r^(k) alpha_c^(k)^T) (.) B^(k), global + salient-refinement
bases) and "2. Kernel innovation" (LUT-BSF tables, virtual columnar mapping, uint32 weight
stream with bit-extracted pattern indices and alpha_r applied in the reduction).
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBPATH = os.path.join(_HERE, "libubw.so")

UBW_OK = 0
UBW_EINVAL, UBW_EUNSUPPORTED, UBW_EALIGN = -1, -2, -3
UBW_ERANGE = -4
UBW_EHIP, UBW_ESIZE, UBW_EWAIT = -5, -6, -7
UBW_F32, UBW_F16 = 0, 1
UBW_SRC_CANON_BITS, UBW_SRC_INT8_SIGNS = 0, 1
MAX_BATCH = 16
MAX_GROUP = 8

# every symbol include/ubw.h declares
EXPORTS = (
    "ubw_status_str", "ubw_version", "ubw_packed_words", "ubw_pack_bases", "ubw_ternary_encode",
    "ubw_build_lut", "ubw_lut_gemv_workspace_bytes", "ubw_workspace_bytes", "ubw_workspace_check",
    "ubw_lut_gemv", "ubw_vcm_gather_refine", "ubw_lut_gemv_refined", "ubw_lut_gemv_refined_noalloc",
    "ubw_check_indices", "ubw_extract_patterns", "ubw_lut_gemv_geometry", "ubw_bench_stream_read",
    "ubw_lut_gemv_multi", "ubw_lut_gemv_gs", "ubw_fit_workspace_bytes", "ubw_fit_bases",
    "ubw_gram", "ubw_saliency_workspace_bytes", "ubw_hessian_saliency",
)


class GemvDesc(ctypes.Structure):
    """Mirror of ubw_gemv_desc (include/ubw.h)."""
    _fields_ = [
        ("packed", ctypes.c_void_p), ("alpha_r", ctypes.c_void_p), ("alpha_c", ctypes.c_void_p), ("nb", ctypes.c_int),
        ("idx", ctypes.c_void_p), ("s", ctypes.c_int64), ("packed_s", ctypes.c_void_p),
        ("alpha_r_s", ctypes.c_void_p), ("alpha_c_s", ctypes.c_void_p), ("ns", ctypes.c_int), ("N", ctypes.c_int64),
        ("y", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
    ]


class UbwError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")
        self.status = status


_lib = None


def lib():
    """The loaded libubw.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBPATH):
        raise ImportError(f"{LIBPATH} is missing: build it with `python -m ultra_bit_weight_uint32_amd.build`")
    L = ctypes.CDLL(LIBPATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "ubw_status_str": ([I], ctypes.c_char_p),
        "ubw_version": ([], I),
        "ubw_packed_words": ([I, I64, I64, I, ctypes.POINTER(I64)], I),
        "ubw_pack_bases": ([P, I, I, I64, I64, I, P, P], I),
        "ubw_ternary_encode": ([P, P, I64, I64, I, P, P, P, P], I),
        "ubw_build_lut": ([P, I, I, P, I, I64, I, P, P], I),
        "ubw_lut_gemv_workspace_bytes": ([I, I64, I64, I, I, ctypes.POINTER(SZ)], I),
        "ubw_workspace_bytes": ([I, I64, I64, I, I, ctypes.POINTER(SZ)], I),
        "ubw_workspace_check": ([P, I, P, ctypes.POINTER(ctypes.c_uint32)], I),
        "ubw_lut_gemv": ([P, P, P, I, I64, I64, I, P, I, I, P, I, P, SZ, P], I),
        "ubw_vcm_gather_refine": ([P, I64, P, P, P, I, I64, I64, I, P, I, I, P, P, SZ, P], I),
        "ubw_check_indices": ([P, I64, I64], I),
        "ubw_extract_patterns": ([P, I, I64, I64, I, P, P], I),
        "ubw_lut_gemv_refined": ([P, P, P, I, P, I64, P, P, P, I, I64, I64, I, P, I, I, P, I, P, SZ, P], I),
        "ubw_lut_gemv_refined_noalloc": ([P, P, P, I, P, I64, P, P, P, I, I64, I64, I, P, I, I, P, I, P], I),
        "ubw_lut_gemv_geometry": ([P, P, P, I, I64, I64, P, I64, P, I, I, P, I, I, I, I, P, SZ, P], I),
        "ubw_bench_stream_read": ([P, I64, P, P], I),
        "ubw_lut_gemv_multi": ([ctypes.POINTER(GemvDesc), I, I64, I, P, I, I, I, P], I),
        "ubw_lut_gemv_gs": ([P, P, P, I, I, P, I64, P, P, P, I, I64, I64, I, P, I, I, P, I, P, SZ, P], I),
        "ubw_fit_workspace_bytes": ([I64, I64, ctypes.POINTER(SZ)], I),
        "ubw_fit_bases": ([P, I, I64, I64, I, I, P, P, P, P, P, SZ, P], I),
        "ubw_gram": ([P, I, I64, I64, ctypes.c_float, P, P], I),
        "ubw_saliency_workspace_bytes": ([I64, I64, ctypes.POINTER(SZ)], I),
        "ubw_hessian_saliency": ([P, I64, ctypes.c_float, P, I64, I64, P, P, P, P, SZ, P], I),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().ubw_status_str(int(status)).decode()


def _check(fn, status):
    if status != UBW_OK:
        raise UbwError(fn, status)


# ---------------------------------------------------------------------------------------------
# torch marshalling helpers

def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtypes):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (no CPU path exists)")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _xdtype(x):
    torch = _torch()
    if x.dtype == torch.float16:
        return UBW_F16
    if x.dtype == torch.float32:
        return UBW_F32
    raise TypeError(f"x must be float16 or float32, got {x.dtype}")


def _as_2d(x):
    return x if x.dim() == 2 else x.reshape(1, -1)


def _words_dtypes():
    torch = _torch()
    return (torch.int32, torch.uint32)


# ---------------------------------------------------------------------------------------------
# the calls (same names as the C ABI without the ubw_ prefix)

def packed_words(nb: int, n: int, k: int, g: int = 8) -> int:
    out = ctypes.c_int64(0)
    _check("ubw_packed_words", lib().ubw_packed_words(nb, n, k, g, ctypes.byref(out)))
    return out.value


def lut_gemv_workspace_bytes(nb: int, n: int, k: int, g: int = 8, batch: int = 1) -> int:
    out = ctypes.c_size_t(0)
    _check("ubw_lut_gemv_workspace_bytes", lib().ubw_lut_gemv_workspace_bytes(nb, n, k, g, batch, ctypes.byref(out)))
    return out.value


workspace_bytes = lut_gemv_workspace_bytes


def workspace_check(workspace, clear: bool = False):
    """Word 0 of a GEMV workspace (None: the static workspace of lut_gemv_refined_noalloc on the
    current device) after the current stream's work has finished: returns (status, word), status
    being UBW_OK, UBW_EWAIT (bit 0: a wait gave up, outputs not written) or UBW_ERANGE (bit 1: a
    salient index out of range or out of order). clear=True zeroes the word afterwards."""
    word = ctypes.c_uint32(0)
    wp = None if workspace is None else _dev(workspace, "workspace", None)
    st = lib().ubw_workspace_check(wp, 1 if clear else 0, _stream(), ctypes.byref(word))
    if st not in (UBW_OK, UBW_EWAIT, UBW_ERANGE):
        raise UbwError("ubw_workspace_check", st)
    return st, word.value


def workspace(n: int, device="cuda"):
    """A zero-filled workspace for GEMV calls with n output rows (reusable on one stream)."""
    torch = _torch()
    return torch.zeros(workspace_bytes(1, n, 1) // 4, dtype=torch.int32, device=device)


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _dev(workspace, "workspace", None), workspace.numel() * workspace.element_size()


def pack_bases(src, nb: int, n: int, k: int, g: int = 8, out=None):
    """Pack canonical uint32 words [nb, n, ceil(k/32)] (int32/uint32 tensor) or int8 signs
    [nb, n, k] into the GPU tile layout; returns an int32 tensor of packed_words() words."""
    torch = _torch()
    if src.dtype == torch.int8:
        fmt = UBW_SRC_INT8_SIGNS
        if tuple(src.shape) != (nb, n, k):
            raise ValueError(f"int8 signs must have shape {(nb, n, k)}, got {tuple(src.shape)}")
    else:
        fmt = UBW_SRC_CANON_BITS
        if tuple(src.shape) != (nb, n, (k + 31) // 32):
            raise ValueError(f"canonical words must have shape {(nb, n, (k + 31) // 32)}, got {tuple(src.shape)}")
    sp = _dev(src, "src", (torch.int8,) + _words_dtypes())
    words = packed_words(nb, n, k, g)
    if out is None:
        out = torch.empty(words, dtype=torch.int32, device=src.device)
    elif out.numel() < words:
        raise ValueError("out is too small")
    _check("ubw_pack_bases", lib().ubw_pack_bases(sp, fmt, nb, n, k, g, _dev(out, "out", _words_dtypes()), _stream()))
    return out


def ternary_encode(w, scale, g: int = 8):
    """Ternary int8 weights [n, k] and per-row scale [n] -> (packed, alpha_r [2, n], alpha_c [2, k])."""
    torch = _torch()
    n, k = w.shape
    wp = _dev(w, "w", (torch.int8,))
    sp = _dev(scale, "scale", (torch.float32,))
    packed = torch.empty(packed_words(2, n, k, g), dtype=torch.int32, device=w.device)
    ar = torch.empty((2, n), dtype=torch.float32, device=w.device)
    ac = torch.empty((2, k), dtype=torch.float32, device=w.device)
    _check("ubw_ternary_encode", lib().ubw_ternary_encode(wp, sp, n, k, g, _dev(packed, "packed", None),
                                                          _dev(ar, "alpha_r", None), _dev(ac, "alpha_c", None),
                                                          _stream()))
    return packed, ar, ac


def build_lut(x, alpha_c, g: int = 8):
    """LUT-BSF tables [batch, nb, ceil(K/g), 2**g] fp32 with alpha_c folded in."""
    torch = _torch()
    x = _as_2d(x)
    batch, k = x.shape
    nb = alpha_c.shape[0]
    if alpha_c.shape[1] != k:
        raise ValueError("alpha_c must be [nb, K]")
    ng = (k + g - 1) // g
    lut = torch.empty((batch, nb, ng, 1 << g), dtype=torch.float32, device=x.device)
    _check("ubw_build_lut", lib().ubw_build_lut(_dev(x, "x", None), _xdtype(x), batch,
                                                _dev(alpha_c, "alpha_c", (torch.float32,)), nb, k, g,
                                                _dev(lut, "lut", None), _stream()))
    return lut


def lut_gemv(packed, alpha_r, alpha_c, x, n: int, k: int, g: int = 8, y=None, accumulate: bool = False,
             workspace=None):
    """y (= or +=) sum_k alpha_r^(k) (.) (B^(k) (alpha_c^(k) (.) x)); x [batch, K] fp16/fp32,
    y [batch, N] fp32. Returns y."""
    torch = _torch()
    x = _as_2d(x)
    batch = x.shape[0]
    nb = alpha_r.shape[0]
    if x.shape[1] != k or tuple(alpha_r.shape) != (nb, n) or tuple(alpha_c.shape) != (nb, k):
        raise ValueError("shape mismatch between x, alpha_r, alpha_c and (n, k)")
    if packed.numel() < packed_words(nb, n, k, g):
        raise ValueError("packed buffer smaller than packed_words()")
    if y is None:
        if accumulate:
            raise ValueError("accumulate=True needs y")
        y = torch.empty((batch, n), dtype=torch.float32, device=x.device)
    if tuple(y.shape) != (batch, n):
        raise ValueError(f"y must be [{batch}, {n}]")
    ws, wsb = _ws(workspace)
    _check("ubw_lut_gemv", lib().ubw_lut_gemv(_dev(packed, "packed", _words_dtypes()),
                                              _dev(alpha_r, "alpha_r", (torch.float32,)),
                                              _dev(alpha_c, "alpha_c", (torch.float32,)), nb, n, k, g,
                                              _dev(x, "x", None), _xdtype(x), batch,
                                              _dev(y, "y", (torch.float32,)), 1 if accumulate else 0,
                                              ws, wsb, _stream()))
    return y


def vcm_gather_refine(idx, packed_s, alpha_r_s, alpha_c_s, x, n: int, k: int, y, g: int = 8, workspace=None):
    """y += salient refinement over the columns idx (int32 [s]); returns y."""
    torch = _torch()
    x = _as_2d(x)
    batch = x.shape[0]
    s = idx.shape[0]
    ns = alpha_r_s.shape[0]
    if x.shape[1] != k or tuple(alpha_r_s.shape) != (ns, n) or tuple(alpha_c_s.shape) != (ns, s):
        raise ValueError("shape mismatch between x, idx, alpha_r_s, alpha_c_s and (n, k)")
    if packed_s.numel() < packed_words(ns, n, s, g):
        raise ValueError("packed_s buffer smaller than packed_words()")
    if tuple(y.shape) != (batch, n):
        raise ValueError(f"y must be [{batch}, {n}]")
    ws, wsb = _ws(workspace)
    _check("ubw_vcm_gather_refine",
           lib().ubw_vcm_gather_refine(_dev(idx, "idx", (torch.int32,)), s, _dev(packed_s, "packed_s", _words_dtypes()),
                                       _dev(alpha_r_s, "alpha_r_s", (torch.float32,)),
                                       _dev(alpha_c_s, "alpha_c_s", (torch.float32,)), ns, n, k, g,
                                       _dev(x, "x", None), _xdtype(x), batch, _dev(y, "y", (torch.float32,)),
                                       ws, wsb, _stream()))
    return y


def lut_gemv_refined(packed, alpha_r, alpha_c, idx, packed_s, alpha_r_s, alpha_c_s, x, n: int, k: int, g: int = 8,
                     y=None, accumulate: bool = False, workspace=None):
    """Main bases plus salient refinement in one launch; returns y [batch, N]."""
    torch = _torch()
    x = _as_2d(x)
    batch = x.shape[0]
    nb, ns, s = alpha_r.shape[0], alpha_r_s.shape[0], idx.shape[0]
    if x.shape[1] != k or tuple(alpha_r.shape) != (nb, n) or tuple(alpha_c.shape) != (nb, k):
        raise ValueError("shape mismatch between x, alpha_r, alpha_c and (n, k)")
    if tuple(alpha_r_s.shape) != (ns, n) or tuple(alpha_c_s.shape) != (ns, s):
        raise ValueError("shape mismatch between idx, alpha_r_s, alpha_c_s and n")
    if packed.numel() < packed_words(nb, n, k, g) or packed_s.numel() < packed_words(ns, n, s, g):
        raise ValueError("packed buffer smaller than packed_words()")
    if y is None:
        if accumulate:
            raise ValueError("accumulate=True needs y")
        y = torch.empty((batch, n), dtype=torch.float32, device=x.device)
    if tuple(y.shape) != (batch, n):
        raise ValueError(f"y must be [{batch}, {n}]")
    ws, wsb = _ws(workspace)
    F32 = (torch.float32,)
    _check("ubw_lut_gemv_refined",
           lib().ubw_lut_gemv_refined(_dev(packed, "packed", _words_dtypes()), _dev(alpha_r, "alpha_r", F32),
                                      _dev(alpha_c, "alpha_c", F32), nb, _dev(idx, "idx", (torch.int32,)), s,
                                      _dev(packed_s, "packed_s", _words_dtypes()), _dev(alpha_r_s, "alpha_r_s", F32),
                                      _dev(alpha_c_s, "alpha_c_s", F32), ns, n, k, g, _dev(x, "x", None),
                                      _xdtype(x), batch, _dev(y, "y", F32), 1 if accumulate else 0, ws, wsb,
                                      _stream()))
    return y


def lut_gemv_refined_noalloc(packed, alpha_r, alpha_c, idx, packed_s, alpha_r_s, alpha_c_s, x, n: int, k: int, y,
                             g: int = 8, accumulate: bool = False):
    """lut_gemv_refined with the library's static workspace (allocates nothing; y is required,
    n <= 65536). Returns y."""
    torch = _torch()
    x = _as_2d(x)
    batch = x.shape[0]
    nb, ns, s = alpha_r.shape[0], alpha_r_s.shape[0], idx.shape[0]
    if x.shape[1] != k or tuple(alpha_r.shape) != (nb, n) or tuple(alpha_c.shape) != (nb, k):
        raise ValueError("shape mismatch between x, alpha_r, alpha_c and (n, k)")
    if tuple(alpha_r_s.shape) != (ns, n) or tuple(alpha_c_s.shape) != (ns, s):
        raise ValueError("shape mismatch between idx, alpha_r_s, alpha_c_s and n")
    if packed.numel() < packed_words(nb, n, k, g) or packed_s.numel() < packed_words(ns, n, s, g):
        raise ValueError("packed buffer smaller than packed_words()")
    if tuple(y.shape) != (batch, n):
        raise ValueError(f"y must be [{batch}, {n}]")
    F32 = (torch.float32,)
    _check("ubw_lut_gemv_refined_noalloc",
           lib().ubw_lut_gemv_refined_noalloc(_dev(packed, "packed", _words_dtypes()), _dev(alpha_r, "alpha_r", F32),
                                              _dev(alpha_c, "alpha_c", F32), nb, _dev(idx, "idx", (torch.int32,)), s,
                                              _dev(packed_s, "packed_s", _words_dtypes()),
                                              _dev(alpha_r_s, "alpha_r_s", F32), _dev(alpha_c_s, "alpha_c_s", F32), ns,
                                              n, k, g, _dev(x, "x", None), _xdtype(x), batch, _dev(y, "y", F32),
                                              1 if accumulate else 0, _stream()))
    return y


GROUP_COLS = 128


def group_scale_cols(k: int) -> int:
    """Blocks of 128 columns per row, padded to an even count (2 * ceil(k / 256))."""
    return 2 * ((int(k) + 255) // 256)


def arrange_group_scales(a):
    """Host-side layout of block scales for lut_gemv_gs: numpy [nb, n, group_scale_cols(k)]
    (block q of row r at [k, r, q]) -> fp16 [nb, ceil(k/256), n, 2], slice-major."""
    import numpy as np
    a = np.asarray(a, dtype=np.float16)
    nb, n, cols = a.shape
    if cols % 2:
        raise ValueError("pad the block count to an even number (group_scale_cols)")
    return np.ascontiguousarray(a.reshape(nb, n, cols // 2, 2).transpose(0, 2, 1, 3))


def lut_gemv_gs(packed, alpha_rg, alpha_c, x, n: int, k: int, g: int = 8, idx=None, packed_s=None, alpha_r_s=None,
                alpha_c_s=None, y=None, accumulate: bool = False, workspace=None):
    """Group-scale variant: alpha_rg fp16 [nb, ceil(k/256), n, 2] (arrange_group_scales) holds
    one row scale per 128 columns; optional refinement (idx, packed_s, alpha_r_s, alpha_c_s) as
    lut_gemv_refined. Returns y [batch, N]."""
    torch = _torch()
    x = _as_2d(x)
    batch = x.shape[0]
    nb = alpha_rg.shape[0]
    if x.shape[1] != k or tuple(alpha_rg.shape) != (nb, (k + 255) // 256, n, 2) or tuple(alpha_c.shape) != (nb, k):
        raise ValueError("shape mismatch between x, alpha_rg, alpha_c and (n, k)")
    if packed.numel() < packed_words(nb, n, k, g):
        raise ValueError("packed buffer smaller than packed_words()")
    F32 = (torch.float32,)
    ref = (None, 0, None, None, None, 0)
    if idx is not None:
        ns, s = alpha_r_s.shape[0], idx.shape[0]
        if tuple(alpha_r_s.shape) != (ns, n) or tuple(alpha_c_s.shape) != (ns, s):
            raise ValueError("shape mismatch between idx, alpha_r_s, alpha_c_s and n")
        if packed_s.numel() < packed_words(ns, n, s, g):
            raise ValueError("packed_s buffer smaller than packed_words()")
        ref = (_dev(idx, "idx", (torch.int32,)), s, _dev(packed_s, "packed_s", _words_dtypes()),
               _dev(alpha_r_s, "alpha_r_s", F32), _dev(alpha_c_s, "alpha_c_s", F32), ns)
    if y is None:
        if accumulate:
            raise ValueError("accumulate=True needs y")
        y = torch.empty((batch, n), dtype=torch.float32, device=x.device)
    if tuple(y.shape) != (batch, n):
        raise ValueError(f"y must be [{batch}, {n}]")
    ws, wsb = _ws(workspace)
    _check("ubw_lut_gemv_gs",
           lib().ubw_lut_gemv_gs(_dev(packed, "packed", _words_dtypes()),
                                 _dev(alpha_rg, "alpha_rg", (torch.float16, torch.int16)),
                                 _dev(alpha_c, "alpha_c", F32), nb, GROUP_COLS, *ref, n, k, g, _dev(x, "x", None),
                                 _xdtype(x), batch, _dev(y, "y", F32), 1 if accumulate else 0, ws, wsb, _stream()))
    return y


def lut_gemv_multi(gemvs, x, k: int, g: int = 8, accumulate: bool = False):
    """Several GEMVs on the same x in one launch. `gemvs` is a list of dicts with keys packed,
    alpha_r, alpha_c, n, y and optionally idx, packed_s, alpha_r_s, alpha_c_s (refinement) and
    workspace; each y is [batch, n] fp32 (written, or added to with accumulate=True). Returns the
    list of outputs."""
    torch = _torch()
    x = _as_2d(x)
    batch = x.shape[0]
    if not 1 <= len(gemvs) <= MAX_GROUP:
        raise ValueError(f"1 to {MAX_GROUP} GEMVs per call")
    if x.shape[1] != k:
        raise ValueError("x must have k columns")
    F32 = (torch.float32,)
    descs = (GemvDesc * len(gemvs))()
    outs = []
    for d, G in zip(descs, gemvs):
        n = G["n"]
        nb = G["alpha_r"].shape[0]
        if tuple(G["alpha_r"].shape) != (nb, n) or tuple(G["alpha_c"].shape) != (nb, k):
            raise ValueError("shape mismatch between alpha_r, alpha_c and (n, k)")
        if G["packed"].numel() < packed_words(nb, n, k, g):
            raise ValueError("packed buffer smaller than packed_words()")
        y = G["y"]
        if tuple(y.shape) != (batch, n):
            raise ValueError(f"y must be [{batch}, {n}]")
        d.packed = _dev(G["packed"], "packed", _words_dtypes()).value
        d.alpha_r = _dev(G["alpha_r"], "alpha_r", F32).value
        d.alpha_c = _dev(G["alpha_c"], "alpha_c", F32).value
        d.nb = nb
        if G.get("idx") is not None:
            s, ns = G["idx"].shape[0], G["alpha_r_s"].shape[0]
            if tuple(G["alpha_r_s"].shape) != (ns, n) or tuple(G["alpha_c_s"].shape) != (ns, s):
                raise ValueError("shape mismatch between idx, alpha_r_s, alpha_c_s and n")
            if G["packed_s"].numel() < packed_words(ns, n, s, g):
                raise ValueError("packed_s buffer smaller than packed_words()")
            d.idx = _dev(G["idx"], "idx", (torch.int32,)).value
            d.s = s
            d.packed_s = _dev(G["packed_s"], "packed_s", _words_dtypes()).value
            d.alpha_r_s = _dev(G["alpha_r_s"], "alpha_r_s", F32).value
            d.alpha_c_s = _dev(G["alpha_c_s"], "alpha_c_s", F32).value
            d.ns = ns
        d.N = n
        d.y = _dev(y, "y", F32).value
        w, d.ws_bytes = _ws(G.get("workspace"))
        d.workspace = w.value if w is not None else None
        outs.append(y)
    _check("ubw_lut_gemv_multi",
           lib().ubw_lut_gemv_multi(descs, len(gemvs), k, g, _dev(x, "x", None), _xdtype(x), batch,
                                    1 if accumulate else 0, _stream()))
    return outs


def fit_workspace_bytes(n: int, k: int) -> int:
    out = ctypes.c_size_t()
    _check("ubw_fit_workspace_bytes", lib().ubw_fit_workspace_bytes(n, k, ctypes.byref(out)))
    return out.value


def fit_bases(w, nb: int, iters: int = 5, residual=None, workspace=None):
    """Fit nb bases to a dense w [N, K] (fp32 or fp16 tensor on the GPU): residual sign
    binarization with `iters` alternating least-squares rounds per base. Returns
    (bits [nb, N, ceil(K/32)] int32 canonical words, alpha_r [nb, N], alpha_c [nb, K],
    residual [N, K] fp32); bits go to pack_bases(..., src is canonical bits)."""
    torch = _torch()
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    dt = {torch.float32: 0, torch.float16: 1}.get(w.dtype)
    if dt is None:
        raise ValueError("w must be float32 or float16")
    dev = w.device
    bits = torch.empty((nb, n, (k + 31) // 32), dtype=torch.int32, device=dev)
    ar = torch.empty((nb, n), dtype=torch.float32, device=dev)
    ac = torch.empty((nb, k), dtype=torch.float32, device=dev)
    if residual is None:
        residual = torch.empty((n, k), dtype=torch.float32, device=dev)
    if tuple(residual.shape) != (n, k) or residual.dtype != torch.float32:
        raise ValueError("residual must be float32 [N, K]")
    need = fit_workspace_bytes(n, k)
    if workspace is None:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=dev)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace smaller than fit_workspace_bytes()")
    _check("ubw_fit_bases", lib().ubw_fit_bases(_dev(w, "w", None), dt, n, k, nb, iters, _dev(bits, "bits", None),
                                                _dev(ar, "alpha_r", None), _dev(ac, "alpha_c", None),
                                                _dev(residual, "residual", None), _dev(workspace, "workspace", None),
                                                need, _stream()))
    return bits, ar, ac, residual


def gram(x, scale: float = 2.0, out=None):
    """H = scale * x^T x on the matrix cores; x fp16 [T, K] on the GPU. Returns H fp32 [K, K]."""
    torch = _torch()
    if x.dim() != 2 or x.dtype != torch.float16:
        raise ValueError("x must be float16 [T, K]")
    t, k = x.shape
    if out is None:
        out = torch.empty((k, k), dtype=torch.float32, device=x.device)
    if tuple(out.shape) != (k, k) or out.dtype != torch.float32:
        raise ValueError("out must be float32 [K, K]")
    _check("ubw_gram", lib().ubw_gram(_dev(x, "x", None), 1, t, k, float(scale), _dev(out, "H", None), _stream()))
    return out


def saliency_workspace_bytes(n: int, k: int) -> int:
    out = ctypes.c_size_t()
    _check("ubw_saliency_workspace_bytes", lib().ubw_saliency_workspace_bytes(n, k, ctypes.byref(out)))
    return out.value


def hessian_saliency(h, w, s: int, damp: float = 0.01, workspace=None):
    """Salient columns from the Hessian h [K, K] fp32 (overwritten: its lower triangle becomes
    the damped Cholesky factor) and the dense weights w [N, K] fp32. Returns (d [K] = diag of
    the damped inverse, score [K], idx [s] int32 ascending, workspace); workspace[0] holds the
    damping lambda and workspace[1] an error code (0 = none)."""
    torch = _torch()
    k = h.shape[0]
    if tuple(h.shape) != (k, k) or h.dtype != torch.float32:
        raise ValueError("h must be float32 [K, K]")
    if w.dim() != 2 or w.shape[1] != k or w.dtype != torch.float32:
        raise ValueError("w must be float32 [N, K]")
    n = w.shape[0]
    need = saliency_workspace_bytes(n, k)
    if workspace is None:
        workspace = torch.empty(need // 4, dtype=torch.float32, device=h.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace smaller than saliency_workspace_bytes()")
    d = torch.empty(k, dtype=torch.float32, device=h.device)
    score = torch.empty(k, dtype=torch.float32, device=h.device)
    idx = torch.empty(s, dtype=torch.int32, device=h.device)
    _check("ubw_hessian_saliency",
           lib().ubw_hessian_saliency(_dev(h, "h", None), k, float(damp), _dev(w, "w", None), n, s, _dev(d, "d", None),
                                      _dev(score, "score", None), _dev(idx, "idx", None),
                                      _dev(workspace, "workspace", None), need, _stream()))
    return d, score, idx, workspace


def check_indices(idx_host, k: int) -> None:
    """Host check: indices ascending, distinct, inside [0, k). idx_host: numpy int32 array."""
    import numpy as np
    a = np.ascontiguousarray(idx_host, dtype=np.int32)
    _check("ubw_check_indices", lib().ubw_check_indices(a.ctypes.data_as(ctypes.c_void_p), a.shape[0], k))


def extract_patterns(packed, nb: int, n: int, k: int, g: int = 8):
    """Pattern indices [nb, n, ceil(k/g)] (int16 storage of uint16 values)."""
    torch = _torch()
    ng = (k + g - 1) // g
    out = torch.empty((nb, n, ng), dtype=torch.int16, device=packed.device)
    _check("ubw_extract_patterns", lib().ubw_extract_patterns(_dev(packed, "packed", _words_dtypes()), nb, n, k, g,
                                                              _dev(out, "out", None), _stream()))
    return out


def lut_gemv_geometry(packed, alpha_r, alpha_c, x, n: int, kv: int, y, *, idx=None, k=None, accumulate=False,
                      rows_per_group=1, workgroups=0, workspace=None, group_scales=False):
    """Main (idx None) or refinement (idx given, k = x's row length) GEMV with an explicit
    launch geometry; for tests and tuning. group_scales=True: main bases with alpha_r the fp16
    group-scale array of lut_gemv_gs."""
    torch = _torch()
    x = _as_2d(x)
    batch = x.shape[0]
    nb = alpha_r.shape[0]
    vcm = idx is not None
    if group_scales and (vcm or tuple(alpha_r.shape) != (nb, (kv + 255) // 256, n, 2)):
        raise ValueError("group scales: main bases only, alpha_r [nb, ceil(k/256), n, 2] fp16")
    mode = 1 if vcm else (2 if group_scales else 0)
    ar_types = (torch.float16, torch.int16) if group_scales else (torch.float32,)
    _check("ubw_lut_gemv_geometry",
           lib().ubw_lut_gemv_geometry(_dev(packed, "packed", _words_dtypes()), _dev(alpha_r, "alpha_r", ar_types),
                                       _dev(alpha_c, "alpha_c", (torch.float32,)), nb, n, kv,
                                       _dev(idx, "idx", (torch.int32,)) if vcm else None, k if vcm else kv,
                                       _dev(x, "x", None), _xdtype(x), batch, _dev(y, "y", (torch.float32,)),
                                       1 if accumulate else 0, mode, rows_per_group, workgroups,
                                       *_ws(workspace), _stream()))
    return y


def bench_stream_read(buf, nbytes: int, out):
    """Measurement helper: one streaming read of nbytes of buf (see include/ubw.h)."""
    _check("ubw_bench_stream_read", lib().ubw_bench_stream_read(_dev(buf, "buf", None), int(nbytes),
                                                                _dev(out, "out", None), _stream()))
