"""CPU-only checks of the C ABI: the library loads, exports every symbol include/ubw.h
declares, and rejects bad arguments on the host before anything is enqueued (no GPU needed:
none of these calls reaches a kernel launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import ultra_bit_weight_uint32_amd as ubw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ubw.h")

EINVAL, EUNSUP, EALIGN, ERANGE, ESIZE = -1, -2, -3, -4, -6
FAKE = ctypes.c_void_p(0x10000)        # 16-byte aligned, never dereferenced on these paths
MISALIGNED = ctypes.c_void_p(0x10004)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(ubw_\w+)\s*\(", text, re.M)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(ubw.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ubw.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert ubw.lib().ubw_version() >= 1


def test_status_strings():
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert ubw.status_str(st).startswith("UBW_") or st == 0
    assert "unknown" in ubw.status_str(-99)


def test_packed_words_sizes():
    # tiles of 256 rows x 256 columns per base: 2048 words each
    assert ubw.packed_words(2, 4096, 4096) == 2 * 16 * 16 * 2048
    assert ubw.packed_words(1, 1, 1) == 2048
    assert ubw.packed_words(3, 257, 257) == 3 * 2 * 2 * 2048
    assert ubw.packed_words(1, 256, 4096, g=4) == 16 * 2048
    out = ctypes.c_int64()
    L = ubw.lib()
    assert L.ubw_packed_words(0, 10, 10, 8, ctypes.byref(out)) == EINVAL
    assert L.ubw_packed_words(1, 0, 10, 8, ctypes.byref(out)) == EINVAL
    assert L.ubw_packed_words(1, 10, 0, 8, ctypes.byref(out)) == EINVAL
    assert L.ubw_packed_words(1, 10, 10, 6, ctypes.byref(out)) == EUNSUP
    assert L.ubw_packed_words(1, 10, 10, 8, None) == EINVAL


def test_workspace_bytes():
    # 16 header words + 64 words per 256-row group
    assert ubw.workspace_bytes(2, 4096, 4096, 8, 1) == 4 * (16 + 64 * 16)
    assert ubw.workspace_bytes(1, 1, 1, 8, 1) == 4 * (16 + 64)
    sz = ctypes.c_size_t()
    L = ubw.lib()
    for fn in (L.ubw_lut_gemv_workspace_bytes, L.ubw_workspace_bytes):
        assert fn(2, 4096, 4096, 8, 1, ctypes.byref(sz)) == 0 and sz.value == 4 * (16 + 64 * 16)
        assert fn(2, 4096, 4096, 8, 17, ctypes.byref(sz)) == EINVAL
        assert fn(2, 4096, 4096, 4, 1, ctypes.byref(sz)) == 0 and sz.value == 4 * 16  # g = 4: header only
        assert fn(2, 4096, 4096, 5, 1, ctypes.byref(sz)) == EUNSUP
        assert fn(2, 4096, 4096, 8, 1, None) == EINVAL


def test_workspace_check_rejects():
    word = ctypes.c_uint32()
    L = ubw.lib()
    assert L.ubw_workspace_check(FAKE, 0, None, None) == EINVAL
    assert L.ubw_workspace_check(None, 0, None, None) == EINVAL
    assert L.ubw_workspace_check(MISALIGNED, 1, None, ctypes.byref(word)) == EALIGN


def noalloc_args(**kw):
    a = dict(packed=FAKE, alpha_r=FAKE, alpha_c=FAKE, nb=2, idx=FAKE, s=10, packed_s=FAKE, alpha_r_s=FAKE,
             alpha_c_s=FAKE, ns=1, N=4096, K=4096, g=8, x=FAKE, x_dtype=1, batch=1, y=FAKE, accumulate=0, stream=None)
    a.update(kw)
    return ubw.lib().ubw_lut_gemv_refined_noalloc(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(N=65537), ERANGE), (dict(N=1 << 20), ERANGE), (dict(idx=None), EINVAL), (dict(packed=None), EINVAL),
    (dict(g=2), EUNSUP), (dict(batch=17), EINVAL), (dict(packed_s=MISALIGNED), EALIGN), (dict(ns=0), EINVAL),
    (dict(g=4, K=40000), EUNSUP), (dict(g=4, s=600), EUNSUP), (dict(g=4, nb=3), EUNSUP),
])
def test_noalloc_rejects_before_touching_the_device(kw, status):
    """Every argument check of the allocation-free entry point runs on the host before the static
    workspace is looked up (no GPU is needed for these)."""
    assert noalloc_args(**kw) == status


def gemv_args(**kw):
    a = dict(packed=FAKE, alpha_r=FAKE, alpha_c=FAKE, nb=2, N=64, K=64, g=8, x=FAKE, x_dtype=1, batch=1,
             y=FAKE, accumulate=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return ubw.lib().ubw_lut_gemv(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(packed=None), EINVAL), (dict(alpha_r=None), EINVAL), (dict(alpha_c=None), EINVAL),
    (dict(x=None), EINVAL), (dict(y=None), EINVAL), (dict(nb=0), EINVAL), (dict(N=0), EINVAL),
    (dict(K=0), EINVAL), (dict(N=-5), EINVAL), (dict(batch=0), EINVAL), (dict(batch=17), EINVAL),
    (dict(x_dtype=7), EUNSUP), (dict(g=2), EUNSUP), (dict(g=5), EUNSUP), (dict(packed=MISALIGNED), EALIGN),
    (dict(ws=None, wsb=8), EINVAL), (dict(ws=MISALIGNED, wsb=4096), EALIGN), (dict(ws=FAKE, wsb=8), ESIZE),
    # group width 4: tables of the whole row in LDS (K = 40000 does not fit), 1, 2 or 4 bases,
    # a workspace of at least the 16 header words
    (dict(g=4, K=40000), EUNSUP), (dict(g=4, K=8192, nb=1), EUNSUP), (dict(g=4, nb=3), EUNSUP),
    (dict(g=4, ws=FAKE, wsb=32), ESIZE),
])
def test_lut_gemv_rejects(kw, status):
    assert gemv_args(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(idx=None), EINVAL), (dict(s=0), EINVAL), (dict(packed_s=None), EINVAL), (dict(ns=0), EINVAL),
    (dict(K=0), EINVAL), (dict(g=2), EUNSUP), (dict(batch=0), EINVAL), (dict(packed_s=MISALIGNED), EALIGN),
    (dict(g=4, s=600), EUNSUP), (dict(g=4, ns=3), EUNSUP),
])
def test_vcm_rejects(kw, status):
    a = dict(idx=FAKE, s=10, packed_s=FAKE, alpha_r_s=FAKE, alpha_c_s=FAKE, ns=2, N=64, K=64, g=8, x=FAKE,
             x_dtype=1, batch=1, y=FAKE, ws=None, wsb=0, stream=None)
    a.update(kw)
    assert ubw.lib().ubw_vcm_gather_refine(*a.values()) == status


def test_geometry_rejects():
    L = ubw.lib()
    base = [FAKE, FAKE, FAKE, 2, 64, 64, None, 64, FAKE, 1, 1, FAKE, 0, 0]
    tail = [None, 0, None]
    assert L.ubw_lut_gemv_geometry(*base, 3, 1, *tail) == ERANGE      # rows_per_group not in {1,2,4}
    assert L.ubw_lut_gemv_geometry(*base, 8, 1, *tail) == ERANGE
    assert L.ubw_lut_gemv_geometry(*base, 1, -1, *tail) == ERANGE     # workgroups < 0
    for batch in (2, 4, 16):                                          # batches: 1 or 2 row tiles
        bb = list(base)
        bb[10] = batch
        assert L.ubw_lut_gemv_geometry(*bb, 4, 1, *tail) == ERANGE
    vcm = list(base)
    vcm[13] = 1                                                       # vcm without idx
    assert L.ubw_lut_gemv_geometry(*vcm, 1, 1, *tail) == EINVAL
    assert L.ubw_lut_gemv_geometry(*base, 1, 1, FAKE, 4, None) == ESIZE


def test_refined_rejects():
    L = ubw.lib()
    args = dict(packed=FAKE, ar=FAKE, ac=FAKE, nb=2, idx=FAKE, s=10, packed_s=FAKE, ar_s=FAKE, ac_s=FAKE, ns=2,
                N=64, K=64, g=8, x=FAKE, x_dtype=1, batch=1, y=FAKE, acc=0, ws=None, wsb=0, stream=None)
    for kw, status in [(dict(idx=None), EINVAL), (dict(s=0), EINVAL), (dict(ns=0), EINVAL), (dict(nb=0), EINVAL),
                       (dict(packed_s=MISALIGNED), EALIGN), (dict(g=2), EUNSUP), (dict(ws=FAKE, wsb=4), ESIZE),
                       (dict(g=4, s=600), EUNSUP), (dict(g=4, K=40000), EUNSUP),
                       (dict(batch=17), EINVAL)]:
        a = dict(args)
        a.update(kw)
        assert L.ubw_lut_gemv_refined(*a.values()) == status, kw


def multi_desc(**kw):
    d = ubw.GemvDesc()
    vals = dict(packed=FAKE.value, alpha_r=FAKE.value, alpha_c=FAKE.value, nb=2, idx=None, s=0, packed_s=None,
                alpha_r_s=None, alpha_c_s=None, ns=0, N=64, y=FAKE.value, workspace=None, ws_bytes=0)
    vals.update(kw)
    for k, v in vals.items():
        setattr(d, k, v)
    return d


def multi_call(descs, K=64, g=8, x=FAKE, x_dtype=1, batch=1):
    arr = (ubw.GemvDesc * max(1, len(descs)))(*descs)
    return ubw.lib().ubw_lut_gemv_multi(arr, len(descs), K, g, x, x_dtype, batch, 0, None)


def test_multi_rejects():
    L = ubw.lib()
    ok = multi_desc()
    assert L.ubw_lut_gemv_multi(None, 1, 64, 8, FAKE, 1, 1, 0, None) == EINVAL       # null descs
    assert multi_call([]) == EINVAL                                                   # count 0
    assert multi_call([multi_desc(y=0x10000 + 256 * i) for i in range(9)]) == EINVAL   # count > UBW_MAX_GROUP
    assert multi_call([ok], g=4) == EUNSUP
    assert multi_call([ok], K=0) == EINVAL
    assert multi_call([ok], x=None) == EINVAL
    assert multi_call([ok], x_dtype=7) == EUNSUP
    assert multi_call([ok], batch=17) == EINVAL
    assert multi_call([ok, multi_desc()]) == EINVAL                                   # same y twice
    ws = 0x20000
    assert multi_call([multi_desc(workspace=ws, ws_bytes=4096),
                       multi_desc(y=0x30000, workspace=ws, ws_bytes=4096)]) == EINVAL  # shared workspace
    # the second desc is the bad one: every desc is checked before anything is enqueued
    for kw, status in [(dict(packed=None), EINVAL), (dict(nb=0), EINVAL), (dict(N=0), EINVAL),
                       (dict(packed=MISALIGNED.value), EALIGN), (dict(workspace=FAKE.value, ws_bytes=8), ESIZE),
                       (dict(workspace=MISALIGNED.value, ws_bytes=4096), EALIGN),
                       (dict(idx=FAKE.value, s=0, packed_s=FAKE.value, alpha_r_s=FAKE.value,
                             alpha_c_s=FAKE.value, ns=2), EINVAL),
                       (dict(idx=FAKE.value, s=10, packed_s=None, alpha_r_s=FAKE.value,
                             alpha_c_s=FAKE.value, ns=2), EINVAL),
                       (dict(idx=FAKE.value, s=10, packed_s=MISALIGNED.value, alpha_r_s=FAKE.value,
                             alpha_c_s=FAKE.value, ns=2), EALIGN),
                       (dict(idx=FAKE.value, s=10, packed_s=FAKE.value, alpha_r_s=FAKE.value,
                             alpha_c_s=FAKE.value, ns=0), EINVAL)]:
        bad = multi_desc(y=0x30000, **kw)
        assert multi_call([ok, bad]) == status, kw


def test_gemv_desc_layout():
    # the binding's struct mirrors ubw_gemv_desc field for field (LP64 layout)
    offs = [(f, getattr(ubw.GemvDesc, f).offset) for f, _ in ubw.GemvDesc._fields_]
    assert offs == [("packed", 0), ("alpha_r", 8), ("alpha_c", 16), ("nb", 24), ("idx", 32), ("s", 40),
                    ("packed_s", 48), ("alpha_r_s", 56), ("alpha_c_s", 64), ("ns", 72), ("N", 80), ("y", 88),
                    ("workspace", 96), ("ws_bytes", 104)]
    assert ctypes.sizeof(ubw.GemvDesc) == 112
    text = open(HEADER).read()
    body = re.search(r"typedef struct ubw_gemv_desc \{(.*?)\} ubw_gemv_desc;", text, re.S).group(1)
    names = re.findall(r"(\w+);", body)
    assert names == [f for f, _ in ubw.GemvDesc._fields_]


def test_gs_rejects():
    L = ubw.lib()
    args = dict(packed=FAKE, arg=FAKE, ac=FAKE, nb=2, gsize=128, idx=None, s=0, packed_s=None, ar_s=None, ac_s=None,
                ns=0, N=64, K=300, g=8, x=FAKE, x_dtype=1, batch=1, y=FAKE, acc=0, ws=None, wsb=0, stream=None)
    ref = dict(idx=FAKE, s=10, packed_s=FAKE, ar_s=FAKE, ac_s=FAKE, ns=2)
    for kw, status in [(dict(arg=None), EINVAL), (dict(gsize=64), EUNSUP), (dict(gsize=0), EUNSUP),
                       (dict(arg=ctypes.c_void_p(0x10002)), EALIGN), (dict(g=4), EUNSUP), (dict(nb=0), EINVAL),
                       (dict(batch=17), EINVAL), (dict(ws=FAKE, wsb=4), ESIZE), (dict(packed=MISALIGNED), EALIGN),
                       (dict(ref, s=0), EINVAL), (dict(ref, packed_s=None), EINVAL), (dict(ref, ns=0), EINVAL),
                       (dict(ref, packed_s=MISALIGNED), EALIGN)]:
        a = dict(args)
        a.update(kw)
        assert L.ubw_lut_gemv_gs(*a.values()) == status, kw
    base = [FAKE, FAKE, FAKE, 2, 64, 64, None, 64, FAKE, 1, 1, FAKE, 0]
    tail = [1, 1, None, 0, None]
    assert L.ubw_lut_gemv_geometry(*base, 3, *tail) == ERANGE                     # mode outside 0..2
    assert L.ubw_lut_gemv_geometry(*base, -1, *tail) == ERANGE
    b2 = list(base)
    b2[1] = ctypes.c_void_p(0x10002)
    assert L.ubw_lut_gemv_geometry(*b2, 2, *tail) == EALIGN                       # group scales: 4-byte aligned


def test_fit_rejects():
    L = ubw.lib()
    sz = ctypes.c_size_t()
    assert L.ubw_fit_workspace_bytes(0, 10, ctypes.byref(sz)) == EINVAL
    assert L.ubw_fit_workspace_bytes(10, 10, None) == EINVAL
    assert L.ubw_fit_workspace_bytes(100, 300, ctypes.byref(sz)) == 0
    assert sz.value == 4 * (2 * 300 + 2 + 5)                      # 2 row chunks of 64, 5 blocks of 64 columns
    need = sz.value
    args = dict(w=FAKE, dt=0, N=100, K=300, nb=2, iters=3, bits=FAKE, ar=FAKE, ac=FAKE, res=FAKE, ws=FAKE,
                wsb=need, stream=None)
    for kw, status in [(dict(w=None), EINVAL), (dict(bits=None), EINVAL), (dict(res=None), EINVAL),
                       (dict(ws=None), EINVAL), (dict(N=0), EINVAL), (dict(K=-1), EINVAL), (dict(nb=0), EINVAL),
                       (dict(nb=65), EINVAL), (dict(iters=-1), EINVAL), (dict(iters=10001), EINVAL),
                       (dict(dt=5), EUNSUP), (dict(ar=ctypes.c_void_p(0x10002)), EALIGN),
                       (dict(wsb=need - 4), ESIZE), (dict(N=65535 * 64 + 1, wsb=1 << 40), ERANGE)]:
        a = dict(args)
        a.update(kw)
        assert L.ubw_fit_bases(*a.values()) == status, kw


def test_saliency_rejects():
    L = ubw.lib()
    assert L.ubw_gram(None, 1, 10, 10, 2.0, FAKE, None) == EINVAL
    assert L.ubw_gram(FAKE, 1, 0, 10, 2.0, FAKE, None) == EINVAL
    assert L.ubw_gram(FAKE, 0, 10, 10, 2.0, FAKE, None) == EUNSUP          # fp16 only
    assert L.ubw_gram(ctypes.c_void_p(0x10001), 1, 10, 10, 2.0, FAKE, None) == EALIGN
    assert L.ubw_gram(FAKE, 1, 10, 65535 * 128 + 1, 2.0, FAKE, None) == ERANGE
    sz = ctypes.c_size_t()
    assert L.ubw_saliency_workspace_bytes(100, 0, ctypes.byref(sz)) == EINVAL
    assert L.ubw_saliency_workspace_bytes(100, 300, ctypes.byref(sz)) == 0
    nblk = 5
    assert sz.value == 4 * (16 + nblk * 4096 + 4096 * nblk * (nblk + 1) // 2 + 2 * 300 + 16 * 300)
    need = sz.value
    args = dict(H=FAKE, K=300, damp=0.01, W=FAKE, N=100, s=10, d=FAKE, score=FAKE, idx=FAKE, ws=FAKE, wsb=need,
                stream=None)
    for kw, status in [(dict(H=None), EINVAL), (dict(idx=None), EINVAL), (dict(ws=None), EINVAL), (dict(s=0), EINVAL),
                       (dict(s=301), EINVAL), (dict(K=0), EINVAL), (dict(damp=-1.0), EINVAL),
                       (dict(damp=float("nan")), EINVAL), (dict(damp=float("inf")), EINVAL),
                       (dict(W=ctypes.c_void_p(0x10002)), EALIGN), (dict(wsb=need - 4), ESIZE),
                       (dict(N=65535 * 64 + 1, wsb=1 << 45), ERANGE)]:
        a = dict(args)
        a.update(kw)
        assert L.ubw_hessian_saliency(*a.values()) == status, kw


def test_other_entry_points_reject():
    L = ubw.lib()
    assert L.ubw_pack_bases(None, 0, 1, 8, 8, 8, FAKE, None) == EINVAL
    assert L.ubw_pack_bases(FAKE, 5, 1, 8, 8, 8, FAKE, None) == EUNSUP
    assert L.ubw_pack_bases(FAKE, 0, 1, 8, 8, 3, FAKE, None) == EUNSUP
    big = 1 << 29                                                      # 2^29 x 2^29 signs: 2^53 bits
    assert L.ubw_pack_bases(FAKE, 0, 1, big, big, 8, FAKE, None) == ERANGE
    assert L.ubw_ternary_encode(FAKE, FAKE, big, big, 8, FAKE, FAKE, FAKE, None) == ERANGE
    assert L.ubw_pack_bases(FAKE, 0, 1, 8, 8, 8, MISALIGNED, None) == EALIGN
    assert L.ubw_ternary_encode(None, FAKE, 8, 8, 8, FAKE, FAKE, FAKE, None) == EINVAL
    assert L.ubw_ternary_encode(FAKE, FAKE, 8, 8, 8, MISALIGNED, FAKE, FAKE, None) == EALIGN
    assert L.ubw_build_lut(FAKE, 1, 0, FAKE, 1, 8, 8, FAKE, None) == EINVAL
    assert L.ubw_build_lut(FAKE, 3, 1, FAKE, 1, 8, 8, FAKE, None) == EUNSUP
    assert L.ubw_build_lut(FAKE, 1, 1, FAKE, 1, 8, 2, FAKE, None) == EUNSUP
    assert L.ubw_extract_patterns(FAKE, 1, 8, 8, 7, FAKE, None) == EUNSUP
    assert L.ubw_extract_patterns(MISALIGNED, 1, 8, 8, 8, FAKE, None) == EALIGN


def test_check_indices_host():
    ubw.check_indices(np.array([0, 3, 9], np.int32), 10)
    for bad in ([3, 3], [4, 2], [-1, 2], [0, 10]):
        with pytest.raises(ubw.UbwError) as e:
            ubw.check_indices(np.array(bad, np.int32), 10)
        assert e.value.status == ERANGE


def test_arrange_group_scales_layout():
    rng = np.random.default_rng(3)
    a = rng.uniform(0, 1, size=(2, 5, 6)).astype(np.float16)
    d = ubw.arrange_group_scales(a)
    assert d.shape == (2, 3, 5, 2) and d.dtype == np.float16 and d.flags.c_contiguous
    for k in range(2):
        for t in range(3):
            for r in range(5):
                for h in range(2):
                    assert d[k, t, r, h] == a[k, r, 2 * t + h]
    with pytest.raises(ValueError):
        ubw.arrange_group_scales(a[:, :, :5])
    assert [ubw.group_scale_cols(k) for k in (1, 128, 129, 256, 257, 700)] == [2, 2, 2, 2, 4, 6]


def test_operands_beyond_32_bit_offsets_rejected():
    """The step addresses every operand through 32-bit buffer offsets: an operand of 2 GiB or more
    is refused on the host (UBW_EUNSUPPORTED) before anything is enqueued."""
    big_n = 300_000_000                                    # 2 bases x 300M rows of fp32 alpha_r: 2.4 GB
    assert gemv_args(N=big_n) == EUNSUP
    assert gemv_args(K=300_000_000) == EUNSUP              # alpha_c 2.4 GB
    assert gemv_args(N=64, K=600_000_000, batch=2) == EUNSUP  # x 2.4 GB
    L = ubw.lib()
    args = dict(packed=FAKE, arg=FAKE, ac=FAKE, nb=2, gsize=128, idx=None, s=0, packed_s=None, ar_s=None, ac_s=None,
                ns=0, N=big_n, K=300, g=8, x=FAKE, x_dtype=1, batch=1, y=FAKE, acc=0, ws=None, wsb=0, stream=None)
    assert L.ubw_lut_gemv_gs(*args.values()) == EUNSUP
