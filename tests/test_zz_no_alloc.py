"""The allocation-free entry point (ubw_lut_gemv_refined_noalloc, static workspace) against
ubw_lut_gemv_refined with a caller's workspace: two calls in a row, the second smaller, each
equal to the existing entry point's result (bit for bit on integer inputs, within the 1e-3
elementwise bar on floats), and the static workspace's error word clear afterwards."""
import numpy as np
import pytest

import ultra_bit_weight_uint32_amd as ubw
from workloads import make_gemv, make_integer_gemv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def dev(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a).to(DEV)


def both(g):
    """(no-alloc result, existing entry point's result) on the same inputs, float64 [batch, n]."""
    args = (ubw.pack_bases(dev(g.bits), g.nb, g.n, g.k), dev(g.alpha_r), dev(g.alpha_c), dev(g.idx),
            ubw.pack_bases(dev(g.bits_s), g.ns, g.n, g.s), dev(g.alpha_r_s), dev(g.alpha_c_s), dev(g.x))
    y0 = torch.full((g.x.shape[0], g.n), float("nan"), device=DEV)
    ubw.lut_gemv_refined_noalloc(*args, g.n, g.k, y0)
    ref = ubw.lut_gemv_refined(*args, g.n, g.k, workspace=ubw.workspace(g.n, DEV))
    torch.cuda.synchronize()
    return y0.cpu().numpy().astype(np.float64), ref.cpu().numpy().astype(np.float64)


def max_rel_err(y, r):
    floor = 1e-3 * np.max(np.abs(r), axis=-1, keepdims=True)
    return float(np.max(np.abs(y - r) / np.maximum(np.maximum(np.abs(r), floor), 1e-30)))


def test_noalloc_matches_workspace_entry_point_two_calls():
    rng = np.random.default_rng(31)
    # first call: the 4096 x 4096 step shape with 205 salient columns (integer-valued: exact)
    a, r = both(make_integer_gemv(rng, 4096, 4096, 2, s=205, ns=2, batch=1))
    assert np.array_equal(a, r)
    # second call, smaller and ragged (fewer row groups than the first left counters for), floats
    a, r = both(make_gemv(rng, "small", 700, 1500, 2, s=70, ns=2, batch=3))
    assert max_rel_err(a, r) <= 1e-3
    assert ubw.workspace_check(None) == (ubw.UBW_OK, 0)


def test_noalloc_rejects_rows_beyond_its_workspace():
    rng = np.random.default_rng(32)
    g = make_integer_gemv(rng, 65537, 64, 1, s=8, ns=1, batch=1)
    packed = torch.zeros(ubw.packed_words(1, g.n, g.k), dtype=torch.int32, device=DEV)
    packed_s = torch.zeros(ubw.packed_words(1, g.n, g.s), dtype=torch.int32, device=DEV)
    y = torch.zeros((1, g.n), device=DEV)
    with pytest.raises(ubw.UbwError) as e:
        ubw.lut_gemv_refined_noalloc(packed, dev(g.alpha_r), dev(g.alpha_c), dev(g.idx), packed_s, dev(g.alpha_r_s),
                                     dev(g.alpha_c_s), dev(g.x), g.n, g.k, y)
    assert e.value.status == -4
