"""GPU parity of the group-width-4 GEMV (whole rows per workgroup) against the CPU oracle.

Same bars as the group-8 tests: bit-exact on integer-valued inputs (unit scales, small integer
activations: every partial sum is an integer below 2**24, so any fp32 order is exact), the
elementwise relative error e <= 1e-3 on float inputs. The oracle's sum does not depend on the
group width (a table entry is the signed sum of its columns), so g = 4 and g = 8 are compared
with the same oracle, and with each other.
"""
import numpy as np
import pytest

import oracle
import ultra_bit_weight_uint32_amd as ubw
from workloads import Gemv, make_gemv, make_integer_gemv

from test_gpu_parity import DEV, TOL, dev, drop_positions, host, index_fault_cases, max_rel_err, oracle_gemv, pack

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run4(g, y=None, accumulate=False, mode="fused", ws=None, g_width=4):
    """The GEMV of a workloads.Gemv at group width 4: fused (main + refinement, one launch) or
    two calls (main, then the refinement accumulated); returns float64 [batch, n]."""
    x = dev(g.x)
    packed = pack(g.bits, g.k)
    if mode == "fused" and g.s:
        y = ubw.lut_gemv_refined(packed, dev(g.alpha_r), dev(g.alpha_c), dev(g.idx), pack(g.bits_s, g.s),
                                 dev(g.alpha_r_s), dev(g.alpha_c_s), x, g.n, g.k, g=g_width, y=y,
                                 accumulate=accumulate, workspace=ws)
    else:
        y = ubw.lut_gemv(packed, dev(g.alpha_r), dev(g.alpha_c), x, g.n, g.k, g=g_width, y=y,
                         accumulate=accumulate, workspace=ws)
        if g.s:
            ubw.vcm_gather_refine(dev(g.idx), pack(g.bits_s, g.s), dev(g.alpha_r_s), dev(g.alpha_c_s), x, g.n, g.k,
                                  y, g=g_width, workspace=ws)
    return host(y).astype(np.float64)


# (n, k, nb, s, ns): ragged rows (not a multiple of 16 or 256), K from 4 columns (one group) up
# to near the largest that fits (1 base: 6000; 2 bases: 4096), chunks of 1, 2, 4 and 8 words,
# and refinements of 1 to 4 bases over 1, 2 and 4 tiles (chunks of 8, 16 and 32 columns)
INT_CASES = [
    (1, 4, 1, 0, 0), (5, 32, 2, 1, 1), (17, 100, 1, 7, 2), (256, 256, 1, 40, 1), (300, 700, 2, 37, 2),
    (333, 1000, 4, 100, 4), (1000, 2048, 2, 205, 2), (513, 3000, 1, 500, 1), (4096, 4096, 2, 205, 2),
    (260, 6000, 1, 256, 1), (700, 4096, 1, 512, 1), (1, 4096, 2, 205, 2), (90, 2000, 1, 1000, 1),
]


@pytest.mark.parametrize("n,k,nb,s,ns", INT_CASES)
@pytest.mark.parametrize("batch", [1, 3, 16])
def test_g4_integer_exact(n, k, nb, s, ns, batch):
    rng = np.random.default_rng(n + 3 * k + 7 * nb + 11 * s + 100 * batch)
    g = make_integer_gemv(rng, n, k, nb, s=s, ns=ns, batch=batch)
    want = oracle_gemv(g)
    for mode in ("fused", "two_calls"):
        y = torch.full((batch, n), float("nan"), device=DEV)   # y = result ignores what y held
        assert np.array_equal(run4(g, y=y, mode=mode), want), mode


@pytest.mark.parametrize("x_dtype", [np.float16, np.float32])
def test_g4_integer_exact_fp32_and_fp16_activations(x_dtype):
    rng = np.random.default_rng(31)
    g = make_integer_gemv(rng, 999, 2500, 2, s=300, ns=2, batch=2, x_dtype=x_dtype)
    assert np.array_equal(run4(g), oracle_gemv(g))


def test_g4_accumulate():
    rng = np.random.default_rng(32)
    g = make_integer_gemv(rng, 700, 1500, 2, s=70, ns=1, batch=2)
    y0 = rng.integers(-100, 100, (2, 700)).astype(np.float32)
    for mode in ("fused", "two_calls"):
        assert np.array_equal(run4(g, y=dev(y0), accumulate=True, mode=mode), oracle_gemv(g) + y0), mode


def test_g4_matches_g8_and_needs_no_workspace():
    """Group widths 4 and 8 give the same exact result on the 4096 x 4096 step; g = 4 runs with
    or without a workspace (only its header word is used) and reports nothing on valid input."""
    rng = np.random.default_rng(33)
    g = make_integer_gemv(rng, 4096, 4096, 2, s=205, ns=2, batch=1)
    want = oracle_gemv(g)
    ws = torch.zeros(16, dtype=torch.int32, device=DEV)
    assert np.array_equal(run4(g, ws=ws), want)
    assert ubw.workspace_check(ws) == (ubw.UBW_OK, 0)
    assert np.array_equal(run4(g, g_width=8, ws=ubw.workspace(4096, DEV)), want)
    assert ubw.lut_gemv_workspace_bytes(2, 4096, 4096, g=4) == 64


@pytest.mark.parametrize("n,k,nb,s,ns,xdt", [
    (256, 512, 1, 0, 0, np.float32), (300, 700, 2, 37, 2, np.float16), (1024, 4096, 2, 205, 2, np.float16),
    (777, 332, 4, 50, 1, np.float32), (4096, 4096, 2, 205, 2, np.float16),
])
@pytest.mark.parametrize("batch", [1, 5])
def test_g4_float_tolerance(n, k, nb, s, ns, xdt, batch):
    rng = np.random.default_rng(n + k + batch + 1)
    g = make_gemv(rng, "f", n, k, nb, s=s, ns=ns, batch=batch, x_dtype=xdt)
    assert max_rel_err(run4(g), oracle_gemv(g)) <= TOL


def test_g4_headline_full_output_b1_and_b16():
    """The 4096 x 4096 step with 2 bases and 205 salient columns in 2 bases (fp16 x, alpha in
    [0.1, 1]): every output at batch 1 and 16 within the float bar, at both group widths."""
    for batch in (1, 16):
        rng = np.random.default_rng(34 + batch)
        g = make_gemv(rng, "headline", 4096, 4096, 2, s=205, ns=2, batch=batch, x_dtype=np.float16)
        want = oracle_gemv(g)
        assert max_rel_err(run4(g), want) <= TOL, batch
        assert max_rel_err(run4(g, g_width=8, ws=ubw.workspace(4096, DEV)), want) <= TOL, batch


@pytest.mark.parametrize("batch", [1, 4])
def test_g4_index_checks(batch):
    """Salient indices checked on the device at g = 4: outside [0, K) or not above the one before
    it sets bit 1 of the workspace header; a column outside [0, K) adds nothing, one out of order
    still adds its term."""
    rng = np.random.default_rng(35 + batch)
    n, k, s = 260, 900, 90
    g = make_integer_gemv(rng, n, k, 1, s=s, ns=2, batch=batch)
    for change, dropped, h in index_fault_cases(g, k, s):
        for mode in ("fused", "two_calls"):
            ws = torch.zeros(16, dtype=torch.int32, device=DEV)
            got = run4(h, mode=mode, ws=ws)
            st, word = ubw.workspace_check(ws, clear=True)
            assert st == ubw.UBW_ERANGE and word == 2, (change, mode, st, word)
            want = oracle_gemv(drop_positions(g, dropped)) if dropped else oracle_gemv(h)
            assert np.array_equal(got, want), (change, mode)


def test_g4_noalloc_matches_refined():
    rng = np.random.default_rng(36)
    for n, k, s, batch in ((4096, 4096, 205, 1), (700, 1500, 70, 3)):
        g = make_integer_gemv(rng, n, k, 2, s=s, ns=2, batch=batch)
        args = (pack(g.bits, k), dev(g.alpha_r), dev(g.alpha_c), dev(g.idx), pack(g.bits_s, s), dev(g.alpha_r_s),
                dev(g.alpha_c_s), dev(g.x), n, k)
        y = torch.full((batch, n), float("nan"), device=DEV)
        ubw.lut_gemv_refined_noalloc(*args, y, g=4)
        assert np.array_equal(host(y).astype(np.float64), oracle_gemv(g))
        assert ubw.workspace_check(None) == (ubw.UBW_OK, 0)


def test_g4_unsupported_shapes_raise():
    """Shapes whose group-4 tables do not fit one workgroup are refused on the host
    (UBW_EUNSUPPORTED), never switched to another width."""
    rng = np.random.default_rng(37)
    for n, k, nb in ((64, 8192, 2), (64, 8192, 1), (64, 100, 3)):
        g = make_integer_gemv(rng, n, k, nb, batch=1)
        with pytest.raises(ubw.UbwError) as e:
            ubw.lut_gemv(pack(g.bits, k), dev(g.alpha_r), dev(g.alpha_c), dev(g.x), n, k, g=4)
        assert e.value.status == ubw.UBW_EUNSUPPORTED


@pytest.mark.parametrize("x_dtype", [np.float16, np.float32])
@pytest.mark.parametrize("k", [64, 61])
def test_g4_unaligned_activations(x_dtype, k):
    """Activation rows that do not start on a 4-element boundary (x offset by one element, or K
    not a multiple of 4) are read one element at a time: same exact result."""
    rng = np.random.default_rng(38 + k)
    g = make_integer_gemv(rng, 300, k, 2, s=20, ns=1, batch=3, x_dtype=x_dtype)
    want = oracle_gemv(g)
    xbig = dev(np.concatenate([np.zeros(1, x_dtype), g.x.reshape(-1)]))
    x = xbig[1:].reshape(3, k)
    y = ubw.lut_gemv_refined(pack(g.bits, k), dev(g.alpha_r), dev(g.alpha_c), dev(g.idx), pack(g.bits_s, g.s),
                             dev(g.alpha_r_s), dev(g.alpha_c_s), x, g.n, k, g=4)
    assert np.array_equal(host(y).astype(np.float64), want)
    assert np.array_equal(run4(g), want)
