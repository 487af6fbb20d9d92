"""GPU parity: the HIP library (through its C ABI) against the CPU oracle, element by element.

Bars: bit-exact for pattern indices, packing and every integer-valued case (unit scales,
integer activations: all partial sums are integers below 2**24, so any fp32 summation order is
exact); for floating-point inputs the elementwise error
    e = max |y - r| / max(|r|, 1e-3 * max_row |r|)
must stay at or below 1e-3 (fp32 accumulation, fp16 activations).
"""
import numpy as np
import pytest

import oracle
import ultra_bit_weight_uint32_amd as ubw
from workloads import (Gemv, single_gemv_256x512, ternary_stack_256x768, attn_proj_7b, mlp_7b, decoder_layer_70b,
                       draw_bits, make_gemv, make_integer_gemv, words_per_row)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-3
DEV = "cuda:0"


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def max_rel_err(y, r):
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    floor = 1e-3 * np.max(np.abs(r), axis=-1, keepdims=True)
    den = np.maximum(np.abs(r), floor)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(y - r) / den))


def pack(bits, k):
    nb, n, _ = bits.shape
    return ubw.pack_bases(dev(bits), nb, n, k)


MODES = ("two_calls", "two_calls_ws", "fused", "fused_ws")


def gpu_gemv(g, packed=None, refine=True, y=None, accumulate=False, mode="fused_ws", ws=None):
    """Main GEMV (+ refinement) of a workloads.Gemv on the GPU; returns float64 [batch, n].
    mode: two calls (lut_gemv then vcm_gather_refine) or the single fused launch, each with a
    workspace (single launch also for y = result) or without one (zero-fill launch first)."""
    packed = pack(g.bits, g.k) if packed is None else packed
    x = dev(g.x)
    if mode.endswith("_ws") and ws is None:
        ws = ubw.workspace(g.n, DEV)
    elif not mode.endswith("_ws"):
        ws = None
    if mode.startswith("fused") and refine and g.s:
        y = ubw.lut_gemv_refined(packed, dev(g.alpha_r), dev(g.alpha_c), dev(g.idx), pack(g.bits_s, g.s),
                                 dev(g.alpha_r_s), dev(g.alpha_c_s), x, g.n, g.k, y=y, accumulate=accumulate,
                                 workspace=ws)
    else:
        y = ubw.lut_gemv(packed, dev(g.alpha_r), dev(g.alpha_c), x, g.n, g.k, y=y, accumulate=accumulate,
                         workspace=ws)
        if refine and g.s:
            ps = pack(g.bits_s, g.s)
            ubw.vcm_gather_refine(dev(g.idx), ps, dev(g.alpha_r_s), dev(g.alpha_c_s), x, g.n, g.k, y, workspace=ws)
    out = host(y).astype(np.float64)
    if ws is not None:
        word = int(host(ws)[0])
        assert word == 0, f"workspace error word {word:#x} (bit 0: a wait gave up, bit 1: a salient index)"
    return out


def oracle_gemv(g, refine=True):
    kw = g.refine_kwargs() if refine else {}
    return oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x, **kw)


# ------------------------------------------------------------------------------------------
# packing and pattern extraction (bit-exact)

SHAPES = [(1, 1), (7, 33), (256, 256), (300, 700), (513, 1000)]


@pytest.mark.parametrize("g_width", [8, 4])
@pytest.mark.parametrize("n,k", SHAPES)
def test_patterns_bit_exact(g_width, n, k):
    rng = np.random.default_rng(n * 1000 + k)
    bits = draw_bits(rng, 2, n, k)   # garbage past column K on purpose
    p = ubw.extract_patterns(pack(bits, k), 2, n, k, g=g_width)
    assert np.array_equal(host(p).view(np.uint16), oracle.patterns(bits, k, g=g_width))


def test_patterns_every_value_in_every_position():
    n, k = 512, 512
    ng = k // 8
    bits = np.zeros((1, n, words_per_row(k)), np.uint32)
    for r in range(n):
        big = 0
        for gi in range(ng):
            big |= ((7 * r + gi) % 256) << (8 * gi)
        for w in range(bits.shape[2]):
            bits[0, r, w] = (big >> (32 * w)) & 0xFFFFFFFF
    p = host(ubw.extract_patterns(pack(bits, k), 1, n, k)).view(np.uint16)
    want = (7 * np.arange(n)[:, None] + np.arange(ng)[None, :]) % 256
    assert np.array_equal(p[0], want)


@pytest.mark.parametrize("n,k", [(5, 40), (300, 700)])
def test_pack_from_int8_signs_matches_canonical(n, k):
    rng = np.random.default_rng(3)
    bits = draw_bits(rng, 3, n, k)
    by = bits.view(np.uint8).reshape(3, n, -1)
    signs = (np.unpackbits(by, axis=2, bitorder="little")[:, :, :k].astype(np.int8) * 2 - 1)
    a = host(pack(bits, k))
    b = host(ubw.pack_bases(dev(signs), 3, n, k))
    assert np.array_equal(a, b)


# ------------------------------------------------------------------------------------------
# LUT-BSF tables

@pytest.mark.parametrize("g_width", [8, 4])
def test_build_lut_integer_exact(g_width):
    rng = np.random.default_rng(4)
    k = 300
    x = rng.integers(-8, 9, (3, k)).astype(np.float16)
    ac = np.ones((2, k), np.float32)
    T = host(ubw.build_lut(dev(x), dev(ac), g=g_width))
    assert np.array_equal(T.astype(np.float64), oracle.lut_tables(x, ac, g=g_width))


@pytest.mark.parametrize("g_width", [8, 4])
@pytest.mark.parametrize("xdt", [np.float16, np.float32])
def test_build_lut_float(g_width, xdt):
    rng = np.random.default_rng(5)
    k = 777
    x = rng.standard_normal((2, k)).astype(xdt)
    ac = rng.uniform(0.05, 0.5, (3, k)).astype(np.float32)
    T = host(ubw.build_lut(dev(x), dev(ac), g=g_width)).astype(np.float64)
    R = oracle.lut_tables(x, ac, g=g_width)
    ng = R.shape[2]
    v = np.abs(ac[None].astype(np.float64) * x[:, None].astype(np.float64))
    v = np.concatenate([v, np.zeros((2, 3, ng * g_width - k))], axis=2).reshape(2, 3, ng, g_width)
    bound = 16 * 2.0 ** -24 * v.sum(-1, keepdims=True)   # fp32 rounding of v and of the sums
    assert np.all(np.abs(T - R) <= bound)


# ------------------------------------------------------------------------------------------
# main GEMV

INT_SHAPES = [(1, 1, 1), (5, 33, 2), (256, 256, 1), (300, 700, 3), (1000, 2050, 2), (4096, 4096, 2)]


@pytest.mark.parametrize("n,k,nb", INT_SHAPES)
@pytest.mark.parametrize("batch", [1, 3, 16])
def test_gemv_integer_exact(n, k, nb, batch):
    rng = np.random.default_rng(n + 7 * k + nb + 100 * batch)
    g = make_integer_gemv(rng, n, k, nb, batch=batch)
    for mode in ("two_calls", "two_calls_ws"):
        assert np.array_equal(gpu_gemv(g, mode=mode), oracle_gemv(g)), mode


@pytest.mark.parametrize("rpg", [1, 2, 4])
@pytest.mark.parametrize("wgs", [1, 2, 3, 5, 7, 0, 100000])
def test_gemv_geometries_integer_exact(rpg, wgs):
    """Every split of the unit list over workgroups gives the same exact result (5 row tiles x
    7 column slices, both ragged; 1, 2, 3 bases), overwriting NaN garbage or accumulating."""
    rng = np.random.default_rng(rpg * 10 + wgs % 97)
    n, k = 4 * 256 + 100, 6 * 256 + 77
    for nb in (1, 2, 3):
        g = make_integer_gemv(rng, n, k, nb, batch=1)
        packed = pack(g.bits, k)
        for ws in (None, ubw.workspace(n, DEV)):
            y = torch.full((1, n), float("nan"), device=DEV)
            ubw.lut_gemv_geometry(packed, dev(g.alpha_r), dev(g.alpha_c), dev(g.x), n, k, y,
                                  rows_per_group=rpg, workgroups=wgs, workspace=ws)
            assert np.array_equal(host(y).astype(np.float64), oracle_gemv(g)), (nb, ws is None)
            if ws is not None:
                assert host(ws)[0] == 0
        y0 = rng.integers(-50, 50, (1, n)).astype(np.float32)
        y = dev(y0)
        ubw.lut_gemv_geometry(packed, dev(g.alpha_r), dev(g.alpha_c), dev(g.x), n, k, y, accumulate=True,
                              rows_per_group=rpg, workgroups=wgs)
        assert np.array_equal(host(y).astype(np.float64), oracle_gemv(g) + y0)


@pytest.mark.parametrize("batch", [2, 4, 8, 16])
def test_gemv_geometries_batched(batch):
    rng = np.random.default_rng(batch)
    n, k = 3 * 256 + 5, 3 * 256 + 1
    g = make_integer_gemv(rng, n, k, 3, batch=batch)
    for rpg in (1, 2):
        for wgs in (1, 4, 0):
            y = torch.zeros((batch, n), device=DEV)
            ubw.lut_gemv_geometry(pack(g.bits, k), dev(g.alpha_r), dev(g.alpha_c), dev(g.x), n, k, y,
                                  rows_per_group=rpg, workgroups=wgs, workspace=ubw.workspace(n, DEV))
            assert np.array_equal(host(y).astype(np.float64), oracle_gemv(g))


@pytest.mark.parametrize("mode", MODES)
def test_gemv_accumulate(mode):
    rng = np.random.default_rng(11)
    g = make_integer_gemv(rng, 700, 1500, 2, s=70, ns=1, batch=2)
    y0 = rng.integers(-100, 100, (2, 700)).astype(np.float32)
    out = gpu_gemv(g, y=dev(y0), accumulate=True, mode=mode)
    assert np.array_equal(out, oracle_gemv(g) + y0)


@pytest.mark.parametrize("mode", MODES)
def test_overwrite_ignores_previous_contents(mode):
    """y = result must not depend on what y held (NaN garbage here)."""
    rng = np.random.default_rng(13)
    g = make_integer_gemv(rng, 900, 3000, 2, s=100, ns=2, batch=3)
    y = torch.full((3, 900), float("nan"), device=DEV)
    assert np.array_equal(gpu_gemv(g, y=y, mode=mode), oracle_gemv(g))


def test_workspace_reused_across_shapes_and_calls():
    """One workspace, many calls of different shapes back to back on one stream: the row-group
    counters stay consistent (every result exact, error word zero)."""
    rng = np.random.default_rng(14)
    ws = ubw.workspace(5000, DEV)
    cases = [make_integer_gemv(rng, n, k, nb, s=s, ns=ns, batch=b)
             for n, k, nb, s, ns, b in ((5000, 2000, 2, 90, 2, 1), (300, 700, 1, 0, 0, 2), (4096, 4096, 2, 205, 2, 1),
                                        (1000, 2600, 3, 33, 1, 4), (5000, 600, 2, 300, 2, 16))]
    for rep in range(3):
        for g in cases:
            mode = "fused_ws" if g.s else "two_calls_ws"
            assert np.array_equal(gpu_gemv(g, mode=mode, ws=ws), oracle_gemv(g)), (rep, g.n, g.k)


def test_one_hot_reads_signs():
    """alpha = 1, x = e_j: y is column j of B as +-1 (sign convention end to end)."""
    rng = np.random.default_rng(12)
    n, k = 256, 512
    bits = draw_bits(rng, 1, n, k)
    packed = pack(bits, k)
    by = bits.view(np.uint8).reshape(1, n, -1)
    signs = np.unpackbits(by, axis=2, bitorder="little")[0, :, :k].astype(np.float64) * 2 - 1
    xs = np.eye(k, dtype=np.float16)
    ar, ac = dev(np.ones((1, n), np.float32)), dev(np.ones((1, k), np.float32))
    for j0 in range(0, k, 16):   # 16 one-hot vectors per call as a batch
        y = ubw.lut_gemv(packed, ar, ac, dev(xs[j0:j0 + 16]), n, k)
        assert np.array_equal(host(y).astype(np.float64), signs[:, j0:j0 + 16].T)


@pytest.mark.parametrize("n,k,nb,xdt", [(256, 512, 1, np.float32), (300, 700, 2, np.float16),
                                        (1024, 4096, 3, np.float16), (777, 333, 2, np.float32)])
@pytest.mark.parametrize("batch", [1, 5])
def test_gemv_float_tolerance(n, k, nb, xdt, batch):
    rng = np.random.default_rng(n + k + batch)
    g = make_gemv(rng, "f", n, k, nb, batch=batch, x_dtype=xdt)
    assert max_rel_err(gpu_gemv(g), oracle_gemv(g)) <= TOL


# ------------------------------------------------------------------------------------------
# salient refinement (VCM)

@pytest.mark.parametrize("k,s", [(64, 1), (700, 37), (4096, 205), (1000, 300), (2000, 1434)])
@pytest.mark.parametrize("batch", [1, 4])
@pytest.mark.parametrize("ns", [1, 2, 3])
def test_vcm_integer_exact(k, s, batch, ns):
    rng = np.random.default_rng(k + s + batch + 10 * ns)
    g = make_integer_gemv(rng, 300, k, 2, s=s, ns=ns, batch=batch)
    for mode in MODES:
        assert np.array_equal(gpu_gemv(g, mode=mode), oracle_gemv(g)), mode


def test_vcm_geometries_integer_exact():
    n, k, s = 600, 3000, 700
    for batch, rpg, wgs in ((2, 1, 0), (2, 1, 1), (2, 1, 3), (1, 2, 3), (1, 2, 0), (1, 4, 5), (1, 1, 7), (2, 2, 0),
                            (3, 2, 3), (7, 2, 0)):
        rng = np.random.default_rng(21 + batch)
        g = make_integer_gemv(rng, n, k, 1, s=s, ns=2, batch=batch)
        ps = pack(g.bits_s, s)
        want = oracle_gemv(g) - oracle_gemv(g, refine=False)
        y = torch.zeros((batch, n), device=DEV)
        ubw.lut_gemv_geometry(ps, dev(g.alpha_r_s), dev(g.alpha_c_s), dev(g.x), n, s, y, idx=dev(g.idx), k=k,
                              accumulate=True, rows_per_group=rpg, workgroups=wgs)
        assert np.array_equal(host(y).astype(np.float64), want), (batch, rpg, wgs)
        y = torch.full((batch, n), float("nan"), device=DEV)
        ubw.lut_gemv_geometry(ps, dev(g.alpha_r_s), dev(g.alpha_c_s), dev(g.x), n, s, y, idx=dev(g.idx), k=k,
                              accumulate=False, rows_per_group=rpg, workgroups=wgs,
                              workspace=ubw.workspace(n, DEV))
        assert np.array_equal(host(y).astype(np.float64), want), (batch, rpg, wgs)


def test_vcm_every_column_salient_doubles():
    rng = np.random.default_rng(22)
    n, k = 300, 500
    g = make_integer_gemv(rng, n, k, 2, batch=2)
    x = dev(g.x)
    packed = pack(g.bits, k)
    y = ubw.lut_gemv(packed, dev(g.alpha_r), dev(g.alpha_c), x, n, k)
    y1 = host(y).copy()
    ubw.vcm_gather_refine(dev(np.arange(k, dtype=np.int32)), packed, dev(g.alpha_r), dev(g.alpha_c), x, n, k, y)
    assert np.array_equal(host(y), 2 * y1)


def drop_positions(g, positions):
    """The same problem with the refinement columns at `positions` contributing nothing (their
    alpha_c_s set to 0; the index list itself is left alone)."""
    h = Gemv(**{f: getattr(g, f) for f in g.__dataclass_fields__})
    h.alpha_c_s = g.alpha_c_s.copy()
    h.alpha_c_s[:, list(positions)] = 0.0
    return h


@pytest.mark.parametrize("batch,k", [(1, 900), (3, 900), (9, 900), (1, 904), (2, 904)])
def test_vcm_index_checks(batch, k):
    """Salient indices are checked on the device: an index outside [0, K) or not above the one
    before it is reported in workspace word 0 (UBW_ERANGE); a column outside [0, K) contributes
    nothing, one out of order still adds its term (the oracle's sum takes any order); a valid
    list reports nothing. Batch 9 runs on the matrix cores, 1 to 3 on the tables: with K = 900
    the activation block (1800 or 5400 bytes, not a multiple of 16) is gathered from memory
    through idx one unit after idx is loaded; with K = 904 (1808 or 3616 bytes) the whole block
    is staged in LDS and gathered there."""
    rng = np.random.default_rng(23 + batch + k)
    n, s = 260, 90
    g = make_integer_gemv(rng, n, k, 1, s=s, ns=2, batch=batch)
    ok_ws = ubw.workspace(n, DEV)
    want = oracle_gemv(g)
    assert np.array_equal(gpu_gemv(g, ws=ok_ws), want)
    assert ubw.workspace_check(ok_ws) == (ubw.UBW_OK, 0)
    for change, dropped, h in index_fault_cases(g, k, s):
        for mode in ("fused_ws", "two_calls_ws"):
            ws = ubw.workspace(n, DEV)
            x = dev(h.x)
            if mode == "fused_ws":
                y = ubw.lut_gemv_refined(pack(h.bits, k), dev(h.alpha_r), dev(h.alpha_c), dev(h.idx), pack(h.bits_s, s),
                                         dev(h.alpha_r_s), dev(h.alpha_c_s), x, n, k, workspace=ws)
            else:
                y = ubw.lut_gemv(pack(h.bits, k), dev(h.alpha_r), dev(h.alpha_c), x, n, k, workspace=ws)
                ubw.vcm_gather_refine(dev(h.idx), pack(h.bits_s, s), dev(h.alpha_r_s), dev(h.alpha_c_s), x, n, k, y,
                                      workspace=ws)
            st, word = ubw.workspace_check(ws, clear=True)
            assert st == ubw.UBW_ERANGE and word == 2, (change, mode, st, word)
            assert ubw.workspace_check(ws) == (ubw.UBW_OK, 0)
            want = oracle_gemv(drop_positions(g, dropped)) if dropped else oracle_gemv(h)
            assert np.array_equal(host(y).astype(np.float64), want), (change, mode)


def index_fault_cases(g, k, s):
    """(change, dropped positions, changed problem) for each index fault: out of range (the
    position is dropped: the expected result is the original problem with its alpha_c_s zeroed
    there) or out of order (nothing dropped: the expected result is the changed problem)."""
    cases = [
        ({0: -1}, [0]),                                 # below 0
        ({s - 1: k}, [s - 1]),                          # at K
        ({s - 1: 2**31 - 1}, [s - 1]),                  # far beyond K
        ({40: int(g.idx[39])}, []),                     # repeats the one before
        ({40: int(g.idx[39]) - 1 if g.idx[39] > 0 else 0, 41: int(g.idx[41])}, []),  # goes down
    ]
    for change, dropped in cases:
        h = Gemv(**{f: getattr(g, f) for f in g.__dataclass_fields__})
        h.idx = g.idx.copy()
        for q, v in change.items():
            h.idx[q] = v
        yield change, dropped, h


def test_progress_beyond_device_capacity():
    """y = result with more workgroups than the device holds at once (1024 single-unit
    workgroups for 16 row groups): a workgroup only ever waits for the first arriver of its row
    group, which is already running, so the launch completes and every result is exact."""
    rng = np.random.default_rng(24)
    n, k = 4096, 16384
    g = make_integer_gemv(rng, n, k, 2, batch=1)
    packed = pack(g.bits, k)
    ws = ubw.workspace(n, DEV)
    want = oracle_gemv(g)
    for wgs in (100000, 700, 513):
        y = torch.full((1, n), float("nan"), device=DEV)
        ubw.lut_gemv_geometry(packed, dev(g.alpha_r), dev(g.alpha_c), dev(g.x), n, k, y, rows_per_group=1,
                              workgroups=wgs, workspace=ws)
        assert np.array_equal(host(y).astype(np.float64), want), wgs
        assert ubw.workspace_check(ws) == (ubw.UBW_OK, 0), wgs


def test_workspace_error_word_decoding():
    """The workspace error word as ubw_workspace_check reports it, bits written from the host (no
    wait is made to run out): bit 0 -> UBW_EWAIT (a wait gave up; it wins over bit 1), bit 1 ->
    UBW_ERANGE, clear=True zeroes the word; a valid GEMV into that workspace leaves a set bit as
    it is (the word is sticky until cleared) and still writes the right y."""
    rng = np.random.default_rng(91)
    g = make_integer_gemv(rng, 777, 900, 2, s=45, ns=1, batch=1)
    ws = ubw.workspace(777, DEV)
    for word, status in ((1, ubw.UBW_EWAIT), (2, ubw.UBW_ERANGE), (3, ubw.UBW_EWAIT)):
        ws[0] = word
        assert ubw.workspace_check(ws) == (status, word)
        assert ubw.workspace_check(ws, clear=True) == (status, word)
        assert ubw.workspace_check(ws) == (ubw.UBW_OK, 0)
    ws[0] = 2
    y = ubw.lut_gemv_refined(pack(g.bits, g.k), dev(g.alpha_r), dev(g.alpha_c), dev(g.idx), pack(g.bits_s, g.s),
                             dev(g.alpha_r_s), dev(g.alpha_c_s), dev(g.x), g.n, g.k,
                             y=torch.full((1, 777), float("nan"), device=DEV), workspace=ws)
    assert np.array_equal(host(y).astype(np.float64), oracle_gemv(g))
    assert ubw.workspace_check(ws, clear=True) == (ubw.UBW_ERANGE, 2)
    assert ubw.workspace_check(ws) == (ubw.UBW_OK, 0)


def test_concurrent_streams_separate_workspaces():
    """Two streams, each with its own workspace, issue full-device y = result launches at the same
    time: the 4096 x 4096 step (2 bases + 205 salient columns) and a 70B gate (28672 x 8192,
    3 bases + 1434 salient columns); integer-valued inputs, so every output of every launch must
    equal the oracle exactly."""
    rng = np.random.default_rng(25)
    gs = [make_integer_gemv(rng, 4096, 4096, 2, s=205, ns=2, batch=1),
          make_integer_gemv(rng, 28672, 8192, 3, s=1434, ns=2, batch=1)]
    wants = [oracle_gemv(g) for g in gs]
    args = []
    for g in gs:
        args.append(dict(packed=pack(g.bits, g.k), ar=dev(g.alpha_r), ac=dev(g.alpha_c), idx=dev(g.idx),
                         ps=pack(g.bits_s, g.s), ars=dev(g.alpha_r_s), acs=dev(g.alpha_c_s), x=dev(g.x),
                         ws=ubw.workspace(g.n, DEV)))
    reps = 60
    outs = [[torch.full((1, g.n), float("nan"), device=DEV) for _ in range(reps)] for g in gs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    torch.cuda._sleep(20_000_000)  # both streams start together once this ends
    gate = torch.cuda.Event()
    gate.record()
    for st in streams:
        st.wait_event(gate)
    for r in range(reps):
        for i, (g, a) in enumerate(zip(gs, args)):
            with torch.cuda.stream(streams[i]):
                ubw.lut_gemv_refined(a["packed"], a["ar"], a["ac"], a["idx"], a["ps"], a["ars"], a["acs"], a["x"],
                                     g.n, g.k, y=outs[i][r], workspace=a["ws"])
    torch.cuda.synchronize()
    for i, g in enumerate(gs):
        with torch.cuda.stream(streams[i]):
            assert ubw.workspace_check(args[i]["ws"]) == (ubw.UBW_OK, 0), g.n
        got = torch.cat(outs[i]).cpu().numpy().astype(np.float64)
        bad = np.flatnonzero(np.any(got != wants[i], axis=1))
        assert bad.size == 0, f"{g.n} x {g.k}: launches {bad[:10].tolist()} differ from the oracle"


@pytest.mark.parametrize("batch", [1, 3])
def test_vcm_float_tolerance(batch):
    rng = np.random.default_rng(24 + batch)
    g = make_gemv(rng, "v", 1000, 3000, 2, s=150, ns=2, batch=batch)
    assert max_rel_err(gpu_gemv(g), oracle_gemv(g)) <= TOL


# ------------------------------------------------------------------------------------------
# ternary weights as two half-scale bases

def test_ternary_encode_patterns_match_oracle_encoding():
    rng = np.random.default_rng(30)
    n, k = 300, 520
    w = rng.integers(-1, 2, (n, k)).astype(np.int8)
    packed, ar, ac = ubw.ternary_encode(dev(w), dev(np.ones(n, np.float32)))
    want = oracle.patterns(oracle.ternary_encode(w, zero_first_plus=True), k)
    assert np.array_equal(host(ubw.extract_patterns(packed, 2, n, k)).view(np.uint16), want)
    assert np.array_equal(host(ar), np.full((2, n), 0.5, np.float32))
    assert np.array_equal(host(ac), np.ones((2, k), np.float32))


def test_ternary_gemv_integer_exact():
    rng = np.random.default_rng(31)
    n, k = 768, 256
    w = rng.integers(-1, 2, (n, k)).astype(np.int8)
    x = rng.integers(-8, 9, (4, k)).astype(np.float16)
    packed, ar, ac = ubw.ternary_encode(dev(w), dev(np.full(n, 2.0, np.float32)))
    y = ubw.lut_gemv(packed, ar, ac, dev(x), n, k)
    assert np.array_equal(host(y).astype(np.float64), oracle.ternary_gemv(w, np.full(n, 2.0, np.float32), x))


def test_ternary_stack_chained():
    """4 x (256 -> 768 -> 256) ternary layers over 64 tokens, fp16 activations between layers.
    Every layer is checked on the GPU's own fp16 input (teacher forcing) at the elementwise 1e-3
    bar. The end-to-end output is compared with the oracle's own chain norm-wise: the two chains
    re-round slightly different fp32 results to fp16 after each of the 8 layers, so outputs
    near zero can differ by more than 1e-3 of themselves while the row stays within ~1e-4 of
    its largest entry."""
    wl = ternary_stack_256x768()
    enc = [ubw.ternary_encode(dev(L.w), dev(L.scale)) for L in wl.ternary]
    xt = dev(wl.tokens)
    worst = 0.0
    for t in range(wl.tokens.shape[0]):
        a = xt[t:t + 1]
        for L, (packed, ar, ac) in zip(wl.ternary, enc):
            n, k = L.w.shape
            y = ubw.lut_gemv(packed, ar, ac, a, n, k)
            r = oracle.ternary_gemv(L.w, L.scale, host(a))
            worst = max(worst, max_rel_err(host(y), r))
            a = y.to(torch.float16)
    assert worst <= TOL
    # end to end, 16 tokens per call (the batch limit of one call)
    for t0 in range(0, wl.tokens.shape[0], ubw.MAX_BATCH):
        a_gpu = xt[t0:t0 + ubw.MAX_BATCH]
        a_ref = wl.tokens[t0:t0 + ubw.MAX_BATCH].astype(np.float64)
        for L, (packed, ar, ac) in zip(wl.ternary, enc):
            n, k = L.w.shape
            a_gpu = ubw.lut_gemv(packed, ar, ac, a_gpu, n, k).to(torch.float16)
            a_ref = oracle.ternary_gemv(L.w, L.scale, a_ref).astype(np.float16).astype(np.float64)
        d = np.abs(host(a_gpu).astype(np.float64) - a_ref).max(axis=1) / np.abs(a_ref).max(axis=1)
        assert d.max() <= 1e-2


# ------------------------------------------------------------------------------------------
# the workloads at full size, in the launch configuration the benchmark uses

def test_single_gemv_256x512_full():
    g = single_gemv_256x512().gemvs[0]
    assert max_rel_err(gpu_gemv(g), oracle_gemv(g)) <= TOL


@pytest.mark.parametrize("mode", MODES)
def test_attn_proj_7b_full(mode):
    g = attn_proj_7b().gemvs[0]
    assert max_rel_err(gpu_gemv(g, mode=mode), oracle_gemv(g)) <= TOL
    assert max_rel_err(gpu_gemv(g, refine=False, mode=mode), oracle_gemv(g, refine=False)) <= TOL


def test_mlp_7b_full():
    wl = mlp_7b()
    for g in wl.gemvs:
        for b in wl.batches:
            gb = g.with_batch(b)
            assert max_rel_err(gpu_gemv(gb), oracle_gemv(gb)) <= TOL, (g.name, b)


def test_large_matrix_five_and_six_rows():
    """5 and 6 rows on the 70B gate shape (3 bases of 28672 x 8192: the matrix cores) and on
    8192 x 8192 with 3 bases (tables at 5 rows, matrix cores at 6): every output against the
    oracle."""
    rng = np.random.default_rng(56)
    for name, n, k in (("gate", 28672, 8192), ("q", 8192, 8192)):
        g = make_gemv(rng, name, n, k, 3, s=410, ns=2, batch=6)
        for b in (5, 6):
            gb = g.with_batch(b)
            assert max_rel_err(gpu_gemv(gb), oracle_gemv(gb)) <= TOL, (name, b)


@pytest.mark.parametrize("name,n,k,nb,s,batches", [
    ("7B up", 11008, 4096, 2, 205, (7, 8)),        # tables at 7 rows, matrix cores at 8
    ("4096 sq", 4096, 4096, 2, 205, (8, 9)),       # tables at 8, matrix cores at 9
    ("70B k", 1024, 8192, 3, 410, (8, 9)),         # tables at 8, matrix cores at 9
])
def test_path_model_crossovers(name, n, k, nb, s, batches):
    """Each side of the path model's crossover for three shapes (the batch before it runs on the
    tables, the batch at it on the matrix cores): every output against the oracle, with salient
    refinement, y = result through the workspace."""
    rng = np.random.default_rng(n + k + nb)
    g = make_gemv(rng, name, n, k, nb, s=s, ns=2, batch=max(batches))
    for b in batches:
        gb = g.with_batch(b)
        assert max_rel_err(gpu_gemv(gb), oracle_gemv(gb)) <= TOL, (name, b)


def test_decoder_layer_70b_full():
    """Every output of all seven 70B-shaped GEMVs (q/k/v/o, gate/up/down; 3 bases + 5% salient
    columns in 2 bases) at batch 1 (tables) and 16 (matrix cores) against the oracle."""
    wl = decoder_layer_70b()
    for g in wl.gemvs:
        for b in wl.batches:
            gb = g.with_batch(b)
            assert max_rel_err(gpu_gemv(gb), oracle_gemv(gb)) <= TOL, (g.name, b)


def test_matrix_cores_against_tables_within_bound():
    """16 activation rows on the matrix cores against the same product on the tables (explicit
    table geometry), every output, within the bound that follows from the arithmetic:
      representation: both paths form v = alpha_c x in fp32 (|err| <= 2^-24 |v|); the matrix
        cores then split v into fp16 hi + lo, |v - hi - lo| < 2^-20 |v| + 2^-38 m (m: the largest
        |v| of the row's 256-column slice);
      summation: fp32 sums of n terms err by at most gamma(n) = n u / (1 - n u), u = 2^-24, times
        the sum of the terms' magnitudes; n <= 514 + nb ceil(K / 256) on the matrix cores (two
        chained 256-term slice sums, the alpha_r product, the hi/lo columns, one add per slice
        and base) and n <= 41 + nb ceil(K / 256) on the tables (table entries of 8 terms, 32
        lookups per lane, the half-wave combine, the alpha_r product, one add per unit).
    With S = sum_k |alpha_r^k| sum_j |v_kj| and M = sum_k |alpha_r^k| sum_slices 256 m, the two
    results differ by at most (2^-20 + 2 u + gamma(n_mfma) + gamma(n_tab)) S + 2^-38 M."""
    rng = np.random.default_rng(57)
    n, k, nb, b = 1000, 4100, 3, 16
    g = make_gemv(rng, "bound", n, k, nb, batch=b, x_dtype=np.float16)
    packed = pack(g.bits, k)
    ym = host(ubw.lut_gemv(packed, dev(g.alpha_r), dev(g.alpha_c), dev(g.x), n, k)).astype(np.float64)
    yt = torch.zeros((b, n), device=DEV)
    ubw.lut_gemv_geometry(packed, dev(g.alpha_r), dev(g.alpha_c), dev(g.x), n, k, yt, rows_per_group=1,
                          workspace=ubw.workspace(n, DEV))
    yt = host(yt).astype(np.float64)
    v = np.abs(g.alpha_c[None].astype(np.float64) * g.x.astype(np.float64)[:, None])     # [b, nb, k]
    ar = np.abs(g.alpha_r.astype(np.float64))                                              # [nb, n]
    S = np.einsum("kr,bk->br", ar, v.sum(-1))
    kt = -(-k // 256)
    vp = np.concatenate([v, np.zeros((b, nb, kt * 256 - k))], -1).reshape(b, nb, kt, 256)
    M = np.einsum("kr,bk->br", ar, 256 * vp.max(-1).sum(-1))
    u = 2.0 ** -24
    gamma = lambda m: m * u / (1 - m * u)
    bound = (2.0 ** -20 + 2 * u + gamma(514 + nb * kt) + gamma(41 + nb * kt)) * S + 2.0 ** -38 * M
    diff = np.abs(ym - yt)
    assert np.all(diff <= bound), float(np.max(diff / bound))
    assert max_rel_err(ym, oracle_gemv(g)) <= TOL and max_rel_err(yt, oracle_gemv(g)) <= TOL


# ------------------------------------------------------------------------------------------
# grouped launches: several GEMVs on one x in one launch

def multi_entry(g, ws=True, y=None):
    e = dict(packed=pack(g.bits, g.k), alpha_r=dev(g.alpha_r), alpha_c=dev(g.alpha_c), n=g.n,
             y=torch.full((g.batch, g.n), float("nan"), device=DEV) if y is None else y)
    if g.s:
        e.update(idx=dev(g.idx), packed_s=pack(g.bits_s, g.s), alpha_r_s=dev(g.alpha_r_s),
                 alpha_c_s=dev(g.alpha_c_s))
    if ws:
        e["workspace"] = ubw.workspace(g.n, DEV)
    return e


def shared_x(gs, x):
    for g in gs:
        g.x = x
    return gs


@pytest.mark.parametrize("batch", [1, 3, 8, 16])
def test_multi_integer_exact(batch):
    """Mixed GEMVs (row counts from 5 to 1100, 1 to 3 bases, with and without refinement) on one
    x: every output exact, written over NaN or added to, with and without workspaces."""
    rng = np.random.default_rng(300 + batch)
    k = 1504   # fp16 x of 3008 bytes: the refinement gather goes through LDS at batch 1
    gs = [make_integer_gemv(rng, 700, k, 2, s=70, ns=1, batch=batch),
          make_integer_gemv(rng, 300, k, 1, batch=batch),
          make_integer_gemv(rng, 1100, k, 3, s=150, ns=2, batch=batch),
          make_integer_gemv(rng, 5, k, 2, s=3, ns=1, batch=batch)]
    shared_x(gs, rng.integers(-8, 9, size=(batch, k)).astype(np.float16))
    ref = [oracle_gemv(g) for g in gs]
    x = dev(gs[0].x)
    for ws in (True, False):
        es = [multi_entry(g, ws=ws) for g in gs]
        outs = ubw.lut_gemv_multi(es, x, k)
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert np.array_equal(host(o).astype(np.float64), r), (i, ws)
        for e in es:
            if ws:
                assert host(e["workspace"])[0] == 0
        y0 = [rng.integers(-50, 50, (batch, g.n)).astype(np.float32) for g in gs]
        for e, a in zip(es, y0):
            e["y"] = dev(a)
        outs = ubw.lut_gemv_multi(es, x, k, accumulate=True)
        for i, (o, r, a) in enumerate(zip(outs, ref, y0)):
            assert np.array_equal(host(o).astype(np.float64), r + a), (i, ws, "accumulate")


def test_multi_eight_gemvs_and_workspace_reuse():
    """UBW_MAX_GROUP GEMVs in one call, then the same workspaces in single calls and a second
    grouped call: the row-group counters stay consistent across calls of both kinds."""
    rng = np.random.default_rng(17)
    k = 777
    gs = [make_integer_gemv(rng, n, k, 1 + i % 3, s=(40 if i % 2 else 0), ns=(1 + i % 2 if i % 2 else 0))
          for i, n in enumerate((64, 1, 513, 256, 257, 900, 33, 1300))]
    shared_x(gs, rng.integers(-8, 9, size=(1, k)).astype(np.float16))
    ref = [oracle_gemv(g) for g in gs]
    x = dev(gs[0].x)
    es = [multi_entry(g) for g in gs]
    for rep in range(3):
        outs = ubw.lut_gemv_multi(es, x, k)
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert np.array_equal(host(o).astype(np.float64), r), (rep, i)
        for g, e in zip(gs, es):   # single calls on the same workspaces in between
            assert np.array_equal(gpu_gemv(g, packed=e["packed"], ws=e["workspace"]), oracle_gemv(g))
    for e in es:
        assert host(e["workspace"])[0] == 0


def test_multi_eight_gemvs_matrix_cores():
    """UBW_MAX_GROUP GEMVs at 12 rows: one matrix-core launch over all their row tiles (each GEMV
    with its own column split), exact, over NaN and accumulated, twice in a row."""
    rng = np.random.default_rng(19)
    k = 1300
    gs = [make_integer_gemv(rng, n, k, 1 + i % 3, s=(40 + 300 * (i % 4 == 1) if i % 2 else 0),
                            ns=(1 + i % 2 if i % 2 else 0), batch=12)
          for i, n in enumerate((64, 1, 513, 256, 257, 900, 33, 1300))]
    shared_x(gs, rng.integers(-8, 9, size=(12, k)).astype(np.float16))
    ref = [oracle_gemv(g) for g in gs]
    x = dev(gs[0].x)
    for ws in (True, False):
        es = [multi_entry(g, ws=ws) for g in gs]
        for rep in range(2):
            outs = ubw.lut_gemv_multi(es, x, k)
            for i, (o, r) in enumerate(zip(outs, ref)):
                assert np.array_equal(host(o).astype(np.float64), r), (ws, rep, i)
        y0 = [rng.integers(-50, 50, (12, g.n)).astype(np.float32) for g in gs]
        for e, a in zip(es, y0):
            e["y"] = dev(a)
        outs = ubw.lut_gemv_multi(es, x, k, accumulate=True)
        for i, (o, r, a) in enumerate(zip(outs, ref, y0)):
            assert np.array_equal(host(o).astype(np.float64), r + a), (ws, i, "accumulate")


def test_multi_matrix_cores_mixed_column_splits():
    """K = 200 at 9 rows: a GEMV without refinement has one slice (plain stores, its extra
    workgroups exit), one with refinement two (zero fill, then atomics), in one launch."""
    rng = np.random.default_rng(29)
    k = 200
    gs = [make_integer_gemv(rng, 300, k, 2, batch=9),
          make_integer_gemv(rng, 700, k, 3, s=50, ns=2, batch=9),
          make_integer_gemv(rng, 17, k, 1, batch=9)]
    shared_x(gs, rng.integers(-8, 9, size=(9, k)).astype(np.float16))
    ref = [oracle_gemv(g) for g in gs]
    es = [multi_entry(g, ws=False) for g in gs]
    outs = ubw.lut_gemv_multi(es, dev(gs[0].x), k)
    for i, (o, r) in enumerate(zip(outs, ref)):
        assert np.array_equal(host(o).astype(np.float64), r), i


def test_multi_single_gemv_matches_single_call():
    rng = np.random.default_rng(23)
    g = make_integer_gemv(rng, 1000, 3000, 3, s=150, ns=2, batch=1)
    out = ubw.lut_gemv_multi([multi_entry(g)], dev(g.x), g.k)[0]
    assert np.array_equal(host(out).astype(np.float64), oracle_gemv(g))


def test_multi_layer_70b_full():
    """70B-shaped q/k/v and gate/up groups on one shared fp16 x each (batch 1 and 16): every
    output against the oracle within the float tolerance."""
    wl = decoder_layer_70b()
    by = {g.name: g for g in wl.gemvs}
    for names in (("q", "k", "v"), ("gate", "up")):
        gs = shared_x([by[nm] for nm in names], by[names[0]].x)
        for b in wl.batches:
            gb = [g.with_batch(b) for g in gs]
            es = [multi_entry(g) for g in gb]
            outs = ubw.lut_gemv_multi(es, dev(gb[0].x), gb[0].k)
            for g, o in zip(gb, outs):
                assert max_rel_err(host(o).astype(np.float64), oracle_gemv(g)) <= TOL, (g.name, b)


# ------------------------------------------------------------------------------------------
# group-scale variant: one fp16 row scale per 128 columns

def gs_scales(rng, g, integer=True, pad_nan=True):
    """[nb, n, 2 ceil(k/256)] fp16 block scales; padding entries (blocks past column k) NaN,
    which the kernel must never read."""
    cols = ubw.group_scale_cols(g.k)
    if integer:
        a = rng.integers(1, 4, size=(g.nb, g.n, cols)).astype(np.float16)
    else:
        a = rng.uniform(0.05, 0.5, size=(g.nb, g.n, cols)).astype(np.float16)
    used = -(-g.k // 128)
    if pad_nan and used < cols:
        a[:, :, used:] = np.float16("nan")
    return a


def gpu_gs(g, arg, refine=True, y=None, accumulate=False, ws=True):
    kw = {}
    if refine and g.s:
        kw = dict(idx=dev(g.idx), packed_s=pack(g.bits_s, g.s), alpha_r_s=dev(g.alpha_r_s),
                  alpha_c_s=dev(g.alpha_c_s))
    w = ubw.workspace(g.n, DEV) if ws else None
    out = ubw.lut_gemv_gs(pack(g.bits, g.k), dev(ubw.arrange_group_scales(arg)), dev(g.alpha_c), dev(g.x), g.n,
                          g.k, y=y,
                          accumulate=accumulate, workspace=w, **kw)
    res = host(out).astype(np.float64)
    if w is not None:
        assert host(w)[0] == 0
    return res


def oracle_gs(g, arg, refine=True):
    kw = g.refine_kwargs() if refine else {}
    return oracle.gemv_gs(g.bits, arg, g.alpha_c, g.x, **kw)


GS_SHAPES = [(300, 700, 2, 0), (513, 1000, 3, 50), (256, 384, 1, 0), (100, 129, 2, 7), (1, 33, 1, 0),
             (700, 1500, 2, 70)]


@pytest.mark.parametrize("n,k,nb,s", GS_SHAPES)
@pytest.mark.parametrize("batch", [1, 3, 16])
def test_gs_integer_exact(n, k, nb, s, batch):
    rng = np.random.default_rng(n + 3 * k + 11 * nb + batch)
    g = make_integer_gemv(rng, n, k, nb, s=s, ns=(2 if s else 0), batch=batch)
    arg = gs_scales(rng, g)
    ref = oracle_gs(g, arg)
    for ws in (True, False):
        y = torch.full((batch, n), float("nan"), device=DEV)
        assert np.array_equal(gpu_gs(g, arg, y=y, ws=ws), ref), ws
    y0 = rng.integers(-50, 50, (batch, n)).astype(np.float32)
    assert np.array_equal(gpu_gs(g, arg, y=dev(y0), accumulate=True), ref + y0)


@pytest.mark.parametrize("rpg", [1, 2, 4])
def test_gs_geometries_integer_exact(rpg):
    rng = np.random.default_rng(40 + rpg)
    n, k = 4 * 256 + 100, 6 * 256 + 77
    for nb in (1, 2, 3):
        g = make_integer_gemv(rng, n, k, nb, batch=1)
        arg = gs_scales(rng, g)
        ref = oracle_gs(g, arg)
        for wgs in (1, 3, 7, 0):
            y = torch.full((1, n), float("nan"), device=DEV)
            ubw.lut_gemv_geometry(pack(g.bits, k), dev(ubw.arrange_group_scales(arg)), dev(g.alpha_c), dev(g.x), n,
                                  k, y, rows_per_group=rpg,
                                  workgroups=wgs, workspace=ubw.workspace(n, DEV), group_scales=True)
            assert np.array_equal(host(y).astype(np.float64), ref), (nb, wgs)


@pytest.mark.parametrize("batch", [1, 4])
def test_gs_float_tolerance(batch):
    """7B attention projection shape with 128-column fp16 group scales and the salient
    refinement, float scales and fp16 x, within the float tolerance."""
    rng = np.random.default_rng(90 + batch)
    g = make_gemv(rng, "gs", 4096, 4096, 2, s=205, ns=2, batch=batch)
    arg = gs_scales(rng, g, integer=False)
    assert max_rel_err(gpu_gs(g, arg), oracle_gs(g, arg)) <= TOL


def test_gs_equal_blocks_match_plain_gemv():
    """Equal block scales along each row: the same product as the per-row call (float)."""
    rng = np.random.default_rng(91)
    g = make_gemv(rng, "gs", 1000, 3000, 2, s=150, ns=1, batch=2)
    arg = np.repeat(g.alpha_r.astype(np.float16)[:, :, None], ubw.group_scale_cols(g.k), axis=2)
    g16 = make_gemv(rng, "gs", 1000, 3000, 2, s=150, ns=1, batch=2)
    g16.bits, g16.alpha_c, g16.x, g16.idx = g.bits, g.alpha_c, g.x, g.idx
    g16.bits_s, g16.alpha_r_s, g16.alpha_c_s = g.bits_s, g.alpha_r_s, g.alpha_c_s
    g16.alpha_r = g.alpha_r.astype(np.float16).astype(np.float32)
    assert max_rel_err(gpu_gs(g, arg), gpu_gemv(g16)) <= TOL


# ------------------------------------------------------------------------------------------
# offline fit (residual sign binarization + alternating least squares)

def fit_matrix(rng, n, k, dtype=np.float32):
    """Anisotropic dense matrix: N(0,1) entries times per-row and per-column magnitudes."""
    w = rng.standard_normal((n, k)) * rng.uniform(0.2, 3, (n, 1)) * rng.uniform(0.2, 3, (1, k))
    return w.astype(dtype)


def check_fit(w, nb, iters):
    wt = dev(w)
    bits, ar, ac, res = ubw.fit_bases(wt, nb, iters)
    bits, ar, ac, res = host(bits).view(np.uint32), host(ar), host(ac), host(res)
    obits, oar, oac, ores = oracle.fit(w, nb, iters)
    w64 = w.astype(np.float64)
    scale = np.abs(w64).max()
    # base 0: the signs of W itself, decided on the same values on both sides
    assert np.array_equal(bits[0], obits[0])
    for kk in range(nb):
        if kk:
            # later bases: signs of a residual that fp32 and fp64 round differently; a sign may
            # differ only where that residual is within rounding of zero
            rk = oracle.fit(w, kk, iters)[3]
            diff = np.unpackbits((bits[kk] ^ obits[kk]).view(np.uint8), axis=-1, bitorder="little")[:, :w.shape[1]]
            if diff.any():
                assert np.abs(rk[diff.astype(bool)]).max() <= 1e-5 * scale, kk
        assert max_rel_err(ar[kk], oar[kk]) <= 1e-4, ("alpha_r", kk)
        assert max_rel_err(ac[kk], oac[kk]) <= 1e-4, ("alpha_c", kk)
    assert np.linalg.norm(res - ores) <= 1e-4 * np.linalg.norm(w64)
    return res


# (a single row is fitted exactly by one base, so its second base would fit rounding noise)
@pytest.mark.parametrize("n,k,nb,iters", [(300, 700, 3, 5), (1, 33, 1, 2), (257, 64, 1, 0), (65, 300, 2, 1),
                                          (1000, 2000, 2, 10)])
def test_fit_matches_oracle(n, k, nb, iters):
    rng = np.random.default_rng(n + k + nb + iters)
    check_fit(fit_matrix(rng, n, k), nb, iters)


def test_fit_fp16_input_and_zeros():
    rng = np.random.default_rng(7)
    w = fit_matrix(rng, 200, 513, np.float16)
    w[::5, ::3] = 0          # sign(0) reads +1 on both sides
    check_fit(w, 2, 3)


def test_fit_4096x4096():
    """4096 x 4096 (the 7B projection), 2 bases, 5 rounds: every scale and the residual."""
    rng = np.random.default_rng(8)
    res = check_fit(fit_matrix(rng, 4096, 4096), 2, 5)
    assert np.isfinite(res).all()


def test_fit_recovers_exact_decomposition_and_error_falls():
    rng = np.random.default_rng(9)
    n, k = 300, 1000
    a = rng.integers(1, 9, n).astype(np.float64)
    b = rng.integers(1, 9, k).astype(np.float64)
    signs = np.where(rng.random((n, k)) < 0.5, -1.0, 1.0)
    w = (np.outer(a, b) * signs).astype(np.float32)
    bits, ar, ac, res = ubw.fit_bases(dev(w), 1, 1)
    words = oracle.fit(w, 1, 0)[0][0]   # the signs of w
    assert np.array_equal(host(bits)[0].view(np.uint32), words)
    assert np.abs(host(res)).max() <= 1e-5 * np.abs(w).max()
    # the residual of a general matrix shrinks with every base
    w = fit_matrix(rng, 500, 700)
    norms = [np.linalg.norm(host(ubw.fit_bases(dev(w), nb, 3)[3])) for nb in (1, 2, 3, 4)]
    assert all(b < a for a, b in zip([np.linalg.norm(w)] + norms, norms))


def test_fit_output_drives_the_gemv():
    """Fitted bases packed and run through the step equal the oracle GEMV of the same bases."""
    rng = np.random.default_rng(10)
    n, k = 700, 1500
    w = fit_matrix(rng, n, k)
    bits, ar, ac, _ = ubw.fit_bases(dev(w), 2, 3)
    x = rng.standard_normal((2, k)).astype(np.float16)
    packed = ubw.pack_bases(bits, 2, n, k)
    y = ubw.lut_gemv(packed, ar, ac, dev(x), n, k, workspace=ubw.workspace(n, DEV))
    r = oracle.gemv(host(bits).view(np.uint32), host(ar), host(ac), x)
    assert max_rel_err(host(y), r) <= TOL


# ------------------------------------------------------------------------------------------
# Hessian-guided saliency: Gram matrix on the matrix cores, blocked Cholesky, selection

@pytest.mark.parametrize("t,k", [(300, 200), (1, 129), (32, 128), (2048, 512), (77, 1000)])
def test_gram_integer_exact(t, k):
    """Integer activations: every product and partial sum is an integer below 2^24, so the
    matrix-core result is exact (pins the operand and result lane layouts)."""
    rng = np.random.default_rng(t + k)
    x = rng.integers(-4, 5, size=(t, k)).astype(np.float16)
    h = host(ubw.gram(dev(x)))
    assert np.array_equal(h.astype(np.float64), oracle.hessian(x))


def test_gram_float():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1024, 1000)).astype(np.float16)
    h = host(ubw.gram(dev(x))).astype(np.float64)
    r = oracle.hessian(x)
    assert np.abs(h - r).max() <= 1e-5 * np.abs(r).max()


def check_saliency(x, w, s, damp=0.01):
    hd = ubw.gram(dev(x))
    h_in = host(hd).astype(np.float64)
    d, score, idx, ws = ubw.hessian_saliency(hd, dev(w), s, damp=damp)
    d, score, idx, ws, L = host(d), host(score), host(idx), host(ws), np.tril(host(hd).astype(np.float64))
    assert ws[1] == 0
    od, oscore, oidx = oracle.saliency(h_in, w, s, damp=damp)
    k = len(d)
    lam = damp * np.mean(np.diag(h_in))
    assert abs(ws[0] - lam) <= 1e-5 * lam
    # the factor: L L^T = H + lambda I
    hd64 = h_in + lam * np.eye(k)
    assert np.abs(L @ L.T - hd64).max() <= 2e-7 * max(k, 500) * np.abs(hd64).max()
    assert max_rel_err(d, od) <= 1e-3
    assert max_rel_err(score, oscore) <= 2e-3
    # the selection is exactly the top s of the GPU's own scores (ties: lower index)...
    own = np.sort(np.lexsort((np.arange(k), -score.astype(np.float64)))[:s])
    assert np.array_equal(idx, own)
    # ...and differs from the oracle's only at scores within rounding of the boundary
    bound = np.sort(oscore)[::-1][s - 1]
    for j in set(idx.tolist()) ^ set(oidx.tolist()):
        assert abs(oscore[j] - bound) <= 4e-3 * bound, j
    return idx


@pytest.mark.parametrize("t,k,n,s", [(500, 64, 40, 5), (300, 300, 100, 31), (2000, 1000, 300, 50), (100, 700, 50, 70),
                                     (1000, 1, 3, 1)])
def test_saliency_matches_oracle(t, k, n, s):
    rng = np.random.default_rng(t + k + n)
    x = (rng.standard_normal((t, k)) * rng.uniform(0.2, 2, (1, k))).astype(np.float16)
    w = rng.standard_normal((n, k)).astype(np.float32)
    check_saliency(x, w, s)


def test_saliency_7b_projection_shape():
    """K = 4096 with 2048 synthetic calibration rows (fewer than K: H is singular and only the
    damping makes it definite), a dense 4096 x 4096 W, 205 salient columns (5%)."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((2048, 4096)) * rng.uniform(0.2, 2, (1, 4096))).astype(np.float16)
    w = rng.standard_normal((4096, 4096)).astype(np.float32)
    idx = check_saliency(x, w, 205)
    ubw.check_indices(idx, 4096)


def test_saliency_flags_a_matrix_that_is_not_definite():
    """-2 I: the mean of the diagonal is negative, so lambda = 1 and H_d = -I has no Cholesky
    factor: the error code is set (the kernels still finish)."""
    k = 100
    h = torch.from_numpy(-2.0 * np.eye(k, dtype=np.float32)).to(DEV)
    w = torch.ones((4, k), device=DEV)
    _, _, _, ws = ubw.hessian_saliency(h, w, 10)
    assert host(ws)[1] != 0


@pytest.mark.parametrize("batch", [5, 6, 13])
@pytest.mark.parametrize("k", [1000, 1501])
def test_batch_chunks_ragged(batch, k):
    """Batches above 4 rows run as 4-row launches: ragged last chunk, activation blocks that go
    through LDS (K = 1000: 4 rows of fp16 fit) or not, each mode of the step, grouped too."""
    rng = np.random.default_rng(batch * 10 + k)
    g = make_integer_gemv(rng, 700, k, 2, s=60, ns=2, batch=batch)
    ref = oracle_gemv(g)
    for mode in MODES:
        y = torch.full((batch, g.n), float("nan"), device=DEV)
        assert np.array_equal(gpu_gemv(g, y=y, mode=mode), ref), mode
    y0 = rng.integers(-50, 50, (batch, g.n)).astype(np.float32)
    assert np.array_equal(gpu_gemv(g, y=dev(y0), accumulate=True), ref + y0)
    h = make_integer_gemv(rng, 300, k, 1, batch=batch)
    shared_x([g, h], g.x)
    outs = ubw.lut_gemv_multi([multi_entry(g), multi_entry(h, ws=False)], dev(g.x), k)
    assert np.array_equal(host(outs[0]).astype(np.float64), ref)
    assert np.array_equal(host(outs[1]).astype(np.float64), oracle_gemv(h))


@pytest.mark.parametrize("batch", [1, 3])
def test_fp32_activations_in_variants(batch):
    """fp32 activations through the group-scale variant and the grouped launch (integer exact)."""
    rng = np.random.default_rng(400 + batch)
    k = 900
    g = make_integer_gemv(rng, 600, k, 2, s=50, ns=1, batch=batch, x_dtype=np.float32)
    h = make_integer_gemv(rng, 300, k, 3, batch=batch, x_dtype=np.float32)
    shared_x([g, h], g.x)
    arg = gs_scales(rng, g)
    assert np.array_equal(gpu_gs(g, arg), oracle_gs(g, arg))
    outs = ubw.lut_gemv_multi([multi_entry(g), multi_entry(h)], dev(g.x), k)
    assert np.array_equal(host(outs[0]).astype(np.float64), oracle_gemv(g))
    assert np.array_equal(host(outs[1]).astype(np.float64), oracle_gemv(h))


# ------------------------------------------------------------------------------------------
# batches the path model sends to the matrix cores (default path) vs the tables (explicit geometry):
# from 9 rows at any size, from 7 rows above ~6.4 MB of weights, from 8 rows above ~3 MB

@pytest.mark.parametrize("n,k,nb,s,ns,batch,xdt,xscale", [
    (300, 200, 2, 0, 0, 9, np.float16, 1.0),         # one slice: one chunk, plain stores
    (1000, 3000, 3, 300, 2, 16, np.float32, 1e4),    # large activations: staging scale < 1
    (777, 1501, 3, 100, 3, 9, np.float32, 1e-5),     # tiny activations: staging scale > 1
    (4100, 700, 1, 37, 1, 12, np.float16, 1.0),      # many row tiles, ragged last tile
    (256, 4096, 2, 205, 2, 16, np.float16, 1.0),     # one row tile, many chunks
    (4100, 6000, 3, 300, 2, 7, np.float16, 1.0),     # 7 rows (9.2 MB of weights), ragged last tile
    (3100, 4500, 2, 45, 1, 8, np.float32, 1.0),      # 8 rows (3.5 MB), ragged slices and tiles
])
def test_matrix_core_batches_match_oracle(n, k, nb, s, ns, batch, xdt, xscale):
    rng = np.random.default_rng(n + k + batch)
    g = make_gemv(rng, "mc", n, k, nb, s=s, ns=ns, batch=batch, x_dtype=np.float32)
    g.x = (g.x * xscale).astype(xdt)
    ref = oracle_gemv(g)
    for mode in MODES:
        y = torch.full((batch, n), float("nan"), device=DEV)
        assert max_rel_err(gpu_gemv(g, y=y, mode=mode), ref) <= TOL, mode
    # accumulate into values of the result's own size (fp32 sums at a larger scale would round
    # away more than the tolerance of a small result)
    y0 = (rng.standard_normal((batch, n)) * np.abs(ref).max()).astype(np.float32)
    got = gpu_gemv(g, y=dev(y0), accumulate=True)
    assert max_rel_err(got, ref + y0.astype(np.float64)) <= TOL


def test_matrix_core_and_tables_agree_and_seven_bases_fall_back():
    """The same integer problem through the matrix cores (default) and the tables (explicit
    geometry) gives the same exact result; with seven bases the default path is the tables."""
    rng = np.random.default_rng(77)
    n, k = 700, 1300
    for nb, ns in ((3, 3), (4, 3)):
        g = make_integer_gemv(rng, n, k, nb, s=90, ns=ns, batch=10)
        ref = oracle_gemv(g)
        assert np.array_equal(gpu_gemv(g, mode="fused"), ref), (nb, ns)
        y = torch.zeros((10, n), device=DEV)
        ubw.lut_gemv_geometry(pack(g.bits, k), dev(g.alpha_r), dev(g.alpha_c), dev(g.x), n, k, y,
                              rows_per_group=1)
        ubw.lut_gemv_geometry(pack(g.bits_s, g.s), dev(g.alpha_r_s), dev(g.alpha_c_s), dev(g.x), n, g.s, y,
                              idx=dev(g.idx), k=k, accumulate=True, rows_per_group=1)
        assert np.array_equal(host(y).astype(np.float64), ref), (nb, ns)


def split_bound(g, x):
    """Per output, sum over bases of |alpha_r| (2^-20 sum_j |v_j| + K 2^-38 max_j |v_j|), v the
    fp32 product alpha_c * x of each activation row: the most the matrix cores' fp16 hi + lo
    representation of v can move a result away from the tables' (include/ubw.h, UBW_MAX_BATCH)."""
    xb = x.astype(np.float32)
    out = np.zeros((x.shape[0], g.n))
    for kk in range(g.nb):
        v = np.abs((g.alpha_c[kk][None, :] * xb).astype(np.float64))
        per_row = 2.0 ** -20 * v.sum(axis=1) + g.k * 2.0 ** -38 * v.max(axis=1)
        out += per_row[:, None] * np.abs(g.alpha_r[kk].astype(np.float64))[None, :]
    return out


def tables_reference(g, x):
    """The same GEMV through the tables at any batch (the geometry export), main bases only."""
    y = torch.zeros((x.shape[0], g.n), device=DEV)
    ubw.lut_gemv_geometry(pack(g.bits, g.k), dev(g.alpha_r), dev(g.alpha_c), dev(x), g.n, g.k, y, rows_per_group=1)
    return host(y).astype(np.float64)


def test_matrix_core_split_bound_one_hot():
    """16 rows on the matrix cores against the tables, each activation row one-hot at its own
    column with a full-precision alpha_c: every output is then alpha_r * (+-v) of one column, exact
    on the tables (fp32 v), so the difference is the hi/lo split's own error, which must stay
    within |alpha_r| (2^-20 |v| + 2^-38 |v|) per base plus the fp32 rounding of the products."""
    rng = np.random.default_rng(26)
    n, k, nb = 512, 1024, 2
    g = make_gemv(rng, "onehot", n, k, nb, batch=16)
    cols = rng.choice(k, 16, replace=False)
    x = np.zeros((16, k), np.float16)
    x[np.arange(16), cols] = (rng.uniform(0.5, 4.0, 16) * rng.choice([-1, 1], 16)).astype(np.float16)
    g.x = x
    y_mm = host(ubw.lut_gemv(pack(g.bits, k), dev(g.alpha_r), dev(g.alpha_c), dev(x), n, k)).astype(np.float64)
    y_tab = tables_reference(g, x)
    prod = sum(np.abs(g.alpha_r[kk].astype(np.float64))[None, :] *
               np.abs((g.alpha_c[kk] * x.astype(np.float32)).astype(np.float64)).max(axis=1)[:, None]
               for kk in range(nb))
    bound = (2.0 ** -20 + 2.0 ** -38) * prod + 4 * 2.0 ** -24 * prod
    diff = np.abs(y_mm - y_tab)
    assert np.all(diff <= bound), float(np.max(diff / bound))
    assert max_rel_err(y_mm, oracle_gemv(g)) <= TOL


@pytest.mark.parametrize("n,k,nb", [(11008, 4096, 2), (4096, 11008, 2)])
def test_matrix_core_vs_tables_16_rows(n, k, nb):
    """7B MLP shapes at 16 rows, every output: the matrix-core result stays within the split
    bound of the tables' result (the two paths' fp32 summation orders differ by far less on these
    inputs) and within the 1e-3 bar of the oracle."""
    rng = np.random.default_rng(27 + n)
    g = make_gemv(rng, "mlp16", n, k, nb, batch=16)
    y_mm = host(ubw.lut_gemv(pack(g.bits, k), dev(g.alpha_r), dev(g.alpha_c), dev(g.x), n, k)).astype(np.float64)
    y_tab = tables_reference(g, g.x)
    assert np.all(np.abs(y_mm - y_tab) <= split_bound(g, g.x))
    assert max_rel_err(y_mm, oracle_gemv(g)) <= TOL


@pytest.mark.parametrize("n,k,batch", [(9 * 256 + 37, 1500, 1), (23 * 256, 777, 1), (10 * 256, 2048, 3),
                                       (17 * 256 - 5, 600, 4), (8 * 256, 1500, 1), (16 * 256 - 100, 900, 2),
                                       (24 * 256, 700, 4)])
def test_xcd_local_row_groups_integer_exact(n, k, batch):
    """y = result with 8 or more row groups: each row group on one XCD, zeroed by a workgroup
    without units at a lower ID (8, 16 and 24 row groups with up to 64 workgroups), or the
    first-arriver protocol (row groups that do not divide over the 8 XCDs, or 100000 workgroups,
    more than the device holds): every split, the refinement alone and main + refinement, NaN
    garbage overwritten, exact."""
    rng = np.random.default_rng(n + k + batch)
    g = make_integer_gemv(rng, n, k, 2, s=max(1, k // 20), ns=2, batch=batch)
    packed, ps = pack(g.bits, k), pack(g.bits_s, g.s)
    ws = ubw.workspace(n, DEV)
    main, full = oracle_gemv(g, refine=False), oracle_gemv(g)
    for wgs in (8, 9, 15, 64, 0, 100000):
        y = torch.full((batch, n), float("nan"), device=DEV)
        ubw.lut_gemv_geometry(packed, dev(g.alpha_r), dev(g.alpha_c), dev(g.x), n, k, y, rows_per_group=1,
                              workgroups=wgs, workspace=ws)
        assert np.array_equal(host(y).astype(np.float64), main), ("main", wgs)
        y = torch.full((batch, n), float("nan"), device=DEV)
        ubw.lut_gemv_geometry(ps, dev(g.alpha_r_s), dev(g.alpha_c_s), dev(g.x), n, g.s, y, idx=dev(g.idx), k=k,
                              rows_per_group=1, workgroups=wgs, workspace=ws)
        assert np.array_equal(host(y).astype(np.float64), full - main), ("refinement", wgs)
        assert ubw.workspace_check(ws) == (ubw.UBW_OK, 0), wgs
    y = torch.full((batch, n), float("nan"), device=DEV)
    assert np.array_equal(gpu_gemv(g, y=y, ws=ws), full)
