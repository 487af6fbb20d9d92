"""Pins for the CPU oracle, checked against things other than itself.

Each test fixes the oracle to something the FluxBin page or plain mathematics determines:
brute-force enumeration of every sign row, closed forms (popcount, all-ones, one-hot, table
symmetries), integer matvecs done by numpy on matrices unpacked by numpy, invariants of the
decomposition W_hat^(k) = (alpha_r^(k) alpha_c^(k)^T) (.) B^(k) ("1. Algorithm innovation"),
and a hand-worked example under tests/golden/.
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import draw_bits, make_gemv, make_integer_gemv, words_per_row

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dense_signs(bits, k):
    """±1 matrix [nb, n, k] unpacked with numpy (independent of the oracle's bit reader)."""
    nb, n, w = bits.shape
    by = np.ascontiguousarray(bits).view(np.uint8).reshape(nb, n, w * 4)
    b01 = np.unpackbits(by, axis=2, bitorder="little")[:, :, :k]
    return b01.astype(np.int64) * 2 - 1


# ---------------------------------------------------------------------------------------------
def test_hand_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    bits = np.array(ex["bits"], np.uint32)
    kw = dict(idx=np.array(ex["idx"], np.int32), bits_s=np.array(ex["bits_s"], np.uint32),
              alpha_r_s=np.array(ex["alpha_r_s"], np.float32), alpha_c_s=np.array(ex["alpha_c_s"], np.float32))
    args = (bits, np.array(ex["alpha_r"], np.float32), np.array(ex["alpha_c"], np.float32),
            np.array(ex["x"], np.float64))
    y = oracle.gemv(*args, **kw)
    assert y[0].tolist() == ex["y"]
    for g in (4, 8):
        assert oracle.lut_gemv(*args, g=g, **kw)[0].tolist() == ex["y"]
    assert oracle.patterns(bits, ex["K"], g=4).tolist() == ex["patterns_g4"]
    assert oracle.patterns(bits, ex["K"], g=8).tolist() == ex["patterns_g8"]


@pytest.mark.parametrize("k", [8, 12])
def test_bruteforce_every_sign_row(k):
    """Row r carries the sign pattern of the integer r: all 2^K rows are present."""
    rng = np.random.default_rng(k)
    n = 1 << k
    bits = np.arange(n, dtype=np.uint32).reshape(1, n, 1)
    alpha_r = np.ones((1, n), np.float32)
    alpha_c = rng.uniform(0.1, 1.0, (1, k)).astype(np.float32)
    x = rng.standard_normal(k)
    x[np.abs(x) < 1e-3] = 0.5
    y = oracle.gemv(bits, alpha_r, alpha_c, x)[0]
    v = alpha_c[0].astype(np.float64) * x
    l1 = np.abs(v).sum()
    # the best sign row matches sign(v) bit by bit, with column j at bit j and bit 1 = +1
    best = sum(1 << j for j in range(k) if v[j] > 0)
    assert int(np.argmax(y)) == best
    assert abs(y.max() - l1) <= 1e-12 * l1
    assert abs(y.min() + l1) <= 1e-12 * l1
    # complement rows negate exactly; all rows sum to zero
    full = n - 1
    assert np.array_equal(y, -y[np.arange(n) ^ full])
    assert abs(y.sum()) <= 1e-9 * l1
    # flipping bit j moves the row's value by 2 v_j
    for j in range(k):
        r = np.arange(n)
        d = y[r] - y[r ^ (1 << j)]
        expect = np.where((r >> j) & 1, 2 * v[j], -2 * v[j])
        assert np.allclose(d, expect, rtol=0, atol=1e-12 * l1)


@pytest.mark.parametrize("k", [1, 31, 32, 33, 100, 257])
def test_popcount_closed_form(k):
    """Unit scales and x = 1: y_r = 2 * popcount(row r's first K bits) - K."""
    rng = np.random.default_rng(100 + k)
    n = 37
    bits = draw_bits(rng, 1, n, k)
    y = oracle.gemv(bits, np.ones((1, n), np.float32), np.ones((1, k), np.float32), np.ones(k))[0]
    mask = (1 << k) - 1
    for r in range(n):
        big = sum(int(w) << (32 * i) for i, w in enumerate(bits[0, r]))
        assert y[r] == 2 * bin(big & mask).count("1") - k


def test_one_hot_reads_one_column():
    rng = np.random.default_rng(7)
    n, k = 41, 70
    bits = draw_bits(rng, 1, n, k)
    signs = dense_signs(bits, k)[0]
    for j in (0, 1, 31, 32, 33, 63, 69):
        x = np.zeros(k)
        x[j] = 1.0
        y = oracle.gemv(bits, np.ones((1, n), np.float32), np.ones((1, k), np.float32), x)[0]
        assert np.array_equal(y, signs[:, j].astype(np.float64))


def test_all_plus_bits_is_rank_one():
    rng = np.random.default_rng(8)
    n, k = 19, 77
    bits = np.full((2, n, words_per_row(k)), 0xFFFFFFFF, np.uint32)
    ar = rng.uniform(0.1, 1, (2, n)).astype(np.float32)
    ac = rng.uniform(0.1, 1, (2, k)).astype(np.float32)
    x = rng.standard_normal(k)
    y = oracle.gemv(bits, ar, ac, x)[0]
    expect = sum(ar[i].astype(np.float64) * float(np.dot(ac[i].astype(np.float64), x)) for i in range(2))
    assert np.allclose(y, expect, rtol=1e-13, atol=0)


def test_integer_matvec_equals_numpy():
    rng = np.random.default_rng(9)
    g = make_integer_gemv(rng, 50, 100, 1, batch=3)
    y = oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x)
    signs = dense_signs(g.bits, g.k)[0]
    expect = g.x.astype(np.int64) @ signs.T
    assert np.array_equal(y, expect.astype(np.float64))


def test_bases_add_up():
    rng = np.random.default_rng(10)
    g = make_integer_gemv(rng, 33, 96, 3, batch=2)
    y = oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x)
    parts = [oracle.gemv(g.bits[i:i + 1], g.alpha_r[i:i + 1], g.alpha_c[i:i + 1], g.x) for i in range(3)]
    assert np.array_equal(y, parts[0] + parts[1] + parts[2])


def test_scale_invariances():
    rng = np.random.default_rng(11)
    g = make_gemv(rng, "t", 40, 64, 2, batch=2)
    y = oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x)
    # alpha_r is a per-row factor of each base
    y2 = oracle.gemv(g.bits, g.alpha_r * 2, g.alpha_c, g.x)
    assert np.array_equal(y2, 2 * y)
    # alpha_c and x meet only through their product (powers of two keep it exact)
    d = np.where(np.arange(64) % 2 == 0, 4.0, 0.5).astype(np.float32)
    y3 = oracle.gemv(g.bits, g.alpha_r, g.alpha_c * d, g.x.astype(np.float64) / d)
    assert np.allclose(y3, y, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("g_width", [1, 2, 4, 8])
@pytest.mark.parametrize("k", [8, 37, 256, 300])
def test_lut_route_equals_dequantized(g_width, k):
    """The table route of the kernel section reaches the dequantized product."""
    rng = np.random.default_rng(1000 * g_width + k)
    s = max(1, k // 20)
    g = make_gemv(rng, "t", 45, k, 2, s=s, ns=2, batch=2)
    y_deq = oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x, **g.refine_kwargs())
    y_lut = oracle.lut_gemv(g.bits, g.alpha_r, g.alpha_c, g.x, g=g_width, **g.refine_kwargs())
    scale = np.abs(g.x.astype(np.float64)).sum(axis=1, keepdims=True) * 4.0
    assert np.all(np.abs(y_lut - y_deq) <= 1e-13 * scale)
    gi = make_integer_gemv(rng, 45, k, 2, s=s, ns=2, batch=2)
    assert np.array_equal(oracle.gemv(gi.bits, gi.alpha_r, gi.alpha_c, gi.x, **gi.refine_kwargs()),
                          oracle.lut_gemv(gi.bits, gi.alpha_r, gi.alpha_c, gi.x, g=g_width, **gi.refine_kwargs()))


@pytest.mark.parametrize("g_width", [4, 8])
def test_table_closed_forms(g_width):
    rng = np.random.default_rng(12)
    k = 3 * g_width + 3   # last group ragged
    ac = rng.uniform(0.1, 1, (2, k)).astype(np.float32)
    x = rng.standard_normal((2, k)).astype(np.float16)
    T = oracle.lut_tables(x, ac, g=g_width)
    ng = T.shape[2]
    full = (1 << g_width) - 1
    for b in range(2):
        for kk in range(2):
            v = ac[kk].astype(np.float64) * x[b].astype(np.float64)
            v = np.concatenate([v, np.zeros(ng * g_width - k)]).reshape(ng, g_width)
            t = T[b, kk]
            assert np.allclose(t[:, full], v.sum(1), rtol=1e-14, atol=1e-14)
            assert np.allclose(t[:, 0], -v.sum(1), rtol=1e-14, atol=1e-14)
            assert np.allclose(t, -t[:, full - np.arange(full + 1)], rtol=0, atol=1e-14)
            for i in range(g_width):
                assert np.allclose(t[:, 1 << i] - t[:, 0], 2 * v[:, i], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("g_width", [4, 8])
def test_patterns_from_constructed_rows(g_width):
    """Row r, group gi holds (7r + gi) mod 2^g; rows are assembled from Python integers."""
    n, k = 40, 8 * g_width + g_width // 2   # ragged last group
    ng = (k + g_width - 1) // g_width
    want = np.zeros((1, n, ng), np.uint16)
    bits = np.zeros((1, n, words_per_row(k)), np.uint32)
    for r in range(n):
        big = 0
        for gi in range(ng):
            p = (7 * r + gi) % (1 << g_width)
            if gi == ng - 1:
                p &= (1 << (k - gi * g_width)) - 1   # columns past K read as zero
            want[0, r, gi] = p
            big |= p << (gi * g_width)
        for w in range(bits.shape[2]):
            bits[0, r, w] = (big >> (32 * w)) & 0xFFFFFFFF
    assert np.array_equal(oracle.patterns(bits, k, g=g_width), want)


def test_padding_bits_ignored():
    rng = np.random.default_rng(13)
    g = make_gemv(rng, "t", 20, 45, 2, batch=1)
    clean = g.bits.copy()
    clean[:, :, -1] &= (1 << (45 - 32)) - 1
    assert np.array_equal(oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x),
                          oracle.gemv(clean, g.alpha_r, g.alpha_c, g.x))
    assert np.array_equal(oracle.patterns(g.bits, 45), oracle.patterns(clean, 45))


def test_ternary_definition_integer_exact():
    rng = np.random.default_rng(14)
    w = rng.integers(-1, 2, (60, 130)).astype(np.int8)
    x = rng.integers(-8, 9, (3, 130)).astype(np.float16)
    y = oracle.ternary_gemv(w, np.ones(60, np.float32), x)
    assert np.array_equal(y, (x.astype(np.int64) @ w.astype(np.int64).T).astype(np.float64))
    sc = rng.uniform(0.01, 0.1, 60).astype(np.float32)
    y2 = oracle.ternary_gemv(w, sc, x)
    assert np.allclose(y2, (x.astype(np.float64) @ w.T.astype(np.float64)) * sc.astype(np.float64), rtol=1e-14)


@pytest.mark.parametrize("zero_first_plus", [True, False])
def test_ternary_two_half_bases(zero_first_plus):
    """w = (B1 + B2)/2 with both bases at row scale s/2 reproduces the ternary layer; the
    choice of (+1,-1) or (-1,+1) for zeros does not matter."""
    rng = np.random.default_rng(15)
    n, k = 48, 200
    w = rng.integers(-1, 2, (n, k)).astype(np.int8)
    enc = oracle.ternary_encode(w, zero_first_plus)
    signs = dense_signs(enc, k)
    assert np.array_equal((signs[0] + signs[1]) // 2, w.astype(np.int64))
    sc = np.full(n, 2.0, np.float32)
    x = rng.integers(-8, 9, (2, k)).astype(np.float16)
    ar = np.stack([sc / 2, sc / 2])
    y = oracle.gemv(enc, ar, np.ones((2, k), np.float32), x)
    assert np.array_equal(y, oracle.ternary_gemv(w, sc, x))


def test_refinement_invariants():
    rng = np.random.default_rng(16)
    n, k = 30, 96
    gi = make_integer_gemv(rng, n, k, 2, batch=2)
    y_main = oracle.gemv(gi.bits, gi.alpha_r, gi.alpha_c, gi.x)
    # every column salient, refinement = copy of the main bases -> exactly double
    idx = np.arange(k, dtype=np.int32)
    y2 = oracle.gemv(gi.bits, gi.alpha_r, gi.alpha_c, gi.x, idx=idx, bits_s=gi.bits,
                     alpha_r_s=gi.alpha_r, alpha_c_s=gi.alpha_c)
    assert np.array_equal(y2, 2 * y_main)
    # permuting salient positions together with their refinement columns changes nothing
    g = make_gemv(rng, "t", n, k, 2, s=23, ns=2, batch=2)
    y_ref = oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x, **g.refine_kwargs())
    perm = rng.permutation(g.s)
    sg = dense_signs(g.bits_s, g.s)[:, :, perm]
    b01 = (sg > 0).astype(np.uint8)
    pad = (-g.s) % 32
    b01 = np.concatenate([b01, np.zeros((2, n, pad), np.uint8)], axis=2)
    bits_p = np.packbits(b01, axis=2, bitorder="little").view(np.uint32).reshape(2, n, -1)
    y_p = oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x, idx=g.idx[perm], bits_s=bits_p,
                      alpha_r_s=g.alpha_r_s, alpha_c_s=g.alpha_c_s[:, perm])
    assert np.allclose(y_p, y_ref, rtol=1e-13, atol=1e-13)
    # one-hot on a salient column: main column plus refinement column
    q = 5
    col = int(g.idx[q])
    x = np.zeros(k)
    x[col] = 1.0
    y1 = oracle.gemv(g.bits, g.alpha_r, g.alpha_c, x, **g.refine_kwargs())[0]
    sm = dense_signs(g.bits, k)[:, :, col]
    ss = dense_signs(g.bits_s, g.s)[:, :, q]
    expect = sum(g.alpha_r[i].astype(np.float64) * float(g.alpha_c[i, col]) * sm[i] for i in range(2)) + \
        sum(g.alpha_r_s[i].astype(np.float64) * float(g.alpha_c_s[i, q]) * ss[i] for i in range(2))
    assert np.allclose(y1, expect, rtol=1e-14, atol=1e-14)
    # a zero activation at every salient column silences the refinement
    x0 = g.x.astype(np.float64).copy()
    x0[:, g.idx] = 0.0
    assert np.allclose(oracle.gemv(g.bits, g.alpha_r, g.alpha_c, x0, **g.refine_kwargs()),
                       oracle.gemv(g.bits, g.alpha_r, g.alpha_c, x0), rtol=1e-14, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# group-scale variant: one row scale per 128-column block

def _gs_problem(rng, n, k, nb, integer):
    gcols = 2 * ((k + 255) // 256)
    if integer:
        g = make_integer_gemv(rng, n, k, nb, batch=2)
        arg = rng.integers(1, 4, size=(nb, n, gcols)).astype(np.float16)
    else:
        g = make_gemv(rng, "gs", n, k, nb, batch=2)
        arg = rng.uniform(0.05, 0.5, size=(nb, n, gcols)).astype(np.float16)
    return g, arg


@pytest.mark.parametrize("k", [77, 128, 200, 256, 300, 700])
def test_gs_constant_blocks_equal_plain(k):
    """Equal scales in every block of a row reduce to the per-row definition, value for value."""
    rng = np.random.default_rng(k)
    g, _ = _gs_problem(rng, 21, k, 2, integer=False)
    arg = np.repeat(g.alpha_r[:, :, None], 2 * ((k + 255) // 256), axis=2)
    assert np.array_equal(oracle.gemv_gs(g.bits, arg, g.alpha_c, g.x), oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x))


@pytest.mark.parametrize("integer", [True, False])
@pytest.mark.parametrize("k", [129, 256, 300, 700])
def test_gs_sum_of_block_restricted_products(integer, k):
    """The product splits over column blocks: block q alone is the per-row definition with
    alpha_r = the block's scales and alpha_c zero outside the block. A wrong block index, a
    dropped block or a block read from the wrong row fails this."""
    rng = np.random.default_rng(1000 + k + integer)
    g, arg = _gs_problem(rng, 17, k, 3, integer)
    y = oracle.gemv_gs(g.bits, arg, g.alpha_c, g.x)
    parts = np.zeros_like(y)
    for q in range(-(-k // 128)):
        ac = np.zeros_like(g.alpha_c)
        ac[:, 128 * q:128 * (q + 1)] = g.alpha_c[:, 128 * q:128 * (q + 1)]
        parts += oracle.gemv(g.bits, arg[:, :, q].astype(np.float32), ac, g.x)
    if integer:
        assert np.array_equal(y, parts)
    else:
        assert np.allclose(y, parts, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_gs_integer_matvec_equals_numpy():
    rng = np.random.default_rng(77)
    k = 300
    g, arg = _gs_problem(rng, 40, k, 2, integer=True)
    signs = dense_signs(g.bits, k)
    scale = np.repeat(arg.astype(np.int64), 128, axis=2)[:, :, :k]   # block scale of every column
    w = (signs * scale).sum(axis=0)
    assert np.array_equal(oracle.gemv_gs(g.bits, arg, g.alpha_c, g.x), (g.x.astype(np.int64) @ w.T).astype(np.float64))


def test_gs_refinement_adds_the_same_branch():
    rng = np.random.default_rng(78)
    g = make_integer_gemv(rng, 30, 500, 2, s=40, ns=2, batch=2)
    arg = rng.integers(1, 4, size=(2, 30, 4)).astype(np.float16)
    with_ref = oracle.gemv_gs(g.bits, arg, g.alpha_c, g.x, **g.refine_kwargs())
    without = oracle.gemv_gs(g.bits, arg, g.alpha_c, g.x)
    branch = oracle.gemv(g.bits, g.alpha_r, g.alpha_c, g.x, **g.refine_kwargs()) - oracle.gemv(
        g.bits, g.alpha_r, g.alpha_c, g.x)
    assert np.array_equal(with_ref, without + branch)


# ---------------------------------------------------------------------------------------------
# offline fit: residual sign binarization + alternating least squares for (alpha_r, alpha_c)

def _sign_bits(m):
    """Canonical words of sign(m) (+1 where m >= 0) via numpy packbits."""
    n, k = m.shape
    b = np.zeros((n, words_per_row(k) * 32), np.uint8)
    b[:, :k] = (m >= 0)
    return np.packbits(b, axis=1, bitorder="little").view(np.uint32).reshape(n, words_per_row(k))


def test_fit_gaussian_one_base_closed_form():
    """N(0,1) entries, one base, no ALS round: alpha = mean|w| ~ sqrt(2/pi) and the residual
    keeps 1 - 2/pi of the energy."""
    rng = np.random.default_rng(200)
    w = rng.standard_normal((512, 2048)).astype(np.float32)
    bits, ar, ac, res = oracle.fit(w, 1, 0)
    assert np.allclose(ar[0], np.abs(w.astype(np.float64)).mean(axis=1), rtol=1e-12)
    assert np.all(ac == 1.0)
    assert abs(ar[0].mean() - np.sqrt(2 / np.pi)) < 5e-3
    assert abs((res ** 2).sum() / (w.astype(np.float64) ** 2).sum() - (1 - 2 / np.pi)) < 5e-3


def test_fit_recovers_an_exact_decomposition():
    """W = (a b^T) (.) B with positive a, b: one base and one ALS round give B exactly and a
    zero residual (|W| has rank one)."""
    rng = np.random.default_rng(201)
    n, k = 70, 333
    a = rng.integers(1, 9, n).astype(np.float64)     # small integers: a b^T is exact in fp32
    b = rng.integers(1, 9, k).astype(np.float64)
    signs = np.where(rng.random((n, k)) < 0.5, -1.0, 1.0)
    w = (np.outer(a, b) * signs).astype(np.float32)
    bits, ar, ac, res = oracle.fit(w, 1, 1)
    assert np.array_equal(bits[0], _sign_bits(w))
    assert np.abs(res).max() < 1e-12 * np.abs(w).max()
    assert np.allclose(np.outer(ar[0], ac[0]), np.abs(w.astype(np.float64)), rtol=1e-12)


def test_fit_als_converges_to_leading_singular_pair():
    """Many ALS rounds are a power iteration on |R|: alpha_r alpha_c^T tends to the best rank-one
    approximation sigma_1 u_1 v_1^T of |W| (numpy SVD)."""
    rng = np.random.default_rng(202)
    w = rng.standard_normal((60, 90)).astype(np.float32)
    bits, ar, ac, res = oracle.fit(w, 1, 300)
    u, sv, vt = np.linalg.svd(np.abs(w.astype(np.float64)))
    best = sv[0] * np.outer(u[:, 0], vt[0])
    assert np.allclose(np.outer(ar[0], ac[0]), best, rtol=1e-8, atol=1e-10)


def test_fit_error_never_increases():
    rng = np.random.default_rng(203)
    w = (rng.standard_normal((200, 300)) * rng.uniform(0.2, 3, (200, 1)) * rng.uniform(0.2, 3, (1, 300))
         ).astype(np.float32)
    by_bases = [np.linalg.norm(oracle.fit(w, nb, 3)[3]) for nb in range(1, 5)]
    assert all(b < a for a, b in zip([np.linalg.norm(w)] + by_bases, by_bases))
    by_rounds = [np.linalg.norm(oracle.fit(w, 1, t)[3]) for t in range(0, 6)]
    assert all(b <= a * (1 + 1e-14) for a, b in zip(by_rounds, by_rounds[1:]))


def test_fit_bases_follow_the_residual():
    """Base k's bits are the signs of the residual left by the first k bases, the residual is
    W minus the dequantized bases, and the scaled bases reconstruct W - residual."""
    rng = np.random.default_rng(204)
    w = rng.standard_normal((50, 130)).astype(np.float32)
    w[::7, ::5] = 0.0          # sign(0) reads +1
    bits, ar, ac, res = oracle.fit(w, 3, 2)
    assert np.array_equal(bits[0], _sign_bits(w))
    for k in (1, 2):
        prev = oracle.fit(w, k, 2)
        assert np.array_equal(bits[k], _sign_bits(prev[3]))
        assert np.allclose(prev[1], ar[:k]) and np.allclose(prev[2], ac[:k])
    signs = dense_signs(bits, 130).astype(np.float64)
    w_hat = sum(np.outer(ar[k], ac[k]) * signs[k] for k in range(3))
    assert np.allclose(w.astype(np.float64) - w_hat, res, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# Hessian-guided saliency

def test_hessian_integer_gram():
    rng = np.random.default_rng(300)
    x = rng.integers(-5, 6, size=(40, 17))
    h = oracle.hessian(x.astype(np.float16))
    assert np.array_equal(h, 2.0 * (x.T.astype(np.int64) @ x).astype(np.float64))


def test_saliency_orthogonal_columns_closed_form():
    """Columns of X orthogonal: H = diag(2 c_j), so [H_d^-1]_jj = 1 / (2 c_j + lambda) and the
    score is sum_r w_rj^2 (2 c_j + lambda)^2."""
    rng = np.random.default_rng(301)
    q, _ = np.linalg.qr(rng.standard_normal((64, 16)))
    c = rng.uniform(0.5, 3, 16)
    x = q * np.sqrt(c)                       # x^T x = diag(c)
    w = rng.standard_normal((9, 16))
    h = oracle.hessian(x)
    lam = 0.05 * np.mean(2 * c)
    d, score, idx = oracle.saliency(h, w, 5, damp=0.05)
    assert np.allclose(d, 1 / (2 * c + lam), rtol=1e-10)
    expect = (w ** 2).sum(axis=0) * (2 * c + lam) ** 2
    assert np.allclose(score, expect, rtol=1e-10)
    assert np.array_equal(idx, np.sort(np.argsort(-expect)[:5]))


def test_saliency_two_by_two_by_hand():
    """H = [[4, 2], [2, 3]], damp 0.5 -> lambda = 0.5 * 3.5 = 1.75, H_d = [[5.75, 2], [2, 4.75]],
    det = 23.3125, [H_d^-1]_00 = 4.75 / 23.3125, [H_d^-1]_11 = 5.75 / 23.3125."""
    h = np.array([[4.0, 2.0], [2.0, 3.0]])
    w = np.array([[1.0, 2.0], [3.0, -1.0]])    # column sums of squares: 10, 5
    d, score, idx = oracle.saliency(h, w, 1, damp=0.5)
    det = 5.75 * 4.75 - 4.0
    assert np.allclose(d, [4.75 / det, 5.75 / det], rtol=1e-14)
    assert np.allclose(score, [10 / d[0] ** 2, 5 / d[1] ** 2], rtol=1e-14)
    assert idx.tolist() == [0]


def test_saliency_permutation_and_ties():
    rng = np.random.default_rng(302)
    x = rng.standard_normal((50, 30))
    w = rng.standard_normal((8, 30))
    d, score, idx = oracle.saliency(oracle.hessian(x), w, 7)
    p = rng.permutation(30)
    dp, sp, ip = oracle.saliency(oracle.hessian(x[:, p]), w[:, p], 7)
    assert np.allclose(dp, d[p], rtol=1e-9) and np.allclose(sp, score[p], rtol=1e-9)
    assert np.array_equal(np.sort(p[ip]), idx)
    # equal scores: the lower index wins; s = K selects every column
    h = np.eye(4) * 2.0
    w = np.ones((3, 4))
    assert oracle.saliency(h, w, 2)[2].tolist() == [0, 1]
    assert oracle.saliency(h, w, 4)[2].tolist() == [0, 1, 2, 3]
