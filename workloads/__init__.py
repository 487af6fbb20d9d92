"""Seeded synthetic inputs for the binary-basis GEMV workloads.

This module only draws random numbers (numpy PCG64) and lays them out in the canonical bit
format; it holds none of the method's arithmetic, so both the CPU oracle and the GPU library
can be fed from it without sharing code.

Canonical bit format: uint32 words [bases][rows][ceil(K/32)]; column j of a row is bit j%32 of
word j//32; bit 1 means +1 and bit 0 means -1. Bits past column K in a row's last word are
left random on purpose: consumers must ignore them.

The workloads stand in for the decode-time linear layers that the FluxBin page evaluates
(LLaMA-2 7B / 70B shapes, "Experimental results") and for the ternary tiny language model of
the FlashLM v6 page (ternary {-1,0,+1} weights, 81% of its parameters). No model weights,
calibration data or datasets are used: weights and activations are drawn from the stated
distributions.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np


def words_per_row(k: int) -> int:
    return (int(k) + 31) // 32


def salient_count(frac: float, k: int) -> int:
    """Number of salient columns: round-half-up of frac * K (5% of 4096 -> 205)."""
    return int(np.floor(frac * k + 0.5))


def draw_bits(rng: np.random.Generator, nb: int, n: int, k: int) -> np.ndarray:
    """i.i.d. Bernoulli(1/2) sign bits as canonical words [nb, n, ceil(k/32)]."""
    return rng.integers(0, 2**32, size=(nb, n, words_per_row(k)), dtype=np.uint32)


def draw_uniform(rng, lo, hi, shape) -> np.ndarray:
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


@dataclass
class Gemv:
    """One binary-basis GEMV problem: main bases, optional salient refinement, activations."""
    name: str
    n: int
    k: int
    bits: np.ndarray            # [nb, n, ceil(k/32)] uint32
    alpha_r: np.ndarray         # [nb, n] float32
    alpha_c: np.ndarray         # [nb, k] float32
    x: np.ndarray               # [batch, k] float16 or float32
    idx: Optional[np.ndarray] = None      # [s] int32, ascending, distinct
    bits_s: Optional[np.ndarray] = None   # [ns, n, ceil(s/32)] uint32
    alpha_r_s: Optional[np.ndarray] = None  # [ns, n] float32
    alpha_c_s: Optional[np.ndarray] = None  # [ns, s] float32

    @property
    def nb(self) -> int:
        return self.bits.shape[0]

    @property
    def batch(self) -> int:
        return self.x.shape[0]

    @property
    def s(self) -> int:
        return 0 if self.idx is None else int(self.idx.shape[0])

    @property
    def ns(self) -> int:
        return 0 if self.bits_s is None else int(self.bits_s.shape[0])

    def refine_kwargs(self) -> dict:
        if self.s == 0:
            return {}
        return dict(idx=self.idx, bits_s=self.bits_s, alpha_r_s=self.alpha_r_s, alpha_c_s=self.alpha_c_s)

    def with_batch(self, b: int) -> "Gemv":
        """Same weights, first b activation rows."""
        g = Gemv(**{f: getattr(self, f) for f in self.__dataclass_fields__})
        g.x = self.x[:b]
        return g


def make_gemv(rng: np.random.Generator, name: str, n: int, k: int, nb: int, *,
              alpha=(0.05, 0.5), s: int = 0, ns: int = 0, batch: int = 1,
              x_dtype=np.float16, relu: bool = False) -> Gemv:
    """Draw one problem in a fixed order: main bits, then (alpha_r, alpha_c) per base, then the
    salient indices, refinement bits, refinement (alpha_r_s, alpha_c_s) per base, then x."""
    bits = draw_bits(rng, nb, n, k)
    ar = np.empty((nb, n), np.float32)
    ac = np.empty((nb, k), np.float32)
    for kk in range(nb):
        ar[kk] = draw_uniform(rng, alpha[0], alpha[1], n)
        ac[kk] = draw_uniform(rng, alpha[0], alpha[1], k)
    g = Gemv(name, n, k, bits, ar, ac, x=None)
    if s > 0 and ns > 0:
        g.idx = np.sort(rng.choice(k, size=s, replace=False)).astype(np.int32)
        g.bits_s = draw_bits(rng, ns, n, s)
        g.alpha_r_s = np.empty((ns, n), np.float32)
        g.alpha_c_s = np.empty((ns, s), np.float32)
        for kk in range(ns):
            g.alpha_r_s[kk] = draw_uniform(rng, alpha[0], alpha[1], n)
            g.alpha_c_s[kk] = draw_uniform(rng, alpha[0], alpha[1], s)
    z = rng.standard_normal((batch, k))
    if relu:
        z = np.maximum(z, 0.0)
    g.x = z.astype(x_dtype)
    return g


def make_integer_gemv(rng: np.random.Generator, n: int, k: int, nb: int, *, s: int = 0, ns: int = 0,
                      batch: int = 1, x_dtype=np.float16, xmax: int = 8) -> Gemv:
    """Unit scales and small integer activations: every partial sum is an integer below 2**24,
    so any fp32 summation order gives the exact result."""
    g = make_gemv(rng, "integer", n, k, nb, alpha=(1.0, 1.0), s=s, ns=ns, batch=batch, x_dtype=x_dtype)
    g.alpha_r[:] = 1.0
    g.alpha_c[:] = 1.0
    if g.s:
        g.alpha_r_s[:] = 1.0
        g.alpha_c_s[:] = 1.0
    g.x = rng.integers(-xmax, xmax + 1, size=(batch, k)).astype(x_dtype)
    return g


# ----------------------------------------------------------------------------------------------
# The five workloads.

@dataclass
class TernaryLayer:
    name: str
    w: np.ndarray        # [n, k] int8 in {-1, 0, +1}
    scale: np.ndarray    # [n] float32 per-row scale


@dataclass
class Workload:
    name: str
    description: str
    gemvs: List[Gemv] = field(default_factory=list)
    ternary: List[TernaryLayer] = field(default_factory=list)
    tokens: Optional[np.ndarray] = None   # [T, d] float16 token vectors (ternary stack)
    batches: Tuple[int, ...] = (1,)


def single_gemv_256x512(seed: int = 0) -> Workload:
    """Single binary GEMV: 256 x 512, one base, alpha ~ U(0.1, 1.0), fp32 x, group width 8."""
    rng = np.random.default_rng(seed)
    g = make_gemv(rng, "gemv256x512", 256, 512, 1, alpha=(0.1, 1.0), x_dtype=np.float32)
    return Workload("binary_256x512", "256x512, 1 base, fp32 x", [g])


def ternary_stack_256x768(seed: int = 0, tokens: int = 64) -> Workload:
    """Ternary tiny-LM linear stack: 4 layers of d=256 -> 768 -> 256, weights in {-1,0,+1} each
    with probability 1/3, per-row scale ~ U(0.01, 0.1), fp16 token vectors, batch 1."""
    rng = np.random.default_rng(seed)
    layers = []
    for li in range(4):
        for nm, n, k in (("up", 768, 256), ("down", 256, 768)):
            w = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
            sc = draw_uniform(rng, 0.01, 0.1, n)
            layers.append(TernaryLayer(f"l{li}_{nm}", w, sc))
    toks = rng.standard_normal((tokens, 256)).astype(np.float16)
    return Workload("ternary_stack", "4 x (256->768->256) ternary, 64 tokens", ternary=layers, tokens=toks)


def attn_proj_7b(seed: int = 0) -> Workload:
    """7B-shaped attention projection: 4096 x 4096, 2 bases, 5% salient columns with 2
    refinement bases, alpha ~ U(0.05, 0.5), fp16 x, batch 1."""
    rng = np.random.default_rng(seed)
    k = 4096
    g = make_gemv(rng, "proj4096", 4096, k, 2, s=salient_count(0.05, k), ns=2)
    return Workload("proj_4096x4096", "4096x4096, 2 bases + 5% salient (2 refinement bases)", [g])


def mlp_7b(seed: int = 0) -> Workload:
    """7B-shaped MLP: up 4096 -> 11008 and down 11008 -> 4096, 2 bases + 3% salient with 1
    refinement base, fp16 x (down input ReLU'd), batch 1, 4, 8 (x drawn at batch 8)."""
    rng = np.random.default_rng(seed)
    up = make_gemv(rng, "up", 11008, 4096, 2, s=salient_count(0.03, 4096), ns=1, batch=8)
    down = make_gemv(rng, "down", 4096, 11008, 2, s=salient_count(0.03, 11008), ns=1, batch=8, relu=True)
    return Workload("mlp_7b", "up 4096->11008, down 11008->4096", [up, down], batches=(1, 4, 8))


def decoder_layer_70b(seed: int = 0) -> Workload:
    """70B-shaped decoder layer: q, k, v, o, gate, up, down with 3 bases + 5% salient columns
    (2 refinement bases), fp16 x, batch 1 and 16 (x drawn at batch 16)."""
    rng = np.random.default_rng(seed)
    shapes = (("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192), ("o", 8192, 8192),
              ("gate", 28672, 8192), ("up", 28672, 8192), ("down", 8192, 28672))
    gs = [make_gemv(rng, nm, n, k, 3, s=salient_count(0.05, k), ns=2, batch=16) for nm, n, k in shapes]
    return Workload("layer_70b", "70B decoder layer, 7 GEMVs", gs, batches=(1, 16))


WORKLOADS = {f.__name__: f for f in (single_gemv_256x512, ternary_stack_256x768, attn_proj_7b, mlp_7b,
                                        decoder_layer_70b)}


def algorithmic_bytes(n: int, k: int, nb: int, batch: int, x_bytes: int, s: int = 0, ns: int = 0) -> int:
    """Bytes one call must move: packed sign bits, scale vectors, activations and outputs, plus
    the refinement branch (its bits, scales and the salient index list)."""
    b = nb * n * words_per_row(k) * 4 + nb * (n + k) * 4 + batch * k * x_bytes + batch * n * 4
    if s and ns:
        b += ns * n * words_per_row(s) * 4 + ns * (n + s) * 4 + 4 * s
    return b
