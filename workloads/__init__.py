"""Seeded synthetic inputs for the FP8 prefill matmul path.

This module only draws random data of the shapes and distributions the
workloads call for.  It contains none of the method's arithmetic (no
dequantisation, no absmax, no scaling, no encoding, no matmul), so both the
CPU oracle's tests and the GPU path's tests/bench can use it without sharing
any of the computation under test.

Every generator takes an explicit seed and uses
``numpy.random.Generator(PCG64(seed))``.  Seeds follow
``1000*cfg + 10*layer + slot`` with slots Q=0, K=1, V=2, O=3, gate=4, up=5,
down=6 and activation inputs 7/8/9.

Block byte layouts follow the public GGUF K-quant super-block formats (the
pages only fix their sizes: 144 bytes per 256 Q4_K weights; Q6_K is 210
bytes per 256 weights):

* Q4_K (144 B): f16 ``d`` | f16 ``dmin`` | 12 bytes of packed 6-bit
  sub-block scales and mins | 128 bytes of 4-bit quants.
* Q6_K (210 B): 128 bytes low 4 bits | 64 bytes high 2 bits |
  16 int8 sub-block scales | f16 ``d``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

QK_K = 256
Q4_K = 12  # GGML type ids
Q6_K = 14
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210}
QTYPE_NAMES = {Q4_K: "Q4_K", Q6_K: "Q6_K"}

SLOT = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6,
        "x_attn": 7, "x_ffn": 8, "x_down": 9}


def seed_for(cfg: int, layer: int, slot: str | int) -> int:
    s = SLOT[slot] if isinstance(slot, str) else int(slot)
    return 1000 * cfg + 10 * layer + s


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _f16_uniform(g: np.random.Generator, count: int, lo=1e-3, hi=2e-2) -> np.ndarray:
    return g.uniform(lo, hi, size=count).astype(np.float16)


def q4k_blocks(seed: int, n: int, k: int) -> np.ndarray:
    """Random Q4_K weight of logical shape [n][k] as uint8 [n*(k/256), 144].

    d, dmin ~ f16(U[1e-3, 2e-2]); the 12 scale bytes and 128 quant bytes are
    uniform bytes, so every 6-bit field and every nibble is uniform.
    """
    assert k % QK_K == 0
    nb = n * (k // QK_K)
    g = rng(seed)
    out = np.empty((nb, 144), dtype=np.uint8)
    out[:, 0:2] = _f16_uniform(g, nb).view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = _f16_uniform(g, nb).view(np.uint8).reshape(nb, 2)
    out[:, 4:144] = g.integers(0, 256, size=(nb, 140), dtype=np.uint8)
    return out


def q6k_blocks(seed: int, n: int, k: int) -> np.ndarray:
    """Random Q6_K weight of logical shape [n][k] as uint8 [n*(k/256), 210].

    ql, qh uniform bytes; the 16 sub-block scales uniform int8 over
    -128..127; d ~ f16(U[1e-3, 2e-2]).
    """
    assert k % QK_K == 0
    nb = n * (k // QK_K)
    g = rng(seed)
    out = np.empty((nb, 210), dtype=np.uint8)
    out[:, 0:208] = g.integers(0, 256, size=(nb, 208), dtype=np.uint8)
    out[:, 208:210] = _f16_uniform(g, nb).view(np.uint8).reshape(nb, 2)
    return out


def weight_blocks(qtype: int, seed: int, n: int, k: int) -> np.ndarray:
    if qtype == Q4_K:
        return q4k_blocks(seed, n, k)
    if qtype == Q6_K:
        return q6k_blocks(seed, n, k)
    raise ValueError(f"unsupported qtype {qtype}")


def act_normal(seed: int, m: int, k: int) -> np.ndarray:
    """fp32 N(0,1) activations [m][k]."""
    return rng(seed).standard_normal((m, k), dtype=np.float32)


def act_silu_gated(seed: int, m: int, k: int) -> np.ndarray:
    """fp32 SiLU(g)*u with g, u ~ N(0,1): the shape of an FFN down input."""
    g = rng(seed)
    a = g.standard_normal((m, k)).astype(np.float64)
    b = g.standard_normal((m, k)).astype(np.float64)
    return (a / (1.0 + np.exp(-a)) * b).astype(np.float32)


def act_student_t(seed: int, m: int, k: int, nu: float = 3.0,
                  n_outlier_channels: int = 8, outlier_scale: float = 100.0) -> np.ndarray:
    """fp32 Student-t(nu) activations with a few channels scaled up.

    Heavy tails plus outlier channels push most values below 2^-6 after
    absmax scaling, which exercises the encoder's flush-to-zero band.
    """
    g = rng(seed)
    x = g.standard_t(nu, size=(m, k))
    ch = g.choice(k, size=min(n_outlier_channels, k), replace=False)
    x[:, ch] *= outlier_scale
    return x.astype(np.float32)


def act_zero(m: int, k: int) -> np.ndarray:
    return np.zeros((m, k), dtype=np.float32)


# --------------------------------------------------------------------------
# Workload catalogue (shapes of the five configurations)
# --------------------------------------------------------------------------

HIDDEN, KV_DIM, FFN = 3584, 512, 18944


@dataclass
class Gemm:
    name: str
    qtype: int
    n: int
    k: int
    w_seed: int


@dataclass
class Group:
    """GEMMs that share one activation quantisation."""
    m: int
    k: int
    act_kind: str  # normal | silu | student_t | zero
    act_seed: int
    gemms: list = field(default_factory=list)

    def activation(self) -> np.ndarray:
        if self.act_kind == "normal":
            return act_normal(self.act_seed, self.m, self.k)
        if self.act_kind == "silu":
            return act_silu_gated(self.act_seed, self.m, self.k)
        if self.act_kind == "student_t":
            return act_student_t(self.act_seed, self.m, self.k)
        if self.act_kind == "zero":
            return act_zero(self.m, self.k)
        raise ValueError(self.act_kind)


def config_groups(cfg: int, layer: int = 0, m: int | None = None) -> list[Group]:
    """The GEMM groups of one configuration (one layer for the sweep)."""
    if cfg == 1:
        return [Group(16, 512, "normal", seed_for(1, 0, "x_attn"),
                      [Gemm("w", Q4_K, 256, 512, seed_for(1, 0, "q"))])]
    if cfg == 2:
        return [Group(512, HIDDEN, "normal", seed_for(2, 0, "x_attn"), [
            Gemm("q", Q4_K, HIDDEN, HIDDEN, seed_for(2, 0, "q")),
            Gemm("k", Q4_K, KV_DIM, HIDDEN, seed_for(2, 0, "k")),
            Gemm("v", Q6_K, KV_DIM, HIDDEN, seed_for(2, 0, "v"))])]
    if cfg == 3:
        return [Group(2048, HIDDEN, "normal", seed_for(3, 0, "x_ffn"), [
                    Gemm("gate", Q4_K, FFN, HIDDEN, seed_for(3, 0, "gate")),
                    Gemm("up", Q4_K, FFN, HIDDEN, seed_for(3, 0, "up"))]),
                Group(2048, FFN, "silu", seed_for(3, 0, "x_down"), [
                    Gemm("down", Q6_K, HIDDEN, FFN, seed_for(3, 0, "down"))])]
    if cfg == 4:
        L = layer
        return [Group(4096, HIDDEN, "normal", seed_for(4, L, "x_attn"), [
                    Gemm("q", Q4_K, HIDDEN, HIDDEN, seed_for(4, L, "q")),
                    Gemm("k", Q4_K, KV_DIM, HIDDEN, seed_for(4, L, "k")),
                    Gemm("v", Q6_K, KV_DIM, HIDDEN, seed_for(4, L, "v"))]),
                Group(4096, HIDDEN, "normal", seed_for(4, L, "o") + 100000, [
                    Gemm("o", Q4_K, HIDDEN, HIDDEN, seed_for(4, L, "o"))]),
                Group(4096, HIDDEN, "normal", seed_for(4, L, "x_ffn"), [
                    Gemm("gate", Q4_K, FFN, HIDDEN, seed_for(4, L, "gate")),
                    Gemm("up", Q4_K, FFN, HIDDEN, seed_for(4, L, "up"))]),
                Group(4096, FFN, "silu", seed_for(4, L, "x_down"), [
                    Gemm("down", Q6_K, HIDDEN, FFN, seed_for(4, L, "down"))])]
    if cfg == 5:
        mm = 37 if m is None else m
        return [Group(mm, HIDDEN, "student_t", seed_for(5, 0, "x_attn") + mm, [
            Gemm("w", Q4_K, 4608, HIDDEN, seed_for(5, 0, "q"))])]
    raise ValueError(f"unknown configuration {cfg}")


CFG5_M = (1, 4, 37, 1000)
CFG4_LAYERS = 28


def gemm_flops(m: int, n: int, k: int) -> float:
    return 2.0 * m * n * k
