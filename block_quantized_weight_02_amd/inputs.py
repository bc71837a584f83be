"""Seeded synthetic inputs for the Q8_0 product, in the canonical layout.

This module only draws random numbers and lays them out; it holds none of the
product's arithmetic, and both the HIP path and the CPU oracle receive what it
returns.  Arrays are numpy, on the host:

* ``x``  -- ``m x K`` bf16 activation, as raw uint16 bit patterns;
* ``q``  -- ``K x N`` int8 weight values (k outer);
* ``s``  -- ``K/32 x N`` fp32 weight scales.

Generators are numpy ``default_rng([seed, j])`` streams with j = 0 for x,
1 for q, 2 for s, 3 for the zero mask.  The shapes are decoder projections of
7-13B-class models (decode: one row; batched decode: 16 rows; 32 rows of a
quantized activation); the laws stand in for real activations and weights.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

BLOCK = 32


@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    K: int
    N: int
    act: str            # "bf16" or "q8_0"
    seed_x: int
    seed_w: int
    x_law: str = "normal"          # "normal" | "normal_zeros30"
    q_law: str = "uniform"         # "uniform" | "block_max127"
    note: str = field(default="", compare=False)


# The workloads, by what they are.
WORKLOADS: Dict[str, Workload] = {
    "decode_k1024_n1024": Workload("decode_k1024_n1024", 1, 1024, 1024, "bf16", 1001, 1001,
                                   note="m=1 K=1024 N=1024, small parity case"),
    "decode_k4096_n4096": Workload("decode_k4096_n4096", 1, 4096, 4096, "bf16", 1002, 1002,
                                   q_law="block_max127",
                                   note="m=1 decode projection, per-block max|q| = 127"),
    "ffn_down_k14336_n4096": Workload("ffn_down_k14336_n4096", 1, 14336, 4096, "bf16", 1003, 1003,
                                      x_law="normal_zeros30",
                                      note="m=1 FFN down-projection, 30% zero activations"),
    "batch16_k4096_n14336": Workload("batch16_k4096_n14336", 16, 4096, 14336, "bf16", 1004, 1004,
                                     note="m=16 batched decode gate/up projection"),
    "q8act_m32_k5120_n40": Workload("q8act_m32_k5120_n40", 32, 5120, 40, "q8_0", 1005, 10051,
                                    note="m=32 Q8_0 activations, N=40 padded to 64"),
    "q8act_m32_k5120_n32000": Workload("q8act_m32_k5120_n32000", 32, 5120, 32000, "q8_0", 1005, 10052,
                                       note="m=32 Q8_0 activations, vocabulary-wide N"),
    "decode_k4096_n14336": Workload("decode_k4096_n14336", 1, 4096, 14336, "bf16", 1006, 1006,
                                    note="m=1 decode gate/up projection, the headline shape"),
    "prefill_m512_k4096_n14336": Workload("prefill_m512_k4096_n14336", 512, 4096, 14336, "bf16",
                                          1007, 1007,
                                          note="m=512 prefill chunk through the gate/up projection"),
    "prefill_q8act_m512_k4096_n14336": Workload("prefill_q8act_m512_k4096_n14336", 512, 4096, 14336,
                                                "q8_0", 1008, 1008,
                                                note="the same chunk with Q8_0 activations"),
    "prefill_m128_k4096_n14336": Workload("prefill_m128_k4096_n14336", 128, 4096, 14336, "bf16",
                                          1013, 1013,
                                          note="m=128 prefill chunk (the tile kernel's row chunks)"),
    "prefill_q8act_m128_k4096_n14336": Workload("prefill_q8act_m128_k4096_n14336", 128, 4096,
                                                14336, "q8_0", 1014, 1014,
                                                note="the m=128 chunk with Q8_0 activations"),
}

HEADLINE = "decode_k4096_n14336"


@dataclass(frozen=True)
class PartsWorkload:
    """Several projections of one activation (one launch in parts)."""
    name: str
    m: int
    K: int
    Ns: tuple
    act: str
    seed_x: int
    seed_w: int
    note: str = field(default="", compare=False)


# The attention's query, key and value projections of the same decoder
# (hidden 4096, 32 query heads and 8 key/value heads of 128).
PARTS_WORKLOADS: Dict[str, PartsWorkload] = {
    "qkv_decode_k4096": PartsWorkload("qkv_decode_k4096", 1, 4096, (4096, 1024, 1024), "bf16",
                                      1009, 1009, note="m=1 decode q/k/v projections"),
    "qkv_batch16_k4096": PartsWorkload("qkv_batch16_k4096", 16, 4096, (4096, 1024, 1024), "bf16",
                                       1010, 1010, note="m=16 batched decode q/k/v projections"),
    "qkv_q8act_m32_k4096": PartsWorkload("qkv_q8act_m32_k4096", 32, 4096, (4096, 1024, 1024),
                                         "q8_0", 1011, 1011,
                                         note="m=32 Q8_0 activations, q/k/v projections"),
    "qkv_prefill_m512_k4096": PartsWorkload("qkv_prefill_m512_k4096", 512, 4096,
                                            (4096, 1024, 1024), "bf16", 1012, 1012,
                                            note="m=512 prefill chunk, q/k/v projections"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, j: int) -> np.random.Generator:
    return np.random.default_rng([seed, j])


def gen_x(m: int, K: int, seed: int, law: str = "normal") -> np.ndarray:
    z = _rng(seed, 0).standard_normal((m, K), dtype=np.float32)
    if law == "normal_zeros30":
        mask = _rng(seed, 3).random((m, K)) < 0.30
        z = np.where(mask, np.float32(0.0), z)
    elif law != "normal":
        raise ValueError(law)
    return f32_to_bf16_bits(z)


def gen_scales(K: int, N: int, seed: int) -> np.ndarray:
    u = _rng(seed, 2).uniform(np.log(1e-4), np.log(1e-2), size=(K // BLOCK, N))
    return np.exp(u).astype(np.float32)


def gen_q(K: int, N: int, seed: int, law: str = "uniform") -> np.ndarray:
    if law == "uniform":
        return _rng(seed, 1).integers(-127, 128, size=(K, N), dtype=np.int8)
    if law == "block_max127":
        # Per block and column: z ~ N(0,1) scaled so the block's largest |z|
        # maps to 127, rounded half away from zero, the largest forced to +-127.
        z = _rng(seed, 1).standard_normal((K // BLOCK, BLOCK, N))
        amax = np.abs(z).max(axis=1, keepdims=True)
        v = z * (127.0 / amax)
        q = np.sign(v) * np.floor(np.abs(v) + 0.5)
        arg = np.abs(z).argmax(axis=1)
        bi, ni = np.meshgrid(np.arange(K // BLOCK), np.arange(N), indexing="ij")
        q[bi, arg, ni] = np.sign(z[bi, arg, ni]) * 127.0
        return np.clip(q, -127, 127).astype(np.int8).reshape(K, N)
    raise ValueError(law)


def generate(w: Workload, n_cols: Optional[int] = None):
    """``(x, q, s)`` for a workload (``n_cols`` truncates N for quick checks)."""
    N = w.N if n_cols is None else n_cols
    x = gen_x(w.m, w.K, w.seed_x, w.x_law)
    q = gen_q(w.K, N, w.seed_w, w.q_law)
    s = gen_scales(w.K, N, w.seed_w)
    return x, q, s


def random_case(m: int, K: int, N: int, seed: int, q_law: str = "uniform",
                x_law: str = "normal"):
    """A small seeded case of any shape: ``(x, q, s)``."""
    return gen_x(m, K, seed, x_law), gen_q(K, N, seed, q_law), gen_scales(K, N, seed)


def gen_bias(N: int, seed: int) -> np.ndarray:
    """fp32 bias of N columns, N(0, 1)."""
    return _rng(seed, 4).standard_normal(N, dtype=np.float32)


def gen_residual(m: int, Npad: int, seed: int) -> np.ndarray:
    """fp32 residual stream, ``m x Npad``, N(0, 8^2) (the order of a
    projection's output at K = 4096 with the weights above)."""
    return (_rng(seed, 5).standard_normal((m, Npad), dtype=np.float32) * 8).astype(np.float32)


def exact_case(m: int, K: int, N: int, seed: int):
    """A case whose product, bias and residual are exact in fp32 whatever the
    summation order, so every rounding-free path gives bit-identical outputs:
    ``(x, q, s, bias, residual)``.

    * x: integers in [-127, 127], each 32-block holding +-127 (so its int8
      quantized form is x itself with scale 1), stored as bf16 bits;
    * q: integers in [-15, 15]; columns 32..63 zero (a zero output block);
    * s: powers of two 2^-4 .. 2^-1;
    * bias, residual: multiples of 2^-4 below 2^10 in magnitude, zero on
      columns 32..63.
    With K <= 512 every partial sum is a multiple of 2^-4 below 2^20.
    """
    if K > 512:
        raise ValueError("exact_case needs K <= 512")
    r = _rng(seed, 6)
    x = r.integers(-126, 127, size=(m, K)).astype(np.float32)
    pos = r.integers(0, BLOCK, size=(m, K // BLOCK))
    sign = np.where(r.random((m, K // BLOCK)) < 0.5, -1.0, 1.0)
    for b in range(K // BLOCK):
        x[np.arange(m), b * BLOCK + pos[:, b]] = 127.0 * sign[:, b]
    q = r.integers(-15, 16, size=(K, N)).astype(np.int8)
    q[:, 32:64] = 0
    s = np.ldexp(1.0, r.integers(-4, 0, size=(K // BLOCK, N))).astype(np.float32)
    Npad = (N + 63) // 64 * 64
    bias = (r.integers(-2 ** 13, 2 ** 13, size=N) / 16.0).astype(np.float32)
    res = (r.integers(-2 ** 13, 2 ** 13, size=(m, Npad)) / 16.0).astype(np.float32)
    bias[32:64] = 0
    res[:, 32:64] = 0
    return f32_to_bf16_bits(x), q, s, bias, res


def generate_pair(w: Workload, n_cols: Optional[int] = None):
    """``(x, qg, sg, qu, su)``: a workload's activation and two weights of its
    shape (a gate and an up projection), the up weight from seed_w + 500000."""
    x, qg, sg = generate(w, n_cols)
    N = w.N if n_cols is None else n_cols
    qu = gen_q(w.K, N, w.seed_w + 500000, w.q_law)
    su = gen_scales(w.K, N, w.seed_w + 500000)
    return x, qg, sg, qu, su


def generate_parts(w: PartsWorkload):
    """``(x, [(q_i, s_i), ...])``: a parts workload's activation and one weight
    per part, part i's from seed_w + 100000 * i."""
    x = gen_x(w.m, w.K, w.seed_x, "normal")
    ws = [(gen_q(w.K, N, w.seed_w + 100000 * i, "uniform"),
           gen_scales(w.K, N, w.seed_w + 100000 * i)) for i, N in enumerate(w.Ns)]
    return x, ws
