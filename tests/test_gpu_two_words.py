"""Parity of the two-word int8 activation path (the two-pass numerics) with the
oracle, through the C ABI.

plan.rs, enum Q8MatKind, variant TwoPassInt8, and struct Buffer field
`quantized`: two int8 words a value and one scale per 32.  The split is this
library's reading (first word and scale as the one-word form, second word the
residual in steps of d/128); the oracle implements the same reading.  The
bar: the words and scales bit-exact, each word's block dots bit-exact, the
product within 1e-5 * sum_k |x_k w_kn| + 1e-6 with x_k = dx * (hi + lo/128).
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_02_amd as q8
import oracle
from block_quantized_weight_02_amd import inputs

pytestmark = pytest.mark.gpu

from tests import gpu_util as g  # noqa: E402

TW = q8.Q8_ACT_Q8_0_TWO_WORDS
REL, ABS = 1e-5, 1e-6


def quantize2(x_bits, pad_rows=False):
    """The two-word buffer of x on the device (optionally inside a buffer the
    size of a 2m-row one-word activation, which the one-word dots read)."""
    m, K = x_bits.shape
    n = q8.q8_act_bytes(2 * m, K) if pad_rows else q8.q8_act_two_words_bytes(m, K)
    buf = g.empty_bytes(n)
    buf.fill_(0x77)
    q8.q8_quantize_act_two_words(g.dev(x_bits.view(np.int16)), buf, m, K)
    torch.cuda.synchronize()
    return buf


def words_host(buf, m, K):
    raw = buf.cpu().numpy()
    hi = raw[: m * K].view(np.int8).reshape(m, K)
    lo = raw[m * K: 2 * m * K].view(np.int8).reshape(m, K)
    off = q8.q8_act_two_words_scales_offset(m, K)
    dx = raw[off: off + m * (K // 32) * 4].view(np.float32).reshape(m, K // 32)
    return hi, lo, dx


def gemv2(buf, Wq, Ws, m, K, N, plan=None):
    return g.gemv(buf, Wq, Ws, m, K, N, TW, plan)


def check(y, z, bnd, N, what):
    err = np.abs(y[:, :N].astype(np.float64) - z)
    lim = REL * bnd + ABS
    assert np.all(err <= lim), f"{what}: max err/lim {np.max(err / lim):.3g}"
    assert (y[:, N:].view(np.uint32) == 0).all(), f"{what}: pad columns not zero"


@pytest.mark.parametrize("m,K", [(1, 64), (3, 2176), (16, 4096), (5, 32), (40, 1024)])
def test_quantize_two_words_bit_exact(m, K):
    x, _, _ = inputs.random_case(m, K, 1, seed=800 + m)
    x[0, :32] = 0                                   # a zero block
    buf = quantize2(x)
    hi, lo, dx = words_host(buf, m, K)
    rh, rl, rd = oracle.quantize_act_two_words(x)
    np.testing.assert_array_equal(hi, rh)
    np.testing.assert_array_equal(lo, rl)
    np.testing.assert_array_equal(dx.view(np.uint32), rd.view(np.uint32))


def test_quantize_two_words_ties():
    # a block with d = 2^-7 holding values whose residuals tie (see the oracle pins)
    v = np.array([127 * 128, 133, 253, -253, 320, -320, 2.5, -2.5, 0], np.float64)
    row = np.zeros(64, np.float32)
    row[:len(v)] = v * 2.0 ** -14
    x = inputs.f32_to_bf16_bits(row)[None, :]
    hi, lo, dx = words_host(quantize2(x), 1, 64)
    rh, rl, rd = oracle.quantize_act_two_words(x)
    np.testing.assert_array_equal(hi, rh)
    np.testing.assert_array_equal(lo, rl)
    np.testing.assert_array_equal(dx.view(np.uint32), rd.view(np.uint32))
    assert list(lo[0, :len(v)]) == [0, 5, -3, 3, -64, 64, 3, -3, 0]


@pytest.mark.parametrize("m,K,N", [(2, 2176, 200), (8, 1024, 96)])
def test_two_word_dots_bit_exact(m, K, N):
    """Each word's int32 block dots: the two-word buffer read as the 2m rows
    of a one-word buffer."""
    x, q, s = inputs.random_case(m, K, N, seed=810 + m)
    buf = quantize2(x, pad_rows=True)
    hi, lo, _ = words_host(buf, m, K)
    Wq, _ = g.pack(q, s)
    # a kernel that reads the rows (the two-word buffer has no block view)
    d = g.block_dots(buf, Wq, 2 * m, K, N, g.plan(q8.Q8_KERNEL_MFMA, 16, 1, 16))
    np.testing.assert_array_equal(d[:m, :, :N], oracle.block_dots(hi, q))
    np.testing.assert_array_equal(d[m:, :, :N], oracle.block_dots(lo, q))


PLANS = [None, (q8.Q8_KERNEL_MFMA, 32, 1, 16), (q8.Q8_KERNEL_MFMA, 32, 3, 8),
         (q8.Q8_KERNEL_MFMA, 32, 2, 4)]


@pytest.mark.parametrize("pl", PLANS)
@pytest.mark.parametrize("m", [1, 3, 8, 16])
@pytest.mark.parametrize("N", [200, 40])
def test_gemv_two_words(m, N, pl):
    K = 2176
    x, q, s = inputs.random_case(m, K, N, seed=820 + m + N)
    buf = quantize2(x)
    Wq, Ws = g.pack(q, s)
    y = gemv2(buf, Wq, Ws, m, K, N, None if pl is None else g.plan(*pl))
    hi, lo, dx = words_host(buf, m, K)
    z, bnd = oracle.gemv_q8_two_words(hi, lo, dx, q, s)
    check(y, z, bnd, N, f"m={m} N={N} plan={pl}")


# The VALU kernel's two-word form (few rows): (m, rows, split_k, waves).
VALU_PLANS = [(1, 1, 1, 8), (1, 1, 3, 4), (2, 2, 2, 16), (3, 4, 1, 16), (4, 4, 3, 8)]


@pytest.mark.parametrize("m,rows,split,waves", VALU_PLANS)
@pytest.mark.parametrize("N", [200, 40])
def test_gemv_two_words_valu(m, rows, split, waves, N):
    K = 2176
    x, q, s = inputs.random_case(m, K, N, seed=850 + m + N)
    buf = quantize2(x)
    Wq, Ws = g.pack(q, s)
    y = gemv2(buf, Wq, Ws, m, K, N, g.plan(q8.Q8_KERNEL_VALU, rows, split, waves))
    hi, lo, dx = words_host(buf, m, K)
    z, bnd = oracle.gemv_q8_two_words(hi, lo, dx, q, s)
    check(y, z, bnd, N, f"VALU m={m} N={N} rows={rows} split={split} waves={waves}")


def test_two_words_valu_exact_case():
    # exact-integer inputs (d = 1, lo = 0): every sum exact in any order
    for m, waves, split in ((1, 8, 1), (2, 16, 2)):
        x, q, s, _, _ = inputs.exact_case(m, 512, 100, seed=38 + m)
        buf = quantize2(x)
        hi, lo, dx = words_host(buf, m, 512)
        assert (lo == 0).all() and (dx == 1.0).all()
        Wq, Ws = g.pack(q, s)
        y = gemv2(buf, Wq, Ws, m, 512, 100, g.plan(q8.Q8_KERNEL_VALU, m, split, waves))
        z, _ = oracle.gemv_q8_two_words(hi, lo, dx, q, s)
        np.testing.assert_array_equal(y[:, :100].astype(np.float64), z)


def test_two_words_one_block_and_exact_case():
    m, K, N = 3, 32, 70
    x, q, s = inputs.random_case(m, K, N, seed=830)
    buf = quantize2(x)
    Wq, Ws = g.pack(q, s)
    y = gemv2(buf, Wq, Ws, m, K, N)
    z, bnd = oracle.gemv_q8_two_words(*words_host(buf, m, K), q, s)
    check(y, z, bnd, N, "K=32")
    # exact-integer inputs: d = 1 and lo = 0 for every block, every sum exact
    x, q, s, _, _ = inputs.exact_case(3, 512, 100, seed=37)
    buf = quantize2(x)
    hi, lo, dx = words_host(buf, 3, 512)
    assert (lo == 0).all() and (dx == 1.0).all()
    Wq, Ws = g.pack(q, s)
    y = gemv2(buf, Wq, Ws, 3, 512, 100)
    z, _ = oracle.gemv_q8_two_words(hi, lo, dx, q, s)
    np.testing.assert_array_equal(y[:, :100].astype(np.float64), z)


def test_two_words_close_to_bf16_product():
    """The second word buys back most of the one-word quantizer's error."""
    m, K, N = 4, 4096, 256
    x, q, s = inputs.random_case(m, K, N, seed=840)
    Wq, Ws = g.pack(q, s)
    y2 = gemv2(quantize2(x), Wq, Ws, m, K, N)
    y1 = g.gemv(g.quantize(x), Wq, Ws, m, K, N, q8.Q8_ACT_Q8_0)
    yb, bnd = oracle.gemv_bf16(x, q, s)
    e2 = np.abs(y2[:, :N] - yb).max()
    e1 = np.abs(y1[:, :N] - yb).max()
    assert e2 < e1 / 20, (e1, e2)


def test_two_words_fused_epilogue():
    m, K, N = 5, 1024, 300
    x, q, s = inputs.random_case(m, K, N, seed=850)
    Npad = q8.q8_padded_cols(N)
    bias = inputs.gen_bias(N, seed=851)
    res = inputs.gen_residual(m, Npad, seed=852)
    buf = quantize2(x)
    Wq, Ws = g.pack(q, s)
    y = torch.full((m, Npad), float("nan"), dtype=torch.float32, device=g.DEV)
    y.copy_(g.dev(res))
    ep = q8.make_epilogue(bias=g.dev(bias), residual=y)
    q8.q8_gemv_fused(buf, Wq, Ws, y, m, K, N, TW, ep)
    torch.cuda.synchronize()
    z, bnd = oracle.gemv_q8_two_words(*words_host(buf, m, K), q, s)
    z = z + bias[None, :].astype(np.float64) + res[:, :N].astype(np.float64)
    bnd = bnd + np.abs(bias)[None, :] + np.abs(res[:, :N])
    check(y.cpu().numpy(), z, bnd, N, "bias + residual in place")


@pytest.mark.parametrize("name", ["decode_k4096_n14336", "batch16_k4096_n14336"])
def test_full_size_two_words(name):
    w = inputs.WORKLOADS[name]
    x, q, s = inputs.generate(w)
    m, K, N = w.m, w.K, w.N
    buf = quantize2(x)
    Wq, Ws = g.pack(q, s)
    y = gemv2(buf, Wq, Ws, m, K, N)
    blocks = np.random.default_rng(w.seed_x + 17).choice(N // 32, size=32, replace=False)
    cols = np.sort((blocks[:, None] * 32 + np.arange(32)[None, :]).ravel())
    hi, lo, dx = words_host(buf, m, K)
    z, bnd = oracle.gemv_q8_two_words(hi, lo, dx, q, s, cols)
    err = np.abs(y[:, cols].astype(np.float64) - z)
    lim = REL * bnd + ABS
    assert np.all(err <= lim), f"{name}: max err/lim {np.max(err / lim):.3g}"


# ------------------------------------------------------------------------------
# the many-row product (q8_gemm) over two-word activations
# ------------------------------------------------------------------------------

def gemm2(buf, Wq, Ws, m, K, N):
    y = torch.full((m, q8.q8_padded_cols(N)), float("nan"), dtype=torch.float32, device=g.DEV)
    q8.q8_gemm(buf, Wq, Ws, y, m, K, N, TW)
    torch.cuda.synchronize()
    return y.cpu().numpy()


GEMM_SHAPES = [(m, K, N) for m in (1, 17, 64, 65, 200) for (K, N) in ((32, 1), (1056, 200), (2176, 257))]


@pytest.mark.parametrize("m,K,N", GEMM_SHAPES)
def test_gemm_two_words(m, K, N):
    x, q, s = inputs.random_case(m, K, N, seed=860 + m + K + N)
    buf = quantize2(x)
    Wq, Ws = g.pack(q, s)
    y = gemm2(buf, Wq, Ws, m, K, N)
    z, bnd = oracle.gemv_q8_two_words(*words_host(buf, m, K), q, s)
    check(y, z, bnd, N, f"gemm two words m={m} K={K} N={N}")


def test_gemm_two_words_most_rows_and_exact():
    m, K, N = q8.Q8_MAX_GEMM_ROWS, 256, 130
    x, q, s = inputs.random_case(m, K, N, seed=870)
    buf = quantize2(x)
    Wq, Ws = g.pack(q, s)
    y = gemm2(buf, Wq, Ws, m, K, N)
    z, bnd = oracle.gemv_q8_two_words(*words_host(buf, m, K), q, s)
    check(y, z, bnd, N, "gemm two words m=8192")
    x, q, s, _, _ = inputs.exact_case(70, 512, 100, seed=38)
    buf = quantize2(x)
    Wq, Ws = g.pack(q, s)
    y = gemm2(buf, Wq, Ws, 70, 512, 100)
    z, _ = oracle.gemv_q8_two_words(*words_host(buf, 70, 512), q, s)
    np.testing.assert_array_equal(y[:, :100].astype(np.float64), z)


def test_gemm_two_words_prefill_full_size():
    w = inputs.WORKLOADS["prefill_q8act_m512_k4096_n14336"]
    x, q, s = inputs.generate(w)
    m, K, N = w.m, w.K, w.N
    buf = quantize2(x)
    Wq, Ws = g.pack(q, s)
    y = gemm2(buf, Wq, Ws, m, K, N)
    blocks = np.random.default_rng(w.seed_x + 19).choice(N // 32, size=16, replace=False)
    cols = np.sort((blocks[:, None] * 32 + np.arange(32)[None, :]).ravel())
    z, bnd = oracle.gemv_q8_two_words(*words_host(buf, m, K), q, s, cols)
    err = np.abs(y[:, cols].astype(np.float64) - z)
    assert np.all(err <= REL * bnd + ABS), np.max(err / (REL * bnd + ABS))
