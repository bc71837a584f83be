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


# ------------------------------------------------------------------------------
# the gated pair and the parts over two-word activations
# ------------------------------------------------------------------------------

def _words_checked(x):
    """The device two-word buffer of x, its words checked bit for bit against
    the oracle's quantizer, and the oracle's words (the references use them)."""
    m, K = x.shape
    buf = quantize2(x)
    hi, lo, dx = words_host(buf, m, K)
    rh, rl, rd = oracle.quantize_act_two_words(x)
    np.testing.assert_array_equal(hi, rh)
    np.testing.assert_array_equal(lo, rl)
    np.testing.assert_array_equal(dx.view(np.uint32), rd.view(np.uint32))
    return buf, (rh, rl, rd)


PAIR_PLANS = [(1, None), (2, None), (3, None), (16, None),
              (1, (q8.Q8_KERNEL_VALU, 1, 2, 8, 1)),
              (4, (q8.Q8_KERNEL_VALU, 4, 1, 16, 1)),
              (8, (q8.Q8_KERNEL_MFMA, 32, 1, 8, 1)),
              (16, (q8.Q8_KERNEL_MFMA, 32, 3, 16, 1))]


@pytest.mark.parametrize("m,pl", PAIR_PLANS)
@pytest.mark.parametrize("N", [200, 40])
def test_gated_pair_two_words(m, pl, N):
    from tests.test_gpu_glu import glu_tolerance, run_glu
    from tests.test_gpu_epilogue import check_quant
    K = 2176
    x, qg, sg = inputs.random_case(m, K, N, seed=900 + m + N)
    _, qu, su = inputs.random_case(m, K, N, seed=950 + m + N)
    bg = inputs.gen_bias(N, seed=901)
    bu = inputs.gen_bias(N, seed=902)
    buf, (rh, rl, rd) = _words_checked(x)
    W = (*g.pack(qg, sg), *g.pack(qu, su))
    plan = None if pl is None else g.plan(*pl)
    y, codes, scales = run_glu(buf, W, m, K, N, TW, bg, bu, quant=True, plan=plan)
    gg, bnd_g = oracle.gemv_q8_two_words(rh, rl, rd, qg, sg)
    uu, bnd_u = oracle.gemv_q8_two_words(rh, rl, rd, qu, su)
    out = oracle.swiglu(gg, uu, bg, bu)
    tol = glu_tolerance(gg, uu, bnd_g, bnd_u, bg, bu, out)
    err = np.abs(y[:, :N].astype(np.float64) - out)
    what = f"pair m={m} plan={pl} N={N}"
    assert np.all(err <= tol), f"{what}: max err/tol {np.max(err / tol):.3g}"
    assert (y[:, N:].view(np.uint32) == 0).all(), f"{what}: pad columns not zero"
    check_quant(codes, scales, out, (tol - ABS) / REL, N, what)


PARTS_PLANS = [(1, None), (2, None), (5, None), (16, None),
               (2, (q8.Q8_KERNEL_VALU, 2, 1, 8, 1)),
               (4, (q8.Q8_KERNEL_VALU, 4, 3, 4, 1)),
               (16, (q8.Q8_KERNEL_MFMA, 32, 2, 16, 1))]


@pytest.mark.parametrize("m,pl", PARTS_PLANS)
@pytest.mark.parametrize("Ns", [(200, 40, 64, 130), (96,)])
def test_parts_two_words(m, pl, Ns):
    from tests.test_gpu_parts import run_parts, check_part
    K = 2176
    seed = 980 + m + sum(Ns)
    x = inputs.gen_x(m, K, seed)
    ws = [(inputs.gen_q(K, N, seed + 10 * i + 1), inputs.gen_scales(K, N, seed + 10 * i + 1))
          for i, N in enumerate(Ns)]
    biases = [inputs.gen_bias(N, seed=seed + i) if i % 2 == 0 else None
              for i, N in enumerate(Ns)]
    buf, (rh, rl, rd) = _words_checked(x)
    packed = [g.pack(q, s) for q, s in ws]
    plan = None if pl is None else g.plan(*pl)
    ys = run_parts(buf, packed, Ns, biases, m, K, TW, plan)
    for i, ((q, s), N, b, y) in enumerate(zip(ws, Ns, biases, ys)):
        z, bnd = oracle.gemv_q8_two_words(rh, rl, rd, q, s)
        z, bnd = oracle.epilogue(z, bnd, b)
        check_part(y, z, bnd, N, f"part {i} m={m} plan={pl} Ns={Ns}")


def test_parts_two_words_match_single_products():
    """Each part equals the single two-word product under the same plan, bit
    for bit (the parts launch walks the same units)."""
    m, K, Ns = 3, 1024, (130, 64)
    x = inputs.gen_x(m, K, 991)
    ws = [(inputs.gen_q(K, N, 992 + i), inputs.gen_scales(K, N, 992 + i)) for i, N in enumerate(Ns)]
    buf, _ = _words_checked(x)
    packed = [g.pack(q, s) for q, s in ws]
    from tests.test_gpu_parts import run_parts
    for pl in ((q8.Q8_KERNEL_VALU, 4, 1, 8, 1), (q8.Q8_KERNEL_MFMA, 32, 1, 16, 1)):
        ys = run_parts(buf, packed, Ns, [None] * len(Ns), m, K, TW, g.plan(*pl))
        for (W, Ws), N, y in zip(packed, Ns, ys):
            y1 = g.gemv(buf, W, Ws, m, K, N, TW, g.plan(*pl))
            np.testing.assert_array_equal(y.view(np.uint32), y1.view(np.uint32))
