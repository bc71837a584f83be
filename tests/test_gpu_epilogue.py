"""Parity of the fused epilogue (bias, residual, quantized output) with the
oracle, through the C ABI.

What the epilogue computes is z = x.W + bias + residual per output, then y = z
and/or z's quantized form per 32 columns (the pages' plan.rs, enum Launch,
variant Gemv, fields `bias` and `quant`; the residual add of its
`gemv_norm_epilogue` note).  The oracle gives x.W and its bound in fp64 and
adds bias and residual (its epilogue), and quantizes with its own fp32-input
quantizer.

The bar:
* exact cases (inputs whose sums are exact in fp32 in any order): y, the
  int8 codes and the scales bit-exact;
* random cases: y within 1e-5 * (sum_k |x_k w_kn| + |bias| + |residual|) + 1e-6;
  each block's scale within that tolerance of the oracle's amax / 127; each
  code within half a step (plus the tolerance) of z, so a code differs from
  the oracle's only where z lies within the tolerance of a rounding tie.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_02_amd as q8
import oracle
from block_quantized_weight_02_amd import inputs

pytestmark = pytest.mark.gpu

from tests import gpu_util as g  # noqa: E402

REL, ABS = 1e-5, 1e-6
BF16, Q8 = q8.Q8_ACT_BF16, q8.Q8_ACT_Q8_0


def run_fused(xin, Wq, Ws, m, K, N, act, bias=None, residual=None, quant=False,
              write_y=True, plan=None, alias=False):
    """One fused call; returns (y or None, codes or None, scales or None)."""
    Npad = q8.q8_padded_cols(N)
    b = g.dev(bias) if bias is not None else None
    if alias:
        y = g.dev(residual)
        r = y
    else:
        y = torch.full((m, Npad), float("nan"), dtype=torch.float32, device=g.DEV) \
            if write_y else None
        r = g.dev(residual) if residual is not None else None
    yq = None
    if quant:
        yq = g.empty_bytes(q8.q8_act_bytes(m, Npad))
        yq.fill_(0x5A)
    ep = q8.make_epilogue(bias=b, residual=r, y_q8=yq, write_y=write_y)
    if plan is None:
        q8.q8_gemv_fused(xin, Wq, Ws, y, m, K, N, act, ep)
    else:
        need = q8.q8_plan_workspace_bytes(plan, m, K, N)
        ws = torch.zeros(need, dtype=torch.uint8, device=g.DEV) if need else None
        q8.q8_gemv_planned_fused(xin, Wq, Ws, y, m, K, N, act, ep, plan, None, ws, need)
    torch.cuda.synchronize()
    yh = y.cpu().numpy() if y is not None else None
    if quant:
        codes, scales = g.act_host(yq, m, Npad)
        np.testing.assert_array_equal(g.act_view(yq, m, Npad), oracle.act_view_ref(codes),
                                      err_msg="quantized output's view")
        return yh, codes, scales
    return yh, None, None


def reference(x, q, s, act, xbuf=None, bias=None, residual=None, cols=None):
    """(z, bound) over the N real columns (or the listed ones), fp64: the
    oracle's product from its own quantizer (Q8_0) and its epilogue."""
    if act == BF16:
        y, bnd = oracle.gemv_bf16(x, q, s, cols)
    else:
        xq, dx = oracle.quantize_act(x)
        y, bnd = oracle.gemv_q8(xq, dx, q, s, cols)
    return oracle.epilogue(y, bnd, bias, residual, cols)


def check_y(y, z, bnd, N, what):
    err = np.abs(y[:, :N].astype(np.float64) - z)
    lim = REL * bnd + ABS
    assert np.all(err <= lim), f"{what}: y max err/lim {np.max(err / lim):.3g}"
    assert (y[:, N:].view(np.uint32) == 0).all(), f"{what}: pad columns not zero"


def check_quant(codes, scales, z, bnd, N, what):
    """Scales and codes against fp64 z within the product's tolerance."""
    m = z.shape[0]
    Npad = codes.shape[1]
    zp = np.zeros((m, Npad))
    zp[:, :N] = z
    tp = np.full((m, Npad), ABS)
    tp[:, :N] = REL * bnd + ABS
    zb = zp.reshape(m, Npad // 32, 32)
    tb = tp.reshape(m, Npad // 32, 32)
    d = scales.astype(np.float64)
    amax = np.abs(zb).max(axis=2)
    tol_d = tb.max(axis=2) / 127 + np.spacing(scales).astype(np.float64)
    bad = np.abs(d - amax / 127) > tol_d
    assert not bad.any(), f"{what}: {bad.sum()} scales off, first {np.argwhere(bad)[0]}"
    c = codes.reshape(m, Npad // 32, 32).astype(np.float64)
    assert np.abs(c).max() <= 127
    # half a step, plus the tolerance, plus the quotient's fp32 rounding
    lim = d[..., None] * (0.5 + 128 * 2.0 ** -23) + tb + tol_d[..., None] * 127
    err = np.abs(c * d[..., None] - zb)
    assert np.all(err <= lim), f"{what}: codes max err/lim {np.max(err / lim):.3g}"
    assert (codes[:, N:] == 0).all(), f"{what}: pad codes not zero"


# ------------------------------------------------------------------------------
# exact cases: bit-exact y, codes and scales
# ------------------------------------------------------------------------------

EXACT_PLANS = [None,
               (q8.Q8_KERNEL_VALU, 4, 1, 8, 1), (q8.Q8_KERNEL_VALU, 4, 3, 16, 1),
               (q8.Q8_KERNEL_VALU, 32, 2, 4, 1),
               (q8.Q8_KERNEL_MFMA, 16, 1, 16, 1), (q8.Q8_KERNEL_MFMA, 32, 4, 8, 1),
               (q8.Q8_KERNEL_MFMA_COLS, 32, 2, 16, 1), (q8.Q8_KERNEL_MFMA_COLS, 16, 5, 8, 2),
               (q8.Q8_KERNEL_MFMA32, 32, 1, 8, 2), (q8.Q8_KERNEL_MFMA32, 32, 3, 4, 1),
               (q8.Q8_KERNEL_MFMA32_DIRECT, 32, 1, 8, 4), (q8.Q8_KERNEL_MFMA32_DIRECT, 32, 2, 8, 8),
               (q8.Q8_KERNEL_MFMA32_TILE, 32, 1, 8, 1), (q8.Q8_KERNEL_MFMA32_TILE, 32, 3, 16, 1),
               (q8.Q8_KERNEL_MFMA32_TILE, 32, 2, 8, 2),
               (q8.Q8_KERNEL_MFMA16_TILE, 16, 1, 8, 1), (q8.Q8_KERNEL_MFMA16_TILE, 16, 4, 4, 1),
               (q8.Q8_KERNEL_MFMA16_TILE, 16, 2, 16, 2), (q8.Q8_KERNEL_MFMA16_TILE, 32, 3, 8, 1)]


@pytest.mark.parametrize("act", [BF16, Q8])
@pytest.mark.parametrize("pl", EXACT_PLANS, ids=lambda p: "default" if p is None else
                         "k{}r{}s{}w{}ks{}".format(*p))
def test_exact_case_bit_exact(act, pl):
    if pl is not None and pl[0] in (q8.Q8_KERNEL_MFMA32, q8.Q8_KERNEL_MFMA32_DIRECT,
                                    q8.Q8_KERNEL_MFMA32_TILE) and act != Q8:
        pytest.skip("the MFMA32 kernel takes Q8_0 activations only")
    if pl is not None and pl[0] == q8.Q8_KERNEL_MFMA16_TILE and pl[4] == 2 and act != BF16:
        pytest.skip("two-block stages are a bf16 form")
    m, K, N = 3, 512, 100
    x, q, s, bias, res = inputs.exact_case(m, K, N, seed=31)
    Wq, Ws = g.pack(q, s)
    xbuf = g.quantize(x) if act == Q8 else None
    xin = xbuf if act == Q8 else g.dev(x.view(np.int16))
    plan = None if pl is None else g.plan(*pl)
    y, codes, scales = run_fused(xin, Wq, Ws, m, K, N, act, bias, res, quant=True, plan=plan)
    z, _ = reference(x, q, s, act, xbuf, bias, res)
    Npad = q8.q8_padded_cols(N)
    zf = np.zeros((m, Npad), np.float32)
    zf[:, :N] = z                           # exact: every value is fp32-representable
    assert np.array_equal(zf[:, :N].astype(np.float64), z)
    np.testing.assert_array_equal(y.view(np.uint32), zf.view(np.uint32))
    rq, rd = oracle.quantize_rows_f32(zf)
    np.testing.assert_array_equal(codes, rq)
    np.testing.assert_array_equal(scales.view(np.uint32), rd.view(np.uint32))
    # columns 32..63 are an all-zero block: scale 0, codes 0
    assert (scales[:, 1] == 0).all() and (codes[:, 32:64] == 0).all()


# ------------------------------------------------------------------------------
# random cases over the kernels and their plans
# ------------------------------------------------------------------------------

RANDOM_PLANS = [
    (1, BF16, None), (3, Q8, None), (16, BF16, None), (32, Q8, None),
    (1, BF16, (q8.Q8_KERNEL_VALU, 1, 5, 8, 1)),
    (8, Q8, (q8.Q8_KERNEL_VALU, 8, 1, 4, 1)),
    (16, BF16, (q8.Q8_KERNEL_MFMA, 16, 3, 16, 1)),
    (32, Q8, (q8.Q8_KERNEL_MFMA, 32, 7, 4, 1)),
    (32, Q8, (q8.Q8_KERNEL_MFMA_COLS, 32, 2, 16, 1)),
    (16, BF16, (q8.Q8_KERNEL_MFMA_COLS, 16, 3, 8, 2)),
    (20, Q8, (q8.Q8_KERNEL_MFMA_COLS, 32, 68, 16, 4)),
    (32, Q8, (q8.Q8_KERNEL_MFMA32, 32, 2, 8, 2)),
    (17, Q8, (q8.Q8_KERNEL_MFMA32, 32, 5, 4, 4)),
    (32, Q8, (q8.Q8_KERNEL_MFMA32, 32, 1, 8, 1)),
    (32, Q8, (q8.Q8_KERNEL_MFMA32_DIRECT, 32, 1, 8, 4)),
    (19, Q8, (q8.Q8_KERNEL_MFMA32_DIRECT, 32, 3, 4, 2)),
    (32, Q8, (q8.Q8_KERNEL_MFMA32_TILE, 32, 1, 8, 1)),
    (25, Q8, (q8.Q8_KERNEL_MFMA32_TILE, 32, 4, 16, 1)),
    (32, Q8, (q8.Q8_KERNEL_MFMA32_TILE, 32, 1, 8, 2)),
    (19, Q8, (q8.Q8_KERNEL_MFMA32_TILE, 32, 3, 4, 2)),
    (16, BF16, (q8.Q8_KERNEL_MFMA16_TILE, 16, 1, 8, 1)),
    (5, Q8, (q8.Q8_KERNEL_MFMA16_TILE, 16, 3, 16, 1)),
    (11, BF16, (q8.Q8_KERNEL_MFMA16_TILE, 16, 7, 4, 1)),
    (16, BF16, (q8.Q8_KERNEL_MFMA16_TILE, 16, 1, 8, 2)),
    (9, BF16, (q8.Q8_KERNEL_MFMA16_TILE, 16, 3, 4, 2)),
    (3, BF16, (q8.Q8_KERNEL_MFMA16_TILE, 16, 1, 16, 2)),
    (32, BF16, (q8.Q8_KERNEL_MFMA16_TILE, 32, 1, 8, 1)),
    (20, Q8, (q8.Q8_KERNEL_MFMA16_TILE, 32, 4, 16, 1)),
    (25, BF16, (q8.Q8_KERNEL_MFMA16_TILE, 32, 2, 4, 1)),
]


@pytest.mark.parametrize("m,act,pl", RANDOM_PLANS)
@pytest.mark.parametrize("N", [200, 20])
def test_random_bias_residual_quant(m, act, pl, N):
    K = 2176
    x, q, s = inputs.random_case(m, K, N, seed=400 + m + N)
    Npad = q8.q8_padded_cols(N)
    bias = inputs.gen_bias(N, seed=401 + m)
    res = inputs.gen_residual(m, Npad, seed=402 + m)
    Wq, Ws = g.pack(q, s)
    xbuf = g.quantize(x) if act == Q8 else None
    xin = xbuf if act == Q8 else g.dev(x.view(np.int16))
    plan = None if pl is None else g.plan(*pl)
    y, codes, scales = run_fused(xin, Wq, Ws, m, K, N, act, bias, res, quant=True, plan=plan)
    z, bnd = reference(x, q, s, act, xbuf, bias, res)
    what = f"m={m} act={act} plan={pl} N={N}"
    check_y(y, z, bnd, N, what)
    check_quant(codes, scales, z, bnd, N, what)


@pytest.mark.parametrize("pl", [(q8.Q8_KERNEL_MFMA_COLS, 32, 1, 16, 1),
                                (q8.Q8_KERNEL_MFMA_COLS, 32, 1, 8, 2)])
def test_cols_kernel_unsplit_bias_and_residual(pl):
    m, K, N = 32, 2176, 200
    x, q, s = inputs.random_case(m, K, N, seed=450)
    Npad = q8.q8_padded_cols(N)
    bias = inputs.gen_bias(N, seed=451)
    res = inputs.gen_residual(m, Npad, seed=452)
    Wq, Ws = g.pack(q, s)
    xbuf = g.quantize(x)
    y, _, _ = run_fused(xbuf, Wq, Ws, m, K, N, Q8, bias, res, plan=g.plan(*pl))
    z, bnd = reference(x, q, s, Q8, xbuf, bias, res)
    check_y(y, z, bnd, N, f"cols {pl}")
    # unsplit, it has no output quantizer
    with pytest.raises(q8.Q8Error) as e:
        run_fused(xbuf, Wq, Ws, m, K, N, Q8, bias, res, quant=True, plan=g.plan(*pl))
    assert e.value.status == 7


@pytest.mark.parametrize("m,act", [(1, BF16), (32, Q8)])
def test_residual_aliases_y(m, act):
    K, N = 1056, 130
    x, q, s = inputs.random_case(m, K, N, seed=460 + m)
    Npad = q8.q8_padded_cols(N)
    res = inputs.gen_residual(m, Npad, seed=461)
    Wq, Ws = g.pack(q, s)
    xbuf = g.quantize(x) if act == Q8 else None
    xin = xbuf if act == Q8 else g.dev(x.view(np.int16))
    y, _, _ = run_fused(xin, Wq, Ws, m, K, N, act, residual=res, alias=True)
    z, bnd = reference(x, q, s, act, xbuf, residual=res)
    check_y(y, z, bnd, N, "aliased residual")


def test_quant_only_without_y():
    m, K, N = 2, 1024, 96
    x, q, s = inputs.random_case(m, K, N, seed=470)
    Wq, Ws = g.pack(q, s)
    _, codes, scales = run_fused(g.dev(x.view(np.int16)), Wq, Ws, m, K, N, BF16,
                                 quant=True, write_y=False)
    z, bnd = reference(x, q, s, BF16)
    check_quant(codes, scales, z, bnd, N, "quant only")


def test_no_epilogue_is_plain_product():
    m, K, N = 4, 2176, 200
    x, q, s = inputs.random_case(m, K, N, seed=480)
    Wq, Ws = g.pack(q, s)
    xin = g.dev(x.view(np.int16))
    y0 = g.gemv(xin, Wq, Ws, m, K, N, BF16)
    y1, _, _ = run_fused(xin, Wq, Ws, m, K, N, BF16)
    np.testing.assert_array_equal(y0.view(np.uint32), y1.view(np.uint32))
    Npad = q8.q8_padded_cols(N)
    y2 = torch.full((m, Npad), float("nan"), dtype=torch.float32, device=g.DEV)
    q8.q8_gemv_fused(xin, Wq, Ws, y2, m, K, N, BF16, None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y0.view(np.uint32), y2.cpu().numpy().view(np.uint32))


def test_quantized_output_feeds_the_next_product():
    """y_q8 is an activation in the Q8_0 layout over K = N_pad: the next
    product reads it directly and agrees with the oracle on those codes."""
    m, K, N, N2 = 3, 1024, 256, 136
    x, q, s = inputs.random_case(m, K, N, seed=490)
    _, q2, s2 = inputs.random_case(1, N, N2, seed=491)
    Wq, Ws = g.pack(q, s)
    Wq2, Ws2 = g.pack(q2, s2)
    yq = g.empty_bytes(q8.q8_act_bytes(m, N))
    ep = q8.make_epilogue(y_q8=yq, write_y=False)
    q8.q8_gemv_fused(g.dev(x.view(np.int16)), Wq, Ws, None, m, K, N, BF16, ep)
    y2 = g.gemv(yq, Wq2, Ws2, m, N, N2, Q8)
    codes, scales = g.act_host(yq, m, N)
    ref, bnd = oracle.gemv_q8(codes, scales, q2, s2)
    err = np.abs(y2[:, :N2] - ref)
    assert np.all(err <= REL * bnd + ABS)


# ------------------------------------------------------------------------------
# full sizes, in the configuration the benchmark times
# ------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["decode_k4096_n14336", "q8act_m32_k5120_n32000"])
def test_full_size_fused(name):
    w = inputs.WORKLOADS[name]
    act = BF16 if w.act == "bf16" else Q8
    x, q, s = inputs.generate(w)
    m, K, N = w.m, w.K, w.N
    Npad = q8.q8_padded_cols(N)
    bias = inputs.gen_bias(N, seed=w.seed_w + 7)
    res = inputs.gen_residual(m, Npad, seed=w.seed_w + 8)
    Wq, Ws = g.pack(q, s)
    xbuf = g.quantize(x) if act == Q8 else None
    xin = xbuf if act == Q8 else g.dev(x.view(np.int16))
    y, codes, scales = run_fused(xin, Wq, Ws, m, K, N, act, bias, res, quant=True)
    z, bnd = reference(x, q, s, act, xbuf, bias, res)
    check_y(y, z, bnd, N, name)
    check_quant(codes, scales, z, bnd, N, name)
