"""Parity of the gated pair (two products of one activation through a SiLU
gate, one launch) with the oracle, through the C ABI.

The pages' plan.rs, enum Launch, variant GemvGlu: out = act(x.wg + bg) *
(x.wu + bu), SwiGLU when no activation is named.  The oracle gives both
products, their bounds and the gated output in fp64.

The bar, from the product's tolerance T = 1e-5 * (sum_k |x_k w_kn| + |b|) +
1e-6 on g and on u, carried through out = silu(g) * u (|silu'| < 1.1):
    |out - out*| <= 1.1 * T_g * (|u*| + T_u) + (|silu(g*)| + 1.1 * T_g) * T_u
                    + 8 * 2^-24 * |out*| + 1e-30
(the last terms: fp32 evaluation of exp, the division and the product).  The
quantized output is checked as in the epilogue tests, with that tolerance.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_02_amd as q8
import oracle
from block_quantized_weight_02_amd import inputs

pytestmark = pytest.mark.gpu

from tests import gpu_util as g  # noqa: E402
from tests.test_gpu_epilogue import check_quant  # noqa: E402

BF16, Q8 = q8.Q8_ACT_BF16, q8.Q8_ACT_Q8_0
REL, ABS = 1e-5, 1e-6


def silu64(v):
    return v / (1.0 + np.exp(-v))


def glu_tolerance(g, u, bnd_g, bnd_u, bg, bu, out):
    G = g + (0 if bg is None else bg.astype(np.float64))
    U = u + (0 if bu is None else bu.astype(np.float64))
    Tg = REL * (bnd_g + (0 if bg is None else np.abs(bg))) + ABS
    Tu = REL * (bnd_u + (0 if bu is None else np.abs(bu))) + ABS
    return (1.1 * Tg * (np.abs(U) + Tu) + (np.abs(silu64(G)) + 1.1 * Tg) * Tu
            + 8 * 2.0 ** -24 * np.abs(out) + 1e-30)


def run_glu(xin, W, m, K, N, act, bg=None, bu=None, quant=False, write_y=True, plan=None):
    Wg, Wgs, Wu, Wus = W
    Npad = q8.q8_padded_cols(N)
    y = torch.full((m, Npad), float("nan"), dtype=torch.float32, device=g.DEV) \
        if write_y else None
    yq = None
    if quant:
        yq = g.empty_bytes(q8.q8_act_bytes(m, Npad))
        yq.fill_(0x5A)
    ep = q8.make_glu_epilogue(bias_g=None if bg is None else g.dev(bg),
                              bias_u=None if bu is None else g.dev(bu), y_q8=yq,
                              write_y=write_y)
    if plan is None:
        q8.q8_gemv_glu(xin, Wg, Wgs, Wu, Wus, y, m, K, N, act, ep)
    else:
        need = q8.q8_glu_workspace_bytes(plan, m, K, N)
        ws = torch.zeros(need, dtype=torch.uint8, device=g.DEV)
        q8.q8_gemv_glu_planned(xin, Wg, Wgs, Wu, Wus, y, m, K, N, act, ep, plan, None, ws, need)
    torch.cuda.synchronize()
    yh = y.cpu().numpy() if y is not None else None
    if quant:
        codes, scales = g.act_host(yq, m, Npad)
        np.testing.assert_array_equal(g.act_view(yq, m, Npad), oracle.act_view_ref(codes),
                                      err_msg="quantized output's view")
        return yh, codes, scales
    return yh, None, None


def setup(x, qg, sg, qu, su, act):
    Wg, Wgs = g.pack(qg, sg)
    Wu, Wus = g.pack(qu, su)
    xbuf = g.quantize(x) if act == Q8 else None
    xin = xbuf if act == Q8 else g.dev(x.view(np.int16))
    return xin, xbuf, (Wg, Wgs, Wu, Wus)


def reference(x, qg, sg, qu, su, act, xbuf, bg, bu, cols=None):
    if act == BF16:
        return oracle.gemv_glu_bf16(x, qg, sg, qu, su, bg, bu, cols)
    xq, dx = oracle.quantize_act(x)
    return oracle.gemv_glu_q8(xq, dx, qg, sg, qu, su, bg, bu, cols)


def check(y, out, gg, uu, bnd_g, bnd_u, bg, bu, N, what):
    tol = glu_tolerance(gg, uu, bnd_g, bnd_u, bg, bu, out)
    err = np.abs(y[:, :N].astype(np.float64) - out)
    assert np.all(err <= tol), f"{what}: max err/tol {np.max(err / tol):.3g}"
    assert (y[:, N:].view(np.uint32) == 0).all(), f"{what}: pad columns not zero"
    return tol


PLANS = [
    (1, BF16, None), (3, Q8, None), (16, BF16, None), (32, Q8, None), (32, BF16, None),
    (1, BF16, (q8.Q8_KERNEL_VALU, 1, 3, 8, 1)),
    (4, Q8, (q8.Q8_KERNEL_VALU, 4, 1, 16, 1)),
    (16, BF16, (q8.Q8_KERNEL_MFMA, 16, 2, 8, 1)),
    (8, BF16, (q8.Q8_KERNEL_MFMA, 16, 3, 4, 1)),
    (5, Q8, (q8.Q8_KERNEL_MFMA, 16, 1, 4, 1)),
    (32, Q8, (q8.Q8_KERNEL_MFMA, 32, 1, 16, 1)),
    (32, Q8, (q8.Q8_KERNEL_MFMA_COLS, 32, 1, 16, 1)),
    (16, BF16, (q8.Q8_KERNEL_MFMA_COLS, 16, 3, 8, 2)),
    (20, Q8, (q8.Q8_KERNEL_MFMA_COLS, 32, 2, 16, 1)),
]


@pytest.mark.parametrize("m,act,pl", PLANS)
@pytest.mark.parametrize("N", [200, 40])
def test_gated_pair(m, act, pl, N):
    K = 2176
    x, qg, sg = inputs.random_case(m, K, N, seed=500 + m + N)
    _, qu, su = inputs.random_case(m, K, N, seed=600 + m + N)
    bg = inputs.gen_bias(N, seed=501)
    bu = inputs.gen_bias(N, seed=502)
    xin, xbuf, W = setup(x, qg, sg, qu, su, act)
    plan = None if pl is None else g.plan(*pl)
    y, codes, scales = run_glu(xin, W, m, K, N, act, bg, bu, quant=True, plan=plan)
    out, gg, uu, bnd_g, bnd_u = reference(x, qg, sg, qu, su, act, xbuf, bg, bu)
    what = f"m={m} act={act} plan={pl} N={N}"
    tol = check(y, out, gg, uu, bnd_g, bnd_u, bg, bu, N, what)
    check_quant(codes, scales, out, (tol - ABS) / REL, N, what)


def test_gated_pair_without_biases_and_y():
    m, K, N = 2, 1024, 96
    x, qg, sg = inputs.random_case(m, K, N, seed=510)
    _, qu, su = inputs.random_case(m, K, N, seed=511)
    xin, xbuf, W = setup(x, qg, sg, qu, su, BF16)
    y, _, _ = run_glu(xin, W, m, K, N, BF16)
    out, gg, uu, bnd_g, bnd_u = reference(x, qg, sg, qu, su, BF16, None, None, None)
    check(y, out, gg, uu, bnd_g, bnd_u, None, None, N, "no biases")
    _, codes, scales = run_glu(xin, W, m, K, N, BF16, quant=True, write_y=False)
    tol = glu_tolerance(gg, uu, bnd_g, bnd_u, None, None, out)
    check_quant(codes, scales, out, (tol - ABS) / REL, N, "quant only")


def test_gated_pair_deterministic():
    """Repeat calls are bit-identical (the carries meet in a fixed order)."""
    m, K, N = 5, 4096, 320
    x, qg, sg = inputs.random_case(m, K, N, seed=520)
    _, qu, su = inputs.random_case(m, K, N, seed=521)
    xin, xbuf, W = setup(x, qg, sg, qu, su, BF16)
    y1, _, _ = run_glu(xin, W, m, K, N, BF16)
    y2, _, _ = run_glu(xin, W, m, K, N, BF16)
    np.testing.assert_array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_exact_products_gate():
    """Exact-integer products (every sum exact in fp32): the gated output is
    within the fp32 SiLU's own rounding of the oracle's."""
    m, K, N = 3, 512, 100
    x, qg, sg, bg, _ = inputs.exact_case(m, K, N, seed=33)
    _, qu, su, bu, _ = inputs.exact_case(m, K, N, seed=34)
    for act in (BF16, Q8):
        xin, xbuf, W = setup(x, qg, sg, qu, su, act)
        y, _, _ = run_glu(xin, W, m, K, N, act, bg, bu)
        out, gg, uu, _, _ = reference(x, qg, sg, qu, su, act, xbuf, bg, bu)
        err = np.abs(y[:, :N].astype(np.float64) - out)
        assert np.all(err <= 8 * 2.0 ** -24 * np.abs(out) + 1e-30), act


@pytest.mark.parametrize("name,act_override", [("decode_k4096_n14336", None),
                                               ("batch16_k4096_n14336", None),
                                               ("batch16_k4096_n14336", "q8_0")])
def test_full_size_gated_pair(name, act_override):
    w = inputs.WORKLOADS[name]
    act = BF16 if (act_override or w.act) == "bf16" else Q8
    x, qg, sg, qu, su = inputs.generate_pair(w)
    m, K, N = w.m, w.K, w.N
    bg = inputs.gen_bias(N, seed=w.seed_w + 11)
    bu = inputs.gen_bias(N, seed=w.seed_w + 12)
    xin, xbuf, W = setup(x, qg, sg, qu, su, act)
    y, codes, scales = run_glu(xin, W, m, K, N, act, bg, bu, quant=True)
    cols = np.arange(N)                         # every column
    out, gg, uu, bnd_g, bnd_u = reference(x, qg, sg, qu, su, act, xbuf, bg, bu, cols)
    tol = glu_tolerance(gg, uu, bnd_g, bnd_u, bg[cols], bu[cols], out)
    err = np.abs(y[:, cols].astype(np.float64) - out)
    assert np.all(err <= tol), f"{name}: max err/tol {np.max(err / tol):.3g}"
    cb = cols.reshape(-1, 32)[:, 0] // 32
    check_quant(codes[:, cols], scales[:, cb], out, (tol - ABS) / REL, len(cols), name)
