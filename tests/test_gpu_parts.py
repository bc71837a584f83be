"""Parity of the product in parts (several projections of one activation in
one launch) with the oracle, through the C ABI.

The pages' plan.rs, enum Launch, variant GemmParts, and struct GemmPart: each
part has its own matrix, optional bias, destination and width, over one
activation.  Part i is checked against the oracle's product of x with W_i plus
bias_i, to the product's tolerance 1e-5 * (sum_k |x_k w_kn| + |b_n|) + 1e-6,
and its pad columns must be zero.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_02_amd as q8
import oracle
from block_quantized_weight_02_amd import inputs

pytestmark = pytest.mark.gpu

from tests import gpu_util as g  # noqa: E402

BF16, Q8 = q8.Q8_ACT_BF16, q8.Q8_ACT_Q8_0
REL, ABS = 1e-5, 1e-6


def setup(x, ws, act):
    packed = [g.pack(q, s) for q, s in ws]
    xbuf = g.quantize(x) if act == Q8 else None
    xin = xbuf if act == Q8 else g.dev(x.view(np.int16))
    return xin, xbuf, packed


def run_parts(xin, packed, Ns, biases, m, K, act, plan=None):
    ys = [torch.full((m, q8.q8_padded_cols(N)), float("nan"), dtype=torch.float32,
                     device=g.DEV) for N in Ns]
    bdev = [None if b is None else g.dev(b) for b in biases]
    parts = [q8.make_part(W, Ws, y, N, bias=b)
             for (W, Ws), y, N, b in zip(packed, ys, Ns, bdev)]
    if plan is None:
        q8.q8_gemv_parts(xin, parts, m, K, act)
    else:
        need = q8.q8_parts_workspace_bytes(plan, parts, m, K)
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=g.DEV)
        q8.q8_gemv_parts_planned(xin, parts, m, K, act, plan, None, ws if need else None, need)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


def reference(x, q, s, act, xbuf, bias, cols=None):
    """(z, bound) of one part, fp64, over `cols` (all when None): the oracle's
    product from its own quantizer (Q8_0) and its epilogue (the bias)."""
    if act == BF16:
        z, bnd = oracle.gemv_bf16(x, q, s, cols)
    else:
        xq, dx = oracle.quantize_act(x)
        z, bnd = oracle.gemv_q8(xq, dx, q, s, cols)
    return oracle.epilogue(z, bnd, bias, None, cols)


def check_part(y, z, bnd, N, what, cols=None):
    yc = y[:, :N] if cols is None else y[:, cols]
    err = np.abs(yc.astype(np.float64) - z)
    lim = REL * bnd + ABS
    assert np.all(err <= lim), f"{what}: max err/lim {np.max(err / lim):.3g}"
    assert (y[:, N:].view(np.uint32) == 0).all(), f"{what}: pad columns not zero"


def small_case(m, K, Ns, seed):
    x = inputs.gen_x(m, K, seed)
    ws = [(inputs.gen_q(K, N, seed + 10 * i + 1), inputs.gen_scales(K, N, seed + 10 * i + 1))
          for i, N in enumerate(Ns)]
    return x, ws


PLANS = [
    (1, BF16, None), (3, Q8, None), (8, Q8, None), (16, BF16, None), (32, Q8, None),
    (32, BF16, None),
    (1, BF16, (q8.Q8_KERNEL_VALU, 1, 3, 8, 1)),
    (2, BF16, (q8.Q8_KERNEL_VALU, 2, 1, 4, 1)),
    (4, Q8, (q8.Q8_KERNEL_VALU, 4, 1, 16, 1)),
    (16, BF16, (q8.Q8_KERNEL_MFMA, 16, 2, 8, 1)),
    (32, Q8, (q8.Q8_KERNEL_MFMA, 32, 1, 16, 1)),
    (32, Q8, (q8.Q8_KERNEL_MFMA, 32, 5, 4, 1)),
    (3, BF16, (q8.Q8_KERNEL_MFMA16_TILE, 16, 2, 16, 1)),
    (16, Q8, (q8.Q8_KERNEL_MFMA16_TILE, 16, 3, 8, 1)),
    (13, BF16, (q8.Q8_KERNEL_MFMA16_TILE, 16, 1, 4, 2)),
    (24, BF16, (q8.Q8_KERNEL_MFMA16_TILE, 32, 2, 16, 1)),
    (32, Q8, (q8.Q8_KERNEL_MFMA16_TILE, 32, 5, 8, 1)),
    (17, Q8, (q8.Q8_KERNEL_MFMA16_TILE, 32, 1, 4, 1)),
]
SHAPES = [(200, 40, 64, 130), (96,), (40, 300)]


@pytest.mark.parametrize("m,act,pl", PLANS)
@pytest.mark.parametrize("Ns", SHAPES)
def test_parts(m, act, pl, Ns):
    K = 2176
    seed = 700 + m + sum(Ns)
    x, ws = small_case(m, K, Ns, seed)
    biases = [inputs.gen_bias(N, seed=seed + i) if i % 2 == 0 else None
              for i, N in enumerate(Ns)]
    xin, xbuf, packed = setup(x, ws, act)
    plan = None if pl is None else g.plan(*pl)
    ys = run_parts(xin, packed, Ns, biases, m, K, act, plan)
    for i, ((q, s), N, b, y) in enumerate(zip(ws, Ns, biases, ys)):
        z, bnd = reference(x, q, s, act, xbuf, b)
        check_part(y, z, bnd, N, f"m={m} act={act} plan={pl} Ns={Ns} part {i}")


def test_parts_match_single_products():
    """A part's output equals the single product of the same plan kind
    bit for bit when the launch gives it the same split (one split each)."""
    m, K, Ns = 2, 1024, (128, 64, 192)
    x, ws = small_case(m, K, Ns, 730)
    xin, xbuf, packed = setup(x, ws, BF16)
    plan = g.plan(q8.Q8_KERNEL_VALU, 2, 1, 8)
    ys = run_parts(xin, packed, Ns, [None] * 3, m, K, BF16, plan)
    for (W, Ws), N, y in zip(packed, Ns, ys):
        single = g.gemv(xin, W, Ws, m, K, N, BF16, plan=plan)
        np.testing.assert_array_equal(y.view(np.uint32), single.view(np.uint32))


def test_parts_deterministic_and_workspace_reuse():
    """Repeat calls are bit-identical, and the library workspace's counters
    are left at zero for the plain product that follows on the stream."""
    m, K, Ns = 5, 4096, (320, 64, 1000)
    x, ws = small_case(m, K, Ns, 740)
    xin, xbuf, packed = setup(x, ws, BF16)
    y1 = run_parts(xin, packed, Ns, [None] * 3, m, K, BF16)
    (W, Ws), N = packed[2], Ns[2]
    single = g.gemv(xin, W, Ws, m, K, N, BF16)
    y2 = run_parts(xin, packed, Ns, [None] * 3, m, K, BF16)
    for a, b in zip(y1, y2):
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    z, bnd = reference(x, *ws[2], BF16, None, None)
    check_part(single, z, bnd, N, "product after parts")


def test_one_block_and_one_part():
    m, K, Ns = 3, 32, (70,)
    for act in (BF16, Q8):
        x, ws = small_case(m, K, Ns, 750)
        xin, xbuf, packed = setup(x, ws, act)
        b = inputs.gen_bias(70, seed=751)
        (y,) = run_parts(xin, packed, Ns, [b], m, K, act)
        z, bnd = reference(x, *ws[0], act, xbuf, b)
        check_part(y, z, bnd, 70, f"K=32 act={act}")


def test_exact_products_parts():
    """Exact-integer products: every part equals the oracle exactly."""
    m, K, N = 3, 512, 100
    x, q1, s1, b1, _ = inputs.exact_case(m, K, N, seed=35)
    _, q2, s2, b2, _ = inputs.exact_case(m, K, N, seed=36)
    for act in (BF16, Q8):
        xin, xbuf, packed = setup(x, [(q1, s1), (q2, s2)], act)
        ys = run_parts(xin, packed, (N, N), [b1, b2], m, K, act)
        for (q, s), b, y in zip([(q1, s1), (q2, s2)], [b1, b2], ys):
            z, _ = reference(x, q, s, act, xbuf, b)
            np.testing.assert_array_equal(y[:, :N].astype(np.float64), z)


@pytest.mark.parametrize("name", sorted(n for n, w in inputs.PARTS_WORKLOADS.items() if w.m <= 32))
def test_full_size_parts(name):
    w = inputs.PARTS_WORKLOADS[name]
    act = BF16 if w.act == "bf16" else Q8
    x, ws = inputs.generate_parts(w)
    biases = [inputs.gen_bias(N, seed=w.seed_w + 20 + i) for i, N in enumerate(w.Ns)]
    xin, xbuf, packed = setup(x, ws, act)
    ys = run_parts(xin, packed, w.Ns, biases, w.m, w.K, act)
    for i, ((q, s), N, b, y) in enumerate(zip(ws, w.Ns, biases, ys)):
        z, bnd = reference(x, q, s, act, xbuf, b)          # every column
        check_part(y, z, bnd, N, f"{name} part {i}")
