"""Parity of the HIP path (through the C ABI) with the CPU oracle.

The bar: integer work (repack bytes, quantized activations, block dots)
bit-exact; fp32 outputs within |y - y*| <= 1e-5 * sum_k |x_k w_kn| + 1e-6, the
bound computed by the oracle in fp64 beside y*.
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


def assert_close(y_gpu, y_ref, bound, what=""):
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y_ref)
    lim = REL * bound + ABS
    bad = ~(err <= lim)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside tolerance; first at {tuple(i)}: "
            f"gpu={y_gpu[tuple(i)]!r} ref={y_ref[tuple(i)]!r} bound={bound[tuple(i)]!r}; "
            f"max err/lim = {np.max(err / lim):.3g}")


def xdev(x_bits):
    return g.dev(x_bits.view(np.int16))


def run_bf16(x, q, s, plan=None):
    m, K = x.shape
    N = q.shape[1]
    Wq, Ws = g.pack(q, s)
    return g.gemv(xdev(x), Wq, Ws, m, K, N, BF16, plan)


def run_q8(x, q, s, plan=None):
    m, K = x.shape
    N = q.shape[1]
    Wq, Ws = g.pack(q, s)
    buf = g.quantize(x)
    return g.gemv(buf, Wq, Ws, m, K, N, Q8, plan), buf


# ------------------------------------------------------------------------------
# repack / unpack (the values are permuted, never changed; pad is zero)
# ------------------------------------------------------------------------------

@pytest.mark.parametrize("K,N", [(32, 1), (64, 40), (1056, 130), (4096, 64), (160, 257)])
def test_repack_unpack_round_trip(K, N):
    _, q, s = inputs.random_case(1, K, N, seed=K + N)
    Wq, Ws = g.pack(q, s)
    q2 = torch.empty((K, N), dtype=torch.int8, device=g.DEV)
    s2 = torch.empty((K // 32, N), dtype=torch.float32, device=g.DEV)
    q8.q8_unpack(Wq, Ws, K, N, q2, s2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q2.cpu().numpy(), q)
    np.testing.assert_array_equal(s2.cpu().numpy().view(np.uint32), s.view(np.uint32))
    # the packed bytes are the canonical bytes plus zeros for the pad columns
    Npad = q8.q8_padded_cols(N)
    packed = np.sort(Wq.cpu().numpy().view(np.int8)[: K * Npad])
    expect = np.sort(np.concatenate([q.ravel(), np.zeros(K * (Npad - N), np.int8)]))
    np.testing.assert_array_equal(packed, expect)
    sp = np.sort(Ws.cpu().numpy()[: (K // 32) * Npad])
    np.testing.assert_array_equal(sp, np.sort(np.concatenate([s.ravel(), np.zeros((K // 32) * (Npad - N), np.float32)])))


@pytest.mark.parametrize("name", ["q8act_m32_k5120_n40", "decode_k4096_n14336",
                                  "ffn_down_k14336_n4096"])
def test_repack_matches_layout_reference(name):
    """q8_repack's bytes are the oracle's numpy statement of the packed layout,
    byte for byte (values) and bit for bit (scales)."""
    w = inputs.WORKLOADS[name]
    _, q, s = inputs.generate(w)
    Wq, Ws = g.pack(q, s)
    v, sc = oracle.repack_ref(q, s)
    np.testing.assert_array_equal(Wq.cpu().numpy()[: v.size].view(np.int8), v)
    np.testing.assert_array_equal(Ws.cpu().numpy()[: sc.size].view(np.uint32), sc.view(np.uint32))


@pytest.mark.parametrize("K,N", [(32, 1), (64, 130), (1056, 200), (160, 257)])
def test_repack_matches_layout_reference_small(K, N):
    _, q, s = inputs.random_case(1, K, N, seed=K * 3 + N)
    Wq, Ws = g.pack(q, s)
    v, sc = oracle.repack_ref(q, s)
    np.testing.assert_array_equal(Wq.cpu().numpy()[: v.size].view(np.int8), v)
    np.testing.assert_array_equal(Ws.cpu().numpy()[: sc.size].view(np.uint32), sc.view(np.uint32))


# ------------------------------------------------------------------------------
# activation quantize: bit-exact
# ------------------------------------------------------------------------------

@pytest.mark.parametrize("m,K,seed", [(1, 32, 1), (3, 96, 2), (32, 5120, 1005), (7, 2176, 3)])
def test_quantize_act_bit_exact(m, K, seed):
    x = inputs.gen_x(m, K, seed)
    xq, dx = g.act_host(g.quantize(x), m, K)
    rq, rd = oracle.quantize_act(x)
    np.testing.assert_array_equal(xq, rq)
    np.testing.assert_array_equal(dx.view(np.uint32), rd.view(np.uint32))


def test_quantize_act_ties_zero_block_and_exact_multiples():
    d = 2.0 ** -7
    row = np.zeros(96, np.float32)
    row[:6] = np.array([127, 2.5, -2.5, 0.5, -1.5, -127], np.float32) * d
    j = np.random.default_rng(5).integers(-127, 128, size=32)
    j[3] = -127
    row[64:] = j * 2.0 ** -3
    x = inputs.f32_to_bf16_bits(row)[None, :]
    xq, dx = g.act_host(g.quantize(x), 1, 96)
    np.testing.assert_array_equal(xq[0, :6], [127, 3, -3, 1, -2, -127])
    assert (xq[0, 6:64] == 0).all() and dx[0, 1] == 0.0 and dx[0, 0] == d
    np.testing.assert_array_equal(xq[0, 64:], j)
    assert dx[0, 2] == 2.0 ** -3


# ------------------------------------------------------------------------------
# block dots: bit-exact int32
# ------------------------------------------------------------------------------

@pytest.mark.parametrize("m,K,N", [(1, 32, 1), (3, 320, 65), (32, 160, 8), (17, 1056, 130)])
def test_block_dots_bit_exact(m, K, N):
    x, q, _ = inputs.random_case(m, K, N, seed=m * 7 + N)
    Wq, _ = g.pack(q, np.ones((K // 32, N), np.float32))
    buf = g.quantize(x)
    xq, _ = oracle.quantize_act(x)
    D = g.block_dots(buf, Wq, m, K, N)
    ref = oracle.block_dots(xq, q)
    np.testing.assert_array_equal(D[:, :, :N].astype(np.int64), ref)
    assert (D[:, :, N:] == 0).all()


def test_block_dots_extremes():
    # |D| reaches 32*127*127: all +-127 values against all +-127 weights
    x = inputs.f32_to_bf16_bits(np.full((2, 64), 1.0, np.float32))
    x[1] = inputs.f32_to_bf16_bits(np.full(64, -1.0, np.float32))
    q = np.full((64, 3), -127, np.int8)
    q[:, 1] = 127
    Wq, _ = g.pack(q, np.ones((2, 3), np.float32))
    buf = g.quantize(x)
    D = g.block_dots(buf, Wq, 2, 64, 3)
    assert D[0, 0, 0] == -516128 and D[0, 0, 1] == 516128 and D[1, 1, 0] == 516128


# ------------------------------------------------------------------------------
# the product, small shapes: several tiles, ragged N, K tails
# ------------------------------------------------------------------------------

SMALL = [(m, K, N) for m in (1, 2, 3, 8, 16, 17, 32)
         for (K, N) in ((32, 1), (768, 40), (1056, 200), (2176, 65))]


@pytest.mark.parametrize("m,K,N", SMALL)
def test_gemv_bf16_small(m, K, N):
    x, q, s = inputs.random_case(m, K, N, seed=1000 + 3 * m + K + N)
    y = run_bf16(x, q, s)
    ref, bnd = oracle.gemv_bf16(x, q, s)
    assert_close(y[:, :N], ref, bnd, f"bf16 m={m} K={K} N={N}")
    assert (y[:, N:].view(np.uint32) == 0).all()


@pytest.mark.parametrize("m,K,N", SMALL)
def test_gemv_q8_small(m, K, N):
    x, q, s = inputs.random_case(m, K, N, seed=2000 + 3 * m + K + N)
    y, _ = run_q8(x, q, s)
    xq, dx = oracle.quantize_act(x)
    ref, bnd = oracle.gemv_q8(xq, dx, q, s)
    assert_close(y[:, :N], ref, bnd, f"q8 m={m} K={K} N={N}")
    assert (y[:, N:].view(np.uint32) == 0).all()


# ------------------------------------------------------------------------------
# every plan the library can launch
# ------------------------------------------------------------------------------

def _plans(m, NB):
    """Every (kernel, rows, split, waves, kslices) combination worth trying;
    the ones the library does not build are rejected with Q8_ERR_PLAN."""
    out = []
    splits = sorted({1, 2, 3, 7, NB})
    for rows in (1, 2, 4, 8, 16, 32):
        if rows < m:
            continue
        for waves in (4, 8, 16):
            for split in splits:
                if split <= NB:
                    out.append((q8.Q8_KERNEL_VALU, rows, split, waves, 1))
    for rows in (16, 32):
        if rows < m:
            continue
        for waves in (4, 8, 16):
            for split in splits:
                if split <= NB:
                    out.append((q8.Q8_KERNEL_MFMA, rows, split, waves, 1))
        for (waves, ks) in ((4, 1), (8, 1), (16, 1), (8, 2), (16, 4)):
            for split in splits:
                if split <= NB:
                    out.append((q8.Q8_KERNEL_MFMA_COLS, rows, split, waves, ks))
    if m <= 32:
        for kernel in (q8.Q8_KERNEL_MFMA32, q8.Q8_KERNEL_MFMA32_DIRECT):
            for (waves, ks) in ((4, 1), (4, 2), (4, 4), (8, 1), (8, 2), (8, 4), (8, 8)):
                for split in splits:
                    if split <= NB:
                        out.append((kernel, 32, split, waves, ks))
        for (waves, tp) in ((4, 1), (8, 1), (16, 1), (4, 2), (8, 2)):
            for split in splits:
                if split <= NB:
                    out.append((q8.Q8_KERNEL_MFMA32_TILE, 32, split, waves, tp))
    if m <= 16:
        for waves in (4, 8, 16):
            for split in splits:
                if split <= NB:
                    for ks in (1, 2):
                        out.append((q8.Q8_KERNEL_MFMA16_TILE, 16, split, waves, ks))
    if m <= 32:
        for waves in (4, 8, 16):
            for split in splits:
                if split <= NB:
                    for ks in (1, 2):
                        out.append((q8.Q8_KERNEL_MFMA16_TILE, 32, split, waves, ks))
    return out


@pytest.mark.parametrize("act", [BF16, Q8])
@pytest.mark.parametrize("m", [1, 5, 16, 32])
def test_every_plan(act, m):
    K, N = 2176, 200
    x, q, s = inputs.random_case(m, K, N, seed=77 + m)
    Wq, Ws = g.pack(q, s)
    if act == BF16:
        xin = xdev(x)
        ref, bnd = oracle.gemv_bf16(x, q, s)
    else:
        xin = g.quantize(x)
        xq, dx = oracle.quantize_act(x)
        ref, bnd = oracle.gemv_q8(xq, dx, q, s)
        Dref = oracle.block_dots(xq, q)
    ran = 0
    for (kernel, rows, split, waves, ks) in _plans(m, K // 32):
        p = g.plan(kernel, rows, split, waves, ks)
        try:
            y = g.gemv(xin, Wq, Ws, m, K, N, act, p)
        except q8.Q8Error as e:
            assert e.status == 7, e   # a plan the library does not build
            continue
        ran += 1
        assert_close(y[:, :N], ref, bnd, f"plan {p}")
        assert (y[:, N:].view(np.uint32) == 0).all()
        if act == Q8:
            D = g.block_dots(xin, Wq, m, K, N, p)
            np.testing.assert_array_equal(D[:, :, :N].astype(np.int64), Dref)
    assert ran > 0


# ------------------------------------------------------------------------------
# the named workloads at full size
# ------------------------------------------------------------------------------

def _sample_cols(N, n=384, seed=0):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, 63, 64, N - 1, N - 2, max(0, N - 64)}
    pick = set(rng.choice(N, size=min(n, N), replace=False).tolist())
    return np.array(sorted(c for c in fixed | pick if 0 <= c < N), np.int64)


@pytest.mark.parametrize("name", [n for n, w in inputs.WORKLOADS.items() if w.m <= q8.Q8_MAX_ROWS])
def test_workload_full_size(name):
    """Every configuration at its full size, in the launch configuration the
    benchmark times (the default plan): every output column against the
    oracle, and in Q8_0 mode every int32 block dot bit for bit."""
    w = inputs.WORKLOADS[name]
    x, q, s = inputs.generate(w)
    m, K, N = w.m, w.K, w.N
    Wq, Ws = g.pack(q, s)
    if w.act == "bf16":
        y = g.gemv(xdev(x), Wq, Ws, m, K, N, BF16)
        ref, bnd = oracle.gemv_bf16(x, q, s)
    else:
        buf = g.quantize(x)                       # bit-equal to the oracle's
        xq, dx = oracle.quantize_act(x)
        y = g.gemv(buf, Wq, Ws, m, K, N, Q8)
        ref, bnd = oracle.gemv_q8(xq, dx, q, s)
        D = g.block_dots(buf, Wq, m, K, N)
        step = 4096                               # the oracle's int64 dots, a slab at a time
        for c0 in range(0, N, step):
            cols = np.arange(c0, min(N, c0 + step))
            np.testing.assert_array_equal(D[:, :, c0:c0 + len(cols)].astype(np.int64),
                                          oracle.block_dots(xq, q, cols),
                                          err_msg=f"{name}: dots of columns {c0}..")
        assert (D[:, :, N:] == 0).all()
        del D
    assert_close(y[:, :N], ref, bnd, name)
    assert (y[:, N:].view(np.uint32) == 0).all()
    assert np.isfinite(y).all()


# ------------------------------------------------------------------------------
# properties
# ------------------------------------------------------------------------------

def test_deterministic_with_split_k():
    x, q, s = inputs.random_case(3, 4096, 512, seed=90)
    Wq, Ws = g.pack(q, s)
    p = g.plan(q8.Q8_KERNEL_VALU, 4, 16)
    y1 = g.gemv(xdev(x), Wq, Ws, 3, 4096, 512, BF16, p)
    y2 = g.gemv(xdev(x), Wq, Ws, 3, 4096, 512, BF16, p)
    np.testing.assert_array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_rows_match_single_row_calls():
    # codegen_cuda/lane/plan.rs, fn is_batch: each row summed as the one-row step sums it
    x, q, s = inputs.random_case(4, 2048, 300, seed=91)
    Wq, Ws = g.pack(q, s)
    p = g.plan(q8.Q8_KERNEL_VALU, 4, 4)
    y = g.gemv(xdev(x), Wq, Ws, 4, 2048, 300, BF16, p)
    for r in range(4):
        p1 = g.plan(q8.Q8_KERNEL_VALU, 1, 4)
        y1 = g.gemv(xdev(x[r:r + 1]), Wq, Ws, 1, 2048, 300, BF16, p1)
        np.testing.assert_array_equal(y1[0].view(np.uint32), y[r].view(np.uint32))


def test_zero_weight_and_one_hot():
    m, K, N = 3, 256, 70
    x, _, _ = inputs.random_case(m, K, N, seed=92)
    y = run_bf16(x, np.zeros((K, N), np.int8), np.zeros((K // 32, N), np.float32))
    assert (y.view(np.uint32) == 0).all()
    q = np.zeros((K, N), np.int8)
    q[37, 65] = 1
    y = run_bf16(x, q, np.ones((K // 32, N), np.float32))
    expect = np.zeros((m, q8.q8_padded_cols(N)), np.float32)
    expect[:, 65] = inputs.bf16_bits_to_f32(x[:, 37])
    np.testing.assert_array_equal(y, expect)


def test_all_ones_gives_row_sums():
    m, K, N = 2, 1024, 64
    x, _, _ = inputs.random_case(m, K, N, seed=93)
    y = run_bf16(x, np.ones((K, N), np.int8), np.ones((K // 32, N), np.float32))
    xv = inputs.bf16_bits_to_f32(x).astype(np.float64)
    rows = xv.sum(axis=1)
    bnd = np.abs(xv).sum(axis=1)
    for n in range(N):
        assert_close(y[:, n], rows, bnd, "all ones")


def test_workspace_too_small_is_rejected():
    m, K, N = 1, 4096, 64
    x, q, s = inputs.random_case(m, K, N, seed=94)
    Wq, Ws = g.pack(q, s)
    p = g.plan(q8.Q8_KERNEL_VALU, 1, 8)
    need = q8.q8_plan_workspace_bytes(p, m, K, N)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=g.DEV)
    y = torch.empty((m, 64), dtype=torch.float32, device=g.DEV)
    with pytest.raises(q8.Q8Error) as e:
        q8.q8_gemv_planned(xdev(x), Wq, Ws, y, m, K, N, BF16, p, None, ws, need - 1)
    assert e.value.status == 5
    with pytest.raises(q8.Q8Error) as e:
        bad = g.plan(q8.Q8_KERNEL_VALU, 1, K // 32 + 1)
        q8.q8_gemv_planned(xdev(x), Wq, Ws, y, m, K, N, BF16, bad, None, ws, need)
    assert e.value.status == 7
    q8.q8_gemv_planned(xdev(x), Wq, Ws, y, m, K, N, BF16, p, None, ws, need)
    torch.cuda.synchronize()
    ref, bnd = oracle.gemv_bf16(x, q, s)
    assert_close(y.cpu().numpy(), ref, bnd, "explicit workspace")


def test_two_streams():
    m, K, N = 2, 4096, 256
    cases = [inputs.random_case(m, K, N, seed=95 + i) for i in range(2)]
    packed = [g.pack(q, s) for (_, q, s) in cases]
    xs = [xdev(x) for (x, _, _) in cases]
    ys = [torch.empty((m, N), dtype=torch.float32, device=g.DEV) for _ in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    torch.cuda.synchronize()
    for _ in range(3):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                q8.q8_gemv(xs[i], packed[i][0], packed[i][1], ys[i], m, K, N, BF16)
    torch.cuda.synchronize()
    for i, (x, q, s) in enumerate(cases):
        ref, bnd = oracle.gemv_bf16(x, q, s)
        assert_close(ys[i].cpu().numpy(), ref, bnd, f"stream {i}")


def test_library_workspace_reused_across_shapes():
    # One stream's library workspace serves calls of different shapes in turn:
    # the split-K counters keep fixed places, so no call sees another's carries.
    shapes = [(1, 2592, 200), (4, 4096, 640), (1, 2592, 200), (2, 8192, 64), (4, 4096, 640)]
    for i, (m, K, N) in enumerate(shapes):
        x, q, s = inputs.random_case(m, K, N, seed=300 + i)
        assert q8.q8_gemv_default_plan(m, K, N, BF16).split_k > 1
        y = run_bf16(x, q, s)
        ref, bnd = oracle.gemv_bf16(x, q, s)
        assert_close(y[:, :N], ref, bnd, f"shape {i}")


def test_row_split_halves():
    """The product split along K (at a block boundary), as a row split across
    devices would run it (int8_model.rs, the row-split projections): each half's
    block dots are the full call's, bit for bit, its quantized activation is
    the full one's blocks, and the halves' outputs sum to the full product
    within the two halves' tolerances."""
    m, K, N, K1 = 3, 2176, 200, 1056
    x, q, s = inputs.random_case(m, K, N, seed=95)
    halves = [(0, K1), (K1, K)]
    xbuf = g.quantize(x)
    xq, dx = g.act_host(xbuf, m, K)
    Wq, _ = g.pack(q, s)
    dots = g.block_dots(xbuf, Wq, m, K, N)
    ysum = np.zeros((m, N))
    for lo, hi in halves:
        xh = np.ascontiguousarray(x[:, lo:hi])
        bh = g.quantize(xh)
        xqh, dxh = g.act_host(bh, m, hi - lo)
        np.testing.assert_array_equal(xqh, xq[:, lo:hi])
        np.testing.assert_array_equal(dxh.view(np.uint32), dx[:, lo // 32:hi // 32].view(np.uint32))
        Wh, Wsh = g.pack(np.ascontiguousarray(q[lo:hi]), np.ascontiguousarray(s[lo // 32:hi // 32]))
        dh = g.block_dots(bh, Wh, m, hi - lo, N)
        np.testing.assert_array_equal(dh, dots[:, lo // 32:hi // 32, :])
        yh = g.gemv(xdev(xh), Wh, Wsh, m, hi - lo, N, BF16)
        ysum += yh[:, :N].astype(np.float64)
    yref, bnd = oracle.gemv_bf16(x, q, s)
    err = np.abs(ysum - yref)
    assert np.all(err <= REL * bnd + 2 * ABS), np.max(err / (REL * bnd + 2 * ABS))


# ------------------------------------------------------------------------------
# maximum sizes
# ------------------------------------------------------------------------------

def test_long_k():
    """K = 2^20 (32768 blocks, a 2 MiB activation row): the default plan and
    explicit VALU and MFMA plans with many K splits, bf16 and int8."""
    m, K, N = 3, 1 << 20, 70
    x, q, s = inputs.random_case(m, K, N, seed=97)
    Wq, Ws = g.pack(q, s)
    ref, bnd = oracle.gemv_bf16(x, q, s)
    for plan in (None, g.plan(q8.Q8_KERNEL_VALU, 4, 3, 8), g.plan(q8.Q8_KERNEL_MFMA, 16, 512, 16)):
        y = g.gemv(xdev(x), Wq, Ws, m, K, N, BF16, plan)
        assert_close(y[:, :N], ref, bnd, f"K=2^20 bf16 plan={plan}")
        assert (y[:, N:].view(np.uint32) == 0).all()
    buf = g.quantize(x)
    xq, dx = g.act_host(buf, m, K)
    rq, rd = oracle.quantize_act(x)
    np.testing.assert_array_equal(xq, rq)
    np.testing.assert_array_equal(dx.view(np.uint32), rd.view(np.uint32))
    ref, bnd = oracle.gemv_q8(xq, dx, q, s)
    y = g.gemv(buf, Wq, Ws, m, K, N, Q8)
    assert_close(y[:, :N], ref, bnd, "K=2^20 int8")


def test_widest_n():
    """N = 2^24 - 5, the widest the library takes (2^18 column tiles, the
    last one ragged), one block of K."""
    m, K, N = 1, 32, (1 << 24) - 5
    x, q, s = inputs.random_case(m, K, N, seed=98)
    Wq, Ws = g.pack(q, s)
    y = g.gemv(xdev(x), Wq, Ws, m, K, N, BF16)
    cols = _sample_cols(N, n=2048, seed=98)
    ref, bnd = oracle.gemv_bf16(x, q, s, cols)
    assert_close(y[:, cols], ref, bnd, "N=2^24-5")
    assert (y[:, N:].view(np.uint32) == 0).all()
    assert y.shape[1] == 1 << 24


def test_long_k_tile_kernels():
    """K = 2^20 on the tile kernels' default plans (their LDS of the split's
    activation scales raises the K split): 20 int8 rows (32x32x32 kernel),
    16 bf16 rows (16x16x32 kernel, both stage sizes) and 24 bf16 rows (its two
    row groups)."""
    K, N = 1 << 20, 70
    for m, act in ((20, Q8), (16, BF16), (24, BF16)):
        x, q, s = inputs.random_case(m, K, N, seed=99 + m)
        Wq, Ws = g.pack(q, s)
        if act == BF16:
            ref, bnd = oracle.gemv_bf16(x, q, s)
            p = q8.q8_gemv_default_plan(m, K, N, BF16)
            assert p.kernel == q8.Q8_KERNEL_MFMA16_TILE and p.rows == (16 if m <= 16 else 32)
            plans = [None]
            if m <= 16:
                plans += [g.plan(q8.Q8_KERNEL_MFMA16_TILE, 16, 64, 16, 2),
                          g.plan(q8.Q8_KERNEL_MFMA16_TILE, 16, 64, 8, 1)]
            for plan in plans:
                y = g.gemv(xdev(x), Wq, Ws, m, K, N, BF16, plan)
                assert_close(y[:, :N], ref, bnd, f"K=2^20 bf16 m={m} plan={plan}")
                assert (y[:, N:].view(np.uint32) == 0).all()
        else:
            buf = g.quantize(x)
            xq, dx = oracle.quantize_act(x)
            ref, bnd = oracle.gemv_q8(xq, dx, q, s)
            p = q8.q8_gemv_default_plan(m, K, N, Q8)
            assert p.kernel == q8.Q8_KERNEL_MFMA32_TILE
            y = g.gemv(buf, Wq, Ws, m, K, N, Q8)
            assert_close(y[:, :N], ref, bnd, f"K=2^20 int8 m={m}")
            assert (y[:, N:].view(np.uint32) == 0).all()


@pytest.mark.parametrize("m,act", [(3, BF16), (17, Q8), (29, BF16)])
def test_widest_n_tile_kernels(m, act):
    """N = 2^24 - 5 on the tile kernels (2^18 workgroups, the last tile
    ragged), one block of K; sampled columns and the tile edges."""
    K, N = 32, (1 << 24) - 5
    x, q, s = inputs.random_case(m, K, N, seed=200 + m)
    Wq, Ws = g.pack(q, s)
    cols = _sample_cols(N, n=2048, seed=200 + m)
    if act == BF16:
        y = g.gemv(xdev(x), Wq, Ws, m, K, N, BF16)
        ref, bnd = oracle.gemv_bf16(x, q, s, cols)
    else:
        buf = g.quantize(x)
        xq, dx = oracle.quantize_act(x)
        y = g.gemv(buf, Wq, Ws, m, K, N, Q8)
        ref, bnd = oracle.gemv_q8(xq, dx, q, s, cols)
    assert_close(y[:, cols], ref, bnd, f"N=2^24-5 m={m}")
    assert (y[:, N:].view(np.uint32) == 0).all()


@pytest.mark.parametrize("m,N,pl", [(32, 130, (q8.Q8_KERNEL_MFMA32_TILE, 32, 1, 8, 2)),
                                    (17, 40, (q8.Q8_KERNEL_MFMA32_TILE, 32, 3, 4, 2)),
                                    (24, 330, (q8.Q8_KERNEL_MFMA32_TILE, 32, 2, 8, 2))])
def test_two_tile_waves_odd_tiles(m, N, pl):
    """The 32x32x32 tile kernel with two column tiles a wave on an odd tile
    count (the last workgroup's second tile is past the weight): every
    column within the bound, pad columns zero, block dots bit for bit."""
    K = 1056
    x, q, s = inputs.random_case(m, K, N, seed=300 + m + N)
    Wq, Ws = g.pack(q, s)
    buf = g.quantize(x)
    xq, dx = oracle.quantize_act(x)
    plan = g.plan(*pl)
    y = g.gemv(buf, Wq, Ws, m, K, N, Q8, plan)
    ref, bnd = oracle.gemv_q8(xq, dx, q, s)
    assert_close(y[:, :N], ref, bnd, f"two tiles m={m} N={N}")
    assert (y[:, N:].view(np.uint32) == 0).all()
    d = g.block_dots(buf, Wq, m, K, N, plan)
    np.testing.assert_array_equal(d[:, :, :N], oracle.block_dots(xq, q))
    assert (d[:, :, N:] == 0).all()
