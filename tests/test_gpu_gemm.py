"""Parity of the many-row product (q8_gemm, the prefill GEMM) with the oracle,
through the C ABI.

Same arithmetic and bar as the GEMV: int8 block dots bit-exact; fp32 outputs
within |y - y*| <= 1e-5 * sum_k |x_k w_kn| + 1e-6 (the oracle's fp64 bound).
Each output's fp32 chain is one FMA per Q8_0 block after the matrix core's
32-term block sum: at K <= 4096 that is at most 128 + 32 roundings, inside
the ~167 the bound allows.
"""
import numpy as np
import pytest
import torch

import block_quantized_weight_02_amd as q8
import oracle
from block_quantized_weight_02_amd import inputs

pytestmark = pytest.mark.gpu

from tests import gpu_util as g  # noqa: E402
from tests.test_gpu_parity import assert_close, xdev, _sample_cols  # noqa: E402

BF16, Q8 = q8.Q8_ACT_BF16, q8.Q8_ACT_Q8_0


def gemm(xin, Wq, Ws, m, K, N, act):
    y = torch.full((m, q8.q8_padded_cols(N)), float("nan"), dtype=torch.float32, device=g.DEV)
    q8.q8_gemm(xin, Wq, Ws, y, m, K, N, act)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def gemm_dots(xbuf, Wq, m, K, N):
    d = torch.full((m, K // 32, q8.q8_padded_cols(N)), -(2 ** 31), dtype=torch.int32,
                   device=g.DEV)
    q8.q8_gemm_block_dots(xbuf, Wq, d, m, K, N)
    torch.cuda.synchronize()
    return d.cpu().numpy()


SHAPES = [(m, K, N) for m in (1, 7, 33, 64, 65, 130, 200, 257, 300, 1100)
          for (K, N) in ((32, 1), (96, 40), (1056, 200), (2176, 257))]


@pytest.mark.parametrize("m,K,N", SHAPES)
def test_gemm_bf16(m, K, N):
    x, q, s = inputs.random_case(m, K, N, seed=3000 + m + K + N)
    Wq, Ws = g.pack(q, s)
    y = gemm(xdev(x), Wq, Ws, m, K, N, BF16)
    ref, bnd = oracle.gemv_bf16(x, q, s)
    assert_close(y[:, :N], ref, bnd, f"gemm bf16 m={m} K={K} N={N}")
    assert (y[:, N:].view(np.uint32) == 0).all()


@pytest.mark.parametrize("m,K,N", SHAPES)
def test_gemm_q8(m, K, N):
    x, q, s = inputs.random_case(m, K, N, seed=4000 + m + K + N)
    Wq, Ws = g.pack(q, s)
    buf = g.quantize(x)
    xq, dx = g.act_host(buf, m, K)
    rq, rd = oracle.quantize_act(x)
    np.testing.assert_array_equal(xq, rq)
    np.testing.assert_array_equal(dx.view(np.uint32), rd.view(np.uint32))
    y = gemm(buf, Wq, Ws, m, K, N, Q8)
    ref, bnd = oracle.gemv_q8(xq, dx, q, s)
    assert_close(y[:, :N], ref, bnd, f"gemm q8 m={m} K={K} N={N}")
    assert (y[:, N:].view(np.uint32) == 0).all()


@pytest.mark.parametrize("m,K,N", [(1, 32, 1), (33, 96, 40), (17, 2176, 257), (64, 1056, 130),
                                   (48, 4096, 640), (100, 1056, 130), (130, 320, 130),
                                   (200, 1056, 64), (300, 320, 130), (1100, 320, 130)])
def test_gemm_block_dots_bit_exact(m, K, N):
    x, q, _ = inputs.random_case(m, K, N, seed=5000 + m + N)
    Wq, _ = g.pack(q, np.ones((K // 32, N), np.float32))
    buf = g.quantize(x)
    xq, _ = g.act_host(buf, m, K)
    D = gemm_dots(buf, Wq, m, K, N)
    np.testing.assert_array_equal(D[:, :, :N].astype(np.int64), oracle.block_dots(xq, q))
    assert (D[:, :, N:] == 0).all()


def test_gemm_extreme_dots():
    # |D| reaches 32 * 127 * 127 with every row and column at the extremes
    m, K, N = 70, 64, 3
    x = inputs.f32_to_bf16_bits(np.where(np.arange(m)[:, None] % 2 == 0, 1.0, -1.0)
                                * np.ones((m, K), np.float32))
    q = np.full((K, N), -127, np.int8)
    q[:, 1] = 127
    Wq, _ = g.pack(q, np.ones((K // 32, N), np.float32))
    D = gemm_dots(g.quantize(x), Wq, m, K, N)
    assert D[0, 0, 0] == -516128 and D[0, 0, 1] == 516128 and D[1, 1, 0] == 516128


def test_gemm_agrees_with_gemv_rows():
    """Row r of the many-row product and the GEMV on the same row are both
    within the tolerance of the oracle; rows do not interact."""
    m, K, N = 96, 2048, 192
    x, q, s = inputs.random_case(m, K, N, seed=5100)
    Wq, Ws = g.pack(q, s)
    y = gemm(xdev(x), Wq, Ws, m, K, N, BF16)
    ref, bnd = oracle.gemv_bf16(x, q, s)
    assert_close(y[:, :N], ref, bnd, "gemm")
    for r in (0, 31, 64, 95):
        y1 = g.gemv(xdev(x[r:r + 1]), Wq, Ws, 1, K, N, BF16)
        assert_close(y1[:, :N], ref[r:r + 1], bnd[r:r + 1], f"gemv row {r}")


def test_gemm_deterministic_and_zero_weight():
    m, K, N = 150, 1024, 300
    x, q, s = inputs.random_case(m, K, N, seed=5200)
    Wq, Ws = g.pack(q, s)
    y1 = gemm(xdev(x), Wq, Ws, m, K, N, BF16)
    y2 = gemm(xdev(x), Wq, Ws, m, K, N, BF16)
    np.testing.assert_array_equal(y1.view(np.uint32), y2.view(np.uint32))
    Wz, Wzs = g.pack(np.zeros_like(q), np.zeros_like(s))
    yz = gemm(xdev(x), Wz, Wzs, m, K, N, BF16)
    assert (yz.view(np.uint32) == 0).all()


def test_gemm_shape_errors():
    with pytest.raises(q8.Q8Error) as e:
        q8.q8_gemm(1 << 20, 1 << 20, 1 << 20, 1 << 20, q8.Q8_MAX_GEMM_ROWS + 1, 64, 8, 0)
    assert e.value.status == 1


@pytest.mark.parametrize("name", ["prefill_m512_k4096_n14336", "prefill_q8act_m512_k4096_n14336",
                                  "prefill_m128_k4096_n14336", "prefill_q8act_m128_k4096_n14336"])
def test_prefill_full_size(name):
    w = inputs.WORKLOADS[name]
    x, q, s = inputs.generate(w)
    m, K, N = w.m, w.K, w.N
    Wq, Ws = g.pack(q, s)
    cols = _sample_cols(N, n=192, seed=w.seed_x)
    if w.act == "bf16":
        y = gemm(xdev(x), Wq, Ws, m, K, N, BF16)
        ref, bnd = oracle.gemv_bf16(x, q, s, cols)
    else:
        buf = g.quantize(x)
        xq, dx = g.act_host(buf, m, K)
        rq, rd = oracle.quantize_act(x)
        np.testing.assert_array_equal(xq, rq)
        np.testing.assert_array_equal(dx.view(np.uint32), rd.view(np.uint32))
        y = gemm(buf, Wq, Ws, m, K, N, Q8)
        ref, bnd = oracle.gemv_q8(xq, dx, q, s, cols)
        # int32 dots bit-exact on 16 rows at full K and N (all 512 rows' dots
        # would take 3.7 GB)
        buf16 = g.quantize(x[:16])
        D = gemm_dots(buf16, Wq, 16, K, N)
        np.testing.assert_array_equal(D[:, :, cols].astype(np.int64),
                                      oracle.block_dots(xq[:16], q, cols))
        del D
    assert_close(y[:, cols], ref, bnd, name)
    assert (y[:, N:].view(np.uint32) == 0).all()
    assert np.isfinite(y).all()


def test_gemm_most_rows():
    """m = Q8_MAX_GEMM_ROWS (8192 rows, 64 row blocks of 128), both formats."""
    m, K, N = q8.Q8_MAX_GEMM_ROWS, 256, 130
    x, q, s = inputs.random_case(m, K, N, seed=5000)
    Wq, Ws = g.pack(q, s)
    y = gemm(xdev(x), Wq, Ws, m, K, N, BF16)
    ref, bnd = oracle.gemv_bf16(x, q, s)
    assert_close(y[:, :N], ref, bnd, "gemm bf16 m=8192")
    assert (y[:, N:].view(np.uint32) == 0).all()
    buf = g.quantize(x)
    xq, dx = g.act_host(buf, m, K)
    y = gemm(buf, Wq, Ws, m, K, N, Q8)
    ref, bnd = oracle.gemv_q8(xq, dx, q, s)
    assert_close(y[:, :N], ref, bnd, "gemm int8 m=8192")


# Up to 64 rows the product streams each column tile once through the
# tile-per-workgroup kernel (16, 32 or 64 rows a wave; 8 waves, or 4 where a
# long K's int8 activation scales fill the LDS, as at K = 14336, also in row
# chunks); a K whose scales do not fit
# even then goes to the GEMM.  Up to 1024 rows, chunks of 64 rows in
# workgroups of their own while tiles x chunks stay within 512 (bf16) or 1024
# (int8).
# Full sizes, sampled columns.
@pytest.mark.parametrize("m,K,N,act", [(17, 4096, 14336, BF16), (48, 4096, 14336, BF16),
                                       (64, 4096, 14336, BF16), (64, 5120, 32000, BF16),
                                       (33, 4096, 14336, Q8), (64, 4096, 14336, Q8),
                                       (64, 14336, 4096, Q8), (64, 16384, 200, Q8),
                                       (128, 4096, 14336, BF16), (200, 4096, 14336, Q8),
                                       (256, 4096, 4096, BF16), (96, 4096, 24576, BF16),
                                       (250, 5120, 1000, Q8), (512, 4096, 2048, BF16),
                                       (1024, 4096, 1024, BF16), (1000, 2048, 2048, Q8),
                                       (130, 14336, 512, Q8)])
def test_gemm_tile_rows_full_size(m, K, N, act):
    x, q, s = inputs.random_case(m, K, N, seed=5300 + m + K // 32 + N)
    Wq, Ws = g.pack(q, s)
    cols = _sample_cols(N, n=160, seed=m + N)
    if act == BF16:
        y = gemm(xdev(x), Wq, Ws, m, K, N, BF16)
        ref, bnd = oracle.gemv_bf16(x, q, s, cols)
    else:
        buf = g.quantize(x)
        xq, dx = g.act_host(buf, m, K)
        y = gemm(buf, Wq, Ws, m, K, N, Q8)
        ref, bnd = oracle.gemv_q8(xq, dx, q, s, cols)
    assert_close(y[:, cols], ref, bnd, f"gemm m={m} K={K} N={N} act={act}")
    assert (y[:, N:].view(np.uint32) == 0).all()
    assert np.isfinite(y).all()


# ------------------------------------------------------------------------------
# the GEMM in parts (plan.rs, GemmParts above the GEMV's rows)
# ------------------------------------------------------------------------------

def gemm_parts(xin, packed, Ns, biases, m, K, act):
    ys = [torch.full((m, q8.q8_padded_cols(N)), float("nan"), dtype=torch.float32,
                     device=g.DEV) for N in Ns]
    bdev = [None if b is None else g.dev(b) for b in biases]
    parts = [q8.make_part(W, Ws, y, N, bias=b)
             for (W, Ws), y, N, b in zip(packed, ys, Ns, bdev)]
    q8.q8_gemm_parts(xin, parts, m, K, act)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


PART_SETS = [(200, 40, 64, 130), (4096, 1024, 1024), (96,), (320, 260)]


def _tile_route(m, K, N, act):
    """Whether the many-row product of N columns takes the tile kernel (the
    library's rule, for K whose activation scales fit the LDS): up to 64 rows
    always, up to 1024 while 64-column tiles x chunks of 64 rows stay within
    512 (bf16) or 1024 (int8) workgroups; two-word activations never."""
    if act not in (BF16, Q8) or m > 1024:
        return False
    chunks, tiles = (m + 63) // 64, (N + 63) // 64
    return chunks == 1 or tiles * chunks <= (512 if act == BF16 else 1024)


@pytest.mark.parametrize("act", [BF16, Q8, q8.Q8_ACT_Q8_0_TWO_WORDS])
@pytest.mark.parametrize("m", [1, 33, 64, 100, 200, 300, 1100])
@pytest.mark.parametrize("Ns", PART_SETS)
def test_gemm_parts(act, m, Ns):
    K = 1056 if max(Ns) < 4096 else 512
    seed = 5000 + m + sum(Ns) + act
    x = inputs.gen_x(m, K, seed)
    ws = [(inputs.gen_q(K, N, seed + 10 * i + 1), inputs.gen_scales(K, N, seed + 10 * i + 1))
          for i, N in enumerate(Ns)]
    biases = [inputs.gen_bias(N, seed=seed + i) if i % 2 == 0 else None
              for i, N in enumerate(Ns)]
    packed = [g.pack(q, s) for q, s in ws]
    if act == BF16:
        xin = xdev(x)
    elif act == Q8:
        xin = g.quantize(x)
        rq, rd = oracle.quantize_act(x)
        xq, dx = g.act_host(xin, m, K)
        np.testing.assert_array_equal(xq, rq)
        np.testing.assert_array_equal(dx.view(np.uint32), rd.view(np.uint32))
    else:
        from tests.test_gpu_two_words import _words_checked
        xin, (rh, rl, rd2) = _words_checked(x)
    ys = gemm_parts(xin, packed, Ns, biases, m, K, act)
    for i, ((q, s), N, b, y) in enumerate(zip(ws, Ns, biases, ys)):
        if act == BF16:
            z, bnd = oracle.gemv_bf16(x, q, s)
        elif act == Q8:
            z, bnd = oracle.gemv_q8(rq, rd, q, s)
        else:
            z, bnd = oracle.gemv_q8_two_words(rh, rl, rd2, q, s)
        z, bnd = oracle.epilogue(z, bnd, b)
        assert_close(y[:, :N], z, bnd, f"gemm part {i} act={act} m={m} Ns={Ns}")
        assert (y[:, N:].view(np.uint32) == 0).all(), f"part {i}: pad columns not zero"
        if b is None and _tile_route(m, K, sum(q8.q8_padded_cols(n) for n in Ns), act) == \
                _tile_route(m, K, N, act):
            y1 = gemm(xin, *packed[i], m, K, N, act)
            np.testing.assert_array_equal(y.view(np.uint32), y1.view(np.uint32),
                                          err_msg=f"part {i} differs from q8_gemm alone")


def test_gemm_parts_qkv_prefill_full_size():
    """The attention's query, key and value projections of a 512-row prefill
    chunk, one launch, every column against the oracle."""
    m, K, Ns = 512, 4096, (4096, 1024, 1024)
    x = inputs.gen_x(m, K, 5100)
    ws = [(inputs.gen_q(K, N, 5101 + i), inputs.gen_scales(K, N, 5101 + i)) for i, N in enumerate(Ns)]
    biases = [inputs.gen_bias(N, seed=5110 + i) for i, N in enumerate(Ns)]
    packed = [g.pack(q, s) for q, s in ws]
    ys = gemm_parts(xdev(x), packed, Ns, biases, m, K, BF16)
    for i, ((q, s), N, b, y) in enumerate(zip(ws, Ns, biases, ys)):
        z, bnd = oracle.gemv_bf16(x, q, s)
        z, bnd = oracle.epilogue(z, bnd, b)
        assert_close(y[:, :N], z, bnd, f"qkv part {i}")


@pytest.mark.parametrize("act", [BF16, Q8])
def test_gemm_parts_tile_rows_full_size(act):
    """A gated pair's two 14336-column projections of a 40-row chunk in one
    launch (tile-per-workgroup kernel): sampled columns against the oracle,
    and the part without a bias bit for bit equal to q8_gemm on it alone."""
    m, K, Ns = 40, 4096, (14336, 14336)
    x = inputs.gen_x(m, K, 5400 + act)
    ws = [(inputs.gen_q(K, N, 5401 + i), inputs.gen_scales(K, N, 5401 + i)) for i, N in enumerate(Ns)]
    biases = [inputs.gen_bias(Ns[0], seed=5410), None]
    packed = [g.pack(q, s) for q, s in ws]
    if act == BF16:
        xin = xdev(x)
    else:
        xin = g.quantize(x)
        xq, dx = g.act_host(xin, m, K)
    ys = gemm_parts(xin, packed, Ns, biases, m, K, act)
    for i, ((q, s), N, b, y) in enumerate(zip(ws, Ns, biases, ys)):
        cols = _sample_cols(N, n=128, seed=i)
        if act == BF16:
            z, bnd = oracle.gemv_bf16(x, q, s, cols)
        else:
            z, bnd = oracle.gemv_q8(xq, dx, q, s, cols)
        z, bnd = oracle.epilogue(z, bnd, b, cols=cols)
        assert_close(y[:, cols], z, bnd, f"tile-rows part {i} act={act}")
        assert (y[:, N:].view(np.uint32) == 0).all()
    y1 = gemm(xin, *packed[1], m, K, Ns[1], act)
    np.testing.assert_array_equal(ys[1].view(np.uint32), y1.view(np.uint32))


@pytest.mark.parametrize("Ns", [(14336, 24576), (4096, 4096)])
def test_gemm_parts_route_of_the_launch(Ns):
    """128 bf16 rows: the parts launch takes the kernel of one product of all
    its columns (14336 + 24576: the GEMM, though 14336 alone takes the tile
    kernel; 4096 + 4096: the tile kernel, as each alone).  Each part against
    the oracle on sampled columns, and against q8_gemm alone bit for bit
    where both take the same kernel, else within the tolerance."""
    m, K = 128, 4096
    x = inputs.gen_x(m, K, 5500)
    ws = [(inputs.gen_q(K, N, 5501 + i), inputs.gen_scales(K, N, 5501 + i)) for i, N in enumerate(Ns)]
    packed = [g.pack(q, s) for q, s in ws]
    xin = xdev(x)
    ys = gemm_parts(xin, packed, Ns, [None, None], m, K, BF16)
    launch = _tile_route(m, K, sum(q8.q8_padded_cols(N) for N in Ns), BF16)
    for i, ((q, s), N, y) in enumerate(zip(ws, Ns, ys)):
        cols = _sample_cols(N, n=96, seed=10 + i)
        z, bnd = oracle.gemv_bf16(x, q, s, cols)
        assert_close(y[:, cols], z, bnd, f"part {i}")
        y1 = gemm(xin, *packed[i], m, K, N, BF16)
        if _tile_route(m, K, N, BF16) == launch:
            np.testing.assert_array_equal(y.view(np.uint32), y1.view(np.uint32))
        else:
            assert_close(y1[:, cols], z, bnd, f"part {i} alone")
