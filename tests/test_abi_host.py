"""The C-ABI library on the host: it loads, exports every function the header
declares, and rejects bad arguments before any device work (no GPU needed:
every call here returns from host-side validation)."""
import ctypes
import os
import re

import pytest

import block_quantized_weight_02_amd as q8
from block_quantized_weight_02_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8gemv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libq8gemv.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 18
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # the binding covers the same set under the same names
    assert sorted(binding.exported_names()) == names


def test_sizes():
    assert q8.q8_padded_cols(40) == 64
    assert q8.q8_padded_cols(64) == 64
    assert q8.q8_padded_cols(65) == 128
    assert q8.q8_padded_cols(0) == -1
    assert q8.q8_packed_values_bytes(5120, 40) == 5120 * 64
    assert q8.q8_packed_scales_bytes(5120, 40) == 160 * 64 * 4
    assert q8.q8_packed_values_bytes(4096, 14336) == 4096 * 14336
    assert q8.q8_packed_values_bytes(33, 14) == 0
    assert q8.q8_act_scales_offset(32, 5120) == 163840
    assert q8.q8_act_view_offset(32, 5120) == 163840 + 32 * 160 * 4
    assert q8.q8_act_bytes(32, 5120) == 163840 + 32 * 160 * 4 + 163840
    assert q8.q8_act_view_offset(3, 96) == 768          # scales at 512, 36 bytes, rounded to 768
    assert q8.q8_act_bytes(3, 96) == q8.q8_act_view_offset(3, 96) + 288
    assert q8.q8_act_scales_offset(1, 32) == 256
    assert q8.q8_layout_version() == 2


def expect(status, fn, *args):
    with pytest.raises(q8.Q8Error) as e:
        fn(*args)
    assert e.value.status == status, e.value
    assert q8.q8_last_error() != ""
    return e.value.message


A = 1 << 20   # a 16-byte aligned fake address; never dereferenced
S0 = 0        # null stream, never reached


@pytest.mark.parametrize("m,K,N", [(0, 64, 8), (33, 64, 8), (1, 0, 8), (1, 48, 8),
                                   (1, 64, 0), (-1, 64, 8), (1, -32, 8)])
def test_gemv_shape_errors(m, K, N):
    msg = expect(1, q8.q8_gemv, A, A, A, A, m, K, N, 0, S0)
    assert ("m =" in msg) or ("K =" in msg) or ("N =" in msg)


def test_whole_block_error_names_declared_and_bound():
    msg = expect(1, q8.q8_gemv, A, A, A, A, 1, 1000, 8, 0, S0)
    assert "declared 1000" in msg and "bound 1024" in msg


def test_act_fmt_error():
    expect(2, q8.q8_gemv, A, A, A, A, 1, 64, 8, 3, S0)
    expect(2, q8.q8_gemv, A, A, A, A, 1, 64, 8, -1, S0)


@pytest.mark.parametrize("which", range(4))
def test_null_errors(which):
    ptrs = [A, A, A, A]
    ptrs[which] = None
    msg = expect(3, q8.q8_gemv, *ptrs, 1, 64, 8, 0, S0)
    assert "NULL" in msg


@pytest.mark.parametrize("which", range(4))
def test_alignment_errors(which):
    ptrs = [A, A, A, A]
    ptrs[which] = A + 8
    expect(4, q8.q8_gemv, *ptrs, 1, 64, 8, 0, S0)


def test_other_entry_points_validate():
    expect(1, q8.q8_repack, A, A, 48, 8, A, A, S0)
    expect(3, q8.q8_repack, None, A, 64, 8, A, A, S0)
    expect(1, q8.q8_unpack, A, A, 64, 0, A, A, S0)
    expect(1, q8.q8_quantize_act, A, A, 0, 64, S0)
    expect(1, q8.q8_quantize_act, A, A, 1, 70, S0)
    expect(4, q8.q8_quantize_act, A + 4, A, 1, 64, S0)
    expect(1, q8.q8_gemv_block_dots, A, A, A, 40, 64, 8, S0)
    expect(3, q8.q8_gemv_block_dots, A, A, None, 1, 64, 8, S0)
    expect(1, q8.q8_gemv_ws, A, A, A, A, 0, 64, 8, 0, S0, None, 0)
    p = q8.q8_plan()
    p.kernel, p.rows, p.split_k, p.waves = 0, 1, 2, 4
    expect(5, q8.q8_gemv_planned, A, A, A, A, 1, 64, 8, 0, p, S0, None, 0)
    p.split_k = 3   # more splits than K/32 blocks
    expect(7, q8.q8_gemv_planned, A, A, A, A, 1, 64, 8, 0, p, S0, None, 0)
    p.split_k, p.rows = 1, 2
    expect(7, q8.q8_gemv_planned, A, A, A, A, 3, 64, 8, 0, p, S0, None, 0)
    expect(4, q8.q8_gemv_ws, A, A, A, A, 1, 64, 8, 0, S0, A + 8, 1 << 20)


def test_status_strings():
    assert q8.q8_status_string(0) == "Q8_OK"
    assert q8.q8_status_string(5) == "Q8_ERR_WORKSPACE"
    assert q8.q8_status_string(99) == "Q8_ERR_UNKNOWN"


def test_fused_epilogue_validation():
    ep = q8.make_epilogue(write_y=False)           # writes nothing
    msg = expect(3, q8.q8_gemv_fused, A, A, A, A, 1, 64, 8, 0, ep, S0)
    assert "neither" in msg
    ep = q8.make_epilogue(bias=A + 4)
    expect(4, q8.q8_gemv_fused, A, A, A, A, 1, 64, 8, 0, ep, S0)
    ep = q8.make_epilogue(residual=A + 8)
    expect(4, q8.q8_gemv_fused, A, A, A, A, 1, 64, 8, 0, ep, S0)
    ep = q8.make_epilogue(y_q8=A + 2, write_y=False)
    expect(4, q8.q8_gemv_fused, A, A, A, None, 1, 64, 8, 0, ep, S0)
    expect(3, q8.q8_gemv_fused, A, A, A, None, 1, 64, 8, 0, q8.make_epilogue(), S0)
    expect(3, q8.q8_gemv_fused, A, A, A, None, 1, 64, 8, 0, None, S0)
    expect(1, q8.q8_gemv_fused, A, A, A, A, 33, 64, 8, 0, None, S0)
    # the column-group kernel quantizes its output only in the split-K finish
    p = q8.q8_plan()
    p.kernel, p.rows, p.split_k, p.waves, p.kslices = 2, 32, 1, 16, 1
    ep = q8.make_epilogue(y_q8=A)
    msg = expect(7, q8.q8_gemv_planned_fused, A, A, A, A, 32, 64, 8, 1, ep, p, S0, None, 0)
    assert "split_k >= 2" in msg


def _t(p):
    return (p.kernel, p.rows, p.split_k, p.waves, p.kslices)


def test_fused_default_plan_for_quantized_output():
    ep_q = q8.make_epilogue(y_q8=A)
    for (m, K, N) in ((32, 5120, 32000), (32, 2176, 200), (32, 32, 40), (16, 4096, 64)):
        plain = q8.q8_gemv_default_plan(m, K, N, 1)
        fused = q8.q8_gemv_fused_default_plan(m, K, N, 1, ep_q)
        if plain.kernel != q8.Q8_KERNEL_MFMA_COLS or plain.split_k >= 2:
            assert _t(fused) == _t(plain)
        elif K >= 64:
            assert _t(fused) == _t(plain)[:2] + (2,) + _t(plain)[3:]
        else:
            assert fused.kernel == q8.Q8_KERNEL_MFMA
        same = q8.q8_gemv_fused_default_plan(m, K, N, 1, q8.make_epilogue(bias=A))
        assert _t(same) == _t(plain)


def test_gated_pair_validation():
    expect(3, q8.q8_gemv_glu, A, A, A, None, A, A, 1, 64, 8, 0, None, S0)
    expect(4, q8.q8_gemv_glu, A, A, A, A, A + 4, A, 1, 64, 8, 0, None, S0)
    expect(1, q8.q8_gemv_glu, A, A, A, A, A, A, 1, 48, 8, 0, None, S0)
    expect(2, q8.q8_gemv_glu, A, A, A, A, A, A, 1, 64, 8, 3, None, S0)
    ep = q8.make_glu_epilogue(write_y=False)
    expect(3, q8.q8_gemv_glu, A, A, A, A, A, A, 1, 64, 8, 0, ep, S0)
    ep = q8.make_glu_epilogue(bias_u=A + 8)
    expect(4, q8.q8_gemv_glu, A, A, A, A, A, A, 1, 64, 8, 0, ep, S0)
    p = q8.q8_gemv_glu_default_plan(1, 64, 8, 0)
    # the two weights' carries always meet in the workspace
    need = q8.q8_glu_workspace_bytes(p, 1, 64, 8)
    assert need >= 4 * 2 ** 20 + 2 * p.split_k * 64 * 4
    expect(5, q8.q8_gemv_glu_planned, A, A, A, A, A, A, 1, 64, 8, 0, None, p, S0, None, 0)
    expect(5, q8.q8_gemv_glu_planned, A, A, A, A, A, A, 1, 64, 8, 0, None, p, S0, A, need - 16)


def test_gated_pair_plan_counts_both_weights():
    # the pair's work is 2 * N_pad columns: its split count is that of a
    # product twice as wide; VALU workgroups beyond one per CU take 4 waves
    for (m, K, N, act) in ((1, 4096, 14336, 0), (1, 4096, 1024, 0), (4, 2048, 200, 1),
                           (16, 4096, 14336, 0)):
        pair = q8.q8_gemv_glu_default_plan(m, K, N, act)
        wide = q8.q8_gemv_default_plan(m, K, 2 * q8.q8_padded_cols(N), act)
        if wide.kernel >= q8.Q8_KERNEL_MFMA32:
            # the tile-per-workgroup kernels run one weight: the pair takes the
            # kernel the product would take without them
            assert pair.kernel in (q8.Q8_KERNEL_VALU, q8.Q8_KERNEL_MFMA, q8.Q8_KERNEL_MFMA_COLS)
            continue
        assert (pair.kernel, pair.rows, pair.split_k, pair.kslices) == \
            (wide.kernel, wide.rows, wide.split_k, wide.kslices)
        if pair.kernel == q8.Q8_KERNEL_VALU:
            assert pair.waves in (wide.waves // 2, wide.waves)
        else:
            assert pair.waves == wide.waves


def _part(N, w=A, s=A, y=A, bias=None):
    return q8.make_part(w, s, y, N, bias=bias)


def test_gemm_parts_validation():
    three = [_part(4096), _part(1024), _part(1024)]
    expect(3, q8.q8_gemm_parts, A, None, 64, 4096, 0, S0)
    expect(1, q8.q8_gemm_parts, A, [], 64, 4096, 0, S0)
    expect(1, q8.q8_gemm_parts, A, [_part(64)] * 5, 64, 4096, 0, S0)
    expect(1, q8.q8_gemm_parts, A, three, 0, 4096, 0, S0)
    expect(1, q8.q8_gemm_parts, A, three, q8.Q8_MAX_GEMM_ROWS + 1, 4096, 0, S0)
    expect(1, q8.q8_gemm_parts, A, three, 64, 48, 0, S0)
    expect(2, q8.q8_gemm_parts, A, three, 64, 4096, 3, S0)
    expect(3, q8.q8_gemm_parts, None, three, 64, 4096, 0, S0)
    expect(4, q8.q8_gemm_parts, A + 2, three, 64, 4096, 0, S0)
    expect(3, q8.q8_gemm_parts, A, [_part(64), _part(64, y=None)], 64, 4096, 0, S0)
    assert "part 1" in q8.q8_last_error()


def test_parts_validation():
    three = [_part(4096), _part(1024), _part(1024)]
    expect(3, q8.q8_gemv_parts, A, None, 1, 4096, 0, S0)
    expect(1, q8.q8_gemv_parts, A, [], 1, 4096, 0, S0)
    expect(1, q8.q8_gemv_parts, A, [_part(64)] * 5, 1, 4096, 0, S0)
    expect(1, q8.q8_gemv_parts, A, [_part(64), _part(0)], 1, 4096, 0, S0)
    expect(1, q8.q8_gemv_parts, A, three, 33, 4096, 0, S0)
    expect(1, q8.q8_gemv_parts, A, three, 1, 48, 0, S0)
    expect(2, q8.q8_gemv_parts, A, three, 1, 4096, 3, S0)
    expect(3, q8.q8_gemv_parts, None, three, 1, 4096, 0, S0)
    expect(3, q8.q8_gemv_parts, A, [_part(64), _part(64, y=None)], 1, 4096, 0, S0)
    assert "part 1" in q8.q8_last_error()
    expect(4, q8.q8_gemv_parts, A, [_part(64), _part(64, s=A + 4)], 1, 4096, 0, S0)
    expect(4, q8.q8_gemv_parts, A, [_part(64, bias=A + 8)], 1, 4096, 0, S0)
    # the padded widths together stay within 2^24 columns
    expect(1, q8.q8_gemv_parts, A, [_part(1 << 24), _part(1)], 1, 64, 0, S0)
    p = q8.q8_gemv_parts_default_plan(three, 1, 4096, 0)
    need = q8.q8_parts_workspace_bytes(p, three, 1, 4096)
    assert need == (4 * 2 ** 20 + p.split_k * 6144 * 4 if p.split_k > 1 else 0)
    if need:
        expect(5, q8.q8_gemv_parts_planned, A, three, 1, 4096, 0, p, S0, None, 0)
        expect(5, q8.q8_gemv_parts_planned, A, three, 1, 4096, 0, p, S0, A, need - 16)
    cols = q8.q8_plan()
    cols.kernel, cols.rows, cols.split_k, cols.waves, cols.kslices = \
        q8.Q8_KERNEL_MFMA_COLS, 32, 1, 16, 1
    expect(7, q8.q8_gemv_parts_planned, A, three, 32, 4096, 1, cols, S0, A, 1 << 30)
    assert q8.q8_parts_workspace_bytes(p, [], 1, 4096) == 0


def test_parts_plan_is_the_side_by_side_product():
    # the parts' columns side by side are one product's work: 1-2 rows the
    # single product's VALU plan; from 3 rows of bf16 or one-word Q8_0 the
    # 16x16x32 tile kernel (which walks parts) with 16 or 32 rows and the
    # split its single-product plan takes, below 128 tiles 16 waves of
    # one-block stages; two-word activations the block-interleaved MFMA kernel
    for (m, K, Ns, act) in ((1, 4096, (4096, 1024, 1024), 0), (8, 4096, (4096, 1024, 1024), 1),
                            (16, 4096, (4096, 1024, 1024), 0), (32, 4096, (100, 30), 1),
                            (4, 2048, (200,), 1), (24, 4096, (8192, 8192), 0),
                            (12, 4096, (14336, 14336), 0)):
        parts = [_part(N) for N in Ns]
        got = q8.q8_gemv_parts_default_plan(parts, m, K, act)
        cols = sum(q8.q8_padded_cols(N) for N in Ns)
        wide = q8.q8_gemv_default_plan(m, K, cols, act)
        if m <= 2:
            assert (got.kernel, got.rows, got.split_k) == (wide.kernel, wide.rows, wide.split_k)
            continue
        assert got.kernel == q8.Q8_KERNEL_MFMA16_TILE and got.rows == (16 if m <= 16 else 32)
        if wide.kernel == q8.Q8_KERNEL_MFMA16_TILE:
            assert (got.rows, got.split_k) == (wide.rows, wide.split_k)
        if cols // 64 < 128:
            assert (got.waves, got.kslices) == (16, 1)
        else:
            assert (got.waves, got.kslices) == (wide.waves, wide.kslices)
        assert 1 <= got.split_k <= K // 32
    got = q8.q8_gemv_parts_default_plan([_part(4096), _part(1024)], 8, 4096,
                                        q8.Q8_ACT_Q8_0_TWO_WORDS)
    assert got.kernel == q8.Q8_KERNEL_MFMA


def test_two_word_rules():
    TW = q8.Q8_ACT_Q8_0_TWO_WORDS
    # sizes: 2m rows of words, then m rows of K/32 scales
    assert q8.q8_act_two_words_scales_offset(3, 64) == 512
    assert q8.q8_act_two_words_bytes(3, 64) == 512 + 3 * 2 * 4
    assert q8.q8_act_two_words_bytes(0, 64) == 0 and q8.q8_act_two_words_bytes(1, 48) == 0
    expect(1, q8.q8_quantize_act_two_words, A, A, 0, 64, S0)
    expect(1, q8.q8_quantize_act_two_words, A, A, 1, 48, S0)
    expect(3, q8.q8_quantize_act_two_words, None, A, 1, 64, S0)
    expect(4, q8.q8_quantize_act_two_words, A, A + 2, 1, 64, S0)
    # GEMV: at most 16 rows, on the MFMA kernel's 32-row tile or (up to 4 rows)
    # the VALU kernel; not the pair or the parts
    expect(1, q8.q8_gemv, A, A, A, A, 17, 64, 8, TW, S0)
    expect(1, q8.q8_gemv_default_plan, 17, 64, 8, TW)
    assert q8.q8_gemv_workspace_bytes(17, 64, 8, TW) == 0
    p = q8.q8_gemv_default_plan(16, 4096, 14336, TW)
    assert (p.kernel, p.rows, p.waves) == (q8.Q8_KERNEL_MFMA, 32, 16)
    p = q8.q8_gemv_default_plan(3, 4096, 14336, TW)
    assert (p.kernel, p.rows) == (q8.Q8_KERNEL_MFMA, 32)
    for m, rows in ((1, 1), (2, 2)):
        p = q8.q8_gemv_default_plan(m, 4096, 14336, TW)
        assert (p.kernel, p.rows) == (q8.Q8_KERNEL_VALU, rows)
    small = q8.q8_gemv_default_plan(1, 4096, 4096, TW)
    assert small.split_k >= 2          # 64 tiles: the splits fill the CUs
    for kernel, rows, waves in ((q8.Q8_KERNEL_VALU, 8, 8), (q8.Q8_KERNEL_MFMA, 16, 16),
                                (q8.Q8_KERNEL_MFMA_COLS, 32, 16)):
        bad = q8.q8_plan()
        bad.kernel, bad.rows, bad.split_k, bad.waves, bad.kslices = kernel, rows, 2, waves, 1
        expect(7, q8.q8_gemv_planned, A, A, A, A, 1, 64, 8, TW, bad, S0, A, 1 << 30)
    # the pair and the parts take two words, within the same row limit
    expect(1, q8.q8_gemv_glu, A, A, A, A, A, A, 17, 64, 8, TW, None, S0)
    expect(1, q8.q8_gemv_glu_default_plan, 17, 64, 8, TW)
    expect(1, q8.q8_gemv_parts, A, [q8.make_part(A, A, A, 64)], 17, 64, TW, S0)
    expect(1, q8.q8_gemv_parts_default_plan, [q8.make_part(A, A, A, 64)], 17, 64, TW)
    expect(3, q8.q8_gemm, None, A, A, A, 64, 64, 8, TW, S0)   # the GEMM takes it


def test_stream_read_argument_errors():
    expect(3, q8.q8_stream_read, None, 1024, 256, 8, 2, A, S0)
    expect(4, q8.q8_stream_read, A + 4, 1024, 256, 8, 2, A, S0)
    expect(1, q8.q8_stream_read, A, 1000, 256, 8, 2, A, S0)       # not whole 16 bytes
    expect(1, q8.q8_stream_read, A, 0, 256, 8, 2, A, S0)
    expect(1, q8.q8_stream_read, A, 1024, 0, 8, 2, A, S0)
    expect(1, q8.q8_stream_read, A, 1024, 256, 17, 2, A, S0)
    expect(1, q8.q8_stream_read, A, 1024, 256, 8, 3, A, S0)
    msg = expect(1, q8.q8_stream_read, A, 1 << 33, 1, 8, 2, A, S0)  # an 8 GiB slice
    assert "slice" in msg


def test_two_block_stages_need_an_even_last_split():
    # the 16x16x32 tile kernel's two-block stages read a pair's two blocks of
    # every row as whole lines; a pair starting at the rows' last block would
    # read past the last row, so plans whose last K split has an odd block
    # count are refused, and the default plan takes one-block stages there
    p = q8.q8_plan()
    p.kernel, p.rows, p.split_k, p.waves, p.kslices = q8.Q8_KERNEL_MFMA16_TILE, 16, 1, 16, 2
    msg = expect(7, q8.q8_gemv_planned, A, A, A, A, 16, 1056, 14336, 0, p, S0, A, 1 << 30)
    assert "even" in msg
    p.split_k = 3          # 33 blocks: splits of 11 -> odd
    expect(7, q8.q8_gemv_planned, A, A, A, A, 16, 1056, 14336, 0, p, S0, A, 1 << 30)
    for (K, N) in ((1056, 14336), (1056, 32000), (4128, 14336)):
        d = q8.q8_gemv_default_plan(16, K, N, 0)
        if d.kernel == q8.Q8_KERNEL_MFMA16_TILE and d.kslices == 2:
            assert (K // 32 // d.split_k) % 2 == 0
