"""Helpers of the GPU tests: device buffers through torch, calls through the
C ABI binding.  No arithmetic of the product lives here."""
import numpy as np
import torch

import block_quantized_weight_02_amd as q8
import oracle

DEV = "cuda:0"


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def empty_bytes(n: int) -> torch.Tensor:
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=DEV)


def pack(q: np.ndarray, s: np.ndarray):
    K, N = q.shape
    Wq = empty_bytes(q8.q8_packed_values_bytes(K, N))
    Ws = torch.empty(q8.q8_packed_scales_bytes(K, N) // 4, dtype=torch.float32, device=DEV)
    q8.q8_repack(dev(q), dev(s), K, N, Wq, Ws)
    return Wq, Ws


def quantize(x_bits: np.ndarray):
    """The HIP quantizer's buffer of x, checked bit for bit against the
    oracle's quantizer before any product reads it (so a product test that
    starts from this buffer compares quantize-then-product end to end)."""
    m, K = x_bits.shape
    buf = empty_bytes(q8.q8_act_bytes(m, K))
    q8.q8_quantize_act(dev(x_bits.view(np.int16)), buf, m, K)
    torch.cuda.synchronize()
    xq, dx = act_host(buf, m, K)
    rq, rd = oracle.quantize_act(x_bits)
    np.testing.assert_array_equal(xq, rq, err_msg="HIP quantizer codes differ from the oracle's")
    np.testing.assert_array_equal(dx.view(np.uint32), rd.view(np.uint32),
                                  err_msg="HIP quantizer scales differ from the oracle's")
    np.testing.assert_array_equal(act_view(buf, m, K), oracle.act_view_ref(rq),
                                  err_msg="HIP quantizer view differs from the oracle's layout")
    return buf


def act_view(buf: torch.Tensor, m: int, K: int) -> np.ndarray:
    """The block-interleaved view region of a quantized activation buffer."""
    off = q8.q8_act_view_offset(m, K)
    return buf.cpu().numpy()[off: off + m * K].view(np.int8)


def act_host(buf: torch.Tensor, m: int, K: int):
    off = q8.q8_act_scales_offset(m, K)
    raw = buf.cpu().numpy()
    xq = raw[: m * K].view(np.int8).reshape(m, K)
    dx = raw[off: off + m * (K // 32) * 4].view(np.float32).reshape(m, K // 32)
    return xq, dx


def gemv(x_dev, Wq, Ws, m, K, N, act, plan=None, workspace=None):
    Npad = q8.q8_padded_cols(N)
    y = torch.full((m, Npad), float("nan"), dtype=torch.float32, device=DEV)
    if plan is None:
        q8.q8_gemv(x_dev, Wq, Ws, y, m, K, N, act)
    else:
        need = q8.q8_plan_workspace_bytes(plan, m, K, N)
        if workspace is None and need:
            workspace = torch.zeros(need, dtype=torch.uint8, device=DEV)
        q8.q8_gemv_planned(x_dev, Wq, Ws, y, m, K, N, act, plan, None, workspace, need)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def block_dots(xbuf, Wq, m, K, N, plan=None):
    Npad = q8.q8_padded_cols(N)
    d = torch.full((m, K // 32, Npad), -(2 ** 31), dtype=torch.int32, device=DEV)
    if plan is None:
        q8.q8_gemv_block_dots(xbuf, Wq, d, m, K, N)
    else:
        q8.q8_gemv_block_dots_planned(xbuf, Wq, d, m, K, N, plan)
    torch.cuda.synchronize()
    return d.cpu().numpy()


def plan(kernel, rows, split_k, waves=4, kslices=1):
    p = q8.q8_plan()
    p.kernel, p.rows, p.split_k, p.waves, p.kslices = kernel, rows, split_k, waves, kslices
    return p
