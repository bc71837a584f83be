"""ctypes binding of libq8gemv.so, the C ABI in include/q8gemv.h.

Argument marshalling only: every function has the C name, takes device
buffers as torch tensors (or raw integer addresses), sizes as ints and an
optional stream (default: torch's current stream on the current device), and
raises ``Q8Error`` carrying the status and ``q8_last_error()`` on failure.
All arithmetic runs in the library's HIP kernels; when the library is not
built, every call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq8gemv.so")

Q8_ACT_BF16 = 0
Q8_ACT_Q8_0 = 1
Q8_ACT_Q8_0_TWO_WORDS = 2
Q8_KERNEL_VALU = 0
Q8_KERNEL_MFMA = 1
Q8_KERNEL_MFMA_COLS = 2
Q8_KERNEL_MFMA32 = 3
Q8_KERNEL_MFMA32_DIRECT = 4
Q8_KERNEL_MFMA32_TILE = 5
Q8_KERNEL_MFMA16_TILE = 6
Q8_MAX_ROWS = 32
Q8_MAX_GEMM_ROWS = 8192
Q8_MAX_PARTS = 4
Q8_MAX_TWO_WORD_ROWS = 16

STATUS = {0: "Q8_OK", 1: "Q8_ERR_SHAPE", 2: "Q8_ERR_ACT_FMT", 3: "Q8_ERR_NULL",
          4: "Q8_ERR_ALIGN", 5: "Q8_ERR_WORKSPACE", 6: "Q8_ERR_HIP", 7: "Q8_ERR_PLAN"}


class Q8Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class q8_plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("kslices", ctypes.c_int32)]

    def __repr__(self):
        return (f"q8_plan(kernel={self.kernel}, rows={self.rows}, split_k={self.split_k}, "
                f"waves={self.waves}, kslices={self.kslices})")


class q8_epilogue(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("residual", ctypes.c_void_p),
                ("y_q8", ctypes.c_void_p), ("write_y", ctypes.c_int32)]


class q8_glu_epilogue(ctypes.Structure):
    _fields_ = [("bias_g", ctypes.c_void_p), ("bias_u", ctypes.c_void_p),
                ("y_q8", ctypes.c_void_p), ("write_y", ctypes.c_int32)]


class q8_part(ctypes.Structure):
    _fields_ = [("W_q8", ctypes.c_void_p), ("W_q8_scale", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int64)]


_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_p = ctypes.c_void_p
_int = ctypes.c_int

# name -> (restype, argtypes)
_SIGS = {
    "q8_padded_cols": (_i64, [_i64]),
    "q8_packed_values_bytes": (_sz, [_i64, _i64]),
    "q8_packed_scales_bytes": (_sz, [_i64, _i64]),
    "q8_act_scales_offset": (_sz, [_i64, _i64]),
    "q8_act_view_offset": (_sz, [_i64, _i64]),
    "q8_act_bytes": (_sz, [_i64, _i64]),
    "q8_act_two_words_scales_offset": (_sz, [_i64, _i64]),
    "q8_act_two_words_bytes": (_sz, [_i64, _i64]),
    "q8_gemv_workspace_bytes": (_sz, [_i64, _i64, _i64, _int]),
    "q8_repack": (_int, [_p, _p, _i64, _i64, _p, _p, _p]),
    "q8_unpack": (_int, [_p, _p, _i64, _i64, _p, _p, _p]),
    "q8_quantize_act": (_int, [_p, _p, _i64, _i64, _p]),
    "q8_quantize_act_two_words": (_int, [_p, _p, _i64, _i64, _p]),
    "q8_gemv": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _p]),
    "q8_gemv_ws": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _p, _p, _sz]),
    "q8_gemv_block_dots": (_int, [_p, _p, _p, _i64, _i64, _i64, _p]),
    "q8_gemv_default_plan": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(q8_plan)]),
    "q8_plan_workspace_bytes": (_sz, [ctypes.POINTER(q8_plan), _i64, _i64, _i64]),
    "q8_gemv_planned": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int,
                               ctypes.POINTER(q8_plan), _p, _p, _sz]),
    "q8_gemv_block_dots_planned": (_int, [_p, _p, _p, _i64, _i64, _i64,
                                          ctypes.POINTER(q8_plan), _p]),
    "q8_gemv_fused": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int,
                             ctypes.POINTER(q8_epilogue), _p]),
    "q8_gemv_planned_fused": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int,
                                     ctypes.POINTER(q8_epilogue), ctypes.POINTER(q8_plan),
                                     _p, _p, _sz]),
    "q8_gemv_fused_default_plan": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(q8_epilogue),
                                          ctypes.POINTER(q8_plan)]),
    "q8_gemv_glu": (_int, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _int,
                           ctypes.POINTER(q8_glu_epilogue), _p]),
    "q8_gemv_glu_planned": (_int, [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _int,
                                   ctypes.POINTER(q8_glu_epilogue), ctypes.POINTER(q8_plan),
                                   _p, _p, _sz]),
    "q8_gemv_glu_default_plan": (_int, [_i64, _i64, _i64, _int, ctypes.POINTER(q8_plan)]),
    "q8_glu_workspace_bytes": (_sz, [ctypes.POINTER(q8_plan), _i64, _i64, _i64]),
    "q8_gemv_parts": (_int, [_p, ctypes.POINTER(q8_part), _int, _i64, _i64, _int, _p]),
    "q8_gemm_parts": (_int, [_p, ctypes.POINTER(q8_part), _int, _i64, _i64, _int, _p]),
    "q8_gemv_parts_planned": (_int, [_p, ctypes.POINTER(q8_part), _int, _i64, _i64, _int,
                                     ctypes.POINTER(q8_plan), _p, _p, _sz]),
    "q8_gemv_parts_default_plan": (_int, [ctypes.POINTER(q8_part), _int, _i64, _i64, _int,
                                          ctypes.POINTER(q8_plan)]),
    "q8_parts_workspace_bytes": (_sz, [ctypes.POINTER(q8_plan), ctypes.POINTER(q8_part), _int,
                                       _i64, _i64]),
    "q8_gemm": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _p]),
    "q8_gemm_block_dots": (_int, [_p, _p, _p, _i64, _i64, _i64, _p]),
    "q8_status_string": (ctypes.c_char_p, [_int]),
    "q8_last_error": (ctypes.c_char_p, []),
    "q8_release_workspaces": (_int, []),
    "q8_stream_read": (_int, [_p, _sz, _int, _int, _int, _p, _p]),
    "q8_gemv_noalloc": (_int, [_p, _p, _p, _p, _i64, _i64, _i64, _int, _p]),
    "q8_noalloc_scratch_bytes": (_sz, []),
    "q8_layout_version": (_int, []),
}

_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded library; raises when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise Q8Error(6, f"{LIB_PATH} is not built: run "
                                 "`python -m block_quantized_weight_02_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                f = getattr(handle, name)
                f.restype = res
                f.argtypes = args
            _lib = handle
    return _lib


def exported_names():
    return list(_SIGS)


def _addr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int) -> None:
    if status != 0:
        msg = lib().q8_last_error()
        raise Q8Error(status, msg.decode() if msg else "")


# ---- sizes ---------------------------------------------------------------------

def q8_padded_cols(N: int) -> int:
    return int(lib().q8_padded_cols(N))


def q8_packed_values_bytes(K: int, N: int) -> int:
    return int(lib().q8_packed_values_bytes(K, N))


def q8_packed_scales_bytes(K: int, N: int) -> int:
    return int(lib().q8_packed_scales_bytes(K, N))


def q8_act_scales_offset(m: int, K: int) -> int:
    return int(lib().q8_act_scales_offset(m, K))


def q8_act_view_offset(m: int, K: int) -> int:
    return int(lib().q8_act_view_offset(m, K))


def q8_act_bytes(m: int, K: int) -> int:
    return int(lib().q8_act_bytes(m, K))


def q8_act_two_words_scales_offset(m: int, K: int) -> int:
    return int(lib().q8_act_two_words_scales_offset(m, K))


def q8_act_two_words_bytes(m: int, K: int) -> int:
    return int(lib().q8_act_two_words_bytes(m, K))


def q8_gemv_workspace_bytes(m: int, K: int, N: int, act_fmt: int) -> int:
    return int(lib().q8_gemv_workspace_bytes(m, K, N, act_fmt))


# ---- calls ----------------------------------------------------------------------

def q8_repack(q_kn, s_kn, K, N, W_q8, W_q8_scale, stream=None) -> None:
    _check(lib().q8_repack(_addr(q_kn), _addr(s_kn), K, N, _addr(W_q8),
                           _addr(W_q8_scale), _stream(stream)))


def q8_unpack(W_q8, W_q8_scale, K, N, q_kn, s_kn, stream=None) -> None:
    _check(lib().q8_unpack(_addr(W_q8), _addr(W_q8_scale), K, N, _addr(q_kn),
                           _addr(s_kn), _stream(stream)))


def q8_quantize_act(x_bf16, x_q8, m, K, stream=None) -> None:
    _check(lib().q8_quantize_act(_addr(x_bf16), _addr(x_q8), m, K, _stream(stream)))


def q8_quantize_act_two_words(x_bf16, x_q8x2, m, K, stream=None) -> None:
    _check(lib().q8_quantize_act_two_words(_addr(x_bf16), _addr(x_q8x2), m, K, _stream(stream)))


def q8_gemv(x, W_q8, W_q8_scale, y, m, K, N, act_fmt, stream=None) -> None:
    _check(lib().q8_gemv(_addr(x), _addr(W_q8), _addr(W_q8_scale), _addr(y),
                         m, K, N, act_fmt, _stream(stream)))


def q8_gemv_ws(x, W_q8, W_q8_scale, y, m, K, N, act_fmt, stream, workspace,
               ws_bytes) -> None:
    _check(lib().q8_gemv_ws(_addr(x), _addr(W_q8), _addr(W_q8_scale), _addr(y),
                            m, K, N, act_fmt, _stream(stream), _addr(workspace),
                            ws_bytes))


def q8_gemv_block_dots(x_q8, W_q8, dots, m, K, N, stream=None) -> None:
    _check(lib().q8_gemv_block_dots(_addr(x_q8), _addr(W_q8), _addr(dots), m, K, N,
                                    _stream(stream)))


def q8_gemv_default_plan(m, K, N, act_fmt) -> q8_plan:
    p = q8_plan()
    _check(lib().q8_gemv_default_plan(m, K, N, act_fmt, ctypes.byref(p)))
    return p


def q8_plan_workspace_bytes(plan: q8_plan, m, K, N) -> int:
    return int(lib().q8_plan_workspace_bytes(ctypes.byref(plan), m, K, N))


def q8_gemv_planned(x, W_q8, W_q8_scale, y, m, K, N, act_fmt, plan: q8_plan,
                    stream=None, workspace=None, ws_bytes=0) -> None:
    _check(lib().q8_gemv_planned(_addr(x), _addr(W_q8), _addr(W_q8_scale), _addr(y),
                                 m, K, N, act_fmt, ctypes.byref(plan), _stream(stream),
                                 _addr(workspace), ws_bytes))


def q8_gemv_block_dots_planned(x_q8, W_q8, dots, m, K, N, plan: q8_plan,
                               stream=None) -> None:
    _check(lib().q8_gemv_block_dots_planned(_addr(x_q8), _addr(W_q8), _addr(dots),
                                            m, K, N, ctypes.byref(plan), _stream(stream)))


def make_epilogue(bias=None, residual=None, y_q8=None, write_y=True) -> q8_epilogue:
    """A ``q8_epilogue`` over device tensors (or raw addresses, or None)."""
    return q8_epilogue(_addr(bias), _addr(residual), _addr(y_q8), 1 if write_y else 0)


def _ep_ref(epilogue):
    return None if epilogue is None else ctypes.byref(epilogue)


def q8_gemv_fused(x, W_q8, W_q8_scale, y, m, K, N, act_fmt, epilogue: q8_epilogue = None,
                  stream=None) -> None:
    _check(lib().q8_gemv_fused(_addr(x), _addr(W_q8), _addr(W_q8_scale), _addr(y),
                               m, K, N, act_fmt, _ep_ref(epilogue), _stream(stream)))


def q8_gemv_planned_fused(x, W_q8, W_q8_scale, y, m, K, N, act_fmt,
                          epilogue: q8_epilogue, plan: q8_plan, stream=None,
                          workspace=None, ws_bytes=0) -> None:
    _check(lib().q8_gemv_planned_fused(_addr(x), _addr(W_q8), _addr(W_q8_scale), _addr(y),
                                       m, K, N, act_fmt, _ep_ref(epilogue),
                                       ctypes.byref(plan), _stream(stream),
                                       _addr(workspace), ws_bytes))


def q8_gemv_fused_default_plan(m, K, N, act_fmt, epilogue: q8_epilogue = None) -> q8_plan:
    p = q8_plan()
    _check(lib().q8_gemv_fused_default_plan(m, K, N, act_fmt, _ep_ref(epilogue),
                                            ctypes.byref(p)))
    return p


def make_glu_epilogue(bias_g=None, bias_u=None, y_q8=None, write_y=True) -> q8_glu_epilogue:
    """A ``q8_glu_epilogue`` over device tensors (or raw addresses, or None)."""
    return q8_glu_epilogue(_addr(bias_g), _addr(bias_u), _addr(y_q8), 1 if write_y else 0)


def q8_gemv_glu(x, Wg_q8, Wg_q8_scale, Wu_q8, Wu_q8_scale, y, m, K, N, act_fmt,
                epilogue: q8_glu_epilogue = None, stream=None) -> None:
    _check(lib().q8_gemv_glu(_addr(x), _addr(Wg_q8), _addr(Wg_q8_scale), _addr(Wu_q8),
                             _addr(Wu_q8_scale), _addr(y), m, K, N, act_fmt,
                             _ep_ref(epilogue), _stream(stream)))


def q8_gemv_glu_planned(x, Wg_q8, Wg_q8_scale, Wu_q8, Wu_q8_scale, y, m, K, N, act_fmt,
                        epilogue: q8_glu_epilogue, plan: q8_plan, stream=None,
                        workspace=None, ws_bytes=0) -> None:
    _check(lib().q8_gemv_glu_planned(_addr(x), _addr(Wg_q8), _addr(Wg_q8_scale),
                                     _addr(Wu_q8), _addr(Wu_q8_scale), _addr(y), m, K, N,
                                     act_fmt, _ep_ref(epilogue), ctypes.byref(plan),
                                     _stream(stream), _addr(workspace), ws_bytes))


def q8_gemv_glu_default_plan(m, K, N, act_fmt) -> q8_plan:
    p = q8_plan()
    _check(lib().q8_gemv_glu_default_plan(m, K, N, act_fmt, ctypes.byref(p)))
    return p


def q8_glu_workspace_bytes(plan: q8_plan, m, K, N) -> int:
    return int(lib().q8_glu_workspace_bytes(ctypes.byref(plan), m, K, N))


def make_part(W_q8, W_q8_scale, y, N, bias=None) -> q8_part:
    """A ``q8_part`` over device tensors (or raw addresses, or None)."""
    return q8_part(_addr(W_q8), _addr(W_q8_scale), _addr(bias), _addr(y), N)


def _parts_ref(parts):
    """(host array, count) of a sequence of ``q8_part``; None passes NULL."""
    if parts is None:
        return None, 0
    parts = list(parts)
    return (q8_part * max(1, len(parts)))(*parts), len(parts)


def q8_gemv_parts(x, parts, m, K, act_fmt, stream=None) -> None:
    arr, n = _parts_ref(parts)
    _check(lib().q8_gemv_parts(_addr(x), arr, n, m, K, act_fmt, _stream(stream)))


def q8_gemm_parts(x, parts, m, K, act_fmt, stream=None) -> None:
    arr, n = _parts_ref(parts)
    _check(lib().q8_gemm_parts(_addr(x), arr, n, m, K, act_fmt, _stream(stream)))


def q8_gemv_parts_planned(x, parts, m, K, act_fmt, plan: q8_plan, stream=None,
                          workspace=None, ws_bytes=0) -> None:
    arr, n = _parts_ref(parts)
    _check(lib().q8_gemv_parts_planned(_addr(x), arr, n, m, K, act_fmt, ctypes.byref(plan),
                                       _stream(stream), _addr(workspace), ws_bytes))


def q8_gemv_parts_default_plan(parts, m, K, act_fmt) -> q8_plan:
    arr, n = _parts_ref(parts)
    p = q8_plan()
    _check(lib().q8_gemv_parts_default_plan(arr, n, m, K, act_fmt, ctypes.byref(p)))
    return p


def q8_parts_workspace_bytes(plan: q8_plan, parts, m, K) -> int:
    arr, n = _parts_ref(parts)
    return int(lib().q8_parts_workspace_bytes(ctypes.byref(plan), arr, n, m, K))


def q8_gemm(x, W_q8, W_q8_scale, y, m, K, N, act_fmt, stream=None) -> None:
    _check(lib().q8_gemm(_addr(x), _addr(W_q8), _addr(W_q8_scale), _addr(y), m, K, N,
                         act_fmt, _stream(stream)))


def q8_gemm_block_dots(x_q8, W_q8, dots, m, K, N, stream=None) -> None:
    _check(lib().q8_gemm_block_dots(_addr(x_q8), _addr(W_q8), _addr(dots), m, K, N,
                                    _stream(stream)))


def q8_status_string(status: int) -> str:
    return lib().q8_status_string(status).decode()


def q8_last_error() -> str:
    return lib().q8_last_error().decode()


def q8_release_workspaces() -> None:
    _check(lib().q8_release_workspaces())


def q8_layout_version() -> int:
    return int(lib().q8_layout_version())


def q8_stream_read(src, nbytes, workgroups, waves, depth, sink, stream=None) -> None:
    _check(lib().q8_stream_read(_addr(src), nbytes, workgroups, waves, depth, _addr(sink),
                                _stream(stream)))


def q8_gemv_noalloc(x, W_q8, W_q8_scale, y, m, K, N, act_fmt, stream=None) -> None:
    _check(lib().q8_gemv_noalloc(_addr(x), _addr(W_q8), _addr(W_q8_scale), _addr(y), m, K, N,
                                 act_fmt, _stream(stream)))


def q8_noalloc_scratch_bytes() -> int:
    return int(lib().q8_noalloc_scratch_bytes())
