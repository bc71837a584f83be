"""The oracle's pins are sharp: each test here plants one plausible mistake in a
copy of q8_oracle.c (a dropped term, a wrong sign, an off-by-one index, a
wrong rounding rule or constant), builds it on the CPU, runs every pin of
test_oracle_pins.py against it, and requires at least one pin to fail.

Every mutation keeps all memory accesses in bounds (indices are shifted
modulo their extent), so a mutant can only compute wrong values.
"""
import inspect
import itertools
import os

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "q8_oracle.c")

# (name, original text, replacement); each original occurs in q8_oracle.c.
MUTANTS = [
    ("bf16 product drops the last term of a block",
     "          blk += t;\n", "          blk += (i == Q8O_BLOCK - 1) ? 0.0 : t;\n"),
    ("bf16 product takes the next block's scale",
     "double sv = (double)s[b * N + n];", "double sv = (double)s[((b + 1) % NB) * N + n];"),
    ("bound loses the absolute value of the scale",
     "bnd += fabs(sv) * blk_abs;", "bnd += sv * blk_abs;"),
    ("bf16 product reads the next activation row",
     "bf16_value(x[r * K + k]) * (double)q[k * N + n]",
     "bf16_value(x[((r + 1) % m) * K + k]) * (double)q[k * N + n]"),
    ("bf16 product reads the neighbouring weight column",
     "bf16_value(x[r * K + k]) * (double)q[k * N + n]",
     "bf16_value(x[r * K + k]) * (double)q[k * N + (n + 1) % N]"),
    ("block dots drop the first term",
     "          acc += (int64_t)xq[r * K + k] * (int64_t)q[k * N + n];\n",
     "          if (i) acc += (int64_t)xq[r * K + k] * (int64_t)q[k * N + n];\n"),
    ("int8 product takes the next block's activation scale",
     "double scale = (double)dx[r * NB + b] * (double)s[b * N + n];",
     "double scale = (double)dx[r * NB + (b + 1) % NB] * (double)s[b * N + n];"),
    ("activation quantizer rounds ties to even",
     "double rv = round_half_away((double)quot);", "double rv = rint((double)quot);"),
    ("activation quantizer divides by 128",
     "float d = (float)(amax / 127.0);", "float d = (float)(amax / 128.0);"),
    ("exact encoder uses amax/126",
     "double d = amax / 127.0;", "double d = amax / 126.0;"),
    ("exact encoder accepts non-integer multiples",
     "if (fabs(v - r) > 1e-9 || fabs(r) > 127.0 || r * d != wv) return 0;",
     "if (fabs(r) > 127.0) return 0;"),
    ("dequant takes the next block's scale",
     "(double)s[(k / Q8O_BLOCK) * N + n]",
     "(double)s[((k / Q8O_BLOCK + 1) % (K / Q8O_BLOCK)) * N + n]"),
    ("output quantizer rounds ties to even",
     "float quot = (float)((double)zb[i] / (double)d);\n          double rv = round_half_away((double)quot);",
     "float quot = (float)((double)zb[i] / (double)d);\n          double rv = rint((double)quot);"),
    ("output quantizer scale reads the neighbouring block",
     "float d = (float)(amax / 127.0);\n      dz[r * NB + b] = d;",
     "float d = (float)(amax / 127.0);\n      dz[r * NB + (b + 1) % NB] = d;"),
    ("SiLU takes sigmoid of +v",
     "double sig = 1.0 / (1.0 + exp(-gv));", "double sig = 1.0 / (1.0 + exp(gv));"),
    ("gated pair drops the up factor",
     "out[r * n + j] = gv * sig * uv;", "out[r * n + j] = gv * sig;"),
    ("gated pair adds the gate bias to the up product",
     "double uv = u[r * n + j] + (bu ? (double)bu[j] : 0.0);",
     "double uv = u[r * n + j] + (bg ? (double)bg[j] : 0.0);"),
    ("two-word residual in steps of 1/127",
     "vl = (int)round_half_away(128.0 * ((double)quot - rh));",
     "vl = (int)round_half_away(127.0 * ((double)quot - rh));"),
    ("two-word residual rounds ties to even",
     "vl = (int)round_half_away(128.0 * ((double)quot - rh));",
     "vl = (int)rint(128.0 * ((double)quot - rh));"),
    ("two-word residual taken from the unrounded quotient's floor",
     "vl = (int)round_half_away(128.0 * ((double)quot - rh));",
     "vl = (int)round_half_away(128.0 * ((double)quot - floor((double)quot)));"),
    ("two-word product reads the first word twice",
     "dot_lo += (int64_t)lo[r * K + k] * w;", "dot_lo += (int64_t)hi[r * K + k] * w;"),
    ("two-word product scales the second word by 1/127",
     "acc += scale * ((double)dot_hi + (double)dot_lo / 128.0);",
     "acc += scale * ((double)dot_hi + (double)dot_lo / 127.0);"),
    ("two-word bound drops the second word",
     "dot_abs += fabs(((double)hi[r * K + k] + (double)lo[r * K + k] / 128.0) * (double)w);",
     "dot_abs += fabs((double)hi[r * K + k] * (double)w);"),
    ("epilogue takes the neighbouring column's bias",
     "v += (double)bias[n];", "v += (double)bias[(n + 1) % ncols];"),
    ("epilogue reads the residual with the output's row stride",
     "v += (double)residual[r * res_stride + n];", "v += (double)residual[r * ncols + n];"),
    ("epilogue bound drops the residual",
     "b += fabs((double)residual[r * res_stride + n]);", "b += 0.0;"),
    ("view rows drop the K tail",
     "return m * ((K + chunk - 1) / chunk) * Q8O_BLOCK;", "return m * (K / chunk) * Q8O_BLOCK;"),
    ("byte model counts 2-byte scales",
     "*weight = K * padded + 4 * (K / Q8O_BLOCK) * padded;",
     "*weight = K * padded + 2 * (K / Q8O_BLOCK) * padded;"),
]


def _pin_calls():
    """Every pin of test_oracle_pins.py as (name, callable) with its
    parametrize cases expanded."""
    calls = []
    for name, fn in sorted(vars(pins).items()):
        if not (name.startswith("test_") and inspect.isfunction(fn)):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            calls.append((name, fn, {}))
            continue
        grids = []
        for mk in marks:
            argnames = [a.strip() for a in mk.args[0].split(",")] if isinstance(mk.args[0], str) \
                else list(mk.args[0])
            cases = [v if len(argnames) > 1 else (v,) for v in mk.args[1]]
            grids.append([dict(zip(argnames, c)) for c in cases])
        for combo in itertools.product(*grids):
            kw = {}
            for d in combo:
                kw.update(d)
            calls.append((name, fn, kw))
    return calls


def _failures():
    failed = []
    for name, fn, kw in _pin_calls():
        try:
            fn(**kw)
        except Exception:   # an assertion, or a wrong-shaped result
            failed.append(name)
    return failed


def test_pins_pass_on_the_oracle():
    assert _failures() == []


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, label, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mutated = src.replace(old, new, 1)
    path = tmp_path / "q8_oracle_mutant.c"
    path.write_text(mutated)
    lib = oracle_build.build(src=str(path), out=str(tmp_path / "liboracle_mutant.so"))
    prev = oracle.swap_library(lib)
    try:
        failed = _failures()
    finally:
        oracle._lib = prev
    assert failed, f"no pin caught: {label}"


# Planted mistakes in the numpy packed-layout reference (oracle.repack_ref):
# each replaces the function with a plausible wrong permutation, and some pin
# of the layout must then fail.
def _swap_halves(q, s):
    K, N = q.shape
    NB, Np = K // 32, (N + 63) // 64 * 64
    qp = np.zeros((K, Np), np.int8)
    qp[:, :N] = q
    v = qp.reshape(NB, 2, 16, Np // 64, 64).transpose(3, 0, 1, 4, 2)[:, :, ::-1]
    return np.ascontiguousarray(v).ravel(), _REPACK(q, s)[1]


def _block_major(q, s):
    K, N = q.shape
    NB, Np = K // 32, (N + 63) // 64 * 64
    qp = np.zeros((K, Np), np.int8)
    qp[:, :N] = q
    v = qp.reshape(NB, 2, 16, Np // 64, 64).transpose(0, 3, 1, 4, 2)
    return np.ascontiguousarray(v).ravel(), _REPACK(q, s)[1]


def _scales_in_column_order(q, s):
    K, N = q.shape
    NB, Np = K // 32, (N + 63) // 64 * 64
    sp = np.zeros((NB, Np), np.float32)
    sp[:, :N] = s
    w = sp.reshape(NB, Np // 64, 64).transpose(1, 0, 2)
    return _REPACK(q, s)[0], np.ascontiguousarray(w).ravel()


def _k_reversed(q, s):
    K, N = q.shape
    NB, Np = K // 32, (N + 63) // 64 * 64
    qp = np.zeros((K, Np), np.int8)
    qp[:, :N] = q
    v = qp.reshape(NB, 2, 16, Np // 64, 64).transpose(3, 0, 1, 4, 2)[..., ::-1]
    return np.ascontiguousarray(v).ravel(), _REPACK(q, s)[1]


def _view_row_major_blocks(xq):
    xq = np.asarray(xq, np.int8)
    return np.ascontiguousarray(xq).ravel()


_REPACK = oracle.repack_ref
LAYOUT_MUTANTS = [("halves swapped", _swap_halves), ("block-major chunks", _block_major),
                  ("scales in column order", _scales_in_column_order),
                  ("k reversed inside a half", _k_reversed)]


@pytest.mark.parametrize("label,fn", LAYOUT_MUTANTS, ids=[m[0] for m in LAYOUT_MUTANTS])
def test_planted_layout_mistake_is_caught(monkeypatch, label, fn):
    monkeypatch.setattr(oracle, "repack_ref", fn)
    failed = [name for name, f, kw in _pin_calls() if "packed_layout" in name
              and not _passes(f, kw)]
    assert failed, f"no layout pin caught: {label}"


def _passes(fn, kw):
    try:
        fn(**kw)
        return True
    except Exception:
        return False


def test_planted_view_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "act_view_ref", _view_row_major_blocks)
    failed = [name for name, f, kw in _pin_calls() if "activation_view" in name
              and not _passes(f, kw)]
    assert failed
