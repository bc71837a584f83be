#!/usr/bin/env python3
"""Benchmark of the Q8_0 weight product on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch: for bf16 activations one
q8_gemv call; for Q8_0 activations q8_quantize_act followed by q8_gemv.  The
weight is repacked once before timing (it is a load-time step).  Inputs are
seeded synthetic tensors of the workload's shape, resident in HBM.  Every
step reads a different copy of the weight, enough copies to span four times
the 256 MB last-level cache, so the weight streams from HBM rather than from
the cache.

`python bench.py --copy-calibration` instead times a plain device-to-device
copy of 256 MiB; profiler byte counters read on it give the factor that turns
the counters into bytes.

Prints ONE JSON line on stdout.  `value` is the whole-job rate in GB/s of
algorithmic bytes (weight values + fp32 scales + activation + output) over
the timed steps; `roofline` prices the product kernel's own average duration
against 8 TB/s.  Every timed region is exactly its step count of launches,
queued behind a bounded device-side hold so that they run back to back (HIP
events on the launch stream around them; see time_loop);
`cpu_baseline` times the CPU oracle on the same workload on this host;
`by_config` gives the same measurement (step and product) at every other
configuration (m = 1, 16 and 32); `fused_epilogue`
times the product with bias, residual and quantized output beside the plain
product, at m = 1 and m = 32, and the gated pair (gate and up through SiLU in
one launch) beside two plain products, at m = 1 and m = 16, and the product
in parts (query, key and value projections of one activation in one launch)
beside the same products one by one, at m = 1 and m = 16, and the two-word
int8 activation (quantize then product) beside the one-word step, at m = 1
and m = 16; `context` gives
the read ceiling (q8_stream_read over the headline's bytes, best of a grid
sweep), the headline with one weight copy reused and a 1 GiB device copy's
rate;
`prefill` times the many-row product (m = 512, and m = 128 on the tile
kernel's row chunks) against the MFMA peak, with
bf16, one-word and two-word int8 activations.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MALL_BYTES = 256 * 2 ** 20      # MI355X Infinity Cache
ROTATE_BYTES = 4 * MALL_BYTES   # weight copies span this much: every read misses the cache
METRIC = "Q8_0 GEMV effective HBM GB/s (% of peak) and weights/s at m=1,16,32"
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w) -> dict:
    """Bytes the product must move once: weight values and scales over the
    padded columns, the activation as the kernel reads it, and the output."""
    Npad = (w.N + 63) // 64 * 64
    values = w.K * Npad
    scales = 4 * (w.K // 32) * Npad
    if w.act == "bf16":
        x = 2 * w.m * w.K
    else:
        x = w.m * w.K + 4 * w.m * (w.K // 32)
    y = 4 * w.m * Npad
    return {"values": values, "scales": scales, "x": x, "y": y,
            "total": values + scales + x + y}


def kernel_name(plan: dict, w) -> str:
    """The kernel a plan launches for a single product, as rocprofv3 names it."""
    act = 0 if w.act == "bf16" else 1
    r, wv, ks = plan["rows"], plan["waves"], plan.get("kslices", 1)
    if plan["kernel"] == 0:
        return f"gemv_valu_kernel<{r}, {act}, false, {wv}, false, false>"
    if plan["kernel"] == 1:
        return f"gemv_mfma_kernel<{r}, {act}, false, {wv}, false, false>"
    if plan["kernel"] == 5:
        return f"gemv_mfma32w_kernel<{wv}, false, {ks}>"
    if plan["kernel"] == 6:
        return (f"gemv_tile16_kernel<{act}, {wv}, false, {'true' if ks == 2 else 'false'}, "
                f"{r // 16}>")
    return f"gemv_mfma_cols_kernel<{r}, {act}, false, {ks}, {wv // (4 * ks)}, false, false>"


def plan_grid(plan: dict, w) -> str:
    """rocprofv3's Grid_Size X x Y x Z (threads) of a tile-per-workgroup
    product launch (kernels 0, 5 and 6: one workgroup per tile and K split)."""
    tiles = (w.N + 63) // 64
    if plan["kernel"] == 5:   # kslices column tiles a workgroup
        ks = plan.get("kslices", 1)
        tiles = (tiles + ks - 1) // ks
    return f"{tiles * 64 * plan['waves']}x{plan['split_k']}x1"


def _code_only(text: str) -> str:
    """C/C++ source with its comments and blank lines removed (string
    literals in these sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def csrc_hash() -> str:
    """Hash of the library's sources, comments aside: the profiler counters
    stay valid for a kernel whose code has not changed."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "block_quantized_weight_02_amd", "csrc")
    for name in sorted(os.listdir(d)):
        with open(os.path.join(d, name), encoding="utf-8") as f:
            h.update(name.encode() + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(PROFILES, f"pmc_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("csrc_hash") != csrc_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


class Setup:
    """Device buffers of one workload: rotating packed weight copies, the
    activation (bf16, and its quantized buffer), the output."""

    def __init__(self, w, rotate=True):
        import torch
        import block_quantized_weight_02_amd as q8
        from block_quantized_weight_02_amd import inputs
        self.w = w
        self.q8 = q8
        dev = "cuda:0"
        x, q, s = inputs.generate(w)
        self.host = (x, q, s)
        K, N, m = w.K, w.N, w.m
        vb, sb = q8.q8_packed_values_bytes(K, N), q8.q8_packed_scales_bytes(K, N)
        self.copies = max(2, math.ceil(ROTATE_BYTES / (vb + sb))) if rotate else 1
        qd = torch.from_numpy(q).to(dev)
        sd = torch.from_numpy(s).to(dev)
        self.W = []
        for _ in range(self.copies):
            Wq = torch.empty(vb, dtype=torch.uint8, device=dev)
            Ws = torch.empty(sb // 4, dtype=torch.float32, device=dev)
            q8.q8_repack(qd, sd, K, N, Wq, Ws)
            self.W.append((Wq, Ws))
        del qd, sd
        self.x = torch.from_numpy(x.view(np.int16)).to(dev)
        self.xq = torch.empty(max(16, q8.q8_act_bytes(m, K)), dtype=torch.uint8, device=dev)
        self.y = torch.empty((m, q8.q8_padded_cols(N)), dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        # pre-marshalled raw arguments: the timed loop is one ctypes call per launch
        lib = q8.lib()
        self._gemv = lib.q8_gemv
        self._quant = lib.q8_quantize_act
        sp = self.stream.cuda_stream
        act = q8.Q8_ACT_BF16 if w.act == "bf16" else q8.Q8_ACT_Q8_0
        xin = self.x.data_ptr() if w.act == "bf16" else self.xq.data_ptr()
        self._gemv_args = [(xin, Wq.data_ptr(), Ws.data_ptr(), self.y.data_ptr(), m, K, N, act, sp)
                           for (Wq, Ws) in self.W]
        self._quant_args = (self.x.data_ptr(), self.xq.data_ptr(), m, K, sp)
        self.plan = q8.q8_gemv_default_plan(m, K, N, act) if m <= q8.Q8_MAX_ROWS else None

    def step(self, i):
        if self.w.act != "bf16":
            rc = self._quant(*self._quant_args)
            if rc:
                raise RuntimeError(self.q8.q8_last_error())
        rc = self._gemv(*self._gemv_args[i % self.copies])
        if rc:
            raise RuntimeError(self.q8.q8_last_error())

    def gemv_only(self, i):
        rc = self._gemv(*self._gemv_args[i % self.copies])
        if rc:
            raise RuntimeError(self.q8.q8_last_error())


_HOLD = {"cycles_per_ms": None}


def _hold_cycles_per_ms():
    """Clock rate of the device-side hold (torch's bounded spin kernel), timed
    once with events."""
    import torch
    if _HOLD["cycles_per_ms"] is None:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record()
        torch.cuda._sleep(2_000_000)
        e1.record()
        torch.cuda.synchronize()
        _HOLD["cycles_per_ms"] = 2_000_000 / max(e0.elapsed_time(e1), 1e-3)
    return _HOLD["cycles_per_ms"]


PREHEAT_MS = 100.0


def preheat(fn, ms=PREHEAT_MS):
    """Untimed launches of `fn` for about `ms` milliseconds of host time before
    a measurement: an idle GPU runs its first launches slower (measured on
    MI355X: the first 20-launch loop of a process 13.2-13.7 us per launch of
    the m=1 product, every later one 11.5-11.7 us, and 11.5-11.7 us for the
    first one after 50 ms of launches), and a decode loop keeps it busy."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < ms * 1e-3:
        fn(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return i


def time_loop(fn, steps, info=None):
    """Milliseconds per step of exactly `steps` steps run back to back on the
    launch stream.

    The launches are queued behind a bounded device-side hold (a spin kernel)
    and the start event is recorded after it, so the host's launch latency
    cannot open gaps between them: the GPU finds every launch already queued.
    That the host finished queueing before the hold ended is checked (the
    start event has not been reached yet); otherwise the hold is lengthened
    and the measurement retaken (at most three times; `info["back_to_back"]`
    says whether it held)."""
    import torch
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    hold_ms = 2.0 + 0.02 * steps           # ~20 us of host time per queued step
    queued = False
    for _ in range(3):
        torch.cuda._sleep(int(hold_ms * _hold_cycles_per_ms()))
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        queued = not e0.query()
        torch.cuda.synchronize()
        if queued:
            break
        hold_ms *= 4
    if info is not None:
        info["back_to_back"] = queued
        info["hold_ms"] = hold_ms
    return e0.elapsed_time(e1) / steps


def measure(w, steps, warmup, rotate=True):
    """One workload's step and product: `warmup` untimed steps, then exactly
    `steps` timed steps back to back; for Q8_0 activations the product alone
    is timed the same way (its launches are the step's minus the quantize)."""
    import torch
    st = Setup(w, rotate=rotate)
    b = algorithmic_bytes(w)
    log(f"[bench] {w.name}: m={w.m} K={w.K} N={w.N} act={w.act} copies={st.copies} "
        f"plan={st.plan} bytes/step={b['total']}")
    preheat(st.gemv_only)
    for i in range(warmup):
        st.step(i)
    torch.cuda.synchronize()
    info = {}
    t0 = time.perf_counter()
    ms = time_loop(st.step, steps, info)
    wall = time.perf_counter() - t0
    gemv_ms = ms if w.act == "bf16" else time_loop(st.gemv_only, steps, info)
    log(f"[bench] {w.name}: {ms * 1e3:.2f} us/step, product kernel {gemv_ms * 1e3:.2f} us/launch "
        f"(back to back: {info['back_to_back']})")
    step_bytes = b["total"]
    weights = w.K * w.N
    res = {
        "workload": w.name, "m": w.m, "K": w.K, "N": w.N, "act": w.act,
        "ms_per_step": ms, "us_per_step": ms * 1e3,
        "gbs": step_bytes / (ms * 1e-3) / 1e9,
        "weights_per_s": weights / (ms * 1e-3),
        "macs_per_s": w.m * weights / (ms * 1e-3),
        "kernel_us_mean": gemv_ms * 1e3,
        "launches_timed": steps, "back_to_back": info["back_to_back"],
        "preheat_ms": PREHEAT_MS,
        "bytes": b, "copies": st.copies, "wall_s": wall,
        "plan": {"kernel": st.plan.kernel, "rows": st.plan.rows,
                 "split_k": st.plan.split_k, "waves": st.plan.waves, "kslices": st.plan.kslices},
    }
    # the product kernel moves every algorithmic byte (its x is the quantized
    # buffer in Q8_0 mode); the quantize launch is counted in the step only
    res["kernel_gbs"] = step_bytes / (res["kernel_us_mean"] * 1e-6) / 1e9
    res["pct_hbm_peak"] = 100.0 * res["gbs"] / HBM_PEAK_GBS
    res["kernel_pct_hbm_peak"] = 100.0 * res["kernel_gbs"] / HBM_PEAK_GBS
    del st
    torch.cuda.empty_cache()
    return res


def read_ceiling(torch, nbytes, steps):
    """The read ceiling at the product's size: q8_stream_read over `nbytes`
    (the product's algorithmic bytes), each launch a different window of a
    1 GiB buffer (as the product rotates its weight copies), over a sweep of
    grid shapes; returns the best and every shape's rate."""
    import block_quantized_weight_02_amd as q8
    span = 2 ** 30
    buf = torch.empty(span, dtype=torch.uint8, device="cuda:0")
    buf.random_(0, 255)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    n = (nbytes + 15) // 16 * 16
    nwin = max(2, (span - n) // n)
    offs = [(i * n) // 256 * 256 for i in range(nwin)]
    base = buf.data_ptr()
    lib = q8.lib()
    sp = torch.cuda.current_stream().cuda_stream
    sink_p = sink.data_ptr()
    rows = []
    for wgs in (224, 256, 512, 1024, 2048):
        for waves in (4, 8, 16):
            for depth in (1, 2, 4):
                def call(i, wgs=wgs, waves=waves, depth=depth):
                    rc = lib.q8_stream_read(base + offs[i % nwin], n, wgs, waves, depth, sink_p, sp)
                    if rc:
                        raise RuntimeError(q8.q8_last_error())
                for i in range(20):
                    call(i)
                ms = time_loop(call, steps)
                rows.append({"workgroups": wgs, "waves": waves, "depth": depth,
                             "us": ms * 1e3, "gbs": n / (ms * 1e-3) / 1e9})
    # the sweep's maximum is biased upward by run-to-run noise: the five
    # fastest shapes are timed three more times and ranked by their median
    top = sorted(rows, key=lambda r: -r["gbs"])[:5]
    for r in top:
        def call(i, r=r):
            rc = lib.q8_stream_read(base + offs[i % nwin], n, r["workgroups"], r["waves"],
                                    r["depth"], sink_p, sp)
            if rc:
                raise RuntimeError(q8.q8_last_error())
        reps = [r["us"]] + [time_loop(call, steps) * 1e3 for _ in range(3)]
        r["us_repeats"] = reps
        r["us_median"] = float(np.median(reps))
        r["gbs_median"] = n / (r["us_median"] * 1e-6) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    best = max(top, key=lambda r: r["gbs_median"])
    best = dict(best, us=best["us_median"], gbs=best["gbs_median"])
    same = [r for r in rows if (r["workgroups"], r["waves"], r["depth"]) == (224, 8, 4)]
    log(f"[bench] read ceiling over {n} B: {best['us']:.2f} us, {best['gbs']:.0f} GB/s "
        f"({best['workgroups']} x {best['waves']} waves, depth {best['depth']})")
    return {"bytes": n, "launches_per_shape": steps, "best": best,
            "product_grid_shape": same[0] if same else None, "sweep": rows}


def measure_fused(w, steps, warmup, rotate=True):
    """The product with its full epilogue (bias, residual add, y, and the
    quantized output for the next projection), against the plain product on
    the same buffers.  Returns per-launch times and the epilogue's extra bytes."""
    import ctypes
    import torch
    st = Setup(w, rotate=rotate)
    q8 = st.q8
    from block_quantized_weight_02_amd import inputs
    m, K, N = w.m, w.K, w.N
    Npad = q8.q8_padded_cols(N)
    bias = torch.from_numpy(inputs.gen_bias(N, seed=w.seed_w + 7)).to("cuda:0")
    res = torch.from_numpy(inputs.gen_residual(m, Npad, seed=w.seed_w + 8)).to("cuda:0")
    yq = torch.empty(q8.q8_act_bytes(m, Npad), dtype=torch.uint8, device="cuda:0")
    ep = q8.make_epilogue(bias=bias, residual=res, y_q8=yq, write_y=True)
    act = q8.Q8_ACT_BF16 if w.act == "bf16" else q8.Q8_ACT_Q8_0
    plan = q8.q8_gemv_fused_default_plan(m, K, N, act, ep)
    fused = q8.lib().q8_gemv_fused
    epp = ctypes.byref(ep)
    args = [a[:8] + (epp, a[8]) for a in st._gemv_args]

    def call(i):
        rc = fused(*args[i % st.copies])
        if rc:
            raise RuntimeError(q8.q8_last_error())

    if w.act != "bf16":
        st.step(0)   # the quantized activation the products read
    for i in range(warmup):
        call(i)
        st.gemv_only(i)
    plain_ms = time_loop(st.gemv_only, steps)
    fused_ms = time_loop(call, steps)
    extra = 4 * N + 4 * m * Npad + m * Npad + 4 * m * (Npad // 32)
    b = algorithmic_bytes(w)["total"] + extra
    del st
    torch.cuda.empty_cache()
    log(f"[bench] fused {w.name}: {fused_ms * 1e3:.2f} us vs plain {plain_ms * 1e3:.2f} us, "
        f"plan={plan}")
    return {"workload": w.name, "epilogue": "bias + residual + y + quantized y",
            "fused_us": fused_ms * 1e3, "plain_us": plain_ms * 1e3,
            "fused_bytes": b, "fused_gbs": b / (fused_ms * 1e-3) / 1e9,
            "plan": {"kernel": plan.kernel, "rows": plan.rows, "split_k": plan.split_k,
                     "waves": plan.waves, "kslices": plan.kslices}}


def measure_glu(w, steps, warmup, rotate=True):
    """The gated pair (gate and up products of one activation through SiLU,
    one launch) against two plain products of the same weights."""
    import ctypes
    import torch
    st = Setup(w, rotate=rotate)
    q8 = st.q8
    m, K, N = w.m, w.K, w.N
    act = q8.Q8_ACT_BF16 if w.act == "bf16" else q8.Q8_ACT_Q8_0
    glu = q8.lib().q8_gemv_glu
    plan = q8.q8_gemv_glu_default_plan(m, K, N, act)
    xin = st.x.data_ptr() if w.act == "bf16" else st.xq.data_ptr()
    sp = st.stream.cuda_stream
    n = st.copies
    args = [(xin, st.W[i][0].data_ptr(), st.W[i][1].data_ptr(), st.W[(i + 1) % n][0].data_ptr(),
             st.W[(i + 1) % n][1].data_ptr(), st.y.data_ptr(), m, K, N, act, None, sp)
            for i in range(n)]

    def call(i):
        rc = glu(*args[i % n])
        if rc:
            raise RuntimeError(q8.q8_last_error())

    def two_products(i):
        st.gemv_only(i)
        st.gemv_only(i + 1)

    if w.act != "bf16":
        st.step(0)
    for i in range(warmup):
        call(i)
        two_products(i)
    two_ms = time_loop(two_products, steps)
    glu_ms = time_loop(call, steps)
    b = algorithmic_bytes(w)
    pair_bytes = 2 * (b["values"] + b["scales"]) + b["x"] + b["y"]
    del st
    torch.cuda.empty_cache()
    log(f"[bench] gated pair {w.name}: {glu_ms * 1e3:.2f} us vs two products {two_ms * 1e3:.2f} us, "
        f"plan={plan}")
    return {"workload": w.name, "glu_us": glu_ms * 1e3, "two_products_us": two_ms * 1e3,
            "bytes": pair_bytes, "glu_gbs": pair_bytes / (glu_ms * 1e-3) / 1e9,
            "plan": {"kernel": plan.kernel, "rows": plan.rows, "split_k": plan.split_k,
                     "waves": plan.waves, "kslices": plan.kslices}}


def measure_parts(pw, steps, warmup, rotate=True, gemm=False):
    """The product in parts (several projections of one activation, one
    launch) against the same products launched one by one; with gemm, the
    many-row forms (q8_gemm_parts against q8_gemm per part)."""
    import torch
    import block_quantized_weight_02_amd as q8
    from block_quantized_weight_02_amd import inputs
    dev = "cuda:0"
    m, K, Ns = pw.m, pw.K, pw.Ns
    act = q8.Q8_ACT_BF16 if pw.act == "bf16" else q8.Q8_ACT_Q8_0
    x, ws = inputs.generate_parts(pw)
    per_copy = sum(q8.q8_packed_values_bytes(K, N) + q8.q8_packed_scales_bytes(K, N) for N in Ns)
    copies = max(2, math.ceil(ROTATE_BYTES / per_copy)) if rotate else 1
    Wd = []
    for (q, s), N in zip(ws, Ns):
        qd, sd = torch.from_numpy(q).to(dev), torch.from_numpy(s).to(dev)
        one = []
        for _ in range(copies):
            Wq = torch.empty(q8.q8_packed_values_bytes(K, N), dtype=torch.uint8, device=dev)
            Ws = torch.empty(q8.q8_packed_scales_bytes(K, N) // 4, dtype=torch.float32, device=dev)
            q8.q8_repack(qd, sd, K, N, Wq, Ws)
            one.append((Wq, Ws))
        Wd.append(one)
        del qd, sd
    xb = torch.from_numpy(x.view(np.int16)).to(dev)
    xq = torch.empty(max(16, q8.q8_act_bytes(m, K)), dtype=torch.uint8, device=dev)
    if act == q8.Q8_ACT_Q8_0:
        q8.q8_quantize_act(xb, xq, m, K)
    xin = xb.data_ptr() if act == q8.Q8_ACT_BF16 else xq.data_ptr()
    ys = [torch.empty((m, q8.q8_padded_cols(N)), dtype=torch.float32, device=dev) for N in Ns]
    sp = torch.cuda.current_stream().cuda_stream
    lib = q8.lib()
    arrs = []
    for c in range(copies):
        parts = [q8.make_part(Wd[i][c][0], Wd[i][c][1], ys[i], N) for i, N in enumerate(Ns)]
        arrs.append((q8.q8_part * len(parts))(*parts))
    singles = [[(xin, Wd[i][c][0].data_ptr(), Wd[i][c][1].data_ptr(), ys[i].data_ptr(), m, K, N,
                 act, sp) for i, N in enumerate(Ns)] for c in range(copies)]
    plan = None if gemm else q8.q8_gemv_parts_default_plan(list(arrs[0]), m, K, act)
    parts_fn = lib.q8_gemm_parts if gemm else lib.q8_gemv_parts
    single_fn = lib.q8_gemm if gemm else lib.q8_gemv
    torch.cuda.synchronize()

    def call(i):
        rc = parts_fn(xin, arrs[i % copies], len(Ns), m, K, act, sp)
        if rc:
            raise RuntimeError(q8.q8_last_error())

    def one_by_one(i):
        for a in singles[i % copies]:
            rc = single_fn(*a)
            if rc:
                raise RuntimeError(q8.q8_last_error())

    for i in range(warmup):
        call(i)
        one_by_one(i)
    sep_ms = time_loop(one_by_one, steps)
    parts_ms = time_loop(call, steps)
    xbytes = 2 * m * K if act == q8.Q8_ACT_BF16 else m * K + 4 * m * (K // 32)
    nbytes = per_copy + xbytes + sum(4 * m * q8.q8_padded_cols(N) for N in Ns)
    del Wd, arrs, singles
    torch.cuda.empty_cache()
    log(f"[bench] parts {pw.name}: {parts_ms * 1e3:.2f} us vs one by one {sep_ms * 1e3:.2f} us, "
        f"plan={plan if plan is not None else 'q8_gemm_parts'}")
    out = {"workload": pw.name, "Ns": list(Ns), "parts_us": parts_ms * 1e3,
           "one_by_one_us": sep_ms * 1e3, "bytes": nbytes,
           "parts_gbs": nbytes / (parts_ms * 1e-3) / 1e9}
    if gemm:
        flops = 2.0 * m * K * sum(Ns)
        out["tflops"] = flops / (parts_ms * 1e-3) / 1e12
        out["frac_of_mfma_peak"] = out["tflops"] / MFMA_PEAK_TFLOPS[pw.act]
    else:
        out["plan"] = {"kernel": plan.kernel, "rows": plan.rows, "split_k": plan.split_k,
                       "waves": plan.waves, "kslices": plan.kslices}
    return out


def measure_two_words(w, steps, warmup, rotate=True):
    """The two-word int8 activation (the two-pass numerics): a step is
    q8_quantize_act_two_words then q8_gemv, beside the one-word step
    (q8_quantize_act then q8_gemv) on the same weights."""
    import torch
    st = Setup(w, rotate=rotate)
    q8 = st.q8
    m, K, N = w.m, w.K, w.N
    lib = q8.lib()
    sp = st.stream.cuda_stream
    x2 = torch.empty(q8.q8_act_two_words_bytes(m, K), dtype=torch.uint8, device="cuda:0")
    tw = q8.Q8_ACT_Q8_0_TWO_WORDS
    gemv_args = [(x2.data_ptr(), Wq.data_ptr(), Ws.data_ptr(), st.y.data_ptr(), m, K, N, tw, sp)
                 for (Wq, Ws) in st.W]
    one_args = [(st.xq.data_ptr(), Wq.data_ptr(), Ws.data_ptr(), st.y.data_ptr(), m, K, N,
                 q8.Q8_ACT_Q8_0, sp) for (Wq, Ws) in st.W]
    quant2 = (st.x.data_ptr(), x2.data_ptr(), m, K, sp)
    plan = q8.q8_gemv_default_plan(m, K, N, tw)

    def ok(rc):
        if rc:
            raise RuntimeError(q8.q8_last_error())

    def two(i):
        ok(lib.q8_quantize_act_two_words(*quant2))
        ok(lib.q8_gemv(*gemv_args[i % st.copies]))

    def two_product(i):
        ok(lib.q8_gemv(*gemv_args[i % st.copies]))

    def one(i):
        ok(st._quant(*st._quant_args))
        ok(lib.q8_gemv(*one_args[i % st.copies]))

    for i in range(warmup):
        two(i)
        one(i)
    product_ms = time_loop(two_product, steps)
    two_ms = time_loop(two, steps)
    one_ms = time_loop(one, steps)
    b = algorithmic_bytes(w)
    xbytes = 2 * m * K + 4 * m * (K // 32)
    nbytes = b["values"] + b["scales"] + xbytes + b["y"]
    del st
    torch.cuda.empty_cache()
    log(f"[bench] two words {w.name}: step {two_ms * 1e3:.2f} us (product {product_ms * 1e3:.2f} us) "
        f"vs one word {one_ms * 1e3:.2f} us, plan={plan}")
    return {"workload": w.name, "two_words_step_us": two_ms * 1e3,
            "two_words_product_us": product_ms * 1e3, "one_word_step_us": one_ms * 1e3,
            "product_bytes": nbytes, "product_gbs": nbytes / (product_ms * 1e-3) / 1e9,
            "plan": {"kernel": plan.kernel, "rows": plan.rows, "split_k": plan.split_k,
                     "waves": plan.waves, "kslices": plan.kslices}}


MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "q8_0": 5000.0}   # MI355X dense, published


def measure_gemm(w, steps, warmup, rotate=True, two_words=False):
    """The many-row product (prefill chunk): q8_gemm per step; with Q8_0
    activations (one or two words) the step also quantizes them (reported
    apart too).  TFLOP/s count the product's 2*m*K*N; the two-word form runs
    twice that on the matrix cores."""
    import torch
    st = Setup(w, rotate=rotate)
    q8 = st.q8
    m, K, N = w.m, w.K, w.N
    act = q8.Q8_ACT_BF16 if w.act == "bf16" else q8.Q8_ACT_Q8_0
    quant, quant_args = st._quant, st._quant_args
    xin = st.x.data_ptr() if w.act == "bf16" else st.xq.data_ptr()
    if two_words:
        act = q8.Q8_ACT_Q8_0_TWO_WORDS
        x2 = torch.empty(q8.q8_act_two_words_bytes(m, K), dtype=torch.uint8, device="cuda:0")
        xin = x2.data_ptr()
        quant = q8.lib().q8_quantize_act_two_words
        quant_args = (st.x.data_ptr(), xin, m, K, st.stream.cuda_stream)
    gemm = q8.lib().q8_gemm
    sp = st.stream.cuda_stream
    args = [(xin, Wq.data_ptr(), Ws.data_ptr(), st.y.data_ptr(), m, K, N, act, sp)
            for (Wq, Ws) in st.W]

    def product(i):
        rc = gemm(*args[i % st.copies])
        if rc:
            raise RuntimeError(q8.q8_last_error())

    def step(i):
        if w.act != "bf16":
            rc = quant(*quant_args)
            if rc:
                raise RuntimeError(q8.q8_last_error())
        product(i)

    for i in range(warmup):
        step(i)
    gemm_ms = time_loop(product, steps)
    step_ms = time_loop(step, steps) if w.act != "bf16" else gemm_ms
    flops = 2.0 * m * K * N
    b = algorithmic_bytes(w)
    peak = MFMA_PEAK_TFLOPS[w.act]
    del st
    torch.cuda.empty_cache()
    tf = flops / (gemm_ms * 1e-3) / 1e12
    form = " two words" if two_words else ""
    log(f"[bench] gemm {w.name}{form}: {gemm_ms * 1e3:.2f} us/launch ({tf:.0f} TFLOP/s, "
        f"{100 * tf / peak:.1f}% of {peak:.0f}), step {step_ms * 1e3:.2f} us")
    return {"workload": w.name, "m": m, "K": K, "N": N,
            "act": w.act + ("_two_words" if two_words else ""),
            "us_per_step": step_ms * 1e3, "kernel_us_mean": gemm_ms * 1e3,
            "tflops": tf, "peak_tflops": peak, "frac_of_mfma_peak": tf / peak,
            "gbs_algorithmic": b["total"] / (gemm_ms * 1e-3) / 1e9}


def cpu_baseline(w, budget_s=12.0):
    """The CPU oracle (as it stands) on this host, on the same workload."""
    import oracle
    from block_quantized_weight_02_amd import inputs
    x, q, s = inputs.generate(w)
    if w.act == "bf16":
        run = lambda: oracle.gemv_bf16(x, q, s)  # noqa: E731
    else:
        def run():
            xq, dx = oracle.quantize_act(x)
            return oracle.gemv_q8(xq, dx, q, s)
    run()  # warm (page in)
    reps, t0 = 0, time.perf_counter()
    while True:
        run()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 200:
            break
    per = el / reps
    b = algorithmic_bytes(w)["total"]
    cores = oracle.threads()
    # the same on one thread (a few products: about 2 s)
    oracle.set_threads(1)
    try:
        t1 = []
        for _ in range(3):
            t0 = time.perf_counter()
            run()
            t1.append(time.perf_counter() - t0)
    finally:
        oracle.set_threads(0)
    per1 = sorted(t1)[1]
    return {"value": b / per / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} full {w.name} products (m={w.m} K={w.K} N={w.N}), "
                      f"{per * 1e3:.1f} ms each, fp64 C oracle, OpenMP",
            "ms_per_step": per * 1e3, "weights_per_s": w.K * w.N / per,
            "one_thread": {"value": b / per1 / 1e9, "ms_per_step": per1 * 1e3,
                           "sample": "median of 3 full products on 1 thread"}}


def bandwidth_context(torch, w, steps):
    """What surrounds the headline number: the same product with one weight
    copy reused (the 256 MB cache may then hold it: 'MALL-hot'), and a plain
    1 GiB device-to-device copy (reads and writes 1 GiB)."""
    st = Setup(w, rotate=False)
    for i in range(50):
        st.gemv_only(i)
    hot_ms = time_loop(st.gemv_only, steps)
    b = algorithmic_bytes(w)["total"]
    del st
    torch.cuda.empty_cache()
    nbytes = 2 ** 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    cms = time_loop(lambda i: dst.copy_(src), 20)
    del src, dst
    torch.cuda.empty_cache()
    return {"mall_hot_us": hot_ms * 1e3, "mall_hot_gbs": b / (hot_ms * 1e-3) / 1e9,
            "copy_1gib_us": cms * 1e3,
            "copy_1gib_gbs_read_plus_write": 2 * nbytes / (cms * 1e-3) / 1e9}


def copy_calibration(torch, nbytes=256 * 2 ** 20, reps=20):
    """A plain copy of known size: reads nbytes and writes nbytes per launch."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    src.random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ms = time_loop(lambda i: dst.copy_(src), reps)
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "launches": reps + 3,
                      "ms_per_copy": ms, "gbs": 2 * nbytes / (ms * 1e-3) / 1e9}), flush=True)


CONFIG_IDS = {"decode_k1024_n1024": "C1", "decode_k4096_n4096": "C2",
              "ffn_down_k14336_n4096": "C3", "batch16_k4096_n14336": "C4",
              "q8act_m32_k5120_n40": "C5a", "q8act_m32_k5120_n32000": "C5b",
              "decode_k4096_n14336": "T"}


def summarize_kernel_trace(path, bench_json=None):
    """Per-kernel dispatch statistics of a rocprofv3 kernel-trace CSV: count,
    mean, median, p10 and p90 of the dispatch durations (us), in order of
    total time.  Given the JSON line that the traced bench.py run printed, each
    configuration's product launches (kernel name and grid from its plan) are
    labelled with the configuration.  Prints one JSON line."""
    import csv
    from block_quantized_weight_02_amd import inputs
    labels = {}
    if bench_json:
        line = [l for l in open(bench_json).read().splitlines() if l.startswith('{"metric"')][-1]
        rec = json.loads(line)
        cfgs = dict(rec.get("by_config", {}))
        cfgs["T"] = {"workload": rec["config"]["workload"], "plan": rec["config"]["plan"]}
        for cid, c in cfgs.items():
            w = inputs.WORKLOADS[c["workload"]]
            labels.setdefault((kernel_name(c["plan"], w), plan_grid(c["plan"], w)), []).append(cid)
    durs = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("KernelName") or row.get("Name")
            t0, t1 = row.get("Start_Timestamp"), row.get("End_Timestamp")
            if not name or t0 is None or t1 is None:
                continue
            # one kernel serves several shapes: the launch's grid tells them apart
            grid = "x".join(str(int(row.get(f"Grid_Size_{a}", 1) or 1)) for a in "XYZ")
            key = (name, grid, int(row.get("Workgroup_Size_X", 0) or 0))
            durs.setdefault(key, []).append((int(t1) - int(t0)) / 1e3)
    out = []
    for (name, grid, wg), d in durs.items():
        a = np.array(d)
        cfg = [c for (k, g), cs in labels.items() if g == grid and k in name for c in cs]
        out.append({"kernel": name, "configs": cfg, "grid_threads": grid, "workgroup": wg,
                    "dispatches": int(a.size), "total_us": float(a.sum()),
                    "mean_us": float(a.mean()), "median_us": float(np.median(a)),
                    "p10_us": float(np.percentile(a, 10)), "p90_us": float(np.percentile(a, 90))})
    out.sort(key=lambda r: -r["total_us"])
    print(json.dumps({"trace": os.path.basename(path), "kernels": out}), flush=True)


def summarize_pmc(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """HBM traffic of one workload's product kernel from four rocprofv3
    counter-collection CSVs: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of a
    `--workload` run, each scaled by what the same counter reads for the
    `--copy-calibration` copy (256 MiB read and written).  The product kernel
    is the gemv kernel (name and grid) with the most dispatches.  Prints one
    JSON record (the `profiles/pmc_<workload>.json` format)."""
    import csv
    from block_quantized_weight_02_amd import inputs
    w = inputs.WORKLOADS[workload]

    def rows(path, cname):
        out = []
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == cname:
                    out.append((r["Kernel_Name"], r.get("Grid_Size", ""), float(r["Counter_Value"])))
        return out

    def product(path, cname):
        groups = {}
        for name, grid, v in rows(path, cname):
            if "gemv_" in name:
                groups.setdefault((name, grid), []).append(v)
        (name, grid), vals = max(groups.items(), key=lambda kv: len(kv[1]))
        return name, grid, vals

    def copy(path, cname):
        return [v for name, _, v in rows(path, cname) if "copyBuffer" in name]

    kname, grid, g_f = product(fetch_csv, "FETCH_SIZE")
    _, _, g_w = product(write_csv, "WRITE_SIZE")
    c_f, c_w = copy(copy_fetch_csv, "FETCH_SIZE"), copy(copy_write_csv, "WRITE_SIZE")
    copy_bytes = 256 * 2 ** 20
    ff = copy_bytes / (float(np.median(c_f)) * 1024)
    wf = copy_bytes / (float(np.median(c_w)) * 1024)
    rd = float(np.mean(g_f)) * 1024 * ff
    wr = float(np.mean(g_w)) * 1024 * wf
    alg = algorithmic_bytes(w)["total"]
    run = (f"python3 bench.py --workload {workload} --no-rows --no-cpu --no-fused --no-prefill "
           "--no-ceiling --no-context --steps 100 --warmup 10")
    rec = {
        "workload": f"{workload} (m={w.m}, K={w.K}, N={w.N}, {w.act} activations)",
        "kernel": kname, "grid_threads": grid,
        "commands": [f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o bench -- {run}",
                     f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o bench -- {run}",
                     "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o copy -- python3 bench.py --copy-calibration",
                     "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o copy -- python3 bench.py --copy-calibration",
                     f"python3 bench.py --summarize-pmc {workload} <fetch csv> <write csv> <copy fetch csv> <copy write csv>"],
        "dispatches": {"gemv": len(g_f), "copy": len(c_f)},
        "FETCH_SIZE_KiB_per_dispatch": {"gemv_mean": float(np.mean(g_f)), "copy_median": float(np.median(c_f))},
        "WRITE_SIZE_KiB_per_dispatch": {"gemv_mean": float(np.mean(g_w)), "copy_median": float(np.median(c_w))},
        "calibration": {"copy_bytes_each_way": copy_bytes, "fetch_factor": ff, "write_factor": wf,
                        "note": "a plain 256 MiB device copy reads and writes 256 MiB; the factors turn each counter's KiB into bytes"},
        "traffic_read_bytes_per_launch": rd, "traffic_write_bytes_per_launch": wr,
        "traffic_bytes_per_launch": rd + wr, "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": (rd + wr) / alg,
        "csrc_hash": csrc_hash(),
    }
    print(json.dumps(rec, indent=2), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None, help="headline workload name (default: the m=1 decode shape)")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the other configurations (m = 1, 16 and 32 shapes)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle leg")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused-epilogue lines")
    ap.add_argument("--no-prefill", action="store_true", help="skip the many-row (prefill) lines")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-ceiling sweep")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the cache-hot headline and the 1 GiB copy")
    ap.add_argument("--no-rotate", action="store_true", help="one weight copy (cache-hot number)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 256 MiB device copy (for profiler counter calibration)")
    ap.add_argument("--summarize-kernel-trace", metavar="CSV", nargs="+", default=None,
                    help="print per-kernel dispatch statistics of a rocprofv3 kernel trace "
                         "(optionally followed by the traced run's output, to label configurations)")
    ap.add_argument("--summarize-pmc", metavar="ARG", nargs=5, default=None,
                    help="WORKLOAD FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV: HBM traffic "
                         "of the workload's product kernel from rocprofv3 counter CSVs")
    args = ap.parse_args()

    if args.summarize_kernel_trace:
        summarize_kernel_trace(*args.summarize_kernel_trace[:2])
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the product shards by columns across GPUs with no collective)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from block_quantized_weight_02_amd import inputs
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import block_quantized_weight_02_amd as q8
    q8.lib()  # fails loudly when the HIP library is not built

    name = args.workload or inputs.HEADLINE
    w = inputs.WORKLOADS[name]
    head = measure(w, args.steps, args.warmup, rotate=not args.no_rotate)

    # every other configuration, product and step, at least 200 launches each
    by_config = {}
    if not args.no_rows:
        for other, cid in CONFIG_IDS.items():
            if other == name:
                continue
            r = measure(inputs.WORKLOADS[other], max(200, args.steps), max(20, args.warmup),
                        rotate=not args.no_rotate)
            by_config[cid] = {
                k: r[k] for k in ("workload", "m", "K", "N", "act", "us_per_step", "gbs",
                                  "pct_hbm_peak", "weights_per_s", "macs_per_s",
                                  "kernel_us_mean", "kernel_gbs", "kernel_pct_hbm_peak",
                                  "launches_timed", "back_to_back", "plan")}
            # HBM bytes per launch from the committed counter record, while the
            # kernel sources are the ones it was taken on
            by_config[cid]["traffic"] = traffic_from_profile(other)

    fused = {}
    if not args.no_fused:
        for other in (name, "q8act_m32_k5120_n32000"):
            r = measure_fused(inputs.WORKLOADS[other], max(200, args.steps // 4),
                              max(20, args.warmup // 4), rotate=not args.no_rotate)
            fused[f"m{inputs.WORKLOADS[other].m}"] = r
        for other in (name, "batch16_k4096_n14336"):
            r = measure_glu(inputs.WORKLOADS[other], max(200, args.steps // 4),
                            max(20, args.warmup // 4), rotate=not args.no_rotate)
            fused[f"glu_m{inputs.WORKLOADS[other].m}"] = r
        for other in ("qkv_decode_k4096", "qkv_batch16_k4096"):
            r = measure_parts(inputs.PARTS_WORKLOADS[other], max(200, args.steps // 4),
                              max(20, args.warmup // 4), rotate=not args.no_rotate)
            fused[f"parts_m{inputs.PARTS_WORKLOADS[other].m}"] = r
        for other in (name, "batch16_k4096_n14336"):
            r = measure_two_words(inputs.WORKLOADS[other], max(200, args.steps // 4),
                                  max(20, args.warmup // 4), rotate=not args.no_rotate)
            fused[f"two_words_m{inputs.WORKLOADS[other].m}"] = r

    prefill = {}
    if not args.no_prefill:
        for other in ("prefill_m512_k4096_n14336", "prefill_q8act_m512_k4096_n14336"):
            prefill[inputs.WORKLOADS[other].act] = measure_gemm(
                inputs.WORKLOADS[other], max(100, args.steps // 10), max(10, args.warmup // 10),
                rotate=not args.no_rotate)
        for other in ("prefill_m128_k4096_n14336", "prefill_q8act_m128_k4096_n14336"):
            prefill[inputs.WORKLOADS[other].act + "_m128"] = measure_gemm(
                inputs.WORKLOADS[other], max(100, args.steps // 10), max(10, args.warmup // 10),
                rotate=not args.no_rotate)
        prefill["q8_0_two_words"] = measure_gemm(
            inputs.WORKLOADS["prefill_q8act_m512_k4096_n14336"], max(100, args.steps // 10),
            max(10, args.warmup // 10), rotate=not args.no_rotate, two_words=True)
        prefill["parts_m512"] = measure_parts(
            inputs.PARTS_WORKLOADS["qkv_prefill_m512_k4096"], max(100, args.steps // 10),
            max(10, args.warmup // 10), rotate=not args.no_rotate, gemm=True)

    context = {}
    if not args.no_ceiling:
        context["read_ceiling"] = read_ceiling(torch, head["bytes"]["total"], 200)
        best = context["read_ceiling"]["best"]["gbs"]
        context["product_frac_of_read_ceiling"] = head["kernel_gbs"] / best
    if not args.no_rows and not args.no_context:
        context.update(bandwidth_context(torch, w, 200))
        log(f"[bench] context: one weight copy {context['mall_hot_us']:.2f} us; 1 GiB copy "
            f"{context['copy_1gib_gbs_read_plus_write']:.0f} GB/s read+write")

    traffic = traffic_from_profile(w.name)
    achieved = head["kernel_gbs"]
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "kernel": kernel_name(head["plan"], w),
            "kernel_us_mean": head["kernel_us_mean"], "launches_timed": head["launches_timed"],
            "back_to_back": head["back_to_back"], "bytes_per_launch": head["bytes"]["total"]}

    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(w)

    out = {
        "metric": METRIC,
        "value": head["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "m": w.m, "K": w.K, "N": w.N, "act": w.act,
                   "weight": "q8_0: int8 values + fp32 scale per 32 rows",
                   "weight_copies": head["copies"], "plan": head["plan"],
                   "parallelism": "single GPU"},
        "pct_hbm_peak": head["pct_hbm_peak"],
        "weights_per_s": head["weights_per_s"],
        "macs_per_s": head["macs_per_s"],
        "roofline": roof,
        "cpu_baseline": cpu,
        "by_config": by_config,
        "fused_epilogue": fused,
        "context": context,
        "prefill": prefill,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
