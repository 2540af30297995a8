#!/usr/bin/env python3
"""Benchmark of the fused quantized SwiGLU expansion on one MI355X.

Headline workload (one "step"): the decode configuration -- M=1, H=2048,
I=5632, 4-bit gs64 gate and up -- run as 1000 calls, each with a fresh x and
one of 40 distinct weight sets in rotation (about 520 MB, more than the
256 MB last-level cache, so every call streams its weights from HBM).
``value`` is weight GB/s over the timed steps.  The 1000 calls of a step are
recorded once into a HIP graph and replayed.

Also reported on the same JSON line:
  * ``roofline`` of the decode kernel against 8 TB/s, with ``practical``: a
    read-only stream of the same bytes in the same 1000-launch graph (what one
    launch per call costs before any arithmetic);
  * ``mfma_measured_peak``: the sustained dense f16 MFMA rate of this GPU on
    random and on kernel-like operands (the MFMA pipes are power limited);
  * ``prefill``: configurations 0 and 2-4, each with value, unit and a
    ``roofline`` block (TFLOP/s against the 2.5 PFLOP/s spec and the measured
    rate; HBM traffic from committed counter summaries);
  * ``cpu_baseline``: the CPU oracle on bounded samples of every
    configuration, with all cores (up to 16) and with one, and the CPU model.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|c2|c3|c4|copy]
                    [--no-prefill] [--no-linear] [--no-mlp] [--no-small-batch] [--no-cpu]
                    [--cpu-seconds S] [--eager]

Unless ``--no-linear``: the quantized linear ``y = x W^T`` at the two down
projections (decode model: M=1, K=5632, N=2048 with rotating weights as
above; M=2048 prefill model: K=14336, N=4096), under ``linear``.

``--workload copy`` times a plain device-to-device copy of one decode call's
algorithmic byte count, 1000 copies per step over 40 rotating sources: the
known-size reference against which the HBM traffic counters are scaled.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused quant-SwiGLU TFLOP/s (prefill) + weight GB/s (M=1 decode), % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/f16 MFMA
ROTATING_SETS = 40
CALLS = 1000


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def weight_bytes(c):
    wg = c.I * c.H * c.bits_g // 8 + 2 * 2 * c.I * (c.H // c.gs_g)
    wu = c.I * c.H * c.bits_u // 8 + 2 * 2 * c.I * (c.H // c.gs_u)
    return wg + wu


def algorithmic_bytes(c, out_bytes=2):
    return weight_bytes(c) + c.M * c.H * 2 + c.M * c.I * out_bytes


PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_PROFILE = os.path.join(PROFILES, "decode_gemv_M1_H2048_I5632_hbm_traffic.md")
GEMV_SOURCES = ["swq_gemv.hip", "swq_device.h", "swq_kernels.h"]
PREFILL_SOURCES = ["swq_prefill.hip", "swq_device.h", "swq_kernels.h"]
PREFILL_TRAFFIC = {2: "prefill_mfma_M512_H2048_I8192_hbm_traffic.md",
                   3: "prefill_mfma_M2048_H4096_I14336_hbm_traffic.md",
                   4: "prefill_mfma_M8192_H2560_I10240_hbm_traffic.md"}


def source_digest(files):
    """First 16 hex digits of the SHA-256 of kernel sources with comments,
    blank space and the LDS-poison debug blocks removed (so an edit of
    comments, or of code the product build does not compile, keeps a measured
    traffic figure valid)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "quantized_swiglu_forward_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"#ifdef SWQ_LDS_POISON.*?#endif", " ", src, flags=re.S)
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def gemv_source_digest():
    return source_digest(GEMV_SOURCES)


def profile_traffic(path, files, key):
    """HBM bytes per launch (or per call) from a committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a copy of known size), or
    None when the kernel's sources changed since the counters were taken."""
    try:
        with open(path) as fh:
            for line in fh:
                if line.startswith("traffic-json:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("source") == source_digest(files):
                        return int(rec[key])
    except (OSError, ValueError, KeyError):
        pass
    return None


def measured_traffic():
    return profile_traffic(TRAFFIC_PROFILE, GEMV_SOURCES, "bytes_per_launch")


def rotating_weight_sets(c, base_dev, n_sets, seed):
    """Set 0 is the seeded problem; the others are drawn on the GPU from the
    same distributions (uniform codes, scales U[0.005,0.02] and biases
    -8*s*U[0.9,1.1] in the activation type), seeded."""
    import torch
    dt16 = torch.float16 if c.act == "f16" else torch.bfloat16
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    sets = [base_dev[1:]]
    for _ in range(n_sets - 1):
        one = []
        for bits, gs in ((c.bits_g, c.gs_g), (c.bits_u, c.gs_u)):
            ng = c.H // gs
            words = torch.randint(-2**31, 2**31 - 1, (c.I, c.H * bits // 32), generator=gen, device="cuda",
                                  dtype=torch.int64).to(torch.int32)
            s = (torch.rand((c.I, ng), generator=gen, device="cuda") * (c.s_hi - c.s_lo) + c.s_lo)
            s = s.to(dt16)
            f = torch.rand((c.I, ng), generator=gen, device="cuda") * 0.2 + 0.9
            b = (-8.0 * s.float() * f).to(dt16)
            one += [words, s, b]
        sets.append(tuple(one))
    return sets


def probe_lib():
    """The benchmark's yardstick kernels (libswq_probe.so, built beside the library)."""
    import ctypes
    path = os.path.join(ROOT, "quantized_swiglu_forward_amd", "libswq_probe.so")
    L = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.swq_probe_mfma_f16.argtypes = [i32, i32, i32, vp, vp]
    L.swq_probe_mfma_f16.restype = i32
    L.swq_probe_read.argtypes = [vp, i64, vp, vp]
    L.swq_probe_read.restype = i32
    L.swq_probe_read_blocks.argtypes = [i64]
    L.swq_probe_read_blocks.restype = i64
    L.swq_probe_empty.argtypes = [i32, vp, vp]
    L.swq_probe_empty.restype = i32
    L.swq_probe_grid_barrier.argtypes = [i32, vp, i32, vp, vp]
    L.swq_probe_grid_barrier.restype = i32
    L.swq_probe_atomic_add.argtypes = [i32, i32, vp, vp]
    L.swq_probe_atomic_add.restype = i32
    L.swq_probe_read_slices.argtypes = [vp, i32, i32, i32, i32, vp, vp]
    L.swq_probe_read_slices.restype = i32
    return L


def graph_call_us(launch, steps, warmup):
    """Microseconds per call of ``launch(i, stream_handle)`` (which enqueues
    one call's kernels and returns 0), CALLS calls per step recorded into
    one HIP graph, timed with HIP events over ``steps`` replays."""
    import torch
    stream = torch.cuda.Stream()

    def step(sh):
        for i in range(CALLS):
            if launch(i, sh) != 0:
                raise RuntimeError("probe launch failed")

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step(stream.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step(torch.cuda.current_stream().cuda_stream)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps):
            g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (steps * CALLS)


def bench_mlp_boundary(steps, warmup):
    """What a whole MLP in one dispatch would pay at decode (M=1, H=Ho=2048,
    I=5632, 4-bit down projection), measured with probe kernels in the decode
    bench's graph setup: the second launch it would save (two dependent
    trivial kernels against one), a grid-wide barrier between its phases
    (352 blocks, as many as the gate/up phase's 16-column tiles), f32
    atomic accumulation of every I-block's partial output (the pages'
    design: 352 blocks, or 22 blocks of 256 inputs, times Ho atomics), and
    the down projection's rows read in the 8-byte I-slices that 16-column
    tiles own, against the same bytes read contiguously."""
    import torch
    L = probe_lib()
    Ho, I = 2048, 5632
    row_bytes = I * 4 // 8
    b16, b256 = I // 16, I // 256
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda")
    counter = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.zeros(Ho, dtype=torch.float32, device="cuda")
    sp, cp, yp = sink.data_ptr(), counter.data_ptr(), y.data_ptr()
    one = graph_call_us(lambda i, sh: L.swq_probe_empty(1, sp, sh), steps, warmup)
    two = graph_call_us(lambda i, sh: L.swq_probe_empty(1, sp, sh) or L.swq_probe_empty(1, sp, sh), steps, warmup)
    empty16 = graph_call_us(lambda i, sh: L.swq_probe_empty(b16, sp, sh), steps, warmup)
    barrier16 = graph_call_us(lambda i, sh: L.swq_probe_grid_barrier(b16, cp, 4096, sp, sh), steps, warmup)
    torch.cuda.synchronize()
    timed_out = int((sink[:b16] != 0).sum().item())
    atomics16 = graph_call_us(lambda i, sh: L.swq_probe_atomic_add(b16, Ho, yp, sh), steps, warmup)
    atomics256 = graph_call_us(lambda i, sh: L.swq_probe_atomic_add(b256, Ho, yp, sh), steps, warmup)
    bufs = [torch.empty(Ho * row_bytes // 4, dtype=torch.int32, device="cuda").fill_(i + 1)
            for i in range(ROTATING_SETS)]
    ptrs = [t.data_ptr() for t in bufs]
    slices8 = graph_call_us(lambda i, sh: L.swq_probe_read_slices(ptrs[i % ROTATING_SETS], Ho, row_bytes, 8, b16,
                                                                  sp, sh), steps, warmup)
    del bufs
    whole = practical_read(Ho * row_bytes, steps, warmup)
    return {"config": f"decode MLP parts: Ho={Ho}, I={I}, 4-bit down projection, {b16} blocks of 16 columns, "
                      f"{CALLS} calls per graph",
            "second_launch_us": round(two - one, 3),
            "grid_barrier_us": round(barrier16 - empty16, 3), "grid_barrier_timeouts": timed_out,
            "atomics_16col_blocks_us": round(atomics16, 3), "atomics_256input_blocks_us": round(atomics256, 3),
            "down_read_8B_slices_us": round(slices8, 3), "down_read_contiguous_us": round(whole, 3)}


def practical_read(nbytes, steps, warmup):
    """The decode call's practical ceiling: a read-only stream of exactly
    ``nbytes`` per launch (16-byte nontemporal loads, one store per block),
    1000 launches per step over 40 rotating buffers in one HIP graph, as the
    decode calls run.  Returns the average launch time in microseconds."""
    import torch
    L = probe_lib()
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(i + 1) for i in range(ROTATING_SETS)]
    sink = torch.empty(int(L.swq_probe_read_blocks(nbytes)), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    def step(sh):
        for i in range(CALLS):
            if L.swq_probe_read(bufs[i % ROTATING_SETS].data_ptr(), nbytes, sink.data_ptr(), sh) != 0:
                raise RuntimeError("read probe launch failed")

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step(stream.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step(torch.cuda.current_stream().cuda_stream)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps):
            g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (steps * CALLS)
    del g, bufs
    return us


def mfma_peak(pattern, iters=3000, reps=5):
    """Sustained dense f16 MFMA rate (TFLOP/s) of back-to-back 32x32x16
    MFMAs, four waves per block and four blocks per compute unit, timed with
    HIP events over ``reps`` launches after one warm-up launch."""
    import torch
    L = probe_lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 4 * cus
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        if L.swq_probe_mfma_f16(blocks, iters, pattern, sink.data_ptr(), stream.cuda_stream) != 0:
            raise RuntimeError("MFMA probe launch failed")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            L.swq_probe_mfma_f16(blocks, iters, pattern, sink.data_ptr(), stream.cuda_stream)
        e1.record(stream)
    torch.cuda.synchronize()
    flops = reps * blocks * 4 * iters * 4 * 32768.0
    return flops / (e0.elapsed_time(e1) * 1e-3) / 1e12


def bench_decode(args):
    import torch

    import quantized_swiglu_forward_amd as swq
    from synth import CONFIGS, make_problem

    c = CONFIGS[1]
    p = make_problem(1)
    dev = swq.to_device(p)
    sets = rotating_weight_sets(c, dev, ROTATING_SETS, seed=101)
    import numpy as np
    xs = torch.from_numpy(np.ascontiguousarray(p.xs).view(np.int16)).cuda().view(torch.bfloat16)  # [1000, H]
    out = torch.empty((CALLS, c.I), dtype=torch.bfloat16, device="cuda")
    L = swq.lib()
    H, I = c.H, c.I
    xrow = H * 2
    orow = I * 2
    ptr_sets = [tuple(t.data_ptr() for t in s) for s in sets]
    x0, o0 = xs.data_ptr(), out.data_ptr()
    assert swq.swiglu_q_get_m_threshold() > 1, "decode must take the matrix-vector path"

    def step(stream_handle, n_sets=ROTATING_SETS):
        for i in range(CALLS):
            wg, sg, bg, wu, su, bu = ptr_sets[i % n_sets]
            rc = L.swiglu_q_forward(x0 + i * xrow, wg, sg, bg, wu, su, bu, 1, H, I, c.bits_g, c.gs_g,
                                    c.bits_u, c.gs_u, 0, o0 + i * orow, stream_handle)
            if rc != 0:
                raise RuntimeError(f"swiglu_q_forward failed: {swq.swiglu_q_strerror(rc)}")

    stream = torch.cuda.Stream()
    graph = None
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step(stream.cuda_stream)               # eager warm-up (also first-use setup)
    torch.cuda.synchronize()
    if not args.eager:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                step(torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
        except Exception as e:                 # noqa: BLE001
            log(f"graph capture failed ({e}); timing eager launches")
            graph = None

    def run_one():
        if graph is not None:
            graph.replay()
        else:
            with torch.cuda.stream(stream):
                step(stream.cuda_stream)

    before = swq.swiglu_q_call_count(swq.SWQ_PATH_GEMV)
    for _ in range(args.warmup):
        run_one()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            run_one()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1)
    ms_step = ms / args.steps
    launches = args.steps * CALLS
    if graph is None:
        assert swq.swiglu_q_call_count(swq.SWQ_PATH_GEMV) - before == (args.warmup + args.steps) * CALLS
    # the same calls on one weight set (13 MB, resident in the last-level
    # cache after the first call): reported separately, never as `value`
    hot = None
    if graph is not None:
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2, stream=stream):
            step(torch.cuda.current_stream().cuda_stream, n_sets=1)
        for _ in range(2):
            g2.replay()
        torch.cuda.synchronize()
        h0 = torch.cuda.Event(enable_timing=True)
        h1 = torch.cuda.Event(enable_timing=True)
        h0.record(stream)
        with torch.cuda.stream(stream):
            for _ in range(5):
                g2.replay()
        h1.record(stream)
        torch.cuda.synchronize()
        hot_us = h0.elapsed_time(h1) * 1e3 / (5 * CALLS)
        hot = {"avg_launch_us": round(hot_us, 3),
               "GB_per_s": round(algorithmic_bytes(c) / (hot_us * 1e-6) / 1e9, 1),
               "note": "one weight set reused by all calls (cache resident); not the headline"}
        del g2
    wb = weight_bytes(c)
    value = wb * CALLS / (ms_step * 1e-3) / 1e9
    avg_launch_us = ms * 1e3 / launches
    achieved = algorithmic_bytes(c) / (avg_launch_us * 1e-6) / 1e9
    prac_us = practical_read(algorithmic_bytes(c), args.steps, max(1, args.warmup)) if graph is not None else None
    res = {
        "value": round(value, 2), "unit": "GB/s", "ms_per_step": round(ms_step, 4),
        "dtype": "f16",
        "config": {"workload": "decode GEMV M=1 H=2048 I=5632, 4-bit gs64 gate and up, "
                               "1000 calls per step with fresh x, 40 rotating weight sets",
                   "M": 1, "H": H, "I": I, "bits_g": c.bits_g, "gs_g": c.gs_g, "bits_u": c.bits_u,
                   "gs_u": c.gs_u, "calls_per_step": CALLS, "weight_sets": ROTATING_SETS,
                   "precision_mode": "MATCH", "launch": "hip graph" if graph is not None else "eager"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "avg_launch_us": round(avg_launch_us, 3),
                     "bytes_per_launch": algorithmic_bytes(c)},
        "wall_s": round(wall, 3),
    }
    if prac_us is not None:
        # a read-only kernel that streams the same bytes in the same graph of
        # 1000 launches over 40 rotating buffers: what one launch per call
        # costs on this GPU before any arithmetic
        res["roofline"]["practical"] = {
            "kernel": "read-only 16-byte stream of the same bytes per launch, same 1000-launch graph, 40 buffers",
            "avg_launch_us": round(prac_us, 3),
            "GB_per_s": round(algorithmic_bytes(c) / (prac_us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(algorithmic_bytes(c) / (prac_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "frac": round(prac_us / avg_launch_us, 4)}
    if hot is not None:
        res["decode_hot_cache"] = hot
    return res


_PROBLEMS = {}


def problem(cfg):
    """The seeded host problem of a configuration (an index or a Config),
    drawn once per run."""
    from synth import make_problem
    if not isinstance(cfg, int):
        return make_problem(cfg, with_calls=False)
    if cfg not in _PROBLEMS:
        _PROBLEMS[cfg] = make_problem(cfg, with_calls=(cfg == 1))
    return _PROBLEMS[cfg]


def bench_prefill_one(cfg, steps, warmup, mode=0, measured_peak=None):
    """One prefill configuration: ``steps`` calls on one stream after
    ``warmup``, timed with HIP events on that stream.  A call is two launches
    (the prep kernel, then the MFMA kernel; three when the columns are split
    in two launches), so the rate is a lower bound on the MFMA kernel's own.
    Config 0 (latency bound) is timed as 200 calls in one HIP graph."""
    import torch

    import quantized_swiglu_forward_amd as swq
    from synth import CONFIGS

    c = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    dev = swq.to_device(problem(cfg))
    out16 = torch.float16 if c.act == "f16" else torch.bfloat16
    out = torch.empty((c.M, c.I), dtype=torch.float32 if mode == 1 else out16, device="cuda")
    stream = torch.cuda.Stream()
    pm = ["MATCH", "F32", "F32_BF16OUT"][mode]
    config = {"workload": c.describe, "M": c.M, "H": c.H, "I": c.I, "bits_g": c.bits_g, "gs_g": c.gs_g,
              "bits_u": c.bits_u, "gs_u": c.gs_u, "precision_mode": pm, "activations": c.act}
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            swq.forward(*dev, c.bits_g, c.gs_g, c.bits_u, c.gs_u, mode=mode, out=out, stream=stream)
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(steps):
            swq.forward(*dev, c.bits_g, c.gs_g, c.bits_u, c.gs_u, mode=mode, out=out, stream=stream)
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    if cfg == 0:
        # latency-bound (no roofline target): the calls recorded into one HIP
        # graph, so the host's launch rate does not set the figure
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(steps):
                swq.forward(*dev, c.bits_g, c.gs_g, c.bits_u, c.gs_u, mode=mode, out=out,
                            stream=torch.cuda.current_stream())
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        with torch.cuda.stream(stream):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        return {"metric": "fused quant-SwiGLU call latency (tiny prefill)", "value": round(us, 2),
                "unit": "us per call", "higher_is_better": False, "dtype": "f16", "config": config,
                "launch": "hip graph of 200 calls",
                "roofline": {"bound": "latency", "note": "233,472 bytes and 4.72 MFLOP per call: no roofline"}}
    flops = 4.0 * c.M * c.H * c.I
    tflops = flops / (ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": profile_traffic(os.path.join(PROFILES, PREFILL_TRAFFIC[cfg]), PREFILL_SOURCES,
                                       "bytes_per_call") if mode == 0 and cfg in PREFILL_TRAFFIC else None,
            "flops_per_call": flops, "algorithmic_bytes_per_call": algorithmic_bytes(c, 4 if mode == 1 else 2)}
    if measured_peak:
        roof["measured_peak"] = round(measured_peak, 1)
        roof["frac_of_measured_peak"] = round(tflops / measured_peak, 4)
    return {"metric": "fused quant-SwiGLU TFLOP/s (prefill)", "value": round(tflops, 2), "unit": "TFLOP/s",
            "ms_per_call": round(ms, 4), "higher_is_better": True, "dtype": "f16", "config": config,
            "roofline": roof}


def bench_decode_spec(c, steps, warmup):
    """The decode call (1000 calls per step on fresh x rows over 40 rotating
    weight sets, one HIP graph) for another quantization spec of the decode
    shape: per-call time and weight bytes per second."""
    import numpy as np
    import torch

    import quantized_swiglu_forward_amd as swq

    p = problem(c)
    dev = swq.to_device(p)
    sets = rotating_weight_sets(c, dev, ROTATING_SETS, seed=103)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    dt16 = torch.float16 if c.act == "f16" else torch.bfloat16
    x = torch.randn((CALLS, c.H), generator=gen, device="cuda").to(dt16)
    out = torch.empty((CALLS, c.I), dtype=dt16, device="cuda")
    L = swq.lib()
    entry = L.swiglu_q_forward_f16 if c.act == "f16" else L.swiglu_q_forward
    ptrs = [tuple(t.data_ptr() for t in st) for st in sets]

    def step(sh):
        for i in range(CALLS):
            wg, sg, bg, wu, su, bu = ptrs[i % ROTATING_SETS]
            rc = entry(x.data_ptr() + i * c.H * 2, wg, sg, bg, wu, su, bu, 1, c.H, c.I, c.bits_g,
                       c.gs_g, c.bits_u, c.gs_u, 0, out.data_ptr() + i * c.I * 2, sh)
            if rc != 0:
                raise RuntimeError(f"swiglu_q_forward failed: {swq.swiglu_q_strerror(rc)}")

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step(stream.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step(torch.cuda.current_stream().cuda_stream)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps):
            g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (steps * CALLS)
    alg = algorithmic_bytes(c)
    return {"config": c.describe, "activations": c.act, "avg_launch_us": round(us, 3),
            "weight_GB_per_s": round(weight_bytes(c) / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_launch": alg}


def bench_decode_rows(M, steps, warmup):
    """The decode shape (H=2048, I=5632, 4-bit gs64) at a few rows per call:
    1000 calls per step on fresh x rows over the 40 rotating weight sets,
    recorded into a HIP graph; per-call time and weight bytes per second.
    Each call takes the dispatcher's path (the matrix-matrix one, with its K
    split, at 128 rows)."""
    import torch

    import quantized_swiglu_forward_amd as swq
    from synth import CONFIGS, make_problem

    c = CONFIGS[1]
    dev = swq.to_device(make_problem(1))
    sets = rotating_weight_sets(c, dev, ROTATING_SETS, seed=101)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(M)
    x = torch.randn((CALLS * M, c.H), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((CALLS * M, c.I), dtype=torch.bfloat16, device="cuda")
    L = swq.lib()
    ptrs = [tuple(t.data_ptr() for t in s) for s in sets]
    x0, o0 = x.data_ptr(), out.data_ptr()
    path = swq.swiglu_q_path_for(M, c.H, c.I)
    before = swq.swiglu_q_call_count(path)

    def step(sh):
        for i in range(CALLS):
            wg, sg, bg, wu, su, bu = ptrs[i % ROTATING_SETS]
            rc = L.swiglu_q_forward(x0 + i * M * c.H * 2, wg, sg, bg, wu, su, bu, M, c.H, c.I, c.bits_g, c.gs_g,
                                    c.bits_u, c.gs_u, 0, o0 + i * M * c.I * 2, sh)
            if rc != 0:
                raise RuntimeError(f"swiglu_q_forward failed: {swq.swiglu_q_strerror(rc)}")

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step(stream.cuda_stream)
    torch.cuda.synchronize()
    assert swq.swiglu_q_call_count(path) - before == CALLS, "not the dispatcher's path"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step(torch.cuda.current_stream().cuda_stream)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps):
            g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (steps * CALLS)
    wb = weight_bytes(c)
    alg = wb + M * (c.H + c.I) * 2
    return {"config": f"decode shape M={M} H={c.H} I={c.I}, 4-bit gs64 gate and up, fresh x per call, "
                      f"{ROTATING_SETS} rotating weight sets, hip graph",
            "path": "matrix-vector" if path == swq.SWQ_PATH_GEMV else
                    "matrix-matrix (prep, MFMA GEMM with its K split, split epilogue: three launches per call)",
            "avg_launch_us": round(us, 3), "weight_GB_per_s": round(wb / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_launch": alg}


def bench_mlp_decode(steps, warmup):
    """The whole MLP at the decode model's shape (M=1, H=2048, I=5632, Ho=2048,
    4-bit gs64 gate, up and down, bf16 residual): 1000 calls per step on fresh
    x rows, 40 rotating sets of all three matrices, recorded into a HIP graph."""
    import torch

    import quantized_swiglu_forward_amd as swq
    from synth import CONFIGS, make_problem

    c = CONFIGS[1]
    dev = swq.to_device(make_problem(1))
    sets = rotating_weight_sets(c, dev, ROTATING_SETS, seed=101)
    Ho, I, H = c.H, c.I, c.H
    gen = torch.Generator(device="cuda")
    gen.manual_seed(17)
    dsets = []
    for _ in range(ROTATING_SETS):
        words = torch.randint(-2**31, 2**31 - 1, (Ho, I * 4 // 32), generator=gen, device="cuda",
                              dtype=torch.int64).to(torch.int32)
        sc = (torch.rand((Ho, I // 64), generator=gen, device="cuda") * 0.015 + 0.005).to(torch.bfloat16)
        bi = (-8.0 * sc.float() * (torch.rand((Ho, I // 64), generator=gen, device="cuda") * 0.2 + 0.9))
        dsets.append((words, sc, bi.to(torch.bfloat16)))
    x = torch.randn((CALLS, H), generator=gen, device="cuda").to(torch.bfloat16)
    res = torch.randn((CALLS, Ho), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((CALLS, Ho), dtype=torch.bfloat16, device="cuda")
    L = swq.lib()
    ptrs = [tuple(t.data_ptr() for t in s) + tuple(t.data_ptr() for t in d) for s, d in zip(sets, dsets)]

    def step(sh):
        for i in range(CALLS):
            wg, sg, bg, wu, su, bu, wd, sd, bd = ptrs[i % ROTATING_SETS]
            rc = L.swiglu_q_mlp(x.data_ptr() + i * H * 2, wg, sg, bg, wu, su, bu, wd, sd, bd,
                                res.data_ptr() + i * Ho * 2, 1, H, I, Ho, 4, 64, 4, 64, 4, 64,
                                swq.SWQ_LINEAR_BF16, out.data_ptr() + i * Ho * 2, sh)
            if rc != 0:
                raise RuntimeError(f"swiglu_q_mlp failed: {swq.swiglu_q_strerror(rc)}")

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step(stream.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step(torch.cuda.current_stream().cuda_stream)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps):
            g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (steps * CALLS)
    wb = weight_bytes(c) + Ho * I * 4 // 8 + 2 * 2 * Ho * (I // 64)
    return {"config": f"whole MLP M=1 H={H} I={I} Ho={Ho}, 4-bit gs64 gate, up and down, bf16 residual, "
                      f"fresh x per call, {ROTATING_SETS} rotating weight sets, hip graph (two launches per call)",
            "avg_call_us": round(us, 3), "weight_GB_per_s": round(wb / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(wb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "weight_bytes": wb}


def bench_mlp_prefill(steps, warmup):
    """The whole MLP of the M=2048 prefill model (H=4096, I=14336, Ho=4096,
    4-bit gs64 everywhere, bf16 residual), one problem, ``steps`` calls."""
    import torch

    import quantized_swiglu_forward_amd as swq
    from synth import make_custom, make_down, make_residual

    M, H, I, Ho = 2048, 4096, 14336, 4096
    p = make_custom(M, H, I, 4, 64, seed=3, x_sigma=0.5, s_lo=0.002, s_hi=0.01)
    wd, sd, bd = make_down(Ho, I, 4, 64, seed=4)
    dev = swq.to_device(p)

    def t16(a):
        return torch.from_numpy(a.view("int16")).cuda().view(torch.bfloat16)

    down = (torch.from_numpy(wd.view("int32")).cuda(), t16(sd), t16(bd))
    res = t16(make_residual(M, Ho, seed=5))
    out = torch.empty((M, Ho), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            swq.mlp(*dev, *down, (4, 64), (4, 64), (4, 64), residual=res, out=out, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            swq.mlp(*dev, *down, (4, 64), (4, 64), (4, 64), residual=res, out=out, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 4.0 * M * H * I + 2.0 * M * I * Ho
    tflops = flops / (ms * 1e-3) / 1e12
    return {"config": f"whole MLP M={M} H={H} I={I} Ho={Ho}, 4-bit gs64 gate, up and down, bf16 residual",
            "ms_per_call": round(ms, 4), "tflops": round(tflops, 2),
            "frac_of_mfma_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)}


def bench_linear(M, K, N, bits, gs, steps, warmup, rotating):
    """The quantized linear at one shape, bf16 output.  ``rotating``: 1000
    calls per step on fresh x rows over 40 weight sets (drawn on the GPU from
    the generator's distributions), recorded into a HIP graph; otherwise
    ``steps`` calls on one problem."""
    import numpy as np
    import torch

    import quantized_swiglu_forward_amd as swq
    from synth import make_custom

    rows = CALLS if rotating else M
    p = make_custom(rows, K, N, bits, gs, bits, gs, seed=K + N, bias_mode="factor")
    dev = swq.to_device(p)
    x, w, s, b = dev[:4]
    wb = N * K * bits // 8 + 2 * 2 * N * (K // gs)
    stream = torch.cuda.Stream()
    if not rotating:
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                swq.linear(x, w, s, b, bits, gs, out=out, stream=stream)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                swq.linear(x, w, s, b, bits, gs, out=out, stream=stream)
            e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tflops = 2.0 * M * K * N / (ms * 1e-3) / 1e12
        return {"config": f"quantized linear M={M} K={K} N={N}, {bits}-bit gs{gs}, bf16 out",
                "ms_per_call": round(ms, 4), "tflops": round(tflops, 2),
                "frac_of_mfma_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    sets = [(w, s, b)]
    for _ in range(ROTATING_SETS - 1):
        words = torch.randint(-2**31, 2**31 - 1, (N, K * bits // 32), generator=gen, device="cuda",
                              dtype=torch.int64).to(torch.int32)
        sc = (torch.rand((N, K // gs), generator=gen, device="cuda") * 0.015 + 0.005).to(torch.bfloat16)
        bi = (-8.0 * sc.float() * (torch.rand((N, K // gs), generator=gen, device="cuda") * 0.2 + 0.9))
        sets.append((words, sc, bi.to(torch.bfloat16)))
    out = torch.empty((CALLS, N), dtype=torch.bfloat16, device="cuda")
    L = swq.lib()
    ptrs = [tuple(t.data_ptr() for t in st) for st in sets]
    x0, o0 = x.data_ptr(), out.data_ptr()

    def step(sh):
        for i in range(CALLS):
            wp, sp, bp = ptrs[i % ROTATING_SETS]
            rc = L.swiglu_q_linear(x0 + i * K * 2, wp, sp, bp, 1, K, N, bits, gs, swq.SWQ_LINEAR_BF16,
                                   o0 + i * N * 2, sh)
            if rc != 0:
                raise RuntimeError(f"swiglu_q_linear failed: {swq.swiglu_q_strerror(rc)}")

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        step(stream.cuda_stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        step(torch.cuda.current_stream().cuda_stream)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(steps):
            g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (steps * CALLS)
    alg = wb + K * 2 + N * 2
    return {"config": f"quantized linear M=1 K={K} N={N}, {bits}-bit gs{gs}, bf16 out, fresh x per call, "
                      f"{ROTATING_SETS} rotating weight sets, hip graph",
            "avg_launch_us": round(us, 3), "weight_GB_per_s": round(wb / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_launch": alg}


def bench_copy(args):
    """Plain copy kernel of a known size: 1000 copies of 12,991,488 bytes per
    step, sources rotating over 40 buffers, recorded into one HIP graph."""
    import torch

    nbytes = 12991488
    srcs = [torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(i) for i in range(ROTATING_SETS)]
    dst = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(3):
            dst.copy_(srcs[i])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(CALLS):
            dst.copy_(srcs[i % ROTATING_SETS])
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    us = ms_step * 1e3 / CALLS
    return {"value": round(2 * nbytes / (us * 1e-6) / 1e9, 2), "unit": "GB/s (read+write)",
            "ms_per_step": round(ms_step, 4), "dtype": "u8",
            "config": {"workload": f"device copy of {nbytes} bytes, 1000 per step, 40 rotating sources",
                       "bytes_read": nbytes, "bytes_written": nbytes, "avg_launch_us": round(us, 3)}}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(threads, seconds):
    """The oracle as it stands (plain C, float64, one output element at a
    time, threaded over elements) on the host, ``threads`` threads, for about
    ``seconds`` per configuration: the decode workload as whole calls on its
    fresh x rows (weight GB/s), config 0 as whole calls (us per call), and
    configs 2-4 on random output elements in batches (TFLOP/s counted as
    4 H flops per element, the call's 4 M H I over its M I elements)."""
    import numpy as np

    import oracle
    from synth import CONFIGS

    res = {}
    # decode: whole calls on the fresh x rows
    c = CONFIGS[1]
    p = problem(1)
    calls, t0 = 0, time.perf_counter()
    x0 = p.x
    while True:
        p.x = p.xs[calls:calls + 1]
        oracle.swiglu_pairs(p, 0, nthreads=threads, want=("h",))
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds or calls >= len(p.xs):
            break
    p.x = x0
    res["c1"] = {"value": round(weight_bytes(c) * calls / el / 1e9, 4), "unit": "GB/s",
                 "sample": f"{calls} whole decode calls (all {c.I} outputs, MATCH) in {el:.2f} s"}
    # config 0: whole calls
    p = problem(0)
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.swiglu_pairs(p, 0, nthreads=threads, want=("h",))
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds / 4:
            break
    res["c0"] = {"value": round(el / calls * 1e6, 1), "unit": "us per call",
                 "sample": f"{calls} whole calls ({p.M * p.I} outputs, MATCH) in {el:.2f} s"}
    for cfg in (2, 3, 4):
        c = CONFIGS[cfg]
        p = problem(cfg)
        rng = np.random.default_rng(cfg)
        batch = 32 * threads
        n, t0 = 0, time.perf_counter()
        while True:
            ms = rng.integers(0, c.M, batch)
            ns = rng.integers(0, c.I, batch)
            oracle.swiglu_pairs(p, 0, ms, ns, nthreads=threads, want=("h",))
            n += batch
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        res[f"c{cfg}"] = {"value": round(4.0 * c.H * n / el / 1e12, 8), "unit": "TFLOP/s",
                          "sample": f"{n} random outputs of the {c.M} x {c.I} call (MATCH) in {el:.2f} s"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode", choices=["decode", "c2", "c3", "c4", "copy"])
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-linear", action="store_true")
    ap.add_argument("--no-small-batch", action="store_true", help="skip the decode shape at 2 to 64 rows")
    ap.add_argument("--no-mlp", action="store_true", help="skip the whole-MLP measurements")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--eager", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=2.5,
                    help="CPU-baseline time per configuration and thread count")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "the fused SwiGLU library runs on one GPU (a multi-GPU layout would shard the I dimension).", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import quantized_swiglu_forward_amd as swq
    swq.lib()

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "data": "synthetic"}
    if args.workload == "decode":
        log("decode: timing ...")
        line.update(bench_decode(args))
    elif args.workload == "copy":
        line.update(bench_copy(args))
        line["metric"] = "plain copy (traffic-counter reference)"
        print(json.dumps(line), flush=True)
        return
    else:
        cfg = int(args.workload[1])
        r = bench_prefill_one(cfg, args.steps, args.warmup)
        line.update({"metric": r["metric"], "value": r["value"], "unit": r["unit"], "ms_per_step": r["ms_per_call"],
                     "dtype": r["dtype"], "config": r["config"], "roofline": r["roofline"]})
    if args.workload == "decode" and not args.no_small_batch:
        log("decode, a few rows per call: timing ...")
        line["decode_small_batch"] = {f"M{m}": bench_decode_rows(m, max(1, args.steps // 4), 2) for m in (2, 4, 8, 16, 32, 64, 128)}
        torch.cuda.empty_cache()
    if not args.no_prefill:
        log("MFMA probe: sustained f16 rate ...")
        peaks = {"random_operands": round(mfma_peak(0), 1), "kernel_like_operands": round(mfma_peak(1), 1)}
        line["mfma_measured_peak"] = {
            "unit": "TFLOP/s", **peaks, "spec": MFMA_F16_PEAK_TFLOPS,
            "kernel": "back-to-back v_mfma_f32_32x32x16_f16, 4 waves per block, 4 blocks per CU",
            "used_as_measured_peak": "kernel_like_operands"}
        pre = {}
        for cfg, mode in ((0, 0), (2, 0), (2, 1), (3, 0), (4, 0)):
            log(f"prefill c{cfg} mode {mode}: timing ...")
            steps = 200 if cfg == 0 else 10
            pre[f"c{cfg}_{['match', 'f32'][mode]}"] = bench_prefill_one(
                cfg, steps=steps, warmup=3, mode=mode, measured_peak=peaks["kernel_like_operands"])
            torch.cuda.empty_cache()
        line["prefill"] = pre
        # the other group size and the third precision mode
        from dataclasses import replace
        from synth import CONFIGS
        log("spec variants: timing ...")
        c3g = replace(CONFIGS[3], name="large_prefill_gs128", gs_g=128, gs_u=128,
                      describe="large prefill M=2048 H=4096 I=14336, 4-bit gs128 gate/up")
        c1g = replace(CONFIGS[1], name="decode_gs128", gs_g=128, gs_u=128, calls=0,
                      describe="decode GEMV M=1 H=2048 I=5632, 4-bit gs128 gate/up, fresh x per call, "
                               "40 rotating weight sets, hip graph")
        # binary16 activations (x, scales and biases float16)
        c3h = replace(CONFIGS[3], name="large_prefill_f16", act="f16",
                      describe="large prefill M=2048 H=4096 I=14336, 4-bit gs64 gate/up, float16 activations")
        c1h = replace(CONFIGS[1], name="decode_f16", act="f16", calls=0,
                      describe="decode GEMV M=1 H=2048 I=5632, 4-bit gs64 gate/up, float16 activations, fresh x "
                               "per call, 40 rotating weight sets, hip graph")
        line["spec_variants"] = {
            "c3_gs128_match": bench_prefill_one(c3g, steps=10, warmup=3, mode=0,
                                                measured_peak=peaks["kernel_like_operands"]),
            "c2_f32_bf16out": bench_prefill_one(2, steps=10, warmup=3, mode=2,
                                                measured_peak=peaks["kernel_like_operands"]),
            "c1_gs128": bench_decode_spec(c1g, max(1, args.steps // 4), 2),
            "c3_f16_match": bench_prefill_one(c3h, steps=10, warmup=3, mode=0,
                                              measured_peak=peaks["kernel_like_operands"]),
            "c1_f16": bench_decode_spec(c1h, max(1, args.steps // 4), 2)}
        torch.cuda.empty_cache()
    if not args.no_linear:
        log("linear: timing ...")
        line["linear"] = {"decode_down_proj": bench_linear(1, 5632, 2048, 4, 64, max(1, args.steps // 4), 2, True),
                          "prefill_down_proj": bench_linear(2048, 14336, 4096, 4, 64, 10, 3, False)}
        torch.cuda.empty_cache()
    if not args.no_mlp:
        log("whole MLP: timing ...")
        line["mlp"] = {"decode": bench_mlp_decode(max(1, args.steps // 4), 2),
                       "prefill": bench_mlp_prefill(10, 3),
                       "one_dispatch_parts": bench_mlp_boundary(max(1, args.steps // 4), 2)}
        torch.cuda.empty_cache()
    if not args.no_cpu:
        log("cpu baseline: the oracle on bounded samples of every configuration ...")
        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count() or 1
        cores = max(1, min(16, cores))
        many = cpu_baseline(cores, args.cpu_seconds)
        one = cpu_baseline(1, args.cpu_seconds)
        line["cpu_baseline"] = {
            "value": many["c1"]["value"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": many["c1"]["sample"], "cpu_model": cpu_model(),
            "configs": {k: {"all_cores": many[k], "one_core": one[k]} for k in sorted(many)},
            "one_core_value": one["c1"]["value"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
