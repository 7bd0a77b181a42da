#!/usr/bin/env python3
"""Benchmark of the Sparse-BitNet BitLinear forward on one MI355X (gfx950).

A step is one pass of the hot path over one batch of synthetic input: per-token INT8 quantization
of the activations, then the n:m-sparse ternary x INT8 matmul with fused dequantization (and, for
the dynamic-sparsity training workload, the absmean + n:m re-pack of the latent weights). Steps
are captured into one HIP graph and replayed, so host launch overhead is not measured; inputs are
resident in HBM before the timed region starts.

Default workload: decode GEMV, 6:8, K=2560 -> N=6912, one token, weights packed once; the packed
weights rotate over enough distinct copies (>= 1 GiB) that every step streams them from HBM.
Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0   # MI355X dense INT8 MFMA
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
LN_EPS = 1e-5             # LayerNorm epsilon of the timed LayerNorm variants
REPEATS = 5               # timed replays per measurement; the median is reported
KERNEL_LAUNCHES = 200     # launches per graph when a kernel is timed on its own (>= 100)
SLEEP_CYCLES = 2_000_000  # GPU busy wait before each timed replay (covers host enqueue latency)
METRIC = "N:M ternary BitLinear dense-equiv TOPS (prefill) + HBM GB/s (decode GEMV)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# The sources of the kernels whose HBM traffic is recorded (the decode GEMVs and the prefill GEMM)
KERNEL_SOURCES = ["sparsity_sbn_quantize_amd/csrc/bitlinear.hip",
                  "sparsity_sbn_quantize_amd/csrc/sbn_common.hpp",
                  "sparsity_sbn_quantize_amd/csrc/gemv.hpp",
                  "sparsity_sbn_quantize_amd/csrc/gemv_i8.hip",
                  "sparsity_sbn_quantize_amd/csrc/gemv_bf16.hip"]


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comment-only lines, trailing // comments and blank lines
    are left out, so editing a comment does not invalidate measured traffic."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            for line in f:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None when missing or
    taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------------------------------------------
# Algorithmic work per launch (what the method must move or compute).
# ------------------------------------------------------------------------------------------------

def rpf_bytes(n_out, K, n, m):
    code_row = ((K // m) * 2 * n + 7) // 8
    mask_row = (K + 7) // 8 if n < m else 0
    return n_out * (code_row + mask_row)


def quantize_bytes(T, K):
    return 2 * T * K + T * K + 4 * T


def forward_bytes(T, K, n_out, n, m):
    return rpf_bytes(n_out, K, n, m) + T * K + 4 * T + 4 + 4 * T * n_out


def pack_bytes(n_out, K, n, m):
    return 4 * n_out * K + rpf_bytes(n_out, K, n, m) + 4


# ------------------------------------------------------------------------------------------------
# GPU helpers.
# ------------------------------------------------------------------------------------------------

class Gpu:
    def __init__(self):
        import torch
        from sparsity_sbn_quantize_amd import binding
        self.torch = torch
        self.b = binding
        binding.lib()  # fails loudly when the HIP library is missing
        torch.cuda.set_device(0)

    def bf16(self, bits):
        import numpy as np
        return self.torch.from_numpy(bits.view(np.int16)).cuda().view(self.torch.bfloat16)

    def f32(self, a):
        return self.torch.from_numpy(a).cuda()

    def graph(self, fn, count):
        """Captures fn(i) for i in range(count) into one HIP graph."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(i)
        torch.cuda.synchronize()
        return g

    def time_graph(self, g, reps=REPEATS):
        """Milliseconds of one replay, between HIP events on the replaying stream: the median of
        `reps` replays. Before each, a GPU-side busy wait keeps the stream occupied while the host
        enqueues the events and the replay, so that host launch latency is not timed."""
        torch = self.torch
        times = []
        for _ in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            torch.cuda._sleep(SLEEP_CYCLES)
            s.record()
            g.replay()
            e.record()
            e.synchronize()
            times.append(s.elapsed_time(e))
        return statistics.median(times)

    def sleep_seconds_per_cycle(self):
        """Seconds per cycle of the GPU busy wait (torch.cuda._sleep), measured once."""
        if getattr(self, "_spc", None) is None:
            torch = self.torch
            n = 4_000_000
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            s.record()
            torch.cuda._sleep(n)
            e.record()
            e.synchronize()
            self._spc = s.elapsed_time(e) * 1e-3 / n
        return self._spc

    def time_eager(self, run, reps=REPEATS):
        """Milliseconds of run(r) (a fixed number of launches, eagerly enqueued) between HIP events,
        the median over r = 0 .. reps-1. A GPU busy wait ahead of each timed region, longer than
        three times the host's measured enqueue time of one run, keeps the host ahead of the GPU,
        so the region times the kernels back to back, not the host."""
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(0)
        host = time.perf_counter() - t0
        torch.cuda.synchronize()
        cycles = int(max(SLEEP_CYCLES, 3.0 * host / self.sleep_seconds_per_cycle()))
        times = []
        for r in range(reps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            torch.cuda._sleep(cycles)
            s.record()
            run(r)
            e.record()
            e.synchronize()
            times.append(s.elapsed_time(e))
        return statistics.median(times)

    def time_launches(self, fn, launches):
        """Milliseconds per launch of fn: a graph of `launches` calls, replayed once untimed, then
        the median of REPEATS timed replays divided by the launch count."""
        g = self.graph(fn, launches)
        g.replay()
        return self.time_graph(g) / launches


def measure_ceilings(gpu, small_bytes):
    """The box's own ceilings (include/sbn_ceilings.h): a streaming read of 2 GiB (HBM), a read of
    `small_bytes` as one launch (the decode step's size; rotated over the 2 GiB buffer, so it comes
    from HBM), INT8 dense and structured-sparse MFMA loops with no memory traffic, and an empty
    kernel's cost per launch in a graph. Each is the median of REPEATS timed replays."""
    import ctypes
    torch, b = gpu.torch, gpu.b
    lib = b.lib()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    big = 2 << 30
    buf = torch.zeros(big // 4, dtype=torch.int32, device="cuda")
    base = buf.data_ptr()
    small = (small_bytes + 4095) // 4096 * 4096
    slots = big // small

    def read_all(i):
        b.check(lib.sbn_ceiling_stream_read(ctypes.c_void_p(base), big, 0xFFFFFFFF, b._ptr(sink),
                                            b._stream(None)))

    def read_small(i):
        b.check(lib.sbn_ceiling_stream_read(ctypes.c_void_p(base + (i % slots) * small), small,
                                            0xFFFFFFFF, b._ptr(sink), b._stream(None)))

    ops = ctypes.c_double(0.0)
    waves, iters = 256 * 8, 4096

    def mfma(i):
        b.check(lib.sbn_ceiling_mfma_i8(iters, waves, b._ptr(sink), ctypes.byref(ops),
                                        b._stream(None)))

    sops = ctypes.c_double(0.0)

    def smfmac(i):
        b.check(lib.sbn_ceiling_smfmac_i8(iters, waves, b._ptr(sink), ctypes.byref(sops),
                                          b._stream(None)))

    def empty(i):
        b.check(lib.sbn_ceiling_empty(b._stream(None)))

    read_ms = gpu.time_launches(read_all, 5)
    small_ms = gpu.time_launches(read_small, KERNEL_LAUNCHES)
    mfma_ms = gpu.time_launches(mfma, 5)
    smfmac_ms = gpu.time_launches(smfmac, 5)
    empty_ms = gpu.time_launches(empty, KERNEL_LAUNCHES)
    del buf
    return {"hbm_read_GBps": big / (read_ms * 1e-3) / 1e9, "hbm_read_bytes": big,
            "small_read_us": small_ms * 1e3, "small_read_bytes": small,
            "small_read_GBps": small / (small_ms * 1e-3) / 1e9,
            "int8_mfma_TOPS": ops.value / (mfma_ms * 1e-3) / 1e12,
            "int8_smfmac_dense_equiv_TOPS": sops.value / (smfmac_ms * 1e-3) / 1e12,
            "empty_kernel_us": empty_ms * 1e3,
            "note": "measured on this GPU: streaming read, one read launch of the decode step's "
                    "size, INT8 MFMA loop, structured-sparse INT8 MFMA loop (2:4, counted "
                    "dense-equivalent), empty kernel (per launch in a graph)"}


def read_launch_ms(gpu, nbytes, launches):
    """Time of one plain read launch of `nbytes` (the ceiling kernel over a 1 GiB buffer, rotated so
    that it comes from HBM): the floor of any single launch that moves those bytes."""
    import ctypes
    torch, b = gpu.torch, gpu.b
    lib = b.lib()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    big = 1 << 30
    buf = torch.zeros(big // 4, dtype=torch.int32, device="cuda")
    base = buf.data_ptr()
    size = (nbytes + 4095) // 4096 * 4096
    slots = big // size

    def read(i):
        b.check(lib.sbn_ceiling_stream_read(ctypes.c_void_p(base + (i % slots) * size), size,
                                            0xFFFFFFFF, b._ptr(sink), b._stream(None)))

    ms = gpu.time_launches(read, launches)
    del buf
    return ms


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return os.cpu_count() or 1


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------------------------------------
# Workloads.
# ------------------------------------------------------------------------------------------------

FUSED_MAX_T = 4  # tokens up to which sbn_bitlinear_fwd_bf16 is a single kernel


def fused_bytes(T, K, n_out, n, m):
    """One-kernel decode step: bf16 x read, int8 x_q and a' written, packed weights and gamma
    read, y written."""
    return rpf_bytes(n_out, K, n, m) + 2 * T * K + T * K + 4 * T + 4 + 4 * T * n_out


def run_decode(gpu, args, T=1, with_cpu=True):
    """Decode: quantize T tokens + n:m forward on weights packed once (sbn_bitlinear_fwd_bf16:
    one kernel for T <= 4, else the quantize kernel and the GEMV)."""
    from sparsity_sbn_quantize_amd import inputs
    torch = gpu.torch
    wl = inputs.W_DECODE
    layer = wl.layers[0]
    n, m = wl.patterns[0]
    K, N = layer.k, layer.n_out
    x_bits, w = inputs.layer_inputs(wl, 0, T)
    xd, wd = gpu.bf16(x_bits), gpu.f32(w)
    R = max(1, -(-args.rotate_bytes // rpf_bytes(N, K, n, m)))
    pws = [gpu.b.PackedWeight(wd, n, m) for _ in range(R)]
    q = torch.empty((T, K), dtype=torch.int8, device="cuda")
    a = torch.empty((T,), dtype=torch.float32, device="cuda")
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    fused = T <= FUSED_MAX_T

    def step(i):
        gpu.b.bitlinear_bf16(xd, pws[i % R], out="f32", y=y, x_q=q, x_absmax=a)

    def gemv_only(i):
        gpu.b.bitlinear(q, a, pws[i % R], out="f32", y=y)

    def quant_only(i):
        gpu.b.quantize_act(xd, out_q=q, out_absmax=a)

    def two_call(i):
        gpu.b.quantize_act(xd, out_q=q, out_absmax=a)
        gpu.b.bitlinear(q, a, pws[i % R], out="f32", y=y)

    # BitLinear operation 1 in front: the parameter-free LayerNorm, fused (one kernel for
    # T <= 4) and as its own kernel
    def ln_step(i):
        gpu.b.bitlinear_bf16(xd, pws[i % R], out="f32", y=y, x_q=q, x_absmax=a, ln_eps=LN_EPS)

    def ln_quant_only(i):
        gpu.b.layernorm_quantize_act(xd, LN_EPS, out_q=q, out_absmax=a)

    # the step equals the two-call path bit for bit
    two_call(0)
    torch.cuda.synchronize()
    y_two = y.clone()
    step(0)
    torch.cuda.synchronize()
    assert torch.equal(y, y_two), "one-call step differs from quantize + forward"
    y_eager = y.clone()
    gw = gpu.graph(step, args.warmup) if args.warmup > 0 else None
    # Exactly K steps per timed region, the median of REPEATS regions over disjoint runs of the
    # rotated copies (no region finds its weights in the last-level cache). Two ways to launch
    # them, both reported: one K-step HIP graph per region, and K eager launches behind a GPU busy
    # wait. A graph replay carries a fixed cost (about 10 us) that K = 20 steps do not amortize,
    # and the host cannot enqueue eager launches as fast as the GPU runs them beyond about 100;
    # the step time is the eager one for K <= 64, the graph one above.
    gss = [gpu.graph(lambda i, o=r * args.steps: step(o + i), args.steps) for r in range(REPEATS)]
    if gw is not None:
        gw.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_graph = statistics.median(gpu.time_graph(g, reps=1) for g in gss)
    assert torch.equal(y, y_eager), "graph replay differs from the eager forward"

    def eager_run(r):
        for i in range(args.steps):
            step(r * args.steps + i)

    ms_eager = gpu.time_eager(eager_run)
    wall = time.perf_counter() - t0
    assert torch.equal(y, y_eager), "eager steps differ from the first forward"
    ms = ms_eager if args.steps <= 64 else ms_graph
    timings = {}
    for name, fn in (("bitlinear_gemv", gemv_only), ("quantize_act", quant_only),
                     ("quantize_act+bitlinear_gemv", two_call),
                     ("layernorm_quantize_act", ln_quant_only),
                     ("bitlinear_gemv (layernorm + quantize fused)", ln_step)):
        if args.lean and name != "bitlinear_gemv":
            continue
        timings[name] = gpu.time_launches(fn, max(args.steps, KERNEL_LAUNCHES))
    # Pack variants on the same weights: the compact plane (GEMV reads nonzero masks + signs)
    # and 16:256 outliers (the step plus the outlier term); fewer rotated copies of each
    variants = {}
    for tag, kw in (() if args.lean else
                    (("compact", {"compact": True}), ("outliers 16:256", {"outliers": 16}))):
        Rv = max(1, R // 2)
        pv = [gpu.b.PackedWeight(wd, n, m, **kw) for _ in range(Rv)]

        def vstep(i, pv=pv, Rv=Rv):
            gpu.b.bitlinear_bf16(xd, pv[i % Rv], out="f32", y=y, x_q=q, x_absmax=a)

        def vgemv(i, pv=pv, Rv=Rv):
            gpu.b.bitlinear(q, a, pv[i % Rv], out="f32", y=y)

        for name, fn in ((f"step ({tag})", vstep), (f"int8 forward ({tag})", vgemv)):
            variants[name] = gpu.time_launches(fn, max(args.steps, KERNEL_LAUNCHES)) * 1e3
        if tag == "compact":
            variants["compact bytes per weight"] = pv[0].query().compact_bytes / (N * K)
        for p in pv:
            p.free()
    # The rank encoding (an export of the same packs, read by no kernel): time per export into one
    # buffer, and its bytes per weight.
    rrb = pws[0].query().rank_row_bytes if not args.lean else 0
    rank_out = gpu.torch.empty((N, rrb), dtype=gpu.torch.uint8, device="cuda")
    lib = gpu.b.lib()

    def rank_export(i):
        gpu.b.check(lib.sbn_packed_export_rank(pws[i % R].handle, gpu.b._ptr(rank_out),
                                               gpu.b._stream(None)))

    if not args.lean:
        variants["rank export"] = gpu.time_launches(rank_export,
                                                    max(args.steps, KERNEL_LAUNCHES)) * 1e3
        variants["rank bytes per weight"] = rrb * N / (N * K)
    ms_step = ms / args.steps
    if fused:
        step_bytes = fused_bytes(T, K, N, n, m)
        kms = gpu.time_launches(step, max(args.steps, KERNEL_LAUNCHES))
        kname, kbytes = "bitlinear_gemv (quantize fused)", step_bytes
        tkey = f"gemv_fused_{n}of{m}_T{T}"
        timings["bitlinear_gemv (quantize fused)"] = kms
    else:
        step_bytes = forward_bytes(T, K, N, n, m) + quantize_bytes(T, K)
        kname, kbytes, kms = "bitlinear_gemv", forward_bytes(T, K, N, n, m), timings["bitlinear_gemv"]
        tkey = f"gemv_{n}of{m}_T{T}"
    achieved = kbytes / (kms * 1e-3) / 1e9
    res = {
        "value": step_bytes / (ms_step * 1e-3) / 1e9, "unit": "GB/s", "ms_per_step": ms_step,
        "wall_s": wall,
        "step_timing": {"method": "eager launches" if args.steps <= 64 else "HIP graph",
                        "graph_ms_per_step": ms_graph / args.steps,
                        "eager_ms_per_step": ms_eager / args.steps},
        "config": {"workload": f"{wl.name}_T{T}", "pattern": f"{n}:{m}", "tokens": T, "K": K,
                   "n_out": N, "weights": "packed once, rotated over %d copies" % R,
                   "step": "one kernel (quantize fused)" if fused else "quantize + GEMV kernels",
                   "step_bytes": step_bytes},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": measured_traffic(tkey),
                     "bytes_per_launch": kbytes, "avg_launch_us": kms * 1e3},
        "kernels_us": {k: v * 1e3 for k, v in timings.items()},
        "pack_variants_us": variants,
    }
    if with_cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_decode(x_bits, w, n, m, step_bytes, args.cpu_seconds)
    for p in pws:
        p.free()
    return res


# Decode shapes with a larger K than the configured workloads (70B- and 13B-style down
# projections), where one launch streams tens of MB of weights: int8 GEMV, weights N(0, 0.02).
LARGE_DECODE = ((8192, 28672, 8, 16), (5120, 13824, 6, 8))


def run_decode_large(gpu, args):
    torch = gpu.torch
    rows = []
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    for (N, K, n, m) in LARGE_DECODE:
        w = torch.randn((N, K), device="cuda", generator=gen) * 0.02
        xs = [(torch.randn((T, K), device="cuda", generator=gen)).to(torch.bfloat16)
              for T in (1, 16)]
        # the positional plane (2 bits per weight), then the compact plane ((m + n) / m bits per
        # weight), each over enough packed copies that the weights stream from HBM
        for plane, kw, bits in (("positional", {}, 2.0), ("compact", {"compact": True},
                                                          (m + n) / m)):
            R = max(1, -(-args.rotate_bytes // int(N * K * bits / 8)))
            pws = [gpu.b.PackedWeight(w, n, m, **kw) for _ in range(R)]
            for x in xs:
                T = x.shape[0]
                q, a = gpu.b.quantize_act(x)
                y = torch.empty((T, N), dtype=torch.float32, device="cuda")
                us = gpu.time_launches(
                    lambda i: gpu.b.bitlinear(q, a, pws[i % R], out="f32", y=y),
                    max(args.steps, 100)) * 1e3
                fb = forward_bytes(T, K, N, n, m)
                rows.append({"n_out": N, "K": K, "pattern": f"{n}:{m}", "tokens": T,
                             "plane": plane, "plane_bits_per_weight": bits, "us": us,
                             "bytes": fb, "GBps": fb / us / 1e3,
                             "frac_hbm": fb / us / 1e3 / HBM_PEAK_GBS})
            for p in pws:
                p.free()
        del w, xs
        torch.cuda.empty_cache()
    return {"workload": "decode_gemv_large_k (int8 GEMV; extra shapes, N(0, 0.02) weights)",
            "rows": rows}


def cpu_decode(x_bits, w, n, m, step_bytes, seconds):
    import oracle
    packed = oracle.pack_nm_ternary(w, n, m)  # packed once, as on the GPU
    steps, t0 = 0, time.perf_counter()
    while True:
        q, a = oracle.quantize_act(x_bits)
        acc = oracle.int_matmul(q, packed["codes"])
        oracle.dequantize(acc, packed["gamma"], a)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds and steps >= 3:
            break
    return {"value": step_bytes * steps / el / 1e9, "unit": "GB/s", "cores": cpu_threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"the full step (quantize + exact fp64 matmul + dequantize), {steps} steps "
                      f"in {el:.1f} s"}


def run_prefill(gpu, args, layer_index=0, steps=None, with_cpu=True, cpu_seconds=None):
    """Prefill GEMM: quantize 2048 tokens + 8:16 forward (weights packed once)."""
    from sparsity_sbn_quantize_amd import inputs
    torch = gpu.torch
    wl = inputs.W_PREFILL
    layer = wl.layers[layer_index]
    n, m = wl.patterns[0]
    T = wl.tokens[0]
    K, N = layer.k, layer.n_out
    steps = steps or args.steps
    x_bits, w = inputs.layer_inputs(wl, layer_index, T)
    xd, wd = gpu.bf16(x_bits), gpu.f32(w)
    pw = gpu.b.PackedWeight(wd, n, m)
    q = torch.empty((T, K), dtype=torch.int8, device="cuda")
    a = torch.empty((T,), dtype=torch.float32, device="cuda")
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")

    def step(i):
        gpu.b.quantize_act(xd, out_q=q, out_absmax=a)
        gpu.b.bitlinear(q, a, pw, out="f32", y=y)

    def gemm_only(i):
        gpu.b.bitlinear(q, a, pw, out="f32", y=y)

    step(0)
    torch.cuda.synchronize()
    y_eager = y.clone()
    ms = gpu.time_launches(step, max(steps, KERNEL_LAUNCHES))
    assert torch.equal(y, y_eager), "graph replay differs from the eager forward"
    gemm_ms = gpu.time_launches(gemm_only, max(steps, KERNEL_LAUNCHES))
    act_ms = {}
    for name, fn in (() if args.lean else
                     (("quantize_act", lambda i: gpu.b.quantize_act(xd, out_q=q, out_absmax=a)),
                      ("layernorm_quantize_act",
                       lambda i: gpu.b.layernorm_quantize_act(xd, LN_EPS, out_q=q,
                                                              out_absmax=a)))):
        act_ms[name] = gpu.time_launches(fn, max(steps, KERNEL_LAUNCHES))
    act_bytes = 3.0 * T * K + 4.0 * T  # bf16 in, int8 + a' out
    ops = 2.0 * T * K * N
    achieved = ops / (gemm_ms * 1e-3) / 1e12
    res = {
        "value": ops / (ms * 1e-3) / 1e12, "unit": "TOPS", "ms_per_step": ms,
        "activation_kernels": {k: {"us": v * 1e3, "GBps": act_bytes / (v * 1e-3) / 1e9,
                                   "frac_hbm": act_bytes / (v * 1e-3) / 1e9 / HBM_PEAK_GBS}
                               for k, v in act_ms.items()},
        "config": {"workload": f"{wl.name}_{layer.name}", "pattern": f"{n}:{m}", "tokens": T,
                   "K": K, "n_out": N, "ops": "dense-equivalent 2*T*K*N"},
        "roofline": {"bound": "mfma", "kernel": "bitlinear_gemm", "achieved": achieved,
                     "peak": INT8_PEAK_TOPS, "unit": "TOP/s", "frac": achieved / INT8_PEAK_TOPS,
                     "traffic": measured_traffic(f"gemm_{n}of{m}_{layer.name}"),
                     "avg_launch_us": gemm_ms * 1e3,
                     # the method's own work: the kept weights' multiply-adds, T*K*N*n/m
                     "algorithmic_macs": T * K * N * n / m,
                     "algorithmic_TMACs_per_s": T * K * N * n / m / (gemm_ms * 1e-3) / 1e12},
    }
    if with_cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_prefill(x_bits, w, n, m, K, N,
                                          cpu_seconds if cpu_seconds else args.cpu_seconds)
    pw.free()
    return res


def cpu_prefill(x_bits, w, n, m, K, N, seconds):
    import oracle
    packed = oracle.pack_nm_ternary(w, n, m)
    tok = 32
    steps, t0 = 0, time.perf_counter()
    while True:
        q, a = oracle.quantize_act(x_bits[:tok])
        acc = oracle.int_matmul(q, packed["codes"])
        oracle.dequantize(acc, packed["gamma"], a)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds and steps >= 2:
            break
    ops = 2.0 * tok * K * N * steps
    return {"value": ops / el / 1e12, "unit": "TOPS", "cores": cpu_threads(), "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"{tok} of the tokens per step (same weights, K, N), {steps} steps in "
                      f"{el:.1f} s"}


# The block's grouped launches: members that read the same input share one launch.
BLOCK_GROUPS = ((0, 1, 2), (3,), (4, 5), (6,))  # Q/K/V, O, gate/up, down


def run_block(gpu, args, pattern, T, steps):
    """2B-style block: Q, K, V, O, gate, up, down BitLinears at T tokens for one n:m pattern.

    A block step quantizes each of the four distinct layer inputs and runs all seven forwards.
    Grouped (the block total): Q/K/V and gate/up each run as one grouped launch; for T <= 4 each
    of the four groups is one kernel that also quantizes its input (sbn_bitlinear_fwd_group_bf16),
    for T = 16 the quantize kernel and the grouped GEMV, for T > 16 the quantize kernel and one GEMM
    per layer. Ungrouped (for comparison): four quantize kernels and seven forwards. Per layer: the
    forward alone on int8 input, and for T <= 4 the one-kernel step of that layer alone. Decode token
    counts rotate over distinct packed copies of the whole block (>= 1 GiB), so weights stream
    from HBM."""
    from sparsity_sbn_quantize_amd import inputs
    torch = gpu.torch
    wl = inputs.W_BLOCK
    n, m = pattern
    layers = wl.layers
    acts = {}
    for layer in layers:
        if layer.act_input not in acts:
            xb = inputs.activations(wl, layer.act_input, T, layer.k)
            acts[layer.act_input] = (gpu.bf16(xb),
                                     torch.empty((T, layer.k), dtype=torch.int8, device="cuda"),
                                     torch.empty((T,), dtype=torch.float32, device="cuda"))
    wds = gpu.block_weights
    ys = [torch.empty((T, l.n_out), dtype=torch.float32, device="cuda") for l in layers]
    weight_bytes = sum(rpf_bytes(l.n_out, l.k, n, m) for l in layers)
    R = max(1, -(-args.rotate_bytes // weight_bytes)) if T <= 16 else 1
    packed = [[gpu.b.PackedWeight(wds[i], n, m) for i in range(len(layers))] for _ in range(R)]
    b = gpu.b

    def ungrouped(i):
        pw = packed[i % R]
        for (xd, q, a) in acts.values():
            b.quantize_act(xd, out_q=q, out_absmax=a)
        for li, layer in enumerate(layers):
            _, q, a = acts[layer.act_input]
            b.bitlinear(q, a, pw[li], out="f32", y=ys[li])

    def grouped(i):
        pw = packed[i % R]
        for grp in BLOCK_GROUPS:
            xd, q, a = acts[layers[grp[0]].act_input]
            members = [pw[li] for li in grp]
            outs = [ys[li] for li in grp]
            if T <= FUSED_MAX_T:
                b.bitlinear_group_bf16(xd, members, out="f32", ys=outs, x_q=q, x_absmax=a)
            else:
                b.quantize_act(xd, out_q=q, out_absmax=a)
                b.bitlinear_group(q, a, members, out="f32", ys=outs)

    # the grouped step equals the ungrouped one bit for bit
    ungrouped(0)
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    grouped(0)
    torch.cuda.synchronize()
    assert all(torch.equal(y, r) for y, r in zip(ys, ref)), "grouped block differs"
    nl = max(steps, KERNEL_LAUNCHES) if T <= 16 else max(steps, 20)
    ms_g = gpu.time_launches(grouped, nl)
    ms_u = gpu.time_launches(ungrouped, nl)
    per_layer = []
    if T <= 16:
        for li, layer in enumerate(layers):
            xd, q, a = acts[layer.act_input]
            fwd_ms = gpu.time_launches(
                lambda i, li=li, q=q, a=a: b.bitlinear(q, a, packed[i % R][li], out="f32",
                                                       y=ys[li]), nl)
            row = {"layer": layer.name, "K": layer.k, "n_out": layer.n_out,
                   "forward_us": fwd_ms * 1e3,
                   "forward_GBps": forward_bytes(T, layer.k, layer.n_out, n, m) /
                   (fwd_ms * 1e-3) / 1e9}
            if T <= FUSED_MAX_T:
                st_ms = gpu.time_launches(
                    lambda i, li=li, xd=xd, q=q, a=a: b.bitlinear_bf16(
                        xd, packed[i % R][li], out="f32", y=ys[li], x_q=q, x_absmax=a), nl)
                row["step_us"] = st_ms * 1e3
                row["step_GBps"] = fused_bytes(T, layer.k, layer.n_out, n, m) / (st_ms * 1e-3) / 1e9
            per_layer.append(row)
        groups = []
        for grp in BLOCK_GROUPS:
            if len(grp) < 2:
                continue
            xd, q, a = acts[layers[grp[0]].act_input]
            outs = [ys[li] for li in grp]
            if T <= FUSED_MAX_T:
                fn = (lambda i, grp=grp, xd=xd, q=q, a=a, outs=outs: b.bitlinear_group_bf16(
                    xd, [packed[i % R][li] for li in grp], out="f32", ys=outs, x_q=q, x_absmax=a))
                gbytes = sum(rpf_bytes(layers[li].n_out, layers[li].k, n, m) + 4 * T *
                             layers[li].n_out + 4 for li in grp) + \
                    quantize_bytes(T, layers[grp[0]].k)
            else:
                fn = (lambda i, grp=grp, q=q, a=a, outs=outs: b.bitlinear_group(
                    q, a, [packed[i % R][li] for li in grp], out="f32", ys=outs))
                gbytes = sum(rpf_bytes(layers[li].n_out, layers[li].k, n, m) + 4 * T *
                             layers[li].n_out + 4 for li in grp) + T * layers[grp[0]].k + 4 * T
            g_ms = gpu.time_launches(fn, nl)
            r_ms = read_launch_ms(gpu, gbytes, nl)
            groups.append({"layers": "/".join(layers[li].name for li in grp), "us": g_ms * 1e3,
                           "bytes": gbytes, "GBps": gbytes / (g_ms * 1e-3) / 1e9,
                           "frac_hbm": gbytes / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "read_launch_us": r_ms * 1e3, "of_read_launch": r_ms / g_ms})
    ops = sum(2.0 * T * l.k * l.n_out for l in layers)
    fb = sum(forward_bytes(T, l.k, l.n_out, n, m) for l in layers)
    qb = sum(quantize_bytes(T, layers[[l.act_input for l in layers].index(ai)].k) for ai in acts)
    for pw in packed:
        for p_ in pw:
            p_.free()
    out = {"pattern": f"{n}:{m}", "tokens": T, "ms_per_step": ms_g,
           "ungrouped_ms_per_step": ms_u, "TOPS": ops / (ms_g * 1e-3) / 1e12,
           "GBps": (fb + qb) / (ms_g * 1e-3) / 1e9,
           "frac_hbm": (fb + qb) / (ms_g * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "weight_bytes": weight_bytes,
           "launches": 4 if T <= FUSED_MAX_T else (8 if T <= 16 else 11)}
    if per_layer:
        out["per_layer"] = per_layer
        out["grouped_launches"] = groups
    return out


def run_train(gpu, args, layer_index, pattern, steps):
    """7B-style dynamic-sparsity training step, forward part: re-pack the fp32 latent weights
    (absmean + n:m mask + ternary codes), quantize the 8192-token input, n:m GEMM."""
    from sparsity_sbn_quantize_amd import inputs
    torch = gpu.torch
    wl = inputs.W_TRAIN
    layer = wl.layers[layer_index]
    n, m = pattern
    T = wl.tokens[0]
    K, N = layer.k, layer.n_out
    x_bits, w = inputs.layer_inputs(wl, layer_index, T)
    xd, wd = gpu.bf16(x_bits), gpu.f32(w)
    del x_bits, w
    # The re-pack reads the latent weights from HBM: the timed packs rotate over distinct copies of
    # them (>= 1 GiB in all, beyond the 256 MB last-level cache), each re-packed into one handle.
    # Each copy carries its own small update (N(0, 1e-4), half a percent of the weights' scale),
    # as consecutive training steps would: masks flip, gamma moves a little.
    RL = max(1, -(-args.rotate_bytes // (4 * N * K)))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1000 + layer_index)
    wds = [wd] + [wd + 1e-4 * torch.randn(wd.shape, device="cuda", generator=gen)
                  for _ in range(RL - 1)]
    pw = gpu.b.PackedWeight(wd, n, m)
    q = torch.empty((T, K), dtype=torch.int8, device="cuda")
    a = torch.empty((T,), dtype=torch.float32, device="cuda")
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")

    def step(i):
        pw.pack(wds[i % RL])
        gpu.b.quantize_act(xd, out_q=q, out_absmax=a)
        gpu.b.bitlinear(q, a, pw, out="f32", y=y)

    def pack_only(i):
        pw.pack(wds[i % RL])

    def gemm_only(i):
        gpu.b.bitlinear(q, a, pw, out="f32", y=y)

    step(0)
    torch.cuda.synchronize()
    res = {}
    for name, fn in (("step", step), ("pack", pack_only), ("gemm", gemm_only)):
        res[name] = gpu.time_launches(fn, max(steps, KERNEL_LAUNCHES))
    pb = pack_bytes(N, K, n, m)
    ops = 2.0 * T * K * N
    out = {"layer": layer.name, "pattern": f"{n}:{m}", "tokens": T, "K": K, "n_out": N,
           "ms_per_step": res["step"], "pack_us": res["pack"] * 1e3,
           "pack_GBps": pb / (res["pack"] * 1e-3) / 1e9,
           "pack_frac_hbm": pb / (res["pack"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "pack_latent_copies": RL,
           "gemm_us": res["gemm"] * 1e3, "gemm_TOPS": ops / (res["gemm"] * 1e-3) / 1e12,
           "gemm_frac_int8": ops / (res["gemm"] * 1e-3) / 1e12 / INT8_PEAK_TOPS,
           "gemm_algorithmic_TMACs_per_s": T * K * N * n / m / (res["gemm"] * 1e-3) / 1e12}
    if (n, m) == (2, 4):
        # 2:4 runs on the structured-sparse MFMA; time the dense-MFMA path on the same weights
        # (positional codes) beside it, and check that both give the same output.
        pw.pack(wd)
        gpu.b.bitlinear(q, a, pw, out="f32", y=y)
        y_sp = y.clone()
        os.environ["SBN_NO_SMFMAC"] = "1"
        try:
            pd = gpu.b.PackedWeight(wd, n, m)
        finally:
            del os.environ["SBN_NO_SMFMAC"]
        yd = torch.empty_like(y)
        gpu.b.bitlinear(q, a, pd, out="f32", y=yd)
        torch.cuda.synchronize()
        assert torch.equal(yd, y_sp), "dense and structured-sparse MFMA paths differ"
        dense_ms = gpu.time_launches(lambda i: gpu.b.bitlinear(q, a, pd, out="f32", y=yd), max(steps, KERNEL_LAUNCHES))
        pd.free()
        out["gemm"] = "structured-sparse MFMA (v_smfmac_i32_16x16x128_i8)"
        out["gemm_dense_mfma_us"] = dense_ms * 1e3
        out["gemm_dense_mfma_frac_int8"] = ops / (dense_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS
    # Straight-through data gradient on the same packed weights: dY bf16 [T][N] -> dX fp32 [T][K]
    # on the bf16 MFMA. The first call after a pack also rebuilds the transposed code plane, so a
    # training step's gradient costs the pack_bwd line (pack, transposed plane, gradient).
    dy = gpu.bf16(inputs.grad_output(wl, layer_index, T))
    dx = torch.empty((T, K), dtype=torch.float32, device="cuda")
    pw.pack(wd)
    gpu.b.bitlinear_bwd_dx(dy, pw, dx=dx)
    torch.cuda.synchronize()
    dx_eager = dx.clone()
    bw = {"bwd": gpu.time_launches(lambda i: gpu.b.bitlinear_bwd_dx(dy, pw, dx=dx),
                                   max(steps, KERNEL_LAUNCHES))}
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_eager), "data-gradient graph replay differs from the eager call"
    bw["pack_bwd"] = gpu.time_launches(lambda i: (pw.pack(wds[i % RL]),
                                                  gpu.b.bitlinear_bwd_dx(dy, pw, dx=dx)),
                                       max(steps, KERNEL_LAUNCHES))
    out["bwd_dx_us"] = bw["bwd"] * 1e3
    out["bwd_dx_TFLOPS"] = ops / (bw["bwd"] * 1e-3) / 1e12
    out["bwd_dx_frac_bf16"] = out["bwd_dx_TFLOPS"] / BF16_PEAK_TFLOPS
    out["pack_transpose_bwd_us"] = bw["pack_bwd"] * 1e3
    del dy, dx, dx_eager, wds
    pw.free()
    return out


def profile_copy(gpu, args):
    """A plain device copy of known size (for scaling HBM byte counters)."""
    torch = gpu.torch
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": 5}))


# Counter runs behind profiles/traffic.json: tag -> (traffic key, kernel-name pattern). Each tag
# names the bench workload that was run under `rocprofv3 --pmc FETCH_SIZE` and, separately,
# `--pmc WRITE_SIZE`; the tag "copy" is `bench.py --profile-copy`.
TRAFFIC_RUNS = {
    # positional codes (form 0) only: the compact variant's GEMV runs in the same workload
    "decode": ("gemv_fused_6of8_T1", r"bitlinear_gemv_bf16_one<0,"),
    "decode16": ("gemv_6of8_T16", r"bitlinear_gemv_i8_deep<0,"),
    "prefill_up": ("gemm_8of16_ffn_up", r"bitlinear_gemm<"),
    "prefill_down": ("gemm_8of16_ffn_down", r"bitlinear_gemm<"),
}


def record_traffic(root):
    """Writes profiles/traffic.json from rocprofv3 counter CSVs under `root`, laid out as
    <tag>_<COUNTER>/run_counter_collection.csv. Bytes per launch = the median per-dispatch counter
    value (KiB) x 1024 x the scale that maps the same counter onto a 1 GiB device copy."""
    import csv
    import re
    import statistics

    def per_dispatch(tag, counter, pattern):
        path = os.path.join(root, f"{tag}_{counter}", "run_counter_collection.csv")
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"].startswith(counter) and re.search(pattern, r["Kernel_Name"]):
                    vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(
                        r["Counter_Value"])
        return list(vals.values())

    copy_bytes = 1 << 30
    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        v = per_dispatch("copy", c, r".")
        scale[c] = copy_bytes / (max(v) * 1024.0)
    out = {"_note": "HBM bytes per launch = FETCH_SIZE x %.3f + WRITE_SIZE x %.3f (KiB x 1024); "
                    "scales from a 1 GiB device copy; valid only for the kernel sources with this "
                    "hash" % (scale["FETCH_SIZE"], scale["WRITE_SIZE"])}
    for tag, (key, pattern) in TRAFFIC_RUNS.items():
        try:
            fetch = statistics.median(per_dispatch(tag, "FETCH_SIZE", pattern))
            write = statistics.median(per_dispatch(tag, "WRITE_SIZE", pattern))
        except (OSError, ValueError, statistics.StatisticsError):
            continue
        out[key] = {"bytes_per_launch": int(round((fetch * scale["FETCH_SIZE"] +
                                                   write * scale["WRITE_SIZE"]) * 1024)),
                    "fetch_bytes": int(round(fetch * scale["FETCH_SIZE"] * 1024)),
                    "write_bytes": int(round(write * scale["WRITE_SIZE"] * 1024)),
                    "source_hash": kernel_source_hash()}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "decode16", "prefill_up", "prefill_down", "block", "train"])
    ap.add_argument("--rotate-bytes", type=int, default=1 << 30,
                    help="distinct packed-weight bytes rotated through (cold HBM)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--profile-copy", action="store_true")
    ap.add_argument("--lean", action="store_true",
                    help="only the workload's step and its dominant kernel (for profiler runs): no "
                         "variants, secondary lines, ceilings or CPU baseline")
    ap.add_argument("--record-traffic", metavar="DIR",
                    help="write profiles/traffic.json from rocprofv3 counter runs under DIR")
    args = ap.parse_args()
    if args.lean:
        args.no_secondary = True
        args.no_cpu_baseline = True
    if args.record_traffic:
        record_traffic(args.record_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    gpu = Gpu()
    if args.profile_copy:
        profile_copy(gpu, args)
        return
    if args.workload == "block":
        large = run_decode_large(gpu, args)
        from sparsity_sbn_quantize_amd import inputs
        gpu.block_weights = [gpu.f32(inputs.latent_weights(inputs.W_BLOCK, i))
                             for i in range(len(inputs.W_BLOCK.layers))]
        rows = [run_block(gpu, args, pat, T, 20 if T > 16 else min(args.steps, 500))
                for pat in inputs.W_BLOCK.patterns for T in inputs.W_BLOCK.tokens]
        print(json.dumps({"workload": inputs.W_BLOCK.name, "rows": rows, "decode_large_k": large}))
        return
    if args.workload == "train":
        rows = [run_train(gpu, args, li, pat, 10) for pat in ((2, 4), (8, 16)) for li in (0, 1)]
        print(json.dumps({"workload": "train_step_7b_ffn_T8192", "rows": rows}))
        return
    if args.workload == "decode":
        res = run_decode(gpu, args, T=1)
    elif args.workload == "decode16":
        res = run_decode(gpu, args, T=16)
    else:
        res = run_prefill(gpu, args, 0 if args.workload == "prefill_up" else 1,
                          steps=min(args.steps, 200))
    line = {"metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1,
            "steps": args.steps if args.workload.startswith("decode") else min(args.steps, 200),
            "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
            "config": res["config"], "roofline": res["roofline"],
            "kernels_us": res.get("kernels_us")}
    if res.get("step_timing"):
        line["step_timing"] = res["step_timing"]
    if res.get("pack_variants_us"):
        line["pack_variants_us"] = res["pack_variants_us"]
    if "activation_kernels" in res:
        line["activation_kernels"] = res["activation_kernels"]
    if "cpu_baseline" in res:
        line["cpu_baseline"] = res["cpu_baseline"]
    ceil = (measure_ceilings(gpu, res["roofline"].get("bytes_per_launch", 1 << 22))
            if not args.lean else None)
    line["ceilings"] = ceil
    rl = line["roofline"]
    if ceil is None:
        pass
    elif rl["bound"] == "hbm":
        rl["measured_peak"] = ceil["hbm_read_GBps"]
        rl["frac_measured"] = rl["achieved"] / ceil["hbm_read_GBps"]
        rl["frac_small_read"] = rl["achieved"] / ceil["small_read_GBps"]
    else:
        rl["measured_peak"] = ceil["int8_mfma_TOPS"]
        rl["frac_measured"] = rl["achieved"] / ceil["int8_mfma_TOPS"]
    if not args.no_secondary and args.workload == "decode":
        sec = []
        r16 = run_decode(gpu, args, T=16, with_cpu=False)
        sec.append({k: r16[k] for k in ("value", "unit", "ms_per_step", "config", "roofline")})
        for li in (0, 1):
            rp = run_prefill(gpu, args, li, steps=50, with_cpu=not args.no_cpu_baseline,
                             cpu_seconds=min(args.cpu_seconds, 5.0))
            sec.append({k: rp[k] for k in ("value", "unit", "ms_per_step", "config", "roofline",
                                           "activation_kernels", "cpu_baseline") if k in rp})
        # both 7B FFN shapes at both patterns of the training-step workload
        for pat in ((2, 4), (8, 16)):
            for li in (0, 1):
                sec.append({"train_step": run_train(gpu, args, li, pat, 5)})
        sec.append({"decode_large_k": run_decode_large(gpu, args)})
        from sparsity_sbn_quantize_amd import inputs
        gpu.block_weights = [gpu.f32(inputs.latent_weights(inputs.W_BLOCK, i))
                             for i in range(len(inputs.W_BLOCK.layers))]
        for T in (1, 16):
            for pat in inputs.W_BLOCK.patterns:
                print(f"[bench] block {pat[0]}:{pat[1]} T={T}", file=sys.stderr, flush=True)
                sec.append({"block": run_block(gpu, args, pat, T, args.steps)})
        del gpu.block_weights
        line["secondary"] = sec
    print(json.dumps(line))


if __name__ == "__main__":
    main()
