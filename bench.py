"""Benchmark of the trellis-coded GEMV hot path on one MI355X.

Default workload: the dense-MLP decode step at batch 1 (gate K2 5120->17408, up K3
5120->17408, down K3 17408->5120, each on its own input), one trellis_gemv_list launch per
step.  Metric: code bytes (in*out*K/8 summed over the three matrices) per second.  The same
JSON line carries the single-matrix latency, the small-batch decode at B = 1, 2, 4, 8, the
MoE decode (8 of 256 experts), the fused routed-expert MLP token (MCG and E4M3 codebooks),
fp16 and FP8 prefill, the roofline of the step's kernel
against HBM with the measured decode ceiling beside it, and the CPU oracle timed on a
bounded sample.

Weights are rotated over enough distinct device copies (> 1 GiB in total) that the 256 MB
Infinity Cache cannot serve them between steps; inputs are resident in HBM before timing.
Every timed leg runs at least 50 ms of the same untimed work first (the GPU's clocks take
~20-30 ms of sustained load to rise after an idle spell), then its W warm-up steps, then
exactly K timed steps; the line's "clock_ramp" says how much ramp work each leg ran.

Prints ONE JSON line (rank 0, N = 1).  --workload selects the other lines (the encoder,
the standalone entry points, the microbenchmarks) or one of the above alone.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
MFMA_F8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
ROTATE_BYTES = 1 << 30
COPY_PROBE_BYTES = 256 << 20   # plain device copy used to calibrate the HBM byte counters
# Counter-derived HBM traffic of the GEMV launch, with the hash of the kernel sources it was
# measured on; the figure is reported only while those sources are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_dense_mlp_b1_hbm_traffic.txt")
GEMV_SOURCES = ["trellis_coded_bit_amd/csrc/gemv.hip", "trellis_coded_bit_amd/csrc/trellis_device.h",
                "trellis_coded_bit_amd/csrc/launch.h"]


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _copies(nbytes_per_copy: int) -> int:
    return max(2, -(-ROTATE_BYTES // max(1, nbytes_per_copy)))


def cpu_baseline_dense(wl, budget_s: float = 12.0):
    """The CPU oracle on a bounded sample: decode + fp64 forward of whole 128-column output
    blocks of the three matrices, round robin, until the time budget is spent."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    names = ["gate", "up", "down"]
    t0 = time.perf_counter()
    nbytes = 0
    blocks = 0
    k = 0
    while time.perf_counter() - t0 < budget_s:
        name = names[k % 3]
        lin = wl.layers[name]
        J = (k // 3) % (lin.out_features // 128)
        O.forward_linear(lin, wl.xs[name], col_blocks=[J])
        nbytes += lin.in_features * 128 * lin.K // 8
        blocks += 1
        k += 1
    dt = time.perf_counter() - t0
    # the two parts separately, on one block of up_proj: decode (codes -> W_hat) and the
    # fp64 forward with W_hat given
    lin = wl.layers["up"]
    sub = np.ascontiguousarray(lin.code[:, 0:8, :])
    t_dec = 1e9
    for _ in range(3):  # (best of three: the first call also warms numpy up)
        t1 = time.perf_counter()
        w = O.decode_tiles(sub, lin.K).astype(np.float64)
        t_dec = min(t_dec, time.perf_counter() - t1)
    xh = O.had_blocks(wl.xs["up"].astype(np.float64) * O.side_scale(lin.rin, lin.s_in))
    t2 = time.perf_counter()
    for _ in range(20):
        O.had_blocks(xh @ w)
    t_fwd = (time.perf_counter() - t2) / 20
    blk_bytes = lin.in_features * 128 * lin.K // 8
    cpu_model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": round(nbytes / dt / 1e9, 6), "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{blocks} whole 128-column output blocks (decode + fp64 forward) of the gate/up/down "
                      f"matrices, round robin, {nbytes / 1e6:.1f} MB of code in {dt:.1f} s; host "
                      f"{cpu_model}, os.cpu_count()={os.cpu_count()}, "
                      f"affinity={len(os.sched_getaffinity(0))}, numpy decode single-threaded, "
                      f"BLAS threads={blas_threads}",
            "decode_only_GBps": round(blk_bytes / t_dec / 1e9, 6),
            "forward_only_GBps_of_code": round(blk_bytes / t_fwd / 1e9, 4)}


def gemv_source_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMV_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per GEMV launch from the committed counter summary (FETCH_SIZE + WRITE_SIZE,
    each scaled by the same counter's reading for a plain copy of known size), or None when
    the summary is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            kv = dict(line.split(":", 1) for line in fh if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != gemv_source_sha256():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(torch):
    """Three plain device-to-device copies of COPY_PROBE_BYTES (the counter calibration)."""
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_read_per_copy": COPY_PROBE_BYTES, "bytes_written_per_copy": COPY_PROBE_BYTES, "copies": 3}


def _capture(torch, fn):
    """Capture fn() into a HIP graph on a side stream (workspaces must be allocated)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


class LayerStack:
    """HIP graphs of consecutive steps, one weight copy per step (copy i % R for step i), as
    the layers of a model follow one another in one captured decode pass.  run(n) replays
    exactly n steps: full graphs of R steps, then one graph of the remainder."""

    def __init__(self, torch, step, R):
        self.torch, self.step, self.R = torch, step, R
        self.graphs = {}

    def _graph(self, n):
        if n not in self.graphs:
            self.graphs[n] = _capture(self.torch, lambda: [self.step(i) for i in range(n)])
        return self.graphs[n]

    def prepare(self, *counts):
        for n in counts:
            if n % self.R:
                self._graph(n % self.R)
        self._graph(self.R)

    def run(self, n):
        for _ in range(n // self.R):
            self._graph(self.R).replay()
        if n % self.R:
            self._graph(n % self.R).replay()


def _per_launch_us(torch, fn, R, reps):
    """Average duration of one launch: a HIP graph of R back-to-back launches (one per
    weight copy), replayed `reps` times between HIP events on the capturing stream's
    successor (the events see the launches' own stream: the replays run on it)."""
    g = _capture(torch, lambda: [fn(i) for i in range(R)])
    _ramp(torch, g.replay, "per_launch", min_ms=RAMP_MS / 2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * R)


# The GPU's clocks rise over the first ~20-30 ms of sustained load after an idle spell (the
# dense step measured 55-58 us per step in its first milliseconds and 43-44 us from ~25 ms
# on).  Every timed leg is therefore preceded by at least RAMP_MS of the same untimed work,
# before its W warm-up steps, so that the K timed steps measure the sustained rate of a
# decode loop that keeps the GPU busy, not the clock ramp.
RAMP_MS = 50.0
RAMP = {"min_ms": RAMP_MS, "legs": {}}


def _ramp(torch, run_once, label, min_ms=RAMP_MS, max_calls=100000):
    """Calls run_once() (untimed) until at least min_ms of GPU time has passed."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    calls = 0
    while calls < max_calls:
        run_once()
        calls += 1
        e1.record()
        e1.synchronize()
        if e0.elapsed_time(e1) >= min_ms:
            break
    RAMP["legs"][label] = {"calls": calls, "ms": round(e0.elapsed_time(e1), 1)}


def _time_steps(torch, step, R, warmup, steps, label="steps"):
    """Eager warm-up over the weight copies, then HIP graphs of consecutive steps (R steps
    per graph, as the layers of a captured decode pass follow one another): the clock ramp,
    `warmup` untimed steps, then exactly `steps` timed.  Returns ms per step."""
    for i in range(R):
        step(i)
    torch.cuda.synchronize()
    stack = LayerStack(torch, step, R)
    stack.prepare(warmup, steps)
    _ramp(torch, lambda: stack.run(R), label)
    stack.run(warmup)
    torch.cuda.synchronize()
    t_s = torch.cuda.Event(enable_timing=True)
    t_e = torch.cuda.Event(enable_timing=True)
    t_s.record()
    stack.run(steps)
    t_e.record()
    torch.cuda.synchronize()
    return t_s.elapsed_time(t_e) / steps


def _weight_copies(tb, base, R):
    """R distinct device copies of the layers' codes (side vectors shared)."""
    return [base] + [{n: tb.TrellisLinear(l.code.clone(), l.rin, l.rout, l.s_in, l.s_out, l.K, l.cb)
                      for n, l in base.items()} for _ in range(R - 1)]


def decode_ceiling(tb, weights_per_code_byte):
    """The decode's vector-instruction ceiling, measured: the products' per-tile decode and
    MFMA sequence (trellis_micro_valu, 4 waves per SIMD, as the products run) in tiles per
    second for the whole chip, in code bytes per second of the given width mix."""
    tb.micro_clock_kernel("valu", "decode_tile_mfma", 4, 4)
    cyc, tick, ms = tb.micro_clock_kernel("valu", "decode_tile_mfma", 4000, 4)
    tiles = 4 * tb.micro_cus() * 4 * 4000 * 16  # SIMDs x waves per SIMD x iterations x tiles
    ghz = float((cyc.double() / (tick.double() * 10.0)).median())
    tiles_per_s = tiles / (ms * 1e-3)
    simds = 4 * tb.micro_cus()
    return {"GBps": round(tiles_per_s * 256 / weights_per_code_byte / 1e9, 1),
            "clocks_per_tile_per_simd": round(simds * ghz * 1e9 / tiles_per_s, 2), "ghz": round(ghz, 3),
            "method": "trellis_micro_valu decode_tile_mfma (K3 decode + one 16x16x32 MFMA per tile, LDS-resident "
                      "words, 4 waves per SIMD), wall time"}


def run_dense(args, torch, tb, synth):
    """The dense-MLP decode step at batch 1: the workload's three matrices (gate K2, up K3,
    down K3, each on its own input) as ONE trellis_gemv_list launch.  Beside it, the same
    matrices as a dependent chain (gate+up one launch, then down), as a model's MLP runs."""
    wl = synth.dense_mlp(args.seed, batch=1)
    names = ["gate", "up", "down"]
    code_bytes = sum(wl.layers[n].code_bytes for n in names)
    weights = sum(wl.layers[n].in_features * wl.layers[n].out_features for n in names)
    flops = 2 * weights
    R = _copies(code_bytes)
    _log(f"dense MLP: {code_bytes / 1e6:.2f} MB code per step, {R} weight copies")
    base = {n: tb.TrellisLinear.from_host(wl.layers[n]) for n in names}
    copies = _weight_copies(tb, base, R)
    xs = [torch.from_numpy(wl.xs[n]).cuda() for n in names]
    ys = [torch.empty((1, wl.layers[n].out_features), dtype=torch.float16, device="cuda") for n in names]
    ws = torch.zeros(tb.trellis_gemv_list_workspace_bytes([base[n] for n in names], 1), dtype=torch.uint8,
                     device="cuda")

    def step(i):
        tb.trellis_gemv_list([copies[i % R][n] for n in names], xs, ys, ws=ws)

    ms_step = _time_steps(torch, step, R, args.warmup, args.steps, "dense")
    launch_us = _per_launch_us(torch, step, R, max(2, args.steps // R))

    def chain(i):  # gate+up (shared x) in one launch, then down
        c = copies[i % R]
        tb.trellis_gemv_list([c["gate"], c["up"]], xs[:2], ys[:2], ws=ws)
        tb.trellis_gemv_list([c["down"]], xs[2:], ys[2:], ws=ws)

    ms_chain = _time_steps(torch, chain, R, args.warmup, args.steps, "dense_chain")
    achieved = code_bytes / (launch_us * 1e-6) / 1e9
    value = code_bytes / (ms_step * 1e-3) / 1e9
    ceiling = decode_ceiling(tb, weights / code_bytes)
    out = {
        "metric": "trellis GEMV code-bytes GB/s (% HBM peak) at batch 1; prefill TFLOP/s",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "dense MLP decode, batch 1: gate K2 5120x17408 + up K3 5120x17408 + down K3 "
                               "17408x5120, each on its own x, as one trellis_gemv_list launch per step; steps over "
                               f"{R} weight copies captured as consecutive layers in HIP graphs",
                   "global_batch": 1, "code_bytes_per_step": code_bytes, "weight_copies_rotated": R,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic()},
        "roofline_kernel": "gemv_kernel<list, mixed K> (the step's one launch)",
        "algorithmic_bytes_per_launch": code_bytes,
        "launch_us": round(launch_us, 2),
        "decode_alu_ceiling": {**ceiling, "frac_of_it": round(achieved / ceiling["GBps"], 4)},
        "hbm_frac_of_step": round(value / HBM_PEAK_GBS, 4),
        "effective_weight_tflops": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "dependent_chain": {"ms_per_step": round(ms_chain, 5),
                            "code_GBps": round(code_bytes / (ms_chain * 1e-3) / 1e9, 1),
                            "what": "gate+up as one launch, then down (two launches), as in a model's MLP"},
    }
    return out, wl


def run_single(args, torch, tb, synth):
    """The single-matrix workload (K2 512 -> 256, s = 1): latency of one trellis_gemv."""
    wl = synth.single_k2(args.seed)
    lin = tb.TrellisLinear.from_host(wl.layers["w"])
    x = torch.from_numpy(wl.xs["w"]).cuda()
    y = torch.empty((1, lin.out_features), dtype=torch.float16, device="cuda")
    ws = torch.zeros(lin.workspace_bytes(tb.TRELLIS_OP_GEMV, 1), dtype=torch.uint8, device="cuda")
    us = _per_launch_us(torch, lambda i: tb.trellis_gemv(lin, x, out=y, ws=ws), 64, 20)
    return {"workload": "single matrix K2 512x256, s = 1, batch 1 (trellis_gemv)", "us_per_call": round(us, 2),
            "code_bytes": wl.layers["w"].code_bytes}


def run_prefill(args, torch, tb, synth, fp8=False):
    """trellis_gemm (fp16 matrix cores) or, with fp8, trellis_gemm_fp8 on the E4M3 variant
    of the same codes (cb = 2; activations quantised per row to E4M3)."""
    wl = synth.prefill(args.seed)
    lin = wl.layers["w"]
    L = tb.TrellisLinear.from_host(lin)
    if fp8:
        L = tb.TrellisLinear(L.code, L.rin, L.rout, L.s_in, L.s_out, L.K, cb=2)
    fn = tb.trellis_gemm_fp8 if fp8 else tb.trellis_gemm
    x = torch.from_numpy(wl.xs["w"]).cuda()
    y = torch.empty((x.shape[0], lin.out_features), dtype=torch.float16, device="cuda")
    _ramp(torch, lambda: fn(L, x, out=y), "prefill_fp8" if fp8 else "prefill")
    for _ in range(max(10, args.warmup)):
        fn(L, x, out=y)
    torch.cuda.synchronize()
    n = max(10, args.steps // 2)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        fn(L, x, out=y)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / n
    flops = 2.0 * x.shape[0] * lin.in_features * lin.out_features
    tf = flops / (ms * 1e-3) / 1e12
    if fp8:
        return {"workload": "FP8 prefill (trellis_gemm_fp8): E4M3 codebook K3 5120x17408, M=2048, E4M3 activations "
                            "with per-row scales", "ms": round(ms, 4), "tflops": round(tf, 1),
                "frac_of_fp8_mfma_peak": round(tf / MFMA_F8_PEAK_TFLOPS, 4)}
    return {"workload": "prefill K3 5120x17408, M=2048", "ms": round(ms, 4), "tflops": round(tf, 1),
            "frac_of_fp16_mfma_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}


def run_small_batch(args, torch, tb, synth, B):
    """Small-batch decode: the workload's three K2 matrices at batch B as one
    trellis_gemv_list launch per step."""
    wl = synth.small_batch(args.seed, batch=B)
    names = ["qkv", "z", "out"]
    code_bytes = sum(wl.layers[n].code_bytes for n in names)
    R = _copies(code_bytes)
    base = {n: tb.TrellisLinear.from_host(wl.layers[n]) for n in names}
    copies = _weight_copies(tb, base, R)
    xs = [torch.from_numpy(wl.xs[n]).cuda() for n in names]
    ys = [torch.empty((B, wl.layers[n].out_features), dtype=torch.float16, device="cuda") for n in names]
    ws = torch.zeros(tb.trellis_gemv_list_workspace_bytes([base[n] for n in names], B), dtype=torch.uint8,
                     device="cuda")

    def step(i):
        tb.trellis_gemv_list([copies[i % R][n] for n in names], xs, ys, ws=ws)

    ms = _time_steps(torch, step, R, args.warmup, args.steps, f"small_batch_B{B}")
    gbs = code_bytes / (ms * 1e-3) / 1e9
    return {"workload": f"small-batch decode K2 B={B} (qkv 5120x10240, z 5120x6144, out 6144x5120; one "
                        "trellis_gemv_list launch per step; consecutive steps over the weight copies in HIP graphs)",
            "B": B, "ms_per_step": round(ms, 5), "code_GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "effective_weight_tflops": round(2 * B * sum(wl.layers[n].in_features * wl.layers[n].out_features
                                                       for n in names) / (ms * 1e-3) / 1e12, 3)}


def run_moe(args, torch, tb, synth):
    """Per token: gate+up over the 8 routed experts (16 products, one launch, shared input
    vectors) and down (8 products, one launch); routes re-drawn every step over 256 experts."""
    layer = synth.moe_layer(args.seed)
    E = len(layer.K)
    dev = lambda l: tb.TrellisLinear.from_host(l)
    gate = [dev(layer.gate[e]) for e in range(E)]
    up = [dev(layer.up[e]) for e in range(E)]
    down = [dev(layer.down[e]) for e in range(E)]
    t_gu = tb.ExpertTable(gate + up, shared_side=0)
    t_d = tb.ExpertTable(down, shared_side=1)
    r_hi = torch.from_numpy(layer.r_hidden_in).cuda()
    s_hi = torch.from_numpy(layer.s_hidden_in).cuda()
    r_ho = torch.from_numpy(layer.r_hidden_out).cuda()
    s_ho = torch.from_numpy(layer.s_hidden_out).cuda()
    n_tok = args.warmup + args.steps + 64
    routes = synth.moe_routes(args.seed, n_tok)
    routes_gu = torch.from_numpy(np.concatenate([routes, routes + E], axis=1).astype(np.int32)).cuda()
    routes_d = torch.from_numpy(routes).cuda()
    xt, xd = synth.moe_token_inputs(args.seed)
    xt = torch.from_numpy(xt[0]).cuda()
    xd = torch.from_numpy(xd).cuda()
    y_gu = torch.empty((16, 2048), dtype=torch.float16, device="cuda")
    y_d = torch.empty((8, 6144), dtype=torch.float16, device="cuda")
    bytes_tok = [sum(layer.expert_code_bytes(int(e)) for e in r) for r in routes]

    nb = max(t_gu.workspace_bytes(16), t_d.workspace_bytes(8))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")

    def step(i):
        tb.trellis_moe_gemv(t_gu, routes_gu[i], xt, False, r_hi, s_hi, 0, out=y_gu, ws=ws)
        tb.trellis_moe_gemv(t_d, routes_d[i], xd, True, r_ho, s_ho, 1, out=y_d, ws=ws)

    for i in range(64):  # warm-up tokens route across most of the 256 experts
        step(i)
    torch.cuda.synchronize()
    # the timed tokens are captured in HIP graphs of 16 tokens each (every token its own
    # freshly drawn routes, read from device memory by the kernels)
    chunk = 16
    n_chunks = max(1, args.steps // chunk)
    graphs = [_capture(torch, lambda c=c: [step(64 + c * chunk + j) for j in range(chunk)]) for c in range(n_chunks)]
    _ramp(torch, graphs[0].replay, "moe")
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for g in graphs:
        g.replay()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / (n_chunks * chunk)
    args = argparse.Namespace(**{**vars(args), "steps": n_chunks * chunk})
    nb = float(np.mean(bytes_tok[64:64 + args.steps]))
    gbs = nb / (ms * 1e-3) / 1e9
    return {"workload": "MoE decode, 8 of 256 GLM-like experts, K in {2,3,4}: gate+up of the routed experts as one "
                        "trellis_moe_gemv launch (16 products, shared rotated input), down as one (8 products); "
                        "routes re-drawn every token; 16 tokens per HIP graph",
            "ms_per_token": round(ms, 5), "code_bytes_per_token": nb, "code_GBps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def run_moe_mlp(args, torch, tb, synth, cb=1):
    """The fused routed-expert MLP of one token (trellis_moe_mlp): gate/up over 16 per-half
    slices of each of the 8 routed experts, silu(g) * u, down, router-weighted sum with one
    output rotation.  Routes and router weights re-drawn every token over 256 experts.  The
    same token computed with the unfused calls (two trellis_moe_gemv launches, the
    activation and the weighted sum as torch ops) is timed beside it."""
    layer = synth.moe_mlp_layer(args.seed)
    E, H = len(layer.down), layer.halves
    if cb != 1:  # the same codes read through the E4M3 codebook (the EXLR8 experts' format)
        for e in range(E):
            for l in layer.gate[e] + layer.up[e] + [layer.down[e]]:
                l.cb = cb
    tables = tb.MoEMLPTables.from_host(layer)
    n_tok = args.warmup + args.steps + 64
    routes = synth.moe_routes(args.seed, n_tok)
    weights = synth.moe_router_weights(args.seed, n_tok)
    r_dev = torch.from_numpy(routes).cuda()
    w_dev = torch.from_numpy(weights).cuda()
    x = torch.from_numpy(synth.make_x(np.random.SeedSequence([args.seed, 0x4D4C58]), 1, layer.hidden)[0]).cuda()
    y = torch.empty(layer.hidden, dtype=torch.float16, device="cuda")
    ws = torch.zeros(tables.workspace_bytes(8), dtype=torch.uint8, device="cuda")
    bytes_tok = [sum(layer.expert_code_bytes(int(e)) for e in r) for r in routes]

    def step(i):
        tb.trellis_moe_mlp(tables, r_dev[i], w_dev[i], x, tables.r_hidden_in, tables.s_hidden_in,
                           tables.r_hidden_out, tables.s_hidden_out, out=y, ws=ws)

    # unfused: the same products through trellis_moe_gemv (gate/up slices of the routed
    # experts as one problem list), the activation and the weighted sum in torch
    slots = torch.arange(2 * H, dtype=torch.int32, device="cuda")
    routes_gu = (r_dev[:, :, None] * (2 * H) + slots[None, None, :]).reshape(n_tok, -1).contiguous()
    y_gu = torch.empty((8 * 2 * H, layer.inter // H), dtype=torch.float16, device="cuda")
    act = torch.empty((8, layer.inter), dtype=torch.float16, device="cuda")
    y_d = torch.empty((8, layer.hidden), dtype=torch.float16, device="cuda")
    ws_u = torch.zeros(max(tables.gate_up.workspace_bytes(16 * H), tables.down.workspace_bytes(8)),
                       dtype=torch.uint8, device="cuda")

    def step_unfused(i):
        tb.trellis_moe_gemv(tables.gate_up, routes_gu[i], x, False, tables.r_hidden_in, tables.s_hidden_in, 0,
                            out=y_gu, ws=ws_u)
        g = y_gu.view(8, 2, layer.inter).float()
        torch.mul(torch.nn.functional.silu(g[:, 0]), g[:, 1], out=act)
        tb.trellis_moe_gemv(tables.down, r_dev[i], act, True, tables.r_hidden_out, tables.s_hidden_out, 1,
                            out=y_d, ws=ws_u)
        torch.mm(w_dev[i][None, :].half(), y_d, out=y.view(1, -1))

    res = {}
    variants = (("fused", step),) if (args.no_unfused or cb != 1) else (("fused", step), ("unfused", step_unfused))
    for name, fn in variants:
        for i in range(64):  # warm-up tokens route across most of the 256 experts
            fn(i)
        torch.cuda.synchronize()
        chunk = 16
        n_chunks = max(1, args.steps // chunk)
        graphs = [_capture(torch, lambda c=c: [fn(64 + c * chunk + j) for j in range(chunk)]) for c in range(n_chunks)]
        _ramp(torch, graphs[0].replay, f"moe_mlp_{name}_cb{cb}")
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for g in graphs:
            g.replay()
        e.record()
        torch.cuda.synchronize()
        res[name] = s.elapsed_time(e) / (n_chunks * chunk)
        del graphs
    steps = n_chunks * chunk
    nb = float(np.mean(bytes_tok[64:64 + steps]))
    ms = res["fused"]
    return {"workload": "fused routed-expert MLP decode (trellis_moe_mlp), 8 of 256 GLM-like experts, hidden 6144, "
                        "intermediate 2048 as 16 gate/up halves per expert with per-half K in {2,3,4}, down K per "
                        "expert; routes and router weights re-drawn every token; 16 tokens per HIP graph; "
                        + ("MCG codebook" if cb == 1 else "E4M3 codebook (cb=2)"),
            "ms_per_token": round(ms, 5), "code_bytes_per_token": nb, "code_GBps": round(nb / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "unfused_ms_per_token": round(res["unfused"], 5) if "unfused" in res else None, "tokens_timed": steps}


def run_encode(args, torch, tb, synth):
    """trellis_encode_tiles on 2048 tiles of N(0, 1.24^2) targets (2 GiB of decisions),
    K = 2, 3, 4, MCG codebook; the oracle's float32 search timed beside it on a few tiles."""
    import oracle as O
    T = 2048
    rng = np.random.default_rng(args.seed)
    tgt_h = (rng.standard_normal((T, 16, 16)) * 1.24371088).astype(np.float32)
    tgt = torch.from_numpy(tgt_h).cuda()
    ws = torch.empty(tb.lib().trellis_encode_workspace_bytes(T), dtype=torch.uint8, device="cuda")
    out = {"workload": f"tail-biting Viterbi encode (trellis_encode_tiles), {T} tiles of 16x16 N(0, 1.24^2) targets, "
                       "MCG codebook", "per_K": {}}
    for K in (2, 3, 4):
        for _ in range(2):
            tb.trellis_encode_tiles(tgt, K, ws=ws)
        torch.cuda.synchronize()
        n = 3
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(n):
            tb.trellis_encode_tiles(tgt, K, ws=ws)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / n
        t0 = time.perf_counter()
        nt = 2
        O.viterbi_encode(tgt_h[:nt], K, dtype=np.float32)
        cpu_s = (time.perf_counter() - t0) / nt
        out["per_K"][K] = {"ms_per_call": round(ms, 3), "tiles_per_s": round(T / (ms * 1e-3), 1),
                           "weights_per_s": round(256 * T / (ms * 1e-3), 1),
                           "state_steps_per_s": round(2 * 256 * 65536 * T / (ms * 1e-3), 1),
                           "cpu_oracle_tiles_per_s": round(1.0 / cpu_s, 3)}
    return out


def run_kernels(args, torch, tb, synth):
    """The standalone entry points on the prefill matrix (K3 5120x17408) and activation
    shape (2048 x 5120), each against HBM: algorithmic bytes (read + written) per call."""
    wl = synth.prefill(args.seed)
    lin = wl.layers["w"]
    code = torch.from_numpy(lin.code).cuda()
    x = torch.from_numpy(wl.xs["w"]).cuda()
    r = torch.from_numpy(lin.rin).cuda()
    sc = torch.from_numpy(lin.s_in).cuda()
    y = torch.empty_like(x)

    def timed(fn, n=20):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(n):
            fn()
        e0.record()
        torch.cuda.synchronize()
        return s0.elapsed_time(e0) / n

    out = {"workload": "standalone entry points: decode of K3 5120x17408 tiles; had128_scale of fp16 [2048, 5120]"}
    code_b = lin.code_bytes
    for name, fn, nbytes in [
        ("trellis_decode_tiles", lambda: tb.trellis_decode_tiles(code, lin.K), code_b + 5120 * 17408 * 2),
        ("trellis_decode_tiles_e4m3", lambda: tb.trellis_decode_tiles_e4m3(code, lin.K), code_b + 5120 * 17408),
        ("had128_scale", lambda: tb.had128_scale(x, r, sc, out=y), 2 * x.numel() * 2 + 5120 * 6),
    ]:
        ms = timed(fn)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 4), "bytes": nbytes, "GBps": round(gbs, 1), "frac_of_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def run_micro(args, torch, tb):
    """The hardware ceilings: cold HBM stream read, vector-instruction issue costs of the
    decode (single instructions and whole per-tile sequences), matrix-instruction rates.
    Clocks are the shader clock (s_memtime); its frequency under each load is reported."""
    out = {"workload": "microbenchmarks: HBM stream read, decode vector-instruction costs, MFMA rates"}
    # cold stream read: 8 GiB (32x the Infinity Cache), 16-byte loads from every CU
    nbytes = 8 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    tb.micro_stream_read(buf)
    torch.cuda.synchronize()
    rates = []
    for blocks in (0, 2048, 4096):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(4):
            tb.micro_stream_read(buf, blocks)
        e1.record()
        torch.cuda.synchronize()
        rates.append((nbytes * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9, blocks))
    best = max(rates)
    out["hbm_stream_read_GBps"] = round(best[0], 1)
    out["hbm_stream_read_frac_of_8TBps"] = round(best[0] / HBM_PEAK_GBS, 4)
    out["hbm_stream_read_by_grid"] = {str(b or "8/CU"): round(r, 1) for r, b in rates}
    del buf
    torch.cuda.empty_cache()
    _log(f"stream read {best[0]:.0f} GB/s")

    simds = 4 * tb.micro_cus()

    def clk(kind, name, iters, wps, per):
        """Per SIMD: wall-clock ns per wave instruction (or tile) over the whole launch, and
        that in shader clocks at the frequency measured in the kernel (s_memtime cycles over
        the 100 MHz s_memrealtime ticks)."""
        tb.micro_clock_kernel(kind, name, 4, wps)  # warm-up
        cyc, tick, ms = tb.micro_clock_kernel(kind, name, iters, wps)
        ghz = float((cyc.double() / (tick.double() * 10.0)).median())
        per_simd = wps * iters * per  # wave instructions (or tiles) each SIMD executes
        ns = ms * 1e6 / per_simd
        return ns * ghz, ghz, ns

    valu = {}
    for name in tb.MICRO_VALU:
        row = {}
        for wps in (1, 2, 4, 8):
            c, ghz, _ = clk("valu", name, 20000, wps, 64)
            row[f"w{wps}"] = round(c, 3)
        row["ghz"] = round(ghz, 3)
        valu[name] = row
    out["valu_clocks_per_wave_instruction_per_simd"] = valu
    dec = {}
    for name in tb.MICRO_DECODE:
        row = {}
        for wps in (1, 2, 4, 8):
            c, ghz, _ = clk("valu", name, 4000, wps, 16)
            row[f"w{wps}"] = round(c, 2)
        row["ghz"] = round(ghz, 3)
        dec[name] = row
    out["decode_clocks_per_tile_per_simd"] = dec
    mf = {}
    for name, (_, macs) in tb.MICRO_MFMA.items():
        row = {}
        for wps in (1, 2, 4):
            c, ghz, ns = clk("mfma", name, 4000, wps, 8)
            row[f"w{wps}_clocks"] = round(c, 2)
            row[f"w{wps}_tflops"] = round(2 * macs / ns * simds / 1e3, 1)
            row[f"w{wps}_ghz"] = round(ghz, 3)
        mf[name] = row
    out["mfma"] = mf
    out["cus"] = tb.micro_cus()
    out["method"] = ("wall time of one launch (events) over the instructions each SIMD issues; clocks at "
                     "the in-kernel s_memtime/s_memrealtime frequency")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="dense", choices=["dense", "small_batch", "moe", "moe_mlp", "prefill", "encode", "kernels", "micro"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="dense: skip the single, small-batch, MoE and fused-MLP lines")
    ap.add_argument("--no-unfused", action="store_true", help="moe_mlp: time only the fused call")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the kernels run one GPU's share of a sharded layer)", file=sys.stderr)
        sys.exit(2)

    import torch
    from trellis_coded_bit_amd import binding as tb
    from trellis_coded_bit_amd import synth
    tb.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.workload == "dense":
        out, wl = run_dense(args, torch, tb, synth)
        if not args.no_extra:
            out["single"] = run_single(args, torch, tb, synth)
            out["small_batch"] = [run_small_batch(args, torch, tb, synth, B) for B in (1, 2, 4, 8)]
            out["moe"] = run_moe(args, torch, tb, synth)
            torch.cuda.empty_cache()
            out["moe_mlp"] = [run_moe_mlp(args, torch, tb, synth), run_moe_mlp(args, torch, tb, synth, cb=2)]
            torch.cuda.empty_cache()
        if not args.no_prefill:
            out["prefill"] = run_prefill(args, torch, tb, synth)
            out["prefill_fp8"] = run_prefill(args, torch, tb, synth, fp8=True)
        if args.copy_probe:
            out["copy_probe"] = copy_probe(torch)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_dense(wl)
        out["clock_ramp"] = RAMP
        print(json.dumps(out), flush=True)
    elif args.workload == "small_batch":
        for B in (1, 2, 4, 8):
            print(json.dumps(run_small_batch(args, torch, tb, synth, B)), flush=True)
    elif args.workload == "moe":
        print(json.dumps(run_moe(args, torch, tb, synth)), flush=True)
    elif args.workload == "moe_mlp":
        print(json.dumps(run_moe_mlp(args, torch, tb, synth)), flush=True)
        print(json.dumps(run_moe_mlp(args, torch, tb, synth, cb=2)), flush=True)
    elif args.workload == "encode":
        print(json.dumps(run_encode(args, torch, tb, synth)), flush=True)
    elif args.workload == "kernels":
        print(json.dumps(run_kernels(args, torch, tb, synth)), flush=True)
    elif args.workload == "micro":
        print(json.dumps(run_micro(args, torch, tb)), flush=True)
    else:
        print(json.dumps(run_prefill(args, torch, tb, synth)), flush=True)
        print(json.dumps(run_prefill(args, torch, tb, synth, fp8=True)), flush=True)


if __name__ == "__main__":
    main()
