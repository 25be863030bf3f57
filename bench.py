"""Benchmark of the trellis-coded GEMV hot path on one MI355X.

Default workload: the dense-MLP decode step at batch 1 (gate K2 5120->17408, up K3
5120->17408, down K3 17408->5120), i.e. three fused trellis_gemv launches per step.
Metric: code bytes (in*out*K/8 summed over the three matrices) per second.

Weights are rotated over enough distinct device copies (> 1 GiB in total) that the 256 MB
Infinity Cache cannot serve them between steps; inputs are resident in HBM before timing.

Prints ONE JSON line (rank 0, N = 1).  Extra workloads (small-batch, MoE, the fused
routed-expert MLP, prefill) are available with --workload for separate measurement lines.
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
# Vector-ALU bound of the codebook decode: 1024 SIMDs at 2.4 GHz; per wave64 of 4 weights
# per lane (256 weights) the hash needs 4 window extractions and 4 32-bit multiplies (half
# lane rate: 4 clocks each) and 4 mask-xors (full rate: 2 clocks each) = 40 clocks.
DECODE_PEAK_WEIGHTS_PER_S = 1024 * 2.4e9 * 256 / 40
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


def run_dense(args, torch, tb, synth):
    """The dense-MLP decode step: gate and up share their input, so they run as one launch
    over a two-entry layer table (trellis_moe_gemv, per-entry K); down is one trellis_gemv."""
    wl = synth.dense_mlp(args.seed, batch=1)
    names = ["gate", "up", "down"]
    code_bytes = sum(wl.layers[n].code_bytes for n in names)
    gu_bytes = wl.layers["gate"].code_bytes + wl.layers["up"].code_bytes
    flops = sum(2 * wl.layers[n].in_features * wl.layers[n].out_features for n in names)
    R = _copies(code_bytes)
    _log(f"dense MLP: {code_bytes / 1e6:.2f} MB code per step, {R} weight copies")
    base = {n: tb.TrellisLinear.from_host(wl.layers[n]) for n in names}
    copies = [base] + [{n: tb.TrellisLinear(base[n].code.clone(), base[n].rin, base[n].rout, base[n].s_in,
                                            base[n].s_out, base[n].K) for n in names} for _ in range(R - 1)]
    tables = [tb.ExpertTable([c["gate"], c["up"]]) for c in copies]
    routed = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    assert np.array_equal(wl.xs["gate"], wl.xs["up"])
    x_gu = torch.from_numpy(wl.xs["gate"][0]).cuda()
    x_d = torch.from_numpy(wl.xs["down"]).cuda()
    y_gu = torch.empty((2, 17408), dtype=torch.float16, device="cuda")
    y_d = torch.empty((1, 5120), dtype=torch.float16, device="cuda")
    nb = max(base["down"].workspace_bytes(tb.TRELLIS_OP_GEMV, 1), tables[0].workspace_bytes(2))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")

    def gate_up(i):
        tb.trellis_moe_gemv(tables[i % R], routed, x_gu, False, out=y_gu, ws=ws)

    def down(i):
        tb.trellis_gemv(copies[i % R]["down"], x_d, out=y_d, ws=ws)

    def step(i):
        gate_up(i)
        down(i)

    # eager warm-up, then HIP graphs of consecutive steps over the weight copies (R steps per
    # graph: the MLPs of R layers in a row, as in one captured decode pass of a model)
    for i in range(R):
        step(i)
    torch.cuda.synchronize()
    stack = LayerStack(torch, step, R)
    stack.prepare(args.warmup, args.steps)
    stack.run(args.warmup)
    torch.cuda.synchronize()
    t_s = torch.cuda.Event(enable_timing=True)
    t_e = torch.cuda.Event(enable_timing=True)
    t_s.record()
    stack.run(args.steps)
    t_e.record()
    torch.cuda.synchronize()
    ms_step = t_s.elapsed_time(t_e) / args.steps
    # per-launch duration of each launch (its two kernels): a graph of R back-to-back launches
    launch_us = {}
    for name, fn in [("gate_up", gate_up), ("down", down)]:
        g = _capture(torch, lambda fn=fn: [fn(i) for i in range(R)])
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(2, args.steps // R)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        launch_us[name] = e0.elapsed_time(e1) * 1e3 / (reps * R)
    # the dominant kernel: the gate+up launch (the larger share of the step)
    achieved = gu_bytes / (launch_us["gate_up"] * 1e-6) / 1e9
    gu_weights = sum(wl.layers[n].in_features * wl.layers[n].out_features for n in ("gate", "up"))
    alu_peak_gbs = DECODE_PEAK_WEIGHTS_PER_S * (gu_bytes / gu_weights) / 1e9
    value = code_bytes / (ms_step * 1e-3) / 1e9
    out = {
        "metric": "trellis GEMV code-bytes GB/s (% HBM peak) at batch 1; prefill TFLOP/s",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "dense MLP decode, batch 1: gate K2 5120x17408 + up K3 5120x17408 (one "
                               "trellis_moe_gemv launch over a 2-entry table, shared x) + down K3 17408x5120 "
                               "(trellis_gemv); steps over 13 weight copies captured as consecutive layers in HIP graphs",
                   "global_batch": 1, "code_bytes_per_step": code_bytes, "weight_copies_rotated": R,
                   "parallelism": "single GPU"},
        # the launch is bound by the decode's vector-ALU work, not by HBM: its peak is the
        # decode bound above, in code bytes per second for this launch's mix of widths
        "roofline": {"bound": "alu", "achieved": round(achieved, 1), "peak": round(alu_peak_gbs, 1), "unit": "GB/s",
                     "frac": round(achieved / alu_peak_gbs, 4), "traffic": measured_traffic()},
        "roofline_hbm": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4)},
        "roofline_kernel": "gate+up launch (gemv_partial_kernel + gemv_finish_kernel over 2 problems)",
        "algorithmic_bytes_per_launch": gu_bytes,
        "hbm_frac_of_step": round(value / HBM_PEAK_GBS, 4),
        "effective_weight_tflops": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "launch_us": {k: round(v, 2) for k, v in launch_us.items()},
    }
    return out, wl


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
    for _ in range(max(10, args.warmup)):  # also lets the clocks settle under the MFMA load
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
    wl = synth.small_batch(args.seed, batch=B)
    names = ["qkv", "z", "out"]
    code_bytes = sum(wl.layers[n].code_bytes for n in names)
    R = _copies(code_bytes)
    base = {n: tb.TrellisLinear.from_host(wl.layers[n]) for n in names}
    copies = [base] + [{n: tb.TrellisLinear(base[n].code.clone(), base[n].rin, base[n].rout, base[n].s_in,
                                            base[n].s_out, base[n].K) for n in names} for _ in range(R - 1)]
    xs = {n: torch.from_numpy(wl.xs[n]).cuda() for n in names}
    ys = {n: torch.empty((B, wl.layers[n].out_features), dtype=torch.float16, device="cuda") for n in names}

    nb = max(base[n].workspace_bytes(tb.TRELLIS_OP_GEMV, B) for n in names)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")

    def step(i):
        for n in names:
            tb.trellis_gemv(copies[i % R][n], xs[n], out=ys[n], ws=ws)

    # HIP graphs of consecutive steps over the weight copies (as for the dense step)
    for i in range(R):
        step(i)
    torch.cuda.synchronize()
    stack = LayerStack(torch, step, R)
    stack.prepare(args.warmup, args.steps)
    stack.run(args.warmup)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    stack.run(args.steps)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    return {"workload": f"small-batch decode K2 B={B} (qkv 5120x10240, z 5120x6144, out 6144x5120; "
                        "three trellis_gemv per step; consecutive steps over the weight copies in HIP graphs)", "ms_per_step": round(ms, 5),
            "code_GBps": round(code_bytes / (ms * 1e-3) / 1e9, 1),
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
    graphs[0].replay()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for g in graphs:
        g.replay()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / (n_chunks * chunk)
    args = argparse.Namespace(**{**vars(args), "steps": n_chunks * chunk})
    nb = float(np.mean(bytes_tok[64:64 + args.steps]))
    return {"workload": "MoE decode, 8 of 256 GLM-like experts, K in {2,3,4}", "ms_per_token": round(ms, 5),
            "code_bytes_per_token": nb, "code_GBps": round(nb / (ms * 1e-3) / 1e9, 1)}


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
        graphs[0].replay()
        torch.cuda.synchronize()
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="dense", choices=["dense", "small_batch", "moe", "moe_mlp", "prefill", "encode", "kernels"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
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
        if not args.no_prefill:
            out["prefill"] = run_prefill(args, torch, tb, synth)
            out["prefill_fp8"] = run_prefill(args, torch, tb, synth, fp8=True)
        if args.copy_probe:
            out["copy_probe"] = copy_probe(torch)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline_dense(wl)
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
    else:
        print(json.dumps(run_prefill(args, torch, tb, synth)), flush=True)
        print(json.dumps(run_prefill(args, torch, tb, synth, fp8=True)), flush=True)


if __name__ == "__main__":
    main()
