"""Benchmark: forward pass of one sparse MoE FFN layer on one MI355X.

Default workload: the MoE++-shaped layer, the largest of the five measured
shapes (T=8192 tokens, d=2048, 16 SwiGLU experts of inner width 5632 plus a
zero, a copy and two constant experts, top-2, tau=0.75, bf16, fp32 router).
A step is one moe_forward over the batch (route -> dispatch -> grouped
GEMM1+SiLU gate -> grouped GEMM2 -> combine), inputs resident in HBM.
Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (datasheet)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (datasheet)
METRIC = "MoE layer tokens/sec at 1 GPU; % of bf16 MFMA peak or HBM GB/s"
COPY_BYTES = 1 << 30
COLD_BYTES = 512 << 20         # read before each cold step: twice the 256 MB MALL
PROFILES = os.path.join(ROOT, "profiles")


def measured_traffic(workload, kernel):
    """HBM bytes per launch of a stage kernel from the committed counter
    summary of the workload (one record, or a list under "records"), or
    None if there is none for the kernel or its source changed since."""
    from mixture_experts_layer_22_amd import profiling as P
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    for rec in data.get("records", [data]):
        if rec.get("kernel") == kernel and rec.get("source_sha256") == P.kernel_source_sha(kernel):
            return rec.get("bytes")
    return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_work(cfg, counts):
    """Per-launch algorithmic FLOPs of each expert stage and the bytes each
    stage kernel must move at the least (each touched expert's weights once,
    the tokens once, its outputs once)."""
    T, d = cfg.T, cfg.d
    es = 2 if cfg.dtype == 1 else 4
    rows_s = T * cfg.n_shared * cfg.f_shared     # shared experts' H columns x tokens
    sh_w = cfg.n_shared * d * cfg.f_shared * es  # one shared weight matrix set, per matrix
    if cfg.router == 1:
        n = T * cfg.k
        touched = int(np.count_nonzero(counts))
        return {
            "expert1_flop": 2.0 * d * n + 4.0 * d * rows_s,
            "expert2_flop": 2.0 * d * n + 2.0 * d * rows_s,
            "weight_bytes": 2 * touched * d * es + 3 * sh_w,
            # k_atomic_h: each touched in-vector and each token once, one
            # fp32 activation per task
            "atomic_h_bytes": (touched + T) * d * es + n * 4,
            # k_atomic_combine: each touched out-vector once, the output, and
            # per task its expert id, gate, sorted position and activation
            "atomic_combine_bytes": (touched + T * (2 if cfg.n_shared else 1)) * d * es
                                    + n * 16,
            # what the combine's row loads request: every task's out-vector
            "atomic_gather_bytes": n * d * es,
            "gemm1_flop": 4.0 * d * rows_s,
            "gemm2_flop": 2.0 * d * rows_s,
        }
    n_ffn = int(np.sum(counts[:cfg.E_ffn]))
    touched = int(np.count_nonzero(counts[:cfg.E_ffn]))
    rows_f = n_ffn * cfg.f + rows_s
    return {
        "expert1_flop": 4.0 * d * rows_f,
        "expert2_flop": 2.0 * d * rows_f,
        "gemm1_flop": 4.0 * d * rows_f,
        "gemm2_flop": 2.0 * d * rows_f,
        "weight_bytes": touched * 3 * d * cfg.f * es + 3 * sh_w,
        # the gated GEMM's operands: weights of touched experts, the tokens,
        # its output H
        "gemm1_bytes": ((touched * 2 * d * cfg.f + cfg.n_shared * 2 * d * cfg.f_shared) + T * d
                        + n_ffn * cfg.f + rows_s) * es,
        # the down projection: its weights, H, and its outputs Y (routed rows
        # and the shared experts' sum)
        "gemm2_bytes": ((touched * d * cfg.f + cfg.n_shared * d * cfg.f_shared) + n_ffn * cfg.f
                        + rows_s + (n_ffn + (T if cfg.n_shared else 0)) * d) * es,
    }


def stage_kernels(cfg):
    """(phase, kernel, bound, work key) of each expert-stage kernel the
    layer launches, in launch order."""
    out = []
    if cfg.router == 1:
        t = "unsigned short" if cfg.dtype == 1 else "float"
        out.append(("atomic", f"k_atomic_h<{t}>", "hbm", "atomic_h_bytes"))
        if cfg.n_shared:
            out.append(("gemm1", "k_gemm_dl<true>", "mfma", "gemm1_flop"))
            out.append(("gemm2", "k_gemm_dl<false>", "mfma", "gemm2_flop"))
        u = next(v for v in (1, 2, 4, 8, 16) if cfg.d <= 512 * v)  # 16-byte units per lane
        out.append(("combine", f"k_atomic_combine<{t}, {u}>", "hbm", "atomic_combine_bytes"))
        return out
    if cfg.dtype != 1:
        return [("gemm1", "k_grouped_gemm_f32<true>", "hbm", "gemm1_bytes"),
                ("gemm2", "k_grouped_gemm_f32<false>", "hbm", "gemm2_bytes")]
    if cfg.T * cfg.k / max(cfg.E_ffn, 1) < 64:
        # decode-sized: the GEMMs stream their weights
        return [("gemm1", "k_grouped_gemm_bf16<1, 4, 1, 2, true>", "hbm", "gemm1_bytes"),
                ("gemm2", "k_grouped_gemm_bf16<1, 4, 1, 2, false>", "hbm", "gemm2_bytes")]
    return [("gemm1", "k_gemm_dl<true>", "mfma", "gemm1_flop"),
            ("gemm2", "k_gemm_dl<false>", "mfma", "gemm2_flop")]


def rooflines(cfg, work, phase_warm, phase_cold):
    """One roofline record per expert-stage kernel.  An HBM-bound kernel is
    rated on steps that each follow a 512 MiB read (nothing of the layer in
    the MALL or the L2s); an MFMA-bound one on warm steps (its weights
    exceed the MALL anyway); both fractions are kept.  The headline record
    is the kernel with the longest measured phase."""
    recs = []
    for phase, kern, bound, key in stage_kernels(cfg):
        w_us, c_us = phase_warm[phase], phase_cold[phase]
        if bound == "hbm":
            peak, unit, scale = PEAK_HBM_GBS, "GB/s", 1e9
        else:
            peak, unit, scale = PEAK_BF16_TFLOPS, "TFLOP/s", 1e12
        ach_w = work[key] / (w_us * 1e-6) / scale if w_us > 0 else 0.0
        ach_c = work[key] / (c_us * 1e-6) / scale if c_us > 0 else 0.0
        ach = ach_c if bound == "hbm" else ach_w
        recs.append({"bound": bound, "kernel": kern, "phase": phase,
                     "timing": "cold" if bound == "hbm" else "warm",
                     "us": c_us if bound == "hbm" else w_us,
                     "achieved": ach, "peak": peak, "unit": unit, "frac": ach / peak,
                     "frac_warm": ach_w / peak, "frac_cold": ach_c / peak,
                     "work": work[key], "work_unit": "B" if bound == "hbm" else "FLOP",
                     "traffic": measured_traffic(cfg.name, kern)})
    head = max(recs, key=lambda r: r["us"])
    return head, recs


def host_cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, budget_s=12.0):
    """Time the CPU oracle, single-threaded and pinned to one host core, on
    batches of the same workload until ~budget_s of CPU work; returns
    tokens/s and the sample description.  The oracle runs as it stands
    (numpy, float64); only its BLAS thread pool is limited to one thread and
    the process is pinned to one core for the duration."""
    from oracle import moe_oracle as O
    from threadpoolctl import threadpool_limits
    prev = os.sched_getaffinity(0)
    core = min(prev)
    n_tok = min(cfg.T, 256)
    done, batches = 0, 0
    try:
        os.sched_setaffinity(0, {core})
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            while True:
                lo = (batches * n_tok) % cfg.T
                sub = dict(inp)
                sub["x"] = inp["x"][lo:lo + n_tok]
                O.forward(cfg.replace(T=sub["x"].shape[0]), sub)
                done += sub["x"].shape[0]
                batches += 1
                el = time.perf_counter() - t0
                if el >= budget_s:
                    break
    finally:
        os.sched_setaffinity(0, prev)
    return {"value": done / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "host_cpu": host_cpu_model(), "pinned_core": core,
            "sample": f"{batches} batches of {n_tok} tokens of the same layer "
                      f"({done} tokens, {el:.1f} s), full layer per batch (route, dispatch, "
                      "experts, combine), numpy float64 with one BLAS thread"}


TAUS = (1.0, 0.75, 0.5, 0.25, 0.1)


class Evictor:
    """Cold caches before a step: a streaming read of a 512 MiB buffer of
    its own (twice the 256 MB MALL), so none of the layer's data is left in
    the MALL or the L2s.  A read, not a write: a written buffer would leave
    about 256 MB of dirty lines whose write-back then competes with the
    step's own reads (measured: a 509 MB weight stream ran 147-160 us after
    a 512 MiB write and 90-104 us after a 512 MiB read, as warm)."""

    def __init__(self, torch, B, stream, dev):
        self.B, self.stream = B, stream
        self.n = COLD_BYTES // 4
        self.buf = torch.ones(self.n, dtype=torch.float32, device=dev)
        self.sums = torch.empty(4096, dtype=torch.float32, device=dev)
        self()                      # the fill's dirty lines go out here
        torch.cuda.synchronize()

    def __call__(self, i=0):
        self.B.moe_probe_stream_read(self.buf, self.n, self.sums, 4096, self.stream)


def traced_phases(torch, B, stream, step_traced, n, evict=None):
    """Mean device time of each phase (us) over n steps bracketed by the
    library's phase events, recorded on the stream the kernels run on.  With
    `evict` (an Evictor), each step starts with cold caches."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(B.MOE_N_PHASES + 1)]
           for _ in range(n)]
    for row in evs:                     # materialise the lazily created events
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(n):
        if evict is not None:
            evict(i)
        step_traced(evs[i])
    torch.cuda.synchronize()
    return {name: 1e3 * float(np.mean([evs[i][p].elapsed_time(evs[i][p + 1])
                                       for i in range(n)]))
            for p, name in enumerate(B.PHASES)}


def expert_stage_us(ph):
    return ph["atomic"] + ph["gemm1"] + ph["gemm2"]


def tau_sweep(args, torch, B, I):
    """MoE++ "Measured effects": a smaller tau sends more tokens to the zero-
    computation experts, so the FFN experts' share of the tasks and the expert
    stage's time fall.  Same weights and tokens at every tau."""
    base = I.CONFIGS["moepp"]
    inp = I.make_inputs(base)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    x = B.to_device(inp["x"], dev)
    T = base.T
    stream = torch.cuda.current_stream()
    ref_us = None
    for tau in TAUS:
        cfg = base.replace(tau=tau)
        layer = B.MoELayer(cfg, inp, dev)
        out = torch.empty((T, cfg.d), dtype=layer.act_dtype, device=dev)
        ws = layer.workspace(T)
        idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
        gate = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            B.moe_forward(layer.dims, layer.weights, x, T, out, ws, idx, gate, stream)
        torch.cuda.synchronize()
        counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=cfg.E)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            B.moe_forward(layer.dims, layer.weights, x, T, out, ws, idx, gate, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        ph = traced_phases(torch, B, stream, lambda ev: B.moe_forward_traced(
            layer.dims, layer.weights, x, T, out, ws, ev, idx, gate, stream),
            max(1, min(args.steps, 10)))
        expert_us = expert_stage_us(ph)
        if ref_us is None:
            ref_us = expert_us
        print(json.dumps({
            "metric": "moepp_tau_sweep", "tau": tau,
            "ffn_task_share": float(counts[:cfg.E_ffn].sum()) / (T * cfg.k),
            "ms_per_step": ms, "tokens_per_s": T / (ms * 1e-3),
            "expert_stage_us": expert_us,
            "expert_stage_speedup_vs_tau1": ref_us / expert_us,
            "phases_us": ph, "config": {"workload": "moepp", "T": T, "steps": args.steps}}),
            flush=True)
        del layer, ws, out


def token_centric_ablation(args, torch, B, I):
    """OmniMoE sec. 2.2 / sec. 4: expert-centric scheduling (dispatch, then
    per-expert activations, then the gathered down projection) against the
    token-centric form (each token gathers its own experts' vectors).  Both
    start from the same routing; the times compared are everything after it."""
    cfg = I.CONFIGS["atomic-pk"]
    inp = I.make_inputs(cfg)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    layer = B.MoELayer(cfg, inp, dev)
    x = B.to_device(inp["x"], dev)
    T = cfg.T
    stream = torch.cuda.current_stream()
    out = torch.empty((T, cfg.d), dtype=layer.act_dtype, device=dev)
    ws = layer.workspace(T)
    idx, gate = layer.route(x)
    for _ in range(args.warmup):
        B.moe_forward(layer.dims, layer.weights, x, T, out, ws, stream=stream)
        B.moe_ablation_atomic_token_centric(layer.dims, layer.weights, x, T, idx, gate, out,
                                            stream)
    torch.cuda.synchronize()
    # expert-centric: the kernels after routing through the stage entry
    # points (dispatch, activations, combine: the same launches as the
    # forward's, without phase markers); the phases of traced forwards
    # are reported beside it
    ph = traced_phases(torch, B, stream, lambda ev: B.moe_forward_traced(
        layer.dims, layer.weights, x, T, out, ws, ev, stream=stream), max(1, min(args.steps, 20)))
    n = T * cfg.k
    counts = torch.empty(cfg.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(cfg.E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    inv = torch.empty(n, dtype=torch.int32, device=dev)
    h = torch.empty(n, dtype=torch.float32, device=dev)

    def expert_centric():
        B.moe_dispatch(layer.dims, idx, T, counts, offsets, perm, inv, ws, stream)
        B.moe_expert_ffn(layer.dims, layer.weights, x, T, idx, perm, offsets, h, None, ws,
                         stream)
        B.moe_combine(layer.dims, layer.weights, x, T, idx, gate, inv, h, None, out, stream)

    def token_centric():
        B.moe_ablation_atomic_token_centric(layer.dims, layer.weights, x, T, idx, gate, out,
                                            stream)

    def per_step_us(fn):
        for _ in range(3):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / args.steps

    ec_us = per_step_us(expert_centric)
    tc_us = per_step_us(token_centric)
    print(json.dumps({
        "metric": "atomic_expert_centric_vs_token_centric",
        "expert_centric_us": ec_us, "expert_centric_phases_us": ph,
        "token_centric_us": tc_us, "token_over_expert_time": tc_us / ec_us,
        "config": {"workload": cfg.name, "T": T, "d": cfg.d, "N": cfg.E, "k": cfg.k,
                   "steps": args.steps}}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU takes some tens of steps to reach its steady clocks and cache
    # state (measured: 20 timed steps after 5 warm-up ones run 6-8 % slower
    # than after 30); the timed region stays well under a second
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="moepp",
                    help="moepp (default, the largest layer), deepseek16b, qwen3-decode, "
                         "atomic-pk, tiny-fp32, or omnimoe (atomic-pk plus a shared MLP)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy a 1 GiB device buffer three times (counter calibration)")
    ap.add_argument("--ablation", action="store_true",
                    help="atomic layer: expert-centric library path against the token-centric "
                         "ablation kernel, one JSON line (not the bench line)")
    ap.add_argument("--tau-sweep", action="store_true",
                    help="MoE++ layer at several tau: one JSON line per tau with the FFN task "
                         "share and the layer / expert-stage times (not the bench line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this layer is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_layer_22_amd import binding as B
    from mixture_experts_layer_22_amd import inputs as I

    if args.calibrate_copy:
        # counter calibration: a device copy of COPY_BYTES (plain loads and
        # stores), then the same bytes streamed once through plain loads and
        # once through direct-to-LDS loads (the expert GEMM's load kind)
        n = COPY_BYTES // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        sums = torch.empty(1024, dtype=torch.float32, device="cuda:0")
        B.moe_probe_stream_read(src, n, sums, 1024)
        B.moe_probe_stream_read_lds(src, n, sums, 1024)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3,
                          "stream_reads": ["k_stream_read", "k_stream_read_lds"]}))
        return

    if args.tau_sweep:
        tau_sweep(args, torch, B, I)
        return
    if args.ablation:
        token_centric_ablation(args, torch, B, I)
        return

    cfg = I.CONFIGS[args.workload]
    log(f"[bench] workload {cfg.name}: generating inputs")
    inp = I.make_inputs(cfg)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    layer = B.MoELayer(cfg, inp, dev)
    x = B.to_device(inp["x"], dev)
    T = cfg.T
    out = torch.empty((T, cfg.d), dtype=layer.act_dtype, device=dev)
    ws = layer.workspace(T)
    idx = torch.empty((T, cfg.k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, cfg.k), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        B.moe_forward(layer.dims, layer.weights, x, T, out, ws, idx, gate, stream)

    def step_traced(events):
        B.moe_forward_traced(layer.dims, layer.weights, x, T, out, ws, events, idx, gate, stream)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=cfg.E)

    # timed region: K steps of the plain forward, inputs resident in HBM
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # phase breakdown: further steps bracketed by the library's phase events
    # (the markers add a little time of their own, so these steps are not
    # part of the timed region), warm and cold
    n_traced = max(1, min(args.steps, 20))
    log(f"[bench] traced steps {n_traced} warm, {n_traced} cold")
    phase_us = traced_phases(torch, B, stream, step_traced, n_traced)
    scratch = Evictor(torch, B, stream, dev)
    phase_cold_us = traced_phases(torch, B, stream, step_traced, n_traced, scratch)

    # per-step spread: steps bracketed one by one, warm, then cold (a 512 MiB
    # read before each step); the per-step events add a little time of
    # their own
    def step_times(n, evict=None):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for i, (a, b) in enumerate(ev):
            if evict is not None:
                evict(i)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        v = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        return {"median": float(np.median(v)), "p10": float(np.percentile(v, 10)),
                "p90": float(np.percentile(v, 90)), "steps": n}

    step_us = step_times(max(1, min(args.steps, 50)))
    cold_step_us = step_times(max(1, min(args.steps, 20)), scratch)
    del scratch

    # measured ceilings (libmoe_probes.so): a streaming read of 2 GiB and a
    # memory-free loop of the GEMM's MFMA, each the best of five runs
    def best_ms(fn):
        best = float("inf")
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b))
        return best

    log("[bench] ceilings")
    # read patterns over 2 GiB: one window moving over the buffer
    # (grid-stride), and every block streaming its own contiguous 1 MiB, with
    # plain and with non-temporal loads
    n_rd, rd_blocks = (2 << 30) // 4, 8192
    rd_buf = torch.ones(n_rd, dtype=torch.float32, device=dev)
    rd_sums = torch.empty(rd_blocks, dtype=torch.float32, device=dev)
    read_grid_gbs = n_rd * 4 / (best_ms(lambda: B.moe_probe_stream_read(
        rd_buf, n_rd, rd_sums, rd_blocks, stream)) * 1e-3) / 1e9
    n_bl = n_rd * 4 // (1 << 20)
    read_blocks_gbs = n_rd * 4 / (best_ms(lambda: B.moe_probe_stream_read_blocks(
        rd_buf, n_rd, rd_sums, n_bl, False, stream)) * 1e-3) / 1e9
    read_nt_gbs = n_rd * 4 / (best_ms(lambda: B.moe_probe_stream_read_blocks(
        rd_buf, n_rd, rd_sums, n_bl, True, stream)) * 1e-3) / 1e9
    read_gbs = max(read_grid_gbs, read_blocks_gbs, read_nt_gbs)
    del rd_buf, rd_sums
    gather_gbs = None
    if cfg.router == I.ROUTER_PRODUCT_KEY:
        # the atomic combine's reads alone: every token's k rows of the W
        # table, this step's routing, nothing else done with them
        aw = layer.weights.tensors["atom_w"]
        g_sums = torch.empty(T, dtype=torch.float32, device=dev)
        row_bytes = cfg.d * aw.element_size()
        gather_gbs = T * cfg.k * row_bytes / (best_ms(lambda: B.moe_probe_row_gather(
            aw, cfg.E, row_bytes, idx, T * cfg.k, cfg.k, g_sums, stream)) * 1e-3) / 1e9
        del g_sums
    mf_iters, mf_blocks = 4096, 512
    mf_out = torch.empty(mf_blocks, dtype=torch.float32, device=dev)
    mf_flop = 2.0 * 16 * 16 * 32 * 16 * 8 * mf_iters * mf_blocks
    mfma_tflops = mf_flop / (best_ms(lambda: B.moe_probe_mfma_loop(
        mf_iters, mf_out, mf_blocks, stream)) * 1e-3) / 1e12
    del mf_out

    # the expert GEMM's K-slice mix alone (one 8-wave block per CU): its
    # MFMAs, + the fragment reads from LDS, + the direct-to-LDS copies of
    # the next K tile from an L2-resident 2 MiB source (issued at the K
    # tile's start, or between the MFMA rows as in the GEMM)
    sl_iters, sl_blocks, sl_rows = 2000, 256, 16384
    sl_src = torch.ones(sl_rows * 64, dtype=torch.bfloat16, device=dev)
    sl_out = torch.empty(sl_blocks, dtype=torch.float32, device=dev)
    sl_flop = 2.0 * 16 * 16 * 32 * 64 * 8 * sl_iters * sl_blocks
    slice_tflops = {name: sl_flop / (best_ms(lambda m=m: B.moe_probe_gemm_slice(
        m, sl_src, sl_rows, sl_iters, sl_out, sl_blocks, stream)) * 1e-3) / 1e12
        for m, name in ((0, "mfma"), (1, "lds_reads"), (2, "lds_reads_copies_at_start"),
                        (3, "lds_reads_copies"))}
    del sl_src, sl_out

    work = algorithmic_work(cfg, counts)
    tokens_per_s = T / (ms_per_step * 1e-3)
    roof, stages = rooflines(cfg, work, phase_us, phase_cold_us)
    # beside the datasheet peaks: what this GPU streams and multiplies when
    # nothing else runs
    ceiling = {"hbm_read_gbs": read_gbs, "hbm_read_grid_stride_gbs": read_grid_gbs,
               "hbm_read_blocks_gbs": read_blocks_gbs, "hbm_read_nontemporal_gbs": read_nt_gbs,
               "mfma_bf16_tflops": mfma_tflops,
               "gemm_slice_tflops": slice_tflops,
               "frac_of_measured": roof["achieved"] / (read_gbs if roof["unit"] == "GB/s"
                                                       else mfma_tflops)}
    if roof["unit"] == "TFLOP/s":
        # against the same K-slice mix with its operands in L2
        ceiling["frac_of_gemm_slice"] = roof["achieved"] / slice_tflops["lds_reads_copies"]
    if gather_gbs is not None:
        # the combine's requested bytes (T k rows) against the same rows
        # gathered by the probe
        comb = [r for r in stages if r["phase"] == "combine"][0]
        ceiling["row_gather_gbs"] = gather_gbs
        ceiling["combine_requested_gbs"] = work["atomic_gather_bytes"] / (comb["us"] * 1e-6) / 1e9
        ceiling["combine_frac_of_gather"] = ceiling["combine_requested_gbs"] / gather_gbs
    expert_flop = work["expert1_flop"] + work["expert2_flop"]
    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == 1 else "f32",
        "data": "synthetic (seeded N(0,1/sqrt(fan_in)) weights, N(0,1) tokens)",
        "config": {"workload": cfg.name, "T": T, "d": cfg.d, "E": cfg.E, "E_ffn": cfg.E_ffn,
                   "k": cfg.k, "f": cfg.f, "n_shared": cfg.n_shared, "f_shared": cfg.f_shared,
                   "router": "product_key" if cfg.router == 1 else "softmax_topk",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "roofline_stages": stages,
        "measured_ceiling": ceiling,
        "phases_us": phase_us,
        "phases_cold_us": phase_cold_us,
        "step_us": step_us,
        "cold_step_us": cold_step_us,
        "layer_expert_tflops": expert_flop / (ms_per_step * 1e-3) / 1e12,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
