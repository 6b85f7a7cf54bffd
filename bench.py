"""Throughput of the MoM layer forward (and decode) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload l380m]

A step is one whole layer forward on one batch of synthetic input: route,
dispatch, projections, chunkwise recurrence, combine.  Inputs are resident in
HBM before the timed region.  The JSON line also carries, for the slowest
stage, its roofline position (HIP events around that stage's launches on the
stream it runs on, taken in a second pass over the same steps so that no event
sits between the kernels of the timed steps), the decode-step throughput of the long-context workload
(256 sequences, one token each, float32 states resident), and the fp64 CPU
checker timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0      # dense bf16 / fp16 matrix cores
FP32_VALU_PEAK_TFLOPS = 157.3  # vector fp32 (packed); 78.6 without packed ops

# Seconds of untimed steps each line runs before its W warm-up steps.  The GPU
# raises its clocks only after about a tenth of a second of load; a handful of
# warm-up steps (a few milliseconds) leaves the timed steps on the way up
# (measured: the 380M-shape step took 0.454-0.456 ms after 5 warm-up steps and
# 0.403-0.413 ms after 200).
CLOCK_WARMUP_S = 0.3


def ramp(fn, seconds=None):
    """Run fn (one untimed step of the line about to be timed) repeatedly for
    `seconds` of wall time; returns the number of steps run."""
    import torch
    seconds = CLOCK_WARMUP_S if seconds is None else seconds
    n = 0
    if seconds <= 0:
        return n
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="l380m")
    p.add_argument("--decode-steps", type=int, default=20)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-single", action="store_true", help="skip the single enlarged-memory line")
    p.add_argument("--no-gla", action="store_true", help="skip the gated linear attention layer line")
    p.add_argument("--no-bwd", action="store_true", help="skip the recurrence-gradient line")
    p.add_argument("--prefill", default="l1b3,m16,long32k",
                   help="other prefill workloads timed after the headline one (comma list; '' for none)")
    p.add_argument("--serial", action="store_true",
                   help="time the steps in order on one stream (default: the layer's two-stream schedule)")
    p.add_argument("--clock-warmup", type=float, default=CLOCK_WARMUP_S,
                   help="seconds of untimed steps before each line's warm-up steps (0 for none)")
    p.add_argument("--traffic", default=None,
                   help="summary of measured HBM bytes per call (default: profiles/traffic_<workload>.json)")
    return p.parse_args()


def stage_costs(cfg, state_in=False):
    """Algorithmic bytes and flops of one launch of each stage for one layer
    forward: every tensor read or written once at its stored width.  The chunk
    stage writes the final states, and reads entering states only when the
    step is given them (state_in)."""
    NT = cfg.B * cfg.T
    K, H, dk, dv, D, M, C = cfg.K, cfg.H, cfg.dk, cfg.dv, cfg.D, cfg.M, cfg.chunk
    N = NT * (K + 1)
    xb = 2 if cfg.dtype == "bf16" else 4
    ab = 2 if cfg.dtype == "bf16" else 4  # q/k/v storage (half or float32)
    n_state = cfg.B * (M + 1)
    c = {}
    c["route"] = dict(bytes=NT * (D * xb + 8 * K) + M * D * xb, flops=2 * NT * D * M)
    c["dispatch"] = dict(bytes=NT * K * 4 * 3 + 2 * NT * H * (M + 1) * 4 + 2 * N * H * 4 + N * 4, flops=0)
    proj_w = (H * dk + (M + 1) * H * (dk + dv)) * D * xb
    c["project"] = dict(bytes=NT * D * xb * (K + 2) + proj_w + (NT * H * dk + N * H * (dk + dv)) * ab,
                        flops=2 * D * (NT * H * dk + N * H * (dk + dv)))
    chunk_flops_row = 6 * C * dk + 4 * C * dv + 6 * dk * dv + (2 * C * C) // 3
    c["chunk"] = dict(bytes=N * H * (2 * dk * ab + dv * ab + 8 + dv * 4) + (2 if state_in else 1) * n_state * H * dk * dv * 4,
                      flops=N * H * chunk_flops_row)
    c["combine"] = dict(bytes=NT * H * dv * 4 * (K + 2) + NT * K * 8, flops=2 * NT * K * H * dv)
    return c


def layer_bound(cfg):
    """Throughput bound of one layer forward from the per-token costs of the
    unfused design: route, dispatch (with a gathered copy of x), combine and
    the chunk recurrence at the HBM peak, the projections at the MFMA peak
    (the chunk stage at whichever of its bytes or flops takes longer).
    Returns (tokens/s, per-stage microseconds)."""
    NT = cfg.B * cfg.T
    K, H, dk, dv, D, C = cfg.K, cfg.H, cfg.dk, cfg.dv, cfg.D, cfg.chunk
    A = K + 1
    bw, mf = HBM_PEAK_GBS * 1e9, MFMA_PEAK_TFLOPS * 1e12
    per_tok = {"route": (2 * D + 8 * K) / bw,
               "dispatch": (2 * D * (1 + K) + 16 * K * H + 12 * K) / bw,
               "project": (2 * D * H * dk + A * 2 * D * H * (dk + dv)) / mf,
               "chunk": max(A * (2 * H * dk * 2 + 2 * H * dv + 8 * H + 4 * H * dv) / bw,
                            A * H * (6 * C * dk + 4 * C * dv + 6 * dk * dv + (2 * C * C) / 3) / mf),
               "combine": (4 * A * H * dv + 8 * K + 4 * H * dv) / bw}
    us = {k: v * NT * 1e6 for k, v in per_tok.items()}
    return NT / (sum(us.values()) * 1e-6), us


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def decode_costs(cfg, n_seq):
    """Algorithmic bytes of the decode kernel (the recurrent step with the
    combine folded in): every state read and written once, q, k, v and the
    gates read, the layer's output row and the router weights."""
    K, H, dk, dv, D, M = cfg.K, cfg.H, cfg.dk, cfg.dv, cfg.D, cfg.M
    state = 2 * n_seq * (K + 1) * H * dk * dv * 4
    io = n_seq * (H * dk * 2 + (K + 1) * H * (dk + dv) * 2 + 2 * H * (M + 1) * 4 + H * dv * 4 + K * 4)
    return dict(bytes=state + io, flops=n_seq * (K + 1) * H * 6 * dk * dv)


def time_cpu_baseline(cfg, inp):
    """The fp64 oracle on the same batch the GPU step processes (about 10-20 s
    on 8-16 host cores for the 380M-shape workload)."""
    from oracle import oracle
    B, T = cfg.B, cfg.T
    NT = B * T
    sl = lambda a: a.reshape(cfg.B, cfg.T, *a.shape[1:])[:B, :T].reshape(NT, *a.shape[1:])
    x, al, be = sl(inp["x"]), sl(inp["alpha"]), sl(inp["beta"])
    oracle.lib()
    t0 = time.perf_counter()
    oracle.layer((B, T, cfg.D, cfg.H, cfg.dk, cfg.dv, cfg.M, cfg.K), x, inp["w_r"], inp["bias"], inp["w_q"],
                 inp["w_k"], inp["w_v"], al, be)
    dt = time.perf_counter() - t0
    return {"value": NT / dt, "unit": "tokens/s", "cores": oracle.threads(), "cpu": cpu_model(), "kind": "oracle",
            "sample": "fp64 oracle, one layer forward over the whole step batch (%d sequences x %d tokens, %.1f s)"
                      % (B, T, dt)}


def time_oracle_sample(cfg, inp, T):
    """The fp64 oracle on the first T tokens of the first sequence of cfg's
    inputs (a bounded sample, a few seconds): tokens/s."""
    from oracle import oracle
    x, al, be = inp["x"][:T], inp["alpha"][:T], inp["beta"][:T]
    oracle.lib()
    t0 = time.perf_counter()
    oracle.layer((1, T, cfg.D, cfg.H, cfg.dk, cfg.dv, cfg.M, cfg.K), x, inp["w_r"], inp["bias"], inp["w_q"],
                 inp["w_k"], inp["w_v"], al, be)
    dt = time.perf_counter() - t0
    return {"value": round(T / dt, 1), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": "fp64 oracle, one sequence x %d tokens of this workload (%.1f s)" % (T, dt)}


def time_gla_layer(cfg, inp, x, alpha, beta, steps, warmup):
    """The same layer, inputs and weights with gated linear attention memories
    (S <- a S + c k v^T) in place of Gated DeltaNet: whole forward steps."""
    import torch
    from mixture_memories_recurrence_amd import mom
    layer = mom.MomLayer(cfg, inp["w_r"], inp["bias"], inp["w_q"], inp["w_k"], inp["w_v"], rule="gla")
    state = torch.empty(cfg.B, cfg.M + 1, cfg.H, cfg.dk, cfg.dv, dtype=torch.float32, device="cuda")
    ramp(lambda: layer.forward(x, alpha, beta, state_out=state))
    for _ in range(warmup):
        layer.forward(x, alpha, beta, state_out=state)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward(x, alpha, beta, state_out=state)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    NT = cfg.B * cfg.T
    return {"workload": "%s layer with gated linear attention memories (same shapes, inputs and weights)" % cfg.name,
            "tokens_per_s": round(NT / (wall / steps), 1), "ms_per_step": round(wall * 1e3 / steps, 4)}


def time_chunk_bwd(cfg, inp, x, alpha, beta, steps, warmup):
    """Gradients for training over the layer's own segments: route, dispatch and
    projections run once (forward), then K timed calls of the recurrence's
    gradients alone (gdn_chunk_bwd) and K of the layer's backward (combine,
    recurrence, dispatch gathers, router weights), with random upstream
    gradients dL/dout and dL/d(final states).  Then K training steps (forward
    and backward) twice: with the forward keeping its chunk factors and states
    for the backward (train=True), and with the backward recomputing them."""
    import torch
    from mixture_memories_recurrence_amd import mom, synth
    layer = mom.MomLayer(cfg, inp["w_r"], inp["bias"], inp["w_q"], inp["w_k"], inp["w_v"])
    _, _, b = layer.forward(x, alpha, beta)
    gr = synth.make_chain_grads(b["N"], cfg.H, cfg.dk, cfg.dv, b["n_seg"], seed=9)
    d_o = torch.from_numpy(gr["d_o"]).cuda()
    dstate = torch.from_numpy(gr["dstate"]).cuda()
    dout = d_o[:b["NT"]].contiguous()
    dstate_l = dstate.view(cfg.B, cfg.M + 1, cfg.H, cfg.dk, cfg.dv)
    stream = torch.cuda.current_stream()

    def timed(fn):
        ramp(fn)
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(lambda: layer.chunk_backward(b, d_o, dstate))
    ms_layer = timed(lambda: layer.backward(x, dout, b, dstate_out=dstate_l))

    def step(train):
        layer.forward(x, alpha, beta, train=train)
        layer.backward(x, dout, b, dstate_out=dstate_l)

    ms_saved = timed(lambda: step(True))
    ms_recompute = timed(lambda: step(False))
    N, NT, H, dk, dv = b["N"], b["NT"], cfg.H, cfg.dk, cfg.dv
    # algorithmic bytes: q (per token), k, v (half), gates, dL/do, dL/dS_out read once;
    # dq, dk, dv, d_alpha, d_beta, dL/dS_in written once (float32)
    n_st = b["n_seg"] * H * dk * dv * 4
    nbytes = (NT * H * dk * 2 + N * H * (dk + dv) * 2 + N * H * 8 + N * H * dv * 4 + n_st
              + N * H * (2 * dk + dv) * 4 + N * H * 8 + n_st)
    return {"workload": "%s recurrence gradients (gdn_chunk_bwd over the layer's %d segments, %d rows)"
                        % (cfg.name, b["n_seg"], N),
            "ms": round(ms, 4), "tokens_per_s": round(NT / (ms * 1e-3), 1),
            "algorithmic_bytes": nbytes, "achieved_gb_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "layer_bwd": {"workload": "%s layer gradients: combine, recurrence, dispatch gathers, router weights "
                                      "(top-k held fixed); not the projections" % cfg.name,
                          "ms": round(ms_layer, 4), "tokens_per_s": round(NT / (ms_layer * 1e-3), 1)},
            "train_step": {"workload": "%s layer forward + the gradients above, one training step" % cfg.name,
                           "ms_saved": round(ms_saved, 4), "ms_recompute": round(ms_recompute, 4),
                           "tokens_per_s": round(NT / (ms_saved * 1e-3), 1)}}


def time_single_memory(steps, warmup):
    """One Gated DeltaNet memory with the 380M layer's active state width (value
    width 768, no router): gdn_chunk_fwd over B sequences as B segments."""
    import torch
    from mixture_memories_recurrence_amd import mom, synth
    sm = synth.SINGLE_MEMORY
    B, T, H, dk, dv = sm["B"], sm["T"], sm["H"], sm["dk"], sm["dv"]
    inp = synth.make_single_memory_inputs(B, T, H, dk, dv, seed=11)
    N = B * T
    cfg = synth.LayerConfig(B, T, 64, H, dk, dv, 1, 1, "bf16", "none", 64, "single")
    dims = mom.dims_of(cfg)
    g = lambda a, dt=torch.float32: torch.from_numpy(a).to(dt).cuda()
    q, k, v = g(inp["q"], torch.float16), g(inp["k"], torch.float16), g(inp["v"], torch.float16)
    alpha, beta = g(inp["alpha"]), g(inp["beta"])
    seg_off = torch.arange(0, N + 1, T, dtype=torch.int32, device="cuda")
    state = torch.empty(B, H, dk, dv, dtype=torch.float32, device="cuda")
    o = torch.empty(N, H, dv, dtype=torch.float32, device="cuda")
    ws = mom.chunk_workspace(dims, B, N)

    def step():
        mom.gdn_chunk_fwd(dims, B, N, N, B, seg_off, None, None, q, k, v, alpha, beta, None, state, o, ws)

    ramp(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(steps):
        step()
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[1]) / steps
    # algorithmic bytes: q, k, v read, o written (fp32), state written, gates read
    nbytes = N * H * (2 * dk * 2 + dv * 2 + 8 + dv * 4) + B * H * dk * dv * 4
    return {"workload": "single Gated DeltaNet memory: B=%d T=%d H=%d dk=%d dv=%d (the 380M layer's active "
                        "state width), half q/k/v, fp32 state and output" % (B, T, H, dk, dv),
            "tokens_per_s": round(N / (wall / steps), 1), "ms_per_step": round(wall * 1e3 / steps, 4),
            "kernel_ms": round(ms, 4), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


STAGES = ["route", "dispatch", "project", "chunk", "combine"]


class Workload:
    """One prefill workload on the GPU: inputs resident in HBM, the layer, its
    buffers, and the two ways of running a step (the layer's own two-stream
    schedule, and the stages in order on one stream with optional events
    between them)."""

    def __init__(self, name):
        import torch
        from mixture_memories_recurrence_amd import mom, synth
        self.mom = mom
        self.cfg = cfg = synth.CONFIGS[name]
        self.inp = inp = synth.make_layer_inputs(cfg, seed=0)
        self.layer = mom.MomLayer(cfg, inp["w_r"], inp["bias"], inp["w_q"], inp["w_k"], inp["w_v"])
        sd = mom.storage_dtype(cfg)
        self.x = torch.from_numpy(inp["x"]).to(sd).cuda()
        self.alpha = torch.from_numpy(inp["alpha"]).cuda()
        self.beta = torch.from_numpy(inp["beta"]).cuda()
        self.state = torch.empty(cfg.B, cfg.M + 1, cfg.H, cfg.dk, cfg.dv, dtype=torch.float32, device="cuda")
        self.b = self.layer.buffers(cfg.B, cfg.T)

    def step_serial(self, ev=None):
        mom, cfg, b, layer = self.mom, self.cfg, self.b, self.layer
        x, alpha, beta = self.x, self.alpha, self.beta
        d, N, NT = b["dims"], b["N"], b["NT"]
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        mom.mom_route_count(d, x, layer.w_r, layer.bias, b["idx"], b["w"], b["ws"])
        rec(1)
        mom.mom_dispatch_counted(d, b["idx"], x, alpha, beta, b["seg_off"], b["perm"], b["inv"], None,
                                 b["alpha_p"], b["beta_p"], b["ws"])
        rec(2)
        mom.mom_project(d, x, b["perm"], b["seg_off"], layer.w_q, layer.w_k, layer.w_v, b["q"], b["k"], b["v"])
        rec(3)
        mom.gdn_chunk_fwd(d, b["n_seg"], N, NT, cfg.B * (cfg.M + 1), b["seg_off"], b["seg_state"], b["perm"],
                          b["q"], b["k"], b["v"], b["alpha_p"], b["beta_p"], None, self.state, b["o"], b["ws_chunk"])
        rec(4)
        mom.mom_combine(d, NT, b["inv"], b["w"], b["o"], b["o"][b["NR"]:], b["out"])
        rec(5)

    def step_overlapped(self):
        # the layer's own schedule: the shared memory's path on a second stream
        self.layer.forward(self.x, self.alpha, self.beta, state_out=self.state)

    def time_steps(self, steps, warmup, serial=False):
        """K whole steps after W warm-up steps, nothing recorded between the
        kernels; returns (wall ms per step, GPU-event ms per step)."""
        import torch
        fn = self.step_serial if serial else self.step_overlapped
        ramp(fn)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        t0 = time.perf_counter()
        ev[0].record()
        for _ in range(steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall * 1e3 / steps, ev[0].elapsed_time(ev[1]) / steps

    def stage_ms(self, steps):
        """Per-stage times: K more steps in order on one stream with an event
        between the stages (each record adds a few microseconds between
        kernels, so these steps are not the timed ones)."""
        import torch
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            self.step_serial(events[i])
        torch.cuda.synchronize()
        return {s: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in range(steps)]))
                for j, s in enumerate(STAGES)}


def stage_table(cfg, st_ms):
    costs = stage_costs(cfg)
    kern = {}
    for s in STAGES:
        t = st_ms[s] * 1e-3
        kern[s] = {"ms": round(st_ms[s], 4), "GB/s": round(costs[s]["bytes"] / t / 1e9, 1),
                   "TFLOP/s": round(costs[s]["flops"] / t / 1e12, 2),
                   "hbm_frac": round(costs[s]["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4),
                   "mfma_frac": round(costs[s]["flops"] / t / 1e12 / MFMA_PEAK_TFLOPS, 4)}
    return kern


def describe(cfg):
    return ("%s: B=%d T=%d D=%d H=%d dk=%d dv=%d M=%d top-%d + shared, %s inputs, fp32 state"
            % (cfg.name, cfg.B, cfg.T, cfg.D, cfg.H, cfg.dk, cfg.dv, cfg.M, cfg.K, cfg.dtype))


def time_prefill(name, steps, warmup, cpu_tokens):
    """Tokens/s of another prefill workload (the layer's two-stream schedule),
    its per-stage times, the fraction of its layer bound, and the oracle on a
    bounded sample of it."""
    import torch
    w = Workload(name)
    cfg = w.cfg
    ms, gpu_ms = w.time_steps(steps, warmup)
    st = w.stage_ms(steps)
    NT = cfg.B * cfg.T
    bound, _ = layer_bound(cfg)
    r = {"workload": describe(cfg), "tokens_per_s": round(NT / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
         "gpu_ms_per_step": round(gpu_ms, 4), "bound_tokens_per_s": round(bound, 1),
         "frac_of_bound": round(NT / (ms * 1e-3) / bound, 4), "stages": stage_table(cfg, st)}
    if cpu_tokens:
        r["cpu_baseline"] = time_oracle_sample(cfg, w.inp, min(cpu_tokens, cfg.T))
    del w
    torch.cuda.empty_cache()
    return r


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from mixture_memories_recurrence_amd import mom, synth

    global CLOCK_WARMUP_S
    CLOCK_WARMUP_S = args.clock_warmup
    w = Workload(args.workload)
    cfg, inp, x, alpha, beta = w.cfg, w.inp, w.x, w.alpha, w.beta
    NT = cfg.B * cfg.T
    ms_per_step, gpu_ms = w.time_steps(args.steps, args.warmup, serial=args.serial)
    value = NT / (ms_per_step * 1e-3)
    st_ms = w.stage_ms(args.steps)
    kern = stage_table(cfg, st_ms)
    costs = stage_costs(cfg)
    dom = max(STAGES, key=lambda s: st_ms[s])
    t = st_ms[dom] * 1e-3
    ai = costs[dom]["flops"] / max(costs[dom]["bytes"], 1)
    if ai > MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        ach, peak, unit, bound = costs[dom]["flops"] / t / 1e12, MFMA_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        ach, peak, unit, bound = costs[dom]["bytes"] / t / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    from mixture_memories_recurrence_amd import pmc_traffic
    tpath = args.traffic or os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                         "traffic_%s.json" % cfg.name)
    traffic = pmc_traffic.load_traffic(tpath, dom, cfg.name)
    roofline = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
                "traffic": traffic, "kernel": "%s (%s)" % (dom, ", ".join(pmc_traffic.stage_kernels(dom, cfg.dtype))),
                "algorithmic_bytes": costs[dom]["bytes"], "algorithmic_flops": costs[dom]["flops"]}
    lb, lb_us = layer_bound(cfg)

    res = {
        "metric": "MoM layer fwd tokens/s (T=2048, M=4 top-2+shared) + decode tokens/s; % roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "gpu_ms_per_step": round(gpu_ms, 4),
        "clock_warmup_s": CLOCK_WARMUP_S,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": describe(cfg), "tokens_per_step": NT, "chunk": cfg.chunk},
        "roofline": roofline,
        "layer_bound": {"tokens_per_s": round(lb, 1), "frac": round(value / lb, 4),
                        "stage_us": {k: round(v, 1) for k, v in lb_us.items()}},
        "stages": kern,
    }
    del w
    if not args.no_decode:
        dcfg = synth.CONFIGS["long32k"]
        n_seq = synth.DECODE_SEQS
        dinp = synth.make_layer_inputs(dataclasses_replace(dcfg, B=1, T=1), seed=0)
        dlayer = mom.MomLayer(dcfg, dinp["w_r"], dinp["bias"], dinp["w_q"], dinp["w_k"], dinp["w_v"])
        states = torch.from_numpy(synth.make_state(dcfg, n_seq, seed=8)).cuda()
        steps_in = []
        for s in range(4):
            d = synth.make_decode_step_inputs(dcfg, n_seq, seed=100 + s)
            steps_in.append((torch.from_numpy(d["x"]).to(torch.bfloat16).cuda(), torch.from_numpy(d["alpha"]).cuda(),
                             torch.from_numpy(d["beta"]).cuda()))
        db = dlayer.buffers(n_seq, 1)
        ramp(lambda: dlayer.decode_step(*steps_in[0], states))
        for i in range(3):
            dlayer.decode_step(*steps_in[i % 4], states)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.decode_steps):
            dlayer.decode_step(*steps_in[i % 4], states)
        torch.cuda.synchronize()
        dwall = time.perf_counter() - t0
        # the decode kernel alone (the recurrent step with the combine folded
        # in), from events around it in further steps
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.decode_steps)]
        for i in range(args.decode_steps):
            xx, aa, bb = steps_in[i % 4]
            dlayer.route_dispatch_project(xx, aa, bb, db)
            ev[i][0].record()
            mom.decode_step_combined("gdn", db["dims"], n_seq, db["idx"], db["inv"], db["w"], db["q"], db["k"],
                                     db["v"], aa, bb, states, db["out"])
            ev[i][1].record()
        torch.cuda.synchronize()
        dk_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        dc = decode_costs(dcfg, n_seq)
        res["decode"] = {"workload": "long32k decode: %d sequences x 1 token, D=%d H=%d dk=%d dv=%d M=%d top-%d, "
                                     "fp32 states [%d,%d,%d,%d,%d] resident" % (n_seq, dcfg.D, dcfg.H, dcfg.dk, dcfg.dv,
                                                                               dcfg.M, dcfg.K, n_seq, dcfg.M + 1,
                                                                               dcfg.H, dcfg.dk, dcfg.dv),
                         "tokens_per_s": round(n_seq * args.decode_steps / dwall, 1),
                         "ms_per_step": round(dwall * 1e3 / args.decode_steps, 4),
                         "decode_kernel_ms": round(dk_ms, 4),
                         "decode_kernel_GB/s": round(dc["bytes"] / (dk_ms * 1e-3) / 1e9, 1),
                         "decode_kernel_hbm_frac": round(dc["bytes"] / (dk_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    if not args.no_gla:
        res["gla_layer"] = time_gla_layer(cfg, inp, x, alpha, beta, args.steps, args.warmup)

    if not args.no_single:
        res["single_memory"] = time_single_memory(args.steps, args.warmup)
    if not args.no_bwd:
        res["chunk_bwd"] = time_chunk_bwd(cfg, inp, x, alpha, beta, args.steps, args.warmup)

    if args.prefill:
        res["prefill"] = {n: time_prefill(n, args.steps, args.warmup, 0 if args.no_cpu_baseline else 512)
                          for n in args.prefill.split(",") if n and n != cfg.name}

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = time_cpu_baseline(cfg, inp)
    print(json.dumps(res), flush=True)


def dataclasses_replace(c, **kw):
    import dataclasses
    return dataclasses.replace(c, **kw)


if __name__ == "__main__":
    main()
