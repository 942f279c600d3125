"""Benchmark of the sparse MoE FFN layer forward on one MI355X.

A step is one pass of the layer's hot path over one batch: route (logits,
scores, biased top-k, renorm) -> dispatch (counting sort + gather, expert
counts) -> grouped SwiGLU gate_up GEMM -> grouped down GEMM -> shared expert
-> combine.  Default workload: T=8192 tokens, hidden 4096, 64 routed experts
top-6, moe_intermediate 2048, one shared expert (2048), sqrtsoftplus scores
with an fp32 selection bias ~N(0, 0.5), renormalised weights, bf16.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_layer(w, device="cuda"):
    import torch  # noqa: F401
    from sparse_mixture_experts_route_amd import _lib as L
    from sparse_mixture_experts_route_amd.layer import MoEFFN
    from workloads import make_inputs
    inp = make_inputs(w, device=device)
    sh = L.make_shape(w.T, w.H, w.E, w.k, w.I, w.Is, w.score, w.renorm, w.shared_gated,
                      L.DTYPE_BF16 if w.dtype == "bf16" else L.DTYPE_FP32)
    params = {k: v for k, v in inp.items() if k not in ("x", "dout", "sel_bias")}
    bias = inp.get("sel_bias")
    layer = MoEFFN(sh, params, sel_bias=bias, rate=1e-3)
    return layer, inp


def _device_sysfs():
    """sysfs directory of the current device's PCI function, or None."""
    import ctypes
    import torch
    try:
        lib = ctypes.CDLL("libamdhip64.so")
        buf = ctypes.create_string_buffer(64)
        if lib.hipDeviceGetPCIBusId(buf, 64, torch.cuda.current_device()) != 0:
            return None
        d = os.path.join("/sys/bus/pci/devices", buf.value.decode().lower())
        return d if os.path.isdir(d) else None
    except OSError:
        return None


def _read_dpm(path):
    """MHz of the level marked current ('*') in a pp_dpm_* file, or None."""
    try:
        with open(path) as f:
            for line in f:
                if "*" in line:
                    v = line.split(":", 1)[1].replace("*", "").strip().lower().replace("mhz", "")
                    return float(v)
    except (OSError, ValueError, IndexError):
        return None
    return None


class ClockSampler:
    """Samples the device's current shader (sclk) and memory (mclk) clock
    levels from sysfs while queued GPU work runs; records nothing when the
    files are not readable."""

    def __init__(self):
        self.dir = _device_sysfs()
        self.sclk, self.mclk = [], []

    def sample_until(self, event, max_s=30.0):
        if self.dir is None:
            return
        t_end = time.perf_counter() + max_s
        while not event.query() and time.perf_counter() < t_end:
            for name, acc in (("pp_dpm_sclk", self.sclk), ("pp_dpm_mclk", self.mclk)):
                v = _read_dpm(os.path.join(self.dir, name))
                if v is not None:
                    acc.append(v)
            time.sleep(0.002)

    def summary(self):
        import statistics
        if not self.sclk and not self.mclk:
            return {"source": "sysfs pp_dpm_sclk / pp_dpm_mclk", "available": False}
        out = {"source": "sysfs pp_dpm_sclk / pp_dpm_mclk, sampled during the timed steps", "samples": len(self.sclk)}
        for name, acc in (("sclk_mhz", self.sclk), ("mclk_mhz", self.mclk)):
            if acc:
                out[name] = {"min": min(acc), "median": statistics.median(acc), "max": max(acc)}
        return out


def timed_steps(step, steps, warmup, clocks=None):
    """`warmup` untimed steps, then exactly `steps` steps, each bracketed by
    its own pair of events on the current stream, with a device
    synchronisation on both sides.  Returns (per-step ms list, wall s)."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        step(i)
        ev[i + 1].record()
    if clocks is not None:
        clocks.sample_until(ev[-1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)], wall


def _stats(per):
    import statistics
    return {"median_ms": statistics.median(per), "mean_ms": sum(per) / len(per), "min_ms": min(per),
            "max_ms": max(per), "steps": len(per)}


def time_forward(w, steps, warmup, profile=True, backward=False):
    """Times `steps` layer steps after `warmup` (median of per-step event
    times, no stage events in that region); with `profile`, a second timed
    region of as many steps records the library's stage events (the
    dominant GEMM's launch duration) and the router and dispatch calls are
    timed on their own.  Returns a dict of results."""
    import torch
    from sparse_mixture_experts_route_amd import _lib as L
    layer, inp = build_layer(w)
    xs = [inp["x"], inp["x"].clone()]          # rotate two copies of the input
    dout = inp.get("dout")
    if backward:
        layer.aux_alpha = 1e-2   # a training step: aux loss in the forward, its term in the backward

    def step(i):
        layer.forward(xs[i % 2], training=backward, save=backward)
        if backward:
            layer.backward(dout)

    clocks = ClockSampler() if profile else None
    per, wall = timed_steps(step, steps, warmup, clocks)
    res = {"timing": _stats(per), "ms_per_step": _stats(per)["median_ms"], "wall_s": wall,
           "clock": clocks.summary() if clocks is not None else None,
           "stages_ms": {}, "n_fwd": 0, "n_bwd": 0, "route_ms": 0.0, "dispatch_ms": 0.0}
    if profile:
        # the stage-timed region: same steps, library stage events on its launch stream
        L.moe_profile_begin(2 * steps)
        per_s, _ = timed_steps(step, steps, 0)
        stages, nf, nb = L.moe_profile_end()
        res.update({"stage_timing": _stats(per_s), "stages_ms": stages, "n_fwd": nf, "n_bwd": nb})
        # router and dispatch calls alone (same stream)
        sh = layer._shape_T(w.T)
        dev = xs[0].device
        P = w.T * w.k
        counts = torch.empty((w.E,), dtype=torch.int32, device=dev)
        offsets = torch.empty((w.E + 1,), dtype=torch.int32, device=dev)
        perm = torch.empty((P,), dtype=torch.int32, device=dev)
        pos = torch.empty((P,), dtype=torch.int32, device=dev)
        # nrep back-to-back calls between two events, outputs allocated
        # beforehand, so the host's per-call overhead stays off the GPU clock
        nrep = max(3, min(steps, 20))
        T, k = w.T, w.k
        wts = torch.empty((T, k), dtype=torch.float32, device=dev)
        ids = torch.empty((T, k), dtype=torch.int64, device=dev)
        gate = torch.empty((T,), dtype=torch.float32, device=dev) if (w.Is and w.shared_gated) else None
        wg = layer.p.get("w_shared_gate") if gate is not None else None
        bias = layer.balance.bias if layer.balance is not None else None

        rws = layer._workspace(sh, L.OP_ROUTE, dev)
        fws = layer._workspace(sh, L.OP_ROUTE_DISPATCH, dev)

        def route(i):
            L.moe_route(sh, xs[i % 2], layer.p["w_router"], wg, bias, None, wts, ids, gate, ws=rws)

        def route_dispatch(i):  # the call the layer makes: routing and the sort together
            L.moe_route_dispatch(sh, xs[i % 2], layer.p["w_router"], wg, bias, None, wts, ids, gate, counts,
                                 offsets, perm, pos, fws)
        out = []
        for fn in (route, route_dispatch):
            fn(0)
            torch.cuda.synchronize()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            for i in range(nrep):
                fn(i)
            e[1].record()
            torch.cuda.synchronize()
            out.append(e[0].elapsed_time(e[1]) / nrep)
        res["route_ms"], rd_ms = out
        res["dispatch_ms"] = rd_ms - res["route_ms"]   # the sort's share of the fused call
    counts = layer.last["counts"].cpu().numpy()
    res["load"] = {"max_segment": int(counts.max()), "mean_segment": float(counts.mean()),
                   "dead_experts": int((counts == 0).sum()), "active_experts": int((counts > 0).sum())}
    del layer, inp, xs
    torch.cuda.empty_cache()
    return res


def time_tp_share(w, n, steps, warmup):
    """One GPU's share of an n-way tensor-parallel layer: route, dispatch, the
    expert MLPs on the share's I/n and Is/n slices (pre-top-k-sum partials),
    then the combine.  The all-reduce that sums the shares' partials between
    the last two needs the other GPUs and is not part of the step."""
    import torch
    from sparse_mixture_experts_route_amd import _lib as L
    from sparse_mixture_experts_route_amd.layer import tp_share_params
    layer, inp = build_layer(w)
    share = tp_share_params(layer.p, n, 0)
    for key in ("w_gate_up", "w_down", "ws_gate_up", "ws_down"):
        layer.p.pop(key, None)
        inp.pop(key, None)
    torch.cuda.empty_cache()
    sh = layer._shape_T(w.T)
    ssh = layer._shape_T(w.T)
    ssh.I, ssh.Is = w.I // n, w.Is // n
    dev = inp["x"].device
    P = w.T * w.k
    xs = [inp["x"], inp["x"].clone()]
    counts = torch.empty((w.E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((w.E + 1,), dtype=torch.int32, device=dev)
    perm = torch.empty((P,), dtype=torch.int32, device=dev)
    pos = torch.empty((P,), dtype=torch.int32, device=dev)
    y = torch.empty((P, w.H), dtype=torch.float32, device=dev)
    sy = torch.empty((w.T, w.H), dtype=torch.float32, device=dev) if w.Is else None
    out = torch.empty_like(xs[0])
    ws_d = layer._workspace(sh, L.OP_DISPATCH, dev)
    ws_p = torch.empty((max(L.workspace_bytes(ssh, L.OP_FFN_PARTIAL), 256),), dtype=torch.uint8, device=dev)
    wst = L.weights_struct(share["w_gate_up"], share["w_down"], share.get("ws_gate_up"), share.get("ws_down"))

    def step(i):
        r = layer._route(xs[i % 2])
        L.moe_dispatch(sh, r["ids"], xs[i % 2], counts, offsets, perm, pos, None, ws_d)
        L.moe_ffn_forward_partial(ssh, wst, xs[i % 2], None, offsets, perm, y, sy, None, ws_p)
        L.moe_combine(sh, y, pos, r["weights"], r["gate"], sy, out)

    per, _ = timed_steps(step, steps, warmup)
    ms = _stats(per)["median_ms"]
    del layer, inp, xs, share, y, sy
    torch.cuda.empty_cache()
    return ms


def time_parallel_block(w, Id, steps, warmup):
    """The parallel dense + MoE block at a workload's shape: route on the
    residual, dispatch, experts on its normalised copy, a dense MLP of width
    Id beside them, the three output norms, residual and layer scalar."""
    import torch
    from sparse_mixture_experts_route_amd.layer import ParallelDenseMoEBlock
    w0 = w.with_(Is=0, shared_gated=False)
    layer, inp = build_layer(w0)
    g = torch.Generator(device="cuda").manual_seed(11)
    dt = inp["x"].dtype
    dense = {"w_gate_up": (torch.randn((2 * Id, w.H), generator=g, device="cuda") * w.H ** -0.5).to(dt),
             "w_down": (torch.randn((w.H, Id), generator=g, device="cuda") * Id ** -0.5).to(dt)}
    norms = {n: torch.ones((w.H,), dtype=dt, device="cuda") for n in
             ("g_pre_moe", "g_post_dense", "g_post_moe", "g_post")}
    blk = ParallelDenseMoEBlock(layer, dense, norms, eps=1e-6, layer_scalar=1.0)
    res = [inp["x"], inp["x"].clone()]
    xd = torch.randn(inp["x"].shape, generator=g, device="cuda").to(dt)
    per, _ = timed_steps(lambda i: blk.forward(res[i % 2], xd), steps, warmup)
    ms = _stats(per)["median_ms"]
    del blk, layer, inp, res, dense
    torch.cuda.empty_cache()
    return ms


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_gemm_dsv4flash_traffic.txt")
GEMM_SRC = os.path.join(ROOT, "sparse_mixture_experts_route_amd", "csrc", "gemm.hip")


def gemm_source_sha256() -> str:
    """SHA-256 of gemm.hip's code: line comments, trailing blanks and empty
    lines removed, so a comment edit does not void recorded counters."""
    import hashlib
    import re
    code = []
    with open(GEMM_SRC) as f:
        for line in f:
            line = re.sub(r"//.*$", "", line).rstrip()
            if line:
                code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()


def recorded_traffic():
    """HBM bytes per routed gate_up launch from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's reading), or
    None when the GEMM source changed after the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("gemm_sha256") != gemm_source_sha256():
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(mib: int):
    """A plain device copy of known size (src and dst of `mib` MiB each), run
    three times: the calibration kernel for the FETCH_SIZE / WRITE_SIZE
    counters."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: {n} bytes read and written per copy, 3 copies")
    del src, dst
    torch.cuda.empty_cache()


def hbm_probe(gib: int = 2, reps: int = 10):
    """The device's achievable HBM rates with the library's plain stream
    kernels (moe_bandwidth_probe): read, write and copy of `gib` GiB, each
    over a few grid sizes, median of `reps` timed launches; the best grid's
    rate per kind (GB/s counts bytes read plus bytes written)."""
    import statistics
    import torch
    from sparse_mixture_experts_route_amd import _lib as L
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {}
    for kind, name, moved in ((0, "read", n), (1, "write", n), (2, "copy", 2 * n)):
        best = None
        for per_cu in (2, 4, 8, 16):
            wgs = per_cu * cus
            ms = []
            for _ in range(reps + 1):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record()
                L.moe_bandwidth_probe(kind, src, dst, n, wgs)
                e[1].record()
                torch.cuda.synchronize()
                ms.append(e[0].elapsed_time(e[1]))
            med = statistics.median(ms[1:])
            gbs = moved / (med / 1e3) / 1e9
            if best is None or gbs > best["GB/s"]:
                best = {"GB/s": gbs, "ms": med, "workgroups_per_cu": per_cu}
        out[name] = best
        log(f"hbm probe {name}: {best['GB/s']:.0f} GB/s ({best['workgroups_per_cu']} workgroups per CU)")
    del src, dst
    torch.cuda.empty_cache()
    return {"note": f"library stream kernels over {gib} GiB buffers, best of 2/4/8/16 workgroups per CU, "
                    f"median of {reps} launches; GB/s counts bytes read plus bytes written", **out}


def cpu_baseline(w, n_tokens=4096):
    """The float64 dense-masked oracle on a bounded token sample of the same
    workload (routing from the oracle's own fp32 logits)."""
    import numpy as np
    import torch
    from oracle import moe_ref as R
    from workloads import make_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    inp = make_inputs(w, device="cuda")
    sel = torch.arange(n_tokens, device="cuda") * (w.T // n_tokens)

    def f(t):
        return t.detach().float().cpu().numpy()
    x = f(inp["x"][sel]).astype(np.float64)
    wr = f(inp["w_router"])
    wgu = f(inp["w_gate_up"])
    wd = f(inp["w_down"])
    sgu = f(inp["ws_gate_up"]) if w.Is else None
    sd = f(inp["ws_down"]) if w.Is else None
    sg = f(inp["w_shared_gate"]) if w.shared_gated else None
    bias = f(inp["sel_bias"]) if "sel_bias" in inp else None
    del inp
    torch.cuda.empty_cache()
    t0 = time.perf_counter()
    R.layer_forward(x, wr, w.k, w.score, w.renorm, wgu, wd, sgu, sd, sg, bias)
    dt = time.perf_counter() - t0
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"dense-masked float64 oracle on {n_tokens} of {w.T} tokens (token stride {w.T // n_tokens}),"
                      f" all {w.E} experts per token; {dt:.1f} s"}


def cpu_baseline_loop(w):
    """The oracle's per-expert loop (the sparse CPU path: SwiGLU on exactly
    the rows each expert received, plus the shared expert) on every token of
    the workload, routing from the oracle's own fp32 logits: the stronger CPU
    baseline, timed apart from the dense-masked one."""
    import numpy as np
    import torch
    from oracle import moe_ref as R
    from workloads import make_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    inp = make_inputs(w, device="cuda")

    def f(t):
        return t.detach().float().cpu().numpy()
    x = f(inp["x"]).astype(np.float64)
    wr = f(inp["w_router"])
    wgu, wd = f(inp["w_gate_up"]), f(inp["w_down"])
    sgu = f(inp["ws_gate_up"]) if w.Is else None
    sd = f(inp["ws_down"]) if w.Is else None
    sg = f(inp["w_shared_gate"]) if w.shared_gated else None
    bias = f(inp["sel_bias"]) if "sel_bias" in inp else None
    del inp
    torch.cuda.empty_cache()
    t0 = time.perf_counter()
    R.layer_forward(x, wr, w.k, w.score, w.renorm, wgu, wd, sgu, sd, sg, bias, loop=True)
    dt = time.perf_counter() - t0
    return {"value": w.T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle (per-expert loop)",
            "sample": f"all {w.T} tokens, each expert's SwiGLU on its own rows; {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv4flash",
                    help="dsv4flash (the headline), another name of workloads.WORKLOADS, or qwen2moe_decode_T<n>")
    ap.add_argument("--backward", action="store_true",
                    help="time the training step (forward with the aux loss, then backward) instead of the forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-primary", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after the timed steps, run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build runs the layer's data-parallel share on a single "
              "MI355X; multi-GPU runs are not part of it (use --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    from sparse_mixture_experts_route_amd import _lib as L
    from workloads import WORKLOADS, decode_workload
    L.load()
    assert torch.cuda.is_available(), "bench needs a HIP device"
    if args.workload.startswith("qwen2moe_decode_T"):
        w = decode_workload(int(args.workload[len("qwen2moe_decode_T"):]))
    else:
        w = WORKLOADS[args.workload]
    log(f"bench: {w.name} T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} Is={w.Is}" + (" (training step)" if args.backward else ""))
    r = time_forward(w, args.steps, args.warmup, backward=args.backward)
    s_step = r["ms_per_step"] / 1e3
    tflops = (3.0 if args.backward else 1.0) * w.fwd_flops() / s_step / 1e12
    P = w.T * w.k
    gu_flops = 2.0 * P * w.H * 2 * w.I
    gu_ms = r["stages_ms"]["gate_up"] / max(1, r["n_fwd"])
    gu_tflops = gu_flops / (gu_ms / 1e3) / 1e12
    b = 2 if w.dtype == "bf16" else 4
    gated = 1 if (w.Is and w.shared_gated) else 0
    # x and the router rows (+ the shared gate's row) read, the fp32 bias
    # read, weights (fp32) and ids (int64) written, the gate (fp32) written;
    # the timed call writes no logits
    route_bytes = w.T * w.H * b + (w.E + gated) * w.H * b + 4 * w.E + 12 * P + 4 * w.T * gated
    # ids in, perm + pos out, counts + offsets (+ the router's per-tile loads,
    # tiles of 16 tokens: written by the router, read by the sort); the row
    # gather is fused into the gate_up GEMM's loads (rows read from x through
    # perm), so no x_sorted
    disp_bytes = 8 * P + 8 * P + 8 * w.E
    comb_bytes = P * w.H * b + 8 * P + w.T * w.H * b * (1 + (1 if w.Is else 0))
    comb_ms = r["stages_ms"]["combine"] / max(1, r["n_fwd"])
    hbm = {
        "route": {"ms": r["route_ms"], "GB/s": route_bytes / (r["route_ms"] / 1e3) / 1e9 if r["route_ms"] else None},
        "dispatch": {"ms": r["dispatch_ms"],
                     "GB/s": disp_bytes / (r["dispatch_ms"] / 1e3) / 1e9 if r["dispatch_ms"] else None},
        "combine": {"ms": comb_ms, "GB/s": comb_bytes / (comb_ms / 1e3) / 1e9 if comb_ms else None},
    }
    for v in hbm.values():
        if v["GB/s"] is not None:
            v["frac_hbm_peak"] = v["GB/s"] / PEAK_HBM_GBS
    stage_avg = {k: v / max(1, r["n_fwd"]) for k, v in r["stages_ms"].items() if v}
    log(f"forward {r['ms_per_step']:.3f} ms/step, {tflops:.1f} TFLOP/s; gate_up {gu_ms:.3f} ms "
        f"({gu_tflops:.1f} TFLOP/s); stages {stage_avg}")
    out = {
        "metric": "MoE layer fwd tokens/s + TFLOP/s (% bf16 MFMA peak), E=64 top-6, 1 MI355X",
        "value": w.T / s_step,
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights, fp32 bias N(0,0.5))",
        "config": {"workload": f"{w.name}: T={w.T} H={w.H} E={w.E} top-{w.k} I={w.I} shared Is={w.Is}"
                               f"{' gated' if w.shared_gated else ''}, "
                               f"{['softmax', 'sigmoid', 'sqrtsoftplus'][w.score]}"
                               f"{' + fp32 selection bias' if w.has_bias else ''}{', renorm' if w.renorm else ''}, "
                               f"{w.dtype}" + (", training step (forward + backward)" if args.backward else ""),
                   "tokens": w.T, "hidden": w.H, "experts": w.E, "top_k": w.k, "moe_intermediate": w.I,
                   "shared_intermediate": w.Is},
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "roofline": {"bound": "mfma", "kernel": "grouped gate_up + SwiGLU GEMM", "achieved": gu_tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": gu_tflops / PEAK_BF16_TFLOPS,
                     # the counters were taken on the headline forward only
                     "traffic": recorded_traffic() if (w.name == "dsv4flash" and not args.backward) else None,
                     "flops_per_launch": gu_flops, "avg_launch_ms": gu_ms},
        "timing": {"ms_per_step": "median of the per-step event times of the timed steps (no stage events "
                                  "in that region)", **r["timing"]},
        "clock": r["clock"],
        "stage_ms": stage_avg,
        "stage_timing": {"note": "a second region of as many steps with the library's stage events recorded; "
                                 "roofline.avg_launch_ms and stage_ms come from it", **r.get("stage_timing", {})},
        "hbm_stages": hbm,
        "load": r["load"],
    }
    if args.copy_probe:
        copy_probe(args.copy_probe)
    if not args.only_primary:
        out["hbm_probe"] = hbm_probe()
        ceiling = max(out["hbm_probe"]["read"]["GB/s"], out["hbm_probe"]["copy"]["GB/s"])
        for v in hbm.values():
            if v["GB/s"] is not None:
                v["frac_probe_ceiling"] = v["GB/s"] / ceiling
    if not args.only_primary:
        other = {}
        cases = [WORKLOADS["qwen2moe"], WORKLOADS["deepseekv3"]] + [decode_workload(t) for t in (16, 64, 256)]
        for wl in cases:
            decode = wl.T <= 256
            rr = time_forward(wl, 50 if decode else 20, 3, profile=False)
            sp = rr["ms_per_step"] / 1e3
            tf = wl.fwd_flops() / sp / 1e12
            other[wl.name] = {"ms_per_step": rr["ms_per_step"], "tokens_per_s": wl.T / sp, "tflops": tf,
                              "pct_bf16_peak": 100 * tf / PEAK_BF16_TFLOPS, "load": rr["load"]}
            log(f"{wl.name}: {rr['ms_per_step']:.3f} ms, {tf:.1f} TFLOP/s")
        wl = WORKLOADS["qwen2moe_train"]
        rr = time_forward(wl, 20, 3, profile=False, backward=True)
        sp = rr["ms_per_step"] / 1e3
        tf = 3.0 * wl.fwd_flops() / sp / 1e12
        other[wl.name + "_fwd_bwd"] = {"ms_per_step": rr["ms_per_step"], "tokens_per_s": wl.T / sp,
                                       "tflops": tf, "pct_bf16_peak": 100 * tf / PEAK_BF16_TFLOPS}
        log(f"{wl.name} fwd+bwd: {rr['ms_per_step']:.3f} ms, {tf:.1f} TFLOP/s")
        n_tp = 8
        ms = time_tp_share(w, n_tp, 20, 3)
        sp = ms / 1e3
        tf = w.with_(I=w.I // n_tp, Is=w.Is // n_tp).fwd_flops() / sp / 1e12
        other[f"{w.name}_tp{n_tp}_share"] = {"ms_per_step": ms, "tokens_per_s": w.T / sp, "tflops": tf,
                                             "pct_bf16_peak": 100 * tf / PEAK_BF16_TFLOPS,
                                             "note": "one share of an 8-way split of I and Is; "
                                                     "the all-reduce between shares is not included"}
        log(f"{w.name} tp{n_tp} share: {ms:.3f} ms, {tf:.1f} TFLOP/s")
        wq = WORKLOADS["qwen2moe"]
        ms = time_parallel_block(wq, wq.Is, 20, 3)
        sp = ms / 1e3
        tf = wq.with_(shared_gated=False).fwd_flops() / sp / 1e12
        other["qwen2moe_parallel_dense_moe_block"] = {
            "ms_per_step": ms, "tokens_per_s": wq.T / sp, "tflops": tf, "pct_bf16_peak": 100 * tf / PEAK_BF16_TFLOPS,
            "note": "router on the residual, experts on its RMS norm, dense SwiGLU MLP of width 5632 beside them, "
                    "three output norms, residual and layer scalar"}
        log(f"qwen2moe parallel block: {ms:.3f} ms, {tf:.1f} TFLOP/s")
        out["other_workloads"] = other
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(w)
        log(f"cpu baseline: {out['cpu_baseline']}")
        if not args.only_primary:
            out["cpu_baseline_loop"] = cpu_baseline_loop(w)
            log(f"cpu baseline (per-expert loop): {out['cpu_baseline_loop']}")
            # the same per-expert loop on the tiny fp32 and Qwen2-MoE-like
            # forwards (context only; the training step has no loop form)
            loops = {}
            for name in ("tiny_fp32", "qwen2moe"):
                loops[name] = cpu_baseline_loop(WORKLOADS[name])
                log(f"cpu baseline (per-expert loop, {name}): {loops[name]}")
            out["cpu_baseline_loop_other"] = loops
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
