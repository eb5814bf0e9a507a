#!/usr/bin/env python3
"""Benchmark of the MoE-layer forward on one MI355X.

The timed loop replays one step captured as a HIP graph (the per-layer calls are also timed
eagerly, reported as eager_ms_per_layer).

One step = one forward of each of L distinct seeded layer instances (the default, Gemma-4
26B-A4B-shaped decode: d_model 2816, 128 experts, top-8, d_ff 704, SwiGLU, Q8_0 weights, bf16
activations, T = 8 tokens, L = 30 layers, ~24 GB of weights resident in HBM), so no layer's
weights are served from the 256 MB Infinity Cache by a previous call.  The metric is MoE-layer
tokens/s = T * L * steps / elapsed, with all inputs resident in HBM before the timed region.

Also reported on the same JSON line:
  roofline     - the dominant kernel (the fused dequant + gate/up + activation kernel) against
                 the 8 TB/s HBM peak: algorithmic bytes per launch (the touched experts' gate/up
                 weights and scales plus x) over its average launch time, measured with HIP events
                 in a pass of its own; roofline.layer holds the whole layer's figure (all of its
                 algorithmic bytes over the whole step time), the quantity the decode target is
                 set on;
  cpu_baseline - the CPU oracle (plain fp64 C) on layer instance 0, timed on this host;
  variants     - the other workloads (the tiny layer, time only; T=1, per-row int8, MiniMax-M3
                 shape, Nemotron latent with zero-skip and dense down, E2M1 SwiGLU, a shared
                 expert, and the int8, Q8_0 and fp8 prefill paths), each with tokens/s and its own
                 roofline fractions.

Algorithmic bytes count what the method must move (touched experts' weights and scales, with
zero-skip only the 16-neuron groups the kernel's own h makes live, router, x, out), never the
workspace kept between kernels.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
I8_PEAK_TOPS = 5000.0          # MI355X dense int8 matrix ops, published (POP/s = 5.0)
F8_PEAK_TFLOPS = 5000.0        # MI355X dense fp8 matrix flops, published: the peak the E4M3
                               # contraction is held to
F16_PEAK_TFLOPS = 2500.0       # MI355X dense fp16 matrix flops, published: the instruction peak of
                               # the f16 matrix cores the E4M3 codes are multiplied on


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gemma_decode")
    ap.add_argument("--T", type=int, default=8)
    ap.add_argument("--fmt", default="q8_0", choices=["q8_0", "i8_row", "e2m1", "fp8_row"])
    ap.add_argument("--plain", action="store_true",
                    help="time the plain row-major int8 layout instead of the tiled one")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--flags", type=int, default=0)
    ap.add_argument("--n-shared", type=int, default=0, help="shared experts beside the routed ones")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (counter scaling)")
    return ap.parse_args()


def copy_calibration():
    """A plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(5):
        b.copy_(a)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / 5
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": ms,
                      "copy_gbs": 2 * n / ms / 1e6}), flush=True)


def expert_gateup_bytes(w) -> int:
    import moe_inputs as mi
    rows, d = w.gate_up_rows, w.d_model
    if w.fmt == mi.FMT_Q8_0:
        return rows * d + rows * (d // 32) * 2
    if w.fmt in (mi.FMT_I8_ROW, mi.FMT_FP8_ROW):
        return rows * d + rows * 4
    return rows * d // 2 + rows * (d // 16) * 2


def expert_down_bytes(w) -> int:
    return __import__("moe_inputs").expert_bytes(w) - expert_gateup_bytes(w)


class Case:
    """L layer instances of one workload, resident on the GPU, with their distinct-expert counts."""

    def __init__(self, w, L, flags=0, tiled=True):
        import torch
        import moe_inputs as mi
        import sparse_moe_expert_router_amd as moe
        self.w, self.L, self.flags = w, L, flags
        self.layers = []
        for i in range(L):
            lay = mi.make_layer(w, i, "cuda")
            if tiled and w.fmt in (mi.FMT_Q8_0, mi.FMT_I8_ROW, mi.FMT_FP8_ROW):
                lay["experts"] = moe.repack_experts(lay["experts"], w.act)  # one-time load step
                torch.cuda.synchronize()
            self.layers.append(lay)
        self.xs = [mi.make_x(w, i, device="cuda") for i in range(L)]
        self.outs = [torch.empty((w.T, w.d_model), device="cuda") for _ in range(L)]
        nbytes = moe.workspace_bytes(w.T, w.k, self.layers[0]["experts"], w.act, flags)
        self.ws = moe.alloc_workspace(nbytes)
        self.distinct = []
        self.active_groups = [] if flags & 1 else None    # zero-skip: groups the down kernel reads
        for i in range(L):
            _, idx, _ = moe.layer_forward(self.xs[i], self.layers[i]["w_router"], self.layers[i]["bias"],
                                          self.layers[i]["experts"], w.k, w.act, flags, ws=self.ws,
                                          want_routing=True)
            self.distinct.append(int(torch.unique(idx).numel()) + w.n_shared)   # + the shared experts
            if self.active_groups is not None:
                self.active_groups.append(self._active_groups(idx))
        torch.cuda.synchronize()

    def _active_groups(self, idx):
        """16-neuron groups the zero-skip down projection of this call had to read: for each
        expert the call touches, the groups in which any of its pairs' h (the kernel's own, read
        back from the workspace) is nonzero.  Counted outside the timed region."""
        import torch
        import sparse_moe_expert_router_amd as moe
        w = self.w
        h = moe.read_intermediates(w.T, w.k, self.layers[0]["experts"], w.act, self.flags, self.ws)
        rows = h.shape[0]
        live = (h.view(rows, w.d_ff // 16, 16) != 0).any(-1)             # [pair row][group]
        ex_of_row = torch.cat([idx.reshape(-1).long(),
                               (w.E + torch.arange(w.n_shared, device=h.device)).repeat_interleave(w.T)])
        per_expert = torch.zeros((w.E + w.n_shared, w.d_ff // 16), dtype=torch.int32, device=h.device)
        per_expert.index_add_(0, ex_of_row, live.int())
        return int((per_expert > 0).sum())

    def step(self):
        import sparse_moe_expert_router_amd as moe
        w = self.w
        for i in range(self.L):
            lay = self.layers[i]
            moe.layer_forward(self.xs[i], lay["w_router"], lay["bias"], lay["experts"], w.k, w.act,
                              self.flags, out=self.outs[i], ws=self.ws)

    def capture(self):
        """One step (the L layer calls) captured as a HIP graph, replayed by the timed loop."""
        import torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        torch.cuda.synchronize()
        return g

    def time(self, steps, warmup, graph=True):
        import torch
        run = self.step
        if graph:
            g = self.capture()
            run = g.replay
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        # one event after every step (a marker between graph launches), so that per-step times
        # come from the same timed region as the total
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            run()
            ev[i + 1].record()
        torch.cuda.synchronize()
        self.step_s = [ev[i].elapsed_time(ev[i + 1]) / 1000.0 for i in range(steps)]
        return ev[0].elapsed_time(ev[steps]) / 1000.0

    def kernel_times(self, steps):
        """Average milliseconds per launch of each kernel, from HIP events around each launch."""
        import torch
        import sparse_moe_expert_router_amd as moe
        torch.cuda.synchronize()
        moe.profile_reset()
        moe.profile_enable(True)
        try:
            for _ in range(steps):
                self.step()
            torch.cuda.synchronize()
            res = moe.profile_collect()
        finally:
            moe.profile_enable(False)
        return {k: (n, ms / n) for k, (n, ms) in res.items()}

    def algorithmic_ops(self):
        """Multiply-adds x 2 per layer call of the prefill GEMMs (int8 or E4M3): for each of the
        P = T k pairs, the gate/up rows (2 d_ff with SwiGLU, d_ff with ReLU^2) times d_model, and
        the down projection's d_model x d_ff (6 P d d_ff with SwiGLU)."""
        w = self.w
        return 2 * w.T * w.k * (w.gate_up_rows * w.d_model + w.d_model * w.d_ff)

    def group_bytes(self):
        """Bytes of one 16-neuron group of an E2M1 down matrix: 16 rows of d_model codes (half a
        byte each) and the group's d_model fp16 scales."""
        return 16 * self.w.d_model // 2 + 2 * self.w.d_model

    def algorithmic_bytes(self):
        """Per layer call, averaged over the L instances: (gate/up kernel bytes, whole layer bytes).

        What the method itself must move, not the workspace it keeps between kernels (h, y and the
        routing records stay out).  Gate/up kernel: the distinct experts' gate/up weights and scales
        and the activations it reads (x, or on the int8 / fp8 prefill paths the 1-byte codes of x
        and their fp32 scales).  Layer: every weight byte of the distinct experts (with zero-skip,
        of the down matrices only the active 16-neuron groups, counted from the kernel's own h),
        the router, x and out.
        """
        w = self.w
        xb = w.T * w.d_model * (2 if w.xtype == 1 else 4)
        D = sum(self.distinct) / len(self.distinct)
        gu_w = D * expert_gateup_bytes(w)
        if self.flags & (4 | 8):
            gu = gu_w + w.T * (w.d_model + 4)
        else:
            gu = gu_w + xb
        dn = D * expert_down_bytes(w)
        if self.active_groups is not None:
            dn = sum(self.active_groups) / len(self.active_groups) * self.group_bytes()
        router = w.E * w.d_model * 4
        out = w.T * w.d_model * 4
        return gu, gu_w + xb + dn + router + out


def variant_specs():
    """The variant workloads timed beside the headline: (workload, layer instances, flags, label);
    a label holding "plain" times the plain row-major int8 layout."""
    import moe_inputs as mi
    return [
        (mi.workload("gemma_decode", T=1), 30, 0, "gemma_decode q8_0"),
        (mi.workload("gemma_decode", T=8), 30, 0, "gemma_decode q8_0 plain layout"),
        (mi.workload("gemma_decode", T=8, fmt=mi.FMT_I8_ROW), 30, 0, "gemma_decode i8_row"),
        (mi.workload("gemma_decode", T=1, fmt=mi.FMT_I8_ROW), 30, 0, "gemma_decode i8_row"),
        (mi.workload("m3_decode", T=1), 8, 0, "m3_decode q8_0"),
        (mi.workload("m3_decode", T=32), 8, 0, "m3_decode q8_0"),
        (mi.workload("nemotron_latent", T=1), 30, 1, "nemotron_latent zero-skip"),
        (mi.workload("nemotron_latent", T=1), 30, 0, "nemotron_latent dense-down"),
        (mi.workload("nemotron_latent", T=8), 30, 1, "nemotron_latent zero-skip batched"),
        (mi.workload("gemma_decode", T=8, fmt=mi.FMT_E2M1), 8, 0, "gemma_decode e2m1 swiglu"),
        (mi.workload("gemma_decode", T=8, n_shared=1), 30, 0, "gemma_decode q8_0 + shared expert"),
        (mi.workload("gemma_prefill", T=2048), 4, 4, "gemma_prefill int8 MFMA"),
        (mi.workload("gemma_prefill", T=2048, fmt=mi.FMT_Q8_0), 4, 4, "gemma_prefill int8 MFMA q8_0 weights"),
        (mi.workload("gemma_prefill", T=2048, fmt=mi.FMT_FP8_ROW), 4, 8, "gemma_prefill fp8 (E4M3) per-row"),
    ]


def traffic_key(w, flags, tiled):
    """Workload key of a stored HBM-traffic reading (profiles/traffic.json)."""
    import moe_inputs as mi
    fmt = {mi.FMT_Q8_0: "q8_0", mi.FMT_I8_ROW: "i8_row", mi.FMT_E2M1: "e2m1", mi.FMT_FP8_ROW: "fp8_row"}[w.fmt]
    lay = "tiled" if tiled and w.fmt != mi.FMT_E2M1 else "plain"
    shared = f":shared={w.n_shared}" if w.n_shared else ""
    return f"{w.name}:T={w.T}:{fmt}:{lay}:flags={flags}{shared}"


def run_case(w, L, steps, warmup, flags=0, label=None, tiled=True, roofline=True):
    """Time L distinct instances of workload w (HIP-graph replay, then eager, then per-kernel HIP
    events) and derive the roofline figures; roofline=False reports the time only."""
    import torch
    c = Case(w, L, flags, tiled)
    elapsed = c.time(steps, warmup, graph=True)
    per_step = sorted(c.step_s)
    eager = c.time(max(2, steps // 2), 1, graph=False)
    kt = c.kernel_times(max(2, min(steps, 5)))
    gu_bytes, layer_bytes = c.algorithmic_bytes()
    calls = steps * L
    res = {
        "workload": label or w.name, "T": w.T, "layers": L, "steps": steps,
        "tokens_per_s": w.T * calls / elapsed, "ms_per_layer": 1e3 * elapsed / calls,
        "ms_per_layer_median": 1e3 * per_step[len(per_step) // 2] / L, "ms_per_layer_min": 1e3 * per_step[0] / L,
        "eager_ms_per_layer": 1e3 * eager / (max(2, steps // 2) * L),
        "distinct_experts_mean": sum(c.distinct) / len(c.distinct),
        "kernels_ms": {k: round(v[1], 5) for k, v in kt.items()},
    }
    if c.active_groups is not None:
        res["active_groups_mean"] = sum(c.active_groups) / len(c.active_groups)
        res["active_group_frac"] = res["active_groups_mean"] / (res["distinct_experts_mean"] * (w.d_ff // 16))
    if not roofline:
        del c
        torch.cuda.empty_cache()
        return res
    res["layer_algorithmic_bytes"] = layer_bytes
    res["layer_hbm_gbs"] = layer_bytes * calls / elapsed / 1e9
    res["layer_hbm_frac"] = res["layer_hbm_gbs"] / HBM_PEAK_GBS
    from sparse_moe_expert_router_amd import profiling
    dom = "gateup_int8" if "gateup_int8" in kt else ("up_e2m1" if "up_e2m1" in kt else None)
    if "ggemm_gateup_i8" in kt:
        fp8 = bool(flags & 8)
        ops = c.algorithmic_ops()
        gu_ms = kt["ggemm_gateup_i8"][1]
        gu_ops = ops * 2 / 3
        peak = F8_PEAK_TFLOPS if fp8 else I8_PEAK_TOPS    # the peak of the contraction's own type
        res["mfma_tops"] = ops * calls / elapsed / 1e12
        res["mfma_peak"] = peak
        res["mfma_frac"] = res["mfma_tops"] / peak
        if fp8:                                        # the f16 matrix cores that multiply the codes
            res["mfma_instruction_peak"] = F16_PEAK_TFLOPS
            res["mfma_frac_of_instruction_peak"] = res["mfma_tops"] / F16_PEAK_TFLOPS
        # the whole layer against its binding roof: the weights (and x, out, router) at the HBM
        # peak outlast its ops at the matrix-core peak
        t_bound = max(layer_bytes / (HBM_PEAK_GBS * 1e9), ops / (peak * 1e12))
        res["layer_bound_frac"] = t_bound / (elapsed / calls)
        traffic = profiling.load_traffic(os.path.join(ROOT, "profiles"), "ggemm_gateup_i8",
                                         traffic_key(w, flags, tiled))
        t_hbm, t_mfma = gu_bytes / (HBM_PEAK_GBS * 1e9), gu_ops / (peak * 1e12)
        mfma_ach = gu_ops / (gu_ms / 1e3) / 1e12
        if t_hbm >= t_mfma:
            ach = gu_bytes / (gu_ms / 1e3) / 1e9
            res["roofline"] = {"kernel": "ggemm_gateup_i8", "bound": "hbm", "achieved": ach,
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                               "traffic": traffic, "algorithmic_bytes_per_launch": gu_bytes,
                               "avg_launch_ms": gu_ms, "mfma_tops": mfma_ach,
                               "mfma_frac": mfma_ach / peak}
        else:
            res["roofline"] = {"kernel": "ggemm_gateup_i8", "bound": "mfma", "achieved": mfma_ach,
                               "peak": peak, "unit": "TOP/s", "frac": mfma_ach / peak,
                               "traffic": traffic, "algorithmic_ops_per_launch": gu_ops,
                               "avg_launch_ms": gu_ms}
        res["roofline"]["layer"] = {"bound": "hbm", "achieved": res["layer_hbm_gbs"], "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": res["layer_hbm_frac"],
                                    "mfma_frac": res["mfma_frac"], "bound_frac": res["layer_bound_frac"]}
        dom = None
    if dom:
        avg_ms = kt[dom][1]
        ach = gu_bytes / (avg_ms / 1e3) / 1e9
        traffic = profiling.load_traffic(os.path.join(ROOT, "profiles"), dom, traffic_key(w, flags, tiled))
        res["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": traffic,
                           "algorithmic_bytes_per_launch": gu_bytes, "avg_launch_ms": avg_ms,
                           "layer": {"bound": "hbm", "achieved": res["layer_hbm_gbs"], "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": res["layer_hbm_frac"],
                                     "algorithmic_bytes_per_call": layer_bytes}}
    del c
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, seconds):
    """The oracle (plain fp64 C, as it stands) on layer instance 0 of the workload, on this host."""
    import moe_inputs as mi
    import oracle
    oracle.build(force=False)
    lay = mi.to_host(mi.make_layer(w, 0, "cuda"))
    x = mi.make_x(w, 0, device="cuda").cpu()
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 1000:
            break
    omp_threads = oracle.get_threads()
    cores = len(os.sched_getaffinity(0))
    # the same forward on one thread (a bounded sample: at least one call, up to ~4 s)
    oracle.set_threads(1)
    try:
        n1, t1 = 0, time.perf_counter()
        while True:
            oracle.layer_forward(x, lay["w_router"], lay["bias"], lay["experts"], w.k, w.act)
            n1 += 1
            el1 = time.perf_counter() - t1
            if el1 >= min(4.0, seconds / 3) or n1 >= 1000:
                break
    finally:
        oracle.set_threads(omp_threads)
    return {"value": w.T * n / el, "unit": "MoE-layer tokens/s", "cores": cores,
            "omp_threads": omp_threads, "kind": "oracle",
            "sample": f"{n} full layer forwards (router + experts, fp64) of instance 0 of the "
                      f"{w.name} workload at T={w.T}, {el:.1f} s; one thread: {n1} forwards, {el1:.1f} s",
            "value_one_core": w.T * n1 / el1}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the layer runs on one GPU's share of experts or tokens). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_inputs as mi
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return

    fmt = mi.FMT_NAMES[args.fmt]
    w = mi.workload(args.workload, T=args.T, fmt=fmt, n_shared=args.n_shared)
    L = args.layers or w.instances
    print(f"# headline: {w.name} T={w.T} fmt={args.fmt} layers={L}", file=sys.stderr, flush=True)
    head = run_case(w, L, args.steps, args.warmup, args.flags, tiled=not args.plain)
    print(f"# headline done: {head['tokens_per_s']:.0f} tok/s", file=sys.stderr, flush=True)

    variants = []
    if not args.no_variants:
        print("# variant: tiny T=4 (time only)", file=sys.stderr, flush=True)
        variants.append(run_case(mi.workload("tiny"), 1, max(5, args.steps // 2), 2, 0, "tiny q8_0",
                                 tiled=False, roofline=False))
        specs = variant_specs()
        for vw, vl, vf, label in specs:
            print(f"# variant: {label} T={vw.T}", file=sys.stderr, flush=True)
            r = run_case(vw, vl, max(5, args.steps // 2), 2, vf, label, tiled="plain" not in label)
            variants.append(r)

    cpu = None
    if not args.no_cpu_baseline:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_seconds)

    line = {
        "metric": "MoE-layer tokens/s + achieved HBM GB/s (decode) / int8 MFMA % (prefill)",
        "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_layer"] * L,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8-weights/bf16-act/fp32-acc",
        "data": "synthetic (seeded N(0, 0.02^2) weights quantised to Q8_0; bf16 N(0,1) activations)",
        "config": {"workload": f"{w.name}: T={w.T}, d_model={w.d_model}, E={w.E}, top-{w.k}, "
                               f"d_ff={w.d_ff}, SwiGLU, {args.fmt} ({'plain' if args.plain else 'tiled'} "
                               f"layout), {L} distinct layers",
                   "global_batch": w.T, "parallelism": "single GPU"},
        "roofline": head.get("roofline"),
        "cpu_baseline": cpu,
        "layer_hbm_gbs": head["layer_hbm_gbs"], "layer_hbm_frac": head["layer_hbm_frac"],
        "eager_ms_per_layer": head["eager_ms_per_layer"],
        "ms_per_layer_median": head["ms_per_layer_median"], "ms_per_layer_min": head["ms_per_layer_min"],
        "timing": "HIP graph replay of one step",
        "kernels_ms": head["kernels_ms"], "distinct_experts_mean": head["distinct_experts_mean"],
        "variants": variants,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
