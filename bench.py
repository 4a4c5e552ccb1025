"""Throughput of the MXFP4 mixture-of-experts expert projection on one MI355X.

A step is one pass of the hot path over one batch of seeded synthetic input:
route + group (mxfp4_moe_route_group), the expert projection
(mxfp4_expert_proj) and, for workloads that have one, the gate-weighted
combine (moe_combine).  A one-token workload routed from logits runs route,
group and projection as one launch (mxfp4_moe_decode, same outputs); the
three-call step is reported beside it.  The headline workload is the gpt-oss-20b gate_up
decode of one token (E=32 experts of [5760, 2880] MXFP4, top-4 from bf16
router logits).  Inputs are resident in HBM before the timed region; every
step reads a different copy of the expert weights (enough copies that one
rotation touches >= 1 GiB) so that the 256 MB last-level cache cannot serve
the weights.  The timed steps are replayed from a HIP graph.

Prints one JSON line.  See --help for the options.
"""
from __future__ import annotations

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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MXFP4_PEAK_TFLOPS = 10100.0    # MI355X dense MXFP4 MFMA, published
METRIC = "MXFP4 expert-proj HBM GB/s (decode) & TFLOP/s (prefill), % of MI355X roofline"
ROTATE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expert_gemv_gate_up_decode_t1.traffic.txt")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "expert_gemm_gate_up_prefill_t4096.traffic.txt")
# the FP6 x FP4 scaled MFMA's sustained rate measured on this part (independent
# v_mfma_scale_f32_32x32x64_f8f6f4 on every CU), halved: each product takes two
# terms, so this is the grouped GEMM's ceiling in algorithmic flops
TWO_TERM_CEILING_TFLOPS = 7700.0 / 2
# The pages' own measured numbers, quoted in the line for context only: whole-
# model decode rates on one NVIDIA H100 80GB (batch 1, 512 prompt + 128 new
# tokens), not a kernel metric, so no ratio is formed with them.
PUBLISHED_CONTEXT = {
    "note": "end-to-end decode tok/s of whole models on one NVIDIA H100 80GB, as the pages report them; "
            "a different metric, workload and machine (vs_baseline stays null)",
    "gpt2_124m_decode_tok_s": {"transformers_eager": 175.29, "transformers_torch_compile": 419.13, "vllm": 696.25,
                               "source": "GPT-2 files page, bench.json (methods)"},
    "gpt_oss_20b_decode_tok_s": {"mxfp4_bytes_read_in_place": 270, "from_dequantized_experts": 202,
                                 "source": "gpt-oss-20b files page, README \"Entries\" (PyTorch on CUDA, H100)"},
}
KERNEL_SOURCES = {
    "expert_gemv": ["mxfp4_mixture_experts_amd/csrc/expert_gemv.hip", "mxfp4_mixture_experts_amd/csrc/common.h",
                    "mxfp4_mixture_experts_amd/csrc/route_common.h"],
    "expert_gemm": ["mxfp4_mixture_experts_amd/csrc/expert_gemm.hip", "mxfp4_mixture_experts_amd/csrc/common.h"],
}


def kernel_source_hash(name: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[name]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, path: str = TRAFFIC_FILE):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source (else None)."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, v = line.split(":", 1)
                vals[key.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ accounting
def algorithmic(p, used, swiglu=False):
    """Minimum bytes each stage must move and the flops of the projection; `used` is the
    number of experts that received at least one routed row.  swiglu: the projection
    writes the bf16 gated activation [T, k, N / 2] instead of fp32 [T, k, N]."""
    KB = p.K // 32
    R = p.T * p.k
    weights = used * p.N * (KB * 16 + KB + 2)           # code blocks + scale bytes + bias
    x = (R if p.x_per_slot else p.T) * p.K * 2
    out = R * (p.N // 2) * 2 if swiglu else R * p.N * 4
    grouping_in = (p.E + 1) * 4 + R * 4
    proj = weights + x + out + grouping_in
    route = (p.T * p.E * 2 if p.logits is not None else 0) + (R * 4 if p.ids_in is not None else 0)
    route += R * 4 + (R * 4 if p.logits is not None else 0) + (p.E + 1) * 4 + R * 4
    comb = (R * p.N * 4 + R * 4 + p.T * p.N * 4) if (p.combine and p.logits is not None and not swiglu) else 0
    flops = 2.0 * R * p.N * p.K
    return {"proj": proj, "route": route, "combine": comb, "step": proj + route + comb, "flops": flops,
            "experts_touched": int(used), "weight_bytes": weights}


# ------------------------------------------------------------------ GPU measurement
def fusable(p):
    """A decode batch routed from logits within the single-launch decode's limits (up to 64
    tokens and 64 experts, K <= 3072), on the projection's automatic path (the GEMV)."""
    R = p.T * p.k
    return (1 <= p.T <= 64 and p.logits is not None and p.ids_in is None and p.E <= 64 and p.K <= 3072
            and R <= 16 * min(R, p.E))


class Workload:
    def __init__(self, cfg_index: int, rotate_bytes: int, path: int = 0, fused: bool = False, swiglu: bool = False,
                 combine_fused: bool = False):
        import torch
        from mxfp4_mixture_experts_amd import synthetic as S
        from mxfp4_mixture_experts_amd.runner import DeviceProblem
        self.torch = torch
        # a workload index, or a problem built by the caller
        self.p = S.make_config(cfg_index) if isinstance(cfg_index, int) else cfg_index
        self.fused = fused and fusable(self.p)
        self.swiglu = swiglu
        # many tokens: the projection with the combine fused in (mxfp4_expert_proj_combine_routed)
        self.combine_fused = combine_fused and self.p.combine and self.p.logits is not None and not swiglu
        self.dp = DeviceProblem(self.p, device="cuda:0", path=path)
        self.dp.route_group()            # the device's own routing decides which experts are touched
        counts = torch.diff(self.dp.offsets.to(torch.int64)).cpu().numpy()
        self.acc = algorithmic(self.p, int((counts > 0).sum()), swiglu)
        touched = max(self.acc["weight_bytes"], 1)
        self.copies = max(1, math.ceil(rotate_bytes / touched))
        self.weights = [(self.dp.blocks, self.dp.scales)]
        for _ in range(self.copies - 1):
            self.weights.append((self.dp.blocks.clone(), self.dp.scales.clone()))
        torch.cuda.synchronize()

    def step(self, i, stream=None):
        b, s = self.weights[i % self.copies]
        if self.combine_fused:
            self.dp.route_group(stream)
            self.dp.proj_combine_routed(stream, blocks=b, scales=s)
            return
        if self.fused and self.swiglu:
            self.decode_swiglu(stream, blocks=b, scales=s)
            return
        if self.fused:
            self.decode(stream, blocks=b, scales=s)
        elif self.swiglu:
            self.dp.route_group(stream)
            self.dp.expert_proj_swiglu(stream, blocks=b, scales=s)
            return
        else:
            self.dp.route_group(stream)
            self.dp.expert_proj(stream, blocks=b, scales=s)
        self.dp.combine(stream)

    def proj_only(self, i, stream=None):
        """The dominant kernel alone: the projection (the single-launch decode when fused)."""
        b, s = self.weights[i % self.copies]
        if self.combine_fused:
            self.dp.proj_combine_routed(stream, blocks=b, scales=s)
        elif self.fused and self.swiglu:
            self.decode_swiglu(stream, blocks=b, scales=s)
        elif self.fused:
            self.decode(stream, blocks=b, scales=s)
        elif self.swiglu:
            self.dp.expert_proj_swiglu(stream, blocks=b, scales=s)
        else:
            self.dp.expert_proj(stream, blocks=b, scales=s)

    def decode(self, stream, blocks, scales):
        """The single-launch decode: mxfp4_moe_decode for one token, mxfp4_moe_decode_batch beyond."""
        if self.p.T == 1:
            self.dp.decode(stream, blocks=blocks, scales=scales)
        else:
            self.dp.decode_batch(stream, blocks=blocks, scales=scales)

    def decode_swiglu(self, stream, blocks, scales):
        if self.p.T == 1:
            self.dp.decode_swiglu(stream, blocks=blocks, scales=scales)
        else:
            self.dp.decode_batch_swiglu(stream, blocks=blocks, scales=scales)

    def capture(self, fn, n):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)                      # one eager call on the capture stream before capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        torch.cuda.synchronize()
        return g

    def time_graph(self, g):
        """(event ms, wall s) of one replay, bracketed by synchronisation."""
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return e0.elapsed_time(e1), t1 - t0


def measure(cfg_index, steps, warmup, rotate_bytes, path=0, kernel_reps=None, fused=False, swiglu=False,
            combine_fused=False):
    """Time `steps` whole-path steps and, separately, back-to-back launches of the
    projection alone (for the kernel's roofline)."""
    w = Workload(cfg_index, rotate_bytes, path, fused, swiglu, combine_fused)
    for i in range(warmup):
        w.step(i)
    w.torch.cuda.synchronize()
    g_steps = w.capture(w.step, steps)
    for _ in range(3):                    # untimed: the instantiated graph's first replays (clocks settle)
        g_steps.replay()
    ms_total, wall = w.time_graph(g_steps)
    kreps = kernel_reps or steps
    g_proj = w.capture(w.proj_only, kreps)
    g_proj.replay()
    # the kernel's own time: the median of five replays of the back-to-back launches
    ms_proj = sorted(w.time_graph(g_proj)[0] for _ in range(5))[2]
    res = {
        "p": w.p, "acc": w.acc, "copies": w.copies, "steps": steps, "fused": w.fused, "combine_fused": w.combine_fused,
        "ms_per_step": ms_total / steps, "wall_s": wall,
        "proj_us": 1e3 * ms_proj / kreps,
    }
    del g_steps, g_proj, w
    return res


def describe(p, swiglu=False):
    name = {
        "tiny": "tiny",
        "gate_up_decode_t1": "gpt-oss-20b gate_up decode",
        "down_decode_t64": "gpt-oss-20b down decode",
        "gate_up_prefill_t4096": "gpt-oss-20b gate_up prefill",
        "down_prefill_zipf_t2048": "gpt-oss-20b down prefill, Zipf(1.2) routing",
        "gate_up_decode_t4": "gpt-oss-20b gate_up decode of a 4-token batch",
        "down_decode_t4": "gpt-oss-20b down decode of a 4-token batch",
    }[p.name]
    if swiglu:
        return (f"{name} + gated activation: E={p.E} N={p.N} K={p.K} T={p.T} top-{p.k}, MXFP4 blocks "
                f"[{p.E},{p.N},{p.K // 32},16] + E8M0 scales, bf16 x [T,K], bf16 activation out [T,k,N/2]")
    return (f"{name}: E={p.E} N={p.N} K={p.K} T={p.T} top-{p.k}, MXFP4 blocks [{p.E},{p.N},{p.K // 32},16] "
            f"+ E8M0 scales, bf16 x {'[T,k,K]' if p.x_per_slot else '[T,K]'}, fp32 out [T,k,N]"
            + (" + combine [T,N]" if p.combine else ""))


def measure_dequant(cfg_index, reps, rotate_bytes):
    """mxfp4_dequantize of a workload's whole expert weight tensor to bf16 (the
    load-time dequantization), weights rotated over copies; graph of `reps`
    launches.  Returns (us per launch, bytes per launch)."""
    import torch
    from mxfp4_mixture_experts_amd import binding as B
    from mxfp4_mixture_experts_amd import synthetic as S
    p = S.make_config(cfg_index)
    blocks = torch.from_numpy(p.blocks).cuda()
    scales = torch.from_numpy(p.scales).cuda()
    copies = max(1, math.ceil(rotate_bytes / (blocks.numel() + scales.numel())))
    ws = [(blocks, scales)] + [(blocks.clone(), scales.clone()) for _ in range(copies - 1)]
    out = torch.empty((p.E, p.N, p.K), dtype=torch.bfloat16, device="cuda")
    B.mxfp4_dequantize(blocks, scales, out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            B.mxfp4_dequantize(ws[i % copies][0], ws[i % copies][1], out)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = blocks.numel() + scales.numel() + out.numel() * 2
    del g, ws, out
    return us, nbytes, copies


def _graph_us(fn, reps):
    """us per call of fn(i) over a graph of `reps` back-to-back calls (one untimed replay first)."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del g
    return us


def measure_router(T, reps, rotate_bytes, H=2880, E=32):
    """mxfp4_moe_router at the gpt-oss-20b widths (H = 2880, E = 32): us per launch
    and algorithmic bytes (x, w, bias, logits); inputs rotated over copies (at most
    64, so a one-token router's inputs stay within the last-level cache)."""
    import torch
    from mxfp4_mixture_experts_amd import binding as B
    from mxfp4_mixture_experts_amd import synthetic as S
    r = S.make_router(T, H, E)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    x, w, b = bf(r.x), bf(r.w), bf(r.bias)
    nbytes = (T * H + E * H + E + T * E) * 2
    copies = max(1, min(64, math.ceil(rotate_bytes / ((T + E) * H * 2))))
    ins = [(x, w)] + [(x.clone(), w.clone()) for _ in range(copies - 1)]
    logits = torch.empty((T, E), dtype=torch.bfloat16, device="cuda")
    us = _graph_us(lambda i: B.mxfp4_moe_router(ins[i % copies][0], ins[i % copies][1], b, T, H, E, logits), reps)
    del ins
    return us, nbytes, copies


def measure_block_decode(reps, rotate_bytes):
    """The whole MoE block for one gpt-oss-20b token, three launches: router ->
    routing + gate/up through the gated activation (mxfp4_moe_decode_swiglu) -> down
    projection of the activations with the combine (mxfp4_expert_proj_combine).  Expert weights rotated over copies (>= rotate_bytes of
    touched weights per rotation).  Returns (us per token, algorithmic bytes, copies)."""
    import torch
    from mxfp4_mixture_experts_amd import binding as B
    from mxfp4_mixture_experts_amd import synthetic as S
    from mxfp4_mixture_experts_amd.runner import DeviceProblem
    H, E, k = 2880, 32, 4
    r = S.make_router(1, H, E)
    gu = S.make_config(1)
    gu.x = r.x
    dn = S.make_custom(E=E, N=H, K=2880, T=1, k=k, x_per_slot=True, route="logits", tag=97, combine=True)
    d1, d2 = DeviceProblem(gu), DeviceProblem(dn)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    rw, rb = bf(r.w), bf(r.bias)
    # the down projection reads the gate/up activations and the gate/up routing
    d2.x = d1.act
    d2.topk_ids, d2.gates, d2.offsets, d2.sorted_rows = d1.topk_ids, d1.gates, d1.offsets, d1.sorted_rows
    acc_gu = algorithmic(gu, k, swiglu=True)
    acc_dn = algorithmic(dn, k)
    # router; routing + gate/up + activation; down with the combine (no per-slot outputs written)
    nbytes = ((H + E * H + E + E) * 2 + acc_gu["proj"] + acc_gu["route"]
              + acc_dn["proj"] - k * H * 4 + k * 4 + H * 4)
    touched = acc_gu["weight_bytes"] + acc_dn["weight_bytes"]
    copies = max(1, math.ceil(rotate_bytes / touched))
    wg = [(d1.blocks, d1.scales)] + [(d1.blocks.clone(), d1.scales.clone()) for _ in range(copies - 1)]
    wd = [(d2.blocks, d2.scales)] + [(d2.blocks.clone(), d2.scales.clone()) for _ in range(copies - 1)]

    def step(i):
        B.mxfp4_moe_router(d1.x, rw, rb, 1, H, E, d1.logits)
        d1.decode_swiglu(blocks=wg[i % copies][0], scales=wg[i % copies][1])
        d2.proj_combine(blocks=wd[i % copies][0], scales=wd[i % copies][1], with_out=False)

    us = _graph_us(step, reps)
    del wg, wd
    return us, nbytes, copies


# ------------------------------------------------------------------ CPU baseline
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg_index, min_seconds=10.0, max_reps=200):
    """The oracle as it stands, on this host's cores (BLAS threads = the CPUs this
    process may run on), on the whole headline step, repeated until at least
    min_seconds of work; then the same once on one thread for comparison."""
    from threadpoolctl import threadpool_info, threadpool_limits
    import oracle.moe_oracle as O
    from mxfp4_mixture_experts_amd import synthetic as S
    p = S.make_config(cfg_index)
    ids = p.ids_in if p.ids_in is not None else O.route_topk(p.logits, p.k)[0]
    acc = algorithmic(p, np.unique(ids).size)
    cores = len(os.sched_getaffinity(0))

    def run(limit, seconds):
        with threadpool_limits(limits=limit):
            used = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
            O.run_problem(p)                      # warm caches and thread pools
            reps, t0 = 0, time.perf_counter()
            while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < seconds):
                O.run_problem(p)
                reps += 1
            return (time.perf_counter() - t0) / reps, reps, used

    t_all, reps, used = run(cores, min_seconds)
    t_one, reps1, _ = run(1, min(min_seconds, 5.0))
    return {"value": round(acc["step"] / t_all / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "cpu_model": _cpu_model(), "cpus_available": cores,
            "value_one_thread": round(acc["step"] / t_one / 1e9, 4),
            "sample": f"the whole {p.name} step (route, group, projection{', combine' if p.combine else ''}) in "
                      f"float64 numpy: {reps} steps of {t_all * 1e3:.1f} ms each with BLAS on {used} threads "
                      f"(the LUT dequantization of the chosen experts is numpy on one thread); on one thread "
                      f"{t_one * 1e3:.1f} ms per step ({reps1} steps)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1, help="workload index 0..4 (default 1: gate_up decode T=1)")
    ap.add_argument("--rotate-bytes", type=int, default=ROTATE_BYTES)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other model-size workloads")
    ap.add_argument("--combine-fused", action="store_true",
                    help="many-token workloads with a combine: the projection with the combine fused in "
                         "(mxfp4_expert_proj_combine_routed) instead of expert_proj + moe_combine")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="run N plain 256 MiB device copies first (counter calibration under rocprofv3)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from mxfp4_mixture_experts_amd import binding as B
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    B.load_library()

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.calibrate_copy):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    head = measure(args.config, args.steps, args.warmup, args.rotate_bytes, fused=True,
                   combine_fused=args.combine_fused)
    p, acc = head["p"], head["acc"]
    # the projection's automatic path: the GEMV while the routed rows average at
    # most 16 per expert they touch, the grouped GEMM beyond
    R = p.T * p.k
    kernel = "expert_gemv" if R <= 16 * min(R, p.E) else "expert_gemm"
    gbs = acc["step"] / (head["ms_per_step"] * 1e-3) / 1e9
    # the fused launch moves the routing bytes too, the fused combine the combine's
    kernel_bytes = acc["proj"] + (acc["route"] if head["fused"] else 0) + (acc["combine"] if head["combine_fused"] else 0)
    proj_gbs = kernel_bytes / (head["proj_us"] * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "published_context": PUBLISHED_CONTEXT,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": describe(p),
            "seed": 0,
            "path": (("moe_decode" if p.T == 1 else "moe_decode_batch")
                     + " (route + group + GEMV in one launch)" if head["fused"] else
                     "route_group + " + ("expert_proj_combine_routed" if head["combine_fused"] else "expert_proj")
                     + "(auto: " + ("GEMV" if kernel == "expert_gemv" else "GEMM") + ")")
                    + (" + combine" if p.combine and not head["combine_fused"] else ""),
            "algorithmic_bytes_per_step": acc["step"],
            "experts_touched": acc["experts_touched"],
            "weight_copies_rotated": head["copies"],
            "timing": "HIP graph replay of the timed steps; events on the replay stream",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(proj_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(proj_gbs / HBM_PEAK_GBS, 4),
            "traffic": read_traffic(kernel),
            "kernel_us": round(head["proj_us"], 3),
            "algorithmic_bytes_per_launch": kernel_bytes,
        },
    }
    if head["fused"]:
        # the same step as three launches (route_group, expert_proj, combine)
        three = measure(args.config, args.steps, args.warmup, args.rotate_bytes, fused=False)
        line["config"]["three_call_step"] = {
            "ms_per_step": round(three["ms_per_step"], 6),
            "GBps": round(acc["step"] / (three["ms_per_step"] * 1e-3) / 1e9, 2),
            "expert_proj_us": round(three["proj_us"], 3),
        }
    if not args.no_secondary:
        sec = []
        # the other model-size workloads, then the two gate_up workloads through
        # the fused gated activation (bf16 [T, k, N / 2], the down projection's input)
        # (the one-token one as a single launch, mxfp4_moe_decode_swiglu)
        # (and the down prefill once more with the combine fused into the grouped GEMM)
        # (the down decode of 64 tokens both as three calls and as one launch,
        # mxfp4_moe_decode_batch, with the combine after it)
        # (and a decode batch of 4 tokens at gate_up, both ways: the one-row-per-workgroup GEMV)
        # (and one at down with the combine, as three calls and with the projection
        # and the combine in one launch, mxfp4_expert_proj_combine_routed on the GEMV path)
        from mxfp4_mixture_experts_amd import synthetic as S
        p4 = S.make_custom(E=32, N=5760, K=2880, T=4, k=4, route="logits", tag=1204)
        p4.name = "gate_up_decode_t4"
        p4d = S.make_custom(E=32, N=2880, K=2880, T=4, k=4, x_per_slot=True, route="logits", combine=True, tag=1205)
        p4d.name = "down_decode_t4"
        for cfg, steps, swiglu, cf, fz in ((2, 100, False, False, False), (2, 100, False, False, True),
                                           (p4, 200, False, False, False), (p4, 200, False, False, True),
                                           (p4d, 200, False, False, False), (p4d, 200, False, True, False),
                                           (3, 20, False, False, False), (4, 40, False, False, False),
                                           (1, 200, True, False, True), (3, 20, True, False, False),
                                           (4, 40, False, True, False)):
            r = measure(cfg, steps, 5, args.rotate_bytes, kernel_reps=steps, swiglu=swiglu, fused=fz,
                        combine_fused=cf)
            a = r["acc"]
            if cfg == 3 and not swiglu:
                # the prefill half of the metric: the grouped GEMM at the gate_up prefill
                tf = a["flops"] / (r["proj_us"] * 1e-6) / 1e12
                line["roofline_prefill"] = {
                    "bound": "mfma",
                    "kernel": "expert_proj grouped-GEMM path: prepare_kernel + expert_gemm_kernel",
                    "workload": describe(r["p"]),
                    "achieved": round(tf, 1),
                    "peak": MXFP4_PEAK_TFLOPS,
                    "unit": "TFLOP/s",
                    "frac": round(tf / MXFP4_PEAK_TFLOPS, 4),
                    "frac_of_two_term_ceiling": round(tf / TWO_TERM_CEILING_TFLOPS, 4),
                    "kernel_us": round(r["proj_us"], 2),
                    "algorithmic_flops_per_launch": a["flops"],
                    "algorithmic_bytes_per_launch": a["proj"],
                    "GBps": round(a["proj"] / (r["proj_us"] * 1e-6) / 1e9, 1),
                    "traffic": read_traffic("expert_gemm", PREFILL_TRAFFIC_FILE),
                }
            t_step = r["ms_per_step"] * 1e-3
            t_proj = r["proj_us"] * 1e-6
            roof_t = max(a["flops"] / (MXFP4_PEAK_TFLOPS * 1e12), a["step"] / (HBM_PEAK_GBS * 1e9))
            # the single launch routes too; the fused combine reads and writes the combine's bytes
            a_proj = a["proj"] + (a["route"] if r["fused"] else 0) + (a["combine"] if cf else 0)
            sec.append({
                "workload": describe(r["p"], swiglu)
                            + ((" (routing + projection + activation in one launch)" if swiglu else
                                " (routing, grouping and projection in one launch: mxfp4_moe_decode_batch"
                                + ("; then the combine)" if r["p"].combine else ")")) if r["fused"] else "")
                            + ((" (route_group + mxfp4_expert_proj_combine_routed: the projection and the "
                                "combine in one launch on the GEMV path; proj_us covers both)"
                                if r["p"].T * r["p"].k <= r["p"].E else
                                " (the combine fused into the grouped GEMM: route_group + "
                                "mxfp4_expert_proj_combine_routed; proj_us covers both)") if cf else ""),
                "ms_per_step": round(r["ms_per_step"], 4),
                "step_GBps": round(a["step"] / t_step / 1e9, 1),
                "step_TFLOPs": round(a["flops"] / t_step / 1e12, 2),
                "proj_us": round(r["proj_us"], 2),
                "proj_GBps": round(a_proj / t_proj / 1e9, 1),
                "proj_TFLOPs": round(a["flops"] / t_proj / 1e12, 2),
                "proj_frac_hbm": round(a_proj / t_proj / 1e9 / HBM_PEAK_GBS, 4),
                "proj_frac_mxfp4_peak": round(a["flops"] / t_proj / 1e12 / MXFP4_PEAK_TFLOPS, 4),
                "step_frac_combined_roofline": round(roof_t / t_step, 4),
                "weight_copies_rotated": r["copies"],
            })
        # the standalone dequantization of the gate_up weights (load-time mirror)
        us, nbytes, copies = measure_dequant(1, 20, args.rotate_bytes)
        sec.append({
            "workload": "gpt-oss-20b gate_up weights MXFP4 [32,5760,90,16] + scales -> bf16 [32,5760,2880] "
                        "(mxfp4_dequantize)",
            "kernel_us": round(us, 2),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_launch": nbytes,
            "weight_copies_rotated": copies,
        })
        # the router GEMV (mxfp4_moe_router) for one token and for a prompt
        for T, reps in ((1, 200), (4096, 40)):
            us, nbytes, copies = measure_router(T, reps, args.rotate_bytes)
            sec.append({
                "workload": f"gpt-oss-20b router: x bf16 [{T},2880] . w bf16 [32,2880]^T + bias -> bf16 logits "
                            f"[{T},32] (mxfp4_moe_router)",
                "kernel_us": round(us, 2),
                "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "bytes_per_launch": nbytes,
                "input_copies_rotated": copies,
            })
        # the whole MoE block for one token, three launches
        us, nbytes, copies = measure_block_decode(200, args.rotate_bytes)
        sec.append({
            "workload": "gpt-oss-20b MoE block, one token: router -> routing + gate_up + gated activation in one "
                        "launch (bf16 [1,4,2880]) -> down [32,2880,90,16] + combine [1,2880] in one launch",
            "us_per_token": round(us, 2),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_hbm": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_token": nbytes,
            "weight_copies_rotated": copies,
        })
        line["secondary"] = sec
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.config)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
