"""Benchmark of the decode-time Any-Precision MoE layer on one MI355X.

One step = one moe_layer_forward call (route + group + gate_up/SiLU + down + combine) over a
synthetic batch already resident in HBM.  The default workload is the largest single-GPU decode
configuration at mixed widths: a Qwen2-57B-A14B-shaped layer (H 3584, 64 experts of
intermediate 2560, top-8, committed widths per (expert, module) drawn from {3, 4, 6, 8}) with 128
decode tokens.  Weight copies are rotated so that the timed steps cannot be served from the
256-MB last-level cache.

Prints one JSON line: value = effective weight GB/s (algorithmic plane + LUT bytes of the blocks
one call reads, divided by the time per call); the rooflines of the gate_up and down kernels
(event times on the launch stream); the CPU oracle timed on the host cores; and, as
sub-records of the same line, every other layer shape of the pages' models (Qwen1.5-MoE-A2.7B
with its shared expert, Mixtral-8x7B, Qwen3-Next-80B-A3B with the Zipf router, the Qwen2 shape
at 1, 8 and 32 tokens, the tiny layer) and the 2048-token chunked prefill.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "µs per MoE decode layer + effective weight GB/s (% of MI355X HBM peak)"
HBM_PEAK_GBS = 8000.0
MFMA_FP16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix-core peak
PROFILES = os.path.join(ROOT, "profiles")
WORKLOADS = {
    "qwen2_57b_a14b_t128": wl.QWEN2_57B_A14B.with_tokens(128),
    "qwen15_moe_a27b": wl.QWEN15_MOE_A27B,
    "mixtral_8x7b": wl.MIXTRAL_8X7B,
    "qwen3_next_80b_a3b": wl.QWEN3_NEXT_80B_A3B,
    "qwen2_57b_a14b_t1": wl.QWEN2_57B_A14B.with_tokens(1),
    "qwen2_57b_a14b_t8": wl.QWEN2_57B_A14B.with_tokens(8),
    "qwen2_57b_a14b_t32": wl.QWEN2_57B_A14B.with_tokens(32),
    "qwen2_57b_a14b_prefill2048": wl.QWEN2_57B_A14B.with_tokens(wl.QWEN2_PREFILL_TOKENS),
    "tiny": wl.TINY,
}
DEFAULT_WORKLOAD = "qwen2_57b_a14b_t128"
# the other decode shapes, reported as sub-records of the default line; "all" = parity on every
# token of the call, else on these tokens (the GPU tests compare every token of every shape)
SUB_WORKLOADS = {
    "qwen15_moe_a27b": "all",
    "mixtral_8x7b": [0, 13, 31],
    "qwen3_next_80b_a3b": "all",
    "qwen2_57b_a14b_t1": "all",
    "qwen2_57b_a14b_t8": "all",
    "qwen2_57b_a14b_t32": [0, 17, 31],
    "tiny": "all",
}
KERNELS = {"apq_gate_up_silu": wl.GATE_UP, "apq_down": wl.DOWN}
DOMINANT = "apq_gate_up_silu"   # the largest byte mover of every decode shape
ENGINE_SOURCES = ["any_precision_expert_router_amd/csrc/apq_engine.hpp",
                  "any_precision_expert_router_amd/csrc/internal.hpp",
                  "any_precision_expert_router_amd/csrc/apq_gate_up.hip",
                  "any_precision_expert_router_amd/csrc/apq_down.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def engine_sha() -> str:
    h = hashlib.sha256()
    for rel in ENGINE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def module_bytes(shape, ids, module, widths):
    """(planes, LUT) bytes of one module over the active experts (+ shared)."""
    planes = lut = 0
    for e in np.unique(ids):
        r, c = wl.block_dims(shape, module, int(e))
        p, l = wl.algorithmic_weight_bytes(r, c, int(widths[e, module]))
        planes, lut = planes + p, lut + l
    if shape.I_shared:
        r, c = wl.block_dims(shape, module, wl.SHARED_EXPERT)
        p, l = wl.algorithmic_weight_bytes(r, c, shape.q_shared)
        planes, lut = planes + p, lut + l
    return planes, lut


def traffic_from_profile(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = os.path.join(PROFILES, f"{kernel}.{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("engine_sha") != engine_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """Host threads the oracle's BLAS may use: the process's cores, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(shape, inputs, budget_s: float, threads: int):
    """The float64 oracle on the host cores: one whole layer call (all tokens), median of runs."""
    import oracle
    from workloads import device as gpu_layers
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    get, sh = gpu_layers.oracle_getters(shape, cache_size=2 * shape.E)
    # draw the blocks first: generating inputs is not the oracle's work
    ids, _ = oracle.route_topk(inputs.logits, shape.k)
    for e in np.unique(ids):
        get(int(e), 0), get(int(e), 1)
    if sh:
        sh(0, 0), sh(0, 1)
    times = []
    ctx = threadpool_limits(limits=threads) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t_end = time.perf_counter() + budget_s
        while len(times) < 3 and (not times or time.perf_counter() + times[-1] < t_end):
            t0 = time.perf_counter()
            oracle.layer_forward(inputs.x, inputs.logits, shape.k, get, shared=sh)
            times.append(time.perf_counter() - t0)
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return statistics.median(times), len(times)


# ---------------------------------------------------------------------------------------------
# device layers and the timed call
# ---------------------------------------------------------------------------------------------
_copies_cache = {}


def layer_copies(apq, torch, shape, dev, copies_gb):
    """The layer's device blocks and page table, plus clones at other addresses (same bytes) so
    that the rotated copies exceed the last-level cache.  Shapes that differ only in their token
    count share one set of weights."""
    from workloads import device as gpu_layers
    key = (shape.workload_id, shape.E, shape.H, shape.I, shape.I_shared)
    if key in _copies_cache:
        return _copies_cache[key]
    _copies_cache.clear()
    torch.cuda.empty_cache()
    base = gpu_layers.device_layer(shape, device=dev)
    copies = [base]
    n_copies = max(1, int(np.ceil(copies_gb * 1e9 / base.weight_bytes)))
    for _ in range(n_copies - 1):
        c = object.__new__(apq.DeviceLayer)
        c.__dict__.update(base.__dict__)
        c.arena = base.arena.clone()
        delta = c.arena.data_ptr() - base.arena.data_ptr()
        tbl = base.table.view(torch.int64).reshape(-1, 4).clone()
        tbl[:, 0] += delta
        tbl[:, 1] += delta
        c.table = tbl.view(torch.uint8).reshape(-1)
        if base.shared is not None:
            sht = base.shared.view(torch.int64).reshape(-1, 4).clone()
            sht[:, 0] += delta
            sht[:, 1] += delta
            c.shared = sht.view(torch.uint8).reshape(-1)
        copies.append(c)
    _copies_cache[key] = copies
    return copies


class LayerCall:
    """One shape's inputs, outputs and workspace on the device, and its step over the copies."""

    def __init__(self, apq, torch, shape, copies, dev):
        self.apq, self.torch, self.shape, self.copies = apq, torch, shape, copies
        self.inputs = wl.gen_layer_inputs(shape)
        self.widths = wl.gen_widths(shape)
        T = shape.T
        self.logits = torch.from_numpy(self.inputs.logits).to(dev)
        self.x = torch.from_numpy(self.inputs.x).to(dev)
        self.y = torch.empty((T, shape.H), dtype=torch.float16, device=dev)
        self.ws = torch.zeros(apq.moe_workspace_bytes(T, shape.E, shape.H, shape.I, shape.k, shape.I_shared),
                              dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()

    def step(self, i, stream=None):
        s, c = self.shape, self.copies[i % len(self.copies)]
        self.apq.moe_layer_forward(self.logits, self.x, s.E, s.H, s.I, s.k, c.table, self.y, self.ws,
                                   shared=c.shared, I_shared=s.I_shared,
                                   stream=self.stream if stream is None else stream)


def check_parity(call, tokens):
    """Layer output of one call against the float64 oracle: relative L2 over the checked tokens
    (all of them, or a list), and the worst single token."""
    from workloads import device as gpu_layers
    import oracle
    shape = call.shape
    call.step(0)
    call.apq.moe_check_device_error(call.ws)
    get, sh = gpu_layers.oracle_getters(shape, cache_size=2 * shape.E + 2)
    toks = list(range(shape.T)) if tokens == "all" else list(tokens)
    ref = oracle.layer_forward(call.inputs.x, call.inputs.logits, shape.k, get, shared=sh,
                               tokens=None if tokens == "all" else toks)
    yc = call.y.float().cpu().numpy()
    err = oracle.rel_l2(yc[toks], ref["y"][toks])
    worst = max(oracle.rel_l2(yc[t], ref["y"][t]) for t in toks)
    log(f"[bench] parity {shape.name} T={shape.T} on {'all' if tokens == 'all' else toks} tokens: "
        f"rel L2 {err:.2e} (worst token {worst:.2e})")
    assert err <= 1e-3, err
    return {"tokens": "all" if tokens == "all" else toks, "rel_l2": float(err), "worst_token_rel_l2": float(worst)}


def time_eager(call, steps, warmup, repeats):
    torch = call.torch
    for i in range(warmup):
        call.step(i)
    torch.cuda.synchronize()
    walls, evs = [], []
    for _ in range(repeats):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(call.stream)
        for i in range(steps):
            call.step(i)
        ev1.record(call.stream)
        torch.cuda.synchronize()
        walls.append((time.perf_counter() - t0) * 1e3)
        evs.append(ev0.elapsed_time(ev1))
    return walls, evs


def per_kernel(call, steps):
    """Average launch time of every library kernel over `steps` calls (HIP events around each
    launch on the launch stream; the launches run back to back)."""
    apq, torch = call.apq, call.torch
    apq.moe_profile_start()
    for i in range(steps):
        call.step(i)
    torch.cuda.synchronize()
    prof = apq.moe_profile_stop()
    return {k: 1e3 * v[0] / v[1] for k, v in prof.items()}


def rooflines(call, ids, kernel_us, workload):
    """Roofline object per FFN kernel: algorithmic plane + LUT bytes of the blocks one launch
    reads, divided by its average launch time, against the 8 TB/s HBM peak."""
    out = {}
    for kname, module in KERNELS.items():
        if kname not in kernel_us:
            continue
        p, l = module_bytes(call.shape, ids, module, call.widths)
        us = kernel_us[kname]
        ach = (p + l) / (us * 1e-6) / 1e9
        out[kname] = {"bound": "hbm", "kernel": kname, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                      "traffic": traffic_from_profile(workload, kname),
                      "algorithmic_bytes_per_launch": int(p + l), "avg_launch_us": round(us, 3)}
    return out


def sub_record(apq, torch, name, dev, args):
    """One other layer shape: parity, then the eager time per layer and the kernel rooflines."""
    from workloads import device as gpu_layers
    import oracle
    shape = WORKLOADS[name]
    log(f"[bench] sub-record {name}: building weights")
    copies = layer_copies(apq, torch, shape, dev, args.copies_gb)
    call = LayerCall(apq, torch, shape, copies, dev)
    parity = None if args.no_check else check_parity(call, SUB_WORKLOADS[name])
    steps = args.sub_steps
    walls, evs = time_eager(call, steps, max(2, args.warmup // 4), 3)
    us = 1e3 * float(np.median(evs)) / steps
    kus = per_kernel(call, steps)
    ids, _ = oracle.route_topk(call.inputs.logits, shape.k)
    pb, lb = gpu_layers.active_weight_bytes(shape, ids, call.widths)
    gbs = (pb + lb) / (us * 1e-6) / 1e9
    log(f"[bench] {name}: {us:.1f} us per layer, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f} %)")
    return {
        "workload": shape.name, "tokens": shape.T, "us_per_layer": round(us, 2),
        "value_GBs": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "widths": sorted(set(int(v) for v in np.unique(call.widths))) + (
            [shape.q_shared] if shape.I_shared else []),
        "active_experts": int(len(np.unique(ids))), "weight_bytes_per_call": int(pb + lb),
        "weight_copies": len(copies), "per_kernel_us": {k: round(v, 3) for k, v in kus.items()},
        "roofline": rooflines(call, ids, kus, name), "parity": parity,
        "timing": f"median of 3 runs of {steps} eager calls between HIP events",
    }


def prefill_row(apq, torch, dev, steps: int, warmup: int, check: bool, copies_gb: float):
    """The chunked-prefill row: one moe_layer_forward over 2048 tokens of the Qwen2-57B-A14B-shaped
    layer, where about 256 tokens meet every expert and the tile kernels take their wide
    matrix-core branch.  Compute-bound: reported as TFLOP/s of the layer's algorithmic flops
    2*T*k*3*H*I against the fp16 MFMA peak."""
    from workloads import device as gpu_layers
    import oracle
    shape = WORKLOADS["qwen2_57b_a14b_prefill2048"]
    log(f"[bench] prefill row: {shape.name}, T={shape.T}")
    call = LayerCall(apq, torch, shape, layer_copies(apq, torch, shape, dev, copies_gb)[:1], dev)
    parity = check_parity(call, [0, 511, 1024, 1537, 2047]) if check else None
    walls, evs = time_eager(call, steps, warmup, 1)
    us = 1e3 * evs[0] / steps
    kus = per_kernel(call, steps)
    ids, _ = oracle.route_topk(call.inputs.logits, shape.k)
    planes_b, lut_b = gpu_layers.active_weight_bytes(shape, ids, call.widths)
    T = shape.T
    flops = 2.0 * T * shape.k * 3 * shape.H * shape.I
    gu_flops = 2.0 * T * shape.k * 2 * shape.I * shape.H
    gu_us = kus["apq_gate_up_silu"]
    gu_tf = gu_flops / (gu_us * 1e-6) / 1e12
    tf = flops / (us * 1e-6) / 1e12
    log(f"[bench] prefill: {us:.1f} us per layer, {tf:.1f} TFLOP/s; gate_up {gu_us:.1f} us = {gu_tf:.1f} TFLOP/s")
    return {
        "workload": shape.name, "tokens": T, "us_per_layer": round(us, 2),
        "TFLOPs": round(tf, 2), "flops_per_layer": flops,
        "weight_GBs": round((planes_b + lut_b) / (us * 1e-6) / 1e9, 1),
        "per_kernel_us": {k: round(v, 3) for k, v in kus.items()},
        "roofline": {"bound": "mfma", "kernel": "apq_gate_up_silu", "achieved": round(gu_tf, 2),
                     "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gu_tf / MFMA_FP16_PEAK_TFLOPS, 4),
                     "algorithmic_flops_per_launch": gu_flops, "avg_launch_us": round(gu_us, 3)},
        "parity": parity, "steps": steps,
        "timing": f"{steps} eager calls between HIP events after {warmup} warmup calls; "
                  "weights (1.25 GB) exceed the last-level cache",
    }


def graph_replay(call, steps, warmup, repeats):
    """The same calls replayed from captured HIP graphs: one graph per weight copy (one layer
    call each), and one graph holding one call per copy in sequence.  Every replay must
    reproduce the eager output bit for bit."""
    apq, torch = call.apq, call.torch
    y_eager = call.y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(call.stream)
    singles, chain = [], torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for i in range(len(call.copies)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                call.step(i, stream=side)
            singles.append(g)
        with torch.cuda.graph(chain, stream=side):
            for i in range(len(call.copies)):
                call.step(i, stream=side)
    call.stream.wait_stream(side)

    def run(fn, n):
        out = []
        for _ in range(repeats):
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            g0.record()
            for i in range(n):
                fn(i)
            g1.record()
            torch.cuda.synchronize()
            out.append(g0.elapsed_time(g1))
        return float(np.median(out))

    for i in range(warmup):
        singles[i % len(singles)].replay()
    torch.cuda.synchronize()
    single_us = 1e3 * run(lambda i: singles[i % len(singles)].replay(), steps) / steps
    same = bool(torch.equal(call.y, y_eager))
    n_chain = max(1, steps // len(call.copies))
    chain.replay()
    torch.cuda.synchronize()
    chain_us = 1e3 * run(lambda i: chain.replay(), n_chain) / (n_chain * len(call.copies))
    same = same and bool(torch.equal(call.y, y_eager))
    log(f"[bench] graph replay: {single_us:.2f} us/layer with one graph per call, {chain_us:.2f} us/layer "
        f"with {len(call.copies)} calls per graph; output identical to eager: {same}")
    assert same, "graph replay output differs from the eager call"
    return {"us_per_layer_one_call_per_graph": round(single_us, 2),
            "us_per_layer_calls_chained_in_one_graph": round(chain_us, 2),
            "calls_per_chained_graph": len(call.copies), "identical_to_eager": same}


def read_ceiling(apq, torch, dev):
    """Achievable streaming-read rate of this device (the library's read probe over 2 GiB)."""
    probe = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        apq.moe_hbm_read_probe(probe, sink)
    torch.cuda.synchronize()
    p0 = torch.cuda.Event(enable_timing=True)
    p1 = torch.cuda.Event(enable_timing=True)
    p0.record()
    for _ in range(5):
        apq.moe_hbm_read_probe(probe, sink)
    p1.record()
    torch.cuda.synchronize()
    gbs = probe.numel() / (p0.elapsed_time(p1) * 1e-3 / 5) / 1e9
    del probe
    log(f"[bench] streaming-read ceiling: {gbs:.1f} GB/s")
    return gbs


def back_to_back_us(torch, stream, launch, n):
    """Average time of `n` launches issued back to back between two events on `stream`."""
    launch(0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / n


def next_rows(apq, torch, call, base, dev, n):
    """Rows beyond the layer call, on the routing of the timed call: online routing statistics,
    residency-aware substitution, LYNX remapping, width planning and commits.  The
    single-workgroup kernels are timed as `n` back-to-back launches between two events (inputs
    prepared beforehand, one copy per launch where a launch rewrites its input)."""
    from workloads import device as gpu_layers
    import oracle
    shape, stream = call.shape, call.stream
    T, E, k = shape.T, shape.E, shape.k
    view = apq.moe_workspace_routing(call.ws, T, E, shape.H, shape.I, k, shape.I_shared)
    ids_ref, _ = oracle.route_topk(call.inputs.logits, k)
    weight_bytes = sum(gpu_layers.active_weight_bytes(shape, ids_ref, call.widths))
    out = {}
    acc = [torch.zeros(E, dtype=torch.int64, device=dev), torch.zeros(E, dtype=torch.float64, device=dev),
           torch.zeros(2, dtype=torch.float64, device=dev)]
    resident = (torch.arange(E, device=dev) % 4 == 0).to(torch.uint8)
    us = back_to_back_us(torch, stream, lambda i: apq.moe_routing_stats(
        view["offsets"], view["pairs"], view["gates"], T, k, E, *acc, resident=resident, stream=stream), n)
    m = float(acc[2][0] / acc[2][1]) if float(acc[2][1]) > 0 else 0.0
    out["routing_stats"] = {
        "us_per_call": round(us, 3), "bytes_per_call": int(4 * (E + 1) + 8 * T * k + 33 * E),
        "substituted_gate_mass_m": round(m, 5),
        "note": "per-expert counts + gate mass + non-resident mass (a quarter of the experts resident), "
                "from the routing results of a layer call; single workgroup"}
    log(f"[bench] routing statistics: {us:.2f} us per call, m = {m:.4f}")

    lg = call.logits.view(T, E)
    ids_in = view["ids"].view(T, k).clone()
    ids_sub = ids_in.unsqueeze(0).repeat(n + 1, 1, 1)
    missed = torch.empty_like(ids_in)
    fetch = torch.empty(E, dtype=torch.uint8, device=dev)
    admit_mass = torch.zeros(E, dtype=torch.float32, device=dev)
    admit = torch.zeros(E, dtype=torch.uint8, device=dev)
    us = back_to_back_us(torch, stream, lambda i: apq.moe_substitute(
        lg, resident, apq.MOE_POLICY_GATE_RULE, ids_sub[i], view["gates"], missed, fetch,
        admit_mass=admit_mass, admit=admit, stream=stream), n)
    out["substitution"] = {
        "us_per_call": round(us, 3), "policy": "0.15 rule + background admission at 0.5",
        "substituted_slots": int((missed >= 0).sum()), "fetched_experts": int(fetch.sum()),
        "note": "a wavefront per token (one workgroup up to 16 tokens; beyond, four tokens per "
                "workgroup, then one workgroup for the fetch flags and admission); a quarter of "
                "the experts resident"}
    log(f"[bench] substitution: {us:.2f} us per call")

    ids_l = ids_in.unsqueeze(0).repeat(n + 1, 1, 1)
    remapped = torch.empty_like(ids_in)
    critical = torch.empty(E, dtype=torch.uint8, device=dev)
    us = back_to_back_us(torch, stream, lambda i: apq.moe_lynx_remap(
        lg, ids_l[i], remapped, critical, stream=stream), n)
    ids_after = ids_l[n].cpu().numpy()
    pb_a, lb_a = gpu_layers.active_weight_bytes(shape, ids_after, call.widths)
    out["lynx_remap"] = {
        "us_per_call": round(us, 3), "distinct_experts_before": int(len(np.unique(ids_ref))),
        "distinct_experts_after": int(len(np.unique(ids_after))),
        "remapped_slots": int((remapped >= 0).sum()), "weight_bytes_before": int(weight_bytes),
        "weight_bytes_after": int(pb_a + lb_a),
        "note": "AffinityBinning with the library's default bin width k/N on the top-2 logit gap; one "
                "workgroup, a wavefront per token; weight bytes are those a layer call would read"}
    log(f"[bench] LYNX remap: {us:.2f} us per call, distinct experts "
        f"{len(np.unique(ids_ref))} -> {len(np.unique(ids_after))}")

    # width planning over every block of the layer (synthetic damage scores rising as the width
    # falls, routed experts with a multiplier) to free a quarter of the weight bytes, on the
    # host; then the commit of all of the layer's descriptors (same values) in stream order
    blocks = [base.block(e, mm) for e in range(E) for mm in (0, 1)]
    if base.shared is not None:
        blocks += [base.shared_block(0), base.shared_block(1)]
    rng = np.random.default_rng(0)
    qc = np.array([b.q for b in blocks], dtype=np.uint8)
    dmg = np.cumsum(rng.random((len(blocks), 8))[:, ::-1], axis=1)[:, ::-1]
    hot = np.concatenate([np.repeat(acc[0].cpu().numpy() > 0, 2), np.zeros(len(blocks) - 2 * E, bool)])
    mult = np.where(hot, 2.0, 1.0)
    target = base.weight_bytes // 4
    plan_args = (qc, np.minimum(qc, 2), [b.rows for b in blocks], [b.cols for b in blocks], dmg, mult, target)
    apq.moe_plan_widths(*plan_args)
    t0 = time.perf_counter()
    reps = 200
    for _ in range(reps):
        q_plan, freed = apq.moe_plan_widths(*plan_args)
    plan_us = (time.perf_counter() - t0) * 1e6 / reps
    index = list(range(2 * E))
    us = back_to_back_us(torch, stream, lambda i: apq.moe_commit_blocks(
        base.table, index, blocks[: 2 * E], stream=stream), n)
    out["width_plan"] = {
        "host_us_per_plan": round(plan_us, 2), "blocks": len(blocks), "target_bytes": int(target),
        "bytes_freed": int(freed), "blocks_lowered": int((q_plan < qc).sum()),
        "commit_us_per_call": round(us, 3), "committed_descriptors": len(index),
        "note": "greedy lowest damage per byte (synthetic scores, multiplier 2 on experts routed "
                "in the timed calls) on the host; commit = stream-ordered page-table write"}
    log(f"[bench] width plan: {plan_us:.1f} us on the host for {len(blocks)} blocks; "
        f"commit of {len(index)} descriptors {us:.2f} us")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--copies-gb", type=float, default=1.2,
                    help="total bytes of rotated weight copies (defeats the last-level cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=30.0)
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed runs of --steps calls each (eager and graph); the median is reported")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the 2048-token chunked-prefill row (matrix-core path)")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--no-sub", action="store_true", help="skip the sub-records of the other shapes")
    ap.add_argument("--sub-steps", type=int, default=100)
    ap.add_argument("--no-next", action="store_true", help="skip the rows beyond the layer call")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one device copy of this many MiB: the known-size "
                         "dispatch that calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the layer is measured on "
                          "one MI355X's share; --gpus must be 1"}), flush=True)
        sys.exit(2)

    import torch
    import any_precision_expert_router_amd as apq
    from workloads import device as gpu_layers
    import oracle

    dev = "cuda:0"
    torch.cuda.set_device(0)
    shape = WORKLOADS[args.workload]
    log(f"[bench] workload {shape.name}, T={shape.T}: building weights")
    copies = layer_copies(apq, torch, shape, dev, args.copies_gb)
    base = copies[0]
    log(f"[bench] {len(copies)} weight copies x {base.weight_bytes / 1e6:.1f} MB")
    call = LayerCall(apq, torch, shape, copies, dev)
    T = shape.T
    ids_ref, _ = oracle.route_topk(call.inputs.logits, shape.k)
    planes_b, lut_b = gpu_layers.active_weight_bytes(shape, ids_ref, call.widths)
    weight_bytes = planes_b + lut_b

    # correctness of the timed configuration on every token of the call
    parity = None if args.no_check else check_parity(call, "all")

    walls, evs = time_eager(call, args.steps, args.warmup, args.repeats)
    wall_ms = float(np.median(walls))
    ev_ms = float(np.median(evs))
    ms_per_step = wall_ms / args.steps
    log(f"[bench] {args.repeats} x {args.steps} steps: median wall {wall_ms:.2f} ms, events {ev_ms:.2f} ms "
        f"-> {1e3 * ms_per_step:.2f} us/layer (events {1e3 * ev_ms / args.steps:.2f}); "
        f"runs {['%.2f' % (1e3 * w / args.steps) for w in walls]} us/layer")

    graph = None if args.no_graph else graph_replay(call, args.steps, args.warmup, args.repeats)
    ceiling = read_ceiling(apq, torch, dev)
    kus = per_kernel(call, args.steps)
    log("[bench] per-kernel (events): " + ", ".join(f"{k} {v:.2f} us" for k, v in kus.items()))
    roofs = rooflines(call, ids_ref, kus, args.workload)
    weakest = min(roofs.values(), key=lambda r: r["frac"])

    nxt = None if args.no_next else next_rows(apq, torch, call, base, dev, args.steps)

    cpu = None
    if not args.no_cpu_baseline:
        threads = cpu_threads()
        med_s, runs = cpu_baseline(shape, call.inputs, args.cpu_budget_s, threads)
        cpu = {"value": round(weight_bytes / med_s / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"one whole layer call ({T} tokens, float64 NumPy, BLAS limited to {threads} "
                         f"threads), median of {runs} runs: {1e3 * med_s:.0f} ms per layer",
               "ms_per_layer": round(1e3 * med_s, 1),
               "host_cores_available": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}
        log(f"[bench] CPU oracle: {1e3 * med_s:.0f} ms per layer on {threads} threads")

    head_cfg = {"workload": shape.name, "tokens": T, "hidden": shape.H, "experts": shape.E,
                "intermediate": shape.I, "top_k": shape.k, "shared_intermediate": shape.I_shared,
                "widths": sorted(set(int(v) for v in np.unique(call.widths))),
                "active_experts": int(len(np.unique(ids_ref))), "weight_bytes_per_call": int(weight_bytes),
                "plane_bytes": int(planes_b), "lut_bytes": int(lut_b), "weight_copies": len(copies)}
    del call

    # shapes that share the headline's weights first (the device copies are reused), then the
    # chunked prefill, then the shapes with weights of their own
    same = [n for n in SUB_WORKLOADS if WORKLOADS[n].workload_id == shape.workload_id]
    order = same + [n for n in SUB_WORKLOADS if n not in same]
    subs, prefill = {}, None
    for name in order:
        if name in same or args.no_prefill or prefill is not None:
            pass
        else:
            prefill = prefill_row(apq, torch, dev, args.prefill_steps, 2, not args.no_check, args.copies_gb)
        if not args.no_sub and name != args.workload:
            subs[name] = sub_record(apq, torch, name, dev, args)
    if prefill is None and not args.no_prefill:
        prefill = prefill_row(apq, torch, dev, args.prefill_steps, 2, not args.no_check, args.copies_gb)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 18   # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")
        del src, dst

    value = weight_bytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "us_per_layer": round(1e3 * ms_per_step, 2),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "planes_only_GBs": round(planes_b / (ms_per_step * 1e-3) / 1e9, 1),
        "repeats": args.repeats,
        "runs_us_per_layer": [round(1e3 * w / args.steps, 2) for w in walls],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp16",
        "data": "synthetic",
        "config": head_cfg,
        "parity": parity,
        "per_kernel_us": {k: round(v, 3) for k, v in kus.items()},
        "hbm_read_ceiling_GBs": round(ceiling, 1),
        "pct_read_ceiling": round(100 * value / ceiling, 2),
        "timing": f"median of {args.repeats} runs of {args.steps} eager moe_layer_forward calls "
                  "(headline, host wall clock around each run); graph_replay replays the same calls "
                  "from captured HIP graphs",
        "graph_replay": graph,
        "roofline": roofs[DOMINANT],
        "roofline_weakest_kernel": weakest,
        "rooflines": roofs,
        "cpu_baseline": cpu,
        "sub_records": subs,
        "prefill_row": prefill,
        "next_rows": nxt,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
