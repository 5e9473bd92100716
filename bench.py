"""Benchmark of the Flint MoE layer on one MI355X.

    python bench.py [--steps K] [--warmup W]
                    [--workload decode32|prefill4096|skew16384|stack47|toy|decode32_mx4|dense32|dense4096]

A step is one pass of the whole layer (router, top-k, dispatch, gate/up +
SwiGLU, down, combine; for stack47 all 47 layers with RMSNorm between them) over
one batch of tokens whose inputs and weights are resident in HBM.  The default
workload is the decode batch: one Flint-shaped layer (H=2048, 256 experts,
top-6, expert width 512, shared width 1024, bf16) on T=32 tokens.  Single-layer
workloads rotate through several independently drawn weight copies so that the
last-level cache cannot serve repeated weight reads.

Prints ONE JSON line.  Beside the headline throughput:
  roofline      the dominant kernel's algorithmic bytes per launch (flops when
                its flop per byte exceed the ridge point, 2.5 PFLOP/s over
                8 TB/s) over its mean launch duration, from HIP events that
                the library stamps at that kernel's own begin and end (hipExtLaunchKernel,
                on the library's stream) during a second pass of the same
                steps, against MI355X's published peak; `traffic` is the HBM
                bytes per launch that the committed rocprofv3 counter summary
                for this kernel and workload records (FETCH_SIZE + WRITE_SIZE,
                scaled by the same counters on a plain copy), or null when the
                kernel's sources have changed since it was taken;
  step_us_percentiles  p10 / median / p90 of single steps (a third pass,
                an event pair around each step);
  device, hbm_read_measured_GBs  the GPU's name, compute units and peak clock
                as the runtime reports them, and the read rate of row sums
                over 1 GiB (a practical ceiling beside the 8 TB/s spec);
  parity        one layer call (weight copy 0) against the oracle, outside
                the timed region: near-tie tokens, tokens whose expert set
                differs, max |gpu - oracle| / rms of the outputs;
  cpu_baseline  the oracle (plain fp64 C) timed on the host on a bounded
                sample of the same workload, on all its threads and on one
                core, with the host's CPU model.
"""
from __future__ import annotations

import argparse
import dataclasses
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# flop per byte above which a kernel is bound by the matrix cores, not by HBM
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
METRIC = "MoE-layer tokens/s (bf16, H=2048, 256e top-6) + % HBM/MFMA roofline"
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "routed_expert_ffn_flint_amd", "csrc")
# the sources each gate/up kernel is built from
KERNEL_SOURCES = {
    "k_expert_stream": ["common.hpp", "gemm_core.hpp", "launch.hpp", "stream.hip"],
    "k_expert_stream_mx4": ["common.hpp", "gemm_core.hpp", "launch.hpp", "stream_mx4.hip"],
    "k_tiled": ["common.hpp", "gemm_core.hpp", "launch.hpp", "tile_sched.hpp", "tiled.hip"],
    "k_fused_decode": ["common.hpp", "gemm_core.hpp", "launch.hpp", "topk.hpp", "fused.hip"],
}
# largest bf16 batch of a MoE layer the library serves with the streaming
# kernels; larger ones go to the tiled kernels (a bf16 dense layer takes the
# tiled kernels at every size)
STREAM_MAX_T = 159


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode32")
    p.add_argument("--tokens", type=int, default=None,
                   help="tokens per step instead of the workload's own (other batch sizes of the same layer)")
    p.add_argument("--copies", type=int, default=4, help="weight copies rotated (single-layer workloads)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true", help="replay the steps from a captured HIP graph")
    p.add_argument("--fused", action="store_true",
                   help="the layer through flint_moe_forward_fused (top-k through down in one persistent kernel; "
                        "bf16 batches of up to 64 tokens)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 5 times (reference for the HBM "
                        "byte counters) and exit")
    return p.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": {"read": n, "write": n}, "launches": 5}))


def device_and_read_rate():
    """The GPU as the runtime reports it (compute units, peak clock) and a
    measured HBM read rate: row sums of a 1 GiB float32 tensor (rows of 1024;
    torch's whole-tensor sum reads at only ~60% of this), best of 6."""
    import torch

    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int, ctypes.c_int]
    dev = torch.cuda.current_device()
    attr = {}
    for name, code in (("clock_khz", 5), ("cus", 63)):  # hipDeviceAttributeClockRate, ...MultiprocessorCount
        v = ctypes.c_int()
        attr[name] = int(v.value) if hip.hipDeviceGetAttribute(ctypes.byref(v), code, dev) == 0 else None
    props = torch.cuda.get_device_properties(dev)
    x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    best = float("inf")
    for _ in range(6):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        x.view(-1, 1024).sum(1)
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b))
    del x
    return ({"name": props.name, "arch": getattr(props, "gcnArchName", None), "cus": attr["cus"],
             "clock_mhz": None if attr["clock_khz"] is None else attr["clock_khz"] / 1000.0},
            (1 << 30) / (best * 1e-3) / 1e9)


class HipEvents:
    """hipEvent_t handles from the process's HIP runtime (the one torch loaded)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(ev)
        return out

    def ms(self, a, b):
        v = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(v), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return v.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def step_percentiles(step, n):
    """p10 / median / p90 of single steps, microseconds: a further pass of n
    steps, each between two events on the library's stream."""
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(evs):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs], dtype=np.float64)
    p10, p50, p90 = np.percentile(us, [10, 50, 90])
    return {"p10": float(p10), "p50": float(p50), "p90": float(p90), "steps": n}


def sources_digest(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def counters_traffic(kernel, workload, digest):
    """HBM bytes per launch from profiles/<kernel>_gate_up.<workload>.hbm_counters.md
    (its json block), if that summary was taken on these very sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_gate_up.{workload}.hbm_counters.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        m = re.search(r"```json\n(.*?)\n```", f.read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("sources_sha256") != digest:
        return None
    return float(rec["traffic_bytes_per_launch"])


def algorithmic(wl, idx_np):
    """Algorithmic HBM bytes and flops of one layer call, per stage.

    Weights count once per distinct expert the batch selects; activations are
    read once; outputs written once (float32 out)."""
    T, H, E, K, I, Is = wl.T, wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter
    eb = 2 if wl.bf16 else 4
    wb = (0.5 + 1.0 / 32) if wl.mx4 else eb  # bytes per expert weight (MXFP4: half-byte code + 1/32 scale)
    distinct = len(np.unique(idx_np))
    gate_up_bytes = distinct * 2 * I * H * wb + 2 * Is * H * wb + T * H * eb + (T * K * I + T * Is) * eb
    down_bytes = distinct * H * I * wb + Is * H * wb + (T * K * I + T * Is) * eb + (T * K + T) * H * 4
    router_bytes = E * H * eb + T * H * eb
    layer_bytes = E * H * eb + (distinct * 3 * I * H + 3 * Is * H) * wb + T * H * eb + T * H * 4
    flops = {
        "router": 2 * T * E * H,
        "gate_up": 4 * T * K * I * H + 4 * T * Is * H,
        "down": 2 * T * K * I * H + 2 * T * Is * H,
    }
    flops["layer"] = flops["router"] + flops["gate_up"] + flops["down"]
    return {"distinct": distinct, "gate_up_bytes": gate_up_bytes, "down_bytes": down_bytes,
            "router_bytes": router_bytes, "layer_bytes": layer_bytes, "flops": flops}


def host_cpu():
    """The host's CPU model (as /proc/cpuinfo names it) and its logical CPUs."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "nproc": os.cpu_count(), "usable": len(os.sched_getaffinity(0))}


def time_calls(fn, n_tok, target_s):
    """Calls fn until about target_s seconds have passed (at most 1000 calls):
    (tokens/s, calls, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 1000:
            return reps * n_tok / el, reps, el


def oracle_baseline(o, run, n_all_tok, n_one_tok, target_s, what):
    """The oracle timed on all the threads its OpenMP loops use (over tokens)
    and on one core: run(n) does one call on the first n tokens."""
    threads = o.threads()
    v_all, r_all, e_all = time_calls(lambda: run(n_all_tok), n_all_tok, target_s)
    o.set_threads(1)
    try:
        v_one, r_one, e_one = time_calls(lambda: run(n_one_tok), n_one_tok, target_s)
    finally:
        o.set_threads(threads)
    return {"value": v_all, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what}, the first {n_all_tok} tokens per call, fp64, {r_all} calls over {e_all:.1f} s "
                      f"on {threads} threads",
            "single_core": {"value": v_one, "unit": "tokens/s", "cores": 1,
                            "sample": f"the first {n_one_tok} tokens per call, {r_one} calls over {e_one:.1f} s"},
            "cpu": host_cpu()}


def host_layer_weights(o, wl, w_dev, experts=None):
    """Exact float32 host copies of a layer's weights for the oracle (MXFP4
    matrices decoded by the oracle itself); with ``experts``, only those
    routed experts' matrices (the rest zero)."""
    from routed_expert_ffn_flint_amd import inputs
    import torch

    def pick(k, v):
        if experts is None or k.split("_")[0] not in ("gate", "up", "down"):
            return v
        keep = torch.as_tensor(sorted(experts), device=v.device, dtype=torch.long)
        out = torch.zeros_like(v)
        out.index_copy_(0, keep, v.index_select(0, keep))
        return out

    if wl.mx4:
        return o.mx4_weights({k: (pick(k, v).cpu().numpy() if k.endswith(("_q", "_s")) else inputs.to_numpy_f32(v))
                              for k, v in w_dev.items()})
    return {k: inputs.to_numpy_f32(pick(k, v) if v is not None else None) for k, v in w_dev.items()}


def cpu_baseline(wl, w_dev, x_dev, target_s):
    """The oracle on the host: whole-layer forward (routing included) of the
    workload's first tokens, on all threads and on one core."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import oracle as orc
    from routed_expert_ffn_flint_amd import inputs

    o = orc.default()
    d = orc.dims(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, wl.bf16)
    wh = host_layer_weights(o, wl, w_dev)
    n_tok = min(wl.T, 32)
    xh = inputs.to_numpy_f32(x_dev[:n_tok])
    return oracle_baseline(o, lambda n: o.forward(d, xh[:n], wh), n_tok, min(n_tok, 4), target_s / 2,
                           f"{wl.name} layer (weight copy 0)")


def parity_report(wl, w_dev, x_dev, out, idx, tw, max_tokens=512):
    """The GPU result of one layer call against the oracle, outside the timed
    region: routing of the checked tokens (near-tie tokens flagged by the
    oracle, tokens whose expert set differs) and max |gpu - oracle| / rms of
    their outputs, the oracle run with the GPU's expert sets (tokens spread
    evenly over the batch when it has more than max_tokens)."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import oracle as orc
    from routed_expert_ffn_flint_amd import inputs
    import torch

    o = orc.default()
    d = orc.dims(wl.hidden, wl.n_experts, wl.top_k, wl.inter, wl.shared_inter, wl.bf16)
    T = x_dev.shape[0]
    rows = np.arange(T) if T <= max_tokens else np.unique(np.linspace(0, T - 1, max_tokens).astype(np.int64))
    sel = torch.as_tensor(rows, device=x_dev.device)
    xh = inputs.to_numpy_f32(x_dev.index_select(0, sel))
    gi = idx.index_select(0, sel).cpu().numpy()
    gw = tw.index_select(0, sel).cpu().numpy()
    router = inputs.to_numpy_f32(w_dev["router"])
    bias = inputs.to_numpy_f32(w_dev.get("bias"))
    o_idx, o_w, tie = o.route(d, xh, router, bias)
    differ = np.any(gi != o_idx, axis=1)
    wh = host_layer_weights(o, wl, w_dev, set(gi.ravel().tolist()))
    ref, _, rw, _ = o.forward(d, xh, wh, force_idx=gi)
    g = out.index_select(0, sel).float().cpu().numpy().astype(np.float64)
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    return {"tokens_checked": int(len(rows)), "near_tie_tokens": int(tie.sum()),
            "sets_differing": int(differ.sum()),
            "max_abs_err_over_rms": float(np.max(np.abs(g - ref)) / rms) if rms > 0 else 0.0,
            "max_weight_err": float(np.max(np.abs(gw - rw))) if gw.size else 0.0,
            "bar": "sets equal except near ties (K-th/(K+1)-th oracle score gap < 1e-5); "
                   "max |delta| <= 1e-2 * rms"}


def bench_dense(args, wl):
    """The dense MLP layer (flint_dense_mlp): same timing scheme as the MoE layer,
    stages gate/up, down and output; every step reads all of the layer's weights."""
    import torch

    from routed_expert_ffn_flint_amd import _lib, api, inputs

    lib = _lib.load()
    dd = api.dense_dims_of(wl)
    T, H, I = wl.T, wl.hidden, wl.inter
    eb = 2 if wl.bf16 else 4
    n_copies = max(1, args.copies)
    layers = [inputs.make_dense(wl, c, "cuda") for c in range(n_copies)]
    x = inputs.make_tokens(wl, device="cuda")
    out = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = api.dense_workspace(dd, T)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptrs = [[ctypes.c_void_p(w[k].data_ptr()) for k in ("gate", "up", "down")] for w in layers]

    def step(i, events=None):
        arr = None if events is None else (ctypes.c_void_p * 6)(*[e.value for e in events])
        g, u, dn = ptrs[i % n_copies]
        st = lib.flint_dense_mlp(ctypes.byref(dd), T, ctypes.c_void_p(x.data_ptr()), g, u, dn,
                                 ctypes.c_void_p(out.data_ptr()), api.F32, ctypes.c_void_p(ws.data_ptr()),
                                 ws.numel(), sp, arr)
        if st != 0:
            raise api.FlintError(st, "flint_dense_mlp")

    for i in range(args.warmup):
        step(i)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / args.steps

    hev = HipEvents()
    n_prof = min(args.steps, 100)
    ev_sets = [hev.create(6) for _ in range(n_prof)]
    for i in range(n_prof):
        step(i, ev_sets[i])
    torch.cuda.synchronize()
    names = ["gate_up", "down", "output"]
    stage_us = {n: float(np.mean([hev.ms(evs[2 * j], evs[2 * j + 1]) for evs in ev_sets]) * 1e3)
                for j, n in enumerate(names)}
    for evs in ev_sets:
        hev.destroy(evs)

    gu_bytes = 2 * I * H * eb + T * H * eb + T * I * eb
    gu_flops = 4 * T * I * H
    layer_bytes = 3 * I * H * eb + T * H * eb + T * H * 4
    layer_flops = 6 * T * I * H
    big = gu_flops / gu_bytes >= RIDGE  # arithmetic intensity of the gate/up kernel
    kernel = "k_tiled"
    digest = sources_digest(kernel)
    kname = f"{kernel}<gate/up> (gate/up GEMM + SwiGLU of the dense layer)"
    traffic = counters_traffic(kernel, wl.name, digest)
    if big:
        achieved = gu_flops / (stage_us["gate_up"] * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / BF16_PEAK_TFLOPS, "traffic": traffic, "kernel": kname,
                    "per_launch": {"flops": gu_flops, "bytes": gu_bytes, "mean_us": stage_us["gate_up"]}}
    else:
        achieved = gu_bytes / (stage_us["gate_up"] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": kname,
                    "per_launch": {"bytes": gu_bytes, "mean_us": stage_us["gate_up"]}}
    roofline["sources_sha256"] = digest
    lt = ms / 1e3
    result = {
        "metric": "dense MLP layer tokens/s (bf16, H=2048, width 6144) + % HBM/MFMA roofline",
        "value": T / lt, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.bf16 else "f32", "data": "synthetic",
        "config": {"workload": f"{wl.name}: one dense gated MLP layer, T={T}, H={H}, width {I}", "T": T,
                   "weight_copies": n_copies, "graph": False, "wall_s": wall},
        "roofline": roofline,
        "layer_roofline": {"hbm_GBs": layer_bytes / lt / 1e9, "hbm_frac": layer_bytes / lt / 1e9 / HBM_PEAK_GBS,
                           "mfma_TFLOPs": layer_flops / lt / 1e12,
                           "mfma_frac": layer_flops / lt / 1e12 / BF16_PEAK_TFLOPS,
                           "algorithmic_bytes": layer_bytes, "flops": layer_flops},
        "stages_us": stage_us,
        "step_us_percentiles": step_percentiles(step, n_prof),
    }
    result["device"], result["hbm_read_measured_GBs"] = device_and_read_rate()
    from oracle import oracle as orc
    o = orc.default()
    w0 = {k: inputs.to_numpy_f32(v) for k, v in layers[0].items()}
    # parity of one call on weight copy 0, outside the timed region
    step(0)
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 512 else np.unique(np.linspace(0, T - 1, 512).astype(np.int64))
    ref = o.dense_mlp(inputs.to_numpy_f32(x)[rows], w0["gate"], w0["up"], w0["down"], h_bf16=wl.bf16)
    g = out.cpu().numpy()[rows].astype(np.float64)
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    result["parity"] = {"tokens_checked": int(len(rows)), "max_abs_err_over_rms": float(np.max(np.abs(g - ref)) / rms),
                        "bar": "max |delta| <= 1e-2 * rms"}
    if not args.no_cpu_baseline:
        n_tok = min(T, 32)
        xh = inputs.to_numpy_f32(x[:n_tok])
        result["cpu_baseline"] = oracle_baseline(
            o, lambda n: o.dense_mlp(xh[:n], w0["gate"], w0["up"], w0["down"], h_bf16=wl.bf16), n_tok,
            min(n_tok, 4), args.cpu_seconds / 2, f"{wl.name} layer (weight copy 0)")
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU: --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)
    import torch

    from routed_expert_ffn_flint_amd import _lib, api, inputs

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    lib = _lib.load()
    wl = inputs.WORKLOADS[args.workload]
    if args.tokens is not None:
        if args.tokens < 1:
            raise SystemExit("--tokens must be at least 1")
        wl = dataclasses.replace(wl, T=args.tokens)
    if wl.dense:
        bench_dense(args, wl)
        return
    d = api.dims_of(wl)
    dev = "cuda"
    torch.cuda.set_device(0)

    stack = wl.layers > 1
    n_copies = wl.layers if stack else max(1, args.copies)
    layers = [inputs.make_layer(wl, c, dev) for c in range(n_copies)]
    wstructs = [api.weights_mx4_struct(d, w) if wl.mx4 else api.weights_struct(d, w) for w in layers]
    x = inputs.make_tokens(wl, device=dev)
    T = wl.T
    ws = api.workspace(d, T, dev)
    out = torch.empty((T, wl.hidden), dtype=torch.float32, device=dev)
    idx = torch.empty((T, wl.top_k), dtype=torch.int32, device=dev)
    tw = torch.empty((T, wl.top_k), dtype=torch.float32, device=dev)
    xs = [torch.empty((T, wl.hidden), dtype=torch.bfloat16, device=dev) for _ in range(2)] if stack else None
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    dref = ctypes.byref(d)
    wsp, wsn = ctypes.c_void_p(ws.data_ptr()), ws.numel()
    outp, idxp, twp = ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(tw.data_ptr())
    xp = ctypes.c_void_p(x.data_ptr())

    def layer_call(c, xin, events=None, norm=None):
        # norm: where the RMSNorm of this layer's output goes (the next layer's
        # input), taken in the layer's combine (flint_moe_forward_rmsnorm)
        arr = None if events is None else (ctypes.c_void_p * 10)(*[e.value for e in events])
        if norm is not None:
            st = lib.flint_moe_forward_rmsnorm(dref, T, xin, ctypes.byref(wstructs[c]), outp, api.F32, norm, 1e-6,
                                               idxp, twp, wsp, wsn, sp, arr)
        elif wl.mx4:
            st = lib.flint_moe_forward_mx4(dref, T, xin, ctypes.byref(wstructs[c]), outp, api.F32, idxp, twp,
                                           wsp, wsn, sp, arr)
        elif args.fused:
            st = lib.flint_moe_forward_fused(dref, T, xin, ctypes.byref(wstructs[c]), outp, api.F32, idxp, twp,
                                             wsp, wsn, sp, arr)
        elif events is None:
            st = lib.flint_moe_forward(dref, T, xin, ctypes.byref(wstructs[c]), outp, api.F32, idxp, twp, wsp, wsn, sp)
        else:
            st = lib.flint_moe_forward_profiled(dref, T, xin, ctypes.byref(wstructs[c]), outp, api.F32, idxp, twp,
                                                wsp, wsn, sp, arr)
        if st != 0:
            raise api.FlintError(st, "flint_moe_forward")

    def step(i, events=None):
        if not stack:
            layer_call(i % n_copies, xp, events[0] if events else None)
            return
        xin = xp
        for l in range(n_copies):
            nxt = ctypes.c_void_p(xs[l % 2].data_ptr()) if l + 1 < n_copies else None
            layer_call(l, xin, events[l] if events else None, nxt)
            xin = nxt

    # routing per copy (for the algorithmic byte counts)
    per_copy = []
    if stack:
        step(0)
    for c in range(n_copies if not stack else 1):
        layer_call(c, xp)
        torch.cuda.synchronize()
        per_copy.append(algorithmic(wl, idx.cpu().numpy()))
    if stack:
        # algorithmic bytes of the stack: every layer's own routing
        per_copy = []
        xin = xp
        for l in range(n_copies):
            nxt = ctypes.c_void_p(xs[l % 2].data_ptr()) if l + 1 < n_copies else None
            layer_call(l, xin, None, nxt)
            torch.cuda.synchronize()
            per_copy.append(algorithmic(wl, idx.cpu().numpy()))
            xin = nxt

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        # one graph holding n_copies consecutive steps (one full weight rotation)
        g = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            sp = ctypes.c_void_p(s2.cuda_stream)
            with torch.cuda.graph(g, stream=s2):
                for i in range(n_copies if not stack else 1):
                    step(i)
        sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        graph = g
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()

    # ---- headline: K steps, bracketed by synchronisation -------------------
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    if graph is not None:
        per = n_copies if not stack else 1
        reps = max(1, args.steps // per)
        for _ in range(reps):
            graph.replay()
        steps_done = reps * per
    else:
        for i in range(args.steps):
            step(i)
        steps_done = args.steps
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / steps_done
    tokens_per_s = T / (ms / 1e3)

    # ---- per-stage timing pass: start/stop events stamped at the stages' own
    # first-kernel begin and last-kernel end, on the library's stream ---------
    hev = HipEvents()
    n_prof = min(args.steps, 100)
    n_layers_step = n_copies if stack else 1
    ev_sets = [[hev.create(10) for _ in range(n_layers_step)] for _ in range(n_prof)]
    for i in range(n_prof):
        step(i, ev_sets[i])
    torch.cuda.synchronize()
    names = ["router", "topk_dispatch", "gate_up", "down", "combine"]
    if args.fused:  # stage 1 is the fused kernel (top-k through down); stages 2 and 3 are empty
        names = ["router", "fused", "_empty2", "_empty3", "combine"]
    stage = {n: [] for n in names}
    for i in range(n_prof):
        for evs in ev_sets[i]:
            for j, n in enumerate(names):
                stage[n].append(hev.ms(evs[2 * j], evs[2 * j + 1]))
    for sets in ev_sets:
        for evs in sets:
            hev.destroy(evs)
    stage_us = {n: float(np.mean(v) * 1e3) for n, v in stage.items() if not n.startswith("_")}

    # algorithmic figures averaged over the copies the steps used
    avg = lambda key: float(np.mean([p[key] for p in per_copy]))  # noqa: E731
    gate_up_bytes = avg("gate_up_bytes")
    layer_bytes = avg("layer_bytes")
    layer_flops = float(np.mean([p["flops"]["layer"] for p in per_copy]))
    gu_flops = float(np.mean([p["flops"]["gate_up"] for p in per_copy]))
    big = gu_flops / gate_up_bytes >= RIDGE  # arithmetic intensity of the gate/up kernel
    kernel = "k_expert_stream_mx4" if wl.mx4 else ("k_expert_stream" if T <= STREAM_MAX_T else "k_tiled")
    kname = f"{kernel}<gate/up> (grouped gate/up GEMM + SwiGLU, routed and shared)"
    if args.fused:
        # the dominant kernel is the fused one: the gate/up and the down bytes
        kernel = "k_fused_decode"
        kname = "k_fused_decode (top-k, dispatch, gate/up + SwiGLU, down)"
        gate_up_bytes = avg("gate_up_bytes") + avg("down_bytes")
        stage_us["gate_up"] = stage_us["fused"]
    digest = sources_digest(kernel)
    traffic = counters_traffic(kernel, wl.name, digest)
    if big:
        achieved = gu_flops / (stage_us["gate_up"] * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / BF16_PEAK_TFLOPS, "traffic": traffic, "kernel": kname,
                    "per_launch": {"flops": gu_flops, "bytes": gate_up_bytes, "mean_us": stage_us["gate_up"]}}
    else:
        achieved = gate_up_bytes / (stage_us["gate_up"] * 1e-6) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": kname,
                    "per_launch": {"bytes": gate_up_bytes, "mean_us": stage_us["gate_up"]}}
    roofline["sources_sha256"] = digest
    layer_time_s = ms / 1e3 / (n_copies if stack else 1)
    layer = {"hbm_GBs": layer_bytes / layer_time_s / 1e9,
             "hbm_frac": layer_bytes / layer_time_s / 1e9 / HBM_PEAK_GBS,
             "mfma_TFLOPs": layer_flops / layer_time_s / 1e12,
             "mfma_frac": layer_flops / layer_time_s / 1e12 / BF16_PEAK_TFLOPS,
             "algorithmic_bytes": layer_bytes, "flops": layer_flops,
             "distinct_experts": avg("distinct")}

    result = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": steps_done, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {'47 stacked' if stack else 'one'} Flint MoE layer(s), T={T}, "
                               f"H={wl.hidden}, E={wl.n_experts} top-{wl.top_k}, I={wl.inter}, "
                               f"Is={wl.shared_inter}" + (", expert weights MXFP4" if wl.mx4 else "")
                               + (", fused decode kernel" if args.fused else ""),
                   "T": T, "weight_copies": n_copies,
                   "graph": bool(graph is not None), "wall_s": wall},
        "roofline": roofline,
        "layer_roofline": layer,
        "stages_us": stage_us,
        "step_us_percentiles": step_percentiles(step, n_prof),
    }
    result["device"], result["hbm_read_measured_GBs"] = device_and_read_rate()
    # parity of one call (weight copy 0 / the stack's first layer), outside the timed region
    layer_call(0, xp)
    torch.cuda.synchronize()
    result["parity"] = parity_report(wl, layers[0], x, out, idx, tw)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, layers[0], x, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
