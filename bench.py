"""Benchmark: one step = one gated GQA attention call (split, QK-norm, partial RoPE,
KV append, causal GQA attention, sigmoid gate) on one batch of synthetic input.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_4b]

Prints one JSON line.  The default workload is the Qwen3.5-4B single-stream
decode (16 query / 4 KV heads, head_dim 256, rotary_dim 64, 4096 cached
tokens, bf16).  Inputs are resident in HBM before timing starts; decode and
verify rotate over enough distinct buffer sets (>= 1 GB) that every step reads
its KV cache from HBM rather than from the 256 MB Infinity Cache.  The K timed
steps are captured in one HIP graph and replayed once, bracketed by HIP events
on the launch stream.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from gated_gqa_attention_amd import binding  # noqa: E402
from gated_gqa_attention_amd.workloads import (DTYPES, WORKLOADS, make_inputs, make_turbo4v_inputs, make_turbo8_inputs,  # noqa: E402
                                               to_paged)

METRIC = "gated-GQA attn tokens/s + effective HBM GB/s (% of peak), 4B geometry decode"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA
ROTATE_BYTES = 1 << 30         # rotate over at least this many bytes of inputs

DEFAULT_STEPS = {"decode_4b": (2000, 200), "verify_24x2": (1000, 100), "ragged_4b": (20, 3),
                 "prefill_4b": (20, 3), "tiny_f32": (1000, 100)}


def algorithmic_work(w, seq_lens, kv="native"):
    """Bytes the method must move and FLOPs it must do per call (QK^T and PV only).

    Returns (total bytes, output bytes, flops).  The output bytes are listed apart
    because a call that splits its keys writes the output from a second, small
    kernel; every other byte is moved by the kernel that streams the KV cache.
    Bytes of one cached row of one KV head: native D elements of the dtype;
    turbo8 D one-byte codes plus D/16 bf16 scales, for K and for V; turbo4v K D
    bf16, V D/2 index bytes plus D/16 E4M3 scale bytes."""
    es = 2 if w.dtype == "bf16" else 4
    B, L, Hq, Hkv, D = w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim
    n = [int(x) for x in seq_lens]
    krow, vrow = {"native": (D * es, D * es), "turbo8": (D + D // 8, D + D // 8),
                  "turbo4v": (2 * D, D // 2 + D // 16)}[kv]
    kv_read = sum(n) * Hkv * (krow + vrow)               # cached K and V rows
    reads = B * L * Hq * 2 * D * es + 2 * B * L * Hkv * D * es + 2 * D * es + 4 * B + 4 * B * L
    out = B * L * Hq * D * es
    writes = out + B * L * Hkv * (krow + vrow)
    keys = sum(nb * L + L * (L + 1) // 2 for nb in n)    # sum over rows of the keys each row sees
    flops = keys * Hq * 4 * D
    return kv_read + reads + writes, out, flops


# Sources that define the kernels of each route (the kernels, their shared
# device code and the launch planner); a traffic figure taken on other
# versions of these files is stale.
ROUTE_SOURCES = {
    "fused_splitk": ("qsa_stream.hip", "qsa_merge.hip", "qsa_device.h", "qsa_internal.h", "qsa_api.hip"),
    "prepared_tiles": ("qsa_prefill.hip", "qsa_rows.hip", "qsa_merge.hip", "qsa_device.h", "qsa_internal.h",
                       "qsa_api.hip"),
}


def kernel_source_hash(route="fused_splitk"):
    """Hash of the sources the kernels of `route` are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_gqa_attention_amd", "csrc")
    for name in ROUTE_SOURCES[route]:
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload, route, per_launch_units=1):
    """HBM bytes per launch from committed rocprofv3 PMC summaries, if they were
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != kernel_source_hash(route):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"]) * per_launch_units
    except (KeyError, ValueError):
        return None


class Call:
    """Device buffers and C-ABI arguments of one buffer set."""

    def __init__(self, w, dev, workspace, max_seq_len, stream, block_size=0):
        self.w, self.dev = w, dev
        self.cfg = binding.make_cfg(
            batch=w.batch, q_len=w.q_len, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
            head_dim=w.head_dim, rotary_dim=w.rotary_dim, rope_theta=w.rope_theta, rms_eps=w.rms_eps,
            dtype=DTYPES[w.dtype], max_seq_len=max_seq_len, q_norm_w=dev["w_q"], k_norm_w=dev["w_k"],
            workspace=workspace, stream=stream)
        if "k_codes" in dev:
            self.kv = binding.make_kv(dev["k_codes"], dev["v_codes"], dev["seq_offset"], dev["capacity"],
                                      k_scales=dev["k_scales"], v_scales=dev["v_scales"])
        elif "v_codes" in dev:                          # bf16 K + Turbo4 V
            self.kv = binding.make_kv(dev["k_cache"], dev["v_codes"], dev["seq_offset"], dev["capacity"],
                                      v_scales=dev["v_scales"])
        elif "block_table" in dev:
            self.kv = binding.make_kv(dev["k_cache"], dev["v_cache"], None, dev["capacity"], dev["block_table"],
                                      block_size)
        else:
            self.kv = binding.make_kv(dev["k_cache"], dev["v_cache"], dev["seq_offset"], dev["capacity"])
        self.ws = workspace
        self.out = torch.empty((w.batch, w.q_len, w.num_q_heads, w.head_dim), dtype=DTYPES[w.dtype],
                               device=dev["q_gate"].device)

    def __call__(self):
        d = self.dev
        binding.gated_attention(self.cfg, self.kv, d["q_gate"], d["k_new"], d["v_new"], d["seq_lens"],
                                d["positions"], self.out)


def kernel_times(calls, stream, n):
    """Average duration (ms) of the attention kernel over n eager calls, from HIP
    events the library records on the launch stream right around that kernel.
    The stream drains before each call, so a dispatch's begin stamp is not
    taken while it waits for the previous call's kernels."""
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    with torch.cuda.stream(stream):
        for a, b in pairs:              # torch creates an event on its first record
            a.record(stream)
            b.record(stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i, (a, b) in enumerate(pairs):
            c = calls[i % len(calls)]
            c.cfg.timing_begin, c.cfg.timing_end = a.cuda_event, b.cuda_event
            stream.synchronize()
            c()
    torch.cuda.synchronize()
    for c in calls:
        c.cfg.timing_begin = c.cfg.timing_end = None
    return sum(a.elapsed_time(b) for a, b in pairs) / n


def copy_calibration(steps=20, nbytes=256 << 20):
    """Plain device-to-device copy of known size (torch's copy kernel): the
    reference point that scales rocprofv3's FETCH_SIZE / WRITE_SIZE counters."""
    dev = torch.device("cuda:0")
    src = torch.randn(nbytes // 4, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "steps": steps,
                      "ms_per_copy": round(ms, 4), "gbs_read_plus_write": round(2 * nbytes / ms / 1e6, 1)}),
          flush=True)


def cpu_baseline(w, inputs, tokens_per_call, budget_s=10.0):
    """The oracle, as is, on this host's cores over a bounded sample of the workload."""
    import numpy as np
    import oracle

    g = oracle.Geometry(w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim, w.rotary_dim,
                        w.rope_theta, w.rms_eps, 0.0, w.dtype)
    total_rows = w.batch * w.q_len * w.num_q_heads
    threads = max(1, oracle.threads())
    # time a few rows (one per core at most, so they run side by side) to size the sample
    rng = np.random.default_rng(0)
    probe = np.sort(rng.choice(total_rows, size=min(total_rows, threads), replace=False)).astype(np.int64)
    kr, vr = oracle.new_kv(g, inputs["k_new"], inputs["v_new"], inputs["w_k"], inputs["positions"])
    t0 = time.perf_counter()
    oracle.attention(g, inputs["q_gate"], inputs["w_q"], inputs["k_cache"], inputs["v_cache"],
                     inputs["seq_offset"], inputs["seq_lens"], inputs["positions"], kr, vr, rows=probe)
    t_row = max(time.perf_counter() - t0, 1e-6)         # wall time of one row per core
    est_full = -(-total_rows // threads) * t_row
    rows_budget = total_rows if est_full <= budget_s else int(budget_s / t_row) * threads
    if rows_budget >= total_rows:
        t0 = time.perf_counter()
        done = 0
        while done == 0 or time.perf_counter() - t0 < budget_s:
            oracle.gated_attention(g, inputs)
            done += 1
        dt = time.perf_counter() - t0
        sample = f"{done} full call(s) of {w.name} ({total_rows} query rows each, append included)"
        tokens = done * tokens_per_call
    else:
        rows = np.sort(rng.choice(total_rows, size=max(1, rows_budget), replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        kr, vr = oracle.new_kv(g, inputs["k_new"], inputs["v_new"], inputs["w_k"], inputs["positions"])
        oracle.attention(g, inputs["q_gate"], inputs["w_q"], inputs["k_cache"], inputs["v_cache"],
                         inputs["seq_offset"], inputs["seq_lens"], inputs["positions"], kr, vr, rows=rows)
        dt = time.perf_counter() - t0
        sample = (f"{len(rows)} of {total_rows} query rows of {w.name} (random, seeded) plus the "
                  f"full append; scaled by rows")
        tokens = tokens_per_call * len(rows) / total_rows
    return {"value": tokens / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3), "cpu_model": cpu_model()}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measure(w, steps, warm, launch="graph", force_splits=0, sets=None, block_size=0, kv="native"):
    """Time one workload: `warm` untimed eager calls, then `steps` calls captured in
    one HIP graph, replayed once untimed and once timed (HIP events on the launch
    stream), then the attention kernel on its own in an eager pass.  block_size >
    0: the cache is laid out in shuffled blocks of that many rows (paged).
    Returns the inputs and a dict of figures."""
    dev = torch.device("cuda:0")
    inputs = {"turbo8": make_turbo8_inputs, "turbo4v": make_turbo4v_inputs}.get(kv, make_inputs)(w)
    max_seq_len = int((inputs["seq_lens"].max() + w.q_len).item())
    base = {k: v.to(dev) for k, v in inputs.items()}
    if block_size:
        base = to_paged(base, block_size, seed=w.seed)
    set_bytes = sum(v.numel() * v.element_size() for v in base.values())
    sets = sets or max(1, min(256, -(-ROTATE_BYTES // set_bytes)))
    if set_bytes * sets > 64 * (1 << 30):
        sets = 1
    stream = torch.cuda.Stream()   # default priority
    probe = binding.make_cfg(
        batch=w.batch, q_len=w.q_len, num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads,
        head_dim=w.head_dim, rotary_dim=w.rotary_dim, rope_theta=w.rope_theta, rms_eps=w.rms_eps,
        dtype=DTYPES[w.dtype], max_seq_len=max_seq_len, q_norm_w=base["w_q"], k_norm_w=base["w_k"],
        force_splits=force_splits, stream=stream)
    ws_bytes = binding.workspace_size(probe)
    plan = binding.describe_plan(probe)

    calls = []
    for i in range(sets):
        d = base if i == 0 else {k: v.clone() for k, v in base.items()}
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        c = Call(w, d, ws, max_seq_len, stream, block_size)
        c.cfg.force_splits = force_splits
        calls.append(c)
    torch.cuda.synchronize()

    with torch.cuda.stream(stream):
        for i in range(warm):
            calls[i % sets]()
    torch.cuda.synchronize()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if launch == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(steps):
                calls[(warm + i) % sets]()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):     # one untimed replay: the graph's first launch sets it up
            graph.replay()
        torch.cuda.synchronize()
        t_host = time.perf_counter()
        with torch.cuda.stream(stream):     # replay() launches on the current stream
            start.record(stream)
            graph.replay()
            end.record(stream)
        torch.cuda.synchronize()
        t_host = time.perf_counter() - t_host
    else:
        t_host = time.perf_counter()
        with torch.cuda.stream(stream):
            start.record(stream)
            for i in range(steps):
                calls[(warm + i) % sets]()
            end.record(stream)
        torch.cuda.synchronize()
        t_host = time.perf_counter() - t_host
    ms = start.elapsed_time(end)
    errs = [int(c.ws[:4].view(torch.int32).item()) for c in calls]
    if any(errs):
        print(f"bench.py: device-side range error flagged on {w.name}: {errs}", file=sys.stderr)
        sys.exit(1)

    # the kernel that streams the KV cache, timed on its own in a separate eager pass
    kernel_ms = kernel_times(calls, stream, min(steps, 500))

    tokens_per_call = w.batch * w.q_len
    bytes_call, out_bytes, flops_call = algorithmic_work(w, inputs["seq_lens"], kv)
    if block_size:                                      # the block table entries the call reads
        bytes_call += 4 * int(((inputs["seq_lens"] + w.q_len + block_size - 1) // block_size).sum())
    fields = dict(kv.split("=") for kv in plan.split())
    route = fields["route"]
    # bytes the streaming kernel moves: all of the call's, except the output when a
    # separate merge kernel writes it
    merged_apart = int(fields["chunks"]) > 1 and fields.get("merge") == "kernel"
    bytes_kernel = bytes_call - (out_bytes if merged_apart else 0)
    step_s = ms / 1e3 / steps
    hbm_bound = route != "prepared_tiles"
    if hbm_bound:
        call_ach, kern_ach = bytes_call / step_s / 1e9, bytes_kernel / (kernel_ms / 1e3) / 1e9
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        call_ach, kern_ach = flops_call / step_s / 1e12, flops_call / (kernel_ms / 1e3) / 1e12
        peak, unit = MFMA_BF16_PEAK_TFS, "TFLOP/s"
    kname = {"fused_splitk": "stream_kernel", "prepared_tiles": "tile_kernel"}.get(route, "rows_f32_kernel")
    if kv != "native":
        kname = "quant_kernel"
    res = {
        "steps": steps, "warmup": warm, "ms_per_step": ms / steps, "tokens_per_s": tokens_per_call / step_s,
        "effective_gbs": bytes_call / step_s / 1e9, "effective_tflops": flops_call / step_s / 1e12,
        "host_wall_s": t_host, "plan": plan, "route": route, "buffer_sets": sets,
        "bound": "hbm" if hbm_bound else "mfma", "unit": unit, "peak": peak,
        "call_achieved": call_ach, "call_frac": call_ach / peak,
        "kernel": kname, "kernel_us": kernel_ms * 1e3, "kernel_achieved": kern_ach,
        "kernel_frac": kern_ach / peak, "bytes_call": bytes_call, "bytes_kernel": bytes_kernel,
        "flops_call": flops_call, "tokens_per_call": tokens_per_call,
        "cached_tokens": int(inputs["seq_lens"].sum()), "block_size": block_size, "kv": kv if kv != "native" else w.dtype,
    }
    del calls, base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return inputs, res


def measure_proj(w, which, steps, warm, hidden=None):
    """Time one projection (which: "qkv" or "o") on the rows of workload w, rotating
    over >= 1 GB of weight sets so that every step streams its weights from HBM.
    Returns figures against the HBM roofline (the weights dominate the bytes)."""
    from gated_gqa_attention_amd.workloads import HIDDEN_4B, make_proj_inputs
    hidden = hidden or HIDDEN_4B
    dev = torch.device("cuda:0")
    p = make_proj_inputs(w, hidden=hidden)
    B, L, Hq, Hkv, D = w.batch, w.q_len, w.num_q_heads, w.num_kv_heads, w.head_dim
    M = B * L
    wkey = "w_qkv" if which == "qkv" else "w_o"
    wbytes = p[wkey].numel() * 2
    sets = max(1, min(256, -(-ROTATE_BYTES // wbytes)))
    weights = [p[wkey].to(dev)] + [p[wkey].to(dev).clone() for _ in range(sets - 1)]
    x = p["x"].to(dev)
    attn = torch.randn((M, Hq * D), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16).to(dev)
    q_gate = torch.empty((B, L, Hq, 2 * D), dtype=torch.bfloat16, device=dev)
    k_new = torch.empty((B, L, Hkv, D), dtype=torch.bfloat16, device=dev)
    v_new = torch.empty_like(k_new)
    y = torch.empty((M, hidden), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.Stream()
    cfg = binding.make_cfg(batch=B, q_len=L, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, rotary_dim=w.rotary_dim,
                           rope_theta=w.rope_theta, rms_eps=w.rms_eps, dtype=torch.bfloat16, max_seq_len=L,
                           q_norm_w=1, k_norm_w=1, stream=stream)

    def call(i):
        if which == "qkv":
            binding.qkv_proj(cfg, x, weights[i % sets], hidden, q_gate, k_new, v_new)
        else:
            binding.o_proj(cfg, attn, weights[i % sets], hidden, y)

    with torch.cuda.stream(stream):
        for i in range(warm):
            call(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            call(warm + i)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        graph.replay()
        end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    if which == "qkv":
        nbytes = wbytes + M * hidden * 2 + (q_gate.numel() + k_new.numel() + v_new.numel()) * 2
    else:
        nbytes = wbytes + M * Hq * D * 2 + M * hidden * 2
    gbs = nbytes / (ms / 1e3) / 1e9
    del weights
    torch.cuda.empty_cache()
    return {"us_per_call": round(ms * 1e3, 3), "steps": steps, "warmup": warm, "rows": M, "hidden": hidden,
            "weight_sets": sets, "algorithmic_bytes": nbytes, "bound": "hbm", "unit": "GB/s",
            "call_achieved": round(gbs, 1), "call_frac": round(gbs / HBM_PEAK_GBS, 4)}


def measure_gdn(w, steps, warm):
    """Time one GatedDeltaNet decode step (qsa_gdn_decode) of workload w in a HIP
    graph, rotating over state sets of >= 1 GB in all so that every step streams
    its recurrent state from HBM.  The state (read and written, fp32) dominates
    the bytes; returns figures against the HBM roofline."""
    from gated_gqa_attention_amd.workloads import make_gdn_inputs
    dev = torch.device("cuda:0")
    x = make_gdn_inputs(w)
    B, C, K, Hv, D = w.batch, w.channels, w.conv_kernel, w.num_v_heads, w.v_head_dim
    per_set = (x["state"].numel() + x["conv_state"].numel()) * 4
    sets = max(1, min(64, -(-ROTATE_BYTES // per_set)))
    fixed = {k: x[k].to(dev) for k in ("qkv", "z", "a", "b", "conv_w", "a_log", "dt_bias", "norm_w")}
    states = [(x["conv_state"].to(dev), x["state"].to(dev)) for _ in range(sets)]
    y = torch.empty((B, Hv, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.Stream()
    cfg = binding.make_gdn_cfg(batch=B, num_k_heads=w.num_k_heads, num_v_heads=Hv, k_head_dim=w.k_head_dim,
                               v_head_dim=D, conv_kernel=K, rms_eps=w.rms_eps, stream=stream.cuda_stream)

    def call(i):
        cs, st = states[i % sets]
        binding.gdn_decode(cfg, fixed["qkv"], fixed["z"], fixed["a"], fixed["b"], fixed["conv_w"], fixed["a_log"],
                           fixed["dt_bias"], fixed["norm_w"], cs, st, y)

    with torch.cuda.stream(stream):
        for i in range(warm):
            call(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(steps):
            call(warm + i)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        graph.replay()
        end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    nbytes = (2 * per_set + (B * C + B * Hv * D + 2 * B * Hv + C * K + Hv + D) * 2 + Hv * 4 + B * Hv * D * 2)
    gbs = nbytes / (ms / 1e3) / 1e9
    del states
    torch.cuda.empty_cache()
    return {"tokens_per_s": round(B / (ms / 1e3), 1), "us_per_call": round(ms * 1e3, 3), "steps": steps,
            "warmup": warm, "batch": B, "state_sets": sets, "algorithmic_bytes": nbytes, "bound": "hbm",
            "unit": "GB/s", "call_achieved": round(gbs, 1), "call_frac": round(gbs / HBM_PEAK_GBS, 4),
            "kernel": "gdn_decode_kernel (one launch per call)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="decode_4b", choices=sorted(WORKLOADS))
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"])
    ap.add_argument("--force-splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only --workload (by default the other bf16 workloads follow as extra keys)")
    ap.add_argument("--sets", type=int, default=None, help="buffer sets to rotate over")
    ap.add_argument("--kv", choices=["native", "turbo8", "turbo4v"], default="native",
                    help="cache storage: the activations' dtype, Turbo8 (E4M3 codes + bf16 scales) or bf16 K + "
                         "Turbo4 V (4-bit Lloyd-Max indices + E4M3 scales)")
    ap.add_argument("--block-size", type=int, default=0,
                    help="lay the cache out in shuffled blocks of this many rows (paged; 0: contiguous)")
    ap.add_argument("--proj", choices=["qkv", "o"], default=None,
                    help="time only the q/k/v (or o) projection at the decode shape and print its figures")
    ap.add_argument("--gdn", choices=["gdn_decode_4b", "gdn_decode_4b_b1"], default=None,
                    help="time only this GatedDeltaNet decode workload and print its figures")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 256 MiB device copy instead (reference for the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the attention core shards by sequence or KV head without any exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    torch.cuda.set_device(torch.device("cuda:0"))
    if args.gdn:
        from gated_gqa_attention_amd.workloads import GDN_WORKLOADS
        print(json.dumps({"gdn": args.gdn, **measure_gdn(GDN_WORKLOADS[args.gdn], args.steps or 200,
                                                         args.warmup or 10)}), flush=True)
        return
    if args.proj:
        print(json.dumps({"proj": args.proj, **measure_proj(WORKLOADS["decode_4b"], args.proj, args.steps or 1000,
                                                            args.warmup or 50)}), flush=True)
        return
    w = WORKLOADS[args.workload]
    steps, warm = DEFAULT_STEPS.get(w.name, (100, 10))
    steps = args.steps if args.steps is not None else steps
    warm = args.warmup if args.warmup is not None else warm
    inputs, r = measure(w, steps, warm, args.launch, args.force_splits, args.sets, args.block_size,
                        args.kv)

    traffic = traffic_from_profiles(w.name, r["route"]) if r["route"] in ROUTE_SOURCES else None
    roof = {"bound": r["bound"], "achieved": round(r["kernel_achieved"], 1), "peak": r["peak"],
            "unit": r["unit"], "frac": round(r["kernel_frac"], 4), "traffic": traffic,
            "kernel": r["kernel"], "kernel_us": round(r["kernel_us"], 3),
            "algorithmic_bytes_per_launch": r["bytes_kernel"],
            "algorithmic_flops_per_launch": r["flops_call"],
            "kernel_share_of_step": round(r["kernel_us"] / 1e3 / r["ms_per_step"], 3),
            # the whole call (every kernel of it, launch gaps included) against the same peak
            "call_achieved": round(r["call_achieved"], 1), "call_frac": round(r["call_frac"], 4)}
    line = {
        "metric": METRIC, "value": round(r["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "ms_per_step": round(r["ms_per_step"], 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) inputs, norm weights 1+N(0,0.1))",
        "config": {"workload": w.name, "batch": w.batch, "q_len": w.q_len,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "rotary_dim": w.rotary_dim, "rope_theta": w.rope_theta,
                   "cached_tokens": r["cached_tokens"], "buffer_sets": r["buffer_sets"],
                   "launch": "hipgraph" if args.launch == "graph" else "eager", "plan": r["plan"]},
        "effective_gbs": round(r["effective_gbs"], 1), "effective_tflops": round(r["effective_tflops"], 3),
        "host_wall_s": round(r["host_wall_s"], 4),
        "roofline": roof,
    }
    if not args.no_cpu_baseline and args.kv == "native":
        line["cpu_baseline"] = cpu_baseline(w, inputs, r["tokens_per_call"])
    del inputs
    if not args.no_extras:
        extras = {}
        for name in ("verify_24x2", "ragged_4b", "prefill_4b"):
            if name == w.name:
                continue
            ew = WORKLOADS[name]
            es, ewarm = DEFAULT_STEPS[name]
            _, x = measure(ew, es, ewarm)
            extras[name] = {
                "tokens_per_s": round(x["tokens_per_s"], 1), "us_per_call": round(x["ms_per_step"] * 1e3, 3),
                "steps": es, "warmup": ewarm, "plan": x["plan"], "bound": x["bound"], "unit": x["unit"],
                "call_achieved": round(x["call_achieved"], 1), "call_frac": round(x["call_frac"], 4),
                "kernel": x["kernel"], "kernel_us": round(x["kernel_us"], 3),
                "kernel_achieved": round(x["kernel_achieved"], 1), "kernel_frac": round(x["kernel_frac"], 4),
                "cached_tokens": x["cached_tokens"]}
        # the ragged batch again, its cache in shuffled blocks of 64 rows (paged)
        _, x = measure(WORKLOADS["ragged_4b"], *DEFAULT_STEPS["ragged_4b"], block_size=64)
        extras["ragged_4b_paged64"] = {
            "tokens_per_s": round(x["tokens_per_s"], 1), "us_per_call": round(x["ms_per_step"] * 1e3, 3),
            "steps": x["steps"], "warmup": x["warmup"], "plan": x["plan"], "block_size": 64, "bound": "hbm",
            "unit": "GB/s", "call_achieved": round(x["call_achieved"], 1), "call_frac": round(x["call_frac"], 4),
            "kernel": x["kernel"], "kernel_us": round(x["kernel_us"], 3),
            "kernel_achieved": round(x["kernel_achieved"], 1), "kernel_frac": round(x["kernel_frac"], 4)}
        # decode and the ragged batch on the quantized caches: Turbo8 (E4M3 codes, bf16
        # scale per 16) and bf16 K + Turbo4 V (4-bit indices, E4M3 scale per 16)
        for kvq in ("turbo8", "turbo4v"):
            for name in ("decode_4b", "ragged_4b"):
                _, x = measure(WORKLOADS[name], *DEFAULT_STEPS[name], kv=kvq)
                extras[f"{name}_{kvq}"] = {
                    "tokens_per_s": round(x["tokens_per_s"], 1), "us_per_call": round(x["ms_per_step"] * 1e3, 3),
                    "steps": x["steps"], "warmup": x["warmup"], "plan": x["plan"], "kv": kvq, "bound": "hbm",
                    "unit": "GB/s", "algorithmic_bytes_per_call": x["bytes_call"],
                    "call_achieved": round(x["call_achieved"], 1), "call_frac": round(x["call_frac"], 4),
                    "kernel": x["kernel"], "kernel_us": round(x["kernel_us"], 3),
                    "kernel_achieved": round(x["kernel_achieved"], 1), "kernel_frac": round(x["kernel_frac"], 4)}
        # the projections either side of the core, at the decode shape (one row)
        extras["qkv_proj_4b"] = measure_proj(WORKLOADS["decode_4b"], "qkv", 1000, 50)
        extras["o_proj_4b"] = measure_proj(WORKLOADS["decode_4b"], "o", 1000, 50)
        # the other layer type of the hybrid model: a GatedDeltaNet decode step
        from gated_gqa_attention_amd.workloads import GDN_WORKLOADS
        extras["gdn_decode_4b"] = measure_gdn(GDN_WORKLOADS["gdn_decode_4b"], 200, 10)
        extras["gdn_decode_4b_b1"] = measure_gdn(GDN_WORKLOADS["gdn_decode_4b_b1"], 1000, 20)
        line["workloads"] = extras
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
