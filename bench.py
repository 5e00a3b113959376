#!/usr/bin/env python3
"""Throughput of one GPU's share of an MoE layer (route -> permute -> grouped FFN -> combine).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mixtral] [--cpu-seconds S]

A step is one pass of the whole layer over one batch of synthetic tokens whose
inputs (tokens, router logits, source ranks, expert weights) are already
resident in HBM.  W untimed steps, then K steps timed with HIP events on the
stream the library launches on; per-call durations come from event pairs
recorded around each of the four calls inside the same timed region.

Prints ONE JSON line: throughput in TFLOP/s (algorithmic: 2*R*H*F per GEMM
matrix, R = routed (token, local expert) rows, padding excluded), tokens/s,
the fraction of the bf16 MFMA peak, a roofline entry for the dominant call
(the grouped FFN: layer0 GEMM + fused activation + layer1 GEMM) and the CPU
oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
RIDGE_FLOP_PER_BYTE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)

# The pages' own figures, quoted beside this build's numbers as context only: they are speedups of
# whole multi-GPU MoE layers / models (communication included) over other systems on NVIDIA GPUs,
# not per-GPU throughput, so nothing here is divided by them.
PAGES_CONTEXT = {
    "comet_moe_layer_speedup_avg": 1.96,
    "comet_end_to_end_speedup_avg": 1.71,
    "tile_signalling_moe_layer_speedup_max": 2.74,
    "tile_signalling_end_to_end_speedup_max": 2.64,
    "source": "Comet (arXiv 2502.19811): abstract, sections 1 and 7; tile-level signalling "
              "follow-up (arXiv 2607.19539): abstract, on 4x A100",
    "note": "context only: speedups of multi-GPU layers over other systems, not comparable to "
            "one GPU's absolute throughput",
}

WORKLOAD_NAMES = {
    "tiny": "tiny MoE layer (256 tokens, hidden 512, FFN 1024, 8 experts top-2, GELU)",
    "mixtral": "Mixtral-shaped MoE layer, one GPU's share (4096 tokens, hidden 4096, FFN 14336, "
               "8 experts top-2, SwiGLU)",
    "fine_grained": "fine-grained MoE layer (8192 tokens, hidden 2048, FFN 1408, 64 experts top-6, "
                    "SwiGLU, Zipf(1.1)-biased router)",
    "ep_share": "expert-parallel share (16384 tokens from 8 source ranks, 8 local of 64 experts, "
                "top-8, hidden 4096, FFN 2048, SwiGLU)",
    "tp2_share": "tensor-parallel rank 0 of 2 of the expert-parallel share (FFN columns 0..1023 of "
                 "8 local experts; partial output)",
    "tp4_share": "tensor-parallel rank 0 of 4 of the expert-parallel share (FFN columns 0..511 of "
                 "8 local experts; partial output)",
    "tp8_share": "tensor-parallel rank 0 of 8 of the expert-parallel share (FFN columns 0..255 of "
                 "8 local experts; partial output)",
    "decode": "decode-sized MoE layer (64 tokens, hidden 7168, FFN 2048, 256 experts top-8, SwiGLU)",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral", choices=list(WORKLOAD_NAMES))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU oracle sample budget in seconds (0 disables the CPU baseline)")
    ap.add_argument("--cu-partition", action="store_true",
                    help="only run the CU-partition sweep (a copy of the remote-labelled token rows on nc CUs "
                         "while the grouped FFN runs on the others) and print its own JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (calibrates the HBM byte "
                         "counters FETCH_SIZE / WRITE_SIZE against a known size) and exit")
    return ap.parse_args()


# HBM traffic of the dominant call, measured with rocprofv3 counters on the same
# kernel sources (profiles/hbm_traffic_grouped_ffn.md); reported only while the
# kernel sources still hash to the values recorded there.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_grouped_ffn.md")
GEMM_SOURCES = [os.path.join(ROOT, "mixture_experts_layer_moe_amd", "csrc", f)
                for f in ("grouped_gemm.hip", "common.h")]


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """Scaled HBM bytes per moe_grouped_ffn launch from the counter summary, or None if stale/absent."""
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256") != gemm_source_hash():
        return None
    entry = rec.get("workloads", {}).get(workload)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


def copy_calibration():
    import torch
    n = 1 << 28  # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 4 * n, "copies": 5}), flush=True)


def cu_partition(args):
    """Stand-in for the communication/computation CU split of thread-block specialisation.

    For nc in a sweep of whole XCDs (32-CU steps), two streams with
    complementary CU masks (default priority) are created: a copy of the
    token rows that come from other source ranks -- the bytes a dispatch
    all-to-all would deliver -- runs on the CUs [0, nc) while the grouped FFN
    runs on [nc, n); the library sizes its persistent grid to the stream's CU
    mask.  Partitions that split an XCD leave that XCD with fewer CUs than
    its round-robin share of a one-workgroup-per-CU grid, which then runs in
    two waves (measured: 1.6-1.8x slower FFN at 8, 16 and 48 CUs), so the
    sweep moves whole XCDs.  Reported per nc: the
    FFN alone on its CUs, the FFN and the copy run together, the copy's rate,
    and the FFN's slowdown against all CUs without the copy.
    """
    import ctypes
    import torch
    from mixture_experts_layer_moe_amd import workloads as W
    from mixture_experts_layer_moe_amd.layer import MoELayer

    name = args.workload if args.workload != "mixtral" else "ep_share"
    cfg = W.CONFIGS[name]
    dev = torch.device("cuda:0")
    d = W.make_inputs(cfg, dev)
    layer = MoELayer.from_inputs(cfg, d)
    layer.run()
    torch.cuda.synchronize()
    n = torch.cuda.get_device_properties(dev).multi_processor_count
    src = d["src_rank"] if d["src_rank"] is not None else torch.ones(cfg.T, dtype=torch.int32, device=dev)
    remote = ((src != 0) & (layer.perm.inv_perm >= 0).any(dim=1)).nonzero().squeeze(1)
    rows = d["x"].index_select(0, remote)
    staging = torch.empty_like(rows)
    comm_bytes = 2 * rows.numel() * rows.element_size()
    hip = ctypes.CDLL("libamdhip64.so")
    words = (n + 31) // 32

    def masked_stream(cus):
        mask = (ctypes.c_uint32 * words)()
        for c in cus:
            mask[c // 32] |= 1 << (c % 32)
        h = ctypes.c_void_p()
        err = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), ctypes.c_uint32(words), mask)
        if err != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed ({err})")
        return h, torch.cuda.ExternalStream(h.value, device=dev)

    def once(stream_f, stream_c, with_comm):
        """One FFN launch on stream_f, with or without the copy on stream_c: (ffn, comm, step) ms."""
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.cuda.synchronize()
        e[0].record(stream_f)
        stream_c.wait_event(e[0])
        layer.ffn(stream_f)
        e[1].record(stream_f)
        if with_comm:
            with torch.cuda.stream(stream_c):
                staging.copy_(rows)
            e[2].record(stream_c)
            stream_f.wait_event(e[2])
        e[3].record(stream_f)
        torch.cuda.synchronize()
        return e[0].elapsed_time(e[1]), e[0].elapsed_time(e[2]) if with_comm else None, e[0].elapsed_time(e[3])

    med = lambda v: sorted(v)[len(v) // 2]

    def paired(stream_f, stream_c, reps):
        """The FFN alone and with the copy, alternating rep by rep after two warm-up pairs, so that
        clock and cache drift fall on both alike: medians of (alone ffn, ffn, comm, step)."""
        for _ in range(2):
            once(stream_f, stream_c, False)
            once(stream_f, stream_c, True)
        a, f, c, st = [], [], [], []
        for _ in range(reps):
            a.append(once(stream_f, stream_c, False)[0])
            r = once(stream_f, stream_c, True)
            f.append(r[0])
            c.append(r[1])
            st.append(r[2])
        return med(a), med(f), med(c), med(st)

    reps = max(5, min(args.steps, 20))
    base = torch.cuda.current_stream()
    for _ in range(2):
        once(base, base, False)
    full_ffn = med([once(base, base, False)[0] for _ in range(reps)])
    curve = []
    per_xcd = n // 8
    for nc in (per_xcd, 2 * per_xcd, 3 * per_xcd, 4 * per_xcd):
        if nc >= n:
            break
        hc, sc = masked_stream(range(nc))
        hf, sf = masked_stream(range(nc, n))
        alone, ffn, comm, step = paired(sf, sc, reps)
        torch.cuda.synchronize()
        hip.hipStreamDestroy(hc)
        hip.hipStreamDestroy(hf)
        curve.append({"comm_cus": nc, "ffn_alone_ms": round(alone, 4), "ffn_with_comm_ms": round(ffn, 4),
                      "comm_ms": round(comm, 4), "comm_GBps": round(comm_bytes / (comm * 1e-3) / 1e9, 1),
                      "step_ms": round(step, 4), "ffn_slowdown": round(ffn / full_ffn, 4)})
    print(json.dumps({"cu_partition": name, "cus": n, "comm_rows": int(remote.numel()),
                      "comm_bytes": comm_bytes, "ffn_all_cus_ms": round(full_ffn, 4), "curve": curve}), flush=True)


def cpu_baseline(cfg, d, seconds):
    """The oracle, as it stands, on a bounded sample of the workload's tokens (rank 0, host cores)."""
    import numpy as np
    import torch
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity set
        threads = len(os.sched_getaffinity(0))

    from mixture_experts_layer_moe_amd import workloads as W
    logits = d["logits"].cpu().numpy()
    xs = d["x"]
    order = np.random.default_rng(0).permutation(cfg.T)
    cache = {}

    def weights(le):
        return cache[le]   # staged before the timer starts (below)

    done, rows, elapsed = 0, 0, 0.0
    for t in order[:64]:
        t = int(t)
        idx_t, _ = O.route_topk(logits[t:t + 1], cfg.k)
        # input staging (untimed): this token's row and its local experts' weights on the host
        for e in idx_t.ravel():
            le = int(e) - cfg.expert_begin
            if 0 <= le < cfg.n_local and le not in cache:
                cache[le] = tuple(None if w is None else w[le].to("cpu", torch.float32).numpy()
                                  for w in (d["w0"], d["w0_up"], d["w1"]))
        x_t = xs[t].to("cpu", torch.float64).numpy()[None, :]
        t0 = time.perf_counter()
        O.moe_layer(x_t, logits[t:t + 1], cfg.k, weights, cfg.act,
                    expert_begin=cfg.expert_begin, E_loc=cfg.n_local)
        elapsed += time.perf_counter() - t0
        done += 1
        rows += int(((idx_t >= cfg.expert_begin) & (idx_t < cfg.expert_begin + cfg.n_local)).sum())
        if len(cache) > 16:   # bound host memory: keep the weights of at most 16 experts
            cache.clear()
        if elapsed >= seconds:
            break
    flop = W.flops(cfg, rows)
    cpu, ram = host_description()
    return {
        "value": flop / elapsed / 1e12,
        "unit": "TFLOP/s",
        "tokens_per_s": done / elapsed,
        "cores": int(threads),
        "kind": "oracle",
        "cpu_model": cpu,
        "host_ram_GiB": ram,
        "sample": f"{done} tokens of the workload ({rows} routed rows), float64 per-token loop, "
                  f"{elapsed:.1f} s on {cpu} ({ram} GiB host RAM)",
    }


def host_description():
    """(CPU model, total host RAM in GiB) from /proc, for the CPU baseline's provenance."""
    cpu = platform.processor() or platform.machine()
    ram = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    ram = round(int(line.split()[1]) / (1 << 20), 1)
                    break
    except OSError:
        pass
    return cpu, ram


def ffn_roofline(cfg, R: int, n_hit: int, ffn_ms: float) -> dict:
    """Roofline entry of moe_grouped_ffn for this workload.

    Algorithmic work per launch: 2*R*H*F_loc flop per weight matrix; algorithmic
    bytes: the weights of every expert that received a row, read once, plus the
    real rows of x_perm (read), act (written and read) and y_perm (written).
    The launch is MFMA-bound when its flop per algorithmic byte exceeds the
    ridge of the published peaks (bf16 MFMA / HBM), else HBM-bound (weight
    streaming: the decode-sized and tiny layers).
    """
    from mixture_experts_layer_moe_amd import workloads as W
    n_mats = 3 if cfg.act == "swiglu" else 2
    flop = W.flops(cfg, R)
    nbytes = n_hit * n_mats * cfg.H * cfg.F_loc * 2 + R * cfg.H * 2 + 2 * R * cfg.F_loc * 2 + R * cfg.H * 4
    entry = {"kernel": "moe_grouped_ffn (layer0 grouped GEMM + fused activation, layer1 grouped GEMM)"}
    if flop / nbytes >= RIDGE_FLOP_PER_BYTE:
        achieved = flop / (ffn_ms * 1e-3) / 1e12
        entry.update(bound="mfma", achieved=round(achieved, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                     frac=round(achieved / PEAK_BF16_TFLOPS, 4))
    else:
        achieved = nbytes / (ffn_ms * 1e-3) / 1e9
        entry.update(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                     frac=round(achieved / PEAK_HBM_GBPS, 4))
    entry["algorithmic_flop"] = flop
    entry["algorithmic_bytes"] = nbytes
    return entry


def copy_and_cold(layer, stream, iters: int = 10):
    """HBM context for the two memory-bound calls, measured outside the timed steps.

    copy_GBps: a plain 1 GiB device-to-device copy (bytes read + written per second).
    permute/combine cold: each call timed alone right after writing a 512 MiB
    scratch buffer, which evicts its inputs from the 256 MiB last-level cache.
    """
    import torch
    dev = layer.out.device
    src = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    cold = {}
    for name, call in (("permute", layer.permute), ("combine", layer.combine)):
        ms = []
        for i in range(iters):
            scratch.fill_(i & 0xFF)
            e0.record(stream)
            call()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        cold[name] = sorted(ms)[len(ms) // 2]
    return copy_gbps, cold


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the layer; runs on more than one GPU are not "
              "part of this build (use --gpus 1).", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.cu_partition:
        cu_partition(args)
        return

    import torch
    from mixture_experts_layer_moe_amd import workloads as W
    from mixture_experts_layer_moe_amd.layer import MoELayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cfg = W.CONFIGS[args.workload]
    d = W.make_inputs(cfg, dev)
    layer = MoELayer.from_inputs(cfg, d)
    stream = torch.cuda.current_stream()

    def timed_steps(lay):
        """W warm-up steps, then K timed steps: (ms per step, per-call ms)."""
        for _ in range(args.warmup):
            lay.run()
        if lay.signalled:
            calls, names = [lay.route, lay.permute, lay.ffn_combine], ["route", "permute", "ffn_combine"]
        else:
            calls, names = [lay.route, lay.permute, lay.ffn, lay.combine], ["route", "permute", "grouped_ffn", "combine"]
        # One event at every call boundary (each record costs the stream a few microseconds, so the end of
        # one step and the start of the next share one): ev[s * n + i] opens call i of step s, ev[-1] closes
        # the last step.
        n = len(calls)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps * n + 1)]
        torch.cuda.synchronize()
        for s in range(args.steps):
            for i, c in enumerate(calls):
                ev[s * n + i].record(stream)
                c()
        ev[-1].record(stream)
        torch.cuda.synchronize()
        return (ev[0].elapsed_time(ev[-1]) / args.steps,
                {nm: sum(ev[s * n + i].elapsed_time(ev[s * n + i + 1]) for s in range(args.steps)) / args.steps
                 for i, nm in enumerate(names)})

    ms_step, per_call = timed_steps(layer)

    # algorithmic work of this batch
    R = int(layer.perm.expert_counts.sum().item())
    n_hit = int((layer.perm.expert_counts > 0).sum().item())
    inv = layer.perm.inv_perm
    T_hit = int((inv >= 0).any(dim=1).sum().item())
    flop = W.flops(cfg, R)
    tflops = flop / (ms_step * 1e-3) / 1e12
    ffn_tflops = flop / (per_call["grouped_ffn"] * 1e-3) / 1e12
    permute_bytes = T_hit * cfg.H * 2 + R * cfg.H * 2
    combine_bytes = R * cfg.H * 4 + cfg.T * cfg.H * 4

    result = {
        "metric": "MoE-layer TFLOP/s and tokens/s on 1 MI355X; % of bf16 MFMA peak",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "tokens": cfg.T, "hidden": cfg.H,
                   "ffn": cfg.F, "ffn_here": cfg.F_loc, "tp": cfg.tp, "experts": cfg.E,
                   "local_experts": cfg.n_local, "top_k": cfg.k,
                   "activation": cfg.act, "tile_m": layer.tile_m, "routed_rows": R},
        "tokens_per_s": round(cfg.T / (ms_step * 1e-3), 1),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "per_call_ms": {n: round(v, 5) for n, v in per_call.items()},
        "permute_GBps": round(permute_bytes / (per_call["permute"] * 1e-3) / 1e9, 1),
        "combine_GBps": round(combine_bytes / (per_call["combine"] * 1e-3) / 1e9, 1),
        "grouped_ffn_TFLOPs": round(ffn_tflops, 2),
        "roofline": dict(ffn_roofline(cfg, R, n_hit, per_call["grouped_ffn"]),
                         traffic=recorded_traffic(args.workload)),
        "cpu_baseline": None,
        "pages_context": PAGES_CONTEXT,
    }
    # The same steps with the permutation fused into layer0's operand load (index-only permute,
    # moe_grouped_ffn_gather), measured after the main line on its own layer buffers.
    gl = MoELayer.from_inputs(cfg, d, fused_gather=True)
    g_ms, g_calls = timed_steps(gl)
    result["fused_gather"] = {"ms_per_step": round(g_ms, 5), "value": round(flop / (g_ms * 1e-3) / 1e12, 3),
                              "per_call_ms": {n: round(v, 5) for n, v in g_calls.items()}}
    del gl
    # The grouped FFN and the combine as one launch with tile-level signals (moe_ffn_combine_fused,
    # 256-row tiles only), also after the main line on its own buffers.
    if layer.tile_m == 256:
        sl = MoELayer.from_inputs(cfg, d, signalled=True)
        s_ms, s_calls = timed_steps(sl)
        result["signalled"] = {"ms_per_step": round(s_ms, 5), "value": round(flop / (s_ms * 1e-3) / 1e12, 3),
                               "per_call_ms": {n: round(v, 5) for n, v in s_calls.items()}}
        del sl
    copy_gbps, cold = copy_and_cold(layer, stream)
    result["copy_GBps"] = round(copy_gbps, 1)
    result["permute_GBps_cold"] = round(permute_bytes / (cold["permute"] * 1e-3) / 1e9, 1)
    result["combine_GBps_cold"] = round(combine_bytes / (cold["combine"] * 1e-3) / 1e9, 1)
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
