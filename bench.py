"""Benchmark of one chunk step of latent-KV (MLA) chunk attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload wan480p] [--no-cpu-baseline]

A step is the whole hot path over one synthetic batch: cache append of the
current chunk (latent down-projection + rotated positional key), query
absorption, the fused latent attention over every cached chunk plus the
current one, and the merge + W_UV up-projection.  Inputs are resident in HBM
before the timed region.  Timing uses HIP events on the stream the library
launches on (torch's current stream): one pair around the K timed steps, with
nothing recorded between kernels; per-kernel durations come from a second pass
of K steps with events around each call.  The line names the library it
measured (path and sha256; an MLA_HIP_LIB override is refused) and the host
CPU the oracle baseline ran on.

Prints one JSON line.  `value` is algorithmic TFLOP/s of the step (absorbed
count: B*Nq*H*[Nk*(4 d_c + 2 d_r) + 4 d_h d_c] plus the append's
2*B*Nq*D*(d_c + d_r)).  `roofline` is for the dominant kernel (the fused
attention: 2(d_c+d_r) + 2 d_c flop per (row, key)); `cpu_baseline` is the
fp64 oracle timed on this host on a bounded sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA chunk-attention TFLOP/s + ms/chunk (480P, d_c=192); % bf16 MFMA peak"
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
HBM_PEAK_GBS = 8000.0
HBM_PEAK_BYTES_S = HBM_PEAK_GBS * 1e9
COPY_BYTES = 1 << 30           # calibration copy of the traffic probe
# sources of the attention kernel that runs at a given latent width
ATTEND_SOURCES = {
    "attend_bf16_kernel": ("latent_kv_cache_chunk_amd/csrc/attend.hip", "latent_kv_cache_chunk_amd/csrc/mla_common.h"),
    "attend_wide_bf16_kernel": ("latent_kv_cache_chunk_amd/csrc/attend_wide.hip",
                                "latent_kv_cache_chunk_amd/csrc/mla_common.h"),
}


def attend_kernel(d_c: int) -> str:
    """The attention kernel of latent width d_c (d_c = 256 runs the single-role kernel)."""
    return "attend_wide_bf16_kernel" if d_c > 192 else "attend_bf16_kernel"


def kernel_source_hash(d_c: int = 192) -> str:
    h = hashlib.sha256()
    for p in ATTEND_SOURCES[attend_kernel(d_c)]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, d_c: int):
    """HBM bytes per attend launch from committed rocprofv3 counters (written by
    latent_kv_cache_chunk_amd.profile_summary), if the kernel source is unchanged."""
    path = os.path.join(ROOT, "profiles", f"attend_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(d_c):
        return None
    return t.get("hbm_bytes_per_launch")


def host_cpu() -> dict:
    """CPU model, the cores this process may run on, and the BLAS thread count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = None
    return {"model": model, "cores": len(os.sched_getaffinity(0)), "blas_threads": blas}


def library_identity(path: str) -> dict:
    h = hashlib.sha256()
    with open(path, "rb") as f:
        for block in iter(lambda: f.read(1 << 20), b""):
            h.update(block)
    return {"path": os.path.relpath(path, ROOT), "sha256": h.hexdigest()}


def cpu_baseline(wl, inputs, n_heads: int) -> dict:
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload:
    every query row of the first `n_heads` heads of sample 0, against all keys."""
    import oracle
    host = host_cpu()
    threads = host["blas_threads"] or host["cores"]
    hh, ii = np.meshgrid(np.arange(min(n_heads, wl.n_heads)), np.arange(wl.n_q), indexing="ij")
    rows = np.stack([np.zeros(hh.size, np.int64), ii.ravel(), hh.ravel()], 1)   # batch 0
    args = [inputs[k].cpu().double().numpy() for k in ("q", "q_r")]
    q_pos = inputs["q_pos"].cpu().numpy()
    w_uk = inputs["w_uk"].cpu().double().numpy()
    w_uv = inputs["w_uv"].cpu().double().numpy()
    cache = inputs["cache"][:, :wl.n_k].cpu().double().numpy()
    chunks = {}
    kv = np.full(len(rows), wl.n_k, np.int64)
    if wl.causal:
        q_start, c = wl.causal
        chunks = dict(q_chunk=(q_start + np.arange(wl.n_q)) // c, k_chunk=np.arange(wl.n_k) // c)
        kv = np.minimum(wl.n_k, ((q_start + rows[:, 1]) // c + 1) * c)
    t0 = time.perf_counter()
    oracle.chunk_attend_rows(rows, args[0], args[1], q_pos, w_uk, w_uv, cache, wl.n_k, wl.scale,
                             split=wl.rope_split, theta=wl.theta, **chunks)
    dt = time.perf_counter() - t0
    flops = float(kv.sum()) * (4 * wl.d_c + 2 * wl.d_r) + len(rows) * 4 * wl.head_dim * wl.d_c
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": host["model"], "cores_available": host["cores"], "blas_threads": host["blas_threads"],
            "sample": f"{len(rows)} rows (all {wl.n_q} queries of heads 0..{min(n_heads, wl.n_heads) - 1}, "
                      f"batch 0) against their visible keys (of {wl.n_k}), fp64 "
                      f"non-absorbed numpy oracle incl. per-head K/V reconstruction; {dt:.1f} s wall; "
                      f"rate = absorbed algorithmic flops of the sample / wall time"}


def _time_calls(fn, steps: int, warmup: int) -> float:
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def compare(wl, dims, t, latent_ms: float, seed: int, dev, steps: int = 20, warmup: int = 3) -> dict:
    """The same chunk step's attention over a dense per-head K/V cache (the
    layout the latent replaces: 2*H*d_h values per token) and in the
    non-absorbed latent form (per-head K_h, V_h materialised from the latent,
    then standard attention), against the absorbed path's absorb + attend +
    up-projection time measured above.  Cache appends are excluded from all three."""
    import torch
    from latent_kv_cache_chunk_amd import mla, synth
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in synth.mha_inputs(wl, seed=seed).items()}
    out = torch.empty((wl.batch, wl.n_q, wl.n_heads, wl.head_dim), dtype=torch.bfloat16, device=dev)
    ws_d = torch.empty(mla.mha_workspace_bytes(wl.batch, wl.n_heads, wl.head_dim, wl.n_q, wl.n_k),
                       dtype=torch.uint8, device=dev)
    dense_ms = _time_calls(lambda: mla.mha_attend(d["q"], d["k"], d["v"], wl.n_k, d["scale"], out=out,
                                                  workspace=ws_d), steps, warmup)
    del d, ws_d
    ws_e = torch.empty(mla.expanded_workspace_bytes(dims, wl.n_q, wl.n_k), dtype=torch.uint8, device=dev)
    exp_ms = _time_calls(lambda: mla.chunk_attend_expanded(dims, t["q"], t["q_r"], t["q_pos"], t["w_uk"], t["w_uv"],
                                                           t["cache"], wl.n_k, wl.scale, out=out, workspace=ws_e),
                         steps, warmup)
    del ws_e
    lat_bytes = mla.cache_bytes(dims, torch.bfloat16, wl.n_k)
    dense_bytes = mla.dense_kv_bytes(dims, torch.bfloat16, wl.n_k)
    return {
        "latent_absorbed_ms": round(latent_ms, 4),
        "dense_mha_ms": round(dense_ms, 4),
        "latent_expanded_ms": round(exp_ms, 4),
        "dense_over_latent_time": round(dense_ms / latent_ms, 3),
        "expanded_over_absorbed_time": round(exp_ms / latent_ms, 3),
        "cache_bytes": {"latent": lat_bytes, "dense_kv": dense_bytes, "ratio": round(dense_bytes / lat_bytes, 2)},
        "flop_per_row_key": {"absorbed": 4 * wl.d_c + 2 * wl.d_r, "expanded": 4 * wl.head_dim + 2 * wl.d_r,
                             "dense": 4 * wl.head_dim},
        "steps": steps,
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan480p")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=12, help="heads whose rows form the oracle sample")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the dense per-head K/V and non-absorbed comparison timings")
    ap.add_argument("--cold", action="store_true",
                    help="flush L2 and the last-level cache with a 512 MB write before every timed step; "
                         "ms_per_step is then the sum of the step's kernel times")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from one captured HIP graph (graph_ms_per_step)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="for rocprofv3 --pmc runs: a plain copy of known size, then a few steps; no timing")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "only one GPU is measured: run with --gpus 1 "
                                   "(the path would shard by batch or query rows over a replicated latent cache)", "n_gpus": args.gpus}))
        return 2

    if os.environ.get("MLA_HIP_LIB"):
        print(json.dumps({"error": "MLA_HIP_LIB is set: the benchmark measures only the in-tree "
                                   "latent_kv_cache_chunk_amd/libmla_hip.so"}))
        return 2
    import torch
    from latent_kv_cache_chunk_amd import mla, synth

    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    dims = mla.Dims(batch=wl.batch, n_heads=wl.n_heads, head_dim=wl.head_dim, d_c=wl.d_c, d_r=wl.d_r,
                    rope=wl.rope_split, rope_theta=wl.theta)
    att = synth.attend_inputs(wl, seed=args.seed)
    app = synth.append_inputs(wl, seed=args.seed)
    t = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in att.items()}
    a = {k: v.to(dev) for k, v in app.items()}
    cache = t["cache"]
    ws = mla.alloc_workspace(dims, torch.bfloat16, wl.n_q, wl.n_k, dev)
    out = torch.empty((wl.batch, wl.n_q, wl.n_heads, wl.head_dim), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        mla.cache_append(dims, a["x"], a["w_dkv"], a["w_kr"], a["pos"], cache, wl.n_cached)
        if ev is not None:
            ev[1].record()
        mla.query_absorb(dims, t["q"], t["q_r"], t["q_pos"], t["w_uk"], wl.scale, wl.n_k, ws)
        if ev is not None:
            ev[2].record()
        mla.latent_attend(dims, cache, wl.n_q, wl.n_k, ws, causal=wl.causal)
        if ev is not None:
            ev[3].record()
        mla.value_upproj(dims, t["w_uv"], out, wl.n_q, wl.n_k, ws)
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.traffic_probe:
        # Calibration for the HBM byte counters: an elementwise kernel (negation)
        # over COPY_BYTES reads and writes exactly that many bytes once each.
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "copy_bytes": COPY_BYTES, "steps": 3, "workload": wl.name}))
        return 0
    # The timed region holds the K steps and nothing else: an event recorded
    # between two kernels adds a few microseconds of its own, so the per-kernel
    # breakdown comes from a second pass of K steps with events around each call.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None
    if flush is None:
        torch.cuda.synchronize()
        start.record()
        for i in range(args.steps):
            step()
        stop.record()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)   # evicts the latent cache and q from L2 and the 256 MB last-level cache
        step(evs[i])
    torch.cuda.synchronize()
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evs])   # [steps, 4]
    ms_step = start.elapsed_time(stop) / args.steps if flush is None else float(np.mean(per.sum(axis=1)))
    append_ms, absorb_ms, attend_ms, upproj_ms = (float(np.mean(per[:, j])) for j in range(4))
    attend_ms_median = float(np.median(per[:, 2]))

    graph_ms = None
    if args.graph:
        # the same step captured once; launch-bound small steps pay one graph launch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / args.steps

    step_flops = wl.attend_flops() + wl.append_flops()
    core_flops = wl.attend_core_flops()
    value = step_flops / (ms_step * 1e-3) / 1e12
    attend_tflops = core_flops / (attend_ms * 1e-3) / 1e12
    traffic = load_traffic(wl.name, wl.d_c)
    minb = wl.min_hbm_bytes()

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs of the workload's shape)",
        "config": {"workload": wl.name, "batch": wl.batch, "n_q": wl.n_q, "n_k": wl.n_k,
                   "heads": wl.n_heads, "head_dim": wl.head_dim, "d_c": wl.d_c, "d_r": wl.d_r,
                   "rope_split": list(wl.rope_split), "d_model": wl.d_model,
                   "chunk_tokens": wl.chunk_tokens or wl.n_q},
        "frac_bf16_peak": round(value / BF16_PEAK_TFLOPS, 4),
        "breakdown_ms": {"append": round(append_ms, 4), "absorb": round(absorb_ms, 4),
                         "attend": round(attend_ms, 4), "attend_median": round(attend_ms_median, 4),
                         "upproj_merge": round(upproj_ms, 4)},
        "mha_equiv_tflops": round(wl.mha_equiv_flops() / (ms_step * 1e-3) / 1e12, 2),
        "cache_state": "cold (512 MB flush before every step)" if args.cold else "hot",
        "graph_ms_per_step": round(graph_ms, 4) if graph_ms is not None else None,
        "min_hbm": {"step_bytes": sum(minb.values()),
                    "step_gb_s": round(sum(minb.values()) / (ms_step * 1e-3) / 1e9, 1),
                    "step_frac_of_8tb_s": round(sum(minb.values()) / (ms_step * 1e-3) / HBM_PEAK_BYTES_S, 4),
                    "append_bytes": minb["append"],
                    "append_gb_s": round(minb["append"] / (append_ms * 1e-3) / 1e9, 1)},
        "roofline": {"kernel": attend_kernel(wl.d_c), "bound": "mfma",
                     "achieved": round(attend_tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attend_tflops / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "traffic_gb_s": round(traffic / (attend_ms * 1e-3) / 1e9, 1) if traffic else None,
                     "traffic_frac_of_8tb_s": round(traffic / (attend_ms * 1e-3) / HBM_PEAK_BYTES_S, 4)
                     if traffic else None,
                     "flop_per_launch": core_flops,
                     "per_unit": f"{4 * wl.d_c + 2 * wl.d_r} flop per visible (row, key); "
                                 f"{wl.batch * wl.n_heads * wl.visible_keys()} visible pairs per launch "
                                 f"({wl.batch * wl.n_q * wl.n_heads} rows, {wl.n_k} keys)"},
        "cpu_baseline": None,
        "library": library_identity(mla.LIB_PATH),
        # The pages' only speed figures: whole-pipeline generation rates on another GPU, for context.
        # They time a full model, not this step, so vs_baseline stays null.
        "context": {"pages_generation_fps": {"latent_cache": 23.96, "per_head_cache_baseline": 18.06},
                    "pages_speedup_claim": 1.23,
                    "setting": "batch 1, whole autoregressive video generation pipeline, one NVIDIA B200; "
                               "not comparable to this kernel-level step"},
    }
    if not args.no_compare and not wl.causal:
        res["comparison"] = compare(wl, dims, t, absorb_ms + attend_ms + upproj_ms, args.seed, dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, att, args.cpu_heads)
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
