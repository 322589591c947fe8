"""Benchmark: batched speculative-decoding verification on one MI355X.

One step = one spec_verify call over the whole batch of the concurrent-batch
workload (B=32 sequences, K=7 drafted positions, V=151936, bf16 target / f32
draft logits, temperature 0.7, top-p 0.9), inputs resident in HBM.  Several
copies of the inputs are rotated so that the 256 MB Infinity Cache cannot
serve a step from the previous one.

Prints one JSON line with the headline metric (verified draft positions/s),
the roofline of the dominant (streaming) kernel measured with HIP events on
the call's stream, and the CPU oracle timed on the host as a baseline.

--mode point measures spec_verify_point instead: the same target rows, with
the drafts given as point masses (each draft row's argmax, the proposals of a
greedy draft head) and no draft logits read.

--mode ragged measures spec_verify_ragged with per-sequence draft lengths
drawn uniformly from 0..K (seeded) and the per-position acceptance counters
on; the bytes counted are those of the rows inside each sequence's length.

--mode hidden measures spec_verify_greedy_hidden: greedy verification of the
same batch shape straight from the target's hidden states (H = 4096, random
bf16 unembedding matrix of 151936 x 4096), the unembedding product fused with
the argmax on the matrix cores.

--mode tree measures spec_verify_tree: the same target-row distributions and
processing over a static 44-node token tree per sequence (4 children of the
root, then 2, 2 and 1 per node), 45 target rows per sequence, the children's
tokens the top candidates of a proposer's noisy copy of the parent row.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified draft positions/sec + HBM GB/s (% peak) at B=32 K=7 V=151936, 1 GPU"
METRIC_RAGGED = ("verified draft positions/sec + HBM GB/s (% peak) at B=32 K<=7 V=151936, 1 GPU, "
                 "per-sequence draft lengths U{0..7} (spec_verify_ragged)")
METRIC_POINT = ("verified draft positions/sec + HBM GB/s (% peak) at B=32 K=7 V=151936, 1 GPU, "
                "point-mass drafts (spec_verify_point)")
METRIC_TREE = ("verified tree nodes/sec + HBM GB/s (% peak) at B=32 N=44 V=151936, 1 GPU, "
               "token trees 4-2-2-1 (spec_verify_tree)")
TREE_BRANCHING = [4, 2, 2, 1]
METRIC_HIDDEN = ("verified draft positions/sec + HBM GB/s (% peak) at B=32 K=7 V=151936 H=4096, 1 GPU, "
                 "greedy from hidden states, unembedding fused (spec_verify_greedy_hidden)")
HIDDEN_H = 4096
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20


def _hip():
    for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
        try:
            L = ctypes.CDLL(name)
            break
        except OSError:
            continue
    else:
        raise RuntimeError("libamdhip64.so not found")
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return L


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "draft_verification_02_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".h", ".hip")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(config_name: str, src_hash: str):
    """HBM bytes per launch from the committed PMC summary, only while the
    kernel sources still match the ones the counters were taken on."""
    path = os.path.join(ROOT, "profiles", "k_row_c3_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != src_hash or d.get("workload") != config_name:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, max_seqs: int, point_tokens=None, lens=None, tree=False):
    import oracle  # CPU baseline leg only

    seqs = list(range(min(w.B, max_seqs)))
    t0 = time.perf_counter()
    if tree:
        par = w.meta["parents"]
        for b in seqs:
            oracle.verify_tree(w.target[b:b + 1], w.tokens[b:b + 1], par[b:b + 1],
                               float(np.float32(w.temperature)), w.top_k, float(np.float32(w.top_p)),
                               w.seed, seq_base=b, diagnostics=False)
        dt = time.perf_counter() - t0
        return {"value": round(len(seqs) * w.K / dt, 3), "unit": "verified tree nodes/s",
                "cores": 1, "kind": "oracle",
                "sample": f"{len(seqs)} of {w.B} sequences of the same workload, single-threaded "
                          f"fp64 C++ oracle, {dt:.2f} s"}
    if lens is not None:
        sub = slice(0, len(seqs))
        oracle.verify_ragged(w.target[sub], w.draft[sub], w.tokens[sub], lens[sub],
                             float(np.float32(w.temperature)), w.top_k, float(np.float32(w.top_p)),
                             w.seed)
        dt = time.perf_counter() - t0
        return {"value": round(int(lens[sub].sum()) / dt, 3), "unit": "verified draft positions/s",
                "cores": 1, "kind": "oracle",
                "sample": f"{len(seqs)} of {w.B} sequences of the same workload, single-threaded "
                          f"fp64 C++ oracle, {dt:.2f} s"}
    for b in seqs:
        if point_tokens is not None:
            oracle.verify_point(w.target[b:b + 1], point_tokens[b:b + 1],
                                float(np.float32(w.temperature)), w.top_k,
                                float(np.float32(w.top_p)), w.seed, seq_base=b, diagnostics=False)
            continue
        oracle.verify(w.target[b:b + 1], w.draft[b:b + 1], w.tokens[b:b + 1],
                      float(np.float32(w.temperature)), w.top_k, float(np.float32(w.top_p)),
                      w.seed, seq_base=b, diagnostics=False)
    dt = time.perf_counter() - t0
    return {"value": round(len(seqs) * w.K / dt, 3), "unit": "verified draft positions/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{len(seqs)} of {w.B} sequences of the same workload, single-threaded "
                      f"fp64 C++ oracle, {dt:.2f} s"}


def _timed_steps(torch, step, steps, warmup, settle_s=0.04):
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    settle = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        step(settle)
        settle += 1
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, settle


def _kernel_ms(torch, binding, step, n):
    hip = _hip()
    evs = []
    for _ in range(2 * n):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        evs.append(h)
    torch.cuda.synchronize()
    for i in range(n):
        binding.profile_events(evs[2 * i].value, evs[2 * i + 1].value)
        step(i)
    torch.cuda.synchronize()
    durs = []
    for i in range(n):
        f = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(f), evs[2 * i], evs[2 * i + 1]) == 0
        durs.append(f.value)
    for h in evs:
        hip.hipEventDestroy(h)
    return float(np.mean(durs))


def bench_hidden(args, torch, binding, wl):
    """Greedy verification from hidden states at the concurrent-batch shape."""
    spec = wl.CONFIG_SPECS[3]
    B, K, V, H = spec["B"], spec["K"], spec["V"], HIDDEN_H
    hidden, w = wl.make_hidden(B, K, V, H, seed=wl.gen_seed(3))
    tokens = np.random.default_rng(wl.verify_seed(3) & 0xFFFFFFFF).integers(0, V, (B, K)).astype(np.int32)
    dev = torch.device("cuda:0")

    def up16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    h_t, w_t, k_t = up16(hidden), up16(w), torch.from_numpy(tokens).to(dev)
    out_t = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((B,), dtype=torch.int32, device=dev)

    def step(i):
        binding.spec_verify_greedy_hidden(h_t, w_t, k_t, out_t, out_n)

    ms, settle = _timed_steps(torch, step, args.steps, args.warmup)
    k_ms = _kernel_ms(torch, binding, step, args.steps)
    R = B * (K + 1)
    ideal = w.nbytes + hidden.nbytes
    flops = 2.0 * R * V * H
    achieved = ideal / (k_ms * 1e-3) / 1e9
    tflops = flops / (k_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC_HIDDEN,
        "value": round(B * K / (ms * 1e-3), 1),
        "unit": "verified draft positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_steps": settle,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 x bf16 -> f32",
        "data": "synthetic (random bf16 hidden states and unembedding matrix)",
        "config": {"workload": f"c3 shape greedy from hidden states B{B} K{K} V{V} H{H}", "B": B, "K": K, "V": V,
                   "H": H, "ideal_bytes": ideal, "flops": flops},
        "roofline": {"bound": "hbm", "kernel": "k_lmhead_argmax", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": None, "kernel_ms": round(k_ms, 5), "kernel_source_hash": kernel_source_hash(),
                     "mfma_tflops": round(tflops, 1), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4)},
    }
    if not args.no_cpu_baseline:
        import oracle  # CPU baseline leg only
        from threadpoolctl import threadpool_limits
        t0 = time.perf_counter()
        with threadpool_limits(limits=1):
            L = oracle.lm_head_logits(hidden[0], w).reshape(1, K + 1, V)
            oracle.verify_greedy_logits64(L, tokens[:1])
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(K / dt, 3), "unit": "verified draft positions/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"1 of {B} sequences ({K + 1} rows), float64 product on one thread, "
                                          f"{dt:.2f} s"}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-settle", dest="settle", action="store_false",
                    help="skip the untimed settle phase after the warmup steps")
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--mode", choices=["general", "point", "ragged", "tree", "hidden"], default="general",
                    help="general: spec_verify with draft logits (the headline); point: "
                         "spec_verify_point with point-mass drafts")
    ap.add_argument("--sets", type=int, default=0, help="input copies rotated (0: auto)")
    ap.add_argument("--cpu-seqs", type=int, default=0, help="sequences of the CPU baseline (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device copy of this many bytes (3 times), for "
                         "calibrating HBM traffic counters, then exit")
    args = ap.parse_args()

    if args.copy_probe:
        import torch
        src = torch.empty(args.copy_probe, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the verifier is data-parallel over sequences and "
              "this build runs on a single MI355X; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from draft_verification_02_amd import binding, workloads as wl

    if args.mode == "hidden":
        return bench_hidden(args, torch, binding, wl)
    point = args.mode == "point"
    ragged = args.mode == "ragged"
    tree = args.mode == "tree"
    if tree:
        spec = dict(wl.CONFIG_SPECS[args.config])
        w = wl.make_tree(spec["B"], TREE_BRANCHING, spec["V"], target_dtype=spec["target_dtype"],
                         temperature=spec["temperature"], top_k=spec.get("top_k", 0),
                         top_p=spec.get("top_p", 1.0), sigma=spec["sigma"], rho=spec["rho"],
                         n_boost=spec["n_boost"], seed=wl.gen_seed(args.config),
                         vseed=wl.verify_seed(args.config),
                         name=spec["name"].split(" ")[0] + f" tree B{spec['B']} N44 4-2-2-1")
    else:
        w = wl.config(args.config)
    if w.greedy:
        raise SystemExit("the headline workload is a sampling workload")
    dev = torch.device("cuda:0")
    # point-mass drafts: the draft rows' argmax, a greedy draft head's proposals
    ptoks = np.argmax(wl.as_f32(w.draft), axis=2).astype(np.int32) if point else None
    ideal = w.target.nbytes if (point or tree) else w.ideal_bytes()
    lens_np = None
    if ragged:
        lens_np = np.random.default_rng(w.seed & 0xFFFFFFFF).integers(0, w.K + 1, w.B).astype(np.int32)
        row_t = w.target[0, 0].nbytes
        row_d = w.draft[0, 0].nbytes
        ideal = int(((lens_np + 1) * row_t + lens_np * row_d).sum())
    n_sets = args.sets or max(4, int(np.ceil(2.5 * MALL_BYTES / ideal)))

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    sets = [(up(w.target), None if (point or tree) else up(w.draft), up(ptoks if point else w.tokens))
            for _ in range(n_sets)]
    par_t = up(np.ascontiguousarray(w.meta["parents"])) if tree else None
    out_p = torch.empty((w.B, w.K), dtype=torch.int32, device=dev) if tree else None
    lens_t = up(lens_np) if ragged else None
    out_t = torch.empty((w.B, w.K + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((w.B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        t, d, k = sets[i % n_sets]
        if tree:
            binding.spec_verify_tree(t, k, par_t, w.temperature, w.top_k, w.top_p, w.seed, stream=stream,
                                     out_tokens=out_t, out_num_accepted=out_n, out_path=out_p)
            return
        if point:
            binding.spec_verify_point(t, k, w.temperature, w.top_k, w.top_p, w.seed, out_t, out_n,
                                      stream=stream)
            return
        if ragged:
            binding.spec_verify_ragged(t, d, k, lens_t, w.temperature, w.top_k, w.top_p, w.seed,
                                       counters=True, out_tokens=out_t, out_num_accepted=out_n,
                                       stream=stream)
            return
        binding.spec_verify(t, d, k, w.temperature, w.top_k, w.top_p, w.seed, out_t, out_n,
                            stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Settle: the GPU takes about 20 ms of sustained work to reach its steady
    # clocks (measured: the first few hundred steps run up to 15% slower).
    # Untimed steps continue for 40 ms after the warmup steps; their count is
    # reported as settle_steps.
    settle = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < 0.04 and args.settle:
        for _ in range(20):
            step(args.warmup + settle)
            settle += 1
        torch.cuda.synchronize()

    # headline: K back-to-back steps between two events on the call stream
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    t_wall = time.perf_counter()
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps

    # dominant kernel: the library records a HIP event pair around its
    # streaming kernel, once per step, on the same stream
    hip = _hip()
    n_ev = args.steps
    evs = []
    for _ in range(2 * n_ev):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        evs.append(h)
    torch.cuda.synchronize()
    for i in range(n_ev):
        binding.profile_events(evs[2 * i].value, evs[2 * i + 1].value)
        step(i)
    torch.cuda.synchronize()
    durs = []
    for i in range(n_ev):
        f = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(f), evs[2 * i], evs[2 * i + 1]) == 0
        durs.append(f.value)
    for h in evs:
        hip.hipEventDestroy(h)
    k_ms = float(np.mean(durs))

    src_hash = kernel_source_hash()
    achieved = ideal / (k_ms * 1e-3) / 1e9
    traffic = None if (point or ragged or tree) else traffic_from_profiles(w.name, src_hash)
    positions = int(lens_np.sum()) if ragged else w.B * w.K
    value = positions / (ms * 1e-3)
    metric = METRIC_TREE if tree else (METRIC_POINT if point else (METRIC_RAGGED if ragged else METRIC))
    if args.config != 3:  # the metric strings above name the concurrent-batch workload
        metric = (f"verified {'tree nodes' if tree else 'draft positions'}/sec + HBM GB/s (% peak) at "
                  f"{w.name}, 1 GPU" + (f", {args.mode} mode" if args.mode != "general" else ""))
    line = {
        "metric": metric,
        "value": round(value, 1),
        "unit": "verified tree nodes/s" if tree else "verified draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+f64",
        "data": "synthetic",
        "config": {"workload": w.name + ("-point" if point else ("-ragged" if ragged else "")),
                   "B": w.B, ("N" if tree else "K"): w.K, "V": w.V,
                   "target": "bf16", "draft": "point mass" if (point or tree) else "f32",
                   "temperature": w.temperature, "top_k": w.top_k,
                   "top_p": w.top_p, "input_sets_rotated": n_sets, "ideal_bytes": ideal},
        "hbm_gbs_step": round(ideal / (ms * 1e-3) / 1e9, 1),
        "pct_peak_step": round(100 * ideal / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "roofline": {"bound": "hbm", "kernel": "k_row", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel_ms": round(k_ms, 5),
                     "kernel_source_hash": src_hash},
        "wall_s_timed": round(t_wall, 4),
    }
    if ragged:
        line["config"]["draft_lens_total"] = positions
    if tree:
        line["config"]["branching"] = TREE_BRANCHING
        line["mean_accepted_path"] = round(float(out_n.float().mean().item()), 3)
    if not args.no_cpu_baseline:
        cpu_seqs = args.cpu_seqs or (8 if tree else 32)
        line["cpu_baseline"] = cpu_baseline(w, cpu_seqs, ptoks, lens_np, tree)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
