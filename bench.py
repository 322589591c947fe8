"""Benchmark: batched speculative-decoding verification on one MI355X.

One step = one verification call over the whole batch of a workload, inputs
resident in HBM.  The default is the concurrent-batch workload (B=32
sequences, K=7 drafted positions, V=151936, bf16 target / f32 draft logits,
temperature 0.7, top-p 0.9) through spec_verify.  Several copies of the
inputs are rotated so that the 256 MB Infinity Cache cannot serve a step from
the previous one.

Prints one JSON line: the headline metric (verified draft positions/s) over
exactly --steps back-to-back steps between two events; the median and p10 /
p90 of the step and of the dominant kernel over at least 100 calls; the
roofline of the dominant kernel (its algorithmic bytes over its average
duration, taken with HIP events attached to its dispatch on the call's
stream); the acceptance telemetry of the batch (tau = mean accepted + 1, the
acceptance rate at each position); and the CPU oracle timed on the host, on
one core and on all the cores the process may use, with its parity summary
against the GPU's outputs (decisions, ambiguous decisions, token mismatches).

--config N picks workload N (1..5; 4 is greedy verification).
--mode point: spec_verify_point, the drafts given as point masses (each draft
row's argmax, a greedy draft head's proposals), no draft logits read.
--mode ragged: spec_verify_ragged with per-sequence draft lengths U{0..K}
(seeded) and the per-position acceptance counters on; the bytes counted are
those of the rows inside each sequence's length.
--mode tree: spec_verify_tree over a static 44-node token tree per sequence
(4 children of the root, then 2, 2 and 1 per node), 45 target rows per
sequence, the children's tokens the top candidates of a proposer's noisy copy
of the parent row.
--mode hidden: spec_verify_greedy_hidden, greedy verification of the same
batch shape straight from the target's hidden states (H = 4096, random bf16
unembedding matrix of 151936 x 4096), the unembedding product fused with the
argmax on the matrix cores.
--mode hidden-sample: spec_verify_hidden, sampling verification of the same
batch shape (T 0.7, top-p 0.9) from target and draft hidden states with the
shared unembedding matrix: the bf16 logits of all 480 rows in one pass over
the matrix, then the verification of spec_verify on them.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

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
METRIC_HIDDEN_SAMPLE = ("verified draft positions/sec + HBM GB/s (% peak) at B=32 K=7 V=151936 H=4096, 1 GPU, "
                        "T 0.7 top-p 0.9 from target and draft hidden states, shared unembedding "
                        "(spec_verify_hidden)")
HIDDEN_H = 4096
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20
DIST_CALLS = 100          # calls behind the medians and percentiles (at least)
MAX_CPU_THREADS = 16      # the host cores one GPU's share of the box holds
ACCEPT_BAND, NUCLEUS_BAND, SAMPLE_BAND = 1e-5, 1e-6, 1e-12


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


def traffic_from_profiles(config_name: str, src_hash: str, kernel: str):
    """HBM bytes per launch from a committed PMC summary of this kernel and
    workload, only while the kernel sources still match the ones the
    counters were taken on."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    for f in sorted(os.listdir(pdir)):
        if not f.endswith("_traffic.json"):
            continue
        with open(os.path.join(pdir, f)) as fh:
            d = json.load(fh)
        if (d.get("kernel_source_hash") == src_hash and d.get("workload") == config_name
                and d.get("kernel", kernel) == kernel):
            return d.get("hbm_bytes_per_launch")
    return None


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
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(MAX_CPU_THREADS, n))


def _oracle_job(w, b, point_tokens=None, lens=None, tree=False, greedy=False):
    """The oracle on sequence b alone (its own global index in the random
    stream), with its diagnostics."""
    import oracle  # CPU baseline leg only
    T, tk, tp = float(np.float32(w.temperature)), w.top_k, float(np.float32(w.top_p))
    sl = slice(b, b + 1)
    if greedy:
        return lambda: oracle.verify_greedy(w.target[sl], w.tokens[sl])
    if tree:
        par = w.meta["parents"]
        return lambda: oracle.verify_tree(w.target[sl], w.tokens[sl], par[sl], T, tk, tp, w.seed, seq_base=b)
    if point_tokens is not None:
        return lambda: oracle.verify_point(w.target[sl], point_tokens[sl], T, tk, tp, w.seed, seq_base=b)
    if lens is not None:
        kb = int(lens[b])

        def ragged():
            d = None if kb == 0 else np.ascontiguousarray(w.draft[sl, :kb])
            return oracle.verify(np.ascontiguousarray(w.target[sl, :kb + 1]), d,
                                 np.ascontiguousarray(w.tokens[sl, :kb]), T, tk, tp, w.seed, seq_base=b)
        return ragged
    return lambda: oracle.verify(w.target[sl], w.draft[sl], w.tokens[sl], T, tk, tp, w.seed, seq_base=b)


def cpu_baseline(w, max_seqs: int, point_tokens=None, lens=None, tree=False, greedy=False,
                 outputs: dict | None = None):
    """The oracle as it stands, timed on the host over a bounded sample of the
    workload's sequences: single-threaded, then the same jobs over all the
    cores the process may use (sequences are independent).  Fills
    ``outputs`` (sequence -> oracle result) when given."""
    seqs = list(range(min(w.B, max_seqs)))
    jobs = [_oracle_job(w, b, point_tokens, lens, tree, greedy) for b in seqs]
    t0 = time.perf_counter()
    res = [j() for j in jobs]
    dt1 = time.perf_counter() - t0
    n = cpu_threads()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as ex:  # the oracle releases the GIL in its C calls
        list(ex.map(lambda j: j(), jobs))
    dtn = time.perf_counter() - t0
    if outputs is not None:
        outputs.update(zip(seqs, res))
    if tree:
        units, unit = len(seqs) * w.K, "verified tree nodes/s"
    elif lens is not None:
        units, unit = int(np.asarray(lens)[:len(seqs)].sum()), "verified draft positions/s"
    else:
        units, unit = len(seqs) * w.K, "verified draft positions/s"
    return {"value": round(units / dt1, 3), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"{len(seqs)} of {w.B} sequences of the same workload, fp64 C++ oracle with "
                      f"diagnostics, {dt1:.2f} s on one core",
            "all_cores": {"value": round(units / dtn, 3), "cores": n, "seconds": round(dtn, 3)},
            "cpu_model": cpu_model()}


def parity_summary(w, g_tok, g_num, outs: dict, lens=None, tree=False, greedy=False):
    """GPU outputs against the oracle on the sequences it ran: decisions
    (accept tests evaluated + one draw per sequence; greedy: the compares
    made + the emitted token), the ambiguous ones by the oracle's margins (an
    accept test with |u q - p| <= 1e-5 q, a draw within 1e-12 S of a
    cumulative boundary, or either made on a row whose nucleus boundary lies
    within 1e-6 of top_p) and the sequences whose tokens differ."""
    dec = amb = bad = 0
    for b, r in outs.items():
        n_o = int(r["num_accepted"][0])
        o_tok = r["tokens"][0]
        bad += int(int(g_num[b]) != n_o or not np.array_equal(g_tok[b, :len(o_tok)], o_tok))
        if greedy or w.temperature == 0:
            kb = w.K if lens is None else int(lens[b])
            dec += n_o + (1 if n_o < kb else 0) + 1
            continue
        am = r["accept_margin"][0]
        ti = r["target_info"][0]
        near = lambda info: bool(info["nucleus_margin"] <= NUCLEUS_BAND)  # noqa: E731
        if tree:
            tested = np.flatnonzero(np.isfinite(am))
            dec += len(tested) + 1
            amb += int((am[tested] <= ACCEPT_BAND).sum())
            path = [c for c in r["path"][0].tolist() if c >= 0]
            stop_row = path[-1] + 1 if path else 0
            amb += int(r["sample_margin"][0] <= SAMPLE_BAND or near(ti[stop_row]))
            continue
        di = r["draft_info"][0] if "draft_info" in r else None
        kb = len(am)
        for k in range(min(n_o + 1, kb)):
            dec += 1
            amb += int(am[k] <= ACCEPT_BAND or near(ti[k]) or (di is not None and near(di[k])))
        dec += 1
        amb += int(r["sample_margin"][0] <= SAMPLE_BAND or near(ti[n_o])
                   or (di is not None and n_o < kb and near(di[n_o])))
    return {"sequences_checked": len(outs), "decisions": dec, "ambiguous_decisions": amb,
            "token_mismatches": bad}


def acceptance(num: np.ndarray, K: int, lens=None):
    """tau (mean tokens emitted per sequence: accepted + 1) and the acceptance
    rate at each position among the sequences whose test there ran."""
    num = np.asarray(num, dtype=np.int64)
    kb = np.full_like(num, K) if lens is None else np.minimum(np.maximum(np.asarray(lens), 0), K)
    rates = []
    for k in range(K):
        tested = int(((num >= k) & (k < kb)).sum())
        rates.append(round(int((num > k).sum()) / tested, 4) if tested else None)
    return round(float((num + 1).mean()), 4), rates


def _events(hip, n):
    evs = []
    for _ in range(n):
        h = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(h)) == 0
        evs.append(h)
    return evs


def kernel_durations(torch, binding, step, n):
    """Durations (ms) of the dominant kernel over n calls: the library
    attaches a HIP event pair to that kernel's dispatch on the call's stream."""
    hip = _hip()
    evs = _events(hip, 2 * n)
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
    return durs


def step_durations(torch, step, n, stream):
    """Durations (ms) of n back-to-back calls, an event between each two."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(n):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(n)]


def dist(xs):
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "mean": round(float(a.mean()), 5), "n": len(a)}


def timed_steps(torch, step, steps, warmup, stream, settle=True):
    """W untimed warmup steps, 40 ms more of untimed steps (the GPU takes
    about 20 ms of sustained work to reach its steady clocks; their count is
    reported as settle_steps), then exactly `steps` back-to-back steps
    between two events on the call stream."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    n_settle = 0
    t0 = time.perf_counter()
    while settle and time.perf_counter() - t0 < 0.04:
        for _ in range(20):
            step(warmup + n_settle)
            n_settle += 1
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    t_wall = time.perf_counter()
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, n_settle, time.perf_counter() - t_wall


def bench_hidden(args, torch, binding, wl, sample=False):
    """Verification from hidden states at the concurrent-batch shape: greedy
    (the argmax fused into the product), or sampling (T 0.7, top-p 0.9) with
    draft states rho * target + sqrt(1 - rho^2) N(0, 1), rho 0.9."""
    spec = wl.CONFIG_SPECS[3]
    B, K, V, H = spec["B"], spec["K"], spec["V"], HIDDEN_H
    T, top_p, rho = spec["temperature"], spec["top_p"], 0.9
    # sampling: weights N(0, 9 / H), so the logits spread as the concurrent
    # batch's rows do (sd 3) and the nucleus is a few hundred tokens
    hidden, w = wl.make_hidden(B, K, V, H, seed=wl.gen_seed(3), w_scale=3.0 / np.sqrt(H) if sample else None)
    rng = np.random.default_rng(wl.verify_seed(3) & 0xFFFFFFFF)
    tokens = rng.integers(0, V, (B, K)).astype(np.int32)
    draft = None
    if sample:
        t32 = wl.bf16_bits_to_f32(hidden)
        draft = wl.f32_to_bf16_bits((rho * t32[:, :K] + np.sqrt(1 - rho * rho) * rng.standard_normal((B, K, H)))
                                    .astype(np.float32))
    dev = torch.device("cuda:0")

    def up16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    h_t, w_t, k_t = up16(hidden), up16(w), torch.from_numpy(tokens).to(dev)
    d_t = up16(draft) if sample else None
    out_t = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    out_n = torch.empty((B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        if sample:
            binding.spec_verify_hidden(h_t, d_t, w_t, k_t, T, 0, top_p, wl.verify_seed(3), out_t, out_n)
        else:
            binding.spec_verify_greedy_hidden(h_t, w_t, k_t, out_t, out_n)

    ms, settle, t_wall = timed_steps(torch, step, args.steps, args.warmup, stream, args.settle)
    n_dist = max(DIST_CALLS, args.steps)
    k_durs = kernel_durations(torch, binding, step, n_dist)
    s_durs = step_durations(torch, step, n_dist, stream)
    k_ms = float(np.mean(k_durs))
    R = B * (K + 1) + (B * K if sample else 0)
    # the product reads the matrix and the states once; the sampling path
    # also writes the bf16 logits of its rows
    ideal = w.nbytes + hidden.nbytes + (draft.nbytes + R * V * 2 if sample else 0)
    flops = 2.0 * R * V * H
    achieved = ideal / (k_ms * 1e-3) / 1e9
    tflops = flops / (k_ms * 1e-3) / 1e12
    src_hash = kernel_source_hash()
    line = {
        "metric": METRIC_HIDDEN_SAMPLE if sample else METRIC_HIDDEN,
        "value": round(B * K / (ms * 1e-3), 1),
        "unit": "verified draft positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "settle_steps": settle,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 x bf16 -> f32",
        "data": "synthetic (random bf16 hidden states and unembedding matrix)",
        "config": {"workload": (f"c3 shape {'T0.7 top-p0.9' if sample else 'greedy'} from hidden states "
                                f"B{B} K{K} V{V} H{H}"), "B": B, "K": K, "V": V,
                   "H": H, "ideal_bytes": ideal, "flops": flops},
        "step_ms": dist(s_durs),
        "roofline": {"bound": "hbm", "kernel": "k_lmhead<store>" if sample else "k_lmhead<argmax>",
                     "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic_from_profiles(f"hidden{'-sample' if sample else ''} B32 K7 V151936 H4096",
                                                      src_hash, "k_lmhead"),
                     "kernel_ms": round(k_ms, 5), "kernel_ms_dist": dist(k_durs),
                     "kernel_source_hash": src_hash,
                     "mfma_tflops": round(tflops, 1), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4)},
        "wall_s_timed": round(t_wall, 4),
    }
    if not args.no_cpu_baseline:
        import oracle  # CPU baseline leg only
        from threadpoolctl import threadpool_limits

        def one(b):
            if sample:
                return oracle.verify_hidden(hidden[b:b + 1], draft[b:b + 1], w, tokens[b:b + 1],
                                            float(np.float32(T)), 0, float(np.float32(top_p)), wl.verify_seed(3),
                                            seq_base=b, diagnostics=False)
            L = oracle.lm_head_logits(hidden[b], w).reshape(1, K + 1, V)
            return oracle.verify_greedy_logits64(L, tokens[b:b + 1])

        t0 = time.perf_counter()
        with threadpool_limits(limits=1):
            one(0)
        dt = time.perf_counter() - t0
        n = cpu_threads()
        t0 = time.perf_counter()
        with threadpool_limits(limits=n):
            one(1)
        dtn = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(K / dt, 3), "unit": "verified draft positions/s", "cores": 1,
                                "kind": "oracle",
                                "sample": f"1 of {B} sequences ({(2 * K + 1) if sample else K + 1} rows), "
                                          f"float64 product and oracle on one thread, {dt:.2f} s",
                                "all_cores": {"value": round(K / dtn, 3), "cores": n, "seconds": round(dtn, 3)},
                                "cpu_model": cpu_model()}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description="Throughput of batched speculative-decoding verification on one "
                                             "GPU; prints one JSON line.")
    ap.add_argument("--gpus", type=int, default=1, help="GPUs (only 1 is supported)")
    ap.add_argument("--steps", type=int, default=200, help="timed steps (one call each)")
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before the settle phase")
    ap.add_argument("--no-settle", dest="settle", action="store_false",
                    help="skip the untimed settle phase after the warmup steps")
    ap.add_argument("--config", type=int, default=3,
                    help="workload 1..5: 1 tiny (B1 K4 V1000), 2 single stream (B1 K15 V151936), "
                         "3 concurrent batch (B32 K7 V151936, the headline), 4 greedy (B64 K15), "
                         "5 large batch (B256 K4 V262144)")
    ap.add_argument("--mode", choices=["general", "point", "ragged", "tree", "hidden", "hidden-sample"],
                    default="general",
                    help="general: spec_verify with draft logits (the headline); point: "
                         "spec_verify_point with point-mass drafts; ragged: spec_verify_ragged with "
                         "per-sequence draft lengths; tree: spec_verify_tree over 44-node token trees; "
                         "hidden: spec_verify_greedy_hidden; hidden-sample: spec_verify_hidden "
                         "(the hidden modes use the concurrent-batch shape)")
    ap.add_argument("--sets", type=int, default=0, help="input copies rotated (0: auto)")
    ap.add_argument("--cpu-seqs", type=int, default=0, help="sequences of the CPU baseline (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle's timing")
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

    if args.mode in ("hidden", "hidden-sample"):
        return bench_hidden(args, torch, binding, wl, sample=args.mode == "hidden-sample")
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
    greedy = w.greedy
    if greedy and args.mode != "general":
        raise SystemExit("greedy workloads run in the general mode only")
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

    sets = [(up(w.target), None if (point or tree or greedy) else up(w.draft), up(ptoks if point else w.tokens))
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

    # headline: exactly --steps back-to-back steps between two events
    ms, settle, t_wall = timed_steps(torch, step, args.steps, args.warmup, stream, args.settle)
    # distributions over at least DIST_CALLS calls: each step between events,
    # and the dominant kernel's own event pair
    n_dist = max(DIST_CALLS, args.steps)
    s_durs = step_durations(torch, step, n_dist, stream)
    k_durs = kernel_durations(torch, binding, step, n_dist)
    k_ms = float(np.mean(k_durs))
    # the outputs of one call on the first input set
    step(0)
    torch.cuda.synchronize()
    g_tok, g_num = out_t.cpu().numpy(), out_n.cpu().numpy()

    src_hash = kernel_source_hash()
    # greedy batches below 512 sequences run in one launch (argmax and prefix)
    kernel = ("k_greedy_rows" if w.B < 512 else "k_row_argmax") if greedy else "k_row"
    achieved = ideal / (k_ms * 1e-3) / 1e9
    workload = w.name + ("-point" if point else ("-ragged" if ragged else ""))
    traffic = traffic_from_profiles(workload, src_hash, kernel)
    positions = int(lens_np.sum()) if ragged else w.B * w.K
    value = positions / (ms * 1e-3)
    metric = METRIC_TREE if tree else (METRIC_POINT if point else (METRIC_RAGGED if ragged else METRIC))
    if args.config != 3:  # the metric strings above name the concurrent-batch workload
        metric = (f"verified {'tree nodes' if tree else 'draft positions'}/sec + HBM GB/s (% peak) at "
                  f"{w.name}, 1 GPU" + (f", {args.mode} mode" if args.mode != "general" else ""))
    tau, rates = acceptance(g_num, w.K, lens_np)
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
        "dtype": "f32+f64" if not greedy else ("bf16" if w.target.dtype == np.uint16 else "f32"),
        "data": "synthetic",
        "config": {"workload": workload,
                   "B": w.B, ("N" if tree else "K"): w.K, "V": w.V,
                   "target": "bf16" if w.target.dtype == np.uint16 else "f32",
                   "draft": ("none (greedy)" if greedy else "point mass" if (point or tree) else
                             ("bf16" if w.draft.dtype == np.uint16 else "f32")),
                   "temperature": w.temperature, "top_k": w.top_k,
                   "top_p": w.top_p, "input_sets_rotated": n_sets, "ideal_bytes": ideal},
        "hbm_gbs_step": round(ideal / (ms * 1e-3) / 1e9, 1),
        "pct_peak_step": round(100 * ideal / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "step_ms": dist(s_durs),
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel_ms": round(k_ms, 5), "kernel_ms_dist": dist(k_durs),
                     "kernel_source_hash": src_hash},
        "acceptance": {"tau": tau, "rate_by_position": rates,
                       "note": "one call's outputs on this batch (tau = mean accepted + 1)"},
        "wall_s_timed": round(t_wall, 4),
    }
    if ragged:
        line["config"]["draft_lens_total"] = positions
    if tree:
        line["config"]["branching"] = TREE_BRANCHING
        line["acceptance"] = {"tau": round(float(g_num.mean()) + 1.0, 4),
                              "note": "mean accepted path length + 1, one call's outputs"}
    if not args.no_cpu_baseline:
        cpu_seqs = args.cpu_seqs or (8 if tree else (64 if greedy else 32))
        outs = {}
        line["cpu_baseline"] = cpu_baseline(w, cpu_seqs, ptoks, lens_np, tree, greedy, outs)
        line["parity"] = parity_summary(w, g_tok, g_num, outs, lens_np, tree, greedy)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
