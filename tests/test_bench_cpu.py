"""Host-side checks of bench.py: the one-GPU guard and the CPU-baseline leg
(the oracle timed on a bounded sample) for every bench mode."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from draft_verification_02_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_for_every_mode():
    w = wl.make(3, 4, 500, target_dtype=wl.BF16, draft_dtype=wl.F32, temperature=0.7, top_p=0.9, seed=5, vseed=6)
    base = bench.cpu_baseline(w, 2)
    assert base["kind"] == "oracle" and base["cores"] == 1 and base["value"] > 0
    assert base["unit"] == "verified draft positions/s" and "2 of 3" in base["sample"]
    ptoks = np.argmax(wl.as_f32(w.draft), axis=2).astype(np.int32)
    assert bench.cpu_baseline(w, 3, point_tokens=ptoks)["value"] > 0
    lens = np.array([0, 4, 2], np.int32)
    assert bench.cpu_baseline(w, 3, lens=lens)["value"] > 0
    t = wl.make_tree(2, [3, 2], 500, temperature=0.7, top_p=0.9, seed=7, vseed=8)
    tb = bench.cpu_baseline(t, 2, tree=True)
    assert tb["unit"] == "verified tree nodes/s" and tb["value"] > 0


def test_all_cores_leg_and_parity_summary():
    """The all-cores timing runs the same oracle jobs; the parity summary of
    the oracle's own outputs against themselves has no mismatch, and counts
    one draw plus the accept tests evaluated per sequence."""
    w = wl.make(4, 3, 700, target_dtype=wl.F32, draft_dtype=wl.F32, temperature=0.8, top_p=0.9, seed=9, vseed=10)
    outs = {}
    base = bench.cpu_baseline(w, 4, outputs=outs)
    assert base["all_cores"]["cores"] >= 1 and base["all_cores"]["value"] > 0 and base["cpu_model"]
    g_tok = np.stack([outs[b]["tokens"][0] for b in range(4)])
    g_num = np.array([outs[b]["num_accepted"][0] for b in range(4)])
    s = bench.parity_summary(w, g_tok, g_num, outs)
    assert s["token_mismatches"] == 0 and s["sequences_checked"] == 4
    assert s["decisions"] == int(sum(min(n + 1, 3) + 1 for n in g_num))
    g_tok2 = g_tok.copy()
    g_tok2[1, 0] = (g_tok2[1, 0] + 1) % 700
    assert bench.parity_summary(w, g_tok2, g_num, outs)["token_mismatches"] == 1
    tau, rates = bench.acceptance(np.array([0, 3, 1, 3]), 3)
    assert tau == 2.75 and rates == [0.75, round(2 / 3, 4), 1.0]
