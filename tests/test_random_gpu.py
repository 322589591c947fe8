"""Seeded sweep of random small configurations on the GPU against the
oracle: vocabulary sizes from 1 to 20000 (tails that fill no tile), K from 0
to 12, batch sizes 1 to 12, every dtype pair, temperatures including greedy,
top-k and top-p on and off, Gaussian and Student-t logits, through the general, point-mass, ragged and tree
entry points.  Every sequence is checked.  The parameters of each case are
printed before it runs."""
import numpy as np
import pytest

from draft_verification_02_amd import workloads as wl

from parity import Report, check_point, check_ragged, check_sampling, check_greedy, check_tree

pytestmark = pytest.mark.gpu


def _case(i):
    r = np.random.default_rng(9000 + i)
    V = int(r.choice([1, 2, 7, 63, 64, 65, 1000, 4097, 8191, 8193, 12345, 20000]))
    K = int(r.integers(0, 13))
    B = int(r.integers(1, 13))
    tdt, ddt = int(r.integers(0, 2)), int(r.integers(0, 2))
    T = float(r.choice([0.0, 0.3, 0.7, 1.0, 1.5]))
    top_k = int(r.choice([0, 0, 1, 5, 50, 100]))
    top_p = float(r.choice([1.0, 1.0, 0.5, 0.9, 0.99]))
    sigma = float(r.choice([0.5, 2.0, 4.0]))
    return dict(V=V, K=K, B=B, tdt=tdt, ddt=ddt, T=T, top_k=top_k, top_p=top_p, sigma=sigma,
                rho=float(r.uniform(0.3, 0.99)), seed=int(r.integers(1, 1 << 30)),
                dist="t3" if i % 3 == 2 else "gauss")


@pytest.mark.parametrize("i", range(80))
def test_random_configuration(i):
    c = _case(i)
    print(f"[case] random {i}: {c}", flush=True)
    w = wl.make(c["B"], c["K"], c["V"], target_dtype=c["tdt"], draft_dtype=c["ddt"], temperature=c["T"],
                top_k=c["top_k"], top_p=c["top_p"], sigma=c["sigma"], rho=c["rho"], seed=c["seed"],
                vseed=c["seed"] + 1, dist=c["dist"])
    rep = Report()
    if c["T"] == 0.0:
        check_greedy(w)
    else:
        check_sampling(w, report=rep, check_stats=(i % 2 == 0))
    toks = np.where(np.random.default_rng(i).random((c["B"], c["K"])) < 0.5, w.tokens,
                    np.argmax(wl.as_f32(w.target[:, :c["K"]]), axis=2) if c["K"] else w.tokens).astype(np.int32)
    if c["T"] > 0.0:  # at temperature 0 the point entry is the greedy path checked above
        check_point(w, toks, report=rep)
    lens = np.random.default_rng(i + 1).integers(-1, c["K"] + 2, c["B"]).astype(np.int32)
    check_ragged(w, lens, report=rep)
    # a tree over the same kind of rows
    # (siblings carry distinct tokens, so at most V of them)
    br = [min(int(x), c["V"]) for x in
          np.random.default_rng(i + 2).integers(1, 4, int(np.random.default_rng(i + 3).integers(0, 4)))]
    t = wl.make_tree(min(c["B"], 6), br, c["V"], target_dtype=c["tdt"], temperature=c["T"], top_k=c["top_k"],
                     top_p=c["top_p"], sigma=c["sigma"], rho=c["rho"], seed=c["seed"] + 7, vseed=c["seed"] + 8)
    check_tree(t, report=rep)
    print(rep)
