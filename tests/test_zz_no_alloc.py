"""The allocation-free entry point (spec_verify_noalloc) against spec_verify.

Both run the same kernels; the allocation-free one carves its scratch from a
fixed static device array instead of a per-stream allocation.  Outputs must
be bitwise equal to spec_verify's on consecutive calls whose sizes shrink (so
scratch contents left by a larger call are in the way of a smaller one), over
the filtered kept-list draw, rows split over workgroups (merged by their
last part through per-row counters), the unfiltered chunked draw with its
arrival counters, and greedy mode; a problem beyond the scratch is refused.
"""
import numpy as np
import pytest
import torch

from draft_verification_02_amd import binding
from draft_verification_02_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _both(w):
    from parity import upload
    t, d, k = upload(w)
    B, K = w.B, w.K
    a_tok, a_num = binding.spec_verify(t, d, k, w.temperature, w.top_k, w.top_p, w.seed)
    n_tok = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
    n_num = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    binding.spec_verify_noalloc(t, d, k, w.temperature, w.top_k, w.top_p, w.seed, n_tok, n_num)
    torch.cuda.synchronize()
    return a_tok.cpu().numpy(), a_num.cpu().numpy(), n_tok.cpu().numpy(), n_num.cpu().numpy()


def _check(w, name):
    print(f"[case] noalloc {name}", flush=True)
    a_tok, a_num, n_tok, n_num = _both(w)
    np.testing.assert_array_equal(n_num, a_num)
    np.testing.assert_array_equal(n_tok, a_tok)


def test_noalloc_matches_spec_verify_on_shrinking_calls():
    # the concurrent-batch workload (kept lists), then smaller calls
    _check(wl.config(3), "c3 B32 K7 V151936 top-p")
    # a single stream: its 31 unfiltered rows are split over many workgroups
    # whose last part merges each row (per-row counters at the scratch's
    # start, which every call must leave at zero), twice in a row
    _check(wl.config(2), "c2 B1 K15 V151936 split rows")
    _check(wl.config(2, rnd=1), "c2 again, next round's inputs")
    _check(wl.make(4, 3, 5003, target_dtype=wl.F32, draft_dtype=wl.BF16, temperature=1.0, rho=0.9,
                   seed=11, vseed=12), "B4 K3 V5003 unfiltered")
    _check(wl.make(3, 2, 4001, temperature=0.8, top_k=30, top_p=0.9, rho=0.85, seed=13, vseed=14),
           "B3 K2 V4001 top-k top-p")
    _check(wl.make(2, 1, 3001, temperature=1.2, rho=0.95, seed=15, vseed=16), "B2 K1 V3001 unfiltered")
    _check(wl.config(4, B=4, V=20000), "greedy B4 K15 V20000")
    _check(wl.make(1, 0, 999, temperature=1.0, seed=17, vseed=18), "B1 K0 bonus only")


def test_noalloc_matches_the_oracle_on_a_small_call():
    from parity import check_sampling
    w = wl.make(3, 4, 7001, temperature=0.9, top_p=0.95, rho=0.9, n_boost=3, seed=19, vseed=20)
    _check(w, "B3 K4 V7001 then oracle")
    check_sampling(w)


def test_noalloc_refuses_problems_beyond_its_scratch():
    print("[case] noalloc too large", flush=True)
    B, K, V = 500, 7, 2048  # 4000 target rows, each with an 80 KiB kept list
    t = torch.zeros((B, K + 1, V), dtype=torch.bfloat16, device="cuda")
    d = torch.zeros((B, K, V), dtype=torch.float32, device="cuda")
    k = torch.zeros((B, K), dtype=torch.int32, device="cuda")
    o = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
    n = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(binding.SpecVerifyError) as e:
        binding.spec_verify_noalloc(t, d, k, 1.0, 0, 0.9, 0, o, n)
    assert e.value.status == binding.SPEC_E_SCRATCH
    torch.cuda.synchronize()
    assert (o == -7).all() and (n == -7).all()  # nothing was launched
