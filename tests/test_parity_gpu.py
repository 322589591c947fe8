"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Workloads are the five measured configurations (full size; the oracle checks
every sequence where it finishes in seconds, otherwise a fixed sample of
sequences computed one by one) plus smaller cases with the same generators
that span several tiles and a ragged tail, and the degenerate cases.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_verification_02_amd import binding
from draft_verification_02_amd import workloads as wl

from parity import check_greedy, check_sampling, f32, gpu_sampling, upload

pytestmark = pytest.mark.gpu


def _print_case(name):
    print(f"[case] {name}", flush=True)


# ---------------------------------------------------------------------------
# Random numbers
# ---------------------------------------------------------------------------

def test_device_uniforms_match_oracle_bitwise():
    _print_case("uniforms")
    seed, B, K = 0xC0FFEE0300000007, 300, 15
    ua, us = binding.rng_uniforms(seed, B, K)
    ua, us = ua.cpu().numpy(), us.cpu().numpy()
    for b in range(B):
        for k in range(K):
            assert ua[b, k] == oracle.u24(seed, b, k, 0)
        for k in range(K + 1):
            assert us[b, k] == oracle.u53(seed, b, k, 1)


# ---------------------------------------------------------------------------
# The five measured workloads
# ---------------------------------------------------------------------------

def test_c1_tiny_all_rounds():
    _print_case("c1 x256 rounds")
    from parity import Report
    rep = Report()
    for rnd in range(wl.C1_ROUNDS):
        w = wl.config(1, rnd)
        check_sampling(w, report=rep)
    print(rep)


def test_c2_block16_single_stream():
    _print_case("c2 full")
    w = wl.config(2)
    print(check_sampling(w))


def test_c2_many_seeds_small_vocab():
    """c2's generator at V=20000 over many seeds: more accept decisions."""
    _print_case("c2-like V=20000 x16 seeds")
    from parity import Report
    rep = Report()
    for rnd in range(16):
        w = wl.config(2, rnd, V=20000, B=4)
        check_sampling(w, report=rep)
    print(rep)


def test_c3_concurrent_batch_full_size_all_sequences():
    _print_case("c3 full, all 32 sequences checked")
    w = wl.config(3)
    print(check_sampling(w))


def test_c3_generator_small_batch_all_sequences():
    _print_case("c3-like B=8 V=40000")
    w = wl.config(3, 1, B=8, V=40000)
    print(check_sampling(w))


def test_c4_greedy_full():
    _print_case("c4 greedy full")
    w = wl.config(4)
    check_greedy(w)
    check_greedy(w, via_verify=True)


def test_c5_large_batch_full_size_sampled():
    _print_case("c5 full, 64 of 256 sequences checked")
    w = wl.config(5)
    print(check_sampling(w, seqs=list(range(0, 256, 4))))


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("V", [1, 2, 7, 8191, 8192, 8193, 12347])
@pytest.mark.parametrize("tdt,ddt", [(wl.F32, wl.F32), (wl.BF16, wl.F32), (wl.BF16, wl.BF16)])
def test_ragged_vocab_and_dtypes(V, tdt, ddt):
    _print_case(f"ragged V={V} dtypes={tdt},{ddt}")
    w = wl.make(3, 4, V, target_dtype=tdt, draft_dtype=ddt, temperature=1.0, rho=0.9,
                seed=V * 7 + tdt, vseed=V + 99)
    check_sampling(w)


@pytest.mark.parametrize("top_k,top_p", [(1, 1.0), (5, 1.0), (50, 0.95), (0, 0.5), (0, 0.99),
                                         (3000, 1.0), (100000, 0.9), (0, 1e-6)])
def test_filters(top_k, top_p):
    _print_case(f"filters top_k={top_k} top_p={top_p}")
    w = wl.make(4, 5, 30011, temperature=0.9, top_k=top_k, top_p=top_p, rho=0.8, n_boost=3,
                seed=top_k + 17, vseed=top_k + 5)
    check_sampling(w)


@pytest.mark.parametrize("top_k,top_p", [(3000, 1.0), (0, 0.99)])
def test_rows_resolved_by_rereading(top_k, top_p):
    """Kept sets larger than the capture reservoir: such rows are resolved by
    re-reading the row (flagged per row); the path must be taken and agree."""
    _print_case(f"re-read resolution top_k={top_k} top_p={top_p}")
    w = wl.make(4, 5, 30011, temperature=0.9, top_k=top_k, top_p=top_p, rho=0.8, n_boost=3,
                seed=top_k + 17, vseed=top_k + 5)
    rep = check_sampling(w)
    assert rep is not None
    _, _, ts, ds = gpu_sampling(w)
    flags = np.concatenate([ts["flags"].ravel(), ds["flags"].ravel()])
    assert (flags & binding.ROW_FILTERED).all()
    assert (flags & binding.ROW_EXACT_PATH).any(), "no row took the re-read path"


def test_ties_at_filter_thresholds():
    """Quantised logits: heavy ties at the top-k value and inside nucleus groups."""
    _print_case("ties")
    rng = np.random.default_rng(9)
    B, K, V = 6, 3, 5000
    x = rng.integers(-8, 9, size=(B, K + 1, V)).astype(np.float32) * np.float32(0.5)
    d = rng.integers(-8, 9, size=(B, K, V)).astype(np.float32) * np.float32(0.5)
    toks = rng.integers(0, V, size=(B, K)).astype(np.int32)
    for top_k, top_p in [(7, 1.0), (40, 0.8), (0, 0.7)]:
        w = wl.Workload("ties", B, K, V, wl.f32_to_bf16_bits(x), d, toks, 1.0, top_k, top_p, 77)
        check_sampling(w)


def test_neg_inf_logits_and_out_of_range_tokens():
    _print_case("-inf and out-of-range")
    rng = np.random.default_rng(10)
    B, K, V = 5, 4, 9000
    x = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    x[:, :, ::3] = -np.inf
    d = (0.7 * x[:, :K] + rng.standard_normal((B, K, V))).astype(np.float32)
    toks = rng.integers(0, V, size=(B, K)).astype(np.int32)
    toks[0, 0] = -1
    toks[1, 1] = V
    toks[2, 0] = 3  # a -inf target logit
    for top_k, top_p in [(0, 1.0), (20, 0.9)]:
        w = wl.Workload("neginf", B, K, V, x, d, toks, 1.0, top_k, top_p, 5)
        check_sampling(w)


def test_k0_bonus_only_and_identical_distributions():
    _print_case("K=0 and identical rows")
    w = wl.make(7, 0, 20000, seed=3, vseed=4)
    check_sampling(w)
    rng = np.random.default_rng(2)
    B, K, V = 4, 6, 10000
    x = (rng.standard_normal((B, K + 1, V)) * 3).astype(np.float32)
    toks = rng.integers(0, V, size=(B, K)).astype(np.int32)
    w = wl.Workload("same", B, K, V, x, x[:, :K].copy(), toks, 1.3, 0, 1.0, 8)
    g_tok, g_num, _, _ = gpu_sampling(w, stats=False)
    assert (g_num == K).all()
    check_sampling(w)


@pytest.mark.parametrize("T", [0.05, 0.37, 2.5])
def test_temperatures(T):
    _print_case(f"T={T}")
    w = wl.make(3, 5, 16385, temperature=T, rho=0.9, n_boost=2, seed=int(T * 100), vseed=1)
    check_sampling(w)


@pytest.mark.parametrize("offset", [-3000.0, 500.0, 20000.0])
@pytest.mark.parametrize("top_p", [0.9, 1.0])
def test_large_logit_offsets(offset, top_p):
    """Logits shifted far from zero (f32 rows): the streamed sums use the
    float just below log2(e)/T and take a 2^(M c_lo) factor into the exact
    units, which grows with |M|; the nucleus target and p(d_k) must still
    match the oracle."""
    _print_case(f"offset {offset} top_p {top_p}")
    w = wl.make(3, 4, 20011, target_dtype=wl.F32, temperature=0.6, top_p=top_p, rho=0.85,
                seed=int(abs(offset)) + 3, vseed=11)
    w.target = (w.target + np.float32(offset)).astype(np.float32)
    w.draft = (w.draft + np.float32(offset)).astype(np.float32)
    check_sampling(w)


def test_greedy_edge_cases():
    _print_case("greedy edges")
    rng = np.random.default_rng(12)
    for (B, K, V) in [(3, 0, 100), (5, 7, 1), (4, 6, 8193), (9, 3, 12347)]:
        x = rng.integers(-3, 4, size=(B, K + 1, V)).astype(np.float32)  # ties
        g = x.argmax(-1).astype(np.int32)
        toks = g[:, :K].copy()
        if K > 0:
            toks[::2, K // 2] = (toks[::2, K // 2] + 1) % max(V, 1)
        for tgt in (x, wl.f32_to_bf16_bits(x)):
            w = wl.Workload("g", B, K, V, tgt, None, toks, 0.0, 0, 1.0, 0)
            check_greedy(w)


@pytest.mark.parametrize("B", [1, 511, 512, 600])
def test_greedy_batches_around_the_single_launch_limit(B):
    """Greedy verification runs in one launch below 512 sequences (the last
    row of each sequence to finish writes its outputs, the last sequence the
    acceptance counts) and in two launches from 512 on: both give the
    oracle's tokens, and the ragged call's counters match their definition,
    on two calls in a row (the arrival counters must be left at zero)."""
    from parity import check_ragged
    _print_case(f"greedy B={B}")
    rng = np.random.default_rng(B)
    K, V = 3, 700
    x = rng.integers(-4, 5, size=(B, K + 1, V)).astype(np.float32)  # ties
    g = x.argmax(-1).astype(np.int32)
    toks = g[:, :K].copy()
    miss = rng.random((B, K)) < 0.3
    toks[miss] = (toks[miss] + 1) % V
    for tgt in (x, wl.f32_to_bf16_bits(x)):
        w = wl.Workload("g", B, K, V, tgt, None, toks, 0.0, 0, 1.0, 0)
        check_greedy(w)
        check_greedy(w, via_verify=True)
        check_ragged(w, _lens(B, K, B + 1))
        check_ragged(w, _lens(B, K, B + 2))


def test_unaligned_rows():
    """bf16 rows of odd length start at 2-byte offsets: element-wise load path."""
    _print_case("unaligned")
    w = wl.make(3, 3, 9999, target_dtype=wl.BF16, draft_dtype=wl.BF16, temperature=1.0,
                top_p=0.9, seed=31, vseed=32)
    check_sampling(w)
    w.temperature = 0.0
    check_greedy(w)


def test_deterministic_and_workspace_reuse():
    _print_case("determinism")
    big = wl.make(6, 5, 50000, top_p=0.9, temperature=0.8, seed=41, vseed=42)
    small = wl.make(2, 2, 3000, seed=43, vseed=44)
    r1 = gpu_sampling(big, stats=False)
    r2 = gpu_sampling(small, stats=False)
    r3 = gpu_sampling(big, stats=False)
    r4 = gpu_sampling(small, stats=False)
    np.testing.assert_array_equal(r1[0], r3[0])
    np.testing.assert_array_equal(r2[0], r4[0])
    check_sampling(big)
    check_sampling(small)


def test_empty_batch_is_noop():
    _print_case("B=0")
    t = torch.zeros((0, 3, 10), device="cuda")
    d = torch.zeros((0, 2, 10), device="cuda")
    k = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    out, n = binding.spec_verify(t, d, k, 1.0)
    torch.cuda.synchronize()
    assert out.shape == (0, 3) and n.shape == (0,)


def test_stats_entry_matches_plain_entry():
    _print_case("stats == plain")
    w = wl.make(5, 4, 20000, top_p=0.9, top_k=100, temperature=0.7, seed=50, vseed=51)
    a = gpu_sampling(w, stats=True)
    b = gpu_sampling(w, stats=False)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# Point-mass drafts (no draft logits)
# ---------------------------------------------------------------------------

def test_point_c3_shape_full_size_sampled():
    """c3's target rows, drafts proposed by the draft rows' argmax."""
    from parity import check_point, point_tokens
    _print_case("point c3 full, 8 sequences checked")
    w = wl.config(3)
    print(check_point(w, point_tokens(w), seqs=[0, 3, 9, 14, 20, 23, 28, 31]))


@pytest.mark.parametrize("cfg,kw", [(3, dict(B=8, V=40000)), (2, dict(B=4, V=20000)),
                                    (5, dict(B=6, V=30011)), (1, {})])
def test_point_small_all_sequences(cfg, kw):
    from parity import Report, check_point, point_tokens
    _print_case(f"point cfg{cfg} {kw}")
    rep = Report()
    for rnd in range(4):
        w = wl.config(cfg, rnd, **kw)
        check_point(w, point_tokens(w), report=rep)
        # proposals that are the sampled draft tokens (in range, any value)
        check_point(w, w.tokens, report=rep)
    print(rep)


def test_point_c5_full_size_sampled():
    from parity import check_point, point_tokens
    _print_case("point c5 full, 16 sequences checked")
    w = wl.config(5)
    print(check_point(w, point_tokens(w), seqs=list(range(0, 256, 16))))


@pytest.mark.parametrize("V", [1, 7, 8193])
@pytest.mark.parametrize("tdt", [wl.F32, wl.BF16])
def test_point_ragged_vocab_and_dtypes(V, tdt):
    from parity import check_point
    _print_case(f"point ragged V={V} tdt={tdt}")
    w = wl.make(3, 4, V, target_dtype=tdt, draft_dtype=wl.F32, temperature=1.0, rho=0.9,
                seed=V * 3 + tdt, vseed=V + 7)
    check_point(w, w.tokens)


def test_point_edge_cases():
    """Out-of-range proposals (always rejected, plain draw from p_0), K = 0,
    a proposal holding all the mass (always accepted), temperature 0
    (greedy), and the point entry against the general entry fed one-hot
    draft rows."""
    from parity import check_point, to_device
    _print_case("point edge cases")
    w = wl.make(6, 3, 5000, temperature=0.8, top_p=0.9, rho=0.9, seed=5, vseed=6)
    toks = w.tokens.copy()
    toks[:3] = -1
    toks[3:, 1] = 5000
    check_point(w, toks)
    w0 = wl.make(5, 0, 777, temperature=1.0, seed=8, vseed=9)
    check_point(w0, np.zeros((5, 0), np.int32))
    t1 = np.full((4, 3, 300), -np.inf, np.float32)
    t1[:, :, 17] = 1.0
    k1 = np.full((4, 2), 17, np.int32)
    tok, num = binding.spec_verify_point(to_device(t1), torch.from_numpy(k1).cuda(), 1.3)
    torch.cuda.synchronize()
    assert (num.cpu().numpy() == 2).all() and (tok.cpu().numpy() == 17).all()
    wg = wl.config(4, B=8, V=20000)
    tg, kg = to_device(wg.target), torch.from_numpy(wg.tokens).cuda()
    a = binding.spec_verify_point(tg, kg, 0.0)
    b = binding.spec_verify_greedy(tg, kg)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # one-hot draft rows through the general entry give the same tokens
    V = 4099
    w1 = wl.make(8, 4, V, temperature=0.9, top_k=40, top_p=0.95, rho=0.8, seed=21, vseed=22)
    oh = np.full((8, 4, V), -np.inf, np.float32)
    bb, kk = np.meshgrid(np.arange(8), np.arange(4), indexing="ij")
    oh[bb, kk, w1.tokens] = 0.0
    tgt, kt = to_device(w1.target), torch.from_numpy(w1.tokens).cuda()
    pa = binding.spec_verify_point(tgt, kt, w1.temperature, w1.top_k, w1.top_p, w1.seed)
    ga = binding.spec_verify(tgt, to_device(oh), kt, w1.temperature, w1.top_k, w1.top_p, w1.seed)
    torch.cuda.synchronize()
    assert torch.equal(pa[0], ga[0]) and torch.equal(pa[1], ga[1])


# ---------------------------------------------------------------------------
# Per-sequence draft lengths and acceptance counters
# ---------------------------------------------------------------------------

def _lens(B, K, seed):
    return np.random.default_rng(seed).integers(0, K + 1, B).astype(np.int32)


def test_ragged_c3_full_size_sampled():
    from parity import check_ragged
    _print_case("ragged c3 full, 8 sequences checked")
    w = wl.config(3)
    print(check_ragged(w, _lens(w.B, w.K, 1), seqs=[0, 2, 7, 12, 19, 25, 30, 31]))


@pytest.mark.parametrize("cfg,kw", [(3, dict(B=8, V=40000)), (2, dict(B=4, V=20000)),
                                    (5, dict(B=6, V=30011)), (1, {}), (4, dict(B=16, V=20000))])
def test_ragged_small_all_sequences(cfg, kw):
    from parity import Report, check_ragged
    _print_case(f"ragged cfg{cfg} {kw}")
    rep = Report()
    for rnd in range(3):
        w = wl.config(cfg, rnd, **kw)
        check_ragged(w, _lens(w.B, w.K, 10 * cfg + rnd), report=rep)
    print(rep)


def test_ragged_lengths_extremes_and_full_equals_plain():
    """All lengths 0 (bonus only), all K (bitwise equal to spec_verify),
    out-of-range lengths (clamped)."""
    from parity import check_ragged, upload
    _print_case("ragged extremes")
    w = wl.make(6, 5, 9000, temperature=0.8, top_p=0.9, rho=0.9, seed=41, vseed=42)
    check_ragged(w, np.zeros(6, np.int32))
    check_ragged(w, np.full(6, 5, np.int32))
    check_ragged(w, np.array([-3, 0, 2, 5, 9, 100], np.int32))
    t, d, k = upload(w)
    a = binding.spec_verify_ragged(t, d, k, torch.full((6,), 5, dtype=torch.int32, device="cuda"),
                                   w.temperature, w.top_k, w.top_p, w.seed)
    b = binding.spec_verify(t, d, k, w.temperature, w.top_k, w.top_p, w.seed)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---------------------------------------------------------------------------
# Long kept-list paths, large K and B
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tdt,V", [(wl.F32, 151936), (wl.BF16, 300007)])
def test_kept_lists_of_rows_with_many_token_blocks(tdt, V):
    """Rows with more than 512 blocks of 64 loads (f32 rows at V = 151936,
    bf16 rows past 262144): the kept list is ranked by the side-by-side
    binary searches instead of block counts."""
    _print_case(f"many blocks tdt={tdt} V={V}")
    w = wl.make(3, 3, V, target_dtype=tdt, draft_dtype=wl.F32, temperature=0.7, top_p=0.9,
                rho=0.8, seed=V + tdt, vseed=V + 1)
    print(check_sampling(w))
    from parity import check_point
    check_point(w, w.tokens)


def test_long_drafts_and_wide_batches():
    """K = 63 (the accept scan spans a full wave) and B = 512 sequences."""
    _print_case("K=63 and B=512")
    w = wl.make(2, 63, 4099, temperature=1.0, top_p=0.95, rho=0.97, seed=63, vseed=64)
    print(check_sampling(w))
    w = wl.make(512, 2, 1000, target_dtype=wl.F32, temperature=0.9, top_k=20, rho=0.8,
                seed=512, vseed=513)
    print(check_sampling(w, check_stats=False))


def test_more_rows_than_one_round_of_workgroups():
    """Batches with more rows than the GPU runs at once (draft rows take the
    first workgroups): general and ragged calls with filters, every sequence
    against the oracle, at a small vocabulary."""
    from parity import check_ragged
    _print_case("rows > one round: B=96 K=7 V=3001")
    w = wl.make(96, 7, 3001, target_dtype=wl.BF16, draft_dtype=wl.F32, temperature=0.7, top_p=0.9,
                rho=(0.6, 0.95), n_boost=4, seed=9601, vseed=9602)
    print(check_sampling(w))
    print(check_ragged(w, _lens(w.B, w.K, 96)))
    w = wl.make(64, 7, 2500, target_dtype=wl.F32, draft_dtype=wl.BF16, temperature=1.0, top_k=40,
                rho=0.8, seed=6401, vseed=6402)
    print(check_sampling(w))


def test_concurrent_streams_have_their_own_workspace():
    """Calls on two streams at once (each with its own workspace), repeated,
    give the results of the same calls made one after another; a token tree
    on a third stream too."""
    from parity import tree_inputs
    _print_case("two streams + tree stream")
    w1 = wl.config(3, B=8, V=40000)
    w2 = wl.make(5, 3, 30011, target_dtype=wl.F32, draft_dtype=wl.BF16, temperature=1.0, top_k=40, rho=0.8,
                 seed=71, vseed=72)
    wt = wl.make_tree(4, [3, 2], 20000, temperature=0.8, top_p=0.95, seed=73, vseed=74)
    a1, a2 = upload(w1), upload(w2)
    tt, tk, tp = tree_inputs(wt)
    torch.cuda.synchronize()

    def call(w, a, stream=None):
        return binding.spec_verify(*a, w.temperature, w.top_k, w.top_p, w.seed, stream=stream)

    r1, r2 = call(w1, a1), call(w2, a2)
    rt = binding.spec_verify_tree(tt, tk, tp, wt.temperature, wt.top_k, wt.top_p, wt.seed)
    torch.cuda.synchronize()
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(s1):
            c1 = call(w1, a1, s1)
        with torch.cuda.stream(s2):
            c2 = call(w2, a2, s2)
        with torch.cuda.stream(s3):
            ct = binding.spec_verify_tree(tt, tk, tp, wt.temperature, wt.top_k, wt.top_p, wt.seed, stream=s3)
        torch.cuda.synchronize()
        for x, y in zip(c1 + c2 + ct, r1 + r2 + rt):
            assert torch.equal(x, y)


def test_drafts_longer_than_a_sequence_workgroup():
    """K = 300 (> 256 threads of the draw workgroup: the output writer reads
    the drafted tokens past the first 256 from memory).  top-k 1 keeps only
    each row's argmax, so argmax proposals are always accepted; sequence 0
    proposes another token at position 280 (rejected there), sequence 1
    accepts all 300 (bonus)."""
    from parity import check_point
    _print_case("K=300")
    w = wl.make(2, 300, 257, target_dtype=wl.F32, draft_dtype=wl.F32, temperature=1.0, top_k=1, sigma=3.0,
                rho=0.9, seed=300, vseed=301)
    toks = np.argmax(wl.as_f32(w.target[:, :w.K]), axis=2).astype(np.int32)
    toks[0, 280] = (toks[0, 280] + 1) % w.V
    print(check_point(w, toks))
    w.tokens = toks
    print(check_sampling(w, check_stats=False))
    r = gpu_sampling(w, stats=False)
    assert r[1].tolist() == [280, 300], r[1]
