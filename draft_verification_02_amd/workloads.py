"""Seeded synthetic inputs for batched speculative-decoding verification.

This module only draws inputs: target logits, draft logits and drafted token
ids with the shapes, dtypes and value distributions of the five workloads the
library is measured on.  It holds none of the verifier's arithmetic (no
temperature processing of the verified rows, no top-k / top-p, no softmax, no
rejection test) and is shared by the tests, the benchmark and the oracle
checks only as a source of bytes.

Random numbers come from numpy's Philox bit generator, one key per
(kind, row), so any row can be regenerated on its own.

Drafted tokens are drawn the way a drafter samples its own proposals: at
temperature T > 0 from softmax(d / T) over the whole vocabulary (the FlashMap
page, section 5, draft_block: softmax of logits / temperature, then a
multinomial draw), realised here as a Gumbel-max draw argmax(d / T + G) so
that no softmax is computed; at T = 0 the draft argmax (lowest index among
equal maxima).  The drafter applies no top-k / top-p, so under the filtered
workloads a drafted token can fall outside the draft's kept set (q = 0).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

F32 = 0
BF16 = 1

# Philox stream kinds (second key word).
_S_TARGET = 1
_S_BOOST = 2
_S_DRAFT = 3
_S_DRAFT_SAMPLE = 4
_S_RHO = 5
_S_TREE = 6
_S_HIDDEN = 7
_S_UNEMBED = 8


def gen_seed(cfg: int, rnd: int = 0) -> int:
    """Seed of the input generator for workload ``cfg``, round ``rnd``."""
    return (0x5EED0000_00000000 + (cfg << 32) + rnd) & 0xFFFFFFFFFFFFFFFF


def verify_seed(cfg: int, rnd: int = 0) -> int:
    """Seed passed to the verifier for workload ``cfg``, round ``rnd``."""
    return (0xC0FFEE00_00000000 + (cfg << 32) + rnd) & 0xFFFFFFFFFFFFFFFF


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    raw 16-bit patterns as uint16.  Inputs must be finite or +-inf."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = u + np.uint32(0x7FFF) + lsb
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen raw bf16 patterns (uint16) to float32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(a: np.ndarray) -> np.ndarray:
    """Float32 view of stored logits of either storage format."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float32)


def dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported logit storage {a.dtype}")


def _rng(seed: int, kind: int, index: int) -> np.random.Generator:
    # One key per (kind, row): streams that share a key but start at nearby
    # counters would overlap, since the counter advances as values are drawn.
    return np.random.Generator(np.random.Philox(key=[seed, (kind << 40) | index]))


@dataclass
class Workload:
    name: str
    B: int
    K: int
    V: int
    target: np.ndarray           # [B, K+1, V] float32 or uint16 (bf16 bits)
    draft: np.ndarray | None     # [B, K, V]
    tokens: np.ndarray           # [B, K] int32
    temperature: float
    top_k: int
    top_p: float
    seed: int
    meta: dict = field(default_factory=dict)

    @property
    def greedy(self) -> bool:
        return self.temperature == 0.0

    def ideal_bytes(self) -> int:
        """Algorithmic bytes of one verification: every target row, plus every
        draft row in sampling mode (greedy reads the target only)."""
        tb = self.B * (self.K + 1) * self.V * self.target.dtype.itemsize
        if self.greedy or self.draft is None:
            return tb
        return tb + self.B * self.K * self.V * self.draft.dtype.itemsize


def make(B: int, K: int, V: int, *, target_dtype: int = BF16, draft_dtype: int = F32,
         temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0,
         dist: str = "gauss", sigma: float = 3.0, rho=0.9, n_boost: int = 0,
         boost: float = 8.0, seed: int = 1, vseed: int | None = None,
         name: str = "custom", threads: int | None = None, with_draft: bool = True) -> Workload:
    """Draw one workload.

    dist="gauss": target x = N(0, sigma^2) (+ ``boost`` on ``n_boost`` distinct
    uniform ids per row), draft d = rho * x_stored + sqrt(1 - rho^2) * N(0, sigma^2).
    dist="t3": target x = sigma * t_3, draft d = rho * x_stored + sqrt(1-rho^2) * sigma * t_3'.
    rho: a number, or a pair (lo, hi) to draw one rho per sequence from U(lo, hi).
    The draft is built from the stored (rounded) target value.  with_draft=False
    draws the target rows only (draft None, tokens zero).
    """
    if dist not in ("gauss", "t3"):
        raise ValueError(dist)
    target = np.empty((B, K + 1, V), dtype=np.uint16 if target_dtype == BF16 else np.float32)
    draft = np.empty((B, K, V) if with_draft else (0,), dtype=np.uint16 if draft_dtype == BF16 else np.float32)
    tokens = np.zeros((B, K), dtype=np.int32)
    if isinstance(rho, (tuple, list)):
        rr = _rng(seed, _S_RHO, 0)
        rhos = rr.uniform(rho[0], rho[1], size=B)
    else:
        rhos = np.full(B, float(rho))

    def one_sequence(b: int) -> None:
        for k in range(K + 1):
            row = b * (K + 1) + k
            g = _rng(seed, _S_TARGET, row)
            if dist == "gauss":
                x = g.standard_normal(V) * sigma
            else:
                x = g.standard_t(3, V) * sigma
            if n_boost:
                ids = _rng(seed, _S_BOOST, row).choice(V, size=min(n_boost, V), replace=False)
                x[ids] += boost
            x32 = x.astype(np.float32)
            if target_dtype == BF16:
                target[b, k] = f32_to_bf16_bits(x32)
            else:
                target[b, k] = x32
            if k == K or not with_draft:
                continue
            stored = as_f32(target[b, k]).astype(np.float64)
            drow = b * K + k
            gd = _rng(seed, _S_DRAFT, drow)
            noise = gd.standard_normal(V) if dist == "gauss" else gd.standard_t(3, V)
            r = rhos[b]
            d = r * stored + np.sqrt(max(0.0, 1.0 - r * r)) * sigma * noise
            d32 = d.astype(np.float32)
            if draft_dtype == BF16:
                draft[b, k] = f32_to_bf16_bits(d32)
            else:
                draft[b, k] = d32
            dv = as_f32(draft[b, k]).astype(np.float64)
            if temperature > 0:
                u = _rng(seed, _S_DRAFT_SAMPLE, drow).random(V)
                with np.errstate(divide="ignore"):
                    gumbel = -np.log(-np.log(u))
                tokens[b, k] = int(np.argmax(dv / temperature + gumbel))
            else:
                tokens[b, k] = int(np.argmax(dv))

    nthreads = threads or min(16, os.cpu_count() or 1)
    if B * (K + 1) * V < (1 << 20) or nthreads <= 1:
        for b in range(B):
            one_sequence(b)
    else:
        with ThreadPoolExecutor(max_workers=nthreads) as ex:
            list(ex.map(one_sequence, range(B)))
    return Workload(name=name, B=B, K=K, V=V, target=target, draft=draft if K > 0 and with_draft else None,
                    tokens=tokens, temperature=float(temperature), top_k=int(top_k),
                    top_p=float(top_p), seed=vseed if vseed is not None else seed,
                    meta={"dist": dist, "sigma": sigma, "rho": rho, "n_boost": n_boost,
                          "rhos": rhos})


def tree_shape(branching) -> np.ndarray:
    """Parent indices of a static token tree in breadth-first order: the root
    has branching[0] children, every node at depth d (1-based) has
    branching[d] children.  Returns int32 [N] (-1 = child of the root)."""
    par, level = [], [-1]
    for m in branching:
        nxt = []
        for u in level:
            for _ in range(m):
                par.append(u)
                nxt.append(len(par) - 1)
        level = nxt
    return np.asarray(par, dtype=np.int32)


def make_tree(B: int, branching, V: int, *, target_dtype: int = BF16, temperature: float = 1.0,
              top_k: int = 0, top_p: float = 1.0, sigma: float = 3.0, rho=0.9, n_boost: int = 0,
              boost: float = 8.0, seed: int = 1, vseed: int | None = None,
              name: str = "tree") -> Workload:
    """A batch of token trees (multi-head / tree speculation).  The target rows
    [B, N+1, V] are drawn as in ``make`` with K = N (row 0 for the root, row
    i+1 after node i); every sequence shares the tree shape of
    ``tree_shape(branching)``, and the children of node u carry the
    ``m`` distinct tokens ranked highest by a proposer's noisy copy of row
    u+1, rho * x + sqrt(1 - rho^2) * sigma * N(0, 1), as draft heads propose
    their top candidates.  ``meta['parents']`` holds the parents [B, N]."""
    par = tree_shape(branching)
    N = len(par)
    w = make(B, N, V, target_dtype=target_dtype, draft_dtype=F32, temperature=temperature,
             top_k=top_k, top_p=top_p, sigma=sigma, rho=rho, n_boost=n_boost, boost=boost,
             seed=seed, vseed=vseed, name=name, with_draft=False)
    kids = [[i for i in range(N) if par[i] == u] for u in range(-1, N)]
    tokens = np.zeros((B, N), dtype=np.int32)
    for b in range(B):
        r = float(w.meta["rhos"][b])
        for u in range(-1, N):
            if not kids[u + 1]:
                continue
            x = as_f32(w.target[b, u + 1]).astype(np.float64)
            g = _rng(seed, _S_TREE, b * (N + 1) + u + 1)
            prop = r * x + np.sqrt(max(0.0, 1.0 - r * r)) * sigma * g.standard_normal(V)
            m = len(kids[u + 1])
            top = np.argpartition(-prop, m - 1)[:m]
            top = top[np.argsort(-prop[top], kind="stable")]
            tokens[b, kids[u + 1]] = top
    w.tokens = tokens
    w.meta["parents"] = np.ascontiguousarray(np.broadcast_to(par, (B, N)))
    w.meta["branching"] = list(branching)
    return w


def make_hidden(B: int, K: int, V: int, H: int, *, seed: int = 1, w_scale: float | None = None):
    """Inputs of greedy verification from hidden states: target hidden states
    [B, K+1, H] ~ N(0, 1) and an unembedding matrix [V, H] ~ N(0, w_scale^2)
    (random weights; w_scale defaults to 1/sqrt(H)), both as bf16 bit
    patterns (uint16), drawn one row at a time from their own streams."""
    if w_scale is None:
        w_scale = 1.0 / np.sqrt(H)
    hidden = np.empty((B, K + 1, H), dtype=np.uint16)
    for r in range(B * (K + 1)):
        hidden.reshape(-1, H)[r] = f32_to_bf16_bits(_rng(seed, _S_HIDDEN, r).standard_normal(H).astype(np.float32))
    w = np.empty((V, H), dtype=np.uint16)
    step = 4096
    for v0 in range(0, V, step):
        g = _rng(seed, _S_UNEMBED, v0 // step)
        n = min(step, V - v0)
        w[v0:v0 + n] = f32_to_bf16_bits((g.standard_normal((n, H), dtype=np.float32) * np.float32(w_scale)))
    return hidden, w


# The five measured workloads (shapes, dtypes, distributions and processing).
CONFIG_SPECS = {
    1: dict(name="c1 tiny sampling B1 K4 V1000 f32/f32", B=1, K=4, V=1000,
            target_dtype=F32, draft_dtype=F32, temperature=1.0, dist="gauss", sigma=3.0,
            rho=0.8, n_boost=0),
    2: dict(name="c2 block-16 single stream B1 K15 V151936 bf16/f32", B=1, K=15, V=151936,
            target_dtype=BF16, draft_dtype=F32, temperature=1.0, dist="gauss", sigma=3.0,
            rho=0.9, n_boost=4),
    3: dict(name="c3 concurrent batch B32 K7 V151936 bf16/f32 T0.7 top-p0.9", B=32, K=7,
            V=151936, target_dtype=BF16, draft_dtype=F32, temperature=0.7, top_p=0.9,
            dist="gauss", sigma=3.0, rho=(0.6, 0.95), n_boost=4),
    4: dict(name="c4 greedy B64 K15 V151936 bf16/bf16", B=64, K=15, V=151936,
            target_dtype=BF16, draft_dtype=BF16, temperature=0.0, dist="gauss", sigma=3.0,
            rho=0.85, n_boost=4),
    5: dict(name="c5 large batch t3 B256 K4 V262144 bf16/f32 top-k50 top-p0.95", B=256, K=4,
            V=262144, target_dtype=BF16, draft_dtype=F32, temperature=1.0, top_k=50,
            top_p=0.95, dist="t3", sigma=2.0, rho=0.8, n_boost=0),
}

C1_ROUNDS = 256


def config(cfg: int, rnd: int = 0, **overrides) -> Workload:
    """Workload ``cfg`` (1..5), round ``rnd``; ``overrides`` replace spec fields
    (e.g. a smaller B for a quick case with the same distributions)."""
    spec = dict(CONFIG_SPECS[cfg])
    spec.update(overrides)
    return make(seed=gen_seed(cfg, rnd), vseed=verify_seed(cfg, rnd), **spec)
