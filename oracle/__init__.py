"""CPU reference (oracle) for batched speculative-decoding verification.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``draft_verification_02_amd``) never imports, links or calls it, and
the two share no code.

The arithmetic lives in ``spec_oracle.cpp`` (plain single-threaded fp64 C++);
this module only builds it with g++ and marshals numpy arrays through ctypes.
Storage formats: float32 logits are ``np.float32`` arrays, bfloat16 logits are
``np.uint16`` arrays holding the raw bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1
PURPOSE_ACCEPT = 0
PURPOSE_SAMPLE = 1


class RowInfo(ctypes.Structure):
    _fields_ = [
        ("max_scaled", ctypes.c_double),
        ("z_kept", ctypes.c_double),
        ("thresh", ctypes.c_double),
        ("n_kept", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("nucleus_margin", ctypes.c_double),
        ("prob_at_token", ctypes.c_double),
    ]


ROW_INFO_DTYPE = np.dtype(
    [
        ("max_scaled", "<f8"),
        ("z_kept", "<f8"),
        ("thresh", "<f8"),
        ("n_kept", "<i4"),
        ("reserved", "<i4"),
        ("nucleus_margin", "<f8"),
        ("prob_at_token", "<f8"),
    ]
)
assert ROW_INFO_DTYPE.itemsize == ctypes.sizeof(RowInfo)


def build_library(force: bool = False) -> str:
    """Compile liboracle.so with g++ (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-o", tmp, _SRC],
            cwd=_HERE,
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build_library()
        L = ctypes.CDLL(_LIB)
        vp, i32, f64, u64, u32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
                                  ctypes.c_uint64, ctypes.c_uint32)
        L.oracle_philox4x32_10.argtypes = [vp, vp, vp]
        L.oracle_philox4x32_10.restype = None
        L.oracle_u24.argtypes = [u64, u32, u32, u32]
        L.oracle_u24.restype = f64
        L.oracle_u53.argtypes = [u64, u32, u32, u32]
        L.oracle_u53.restype = f64
        L.oracle_process_row.argtypes = [vp, i32, i32, f64, i32, f64, vp, vp]
        L.oracle_process_row.restype = i32
        L.oracle_verify.argtypes = [vp, i32, vp, i32, vp, i32, i32, i32, f64, i32, f64,
                                    u64, i32, vp, vp, vp, vp, vp, vp]
        L.oracle_verify.restype = i32
        L.oracle_verify_point.argtypes = [vp, i32, vp, i32, i32, i32, f64, i32, f64, u64, i32,
                                          vp, vp, vp, vp, vp]
        L.oracle_verify_point.restype = i32
        L.oracle_verify_tree.argtypes = [vp, i32, vp, vp, i32, i32, i32, f64, i32, f64, u64, i32,
                                         vp, vp, vp, vp, vp, vp]
        L.oracle_verify_tree.restype = i32
        L.oracle_verify_greedy.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp]
        L.oracle_verify_greedy.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported logit storage {a.dtype}")


def philox(counter, key) -> np.ndarray:
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def u24(seed: int, b: int, k: int, purpose: int) -> float:
    return lib().oracle_u24(seed, b, k, purpose)


def u53(seed: int, b: int, k: int, purpose: int) -> float:
    return lib().oracle_u53(seed, b, k, purpose)


def process_row(row: np.ndarray, temperature: float, top_k: int = 0, top_p: float = 1.0):
    """Processed distribution of one row: (prob[V] float64, info record)."""
    row = np.ascontiguousarray(row)
    V = row.shape[-1]
    prob = np.zeros(V, dtype=np.float64)
    info = np.zeros(1, dtype=ROW_INFO_DTYPE)
    rc = lib().oracle_process_row(_ptr(row), dtype_code(row), V, float(temperature),
                                  int(top_k), float(top_p), _ptr(prob), _ptr(info))
    if rc:
        raise ValueError(f"oracle_process_row failed ({rc})")
    return prob, info[0]


def verify(target, draft, tokens, temperature, top_k=0, top_p=1.0, seed=0, seq_base=0,
           diagnostics=True):
    """Sampling-mode (or, at temperature 0, greedy) verification.

    target: [B, K+1, V] (float32 or bf16-as-uint16); draft: [B, K, V];
    tokens: [B, K] int32.  Returns a dict with ``tokens`` [B, K+1],
    ``num_accepted`` [B] and, if ``diagnostics``, ``accept_margin`` [B, K],
    ``sample_margin`` [B], ``target_info`` [B, K+1], ``draft_info`` [B, K].
    """
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    draft = None if draft is None else np.ascontiguousarray(draft)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, K)
    out_tok = np.empty((B, K + 1), dtype=np.int32)
    out_n = np.empty(B, dtype=np.int32)
    am = sm = ti = di = None
    if diagnostics and temperature > 0:
        am = np.full((B, K), np.nan)
        sm = np.zeros(B)
        ti = np.zeros((B, K + 1), dtype=ROW_INFO_DTYPE)
        di = np.zeros((B, K), dtype=ROW_INFO_DTYPE)
    ddt = dtype_code(draft) if draft is not None else F32
    rc = lib().oracle_verify(_ptr(target), dtype_code(target), _ptr(draft), ddt, _ptr(tokens),
                             B, K, V, float(temperature), int(top_k), float(top_p),
                             int(seed) & 0xFFFFFFFFFFFFFFFF, int(seq_base), _ptr(out_tok),
                             _ptr(out_n), _ptr(am), _ptr(sm), _ptr(ti), _ptr(di))
    if rc:
        raise ValueError(f"oracle_verify failed ({rc})")
    res = {"tokens": out_tok, "num_accepted": out_n}
    if am is not None:
        res.update(accept_margin=am, sample_margin=sm, target_info=ti, draft_info=di)
    return res


def verify_point(target, tokens, temperature, top_k=0, top_p=1.0, seed=0, seq_base=0,
                 diagnostics=True):
    """Verification against point-mass drafts (no draft logits): target
    [B, K+1, V], tokens [B, K].  Same result dict as ``verify`` (without
    ``draft_info``)."""
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, K)
    out_tok = np.empty((B, K + 1), dtype=np.int32)
    out_n = np.empty(B, dtype=np.int32)
    am = sm = ti = None
    if diagnostics and temperature > 0:
        am = np.full((B, K), np.nan)
        sm = np.zeros(B)
        ti = np.zeros((B, K + 1), dtype=ROW_INFO_DTYPE)
    rc = lib().oracle_verify_point(_ptr(target), dtype_code(target), _ptr(tokens), B, K, V,
                                   float(temperature), int(top_k), float(top_p),
                                   int(seed) & 0xFFFFFFFFFFFFFFFF, int(seq_base), _ptr(out_tok),
                                   _ptr(out_n), _ptr(am), _ptr(sm), _ptr(ti))
    if rc:
        raise ValueError(f"oracle_verify_point failed ({rc})")
    res = {"tokens": out_tok, "num_accepted": out_n}
    if am is not None:
        res.update(accept_margin=am, sample_margin=sm, target_info=ti)
    return res


def verify_tree(target, tokens, parents, temperature, top_k=0, top_p=1.0, seed=0, seq_base=0,
                diagnostics=True):
    """Token-tree verification: target [B, N+1, V] (row 0 the root, row i+1
    after node i), tokens [B, N], parents [B, N] (-1 = root, else an index
    below the node's own).  Returns ``tokens`` [B, N+1], ``num_accepted`` [B],
    ``path`` [B, N] and, with ``diagnostics`` at temperature > 0,
    ``accept_margin`` [B, N], ``sample_margin`` [B], ``target_info`` [B, N+1]."""
    target = np.ascontiguousarray(target)
    B, N1, V = target.shape
    N = N1 - 1
    tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, N)
    parents = np.ascontiguousarray(parents, dtype=np.int32).reshape(B, N)
    out_tok = np.empty((B, N + 1), dtype=np.int32)
    out_n = np.empty(B, dtype=np.int32)
    path = np.empty((B, N), dtype=np.int32)
    am = sm = ti = None
    if diagnostics and temperature > 0:
        am = np.full((B, N), np.nan)
        sm = np.zeros(B)
        ti = np.zeros((B, N + 1), dtype=ROW_INFO_DTYPE)
    rc = lib().oracle_verify_tree(_ptr(target), dtype_code(target), _ptr(tokens), _ptr(parents), B, N,
                                  V, float(temperature), int(top_k), float(top_p),
                                  int(seed) & 0xFFFFFFFFFFFFFFFF, int(seq_base), _ptr(out_tok),
                                  _ptr(out_n), _ptr(path), _ptr(am), _ptr(sm), _ptr(ti))
    if rc:
        raise ValueError(f"oracle_verify_tree failed ({rc})")
    res = {"tokens": out_tok, "num_accepted": out_n, "path": path}
    if am is not None:
        res.update(accept_margin=am, sample_margin=sm, target_info=ti)
    return res


def verify_ragged(target, draft, tokens, draft_lens, temperature, top_k=0, top_p=1.0, seed=0,
                  point=False):
    """Per-sequence draft lengths: sequence b verifies only its first
    draft_lens[b] drafted tokens (0 <= draft_lens[b] <= K), against target rows
    0..draft_lens[b] (the bonus token comes from row draft_lens[b]); the rows past
    them are not part of the problem.  Each sequence is the plain verification
    of its own prefix of the padded [B, K+1, V] / [B, K, V] / [B, K] inputs,
    with its own global sequence index in the random stream.  Outputs are
    padded with -1 to K+1.  Also returns the per-position acceptance
    counters: tested[k] = sequences whose accept test at position k ran,
    accepted[k] = sequences that accepted position k."""
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    lens = np.asarray(draft_lens, dtype=np.int64).reshape(B)
    if (lens < 0).any() or (lens > K).any():
        raise ValueError("draft_lens out of [0, K]")
    out_tok = np.full((B, K + 1), -1, dtype=np.int32)
    out_n = np.zeros(B, dtype=np.int32)
    tested = np.zeros(K, dtype=np.int64)
    accepted = np.zeros(K, dtype=np.int64)
    for b in range(B):
        kb = int(lens[b])
        t = target[b:b + 1, :kb + 1]
        tk = np.ascontiguousarray(tokens[b:b + 1, :kb])
        if point:
            r = verify_point(t, tk, temperature, top_k, top_p, seed, seq_base=b, diagnostics=False)
        elif temperature == 0:
            r = verify_greedy(t, tk)
        else:
            d = None if kb == 0 else draft[b:b + 1, :kb]
            r = verify(t, d, tk, temperature, top_k, top_p, seed, seq_base=b, diagnostics=False)
        n = int(r["num_accepted"][0])
        out_tok[b, :kb + 1] = r["tokens"][0]
        out_n[b] = n
        tested[:min(n + 1, kb)] += 1
        accepted[:n] += 1
    return {"tokens": out_tok, "num_accepted": out_n, "tested": tested, "accepted": accepted}


def verify_greedy(target, tokens):
    target = np.ascontiguousarray(target)
    B, K1, V = target.shape
    K = K1 - 1
    tokens = np.ascontiguousarray(tokens, dtype=np.int32).reshape(B, K)
    out_tok = np.empty((B, K + 1), dtype=np.int32)
    out_n = np.empty(B, dtype=np.int32)
    rc = lib().oracle_verify_greedy(_ptr(target), dtype_code(target), _ptr(tokens), B, K, V,
                                    _ptr(out_tok), _ptr(out_n))
    if rc:
        raise ValueError(f"oracle_verify_greedy failed ({rc})")
    return {"tokens": out_tok, "num_accepted": out_n}


# ---------------------------------------------------------------------------
# Greedy verification from the target's last hidden states (the unembedding
# product computed here, in float64): "FlashMap: Flow Map Speculative
# Decoding and the Mathematical Elimination of Suffix Decay", section 3
# (logits of position k are the hidden state times the unembedding matrix
# transposed), with the greedy rule of "DFlash", section 4 (accept while the
# draft equals the target argmax, then emit the target's token).
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (uint16)."""
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def lm_head_logits(hidden_bits: np.ndarray, w_bits: np.ndarray, chunk: int = 8192) -> np.ndarray:
    """Logits [R, V] = hidden [R, H] @ W^T, W [V, H], both bf16 bit patterns,
    in float64 (a library matmul over vocabulary chunks)."""
    h = bf16_to_f64(hidden_bits)
    V = w_bits.shape[0]
    out = np.empty((h.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, chunk):
        out[:, v0:v0 + chunk] = h @ bf16_to_f64(w_bits[v0:v0 + chunk]).T
    return out


def lm_head_abs_sums(hidden_bits: np.ndarray, w_bits: np.ndarray, chunk: int = 8192) -> np.ndarray:
    """sum_h |hidden_h * W_vh| for every (row, token): the scale of the
    rounding error of any summation order of the dot product."""
    h = np.abs(bf16_to_f64(hidden_bits))
    V = w_bits.shape[0]
    out = np.empty((h.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, chunk):
        out[:, v0:v0 + chunk] = h @ np.abs(bf16_to_f64(w_bits[v0:v0 + chunk])).T
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 values rounded to the nearest bfloat16 value (8 significant
    bits), ties to the even significand, as bf16 bit patterns (uint16).  The
    inputs are finite and in bf16's normal range (or zero).  The logits of a
    bf16 LM head are its products rounded this way."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                  # x = m 2^e with 0.5 <= |m| < 1
    q = np.rint(m * 256.0)              # 8 significant bits, halves to even
    y = np.ldexp(q, e - 8)              # exact, and exact in float32 too
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def lm_head_logits_bf16(hidden_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """Logits [R, V] = hidden [R, H] @ W^T rounded to bf16 (bit patterns):
    the float64 product (exact for small-integer inputs) through round_bf16."""
    return round_bf16(lm_head_logits(hidden_bits, w_bits))


def verify_hidden(target_hidden, draft_hidden, w_bits, tokens, temperature, top_k=0, top_p=1.0, seed=0,
                  seq_base=0, diagnostics=True):
    """Verification from hidden states with a shared unembedding: the logits
    of target rows [B, K+1, H] and draft rows [B, K, H] are their products
    with w [V, H] rounded to bf16, then ``verify`` (greedy at temperature 0).
    Returns verify's dict plus ``target_logits`` and ``draft_logits``."""
    B, K1, H = target_hidden.shape
    K = K1 - 1
    V = w_bits.shape[0]
    tl = lm_head_logits_bf16(target_hidden.reshape(-1, H), w_bits).reshape(B, K1, V)
    dl = None
    if K > 0 and temperature > 0:
        dl = lm_head_logits_bf16(draft_hidden.reshape(-1, H), w_bits).reshape(B, K, V)
    r = verify(tl, dl, tokens, temperature, top_k, top_p, seed, seq_base=seq_base, diagnostics=diagnostics)
    r["target_logits"] = tl
    r["draft_logits"] = dl
    return r


def verify_greedy_logits64(logits: np.ndarray, tokens: np.ndarray):
    """Greedy verification on float64 logits [B, K+1, V]: g_k = argmax of row
    k (lowest index among equal maxima); accept while d_k == g_k, then emit
    g_j; pad with -1.  Returns tokens [B, K+1] and num_accepted [B]."""
    B, K1, V = logits.shape
    K = K1 - 1
    out = np.full((B, K + 1), -1, dtype=np.int32)
    num = np.zeros(B, dtype=np.int32)
    for b in range(B):
        g = [int(np.argmax(logits[b, k])) for k in range(K + 1)]  # first occurrence of the maximum
        j = K
        for k in range(K):
            if int(tokens[b, k]) != g[k]:
                j = k
                break
        out[b, :j] = tokens[b, :j]
        out[b, j] = g[j]
        num[b] = j
    return out, num
