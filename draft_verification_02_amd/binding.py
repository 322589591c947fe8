"""Thin Python binding of libspecverify.so (argument marshalling only).

Every step of the verification runs in the library's HIP kernels; this module
checks shapes and dtypes of torch tensors, passes device pointers and the
current HIP stream through ctypes, and raises on a non-zero status.  It raises
ImportError-style RuntimeError when the library has not been built: there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

from ._build import LIB

SPEC_DTYPE_F32 = 0
SPEC_DTYPE_BF16 = 1

ROW_FILTERED = 0x1
ROW_EXACT_PATH = 0x2

SPEC_E_SCRATCH = 5
NOALLOC_SCRATCH_BYTES = 32 << 20

# Layout of spec_row_stats_t (32 bytes), for viewing a stats tensor from numpy.
ROW_STATS_FIELDS = [("max_logit", "<f4"), ("thresh", "<f4"), ("n_kept", "<i4"),
                    ("flags", "<i4"), ("z_kept", "<f8"), ("prob_at_token", "<f8")]
ROW_STATS_BYTES = 32

EXPORTS = ["spec_verify", "spec_verify_noalloc", "spec_verify_ragged", "spec_verify_point", "spec_verify_tree", "spec_verify_greedy",
           "spec_verify_greedy_hidden", "spec_lm_head_logits", "spec_verify_hidden",
           "spec_verify_stats",
           "spec_rng_uniforms", "spec_profile_events", "spec_status_string", "spec_release_workspace"]

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


def load(path: str = LIB) -> ctypes.CDLL:
    """Load the HIP library (fails loudly when it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library {path} is not built; run __graft_entry__.build() "
            "(hipcc --offload-arch=gfx950) first")
    L = ctypes.CDLL(path)
    vp, i32, f32, u64, f64p = (ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint64,
                               ctypes.c_void_p)
    L.spec_verify.argtypes = [vp, vp, vp, i32, i32, i32, f32, i32, f32, u64, vp, vp, vp, i32, i32]
    L.spec_verify.restype = i32
    L.spec_verify_noalloc.argtypes = [vp, vp, vp, i32, i32, i32, f32, i32, f32, u64, vp, vp, vp, i32, i32]
    L.spec_verify_noalloc.restype = i32
    L.spec_verify_ragged.argtypes = [vp, vp, vp, vp, i32, i32, i32, f32, i32, f32, u64, vp, vp, vp, vp,
                                     vp, i32, i32]
    L.spec_verify_ragged.restype = i32
    L.spec_verify_point.argtypes = [vp, vp, i32, i32, i32, f32, i32, f32, u64, vp, vp, vp, i32]
    L.spec_verify_point.restype = i32
    L.spec_verify_tree.argtypes = [vp, vp, vp, i32, i32, i32, f32, i32, f32, u64, vp, vp, vp, vp, i32]
    L.spec_verify_tree.restype = i32
    L.spec_verify_greedy_hidden.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, vp]
    L.spec_verify_greedy_hidden.restype = i32
    L.spec_lm_head_logits.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    L.spec_lm_head_logits.restype = i32
    L.spec_verify_hidden.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, f32, u64, vp, vp, vp]
    L.spec_verify_hidden.restype = i32
    L.spec_verify_greedy.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, i32]
    L.spec_verify_greedy.restype = i32
    L.spec_verify_stats.argtypes = [vp, vp, vp, i32, i32, i32, f32, i32, f32, u64, vp, vp, vp,
                                    i32, i32, vp, vp]
    L.spec_verify_stats.restype = i32
    L.spec_rng_uniforms.argtypes = [u64, i32, i32, f64p, f64p, vp]
    L.spec_rng_uniforms.restype = i32
    L.spec_profile_events.argtypes = [vp, vp]
    L.spec_profile_events.restype = i32
    L.spec_status_string.argtypes = [i32]
    L.spec_status_string.restype = ctypes.c_char_p
    L.spec_release_workspace.argtypes = []
    L.spec_release_workspace.restype = None
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != 0:
        msg = load().spec_status_string(rc).decode()
        raise SpecVerifyError(f"spec_verify status {rc}: {msg}", rc)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SPEC_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return SPEC_DTYPE_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _outputs(B, K, device, out_tokens, out_num):
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=device)
    if out_num is None:
        out_num = torch.empty((B,), dtype=torch.int32, device=device)
    assert out_tokens.dtype == torch.int32 and out_tokens.numel() == B * (K + 1)
    assert out_num.dtype == torch.int32 and out_num.numel() == B
    _dev(out_tokens, "out_tokens")
    _dev(out_num, "out_num_accepted")
    return out_tokens, out_num


def _shapes(target, draft, tokens, need_draft=True):
    _dev(target, "target_logits")
    B, K1, V = target.shape
    K = K1 - 1
    if K > 0:
        if need_draft:
            assert draft is not None and tuple(draft.shape) == (B, K, V), "draft must be [B, K, V]"
            _dev(draft, "draft_logits")
        assert tokens is not None and tokens.dtype == torch.int32 and tuple(tokens.shape) == (B, K)
        _dev(tokens, "draft_tokens")
    return B, K, V


def spec_verify(target: torch.Tensor, draft: torch.Tensor | None, tokens: torch.Tensor | None,
                temperature: float, top_k: int = 0, top_p: float = 1.0, seed: int = 0,
                out_tokens=None, out_num_accepted=None, stream=None):
    """Verify a batch: target [B, K+1, V], draft [B, K, V] (bf16 or f32),
    tokens [B, K] int32.  Returns (out_tokens [B, K+1], out_num_accepted [B])."""
    B, K, V = _shapes(target, draft, tokens, need_draft=temperature > 0)
    out_tokens, out_num = _outputs(B, K, target.device, out_tokens, out_num_accepted)
    use_draft = draft is not None and K > 0 and temperature > 0
    ddt = _dtype_code(draft) if use_draft else SPEC_DTYPE_F32
    rc = load().spec_verify(_ptr(target), _ptr(draft) if use_draft else None,
                            _ptr(tokens) if K > 0 else None, B, K, V, float(temperature),
                            int(top_k), float(top_p), int(seed) & 0xFFFFFFFFFFFFFFFF,
                            _ptr(out_tokens), _ptr(out_num), _stream_handle(stream),
                            _dtype_code(target), ddt)
    _check(rc)
    return out_tokens, out_num


def spec_verify_noalloc(target: torch.Tensor, draft: torch.Tensor | None, tokens: torch.Tensor | None,
                        temperature: float, top_k: int, top_p: float, seed: int,
                        out_tokens: torch.Tensor, out_num_accepted: torch.Tensor, stream=None):
    """spec_verify through the allocation-free entry point: the library's
    scratch is its fixed static device array, and the outputs must be given
    (this wrapper allocates nothing either).  Raises SpecVerifyError with
    status SPEC_E_SCRATCH when the problem does not fit."""
    B, K, V = _shapes(target, draft, tokens, need_draft=temperature > 0)
    assert out_tokens is not None and out_num_accepted is not None, "outputs must be given"
    out_tokens, out_num = _outputs(B, K, target.device, out_tokens, out_num_accepted)
    use_draft = draft is not None and K > 0 and temperature > 0
    ddt = _dtype_code(draft) if use_draft else SPEC_DTYPE_F32
    rc = load().spec_verify_noalloc(_ptr(target), _ptr(draft) if use_draft else None,
                                    _ptr(tokens) if K > 0 else None, B, K, V, float(temperature),
                                    int(top_k), float(top_p), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                    _ptr(out_tokens), _ptr(out_num), _stream_handle(stream),
                                    _dtype_code(target), ddt)
    _check(rc)
    return out_tokens, out_num


def spec_verify_ragged(target: torch.Tensor, draft: torch.Tensor | None, tokens: torch.Tensor | None,
                       lens: torch.Tensor, temperature: float, top_k: int = 0, top_p: float = 1.0,
                       seed: int = 0, counters: bool = True, out_tokens=None, out_num_accepted=None,
                       stream=None):
    """Per-sequence draft lengths lens [B] int32 (device).  Returns
    (out_tokens [B, K+1], out_num_accepted [B], tested [K], accepted [K]);
    the counters are None when ``counters`` is False."""
    B, K, V = _shapes(target, draft, tokens, need_draft=temperature > 0)
    assert lens.dtype == torch.int32 and tuple(lens.shape) == (B,)
    _dev(lens, "draft_lens")
    out_tokens, out_num = _outputs(B, K, target.device, out_tokens, out_num_accepted)
    tested = accepted = None
    if counters:
        tested = torch.empty((K,), dtype=torch.int32, device=target.device)
        accepted = torch.empty((K,), dtype=torch.int32, device=target.device)
    use_draft = draft is not None and K > 0 and temperature > 0
    ddt = _dtype_code(draft) if use_draft else SPEC_DTYPE_F32
    rc = load().spec_verify_ragged(_ptr(target), _ptr(draft) if use_draft else None,
                                   _ptr(tokens) if K > 0 else None, _ptr(lens), B, K, V,
                                   float(temperature), int(top_k), float(top_p),
                                   int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out_tokens), _ptr(out_num),
                                   _ptr(tested), _ptr(accepted), _stream_handle(stream),
                                   _dtype_code(target), ddt)
    _check(rc)
    return out_tokens, out_num, tested, accepted


def spec_verify_point(target: torch.Tensor, tokens: torch.Tensor | None, temperature: float,
                      top_k: int = 0, top_p: float = 1.0, seed: int = 0, out_tokens=None,
                      out_num_accepted=None, stream=None):
    """Verify point-mass drafts (no draft logits): target [B, K+1, V],
    tokens [B, K] int32.  Returns (out_tokens [B, K+1], out_num_accepted [B])."""
    B, K, V = _shapes(target, None, tokens, need_draft=False)
    out_tokens, out_num = _outputs(B, K, target.device, out_tokens, out_num_accepted)
    rc = load().spec_verify_point(_ptr(target), _ptr(tokens) if K > 0 else None, B, K, V,
                                  float(temperature), int(top_k), float(top_p),
                                  int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out_tokens), _ptr(out_num),
                                  _stream_handle(stream), _dtype_code(target))
    _check(rc)
    return out_tokens, out_num


def spec_verify_tree(target: torch.Tensor, tokens: torch.Tensor | None, parents: torch.Tensor | None,
                     temperature: float, top_k: int = 0, top_p: float = 1.0, seed: int = 0,
                     path: bool = True, stream=None, out_tokens=None, out_num_accepted=None,
                     out_path=None):
    """Verify a token tree per sequence: target [B, N+1, V] (row 0 the root,
    row i+1 after node i), tokens [B, N] and parents [B, N] int32 (-1 = root,
    else an index below the node's own).  Returns (out_tokens [B, N+1],
    out_num_accepted [B], out_path [B, N] or None)."""
    _dev(target, "target_logits")
    B, N1, V = target.shape
    N = N1 - 1
    if N > 0:
        for t, name in ((tokens, "node_tokens"), (parents, "parents")):
            assert t is not None and t.dtype == torch.int32 and tuple(t.shape) == (B, N), name
            _dev(t, name)
    out_tokens, out_num = _outputs(B, N, target.device, out_tokens, out_num_accepted)
    if out_path is None and path:
        out_path = torch.empty((B, N), dtype=torch.int32, device=target.device)
    if out_path is not None:
        assert out_path.dtype == torch.int32 and out_path.numel() == B * N
        _dev(out_path, "out_path")
    rc = load().spec_verify_tree(_ptr(target), _ptr(tokens) if N > 0 else None,
                                 _ptr(parents) if N > 0 else None, B, N, V, float(temperature), int(top_k),
                                 float(top_p), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out_tokens),
                                 _ptr(out_num), _ptr(out_path) if N > 0 else None, _stream_handle(stream),
                                 _dtype_code(target))
    _check(rc)
    return out_tokens, out_num, out_path


def spec_verify_greedy_hidden(hidden: torch.Tensor, w_unembed: torch.Tensor, tokens: torch.Tensor | None,
                              out_tokens=None, out_num_accepted=None, stream=None):
    """Greedy verification from hidden states: hidden [B, K+1, H] bf16, the
    unembedding matrix w_unembed [V, H] bf16, tokens [B, K] int32.  Returns
    (out_tokens [B, K+1], out_num_accepted [B])."""
    _dev(hidden, "hidden")
    _dev(w_unembed, "w_unembed")
    if hidden.dtype != torch.bfloat16 or w_unembed.dtype != torch.bfloat16:
        raise TypeError("hidden states and unembedding matrix must be bfloat16")
    B, K1, H = hidden.shape
    K = K1 - 1
    V, H2 = w_unembed.shape
    assert H2 == H, "hidden size mismatch"
    if K > 0:
        assert tokens is not None and tokens.dtype == torch.int32 and tuple(tokens.shape) == (B, K)
        _dev(tokens, "draft_tokens")
    out_tokens, out_num = _outputs(B, K, hidden.device, out_tokens, out_num_accepted)
    rc = load().spec_verify_greedy_hidden(_ptr(hidden), _ptr(w_unembed), _ptr(tokens) if K > 0 else None, B, K, V,
                                          H, _ptr(out_tokens), _ptr(out_num), _stream_handle(stream))
    _check(rc)
    return out_tokens, out_num


def spec_lm_head_logits(hidden: torch.Tensor, w_unembed: torch.Tensor, out=None, stream=None) -> torch.Tensor:
    """bf16 logits [R, V] of hidden [R, H] (bf16) and w_unembed [V, H] (bf16)."""
    _dev(hidden, "hidden")
    _dev(w_unembed, "w_unembed")
    assert hidden.dtype == torch.bfloat16 and w_unembed.dtype == torch.bfloat16
    R, H = hidden.shape
    V, H2 = w_unembed.shape
    assert H == H2, "hidden and w_unembed disagree on H"
    if out is None:
        out = torch.empty((R, V), dtype=torch.bfloat16, device=hidden.device)
    assert out.dtype == torch.bfloat16 and out.numel() == R * V
    _dev(out, "out_logits")
    _check(load().spec_lm_head_logits(_ptr(hidden), _ptr(w_unembed), R, V, H, _ptr(out), _stream_handle(stream)))
    return out


def spec_verify_hidden(target_hidden: torch.Tensor, draft_hidden: torch.Tensor | None, w_unembed: torch.Tensor,
                       tokens: torch.Tensor | None, temperature: float, top_k: int = 0, top_p: float = 1.0,
                       seed: int = 0, out_tokens=None, out_num_accepted=None, stream=None):
    """Verification from hidden states with a shared unembedding: target_hidden
    [B, K+1, H], draft_hidden [B, K, H], w_unembed [V, H] (all bf16), tokens
    [B, K] int32.  Returns (out_tokens [B, K+1], out_num_accepted [B])."""
    _dev(target_hidden, "target_hidden")
    _dev(w_unembed, "w_unembed")
    B, K1, H = target_hidden.shape
    K = K1 - 1
    V = w_unembed.shape[0]
    assert target_hidden.dtype == torch.bfloat16 and w_unembed.dtype == torch.bfloat16
    assert tuple(w_unembed.shape) == (V, H)
    use_draft = K > 0 and temperature > 0
    if use_draft:
        assert draft_hidden is not None and tuple(draft_hidden.shape) == (B, K, H)
        assert draft_hidden.dtype == torch.bfloat16
        _dev(draft_hidden, "draft_hidden")
    if K > 0:
        assert tokens is not None and tokens.dtype == torch.int32 and tuple(tokens.shape) == (B, K)
        _dev(tokens, "draft_tokens")
    out_tokens, out_num = _outputs(B, K, target_hidden.device, out_tokens, out_num_accepted)
    rc = load().spec_verify_hidden(_ptr(target_hidden), _ptr(draft_hidden) if use_draft else None, _ptr(w_unembed),
                                   _ptr(tokens) if K > 0 else None, B, K, V, H, float(temperature), int(top_k),
                                   float(top_p), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(out_tokens), _ptr(out_num),
                                   _stream_handle(stream))
    _check(rc)
    return out_tokens, out_num


def spec_verify_greedy(target: torch.Tensor, tokens: torch.Tensor | None, out_tokens=None,
                       out_num_accepted=None, stream=None):
    _dev(target, "target_logits")
    B, K1, V = target.shape
    K = K1 - 1
    if K > 0:
        assert tokens is not None and tokens.dtype == torch.int32 and tuple(tokens.shape) == (B, K)
        _dev(tokens, "draft_tokens")
    out_tokens, out_num = _outputs(B, K, target.device, out_tokens, out_num_accepted)
    rc = load().spec_verify_greedy(_ptr(target), _ptr(tokens) if K > 0 else None, B, K, V,
                                   _ptr(out_tokens), _ptr(out_num), _stream_handle(stream),
                                   _dtype_code(target))
    _check(rc)
    return out_tokens, out_num


def spec_verify_stats(target, draft, tokens, temperature, top_k=0, top_p=1.0, seed=0,
                      stream=None):
    """spec_verify plus per-row intermediates.  Returns
    (out_tokens, out_num_accepted, target_stats uint8[B, K+1, 32], draft_stats uint8[B, K, 32])."""
    B, K, V = _shapes(target, draft, tokens)
    out_tokens, out_num = _outputs(B, K, target.device, None, None)
    ts = torch.empty((B, K + 1, ROW_STATS_BYTES), dtype=torch.uint8, device=target.device)
    ds = torch.empty((B, max(K, 0), ROW_STATS_BYTES), dtype=torch.uint8, device=target.device)
    ddt = _dtype_code(draft) if (draft is not None and K > 0) else SPEC_DTYPE_F32
    rc = load().spec_verify_stats(_ptr(target), _ptr(draft) if K > 0 else None,
                                  _ptr(tokens) if K > 0 else None, B, K, V, float(temperature),
                                  int(top_k), float(top_p), int(seed) & 0xFFFFFFFFFFFFFFFF,
                                  _ptr(out_tokens), _ptr(out_num), _stream_handle(stream),
                                  _dtype_code(target), ddt, _ptr(ts),
                                  _ptr(ds) if K > 0 else None)
    _check(rc)
    return out_tokens, out_num, ts, ds


def rng_uniforms(seed: int, B: int, K: int, device="cuda", stream=None):
    ua = torch.empty((B, K), dtype=torch.float64, device=device)
    us = torch.empty((B, K + 1), dtype=torch.float64, device=device)
    rc = load().spec_rng_uniforms(int(seed) & 0xFFFFFFFFFFFFFFFF, B, K,
                                  _ptr(ua) if K > 0 else None, _ptr(us), _stream_handle(stream))
    _check(rc)
    return ua, us


def profile_events(before, after) -> None:
    """Arm the measurement hook with two hipEvent_t handles (ints) or clear it."""
    _check(load().spec_profile_events(ctypes.c_void_p(before) if before else None,
                                      ctypes.c_void_p(after) if after else None))


def release_workspace() -> None:
    load().spec_release_workspace()
