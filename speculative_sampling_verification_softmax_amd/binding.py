"""ctypes binding of libspec_softmax.so (the C ABI in include/spec_softmax.h).

Argument marshalling only: every step of the verify runs in the HIP kernels.
torch tensors supply device memory (``data_ptr()``) and the stream
(``torch.cuda.current_stream().cuda_stream``); nothing is computed in Python.
There is no CPU fallback: if the library is missing or no GPU is present the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspec_softmax.so")

SPEC_DTYPE_F32 = 0
SPEC_DTYPE_BF16 = 1
SPEC_OK = 0
SPEC_MAX_K = 64
SPEC_MAX_V = 1 << 20
SPEC_MAX_ROWS = 4194303
SPEC_NOALLOC_SCRATCH_BYTES = 8 << 20
SPEC_ERR_UNSUPPORTED = 2

EXPORTS = ("spec_softmax_stats", "spec_verify", "spec_residual_sample", "spec_status_string",
           "spec_verify_step_workspace_size", "spec_verify_step", "spec_verify_step_noalloc",
           "spec_greedy_verify", "spec_sample", "spec_filter", "spec_verify_sample")

_lib = None


class SpecError(RuntimeError):
    pass


def load(path: str = LIB_PATH):
    """Load the HIP library (no build, no fallback) and declare signatures."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path)
    return _lib


def open_library(path: str):
    """A library with this header's entry points (the library itself, or its
    measurement build) loaded from `path`, its signatures declared; load()
    keeps the one the wrappers call."""
    if not os.path.exists(path):
        raise SpecError(f"{path} is missing: build it with "
                        "`python -m speculative_sampling_verification_softmax_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.spec_softmax_stats.argtypes = [vp, vp, i32, i32, i32, i32, f32, vp, vp, vp]
    L.spec_softmax_stats.restype = i32
    L.spec_verify.argtypes = [vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, vp, vp]
    L.spec_verify.restype = i32
    L.spec_residual_sample.argtypes = [vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, f32,
                                       vp, vp, vp]
    L.spec_residual_sample.restype = i32
    L.spec_verify_step_workspace_size.argtypes = [i32, i32, i32, i32]
    L.spec_verify_step_workspace_size.restype = ctypes.c_size_t
    L.spec_verify_step.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, f32, vp, vp, vp, vp, vp,
                                   vp, vp, ctypes.c_size_t, vp]
    L.spec_verify_step.restype = i32
    L.spec_verify_step_noalloc.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, f32, vp, vp, vp,
                                           vp, vp, vp, vp]
    L.spec_verify_step_noalloc.restype = i32
    L.spec_greedy_verify.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, vp, vp, vp]
    L.spec_greedy_verify.restype = i32
    L.spec_sample.argtypes = [vp, i32, i32, i32, f32, vp, vp, vp, vp]
    L.spec_sample.restype = i32
    L.spec_verify_sample.argtypes = [vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, f32, vp, vp, vp,
                                     vp, vp]
    L.spec_verify_sample.restype = i32
    L.spec_filter.argtypes = [vp, i32, i32, i32, f32, i32, f32, vp, vp, vp, vp]
    L.spec_filter.restype = i32
    L.spec_status_string.argtypes = [i32]
    L.spec_status_string.restype = ctypes.c_char_p
    return L


def status_string(rc: int) -> str:
    return load().spec_status_string(int(rc)).decode()


def _check(rc: int, what: str):
    if rc != SPEC_OK:
        raise SpecError(f"{what}: {status_string(rc)}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SPEC_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return SPEC_DTYPE_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _shapes(target: torch.Tensor, draft: torch.Tensor):
    if target.dim() != 3 or draft.dim() != 3:
        raise ValueError("target must be [B][K+1][V] and draft [B][K][V]")
    B, K1, V = target.shape
    K = K1 - 1
    if tuple(draft.shape) != (B, K, V):
        raise ValueError(f"draft must be {(B, K, V)}, got {tuple(draft.shape)}")
    if draft.dtype != target.dtype:
        raise TypeError("target and draft must share a dtype")
    return B, K, V


def softmax_stats(target: torch.Tensor, draft: torch.Tensor, T: float,
                  target_stats: Optional[torch.Tensor] = None,
                  draft_stats: Optional[torch.Tensor] = None, stream=None):
    """spec_softmax_stats: returns (target_stats [B][K+1][2], draft_stats [B][K][2])."""
    B, K, V = _shapes(target, draft)
    dev = target.device
    if target_stats is None:
        target_stats = torch.empty((B, K + 1, 2), dtype=torch.float32, device=dev)
    if draft_stats is None:
        draft_stats = torch.empty((B, K, 2), dtype=torch.float32, device=dev)
    rc = load().spec_softmax_stats(
        _dev(target, "target"), _dev(draft, "draft"), _dtype_code(target), B, K, V, float(T),
        _dev(target_stats, "target_stats", torch.float32, (B, K + 1, 2)),
        _dev(draft_stats, "draft_stats", torch.float32, (B, K, 2)), _stream(stream))
    _check(rc, "spec_softmax_stats")
    return target_stats, draft_stats


def verify(target, draft, tokens, uniforms, target_stats, draft_stats, T: float,
           num_accepted=None, out_tokens=None, probs=True, stream=None):
    """spec_verify: returns (num_accepted [B], out_tokens [B][K+1], probs [B][K][2] or None)."""
    B, K, V = _shapes(target, draft)
    dev = target.device
    if num_accepted is None:
        num_accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if probs is True:
        probs = torch.empty((B, K, 2), dtype=torch.float32, device=dev)
    elif probs is False:
        probs = None
    pp = None if probs is None else _dev(probs, "probs", torch.float32, (B, K, 2))
    rc = load().spec_verify(
        _dev(target, "target"), _dev(draft, "draft"), _dtype_code(target),
        _dev(tokens, "tokens", torch.int32, (B, K)),
        _dev(uniforms, "uniforms", torch.float32, (B, K + 1)),
        _dev(target_stats, "target_stats", torch.float32, (B, K + 1, 2)),
        _dev(draft_stats, "draft_stats", torch.float32, (B, K, 2)),
        B, K, V, float(T),
        _dev(num_accepted, "num_accepted", torch.int32, (B,)),
        _dev(out_tokens, "out_tokens", torch.int32, (B, K + 1)), pp, _stream(stream))
    _check(rc, "spec_verify")
    return num_accepted, out_tokens, probs


def residual_sample(target, draft, uniforms, target_stats, draft_stats, num_accepted, T: float,
                    out_tokens, num_emitted=True, stream=None):
    """spec_residual_sample: fills out_tokens[b][num_accepted[b]]; returns num_emitted."""
    B, K, V = _shapes(target, draft)
    if num_emitted is True:
        num_emitted = torch.empty(B, dtype=torch.int32, device=target.device)
    elif num_emitted is False:
        num_emitted = None
    ne = None if num_emitted is None else _dev(num_emitted, "num_emitted", torch.int32, (B,))
    rc = load().spec_residual_sample(
        _dev(target, "target"), _dev(draft, "draft"), _dtype_code(target),
        _dev(uniforms, "uniforms", torch.float32, (B, K + 1)),
        _dev(target_stats, "target_stats", torch.float32, (B, K + 1, 2)),
        _dev(draft_stats, "draft_stats", torch.float32, (B, K, 2)),
        _dev(num_accepted, "num_accepted", torch.int32, (B,)),
        B, K, V, float(T), _dev(out_tokens, "out_tokens", torch.int32, (B, K + 1)), ne,
        _stream(stream))
    _check(rc, "spec_residual_sample")
    return num_emitted


def verify_all(target, draft, tokens, uniforms, T: float, stream=None) -> dict:
    """The whole verify (stats, accept scan, final draw) on one stream."""
    ts, ds = softmax_stats(target, draft, T, stream=stream)
    n, out, probs = verify(target, draft, tokens, uniforms, ts, ds, T, stream=stream)
    ne = residual_sample(target, draft, uniforms, ts, ds, n, T, out, stream=stream)
    return dict(target_stats=ts, draft_stats=ds, num_accepted=n, out_tokens=out, probs=probs,
                num_emitted=ne)


def verify_sample(target, draft, tokens, uniforms, target_stats, draft_stats, T: float,
                  num_accepted=None, out_tokens=None, probs=True, num_emitted=True,
                  stream=None):
    """spec_verify_sample: the accept scan and the final draw in one launch.
    Returns (num_accepted, out_tokens, probs or None, num_emitted or None)."""
    B, K, V = _shapes(target, draft)
    dev = target.device
    if num_accepted is None:
        num_accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if probs is True:
        probs = torch.empty((B, K, 2), dtype=torch.float32, device=dev)
    elif probs is False:
        probs = None
    if num_emitted is True:
        num_emitted = torch.empty(B, dtype=torch.int32, device=dev)
    elif num_emitted is False:
        num_emitted = None
    pp = None if probs is None else _dev(probs, "probs", torch.float32, (B, K, 2))
    ne = None if num_emitted is None else _dev(num_emitted, "num_emitted", torch.int32, (B,))
    rc = load().spec_verify_sample(
        _dev(target, "target"), _dev(draft, "draft"), _dtype_code(target),
        _dev(tokens, "tokens", torch.int32, (B, K)),
        _dev(uniforms, "uniforms", torch.float32, (B, K + 1)),
        _dev(target_stats, "target_stats", torch.float32, (B, K + 1, 2)),
        _dev(draft_stats, "draft_stats", torch.float32, (B, K, 2)),
        B, K, V, float(T),
        _dev(num_accepted, "num_accepted", torch.int32, (B,)),
        _dev(out_tokens, "out_tokens", torch.int32, (B, K + 1)), pp, ne, _stream(stream))
    _check(rc, "spec_verify_sample")
    return num_accepted, out_tokens, probs, num_emitted


def verify_two_call(target, draft, tokens, uniforms, T: float, stream=None) -> dict:
    """The whole verify as two calls: stats, then accept scan + final draw."""
    ts, ds = softmax_stats(target, draft, T, stream=stream)
    n, out, probs, ne = verify_sample(target, draft, tokens, uniforms, ts, ds, T, stream=stream)
    return dict(target_stats=ts, draft_stats=ds, num_accepted=n, out_tokens=out, probs=probs,
                num_emitted=ne)


def workspace_size(B: int, K: int, V: int, dtype: torch.dtype) -> int:
    """Bytes of workspace spec_verify_step needs for this shape."""
    code = SPEC_DTYPE_F32 if dtype == torch.float32 else SPEC_DTYPE_BF16
    n = load().spec_verify_step_workspace_size(B, K, V, code)
    if n == 0:
        raise ValueError(f"invalid shape B={B} K={K} V={V}")
    return int(n)


def new_workspace(B: int, K: int, V: int, dtype: torch.dtype, device) -> torch.Tensor:
    """A zeroed workspace for spec_verify_step (reusable: each completed call
    leaves its counters zero)."""
    return torch.zeros(workspace_size(B, K, V, dtype), dtype=torch.uint8, device=device)


def _step_outputs(B, K, dev, target_stats, draft_stats, num_accepted, out_tokens, probs,
                  num_emitted):
    if target_stats is None:
        target_stats = torch.empty((B, K + 1, 2), dtype=torch.float32, device=dev)
    if draft_stats is None:
        draft_stats = torch.empty((B, K, 2), dtype=torch.float32, device=dev)
    if num_accepted is None:
        num_accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    if probs is True:
        probs = torch.empty((B, K, 2), dtype=torch.float32, device=dev)
    elif probs is False:
        probs = None
    if num_emitted is True:
        num_emitted = torch.empty(B, dtype=torch.int32, device=dev)
    elif num_emitted is False:
        num_emitted = None
    return target_stats, draft_stats, num_accepted, out_tokens, probs, num_emitted


def verify_step(target, draft, tokens, uniforms, T: float, workspace: torch.Tensor,
                target_stats=None, draft_stats=None, num_accepted=None, out_tokens=None,
                probs=True, num_emitted=True, stream=None) -> dict:
    """spec_verify_step: the whole verify in two launches that split rows and
    sequences over several workgroups when the batch is small."""
    B, K, V = _shapes(target, draft)
    ts, ds, n, out, pr, ne = _step_outputs(B, K, target.device, target_stats, draft_stats,
                                           num_accepted, out_tokens, probs, num_emitted)
    if workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    rc = load().spec_verify_step(
        _dev(target, "target"), _dev(draft, "draft"), _dtype_code(target),
        _dev(tokens, "tokens", torch.int32, (B, K)),
        _dev(uniforms, "uniforms", torch.float32, (B, K + 1)), B, K, V, float(T),
        _dev(ts, "target_stats", torch.float32, (B, K + 1, 2)),
        _dev(ds, "draft_stats", torch.float32, (B, K, 2)),
        _dev(n, "num_accepted", torch.int32, (B,)),
        _dev(out, "out_tokens", torch.int32, (B, K + 1)),
        None if pr is None else _dev(pr, "probs", torch.float32, (B, K, 2)),
        None if ne is None else _dev(ne, "num_emitted", torch.int32, (B,)),
        _dev(workspace, "workspace"), workspace.numel(), _stream(stream))
    _check(rc, "spec_verify_step")
    return dict(target_stats=ts, draft_stats=ds, num_accepted=n, out_tokens=out, probs=pr,
                num_emitted=ne)


def verify_step_noalloc(target, draft, tokens, uniforms, T: float, target_stats=None,
                        draft_stats=None, num_accepted=None, out_tokens=None, probs=True,
                        num_emitted=True, stream=None) -> dict:
    """spec_verify_step_noalloc: spec_verify_step on the library's own static
    scratch (no workspace; calls that overlap on one GPU race)."""
    B, K, V = _shapes(target, draft)
    ts, ds, n, out, pr, ne = _step_outputs(B, K, target.device, target_stats, draft_stats,
                                           num_accepted, out_tokens, probs, num_emitted)
    rc = load().spec_verify_step_noalloc(
        _dev(target, "target"), _dev(draft, "draft"), _dtype_code(target),
        _dev(tokens, "tokens", torch.int32, (B, K)),
        _dev(uniforms, "uniforms", torch.float32, (B, K + 1)), B, K, V, float(T),
        _dev(ts, "target_stats", torch.float32, (B, K + 1, 2)),
        _dev(ds, "draft_stats", torch.float32, (B, K, 2)),
        _dev(n, "num_accepted", torch.int32, (B,)),
        _dev(out, "out_tokens", torch.int32, (B, K + 1)),
        None if pr is None else _dev(pr, "probs", torch.float32, (B, K, 2)),
        None if ne is None else _dev(ne, "num_emitted", torch.int32, (B,)), _stream(stream))
    _check(rc, "spec_verify_step_noalloc")
    return dict(target_stats=ts, draft_stats=ds, num_accepted=n, out_tokens=out, probs=pr,
                num_emitted=ne)


def greedy_verify(target, tokens, target_argmax=None, num_accepted=None, out_tokens=None,
                  num_emitted=True, stream=None) -> dict:
    """spec_greedy_verify: target [B][K+1][V] logits, tokens [B][K] int32."""
    if target.dim() != 3:
        raise ValueError("target must be [B][K+1][V]")
    B, K1, V = target.shape
    K = K1 - 1
    dev = target.device
    if target_argmax is None:
        target_argmax = torch.empty((B, K1), dtype=torch.int32, device=dev)
    if num_accepted is None:
        num_accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty((B, K1), dtype=torch.int32, device=dev)
    if num_emitted is True:
        num_emitted = torch.empty(B, dtype=torch.int32, device=dev)
    elif num_emitted is False:
        num_emitted = None
    rc = load().spec_greedy_verify(
        _dev(target, "target"), _dtype_code(target), _dev(tokens, "tokens", torch.int32, (B, K)),
        B, K, V, _dev(target_argmax, "target_argmax", torch.int32, (B, K1)),
        _dev(num_accepted, "num_accepted", torch.int32, (B,)),
        _dev(out_tokens, "out_tokens", torch.int32, (B, K1)),
        None if num_emitted is None else _dev(num_emitted, "num_emitted", torch.int32, (B,)),
        _stream(stream))
    _check(rc, "spec_greedy_verify")
    return dict(argmax=target_argmax, num_accepted=num_accepted, out_tokens=out_tokens,
                num_emitted=num_emitted)


def sample(logits, uniforms, T: float, row_stats=None, tokens=None, stream=None) -> dict:
    """spec_sample: one token per row of logits [..., V] from softmax(row / T)."""
    V = logits.shape[-1]
    R = logits.numel() // V
    dev = logits.device
    if row_stats is None:
        row_stats = torch.empty((R, 2), dtype=torch.float32, device=dev)
    if tokens is None:
        tokens = torch.empty(R, dtype=torch.int32, device=dev)
    if uniforms.numel() != R:
        raise ValueError(f"uniforms must hold {R} values")
    rc = load().spec_sample(_dev(logits, "logits"), _dtype_code(logits), R, V, float(T),
                            _dev(uniforms, "uniforms", torch.float32),
                            _dev(row_stats, "row_stats", torch.float32, (R, 2)),
                            _dev(tokens, "tokens", torch.int32, (R,)), _stream(stream))
    _check(rc, "spec_sample")
    shape = tuple(logits.shape[:-1])
    return dict(tokens=tokens.view(shape), row_stats=row_stats.view(shape + (2,)))


def filter_rows(logits, T: float, top_k: int = 0, top_p: float = 1.0, out=None,
                thresholds=None, inplace: bool = False, write_rows: bool = True,
                stats=None, stream=None) -> dict:
    """spec_filter: top-k / nucleus thresholds of each row of logits [..., V]
    and the rows with the removed tokens set to -inf (written into `out`, a
    new tensor by default, or into logits itself when inplace; not written
    at all when write_rows is False).  stats: True for a new [..., 2] tensor
    of the filtered rows' {m, s}, or a float32 tensor to fill; None: none."""
    V = logits.shape[-1]
    R = logits.numel() // V
    dev = logits.device
    shape = tuple(logits.shape[:-1])
    if thresholds is None:
        thresholds = torch.empty(R, dtype=torch.float32, device=dev)
    if stats is True:
        stats = torch.empty(shape + (2,), dtype=torch.float32, device=dev)
    if not write_rows:
        out = None
    elif inplace:
        out = logits
    elif out is None:
        out = torch.empty_like(logits)
    out_ptr = None if out is None else _dev(out, "out", logits.dtype, tuple(logits.shape))
    st_ptr = None if stats is None else _dev(stats, "stats", torch.float32, shape + (2,))
    rc = load().spec_filter(_dev(logits, "logits"), _dtype_code(logits), R, V, float(T),
                            int(top_k), float(top_p),
                            _dev(thresholds, "thresholds", torch.float32, (R,)), st_ptr, out_ptr,
                            _stream(stream))
    _check(rc, "spec_filter")
    return dict(filtered=out, thresholds=thresholds.view(shape), stats=stats)
