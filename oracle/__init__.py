"""fp64 CPU oracle for the speculative-sampling verify step (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
never imports, links or calls it, and it imports nothing from the GPU library.

The arithmetic lives in ``spec_oracle.c`` (plain C, binary64, built with gcc
without fast-math).  What each function computes, and which passage of the
wikillm.com card "Accelerating Large Language Model Decoding with Speculative
Sampling" (arXiv 2302.01318) it follows, is stated in ``spec_oracle.h``.

Pins (tests that tie this oracle to the mathematics rather than to itself):
``tests/test_oracle_pins.py`` and ``tests/test_oracle_laws.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "spec_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_F32 = 0
DTYPE_BF16 = 1

_lib = None


def build(verbose: bool = False) -> str:
    """Compile spec_oracle.c into liboracle.so next to it (gcc, -O2, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    """Load liboracle.so, building it first only when it does not exist."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    L.oracle_softmax_row.argtypes = [vp, i32, i32, f64, vp, vp, vp]
    L.oracle_softmax_row.restype = i32
    L.oracle_accept.argtypes = [f64, f64, f64, vp]
    L.oracle_accept.restype = i32
    L.oracle_residual_weights.argtypes = [vp, vp, i32, vp]
    L.oracle_residual_weights.restype = i32
    L.oracle_inverse_cdf.argtypes = [vp, i32, f64, vp]
    L.oracle_inverse_cdf.restype = i32
    L.oracle_verify_dists.argtypes = [vp, vp, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp]
    L.oracle_verify_dists.restype = i32
    L.oracle_verify.argtypes = [vp, vp, i32, i32, i32, i32, f64, vp, vp,
                                vp, vp, vp, vp, vp, vp, vp, vp, vp, i32]
    L.oracle_verify.restype = i32
    L.oracle_final_draw.argtypes = [vp, vp, i32, i32, i32, i32, f64, vp, vp, vp, vp, vp, i32]
    L.oracle_final_draw.restype = i32
    L.oracle_argmax_row.argtypes = [vp, i32, i32, vp]
    L.oracle_argmax_row.restype = i32
    L.oracle_greedy_verify.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32]
    L.oracle_greedy_verify.restype = i32
    L.oracle_sample_rows.argtypes = [vp, i32, i64, i32, f64, vp, vp, vp, i32]
    L.oracle_sample_rows.restype = i32
    L.oracle_filter_threshold.argtypes = [vp, i32, i32, f64, i32, f64, vp]
    L.oracle_filter_threshold.restype = i32
    L.oracle_verify_filtered.argtypes = [vp, vp, i32, i32, i32, i32, f64, i32, f64, vp, vp, vp, vp,
                                         vp, vp, vp, vp, vp, vp, vp, vp, vp, i32]
    L.oracle_verify_filtered.restype = i32
    _lib = L
    return L


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _logits(a: np.ndarray) -> tuple[np.ndarray, int]:
    """Accept float32 logits, or bf16 logits given as their raw uint16 bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, DTYPE_F32
    if a.dtype == np.uint16:
        return a, DTYPE_BF16
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {a.dtype}")


def softmax_row(row: np.ndarray, T: float):
    """Return (prob[V] float64, M, S) or None when the row defines no distribution."""
    row, dt = _logits(row)
    V = row.shape[-1]
    prob = np.empty(V, np.float64)
    M = ctypes.c_double()
    S = ctypes.c_double()
    rc = lib().oracle_softmax_row(_ptr(row), dt, V, float(T), _ptr(prob),
                                  ctypes.byref(M), ctypes.byref(S))
    if rc != 0:
        return None
    return prob, M.value, S.value


def accept(q: float, p: float, u: float) -> tuple[bool, float]:
    d = ctypes.c_double()
    r = lib().oracle_accept(float(q), float(p), float(u), ctypes.byref(d))
    return bool(r), d.value


def residual_weights(q: np.ndarray, p: np.ndarray) -> tuple[np.ndarray, bool]:
    q = np.ascontiguousarray(q, np.float64)
    p = np.ascontiguousarray(p, np.float64)
    w = np.empty_like(q)
    fell_back = lib().oracle_residual_weights(_ptr(q), _ptr(p), q.shape[0], _ptr(w))
    return w, bool(fell_back)


def inverse_cdf(w: np.ndarray, u: float) -> tuple[int, float]:
    w = np.ascontiguousarray(w, np.float64)
    d = ctypes.c_double()
    x = lib().oracle_inverse_cdf(_ptr(w), w.shape[0], float(u), ctypes.byref(d))
    return int(x), d.value


def verify_dists(q: np.ndarray, p: np.ndarray, tokens: np.ndarray, uniforms: np.ndarray) -> dict:
    """Steps 3-4 of the verify on known distributions q [K+1][V], p [K][V] for
    N runs: tokens [N][K] int32, uniforms [N][K+1] float32."""
    q = np.ascontiguousarray(q, np.float64)
    p = np.ascontiguousarray(p, np.float64)
    K, V = p.shape
    assert q.shape == (K + 1, V)
    tokens = np.ascontiguousarray(tokens, np.int32)
    uniforms = np.ascontiguousarray(uniforms, np.float32)
    N = tokens.shape[0]
    assert tokens.shape == (N, K) and uniforms.shape == (N, K + 1)
    out = dict(
        num_accepted=np.empty(N, np.int32),
        out_tokens=np.empty((N, K + 1), np.int32),
        accept_dist=np.empty((N, K), np.float64),
        draw_dist=np.empty(N, np.float64),
        draw_kind=np.empty(N, np.int32),
    )
    rc = lib().oracle_verify_dists(_ptr(q), _ptr(p), K, V, N, _ptr(tokens), _ptr(uniforms),
                                   _ptr(out["num_accepted"]), _ptr(out["out_tokens"]),
                                   _ptr(out["accept_dist"]), _ptr(out["draw_dist"]),
                                   _ptr(out["draw_kind"]))
    if rc != 0:
        raise ValueError(f"oracle_verify_dists failed ({rc})")
    return out


def verify(target: np.ndarray, draft: np.ndarray, tokens: np.ndarray, uniforms: np.ndarray,
           T: float, nthreads: int = 0) -> dict:
    """Full verify from logits.  target [B][K+1][V], draft [B][K][V] as float32
    or bf16 bits (uint16); tokens [B][K] int32; uniforms [B][K+1] float32."""
    target, dt = _logits(target)
    draft, dt2 = _logits(draft)
    assert dt == dt2
    B, K1, V = target.shape
    K = K1 - 1
    assert draft.shape == (B, K, V)
    tokens = np.ascontiguousarray(tokens, np.int32)
    uniforms = np.ascontiguousarray(uniforms, np.float32)
    assert tokens.shape == (B, K) and uniforms.shape == (B, K + 1)
    out = dict(
        target_stats=np.empty((B, K + 1, 2), np.float64),
        draft_stats=np.empty((B, K, 2), np.float64),
        num_accepted=np.empty(B, np.int32),
        out_tokens=np.empty((B, K + 1), np.int32),
        num_emitted=np.empty(B, np.int32),
        probs=np.empty((B, K, 2), np.float64),
        accept_dist=np.empty((B, K), np.float64),
        draw_dist=np.empty(B, np.float64),
        draw_kind=np.empty(B, np.int32),
    )
    rc = lib().oracle_verify(_ptr(target), _ptr(draft), dt, B, K, V, float(T),
                             _ptr(tokens), _ptr(uniforms),
                             _ptr(out["target_stats"]), _ptr(out["draft_stats"]),
                             _ptr(out["num_accepted"]), _ptr(out["out_tokens"]),
                             _ptr(out["num_emitted"]), _ptr(out["probs"]),
                             _ptr(out["accept_dist"]), _ptr(out["draw_dist"]),
                             _ptr(out["draw_kind"]), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_verify failed ({rc})")
    return out


def final_draw(target: np.ndarray, draft: np.ndarray, uniforms: np.ndarray,
               num_accepted: np.ndarray, T: float, nthreads: int = 0) -> dict:
    """Residual/bonus draw alone for caller-supplied accepted counts."""
    target, dt = _logits(target)
    draft, _ = _logits(draft)
    B, K1, V = target.shape
    K = K1 - 1
    uniforms = np.ascontiguousarray(uniforms, np.float32)
    n = np.ascontiguousarray(num_accepted, np.int32)
    out = dict(token=np.empty(B, np.int32), draw_dist=np.empty(B, np.float64),
               draw_kind=np.empty(B, np.int32))
    rc = lib().oracle_final_draw(_ptr(target), _ptr(draft), dt, B, K, V, float(T),
                                 _ptr(uniforms), _ptr(n), _ptr(out["token"]),
                                 _ptr(out["draw_dist"]), _ptr(out["draw_kind"]), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_final_draw failed ({rc})")
    return out


def argmax_row(row: np.ndarray) -> int | None:
    """First index of the row's maximum, or None when the row defines no
    distribution (a NaN, or a maximum that is not finite)."""
    row, dt = _logits(np.ascontiguousarray(row))
    idx = np.zeros(1, np.int32)
    rc = lib().oracle_argmax_row(_ptr(row), dt, int(row.shape[-1]), _ptr(idx))
    return None if rc != 0 else int(idx[0])


def greedy_verify(target: np.ndarray, tokens: np.ndarray, nthreads: int = 0) -> dict:
    """Greedy verify: target [B][K+1][V] (float32 or bf16 bits), tokens [B][K]."""
    target, dt = _logits(target)
    B, K1, V = target.shape
    K = K1 - 1
    tokens = np.ascontiguousarray(tokens, np.int32)
    assert tokens.shape == (B, K)
    out = dict(argmax=np.empty((B, K1), np.int32), num_accepted=np.empty(B, np.int32),
               out_tokens=np.empty((B, K1), np.int32), num_emitted=np.empty(B, np.int32))
    rc = lib().oracle_greedy_verify(_ptr(target), dt, B, K, V, _ptr(tokens), _ptr(out["argmax"]),
                                    _ptr(out["num_accepted"]), _ptr(out["out_tokens"]),
                                    _ptr(out["num_emitted"]), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_greedy_verify failed ({rc})")
    return out


def sample_rows(logits: np.ndarray, uniforms: np.ndarray, T: float, nthreads: int = 0) -> dict:
    """Draw one token from softmax(row / T) for every row of logits [..., V]
    with the matching uniform (inverse CDF in ascending token id)."""
    logits, dt = _logits(logits)
    V = logits.shape[-1]
    R = int(np.prod(logits.shape[:-1]))
    u = np.ascontiguousarray(uniforms, np.float32).reshape(-1)
    assert u.size == R
    out = dict(tokens=np.empty(R, np.int32), dist=np.empty(R, np.float64))
    rc = lib().oracle_sample_rows(_ptr(logits), dt, R, V, float(T), _ptr(u), _ptr(out["tokens"]),
                                  _ptr(out["dist"]), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_sample_rows failed ({rc})")
    shape = logits.shape[:-1]
    return dict(tokens=out["tokens"].reshape(shape), dist=out["dist"].reshape(shape))


def filter_threshold(row: np.ndarray, T: float, top_k: int = 0, top_p: float = 1.0):
    """Logit threshold of the decoding transforms on one row (-inf: nothing
    removed), or None when the row defines no distribution."""
    row, dt = _logits(np.ascontiguousarray(row))
    t = np.zeros(1, np.float64)
    rc = lib().oracle_filter_threshold(_ptr(row), dt, int(row.shape[-1]), float(T), int(top_k),
                                       float(top_p), _ptr(t))
    return None if rc != 0 else float(t[0])


def verify_filtered(target: np.ndarray, draft: np.ndarray, tokens: np.ndarray,
                    uniforms: np.ndarray, T: float, top_k: int = 0, top_p: float = 1.0,
                    nthreads: int = 0) -> dict:
    """verify() on the rows after temperature, top-k and nucleus."""
    target, dt = _logits(target)
    draft, dt2 = _logits(draft)
    assert dt == dt2
    B, K1, V = target.shape
    K = K1 - 1
    tokens = np.ascontiguousarray(tokens, np.int32)
    uniforms = np.ascontiguousarray(uniforms, np.float32)
    out = dict(
        target_thr=np.empty((B, K + 1), np.float64), draft_thr=np.empty((B, K), np.float64),
        target_stats=np.empty((B, K + 1, 2), np.float64), draft_stats=np.empty((B, K, 2), np.float64),
        num_accepted=np.empty(B, np.int32), out_tokens=np.empty((B, K + 1), np.int32),
        num_emitted=np.empty(B, np.int32), probs=np.empty((B, K, 2), np.float64),
        accept_dist=np.empty((B, K), np.float64), draw_dist=np.empty(B, np.float64),
        draw_kind=np.empty(B, np.int32))
    rc = lib().oracle_verify_filtered(
        _ptr(target), _ptr(draft), dt, B, K, V, float(T), int(top_k), float(top_p), _ptr(tokens),
        _ptr(uniforms), _ptr(out["target_thr"]), _ptr(out["draft_thr"]), _ptr(out["target_stats"]),
        _ptr(out["draft_stats"]), _ptr(out["num_accepted"]), _ptr(out["out_tokens"]),
        _ptr(out["num_emitted"]), _ptr(out["probs"]), _ptr(out["accept_dist"]),
        _ptr(out["draw_dist"]), _ptr(out["draw_kind"]), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_verify_filtered failed ({rc})")
    return out
