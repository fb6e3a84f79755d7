"""Plain CPU oracle for block-hybrid attention (fp64).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``; nothing in the product package
imports it.  The arithmetic lives in ``hybrid_oracle.c`` (plain loops, fp64,
one function per operation, each citing the passage of the pages it follows);
this module only compiles it with gcc and marshals numpy arrays.

Every function takes float arrays of any precision and upcasts them exactly to
fp64, so the oracle sees bit-for-bit the same values as the GPU path.  Results
are fp64 and unrounded.

Layouts: active-block tensors ``[n_req, blk, H, d]``; state
``[n_slots, H, d, d]`` with ``S[slot, h, f, c]`` (``f`` = feature of phi(k),
``c`` = value dimension); prompts / prefixes packed ``[total, H, d]`` with
``cu_seqlens[n_req + 1]``.

Parity: every function here is pinned by ``tests/test_oracle_pins.py``
(library routines, closed forms, invariants, brute force and a hand-derived
worked example); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hybrid_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I32 = ctypes.POINTER(ctypes.c_int32)
_I64 = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile ``hybrid_oracle.c`` into ``liboracle.so`` (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
            lib.oracle_num_threads.restype = ctypes.c_int
            lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
            lib.oracle_set_num_threads.restype = None
            i = ctypes.c_int
            lib.oracle_step.argtypes = [_D, _D, _D, _D, _I32, _I32, _D] + [i] * 5 + [ctypes.c_double, i]
            lib.oracle_commit.argtypes = [_D, _D, _D, _I32, _I32] + [i] * 6
            lib.oracle_prefill.argtypes = [_D, _D, _I64, _D, _I32] + [i] * 5
            for fn in (lib.oracle_step_recompute, lib.oracle_step_norm_recompute):
                fn.argtypes = [_D, _D, _D, _D, _D, _I64, _I32, _D] + [i] * 4 + [ctypes.c_double, i]
            lib.oracle_exact_step.argtypes = [_D, _D, _D, _D, _D, _I64, _I32, _D] + [i] * 4 + [ctypes.c_double]
            lib.oracle_step_norm.argtypes = [_D, _D, _D, _D, _D, _I32, _I32, _D] + [i] * 5 + [ctypes.c_double, i]
            lib.oracle_znorm_commit.argtypes = [_D, _D, _I32, _I32] + [i] * 6
            lib.oracle_znorm_prefill.argtypes = [_D, _I64, _D, _I32] + [i] * 5
            for fn in (lib.oracle_step, lib.oracle_commit, lib.oracle_prefill,
                       lib.oracle_step_recompute, lib.oracle_exact_step, lib.oracle_step_norm,
                       lib.oracle_znorm_commit, lib.oracle_znorm_prefill, lib.oracle_step_norm_recompute):
                fn.restype = None
            _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    a = _np(a)
    return np.ascontiguousarray(a, dtype=np.float64)


def _np(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor (bf16 is upcast exactly through fp32)
        import torch
        t = a.detach().cpu()
        if t.dtype == torch.bfloat16 or t.dtype == torch.float16:
            t = t.float()
        return t.numpy()
    return np.asarray(a)


def _i32(a, n) -> np.ndarray | None:
    if a is None:
        return None
    a = np.ascontiguousarray(_np(a), dtype=np.int32)
    assert a.shape == (n,)
    return a


def _p(a, typ):
    return None if a is None else a.ctypes.data_as(typ)


# The feature maps phi (hybrid_oracle.c): "relu" max(x, 0), the pages' worked
# example; "elu1" ELU(x) + 1 (x + 1 for x > 0, e^x otherwise).
PHI = {"relu": 0, "elu1": 1}


def _map(phi: str) -> int:
    if phi not in PHI:
        raise ValueError(f"unknown feature map {phi!r} (one of {sorted(PHI)})")
    return PHI[phi]


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """OpenMP threads of the following calls (the units of a call are spread
    over them; nothing inside a unit changes)."""
    _load().oracle_set_num_threads(int(n))


def step(q, k, v, S, slots=None, blk_lens=None, scale=None, phi="relu") -> np.ndarray:
    """O = Softmax(scale Q_a K_a^T) V_a + phi(Q_a) S per (request, head).

    Rows at or past ``blk_lens[r]`` are returned as zeros (never written)."""
    q, k, v, S = _f64(q), _f64(k), _f64(v), _f64(S)
    n_req, blk, H, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    n_slots = S.shape[0]
    assert S.shape == (n_slots, H, d, d)
    slots = _i32(slots if slots is not None else np.arange(n_req), n_req)
    bl = _i32(blk_lens, n_req)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros_like(q)
    _load().oracle_step(_p(q, _D), _p(k, _D), _p(v, _D), _p(S, _D), _p(slots, _I32),
                        _p(bl, _I32), _p(out, _D), n_req, n_slots, H, blk, d, float(scale), _map(phi))
    return out


def commit(k, v, S, slots=None, blk_lens=None, phi="relu") -> np.ndarray:
    """Returns S + phi(K)^T V for each request's slot (a new fp64 array)."""
    k, v = _f64(k), _f64(v)
    S = np.array(_f64(S), copy=True)
    n_req, blk, H, d = k.shape
    n_slots = S.shape[0]
    assert S.shape == (n_slots, H, d, d) and v.shape == k.shape
    slots = _i32(slots if slots is not None else np.arange(n_req), n_req)
    bl = _i32(blk_lens, n_req)
    _load().oracle_commit(_p(k, _D), _p(v, _D), _p(S, _D), _p(slots, _I32), _p(bl, _I32),
                          n_req, n_slots, H, blk, d, _map(phi))
    return S


def prefill(k, v, cu_seqlens, S=None, slots=None, n_slots=None, phi="relu") -> np.ndarray:
    """Returns the state with each request's slot overwritten by
    sum_t phi(k_t)^T v_t over its prompt (packed [total, H, d])."""
    k, v = _f64(k), _f64(v)
    total, H, d = k.shape
    cu = np.ascontiguousarray(_np(cu_seqlens), dtype=np.int64)
    n_req = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == total and np.all(np.diff(cu) >= 0)
    if S is None:
        S = np.zeros((n_slots if n_slots is not None else n_req, H, d, d))
    S = np.array(_f64(S), copy=True)
    slots = _i32(slots if slots is not None else np.arange(n_req), n_req)
    _load().oracle_prefill(_p(k, _D), _p(v, _D), _p(cu, _I64), _p(S, _D), _p(slots, _I32),
                           n_req, S.shape[0], H, d, _map(phi))
    return S


def _prefix_form(fn, q, k, v, kp, vp, cu_seqlens, blk_lens, scale, *extra):
    q, k, v, kp, vp = _f64(q), _f64(k), _f64(v), _f64(kp), _f64(vp)
    n_req, blk, H, d = q.shape
    cu = np.ascontiguousarray(_np(cu_seqlens), dtype=np.int64)
    assert cu.shape == (n_req + 1,) and kp.shape[1:] == (H, d) and vp.shape == kp.shape
    bl = _i32(blk_lens, n_req)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros_like(q)
    fn(_p(q, _D), _p(k, _D), _p(v, _D), _p(kp, _D), _p(vp, _D), _p(cu, _I64), _p(bl, _I32),
       _p(out, _D), n_req, H, blk, d, float(scale), *extra)
    return out


def step_recompute(q, k, v, kp, vp, cu_seqlens, blk_lens=None, scale=None, phi="relu") -> np.ndarray:
    """The formula's own form: softmax part + (phi(Q_a) phi(K_p)^T) V_p from the
    retained prefix keys/values (packed [total, H, d])."""
    return _prefix_form(_load().oracle_step_recompute, q, k, v, kp, vp, cu_seqlens, blk_lens, scale, _map(phi))


def exact_step(q, k, v, kp, vp, cu_seqlens, blk_lens=None, scale=None) -> np.ndarray:
    """Exact softmax over [prefix; active block]: the step the method replaces."""
    return _prefix_form(_load().oracle_exact_step, q, k, v, kp, vp, cu_seqlens, blk_lens, scale)


# ---------------------------------------------------------------------------
# Normalised variant: the block's softmax scores and the prefix's linear scores
# share one denominator, which needs z = sum phi(k_p) ([n_slots, H, d]) next to
# S (a reading of the pages' LoLCATs-based retrofit; see hybrid_oracle.c).


def step_norm(q, k, v, S, z, slots=None, blk_lens=None, scale=None, phi="relu") -> np.ndarray:
    """O_i = (sum_j exp(l_ij) v_j + phi(q_i) S) / (sum_j exp(l_ij) + phi(q_i) . z)
    per (request, head); rows at or past ``blk_lens[r]`` are zeros."""
    q, k, v, S, z = _f64(q), _f64(k), _f64(v), _f64(S), _f64(z)
    n_req, blk, H, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    n_slots = S.shape[0]
    assert S.shape == (n_slots, H, d, d) and z.shape == (n_slots, H, d)
    slots = _i32(slots if slots is not None else np.arange(n_req), n_req)
    bl = _i32(blk_lens, n_req)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros_like(q)
    _load().oracle_step_norm(_p(q, _D), _p(k, _D), _p(v, _D), _p(S, _D), _p(z, _D), _p(slots, _I32),
                             _p(bl, _I32), _p(out, _D), n_req, n_slots, H, blk, d, float(scale), _map(phi))
    return out


def znorm_commit(k, z, slots=None, blk_lens=None, phi="relu") -> np.ndarray:
    """Returns z + sum_j phi(k_j) over each request's valid block rows."""
    k = _f64(k)
    z = np.array(_f64(z), copy=True)
    n_req, blk, H, d = k.shape
    n_slots = z.shape[0]
    assert z.shape == (n_slots, H, d)
    slots = _i32(slots if slots is not None else np.arange(n_req), n_req)
    bl = _i32(blk_lens, n_req)
    _load().oracle_znorm_commit(_p(k, _D), _p(z, _D), _p(slots, _I32), _p(bl, _I32), n_req, n_slots, H, blk, d,
                                _map(phi))
    return z


def znorm_prefill(k, cu_seqlens, z=None, slots=None, n_slots=None, phi="relu") -> np.ndarray:
    """Returns z with each request's slot overwritten by sum_t phi(k_t) over its
    prompt (packed [total, H, d])."""
    k = _f64(k)
    total, H, d = k.shape
    cu = np.ascontiguousarray(_np(cu_seqlens), dtype=np.int64)
    n_req = cu.shape[0] - 1
    assert cu[0] == 0 and cu[-1] == total and np.all(np.diff(cu) >= 0)
    if z is None:
        z = np.zeros((n_slots if n_slots is not None else n_req, H, d))
    z = np.array(_f64(z), copy=True)
    slots = _i32(slots if slots is not None else np.arange(n_req), n_req)
    _load().oracle_znorm_prefill(_p(k, _D), _p(cu, _I64), _p(z, _D), _p(slots, _I32), n_req, z.shape[0], H, d,
                                 _map(phi))
    return z


def step_norm_recompute(q, k, v, kp, vp, cu_seqlens, blk_lens=None, scale=None, phi="relu") -> np.ndarray:
    """The normalised output with one weight per key: exp(l_ij) for block keys
    and phi(q_i) . phi(k_t) for the retained prefix tokens (packed [total, H, d])."""
    return _prefix_form(_load().oracle_step_norm_recompute, q, k, v, kp, vp, cu_seqlens, blk_lens, scale,
                        _map(phi))
