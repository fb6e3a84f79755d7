"""ctypes binding of libhybrid_attn.so: argument marshalling only.

The functions carry the C ABI's names and take torch tensors on the GPU; they
check shapes and dtypes, pass raw device pointers and the current HIP stream,
and raise ``HybridAttnError`` on any non-OK status.  All computation happens
in the library's HIP kernels; there is no fallback of any kind, and a missing
library is an error.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

import torch

from .build import LIB as LIB_PATH

HA_OK, HA_ERR_INVALID_ARG, HA_ERR_UNSUPPORTED, HA_ERR_HIP = 0, 1, 2, 3
HA_F32, HA_BF16 = 0, 1
HA_PHI_RELU, HA_PHI_ELU1 = 0, 1
FEATURE_MAPS = {"relu": HA_PHI_RELU, "elu1": HA_PHI_ELU1}
MAX_BLK = 256
EXACT_MAX_BLK = 128

_lock = threading.Lock()
_lib = None


class HybridAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed with status {status}: {message}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the shared library; raises if it is not built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() or "
                               "python -m block_hybrid_linear_amd.build")
        lib = ctypes.CDLL(path)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        lib.hybrid_attn_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, ctypes.c_int, vp]
        lib.hybrid_state_commit.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp]
        lib.hybrid_attn_step_commit.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                                ctypes.c_int, vp]
        lib.hybrid_state_prefill.argtypes = [vp, vp, vp, i64, i64, vp, vp, i32, i32, i32, i32, i32, vp, sz,
                                             ctypes.c_int, vp]
        lib.hybrid_state_prefill_noalloc.argtypes = [vp, vp, vp, i64, i64, vp, vp, i32, i32, i32, i32, i32,
                                                     ctypes.c_int, vp]
        lib.hybrid_state_prefill_workspace_bytes.argtypes = [i32, i32, i32, i64, i64, i32]
        lib.hybrid_state_prefill_workspace_bytes.restype = sz
        lib.hybrid_exact_step.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, vp, i32, i32, i32, i32, f32, i32, vp, sz,
                                          ctypes.c_int, vp]
        lib.hybrid_exact_step_workspace_bytes.argtypes = [i32, i32, i32, i32]
        lib.hybrid_exact_step_workspace_bytes.restype = sz
        lib.hybrid_attn_step_norm.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                              ctypes.c_int, vp]
        lib.hybrid_attn_step_commit_norm.argtypes = lib.hybrid_attn_step_norm.argtypes
        lib.hybrid_state_commit_norm.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int, vp]
        lib.hybrid_state_prefill_norm.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, i32, i32, i32, i32, i32, vp,
                                                  sz, ctypes.c_int, vp]
        lib.hybrid_attn_step_phi.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32,
                                             ctypes.c_int, ctypes.c_int, vp]
        lib.hybrid_attn_step_commit_phi.argtypes = lib.hybrid_attn_step_phi.argtypes
        lib.hybrid_state_commit_phi.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.c_int,
                                                ctypes.c_int, vp]
        lib.hybrid_state_prefill_phi.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp, i32, i32, i32, i32, i32, vp, sz,
                                                 ctypes.c_int, ctypes.c_int, vp]
        for fn in (lib.hybrid_attn_step_phi, lib.hybrid_attn_step_commit_phi, lib.hybrid_state_commit_phi,
                   lib.hybrid_state_prefill_phi):
            fn.restype = ctypes.c_int
        for fn in (lib.hybrid_attn_step, lib.hybrid_state_commit, lib.hybrid_state_prefill, lib.hybrid_exact_step,
                   lib.hybrid_attn_step_commit, lib.hybrid_attn_step_norm, lib.hybrid_attn_step_commit_norm,
                   lib.hybrid_state_commit_norm, lib.hybrid_state_prefill_norm, lib.hybrid_state_prefill_noalloc):
            fn.restype = ctypes.c_int
        lib.hybrid_last_error.argtypes = []
        lib.hybrid_last_error.restype = ctypes.c_char_p
        lib.hybrid_abi_version.argtypes = []
        lib.hybrid_abi_version.restype = ctypes.c_int32
        _lib = lib
        return lib


def _check(fn: str, status: int) -> None:
    if status != HA_OK:
        msg = load_library().hybrid_last_error().decode(errors="replace")
        raise HybridAttnError(fn, status, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HA_BF16
    if t.dtype == torch.float32:
        return HA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _opt(t, name, dtype) -> int | None:
    return None if t is None else _dev(t, name, dtype)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _on_stream(stream):
    """Context in which tensors are allocated (and filled) on ``stream``, so
    that the caching allocator orders their reuse, and any fill kernel, with
    the library's kernels on that stream; a no-op for the current stream."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream))
    return torch.cuda.stream(stream)


def abi_version() -> int:
    return load_library().hybrid_abi_version()


def _step_args(q, k, v, state, slots, out, blk_lens, scale):
    n_req, blk, H, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if state.dim() != 4 or tuple(state.shape[1:]) != (H, d, d):
        raise ValueError(f"state must be [n_slots, {H}, {d}, {d}]")
    if slots.shape != (n_req,):
        raise ValueError("slots must be [n_req]")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if blk_lens is not None and blk_lens.shape != (n_req,):
        raise ValueError("blk_lens must be [n_req]")
    if scale is None:
        scale = d ** -0.5
    return (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(state, "state", torch.float32),
            _dev(slots, "slots", torch.int32), _dev(out, "out"), _opt(blk_lens, "blk_lens", torch.int32),
            n_req, state.shape[0], H, blk, d, float(scale), _dtype_code(q))


def hybrid_attn_step(q, k, v, state, slots, out=None, blk_lens=None, scale=None, stream=None):
    """out = Softmax(scale Q K^T) V + ReLU(Q) S[slots] for q/k/v [n_req, blk, H, d];
    state [n_slots, H, d, d] fp32 (each d x d block stores S transposed)."""
    if out is None:
        with _on_stream(stream):
            out = torch.zeros_like(q)
    args = _step_args(q, k, v, state, slots, out, blk_lens, scale)
    _check("hybrid_attn_step", load_library().hybrid_attn_step(*args, _stream(stream)))
    return out


def prepare_step(q, k, v, state, slots, out, blk_lens=None, scale=None, stream=None):
    """Validates and marshals once; returns a callable that enqueues the same
    step again (one ctypes call) -- for loops that re-run a step on buffers
    whose contents change but whose storage does not."""
    args = _step_args(q, k, v, state, slots, out, blk_lens, scale) + (_stream(stream),)
    fn = load_library().hybrid_attn_step

    def run():
        st = fn(*args)
        if st != HA_OK:
            _check("hybrid_attn_step", st)
    return run


def hybrid_attn_step_commit(q, k, v, state, slots, out=None, blk_lens=None, scale=None, stream=None):
    """The step from the current state (as hybrid_attn_step), then
    state[slots] += ReLU(K)^T V in the same pass: the last denoising step of a
    block fused with its commit.  Requests must use distinct slots."""
    if out is None:
        with _on_stream(stream):
            out = torch.zeros_like(q)
    args = _step_args(q, k, v, state, slots, out, blk_lens, scale)
    _check("hybrid_attn_step_commit", load_library().hybrid_attn_step_commit(*args, _stream(stream)))
    return out


def prepare_step_commit(q, k, v, state, slots, out, blk_lens=None, scale=None, stream=None):
    """Prepared form of hybrid_attn_step_commit (see prepare_step)."""
    args = _step_args(q, k, v, state, slots, out, blk_lens, scale) + (_stream(stream),)
    fn = load_library().hybrid_attn_step_commit

    def run():
        st = fn(*args)
        if st != HA_OK:
            _check("hybrid_attn_step_commit", st)
    return run


def _commit_args(k, v, state, slots, blk_lens):
    n_req, blk, H, d = k.shape
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k, v must share shape and dtype")
    if state.dim() != 4 or tuple(state.shape[1:]) != (H, d, d):
        raise ValueError(f"state must be [n_slots, {H}, {d}, {d}]")
    if slots.shape != (n_req,):
        raise ValueError("slots must be [n_req]")
    if blk_lens is not None and blk_lens.shape != (n_req,):
        raise ValueError("blk_lens must be [n_req]")
    return (_dev(k, "k"), _dev(v, "v"), _dev(state, "state", torch.float32), _dev(slots, "slots", torch.int32),
            _opt(blk_lens, "blk_lens", torch.int32), n_req, state.shape[0], H, blk, d, _dtype_code(k))


def hybrid_state_commit(k, v, state, slots, blk_lens=None, stream=None):
    """state[slots] += ReLU(K)^T V (stored transposed), in place."""
    args = _commit_args(k, v, state, slots, blk_lens)
    _check("hybrid_state_commit", load_library().hybrid_state_commit(*args, _stream(stream)))
    return state


def prepare_commit(k, v, state, slots, blk_lens=None, stream=None):
    """Prepared form of hybrid_state_commit (see prepare_step)."""
    args = _commit_args(k, v, state, slots, blk_lens) + (_stream(stream),)
    fn = load_library().hybrid_state_commit

    def run():
        st = fn(*args)
        if st != HA_OK:
            _check("hybrid_state_commit", st)
    return run


def hybrid_state_prefill_workspace_bytes(n_req, heads, d, total_tokens, max_len, chunk=256) -> int:
    return int(load_library().hybrid_state_prefill_workspace_bytes(n_req, heads, d, total_tokens, max_len, chunk))


def _prefill_args(k, v, cu_seqlens, state, slots, max_len, chunk, workspace, stream=None):
    total, H, d = k.shape
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k, v must share shape and dtype")
    n_req = cu_seqlens.shape[0] - 1
    if state.dim() != 4 or tuple(state.shape[1:]) != (H, d, d):
        raise ValueError(f"state must be [n_slots, {H}, {d}, {d}]")
    if slots.shape != (n_req,):
        raise ValueError("slots must be [n_req]")
    if max_len is None:
        max_len = 0     # only an upper bound; the kernels do not need it
    need = hybrid_state_prefill_workspace_bytes(n_req, H, d, total, max_len, chunk)
    if workspace is None:
        with _on_stream(stream):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
    args = (_dev(k, "k"), _dev(v, "v"), _dev(cu_seqlens, "cu_seqlens", torch.int64), total, max_len,
            _dev(state, "state", torch.float32), _dev(slots, "slots", torch.int32), n_req, state.shape[0], H, d,
            chunk, _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _dtype_code(k))
    return args, workspace


def hybrid_state_prefill(k, v, cu_seqlens, state, slots, max_len=None, chunk=256, workspace=None,
                         stream=None):
    """state[slots[r]] = sum over prompt r of ReLU(k_t)^T v_t (overwrite).

    k, v packed [total, H, d]; cu_seqlens int64 [n_req + 1] on the GPU.
    ``max_len`` (host int) is an optional upper bound of the prompt lengths.
    ``workspace`` is a GPU uint8 tensor of at least
    ``hybrid_state_prefill_workspace_bytes`` bytes (contents on entry do not
    matter); if omitted one is allocated through torch."""
    args, _ws = _prefill_args(k, v, cu_seqlens, state, slots, max_len, chunk, workspace, stream)
    _check("hybrid_state_prefill", load_library().hybrid_state_prefill(*args, _stream(stream)))
    return state


def prepare_prefill(k, v, cu_seqlens, state, slots, max_len=None, chunk=256, workspace=None, stream=None):
    """Prepared form of hybrid_state_prefill (see prepare_step); keeps its
    workspace alive."""
    args, ws = _prefill_args(k, v, cu_seqlens, state, slots, max_len, chunk, workspace, stream)
    args = args + (_stream(stream),)
    fn = load_library().hybrid_state_prefill

    def run():
        st = fn(*args)
        if st != HA_OK:
            _check("hybrid_state_prefill", st)
    run.workspace = ws
    return run


NOALLOC_SCRATCH_BYTES = 128 << 20


def hybrid_state_prefill_noalloc(k, v, cu_seqlens, state, slots, max_len=None, chunk=256, stream=None):
    """hybrid_state_prefill with the library's own device scratch as the
    workspace: nothing is allocated by the call (for graph capture and
    callers that cannot allocate).  Calls that overlap on one GPU race on
    that scratch."""
    total, H, d = k.shape
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k, v must share shape and dtype")
    n_req = cu_seqlens.shape[0] - 1
    if state.dim() != 4 or tuple(state.shape[1:]) != (H, d, d):
        raise ValueError(f"state must be [n_slots, {H}, {d}, {d}]")
    if slots.shape != (n_req,):
        raise ValueError("slots must be [n_req]")
    args = (_dev(k, "k"), _dev(v, "v"), _dev(cu_seqlens, "cu_seqlens", torch.int64), total,
            0 if max_len is None else max_len, _dev(state, "state", torch.float32), _dev(slots, "slots", torch.int32),
            n_req, state.shape[0], H, d, chunk, _dtype_code(k))
    _check("hybrid_state_prefill_noalloc", load_library().hybrid_state_prefill_noalloc(*args, _stream(stream)))
    return state


def hybrid_exact_step_workspace_bytes(n_req, heads, blk, d) -> int:
    return int(load_library().hybrid_exact_step_workspace_bytes(n_req, heads, blk, d))


def _exact_args(q, k, v, k_cache, v_cache, cu_prefix, out, blk_lens, scale, chunk, workspace, stream=None):
    n_req, blk, H, d = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if k_cache.dim() != 3 or tuple(k_cache.shape[1:]) != (H, d) or v_cache.shape != k_cache.shape:
        raise ValueError(f"k_cache, v_cache must be [total_prefix, {H}, {d}]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("the prefix cache must have the dtype of q")
    if cu_prefix.shape != (n_req + 1,):
        raise ValueError("cu_prefix must be [n_req + 1]")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if blk_lens is not None and blk_lens.shape != (n_req,):
        raise ValueError("blk_lens must be [n_req]")
    if scale is None:
        scale = d ** -0.5
    need = hybrid_exact_step_workspace_bytes(n_req, H, blk, d)
    if workspace is None:
        with _on_stream(stream):
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    total = k_cache.shape[0]
    args = (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(k_cache, "k_cache") if total else None,
            _dev(v_cache, "v_cache") if total else None, _dev(cu_prefix, "cu_prefix", torch.int64), total,
            _dev(out, "out"), _opt(blk_lens, "blk_lens", torch.int32), n_req, H, blk, d, float(scale), chunk,
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _dtype_code(q))
    return args, workspace


def hybrid_exact_step(q, k, v, k_cache, v_cache, cu_prefix, out=None, blk_lens=None, scale=None, chunk=256,
                      workspace=None, stream=None):
    """out = Softmax(scale Q [K_p; K]^T) [V_p; V]: exact attention of the active
    block q/k/v [n_req, blk, H, d] over its prefix (k_cache/v_cache packed
    [total_prefix, H, d], request r owns rows cu_prefix[r]..cu_prefix[r+1]-1)
    and itself -- the step block-hybrid attention replaces."""
    if out is None:
        with _on_stream(stream):
            out = torch.zeros_like(q)
    args, _ws = _exact_args(q, k, v, k_cache, v_cache, cu_prefix, out, blk_lens, scale, chunk, workspace, stream)
    _check("hybrid_exact_step", load_library().hybrid_exact_step(*args, _stream(stream)))
    return out


def prepare_exact_step(q, k, v, k_cache, v_cache, cu_prefix, out, blk_lens=None, scale=None, chunk=256,
                       workspace=None, stream=None):
    """Prepared form of hybrid_exact_step (see prepare_step); keeps its
    workspace alive."""
    args, ws = _exact_args(q, k, v, k_cache, v_cache, cu_prefix, out, blk_lens, scale, chunk, workspace, stream)
    args = args + (_stream(stream),)
    fn = load_library().hybrid_exact_step

    def run():
        st = fn(*args)
        if st != HA_OK:
            _check("hybrid_exact_step", st)
    run.workspace = ws
    return run


# ---------------------------------------------------------------------------
# Normalised variant: one denominator for the block's softmax scores and the
# prefix's linear scores, with z = sum phi(k) [n_slots, H, d] fp32 next to S.

def _check_z(z, state):
    n_slots, H, d = state.shape[0], state.shape[1], state.shape[2]
    if z.dim() != 3 or tuple(z.shape) != (n_slots, H, d):
        raise ValueError(f"z must be [{n_slots}, {H}, {d}]")
    return _dev(z, "z", torch.float32)


def _with_z(args, z, state, at):
    """Inserts z's pointer into a marshalled argument tuple at position `at`."""
    return args[:at] + (_check_z(z, state),) + args[at:]


def hybrid_attn_step_norm(q, k, v, state, z, slots, out=None, blk_lens=None, scale=None, stream=None):
    """out_i = (sum_j exp(l_ij) v_j + ReLU(q_i) S) / (sum_j exp(l_ij) + ReLU(q_i).z)
    for q/k/v [n_req, blk, H, d], state [n_slots, H, d, d], z [n_slots, H, d]."""
    if out is None:
        with _on_stream(stream):
            out = torch.zeros_like(q)
    args = _with_z(_step_args(q, k, v, state, slots, out, blk_lens, scale), z, state, 4)
    _check("hybrid_attn_step_norm", load_library().hybrid_attn_step_norm(*args, _stream(stream)))
    return out


def prepare_step_norm(q, k, v, state, z, slots, out, blk_lens=None, scale=None, stream=None):
    """Prepared form of hybrid_attn_step_norm (see prepare_step)."""
    args = _with_z(_step_args(q, k, v, state, slots, out, blk_lens, scale), z, state, 4) + (_stream(stream),)
    fn = load_library().hybrid_attn_step_norm

    def run():
        st = fn(*args)
        if st != HA_OK:
            _check("hybrid_attn_step_norm", st)
    return run


def hybrid_attn_step_commit_norm(q, k, v, state, z, slots, out=None, blk_lens=None, scale=None, stream=None):
    """hybrid_attn_step_norm from the current S and z, then S += ReLU(K)^T V and
    z += sum_j ReLU(k_j) in the same call.  Requests must use distinct slots."""
    if out is None:
        with _on_stream(stream):
            out = torch.zeros_like(q)
    args = _with_z(_step_args(q, k, v, state, slots, out, blk_lens, scale), z, state, 4)
    _check("hybrid_attn_step_commit_norm", load_library().hybrid_attn_step_commit_norm(*args, _stream(stream)))
    return out


def prepare_step_commit_norm(q, k, v, state, z, slots, out, blk_lens=None, scale=None, stream=None):
    """Prepared form of hybrid_attn_step_commit_norm (see prepare_step)."""
    args = _with_z(_step_args(q, k, v, state, slots, out, blk_lens, scale), z, state, 4) + (_stream(stream),)
    fn = load_library().hybrid_attn_step_commit_norm

    def run():
        st = fn(*args)
        if st != HA_OK:
            _check("hybrid_attn_step_commit_norm", st)
    return run


def hybrid_state_commit_norm(k, v, state, z, slots, blk_lens=None, stream=None):
    """state[slots] += ReLU(K)^T V and z[slots] += sum_j ReLU(k_j), in place."""
    args = _with_z(_commit_args(k, v, state, slots, blk_lens), z, state, 3)
    _check("hybrid_state_commit_norm", load_library().hybrid_state_commit_norm(*args, _stream(stream)))
    return state


def hybrid_state_prefill_norm(k, v, cu_seqlens, state, z, slots, max_len=None, chunk=256, workspace=None,
                              stream=None):
    """state[slots[r]] and z[slots[r]] overwritten by the sums over prompt r of
    ReLU(k_t)^T v_t and ReLU(k_t) (see hybrid_state_prefill)."""
    args, _ws = _prefill_args(k, v, cu_seqlens, state, slots, max_len, chunk, workspace, stream)
    args = _with_z(args, z, state, 6)
    _check("hybrid_state_prefill_norm", load_library().hybrid_state_prefill_norm(*args, _stream(stream)))
    return state


def prepare_prefill_norm(k, v, cu_seqlens, state, z, slots, max_len=None, chunk=256, workspace=None, stream=None):
    """Prepared form of hybrid_state_prefill_norm; keeps its workspace alive."""
    args, ws = _prefill_args(k, v, cu_seqlens, state, slots, max_len, chunk, workspace, stream)
    args = _with_z(args, z, state, 6) + (_stream(stream),)
    fn = load_library().hybrid_state_prefill_norm

    def run():
        st = fn(*args)
        if st != HA_OK:
            _check("hybrid_state_prefill_norm", st)
    run.workspace = ws
    return run


# ---------------------------------------------------------------------------
# The calls with the feature map as an argument ("relu" or "elu1"); z = None
# gives the plain sum, a z tensor [n_slots, H, d] the normalised variant.

def _phi_code(phi) -> int:
    if isinstance(phi, str):
        if phi not in FEATURE_MAPS:
            raise ValueError(f"unknown feature map {phi!r} (one of {sorted(FEATURE_MAPS)})")
        return FEATURE_MAPS[phi]
    return int(phi)


def _opt_z(z, state):
    return None if z is None else _check_z(z, state)


def hybrid_attn_step_phi(q, k, v, state, slots, phi, z=None, out=None, blk_lens=None, scale=None, stream=None):
    """hybrid_attn_step (z = None) or hybrid_attn_step_norm (z given) with the
    feature map ``phi`` ("relu" or "elu1")."""
    if out is None:
        with _on_stream(stream):
            out = torch.zeros_like(q)
    a = _step_args(q, k, v, state, slots, out, blk_lens, scale)
    args = a[:4] + (_opt_z(z, state),) + a[4:13] + (_phi_code(phi), a[13])
    _check("hybrid_attn_step_phi", load_library().hybrid_attn_step_phi(*args, _stream(stream)))
    return out


def hybrid_attn_step_commit_phi(q, k, v, state, slots, phi, z=None, out=None, blk_lens=None, scale=None,
                                stream=None):
    """The step from the current state, then state (and z) updated by the
    block, with the feature map ``phi``.  Requests must use distinct slots."""
    if out is None:
        with _on_stream(stream):
            out = torch.zeros_like(q)
    a = _step_args(q, k, v, state, slots, out, blk_lens, scale)
    args = a[:4] + (_opt_z(z, state),) + a[4:13] + (_phi_code(phi), a[13])
    _check("hybrid_attn_step_commit_phi", load_library().hybrid_attn_step_commit_phi(*args, _stream(stream)))
    return out


def hybrid_state_commit_phi(k, v, state, slots, phi, z=None, blk_lens=None, stream=None):
    """state[slots] += phi(K)^T V (and z += sum phi(k) when z is given)."""
    a = _commit_args(k, v, state, slots, blk_lens)
    args = a[:3] + (_opt_z(z, state),) + a[3:10] + (_phi_code(phi), a[10])
    _check("hybrid_state_commit_phi", load_library().hybrid_state_commit_phi(*args, _stream(stream)))
    return state


def hybrid_state_prefill_phi(k, v, cu_seqlens, state, slots, phi, z=None, max_len=None, chunk=256, workspace=None,
                             stream=None):
    """state[slots[r]] (and z[slots[r]]) overwritten by the sums over prompt r
    of phi(k_t)^T v_t (and phi(k_t)), with the feature map ``phi``."""
    a, _ws = _prefill_args(k, v, cu_seqlens, state, slots, max_len, chunk, workspace, stream)
    args = a[:6] + (_opt_z(z, state),) + a[6:14] + (_phi_code(phi), a[14])
    _check("hybrid_state_prefill_phi", load_library().hybrid_state_prefill_phi(*args, _stream(stream)))
    return state
