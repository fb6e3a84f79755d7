"""The C-ABI library on a host without a GPU: it loads, exports every symbol
the header declares, and rejects bad arguments before touching the GPU.
These calls never launch a kernel: validation fails first, or n_req == 0."""
import ctypes
import os
import re

import pytest

import block_hybrid_linear_amd as bh
from block_hybrid_linear_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hybrid_attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from block_hybrid_linear_amd.build import build_library
        build_library()
    return bh.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hybrid_\w+)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for n in ("hybrid_attn_step", "hybrid_attn_step_commit", "hybrid_state_commit", "hybrid_state_prefill",
              "hybrid_state_prefill_workspace_bytes", "hybrid_exact_step", "hybrid_exact_step_workspace_bytes",
              "hybrid_attn_step_norm", "hybrid_attn_step_commit_norm", "hybrid_state_commit_norm",
              "hybrid_state_prefill_norm", "hybrid_state_prefill_noalloc", "hybrid_attn_step_phi",
              "hybrid_attn_step_commit_phi", "hybrid_state_commit_phi", "hybrid_state_prefill_phi",
              "hybrid_last_error", "hybrid_abi_version"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version(lib):
    assert bh.abi_version() == 2


N = None


def step(lib, q=1, k=1, v=1, state=1, slots=1, out=1, n_req=2, n_slots=2, heads=4, blk=32, d=64,
         scale=0.125, dtype=binding.HA_BF16):
    return lib.hybrid_attn_step(q, k, v, state, slots, out, None, n_req, n_slots, heads, blk, d, scale,
                                dtype, None)


def step_commit(lib, q=1, k=1, v=1, state=1, slots=1, out=1, n_req=2, n_slots=2, heads=4, blk=32, d=64,
                scale=0.125, dtype=binding.HA_BF16):
    return lib.hybrid_attn_step_commit(q, k, v, state, slots, out, None, n_req, n_slots, heads, blk, d, scale,
                                       dtype, None)


def commit(lib, k=1, v=1, state=1, slots=1, n_req=2, n_slots=2, heads=4, blk=32, d=64, dtype=binding.HA_BF16):
    return lib.hybrid_state_commit(k, v, state, slots, None, n_req, n_slots, heads, blk, d, dtype, None)


def prefill(lib, k=1, v=1, cu=1, total=100, max_len=60, state=1, slots=1, n_req=2, n_slots=2, heads=4, d=64,
            chunk=256, ws=1, ws_bytes=1 << 40, dtype=binding.HA_BF16):
    return lib.hybrid_state_prefill(k, v, cu, total, max_len, state, slots, n_req, n_slots, heads, d, chunk,
                                    ws, ws_bytes, dtype, None)


def exact(lib, q=1, k=1, v=1, kc=1, vc=1, cu=1, total=100, out=1, n_req=2, heads=4, blk=32, d=64, scale=0.125,
          chunk=256, ws=1, ws_bytes=1 << 40, dtype=binding.HA_BF16):
    return lib.hybrid_exact_step(q, k, v, kc, vc, cu, total, out, None, n_req, heads, blk, d, scale, chunk, ws,
                                 ws_bytes, dtype, None)


def step_norm(lib, q=1, k=1, v=1, state=1, z=1, slots=1, out=1, n_req=2, n_slots=2, heads=4, blk=32, d=64,
              scale=0.125, dtype=binding.HA_BF16):
    return lib.hybrid_attn_step_norm(q, k, v, state, z, slots, out, None, n_req, n_slots, heads, blk, d, scale,
                                     dtype, None)


def step_commit_norm(lib, q=1, k=1, v=1, state=1, z=1, slots=1, out=1, n_req=2, n_slots=2, heads=4, blk=32, d=64,
                     scale=0.125, dtype=binding.HA_BF16):
    return lib.hybrid_attn_step_commit_norm(q, k, v, state, z, slots, out, None, n_req, n_slots, heads, blk, d,
                                            scale, dtype, None)


def commit_norm(lib, k=1, v=1, state=1, z=1, slots=1, n_req=2, n_slots=2, heads=4, blk=32, d=64,
                dtype=binding.HA_BF16):
    return lib.hybrid_state_commit_norm(k, v, state, z, slots, None, n_req, n_slots, heads, blk, d, dtype, None)


def prefill_norm(lib, k=1, v=1, cu=1, total=100, max_len=60, state=1, z=1, slots=1, n_req=2, n_slots=2, heads=4,
                 d=64, chunk=256, ws=1, ws_bytes=1 << 40, dtype=binding.HA_BF16):
    return lib.hybrid_state_prefill_norm(k, v, cu, total, max_len, state, z, slots, n_req, n_slots, heads, d, chunk,
                                         ws, ws_bytes, dtype, None)


def last(lib):
    return lib.hybrid_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d=100), binding.HA_ERR_UNSUPPORTED, "head dim"),
    (dict(d=48), binding.HA_ERR_UNSUPPORTED, "head dim"),
    (dict(dtype=7), binding.HA_ERR_UNSUPPORTED, "dtype"),
    (dict(blk=0), binding.HA_ERR_INVALID_ARG, "blk"),
    (dict(blk=257), binding.HA_ERR_INVALID_ARG, "blk"),
    (dict(n_req=-1), binding.HA_ERR_INVALID_ARG, "n_req"),
    (dict(n_slots=0), binding.HA_ERR_INVALID_ARG, "n_slots"),
    (dict(heads=0), binding.HA_ERR_INVALID_ARG, "heads"),
    (dict(scale=float("inf")), binding.HA_ERR_INVALID_ARG, "scale"),
    (dict(scale=float("nan")), binding.HA_ERR_INVALID_ARG, "scale"),
    (dict(q=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
    (dict(state=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
    (dict(slots=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
    (dict(out=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
])
def test_step_rejects(lib, kw, status, msg):
    assert step(lib, **kw) == status
    assert msg in last(lib) and "hybrid_attn_step" in last(lib)
    assert step_commit(lib, **kw) == status
    assert msg in last(lib) and "hybrid_attn_step_commit" in last(lib)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d=8), binding.HA_ERR_UNSUPPORTED, "head dim"),
    (dict(dtype=-1), binding.HA_ERR_UNSUPPORTED, "dtype"),
    (dict(blk=1000), binding.HA_ERR_INVALID_ARG, "blk"),
    (dict(heads=-3), binding.HA_ERR_INVALID_ARG, "heads"),
    (dict(k=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
    (dict(state=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
])
def test_commit_rejects(lib, kw, status, msg):
    assert commit(lib, **kw) == status
    assert msg in last(lib) and "hybrid_state_commit" in last(lib)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d=256), binding.HA_ERR_UNSUPPORTED, "head dim"),
    (dict(dtype=2), binding.HA_ERR_UNSUPPORTED, "dtype"),
    (dict(chunk=0), binding.HA_ERR_INVALID_ARG, "chunk"),
    (dict(total=-1), binding.HA_ERR_INVALID_ARG, "total_tokens"),
    (dict(max_len=-5), binding.HA_ERR_INVALID_ARG, "max_len"),
    (dict(cu=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
    (dict(k=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
    (dict(ws_bytes=10), binding.HA_ERR_INVALID_ARG, "workspace"),
    (dict(ws=None), binding.HA_ERR_INVALID_ARG, "workspace"),
    (dict(n_req=70000), binding.HA_ERR_INVALID_ARG, "65535"),
])
def test_prefill_rejects(lib, kw, status, msg):
    assert prefill(lib, **kw) == status
    assert msg in last(lib) and "hybrid_state_prefill" in last(lib)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d=48), binding.HA_ERR_UNSUPPORTED, "head dim"),
    (dict(dtype=3), binding.HA_ERR_UNSUPPORTED, "dtype"),
    (dict(blk=0), binding.HA_ERR_INVALID_ARG, "blk"),
    (dict(blk=129), binding.HA_ERR_INVALID_ARG, "blk"),
    (dict(heads=0), binding.HA_ERR_INVALID_ARG, "heads"),
    (dict(n_req=-2), binding.HA_ERR_INVALID_ARG, "n_req"),
    (dict(scale=float("inf")), binding.HA_ERR_INVALID_ARG, "scale"),
    (dict(chunk=0), binding.HA_ERR_INVALID_ARG, "chunk"),
    (dict(total=-1), binding.HA_ERR_INVALID_ARG, "total_prefix"),
    (dict(q=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
    (dict(cu=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
    (dict(out=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
    (dict(kc=None), binding.HA_ERR_INVALID_ARG, "k_cache"),
    (dict(ws_bytes=10), binding.HA_ERR_INVALID_ARG, "workspace"),
    (dict(ws=None), binding.HA_ERR_INVALID_ARG, "workspace"),
])
def test_exact_rejects(lib, kw, status, msg):
    assert exact(lib, **kw) == status
    assert msg in last(lib) and "hybrid_exact_step" in last(lib)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d=100), binding.HA_ERR_UNSUPPORTED, "head dim"),
    (dict(blk=257), binding.HA_ERR_INVALID_ARG, "blk"),
    (dict(scale=float("nan")), binding.HA_ERR_INVALID_ARG, "scale"),
    (dict(z=None), binding.HA_ERR_INVALID_ARG, "z"),
    (dict(state=None), binding.HA_ERR_INVALID_ARG, "non-NULL"),
])
def test_norm_calls_reject(lib, kw, status, msg):
    """The normalised calls keep their plain counterparts' checks and require z."""
    for fn, name in ((step_norm, "hybrid_attn_step_norm"), (step_commit_norm, "hybrid_attn_step_commit_norm")):
        assert fn(lib, **kw) == status
        assert msg in last(lib) and name in last(lib)
    ckw = {key: val for key, val in kw.items() if key != "scale"}
    if ckw:
        assert commit_norm(lib, **ckw) == status
        assert msg in last(lib) and "hybrid_state_commit_norm" in last(lib)
    pkw = {key: val for key, val in kw.items() if key not in ("scale", "blk")}
    if pkw:
        assert prefill_norm(lib, **pkw) == status
        assert msg in last(lib) and "hybrid_state_prefill_norm" in last(lib)


A = 1 << 12   # a fake, suitably aligned device address (never dereferenced: the calls fail validation)


@pytest.mark.parametrize("call,kw,msg", [
    ("step", dict(q=A + 2), "16-byte"),
    ("step", dict(state=A + 8), "16-byte"),
    ("step_commit", dict(out=A + 4), "16-byte"),
    ("commit", dict(v=A + 4), "16-byte"),
    ("prefill", dict(k=A + 8), "16-byte"),
    ("prefill", dict(ws=A + 16), "256-byte"),
    ("exact", dict(vc=A + 2), "16-byte"),
    ("exact", dict(out=A + 8), "16-byte"),
    ("exact", dict(ws=A + 128), "256-byte"),
    ("step_norm", dict(z=A + 4), "16-byte"),
    ("commit_norm", dict(z=A + 8), "16-byte"),
    ("prefill_norm", dict(z=A + 12), "16-byte"),
])
def test_misaligned_pointers_rejected(lib, call, kw, msg):
    fn = {"step": step, "step_commit": step_commit, "commit": commit, "prefill": prefill, "exact": exact,
          "step_norm": step_norm, "commit_norm": commit_norm, "prefill_norm": prefill_norm}[call]
    base = {"step": dict(q=A, k=A, v=A, state=A, slots=A, out=A),
            "step_commit": dict(q=A, k=A, v=A, state=A, slots=A, out=A),
            "commit": dict(k=A, v=A, state=A, slots=A),
            "prefill": dict(k=A, v=A, cu=A, state=A, slots=A, ws=A),
            "exact": dict(q=A, k=A, v=A, kc=A, vc=A, cu=A, out=A, ws=A),
            "step_norm": dict(q=A, k=A, v=A, state=A, slots=A, out=A),
            "commit_norm": dict(k=A, v=A, state=A, slots=A),
            "prefill_norm": dict(k=A, v=A, cu=A, state=A, slots=A, ws=A)}[call]
    base.update(kw)
    assert fn(lib, **base) == binding.HA_ERR_INVALID_ARG
    assert msg in last(lib)


def test_empty_batches_are_noops(lib):
    """n_req == 0 returns OK without touching any pointer (all NULL here)."""
    assert step(lib, q=None, k=None, v=None, state=None, slots=None, out=None, n_req=0) == binding.HA_OK
    assert step_commit(lib, q=None, k=None, v=None, state=None, slots=None, out=None, n_req=0) == binding.HA_OK
    assert commit(lib, k=None, v=None, state=None, slots=None, n_req=0) == binding.HA_OK
    assert prefill(lib, k=None, v=None, cu=None, state=None, slots=None, ws=None, ws_bytes=0,
                   n_req=0) == binding.HA_OK
    assert exact(lib, q=None, k=None, v=None, kc=None, vc=None, cu=None, out=None, ws=None, ws_bytes=0,
                 n_req=0) == binding.HA_OK
    assert step_norm(lib, q=None, k=None, v=None, state=None, z=None, slots=None, out=None,
                     n_req=0) == binding.HA_OK
    assert commit_norm(lib, k=None, v=None, state=None, z=None, slots=None, n_req=0) == binding.HA_OK
    assert prefill_norm(lib, k=None, v=None, cu=None, state=None, z=None, slots=None, ws=None, ws_bytes=0,
                        n_req=0) == binding.HA_OK


def test_noalloc_prefill_validates_before_touching_the_gpu(lib):
    """The prefill that uses the library's own scratch: an empty batch is a
    no-op, and a call needing more than the scratch's fixed maximum, or with
    bad arguments, is rejected before any device call."""
    fn = lib.hybrid_state_prefill_noalloc
    assert fn(None, None, None, 0, 0, None, None, 0, 2, 4, 64, 256, binding.HA_BF16, None) == binding.HA_OK
    need = bh.hybrid_state_prefill_workspace_bytes(64, 32, 128, 10 ** 6, 0, 256)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    assert fn(1, 1, 1, 10 ** 6, 0, 1, 1, 64, 64, 32, 128, 256, binding.HA_BF16, None) == binding.HA_ERR_INVALID_ARG
    assert "scratch" in lib.hybrid_last_error().decode()
    assert bh.hybrid_state_prefill_workspace_bytes(47, 32, 128, 10 ** 6, 0, 256) <= binding.NOALLOC_SCRATCH_BYTES
    assert fn(1, 1, 1, 100, 0, 1, 1, 2, 2, 4, 48, 256, binding.HA_BF16, None) == binding.HA_ERR_UNSUPPORTED
    assert fn(1, 1, 1, 100, 0, 1, 1, 2, 2, 4, 64, 0, binding.HA_BF16, None) == binding.HA_ERR_INVALID_ARG
    assert fn(1, 1, 1, 100, 0, 1, 1, -1, 2, 4, 64, 256, binding.HA_BF16, None) == binding.HA_ERR_INVALID_ARG


def test_feature_map_calls_validate(lib):
    """The *_phi calls reject an unknown map (unsupported) and keep the plain
    calls' checks; an empty batch is a no-op."""
    bf = binding.HA_BF16
    assert lib.hybrid_attn_step_phi(1, 1, 1, 1, None, 1, 1, None, 2, 2, 4, 32, 64, 0.1, 5, bf, None) \
        == binding.HA_ERR_UNSUPPORTED
    assert "feature map" in last(lib)
    assert lib.hybrid_attn_step_commit_phi(1, 1, 1, 1, None, 1, 1, None, 2, 2, 4, 32, 64, 0.1, -1, bf, None) \
        == binding.HA_ERR_UNSUPPORTED
    assert lib.hybrid_state_commit_phi(1, 1, 1, None, 1, None, 2, 2, 4, 32, 64, 2, bf, None) \
        == binding.HA_ERR_UNSUPPORTED
    assert lib.hybrid_state_prefill_phi(1, 1, 1, 100, 0, 1, None, 1, 2, 2, 4, 64, 256, 1, 1 << 40, 9, bf, None) \
        == binding.HA_ERR_UNSUPPORTED
    assert lib.hybrid_attn_step_phi(1, 1, 1, 1, None, 1, 1, None, 2, 2, 4, 300, 64, 0.1, 1, bf, None) \
        == binding.HA_ERR_INVALID_ARG
    assert lib.hybrid_attn_step_phi(None, None, None, None, None, None, None, None, 0, 2, 4, 32, 64, 0.1, 1, bf,
                                    None) == binding.HA_OK


def test_prefill_workspace_size(lib):
    """Plan (n_req + 2 int64, padded to 256 bytes) + one fp32 partial of
    d x d + d floats (S and the normalised variant's z) per (slice, unit)
    slot: max(512 (2048 for d = 32), heads) + n_req * heads slots."""
    f = bh.hybrid_state_prefill_workspace_bytes
    plan = lambda n: ((n + 2) * 8 + 255) // 256 * 256  # noqa: E731
    assert f(2, 4, 64, 100, 0, 256) == plan(2) + (512 + 8) * (64 * 64 + 64) * 4
    assert f(8, 32, 128, 10 ** 6, 65536, 256) == plan(8) + (512 + 256) * (128 * 128 + 128) * 4
    assert f(1, 1, 32, 0, 0, 1) == plan(1) + (2048 + 1) * (32 * 32 + 32) * 4
    assert f(40, 2, 16, 0, 0, 7) == plan(40) + (512 + 80) * (16 * 16 + 16) * 4
    assert f(2, 600, 64, 10, 0, 256) == plan(2) + (600 + 1200) * (64 * 64 + 64) * 4
    assert f(1, 3000, 32, 10, 0, 256) == plan(1) + (3000 + 3000) * (32 * 32 + 32) * 4
    assert f(0, 1, 16, 0, 10, 1) == 0
    assert f(3, 1, 16, 0, 10, 0) == 0


def test_exact_workspace_size(lib):
    """Plan as for prefill + (slices + n_req * heads) partials of R rows x
    (d + 2) floats (output row, max, sum), R = 32 / 64 / 128 for blk up to
    32 / 64 / 128; slices = 256 x workgroups per compute unit of the
    variant, 1024 for d = 16."""
    f = bh.hybrid_exact_step_workspace_bytes
    plan = lambda n: ((n + 2) * 8 + 255) // 256 * 256  # noqa: E731
    assert f(64, 32, 32, 128) == plan(64) + (768 + 2048) * 32 * 130 * 4
    assert f(3, 5, 33, 16) == plan(3) + (1024 + 15) * 64 * 18 * 4
    assert f(2, 3, 65, 32) == plan(2) + (1024 + 6) * 128 * 34 * 4
    assert f(1, 1, 128, 64) == plan(1) + (512 + 1) * 128 * 66 * 4
    assert f(5, 2, 40, 64) == plan(5) + (1024 + 10) * 64 * 66 * 4
    assert f(5, 2, 8, 32) == plan(5) + (2304 + 10) * 32 * 34 * 4
    assert f(1, 1, 100, 128) == plan(1) + (256 + 1) * 128 * 130 * 4
    assert f(0, 1, 32, 64) == 0 and f(2, 2, 0, 64) == 0 and f(2, 2, 129, 64) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError, match="GPU"):
        bh.hybrid_attn_step(q, q, q, torch.zeros(1, 1, 16, 16), torch.zeros(1, dtype=torch.int32))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        binding._lib_saved = binding._lib
        try:
            binding._lib = None
            binding.load_library(str(tmp_path / "nope.so"))
        finally:
            binding._lib = binding._lib_saved


def test_header_is_plain_c_and_links(tmp_path):
    """include/hybrid_attn.h compiles as C11 (gcc, -Wall -Wextra -Werror) in
    a program that links libhybrid_attn.so and libamdhip64 with no C++ or
    torch; the GPU test runs the same program."""
    import importlib.util
    here = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location("c_consumer_build", os.path.join(here, "c_consumer", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    exe = mod.build_consumer(str(tmp_path / "abi_consumer"))
    assert os.path.getsize(exe) > 0
