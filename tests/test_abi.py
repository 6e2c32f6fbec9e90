"""The C-ABI library loads and exports every entry point include/pa.h
declares; host-side argument checks return their status codes without
touching a GPU (null pointers and bad sizes are rejected before any launch)."""
import ctypes
import os
import subprocess
import sys

import pytest

import ragged_paged_attention_amd as rpa
from ragged_paged_attention_amd import _lib


def test_library_loads_and_exports_all_declared_symbols():
    lib = rpa.library()
    names = rpa.declared_symbols()
    assert {"pa_build_metadata", "pa_write_kv", "pa_attention", "pa_attention_workspace_size",
            "pa_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libpa.so does not export {n}"
    out = subprocess.run(["nm", "-D", "--defined-only", rpa.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported


def test_version_and_status_strings():
    assert rpa.pa_version() >= 100
    for code in range(8):
        assert rpa.status_string(code).startswith("PA_")


def test_validation_switch_roundtrip():
    prev = rpa.pa_set_validation(1)
    assert rpa.pa_set_validation(prev) == 1
    assert rpa.pa_set_validation(2) == -1


def test_trace_switch_roundtrip():
    prev = rpa.pa_set_trace(1)
    assert rpa.pa_set_trace(prev) == 1
    assert rpa.pa_set_trace(-1) == -1


@pytest.mark.parametrize("value,expected", [("1", ["1", "1"]), ("yes", ["1", "1"]), ("0", ["0", "0"]),
                                            ("", ["0", "0"])])
def test_environment_sets_trace_and_validation_at_load(value, expected):
    """PA_TRACE and PA_VALIDATE in the environment at load time give the
    switches' initial values (a fresh process: the library reads them once)."""
    code = "import ragged_paged_attention_amd as r; print(r.pa_set_trace(0), r.pa_set_validation(0))"
    env = {**os.environ, "PA_TRACE": value, "PA_VALIDATE": value}
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], env=env, cwd=root, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split() == expected


def test_kernel_policy_roundtrip():
    prev = rpa.pa_set_kernel_policy(rpa.PA_POLICY_GENERIC)
    assert rpa.pa_set_kernel_policy(prev) == rpa.PA_POLICY_GENERIC
    assert rpa.pa_set_kernel_policy(7) == -1


def test_host_side_rejections_need_no_gpu():
    lib = _lib.library()
    NULL = None
    # negative sizes
    assert lib.pa_build_metadata(NULL, NULL, -1, 0, NULL, 0, 1, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == 2
    # missing outputs
    assert lib.pa_build_metadata(NULL, NULL, 0, 0, NULL, 0, 1, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == 1
    # bad dtype
    assert lib.pa_write_kv(NULL, NULL, NULL, 1, 1, 1, NULL, NULL, 1, 1, 9, NULL, NULL) == 3
    # num_blocks * block_size overflowing int32 slots
    assert lib.pa_write_kv(NULL, NULL, NULL, 1, 1, 1, NULL, NULL, 1 << 20, 1 << 12, 1, NULL, NULL) == 2
    # nothing to write is fine
    assert lib.pa_write_kv(NULL, NULL, NULL, 0, 1, 1, NULL, NULL, 1, 1, 1, NULL, NULL) == 0
    att = lambda **kw: lib.pa_attention(*_attn_args(**kw))
    assert att(Hq=6, Hkv=4) == 2          # Hq % Hkv != 0
    assert att(D=512) == 4                # head_dim > 256
    assert att(T=0) == 0                  # empty batch: nothing to do
    assert att() == 1                     # null pointers
    assert att(max_q=0) == 2              # size hints must be >= 1
    assert att(scale=float("nan")) == 7   # non-finite softmax scale
    assert att(scale=float("inf")) == 7
    assert lib.pa_attention_workspace_size(4, 100, 32, 32, 128, 1, 2001) >= 0
    # the fused write + attention: pa_write_kv's checks, then pa_attention's
    wa = lambda **kw: lib.pa_write_kv_attention(*_write_attn_args(**kw))
    assert wa(dtype=9) == 3               # bad dtype
    assert wa(NB=1 << 20, bs=1 << 12) == 2  # slots overflowing int32
    assert wa(T=0) == 0                   # empty batch: nothing to do
    assert wa() == 1                      # null new rows
    assert wa(fake_rows=True, Hq=6, Hkv=4) == 2   # then the attention's own checks
    assert wa(fake_rows=True, scale=float("nan")) == 7
    cp = lambda nsrc=4, ndst=4, n=1, bb=8192, ptr=16: lib.pa_copy_blocks(ptr, ptr, ptr, ptr, nsrc, ndst, ptr, n, bb,
                                                                          NULL, NULL)
    assert cp(bb=8200) == 2               # block bytes not a multiple of 16
    assert cp(nsrc=0) == 2
    assert cp(n=-1) == 2
    assert cp(ptr=8) == 2                 # pools not 16-byte aligned
    assert cp(ptr=None) == 1
    assert cp(n=0, ptr=None) == 0         # nothing to copy


def test_noalloc_refuses_calls_beyond_its_scratch_without_a_gpu():
    """pa_attention_noalloc checks the call's workspace need against its
    static scratch before any HIP call: too large a call is refused with
    PA_ERR_WORKSPACE (the pointers below are never dereferenced)."""
    lib = _lib.library()
    fake = ctypes.c_void_p(1 << 20)
    S, T, Hq, Hkv, D, max_q, max_l = 256, 8192, 32, 8, 128, 497, 8192
    need = lib.pa_attention_workspace_size(S, T, Hq, Hkv, D, max_q, max_l)
    assert need > rpa.PA_NOALLOC_SCRATCH_BYTES
    args = [fake] * 6 + [S, T, Hq, Hkv, D, 16, 40000, 512, max_q, max_l, ctypes.c_float(0.088), 1, fake, None,
                         None]
    assert lib.pa_attention_noalloc(*args) == 5
    assert lib.pa_attention_noalloc(*([None] * 6 + args[6:])) == 1   # null pointers come first


def _attn_args(T=3, Hq=4, Hkv=2, D=16, max_q=2, S=2, scale=0.25):
    return [None] * 6 + [S, T, Hq, Hkv, D, 16, 8, 4, max_q, 8, ctypes.c_float(scale), 1, None, None, 0, None, None]


def _write_attn_args(T=3, Hq=4, Hkv=2, D=16, max_q=2, S=2, scale=0.25, dtype=1, NB=8, bs=16, fake_rows=False):
    rows = [ctypes.c_void_p(1 << 20)] * 3 if fake_rows else [None] * 3   # never dereferenced: checks come first
    return rows + [None] * 6 + [S, T, Hq, Hkv, D, bs, NB, 4, max_q, 8, ctypes.c_float(scale), dtype, None, None, 0,
                                None, None]
