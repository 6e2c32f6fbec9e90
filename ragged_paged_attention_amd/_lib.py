"""ctypes binding to libpa.so: argument marshalling only.

Each function here has the name of the C entry point it calls and forwards
device pointers (from torch tensors), sizes and the current HIP stream.  Every
step of the computation runs in the library's HIP kernels; torch is used only
to own device memory and to name the stream.  If the library is missing the
import fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "pa.h")
HEADERS = [HEADER, os.path.join(os.path.dirname(PKG), "include", "pa_bench.h")]

PA_F32, PA_BF16, PA_F16 = 0, 1, 2
PA_POLICY_AUTO, PA_POLICY_GENERIC, PA_POLICY_FAST = 0, 1, 2
PA_DERR_QLEN_GT_SEQLEN, PA_DERR_TOKEN_SUM, PA_DERR_BLOCK_OOB, PA_DERR_SLOT_OOB, PA_DERR_OVERFLOW = 1, 2, 4, 8, 16
PA_DERR_HINT = 32
PA_DERR_DUP_SLOT = 64
PA_NOALLOC_SCRATCH_BYTES = 64 << 20   # include/pa.h


class PAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        extra = ""
        if status == 6:
            extra = " [" + _lib.pa_last_hip_error().decode() + "]"
        super().__init__(f"{where}: {status_string(status)} (status {status}){extra}")


def _load() -> ctypes.CDLL:
    # One process must hold one HIP runtime.  torch ships its own
    # libamdhip64.so.7; importing torch first makes libpa bind to that copy
    # (same soname) instead of loading /opt/rocm's alongside it, which would
    # leave two runtimes fighting over the device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python ragged_paged_attention_amd/build.py` "
                          "(there is no non-HIP fallback)")
    return ctypes.CDLL(LIB_PATH)


_lib = _load()

_i32, _p, _f32, _size = ctypes.c_int32, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t

_lib.pa_status_string.restype = ctypes.c_char_p
_lib.pa_status_string.argtypes = [_i32]
_lib.pa_last_hip_error.restype = ctypes.c_char_p
_lib.pa_last_hip_error.argtypes = []
_lib.pa_version.restype = _i32
_lib.pa_version.argtypes = []
_lib.pa_set_kernel_policy.restype = _i32
_lib.pa_set_kernel_policy.argtypes = [_i32]
_lib.pa_set_validation.restype = _i32
_lib.pa_set_validation.argtypes = [_i32]
_lib.pa_set_trace.restype = _i32
_lib.pa_set_trace.argtypes = [_i32]
_lib.pa_build_metadata.restype = _i32
_lib.pa_build_metadata.argtypes = [_p, _p, _i32, _i32, _p, _i32, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p]
_lib.pa_write_kv.restype = _i32
_lib.pa_write_kv.argtypes = [_p, _p, _p, _i32, _i32, _i32, _p, _p, _i32, _i32, _i32, _p, _p]
_lib.pa_copy_blocks.restype = _i32
_lib.pa_copy_blocks.argtypes = [_p, _p, _p, _p, _i32, _i32, _p, _i32, ctypes.c_int64, _p, _p]
_lib.pa_attention_workspace_size.restype = _size
_lib.pa_attention_workspace_size.argtypes = [_i32] * 7
_lib.pa_bench_stream_read.restype = _i32
_lib.pa_bench_stream_read.argtypes = [_p, _size, _p, _p]
_lib.pa_bench_paged_read.restype = _i32
_lib.pa_bench_paged_read.argtypes = [_p, _p, _p, _p] + [_i32] * 6 + [_p, _p]
class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


_lib.pa_bench_timing_begin.restype = _i32
_lib.pa_bench_timing_begin.argtypes = []
_lib.pa_bench_timing_end.restype = _i32
_lib.pa_bench_timing_end.argtypes = [ctypes.POINTER(KernelTime), _i32, ctypes.POINTER(_i32)]
_lib.pa_attention.restype = _i32
_lib.pa_attention.argtypes = [_p, _p, _p, _p, _p, _p] + [_i32] * 10 + [_f32, _i32, _p, _p, _size, _p, _p]
_lib.pa_write_kv_attention.restype = _i32
_lib.pa_write_kv_attention.argtypes = [_p] * 9 + [_i32] * 10 + [_f32, _i32, _p, _p, _size, _p, _p]
_lib.pa_attention_noalloc.restype = _i32
_lib.pa_attention_noalloc.argtypes = [_p, _p, _p, _p, _p, _p] + [_i32] * 10 + [_f32, _i32, _p, _p, _p]


def declared_symbols() -> list:
    """Names of the functions include/pa.h and include/pa_bench.h declare."""
    names = set()
    for h in HEADERS:
        with open(h) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text))
    return sorted(names)


def library() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.pa_status_string(int(status)).decode()


def pa_version() -> int:
    return int(_lib.pa_version())


def pa_set_kernel_policy(policy: int) -> int:
    return int(_lib.pa_set_kernel_policy(int(policy)))


def pa_set_validation(on: int) -> int:
    return int(_lib.pa_set_validation(int(on)))


def pa_set_trace(on: int) -> int:
    return int(_lib.pa_set_trace(int(on)))


# --------------------------------------------------------------------------
# torch marshalling helpers
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return PA_F32
    if dt == torch.bfloat16:
        return PA_BF16
    if dt == torch.float16:
        return PA_F16
    raise TypeError(f"unsupported dtype {dt}")


def _check(status: int, where: str):
    if status != 0:
        raise PAError(status, where)


def _need(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------
def pa_build_metadata(query_lens, seq_lens, num_tokens: int, block_tables=None, block_size: int = 1,
                      num_blocks: int = 1, out: dict | None = None, d_err=None) -> dict:
    """Calls pa_build_metadata.  Returns a dict of device int32 tensors:
    query_start_loc, seq_start_loc, positions, token_to_seq, slot_mapping
    (None without a table) and stats."""
    torch = _torch()
    i32 = torch.int32
    _need(query_lens, "query_lens", i32)
    _need(seq_lens, "seq_lens", i32)
    _need(block_tables, "block_tables", i32)
    dev = query_lens.device
    S = int(query_lens.shape[0])
    out = dict(out or {})
    for name, n in (("query_start_loc", S + 1), ("seq_start_loc", S + 1), ("positions", num_tokens),
                    ("token_to_seq", num_tokens), ("stats", 6)):
        if out.get(name) is None:
            out[name] = torch.empty(n, dtype=i32, device=dev)
    if block_tables is not None and out.get("slot_mapping") is None:
        out["slot_mapping"] = torch.empty(num_tokens, dtype=i32, device=dev)
    if block_tables is None:
        out["slot_mapping"] = None
    MB = int(block_tables.shape[1]) if block_tables is not None else 0
    st = _lib.pa_build_metadata(_ptr(query_lens), _ptr(seq_lens), S, int(num_tokens), _ptr(block_tables),
                                MB, int(block_size), int(num_blocks), _ptr(out["query_start_loc"]),
                                _ptr(out["seq_start_loc"]), _ptr(out["positions"]), _ptr(out["token_to_seq"]),
                                _ptr(out["slot_mapping"]), _ptr(out["stats"]), _ptr(d_err), _stream(dev))
    _check(st, "pa_build_metadata")
    return out


def pa_write_kv(k, v, slot_mapping, k_cache, v_cache, d_err=None) -> None:
    """Calls pa_write_kv.  k, v: [T, Hkv, D]; caches [NB, BS, Hkv, D]."""
    torch = _torch()
    for t, n in ((k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, n, k.dtype)
    _need(slot_mapping, "slot_mapping", torch.int32)
    T, Hkv, D = (int(x) for x in k.shape)
    NB, BS = int(k_cache.shape[0]), int(k_cache.shape[1])
    if tuple(k_cache.shape[2:]) != (Hkv, D) or v_cache.shape != k_cache.shape or v.shape != k.shape:
        raise ValueError("shape mismatch between new rows and caches")
    st = _lib.pa_write_kv(_ptr(k), _ptr(v), _ptr(slot_mapping), T, Hkv, D, _ptr(k_cache), _ptr(v_cache),
                          NB, BS, _dtype_code(k.dtype), _ptr(d_err), _stream(k.device))
    _check(st, "pa_write_kv")


def pa_copy_blocks(src_k, src_v, dst_k, dst_v, pairs, d_err=None, stream_device=None) -> None:
    """Calls pa_copy_blocks.  Pools [NB, BS, Hkv, D] (device or pinned host),
    pairs [n, 2] int32 (source block, destination block), device-accessible."""
    torch = _torch()
    for t, n in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{n} must be device memory or pinned host memory")
    if pairs.dtype != torch.int32 or not pairs.is_contiguous() or (not pairs.is_cuda and not pairs.is_pinned()):
        raise ValueError("pairs must be a contiguous int32 device (or pinned) tensor")
    if src_k.shape[1:] != dst_k.shape[1:] or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination blocks differ in shape or dtype")
    block_bytes = src_k[0].numel() * src_k.element_size()
    dev = next((t.device for t in (src_k, dst_k, pairs) if t.is_cuda), torch.device("cuda"))
    st = _lib.pa_copy_blocks(_ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v), int(src_k.shape[0]),
                             int(dst_k.shape[0]), _ptr(pairs), int(pairs.shape[0]), int(block_bytes), _ptr(d_err),
                             _stream(dev))
    _check(st, "pa_copy_blocks")


def pa_attention_workspace_size(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_query_len,
                                max_seq_len) -> int:
    return int(_lib.pa_attention_workspace_size(int(num_seqs), int(num_tokens), int(num_q_heads),
                                                int(num_kv_heads), int(head_dim), int(max_query_len),
                                                int(max_seq_len)))


def pa_attention(q, k_cache, v_cache, block_tables, query_start_loc, seq_lens, max_query_len: int,
                 max_seq_len: int, scale: float, out=None, workspace=None, d_err=None):
    """Calls pa_attention.  q [T, Hq, D]; caches [NB, BS, Hkv, D]; returns out."""
    torch = _torch()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out")):
        _need(t, n, q.dtype)
    for t, n in ((block_tables, "block_tables"), (query_start_loc, "query_start_loc"), (seq_lens, "seq_lens")):
        _need(t, n, torch.int32)
    T, Hq, D = (int(x) for x in q.shape)
    NB, BS, Hkv = int(k_cache.shape[0]), int(k_cache.shape[1]), int(k_cache.shape[2])
    if int(k_cache.shape[3]) != D or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape mismatch")
    S = int(seq_lens.shape[0])
    if out is None:
        out = torch.empty_like(q)
    need = pa_attention_workspace_size(S, T, Hq, Hkv, D, max_query_len, max_seq_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.pa_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(query_start_loc),
                           _ptr(seq_lens), S, T, Hq, Hkv, D, BS, NB, int(block_tables.shape[1]),
                           int(max_query_len), int(max_seq_len), float(scale), _dtype_code(q.dtype),
                           _ptr(out), _ptr(workspace), wbytes, _ptr(d_err), _stream(q.device))
    _check(st, "pa_attention")
    return out


def pa_write_kv_attention(k, v, slot_mapping, q, k_cache, v_cache, block_tables, query_start_loc, seq_lens,
                          max_query_len: int, max_seq_len: int, scale: float, out=None, workspace=None,
                          d_err=None):
    """Calls pa_write_kv_attention: pa_write_kv(k, v, slot_mapping, ...) then
    pa_attention(q, ...), in one call.  k, v [T, Hkv, D]; q [T, Hq, D];
    caches [NB, BS, Hkv, D] (written); returns out."""
    torch = _torch()
    for t, n in ((k, "k"), (v, "v"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out")):
        _need(t, n, q.dtype)
    for t, n in ((slot_mapping, "slot_mapping"), (block_tables, "block_tables"),
                 (query_start_loc, "query_start_loc"), (seq_lens, "seq_lens")):
        _need(t, n, torch.int32)
    T, Hq, D = (int(x) for x in q.shape)
    NB, BS, Hkv = int(k_cache.shape[0]), int(k_cache.shape[1]), int(k_cache.shape[2])
    if int(k_cache.shape[3]) != D or v_cache.shape != k_cache.shape or tuple(k.shape) != (T, Hkv, D) or \
            v.shape != k.shape:
        raise ValueError("shape mismatch between new rows, queries and caches")
    S = int(seq_lens.shape[0])
    if out is None:
        out = torch.empty_like(q)
    need = pa_attention_workspace_size(S, T, Hq, Hkv, D, max_query_len, max_seq_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.pa_write_kv_attention(_ptr(k), _ptr(v), _ptr(slot_mapping), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(block_tables), _ptr(query_start_loc), _ptr(seq_lens), S, T, Hq, Hkv, D,
                                    BS, NB, int(block_tables.shape[1]), int(max_query_len), int(max_seq_len),
                                    float(scale), _dtype_code(q.dtype), _ptr(out), _ptr(workspace), wbytes,
                                    _ptr(d_err), _stream(q.device))
    _check(st, "pa_write_kv_attention")
    return out


def pa_attention_noalloc(q, k_cache, v_cache, block_tables, query_start_loc, seq_lens, max_query_len: int,
                         max_seq_len: int, scale: float, out=None, d_err=None):
    """Calls pa_attention_noalloc (the library's static scratch instead of a
    workspace).  Same shapes as pa_attention; returns out."""
    torch = _torch()
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (out, "out")):
        _need(t, n, q.dtype)
    for t, n in ((block_tables, "block_tables"), (query_start_loc, "query_start_loc"), (seq_lens, "seq_lens")):
        _need(t, n, torch.int32)
    T, Hq, D = (int(x) for x in q.shape)
    NB, BS, Hkv = int(k_cache.shape[0]), int(k_cache.shape[1]), int(k_cache.shape[2])
    if int(k_cache.shape[3]) != D or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape mismatch")
    if out is None:
        out = torch.empty_like(q)
    st = _lib.pa_attention_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                   _ptr(query_start_loc), _ptr(seq_lens), int(seq_lens.shape[0]), T, Hq, Hkv, D,
                                   BS, NB, int(block_tables.shape[1]), int(max_query_len), int(max_seq_len),
                                   float(scale), _dtype_code(q.dtype), _ptr(out), _ptr(d_err), _stream(q.device))
    _check(st, "pa_attention_noalloc")
    return out


# --------------------------------------------------------------------------
# measurement helpers (include/pa_bench.h)
# --------------------------------------------------------------------------
def pa_bench_stream_read(buf, sink) -> None:
    """Reads every byte of the contiguous device tensor `buf` once."""
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.pa_bench_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(buf.device)), "pa_bench_stream_read")


def pa_bench_paged_read(k_cache, v_cache, block_tables, seq_lens, max_seq_len: int, sink) -> None:
    """Reads the K/V rows of every sequence through its block table, no math."""
    NB, BS, Hkv = int(k_cache.shape[0]), int(k_cache.shape[1]), int(k_cache.shape[2])
    st = _lib.pa_bench_paged_read(_ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
                                  int(seq_lens.shape[0]), Hkv, BS, NB, int(block_tables.shape[1]),
                                  int(max_seq_len), _ptr(sink), _stream(k_cache.device))
    _check(st, "pa_bench_paged_read")


def pa_bench_timing_begin() -> None:
    _check(_lib.pa_bench_timing_begin(), "pa_bench_timing_begin")


def pa_bench_timing_end() -> dict:
    """{kernel name: (launches, total ms)} for the launches since begin()."""
    arr = (KernelTime * 32)()
    n = _i32(0)
    _check(_lib.pa_bench_timing_end(arr, 32, ctypes.byref(n)), "pa_bench_timing_end")
    return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms)) for i in range(n.value)}
