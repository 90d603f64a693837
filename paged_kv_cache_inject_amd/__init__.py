"""Python binding of libpkv (include/pkv.h): argument marshalling only.

Every function here has the name of the C entry point it calls and forwards
its arguments: torch tensors become device or host pointers, the current
torch stream becomes the HIP stream, and a negative status raises PkvError
with the library's message.  No step of the hot path runs in Python.

Loading fails loudly when the built library is missing: there is no
fallback.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
PKV_E_INVALID = -1
PKV_E_OOM = -2
PKV_E_RANGE = -3
PKV_E_OVERLAP = -4
PKV_E_WORKSPACE = -5
PKV_E_HIP = -6
PKV_E_UNSUPPORTED = -7
STATUS_NAMES = {0: "OK", -1: "INVALID", -2: "OOM", -3: "RANGE", -4: "OVERLAP",
                -5: "WORKSPACE", -6: "HIP", -7: "UNSUPPORTED"}

PKV_F32, PKV_BF16, PKV_F16, PKV_FP8E4M3 = 0, 1, 2, 3
DTYPE_CODES = {"f32": PKV_F32, "bf16": PKV_BF16, "f16": PKV_F16, "fp8": PKV_FP8E4M3}
PKV_ROPE_PAIRS, PKV_ROPE_HALVES, PKV_ROPE_NONE = 0, 1, 2
ROPE_CODES = {"pairs": PKV_ROPE_PAIRS, "halves": PKV_ROPE_HALVES, "none": PKV_ROPE_NONE}
BLOCK_TOKENS = 16
PKV_NOALLOC_SCRATCH_BYTES = 16 << 20     # static scratch of the allocation-free step


class PkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS_NAMES.get(status, "?"), status, msg))
        self.status = status
        self.code = STATUS_NAMES.get(status, "?")


class pkv_pool(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("layer_stride", ctypes.c_int64), ("block_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p)]


class pkv_src(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("layer_stride", ctypes.c_int64), ("token_stride", ctypes.c_int64),
                ("n_tokens", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("_reserved", ctypes.c_int32)]


class pkv_run(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
                ("dst_pos", ctypes.c_int32), ("_reserved", ctypes.c_int32),
                ("src_token", ctypes.c_int64)]


class pkv_cache_config(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("max_seqs", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("block_tokens", ctypes.c_int32),
                ("free_list_seed", ctypes.c_uint64)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "pkv_abi_version": (_I32, []),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_kv_bytes": (ctypes.c_uint64, [_I32, _I32, _I32, _I32, _I64]),
    "pkv_cache_create": (_I32, [ctypes.POINTER(pkv_cache_config), ctypes.POINTER(_P)]),
    "pkv_cache_destroy": (None, [_P]),
    "pkv_alloc_blocks": (_I32, [_P, _I32, _I64]),
    "pkv_set_blocks": (_I32, [_P, _I32, _P, _I32, _I64]),
    "pkv_extend": (_I32, [_P, _P, _I32, _I32, _P]),
    "pkv_free_seq": (_I32, [_P, _I32]),
    "pkv_block_table": (_I32, [_P, _P, _I32, _P, _P]),
    "pkv_table_width": (_I32, [_P]),
    "pkv_num_free_blocks": (_I32, [_P]),
    "pkv_free_list": (_I32, [_P, _P, _I32]),
    "pkv_fork": (_I32, [_P, _I32, _I32]),
    "pkv_block_refcount": (_I32, [_P, _I32]),
    "pkv_pending_copies": (_I32, [_P, _P, _I32]),
    "pkv_copy_blocks": (_I32, [_P, ctypes.POINTER(pkv_pool), _P]),
    "pkv_prefix_match": (_I32, [_P, _I32, _P, _I64, _P]),
    "pkv_prefix_commit": (_I32, [_P, _I32, _P, _I64]),
    "pkv_prefix_cached_blocks": (_I32, [_P]),
    "pkv_trim_window": (_I32, [_P, _P, _I32, _I32, _P]),
    "pkv_rope_table": (_I32, [_I32, ctypes.c_double, _I32, _P, _P]),
    "pkv_inject_workspace_bytes": (_SZ, [_P, _I32]),
    "pkv_host_alloc": (_I32, [_SZ, ctypes.POINTER(_P)]),
    "pkv_host_free": (_I32, [_P]),
    "pkv_inject": (_I32, [_P, ctypes.POINTER(pkv_pool), ctypes.POINTER(pkv_src), _P, _I32,
                          _I32, _I32, _I32, _P, _P, _I32, _P, _SZ, _P]),
    "pkv_append_kv": (_I32, [ctypes.POINTER(pkv_pool), _I32, _P, _I32, _P, _I32, _I32, _P, _P,
                             _I32, _I32, _P, _P, _I32, _P]),
    "pkv_decode_plan_create": (_I32, [_P, _I32, _I32, _I32, _I32, _I32, _I32,
                                      ctypes.POINTER(_P)]),
    "pkv_decode_plan_destroy": (None, [_P]),
    "pkv_decode_plan_items": (_I32, [_P]),
    "pkv_decode_plan_part_tokens": (_I32, [_P]),
    "pkv_decode_plan_waves": (_I32, [_P]),
    "pkv_decode_workspace_bytes": (_SZ, [_P]),
    "pkv_decode_plan_upload": (_I32, [_P, _P, _SZ, _P]),
    "pkv_decode_attention": (_I32, [_P, ctypes.POINTER(pkv_pool), _I32, _P, _I32,
                                    ctypes.c_float, _P, _I32, _P, _P, _P, _SZ, _P]),
    "pkv_append_decode_attention": (_I32, [_P, ctypes.POINTER(pkv_pool), _I32, _P, _I32,
                                           ctypes.c_float, _P, _I32, _P, _P, _I32, _P, _P, _I32,
                                           _P, _P, _P, _SZ, _P]),
    "pkv_append_decode_attention_noalloc": (_I32, [_P, ctypes.POINTER(pkv_pool), _I32, _P, _I32,
                                                   ctypes.c_float, _P, _I32, _P, _P, _I32, _P, _P,
                                                   _I32, _P, _P, _P]),
    "pkv_bw_probe": (_I32, [_P, _SZ, _P, _P]),
    "pkv_kernel_timing": (_I32, [_I32]),
    "pkv_kernel_times": (_I32, [_P, _I32]),
}

_lib = None


def load_library(path: str = LIB_PATH):
    """Load libpkv.so; raises if it is missing or lacks a declared symbol."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libpkv.so is not built (%s); run paged_kv_cache_inject_amd/build.py"
                          % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status < 0:
        raise PkvError(status, _lib.pkv_last_error().decode())
    return status


def _ptr(t):
    """Device or host address of a torch tensor or numpy array (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return t.ctypes.data


def _stream(stream=None):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------
# Library
# ---------------------------------------------------------------------------
def pkv_abi_version() -> int:
    return load_library().pkv_abi_version()


def pkv_last_error() -> str:
    return load_library().pkv_last_error().decode()


def pkv_kv_bytes(n_layers, n_kv_heads, head_dim, elem_bytes, n_tokens) -> int:
    return load_library().pkv_kv_bytes(n_layers, n_kv_heads, head_dim, elem_bytes, n_tokens)


# ---------------------------------------------------------------------------
# Allocator
# ---------------------------------------------------------------------------
def pkv_cache_create(num_blocks, max_seqs, max_blocks_per_seq, free_list_seed=0, block_tokens=16):
    lib = load_library()
    cfg = pkv_cache_config(num_blocks, max_seqs, max_blocks_per_seq, block_tokens, free_list_seed)
    h = ctypes.c_void_p()
    _check(lib.pkv_cache_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def pkv_cache_destroy(cache):
    load_library().pkv_cache_destroy(cache)


def pkv_alloc_blocks(cache, seq, n_tokens):
    _check(load_library().pkv_alloc_blocks(cache, seq, n_tokens))


def pkv_set_blocks(cache, seq, ids, length):
    import numpy as np
    a = np.ascontiguousarray(ids, dtype=np.int32)
    _check(load_library().pkv_set_blocks(cache, seq, a.ctypes.data, len(a), length))


def pkv_extend(cache, seqs, n_new):
    """Returns the int64 array of first new positions."""
    import numpy as np
    s = np.ascontiguousarray(seqs, dtype=np.int32)
    first = np.zeros(len(s), dtype=np.int64)
    _check(load_library().pkv_extend(cache, s.ctypes.data, len(s), n_new, first.ctypes.data))
    return first


def pkv_free_seq(cache, seq):
    _check(load_library().pkv_free_seq(cache, seq))


def pkv_table_width(cache) -> int:
    return load_library().pkv_table_width(cache)


def pkv_block_table(cache, seqs, max_blocks_per_seq=None):
    """Returns (int32 table of 16-token planes [n][pkv_table_width], int64
    lens [n]); max_blocks_per_seq, if given, must match the cache's width."""
    import numpy as np
    s = np.ascontiguousarray(seqs, dtype=np.int32)
    width = pkv_table_width(cache)
    if max_blocks_per_seq is not None and max_blocks_per_seq != width:
        raise ValueError("table width is %d, not %d" % (width, max_blocks_per_seq))
    table = np.empty((len(s), width), dtype=np.int32)
    lens = np.empty(len(s), dtype=np.int64)
    _check(load_library().pkv_block_table(cache, s.ctypes.data, len(s), table.ctypes.data,
                                          lens.ctypes.data))
    return table, lens


def pkv_num_free_blocks(cache) -> int:
    return load_library().pkv_num_free_blocks(cache)


def pkv_free_list(cache):
    import numpy as np
    n = pkv_num_free_blocks(cache)
    out = np.empty(max(n, 1), dtype=np.int32)
    got = _check(load_library().pkv_free_list(cache, out.ctypes.data, n))
    return out[:got].tolist()


# ---------------------------------------------------------------------------
# Sharing: fork, copy-on-write copies, prefix cache
# ---------------------------------------------------------------------------
def pkv_fork(cache, src_seq, dst_seq):
    _check(load_library().pkv_fork(cache, src_seq, dst_seq))


def pkv_block_refcount(cache, block) -> int:
    return _check(load_library().pkv_block_refcount(cache, block))


def pkv_pending_copies(cache):
    """Queued copy-on-write pairs as a list of (src, dst), oldest first."""
    import numpy as np
    lib = load_library()
    n = _check(lib.pkv_pending_copies(cache, None, 0))
    out = np.empty((max(n, 1), 2), dtype=np.int32)
    _check(lib.pkv_pending_copies(cache, out.ctypes.data, n))
    return [tuple(int(x) for x in r) for r in out[:n]]


def pkv_copy_blocks(cache, pool, stream=None):
    _check(load_library().pkv_copy_blocks(cache, ctypes.byref(pool), _stream(stream)))


def _keys(keys):
    import numpy as np
    return np.ascontiguousarray(np.asarray(keys, dtype=np.uint64).reshape(-1))


def pkv_prefix_match(cache, seq, keys) -> int:
    """Share the longest cached chain matching ``keys``; returns matched tokens."""
    k = _keys(keys)
    out = ctypes.c_int64(0)
    _check(load_library().pkv_prefix_match(cache, seq, k.ctypes.data if len(k) else None,
                                           len(k), ctypes.byref(out)))
    return int(out.value)


def pkv_prefix_commit(cache, seq, keys):
    k = _keys(keys)
    _check(load_library().pkv_prefix_commit(cache, seq, k.ctypes.data if len(k) else None,
                                            len(k)))


def pkv_prefix_cached_blocks(cache) -> int:
    return load_library().pkv_prefix_cached_blocks(cache)


def pkv_trim_window(cache, seqs, window) -> int:
    """Drop blocks wholly before each sequence's last ``window`` positions;
    returns the number of table entries dropped."""
    import numpy as np
    s = np.ascontiguousarray(seqs, dtype=np.int32)
    out = ctypes.c_int64(0)
    _check(load_library().pkv_trim_window(cache, s.ctypes.data if len(s) else None, len(s),
                                          window, ctypes.byref(out)))
    return int(out.value)


# ---------------------------------------------------------------------------
# Rotary table
# ---------------------------------------------------------------------------
def pkv_rope_table(head_dim, base, max_pos):
    """Returns (cos, sin) as float32 numpy arrays [max_pos][head_dim/2]."""
    import numpy as np
    cos = np.empty((max_pos, head_dim // 2), dtype=np.float32)
    sin = np.empty((max_pos, head_dim // 2), dtype=np.float32)
    _check(load_library().pkv_rope_table(head_dim, base, max_pos, cos.ctypes.data,
                                         sin.ctypes.data))
    return cos, sin


# ---------------------------------------------------------------------------
# Descriptors
# ---------------------------------------------------------------------------
def make_pool(k, v, n_layers, num_blocks, n_kv_heads, head_dim, dtype,
              layer_stride, block_stride, head_stride, k_scale=None, v_scale=None,
              scale_mode=0) -> pkv_pool:
    """scale_mode (fp8 pools): 0 scales per (layer, KV head), 1 per (layer,
    block, KV head)."""
    return pkv_pool(n_layers, num_blocks, n_kv_heads, head_dim, DTYPE_CODES[dtype], scale_mode,
                    _ptr(k), _ptr(v), layer_stride, block_stride, head_stride, _ptr(k_scale),
                    _ptr(v_scale))


def make_src(k, v, layer_stride, token_stride, n_tokens, dtype=None) -> pkv_src:
    """dtype defaults to the torch dtype of k ("f32", "bf16", "f16")."""
    if dtype is None:
        dtype = {"torch.float32": "f32", "torch.bfloat16": "bf16",
                 "torch.float16": "f16"}[str(k.dtype)]
    return pkv_src(_ptr(k), _ptr(v), layer_stride, token_stride, n_tokens, DTYPE_CODES[dtype], 0)


def _dtype_of(t, default):
    if t is None or not hasattr(t, "dtype"):
        return default
    return {"torch.float32": PKV_F32, "torch.bfloat16": PKV_BF16,
            "torch.float16": PKV_F16}.get(str(t.dtype), default)


def make_runs(runs):
    arr = (pkv_run * max(1, len(runs)))()
    for i, (seq, n, pos, src) in enumerate(runs):
        arr[i] = pkv_run(int(seq), int(n), int(pos), 0, int(src))
    return arr


# ---------------------------------------------------------------------------
# Inject / append
# ---------------------------------------------------------------------------
def pkv_inject_workspace_bytes(runs) -> int:
    arr = runs if isinstance(runs, ctypes.Array) else make_runs(runs)
    return load_library().pkv_inject_workspace_bytes(arr, len(arr))


def pkv_host_alloc(n_bytes) -> int:
    """Pinned host memory of exactly n_bytes; returns its address."""
    out = _P()
    _check(load_library().pkv_host_alloc(int(n_bytes), ctypes.byref(out)))
    return int(out.value)


def pkv_host_free(addr):
    _check(load_library().pkv_host_free(addr))


def host_view(addr, n_bytes):
    """uint8 numpy view of n_bytes of host memory at addr (no copy)."""
    import numpy as np
    return np.ctypeslib.as_array((ctypes.c_uint8 * int(n_bytes)).from_address(int(addr)))


def pkv_inject(cache, pool: pkv_pool, src: pkv_src, runs, layer_begin, layer_end, rope_mode,
               cos, sin, max_pos, workspace, stream=None):
    arr = runs if isinstance(runs, ctypes.Array) else make_runs(runs)
    n = len(arr) if not isinstance(runs, (list, tuple)) else len(runs)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load_library().pkv_inject(cache, ctypes.byref(pool), ctypes.byref(src), arr, n,
                                     layer_begin, layer_end, ROPE_CODES.get(rope_mode, rope_mode),
                                     _ptr(cos), _ptr(sin), max_pos, _ptr(workspace), ws_bytes,
                                     _stream(stream)))


def pkv_append_kv(pool: pkv_pool, layer, tables, first_pos, n_new, k_new, v_new, rope_mode,
                  cos, sin, max_pos, stream=None, new_dtype=None):
    """new_dtype defaults to the torch dtype of k_new."""
    nd = DTYPE_CODES[new_dtype] if isinstance(new_dtype, str) else _dtype_of(k_new, pool.dtype)
    _check(load_library().pkv_append_kv(ctypes.byref(pool), layer, _ptr(tables),
                                        tables.shape[1], _ptr(first_pos), first_pos.shape[0],
                                        n_new, _ptr(k_new), _ptr(v_new), nd,
                                        ROPE_CODES.get(rope_mode, rope_mode), _ptr(cos), _ptr(sin),
                                        max_pos, _stream(stream)))


# ---------------------------------------------------------------------------
# Decode
# ---------------------------------------------------------------------------
def pkv_decode_plan_create(lens, n_q_heads, n_kv_heads, head_dim, part_tokens=0, window=0):
    """window > 0: each sequence attends to its last ``window`` positions."""
    import numpy as np
    a = np.ascontiguousarray(lens, dtype=np.int64)
    h = ctypes.c_void_p()
    _check(load_library().pkv_decode_plan_create(a.ctypes.data, len(a), n_q_heads, n_kv_heads,
                                                 head_dim, part_tokens, window, ctypes.byref(h)))
    return h


def pkv_decode_plan_destroy(plan):
    load_library().pkv_decode_plan_destroy(plan)


def pkv_decode_plan_items(plan) -> int:
    return load_library().pkv_decode_plan_items(plan)


def pkv_decode_plan_part_tokens(plan) -> int:
    return load_library().pkv_decode_plan_part_tokens(plan)


def pkv_decode_plan_waves(plan) -> int:
    return load_library().pkv_decode_plan_waves(plan)


def pkv_decode_workspace_bytes(plan) -> int:
    return load_library().pkv_decode_workspace_bytes(plan)


def pkv_decode_plan_upload(plan, workspace, stream=None):
    _check(load_library().pkv_decode_plan_upload(plan, _ptr(workspace),
                                                 workspace.numel() * workspace.element_size(),
                                                 _stream(stream)))


def pkv_decode_attention(plan, pool: pkv_pool, layer, q, tables, out, lse, workspace,
                         scale=0.0, stream=None, q_dtype=None):
    """q_dtype defaults to the torch dtype of q."""
    qd = DTYPE_CODES[q_dtype] if isinstance(q_dtype, str) else _dtype_of(q, pool.dtype)
    _check(load_library().pkv_decode_attention(plan, ctypes.byref(pool), layer, _ptr(q), qd,
                                               float(scale), _ptr(tables), tables.shape[1],
                                               _ptr(out), _ptr(lse), _ptr(workspace),
                                               workspace.numel() * workspace.element_size(),
                                               _stream(stream)))


def pkv_append_decode_attention(plan, pool: pkv_pool, layer, q, tables, k_new, v_new, rope_mode,
                                cos, sin, max_pos, out, lse, workspace, scale=0.0, stream=None,
                                q_dtype=None):
    """k_new, v_new: [n_seqs][n_kv_heads][head_dim] in q's format (q_dtype
    defaults to the torch dtype of q)."""
    qd = DTYPE_CODES[q_dtype] if isinstance(q_dtype, str) else _dtype_of(q, pool.dtype)
    _check(load_library().pkv_append_decode_attention(
        plan, ctypes.byref(pool), layer, _ptr(q), qd, float(scale), _ptr(tables), tables.shape[1],
        _ptr(k_new), _ptr(v_new), ROPE_CODES.get(rope_mode, rope_mode), _ptr(cos), _ptr(sin),
        max_pos, _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


def pkv_append_decode_attention_noalloc(plan, pool: pkv_pool, layer, q, tables, k_new, v_new,
                                        rope_mode, cos, sin, max_pos, out, lse, scale=0.0,
                                        stream=None, q_dtype=None):
    """The decode step with the library's static device scratch as its
    workspace (no workspace argument, no plan upload)."""
    qd = DTYPE_CODES[q_dtype] if isinstance(q_dtype, str) else _dtype_of(q, pool.dtype)
    _check(load_library().pkv_append_decode_attention_noalloc(
        plan, ctypes.byref(pool), layer, _ptr(q), qd, float(scale), _ptr(tables), tables.shape[1],
        _ptr(k_new), _ptr(v_new), ROPE_CODES.get(rope_mode, rope_mode), _ptr(cos), _ptr(sin),
        max_pos, _ptr(out), _ptr(lse), _stream(stream)))


def pkv_kernel_timing(enable: bool):
    _check(load_library().pkv_kernel_timing(1 if enable else 0))


def pkv_kernel_times(max_n=1 << 20):
    """Durations (ms, numpy float32) of the decode launches recorded since
    timing was switched on; releases them."""
    import numpy as np
    buf = np.empty(max_n, dtype=np.float32)
    n = _check(load_library().pkv_kernel_times(buf.ctypes.data, max_n))
    return buf[:min(n, max_n)].copy()


def pkv_bw_probe(src, sink, stream=None):
    _check(load_library().pkv_bw_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                       _stream(stream)))


# ---------------------------------------------------------------------------
# Object facade over the allocator handle (marshalling only; every method is
# the C entry point of the same name without the "pkv_" prefix).
# ---------------------------------------------------------------------------
class Cache:
    """A ``pkv_cache`` handle: host allocator, tables, sharing, prefix cache.

    ``Cache(num_blocks, max_seqs, max_blocks_per_seq, free_list_seed=0,
    block_tokens=16)``; release with ``close()`` (or use it in ``with``)."""

    def __init__(self, num_blocks, max_seqs, max_blocks_per_seq, free_list_seed=0,
                 block_tokens=16):
        self.handle = pkv_cache_create(num_blocks, max_seqs, max_blocks_per_seq, free_list_seed,
                                       block_tokens)

    def close(self):
        if self.handle is not None:
            pkv_cache_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc_blocks(self, seq, n_tokens):
        pkv_alloc_blocks(self.handle, seq, n_tokens)

    def set_blocks(self, seq, ids, length):
        pkv_set_blocks(self.handle, seq, ids, length)

    def extend(self, seqs, n_new):
        return pkv_extend(self.handle, seqs, n_new)

    def free_seq(self, seq):
        pkv_free_seq(self.handle, seq)

    def block_table(self, seqs):
        return pkv_block_table(self.handle, seqs)

    def table_width(self):
        return pkv_table_width(self.handle)

    def num_free_blocks(self):
        return pkv_num_free_blocks(self.handle)

    def free_list(self):
        return pkv_free_list(self.handle)

    def fork(self, src_seq, dst_seq):
        pkv_fork(self.handle, src_seq, dst_seq)

    def block_refcount(self, block):
        return pkv_block_refcount(self.handle, block)

    def pending_copies(self):
        return pkv_pending_copies(self.handle)

    def copy_blocks(self, pool, stream=None):
        pkv_copy_blocks(self.handle, pool, stream)

    def prefix_match(self, seq, keys):
        return pkv_prefix_match(self.handle, seq, keys)

    def prefix_commit(self, seq, keys):
        pkv_prefix_commit(self.handle, seq, keys)

    def prefix_cached_blocks(self):
        return pkv_prefix_cached_blocks(self.handle)

    def trim_window(self, seqs, window):
        return pkv_trim_window(self.handle, seqs, window)

    def inject(self, pool, src, runs, layer_begin, layer_end, rope_mode, cos, sin, max_pos,
               workspace, stream=None):
        pkv_inject(self.handle, pool, src, runs, layer_begin, layer_end, rope_mode, cos, sin,
                   max_pos, workspace, stream)
