"""Python binding of libpagedkv (paged KV cache + decode attention on MI355X).

Argument marshalling only: every computation runs in the HIP kernels of
libpagedkv.so, and every bookkeeping step in its C++ host core.  PyTorch
provides device memory and streams.  If the library is not built, importing
this package still works but the first call raises ``LibraryMissing``; there is
no fallback implementation.

The names follow the C ABI (include/pagedkv.h): ``kv_pool_create``,
``kv_append``, ``paged_decode``, ... ; ``KVPool`` wraps a pool handle.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

F32, F16, BF16, FP8_E4M3, INT8_MINMAX = 0, 1, 2, 3, 4
OK, ERR_INVALID_ARG, ERR_NO_BLOCKS, ERR_OUT_OF_RANGE, ERR_STATE, ERR_UNSUPPORTED, ERR_DEVICE = range(7)
BLOCK = 16
NOALLOC_SCRATCH_BYTES = 32 << 20   # PKV_NOALLOC_SCRATCH_BYTES of include/pagedkv.h

_lib = None


class LibraryMissing(ImportError):
    pass


class PagedKVError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where} failed with status {code}: {msg}")
        self.code = code


class PoolInfo(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("pool_bytes", ctypes.c_uint64), ("block_bytes", ctypes.c_uint64),
                ("total_bytes", ctypes.c_uint64),
                ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("elem_bytes", ctypes.c_int32),
                ("free_blocks", ctypes.c_int32), ("used_blocks", ctypes.c_int32),
                ("shared_blocks", ctypes.c_int32), ("live_seqs", ctypes.c_int32),
                ("host_only", ctypes.c_int32), ("partition_tokens", ctypes.c_int32),
                ("cached_blocks", ctypes.c_int32), ("evictable_blocks", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class KernelStat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64),
                ("dropped", ctypes.c_int64), ("total_ms", ctypes.c_double)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_PI32 = ctypes.POINTER(ctypes.c_int32)

_SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "kv_cache_bytes": (ctypes.c_uint64, [_I32, _I32, _I32, _I32, ctypes.c_int64, ctypes.c_int64]),
    "kv_pool_create": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _P, ctypes.POINTER(_P)]),
    "kv_pool_create_host_only": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _P, ctypes.POINTER(_P)]),
    "kv_pool_destroy": (ctypes.c_int, [_P]),
    "kv_pool_info": (ctypes.c_int, [_P, ctypes.POINTER(PoolInfo)]),
    "kv_pool_set_fp8_scales": (ctypes.c_int, [_P, _P, _P]),
    "kv_seq_create": (ctypes.c_int, [_P, _PI32]),
    "kv_seq_reserve": (ctypes.c_int, [_P, _I32, _I32, _P]),
    "kv_batch_reserve": (ctypes.c_int, [_P, _P, _I32, _P, _P]),
    "kv_seq_fork": (ctypes.c_int, [_P, _I32, _I32, _PI32]),
    "kv_seq_free": (ctypes.c_int, [_P, _I32]),
    "kv_block_hash": (ctypes.c_uint64, [ctypes.c_uint64, ctypes.c_uint64, _P]),
    "kv_prefix_register": (ctypes.c_int, [_P, _I32, _P, _I32, ctypes.c_uint64, _PI32]),
    "kv_seq_create_cached": (ctypes.c_int, [_P, _P, _I32, ctypes.c_uint64, _PI32, _PI32]),
    "kv_prefix_evict_all": (ctypes.c_int, [_P]),
    "kv_pending_copies": (ctypes.c_int, [_P, _P, _P, _I32, _PI32]),
    "kv_apply_copies": (ctypes.c_int, [_P, _P]),
    "kv_seq_length": (ctypes.c_int, [_P, _I32, _PI32]),
    "kv_block_tables": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P]),
    "kv_block_refcount": (ctypes.c_int, [_P, _I32, _PI32]),
    "kv_free_list": (ctypes.c_int, [_P, _P, _I32, _PI32]),
    "kv_append": (ctypes.c_int, [_P, _P, _I32, _P, _P, _I32, _P]),
    "paged_decode": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _I32, _P, _I32, ctypes.c_float,
                                    _P, _P, ctypes.c_size_t, _P]),
    "paged_decode_noalloc": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _I32, _P, _I32, ctypes.c_float,
                                            _P, _P]),
    "paged_decode_workspace_bytes": (ctypes.c_size_t, [_P, _I32, _I32, _I32]),
    "kv_seq_swap_bytes": (ctypes.c_int, [_P, _I32, ctypes.POINTER(ctypes.c_size_t)]),
    "kv_seq_swap_out": (ctypes.c_int, [_P, _I32, _P, ctypes.c_size_t, _P]),
    "kv_seq_swap_in": (ctypes.c_int, [_P, _I32, _P, ctypes.c_size_t, _P]),
    "paged_prefill": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _I32, _I32, _P, _I32, _P, ctypes.c_float,
                                     _I32, _P, _P]),
    "paged_decode_set_partition": (ctypes.c_int, [_P, _I32]),
    "paged_decode_partition_tokens": (ctypes.c_int32, [_P, _I32, _I32, _I32]),
    "kv_pool_copy_to_host": (ctypes.c_int, [_P, _P, _P]),
    "pkv_profile_enable": (ctypes.c_int, [_P, _I32]),
    "pkv_profile_read": (ctypes.c_int, [_P, ctypes.POINTER(KernelStat), _I32, _PI32]),
    "pkv_copy": (ctypes.c_int, [_P, _P, ctypes.c_size_t, _P]),
    "pkv_read_probe": (ctypes.c_int, [_P, ctypes.c_size_t, _I32, _P, ctypes.c_int64, _I32, _P, _P]),
}
EXPORTED = tuple(_SIGNATURES)


def lib():
    """The loaded libpagedkv.so (raises LibraryMissing if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                                 "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().pkv_last_error().decode()


def _check(rc: int, where: str) -> None:
    if rc != OK:
        raise PagedKVError(rc, where, last_error())


def kv_cache_bytes(layers, kv_heads, head_dim, elem_bytes, tokens=1, seqs=1) -> int:
    return int(lib().kv_cache_bytes(layers, kv_heads, head_dim, elem_bytes, tokens, seqs))


def kv_block_hash(parent: int, ns: int, tokens) -> int:
    t, tp = _np_i32(tokens)
    if len(t) != BLOCK:
        raise ValueError("a block has 16 tokens")
    return int(lib().kv_block_hash(parent, ns, tp))


# --------------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


_TORCH_DTYPES = None


def torch_dtype(code: int):
    global _TORCH_DTYPES
    torch = _torch()
    if _TORCH_DTYPES is None:
        _TORCH_DTYPES = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16,
                         FP8_E4M3: torch.uint8, INT8_MINMAX: torch.uint8}
    return _TORCH_DTYPES[code]


def dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.uint8: FP8_E4M3,
         torch.float8_e4m3fn: FP8_E4M3}
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name, dtype=None, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _np_i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------- pool
class KVPool:
    """A block pool (kv_pool_t) and its sequences."""

    def __init__(self, num_blocks, kv_heads, head_dim, dtype, block_size=BLOCK, free_order=None,
                 host_only=False):
        handle = ctypes.c_void_p()
        order_ptr = None
        if free_order is not None:
            self._order, order_ptr = _np_i32(free_order)
            if self._order.shape != (num_blocks,):
                raise ValueError("free_order must have num_blocks entries")
        fn = lib().kv_pool_create_host_only if host_only else lib().kv_pool_create
        _check(fn(num_blocks, block_size, kv_heads, head_dim, dtype, order_ptr, ctypes.byref(handle)),
               "kv_pool_create")
        self.handle = handle
        self.num_blocks, self.kv_heads, self.head_dim, self.dtype = num_blocks, kv_heads, head_dim, dtype
        self.block_size = block_size
        self.host_only = host_only

    # -- lifetime
    def close(self):
        if getattr(self, "handle", None):
            _check(lib().kv_pool_destroy(self.handle), "kv_pool_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- metadata
    def info(self) -> dict:
        inf = PoolInfo()
        _check(lib().kv_pool_info(self.handle, ctypes.byref(inf)), "kv_pool_info")
        return inf.as_dict()

    def set_fp8_scales(self, k_scale, v_scale):
        k = np.ascontiguousarray(k_scale, dtype=np.float32)
        v = np.ascontiguousarray(v_scale, dtype=np.float32)
        if k.shape != (self.kv_heads,) or v.shape != (self.kv_heads,):
            raise ValueError("one scale per KV head")
        _check(lib().kv_pool_set_fp8_scales(self.handle, k.ctypes.data_as(_P), v.ctypes.data_as(_P)),
               "kv_pool_set_fp8_scales")

    def seq_create(self) -> int:
        sid = ctypes.c_int32()
        _check(lib().kv_seq_create(self.handle, ctypes.byref(sid)), "kv_seq_create")
        return sid.value

    def seq_reserve(self, seq: int, n_tokens: int) -> np.ndarray:
        slots = np.empty(max(n_tokens, 0), np.int32)
        _check(lib().kv_seq_reserve(self.handle, seq, n_tokens, slots.ctypes.data_as(_P) if n_tokens > 0 else None),
               "kv_seq_reserve")
        return slots

    def batch_reserve(self, seqs, n_tokens=None) -> np.ndarray:
        """kv_batch_reserve: slots for every (sequence, count), concatenated in order."""
        s, sp = _np_i32(seqs)
        if n_tokens is None:
            total, cp = len(s), None
        else:
            c, cp = _np_i32(n_tokens)
            if c.shape != s.shape:
                raise ValueError("one count per sequence")
            total = int(c.sum())
        slots = np.empty(max(total, 1), np.int32)
        _check(lib().kv_batch_reserve(self.handle, sp, len(s), cp, slots.ctypes.data_as(_P)), "kv_batch_reserve")
        return slots[:total]

    def seq_fork(self, parent: int, n_shared_tokens: int) -> int:
        child = ctypes.c_int32()
        _check(lib().kv_seq_fork(self.handle, parent, n_shared_tokens, ctypes.byref(child)), "kv_seq_fork")
        return child.value

    def prefix_register(self, seq: int, tokens, ns: int = 0) -> int:
        """kv_prefix_register: publish seq's full blocks holding tokens; returns how many were new."""
        t, tp = _np_i32(tokens)
        n = ctypes.c_int32()
        _check(lib().kv_prefix_register(self.handle, seq, tp if len(t) else None, len(t), ns, ctypes.byref(n)),
               "kv_prefix_register")
        return n.value

    def seq_create_cached(self, tokens, ns: int = 0):
        """kv_seq_create_cached: (seq, cached tokens) starting on the longest cached prefix."""
        t, tp = _np_i32(tokens)
        sid, hit = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().kv_seq_create_cached(self.handle, tp if len(t) else None, len(t), ns, ctypes.byref(sid),
                                          ctypes.byref(hit)), "kv_seq_create_cached")
        return sid.value, hit.value

    def prefix_evict_all(self) -> None:
        _check(lib().kv_prefix_evict_all(self.handle), "kv_prefix_evict_all")

    def pending_copies(self):
        """Copy-on-write block copies owed to the device: list of (src, dst)."""
        n = ctypes.c_int32()
        cap = self.num_blocks
        src = np.empty(cap, np.int32)
        dst = np.empty(cap, np.int32)
        _check(lib().kv_pending_copies(self.handle, src.ctypes.data_as(_P), dst.ctypes.data_as(_P), cap,
                                       ctypes.byref(n)), "kv_pending_copies")
        return list(zip(src[: n.value].tolist(), dst[: n.value].tolist()))

    def apply_copies(self, stream=None) -> None:
        _check(lib().kv_apply_copies(self.handle, None if self.host_only else _stream(stream)), "kv_apply_copies")

    def seq_free(self, seq: int) -> None:
        _check(lib().kv_seq_free(self.handle, seq), "kv_seq_free")

    def seq_length(self, seq: int) -> int:
        n = ctypes.c_int32()
        _check(lib().kv_seq_length(self.handle, seq, ctypes.byref(n)), "kv_seq_length")
        return n.value

    def block_tables(self, seqs, max_blocks_per_seq: int):
        s, sp = _np_i32(seqs)
        tables = np.empty((len(s), max_blocks_per_seq), np.int32)
        lens = np.empty(len(s), np.int32)
        _check(lib().kv_block_tables(self.handle, sp, len(s), max_blocks_per_seq,
                                     tables.ctypes.data_as(_P), lens.ctypes.data_as(_P)), "kv_block_tables")
        return tables, lens

    def block_refcount(self, block: int) -> int:
        n = ctypes.c_int32()
        _check(lib().kv_block_refcount(self.handle, block, ctypes.byref(n)), "kv_block_refcount")
        return n.value

    def free_list(self) -> np.ndarray:
        out = np.empty(self.num_blocks, np.int32)
        n = ctypes.c_int32()
        _check(lib().kv_free_list(self.handle, out.ctypes.data_as(_P), self.num_blocks, ctypes.byref(n)),
               "kv_free_list")
        return out[: n.value].copy()

    # -- device work
    def append(self, slot_mapping, k_new, v_new, stream=None):
        """kv_append: slot_mapping int32 [T], k_new/v_new [T][kv_heads][head_dim] on the device."""
        torch = _torch()
        T = int(slot_mapping.shape[0])
        shape = (T, self.kv_heads, self.head_dim)
        sp = _dev(slot_mapping, "slot_mapping", torch.int32)
        kp = _dev(k_new, "k_new", shape=shape)
        vp = _dev(v_new, "v_new", dtype=k_new.dtype, shape=shape)
        _check(lib().kv_append(self.handle, sp, T, kp, vp, dtype_code(k_new), _stream(stream)), "kv_append")

    def workspace_bytes(self, B: int, H_q: int, max_context_len: int) -> int:
        return int(lib().paged_decode_workspace_bytes(self.handle, B, H_q, max_context_len))

    def partition_tokens(self, B: int, H_q: int, max_context_len: int) -> int:
        return int(lib().paged_decode_partition_tokens(self.handle, B, H_q, max_context_len))

    def set_partition(self, tokens: int) -> None:
        _check(lib().paged_decode_set_partition(self.handle, tokens), "paged_decode_set_partition")

    def decode(self, q, block_tables, context_lens, max_context_len: int, scale: float, out=None,
               workspace=None, stream=None):
        """paged_decode: q [B][H_q][head_dim] -> out of the same shape and dtype."""
        torch = _torch()
        B, H_q, D = (int(x) for x in q.shape)
        if D != self.head_dim:
            raise ValueError("q head_dim does not match the pool")
        if out is None:
            out = torch.empty_like(q)
        qp = _dev(q, "q")
        op = _dev(out, "out", dtype=q.dtype, shape=q.shape)
        tp = _dev(block_tables, "block_tables", torch.int32)
        if block_tables.dim() != 2 or block_tables.shape[0] != B:
            raise ValueError("block_tables must be [B][max_blocks_per_seq]")
        lp = _dev(context_lens, "context_lens", torch.int32, shape=(B,))
        need = self.workspace_bytes(B, H_q, max_context_len)
        if need and workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        wp = _dev(workspace, "workspace") if workspace is not None else None
        wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        _check(lib().paged_decode(self.handle, qp, dtype_code(q), B, H_q, tp, int(block_tables.shape[1]), lp,
                                  int(max_context_len), float(scale), op, wp, wbytes, _stream(stream)),
               "paged_decode")
        return out

    def decode_noalloc(self, q, block_tables, context_lens, max_context_len: int, scale: float, out=None,
                       stream=None):
        """paged_decode_noalloc: as decode(), with the library's fixed device
        scratch instead of a workspace (the call itself allocates nothing; an
        `out` of None is allocated here, before the call)."""
        torch = _torch()
        B, H_q, D = (int(x) for x in q.shape)
        if D != self.head_dim:
            raise ValueError("q head_dim does not match the pool")
        if out is None:
            out = torch.empty_like(q)
        qp = _dev(q, "q")
        op = _dev(out, "out", dtype=q.dtype, shape=q.shape)
        tp = _dev(block_tables, "block_tables", torch.int32)
        if block_tables.dim() != 2 or block_tables.shape[0] != B:
            raise ValueError("block_tables must be [B][max_blocks_per_seq]")
        lp = _dev(context_lens, "context_lens", torch.int32, shape=(B,))
        _check(lib().paged_decode_noalloc(self.handle, qp, dtype_code(q), B, H_q, tp, int(block_tables.shape[1]), lp,
                                          int(max_context_len), float(scale), op, _stream(stream)),
               "paged_decode_noalloc")
        return out

    def swap_bytes(self, seq: int) -> int:
        n = ctypes.c_size_t()
        _check(lib().kv_seq_swap_bytes(self.handle, seq, ctypes.byref(n)), "kv_seq_swap_bytes")
        return n.value

    def swap_out(self, seq: int, host=None, stream=None):
        """kv_seq_swap_out into `host` (a CPU tensor, pinned is fastest; allocated
        pinned if None; none on a metadata-only pool).  Returns the host tensor."""
        torch = _torch()
        nbytes = self.swap_bytes(seq)
        if host is None and not self.host_only:
            host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        ptr, size = (None, 0) if host is None else (ctypes.c_void_p(host.data_ptr()), host.numel() * host.element_size())
        if host is not None and (host.is_cuda or not host.is_contiguous()):
            raise ValueError("host must be a contiguous CPU tensor")
        _check(lib().kv_seq_swap_out(self.handle, seq, ptr, size, None if self.host_only else _stream(stream)),
               "kv_seq_swap_out")
        return host

    def swap_in(self, seq: int, host=None, stream=None) -> None:
        ptr, size = (None, 0) if host is None else (ctypes.c_void_p(host.data_ptr()), host.numel() * host.element_size())
        if host is not None and (host.is_cuda or not host.is_contiguous()):
            raise ValueError("host must be a contiguous CPU tensor")
        _check(lib().kv_seq_swap_in(self.handle, seq, ptr, size, None if self.host_only else _stream(stream)),
               "kv_seq_swap_in")

    def prefill(self, q, q_start, block_tables, context_lens, max_q_len: int, scale: float, causal: bool = True,
                out=None, stream=None):
        """paged_prefill: q [total_q][H_q][head_dim], sequence s owning query rows
        q_start[s] .. q_start[s+1]-1 (its last positions) -> out of the same shape."""
        torch = _torch()
        T, H_q, D = (int(x) for x in q.shape)
        if D != self.head_dim:
            raise ValueError("q head_dim does not match the pool")
        if out is None:
            out = torch.empty_like(q)
        n = int(context_lens.shape[0])
        qp = _dev(q, "q")
        op = _dev(out, "out", dtype=q.dtype, shape=q.shape)
        sp = _dev(q_start, "q_start", torch.int32, shape=(n + 1,))
        tp = _dev(block_tables, "block_tables", torch.int32)
        if block_tables.dim() != 2 or block_tables.shape[0] != n:
            raise ValueError("block_tables must be [n_seqs][max_blocks]")
        lp = _dev(context_lens, "context_lens", torch.int32, shape=(n,))
        _check(lib().paged_prefill(self.handle, qp, dtype_code(q), n, H_q, sp, T, int(max_q_len), tp,
                                   int(block_tables.shape[1]), lp, float(scale), 1 if causal else 0, op,
                                   _stream(stream)), "paged_prefill")
        return out

    def copy_to_host(self):
        """(K, V) pool contents as uint8 numpy arrays of pool_bytes each."""
        nbytes = self.info()["pool_bytes"]
        k = np.empty(nbytes, np.uint8)
        v = np.empty(nbytes, np.uint8)
        _check(lib().kv_pool_copy_to_host(self.handle, k.ctypes.data_as(_P), v.ctypes.data_as(_P)),
               "kv_pool_copy_to_host")
        return k, v

    def profile_enable(self, on: bool = True) -> None:
        _check(lib().pkv_profile_enable(self.handle, 1 if on else 0), "pkv_profile_enable")

    def profile_read(self) -> dict:
        arr = (KernelStat * 16)()
        n = ctypes.c_int32()
        _check(lib().pkv_profile_read(self.handle, arr, 16, ctypes.byref(n)), "pkv_profile_read")
        return {arr[i].name.decode(): {"launches": arr[i].launches, "dropped": arr[i].dropped,
                                       "total_ms": arr[i].total_ms} for i in range(n.value)}


def copy(dst, src, stream=None) -> None:
    """pkv_copy: plain 16-byte device copy of src into dst (same byte size)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("size mismatch")
    _check(lib().pkv_copy(_dev(dst, "dst"), _dev(src, "src"), nbytes, _stream(stream)), "pkv_copy")


def read_probe(src, sink, nontemporal: bool, order=None, chunk_bytes: int = 0, stream=None) -> None:
    """pkv_read_probe: read src (plain or nontemporal 16-byte loads), in address
    order, or chunk by chunk in the order of the device int32 tensor `order`
    (chunks of chunk_bytes), and XOR the XOR of the 32-bit words read into
    sink (a device int32 tensor of one element)."""
    torch = _torch()
    if order is None:
        optr, n_order = None, 0
    else:
        optr, n_order = _dev(order, "order", torch.int32), order.numel()
    _check(lib().pkv_read_probe(_dev(src, "src"), src.numel() * src.element_size(), int(bool(nontemporal)),
                                optr, n_order, int(chunk_bytes), _dev(sink, "sink", torch.int32, (1,)),
                                _stream(stream)), "pkv_read_probe")


# C-ABI names as plain functions over a KVPool.
def kv_pool_create(num_blocks, block_size, kv_heads, head_dim, dtype, initial_free_order=None) -> KVPool:
    return KVPool(num_blocks, kv_heads, head_dim, dtype, block_size=block_size, free_order=initial_free_order)


def kv_append(pool: KVPool, slot_mapping, k_new, v_new, stream=None):
    return pool.append(slot_mapping, k_new, v_new, stream)


def paged_decode(pool: KVPool, q, block_tables, context_lens, max_context_len, scale, out=None,
                 workspace=None, stream=None):
    return pool.decode(q, block_tables, context_lens, max_context_len, scale, out, workspace, stream)


def paged_decode_noalloc(pool: KVPool, q, block_tables, context_lens, max_context_len, scale, out=None,
                         stream=None):
    return pool.decode_noalloc(q, block_tables, context_lens, max_context_len, scale, out, stream)
