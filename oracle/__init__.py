"""fp64 CPU oracle for paged decode attention -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
this package never imports the product: the two share no code.

Contents
  * ``liboracle.so`` (built from ``oracle.c`` by ``oracle/build.py``): the KV
    size formula, exact widening of f16/bf16/E4M3 to double, the OCP E4M3
    encoder, and two-pass fp64 decode attention over de-paged K/V.
  * ``causal_attention`` below: full no-cache causal attention (every query
    row attends to all earlier rows), the "recompute everything" path that the
    cached decode must reproduce.
  * ``allocator_model``: a pure-Python model of the block pool allocator.
  * ``int8_minmax``: the INT8 per-block min-max codes, their values, and a
    model of the tiles as appends leave them.

Pins (checked by the CPU tests, never by the oracle against itself):
  kv_cache_bytes   -- numbers the pages print (tests/golden/kv_sizes.json)
  f16/bf16 widen   -- numpy float16 and torch bfloat16 on all 65536 patterns
  E4M3 decode      -- torch.float8_e4m3fn on all 256 codes; spec constants
  E4M3 encode      -- torch's RNE cast inside the finite range; saturation
                      and NaN from the specification
  INT8 min-max     -- the page's formula on closed-form inputs, the half-step
                      round-trip bound, range = min/max of the raw inputs since
                      row 0, untouched rows when the range holds, and the
                      re-encode error bound over whole fill sequences
  decode attention -- numpy textbook softmax, closed forms (single token,
                      two tokens, q = 0, constant V), GQA == repeated-KV MHA,
                      cached decode == causal recompute
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import allocator_model  # noqa: F401  (re-exported)
from . import int8_minmax  # noqa: F401  (re-exported)

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "liboracle.so")

F32, F16, BF16, E4M3 = 0, 1, 2, 3
F64 = 5     # K/V given as fp64 values (INT8 pools: the values their codes stand for)
_NP_STORAGE = {F32: np.float32, F16: np.float16, BF16: np.uint16, E4M3: np.uint8, F64: np.float64}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = bind(_LIB_PATH)
    return _lib


def bind(path: str):
    """Load an oracle shared library at `path` and declare its signatures."""
    L = ctypes.CDLL(path)
    L.oracle_kv_cache_bytes.restype = ctypes.c_uint64
    L.oracle_kv_cache_bytes.argtypes = [ctypes.c_int64] * 6
    L.oracle_f16_to_f64.restype = ctypes.c_double
    L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_to_f64.restype = ctypes.c_double
    L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.oracle_e4m3_to_f64.restype = ctypes.c_double
    L.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    L.oracle_e4m3_from_f32.restype = ctypes.c_uint8
    L.oracle_e4m3_from_f32.argtypes = [ctypes.c_float]
    L.oracle_e4m3_encode_f32_array.restype = None
    L.oracle_e4m3_encode_f32_array.argtypes = [ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_void_p, ctypes.c_int32]
    L.oracle_widen_array.restype = None
    L.oracle_widen_array.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                     ctypes.c_void_p]
    L.oracle_decode_attention.restype = ctypes.c_int
    L.oracle_decode_attention.argtypes = [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]
    L.oracle_prefill_attention.restype = ctypes.c_int
    L.oracle_prefill_attention.argtypes = [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    L.oracle_num_threads.restype = ctypes.c_int
    return L


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def kv_cache_bytes(layers, kv_heads, head_dim, elem_bytes, tokens=1, seqs=1) -> int:
    """KV size formula 2*L*H_kv*d*bytes*tokens*seqs (0 on invalid input)."""
    return int(lib().oracle_kv_cache_bytes(layers, kv_heads, head_dim, elem_bytes, tokens, seqs))


def widen(stored: np.ndarray, dtype_code: int) -> np.ndarray:
    """Exact float64 value of stored f32/f16/bf16(uint16 bits)/E4M3(uint8 codes)."""
    a = np.ascontiguousarray(stored, dtype=_NP_STORAGE[dtype_code])
    out = np.empty(a.shape, dtype=np.float64)
    lib().oracle_widen_array(_ptr(a), dtype_code, a.size, _ptr(out))
    return out


def e4m3_encode(x: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """OCP E4M3 codes of float32 values: RNE, saturating to +-448, NaN -> 0x7F."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_f32_array(_ptr(a), a.size, _ptr(out), nthreads)
    return out


def decode_attention(q: np.ndarray, q_dtype: int, K: np.ndarray, V: np.ndarray, kv_dtype: int,
                     tok_off: np.ndarray, lens: np.ndarray, scale: float, *,
                     k_scale=None, v_scale=None, nthreads: int = 0) -> np.ndarray:
    """fp64 decode attention over de-paged K/V.

    q: [B][H_q][D] storage of q_dtype; K, V: [total_tokens][H_kv][D] storage of
    kv_dtype; sequence b owns tokens tok_off[b] .. tok_off[b]+lens[b]-1.
    Returns out [B][H_q][D] float64.
    """
    q = np.ascontiguousarray(q, dtype=_NP_STORAGE[q_dtype])
    K = np.ascontiguousarray(K, dtype=_NP_STORAGE[kv_dtype])
    V = np.ascontiguousarray(V, dtype=_NP_STORAGE[kv_dtype])
    B, H_q, D = q.shape
    assert K.ndim == 3 and K.shape == V.shape and K.shape[2] == D
    H_kv = K.shape[1]
    tok_off = np.ascontiguousarray(tok_off, dtype=np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    assert tok_off.shape == (B,) and lens.shape == (B,)
    for b in range(B):
        if lens[b] > 0:
            assert 0 <= tok_off[b] and tok_off[b] + lens[b] <= K.shape[0]
    ks = vs = None
    if kv_dtype == E4M3:
        ks = np.ascontiguousarray(k_scale, dtype=np.float32)
        vs = np.ascontiguousarray(v_scale, dtype=np.float32)
        assert ks.shape == (H_kv,) and vs.shape == (H_kv,)
    out = np.empty((B, H_q, D), dtype=np.float64)
    rc = lib().oracle_decode_attention(
        B, H_q, H_kv, D, _ptr(q), q_dtype, _ptr(K), _ptr(V), kv_dtype,
        _ptr(tok_off), _ptr(lens),
        _ptr(ks) if ks is not None else None, _ptr(vs) if vs is not None else None,
        float(np.float32(scale)), nthreads, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_decode_attention rejected its arguments")
    return out


def prefill_attention(q: np.ndarray, q_dtype: int, q_start, K: np.ndarray, V: np.ndarray, kv_dtype: int,
                      tok_off, lens, scale: float, *, causal: bool = True,
                      k_scale=None, v_scale=None, nthreads: int = 0) -> np.ndarray:
    """fp64 multi-query attention over de-paged K/V (oracle_prefill_attention).

    q: [T][H_q][D] storage of q_dtype, sequence s owning query rows
    q_start[s] .. q_start[s+1]-1 (its last positions); K, V: [tokens][H_kv][D]
    storage of kv_dtype, sequence s owning tok_off[s] .. tok_off[s]+lens[s]-1.
    Returns out [T][H_q][D] float64.
    """
    q = np.ascontiguousarray(q, dtype=_NP_STORAGE[q_dtype])
    K = np.ascontiguousarray(K, dtype=_NP_STORAGE[kv_dtype])
    V = np.ascontiguousarray(V, dtype=_NP_STORAGE[kv_dtype])
    T, H_q, D = q.shape
    assert K.ndim == 3 and K.shape == V.shape and K.shape[2] == D
    H_kv = K.shape[1]
    q_start = np.ascontiguousarray(q_start, dtype=np.int64)
    tok_off = np.ascontiguousarray(tok_off, dtype=np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    S = len(lens)
    assert q_start.shape == (S + 1,) and tok_off.shape == (S,) and q_start[S] == T
    for s in range(S):
        assert 0 <= tok_off[s] and tok_off[s] + lens[s] <= K.shape[0]
    ks = vs = None
    if kv_dtype == E4M3:
        ks = np.ascontiguousarray(k_scale, dtype=np.float32)
        vs = np.ascontiguousarray(v_scale, dtype=np.float32)
        assert ks.shape == (H_kv,) and vs.shape == (H_kv,)
    out = np.empty((T, H_q, D), dtype=np.float64)
    rc = lib().oracle_prefill_attention(
        S, H_q, H_kv, D, _ptr(q), q_dtype, _ptr(q_start), _ptr(K), _ptr(V), kv_dtype,
        _ptr(tok_off), _ptr(lens),
        _ptr(ks) if ks is not None else None, _ptr(vs) if vs is not None else None,
        float(np.float32(scale)), 1 if causal else 0, nthreads, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_prefill_attention rejected its arguments")
    return out


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Full no-cache causal attention in float64 (small inputs only).

    q, k, v: [T][H][D] float64 (same head count).  Row t attends to rows
    0..t: the whole history is recomputed for every position, the path the
    KV cache replaces ([mlqm] 一/三, [xph] "核心概念").  Returns [T][H][D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, D = q.shape
    out = np.zeros((T, H, D))
    for h in range(H):
        scores = float(scale) * (q[:, h, :] @ k[:, h, :].T)          # [T][T]
        scores[np.triu_indices(T, 1)] = -np.inf                       # future rows hidden
        scores -= scores.max(axis=1, keepdims=True)
        w = np.exp(scores)
        w /= w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ v[:, h, :]
    return out
