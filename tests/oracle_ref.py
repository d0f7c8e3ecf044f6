"""Oracle expectations for a workload (test side only).

The oracle never reads the device pool for attention: it regenerates each
sequence's logical K/V from the workload's seed and runs the fp64 oracle on
them.  For FP8 workloads it quantises the same bf16 source with its own OCP
encoder and the same fp32 inverse scales, then attends over the dequantised
values decode(code) * scale.
"""
from __future__ import annotations

import numpy as np

import oracle
import workloads as wl


def fp8_codes(x_bf16_bits: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Oracle E4M3 codes of bf16 values: code = E4M3(x * fp32(1/scale)) per head (axis 1)."""
    inv = (np.float32(1.0) / scale.astype(np.float32)).astype(np.float32)
    x = wl.bf16_bits_to_f32(x_bf16_bits) * inv[None, :, None]
    return oracle.e4m3_encode(x.astype(np.float32))


APPEND_CHUNK_TOKENS = 1 << 16      # the harness appends a prefill in calls of this many tokens


def int8_values(w: wl.Workload, b: int, n: int):
    """fp64 values [n][H_kv][D] of sequence b's K and V in an INT8 pool, from the
    oracle's tile model fed the same append calls the harness makes: the
    prefill in chunks, then the decode step's token on its own."""
    from oracle import int8_minmax as i8
    K, V = w.kv(b)
    K, V = wl.storage_to_f32(K[:n], w.src_dtype), wl.storage_to_f32(V[:n], w.src_dtype)
    store = i8.TileStore(w.H_kv, w.D)
    n_pre = min(n, int(w.prefill[b]))
    for s in range(0, n_pre, APPEND_CHUNK_TOKENS):
        e = min(n_pre, s + APPEND_CHUNK_TOKENS)
        store.append(np.arange(s, e), K[s:e], V[s:e])
    for t in range(n_pre, n):
        store.append(np.array([t]), K[t:t + 1], V[t:t + 1])
    blocks = np.arange(-(-n // wl.BLOCK))
    return store.values("k", blocks, n), store.values("v", blocks, n)


def expected(w: wl.Workload, seqs=None, step: int = 0, lens_override=None, nthreads: int = 0):
    """fp64 oracle output [len(seqs)][H_q][D] for the given sequence indices."""
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    lens = w.lens if lens_override is None else np.asarray(lens_override, np.int32)
    Ks, Vs, off, ln = [], [], [], []
    t = 0
    scales = w.fp8_scales()
    kv_code = oracle.F64 if w.kv_dtype == wl.INT8 else w.kv_dtype
    for b in seqs:
        n = int(lens[b])
        if w.kv_dtype == wl.INT8:
            K, V = int8_values(w, b, n)
        else:
            K, V = w.kv(b)
            K, V = K[:n], V[:n]
        if w.kv_dtype == wl.E4M3:
            K, V = fp8_codes(K, scales[0]), fp8_codes(V, scales[1])
        Ks.append(K)
        Vs.append(V)
        off.append(t)
        ln.append(n)
        t += n
    shape = (0, w.H_kv, w.D)
    empty = np.float64 if w.kv_dtype == wl.INT8 else wl._NP[w.kv_dtype]
    K = np.concatenate(Ks) if t else np.zeros(shape, empty)
    V = np.concatenate(Vs) if t else np.zeros(shape, empty)
    q = w.q(step)[seqs]
    kw = {}
    if w.kv_dtype == wl.E4M3:
        kw = dict(k_scale=scales[0], v_scale=scales[1])
    return oracle.decode_attention(q, w.q_dtype, K, V, kv_code, np.array(off, np.int64),
                                   np.array(ln, np.int32), w.scale, nthreads=nthreads, **kw)


TOL = {wl.F32: 1e-4, wl.F16: 5e-3, wl.BF16: 5e-3, wl.E4M3: 1e-2, wl.INT8: 5e-3}
_FRAC_BITS = {wl.F32: 23, wl.F16: 10, wl.BF16: 7}
_MIN_EXP = {wl.F32: -126, wl.F16: -14, wl.BF16: -126}


def half_ulp(x: np.ndarray, out_dtype: int) -> np.ndarray:
    """Half a unit in the last place of the output format at |x|: the error of
    storing the exact result in that format, which no kernel can avoid."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))), _MIN_EXP[out_dtype])
    e = np.maximum(e, _MIN_EXP[out_dtype])
    return np.ldexp(1.0, (e - _FRAC_BITS[out_dtype] - 1).astype(np.int64))


# Below this magnitude of the oracle's output the raw error is held to the
# tolerance: half an ulp of bf16 there is at most 2^-8 < 5e-3, so storing the
# exact result in any output format here fits inside every tolerance.
RAW_REGION = 2.0


def parity_error(got: np.ndarray, want: np.ndarray, out_dtype: int) -> float:
    """The figure held to TOL.  Per element, |got - want| where |want| < 2, and
    |got - want| - half_ulp(want) where |want| >= 2: above 2 the output format's
    own rounding of the exact result (half an ulp, 0.125 for bf16 at 52) is no
    computation error and is allowed on top of TOL, capped by construction at
    half an ulp.  The maximum over all elements is returned."""
    if got.size == 0:
        return 0.0
    d = np.abs(got - want)
    big = np.abs(want) >= RAW_REGION
    return float(np.max(np.where(big, d - half_ulp(want, out_dtype), d)))


def raw_error(got: np.ndarray, want: np.ndarray) -> dict:
    """max |got - want| over all elements, over |want| < 2, and the largest |want|."""
    if got.size == 0:
        return {"raw_max_abs": 0.0, "raw_max_abs_below_2": 0.0, "max_abs_out": 0.0}
    d = np.abs(got - want)
    small = np.abs(want) < RAW_REGION
    return {"raw_max_abs": float(d.max()), "raw_max_abs_below_2": float(d[small].max()) if small.any() else 0.0,
            "max_abs_out": float(np.abs(want).max())}


def error_beyond_output_rounding(got: np.ndarray, want: np.ndarray, out_dtype: int) -> float:
    """max(|got - want| - half_ulp(want)): the error beyond what storing the exact
    result in the output format costs.  The prefill tolerance: its P.V product
    takes the softmax weights in q's 16-bit format (8 significant bits for
    bf16), a rounding of its own on top of the output's, which the raw decode
    rule leaves no room for at |out| near 2."""
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - want) - half_ulp(want, out_dtype)))
