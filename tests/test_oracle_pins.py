"""Pins of the fp64 oracle against things other than itself (CPU only).

Every check here compares the oracle with a number a page prints, a library
routine of a different formulation, a specification constant or a closed
form.  The checks are plain functions (``check_*``) so that the planted-
mistake tests can run them against deliberately broken oracle builds.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# KV size formula
# ---------------------------------------------------------------------------
def check_kv_sizes():
    g = _golden("kv_sizes.json")
    for e in g["exact"]:
        got = oracle.kv_cache_bytes(e["layers"], e["kv_heads"], e["head_dim"], e["elem_bytes"],
                                    e["tokens"], e["seqs"])
        assert got == e["bytes"], (e["cite"], got)
    for e in g["approx"]:
        got = oracle.kv_cache_bytes(e["layers"], e["kv_heads"], e["head_dim"], e["elem_bytes"],
                                    e["tokens"], e["seqs"])
        assert abs(got - e["printed"]) <= e["rel_tol"] * e["printed"], (e["cite"], got)
    b = g["budget"]
    per_tok = oracle.kv_cache_bytes(b["layers"], b["kv_heads"], b["head_dim"], b["elem_bytes"], 1, 1)
    tokens = (b["budget_gib"] * 1024**3) // per_tok
    assert tokens == b["tokens"]
    assert tokens // 4096 == b["requests_at_4096"]


def test_kv_sizes_printed_on_pages():
    check_kv_sizes()


def test_kv_sizes_reject_invalid_shapes():
    # the budget script on m.lqnn.cn/news/219451 §2 refuses non-positive structure
    assert oracle.kv_cache_bytes(0, 8, 128, 2, 1, 1) == 0
    assert oracle.kv_cache_bytes(32, 8, 128, 0, 1, 1) == 0
    assert oracle.kv_cache_bytes(32, 8, 128, 2, -1, 1) == 0
    assert oracle.kv_cache_bytes(32, 8, 128, 2, 0, 1) == 0


# ---------------------------------------------------------------------------
# Exact widening of stored values
# ---------------------------------------------------------------------------
def check_f16_widen():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.widen(bits.view(np.float16), oracle.F16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def check_bf16_widen():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.widen(bits, oracle.BF16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f16_widen_all_patterns():
    check_f16_widen()


def test_bf16_widen_all_patterns():
    check_bf16_widen()


# ---------------------------------------------------------------------------
# OCP E4M3 codec
# ---------------------------------------------------------------------------
def _torch_e4m3_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).to(torch.float64).numpy()


def check_e4m3_decode():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.widen(codes, oracle.E4M3)
    ref = _torch_e4m3_decode()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # specification constants: bias 7, max 448, min subnormal 2^-9, min normal 2^-6,
    # S.1111.111 is NaN and there are no infinities
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0**-9 and got[0x08] == 2.0**-6
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and nan.sum() == 2
    assert not np.isinf(got).any()
    assert got[0x38] == 1.0                       # exponent field 7 = bias


def test_e4m3_decode_all_codes():
    check_e4m3_decode()


def _e4m3_critical_inputs():
    """Every midpoint between neighbouring codes, one float ulp either side,
    the codes themselves, plus random floats inside the finite range."""
    pos = oracle.widen(np.arange(127, dtype=np.uint8), oracle.E4M3)     # 0 .. 448
    mids = (pos[:-1] + pos[1:]) / 2
    m32 = mids.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mids)                 # midpoints are floats
    xs = [pos.astype(np.float32), m32,
          np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(-np.inf))]
    rng = np.random.default_rng(7)
    xs.append(rng.uniform(0, 448, 200000).astype(np.float32))
    xs.append((rng.uniform(0, 1, 200000) * 2.0**rng.integers(-24, 0, 200000)).astype(np.float32))
    x = np.concatenate(xs)
    return np.concatenate([x, -x])


def check_e4m3_encode():
    x = _e4m3_critical_inputs()
    got = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]
    # encode(decode(c)) == c on every finite code (+0 and -0 included)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.widen(codes, oracle.E4M3).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    # saturation beyond the largest finite value (outliers saturate), NaN code
    big = np.array([448.0, 449.0, 464.0, 480.0, 1e6, np.inf, 3.4e38], np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)
    assert oracle.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_e4m3_encode_rne_saturating():
    check_e4m3_encode()


# ---------------------------------------------------------------------------
# Decode attention
# ---------------------------------------------------------------------------
def _textbook(q64, K64, V64, tok_off, lens, scale):
    """softmax(scale * q K^T) V per (b, h) with scipy's softmax and numpy matmul."""
    B, H_q, D = q64.shape
    H_kv = K64.shape[1]
    G = H_q // H_kv
    out = np.zeros((B, H_q, D))
    for b in range(B):
        n = int(lens[b])
        if n <= 0:
            continue
        for h in range(H_q):
            g = h // G
            Kb = K64[tok_off[b]:tok_off[b] + n, g, :]
            Vb = V64[tok_off[b]:tok_off[b] + n, g, :]
            w = scipy.special.softmax(np.float64(np.float32(scale)) * (Kb @ q64[b, h]))
            out[b, h] = w @ Vb
    return out


def _random_case(seed, B, H_q, H_kv, D, lens, dtype):
    rng = np.random.default_rng(seed)
    T = int(np.sum(lens))
    tok_off = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    q = wl.cast_to_storage(rng.standard_normal((B, H_q, D)).astype(np.float32), dtype)
    K = wl.cast_to_storage(rng.standard_normal((T, H_kv, D)).astype(np.float32), dtype)
    V = wl.cast_to_storage(rng.standard_normal((T, H_kv, D)).astype(np.float32), dtype)
    return q, K, V, tok_off, np.asarray(lens, np.int32)


def check_attention_textbook():
    cases = [(11, 3, 8, 2, 16, [1, 7, 33], oracle.F32, 0.25),
             (12, 2, 5, 1, 32, [16, 40], oracle.F16, 1 / math.sqrt(32)),
             (13, 2, 6, 3, 8, [5, 18], oracle.BF16, 0.7)]
    for seed, B, Hq, Hkv, D, lens, dt, scale in cases:
        q, K, V, off, ln = _random_case(seed, B, Hq, Hkv, D, lens, dt)
        got = oracle.decode_attention(q, dt, K, V, dt, off, ln, scale)
        ref = _textbook(oracle.widen(q, dt), oracle.widen(K, dt), oracle.widen(V, dt), off, ln, scale)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_attention_vs_textbook_softmax():
    check_attention_textbook()


def check_attention_closed_forms():
    rng = np.random.default_rng(3)
    D = 16
    # single-token context: the weight is exactly 1, out = V_0 exactly
    q = rng.standard_normal((1, 2, D)).astype(np.float32)
    K = rng.standard_normal((1, 2, D)).astype(np.float32)
    V = rng.standard_normal((1, 2, D)).astype(np.float32)
    out = oracle.decode_attention(q, oracle.F32, K, V, oracle.F32, [0], [1], 0.25)
    assert np.array_equal(out[0], V[0].astype(np.float64))
    # q = 0: uniform weights, out = mean of V
    n = 9
    K = rng.standard_normal((n, 1, D)).astype(np.float32)
    V = rng.standard_normal((n, 1, D)).astype(np.float32)
    out = oracle.decode_attention(np.zeros((1, 1, D), np.float32), oracle.F32, K, V, oracle.F32,
                                  [0], [n], 0.25)
    np.testing.assert_allclose(out[0, 0], V[:, 0].astype(np.float64).mean(axis=0), atol=1e-14)
    # constant V: out = that constant
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    Vc = np.full((n, 1, D), 0.375, np.float32)
    out = oracle.decode_attention(q, oracle.F32, K, Vc, oracle.F32, [0], [n], 0.25)
    np.testing.assert_allclose(out[0, 0], 0.375, atol=1e-15)
    # two tokens: out = sigmoid(z0 - z1) V0 + sigmoid(z1 - z0) V1
    K2 = rng.standard_normal((2, 1, D)).astype(np.float32)
    V2 = rng.standard_normal((2, 1, D)).astype(np.float32)
    s = 0.3
    z = [float(np.float32(s)) * float(np.dot(q[0, 0].astype(np.float64), K2[j, 0].astype(np.float64)))
         for j in range(2)]
    sig = lambda t: 1.0 / (1.0 + math.exp(-t))
    ref = sig(z[0] - z[1]) * V2[0, 0].astype(np.float64) + sig(z[1] - z[0]) * V2[1, 0].astype(np.float64)
    out = oracle.decode_attention(q, oracle.F32, K2, V2, oracle.F32, [0], [2], s)
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-14)
    # one key aligned with q and scaled up: out tends to its value
    Kl = rng.standard_normal((n, 1, D)).astype(np.float32)
    Kl[4, 0] = 50.0 * q[0, 0]
    out = oracle.decode_attention(q, oracle.F32, Kl, V, oracle.F32, [0], [n], 1.0)
    np.testing.assert_allclose(out[0, 0], V[4, 0].astype(np.float64), atol=1e-12)
    # empty context: zeros
    out = oracle.decode_attention(q, oracle.F32, K, V, oracle.F32, [0], [0], 0.25)
    assert np.array_equal(out, np.zeros_like(out))


def test_attention_closed_forms():
    check_attention_closed_forms()


def check_gqa_equals_repeated_mha():
    # several query heads sharing one KV head (mlqm.cn/news/394450, 六) equals MHA
    # with each KV head repeated G times, consecutive query heads per group
    B, Hq, Hkv, D = 2, 10, 2, 16
    lens = [13, 30]
    q, K, V, off, ln = _random_case(21, B, Hq, Hkv, D, lens, oracle.F32)
    gqa = oracle.decode_attention(q, oracle.F32, K, V, oracle.F32, off, ln, 0.25)
    G = Hq // Hkv
    Kr = np.repeat(K, G, axis=1)
    Vr = np.repeat(V, G, axis=1)
    mha = oracle.decode_attention(q, oracle.F32, Kr, Vr, oracle.F32, off, ln, 0.25)
    assert np.array_equal(gqa, mha)
    # and it is not trivially so: a different head->group map gives other values
    Kalt = np.tile(K, (1, G, 1))
    Valt = np.tile(V, (1, G, 1))
    alt = oracle.decode_attention(q, oracle.F32, Kalt, Valt, oracle.F32, off, ln, 0.25)
    assert not np.allclose(alt, gqa)


def test_gqa_equals_repeated_mha():
    check_gqa_equals_repeated_mha()


def check_cached_decode_equals_recompute():
    # The walk-through on mlqm.cn/news/394450 (四): d_model 64, 4 heads of 16,
    # 5-token prompt then 3 decode steps, cache 5 -> 8.  Each decode step's output
    # must equal the last row of full no-cache causal attention over the history.
    x, Wq, Wk, Wv = wl.mini_model_inputs(seed=99, n_tokens=8)
    H, dk = 4, 16
    Q = (x @ Wq).reshape(8, H, dk)
    Kx = (x @ Wk).reshape(8, H, dk)
    Vx = (x @ Wv).reshape(8, H, dk)
    scale = float(np.float32(1 / math.sqrt(dk)))
    full = oracle.causal_attention(Q, Kx, Vx, scale)
    for t in range(5, 9):                       # context lengths after prefill / each step
        # the oracle takes stored values; float32 storage of the projections
        q32 = Q[t - 1:t].astype(np.float32)
        K32, V32 = Kx[:t].astype(np.float32), Vx[:t].astype(np.float32)
        dec = oracle.decode_attention(q32, oracle.F32, K32, V32, oracle.F32, [0], [t], scale)
        Q32 = Q[:t].astype(np.float32).astype(np.float64)
        ref = oracle.causal_attention(Q32, K32.astype(np.float64), V32.astype(np.float64), scale)[t - 1]
        np.testing.assert_allclose(dec[0], ref, atol=1e-12)
        # and against the recompute from the float64 history (only float32 storage rounding apart)
        np.testing.assert_allclose(dec[0], full[t - 1], atol=1e-5)


def test_cached_decode_equals_recompute():
    check_cached_decode_equals_recompute()


def check_fp8_attention_on_dequantised_values():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, lens = 2, 4, 2, 16, [20, 35]
    T = sum(lens)
    off = np.array([0, lens[0]], np.int64)
    q = wl.f32_to_bf16_bits(rng.standard_normal((B, Hq, D)).astype(np.float32))
    codes_k = rng.integers(0, 256, (T, Hkv, D)).astype(np.uint8)
    codes_v = rng.integers(0, 256, (T, Hkv, D)).astype(np.uint8)
    codes_k[(codes_k & 0x7F) == 0x7F] = 0x11        # no NaN codes in live data
    codes_v[(codes_v & 0x7F) == 0x7F] = 0x22
    ks = np.array([0.03, 0.5], np.float32)
    vs = np.array([0.25, 0.0078125], np.float32)
    got = oracle.decode_attention(q, oracle.BF16, codes_k, codes_v, oracle.E4M3, off, lens, 0.25,
                                  k_scale=ks, v_scale=vs)
    dec = _torch_e4m3_decode()
    K64 = dec[codes_k] * ks.astype(np.float64)[None, :, None]
    V64 = dec[codes_v] * vs.astype(np.float64)[None, :, None]
    ref = _textbook(wl.bf16_bits_to_f32(q).astype(np.float64), K64, V64, off, lens, 0.25)
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_fp8_attention_on_dequantised_values():
    check_fp8_attention_on_dequantised_values()


# ---------------------------------------------------------------------------
# Multi-query (prefill / chunked prefill) attention
# ---------------------------------------------------------------------------
def _prefill_case(seed, lens, q_lens, H_q, H_kv, D, dtype):
    rng = np.random.default_rng(seed)
    q_start = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    tok_off = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    q = wl.cast_to_storage(rng.standard_normal((int(q_start[-1]), H_q, D)).astype(np.float32), dtype)
    K = wl.cast_to_storage(rng.standard_normal((int(np.sum(lens)), H_kv, D)).astype(np.float32), dtype)
    V = wl.cast_to_storage(rng.standard_normal((int(np.sum(lens)), H_kv, D)).astype(np.float32), dtype)
    return q, q_start, K, V, tok_off, np.asarray(lens, np.int32)


def _sdpa_reference(q64, q_start, K64, V64, tok_off, lens, scale, causal):
    """torch's scaled_dot_product_attention in float64, one sequence at a time,
    KV heads repeated per query group, with an explicit mask: query i of a chunk
    of q_len at the end of n positions may see j <= n - q_len + i."""
    H_q, H_kv = q64.shape[1], K64.shape[1]
    out = np.zeros_like(q64)
    for s in range(len(lens)):
        n, a, b = int(lens[s]), int(q_start[s]), int(q_start[s + 1])
        Q = torch.from_numpy(q64[a:b]).permute(1, 0, 2)                           # [H][L][D]
        Ks = torch.from_numpy(K64[tok_off[s]:tok_off[s] + n]).permute(1, 0, 2)
        Vs = torch.from_numpy(V64[tok_off[s]:tok_off[s] + n]).permute(1, 0, 2)
        Ks = Ks.repeat_interleave(H_q // H_kv, dim=0).contiguous()
        Vs = Vs.repeat_interleave(H_q // H_kv, dim=0).contiguous()
        L = b - a
        mask = torch.ones(L, n, dtype=torch.bool)
        if causal:
            mask = torch.arange(n)[None, :] <= (n - L + torch.arange(L))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            Q, Ks, Vs, attn_mask=mask, scale=float(np.float32(scale)))
        out[a:b] = o.permute(1, 0, 2).numpy()
    return out


def check_prefill_vs_library_attention():
    # chunks at the end of a cached context, GQA, causal and unmasked
    cases = [(31, [12, 40, 5], [12, 9, 1], 8, 2, 16, oracle.F32, 0.25),
             (32, [64, 33], [17, 33], 6, 3, 32, oracle.BF16, 1 / math.sqrt(32)),
             (33, [20], [7], 4, 4, 8, oracle.F16, 0.6)]
    for seed, lens, q_lens, Hq, Hkv, D, dt, scale in cases:
        q, qs, K, V, off, ln = _prefill_case(seed, lens, q_lens, Hq, Hkv, D, dt)
        for causal in (True, False):
            got = oracle.prefill_attention(q, dt, qs, K, V, dt, off, ln, scale, causal=causal)
            ref = _sdpa_reference(oracle.widen(q, dt), qs, oracle.widen(K, dt), oracle.widen(V, dt),
                                  off, ln, scale, causal)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_prefill_vs_library_attention():
    check_prefill_vs_library_attention()


def check_prefill_single_token_is_decode():
    # a chunk of one token at the end of the context is the decode step
    q, qs, K, V, off, ln = _prefill_case(34, [9, 30, 1], [1, 1, 1], 8, 2, 16, oracle.BF16)
    pre = oracle.prefill_attention(q, oracle.BF16, qs, K, V, oracle.BF16, off, ln, 0.3)
    dec = oracle.decode_attention(q, oracle.BF16, K, V, oracle.BF16, off, ln, 0.3)
    np.testing.assert_allclose(pre, dec, rtol=0, atol=1e-13)


def test_prefill_single_token_is_decode():
    check_prefill_single_token_is_decode()


def check_prefill_chunks_compose():
    # mlqm.cn/news/394450, 七 (chunked prefill): a prompt of 12 tokens processed as
    # chunks of 5 and 7 gives what one chunk of 12 gives, token for token
    q, qs, K, V, off, ln = _prefill_case(35, [12], [12], 4, 2, 16, oracle.F32)
    whole = oracle.prefill_attention(q, oracle.F32, qs, K, V, oracle.F32, off, ln, 0.25)
    first = oracle.prefill_attention(q[:5], oracle.F32, [0, 5], K[:5], V[:5], oracle.F32, [0], [5], 0.25)
    second = oracle.prefill_attention(q[5:], oracle.F32, [0, 7], K, V, oracle.F32, [0], [12], 0.25)
    np.testing.assert_allclose(np.concatenate([first, second]), whole, rtol=0, atol=1e-13)
    # and each row equals decode with the context that row sees
    for t in range(12):
        dec = oracle.decode_attention(q[t:t + 1], oracle.F32, K, V, oracle.F32, [0], [t + 1], 0.25)
        np.testing.assert_allclose(whole[t], dec[0], rtol=0, atol=1e-13)


def test_prefill_chunks_compose():
    check_prefill_chunks_compose()


def check_prefill_fp8_on_dequantised_values():
    rng = np.random.default_rng(36)
    lens, q_lens, Hq, Hkv, D = [25, 14], [6, 14], 4, 2, 16
    qs = np.array([0, 6, 20], np.int64)
    off = np.array([0, 25], np.int64)
    q = wl.f32_to_bf16_bits(rng.standard_normal((20, Hq, D)).astype(np.float32))
    codes_k = rng.integers(0, 256, (39, Hkv, D)).astype(np.uint8)
    codes_v = rng.integers(0, 256, (39, Hkv, D)).astype(np.uint8)
    codes_k[(codes_k & 0x7F) == 0x7F] = 0x11
    codes_v[(codes_v & 0x7F) == 0x7F] = 0x22
    ks = np.array([0.03, 0.5], np.float32)
    vs = np.array([0.25, 0.0078125], np.float32)
    got = oracle.prefill_attention(q, oracle.BF16, qs, codes_k, codes_v, oracle.E4M3, off, lens, 0.25,
                                   k_scale=ks, v_scale=vs)
    dec = _torch_e4m3_decode()
    K64 = dec[codes_k] * ks.astype(np.float64)[None, :, None]
    V64 = dec[codes_v] * vs.astype(np.float64)[None, :, None]
    ref = _sdpa_reference(wl.bf16_bits_to_f32(q).astype(np.float64), qs, K64, V64, off, lens, 0.25, True)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_prefill_fp8_on_dequantised_values():
    check_prefill_fp8_on_dequantised_values()


def test_prefill_rejects_chunk_longer_than_context():
    q, qs, K, V, off, ln = _prefill_case(37, [4], [4], 2, 2, 8, oracle.F32)
    with pytest.raises(ValueError):
        oracle.prefill_attention(q, oracle.F32, qs, K, V, oracle.F32, off, np.array([3], np.int32), 0.5)


ALL_CHECKS = [check_kv_sizes, check_f16_widen, check_bf16_widen, check_e4m3_decode,
              check_e4m3_encode, check_attention_textbook, check_attention_closed_forms,
              check_gqa_equals_repeated_mha, check_cached_decode_equals_recompute,
              check_fp8_attention_on_dequantised_values, check_prefill_vs_library_attention,
              check_prefill_single_token_is_decode, check_prefill_chunks_compose,
              check_prefill_fp8_on_dequantised_values]


# ---------------------------------------------------------------------------
# INT8 per-block min-max codes ([moo] §3.3): q = round((k - k_min) / (k_max - k_min) * 255)
# ---------------------------------------------------------------------------
from fractions import Fraction  # noqa: E402

from oracle import int8_minmax as _i8  # noqa: E402


def _half_even(fr: Fraction) -> int:
    lo = fr.numerator // fr.denominator
    rem = fr - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        return lo + 1
    return lo


def check_int8_formula(m=_i8):
    """Inputs for which every fp32 step of the formula is exact, against the
    formula evaluated in rationals with round-half-even."""
    cases = [(0.0, 256.0, [float(k) for k in range(257)]),          # t = k/256, codes 255k/256
             (-3.0, 5.0, [-3.0 + j for j in range(9)]),             # t = j/8
             (-1.0, 1.0, [-1.0, -0.5, 0.0, 0.5, 1.0])]              # 0 -> 127.5 -> 128 (even)
    for lo, hi, xs in cases:
        got = m.encode(np.array(xs, np.float32), lo, hi)
        want = [_half_even((Fraction(x) - Fraction(lo)) / (Fraction(hi) - Fraction(lo)) * 255) for x in xs]
        assert got.tolist() == want, (lo, hi)
    assert m.encode(np.float32(0.0), -1.0, 1.0) == 128
    # degenerate range: code 0, standing for the value itself
    assert m.encode(np.float32(2.5), 2.5, 2.5) == 0 and m.value(np.uint8(0), 2.5, 2.5) == 2.5


def check_int8_round_trip(m=_i8):
    """A code stands for its input within half a step; the range's ends are exact."""
    rng = np.random.default_rng(41)
    for lo, hi in [(-2.5, 3.75), (0.001, 0.002), (-100.0, -99.0), (-1e-3, 7e3)]:
        lo, hi = np.float32(lo), np.float32(hi)
        x = rng.uniform(lo, hi, 4000).astype(np.float32)
        x[:2] = (lo, hi)
        c = m.encode(x, lo, hi)
        assert c[0] == 0 and c[1] == 255
        half = (float(hi) - float(lo)) / 510.0
        assert np.all(np.abs(m.value(c, lo, hi) - x) <= half * (1 + 1e-4)), (lo, hi)
        assert m.value(np.uint8(0), lo, hi) == float(lo) and m.value(np.uint8(255), lo, hi) == float(hi)


def check_int8_fill_invariants(m=_i8):
    """Tiles filled a random number of rows per call: the range is the min and
    max of the raw values since row 0, rows keep their codes while the range
    holds, every row stays within its accumulated re-encode bound of its raw
    value, and writing row 0 again starts the tile over."""
    rng = np.random.default_rng(43)
    H, D = 2, 16
    for trial in range(25):
        store = m.TileStore(H, D)
        for b in (3, 7):
            raw = {"k": [], "v": []}
            bound = {"k": np.zeros((16, H)), "v": np.zeros((16, H))}
            row = 0
            while row < 16:
                n = int(min(rng.integers(1, 6), 16 - row))
                scale = float(rng.choice([0.25, 1.0, 4.0]))
                K = (rng.standard_normal((n, H, D)) * scale).astype(np.float32)
                V = (rng.standard_normal((n, H, D)) * scale).astype(np.float32)
                before = {(kind, g): store.tile(kind, b, g) for kind in "kv" for g in range(H)}
                store.append(np.arange(n) + 16 * b + row, K, V)
                for kind, X in (("k", K), ("v", V)):
                    raw[kind].extend(X)
                    R = np.stack(raw[kind])                                    # [rows][H][D]
                    for g in range(H):
                        codes, (lo, hi) = store.tile(kind, b, g)
                        assert lo == R[:, g].min() and hi == R[:, g].max(), (trial, kind, row)
                        old_codes, (olo, ohi) = before[(kind, g)]
                        if row > 0 and (olo, ohi) == (lo, hi):
                            assert np.array_equal(codes[:row], old_codes[:row])
                        half = (float(hi) - float(lo)) / 510.0 * (1 + 1e-4) + 1e-6 * max(abs(float(lo)), abs(float(hi)))
                        if row > 0 and (olo, ohi) != (lo, hi):
                            bound[kind][:row, g] += half                       # one more re-encode
                        bound[kind][row:row + n, g] = half
                        err = np.abs(m.value(codes[:row + n], lo, hi) - R[:, g]).max(axis=1)
                        assert np.all(err <= bound[kind][:row + n, g]), (trial, kind, row)
                row += n
        # row 0 again: the tile starts over with this call's values alone
        K = rng.standard_normal((1, H, D)).astype(np.float32) * 0.01
        store.append(np.array([16 * 3]), K, K)
        for g in range(H):
            _, (lo, hi) = store.tile("k", 3, g)
            assert lo == K[0, g].min() and hi == K[0, g].max()


def check_int8_one_shot(m=_i8):
    """The page's formula applied once per (tile, head): closed forms, the
    rational formula with round-half-even, half a step of error, and tiles and
    heads that never see each other's values."""
    # a tile holding exactly the grid k_min + k * (k_max - k_min) / 255 maps onto itself
    grid = np.arange(256, dtype=np.float64).reshape(16, 1, 16) * 0.5 - 3.0     # -3 .. 124.5 step 0.5
    assert np.array_equal(m.one_shot_values(grid), grid)
    # constant tile: its constant; a lone row of one value too
    const = np.full((16, 2, 8), 0.7)
    assert np.array_equal(m.one_shot_values(const), const)
    rng = np.random.default_rng(45)
    # dyadic values: every fp64 step of the formula is exact, so the codes equal
    # the rational formula with round-half-even (ties included)
    for trial in range(20):
        x = rng.integers(-64, 65, size=(16, 1, 4)).astype(np.float64) / 8.0
        x[0, 0, 0], x[1, 0, 0] = -8.0, 8.0                                       # span 16: exact /255 steps
        v = m.one_shot_values(x)
        lo, hi = Fraction(-8), Fraction(8)
        for xi, vi in zip(x.reshape(-1), v.reshape(-1)):
            q = _half_even((Fraction(float(xi)) - lo) / (hi - lo) * 255)
            assert float(vi) == float(lo + q * (hi - lo) / 255), (xi, vi, q)   # both correctly rounded
    # random tiles: within half a step of the input, ends exact, a partial last
    # tile ranges over its own rows only, heads are independent
    for n in (1, 15, 16, 17, 40, 77):
        x = (rng.standard_normal((n, 3, 8)) * np.array([1.0, 10.0, 0.01])[None, :, None]).astype(np.float32)
        x = x.astype(np.float64)                                                 # fp32 values, as the pools hold
        v = m.one_shot_values(x)
        for j0 in range(0, n, 16):
            t, tv = x[j0:j0 + 16], v[j0:j0 + 16]
            for h in range(3):
                lo, hi = t[:, h].min(), t[:, h].max()
                assert np.all(np.abs(tv[:, h] - t[:, h]) <= (hi - lo) / 510 * (1 + 1e-9))
                assert tv[:, h].min() == lo and tv[:, h].max() == hi
            assert np.array_equal(m.one_shot_values(t), tv)                      # the tile alone
        y = x.copy()
        y[:, 1] *= 1000.0
        if n > 16:
            y[16:32, 0] += 5.0                                                   # another tile of head 0
        w = m.one_shot_values(y)
        assert np.array_equal(w[:, 2], v[:, 2]) and np.array_equal(w[:16, 0], v[:16, 0])


def _ranges_after_each_row(col):
    """(k_min, k_max) of rows 0..t of one head's tile, for every t (raw values)."""
    flat = col.reshape(col.shape[0], -1)
    return np.minimum.accumulate(flat.min(axis=1)), np.maximum.accumulate(flat.max(axis=1))


def check_int8_token_fill_vs_one_shot(m=_i8):
    """Tiles filled one token per call (the decode pattern), with the model of
    the appends: every dequantised value lies within the sum of half steps of
    the ranges its row lived under (counted from the raw data alone: one for
    its own write, one per later range move) of its raw value, and within that
    plus half a final step of the page's one-shot value.  Returns the largest
    errors against the raw values (token fill, one-shot)."""
    rng = np.random.default_rng(46)
    H, D, n = 2, 64, 16 * 12 + 5
    worst_fill = worst_once = 0.0
    for trial in range(4):
        X = {kind: (rng.standard_normal((n, H, D)) * rng.choice([0.3, 1.0, 3.0])).astype(np.float32) for kind in "kv"}
        store = m.TileStore(H, D)
        for t in range(n):
            store.append(np.array([t]), X["k"][t:t + 1], X["v"][t:t + 1])
        blocks = np.arange(-(-n // 16))
        for kind in "kv":
            x = X[kind].astype(np.float64)
            lib = store.values(kind, blocks, n)
            once = m.one_shot_values(x)
            for j0 in range(0, n, 16):
                rows = min(16, n - j0)
                for h in range(H):
                    lo, hi = _ranges_after_each_row(x[j0:j0 + rows, h])
                    half = (hi - lo) / 510.0 * (1 + 1e-4) + 1e-6 * np.maximum(np.abs(lo), np.abs(hi))
                    moved = np.r_[False, (lo[1:] != lo[:-1]) | (hi[1:] != hi[:-1])]
                    for r in range(rows):
                        bound = half[r] + half[r + 1:][moved[r + 1:]].sum()
                        err = np.abs(lib[j0 + r, h] - x[j0 + r, h]).max()
                        assert err <= bound, (trial, kind, j0, h, r, err, bound)
                        assert np.abs(lib[j0 + r, h] - once[j0 + r, h]).max() <= bound + half[-1]
            worst_fill = max(worst_fill, float(np.abs(lib - x).max() / x.std()))
            worst_once = max(worst_once, float(np.abs(once - x).max() / x.std()))
    return worst_fill, worst_once


def check_f64_storage_path():
    """Attention on fp64 storage: equal to fp32 storage of the same values, and
    to the textbook softmax on values that fp32 cannot hold."""
    rng = np.random.default_rng(44)
    q = rng.standard_normal((2, 4, 16)).astype(np.float32)
    K = rng.standard_normal((50, 2, 16)).astype(np.float32)
    V = rng.standard_normal((50, 2, 16)).astype(np.float32)
    off, lens = np.array([0, 20]), np.array([20, 30], np.int32)
    a = oracle.decode_attention(q, oracle.F32, K, V, oracle.F32, off, lens, 0.25)
    b = oracle.decode_attention(q, oracle.F32, K.astype(np.float64), V.astype(np.float64), oracle.F64, off, lens, 0.25)
    assert np.array_equal(a, b)
    K64 = rng.standard_normal((50, 2, 16)) * (1 + 1e-9)
    V64 = rng.standard_normal((50, 2, 16)) * (1 + 1e-9)
    got = oracle.decode_attention(q, oracle.F32, K64, V64, oracle.F64, off, lens, 0.25)
    ref = _textbook(q.astype(np.float64), K64, V64, off, lens, 0.25)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_int8_formula_closed_forms():
    check_int8_formula()


def test_int8_round_trip_half_step():
    check_int8_round_trip()


def test_int8_fill_invariants():
    check_int8_fill_invariants()


def test_int8_one_shot_formula():
    check_int8_one_shot()


def test_int8_token_fill_within_its_bound_of_raw_and_one_shot():
    fill, once = check_int8_token_fill_vs_one_shot()
    # the token-at-a-time fill drifts further than one quantisation, but stays
    # within the sum of its own half steps (asserted per element above)
    assert once < fill < 16 * once


def test_int8_tile_store_rename():
    """Renaming blocks moves whole tiles at once, also when a new id is
    another pair's old id (a swap of two ids, and a chain 1 -> 2 -> 5)."""
    rng = np.random.default_rng(44)
    store = _i8.TileStore(2, 16)
    for b in (1, 2, 3):
        K = rng.standard_normal((16, 2, 16)).astype(np.float32) * (b + 1)
        store.append(np.arange(16) + 16 * b, K, -K)
    snap = {(kind, b, g): store.tile(kind, b, g) for kind in "kv" for b in (1, 2, 3) for g in range(2)}
    store.rename([(1, 2), (2, 1)])
    store.rename([(1, 5), (3, 1)])
    # after both calls: old 1 -> 2, old 2 -> 1 -> 5, old 3 -> 1
    for old, new in ((1, 2), (2, 5), (3, 1)):
        for kind in "kv":
            for g in range(2):
                codes, (lo, hi) = store.tile(kind, new, g)
                want_codes, (wlo, whi) = snap[(kind, old, g)]
                assert np.array_equal(codes, want_codes) and lo == wlo and hi == whi, (old, new, kind, g)


def test_f64_storage_path():
    check_f64_storage_path()
