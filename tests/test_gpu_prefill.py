"""GPU parity of paged_prefill (multi-query attention over the paged cache)
against the fp64 oracle's prefill_attention, through the C ABI.

Each case lays random K/V for every position of every sequence into a pool
with a scattered free list (kv_append, the chunk's own tokens included), then
attends a chunk of query tokens at the end of each context.  The oracle gets
the same stored values in logical order (for FP8 pools, its own E4M3 codes of
the same bf16 source).  Tolerances and the output-rounding allowance are the
decode ones.
"""
import math
import sys

import numpy as np
import pytest

import harness
import oracle
import paged_kv_cache_152_amd as pkv
import workloads as wl
from tests.oracle_ref import TOL, error_beyond_output_rounding, fp8_codes

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(*a):
    print(*a, flush=True, file=sys.stderr)


class Case:
    """Sequences with (context length n, chunk length q_len) laid into one pool."""

    def __init__(self, kv_dt, H_q, H_kv, D, shapes, seed, q_dt=None, poison=False, free_order=None):
        rng = np.random.default_rng(seed)
        self.kv_dt, self.H_q, self.H_kv, self.D = kv_dt, H_q, H_kv, D
        self.q_dt = q_dt if q_dt is not None else (wl.BF16 if kv_dt == wl.E4M3 else kv_dt)
        src_dt = wl.BF16 if kv_dt == wl.E4M3 else kv_dt
        self.lens = np.array([n for n, _ in shapes], np.int32)
        self.q_lens = np.array([ql for _, ql in shapes], np.int32)
        self.q_start = np.concatenate([[0], np.cumsum(self.q_lens)]).astype(np.int32)
        nb = int(sum(-(-n // 16) for n in self.lens)) + 3
        order = rng.permutation(nb)
        if free_order is not None:
            order = free_order(nb)
        self.pool = pkv.KVPool(nb, H_kv, D, kv_dt, free_order=order)
        self.K = [wl.cast_to_storage(rng.standard_normal((n, H_kv, D)).astype(np.float32), src_dt)
                  for n in self.lens]
        self.V = [wl.cast_to_storage(rng.standard_normal((n, H_kv, D)).astype(np.float32), src_dt)
                  for n in self.lens]
        self.scales = None
        if kv_dt == wl.E4M3:
            allk = np.concatenate(self.K)
            allv = np.concatenate(self.V)
            ks = np.abs(wl.bf16_bits_to_f32(allk)).max(axis=(0, 2)) / 448.0
            vs = np.abs(wl.bf16_bits_to_f32(allv)).max(axis=(0, 2)) / 448.0
            self.scales = (ks.astype(np.float32), vs.astype(np.float32))
            self.pool.set_fp8_scales(*self.scales)
        if poison:
            nan = torch.full((nb * 16, H_kv, D), float("nan"),
                             dtype=torch.bfloat16 if src_dt == wl.BF16 else pkv.torch_dtype(src_dt), device="cuda")
            self.pool.append(torch.arange(nb * 16, dtype=torch.int32, device="cuda"), nan, nan)
        self.seqs = []
        for n, K, V in zip(self.lens, self.K, self.V):
            s = self.pool.seq_create()
            slots = self.pool.seq_reserve(s, int(n))
            self.pool.append(torch.from_numpy(slots).cuda(), harness.to_device(K, src_dt),
                             harness.to_device(V, src_dt))
            self.seqs.append(s)
        self.q = wl.cast_to_storage(rng.standard_normal((int(self.q_start[-1]), H_q, D)).astype(np.float32),
                                    self.q_dt)
        self.scale = float(np.float32(1 / math.sqrt(D)))

    def run(self, causal=True):
        mb = max(1, int(max(-(-n // 16) for n in self.lens)))
        tables, lens = self.pool.block_tables(self.seqs, mb)
        out = self.pool.prefill(harness.to_device(self.q, self.q_dt), torch.from_numpy(self.q_start).cuda(),
                                torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                                int(self.q_lens.max()), self.scale, causal=causal)
        torch.cuda.synchronize()
        return harness.out_to_f64(out)

    def oracle_kv(self):
        if self.kv_dt == wl.E4M3:
            K = np.concatenate([fp8_codes(k, self.scales[0]) for k in self.K])
            V = np.concatenate([fp8_codes(v, self.scales[1]) for v in self.V])
        else:
            K, V = np.concatenate(self.K), np.concatenate(self.V)
        return K, V

    def expected(self, causal=True):
        K, V = self.oracle_kv()
        off = np.concatenate([[0], np.cumsum(self.lens)[:-1]]).astype(np.int64)
        kw = dict(k_scale=self.scales[0], v_scale=self.scales[1]) if self.scales else {}
        return oracle.prefill_attention(self.q, self.q_dt, self.q_start, K, V, self.kv_dt, off, self.lens,
                                        self.scale, causal=causal, **kw)

    def close(self):
        self.pool.close()


def check(got, want, kv_dt, q_dt, what):
    """Error beyond the output format's rounding <= TOL (the prefill rule: the
    weights enter P.V in q's 16-bit format); the raw max-abs is reported."""
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = error_beyond_output_rounding(got, want, q_dt)
    raw = float(np.abs(got - want).max()) if got.size else 0.0
    assert err <= TOL[kv_dt], f"{what}: err {err:.3e} beyond output rounding (raw {raw:.3e}) > {TOL[kv_dt]:.0e}"
    return raw


SHAPES = [(37, 37), (300, 45), (129, 1), (64, 16), (17, 3)]


@pytest.mark.parametrize("kv_dt", [wl.F16, wl.BF16, wl.E4M3])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8, 11, 16, 24, 32])
def test_prefill_vs_oracle(kv_dt, D, G):
    """Every row-group shape: G <= 16 query heads share one row group (32 / G
    tokens per wave, padding rows when G does not divide 32); 24 and 32 split
    into two groups of 12 and of 16."""
    H_kv = 2
    c = Case(kv_dt, G * H_kv, H_kv, D, SHAPES, seed=1000 + 10 * G + D + kv_dt)
    for causal in (True, False):
        err = check(c.run(causal), c.expected(causal), kv_dt, c.q_dt, f"dt={kv_dt} D={D} G={G} causal={causal}")
        say(f"prefill dt={kv_dt} D={D} G={G} causal={causal}: err {err:.2e}")
    c.close()


def test_prefill_fp8_pool_with_f16_queries():
    c = Case(wl.E4M3, 8, 2, 128, SHAPES, seed=5, q_dt=wl.F16)
    check(c.run(), c.expected(), wl.E4M3, wl.F16, "fp8 pool, f16 q")
    c.close()


def test_prefill_large_group_splits_heads():
    # 20 query heads per KV head: rows cover groups of 10 heads (one token per row set)
    c = Case(wl.BF16, 40, 2, 128, [(100, 20), (33, 33)], seed=6)
    check(c.run(), c.expected(), wl.BF16, wl.BF16, "G=20")
    c.close()


def test_prefill_dead_slots_and_placement():
    """NaN in every non-live slot changes nothing, and the physical placement of
    the blocks does not change a bit."""
    shapes = [(150, 40), (31, 31), (16, 5)]
    clean = Case(wl.BF16, 16, 4, 128, shapes, seed=7)
    a = clean.run()
    dirty = Case(wl.BF16, 16, 4, 128, shapes, seed=7, poison=True)
    b = dirty.run()
    lin = Case(wl.BF16, 16, 4, 128, shapes, seed=7, free_order=lambda nb: np.arange(nb, dtype=np.int32))
    c = lin.run()
    assert np.isfinite(b).all()
    assert np.array_equal(a, b) and np.array_equal(a, c)
    check(a, clean.expected(), wl.BF16, wl.BF16, "clean")
    for x in (clean, dirty, lin):
        x.close()


def test_one_token_chunk_matches_decode():
    c = Case(wl.F16, 32, 8, 128, [(1000, 1), (333, 1), (17, 1)], seed=8)
    pre = c.run()
    mb = max(-(-n // 16) for n in c.lens)
    tables, lens = c.pool.block_tables(c.seqs, mb)
    out = c.pool.decode(harness.to_device(c.q, wl.F16), torch.from_numpy(tables).cuda(),
                        torch.from_numpy(lens).cuda(), int(c.lens.max()), c.scale)
    dec = harness.out_to_f64(out)
    assert np.abs(pre - dec).max() <= 2 * TOL[wl.F16]
    check(pre, c.expected(), wl.F16, wl.F16, "one-token chunk")
    c.close()


def test_chunks_compose():
    """A 200-token prompt attended as chunks of 64, 64 and 72 (each after the
    previous ones are cached) gives what one 200-token chunk gives."""
    c = Case(wl.BF16, 16, 4, 128, [(200, 200)], seed=9)
    whole = c.run()
    mb = -(-200 // 16)
    tables, _ = c.pool.block_tables(c.seqs, mb)
    parts, start = [], 0
    for ql in (64, 64, 72):
        n = start + ql
        q = torch.from_numpy(c.q[start:n].view(np.int16)).cuda().view(torch.bfloat16)
        out = c.pool.prefill(q, torch.tensor([0, ql], dtype=torch.int32, device="cuda"),
                             torch.from_numpy(tables).cuda(), torch.tensor([n], dtype=torch.int32, device="cuda"),
                             ql, c.scale)
        parts.append(harness.out_to_f64(out))
        start = n
    pieces = np.concatenate(parts)
    assert np.abs(pieces - whole).max() <= TOL[wl.BF16]
    check(whole, c.expected(), wl.BF16, wl.BF16, "whole")
    c.close()


def test_prefill_deterministic():
    c = Case(wl.BF16, 32, 8, 128, [(700, 128), (90, 90)], seed=10)
    outs = [c.run() for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    c.close()


@pytest.mark.parametrize("kv_dt", [wl.BF16, wl.E4M3])
def test_prefill_long_context_sampled(kv_dt):
    """2 sequences of 2048 cached tokens plus a 512-token chunk, Llama-3-8B heads
    (the prefill8b shape, and prefill8b_fp8 with an FP8 pool): sampled rows
    against the oracle (a row at position p is the one-token chunk with
    context p + 1)."""
    c = Case(kv_dt, 32, 8, 128, [(2560, 512), (2304, 256)], seed=11)
    got = c.run()
    K, V = c.oracle_kv()
    kw = dict(k_scale=c.scales[0], v_scale=c.scales[1]) if c.scales else {}
    off = [0, int(c.lens[0])]
    rows = [0, 1, 255, 256, 511, 512, 700, 767]
    for t in rows:
        s = 0 if t < c.q_start[1] else 1
        i = t - c.q_start[s]
        p = int(c.lens[s]) - int(c.q_lens[s]) + i
        want = oracle.prefill_attention(c.q[t:t + 1], c.q_dt, [0, 1], K, V, kv_dt, [off[s]], [p + 1],
                                        c.scale, **kw)
        check(got[t:t + 1], want, kv_dt, c.q_dt, f"row {t}")
    c.close()


@pytest.mark.parametrize("kv_dt", [wl.BF16, wl.E4M3])
def test_prefill_very_long_context_sampled(kv_dt):
    """A 256-token chunk after 65,280 cached tokens (4080 blocks, 2048 stages
    for the last query tile) beside a short sequence: sampled rows against the
    oracle."""
    c = Case(kv_dt, 32, 8, 128, [(65536, 256), (300, 45)], seed=13)
    got = c.run()
    K, V = c.oracle_kv()
    kw = dict(k_scale=c.scales[0], v_scale=c.scales[1]) if c.scales else {}
    off = [0, int(c.lens[0])]
    rows = [0, 127, 128, 255, 256, 300]
    for t in rows:
        s = 0 if t < c.q_start[1] else 1
        i = t - c.q_start[s]
        p = int(c.lens[s]) - int(c.q_lens[s]) + i
        want = oracle.prefill_attention(c.q[t:t + 1], c.q_dt, [0, 1], K, V, kv_dt, [off[s]], [p + 1],
                                        c.scale, **kw)
        check(got[t:t + 1], want, kv_dt, c.q_dt, f"row {t}")
    c.close()


@pytest.mark.parametrize("scale", [-0.09, 0.0])
@pytest.mark.parametrize("kv_dt", [wl.BF16, wl.E4M3])
def test_prefill_scale_sign(scale, kv_dt):
    """A negative softmax scale (the logits' order reverses) and a zero scale
    (uniform weights over the visible positions) against the oracle."""
    c = Case(kv_dt, 16, 4, 128, [(300, 45), (40, 40)], seed=12)
    c.scale = float(np.float32(scale))
    check(c.run(), c.expected(), kv_dt, c.q_dt, f"scale={scale}")
    c.close()


_DET_SHAPES = [(300, 100), (129, 64), (64, 64), (17, 17), (1000, 33)]


@pytest.mark.parametrize("kv_dt,D,G,shapes", [
    (wl.BF16, 128, 4, _DET_SHAPES), (wl.F16, 128, 1, _DET_SHAPES), (wl.BF16, 64, 8, _DET_SHAPES),
    (wl.F16, 64, 5, _DET_SHAPES), (wl.E4M3, 128, 4, _DET_SHAPES),
    (wl.BF16, 128, 4, [(150, 40), (31, 31), (16, 5)]), (wl.F16, 128, 1, [(2560, 512), (700, 90)]),
    (wl.BF16, 64, 8, [(150, 40), (31, 31)]), (wl.BF16, 128, 8, [(2304, 256), (40, 40)])])
def test_prefill_bit_identical_across_runs(kv_dt, D, G, shapes):
    """Twelve runs of the same launch give the same bits (no order or timing
    dependence in staging, softmax or the accumulation), over contexts whose
    last stage is partial, exactly full, or a single block.  An unguarded VALU
    read of a matrix-core result once showed up here as one-ulp differences
    between runs, and only under some launch orders, so the runs are many."""
    c = Case(kv_dt, 2 * G, 2, D, shapes, seed=13 + D + G + len(shapes))
    outs = [c.run() for _ in range(12)]
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"run {i} differs in {int((outs[0] != o).sum())} elements"
    check(outs[0], c.expected(), kv_dt, c.q_dt, "deterministic case")
    c.close()
