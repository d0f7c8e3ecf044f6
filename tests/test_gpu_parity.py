"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bit-exact where the result is integer or a stored copy (append contents, FP8
codes, single-token contexts, placement and NaN-masking invariance,
determinism); within the fixed tolerances elsewhere: max |out - oracle| <=
1e-4 for fp32 KV, 5e-3 for fp16/bf16 KV, 1e-2 for FP8 KV (oracle on the same
dequantised values).
"""
import math
import sys

import numpy as np
import pytest

import harness
import oracle
import paged_kv_cache_152_amd as pkv
import workloads as wl
from tests.oracle_ref import TOL, expected, fp8_codes, parity_error, raw_error

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

E4M3_TABLE = oracle.widen(np.arange(256, dtype=np.uint8), oracle.E4M3)


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def dev(a, code):
    return harness.to_device(a, code)


def run_case(w, partition=0, poison=False, free_order=None):
    """Prepare workload w on the GPU, run one decode step, return out as float64."""
    prep = harness.prepare(w, poison=poison, free_order=free_order, partition_tokens=partition)
    out = prep.step()
    torch.cuda.synchronize()
    res = harness.out_to_f64(out)
    prep.pool.close()
    return res


def assert_close(got, want, kv_dtype, what="", out_dtype=None):
    """|got - want| <= TOL[kv dtype] on every element whose oracle value is below
    2 in magnitude, and <= TOL + half an ulp of the output format above that
    (the output is stored in the q dtype: bf16 for FP8 and INT8 pools, else the
    KV dtype).  Returns the raw max |got - want|."""
    if out_dtype is None:
        out_dtype = wl.BF16 if kv_dtype in (wl.E4M3, wl.INT8) else kv_dtype
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = parity_error(got, want, out_dtype)
    raw = raw_error(got, want)
    assert err <= TOL[kv_dtype], (f"{what}: err {err:.3e} > {TOL[kv_dtype]:.0e} (raw {raw['raw_max_abs']:.3e}, "
                                  f"below |out| 2: {raw['raw_max_abs_below_2']:.3e}, max |out| {raw['max_abs_out']:.3g})")
    return raw["raw_max_abs"]


# --------------------------------------------------------------------------- codec
def test_fp8_codes_and_hardware_decode_all_256_codes():
    """Every E4M3 code survives append (encoder) and decode (hardware cvt) exactly."""
    pool = pkv.KVPool(4, 1, 128, pkv.FP8_E4M3)
    pool.set_fp8_scales([1.0], [1.0])
    vals = E4M3_TABLE.astype(np.float32).reshape(2, 1, 128)          # codes 0..127, 128..255
    src = dev(wl.cast_to_storage(vals, wl.BF16), wl.BF16)             # exact in bf16 (NaN stays NaN)
    kz = torch.zeros_like(src)
    s0, s1 = pool.seq_create(), pool.seq_create()
    slots = np.concatenate([pool.seq_reserve(s0, 1), pool.seq_reserve(s1, 1)])
    pool.append(torch.from_numpy(slots).cuda(), kz, src)
    kbuf, vbuf = pool.copy_to_host()
    codes = vbuf.reshape(4, 16, 128)[slots // 16, slots % 16].reshape(-1)
    want = np.arange(256, dtype=np.uint8)
    want[0xFF] = 0x7F                                                 # NaN input encodes as 0x7F
    assert np.array_equal(codes, want)
    tables, lens = pool.block_tables([s0, s1], 1)
    q = torch.ones((2, 1, 128), dtype=torch.bfloat16, device="cuda")
    out = harness.out_to_f64(pool.decode(q, torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda(),
                                         1, 0.1))
    ref = E4M3_TABLE.copy()
    ref[0xFF] = np.nan
    got = out.reshape(-1)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    pool.close()


def test_fp32_to_e4m3_all_2p32_patterns():
    """The device encoder equals the oracle encoder on every fp32 bit pattern."""
    H, D = 8, 128
    per_tok = H * D
    chunk = 1 << 27                                    # K and V each: 2^27 patterns per call
    T = chunk // per_tok
    nb = T // 16
    pool = pkv.KVPool(nb, H, D, pkv.FP8_E4M3)
    pool.set_fp8_scales(np.ones(H, np.float32), np.ones(H, np.float32))
    slots = torch.arange(T, dtype=torch.int32, device="cuda")
    for start in range(0, 1 << 32, 2 * chunk):
        as_i32 = lambda a: ((a + 2**31) % 2**32 - 2**31).to(torch.int32)   # same 32 bits, signed
        pk = as_i32(torch.arange(start, start + chunk, dtype=torch.int64, device="cuda"))
        pv = as_i32(torch.arange(start + chunk, start + 2 * chunk, dtype=torch.int64, device="cuda"))
        pool.append(slots, pk.view(torch.float32).view(T, H, D), pv.view(torch.float32).view(T, H, D))
        kb, vb = pool.copy_to_host()
        for buf, base in ((kb, start), (vb, start + chunk)):
            got = buf.reshape(nb, H, 16, D).transpose(0, 2, 1, 3).reshape(-1)
            pat = (np.arange(base, base + chunk, dtype=np.uint64) & 0xFFFFFFFF).astype(np.uint32)
            want = oracle.e4m3_encode(pat.view(np.float32))
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, f"patterns {pat[bad[:5]]} -> {got[bad[:5]]}, oracle {want[bad[:5]]}"
        say(f"e4m3 exhaustive: {start + 2 * chunk:#x} / 0x100000000")
    pool.close()


# -------------------------------------------------------------------------- append
@pytest.mark.parametrize("dt,D", [(wl.F32, 16), (wl.F32, 128), (wl.F16, 128), (wl.F16, 64), (wl.BF16, 128),
                                  (wl.BF16, 16)])
def test_append_bit_exact(dt, D):
    rng = np.random.default_rng(D + dt)
    H, nb, T = 3, 20, 150
    pool = pkv.KVPool(nb, H, D, dt)
    slots = rng.permutation(nb * 16)[:T].astype(np.int32)
    slots[::37] = -1                                   # skipped tokens
    K = wl.cast_to_storage(rng.standard_normal((T, H, D)).astype(np.float32), dt)
    V = wl.cast_to_storage(rng.standard_normal((T, H, D)).astype(np.float32), dt)
    pool.append(torch.from_numpy(slots).cuda(), dev(K, dt), dev(V, dt))
    kb, vb = pool.copy_to_host()
    item = wl._NP[dt]
    for buf, src in ((kb, K), (vb, V)):
        p = buf.view(item).reshape(nb, H, 16, D)
        live = slots >= 0
        got = p[slots[live] // 16, :, slots[live] % 16]                 # [T'][H][D]
        assert np.array_equal(got.view(np.uint8), src[live].view(np.uint8))
        mask = np.ones(nb * 16, bool)
        mask[slots[live]] = False
        untouched = p.transpose(0, 2, 1, 3).reshape(nb * 16, H, D)[mask]
        assert not np.any(untouched.view(np.uint8))                     # pool starts zeroed
    pool.close()


@pytest.mark.parametrize("src", [wl.BF16, wl.F32])
def test_append_fp8_codes_match_oracle(src):
    rng = np.random.default_rng(3)
    H, D, nb, T = 4, 128, 12, 180
    pool = pkv.KVPool(nb, H, D, pkv.FP8_E4M3)
    ks = np.array([0.01, 0.5, 3.0, 1e-3], np.float32)
    vs = np.array([0.2, 0.07, 1.0, 11.0], np.float32)
    pool.set_fp8_scales(ks, vs)
    slots = rng.permutation(nb * 16)[:T].astype(np.int32)
    x = (rng.standard_normal((2, T, H, D)) * 4).astype(np.float32)
    x[0, 5, 1, :8] = [np.inf, -np.inf, np.nan, 1e30, -1e30, 0.0, -0.0, 1e-30]
    if src == wl.BF16:
        K, V = wl.cast_to_storage(x[0], wl.BF16), wl.cast_to_storage(x[1], wl.BF16)
        xk, xv = wl.bf16_bits_to_f32(K), wl.bf16_bits_to_f32(V)
    else:
        K, V = x[0], x[1]
        xk, xv = K, V
    pool.append(torch.from_numpy(slots).cuda(), dev(K, src), dev(V, src))
    kb, vb = pool.copy_to_host()
    for buf, xx, sc in ((kb, xk, ks), (vb, xv, vs)):
        inv = (np.float32(1) / sc).astype(np.float32)
        want = oracle.e4m3_encode((xx * inv[None, :, None]).astype(np.float32))
        got = buf.reshape(nb, H, 16, D)[slots // 16, :, slots % 16]
        assert np.array_equal(got, want)
    pool.close()


# ------------------------------------------------------------------ small decodes
def _small(dt, Hq, Hkv, D, lens, seed=7):
    return wl.custom(seed, lens, Hq, Hkv, D, dt)


@pytest.mark.parametrize("dt", [wl.F32, wl.F16, wl.BF16, wl.E4M3])
def test_single_token_context_is_v0(dt):
    """n = 1: the only weight is exactly 1, so out = V_0 (bit-exact up to the output cast)."""
    w = _small(dt, 8, 2, 128 if dt != wl.F32 else 16, [1, 1, 1])
    got = run_case(w)
    if dt == wl.E4M3:
        sc = w.fp8_scales()[1]
        for b in range(w.B):
            _, V = w.kv(b)
            v = oracle.widen(fp8_codes(V[:1], sc), oracle.E4M3)[0] * sc.astype(np.float64)[:, None]
            want = wl.bf16_bits_to_f32(wl.cast_to_storage(v.astype(np.float32), wl.BF16)).astype(np.float64)
            assert np.array_equal(got[b].reshape(2, 4, -1), np.repeat(want[:, None], 4, axis=1))
    else:
        for b in range(w.B):
            _, V = w.kv(b)
            want = oracle.widen(V[0], dt)                                 # [H_kv][D]
            assert np.array_equal(got[b].reshape(2, 4, -1), np.repeat(want[:, None], 4, axis=1))


CASES = [
    # dtype, H_q, H_kv, D, lens
    (wl.F32, 4, 4, 16, [32, 25, 1, 17]),
    (wl.F32, 8, 2, 128, [300, 65, 16]),
    (wl.F32, 10, 2, 64, [129, 64, 200]),
    (wl.F16, 32, 32, 128, [1000, 333, 17]),
    (wl.F16, 40, 8, 128, [1000, 15, 513]),
    (wl.F16, 6, 2, 64, [777, 31]),
    (wl.F16, 4, 4, 16, [100, 33]),
    (wl.BF16, 32, 8, 128, [1000, 333, 17, 129]),
    (wl.BF16, 16, 2, 128, [640, 1]),
    (wl.BF16, 8, 8, 64, [200, 300]),
    (wl.E4M3, 32, 8, 128, [1000, 333, 17]),
    (wl.E4M3, 16, 4, 64, [500, 33]),
    (wl.E4M3, 4, 4, 16, [90, 7]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("partition", [64, 512, 0])
def test_decode_small_vs_oracle(case, partition):
    dt, Hq, Hkv, D, lens = CASES[case]
    w = _small(dt, Hq, Hkv, D, lens, seed=100 + case)
    if dt == wl.E4M3:
        w.outlier_p = 0.01
    got = run_case(w, partition=partition)
    want = expected(w)
    err = assert_close(got, want, dt, f"case {case} P={partition}")
    say(f"case {case} dt={dt} G={Hq // Hkv} D={D} P={partition}: max err {err:.2e}")


@pytest.mark.parametrize("dt", [wl.F32, wl.F16, wl.BF16, wl.E4M3])
def test_many_partitions_merge(dt):
    """Contexts of up to 47 partitions mixed with one-partition rows: the
    log-sum-exp merge matches the oracle and repeats bit for bit."""
    D = 16 if dt == wl.F32 else 128
    w = _small(dt, 16, 4, D, [3000, 64, 1, 2049, 16, 700, 3001, 65], seed=61)
    prep = harness.prepare(w, partition_tokens=64)
    prep.append_step()
    runs = [harness.out_to_f64(prep.decode()) for _ in range(3)]
    prep.pool.close()
    assert all(np.array_equal(runs[0], r) for r in runs[1:])
    assert_close(runs[0], expected(w), dt, "many partitions")


def test_batch_beyond_one_plan_workgroup():
    """1100 sequences (more than the plan kernel's 1024 threads, so its loop
    over later sequences runs), lengths over several partitions and short
    ones: every sequence against the oracle."""
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.choice([1, 17, 64, 300, 700, 1500], size=1100)]
    w = _small(wl.BF16, 8, 2, 128, lens, seed=78)
    got = run_case(w, partition=256)
    assert_close(got, expected(w), wl.BF16, "1100 sequences")


@pytest.mark.parametrize("dt", [wl.BF16, wl.E4M3])
def test_uniform_lengths_automatic_partition(dt):
    """Every context the same length with the automatic partition: the plan
    kernel re-cuts the contexts into partitions that fill whole rounds of the
    grid.  Parity with the oracle, and agreement with a fixed partition."""
    w = _small(dt, 32, 8, 128, [5000] * 8, seed=71)
    auto = run_case(w, partition=0)
    fixed = run_case(w, partition=1024)
    want = expected(w)
    assert_close(auto, want, dt, "automatic")
    assert_close(fixed, want, dt, "fixed 1024")


@pytest.mark.parametrize("D", [16, 64, 128])
@pytest.mark.parametrize("dt", [wl.F32, wl.BF16, wl.F16, wl.E4M3])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 6, 7, 8, 12, 16])
def test_every_group_size(dt, G, D):
    """Every query-head group size the kernels instantiate (1 to 8 heads per
    workgroup; 12 and 16 split into groups of 6 and 8), on the vector kernel
    (all dtypes at head_dim 16 and 64, fp32 and groups 1-2 at 128) and the
    matrix-core kernel (16-bit and FP8 at 128, groups 3 and up), against the
    oracle over one-partition and multi-partition contexts."""
    w = _small(dt, 2 * G, 2, D, [700, 1, 129, 2100], seed=90 + G + D)
    for P in (256, 0):
        got = run_case(w, partition=P)
        assert_close(got, expected(w), dt, f"G={G} P={P}")


def test_brute_force_sweep():
    """Random small shapes across dtypes, groups 1/2/4/5, head dims and edge lengths."""
    rng = np.random.default_rng(2024)
    edge = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]
    for i in range(40):
        dt = [wl.F32, wl.F16, wl.BF16, wl.E4M3][i % 4]
        G = [1, 2, 4, 5][(i // 4) % 4]
        D = [16, 64, 128][i % 3]
        Hkv = int(rng.integers(1, 4))
        B = int(rng.integers(1, 5))
        lens = [int(rng.choice(edge)) if rng.random() < 0.6 else int(rng.integers(1, 301)) for _ in range(B)]
        P = int(rng.choice([64, 128, 256, 0]))
        w = _small(dt, G * Hkv, Hkv, D, lens, seed=1000 + i)
        got = run_case(w, partition=P)
        assert_close(got, expected(w), dt, f"sweep {i}: dt={dt} G={G} D={D} lens={lens} P={P}")


# --------------------------------------------------------------- invariances
def test_placement_invariance_bit_exact():
    """Any physical placement of the blocks gives the bit-identical output."""
    w = _small(wl.BF16, 16, 4, 128, [700, 64, 333], seed=5)
    a = run_case(w, free_order=np.arange(w.num_blocks, dtype=np.int32))
    b = run_case(w, free_order=w.free_order)
    c = run_case(w, free_order=np.arange(w.num_blocks, dtype=np.int32)[::-1].copy())
    assert np.array_equal(a, b) and np.array_equal(a, c)


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16, wl.E4M3, wl.F32])
def test_nan_in_dead_slots_is_masked(dt):
    """NaN in every non-live slot (block tails, free blocks) changes nothing."""
    D = 16 if dt == wl.F32 else 128
    w = _small(dt, 8, 2, D, [37, 100, 1, 250], seed=11)
    clean = run_case(w, partition=64)
    dirty = run_case(w, partition=64, poison=True)
    assert np.isfinite(dirty).all()
    assert np.array_equal(clean, dirty)


def test_gqa_matches_repeated_kv_mha():
    G, Hkv, D = 4, 2, 128
    w = _small(wl.F16, G * Hkv, Hkv, D, [300, 77], seed=21)
    gqa = run_case(w, partition=128)
    # MHA pool holding each KV head repeated G times, filled from the same logical K/V
    pool = pkv.KVPool(w.num_blocks * G, G * Hkv, D, wl.F16)
    pool.set_partition(128)
    seqs = []
    for b in range(w.B):
        s = pool.seq_create()
        seqs.append(s)
        K, V = w.kv(b)
        n = int(w.lens[b])
        sl = pool.seq_reserve(s, n)
        pool.append(torch.from_numpy(sl).cuda(), dev(np.repeat(K[:n], G, axis=1), wl.F16),
                    dev(np.repeat(V[:n], G, axis=1), wl.F16))
    t, l = pool.block_tables(seqs, w.max_blocks_per_seq())
    out = pool.decode(dev(w.q(), wl.F16), torch.from_numpy(t).cuda(), torch.from_numpy(l).cuda(), w.max_len(),
                      w.scale)
    mha = harness.out_to_f64(out)
    pool.close()
    assert np.abs(gqa - mha).max() <= 1e-3
    assert_close(gqa, expected(w), wl.F16)


def test_deterministic():
    w = _small(wl.BF16, 32, 8, 128, [2000, 1500, 9], seed=31)
    prep = harness.prepare(w, partition_tokens=256)
    prep.append_step()
    outs = [harness.out_to_f64(prep.decode()) for _ in range(3)]
    prep.pool.close()
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


@pytest.mark.parametrize("dt,Hq,Hkv", [(wl.F16, 8, 8), (wl.BF16, 32, 8), (wl.F16, 40, 8), (wl.E4M3, 32, 8)])
def test_decode_bit_identical_across_runs(dt, Hq, Hkv):
    """Twelve launches of one decode give the same bits, on the vector kernel
    (MHA) and the matrix-core kernel (groups 4 and 5, FP8): the work list
    decides which workgroup computes an item, never the item's arithmetic or
    the order of the merge."""
    w = _small(dt, Hq, Hkv, 128, [3000, 1, 2049, 700, 4100, 16, 9000, 257], seed=71 + Hq)
    prep = harness.prepare(w, partition_tokens=256)
    prep.append_step()
    outs = [harness.out_to_f64(prep.decode()) for _ in range(12)]
    prep.pool.close()
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"run {i} differs in {int((outs[0] != o).sum())} elements"
    assert_close(outs[0], expected(w), dt, "deterministic")


@pytest.mark.parametrize("name", ["gqa8b", "fp8"])
def test_full_size_decode_bit_identical_across_runs(name):
    """Five launches at full size (768 resident workgroups taking items from
    the work list under full HBM load) give the same bits."""
    w = wl.make(name)
    prep = harness.prepare(w)
    prep.append_step()
    outs = [harness.out_to_f64(prep.decode()) for _ in range(5)]
    prep.pool.close()
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"{name}: run {i} differs in {int((outs[0] != o).sum())} elements"


def test_zero_lengths_and_bad_table_entries():
    w = _small(wl.F16, 8, 2, 128, [100, 40], seed=41)
    prep = harness.prepare(w, partition_tokens=64)
    prep.append_step()
    # a zero-length row, and a table entry outside the pool
    lens = prep.lens.clone()
    lens[1] = 0
    out = harness.out_to_f64(prep.pool.decode(prep.q, prep.tables, lens, prep.max_len, w.scale))
    assert np.array_equal(out[1], np.zeros_like(out[1]))
    assert_close(out[0], expected(w, seqs=[0])[0], wl.F16)
    tables = prep.tables.clone()
    tables[0, 2] = w.num_blocks + 5                  # tokens 32..47 count as absent
    tables[0, 3] = -7                                # tokens 48..63 count as absent
    out = harness.out_to_f64(prep.pool.decode(prep.q, tables, prep.lens, prep.max_len, w.scale))
    assert np.isfinite(out).all()
    # the result equals attention over the remaining tokens
    K, V = w.kv(0)
    keep = np.r_[0:32, 64:100]
    q = w.q()[:1]
    ref = oracle.decode_attention(q, wl.F16, K[keep], V[keep], wl.F16, [0], [len(keep)], w.scale)
    assert_close(out[0], ref[0], wl.F16)
    # lengths beyond the host bound are clamped, never read past the table
    lens = prep.lens.clone()
    lens[0] = 10**6
    out = harness.out_to_f64(prep.pool.decode(prep.q, prep.tables, lens, prep.max_len, w.scale))
    assert np.isfinite(out).all()
    prep.pool.close()


# ------------------------------------------------------------------ configurations
def test_tiny_config_cached_decode_equals_recompute():
    """1 seq, 4 heads, d 16, fp32: prefill 24 then 8 steps; each step equals the
    oracle recomputing attention over the whole history from the seed."""
    w = wl.make("tiny")
    pool = pkv.KVPool(w.num_blocks, w.H_kv, w.D, w.kv_dtype, free_order=w.free_order)
    s = pool.seq_create()
    K, V = w.kv(0)
    sl = pool.seq_reserve(s, int(w.prefill[0]))
    pool.append(torch.from_numpy(sl).cuda(), dev(K[:24], wl.F32), dev(V[:24], wl.F32))
    for step in range(w.decode_steps):
        n = 24 + step + 1
        sl = pool.seq_reserve(s, 1)
        pool.append(torch.from_numpy(sl).cuda(), dev(K[n - 1:n], wl.F32), dev(V[n - 1:n], wl.F32))
        t, l = pool.block_tables([s], 2)
        assert l[0] == n and (t[0] >= 0).sum() == 2
        out = harness.out_to_f64(pool.decode(dev(w.q(step), wl.F32), torch.from_numpy(t).cuda(),
                                             torch.from_numpy(l).cuda(), 32, w.scale))
        want = oracle.decode_attention(w.q(step), wl.F32, K[:n], V[:n], wl.F32, [0], [n], w.scale)
        assert_close(out, want, wl.F32, f"step {step}")
    pool.close()


def test_mini_model_walkthrough():
    """d_model 64, 4 heads of 16: prefill 5 tokens then 3 decode steps (cache 5 -> 8).
    Each step's paged decode equals full no-cache causal attention's last row."""
    x, Wq, Wk, Wv = wl.mini_model_inputs(seed=7, n_tokens=8)
    H, dk = 4, 16
    Q = (x @ Wq).reshape(8, H, dk).astype(np.float32)
    Kx = (x @ Wk).reshape(8, H, dk).astype(np.float32)
    Vx = (x @ Wv).reshape(8, H, dk).astype(np.float32)
    scale = float(np.float32(1 / math.sqrt(dk)))
    full = oracle.causal_attention(Q.astype(np.float64), Kx.astype(np.float64), Vx.astype(np.float64), scale)
    pool = pkv.KVPool(4, H, dk, pkv.F32, free_order=[2, 0, 3, 1])
    s = pool.seq_create()
    sl = pool.seq_reserve(s, 5)
    pool.append(torch.from_numpy(sl).cuda(), dev(Kx[:5], wl.F32), dev(Vx[:5], wl.F32))
    for t in range(5, 9):
        if t > 5:
            sl = pool.seq_reserve(s, 1)
            pool.append(torch.from_numpy(sl).cuda(), dev(Kx[t - 1:t], wl.F32), dev(Vx[t - 1:t], wl.F32))
        tb, ln = pool.block_tables([s], 1)
        out = harness.out_to_f64(pool.decode(dev(Q[t - 1:t], wl.F32), torch.from_numpy(tb).cuda(),
                                             torch.from_numpy(ln).cuda(), 16, scale))
        assert np.abs(out[0] - full[t - 1]).max() <= 1e-4
    pool.close()


FULL_CHUNK = 32      # sequences per oracle call (bounds the host memory of one call)


@pytest.mark.parametrize("name", ["mha7b", "gqa8b", "mixed", "fp8", "int8"])
def test_full_size_config_every_sequence(name):
    """Full-size workloads in the launch configuration the benchmark times:
    every sequence, every head and every output element against the oracle.
    Prints the raw max |out - oracle| over all elements and over |oracle| < 2."""
    w = wl.make(name)
    w.cache_kv = True                      # the oracle reads the K/V the pool was filled with
    say(f"{name}: preparing {w.B} seqs, {w.num_blocks} blocks")
    prep = harness.prepare(w)
    out = prep.step()
    torch.cuda.synchronize()
    got = harness.out_to_f64(out)
    assert np.isfinite(got).all()
    if w.sharers:
        info = prep.pool.info()
        assert info["shared_blocks"] == w.prefix_tokens // 16
        for blk in prep.host_tables[w.sharers[0], : w.prefix_tokens // 16]:
            assert prep.pool.block_refcount(int(blk)) == len(w.sharers)
    prep.pool.close()
    want = np.concatenate([expected(w, seqs=range(s0, min(w.B, s0 + FULL_CHUNK)))
                           for s0 in range(0, w.B, FULL_CHUNK)])
    w._kv_cache.clear()
    raw = assert_close(got, want, w.kv_dtype, name)
    r = raw_error(got, want)
    say(f"PARITY {name}: all {w.B} sequences, {got.size} outputs; raw max-abs {r['raw_max_abs']:.3e}, "
        f"over |oracle| < 2 {r['raw_max_abs_below_2']:.3e}, max |oracle| {r['max_abs_out']:.3g}; "
        f"held to {TOL[w.kv_dtype]:.0e}")
    assert raw == r["raw_max_abs"]


@pytest.mark.parametrize("partition", [0, 256])
def test_very_long_context(partition):
    """One sequence of 262,144 tokens (GQA 32/8, bf16; 1 GiB of K/V) beside two
    short ones: the automatic partition and 256-token partitions (1024 of them,
    the merge's general loop), every output against the oracle."""
    w = wl.custom(91, [262144, 17, 3000], 32, 8, 128, wl.BF16)
    w.cache_kv = True
    say(f"[test] very long context, partition {partition}: {w.num_blocks} blocks")
    prep = harness.prepare(w, partition_tokens=partition)
    out = prep.step()
    torch.cuda.synchronize()
    got = harness.out_to_f64(out)
    prep.pool.close()
    want = expected(w)
    w._kv_cache.clear()
    err = assert_close(got, want, wl.BF16, f"262144 tokens P={partition}")
    say(f"very long context P={partition}: raw max-abs {err:.2e}")


# ------------------------------------------------------------------ closed forms
# softmax(s q K^T) V (www.mlqm.cn/news/394450, section 二) in cases where the
# result has a form of its own: s = 0 or q = 0 weighs every token equally (the
# mean of V), a constant V comes back unchanged, and two tokens mix by the
# logistic function of their logit difference.  Each is checked on the vector
# kernel (MHA, small groups, fp32 and head_dim 16 / 64) and on the matrix-core
# kernel (groups >= 3 at head_dim 128), over one and several partitions.
KERNEL_SHAPES = [
    # dtype, D, G        kernel
    (wl.F32, 16, 1),     # vector
    (wl.F16, 128, 1),    # vector
    (wl.BF16, 64, 2),    # vector
    (wl.E4M3, 64, 1),    # vector
    (wl.BF16, 128, 4),   # matrix cores
    (wl.F16, 128, 5),    # matrix cores
    (wl.E4M3, 128, 4),   # matrix cores
]


class ClosedFormPool:
    """A pool holding given per-sequence K/V (stored dtype values; bf16 sources for FP8)."""

    def __init__(self, dt, D, G, Ks, Vs, partition, seed):
        self.dt, self.D, self.G = dt, D, G
        self.H_kv = Ks[0].shape[1]
        self.src = wl.BF16 if dt == wl.E4M3 else dt
        nb = sum(-(-len(k) // 16) for k in Ks) + 3
        rng = np.random.default_rng(seed)
        self.pool = pkv.KVPool(nb, self.H_kv, D, dt, free_order=rng.permutation(nb))
        self.pool.set_partition(partition)
        self.vscale = None
        if dt == wl.E4M3:
            self.kscale = np.full(self.H_kv, 0.02, np.float32)
            self.vscale = np.full(self.H_kv, 0.0078125, np.float32)      # 2^-7: codes * scale exact in fp32
            self.pool.set_fp8_scales(self.kscale, self.vscale)
        self.seqs = []
        for K, V in zip(Ks, Vs):
            s = self.pool.seq_create()
            self.seqs.append(s)
            sl = self.pool.seq_reserve(s, len(K))
            self.pool.append(torch.from_numpy(sl).cuda(), dev(K, self.src), dev(V, self.src))
        self.tables, self.lens = self.pool.block_tables(self.seqs, max(-(-len(k) // 16) for k in Ks))

    def values(self, X, which):
        """fp64 values the pool holds for source rows X (FP8: decoded codes times the scale)."""
        if self.dt == wl.E4M3:
            sc = self.kscale if which == "k" else self.vscale
            return oracle.widen(fp8_codes(X, sc), oracle.E4M3) * sc.astype(np.float64)[None, :, None]
        return oracle.widen(X, self.dt)

    def decode(self, q, scale):
        qd = wl.BF16 if self.dt == wl.E4M3 else self.dt
        out = self.pool.decode(dev(q, qd), torch.from_numpy(self.tables).cuda(), torch.from_numpy(self.lens).cuda(),
                               int(self.lens.max()), scale)
        torch.cuda.synchronize()
        return harness.out_to_f64(out)

    def close(self):
        self.pool.close()


def _src(rng, shape, dt):
    return wl.cast_to_storage(rng.standard_normal(shape).astype(np.float32), wl.BF16 if dt == wl.E4M3 else dt)


@pytest.mark.parametrize("partition", [256, 0])
@pytest.mark.parametrize("shape", range(len(KERNEL_SHAPES)))
def test_closed_form_equal_weights_give_mean_of_v(shape, partition):
    """s = 0, and separately q = 0: every weight is 1/n, so out = mean_j V_j."""
    dt, D, G = KERNEL_SHAPES[shape]
    rng = np.random.default_rng(500 + shape)
    H_kv, lens = 2, [1, 17, 300, 2100]
    Ks = [_src(rng, (n, H_kv, D), dt) for n in lens]
    Vs = [_src(rng, (n, H_kv, D), dt) for n in lens]
    c = ClosedFormPool(dt, D, G, Ks, Vs, partition, seed=shape)
    mean = np.stack([c.values(V, "v").mean(axis=0) for V in Vs])                 # [B][H_kv][D]
    want = np.repeat(mean, G, axis=1)                                             # q head h -> KV head h // G
    qd = wl.BF16 if dt == wl.E4M3 else dt
    q = _src(rng, (len(lens), G * H_kv, D), qd)
    e1 = assert_close(c.decode(q, 0.0), want, dt, "scale 0")
    zero = wl.cast_to_storage(np.zeros((len(lens), G * H_kv, D), np.float32), qd)
    e2 = assert_close(c.decode(zero, float(np.float32(1 / math.sqrt(D)))), want, dt, "q = 0")
    say(f"closed form mean: dt={dt} D={D} G={G} P={partition}: raw {e1:.2e} (s = 0), {e2:.2e} (q = 0)")
    c.close()


@pytest.mark.parametrize("partition", [256, 0])
@pytest.mark.parametrize("shape", range(len(KERNEL_SHAPES)))
def test_closed_form_constant_values_come_back(shape, partition):
    """V_j = c for every token (per KV head and dim), any keys: out = c."""
    dt, D, G = KERNEL_SHAPES[shape]
    rng = np.random.default_rng(600 + shape)
    H_kv, lens = 2, [1, 17, 300, 2100]
    Ks = [_src(rng, (n, H_kv, D), dt) for n in lens]
    row = _src(rng, (1, H_kv, D), dt)
    if dt == wl.E4M3:                      # values on the E4M3 grid times the V scale, so c is stored exactly
        grid = wl.cast_to_storage((oracle.widen(fp8_codes(row, np.full(H_kv, 0.0078125, np.float32)), oracle.E4M3)
                                   * 0.0078125).astype(np.float32), wl.BF16)
        row = grid
    Vs = [np.repeat(row, n, axis=0) for n in lens]
    c = ClosedFormPool(dt, D, G, Ks, Vs, partition, seed=shape)
    cval = c.values(row, "v")[0]                                                  # [H_kv][D]
    want = np.repeat(np.repeat(cval[None], len(lens), axis=0), G, axis=1)
    qd = wl.BF16 if dt == wl.E4M3 else dt
    q = wl.cast_to_storage((rng.standard_normal((len(lens), G * H_kv, D)) * 3).astype(np.float32), qd)
    e = assert_close(c.decode(q, float(np.float32(1 / math.sqrt(D)))), want, dt, "constant V")
    say(f"closed form constant V: dt={dt} D={D} G={G} P={partition}: raw {e:.2e}")
    c.close()


@pytest.mark.parametrize("shape", range(len(KERNEL_SHAPES)))
def test_closed_form_two_tokens_mix_by_logistic(shape):
    """n = 2: out = sigma(z0 - z1) V0 + sigma(z1 - z0) V1 with z_j = s <q, K_j>,
    evaluated in fp64 from the stored values (no softmax routine)."""
    dt, D, G = KERNEL_SHAPES[shape]
    rng = np.random.default_rng(700 + shape)
    H_kv, B = 2, 6
    Ks = [_src(rng, (2, H_kv, D), dt) for _ in range(B)]
    Vs = [_src(rng, (2, H_kv, D), dt) for _ in range(B)]
    c = ClosedFormPool(dt, D, G, Ks, Vs, 0, seed=shape)
    qd = wl.BF16 if dt == wl.E4M3 else dt
    q = _src(rng, (B, G * H_kv, D), qd)
    s = float(np.float32(1 / math.sqrt(D)))
    got = c.decode(q, s)
    qv = oracle.widen(q, qd)
    want = np.empty_like(got)
    for b in range(B):
        K, V = c.values(Ks[b], "k"), c.values(Vs[b], "v")
        for h in range(G * H_kv):
            g = h // G
            dz = s * (qv[b, h] @ K[0, g] - qv[b, h] @ K[1, g])
            a = 1.0 / (1.0 + math.exp(-dz))
            want[b, h] = a * V[0, g] + (1.0 - a) * V[1, g]
    e = assert_close(got, want, dt, "two tokens")
    say(f"closed form two tokens: dt={dt} D={D} G={G}: raw {e:.2e}")
    c.close()


def test_copy_on_write_branches_decode_their_own_history():
    """Beam-style forks at a partial block (cf-1.com/news/5824798 §3.3): every branch
    appends its own tokens; each must attend to the shared prompt plus its own tail,
    the shared full blocks stay shared, and no branch sees another's writes."""
    rng = np.random.default_rng(17)
    H_kv, G, D, n0 = 2, 3, 128, 37
    pool = pkv.KVPool(24, H_kv, D, pkv.F16, free_order=rng.permutation(24))
    parent = pool.seq_create()
    K0 = rng.standard_normal((n0, H_kv, D)).astype(np.float16)
    V0 = rng.standard_normal((n0, H_kv, D)).astype(np.float16)
    pool.append(torch.from_numpy(pool.seq_reserve(parent, n0)).cuda(), dev(K0, wl.F16), dev(V0, wl.F16))
    seqs = [parent] + [pool.seq_fork(parent, n0) for _ in range(3)]
    hist = {s: (K0, V0) for s in seqs}
    shared_full = pool.block_tables([parent], 8)[0][0][:2].copy()
    for step in range(20):
        slots = pool.batch_reserve(seqs)
        if step == 0:
            assert len(pool.pending_copies()) == 3             # three writers copy, the last owns it
        k = rng.standard_normal((len(seqs), H_kv, D)).astype(np.float16)
        v = rng.standard_normal((len(seqs), H_kv, D)).astype(np.float16)
        pool.append(torch.from_numpy(slots).cuda(), dev(k, wl.F16), dev(v, wl.F16))
        assert pool.pending_copies() == []
        for i, s in enumerate(seqs):
            hist[s] = (np.concatenate([hist[s][0], k[i:i + 1]]), np.concatenate([hist[s][1], v[i:i + 1]]))
        tables, lens = pool.block_tables(seqs, 8)
        q = rng.standard_normal((len(seqs), G * H_kv, D)).astype(np.float16)
        out = harness.out_to_f64(pool.decode(dev(q, wl.F16), torch.from_numpy(tables).cuda(),
                                             torch.from_numpy(lens).cuda(), int(lens.max()), 1 / math.sqrt(D)))
        for i, s in enumerate(seqs):
            Kh, Vh = hist[s]
            want = oracle.decode_attention(q[i:i + 1], wl.F16, Kh, Vh, wl.F16, [0], [len(Kh)], 1 / math.sqrt(D))
            assert_close(out[i:i + 1], want, wl.F16, f"step {step} branch {i}")
    for blk in shared_full:
        assert pool.block_refcount(int(blk)) == len(seqs)
    pool.close()


def test_prefix_cache_reuse_decodes_the_cached_prompt():
    """Prefix caching (cf-1.com/news/5824798 §3.3; m.lqnn.cn/news/219451 §3): a
    request whose prompt starts like a registered one takes over the cached full
    blocks and computes K/V only for the rest; its decode must equal the oracle
    over (cached prefix K/V + its own tail).  Blocks released by every holder stay
    reusable until allocation evicts them, and an evicted block then holds the
    new owner's data only."""
    rng = np.random.default_rng(23)
    H_kv, G, D, N = 2, 4, 128, 48
    dt, scale = wl.BF16, 1 / math.sqrt(D)
    pool = pkv.KVPool(N, H_kv, D, pkv.BF16, free_order=rng.permutation(N))

    def kv(n):
        return (rng.standard_normal((n, H_kv, D)).astype(np.float32),
                rng.standard_normal((n, H_kv, D)).astype(np.float32))

    def put(seq, K, V):
        slots = pool.seq_reserve(seq, len(K))
        pool.append(torch.from_numpy(slots).cuda(), dev(wl.f32_to_bf16_bits(K), dt), dev(wl.f32_to_bf16_bits(V), dt))

    def check(seqs, hist, what):
        tables, lens = pool.block_tables(seqs, N)
        q = wl.f32_to_bf16_bits(rng.standard_normal((len(seqs), G * H_kv, D)).astype(np.float32))
        out = harness.out_to_f64(pool.decode(dev(q, dt), torch.from_numpy(tables).cuda(),
                                             torch.from_numpy(lens).cuda(), int(lens.max()), scale))
        for i, (K, V) in enumerate(hist):
            assert lens[i] == len(K)
            Kb, Vb = wl.f32_to_bf16_bits(K), wl.f32_to_bf16_bits(V)
            want = oracle.decode_attention(q[i:i + 1], dt, Kb, Vb, dt, [0], [len(K)], scale)
            assert_close(out[i:i + 1], want, dt, f"{what} seq {i}")

    prompt = [int(t) for t in rng.integers(0, 32000, size=300)]   # 18 full blocks + 12 tokens
    a = pool.seq_create()
    KA, VA = kv(300)
    put(a, KA, VA)
    assert pool.prefix_register(a, prompt, ns=5) == 18
    # B shares 17 blocks (272 tokens), then diverges
    b_prompt = prompt[:272] + [int(t) for t in rng.integers(0, 32000, size=40)]
    b, hit = pool.seq_create_cached(b_prompt, ns=5)
    assert hit == 272 and pool.block_tables([b], 32)[0][0][:17].tolist() == pool.block_tables([a], 32)[0][0][:17].tolist()
    assert pool.seq_create_cached(prompt, ns=6)[1] == 0                 # other namespace
    KB, VB = kv(40)
    put(b, KB, VB)
    hist_b = (np.concatenate([KA[:272], KB]), np.concatenate([VA[:272], VB]))
    check([a, b], [(KA, VA), hist_b], "shared prefix")
    # A finishes: its keyed block 17 stays evictable, its partial block is freed
    pool.seq_free(a)
    info = pool.info()
    assert info["evictable_blocks"] == 1 and info["cached_blocks"] == 18
    c, hit = pool.seq_create_cached(prompt + [1, 2, 3], ns=5)
    assert hit == 288 and pool.info()["evictable_blocks"] == 0
    KC, VC = kv(15)
    put(c, KC, VC)
    hist_c = (np.concatenate([KA[:288], KC]), np.concatenate([VA[:288], VC]))
    check([b, c], [hist_b, hist_c], "reuse after release")
    # everyone leaves; a long sequence then needs every block: the cache is evicted
    pool.seq_free(b)
    pool.seq_free(c)
    assert pool.info()["evictable_blocks"] == 18
    d = pool.seq_create()
    KD, VD = kv(N * 16)
    put(d, KD, VD)
    info = pool.info()
    assert info["cached_blocks"] == 0 and info["free_blocks"] == 0
    check([d], [(KD, VD)], "after eviction")
    pool.seq_free(d)
    assert pool.seq_create_cached(prompt, ns=5)[1] == 0
    pool.close()
