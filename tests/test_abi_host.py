"""C-ABI library on the CPU: it loads, exports what include/pagedkv.h declares,
its allocator matches the Python model bit for bit, and it validates arguments.

No GPU is touched: allocator tests use metadata-only (host-only) pools, and
the device entry points are called only with arguments they must refuse
before any device work.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_cache_152_amd as pkv
from oracle.allocator_model import AllocError, BlockPoolModel

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pagedkv.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|uint64_t|size_t|int32_t|char\s*\*|void)\s*\**\s*"
                                 r"(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_binding_surface():
    names = _declared()
    assert "kv_pool_create" in names and "kv_append" in names and "paged_decode" in names
    assert sorted(pkv.EXPORTED) == names


def test_library_exports_every_declared_symbol():
    L = pkv.lib()
    for name in _declared():
        assert hasattr(L, name), name
    # and nothing but the C ABI (internal C++ symbols are hidden)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == _declared()


def test_kv_cache_bytes_matches_formula():
    assert pkv.kv_cache_bytes(32, 32, 128, 2, 1, 1) == 524288
    assert pkv.kv_cache_bytes(40, 8, 128, 2, 1, 1) == 163840
    assert pkv.kv_cache_bytes(2, 2, 4, 2, 10, 1) == 640
    assert pkv.kv_cache_bytes(0, 2, 4, 2, 10, 1) == 0


def _code(e):
    return e.code


MAP = {1: pkv.ERR_INVALID_ARG, 2: pkv.ERR_NO_BLOCKS, 3: pkv.ERR_OUT_OF_RANGE, 4: pkv.ERR_STATE}


def _compare(pool, model, live):
    assert list(pool.free_list()) == model.free_list()
    for b in range(model.N):
        assert pool.block_refcount(b) == model.refcount(b)
    resident = [s for s in live if s not in model.swapped]
    if resident:
        mb = max(1, max(len(model.table(s)) for s in resident))
        t, l = pool.block_tables(resident, mb)
        mt, ml = model.tables(resident, mb)
        assert np.array_equal(t, np.array(mt, np.int32)) and list(l) == ml
    for s in live:
        assert pool.seq_length(s) == model.length(s)
    info = pool.info()
    assert info["free_blocks"] == len(model.free_list())
    assert info["shared_blocks"] == model.shared_blocks()
    assert info["live_seqs"] == len(live)
    assert info["cached_blocks"] == len(model.cache) and info["evictable_blocks"] == len(model.lru)


_TOKS = {}


def _tokens(seq, n):
    """Deterministic token ids for a sequence's first n positions (few distinct
    prompts, so prefixes repeat across sequences)."""
    base = _TOKS.get(seq, [])
    while len(base) < n:
        base = base + [(seq % 3) * 1000 + len(base) % 37]
    _TOKS[seq] = base
    return base[:n]


@pytest.mark.parametrize("seed", range(12))
def test_allocator_matches_model_on_random_traces(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(8, 65))
    order = rng.permutation(n)
    pool = pkv.KVPool(n, 2, 16, pkv.F32, free_order=order, host_only=True)
    model = BlockPoolModel(n, 16, free_order=order)
    live = []
    _TOKS.clear()
    hits = evicted = swaps = 0
    for step in range(800):
        cached_before = len(model.cache)
        op = int(rng.integers(0, 10))
        resident = [x for x in live if x not in model.swapped]
        if op == 8 and resident:                        # swap a sequence out (no data on this pool)
            s = resident[int(rng.integers(len(resident)))]
            model.swap_out(s)
            assert pool.swap_out(s) is None
            swaps += 1
        elif op == 9 and model.swapped & set(live):     # and back in
            s = sorted(model.swapped & set(live))[int(rng.integers(len(model.swapped & set(live))))]
            try:
                model.swap_in(s)
            except AllocError as e:
                with pytest.raises(pkv.PagedKVError) as got:
                    pool.swap_in(s)
                assert got.value.code == MAP[e.code]
            else:
                pool.swap_in(s)
        elif op in (5, 6, 3) and not resident:
            pass
        elif op == 5 and live:                          # publish a sequence's blocks
            s = resident[int(rng.integers(len(resident)))]
            toks = _tokens(s, model.length(s))
            assert pool.prefix_register(s, toks, ns=s % 3) == model.prefix_register(s, toks, ns=s % 3)
        elif op == 6 and live:                          # a request reusing a cached prefix
            s = resident[int(rng.integers(len(resident)))]
            toks = _tokens(s, model.length(s)) + [7] * int(rng.integers(0, 20))
            a, b = pool.seq_create_cached(toks, ns=s % 3), model.seq_create_cached(toks, ns=s % 3)
            assert a == b
            live.append(a[0])
            _TOKS[a[0]] = toks[: a[1]]
            hits += a[1] // 16
        elif op == 7 and rng.random() < 0.05:
            pool.prefix_evict_all()
            model.prefix_evict_all()
        elif op == 0 or not live:
            a, b = pool.seq_create(), model.seq_create()
            assert a == b
            live.append(a)
        elif op in (1, 2):
            s = live[int(rng.integers(len(live)))]
            k = int(rng.integers(0, 40))
            try:
                want = model.reserve(s, k)
            except AllocError as e:
                with pytest.raises(pkv.PagedKVError) as got:
                    pool.seq_reserve(s, k)
                assert got.value.code == MAP[e.code]
            else:
                assert list(pool.seq_reserve(s, k)) == want
            assert pool.seq_length(s) == model.length(s)
        elif op == 3:
            p = resident[int(rng.integers(len(resident)))]
            k = int(rng.integers(0, model.length(p) + 1))      # any length: partial blocks shared
            a, b = pool.seq_fork(p, k), model.fork(p, k)
            assert a == b
            live.append(a)
        else:
            s = live.pop(int(rng.integers(len(live))))
            pool.seq_free(s)
            model.free_seq(s)
        model.check_invariants()
        if op in (1, 2) and len(model.cache) < cached_before:
            evicted += cached_before - len(model.cache)
        if step % 25 == 0:
            _compare(pool, model, live)
            assert pool.pending_copies() == model.take_copies()
            pool.apply_copies()
            assert pool.pending_copies() == []
    _compare(pool, model, live)
    assert pool.pending_copies() == model.take_copies()
    pool.close()
    print(f"seed {seed}: {hits} cached blocks reused, {evicted} evicted by allocation, {swaps} swaps")
    assert hits > 0 and swaps > 0


def test_allocator_errors():
    pool = pkv.KVPool(4, 1, 16, pkv.F16, host_only=True)
    s = pool.seq_create()
    pool.seq_reserve(s, 40)
    before = (pool.block_tables([s], 4), list(pool.free_list()))
    with pytest.raises(pkv.PagedKVError) as e:
        pool.seq_reserve(s, 40)
    assert e.value.code == pkv.ERR_NO_BLOCKS
    after = (pool.block_tables([s], 4), list(pool.free_list()))
    assert np.array_equal(before[0][0], after[0][0]) and before[1] == after[1]
    for bad in (48, -16):
        with pytest.raises(pkv.PagedKVError) as e:
            pool.seq_fork(s, bad)
        assert e.value.code == pkv.ERR_INVALID_ARG
    with pytest.raises(pkv.PagedKVError) as e:
        pool.block_tables([s], 2)
    assert e.value.code == pkv.ERR_OUT_OF_RANGE
    t, l = pool.block_tables([s], 5)
    assert list(t[0][3:]) == [-1, -1] and l[0] == 40
    pool.seq_free(s)
    for fn in (lambda: pool.seq_free(s), lambda: pool.seq_reserve(s, 1), lambda: pool.seq_length(s),
               lambda: pool.block_tables([s], 4), lambda: pool.seq_fork(s, 0), lambda: pool.seq_free(999)):
        with pytest.raises(pkv.PagedKVError) as e:
            fn()
        assert e.value.code == pkv.ERR_STATE
    with pytest.raises(pkv.PagedKVError) as e:
        pool.block_refcount(4)
    assert e.value.code == pkv.ERR_INVALID_ARG
    pool.close()


def test_pool_create_validation():
    cases = [((0, 1, 16, pkv.F16), pkv.ERR_INVALID_ARG), ((4, 0, 16, pkv.F16), pkv.ERR_INVALID_ARG),
             ((4, 1, 0, pkv.F16), pkv.ERR_INVALID_ARG), ((4, 1, 96, pkv.F16), pkv.ERR_UNSUPPORTED),
             ((4, 1, 127, pkv.F16), pkv.ERR_UNSUPPORTED), ((4, 1, 16, 9), pkv.ERR_UNSUPPORTED)]
    for args, code in cases:
        with pytest.raises(pkv.PagedKVError) as e:
            pkv.KVPool(*args, host_only=True)
        assert e.value.code == code, args
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.KVPool(4, 1, 16, pkv.F16, block_size=32, host_only=True)
    assert e.value.code == pkv.ERR_UNSUPPORTED
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.KVPool(4, 1, 16, pkv.F16, free_order=[0, 1, 1, 3], host_only=True)
    assert e.value.code == pkv.ERR_INVALID_ARG


def test_pool_info_bytes():
    # [moo] §3.1 layout for one layer: K and V each num_blocks * H_kv * 16 * d * elem
    for dt, e in ((pkv.F32, 4), (pkv.F16, 2), (pkv.BF16, 2), (pkv.FP8_E4M3, 1)):
        p = pkv.KVPool(10, 8, 128, dt, host_only=True)
        inf = p.info()
        assert inf["pool_bytes"] == 10 * 8 * 16 * 128 * e
        assert inf["block_bytes"] == 16 * 128 * e
        assert inf["host_only"] == 1 and inf["total_bytes"] == 0
        assert inf["free_blocks"] == 10 and inf["used_blocks"] == 0
        p.close()


def test_int8_pool_layout_and_pairings():
    """INT8 min-max pools: a tile is 16 x head_dim codes plus a 16-byte header;
    appends take BF16 / F16 / F32 sources only; decode takes BF16 or F16
    queries; prefill has no INT8 kernel; FP8 scales do not apply."""
    L = pkv.lib()
    for D in (16, 64, 128):
        p = pkv.KVPool(10, 8, D, pkv.INT8_MINMAX, host_only=True)
        inf = p.info()
        assert inf["block_bytes"] == 16 * D + 16 and inf["elem_bytes"] == 1
        assert inf["pool_bytes"] == 10 * 8 * (16 * D + 16)
        p.close()
    p = pkv.KVPool(8, 2, 128, pkv.INT8_MINMAX, host_only=True)
    h = p.handle
    fake = ctypes.c_void_p(0x10000)     # never dereferenced: every call below is refused on the host
    ap = lambda dt: L.kv_append(h, fake, 3, fake, fake, dt, None)
    for dt in (pkv.BF16, pkv.F16, pkv.F32):
        assert ap(dt) == pkv.ERR_STATE                 # accepted pairing; host-only pool
    for dt in (pkv.FP8_E4M3, pkv.INT8_MINMAX):
        assert ap(dt) == pkv.ERR_UNSUPPORTED
    dec = lambda qdt: L.paged_decode(h, fake, qdt, 2, 8, fake, 4, fake, 64, 0.125, fake, None, 0, None)
    assert dec(pkv.BF16) == pkv.ERR_STATE and dec(pkv.F16) == pkv.ERR_STATE
    assert dec(pkv.F32) == pkv.ERR_UNSUPPORTED
    pre = L.paged_prefill(h, fake, pkv.BF16, 1, 8, fake, 4, 4, fake, 4, fake, 0.1, 1, fake, None)
    assert pre == pkv.ERR_UNSUPPORTED
    with pytest.raises(pkv.PagedKVError) as e:
        p.set_fp8_scales([1.0, 1.0], [1.0, 1.0])
    assert e.value.code == pkv.ERR_STATE
    p.close()


def test_fp8_scale_validation():
    p = pkv.KVPool(4, 2, 128, pkv.FP8_E4M3, host_only=True)
    p.set_fp8_scales([0.5, 0.25], [1.0, 2.0])
    for bad in ([0.0, 1.0], [-1.0, 1.0], [np.inf, 1.0], [np.nan, 1.0]):
        with pytest.raises(pkv.PagedKVError) as e:
            p.set_fp8_scales(bad, [1.0, 1.0])
        assert e.value.code == pkv.ERR_INVALID_ARG
    q = pkv.KVPool(4, 2, 128, pkv.F16, host_only=True)
    with pytest.raises(pkv.PagedKVError) as e:
        q.set_fp8_scales([1.0, 1.0], [1.0, 1.0])
    assert e.value.code == pkv.ERR_STATE


def test_device_calls_validate_before_device_work():
    """paged_decode / kv_append on a host-only pool: argument errors first, then STATE."""
    L = pkv.lib()
    p = pkv.KVPool(8, 2, 128, pkv.F16, host_only=True)
    h = p.handle
    fake = ctypes.c_void_p(0x10000)     # never dereferenced: every call below is refused on the host
    dec = lambda **kw: L.paged_decode(h, kw.get("q", fake), kw.get("qdt", pkv.F16), kw.get("B", 2),
                                      kw.get("H", 8), kw.get("t", fake), kw.get("mb", 4), kw.get("l", fake),
                                      kw.get("ml", 64), kw.get("s", 0.125), kw.get("o", fake), kw.get("w", None),
                                      kw.get("wb", 0), None)
    assert dec(H=7) == pkv.ERR_INVALID_ARG            # not a multiple of kv_heads
    assert dec(B=-1) == pkv.ERR_INVALID_ARG
    assert dec(B=70000) == pkv.ERR_INVALID_ARG
    assert dec(mb=0) == pkv.ERR_INVALID_ARG
    assert dec(ml=-1) == pkv.ERR_INVALID_ARG
    assert dec(s=float("nan")) == pkv.ERR_INVALID_ARG
    assert dec(q=None) == pkv.ERR_INVALID_ARG
    assert dec(q=ctypes.c_void_p(0x10008)) == pkv.ERR_INVALID_ARG   # misaligned
    assert dec(qdt=pkv.BF16) == pkv.ERR_UNSUPPORTED   # q dtype must match an f16 pool
    assert dec(qdt=17) == pkv.ERR_INVALID_ARG
    p.set_partition(64)
    assert dec(ml=1000, mb=100) == pkv.ERR_INVALID_ARG   # workspace needed, none given
    assert p.workspace_bytes(2, 8, 1000) > 0
    p.set_partition(0)
    assert dec() == pkv.ERR_STATE                     # valid call, but no device memory
    ap = lambda **kw: L.kv_append(h, kw.get("s", fake), kw.get("T", 3), kw.get("k", fake), kw.get("v", fake),
                                  kw.get("dt", pkv.F16), None)
    assert ap(T=-1) == pkv.ERR_INVALID_ARG
    assert ap(dt=pkv.BF16) == pkv.ERR_UNSUPPORTED
    assert ap(k=None) == pkv.ERR_INVALID_ARG
    assert ap(v=ctypes.c_void_p(0x10004)) == pkv.ERR_INVALID_ARG
    assert ap() == pkv.ERR_STATE
    for bad in (1, 63, 100, 2**21):
        with pytest.raises(pkv.PagedKVError):
            p.set_partition(bad)
    p.close()


def test_probes_validate_before_device_work():
    """pkv_copy and pkv_read_probe refuse bad arguments on the host, before any
    launch (the pointers below are never dereferenced)."""
    L = pkv.lib()
    fake = ctypes.c_void_p(0x10000)
    odd = ctypes.c_void_p(0x10008)
    assert L.pkv_copy(None, fake, 64, None) == pkv.ERR_INVALID_ARG
    assert L.pkv_copy(fake, fake, 24, None) == pkv.ERR_INVALID_ARG          # not a multiple of 16
    assert L.pkv_copy(odd, fake, 64, None) == pkv.ERR_INVALID_ARG           # misaligned
    rp = lambda **kw: L.pkv_read_probe(kw.get("src", fake), kw.get("n", 1 << 20), kw.get("nt", 1),
                                       kw.get("order", None), kw.get("no", 0), kw.get("cb", 0),
                                       kw.get("sink", fake), None)
    assert rp(src=None) == pkv.ERR_INVALID_ARG
    assert rp(sink=None) == pkv.ERR_INVALID_ARG
    assert rp(n=24) == pkv.ERR_INVALID_ARG
    assert rp(src=odd) == pkv.ERR_INVALID_ARG
    assert rp(sink=ctypes.c_void_p(0x10002)) == pkv.ERR_INVALID_ARG
    assert rp(nt=2) == pkv.ERR_INVALID_ARG
    for cb in (0, -4096, 2048, 3 * 4096):                                      # not 4096 x 2^k
        assert rp(order=fake, no=4, cb=cb) == pkv.ERR_INVALID_ARG
    assert rp(order=fake, no=4, cb=1 << 21) == pkv.ERR_INVALID_ARG          # 1 MiB buffer, 2 MiB chunks
    assert rp(order=fake, no=-1, cb=4096) == pkv.ERR_INVALID_ARG
    assert rp(order=ctypes.c_void_p(0x10002), no=4, cb=4096) == pkv.ERR_INVALID_ARG


def test_decode_noalloc_validates_and_bounds_its_scratch():
    """paged_decode_noalloc: the same argument checks as paged_decode; sizes whose
    workspace exceeds the fixed scratch are refused with OUT_OF_RANGE before any
    device work; a host-only pool then gives STATE."""
    L = pkv.lib()
    p = pkv.KVPool(8, 8, 128, pkv.F16, host_only=True)
    h = p.handle
    fake = ctypes.c_void_p(0x10000)     # never dereferenced: every call below is refused on the host
    dec = lambda **kw: L.paged_decode_noalloc(h, kw.get("q", fake), pkv.F16, kw.get("B", 2), kw.get("H", 40),
                                              fake, kw.get("mb", 4096), fake, kw.get("ml", 64), 0.125, fake, None)
    assert dec(H=7) == pkv.ERR_INVALID_ARG
    assert dec(q=None) == pkv.ERR_INVALID_ARG
    assert dec() == pkv.ERR_STATE
    # the mixed-traffic shape (256 sequences up to 65536 tokens, 40 query heads) needs more than the scratch
    big = p.workspace_bytes(256, 40, 65536)
    assert big > pkv.NOALLOC_SCRATCH_BYTES
    assert dec(B=256, ml=65536) == pkv.ERR_OUT_OF_RANGE
    assert "scratch" in pkv.last_error()
    # a Llama-3-8B-shaped batch (64 sequences up to 8192 tokens, 32 query heads) fits
    q = pkv.KVPool(8, 8, 128, pkv.BF16, host_only=True)
    assert 0 < q.workspace_bytes(64, 32, 8192) <= pkv.NOALLOC_SCRATCH_BYTES
    p.close()
    q.close()


def test_partition_heuristic_is_multiple_of_64():
    p = pkv.KVPool(8, 8, 128, pkv.BF16, host_only=True)
    for B, Hq, ml in ((1, 32, 1), (64, 32, 8192), (256, 40, 65536), (16, 8, 100), (1, 8, 0)):
        P = p.partition_tokens(B, Hq, ml)
        assert P >= 64 and P % 64 == 0
        if ml <= P:
            assert p.workspace_bytes(B, Hq, ml) == 0
    p.close()


def test_batch_reserve_matches_single_reserves():
    """kv_batch_reserve == the model's reserves in order; all or nothing when the pool runs out."""
    import copy
    rng = np.random.default_rng(5)
    order = rng.permutation(40)
    a = pkv.KVPool(40, 2, 16, pkv.F16, free_order=order, host_only=True)
    m = BlockPoolModel(40, 16, free_order=order)
    seqs = [a.seq_create() for _ in range(5)]
    for _ in seqs:
        m.seq_create()
    # two forks at partial-block lengths, so batches exercise copy-on-write
    a.seq_reserve(seqs[0], 21)
    m.reserve(seqs[0], 21)
    for _ in range(2):
        seqs.append(a.seq_fork(seqs[0], 21))
        m.fork(seqs[0], 21)
    refused = 0
    for step in range(60):
        counts = rng.integers(0, 9, size=7)
        batch = [int(x) for x in rng.choice(seqs, size=7)]      # repeats allowed
        trial = copy.deepcopy(m)
        try:
            want = []
            for s, k in zip(batch, counts):
                want += trial.reserve(s, int(k))
        except AllocError as e:
            assert e.code == NO_BLOCKS_CODE
            with pytest.raises(pkv.PagedKVError) as got:
                a.batch_reserve(batch, counts)
            assert got.value.code == pkv.ERR_NO_BLOCKS
            refused += 1
        else:
            m = trial
            assert list(a.batch_reserve(batch, counts)) == want
        assert list(a.free_list()) == m.free_list()
        assert [a.seq_length(s) for s in seqs] == [m.length(s) for s in seqs]
        assert a.pending_copies() == m.pending
        if step % 10 == 9:                                       # release one to keep going
            s = seqs.pop(0)
            a.seq_free(s)
            m.free_seq(s)
            seqs.append(a.seq_create())
            m.seq_create()
    assert refused > 0
    a.close()


NO_BLOCKS_CODE = 2


def test_block_hash_matches_model():
    from oracle.allocator_model import block_key
    rng = np.random.default_rng(1)
    parent = 0
    for i in range(50):
        toks = rng.integers(-2**31, 2**31 - 1, size=16)
        ns = int(rng.integers(0, 2**63))
        k = pkv.kv_block_hash(parent, ns, toks)
        assert k == block_key(parent, ns, [int(t) for t in toks])
        parent = k


def test_prefill_validates_before_device_work():
    """paged_prefill on a host-only pool: argument errors first, then STATE."""
    L = pkv.lib()
    fake = ctypes.c_void_p(0x10000)
    p = pkv.KVPool(8, 2, 128, pkv.BF16, host_only=True)
    h = p.handle
    pre = lambda **kw: L.paged_prefill(h, kw.get("q", fake), kw.get("qdt", pkv.BF16), kw.get("S", 2), kw.get("H", 8),
                                       kw.get("qs", fake), kw.get("T", 10), kw.get("mq", 8), kw.get("t", fake),
                                       kw.get("mb", 4), kw.get("l", fake), kw.get("s", 0.1), kw.get("c", 1),
                                       kw.get("o", fake), None)
    assert pre(H=7) == pkv.ERR_INVALID_ARG
    assert pre(S=-1) == pkv.ERR_INVALID_ARG
    assert pre(T=-1) == pkv.ERR_INVALID_ARG
    assert pre(mb=0) == pkv.ERR_INVALID_ARG
    assert pre(s=float("inf")) == pkv.ERR_INVALID_ARG
    assert pre(qs=None) == pkv.ERR_INVALID_ARG
    assert pre(o=ctypes.c_void_p(0x10004)) == pkv.ERR_INVALID_ARG      # misaligned
    assert pre(qdt=pkv.F16) == pkv.ERR_UNSUPPORTED                    # q must match a bf16 pool
    assert pre() == pkv.ERR_STATE
    assert pre(T=0) == pkv.ERR_STATE and pre(S=0) == pkv.ERR_STATE    # as paged_decode: no device
    p.close()
    for dt, D in ((pkv.F32, 128), (pkv.BF16, 16)):                    # no prefill kernel for these
        q = pkv.KVPool(8, 2, D, dt, host_only=True)
        assert L.paged_prefill(q.handle, fake, dt, 1, 2, fake, 1, 1, fake, 1, fake, 0.1, 1, fake, None) \
            == pkv.ERR_UNSUPPORTED
        q.close()


def test_bench_traffic_summary_from_counter_csvs(tmp_path, monkeypatch):
    """bench.py --traffic-from: per-dispatch counter sums averaged per kernel,
    scaled by the copy kernel's reading of its known 2 GiB, summed over the
    decode call's kernels."""
    import csv
    import json
    import bench
    rows = {"FETCH_SIZE": [("pkv::pkv_copy_kernel(x)", 1, 1048576.0), ("pkv::pkv_copy_kernel(x)", 2, 1048576.0),
                           ("pkv::paged_decode_plan(p)", 3, 1.0),
                           ("void pkv::paged_decode_partition_gqa<2, 2, 4>(p)", 4, 500000.0),
                           ("void pkv::paged_decode_partition_gqa<2, 2, 4>(p)", 5, 600000.0),
                           ("void pkv::paged_decode_reduce<2, 128>(p)", 6, 2000.0)],
            "WRITE_SIZE": [("pkv::pkv_copy_kernel(x)", 1, 2097152.0), ("pkv::paged_decode_plan(p)", 3, 2.0),
                           ("void pkv::paged_decode_partition_gqa<2, 2, 4>(p)", 4, 4000.0),
                           ("void pkv::paged_decode_reduce<2, 128>(p)", 6, 500.0)]}
    dirs = []
    for counter, data in rows.items():
        d = tmp_path / counter
        d.mkdir()
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            wr = csv.writer(f)
            wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            for name, disp, val in data:
                wr.writerow([disp, name, counter, val / 2])          # two rows per dispatch, summed
                wr.writerow([disp, name, counter, val / 2])
        dirs.append(str(d))
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_hash", lambda kernel="x": "h")
    args = type("A", (), {"traffic_from": dirs, "workload": "gqa8b", "partition": 0})()
    bench.traffic_summary(args)
    t = json.load(open(prof / "traffic_paged_decode_partition_gqa8b.json"))
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    part = t["per_kernel"]["paged_decode_partition"]
    assert part["fetch_bytes"] == 550000 * 1024 * 2 and part["write_bytes"] == 4000 * 1024
    assert t["bytes_per_launch"] == part["fetch_bytes"] + part["write_bytes"]
    assert t["call_bytes"] == (1 + 550000 + 2000) * 2048 + (2 + 4000 + 500) * 1024
