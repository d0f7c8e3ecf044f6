"""Seeded synthetic inputs for paged decode attention.

This module holds random numbers, shapes and length mixes only -- none of the
attention arithmetic.  Both the HIP library's harness and the CPU oracle read
their inputs from here; nothing here imports either of them.

Five workloads, each one decode step of one layer (block size 16):
  tiny       1 seq, 4 q / 4 kv heads, d 16, fp32, 64-block pool; prefill 24
             tokens then 8 decode steps with an append each (context 25..32)
  mha7b      Llama-2-7B-shaped MHA: 32/32 heads, d 128, fp16, batch 16,
             every context 4096, pool of exactly 4096 blocks
  gqa8b      Llama-3-8B-shaped GQA: 32 q / 8 kv heads, d 128, bf16, batch 64,
             context ~ U[128, 8192]
  mixed      40 q / 8 kv heads, d 128, fp16, batch 256: 230 short contexts
             U[256, 2048], 26 long U[16384, 65536]; 16 short sequences share a
             2048-token prefix (128 blocks, refcount 16) and add U[256, 2048]
  fp8        FP8-E4M3 KV, 32 q / 8 kv heads, d 128, batch 32, every context
             32768; K, V ~ N(0,1) with 0.1% elements x20, cast to bf16;
             per-kv-head scales absmax / 448; q bf16

Value recipe: float32 N(0,1) from torch's CPU generator (Mersenne Twister,
reproducible for a seed whatever the thread count), cast with round-to-
nearest-even to the stored dtype.  Each sequence draws from its own generator,
seeded from a numpy SeedSequence child, so any subset of sequences can be
generated alone, and several at once on a thread pool.  Pools hold 1.25x
the blocks the batch needs (tiny: 64, mha7b: exactly the need), and the free
list starts as a seeded permutation, which scatters the physical blocks.
These stand in for the Llama-2-7B / Llama-3-8B / long-tail traffic shapes the
pages discuss; no model weights or traces are used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F32, F16, BF16, E4M3, INT8 = 0, 1, 2, 3, 4
BLOCK = 16
_NP = {F32: np.float32, F16: np.float16, BF16: np.uint16, E4M3: np.uint8, INT8: np.uint8}
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2, E4M3: 1, INT8: 1}
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16", E4M3: "fp8_e4m3", INT8: "int8_minmax"}


def storage_to_f32(x: np.ndarray, dtype: int) -> np.ndarray:
    """Exact float32 values of f32 / f16 / bf16 (uint16 bits) storage."""
    if dtype == BF16:
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=_NP[dtype]).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    return cast_to_storage(x, BF16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def cast_to_storage(x, dtype: int) -> np.ndarray:
    """float32 values (numpy or torch CPU) -> stored dtype, round to nearest even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)) if isinstance(x, np.ndarray) else x
    if dtype == F32:
        return t.to(torch.float32).numpy()
    if dtype == F16:
        return t.to(torch.float16).numpy()
    if dtype == BF16:
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError("no direct cast to this storage dtype")


def _torch_gen(ss: np.random.SeedSequence):
    import torch
    return torch.Generator().manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] >> 1))


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    H_q: int
    H_kv: int
    D: int
    kv_dtype: int            # pool storage dtype
    q_dtype: int             # q / out / appended k,v dtype
    lens: np.ndarray         # int32 [B], final context length (includes the new token)
    num_blocks: int
    free_order: np.ndarray   # int32 permutation of 0..num_blocks-1
    prefill: np.ndarray      # int32 [B], tokens present before the decode steps
    decode_steps: int = 1
    sharers: list = field(default_factory=list)   # sequence indices sharing the prefix
    prefix_tokens: int = 0
    outlier_p: float = 0.0
    outlier_mult: float = 1.0
    cache_kv: bool = False   # keep generated K/V in host memory (FP8: scales need a full pass)
    _scales: tuple | None = None
    _kv_cache: dict = field(default_factory=dict)

    # ------------------------------------------------------------------
    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), rounded to float32."""
        return float(np.float32(1.0 / math.sqrt(self.D)))

    @property
    def src_dtype(self) -> int:
        """dtype of the K/V handed to kv_append (bf16 for an FP8 or INT8 pool)."""
        return BF16 if self.kv_dtype in (E4M3, INT8) else self.kv_dtype

    def step_lens(self) -> np.ndarray:
        """Context lengths during the first decode step (prefill + the new token)."""
        return np.minimum(self.lens, self.prefill + 1).astype(np.int32)

    def kv_bytes(self, lens) -> int:
        """Algorithmic K+V bytes of attending once over contexts `lens`: every live
        element once, plus for INT8 pools each touched tile's 16-byte header."""
        lens = np.asarray(lens).astype(np.int64)
        n = int(lens.sum()) * self.H_kv * self.D * 2 * ELEM_BYTES[self.kv_dtype]
        if self.kv_dtype == INT8:
            n += int(((lens + BLOCK - 1) // BLOCK).sum()) * self.H_kv * 2 * 16
        return n

    def kv_bytes_per_step(self) -> int:
        """Algorithmic K+V bytes the first decode step reads."""
        return self.kv_bytes(self.step_lens())

    def max_len(self) -> int:
        return int(self.lens.max()) if self.B else 0

    def max_blocks_per_seq(self) -> int:
        return -(-self.max_len() // BLOCK)

    # ------------------------------------------------------------------
    def _children(self):
        # children 0..B-1: sequences; B: prefix; B+1: queries; B+2..: decode-step queries
        return np.random.SeedSequence(self.seed).spawn(self.B + 2 + self.decode_steps)

    def _normal(self, ss, n: int):
        """n float32 N(0,1) draws (torch CPU tensor); outliers x mult with prob outlier_p."""
        import torch
        g = _torch_gen(ss)
        x = torch.randn(n, generator=g, dtype=torch.float32)
        if self.outlier_p > 0:
            hit = torch.rand(n, generator=g, dtype=torch.float32) < self.outlier_p
            x[hit] *= self.outlier_mult
        return x

    def own_tokens(self, b: int) -> int:
        """Tokens of sequence b not covered by the shared prefix."""
        return int(self.lens[b]) - (self.prefix_tokens if b in self.sharers else 0)

    def kv(self, b: int):
        """Logical (de-paged) K_b, V_b: [n_b][H_kv][D] in src_dtype storage."""
        if b in self._kv_cache:
            return self._kv_cache[b]
        kv = self._kv(b)
        if self.cache_kv:
            self._kv_cache[b] = kv
        return kv

    def _kv(self, b: int):
        kids = self._children()
        n_own = self.own_tokens(b)
        per = self.H_kv * self.D
        x = self._normal(kids[b], 2 * n_own * per)
        K = x[: n_own * per].reshape(n_own, self.H_kv, self.D)
        V = x[n_own * per:].reshape(n_own, self.H_kv, self.D)
        if b in self.sharers:
            import torch
            pK, pV = self.prefix_kv_f32(kids)
            K = torch.cat([pK, K])
            V = torch.cat([pV, V])
        return cast_to_storage(K, self.src_dtype), cast_to_storage(V, self.src_dtype)

    def kv_many(self, seqs, workers: int = 8):
        """Yield (b, K_b, V_b) in the order of `seqs`, generating ahead on a thread pool."""
        import concurrent.futures as cf
        seqs = list(seqs)
        with cf.ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
            futs = {}
            ahead = max(1, workers)
            for i, b in enumerate(seqs[:ahead]):
                futs[i] = ex.submit(self.kv, b)
            for i, b in enumerate(seqs):
                K, V = futs.pop(i).result()
                if i + ahead < len(seqs):
                    futs[i + ahead] = ex.submit(self.kv, seqs[i + ahead])
                yield b, K, V

    def prefix_kv_f32(self, kids=None):
        kids = kids if kids is not None else self._children()
        per = self.H_kv * self.D
        p = self.prefix_tokens
        x = self._normal(kids[self.B], 2 * p * per)
        return x[: p * per].reshape(p, self.H_kv, self.D), x[p * per:].reshape(p, self.H_kv, self.D)

    def q(self, step: int = 0) -> np.ndarray:
        """Queries of decode step `step`: [B][H_q][D] in q_dtype storage."""
        import torch
        kids = self._children()
        x = torch.randn(self.B * self.H_q * self.D, generator=_torch_gen(kids[self.B + 1 + step]),
                        dtype=torch.float32)
        return cast_to_storage(x.reshape(self.B, self.H_q, self.D), self.q_dtype)

    def fp8_scales(self):
        """Per-kv-head static scales absmax/448 over all generated K (resp. V)."""
        if self.kv_dtype != E4M3:
            return None
        if self._scales is None:
            kmax = np.zeros(self.H_kv, np.float32)
            vmax = np.zeros(self.H_kv, np.float32)
            import torch
            amax = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).abs().amax(dim=(0, 2)) \
                .to(torch.float32).numpy()
            for b, K, V in self.kv_many(range(self.B)):
                kmax = np.maximum(kmax, amax(K))
                vmax = np.maximum(vmax, amax(V))
            self._scales = ((kmax / np.float32(448.0)).astype(np.float32),
                            (vmax / np.float32(448.0)).astype(np.float32))
        return self._scales

    def build_plan(self):
        """How the batch is laid into the pool, in order.

        ("new", b, n)          create sequence b and reserve its first n tokens
        ("fork", b, owner, p)  sequence b shares the first p tokens of `owner`
        ("grow", b, n)         reserve n more tokens for sequence b
        Sequences are built in index order; the first sharer owns the prefix.
        The final decode token of every sequence is a separate ("grow", b, 1)
        per decode step, issued for all b after the prefill.
        """
        plan = []
        owner = min(self.sharers) if self.sharers else None
        for b in range(self.B):
            n_pre = int(self.prefill[b])
            if b in self.sharers and b != owner:
                plan.append(("fork", b, owner, self.prefix_tokens))
                plan.append(("grow", b, n_pre - self.prefix_tokens))
            else:
                plan.append(("new", b, n_pre))
        return plan


def _pool_blocks(lens, sharers, prefix_tokens, slack: float) -> int:
    need = int(sum(-(-int(n) // BLOCK) for n in lens))
    if sharers:
        need -= (len(sharers) - 1) * (prefix_tokens // BLOCK)
    return int(math.ceil(need * slack))


def make(name: str) -> Workload:
    """One of: tiny, mha7b, gqa8b, mixed, fp8."""
    if name == "tiny":
        seed, B, Hq, Hkv, D, kvd, qd = 1, 1, 4, 4, 16, F32, F32
        lens = np.array([32], np.int32)
        nb = 64
        steps = 8
        pre = lens - steps
    elif name == "mha7b":
        seed, B, Hq, Hkv, D, kvd, qd = 2, 16, 32, 32, 128, F16, F16
        lens = np.full(B, 4096, np.int32)
        nb = _pool_blocks(lens, [], 0, 1.0)
        steps, pre = 1, lens - 1
    elif name == "gqa8b":
        seed, B, Hq, Hkv, D, kvd, qd = 3, 64, 32, 8, 128, BF16, BF16
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed + 2000)))
        lens = rng.integers(128, 8192, size=B, endpoint=True).astype(np.int32)
        nb = _pool_blocks(lens, [], 0, 1.25)
        steps, pre = 1, lens - 1
    elif name == "mixed":
        seed, B, Hq, Hkv, D, kvd, qd = 4, 256, 40, 8, 128, F16, F16
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed + 2000)))
        n_long = round(0.1 * B)
        perm = rng.permutation(B)
        long_idx, short_idx = perm[:n_long], perm[n_long:]
        lens = np.zeros(B, np.int32)
        lens[long_idx] = rng.integers(16384, 65536, size=n_long, endpoint=True)
        lens[short_idx] = rng.integers(256, 2048, size=B - n_long, endpoint=True)
        sharers = sorted(int(i) for i in short_idx)[:16]
        for b in sharers:
            lens[b] = 2048 + int(rng.integers(256, 2048, endpoint=True))
        nb = _pool_blocks(lens, sharers, 2048, 1.25)
        steps, pre = 1, lens - 1
        w = Workload(name, seed, B, Hq, Hkv, D, kvd, qd, lens, nb, None, pre, steps,
                     sharers=sharers, prefix_tokens=2048)
        w.free_order = _free_order(seed, nb)
        return w
    elif name == "int8":
        # the fp8 workload's shape and values (same seed), stored as INT8 min-max codes
        seed, B, Hq, Hkv, D, kvd, qd = 5, 32, 32, 8, 128, INT8, BF16
        lens = np.full(B, 32768, np.int32)
        nb = _pool_blocks(lens, [], 0, 1.25)
        steps, pre = 1, lens - 1
        w = Workload(name, seed, B, Hq, Hkv, D, kvd, qd, lens, nb, None, pre, steps,
                     outlier_p=0.001, outlier_mult=20.0)
        w.free_order = _free_order(seed, nb)
        return w
    elif name == "fp8":
        seed, B, Hq, Hkv, D, kvd, qd = 5, 32, 32, 8, 128, E4M3, BF16
        lens = np.full(B, 32768, np.int32)
        nb = _pool_blocks(lens, [], 0, 1.25)
        steps, pre = 1, lens - 1
        w = Workload(name, seed, B, Hq, Hkv, D, kvd, qd, lens, nb, None, pre, steps,
                     outlier_p=0.001, outlier_mult=20.0, cache_kv=True)
        w.free_order = _free_order(seed, nb)
        return w
    else:
        raise KeyError(name)
    w = Workload(name, seed, B, Hq, Hkv, D, kvd, qd, lens, nb, None, pre.astype(np.int32), steps)
    w.free_order = _free_order(seed, nb)
    return w


def _free_order(seed: int, nb: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed + 1000)))
    return rng.permutation(nb).astype(np.int32)


def custom(seed: int, lens, H_q: int, H_kv: int, D: int, kv_dtype: int, q_dtype: int | None = None,
           num_blocks: int | None = None, outlier_p: float = 0.0) -> Workload:
    """A small workload of the same recipe with arbitrary shapes (parity sweeps)."""
    lens = np.asarray(lens, dtype=np.int32)
    if q_dtype is None:
        q_dtype = BF16 if kv_dtype in (E4M3, INT8) else kv_dtype
    nb = num_blocks if num_blocks is not None else max(1, _pool_blocks(np.maximum(lens, 1), [], 0, 1.25) + 2)
    w = Workload(f"custom{seed}", seed, len(lens), H_q, H_kv, D, kv_dtype, q_dtype, lens, nb,
                 _free_order(seed, nb), np.maximum(lens - 1, 0).astype(np.int32), 1,
                 outlier_p=outlier_p, outlier_mult=20.0)
    return w


def mini_model_inputs(seed: int, n_tokens: int, d_model: int = 64):
    """Embeddings x_t ~ N(0,1)^d_model and projections W ~ 0.1 * N(0,1), float64.

    The shape of the NumPy walk-through on [mlqm] www.mlqm.cn/news/394450,
    section 四 (d_model 64, 4 heads of 16).
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    x = rng.standard_normal((n_tokens, d_model))
    Wq = rng.standard_normal((d_model, d_model)) * 0.1
    Wk = rng.standard_normal((d_model, d_model)) * 0.1
    Wv = rng.standard_normal((d_model, d_model)) * 0.1
    return x, Wq, Wk, Wv


# ---------------------------------------------------------------------------
# Multi-query (chunked prefill) workload
# ---------------------------------------------------------------------------
@dataclass
class PrefillWorkload:
    """B sequences, each with `cached` tokens already in the cache and a chunk of
    `chunk` new tokens (their K/V appended, then attended causally).  Values
    N(0,1) per sequence from child seeds of `seed`; queries from child B."""
    name: str
    seed: int
    B: int
    H_q: int
    H_kv: int
    D: int
    kv_dtype: int
    cached: int
    chunk: int
    causal: bool = True

    @property
    def n(self) -> int:
        return self.cached + self.chunk

    @property
    def src_dtype(self) -> int:
        """Storage of the generated K/V and of q: bf16 for an FP8 pool (the codes
        are made by kv_append), else the pool's own type."""
        return BF16 if self.kv_dtype == E4M3 else self.kv_dtype

    def fp8_scales(self):
        """Per-kv-head static scales absmax/448 over all generated K (resp. V);
        None unless the pool is FP8."""
        if self.kv_dtype != E4M3:
            return None
        kmax = np.zeros(self.H_kv, np.float32)
        vmax = np.zeros(self.H_kv, np.float32)
        for b in range(self.B):
            K, V = self.kv(b)
            kmax = np.maximum(kmax, np.abs(bf16_bits_to_f32(K)).max(axis=(0, 2)))
            vmax = np.maximum(vmax, np.abs(bf16_bits_to_f32(V)).max(axis=(0, 2)))
        return (kmax / np.float32(448.0)).astype(np.float32), (vmax / np.float32(448.0)).astype(np.float32)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.D)))

    @property
    def num_blocks(self) -> int:
        return self.B * -(-self.n // BLOCK)

    def _children(self):
        return np.random.SeedSequence(self.seed).spawn(self.B + 1)

    def kv(self, b: int):
        """K_b, V_b: [n][H_kv][D] in the source storage dtype (bf16 bits, f16)."""
        import torch
        g = _torch_gen(self._children()[b])
        per = self.n * self.H_kv * self.D
        x = torch.randn(2 * per, generator=g, dtype=torch.float32)
        K = x[:per].reshape(self.n, self.H_kv, self.D)
        V = x[per:].reshape(self.n, self.H_kv, self.D)
        return cast_to_storage(K, self.src_dtype), cast_to_storage(V, self.src_dtype)

    def q(self) -> np.ndarray:
        """[B * chunk][H_q][D], sequence b owning rows b*chunk .. (b+1)*chunk - 1."""
        import torch
        x = torch.randn(self.B * self.chunk * self.H_q * self.D, generator=_torch_gen(self._children()[self.B]),
                        dtype=torch.float32)
        return cast_to_storage(x.reshape(self.B * self.chunk, self.H_q, self.D), self.src_dtype)

    def flops(self) -> int:
        """Algorithmic flops of one launch: 2 D for q.k and 2 D for p.v per (query
        row, visible position); causal: row i of a chunk sees cached + i + 1."""
        if self.causal:
            visible = self.chunk * self.cached + self.chunk * (self.chunk + 1) // 2
        else:
            visible = self.chunk * self.n
        return self.B * self.H_q * visible * 4 * self.D

    def kv_bytes(self) -> int:
        """K+V bytes of the contexts (each read at least once)."""
        return self.B * self.n * self.H_kv * self.D * 2 * ELEM_BYTES[self.kv_dtype]


def make_prefill(name: str) -> PrefillWorkload:
    """prefill8b: Llama-3-8B heads (32 q / 8 kv, d 128), bf16, 16 sequences of
    2048 cached tokens plus a 512-token chunk, causal.  prefill8b_fp8: the same
    values appended into an FP8-E4M3 pool (per-head scales absmax / 448), q bf16."""
    if name == "prefill8b":
        return PrefillWorkload(name, 6, 16, 32, 8, 128, BF16, 2048, 512)
    if name == "prefill8b_fp8":
        return PrefillWorkload(name, 6, 16, 32, 8, 128, E4M3, 2048, 512)
    raise ValueError(f"unknown prefill workload {name!r}")
