"""INT8 per-block min-max KV codes: the oracle's model -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use this module.  The product never imports it, and it
imports nothing of the product.

What the page fixes ([moo] www.mooersco.com/news/1484987 §3.3, quantisation
strategies, the INT8 KV-cache item): the keys (and values) of a block are
stored as codes

    q = round((k - k_min) / (k_max - k_min) * 255)

with two parameters, k_min and k_max, kept per block.

Readings where the page is silent (each is also listed in the design notes):
  R1  One (k_min, k_max) per (block, KV head) tile, separately for K and V:
      the tile is the unit the pool stores per head.
  R2  Every step in IEEE fp32, in the formula's order: d = x - k_min,
      t = d / (k_max - k_min), code = round-half-even(t * 255), clamped to
      [0, 255].  k_max == k_min gives code 0; a NaN gives code 0.
  R3  A code stands for k_min + code * (k_max - k_min) / 255 (the inverse of
      the formula); attention uses that value, in fp64.
  R4  A block fills a call at a time.  Its range is the min and max of every
      value written into the tile since its row 0 was last written: a call
      that writes row 0 starts the tile afresh (its other rows no longer
      count); any other call widens the range to take its values and, if the
      range moved, re-encodes every other row of the tile.  A re-encoded
      row's fp32 value is k_min + code * step with step = (k_max - k_min) / 255
      (product and sum rounded separately), quantised again under the new
      range (R2).  All rows one call writes into one tile are taken together.
      An unwritten tile reads as codes 0 and range (0, 0), like a
      zero-filled pool.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
BLOCK = 16


def encode(x, k_min, k_max) -> np.ndarray:
    """Codes of fp32 values under the range (k_min, k_max) (R2)."""
    x = np.asarray(x, dtype=np.float32)
    lo, hi = F32(k_min), F32(k_max)
    if not hi > lo:
        return np.zeros(x.shape, dtype=np.uint8)
    with np.errstate(invalid="ignore", over="ignore"):
        d = x - lo                              # fp32
        t = d / (hi - lo)                       # fp32, correctly rounded division
        c = np.rint(t * F32(255))               # fp32 product, round half to even
    c = np.where(np.isnan(c), F32(0), np.clip(c, F32(0), F32(255)))
    return c.astype(np.uint8)


def step(k_min, k_max) -> np.float32:
    """(k_max - k_min) / 255 in fp32."""
    return F32(F32(k_max) - F32(k_min)) / F32(255)


def value_f32(codes, k_min, k_max) -> np.ndarray:
    """fp32 value of codes, as a re-encode reads it (R4): k_min + code * step."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float32)
    return F32(k_min) + c * step(k_min, k_max)


def value(codes, k_min, k_max) -> np.ndarray:
    """The value a code stands for (R3), in fp64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    lo, hi = float(F32(k_min)), float(F32(k_max))
    # = lo + c (hi - lo) / 255; both products are exact in fp64, so codes 0 and
    # 255 give k_min and k_max exactly
    return (lo * (255.0 - c) + hi * c) / 255.0


class TileStore:
    """The INT8 pool as appends leave it: per (tensor, block, KV head) a tile of
    16 rows of head_dim codes and its range (R1, R4).  Keys are physical
    block ids, so the model follows the same slots as the library."""

    def __init__(self, H_kv: int, D: int):
        self.H_kv, self.D = H_kv, D
        self.codes: dict = {}
        self.range: dict = {}

    def tile(self, kind: str, block: int, head: int):
        key = (kind, block, head)
        codes = self.codes.get(key)
        if codes is None:
            codes = np.zeros((BLOCK, self.D), dtype=np.uint8)
        return codes, self.range.get(key, (F32(0), F32(0)))

    def append(self, slots, K, V) -> None:
        """One append call: token t goes to slot slots[t] (block slot // 16, row
        slot % 16); K and V are [T][H_kv][D] fp32 values.  Negative slots are
        skipped.  Slots must be distinct."""
        K = np.asarray(K, dtype=np.float32)
        V = np.asarray(V, dtype=np.float32)
        rows_of: dict = {}
        for t, s in enumerate(np.asarray(slots).tolist()):
            if s < 0:
                continue
            rows = rows_of.setdefault(s // BLOCK, {})
            assert s % BLOCK not in rows, "duplicate slot in one call"
            rows[s % BLOCK] = t
        for block, rows in rows_of.items():
            for g in range(self.H_kv):
                self._write("k", block, g, {r: K[t, g] for r, t in rows.items()})
                self._write("v", block, g, {r: V[t, g] for r, t in rows.items()})

    def _write(self, kind: str, block: int, head: int, new: dict) -> None:
        codes, (old_lo, old_hi) = self.tile(kind, block, head)
        codes = codes.copy()
        vals = np.stack(list(new.values()))
        lo, hi = F32(np.min(vals)), F32(np.max(vals))
        if 0 not in new:                        # the tile continues: widen, re-encode the rest
            lo, hi = min(old_lo, lo), max(old_hi, hi)
            if (lo, hi) != (old_lo, old_hi):
                rest = [r for r in range(BLOCK) if r not in new]
                codes[rest] = encode(value_f32(codes[rest], old_lo, old_hi), lo, hi)
        for r, x in new.items():
            codes[r] = encode(x, lo, hi)
        self.codes[(kind, block, head)] = codes
        self.range[(kind, block, head)] = (F32(lo), F32(hi))

    def copy_block(self, src: int, dst: int) -> None:
        """A whole-block copy (copy-on-write, swap): codes and ranges move alike."""
        for kind in ("k", "v"):
            for g in range(self.H_kv):
                codes, rng = self.tile(kind, src, g)
                self.codes[(kind, dst, g)] = codes.copy()
                self.range[(kind, dst, g)] = rng

    def values(self, kind: str, blocks, n: int) -> np.ndarray:
        """fp64 values [n][H_kv][D] of the first n tokens of a sequence whose
        block table starts with `blocks` (R3)."""
        out = np.empty((n, self.H_kv, self.D), dtype=np.float64)
        for j in range(n):
            b, r = blocks[j // BLOCK], j % BLOCK
            for g in range(self.H_kv):
                codes, (lo, hi) = self.tile(kind, b, g)
                out[j, g] = value(codes[r], lo, hi)
        return out
