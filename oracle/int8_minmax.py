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
    """Codes of fp32 values under the range (k_min, k_max) (R2); k_min and
    k_max may be arrays that broadcast against x."""
    x = np.asarray(x, dtype=np.float32)
    lo, hi = np.asarray(k_min, dtype=np.float32), np.asarray(k_max, dtype=np.float32)
    ok = hi > lo
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        d = x - lo                                              # fp32
        t = d / np.where(ok, hi - lo, np.float32(1))            # fp32, correctly rounded division
        c = np.rint(t * F32(255))                               # fp32 product, round half to even
    c = np.where(np.isnan(c), F32(0), np.clip(c, F32(0), F32(255)))
    return np.where(ok, c, F32(0)).astype(np.uint8)


def step(k_min, k_max):
    """(k_max - k_min) / 255 in fp32."""
    return (np.asarray(k_max, dtype=np.float32) - np.asarray(k_min, dtype=np.float32)) / F32(255)


def value_f32(codes, k_min, k_max) -> np.ndarray:
    """fp32 value of codes, as a re-encode reads it (R4): k_min + code * step."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float32)
    return np.asarray(k_min, dtype=np.float32) + c * step(k_min, k_max)


def value(codes, k_min, k_max) -> np.ndarray:
    """The value a code stands for (R3), in fp64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    lo = np.asarray(k_min, dtype=np.float32).astype(np.float64)
    hi = np.asarray(k_max, dtype=np.float32).astype(np.float64)
    # = lo + c (hi - lo) / 255; both products are exact in fp64, so codes 0 and
    # 255 give k_min and k_max exactly
    return (lo * (255.0 - c) + hi * c) / 255.0


class TileStore:
    """The INT8 pool as appends leave it: per (tensor, block) the tiles of all
    KV heads -- codes [H_kv][16][D] and ranges lo, hi [H_kv] (R1, R4).  Keys
    are physical block ids, so the model follows the same slots as the
    library.  Each head's tile is handled on its own; the heads of one block
    are only evaluated together."""

    def __init__(self, H_kv: int, D: int):
        self.H_kv, self.D = H_kv, D
        self.blocks: dict = {}

    def _block(self, kind: str, block: int):
        b = self.blocks.get((kind, block))
        if b is None:
            b = (np.zeros((self.H_kv, BLOCK, self.D), dtype=np.uint8),
                 np.zeros(self.H_kv, dtype=np.float32), np.zeros(self.H_kv, dtype=np.float32))
        return b

    def tile(self, kind: str, block: int, head: int):
        codes, lo, hi = self._block(kind, block)
        return codes[head], (lo[head], hi[head])

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
            r = np.array(sorted(rows))
            t = np.array([rows[i] for i in r.tolist()])
            self._write("k", block, r, K[t].transpose(1, 0, 2))
            self._write("v", block, r, V[t].transpose(1, 0, 2))

    def _write(self, kind: str, block: int, rows: np.ndarray, new: np.ndarray) -> None:
        """Rows `rows` of every head's tile get new[h] ([H_kv][len(rows)][D])."""
        codes, old_lo, old_hi = (a.copy() for a in self._block(kind, block))
        lo, hi = new.min(axis=(1, 2)), new.max(axis=(1, 2))
        if 0 not in rows:                       # the tile continues: widen, re-encode the rest
            lo, hi = np.minimum(old_lo, lo), np.maximum(old_hi, hi)
            rest = np.setdiff1d(np.arange(BLOCK), rows)
            for h in np.flatnonzero((lo != old_lo) | (hi != old_hi)):
                codes[h, rest] = encode(value_f32(codes[h, rest], old_lo[h], old_hi[h]), lo[h], hi[h])
        codes[:, rows] = encode(new, lo[:, None, None], hi[:, None, None])
        self.blocks[(kind, block)] = (codes, lo.astype(np.float32), hi.astype(np.float32))

    def copy_block(self, src: int, dst: int) -> None:
        """A whole-block copy (copy-on-write, swap): codes and ranges move alike."""
        for kind in ("k", "v"):
            self.blocks[(kind, dst)] = tuple(a.copy() for a in self._block(kind, src))

    def rename(self, pairs) -> None:
        """Blocks that moved to new ids all at once (a swap-out and swap-in):
        for each (old, new) the tiles held at `old` before the call are held
        at `new` afterwards.  A new id may be another pair's old id."""
        snap = {(kind, a): tuple(x.copy() for x in self._block(kind, a)) for a, _ in pairs for kind in ("k", "v")}
        for a, b in pairs:
            for kind in ("k", "v"):
                self.blocks[(kind, b)] = snap[(kind, a)]

    def values(self, kind: str, blocks, n: int) -> np.ndarray:
        """fp64 values [n][H_kv][D] of the first n tokens of a sequence whose
        block table starts with `blocks` (R3)."""
        out = np.empty((n, self.H_kv, self.D), dtype=np.float64)
        for j in range(-(-n // BLOCK)):
            codes, lo, hi = self._block(kind, int(blocks[j]))
            rows = min(BLOCK, n - BLOCK * j)
            out[BLOCK * j:BLOCK * j + rows] = value(codes[:, :rows], lo[:, None, None], hi[:, None, None]).transpose(1, 0, 2)
        return out


def one_shot_values(x) -> np.ndarray:
    """The page's formula applied once per (16-row tile, KV head) over the rows
    the tile finally holds -- the plain definition, independent of how appends
    filled the tile.

    x: [n][H_kv][D] values of one sequence in logical order (any float type).
    Tile j holds rows 16j .. min(16j + 16, n) - 1.  For each tile and head, in
    fp64: k_min, k_max over the tile's rows and dims, q = round-half-even(
    (x - k_min) / (k_max - k_min) * 255), and the value a code stands for,
    k_min + q * (k_max - k_min) / 255, evaluated as (k_min * (255 - q) +
    k_max * q) / 255 so that codes 0 and 255 give k_min and k_max exactly for
    fp32-representable inputs.  A constant tile (k_max == k_min) stands for
    its constant.  Returns fp64 [n][H_kv][D]."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    out = np.empty_like(x)
    for j0 in range(0, n, BLOCK):
        tile = x[j0:j0 + BLOCK]                                # [rows][H][D]
        k_min = tile.min(axis=(0, 2))[None, :, None]
        k_max = tile.max(axis=(0, 2))[None, :, None]
        span = k_max - k_min
        flat = span == 0
        q = np.rint((tile - k_min) / np.where(flat, 1.0, span) * 255.0)
        out[j0:j0 + BLOCK] = np.where(flat, tile, (k_min * (255.0 - q) + k_max * q) / 255.0)
    return out
