"""Pure-Python model of the paged KV block pool -- TEST INFRASTRUCTURE.

Used only by the tests, to compare the native allocator bit for bit (block
tables, slot mappings, lengths, refcounts and the free list) after every
operation of random traces.  It shares no code with the library.

What the pages fix, and where:
  * K/V live in fixed-size physical blocks (16 tokens by default) in one pool;
    a per-sequence block table maps logical block i to a physical block, and
    physical placement is irrelevant ([cf1] www.cf-1.com/news/5824798, §3.1).
  * Blocks are taken from a global free list on demand, when the current
    block is full; only the last block of a sequence can be partly filled
    ([cf1] §3.2).  Pre-allocation makes an append a mere index move
    ([moo] www.mooersco.com/news/1484987, §2.2).
  * Several block tables may point at the same physical blocks (shared
    prefix, beam search, parallel sampling); a block is reclaimed when nobody
    references it ([cf1] §2.3, §3.3; [lqnn] m.lqnn.cn/news/219451, §3).

What the pages leave open, and the reading taken here:
  * Free-list order: a FIFO deque seeded from a caller-given order; allocation
    pops the front, release pushes to the back.  A freed sequence releases its
    blocks deepest first (reverse logical order), so that a cached prefix chain
    is evicted from its tail and its root stays findable longest.
  * A fork at any length n shares the first ceil(n / bs) blocks.  Writing into
    a shared, partly filled last block first takes a fresh block from the free
    list and records a block copy old -> fresh (copy-on-write, [cf1] §3.3); the
    old block loses one holder.  The copy block is taken before any new block.
  * Reserve is all-or-nothing: without enough free blocks nothing changes.
  * Slot of logical position p: table[p // bs] * bs + p % bs.
  * Swap ([cf1] §2.2 demand paging: blocks not in use may live in host memory
    and are brought back when needed): swap-out releases a sequence's blocks
    exactly as freeing it would (deepest first) but keeps the sequence, its
    length and its token contents (on the host); swap-in takes ceil(n / bs)
    fresh blocks, all or nothing, in logical order.  A swapped sequence
    cannot grow, fork, be registered or appear in a table until swapped in.
  * Prefix cache ([cf1] §3.3 content hash per block; [lqnn] §3 the cache
    identity includes the model/tenant namespace): full block i of a prompt
    has key_i = H(key_{i-1}, ns, its 16 tokens), key_{-1} = 0, with H the
    SplitMix64 output function folded over parent, namespace and tokens.  A
    block is shared only on an exact token match.  Cached blocks nobody holds
    stay findable in an LRU list; allocation takes the free list first, then
    evicts the least recently released cached block.
"""
from __future__ import annotations

from collections import deque

OK, INVALID_ARG, NO_BLOCKS, OUT_OF_RANGE, STATE = 0, 1, 2, 3, 4
INT32_MAX = 2**31 - 1
MASK64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """SplitMix64 (Steele, Lea, Flood; Vigna's reference): advance the state by
    the golden gamma and return the mixed output."""
    z = (x + 0x9E3779B97F4A7C15) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def block_key(parent: int, ns: int, tokens) -> int:
    h = splitmix64(parent ^ splitmix64(ns & MASK64))
    for t in tokens:
        h = splitmix64(h ^ (int(t) & 0xFFFFFFFF))
    return h


class AllocError(Exception):
    def __init__(self, code: int, msg: str = ""):
        super().__init__(msg or str(code))
        self.code = code


class BlockPoolModel:
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise AllocError(INVALID_ARG, "num_blocks and block_size must be > 0")
        order = list(range(num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError(INVALID_ARG, "free order must be a permutation of 0..N-1")
        self.N = num_blocks
        self.bs = block_size
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.seqs = {}          # id -> [blocks list, length]
        self.next_id = 0
        self.pending = []       # copy-on-write block copies (src, dst), oldest first
        self.cache = {}         # content key -> block
        self.key_of = {}        # cached block -> (key, tokens)
        self.lru = []           # cached blocks nobody holds, oldest release first
        self.swapped = set()    # sequences whose blocks live on the host

    def _take(self) -> int:
        if self.free:
            b = self.free.popleft()
        else:
            b = self.lru.pop(0)
            key, _ = self.key_of.pop(b)
            del self.cache[key]
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        if b in self.key_of:
            self.lru.append(b)
        else:
            self.free.append(b)

    def available(self) -> int:
        return len(self.free) + len(self.lru)

    # -- sequences -------------------------------------------------------
    def seq_create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = [[], 0]
        return sid

    def _get(self, sid, resident: bool = True):
        if sid not in self.seqs:
            raise AllocError(STATE, f"unknown or freed sequence {sid}")
        if resident and sid in self.swapped:
            raise AllocError(STATE, f"sequence {sid} is swapped out")
        return self.seqs[sid]

    # -- swap ----------------------------------------------------------------
    def swap_out(self, sid: int) -> int:
        """Release the blocks of sid (deepest first); returns how many it held."""
        blocks, _ = self._get(sid)
        n = len(blocks)
        for b in reversed(blocks):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self._release(b)
        self.seqs[sid][0] = []
        self.swapped.add(sid)
        return n

    def swap_in(self, sid: int):
        """Fresh blocks for every block of sid, all or nothing; returns the table."""
        if sid not in self.seqs or sid not in self.swapped:
            raise AllocError(STATE, f"sequence {sid} is not swapped out")
        length = self.seqs[sid][1]
        need = -(-length // self.bs)
        if need > self.available():
            raise AllocError(NO_BLOCKS, "not enough free blocks")
        self.seqs[sid][0] = [self._take() for _ in range(need)]
        self.swapped.discard(sid)
        return list(self.seqs[sid][0])

    def reserve(self, sid: int, n: int):
        """Append n token positions; return their slots."""
        s = self._get(sid)
        if n < 0:
            raise AllocError(INVALID_ARG, "n_tokens < 0")
        blocks, length = s
        new_len = length + n
        if new_len > INT32_MAX:
            raise AllocError(OUT_OF_RANGE, "sequence length overflow")
        cow = n > 0 and length % self.bs != 0 and self.ref[blocks[-1]] > 1
        need = -(-new_len // self.bs) - len(blocks)
        if need + cow > self.available():
            raise AllocError(NO_BLOCKS, "not enough free blocks")
        if cow:
            old, fresh = blocks[-1], self._take()
            self.ref[old] -= 1
            blocks[-1] = fresh
            self.pending.append((old, fresh))
        for _ in range(need):
            blocks.append(self._take())
        slots = [blocks[p // self.bs] * self.bs + p % self.bs for p in range(length, new_len)]
        s[1] = new_len
        return slots

    def fork(self, parent: int, n_shared: int) -> int:
        p = self._get(parent)
        if n_shared < 0 or n_shared > p[1]:
            raise AllocError(INVALID_ARG, "fork length must be in [0, parent length]")
        shared = p[0][: -(-n_shared // self.bs)]
        for b in shared:
            self.ref[b] += 1
        sid = self.seq_create()
        self.seqs[sid] = [list(shared), n_shared]
        return sid

    def free_seq(self, sid: int) -> None:
        blocks, _ = self._get(sid, resident=False)
        self.swapped.discard(sid)
        for b in reversed(blocks):
            self.ref[b] -= 1
            assert self.ref[b] >= 0
            if self.ref[b] == 0:
                self._release(b)
        del self.seqs[sid]

    # -- prefix cache ------------------------------------------------------
    def prefix_register(self, sid: int, tokens, ns: int = 0) -> int:
        blocks, length = self._get(sid)
        if len(tokens) > length:
            raise AllocError(OUT_OF_RANGE, "more tokens than the sequence holds")
        key, added = 0, 0
        for i in range(len(tokens) // self.bs):
            chunk = [int(t) for t in tokens[i * self.bs:(i + 1) * self.bs]]
            key = block_key(key, ns, chunk)
            b = blocks[i]
            if key in self.cache or b in self.key_of:
                continue
            self.cache[key] = b
            self.key_of[b] = (key, chunk)
            added += 1
        return added

    def seq_create_cached(self, tokens, ns: int = 0):
        key, hits = 0, []
        for i in range(len(tokens) // self.bs):
            chunk = [int(t) for t in tokens[i * self.bs:(i + 1) * self.bs]]
            key = block_key(key, ns, chunk)
            b = self.cache.get(key)
            if b is None or self.key_of[b][1] != chunk:
                break
            hits.append(b)
        sid = self.seq_create()
        for b in hits:
            if self.ref[b] == 0:
                self.lru.remove(b)
            self.ref[b] += 1
        self.seqs[sid] = [hits, len(hits) * self.bs]
        return sid, len(hits) * self.bs

    def prefix_evict_all(self) -> None:
        for b in self.lru:
            self.free.append(b)
        self.lru = []
        self.cache = {}
        self.key_of = {}

    # -- queries -----------------------------------------------------------
    def length(self, sid: int) -> int:
        return self._get(sid, resident=False)[1]

    def table(self, sid: int):
        return list(self._get(sid)[0])

    def tables(self, sids, max_blocks: int):
        rows, lens = [], []
        for sid in sids:
            blocks, length = self._get(sid)
            if len(blocks) > max_blocks:
                raise AllocError(OUT_OF_RANGE, "table wider than max_blocks_per_seq")
            rows.append(blocks + [-1] * (max_blocks - len(blocks)))
            lens.append(length)
        return rows, lens

    def refcount(self, block: int) -> int:
        if not 0 <= block < self.N:
            raise AllocError(INVALID_ARG, "block out of range")
        return self.ref[block]

    def free_list(self):
        return list(self.free)

    def take_copies(self):
        """The owed copy-on-write copies, clearing the list (as a device call does)."""
        out, self.pending = self.pending, []
        return out

    def shared_blocks(self) -> int:
        return sum(1 for r in self.ref if r > 1)

    # -- invariants ([cf1] §3.2, §3.3) ----------------------------------------
    def check_invariants(self) -> None:
        holders = [0] * self.N
        for sid, (blocks, length) in self.seqs.items():
            if sid in self.swapped:
                assert blocks == [], "a swapped sequence holds blocks"
                continue
            assert len(blocks) == -(-length // self.bs), "blocks != ceil(len / bs)"
            for b in blocks:
                holders[b] += 1
        free_set, lru_set = set(self.free), set(self.lru)
        assert len(free_set) == len(self.free), "a block is in the free list twice"
        assert len(lru_set) == len(self.lru) and not (free_set & lru_set)
        for b in range(self.N):
            if b in free_set or b in lru_set:
                assert self.ref[b] == 0 and holders[b] == 0
            else:
                assert self.ref[b] == holders[b] and self.ref[b] > 0, f"refcount mismatch on {b}"
        assert all(b in self.key_of for b in self.lru) and not any(b in self.key_of for b in self.free)
        assert all(self.cache[k] == b for b, (k, _) in self.key_of.items()) and len(self.cache) == len(self.key_of)
        assert len(self.free) + len(self.lru) + sum(1 for r in self.ref if r > 0) == self.N
