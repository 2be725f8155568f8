"""Block-pool allocator replica (oracle; test infrastructure only).

What the pages fix: blocks of a fixed number of tokens come from one shared
pool as tokens arrive («¿Cómo gestiona Paged Attention la caché KV…?» "PagedAttention divide el estado KV en bloques
de tamaño fijo"); each sequence keeps a block table mapping logical order to
physical blocks («¿Cómo gestiona Paged Attention la caché KV…?»; «PagedAttention e vLLM» "Approfondimento tecnico"; «Paged Attention optimiza el uso de memoria»); the
runtime keeps reference counts («¿Cómo gestiona Paged Attention la caché KV…?» "La gestión de bloques…"); finished
requests return their unshared blocks to the pool at once («¿Cómo gestiona Paged Attention la caché KV…?» "Los
bloques liberados…", «Paged Attention optimiza el uso de memoria»); identical prefixes point at the same blocks
and a writer copies only the page it would change («PagedAttention e vLLM»; «Paged Attention optimiza el uso de memoria» on
copy-on-write); release must not free blocks still in use and no request may
see another's private continuation («Servicio…presupuesto de memoria» §8).

Readings where the pages are silent (each is one of several correct
choices; the library follows the same ones so allocator state can be
compared bit for bit):

* free list is a stack: ``init`` pushes the initial order reversed, so pops
  return ``perm[0], perm[1], ...``; freed blocks are pushed on top;
* sequence ids start at 0 and are never reused;
* a batched append serves ids in the order given; a duplicate id in one
  batch is invalid;
* the token at position ``pos`` needs a fresh block when ``pos % B == 0``;
  otherwise, if its block is shared (refcount > 1), the writer takes a fresh
  block, the shared block loses one reference, and the pair (old, new) is
  recorded so the whole block's contents can be copied;
* slot number = block id · B + pos % B;
* release walks the table in logical order and pushes each block whose
  count drops to zero;
* every call is all-or-nothing: on pool exhaustion nothing changes.

Sliding window («¿Cuánta memoria reservar para la caché KV?», "Adaptar…": a
layer with windowed attention keeps a bounded history; «¿Cómo gestiona…?»:
a window changes how much state a sequence keeps, paging how it is
allocated): ``release_before(sid, pos)`` gives back every block whose
positions all lie before ``pos``, walking the table in logical order as a
release does; its table entry becomes ``HOLE`` (-1) so the table stays
indexed by position.  ``pos`` may not exceed the length, so the block being
filled is never released.

Prefix cache («Servicio…presupuesto de memoria» §8: reusing the KV state of
identical prefixes saves repeated work; the cache key must identify every
input that shapes the state, model version and configuration included;
reused pages must not expose or let anyone change another request's private
continuation; cancelling and evicting drop references without freeing pages
in use.  «PagedAttention e vLLM»: a long shared system prompt is processed
once, not again for every request).  Readings taken:

* only full blocks are cached (a partial block is still being written);
* an entry is keyed exactly by (namespace, parent entry, the block's B token
  ids) — the namespace stands for the model version and configuration, the
  parent for everything before the block — and holds one reference to its
  block;
* ``prefix_register(sid, tokens, ns)`` walks the sequence's full blocks from
  position 0: a known key is touched (and, if it names another block with
  the same content, kept), an unknown key becomes a new entry for the
  sequence's block; it stops at a released block (a hole);
* ``prefix_match(tokens, ns)`` creates a sequence made of the longest chain
  of cached blocks that matches the tokens' leading full blocks (one more
  reference per block, as a fork) and touches the chain; the new sequence's
  next token starts a fresh block, so cached blocks are never written;
* ``prefix_evict(k)`` repeatedly drops the least recently used entry among
  those with no child entry whose block only the cache holds (count 1),
  deeper entries first on equal use, until k blocks are free again or none
  qualifies; ``prefix_clear()`` drops every entry;
* use is a logical clock that advances once per register or match call.
"""
from __future__ import annotations

import copy
from typing import Dict, List, Sequence, Tuple


class AllocError(Exception):
    pass


class NoBlocks(AllocError):
    pass


class BadSeq(AllocError):
    pass


class Invalid(AllocError):
    pass


HOLE = -1      # table entry of a block released by release_before


class Allocator:
    def __init__(self, num_blocks: int, block: int = 16, perm: Sequence[int] = None):
        if num_blocks < 1 or block < 1:
            raise Invalid("num_blocks and block must be positive")
        if perm is None:
            perm = list(range(num_blocks))
        perm = [int(x) for x in perm]
        if sorted(perm) != list(range(num_blocks)):
            raise Invalid("perm must be a permutation of 0..num_blocks-1")
        self.N = num_blocks
        self.B = block
        self.free: List[int] = list(reversed(perm))
        self.ref: List[int] = [0] * num_blocks
        self.seqs: Dict[int, Tuple[int, List[int]]] = {}
        self.next_id = 0
        # prefix cache: key (ns, parent entry, tokens) -> entry index;
        # entry index -> [key, block, last_use, depth, children]
        self.pc_index: Dict[tuple, int] = {}
        self.pc: Dict[int, list] = {}
        self.pc_next = 0
        self.pc_clock = 0

    # -- sequences ---------------------------------------------------------
    def create(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = (0, [])
        return sid

    def fork(self, parent: int) -> int:
        if parent not in self.seqs:
            raise BadSeq(parent)
        n, table = self.seqs[parent]
        for b in table:
            if b != HOLE:
                self.ref[b] += 1
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = (n, list(table))
        return sid

    def free_seq(self, sid: int) -> None:
        if sid not in self.seqs:
            raise BadSeq(sid)
        _, table = self.seqs.pop(sid)
        for b in table:
            if b == HOLE:
                continue
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    def release_before(self, sid: int, pos: int) -> int:
        """Release the blocks of ``sid`` that hold only positions < ``pos``
        (block i with (i + 1)·B <= pos) and are not holes yet, in logical
        order; returns how many were released."""
        if sid not in self.seqs:
            raise BadSeq(sid)
        n, table = self.seqs[sid]
        if pos < 0 or pos > n:
            raise Invalid("release position outside [0, length]")
        released = 0
        for i in range(pos // self.B):
            b = table[i]
            if b == HOLE:
                continue
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
            table[i] = HOLE
            released += 1
        return released

    # -- slot reservation ----------------------------------------------------
    def _append_one(self, sid: int, cow: List[Tuple[int, int]]) -> int:
        n, table = self.seqs[sid]
        pos = n
        if pos % self.B == 0:
            if not self.free:
                raise NoBlocks()
            b = self.free.pop()
            self.ref[b] = 1
            table.append(b)
        else:
            last = table[-1]
            if self.ref[last] > 1:
                if not self.free:
                    raise NoBlocks()
                nb = self.free.pop()
                self.ref[last] -= 1
                self.ref[nb] = 1
                cow.append((last, nb))
                table[-1] = nb
        slot = table[pos // self.B] * self.B + pos % self.B
        self.seqs[sid] = (n + 1, table)
        return slot

    def _transaction(self, fn):
        saved = (list(self.free), list(self.ref),
                 {k: (v[0], list(v[1])) for k, v in self.seqs.items()}, self.next_id)
        try:
            return fn()
        except AllocError:
            self.free, self.ref, self.seqs, self.next_id = saved
            raise

    # -- prefix cache --------------------------------------------------------
    def prefix_register(self, sid: int, tokens: Sequence[int], ns: int) -> int:
        """Enter the full blocks of ``sid`` (token ids ``tokens`` for its
        positions 0..) into the cache; returns the number of new entries."""
        if sid not in self.seqs:
            raise BadSeq(sid)
        n, table = self.seqs[sid]
        tokens = [int(t) for t in tokens]
        if len(tokens) < n:
            raise Invalid("fewer token ids than the sequence holds")
        self.pc_clock += 1
        parent, added = -1, 0
        for i in range(n // self.B):
            b = table[i]
            if b == HOLE:
                break
            key = (int(ns), parent, tuple(tokens[i * self.B:(i + 1) * self.B]))
            e = self.pc_index.get(key)
            if e is None:
                e = self.pc_next
                self.pc_next += 1
                self.pc_index[key] = e
                self.pc[e] = [key, b, self.pc_clock, i, 0]
                if parent >= 0:
                    self.pc[parent][4] += 1
                self.ref[b] += 1
                added += 1
            else:
                self.pc[e][2] = self.pc_clock
            parent = e
        return added

    def prefix_match(self, tokens: Sequence[int], ns: int) -> Tuple[int, int]:
        """New sequence sharing the longest cached chain of the tokens'
        leading full blocks; returns (sequence id, matched tokens)."""
        tokens = [int(t) for t in tokens]
        self.pc_clock += 1
        parent, chain = -1, []
        for i in range(len(tokens) // self.B):
            e = self.pc_index.get((int(ns), parent, tuple(tokens[i * self.B:(i + 1) * self.B])))
            if e is None:
                break
            chain.append(e)
            parent = e
        table = []
        for e in chain:
            self.pc[e][2] = self.pc_clock
            b = self.pc[e][1]
            self.ref[b] += 1
            table.append(b)
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = (len(table) * self.B, table)
        return sid, len(table) * self.B

    def _pc_drop(self, e: int) -> None:
        key, b, _, _, _ = self.pc.pop(e)
        del self.pc_index[key]
        if key[1] >= 0:
            self.pc[key[1]][4] -= 1
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)

    def prefix_evict(self, k: int) -> int:
        """Free up to k blocks held only by the cache (LRU leaves first);
        returns the number freed."""
        if k < 0:
            raise Invalid("negative count")
        freed = 0
        while freed < k:
            cands = [(v[2], -v[3], e) for e, v in self.pc.items() if v[4] == 0 and self.ref[v[1]] == 1]
            if not cands:
                break
            self._pc_drop(min(cands)[2])
            freed += 1
        return freed

    def prefix_clear(self) -> int:
        """Drop every entry (children before parents); returns how many."""
        n = 0
        for e in sorted(self.pc, key=lambda e: (-self.pc[e][3], e)):
            self._pc_drop(e)
            n += 1
        return n

    def prefix_snapshot(self):
        """[(entry, ns, parent, tokens, block, last_use)] by entry index."""
        return [(e, v[0][0], v[0][1], list(v[0][2]), v[1], v[2]) for e, v in sorted(self.pc.items())]

    def append(self, ids: Sequence[int]):
        """One token for each id, in order.  Returns (slots, cow_pairs)."""
        ids = [int(i) for i in ids]
        if len(set(ids)) != len(ids):
            raise Invalid("duplicate id in batch")
        for i in ids:
            if i not in self.seqs:
                raise BadSeq(i)

        def run():
            cow: List[Tuple[int, int]] = []
            slots = [self._append_one(i, cow) for i in ids]
            return slots, cow
        return self._transaction(run)

    def extend(self, sid: int, k: int):
        """k successive one-token appends of ``sid``; all-or-nothing."""
        if sid not in self.seqs:
            raise BadSeq(sid)
        if k < 0:
            raise Invalid("negative count")

        def run():
            cow: List[Tuple[int, int]] = []
            slots = [self._append_one(sid, cow) for _ in range(k)]
            return slots, cow
        return self._transaction(run)

    # -- inspection ----------------------------------------------------------
    def length(self, sid: int) -> int:
        return self.seqs[sid][0]

    def table(self, sid: int) -> List[int]:
        return list(self.seqs[sid][1])

    def snapshot(self):
        """(free stack bottom..top, refcounts, [(id, len, table)] by id, next_id)."""
        return (list(self.free), list(self.ref),
                [(k, v[0], list(v[1])) for k, v in sorted(self.seqs.items())],
                self.next_id)

    def stats(self):
        used = self.N - len(self.free)
        sum_len = sum(v[0] for v in self.seqs.values())
        tail = sum(self.B * len(v[1]) - v[0] for v in self.seqs.values())
        return {"free": len(self.free), "used": used, "sum_len": sum_len,
                "sum_ref": sum(self.ref), "tail_waste": tail, "num_seqs": len(self.seqs)}

    def check_invariants(self) -> None:
        """Raise AssertionError if the state breaks a pool invariant."""
        assert sum(self.ref) == sum(sum(1 for b in t if b != HOLE) for _, t in self.seqs.values()) + len(self.pc)
        live = {b for b in range(self.N) if self.ref[b] > 0}
        assert len(set(self.free)) == len(self.free)
        assert live.isdisjoint(self.free)
        assert live | set(self.free) == set(range(self.N))
        for b in range(self.N):
            assert self.ref[b] >= 0
        counts = [0] * self.N
        for n, t in self.seqs.values():
            assert len(t) == -(-n // self.B)
            assert 0 <= self.B * len(t) - n <= self.B - 1 or n == 0
            for b in t:
                if b != HOLE:
                    counts[b] += 1
            # holes only at the head, and never the block being filled
            live_from = next((i for i, b in enumerate(t) if b != HOLE), len(t))
            assert all(b != HOLE for b in t[live_from:])
            assert n % self.B == 0 or live_from < len(t)
        for v in self.pc.values():
            counts[v[1]] += 1
        assert counts == self.ref
        # every entry's parent exists and counts it as a child
        kids = {e: 0 for e in self.pc}
        for e, v in self.pc.items():
            if v[0][1] >= 0:
                assert v[0][1] in self.pc
                kids[v[0][1]] += 1
        assert all(kids[e] == self.pc[e][4] for e in self.pc)

    def clone(self) -> "Allocator":
        return copy.deepcopy(self)


def run_script(alloc: Allocator, ops, on_slots=None):
    """Execute a workload script.  ``on_slots(op, sid_or_ids, slots, cow)`` is
    called after each extend/append so a caller can write values.  Errors
    from the allocator propagate."""
    for op in ops:
        kind = op[0]
        if kind == "create":
            alloc.create()
        elif kind == "fork":
            alloc.fork(op[1])
        elif kind == "free":
            alloc.free_seq(op[1])
        elif kind == "release":
            alloc.release_before(op[1], op[2])
        elif kind == "window":              # keep the last op[2] positions
            alloc.release_before(op[1], max(0, alloc.length(op[1]) - op[2]))
        elif kind == "register":            # ("register", sid, tokens, ns)
            alloc.prefix_register(op[1], op[2], op[3])
        elif kind == "match":               # ("match", tokens, ns)
            alloc.prefix_match(op[1], op[2])
        elif kind == "evict":
            alloc.prefix_evict(op[1])
        elif kind == "clear":
            alloc.prefix_clear()
        elif kind == "register_stream":     # ("register_stream", sid, stream, ns)
            from workloads import stream_tokens
            if op[1] not in alloc.seqs:
                raise BadSeq(op[1])
            alloc.prefix_register(op[1], stream_tokens(op[2], alloc.length(op[1])), op[3])
        elif kind == "match_stream":        # ("match_stream", stream, n, ns)
            from workloads import stream_tokens
            alloc.prefix_match(stream_tokens(op[1], op[2]), op[3])
        elif kind == "extend":
            slots, cow = alloc.extend(op[1], op[2])
            if on_slots:
                on_slots(op, op[1], slots, cow)
        elif kind == "append":
            ids = [e[0] for e in op[1]]
            slots, cow = alloc.append(ids)
            if on_slots:
                on_slots(op, ids, slots, cow)
        else:
            raise ValueError(kind)
