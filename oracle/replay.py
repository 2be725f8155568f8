"""Run a workload script through the oracle allocator and pool (test infra).

The workload object only supplies inputs (script, initial free order, shapes,
logical per-sequence K/V values).  Here the oracle's own allocator decides
every slot, its own pool receives the values, copy-on-write pairs are copied
before the new token is written, and the decode inputs (tables, lengths)
are read back from the oracle's own state.
"""
from __future__ import annotations

import numpy as np

from .allocator import Allocator, run_script
from .pool import Pool


class Replay:
    def __init__(self, wl, layers=None):
        self.wl = wl
        self.alloc = Allocator(wl.num_blocks, wl.block, wl.perm)
        n_layers = wl.layers if layers is None else layers
        self.pool = Pool(wl.num_blocks, wl.Hkv, wl.d, wl.cache_dtype, wl.block, layers=n_layers,
                         lazy_layers=True)
        self.log = []          # (op kind, ids, slots, cow pairs) per extend/append

    def run(self, ops, values=None, sources=None):
        """Execute ``ops``; ``values`` maps layer -> (k_bits, v_bits) logical
        arrays [sum n][Hkv][d]; every listed layer receives the tokens.
        ``sources``: optional set of logical sequences whose tokens are
        written (the allocator still runs every op; other slots keep their
        poison) — for spot checks of batches too large to fill whole."""
        offs = self.wl.offsets
        values = values or {}

        def on_slots(op, ids, slots, cow):
            self.log.append((op[0], ids, list(slots), list(cow)))
            for a, b in cow:
                self.pool.copy_block(a, b)
            if op[0] == "extend":
                _, sid, k, src, pos = op
                rows = np.arange(offs[src] + pos, offs[src] + pos + k)
                keep = np.full(k, sources is None or src in sources)
            else:
                rows = np.array([offs[src] + pos for (_, src, pos) in op[1]], dtype=np.int64)
                keep = np.array([sources is None or src in sources for (_, src, _) in op[1]], dtype=bool)
            if not keep.any():
                return
            sl = np.asarray(slots)[keep]
            for layer, (kb, vb) in values.items():
                self.pool.scatter(layer, sl, kb[rows[keep]], vb[rows[keep]])

        run_script(self.alloc, ops, on_slots)
        return self

    def tables(self):
        return [self.alloc.table(sid) for sid in self.wl.seq_ids]

    def lengths(self):
        return [self.alloc.length(sid) for sid in self.wl.seq_ids]
