"""Pins of the oracle allocator: hand-derived scenarios and invariants."""
import json
import os

import numpy as np
import pytest

import workloads
from conftest import GOLDEN
from oracle import allocator as A

with open(os.path.join(GOLDEN, "allocator_scripts.json")) as f:
    GOLD = json.load(f)

ERR = {"NO_BLOCKS": A.NoBlocks, "INVALID": A.Invalid, "BAD_SEQ": A.BadSeq}


def run_golden_steps(alloc, steps):
    for st in steps:
        op = st["op"]
        before = alloc.snapshot()
        if "error" in st:
            with pytest.raises(ERR[st["error"]]):
                _apply(alloc, op)
            assert alloc.snapshot() == before, "failed call changed state"
            continue
        res = _apply(alloc, op)
        if "id" in st:
            assert res == st["id"]
        if "released" in st:
            assert res == st["released"], op
        if "slots" in st:
            slots, cow = res
            assert slots == st["slots"], op
            assert [list(p) for p in cow] == st["cow"], op
        alloc.check_invariants()


def _apply(alloc, op):
    k = op[0]
    if k == "create":
        return alloc.create()
    if k == "fork":
        return alloc.fork(op[1])
    if k == "free":
        return alloc.free_seq(op[1])
    if k == "extend":
        return alloc.extend(op[1], op[2])
    if k == "append":
        return alloc.append(op[1])
    if k == "release":
        return alloc.release_before(op[1], op[2])
    raise ValueError(k)


SCRIPTED = {sc["name"]: sc for sc in GOLD["scenarios"] if "steps" in sc}


@pytest.mark.parametrize("which", ["fork_cow_free_oom", "sliding_window_release"])
def test_golden_scenarios(which):
    sc = SCRIPTED[which]
    alloc = A.Allocator(sc["num_blocks"], sc["block"], sc["perm"])
    run_golden_steps(alloc, sc["steps"])
    free, ref, seqs, next_id = alloc.snapshot()
    assert free == sc["final"]["free"]
    assert ref == sc["final"]["ref"]
    assert [[i, n, t] for i, n, t in seqs] == sc["final"]["seqs"]
    assert next_id == sc["final"]["next_id"]


def test_golden_tiny_layout():
    sc = GOLD["scenarios"][1]
    wl = workloads.tiny()
    assert list(wl.lengths) == sc["lengths"] and wl.num_blocks == sc["num_blocks"]
    alloc = A.Allocator(wl.num_blocks, wl.block, wl.perm)
    A.run_script(alloc, wl.setup_ops)
    slots, cow = alloc.append([e[0] for e in wl.step_ops[0][1]])
    assert cow == []
    perm = [int(x) for x in wl.perm]
    assert [alloc.table(s) for s in wl.seq_ids] == [[perm[i] for i in row] for row in sc["tables_as_perm_index"]]
    assert slots == [perm[i] * 16 + o for i, o in sc["step_slots_as"]]
    st = alloc.stats()
    assert st["used"] == sc["blocks_used"]
    assert [16 * len(alloc.table(s)) - alloc.length(s) for s in wl.seq_ids] == sc["tails"]


def test_pops_follow_perm_and_lifo_reuse():
    alloc = A.Allocator(6, 2, [3, 1, 4, 0, 5, 2])
    a = alloc.create()
    slots, _ = alloc.extend(a, 6)
    assert alloc.table(a) == [3, 1, 4]
    assert slots == [6, 7, 2, 3, 8, 9]
    alloc.free_seq(a)
    # released in logical order onto the stack: 3, 1, 4 -> next pops 4, 1, 3
    b = alloc.create()
    alloc.extend(b, 5)
    assert alloc.table(b) == [4, 1, 3]


def test_cow_copy_only_when_shared_partial():
    alloc = A.Allocator(10, 4)
    p = alloc.create()
    alloc.extend(p, 8)                      # block-aligned
    c = alloc.fork(p)
    slots, cow = alloc.append([c])          # pos 8: fresh block, no copy
    assert cow == []
    alloc.append([p])                       # parent too: fresh block, no copy
    c2 = alloc.fork(c)                      # c has len 9: shares a partial block
    _, cow = alloc.append([c2])
    assert len(cow) == 1 and cow[0][0] == alloc.table(c)[-1]
    _, cow = alloc.append([c])              # last holder writes in place
    assert cow == []


def test_free_parent_keeps_children_blocks():
    alloc = A.Allocator(8, 4)
    p = alloc.create()
    alloc.extend(p, 8)
    kids = [alloc.fork(p) for _ in range(3)]
    alloc.free_seq(p)
    assert alloc.stats()["free"] == 6
    assert all(alloc.ref[b] == 3 for b in alloc.table(kids[0]))
    for k in kids:
        alloc.free_seq(k)
    assert alloc.stats()["free"] == 8 and sum(alloc.ref) == 0


def test_oom_rolls_back_whole_batch():
    alloc = A.Allocator(3, 4)
    a, b = alloc.create(), alloc.create()
    alloc.extend(a, 4)
    alloc.extend(b, 4)
    before = alloc.snapshot()
    # a needs a fresh block (pos 4), b needs one too, only one left
    with pytest.raises(A.NoBlocks):
        alloc.append([a, b])
    assert alloc.snapshot() == before
    with pytest.raises(A.NoBlocks):
        alloc.extend(a, 9)
    assert alloc.snapshot() == before


@pytest.mark.parametrize("seed,windows", [(0, False), (1, False), (2, True), (3, True)])
def test_random_ops_invariants(seed, windows):
    ops = workloads.random_op_script(seed, 2500, windows=windows)
    alloc = A.Allocator(24, 4, np.random.default_rng(seed).permutation(24))
    fails = 0
    for op in ops:
        before = alloc.snapshot()
        try:
            if op[0] == "append":
                ids = [e[0] for e in op[1]]
                slots, cow = alloc.append(ids)
                assert len(set(slots)) == len(slots)
                # every written slot lies in a block this sequence alone holds
                for s in slots:
                    assert alloc.ref[s // 4] == 1
            else:
                A.run_script(alloc, [op])
        except A.NoBlocks:
            fails += 1
            assert alloc.snapshot() == before
        alloc.check_invariants()
    assert fails > 0, "the script should exhaust the small pool sometimes"
