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


def _tokens(sc, name):
    toks = sc.get("tokens", {})
    if name in toks:
        return toks[name]
    return toks[name[0]][:int(name[1:])]          # e.g. "B10": the first 10 of B


def run_golden_steps(alloc, steps, sc=None):
    for k, st in enumerate(steps):
        op = list(st["op"])
        if op[0] == "register":
            op[2] = _tokens(sc, op[2])
        elif op[0] == "match":
            op[1] = _tokens(sc, op[1])
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
        if "added" in st:
            assert res == st["added"], op
        if "freed" in st:
            assert res == st["freed"], op
        if "match" in st:
            assert list(res) == st["match"], op
        if sc is not None and str(k) in sc.get("cache_after_step", {}):
            assert [list(e) for e in alloc.prefix_snapshot()] == sc["cache_after_step"][str(k)], k
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
    if k == "register":
        return alloc.prefix_register(op[1], op[2], op[3])
    if k == "match":
        return alloc.prefix_match(op[1], op[2])
    if k == "evict":
        return alloc.prefix_evict(op[1])
    raise ValueError(k)


SCRIPTED = {sc["name"]: sc for sc in GOLD["scenarios"] if "steps" in sc}


@pytest.mark.parametrize("which", ["fork_cow_free_oom", "sliding_window_release", "prefix_cache"])
def test_golden_scenarios(which):
    sc = SCRIPTED[which]
    alloc = A.Allocator(sc["num_blocks"], sc["block"], sc["perm"])
    run_golden_steps(alloc, sc["steps"], sc)
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


@pytest.mark.parametrize("seed,windows,prefix", [(0, False, False), (1, False, False), (2, True, False),
                                                 (3, True, False), (4, False, True), (5, True, True)])
def test_random_ops_invariants(seed, windows, prefix):
    ops = workloads.random_op_script(seed, 2500, windows=windows, prefix=prefix)
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


def test_prefix_cache_namespace_and_exact_keys():
    """A different namespace (model version / configuration) or a different
    earlier block never matches, even with identical block tokens."""
    alloc = A.Allocator(12, 4)
    a = alloc.create()
    alloc.extend(a, 12)
    toks = list(range(100, 112))
    assert alloc.prefix_register(a, toks, ns=1) == 3
    _, got = alloc.prefix_match(toks, ns=2)
    assert got == 0
    _, got = alloc.prefix_match([0, 0, 0, 0] + toks[4:], ns=1)     # same blocks 1-2, other first block
    assert got == 0
    _, got = alloc.prefix_match(toks[:11], ns=1)                   # only full blocks match
    assert got == 8
    alloc.check_invariants()


def test_prefix_cache_shared_blocks_are_never_written():
    """A sequence built from cached blocks writes its next token into a
    fresh block: no copy-on-write pair, no slot inside a cached block."""
    alloc = A.Allocator(16, 4)
    a = alloc.create()
    alloc.extend(a, 10)
    alloc.prefix_register(a, list(range(10)), ns=0)
    cached = {v[1] for v in alloc.pc.values()}
    sid, got = alloc.prefix_match(list(range(10)) + [77, 78], ns=0)
    assert got == 8
    slots, cow = alloc.extend(sid, 5)
    assert cow == [] and not any(s // 4 in cached for s in slots)
    slots, cow = alloc.append([sid, a])
    assert cow == [] and not any(s // 4 in cached for s in slots)
    alloc.check_invariants()


def test_prefix_evict_never_frees_blocks_in_use():
    alloc = A.Allocator(8, 4)
    a = alloc.create()
    alloc.extend(a, 8)
    alloc.prefix_register(a, list(range(8)), ns=0)
    assert alloc.prefix_evict(5) == 0            # the sequence still holds both blocks
    alloc.free_seq(a)
    assert alloc.prefix_evict(1) == 1            # the leaf goes first
    assert [e[3] for e in alloc.prefix_snapshot()] == [[0, 1, 2, 3]]
    assert alloc.prefix_clear() == 1
    assert len(alloc.free) == 8
    alloc.check_invariants()
