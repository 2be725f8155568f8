"""GPU parity on the five decode workloads at their full sizes.

Small ones are compared on every output; the 32K-token batch and the
32-layer step on sampled (sequence, head) rows that the oracle computes one
by one.  Allocator state and the pool bytes are compared exactly.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from gpu_common import (check_allocator, check_pool, compare_out, need_gpu, note, oracle_out,
                        oracle_replay, run_gpu)

pytestmark = pytest.mark.gpu


def test_tiny_config():
    need_gpu()
    wl = workloads.tiny()
    note(wl.description)
    q, k, v = wl.tensors(device="cuda")
    eng, log, out = run_gpu(wl, {0: k}, {0: v}, q)
    rp = oracle_replay(wl, {0: k}, {0: v})
    check_allocator(eng, rp, log)
    check_pool(eng, rp)
    compare_out(out[0], oracle_out(rp, wl, q))


def test_single_layer_config_and_permutation():
    need_gpu()
    wl = workloads.single_layer()
    note(wl.description)
    q, k, v = wl.tensors(device="cuda")
    eng, log, out = run_gpu(wl, {0: k}, {0: v}, q)
    rp = oracle_replay(wl, {0: k}, {0: v})
    check_allocator(eng, rp, log)
    check_pool(eng, rp)
    e = compare_out(out[0], oracle_out(rp, wl, q))
    note(f"  max_abs={e[0]:.3e} row_rel={e[1]:.3e}")
    del eng
    wl2 = dataclasses.replace(wl, perm=np.random.default_rng(1001).permutation(wl.num_blocks).astype(np.int32))
    _, _, out2 = run_gpu(wl2, {0: k}, {0: v}, q)
    assert torch.equal(out[0].view(torch.int16), out2[0].view(torch.int16))


def test_shared_prefix_config_and_private_twin():
    need_gpu()
    sh = workloads.shared_prefix()
    pr = workloads.shared_prefix(private_copies=True)
    note(sh.description)
    q, k, v = sh.tensors(device="cuda")
    offs = sh.offsets
    for s in range(1, sh.S):
        k[offs[s]:offs[s] + 1024] = k[0:1024]
        v[offs[s]:offs[s] + 1024] = v[0:1024]
    eng, log, out_s = run_gpu(sh, {0: k}, {0: v}, q)
    rp = oracle_replay(sh, {0: k}, {0: v})
    check_allocator(eng, rp, log)
    check_pool(eng, rp)
    # 64 prefix blocks, each referenced by all 128 sequences
    assert sum(1 for r in rp.alloc.ref if r == sh.S) == 64
    e = compare_out(out_s[0], oracle_out(rp, sh, q))
    note(f"  max_abs={e[0]:.3e} row_rel={e[1]:.3e}")
    del eng
    _, _, out_p = run_gpu(pr, {0: k}, {0: v}, q)
    assert torch.equal(out_s[0].view(torch.int16), out_p[0].view(torch.int16))


def test_long_context_config_sampled():
    need_gpu()
    wl = workloads.long_context()
    note(wl.description)
    q, k, v = wl.tensors(device="cuda")
    eng, log, out = run_gpu(wl, {0: k}, {0: v}, q)
    rp = oracle_replay(wl, {0: k}, {0: v})
    check_allocator(eng, rp, log)
    check_pool(eng, rp)
    rows = [(s, h) for s in (0, 6, 15) for h in (0, 7, 8, 33, 63)]
    e = compare_out(out[0], oracle_out(rp, wl, q, rows=rows), rows=rows)
    note(f"  sampled rows max_abs={e[0]:.3e} row_rel={e[1]:.3e}")
    assert torch.isfinite(out[0].float()).all()


def test_full_step_config_sampled():
    need_gpu()
    wl = workloads.full_step()
    note(wl.description)
    layers = (0, 31)
    ts = {l: wl.tensors(l, device="cuda") for l in layers}
    k = {l: ts[l][1] for l in layers}
    v = {l: ts[l][2] for l in layers}
    q = {l: ts[l][0] for l in layers}
    eng, log, out = run_gpu(wl, k, v, q, layers=layers, engine_layers=wl.layers)
    rp = oracle_replay(wl, k, v, layers=layers)
    check_allocator(eng, rp, log)
    longest = int(np.argmax(wl.lengths))
    rows = [(s, h) for s in (0, 17, 100, 255, longest) for h in (0, 13, 31)]
    for l in layers:
        check_pool(eng, rp, l)
        e = compare_out(out[l], oracle_out(rp, wl, q[l], layer=l, rows=rows), rows=rows)
        note(f"  layer {l} sampled rows max_abs={e[0]:.3e} row_rel={e[1]:.3e}")
        assert torch.isfinite(out[l].float()).all()
