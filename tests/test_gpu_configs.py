"""GPU parity on the five decode workloads at their full sizes, every
output row against the oracle; allocator state and pool bytes exactly.
The 32K-token batch (bf16 and 8-bit caches) and the 32-layer step are
decoded the way the benchmark decodes them, with the step's new token
handed to the decode call, and checked bit for bit against the same step
done with a separate kv_append_last.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from gpu_common import (check_allocator, check_pool, check_pool_layer, check_same_bits, compare_out, decode_step,
                        need_gpu, note, oracle_out, oracle_replay, run_gpu, step_inputs)

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


def _plan(eng, wl, q, layer=0, **kw):
    from paged_kv_cache_08_amd import pkv as P
    info, _ = P.pkv_decode_plan(eng.decode_args(layer, q, torch.empty_like(q), wl.max_len, **kw), with_cells=False)
    return info


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_long_context_config(cache):
    """The 32K-token batch decoded as the benchmark decodes it: the step's
    new token handed to the decode call (written by the partial kernel),
    runs of several partitions per wave (the deep pipeline for the bf16
    cache).  Pool and output bits equal those of the same step done by
    kv_append_last + decode; allocator, pool and every (sequence, head)
    row against the oracle."""
    need_gpu()
    wl = workloads.long_context()
    if cache == "fp8":
        wl = workloads.fp8_cache(wl)
    note(wl.description)
    q, k, v = wl.tensors(device="cuda")
    fus, out_f = decode_step(wl, {0: k}, {0: v}, {0: q}, fused=True)
    ids, rows = step_inputs(wl, k)
    info = _plan(fus, wl, q, k_new=k.index_select(0, rows), v_new=v.index_select(0, rows))
    note(f"  plan: depth {info.pipeline_depth}, {info.partitions_per_wave} partitions per wave, "
         f"fused append {info.fused_append}, {info.cells} cells")
    assert info.fused_append == 1 and info.partitions_per_wave > 1 and not info.work_list
    assert info.pipeline_depth == (5 if cache == "bf16" else 4)
    sep, out_s = decode_step(wl, {0: k}, {0: v}, {0: q}, fused=False)
    for a, b, what in ((fus.k[0], sep.k[0], "K pool"), (fus.v[0], sep.v[0], "V pool"), (out_f[0], out_s[0], "output")):
        check_same_bits(a, b, what)
    if cache == "fp8":
        check_same_bits(fus.ks[0], sep.ks[0], "K scales")
        check_same_bits(fus.vs[0], sep.vs[0], "V scales")
    del sep
    rp = oracle_replay(wl, {0: k}, {0: v})
    assert fus.snapshot() == tuple(rp.alloc.snapshot())
    check_pool(fus, rp)
    e = compare_out(out_f[0], oracle_out(rp, wl, q))
    note(f"  all {wl.S * wl.Hq} rows max_abs={e[0]:.3e} row_rel={e[1]:.3e}")


def test_full_step_config():
    """The 32-layer step at full size: layers 0 and 31 (their own K/V and
    queries), the new token handed to the decode call as the benchmark does
    (the library picks the fused or the separate append for this batch),
    bits equal to the kv_append_last step; allocator, pools and every
    (sequence, head) row of both layers against the oracle."""
    need_gpu()
    wl = workloads.full_step()
    note(wl.description)
    layers = (0, 31)
    ts = {l: wl.tensors(l, device="cuda") for l in layers}
    k = {l: ts[l][1] for l in layers}
    v = {l: ts[l][2] for l in layers}
    q = {l: ts[l][0] for l in layers}
    fus, out_f = decode_step(wl, k, v, q, fused=True, layers=layers)
    sep, out_s = decode_step(wl, k, v, q, fused=False, layers=layers)
    for i, l in enumerate(layers):
        check_same_bits(fus.k[i], sep.k[i], f"K pool of layer {l}")
        check_same_bits(fus.v[i], sep.v[i], f"V pool of layer {l}")
        check_same_bits(out_f[l], out_s[l], f"output of layer {l}")
    del sep
    rp = oracle_replay(wl, k, v, layers=layers)
    assert fus.snapshot() == tuple(rp.alloc.snapshot())
    for i, l in enumerate(layers):
        check_pool_layer(fus, i, rp, l)
        e = compare_out(out_f[l], oracle_out(rp, wl, q[l], layer=l))
        note(f"  layer {l}: all {wl.S * wl.Hq} rows max_abs={e[0]:.3e} row_rel={e[1]:.3e}")
