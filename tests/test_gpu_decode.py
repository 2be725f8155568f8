"""GPU parity: the library (allocator, kv_append, copy_blocks, decode
kernels) against the CPU oracle on the same seeded inputs.

Allocator state, slot mappings and the pool contents are compared bit for
bit (free and tail slots hold NaN poison on both sides); attention outputs
within max |err| <= 2e-2 and row-normwise relative error <= 1e-2.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from gpu_common import (check_allocator, check_pool, compare_out, need_gpu, note, oracle_out,
                        oracle_replay, run_gpu)

pytestmark = pytest.mark.gpu


def _full_case(wl, partition=0, scale=None, q_scale=1.0):
    need_gpu()
    note(f"case: {wl.description} partition={partition} q_scale={q_scale}")
    q, k, v = wl.tensors(device="cuda")
    if q_scale != 1.0:
        q = (q.float() * q_scale).to(q.dtype)
    eng, log, out = run_gpu(wl, {0: k}, {0: v}, q, partition=partition, scale=scale)
    rp = oracle_replay(wl, {0: k}, {0: v})
    check_allocator(eng, rp, log)
    check_pool(eng, rp)
    ref = oracle_out(rp, wl, q, scale=scale)
    err = compare_out(out[0], ref)
    note(f"  max_abs={err[0]:.3e} row_rel={err[1]:.3e}")
    return eng, log, out[0], ref


def test_tiny():
    _full_case(workloads.tiny())


SHAPES = [
    # S, Hq, Hkv, d, dtype, max_len
    (5, 8, 2, 128, "bf16", 300),
    (4, 40, 8, 128, "bf16", 1100),
    (3, 40, 2, 128, "bf16", 700),       # 20 query heads per KV head: two head groups
    (6, 8, 1, 64, "bf16", 200),         # one KV head, d = 64
    (3, 4, 4, 128, "f32", 900),         # MHA fp32, several partitions
    (4, 12, 3, 64, "f32", 600),
    (4, 64, 8, 128, "bf16", 2100),
    (2, 64, 1, 128, "bf16", 150),       # 64 query heads on one KV head
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_shapes(shape):
    S, Hq, Hkv, d, dt, ml = shape
    _full_case(workloads.random_small(40 + len(str(shape)), S=S, Hq=Hq, Hkv=Hkv, d=d, dtype=dt, max_len=ml))


EDGE = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1023, 1024, 1025, 1535]


@pytest.mark.parametrize("partition", [0, 32, 64, 1024])
def test_edge_lengths(partition):
    wl = workloads.with_lengths(EDGE, Hq=16, Hkv=4, d=128, dtype="bf16", seed=partition + 1)
    _full_case(wl, partition=partition)


@pytest.mark.parametrize("longest", [1024, 1025], ids=["32 partitions (row reduce)", "33 partitions (wide reduce)"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_reduce_kernel_boundary(longest, dtype, d):
    """Launches whose partition bound is at most 32 merge one row per wave,
    larger ones with a 256-lane workgroup per row; both against the oracle
    at the boundary, with every row's partition count from 1 to the bound."""
    lengths = [1, 31, 32, 33, 97, 480, 512, 513, 1000, longest]
    wl = workloads.with_lengths(lengths, Hq=8, Hkv=2, d=d, dtype=dtype, seed=longest + d)
    _full_case(wl, partition=32)


def test_edge_lengths_fp32():
    wl = workloads.with_lengths(EDGE, Hq=4, Hkv=1, d=64, dtype="f32", seed=5)
    _full_case(wl)


def test_extreme_logits():
    wl = workloads.random_small(61, S=4, Hq=8, Hkv=2, d=128, dtype="bf16", max_len=700)
    _full_case(wl, q_scale=3000.0)


def test_custom_scale():
    wl = workloads.random_small(62, S=3, Hq=8, Hkv=2, d=128, dtype="bf16", max_len=600)
    _full_case(wl, scale=0.37)


def test_permutation_gives_identical_bits():
    need_gpu()
    wl = workloads.random_small(70, S=6, Hq=16, Hkv=4, d=128, dtype="bf16", max_len=1500)
    q, k, v = wl.tensors(device="cuda")
    _, _, out1 = run_gpu(wl, {0: k}, {0: v}, q)
    wl2 = dataclasses.replace(wl, perm=np.random.default_rng(123).permutation(wl.num_blocks).astype(np.int32))
    _, _, out2 = run_gpu(wl2, {0: k}, {0: v}, q)
    assert torch.equal(out1[0].view(torch.int16), out2[0].view(torch.int16))


def test_shared_prefix_equals_private_copies_bits():
    need_gpu()
    kw = dict(seed=9, S=12, prefix=256, lo=16, hi=200)
    sh = workloads.shared_prefix(**kw)
    pr = workloads.shared_prefix(private_copies=True, **kw)
    q, k, v = sh.tensors(device="cuda")
    offs = sh.offsets
    for s in range(1, sh.S):       # every logical sequence carries sequence 0's prefix
        k[offs[s]:offs[s] + 256] = k[0:256]
        v[offs[s]:offs[s] + 256] = v[0:256]
    eng, log, out_s = run_gpu(sh, {0: k}, {0: v}, q)
    _, _, out_p = run_gpu(pr, {0: k}, {0: v}, q)
    assert torch.equal(out_s[0].view(torch.int16), out_p[0].view(torch.int16))
    rp = oracle_replay(sh, {0: k}, {0: v})
    check_allocator(eng, rp, log)
    check_pool(eng, rp)
    compare_out(out_s[0], oracle_out(rp, sh, q))


def _cow_workload(dtype="bf16", d=128):
    lengths = np.array([21, 21, 21, 37])
    ops = [("create",), ("extend", 0, 20, 0, 0), ("fork", 0), ("fork", 0),
           ("append", [(1, 1, 20), (2, 2, 20), (0, 0, 20)]),
           ("fork", 1), ("extend", 3, 15, 3, 21)]
    # seq 3 forks seq 1 at length 21 (inside a block), extends 15 tokens and
    # appends its 37th in the checked step
    step = [("append", [(3, 3, 36)])]
    return workloads.Workload("cow", 1, 8, 2, d, dtype, lengths, 12, np.arange(12, dtype=np.int32)[::-1].copy(),
                              ops, step, [0, 1, 2, 3], 77, description="fork/copy-on-write script")


def test_copy_on_write():
    wl = _cow_workload()
    eng, log, out, ref = _full_case(wl)
    # the batch append copied the shared partial block for seqs 1 and 2, not 0;
    # the extend of seq 3 copied the block it shared with seq 1
    assert [len(c) for _, _, _, c in log] == [0, 2, 1, 0]


def test_copy_on_write_fp32_two_layers():
    need_gpu()
    wl = _cow_workload("f32", 64)
    wl = dataclasses.replace(wl, layers=2)
    t0 = wl.tensors(0, device="cuda")
    t1 = wl.tensors(1, device="cuda")
    k = {0: t0[1], 1: t1[1]}
    v = {0: t0[2], 1: t1[2]}
    eng, log, out = run_gpu(wl, k, v, {0: t0[0], 1: t1[0]}, layers=(0, 1))
    assert any(c for _, _, _, c in log), "script should copy on write"
    rp = oracle_replay(wl, k, v, layers=(0, 1))
    check_allocator(eng, rp, log)
    for layer, q in ((0, t0[0]), (1, t1[0])):
        check_pool(eng, rp, layer)
        compare_out(out[layer], oracle_out(rp, wl, q, layer=layer))


def test_invalid_rows_become_nan():
    need_gpu()
    import paged_kv_cache_08_amd.pkv as P
    wl = workloads.random_small(80, S=5, Hq=8, Hkv=2, d=128, dtype="bf16", max_len=900, min_len=600)
    q, k, v = wl.tensors(device="cuda")
    eng, _, out = run_gpu(wl, {0: k}, {0: v}, q)
    good = out[0].clone()
    tables, lens = eng.tables.clone(), eng.lens.clone()
    lens[1] = 0                          # empty sequence
    lens[2] = wl.max_len + 1             # beyond the declared bound
    tables[3, 1] = wl.num_blocks         # block id outside the pool
    out2 = torch.empty_like(q)
    a = P.decode_args(q, out2, eng.k[0], eng.v[0], tables, lens, wl.Hkv, wl.num_blocks, wl.max_len)
    ws = torch.empty(P.pkv_decode_workspace_bytes(wl.S, wl.Hq, wl.d, wl.max_len), dtype=torch.uint8, device="cuda")
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    P.pkv_paged_attention_decode(a)
    torch.cuda.synchronize()
    for s in (1, 2, 3):
        assert torch.isnan(out2[s].float()).all(), s
    for s in (0, 4):
        assert torch.equal(out2[s].view(torch.int16), good[s].view(torch.int16))


def test_wave_split_does_not_change_bits():
    """The work split (partitions streamed per wave, chosen from the host
    length hint) must not change a single output bit."""
    need_gpu()
    import paged_kv_cache_08_amd.pkv as P
    wl = workloads.with_lengths([3072] * 8, Hq=32, Hkv=8, d=128, dtype="bf16", seed=21)
    q, k, v = wl.tensors(device="cuda")
    eng, _, out = run_gpu(wl, {0: k}, {0: v}, q, partition=32)
    with_hint = out[0]
    no_hint = torch.empty_like(q)
    a = eng.decode_args(0, q, no_hint, wl.max_len)
    a.host_seq_lens = None                   # no hint: one partition per wave
    P.pkv_paged_attention_decode(a)
    torch.cuda.synchronize()
    assert torch.equal(with_hint.view(torch.int16), no_hint.view(torch.int16))
    rp = oracle_replay(wl, {0: k}, {0: v})
    compare_out(with_hint, oracle_out(rp, wl, q))


ORDER_CASES = {
    "bf16, 4 heads per KV head": lambda: workloads.random_small(95, S=37, Hq=16, Hkv=4, d=128, dtype="bf16",
                                                                max_len=1500, min_len=1),
    "8-bit cache": lambda: workloads.fp8_cache(workloads.random_small(96, S=29, Hq=16, Hkv=2, d=128, dtype="bf16",
                                                                      max_len=1500, min_len=1)),
    "32 heads per KV head": lambda: workloads.random_small(97, S=11, Hq=64, Hkv=2, d=64, dtype="bf16",
                                                           max_len=1500, min_len=1),
    # with 32-token partitions: up to 122 partitions, ~18k listed cells
    "300 sequences": lambda: workloads.random_small(98, S=300, Hq=8, Hkv=2, d=64, dtype="bf16", max_len=3900,
                                                    min_len=1),
}


@pytest.mark.parametrize("window", [0, 700])
@pytest.mark.parametrize("case", list(ORDER_CASES))
@pytest.mark.parametrize("partition", [32, 512])
def test_dispatch_order_does_not_change_bits(partition, case, window):
    """Mixed lengths: from the host hint the launch lists only the partitions
    the hint names, largest first; the last listed partition of a sequence
    and sweep waves take whatever the device lengths add.  Any hint (right,
    missing, shuffled, reversed, out of range, all at the bound, all zero)
    must give the bits of the launch without a hint, with and without a
    sliding window."""
    need_gpu()
    import numpy as np
    import paged_kv_cache_08_amd.pkv as P
    wl = ORDER_CASES[case]()
    q, k, v = wl.tensors(device="cuda")
    eng, _, _ = run_gpu(wl, {0: k}, {0: v}, partition=partition)
    first = torch.empty_like(q)                 # without a hint: the plain grid
    a = eng.decode_args(0, q, first, wl.max_len, window=window)
    a.host_seq_lens = None
    P.pkv_paged_attention_decode(a)
    torch.cuda.synchronize()
    ref = first.view(torch.int16).clone()
    lens = np.asarray(eng.host_lens[:wl.S], dtype=np.int32)
    rng = np.random.default_rng(3)
    hints = {"none": None, "right": lens.copy(), "shuffled": rng.permutation(lens).astype(np.int32),
             "reversed": lens[::-1].copy(), "out of range": np.where(lens % 3 == 0, -4, wl.max_len + 9).astype(np.int32),
             "at the bound": np.full(wl.S, wl.max_len, dtype=np.int32), "zeros": np.zeros(wl.S, dtype=np.int32)}
    for name, hint in hints.items():
        note(f"dispatch order: {case}, partition {partition}, window {window}, hint {name}")
        again = torch.empty_like(q)
        a = eng.decode_args(0, q, again, wl.max_len, window=window)
        a.host_seq_lens = None
        if hint is not None:
            a.host_seq_lens, a._keep = hint.ctypes.data, hint
        P.pkv_paged_attention_decode(a)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), ref), name
    rp = oracle_replay(wl, {0: k}, {0: v})
    compare_out(first, oracle_out(rp, wl, q, window=window))


@pytest.mark.parametrize("make", [workloads.tiny, lambda: _cow_workload(),
                                  lambda: workloads.random_small(90, S=7, Hq=8, Hkv=2, d=128, dtype="bf16",
                                                                 max_len=300)],
                         ids=["tiny", "cow", "random"])
def test_step_append_matches_oracle(make):
    """Setup through extend/append with slot mappings, then the checked step
    through the step form (tables upload + kv_append_last)."""
    need_gpu()
    from paged_kv_cache_08_amd.engine import PagedDecodeEngine
    wl = make()
    note(f"step append: {wl.description}")
    q, k, v = wl.tensors(device="cuda")
    eng = PagedDecodeEngine(1, wl.Hkv, wl.d, wl.num_blocks, wl.dtype, init_perm=wl.perm)
    log = eng.run_script(wl.setup_ops, wl, {0: k}, {0: v})
    (kind, entries), = wl.step_ops
    offs = wl.offsets
    rows = torch.tensor([offs[src] + pos for (_, src, pos) in entries], device="cuda")
    ids = [e[0] for e in entries]
    slots, cow = eng.step_append(ids, {0: (k.index_select(0, rows), v.index_select(0, rows))})
    log.append(("append", ids, slots, cow))
    eng.sync(wl.seq_ids)                     # the decode batch may differ from the appended ids
    out = eng.decode(0, q, max_seq_len=wl.max_len)
    torch.cuda.synchronize()
    rp = oracle_replay(wl, {0: k}, {0: v})
    check_allocator(eng, rp, log)
    check_pool(eng, rp)
    compare_out(out, oracle_out(rp, wl, q))



@pytest.mark.parametrize("dtype,d,Hkv", [
    ("bf16", 128, 6),    # 4 heads per wave: the second wave has heads 4 and 5 only
    ("bf16", 64, 3),     # 8 heads per wave, 3 present
    ("bf16", 256, 3),    # 2 heads per wave
    ("f32", 16, 5),      # 16 heads per wave
    ("f32", 128, 3),     # 2 heads per wave
    ("bf16", 96, 3),     # 12 chunks per row do not divide a wave: one wave per row
    ("fp8", 128, 6),     # 8-bit pool: 4 heads per wave, eight values per lane
    ("fp8", 64, 9),      # 8 heads per wave: the second wave has head 8 only
    ("fp8", 192, 2),     # one wave per row
])
def test_append_shapes_match_oracle(dtype, d, Hkv):
    """Both append forms (slot mapping for the set-up, last position for the
    step) write the oracle's pool bit for bit at head dims and head counts
    that fill a wave's head group raggedly or not at all."""
    need_gpu()
    from paged_kv_cache_08_amd.engine import PagedDecodeEngine
    wl = workloads.random_small(91, S=5, Hq=Hkv, Hkv=Hkv, d=d, dtype="bf16" if dtype == "fp8" else dtype,
                                max_len=70)
    if dtype == "fp8":
        wl = workloads.fp8_cache(wl)
    note(f"append shapes: {wl.description}, {wl.cache_dtype} cache")
    q, k, v = wl.tensors(device="cuda")
    eng = PagedDecodeEngine(1, wl.Hkv, wl.d, wl.num_blocks, wl.cache_dtype, init_perm=wl.perm)
    log = eng.run_script(wl.setup_ops, wl, {0: k}, {0: v})
    (kind, entries), = wl.step_ops
    offs = wl.offsets
    rows = torch.tensor([offs[src] + pos for (_, src, pos) in entries], device="cuda")
    ids = [e[0] for e in entries]
    slots, cow = eng.step_append(ids, {0: (k.index_select(0, rows), v.index_select(0, rows))})
    log.append(("append", ids, slots, cow))
    torch.cuda.synchronize()
    rp = oracle_replay(wl, {0: k}, {0: v})
    check_allocator(eng, rp, log)
    check_pool(eng, rp)


def test_workspace_reuse_and_garbage():
    """The split-K workspace may hold anything: repeated calls on one
    workspace, and a workspace full of random bytes, give the same bits, with
    and without the host length hint."""
    need_gpu()
    import paged_kv_cache_08_amd.pkv as P
    wl = workloads.with_lengths([2900] * 6, Hq=16, Hkv=4, d=128, dtype="bf16", seed=33)
    q, k, v = wl.tensors(device="cuda")
    eng, _, out = run_gpu(wl, {0: k}, {0: v}, q)
    ref_bits = out[0].view(torch.int16).clone()
    for trial in range(4):
        if trial >= 2:
            g = torch.Generator(device="cuda").manual_seed(5 + trial)
            eng.workspace.copy_(torch.randint(0, 256, eng.workspace.shape, generator=g, device="cuda",
                                              dtype=torch.int32).to(torch.uint8))
        again = torch.empty_like(q)
        a = eng.decode_args(0, q, again, wl.max_len)
        if trial % 2:
            a.host_seq_lens = None
        P.pkv_paged_attention_decode(a)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), ref_bits), trial
    rp = oracle_replay(wl, {0: k}, {0: v})
    compare_out(out[0], oracle_out(rp, wl, q))


@pytest.mark.parametrize("offset", [0, 1], ids=["16-byte aligned", "4-byte aligned"])
def test_sync_tables_writes_exactly_the_rows(offset):
    """pkv_sync_tables writes each row (table, then -1 padding) and the
    lengths, whether the table buffer allows 16-byte copies or not, with a
    row count that leaves a ragged tail, and nothing around them."""
    need_gpu()
    from paged_kv_cache_08_amd import pkv as P
    from paged_kv_cache_08_amd.engine import PagedDecodeEngine
    wl = workloads.with_lengths([1, 17, 33, 100, 257], Hq=4, Hkv=1, d=64, dtype="f32", seed=3)
    eng = PagedDecodeEngine(1, wl.Hkv, wl.d, wl.num_blocks, wl.cache_dtype, init_perm=wl.perm)
    eng.run_script(wl.setup_ops + wl.step_ops, None)
    ids = list(wl.seq_ids)
    n, mb = len(ids), 23                                    # 115 entries: not a multiple of 4
    buf = torch.full((n * mb + offset + 8,), -7, dtype=torch.int32, device="cuda")
    tab = buf[offset:offset + n * mb].view(n, mb)
    lens = torch.full((n + 2,), -7, dtype=torch.int32, device="cuda")
    host = np.zeros(n, dtype=np.int32)
    P.pkv_sync_tables(eng.pool, ids, tab, lens[1:n + 1], host)
    torch.cuda.synchronize()
    want = np.full((n, mb), -1, dtype=np.int32)
    for r, i in enumerate(ids):
        t = P.pkv_seq_table(eng.pool, i)
        want[r, :len(t)] = t
    got = buf.cpu().numpy()
    assert (got[:offset] == -7).all() and (got[offset + n * mb:] == -7).all()
    assert np.array_equal(got[offset:offset + n * mb].reshape(n, mb), want)
    want_lens = np.array([P.pkv_seq_length(eng.pool, i) for i in ids], dtype=np.int32)
    assert np.array_equal(lens.cpu().numpy()[1:n + 1], want_lens) and np.array_equal(host, want_lens)
    assert lens[0].item() == -7 and lens[n + 1].item() == -7


def test_sync_tables_ring_keeps_every_upload():
    """Successive uploads, on two streams that alternate within the pool's
    groups of four and behind a long matrix product, each land their own
    step's tables and lengths: no staging buffer is refilled while an upload
    that reads it is still queued."""
    need_gpu()
    from paged_kv_cache_08_amd import pkv as P
    from paged_kv_cache_08_amd.engine import PagedDecodeEngine
    wl = workloads.with_lengths([15, 16, 31, 47, 64, 100], Hq=4, Hkv=1, d=64, dtype="f32", seed=5, slack=2.0)
    eng = PagedDecodeEngine(1, wl.Hkv, wl.d, wl.num_blocks, wl.cache_dtype, init_perm=wl.perm)
    eng.run_script(wl.setup_ops + wl.step_ops, None)
    ids = list(wl.seq_ids)
    n, mb, uploads = len(ids), 16, 27
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    tabs = [torch.full((n, mb), -7, dtype=torch.int32, device="cuda") for _ in range(uploads)]
    lens = [torch.full((n,), -7, dtype=torch.int32, device="cuda") for _ in range(uploads)]
    busy = [torch.randn((6144, 6144), device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    for st, a in zip((main, side), busy):    # keep both streams busy for a while
        with torch.cuda.stream(st):
            for _ in range(4):
                a.copy_(a @ a / 80.0)
    want_tab, want_len = [], []
    for u in range(uploads):
        P.pkv_append_slots(eng.pool, ids)
        t = np.full((n, mb), -1, dtype=np.int32)
        for r, i in enumerate(ids):
            row = P.pkv_seq_table(eng.pool, i)
            t[r, :len(row)] = row
        want_tab.append(t)
        want_len.append(np.array([P.pkv_seq_length(eng.pool, i) for i in ids], dtype=np.int32))
        st = side if u % 3 == 1 else main
        P.pkv_sync_tables(eng.pool, ids, tabs[u], lens[u], stream=st)
    torch.cuda.synchronize()
    for u in range(uploads):
        assert np.array_equal(tabs[u].cpu().numpy(), want_tab[u]), f"upload {u}: tables"
        assert np.array_equal(lens[u].cpu().numpy(), want_len[u]), f"upload {u}: lengths"
