"""GPU parity of chunked paged prefill: the chunk's K/V are appended through
the library, then every new token attends causally over its sequence through
the block table; compared with the oracle's prefill on the same inputs."""
import numpy as np
import pytest
import torch

import workloads
from gpu_common import check_allocator, check_pool, need_gpu, note, oracle_replay, run_gpu
from helpers import bits
from oracle import attention as OA
from oracle.pool import to_f64

pytestmark = pytest.mark.gpu

ATOL = 2e-2
ROW_RTOL = 1e-2


def compare(out, ref, rows=None):
    g = out.detach().float().cpu().double().numpy()
    if rows is not None:
        g = np.stack([g[r, h] for r, h in rows])
        ref = np.stack([ref[r, h] for r, h in rows])
    g = g.reshape(-1, g.shape[-1])
    ref = ref.reshape(-1, ref.shape[-1])
    assert np.all(np.isfinite(g)), "non-finite output"
    err = np.abs(g - ref)
    row_rel = float((err.max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-300)).max())
    assert err.max() <= ATOL, f"max abs err {err.max()}"
    assert row_rel <= ROW_RTOL, f"row-normwise rel err {row_rel}"
    return float(err.max()), row_rel


def run_prefill_case(wl, window=0, rows=None, check_state=True):
    need_gpu()
    note(f"prefill window={window}: {wl.description}")
    _, k, v = wl.tensors(device="cuda")
    q = wl.prefill_queries(device="cuda")
    eng, log, _ = run_gpu(wl, {0: k}, {0: v})
    out = eng.prefill(0, q, list(map(int, wl.chunk_lens)), max_seq_len=wl.max_len, window=window)
    torch.cuda.synchronize()
    rp = oracle_replay(wl, {0: k}, {0: v})
    if check_state:
        check_allocator(eng, rp, log)
        check_pool(eng, rp)
    ref = OA.prefill(rp.pool, 0, rp.tables(), rp.lengths(), wl.chunk_lens, to_f64(bits(q.cpu()), wl.dtype), wl.Hq,
                     window=window, rows=None if rows is None else set(rows))
    e = compare(out, ref, rows)
    note(f"  max_abs={e[0]:.3e} row_rel={e[1]:.3e}")
    return eng, out


CASES = [
    # contexts, chunks, Hq, Hkv, d
    ([0], [1], 8, 2, 128),
    ([0], [64], 8, 2, 128),
    ([0, 5, 100], [17, 64, 130], 8, 2, 128),
    ([300, 0, 1000], [257, 500, 33], 32, 8, 128),
    ([7, 0], [190, 77], 16, 16, 128),            # MHA: 256 rows = 256 positions per workgroup
    ([0, 40], [300, 61], 64, 8, 128),            # 8 heads per KV head
    ([33, 0], [100, 129], 40, 8, 128),           # 5 heads per KV head (rows straddle positions)
    ([0, 12], [150, 70], 8, 1, 64),              # d = 64
    ([1023, 64], [1, 1], 8, 2, 128),             # decode-shaped chunks
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}x{c[3]}x{c[4]}")
def test_prefill_parity(case):
    contexts, chunks, Hq, Hkv, d = case
    wl = workloads.prefill_chunks(contexts, chunks, Hq, Hkv, d, seed=sum(chunks) + Hq)
    run_prefill_case(wl)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}x{c[3]}x{c[4]}")
def test_prefill_parity_8bit_cache(case):
    """The same batches over an 8-bit (E4M3) cache: the call dequantises the
    blocks the sequences hold into a bf16 copy, then attends; compared with
    exact attention over the dequantised cache (codes and scales bit-exact
    with the oracle's pool)."""
    contexts, chunks, Hq, Hkv, d = case
    wl = workloads.fp8_cache(workloads.prefill_chunks(contexts, chunks, Hq, Hkv, d, seed=sum(chunks) + Hq + 1))
    run_prefill_case(wl)


@pytest.mark.parametrize("window", [16, 65, 200])
def test_prefill_window_8bit_cache(window):
    wl = workloads.fp8_cache(workloads.prefill_chunks([0, 90, 500], [150, 70, 129], 16, 4, 128, seed=window + 1))
    run_prefill_case(wl, window=window)


def test_prefill_bad_block_gives_nan_rows_8bit_cache():
    need_gpu()
    wl = workloads.fp8_cache(workloads.prefill_chunks([64, 64], [40, 40], 8, 2, 128, seed=12))
    _, k, v = wl.tensors(device="cuda")
    q = wl.prefill_queries(device="cuda")
    eng, _, _ = run_gpu(wl, {0: k}, {0: v})
    eng.tables[1, 2] = wl.num_blocks              # sequence 1 reads a block outside the pool
    out = eng.prefill(0, q, [40, 40], max_seq_len=wl.max_len)
    torch.cuda.synchronize()
    assert torch.isnan(out[40:].float()).all()
    assert torch.isfinite(out[:40].float()).all()


@pytest.mark.parametrize("window", [1, 16, 63, 64, 65, 200])
def test_prefill_window(window):
    wl = workloads.prefill_chunks([0, 90, 500], [150, 70, 129], 16, 4, 128, seed=window)
    run_prefill_case(wl, window=window)


def test_prefill_single_token_matches_decode_kernel():
    """m = 1 is a decode step: the prefill kernel and the decode kernel agree
    within the tolerance on the same cache (different reduction orders)."""
    need_gpu()
    wl = workloads.prefill_chunks([100, 0, 700], [1, 1, 1], 16, 4, 128, seed=3)
    eng, out = run_prefill_case(wl)
    q = wl.prefill_queries(device="cuda")
    dec = eng.decode(0, q, max_seq_len=wl.max_len)
    torch.cuda.synchronize()
    assert (out.float() - dec.float()).abs().max().item() <= 1e-2


def test_prefill_extreme_logits():
    need_gpu()
    wl = workloads.prefill_chunks([50, 0], [90, 70], 8, 2, 128, seed=9)
    _, k, v = wl.tensors(device="cuda")
    q = (wl.prefill_queries(device="cuda").float() * 3000.0).to(torch.bfloat16)
    eng, log, _ = run_gpu(wl, {0: k}, {0: v})
    out = eng.prefill(0, q, list(map(int, wl.chunk_lens)), max_seq_len=wl.max_len)
    torch.cuda.synchronize()
    rp = oracle_replay(wl, {0: k}, {0: v})
    ref = OA.prefill(rp.pool, 0, rp.tables(), rp.lengths(), wl.chunk_lens, to_f64(bits(q.cpu()), "bf16"), wl.Hq)
    compare(out, ref)


def test_prefill_permutation_keeps_bits():
    need_gpu()
    import dataclasses
    wl = workloads.prefill_chunks([200, 17], [300, 90], 32, 8, 128, seed=10)
    _, out1 = run_prefill_case(wl)
    wl2 = dataclasses.replace(wl, perm=np.random.default_rng(5).permutation(wl.num_blocks).astype(np.int32))
    _, out2 = run_prefill_case(wl2)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_prefill_bad_block_gives_nan_rows():
    need_gpu()
    wl = workloads.prefill_chunks([64, 64], [40, 40], 8, 2, 128, seed=11)
    _, k, v = wl.tensors(device="cuda")
    q = wl.prefill_queries(device="cuda")
    eng, _, _ = run_gpu(wl, {0: k}, {0: v})
    eng.tables[1, 2] = wl.num_blocks              # sequence 1 reads a block outside the pool
    out = eng.prefill(0, q, [40, 40], max_seq_len=wl.max_len)
    torch.cuda.synchronize()
    assert torch.isnan(out[40:].float()).all()
    assert torch.isfinite(out[:40].float()).all()


@pytest.mark.parametrize("name", ["prefill_prompts", "prefill_chunked", "prefill_chunked_fp8"])
def test_prefill_configs(name):
    """The measured prefill batches at full size: every query head of every
    sequence at the query positions around the kernel's boundaries — both
    ends of each chunk, 16-token cache blocks, 64-token K/V tiles, the
    workgroup's 384 (position, head) rows (96 positions at four heads per
    KV head) — plus random positions; pool and allocator exactly."""
    wl = workloads.CONFIGS[name]()
    G = wl.Hq // wl.Hkv
    per_wg = 384 // G
    rng = np.random.default_rng(0)
    rows = []
    r0 = 0
    for m in map(int, wl.chunk_lens):
        pos = {0, 1, m - 2, m - 1}
        for step in (16, 64, per_wg):
            for b in range(step, m, step * 7):           # a spread of boundaries, both sides
                pos |= {b - 1, b, b + 1}
            pos |= {m - step - 1, m - step}
        pos |= set(map(int, rng.integers(0, m, 8)))
        rows += [(r0 + i, h) for i in sorted(p for p in pos if 0 <= p < m) for h in range(wl.Hq)]
        r0 += m
    note(f"  {len(rows)} (row, head) pairs")
    run_prefill_case(wl, rows=rows, check_state=True)
