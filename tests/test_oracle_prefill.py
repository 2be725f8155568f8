"""Pins of the chunked (paged) prefill oracle: causal attention of each new
token over its sequence's positions up to itself, through the block table."""
import math

import numpy as np
import pytest
import torch

import workloads
from helpers import bits
from oracle import attention as OA
from oracle.pool import to_f64
from oracle.replay import Replay


def run_prefill(wl, window=0):
    q = wl.prefill_queries()
    _, k, v = wl.tensors()
    rp = Replay(wl).run(wl.setup_ops + wl.step_ops, {0: (bits(k), bits(v))})
    out = OA.prefill(rp.pool, 0, rp.tables(), rp.lengths(), wl.chunk_lens, to_f64(bits(q), wl.dtype), wl.Hq,
                     window=window)
    return rp, q, k, v, out


def brute(wl, q, k, v, window=0):
    """Pure-Python loops over the logical tensors."""
    G = wl.Hq // wl.Hkv
    d = wl.d
    qq, kk, vv = (t.to(torch.float64).tolist() for t in (q, k, v))
    offs, qoffs = wl.offsets, wl.query_offsets
    out = []
    for s in range(wl.S):
        n, m = int(wl.lengths[s]), int(wl.chunk_lens[s])
        for i in range(m):
            p = n - m + i
            lo = max(0, p - window + 1) if window > 0 else 0
            row = []
            for h in range(wl.Hq):
                g = h // G
                sc = [sum(qq[qoffs[s] + i][h][j] * kk[offs[s] + t][g][j] for j in range(d)) / math.sqrt(d)
                      for t in range(lo, p + 1)]
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                z = sum(w)
                row.append([sum(w[t - lo] * vv[offs[s] + t][g][j] for t in range(lo, p + 1)) / z
                            for j in range(d)])
            out.append(row)
    return np.array(out)


@pytest.mark.parametrize("window", [0, 1, 7, 20])
def test_prefill_matches_brute_force(window):
    wl = workloads.prefill_chunks([0, 5, 19], [9, 12, 6], Hq=4, Hkv=2, d=16, seed=3)
    rp, q, k, v, out = run_prefill(wl, window)
    assert np.max(np.abs(out - brute(wl, q, k, v, window))) <= 1e-13


def test_whole_prompt_matches_causal_sdpa():
    """Context 0: the library routine's causal attention (fp64, K/V repeated
    over the query-head groups)."""
    wl = workloads.prefill_chunks([0, 0], [70, 33], Hq=6, Hkv=2, d=32, seed=4)
    rp, q, k, v, out = run_prefill(wl)
    G = wl.Hq // wl.Hkv
    for s in range(wl.S):
        a, b = wl.query_offsets[s], wl.query_offsets[s + 1]
        ka, kb = wl.offsets[s], wl.offsets[s + 1]
        Q = q[a:b].double().transpose(0, 1)                              # [Hq][m][d]
        K = k[ka:kb].double().transpose(0, 1).repeat_interleave(G, 0)    # [Hq][n][d]
        V = v[ka:kb].double().transpose(0, 1).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
        assert np.max(np.abs(out[a:b] - ref.transpose(0, 1).numpy())) <= 1e-12


def test_chunk_equals_rows_of_whole_prompt():
    """Prefilling [c, n) over a cached context gives the rows c..n-1 of
    prefilling [0, n) at once (up to BLAS rounding order)."""
    whole = workloads.prefill_chunks([0], [90], Hq=4, Hkv=1, d=16, seed=5)
    _, q, _, _, out_whole = run_prefill(whole)
    part = workloads.prefill_chunks([61], [29], Hq=4, Hkv=1, d=16, seed=5)
    qp = q[61:]
    _, k, v = part.tensors()
    rp = Replay(part).run(part.setup_ops + part.step_ops, {0: (bits(k), bits(v))})
    out = OA.prefill(rp.pool, 0, rp.tables(), rp.lengths(), part.chunk_lens, to_f64(bits(qp), "bf16"), 4)
    assert np.max(np.abs(out - out_whole[61:])) <= 1e-15


def test_single_new_token_is_decode():
    wl = workloads.prefill_chunks([40, 0, 77], [1, 1, 1], Hq=8, Hkv=2, d=32, seed=6)
    rp, q, k, v, out = run_prefill(wl)
    dec = OA.decode(rp.pool, 0, rp.tables(), rp.lengths(), to_f64(bits(q), "bf16"), wl.Hq)
    assert np.max(np.abs(out - dec)) <= 1e-15       # same formula; only BLAS blocking differs


def test_first_query_of_empty_context_returns_its_value():
    wl = workloads.prefill_chunks([0], [5], Hq=2, Hkv=1, d=16, seed=7)
    rp, q, k, v, out = run_prefill(wl)
    assert np.array_equal(out[0, 0], v[0, 0].double().numpy())
    assert np.array_equal(out[0, 1], v[0, 0].double().numpy())


def test_prefill_flops_count():
    wl = workloads.prefill_chunks([3, 0], [2, 4], Hq=2, Hkv=1, d=8)
    # sequence 0: queries at 3, 4 see 4 + 5 keys; sequence 1: 1 + 2 + 3 + 4
    assert wl.prefill_flops() == 4 * 8 * 2 * (4 + 5 + 1 + 2 + 3 + 4)
    assert wl.prefill_flops(window=2) == 4 * 8 * 2 * (2 + 2 + 1 + 2 + 2 + 2)


def _torch_dequantized(x: torch.Tensor) -> torch.Tensor:
    """fp64 copy of bf16 rows [..][d] as an 8-bit cache holds them, through
    torch: per-row fp32 scale amax/448, codes by torch's E4M3 conversion."""
    x32 = x.to(torch.float32)
    s = x32.abs().amax(dim=-1, keepdim=True) / torch.tensor(448.0, dtype=torch.float32)
    y = torch.where(s > 0, x32 / torch.where(s > 0, s, torch.ones_like(s)), torch.zeros_like(x32))
    return y.to(torch.float8_e4m3fn).to(torch.float64) * s.to(torch.float64)


@pytest.mark.parametrize("window", [0, 7])
def test_prefill_over_8bit_cache_matches_brute_force(window):
    """The prefill oracle over an 8-bit pool is exact attention over the
    dequantised cache: brute force on K/V quantised by torch."""
    wl = workloads.fp8_cache(workloads.prefill_chunks([0, 5, 19], [9, 12, 6], Hq=4, Hkv=2, d=64, seed=4))
    rp, q, k, v, out = run_prefill(wl, window)
    ref = brute(wl, q, _torch_dequantized(k), _torch_dequantized(v), window)
    assert np.max(np.abs(out - ref)) <= 1e-13
