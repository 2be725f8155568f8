"""Pins of the oracle's paged gather + fp64 attention.

Each check fixes the oracle to something other than itself: pure-Python
brute force on the unpaged logical tensors, torch's scaled-dot-product
attention in fp64, closed-form special cases, scipy's softmax on extreme
logits, and invariances the pages state (placement does not change meaning;
shared and copied prefixes give the same result; forks are isolated).
"""
import math

import numpy as np
import pytest
import torch

import workloads
from helpers import bits, brute_force, oracle_run
from oracle import attention as OA
from oracle.allocator import Allocator
from oracle.pool import Pool, to_f64
from oracle.replay import Replay


def _small_cases():
    return [
        workloads.tiny(),
        workloads.random_small(11, S=3, Hq=6, Hkv=2, d=16, dtype="bf16", max_len=40),
        workloads.random_small(12, S=2, Hq=5, Hkv=5, d=8, dtype="f32", max_len=35),
        workloads.random_small(13, S=2, Hq=8, Hkv=1, d=16, dtype="bf16", max_len=20),
    ]


@pytest.mark.parametrize("wl", _small_cases(), ids=lambda w: w.description)
def test_brute_force(wl):
    q, k, v = wl.tensors()
    _, out = oracle_run(wl, q, k, v)
    ref = brute_force(wl, q, k, v)
    assert np.max(np.abs(out - ref)) <= 1e-13


@pytest.mark.parametrize("seed", range(3))
def test_sdpa_fp64(seed):
    wl = workloads.random_small(20 + seed, S=4, Hq=12, Hkv=4, d=32, dtype="bf16", max_len=200)
    q, k, v = wl.tensors()
    _, out = oracle_run(wl, q, k, v)
    offs = wl.offsets
    G = wl.G
    for s in range(wl.S):
        ks = k[offs[s]:offs[s + 1]].to(torch.float64).transpose(0, 1)   # [Hkv][n][d]
        vs = v[offs[s]:offs[s + 1]].to(torch.float64).transpose(0, 1)
        ks = ks.repeat_interleave(G, dim=0).contiguous()
        vs = vs.repeat_interleave(G, dim=0).contiguous()
        qs = q[s].to(torch.float64)[:, None, :]                           # [Hq][1][d]
        ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs)[:, 0, :]
        assert np.max(np.abs(out[s] - ref.numpy())) <= 1e-12


def _pool_one(K, V, dtype="f32", block=4, perm=None):
    """One sequence of len(K) tokens, one KV head, written through the oracle."""
    n, d = K.shape
    nb = -(-n // block) + 2
    alloc = Allocator(nb, block, perm)
    sid = alloc.create()
    slots, _ = alloc.extend(sid, n)
    pool = Pool(nb, 1, d, dtype, block)
    t = torch.tensor(K, dtype=torch.float32)[:, None, :]
    u = torch.tensor(V, dtype=torch.float32)[:, None, :]
    pool.scatter(0, slots, bits(t), bits(u))
    return pool, alloc.table(sid)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(0)
    K = rng.standard_normal((1, 8)).astype(np.float32)
    V = rng.standard_normal((1, 8)).astype(np.float32)
    pool, table = _pool_one(K, V)
    q = rng.standard_normal((1, 3, 8))
    out = OA.decode(pool, 0, [table], [1], q, 3)
    assert np.array_equal(out[0], np.repeat(V.astype(np.float64), 3, axis=0))


def test_zero_query_or_equal_keys_give_mean_value():
    rng = np.random.default_rng(1)
    n, d = 13, 8
    K = rng.standard_normal((n, d)).astype(np.float32)
    V = rng.standard_normal((n, d)).astype(np.float32)
    pool, table = _pool_one(K, V)
    out = OA.decode(pool, 0, [table], [n], np.zeros((1, 1, d)), 1)
    assert np.allclose(out[0, 0], V.astype(np.float64).mean(0), atol=1e-15, rtol=0)
    Keq = np.repeat(K[:1], n, axis=0)
    pool, table = _pool_one(Keq, V)
    out = OA.decode(pool, 0, [table], [n], rng.standard_normal((1, 1, d)), 1)
    assert np.allclose(out[0, 0], V.astype(np.float64).mean(0), atol=1e-15, rtol=0)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(2)
    n, d = 21, 8
    K = rng.standard_normal((n, d)).astype(np.float32) * 0.01
    V = rng.standard_normal((n, d)).astype(np.float32)
    K[9] = 0.0
    K[9, 0] = 1e4 * math.sqrt(d)      # q·k·scale ≈ 1e4 above the rest for q = e0
    pool, table = _pool_one(K, V)
    q = np.zeros((1, 1, d))
    q[0, 0, 0] = 1.0
    out = OA.decode(pool, 0, [table], [n], q, 1)
    assert np.array_equal(out[0, 0], V[9].astype(np.float64))


def test_extreme_logits_match_scipy_softmax():
    from scipy.special import softmax
    rng = np.random.default_rng(3)
    n, d = 40, 16
    K = rng.standard_normal((n, d)).astype(np.float32)
    V = rng.standard_normal((n, d)).astype(np.float32)
    pool, table = _pool_one(K, V)
    q = rng.standard_normal((1, 2, d)) * 3000.0     # logits of order ±1e4
    out = OA.decode(pool, 0, [table], [n], q, 2)
    assert np.all(np.isfinite(out))
    K64, V64 = K.astype(np.float64), V.astype(np.float64)
    for h in range(2):
        w = softmax(q[0, h] @ K64.T / math.sqrt(d))
        assert np.max(np.abs(out[0, h] - w @ V64)) <= 1e-12


@pytest.mark.parametrize("seed", range(8))
def test_online_softmax_equals_dense(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 600))
    d = 16
    q = rng.standard_normal((3, d))
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    dense = OA.attend(q, K, V, 1 / math.sqrt(d))
    for chunk in (1, 3, 16, 512, n):
        assert np.max(np.abs(OA.attend_online(q, K, V, 1 / math.sqrt(d), chunk) - dense)) <= 1e-15


@pytest.mark.parametrize("seed", range(8))
def test_split_merge_equals_dense(seed):
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(1, 1500))
    d = 16
    q = rng.standard_normal((4, d))
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    dense = OA.attend(q, K, V, 1 / math.sqrt(d))
    for part in (16, 512, n):
        assert np.max(np.abs(OA.attend_split(q, K, V, 1 / math.sqrt(d), part) - dense)) <= 1e-15


def test_permutation_invariance():
    wl = workloads.random_small(31, S=5, Hq=4, Hkv=2, d=16, dtype="bf16", max_len=70)
    q, k, v = wl.tensors()
    _, out1 = oracle_run(wl, q, k, v)
    wl.perm = np.random.default_rng(99).permutation(wl.num_blocks).astype(np.int32)
    rp2, out2 = oracle_run(wl, q, k, v)
    assert np.array_equal(out1, out2)


def test_shared_prefix_equals_private_copies():
    kw = dict(seed=5, S=6, prefix=48, lo=16, hi=40)
    shared = workloads.shared_prefix(**kw)
    private = workloads.shared_prefix(private_copies=True, **kw)
    shared.Hq, shared.Hkv, shared.d = private.Hq, private.Hkv, private.d = 4, 2, 16
    q, k, v = shared.tensors()
    # logical sequence s carries the prefix of logical sequence 0 in both forms
    offs = shared.offsets
    for s in range(1, shared.S):
        k[offs[s]:offs[s] + 48] = k[0:48]
        v[offs[s]:offs[s] + 48] = v[0:48]
    rps, out_s = oracle_run(shared, q, k, v)
    rpp, out_p = oracle_run(private, q, k, v)
    assert np.array_equal(out_s, out_p)
    # the shared form really shares: 3 prefix blocks with refcount S
    t0 = rps.tables()[0][:3]
    assert all(rps.alloc.ref[b] == shared.S for b in t0)
    assert all(rps.tables()[s][:3] == t0 for s in range(shared.S))


def test_fork_isolation():
    """After a fork inside a block, each side's appends stay private."""
    d, B = 8, 4
    rng = np.random.default_rng(4)
    alloc = Allocator(10, B)
    pool = Pool(10, 1, d, "f32", B)
    tok = lambda n: torch.tensor(rng.standard_normal((n, 1, d)), dtype=torch.float32)
    p = alloc.create()
    kv = tok(6), tok(6)
    slots, _ = alloc.extend(p, 6)
    pool.scatter(0, slots, bits(kv[0]), bits(kv[1]))
    c = alloc.fork(p)
    q = rng.standard_normal((1, 1, d))
    before = OA.decode(pool, 0, [alloc.table(p)], [6], q, 1)
    kc, vc = tok(1), tok(1)
    slots, cow = alloc.append([c])
    assert len(cow) == 1
    for a, b in cow:
        pool.copy_block(a, b)
    pool.scatter(0, slots, bits(kc), bits(vc))
    after = OA.decode(pool, 0, [alloc.table(p)], [alloc.length(p)], q, 1)
    assert np.array_equal(before, after)          # parent unaffected by child write
    kp, vp = tok(1), tok(1)
    slots, cow = alloc.append([p])
    assert cow == []                               # parent now sole holder
    pool.scatter(0, slots, bits(kp), bits(vp))
    Kc, Vc = pool.gather(0, alloc.table(c), 7, 0)
    assert np.array_equal(Kc[6], kc.double().numpy()[0, 0])
    assert np.array_equal(Kc[:6], kv[0].double().numpy()[:, 0])
    Kp, _ = pool.gather(0, alloc.table(p), 7, 0)
    assert np.array_equal(Kp[6], kp.double().numpy()[0, 0])


def test_pool_layout_bytes():
    """The documented layout: K element j of slot o at [blk][h][j//x][o][j%x],
    V element j at [blk][h][o//4][j//4][j%4][o%4] (x = 8 for bf16)."""
    d, B = 16, 4
    pool = Pool(3, 2, d, "bf16", B)
    k = torch.arange(2 * d, dtype=torch.float32).reshape(1, 2, d).to(torch.bfloat16)
    v = (torch.arange(2 * d, dtype=torch.float32) + 100).reshape(1, 2, d).to(torch.bfloat16)
    pool.scatter(0, [2 * B + 3], bits(k), bits(v))     # block 2, slot 3
    K, V = pool.K[0], pool.V[0]
    kb, vb = bits(k), bits(v)
    for h in range(2):
        for j in range(d):
            assert K[2, h, j // 8, 3, j % 8] == kb[0, h, j]
            assert V[2, h, 0, j // 4, j % 4, 3] == vb[0, h, j]
    flatK = K.reshape(-1)
    # byte offset of element (blk 2, h 1, j 11, slot 3) in the flat K array
    off = (((2 * 2 + 1) * (d // 8) + 11 // 8) * B + 3) * 8 + 11 % 8
    assert flatK[off] == kb[0, 1, 11]
    # and in the flat V array: four columns of four tokens per 16 values
    flatV = V.reshape(-1)
    off = ((((2 * 2 + 1) * (B // 4) + 3 // 4) * (d // 4) + 11 // 4) * 4 + 11 % 4) * 4 + 3 % 4
    assert flatV[off] == vb[0, 1, 11]
    assert np.all(K[0] == 0x7FC0) and np.all(V[1] == 0x7FC0)
