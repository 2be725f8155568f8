"""Seeded synthetic decode workloads shared by the tests and the benchmark.

This module only draws inputs: sequence lengths, pool permutations, the
script of allocator operations that builds each batch, and the query / key /
value tensors.  It holds none of the method's arithmetic (no slot, table or
attention computation); the CPU oracle and the HIP library each run the
script through their own allocator and kernels.

The five workloads follow the decode configurations the library is measured
on (tiny fp32 case, single-layer GQA batch, shared-prefix copy-on-write batch,
32K-token split-K batch, 32-layer MHA decode step).  Inputs are synthetic:
lengths from the stated distributions with ``numpy.random.default_rng(seed)``,
tensor values N(0, 1) drawn in fp32 by a seeded ``torch.Generator`` and
rounded to the storage dtype (round-to-nearest-even).

Script operations (ids are assigned 0, 1, 2, ... in create/fork order):

* ``("create",)``                      new empty sequence
* ``("extend", sid, k, src, pos)``     reserve k slots for ``sid``; their
  values are tokens ``pos .. pos+k-1`` of logical sequence ``src``
* ``("fork", parent)``                 child shares all of parent's blocks
* ``("free", sid)``                    release a sequence
* ``("append", [(sid, src, pos), ...])``  one new token for each listed id,
  in list order (the batched decode append)
* ``("release", sid, pos)``            sliding window: give back the blocks
  holding only positions < pos
* ``("window", sid, W)``               the same with pos = max(0, length - W)
* ``("register", sid, tokens, ns)``    enter sid's full blocks into the prefix
  cache under token ids ``tokens`` and namespace ``ns``
* ``("match", tokens, ns)``            new sequence from the cached chain
* ``("evict", k)`` / ``("clear",)``    prefix-cache eviction
* ``("register_stream", sid, stream, ns)`` / ``("match_stream", stream, n, ns)``
  the same with the token ids of a synthetic stream (``stream_tokens``)
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16  # tokens per block (page size)


@dataclasses.dataclass
class Workload:
    name: str
    layers: int
    Hq: int
    Hkv: int
    d: int
    dtype: str                 # "f32" or "bf16"
    lengths: np.ndarray        # attended length n_s of each checked sequence
    num_blocks: int
    perm: np.ndarray           # initial free-list order (a permutation)
    setup_ops: list            # builds the batch up to n_s - 1 tokens
    step_ops: list             # the checked decode append (one token each)
    seq_ids: List[int]         # pool id of checked sequence s
    seed: int
    block: int = BLOCK
    partition: int = 512
    description: str = ""
    kv_dtype: str = ""         # cache element type if it differs: "fp8" (E4M3 codes)
    chunk: Optional[np.ndarray] = None   # prefill: new tokens (queries) per sequence

    @property
    def S(self) -> int:
        return int(len(self.lengths))

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def offsets(self) -> np.ndarray:
        o = np.zeros(self.S + 1, dtype=np.int64)
        o[1:] = np.cumsum(self.lengths)
        return o

    @property
    def total_tokens(self) -> int:
        return int(self.lengths.sum())

    @property
    def max_len(self) -> int:
        return int(self.lengths.max())

    @property
    def chunk_lens(self) -> np.ndarray:
        """Queries per sequence: the prefill chunk, or 1 (the decode step)."""
        return self.chunk if self.chunk is not None else np.ones(self.S, dtype=np.int64)

    @property
    def query_offsets(self) -> np.ndarray:
        o = np.zeros(self.S + 1, dtype=np.int64)
        o[1:] = np.cumsum(self.chunk_lens)
        return o

    def prefill_queries(self, layer: int = 0, device="cpu"):
        """Queries of a prefill batch, [sum chunk][Hq][d], N(0,1) drawn in fp32
        from their own generator and rounded to the workload dtype."""
        import torch
        dt = torch.float32 if self.dtype == "f32" else torch.bfloat16
        g = torch.Generator(device=device)
        g.manual_seed(self.seed * 1000003 + 7919 + layer)
        return torch.randn((int(self.chunk_lens.sum()), self.Hq, self.d), generator=g, device=device,
                           dtype=torch.float32).to(dt)

    def prefill_flops(self, window: int = 0) -> int:
        """Multiply-adds x 2 of QK and PV over the causal pairs (query,
        key) of the chunk: 4 d Hq per pair."""
        pairs = 0
        for n, m in zip(self.lengths, self.chunk_lens):
            n, m = int(n), int(m)
            keys = np.arange(n - m, n) + 1                      # keys 0..p of query at p
            if window > 0:
                keys = np.minimum(keys, window)
            pairs += int(keys.sum())
        return 4 * self.d * self.Hq * pairs

    def kv_bytes_per_token_head(self) -> int:
        """K+V bytes of one token of one KV head in one layer (for the 8-bit
        cache: one byte per value plus a 4-byte scale, for K and for V)."""
        if self.cache_dtype == "fp8":
            return 2 * (self.d + 4)
        return 2 * self.d * self.itemsize

    def kv_bytes_per_layer(self) -> int:
        """Algorithmic K+V bytes one decode attention call reads."""
        return self.total_tokens * self.Hkv * self.kv_bytes_per_token_head()

    def tensors(self, layer: int = 0, device="cpu"):
        """(q [S][Hq][d], k_log [sum n][Hkv][d], v_log [sum n][Hkv][d]).

        Drawn N(0,1) in fp32 from a generator seeded by (seed, layer) on
        ``device`` and rounded to the workload dtype.  The same call on the
        same device always returns the same values.
        """
        import torch
        dt = torch.float32 if self.dtype == "f32" else torch.bfloat16
        g = torch.Generator(device=device)
        g.manual_seed(self.seed * 1000003 + layer)
        T = self.total_tokens
        q = torch.randn((self.S, self.Hq, self.d), generator=g, device=device,
                        dtype=torch.float32).to(dt)
        k = torch.randn((T, self.Hkv, self.d), generator=g, device=device,
                        dtype=torch.float32).to(dt)
        v = torch.randn((T, self.Hkv, self.d), generator=g, device=device,
                        dtype=torch.float32).to(dt)
        return q, k, v


def _pool_perm(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.permutation(n).astype(np.int32)


def _private_script(lengths: Sequence[int]):
    """Each checked sequence is its own pool sequence (ids 0..S-1)."""
    setup = [("create",) for _ in lengths]
    for s, n in enumerate(lengths):
        if n - 1 > 0:
            setup.append(("extend", s, int(n) - 1, s, 0))
    step = [("append", [(s, s, int(n) - 1) for s, n in enumerate(lengths)])]
    return setup, step, list(range(len(lengths)))


def _blocks_needed(lengths, block=BLOCK) -> int:
    return int(sum(-(-int(n) // block) for n in lengths))


def tiny(seed: int = 0) -> Workload:
    """1 layer, lengths {1,7,16,33}, B=16, 4 Q heads / 1 KV head, d=64,
    fp32, blocks drawn by a seeded permutation of a 32-block pool."""
    rng = np.random.default_rng(seed)
    lengths = np.array([1, 7, 16, 33], dtype=np.int64)
    setup, step, ids = _private_script(lengths)
    return Workload("tiny", 1, 4, 1, 64, "f32", lengths, 32, _pool_perm(rng, 32),
                    setup, step, ids, seed,
                    description="1 layer, S=4, n={1,7,16,33}, Hq=4, Hkv=1, d=64, fp32, 32-block pool")


def single_layer(seed: int = 1, S: int = 64, max_len: int = 4096) -> Workload:
    """64 sequences, lengths uniform in [1,4096], 32 Q / 8 KV heads, d=128,
    bf16, pool sized to 1.25x the blocks needed, random placement."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, max_len, size=S, endpoint=True).astype(np.int64)
    nb = math.ceil(1.25 * _blocks_needed(lengths))
    setup, step, ids = _private_script(lengths)
    return Workload("single_layer", 1, 32, 8, 128, "bf16", lengths, nb, _pool_perm(rng, nb),
                    setup, step, ids, seed,
                    description=f"1 layer, S={S}, n~U[1,{max_len}], Hq=32, Hkv=8, d=128, bf16")


def shared_prefix(seed: int = 2, S: int = 128, prefix: int = 1024, lo: int = 16,
                  hi: int = 512, private_copies: bool = False) -> Workload:
    """128 sequences sharing one 1024-token prefix by reference count, plus
    private suffixes uniform in [16,512]; 40 Q / 8 KV heads, d=128, bf16.

    With ``private_copies`` every sequence writes its own copy of the same
    prefix values instead (the twin the shared layout is checked against).
    Logical sequence s holds the prefix tokens at positions 0..prefix-1 in
    both forms; the shared form writes them once, from logical sequence 0.
    """
    rng = np.random.default_rng(seed)
    suffix = rng.integers(lo, hi, size=S, endpoint=True).astype(np.int64)
    lengths = prefix + suffix
    if private_copies:
        nb = math.ceil(1.25 * _blocks_needed(lengths))
        perm = _pool_perm(rng, nb)
        setup = [("create",) for _ in range(S)]
        for s in range(S):
            # prefix values are those of logical sequence 0 (identical for all)
            setup.append(("extend", s, prefix, 0, 0))
            if suffix[s] - 1 > 0:
                setup.append(("extend", s, int(suffix[s]) - 1, s, prefix))
        step = [("append", [(s, s, int(lengths[s]) - 1) for s in range(S)])]
        ids = list(range(S))
        name = "shared_prefix_private"
    else:
        nb = math.ceil(1.25 * (prefix // BLOCK + _blocks_needed(suffix)))
        perm = _pool_perm(rng, nb)
        setup = [("create",), ("extend", 0, prefix, 0, 0)]
        for s in range(S):
            setup.append(("fork", 0))
        for s in range(S):
            if suffix[s] - 1 > 0:
                setup.append(("extend", s + 1, int(suffix[s]) - 1, s, prefix))
        setup.append(("free", 0))
        step = [("append", [(s + 1, s, int(lengths[s]) - 1) for s in range(S)])]
        ids = [s + 1 for s in range(S)]
        name = "shared_prefix"
    return Workload(name, 1, 40, 8, 128, "bf16", lengths, nb, perm, setup, step, ids, seed,
                    description=f"1 layer, S={S}, shared {prefix}-token prefix + U[{lo},{hi}] suffix, "
                                f"Hq=40, Hkv=8, d=128, bf16" + (", private copies" if private_copies else ""))


def long_context(seed: int = 3, S: int = 16, n: int = 32768) -> Workload:
    """16 sequences of 32768 tokens, 64 Q / 8 KV heads, d=128, bf16, random
    physical block order, 512-token split-K partitions."""
    rng = np.random.default_rng(seed)
    lengths = np.full(S, n, dtype=np.int64)
    nb = math.ceil(1.25 * _blocks_needed(lengths))
    setup, step, ids = _private_script(lengths)
    return Workload("long_context", 1, 64, 8, 128, "bf16", lengths, nb, _pool_perm(rng, nb),
                    setup, step, ids, seed,
                    description=f"1 layer, S={S}, n={n}, Hq=64, Hkv=8, d=128, bf16, 512-token partitions")


def full_step(seed: int = 4, S: int = 256, layers: int = 32, mean: float = 500.0,
              cap: int = 8192) -> Workload:
    """32 layers, 256 sequences, context geometric with mean 500 capped at
    8192, 32 Q / 32 KV heads (MHA), d=128, bf16; the decode step appends one
    token per sequence and attends over context + 1."""
    rng = np.random.default_rng(seed)
    ctx = np.minimum(rng.geometric(1.0 / mean, size=S), cap).astype(np.int64)
    lengths = ctx + 1
    nb = math.ceil(1.25 * _blocks_needed(lengths))
    setup, step, ids = _private_script(lengths)
    return Workload("full_step", layers, 32, 32, 128, "bf16", lengths, nb, _pool_perm(rng, nb),
                    setup, step, ids, seed,
                    description=f"{layers} layers, S={S}, context~min(Geom(1/{mean:g}),{cap})+1, "
                                f"Hq=Hkv=32, d=128, bf16")


def random_small(seed: int, S: int, Hq: int, Hkv: int, d: int, dtype: str,
                 max_len: int, min_len: int = 1, slack: float = 1.25) -> Workload:
    """A small randomized private-sequence workload for edge-case tests."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(min_len, max_len, size=S, endpoint=True).astype(np.int64)
    nb = max(1, math.ceil(slack * _blocks_needed(lengths)))
    setup, step, ids = _private_script(lengths)
    return Workload(f"random_{seed}", 1, Hq, Hkv, d, dtype, lengths, nb, _pool_perm(rng, nb),
                    setup, step, ids, seed,
                    description=f"S={S}, n~U[{min_len},{max_len}], Hq={Hq}, Hkv={Hkv}, d={d}, {dtype}")


def with_lengths(lengths, Hq: int, Hkv: int, d: int, dtype: str, seed: int = 7,
                 slack: float = 1.25) -> Workload:
    """Private sequences with the given attended lengths."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    nb = max(1, math.ceil(slack * _blocks_needed(lengths)))
    setup, step, ids = _private_script(lengths)
    return Workload(f"lengths_{seed}", 1, Hq, Hkv, d, dtype, lengths, nb, _pool_perm(rng, nb),
                    setup, step, ids, seed,
                    description=f"S={len(lengths)}, n={list(map(int, lengths))[:8]}..., Hq={Hq}, Hkv={Hkv}, d={d}, {dtype}")


def prefill_chunks(contexts, chunks, Hq: int, Hkv: int, d: int, dtype: str = "bf16", seed: int = 11,
                   slack: float = 1.25, name: str = "prefill") -> Workload:
    """Sequence s holds contexts[s] cached tokens and receives chunks[s] new
    ones, whose K/V are appended (one extend each) before the chunk's
    queries attend causally to everything up to themselves."""
    rng = np.random.default_rng(seed)
    contexts = np.asarray(contexts, dtype=np.int64)
    chunks = np.asarray(chunks, dtype=np.int64)
    lengths = contexts + chunks
    nb = max(1, math.ceil(slack * _blocks_needed(lengths)))
    setup = [("create",) for _ in lengths]
    for s, c in enumerate(contexts):
        if c > 0:
            setup.append(("extend", s, int(c), s, 0))
    step = [("extend", s, int(m), s, int(c)) for s, (c, m) in enumerate(zip(contexts, chunks))]
    return Workload(name, 1, Hq, Hkv, d, dtype, lengths, nb, _pool_perm(rng, nb), setup, step,
                    list(range(len(lengths))), seed, chunk=chunks,
                    description=f"prefill S={len(lengths)}, context={list(map(int, contexts))[:6]}, "
                                f"chunk={list(map(int, chunks))[:6]}, Hq={Hq}, Hkv={Hkv}, d={d}, {dtype}")


def prefill_prompts(seed: int = 12) -> Workload:
    """8 prompts of 4096 tokens each prefilled from an empty cache, 32 query /
    8 KV heads, d = 128, bf16 (the prefill measured for throughput)."""
    return prefill_chunks([0] * 8, [4096] * 8, 32, 8, 128, "bf16", seed, name="prefill_prompts")


def prefill_chunked(seed: int = 13) -> Workload:
    """8 sequences with 8192 cached tokens each taking a 1024-token chunk,
    32 query / 8 KV heads, d = 128, bf16 (chunked prefill over a cache)."""
    return prefill_chunks([8192] * 8, [1024] * 8, 32, 8, 128, "bf16", seed, name="prefill_chunked")


def fp8_cache(wl: Workload) -> Workload:
    """The same workload with an 8-bit (E4M3) KV cache: the same bf16 input
    values, quantised per (token, head) row when they are written."""
    if wl.dtype != "bf16":
        raise ValueError("the 8-bit cache takes bf16 tokens and queries")
    return dataclasses.replace(wl, name=wl.name + "_fp8", kv_dtype="fp8",
                               description=wl.description + ", fp8 (e4m3) KV cache")


CONFIGS = {
    "tiny": tiny,
    "single_layer": single_layer,
    "shared_prefix": shared_prefix,
    "long_context": long_context,
    "full_step": full_step,
    "long_context_fp8": lambda seed=3, **kw: fp8_cache(long_context(seed, **kw)),
    "full_step_fp8": lambda seed=4, **kw: fp8_cache(full_step(seed, **kw)),
    "prefill_prompts": prefill_prompts,
    "prefill_chunked": prefill_chunked,
    "prefill_prompts_fp8": lambda seed=12, **kw: fp8_cache(prefill_prompts(seed, **kw)),
    "prefill_chunked_fp8": lambda seed=13, **kw: fp8_cache(prefill_chunked(seed, **kw)),
}


def stream_tokens(stream: int, n: int) -> List[int]:
    """Synthetic token ids: stream k shares its first 12·(k + 1) tokens with
    every other stream, then continues with ids of its own."""
    shared = 12 * (stream + 1)
    return [p % 97 if p < shared else 1000 * (stream + 1) + p for p in range(n)]


def random_op_script(seed: int, n_ops: int, max_live: int = 12, max_extend: int = 40, windows: bool = False,
                     prefix: bool = False):
    """A random allocator-only script (no tensor values) for allocator tests:
    create / extend / fork / free / batched append (and, with ``windows``,
    sliding-window releases), ids valid at issue time."""
    rng = np.random.default_rng(seed)
    ops = []
    live: List[int] = []
    next_id = 0
    for _ in range(n_ops):
        r = rng.random()
        if r < 0.12 or not live:
            ops.append(("create",))
            live.append(next_id)
            next_id += 1
        elif r < 0.40:
            sid = int(rng.choice(live))
            ops.append(("extend", sid, int(rng.integers(0, max_extend + 1)), 0, 0))
        elif r < 0.52 and len(live) < max_live:
            p = int(rng.choice(live))
            ops.append(("fork", p))
            live.append(next_id)
            next_id += 1
        elif r < 0.64:
            sid = int(rng.choice(live))
            ops.append(("free", sid))
            live.remove(sid)
        elif windows and r < 0.74:
            ops.append(("window", int(rng.choice(live)), int(rng.integers(0, 3 * max_extend))))
        elif prefix and r < 0.84:
            q = rng.random()
            ns = int(rng.integers(0, 2))
            if q < 0.4:
                ops.append(("register_stream", int(rng.choice(live)), int(rng.integers(0, 4)), ns))
            elif q < 0.75 and len(live) < max_live:
                ops.append(("match_stream", int(rng.integers(0, 4)), int(rng.integers(0, 3 * max_extend)), ns))
                live.append(next_id)
                next_id += 1
            elif q < 0.95:
                ops.append(("evict", int(rng.integers(0, 6))))
            else:
                ops.append(("clear",))
        else:
            k = int(rng.integers(1, len(live) + 1))
            ids = [int(x) for x in rng.choice(live, size=k, replace=False)]
            ops.append(("append", [(i, 0, 0) for i in ids]))
    return ops
