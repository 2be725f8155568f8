"""Exact decode attention in fp64 (oracle; test infrastructure only).

«Servicio…presupuesto de memoria» §6 ("La atención exacta sigue teniendo un contrato numérico"): dense
attention forms scaled query-key scores, applies softmax and weights the
values; an IO-aware implementation may process blocks while carrying running
normalisation statistics, which changes the evaluation order, not the
operation.  «¿Cuánta memoria reservar para la caché KV?» ("Emplear las cabezas KV, en particular con GQA"): with
grouped-query attention several query heads share one KV head (e.g. 40 query
heads over 8 KV heads, five per group); the cache stores KV heads only.

Readings (where the pages are silent):
* sliding window («¿Cuánta memoria reservar para la caché KV?», "Adaptar…":
  windowed layers keep a bounded history): with window W > 0 the query of
  a sequence of length n attends to positions max(0, n - W) .. n - 1 only;
  W = 0 is full attention;
* score scale: 1/sqrt(d) by default, passed in explicitly;
* query head h uses KV head floor(h / G), G = Hq / Hkv (contiguous groups,
  the repeat-interleave convention);
* decode attends over every stored token of the sequence, the one just
  appended included; a sequence needs at least one token.
"""
from __future__ import annotations

import math

import numpy as np

from .pool import Pool, to_f64


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q Kᵀ · scale) V for query rows q [G][d], keys/values [n][d]."""
    X = (q @ K.T) * scale
    X = X - X.max(axis=1, keepdims=True)
    P = np.exp(X)
    return (P @ V) / P.sum(axis=1, keepdims=True)


def attend_online(q, K, V, scale: float, chunk: int) -> np.ndarray:
    """The same result computed chunk by chunk with running statistics:
    per query row a running maximum m, running sum l and an unnormalised
    accumulator, rescaled whenever the maximum grows («Servicio…presupuesto de memoria» §6, §9)."""
    G, d = q.shape
    m = np.full((G, 1), -np.inf)
    l = np.zeros((G, 1))
    acc = np.zeros((G, V.shape[1]))
    for lo in range(0, K.shape[0], chunk):
        X = (q @ K[lo:lo + chunk].T) * scale
        m_new = np.maximum(m, X.max(axis=1, keepdims=True))
        alpha = np.exp(m - m_new)
        P = np.exp(X - m_new)
        l = l * alpha + P.sum(axis=1, keepdims=True)
        acc = acc * alpha + P @ V[lo:lo + chunk]
        m = m_new
    return acc / l


def partial_stats(q, K, V, scale: float):
    """(m, l, acc) of one partition: max score, sum of exp(score - m) and the
    unnormalised exp-weighted value sum."""
    X = (q @ K.T) * scale
    m = X.max(axis=1, keepdims=True)
    P = np.exp(X - m)
    return m, P.sum(axis=1, keepdims=True), P @ V


def merge_stats(parts) -> np.ndarray:
    """Combine per-partition (m, l, acc): rescale every partition to the
    common maximum, then divide the summed accumulators by the summed sums."""
    M = np.max(np.concatenate([p[0] for p in parts], axis=1), axis=1, keepdims=True)
    L = sum(p[1] * np.exp(p[0] - M) for p in parts)
    A = sum(p[2] * np.exp(p[0] - M) for p in parts)
    return A / L


def attend_split(q, K, V, scale: float, part: int) -> np.ndarray:
    """Split the keys into partitions of ``part`` tokens, summarise each
    independently and merge the summaries."""
    parts = [partial_stats(q, K[lo:lo + part], V[lo:lo + part], scale)
             for lo in range(0, K.shape[0], part)]
    return merge_stats(parts)


def decode(pool: Pool, layer: int, tables, lengths, q: np.ndarray, Hq: int,
           scale: float = None, heads=None, window: int = 0) -> np.ndarray:
    """out[s][h] = attention of query head h of sequence s over the sequence's
    gathered keys/values of KV head floor(h/G) (the last ``window`` of them
    when window > 0).

    ``q`` is float64 [S][Hq][d] (already upcast).  ``heads`` optionally limits
    the (s, h) pairs computed; others are left NaN.
    """
    S = len(lengths)
    d = pool.d
    G = Hq // pool.Hkv
    if Hq % pool.Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.full((S, Hq, d), np.nan)
    for s in range(S):
        n = int(lengths[s])
        if n < 1:
            raise ValueError("a sequence needs at least one token")
        for g in range(pool.Hkv):
            hs = [h for h in range(g * G, (g + 1) * G) if heads is None or (s, h) in heads]
            if not hs:
                continue
            start = max(0, n - window) if window > 0 else 0
            Kc, Vc = pool.gather(layer, tables[s], n, g, start=start)
            out[s, hs] = attend(q[s, hs], Kc, Vc, scale)
    return out


def prefill(pool: Pool, layer: int, tables, lengths, chunk_lens, q: np.ndarray, Hq: int,
            scale: float = None, window: int = 0, rows=None) -> np.ndarray:
    """Chunked (paged) prefill: the last ``chunk_lens[s]`` of the
    ``lengths[s]`` tokens of sequence s are new, and each is a query.  Query
    i of sequence s sits at position p = lengths[s] - chunk_lens[s] + i and
    attends causally to positions 0 .. p (the last ``window`` of them when
    window > 0), through the block table.  With one new token this is the
    decode step.

    «Servicio…presupuesto de memoria» §6: exact attention — scaled scores,
    softmax, weighted values; «…» §2 and §4: prefill work has another shape
    than decode steps (many queries at once).

    ``q`` is float64 [T][Hq][d], T = sum(chunk_lens), the rows of sequence s
    after those of sequences 0 .. s-1.  Returns float64 [T][Hq][d];
    ``rows`` optionally limits the (row, head) pairs computed (others NaN).
    """
    d = pool.d
    G = Hq // pool.Hkv
    if Hq % pool.Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    T = int(sum(chunk_lens))
    out = np.full((T, Hq, d), np.nan)
    r0 = 0
    for s, (n, m) in enumerate(zip(lengths, chunk_lens)):
        n, m = int(n), int(m)
        if m < 1 or m > n:
            raise ValueError("a chunk holds 1 .. length tokens")
        c = n - m
        pos = c + np.arange(m)                                 # query positions
        lo = pos - window + 1 if window > 0 else np.zeros(m, dtype=np.int64)
        start = int(max(0, lo.min()))
        keys = np.arange(start, n)
        allowed = (keys[None, :] <= pos[:, None]) & (keys[None, :] >= lo[:, None])
        for g in range(pool.Hkv):
            todo = {}
            for h in range(g * G, (g + 1) * G):
                idx = np.arange(m) if rows is None else np.array(
                    [i for i in range(m) if (r0 + i, h) in rows], dtype=np.int64)
                if idx.size:
                    todo[h] = idx
            if not todo:
                continue
            Kc, Vc = pool.gather(layer, tables[s], n, g, start=start)
            for h, idx in todo.items():
                X = (q[r0 + idx, h] @ Kc.T) * scale
                X = np.where(allowed[idx], X, -np.inf)
                X = X - X.max(axis=1, keepdims=True)
                P = np.exp(X)
                out[r0 + idx, h] = (P @ Vc) / P.sum(axis=1, keepdims=True)
        r0 += m
    return out

