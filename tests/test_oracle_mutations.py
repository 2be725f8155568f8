"""Plant plausible mistakes in the oracle (on the CPU) and check a pin fails.

Each mutation is applied with monkeypatch to one oracle function; the named
pin must then raise.  This shows the pins are sensitive to a dropped term, a
wrong index, a transposed operand or a wrong allocator policy.
"""
import math

import numpy as np
import pytest

import test_oracle_accounting as T_acc
import test_oracle_allocator as T_alloc
import test_oracle_attention as T_att
import test_oracle_fp8 as T_fp8
import test_oracle_window as T_win
import test_oracle_prefill as T_pre
import workloads
from oracle import accounting, allocator, attention, fp8, pool


def _fails(fn, *args):
    with pytest.raises((AssertionError, FloatingPointError, ValueError, IndexError)):
        with np.errstate(all="ignore"):
            fn(*args)


def test_dropped_scale(monkeypatch):
    def attend(q, K, V, scale):
        X = q @ K.T
        X = X - X.max(axis=1, keepdims=True)
        P = np.exp(X)
        return (P @ V) / P.sum(axis=1, keepdims=True)
    monkeypatch.setattr(attention, "attend", attend)
    _fails(T_att.test_brute_force, workloads.tiny())


def test_wrong_shift_sign(monkeypatch):
    def attend(q, K, V, scale):
        X = (q @ K.T) * scale
        X = X + X.max(axis=1, keepdims=True)
        P = np.exp(X)
        return (P @ V) / P.sum(axis=1, keepdims=True)
    monkeypatch.setattr(attention, "attend", attend)
    _fails(T_att.test_extreme_logits_match_scipy_softmax)


def test_wrong_gqa_mapping(monkeypatch):
    orig = pool.Pool.gather

    def decode(pl, layer, tables, lengths, q, Hq, scale=None, heads=None, window=0):
        S, d = len(lengths), pl.d
        scale = 1 / math.sqrt(d) if scale is None else scale
        out = np.zeros((S, Hq, d))
        for s in range(S):
            for h in range(Hq):
                Kc, Vc = orig(pl, layer, tables[s], int(lengths[s]), h % pl.Hkv)
                out[s, h] = attention.attend(q[s, h:h + 1], Kc, Vc, scale)[0]
        return out
    monkeypatch.setattr(attention, "decode", decode)
    wl = workloads.random_small(11, S=3, Hq=6, Hkv=2, d=16, dtype="bf16", max_len=40)
    _fails(T_att.test_brute_force, wl)


def test_transposed_value_gather(monkeypatch):
    def gather(self, layer, table, n, head, start=0):
        nblk = -(-n // self.B)
        blocks = np.asarray(table[:nblk])
        kb = self.K[layer][blocks, head].transpose(0, 2, 1, 3).reshape(nblk * self.B, self.d)
        vb = self.V[layer][blocks, head].reshape(nblk * self.B, self.d)   # token and column order not swapped
        return pool.to_f64(kb[:n], self.dtype), pool.to_f64(vb[:n], self.dtype)
    monkeypatch.setattr(pool.Pool, "gather", gather)
    _fails(T_att.test_brute_force, workloads.tiny())


def test_off_by_one_block_index(monkeypatch):
    def scatter(self, layer, slots, k_bits, v_bits):
        self._materialize(layer)
        for i, slot in enumerate(slots):
            b, o = divmod(int(slot) + 1, self.B)
            if b >= self.N:
                b = 0
            self.K[layer][b, :, :, o, :] = k_bits[i].reshape(self.Hkv, self.d // self.x, self.x)
            self.V[layer][b, :, o // 4, :, :, o % 4] = v_bits[i].reshape(self.Hkv, self.d // 4, 4)
    monkeypatch.setattr(pool.Pool, "scatter", scatter)
    _fails(T_att.test_brute_force, workloads.random_small(11, S=3, Hq=6, Hkv=2, d=16, dtype="bf16", max_len=40))


def test_merge_without_rescale(monkeypatch):
    def merge(parts):
        return sum(p[2] for p in parts) / sum(p[1] for p in parts)
    monkeypatch.setattr(attention, "merge_stats", merge)
    _fails(T_att.test_split_merge_equals_dense, 3)


def test_online_without_rescale(monkeypatch):
    def online(q, K, V, scale, chunk):
        l = np.zeros((q.shape[0], 1))
        acc = np.zeros((q.shape[0], V.shape[1]))
        for lo in range(0, K.shape[0], chunk):
            X = (q @ K[lo:lo + chunk].T) * scale
            P = np.exp(X - X.max(axis=1, keepdims=True))
            l = l + P.sum(axis=1, keepdims=True)
            acc = acc + P @ V[lo:lo + chunk]
        return acc / l
    monkeypatch.setattr(attention, "attend_online", online)
    _fails(T_att.test_online_softmax_equals_dense, 0)


def test_fifo_free_list(monkeypatch):
    orig = allocator.Allocator.__init__

    def init(self, *a, **k):
        orig(self, *a, **k)
        self.free = list(reversed(self.free))       # pops now give perm[-1] first
    monkeypatch.setattr(allocator.Allocator, "__init__", init)
    _fails(T_alloc.test_golden_scenarios, "fork_cow_free_oom")


def test_no_copy_on_write(monkeypatch):
    def append_one(self, sid, cow):
        n, table = self.seqs[sid]
        if n % self.B == 0:
            if not self.free:
                raise allocator.NoBlocks()
            b = self.free.pop()
            self.ref[b] = 1
            table.append(b)
        slot = table[n // self.B] * self.B + n % self.B
        self.seqs[sid] = (n + 1, table)
        return slot
    monkeypatch.setattr(allocator.Allocator, "_append_one", append_one)
    _fails(T_alloc.test_golden_scenarios, "fork_cow_free_oom")
    _fails(T_att.test_fork_isolation)


def test_free_ignores_refcount(monkeypatch):
    def free_seq(self, sid):
        if sid not in self.seqs:
            raise allocator.BadSeq(sid)
        _, table = self.seqs.pop(sid)
        for b in table:
            self.ref[b] = 0
            if b not in self.free:
                self.free.append(b)
    monkeypatch.setattr(allocator.Allocator, "free_seq", free_seq)
    _fails(T_alloc.test_free_parent_keeps_children_blocks)


def test_dropped_factor_two(monkeypatch):
    monkeypatch.setattr(accounting, "kv_bytes_per_token", lambda L, H, d, b: L * H * d * b)
    _fails(T_acc.test_bytes_per_token, T_acc.GOLD["bytes_per_token"][0])


def test_floor_instead_of_ceil(monkeypatch):
    monkeypatch.setattr(accounting, "blocks_for", lambda T, B: T // B)
    _fails(T_acc.test_pages_for_500_tokens)


# -- 8-bit cache ---------------------------------------------------------------

def _fp8_case():
    return lambda: workloads.random_small(21, S=4, Hq=8, Hkv=2, d=64, dtype="bf16", max_len=70)


def test_fp8_ties_away_from_zero(monkeypatch):
    orig = fp8.encode

    def encode(y):
        y = np.asarray(y, dtype=np.float64)
        return orig(y + np.sign(y) * np.abs(y) * 2.0 ** -30)     # nudges every tie upwards
    monkeypatch.setattr(fp8, "encode", encode)
    _fails(T_fp8.test_encode_matches_library_rounding)


def test_fp8_scale_off_by_one(monkeypatch):
    def quantize_rows(x):
        x = np.asarray(x, dtype=np.float32)
        scale = (np.max(np.abs(x), axis=-1) / np.float32(447)).astype(np.float32)
        safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
        codes = np.where(scale[..., None] > 0, fp8.encode((x / safe[..., None]).astype(np.float32)), 0)
        return codes.astype(np.uint8), scale
    monkeypatch.setattr(fp8, "quantize_rows", quantize_rows)
    _fails(T_fp8.test_paged_fp8_attention_matches_brute_force, _fp8_case())


def test_fp8_value_columns_swapped(monkeypatch):
    orig = pool.Pool.gather

    def gather(self, layer, table, n, head, start=0):
        K, V = orig(self, layer, table, n, head, start)
        if self.dtype == "fp8":       # columns 4c + b read as 4b + c inside each group of 16
            V = V.reshape(V.shape[0], -1, 4, 4).transpose(0, 1, 3, 2).reshape(V.shape[0], -1)
        return K, V
    monkeypatch.setattr(pool.Pool, "gather", gather)
    _fails(T_fp8.test_paged_fp8_attention_matches_brute_force, _fp8_case())


def test_fp8_one_scale_per_block(monkeypatch):
    orig = pool.Pool.gather

    def gather(self, layer, table, n, head, start=0):
        K, V = orig(self, layer, table, n, head, start)
        if self.dtype == "fp8":       # every token scaled as its block's first one
            ks = self.KS[layer][np.asarray(table[:-(-n // self.B)]), head].view(np.float32).astype(np.float64)
            first = np.repeat(ks[:, :1], self.B, axis=1).reshape(-1)[:n]
            K = K / ks.reshape(-1)[:n, None] * first[:, None]
        return K, V
    monkeypatch.setattr(pool.Pool, "gather", gather)
    _fails(T_fp8.test_paged_fp8_attention_matches_brute_force, _fp8_case())


# -- sliding window --------------------------------------------------------------

def test_window_off_by_one(monkeypatch):
    orig = attention.decode

    def decode(*a, window=0, **k):
        return orig(*a, window=window + 1 if window > 0 else 0, **k)
    monkeypatch.setattr(attention, "decode", decode)
    _fails(T_win.test_window_matches_brute_force, 5)


def test_window_gather_from_block_start(monkeypatch):
    orig = pool.Pool.gather

    def gather(self, layer, table, n, head, start=0):       # starts at the window's block, not its token
        return orig(self, layer, table, n, head, start=(start // self.B) * self.B)
    monkeypatch.setattr(pool.Pool, "gather", gather)
    _fails(T_win.test_window_matches_brute_force, 5)


def test_window_release_keeps_one_block_too_many(monkeypatch):
    orig = allocator.Allocator.release_before

    def release_before(self, sid, pos):
        return orig(self, sid, max(0, pos - self.B))
    monkeypatch.setattr(allocator.Allocator, "release_before", release_before)
    _fails(T_alloc.test_golden_scenarios, "sliding_window_release")


# -- prefill -------------------------------------------------------------------

def _mutated_prefill(allowed_fn):
    """A prefill whose key mask is allowed_fn(keys, positions) (brute layout)."""
    def prefill(pool_, layer, tables, lengths, chunk_lens, q, Hq, scale=None, window=0, rows=None):
        d = pool_.d
        G = Hq // pool_.Hkv
        scale = 1 / math.sqrt(d) if scale is None else scale
        out = np.zeros((int(sum(chunk_lens)), Hq, d))
        r0 = 0
        for s, (n, m) in enumerate(zip(lengths, chunk_lens)):
            n, m = int(n), int(m)
            ok = allowed_fn(np.arange(n)[None, :], (n - m + np.arange(m))[:, None], np.arange(m)[:, None])
            for g in range(pool_.Hkv):
                Kc, Vc = pool_.gather(layer, tables[s], n, g)
                for h in range(g * G, (g + 1) * G):
                    X = np.where(ok, q[r0:r0 + m, h] @ Kc.T * scale, -np.inf)
                    P = np.exp(X - X.max(1, keepdims=True))
                    P = np.nan_to_num(P)
                    out[r0:r0 + m, h] = P @ Vc / np.maximum(P.sum(1, keepdims=True), 1e-300)
            r0 += m
        return out
    return prefill


def test_prefill_causal_off_by_one(monkeypatch):
    # each query misses its own position
    monkeypatch.setattr(attention, "prefill", _mutated_prefill(lambda t, p, i: t < p))
    _fails(T_pre.test_prefill_matches_brute_force, 0)


def test_prefill_mask_ignores_context(monkeypatch):
    # positions counted from the chunk start instead of the sequence start
    monkeypatch.setattr(attention, "prefill", _mutated_prefill(lambda t, p, i: t <= i))
    _fails(T_pre.test_prefill_matches_brute_force, 0)
