"""Physical K/V pool in the library's byte layout (oracle; test infrastructure).

«¿Cómo gestiona Paged Attention la caché KV…?» ("PagedAttention divide el estado KV…"): K/V blocks may sit anywhere
in physical memory; a per-sequence block table maps the request's logical
token order onto them, and the model still attends over the right sequence —
the indirection moves data, it does not change its meaning.  «PagedAttention e vLLM»
("Approfondimento tecnico"): each page holds the keys and values of a fixed
number of tokens.

Layout (the library's documented format, restated here with NumPy indexing;
B = tokens per block, x = 16 bytes / element size, so x = 4 for fp32 and 8
for bf16):

* K of layer l: ``K[l][block][head][d // x][B][x]`` — element ``j`` of
  token slot ``o`` sits at ``[block][head][j // x][o][j % x]``;
* V of layer l: ``V[l][block][head][B // 4][d // 4][4][4]`` — element ``j``
  of slot ``o`` sits at ``[block][head][o // 4][j // 4][j % 4][o % 4]``: every
  run of four values holds one column of four consecutive tokens, and one
  token's row fills a quarter of the block tile.

Values are stored as raw bit patterns (uint32 for fp32, uint16 for bf16) so
that the pool can be compared bit for bit.  Slots nothing has written hold a
quiet-NaN poison pattern.

8-bit cache (``dtype="fp8"``, E4M3 codes, see ``oracle.fp8``): new tokens
arrive as bf16 bit patterns and are quantised per (token, head) row when they
are written.  x = 16, d a multiple of 64, B = 16, and

* K codes: ``K[l][block][head][d // 16][B][16]`` (as above);
* V codes: ``V[l][block][head][d // 64][B // 4][16][4][4]`` — value column
  ``j = 64a + 4c + b`` of token slot ``o = 4u + w`` sits at
  ``[block][head][a][u][c][b][w]``: every 16-byte run holds four columns of
  four consecutive tokens;
* scales: ``KS[l][block][head][B]`` and ``VS[l][block][head][B]``, fp32 bit
  patterns, one per token slot.

Poison: code 0x7F (NaN) and the fp32 quiet NaN for scales.
"""
from __future__ import annotations

import numpy as np

from . import fp8

POISON = {"f32": np.uint32(0x7FC00000), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}
BITS = {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8}
ITEMSIZE = {"f32": 4, "bf16": 2, "fp8": 1}


def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored bit patterns to float64."""
    if dtype == "f32":
        return np.ascontiguousarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)
    if dtype == "bf16":
        wide = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


class Pool:
    def __init__(self, num_blocks: int, Hkv: int, d: int, dtype: str, block: int = 16,
                 layers: int = 1, lazy_layers: bool = False):
        self.N, self.Hkv, self.d, self.dtype, self.B = num_blocks, Hkv, d, dtype, block
        self.itemsize = ITEMSIZE[dtype]
        self.x = 16 // self.itemsize
        if d % self.x:
            raise ValueError("head dim must be a multiple of 16 bytes")
        if block % 4 or d % 4:
            raise ValueError("the value layout needs block and head dim multiples of 4")
        if dtype == "fp8" and (d % 64 or block != 16):
            raise ValueError("the 8-bit layout needs d % 64 == 0 and B == 16")
        self.layers = layers
        self.K = [None] * layers
        self.V = [None] * layers
        self.KS = [None] * layers          # fp8 only: per-slot scales
        self.VS = [None] * layers
        if not lazy_layers:
            for l in range(layers):
                self._materialize(l)

    def _materialize(self, l: int) -> None:
        if self.K[l] is None:
            self.K[l] = np.full((self.N, self.Hkv, self.d // self.x, self.B, self.x),
                                POISON[self.dtype], dtype=BITS[self.dtype])
            if self.dtype == "fp8":
                self.V[l] = np.full((self.N, self.Hkv, self.d // 64, self.B // 4, 16, 4, 4),
                                    POISON["fp8"], dtype=np.uint8)
                self.KS[l] = np.full((self.N, self.Hkv, self.B), POISON["f32"], dtype=np.uint32)
                self.VS[l] = np.full((self.N, self.Hkv, self.B), POISON["f32"], dtype=np.uint32)
            else:
                self.V[l] = np.full((self.N, self.Hkv, self.B // 4, self.d // 4, 4, 4),
                                    POISON[self.dtype], dtype=BITS[self.dtype])

    def scatter(self, layer: int, slots, k_bits: np.ndarray, v_bits: np.ndarray) -> None:
        """Write token i's K/V ([Hkv][d] bit patterns) into ``slots[i]``."""
        self._materialize(layer)
        K, V = self.K[layer], self.V[layer]
        if self.dtype == "fp8":
            # new tokens arrive as bf16 bit patterns; quantise row by row
            kc, ks = fp8.quantize_rows(to_f64(k_bits, "bf16").astype(np.float32))   # [n][Hkv][d], [n][Hkv]
            vc, vs = fp8.quantize_rows(to_f64(v_bits, "bf16").astype(np.float32))
            for i, slot in enumerate(slots):
                b, o = divmod(int(slot), self.B)
                K[b, :, :, o, :] = kc[i].reshape(self.Hkv, self.d // 16, 16)
                V[b, :, :, o // 4, :, :, o % 4] = vc[i].reshape(self.Hkv, self.d // 64, 16, 4)
                self.KS[layer][b, :, o] = ks[i].view(np.uint32)
                self.VS[layer][b, :, o] = vs[i].view(np.uint32)
            return
        for i, slot in enumerate(slots):
            b, o = divmod(int(slot), self.B)
            K[b, :, :, o, :] = k_bits[i].reshape(self.Hkv, self.d // self.x, self.x)
            V[b, :, o // 4, :, :, o % 4] = v_bits[i].reshape(self.Hkv, self.d // 4, 4)

    def copy_block(self, src: int, dst: int) -> None:
        """Copy-on-write: block ``dst`` becomes a copy of ``src`` in every layer."""
        for l in range(self.layers):
            if self.K[l] is not None:
                self.K[l][dst] = self.K[l][src]
                self.V[l][dst] = self.V[l][src]
                if self.dtype == "fp8":
                    self.KS[l][dst] = self.KS[l][src]
                    self.VS[l][dst] = self.VS[l][src]

    def gather(self, layer: int, table, n: int, head: int, start: int = 0):
        """Contiguous fp64 (K [n - start][d], V [n - start][d]) of tokens
        start .. n-1 of one sequence and KV head: logical token t comes from
        block ``table[t // B]``, slot ``t % B`` (blocks before start // B are
        not read; a sliding window may have released them)."""
        self._materialize(layer)
        first = start // self.B
        if start:
            K, V = self.gather(layer, list(table[first:]), n - first * self.B, head)
            off = start - first * self.B
            return K[off:], V[off:]
        nblk = -(-n // self.B)
        blocks = np.asarray(table[:nblk], dtype=np.int64)
        if np.any(blocks < 0):
            raise ValueError("gather reached a released block")
        kb = self.K[layer][blocks, head]                 # [nblk][d/x][B][x]
        kb = kb.transpose(0, 2, 1, 3).reshape(nblk * self.B, self.d)
        if self.dtype == "fp8":
            vb = self.V[layer][blocks, head]             # [nblk][d/64][B/4][16][4][4]
            vb = vb.transpose(0, 2, 5, 1, 3, 4).reshape(nblk * self.B, self.d)
            ks = self.KS[layer][blocks, head].reshape(-1).view(np.float32).astype(np.float64)
            vs = self.VS[layer][blocks, head].reshape(-1).view(np.float32).astype(np.float64)
            kf = fp8.decode(kb[:n]) * ks[:n, None]
            vf = fp8.decode(vb[:n]) * vs[:n, None]
            return kf, vf
        vb = self.V[layer][blocks, head]                 # [nblk][B/4][d/4][4][4]
        vb = vb.transpose(0, 1, 4, 2, 3).reshape(nblk * self.B, self.d)
        return to_f64(kb[:n], self.dtype), to_f64(vb[:n], self.dtype)
