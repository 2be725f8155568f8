"""A decode-step driver over the C ABI: device pools as torch tensors, the
host allocator, copy-on-write copies, kv_append and paged decode attention.

torch provides device memory and streams only; every step of the path is a
libpkv call (host allocator or HIP kernel).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch

from . import pkv as P

# cache dtype -> (cache tensor dtype, pool dtype, token/query dtype)
_DT = {"f32": (torch.float32, P.PKV_F32, torch.float32),
       "bf16": (torch.bfloat16, P.PKV_BF16, torch.bfloat16),
       "fp8": (torch.uint8, P.PKV_FP8_E4M3, torch.bfloat16)}


class PagedDecodeEngine:
    def __init__(self, num_layers: int, num_kv_heads: int, head_dim: int, num_blocks: int,
                 dtype: str = "bf16", block_size: int = 16, init_perm=None, device="cuda",
                 poison: bool = True, partition: int = 0):
        self.L, self.Hkv, self.d, self.N, self.B = num_layers, num_kv_heads, head_dim, num_blocks, block_size
        self.dtype = dtype                 # cache dtype: "f32", "bf16" or "fp8"
        self.tdtype, self.cdtype, self.qdtype = _DT[dtype]
        self.device = torch.device(device)
        self.partition = partition
        numel = num_blocks * num_kv_heads * head_dim * block_size
        fill = (0x7F if dtype == "fp8" else float("nan")) if poison else 0   # 0x7F: the E4M3 NaN
        self.k = [torch.full((numel,), fill, dtype=self.tdtype, device=self.device) for _ in range(num_layers)]
        self.v = [torch.full((numel,), fill, dtype=self.tdtype, device=self.device) for _ in range(num_layers)]
        self.ks = self.vs = None
        if dtype == "fp8":                 # one fp32 scale per (slot, KV head)
            sfill = float("nan") if poison else 0.0
            nsc = num_blocks * num_kv_heads * block_size
            self.ks = [torch.full((nsc,), sfill, dtype=torch.float32, device=self.device) for _ in range(num_layers)]
            self.vs = [torch.full((nsc,), sfill, dtype=torch.float32, device=self.device) for _ in range(num_layers)]
        self.pool = P.pkv_pool_create(num_layers, num_kv_heads, head_dim, block_size, num_blocks,
                                      self.cdtype, self.k, self.v, init_perm, self.ks, self.vs)
        self.tables = None
        self.lens = None
        self.host_lens = None      # host copy of the last uploaded lengths
        self.workspace = None

    # -- allocator + writes ------------------------------------------------
    def create(self) -> int:
        return P.pkv_seq_create(self.pool)

    def fork(self, parent: int) -> int:
        return P.pkv_seq_fork(self.pool, parent)

    def free(self, sid: int) -> None:
        P.pkv_seq_free(self.pool, sid)

    def _write(self, slots: np.ndarray, cow, values: Optional[Dict[int, Tuple[torch.Tensor, torch.Tensor]]],
               stream=None):
        if cow:
            P.pkv_copy_blocks(self.pool, cow, stream)
        if values:
            dev_slots = torch.from_numpy(np.ascontiguousarray(slots)).to(self.device, non_blocking=False)
            for layer, (kk, vv) in values.items():
                P.pkv_kv_append(self.pool, layer, kk.contiguous(), vv.contiguous(), dev_slots, stream)

    def extend(self, sid: int, ntok: int, values=None, stream=None):
        """Reserve ntok slots; values: {layer: (k [ntok][Hkv][d], v)} device tensors."""
        slots, cow = P.pkv_seq_extend(self.pool, sid, ntok)
        self._write(slots, cow, values, stream)
        return slots, cow

    def append(self, ids: Sequence[int], values=None, stream=None):
        """One token per id; values: {layer: (k [n][Hkv][d], v)} device tensors."""
        slots, cow = P.pkv_append_slots(self.pool, ids)
        self._write(slots, cow, values, stream)
        return slots, cow

    def run_script(self, ops, wl=None, k_log=None, v_log=None, layers: Sequence[int] = (0,), stream=None):
        """Execute a workload script; token values are rows of the logical
        tensors (dict layer -> tensor [sum n][Hkv][d]) selected by the ops."""
        offs = None if wl is None else wl.offsets
        log = []
        for op in ops:
            kind = op[0]
            if kind == "create":
                self.create()
            elif kind == "fork":
                self.fork(op[1])
            elif kind == "free":
                self.free(op[1])
            elif kind == "release":
                P.pkv_seq_release_before(self.pool, op[1], op[2])
            elif kind == "window":             # keep the last op[2] positions
                P.pkv_seq_release_before(self.pool, op[1], max(0, self.length(op[1]) - op[2]))
            elif kind in ("extend", "append"):
                if kind == "extend":
                    _, sid, k, src, pos = op
                    rows = torch.arange(offs[src] + pos, offs[src] + pos + k) if offs is not None else None
                else:
                    rows = (torch.tensor([offs[src] + pos for (_, src, pos) in op[1]])
                            if offs is not None else None)
                vals = None
                if k_log is not None and rows is not None:
                    rd = rows.to(self.device)
                    vals = {l: (k_log[l].index_select(0, rd), v_log[l].index_select(0, rd)) for l in layers}
                if kind == "extend":
                    slots, cow = self.extend(op[1], op[2], vals, stream)
                    log.append(("extend", op[1], slots, cow))
                else:
                    ids = [e[0] for e in op[1]]
                    slots, cow = self.append(ids, vals, stream)
                    log.append(("append", ids, slots, cow))
            else:
                raise ValueError(kind)
        return log

    def step_append(self, ids: Sequence[int], values=None, max_blocks: Optional[int] = None, stream=None):
        """Decode-step append: reserve one slot per id on the host, copy any
        shared partial blocks, upload tables and lengths, and write each new
        token at its row's last position (kv_append_last) in every layer of
        ``values`` ({layer: (k [n][Hkv][d], v)})."""
        slots, cow = P.pkv_append_slots(self.pool, ids)
        if cow:
            P.pkv_copy_blocks(self.pool, cow, stream)
        self.sync(ids, max_blocks, stream)
        for layer, (kk, vv) in (values or {}).items():
            P.pkv_kv_append_last(self.pool, layer, kk.contiguous(), vv.contiguous(), self.tables, self.lens, stream)
        return slots, cow

    # -- decode ------------------------------------------------------------
    def sync(self, ids: Sequence[int], max_blocks: Optional[int] = None, stream=None):
        n = len(ids)
        if max_blocks is None:
            max_blocks = max(1, max(len(P.pkv_seq_table(self.pool, i)) for i in ids))
        if self.tables is None or self.tables.shape != (n, max_blocks):
            self.tables = torch.empty((n, max_blocks), dtype=torch.int32, device=self.device)
            self.lens = torch.empty((n,), dtype=torch.int32, device=self.device)
            self.host_lens = np.zeros(n, dtype=np.int32)
        P.pkv_sync_tables(self.pool, ids, self.tables, self.lens, self.host_lens, stream)
        return self.tables, self.lens

    def decode_args(self, layer: int, q: torch.Tensor, out: torch.Tensor, max_seq_len: int,
                    scale: Optional[float] = None, window: int = 0, k_new=None, v_new=None):
        need = P.pkv_decode_workspace_bytes(q.shape[0], q.shape[1], self.d, max_seq_len, self.partition)
        if need and (self.workspace is None or self.workspace.numel() < need):
            self.workspace = torch.empty((need,), dtype=torch.uint8, device=self.device)
        return P.decode_args(q, out, self.k[layer], self.v[layer], self.tables, self.lens, self.Hkv, self.N,
                             max_seq_len, scale, self.partition, self.workspace if need else None, self.B,
                             host_seq_lens=self.host_lens,
                             k_scale=None if self.ks is None else self.ks[layer],
                             v_scale=None if self.vs is None else self.vs[layer], window=window,
                             k_new=k_new, v_new=v_new)

    def decode(self, layer: int, q: torch.Tensor, max_seq_len: int, out: Optional[torch.Tensor] = None,
               scale: Optional[float] = None, stream=None, window: int = 0, k_new=None,
               v_new=None) -> torch.Tensor:
        """Decode one layer of the synced batch.  k_new / v_new ([S][Hkv][d]):
        the step's new token of each sequence, appended at its last position
        by the decode kernel itself (in place of kv_append_last)."""
        if out is None:
            out = torch.empty_like(q)
        a = self.decode_args(layer, q, out, max_seq_len, scale, window, k_new, v_new)
        P.pkv_paged_attention_decode(a, stream)
        return out

    def prefill(self, layer: int, q: torch.Tensor, chunk_lens: Sequence[int], max_seq_len: int,
                out: Optional[torch.Tensor] = None, scale: Optional[float] = None, window: int = 0,
                stream=None) -> torch.Tensor:
        """Chunked prefill of the synced batch: q [sum chunk_lens][Hq][d], the
        rows of batch entry i being its last chunk_lens[i] tokens (already
        written).  Returns out, shaped like q."""
        if out is None:
            out = torch.empty_like(q)
        qs = np.zeros(len(chunk_lens) + 1, dtype=np.int32)
        qs[1:] = np.cumsum(chunk_lens)
        self.query_start = torch.from_numpy(qs).to(self.device)
        ks = vs = ws = None
        if self.ks is not None:       # 8-bit cache: its scales and the bf16 copy's workspace
            ks, vs = self.ks[layer], self.vs[layer]
            nbytes = P.pkv_prefill_workspace_bytes(len(chunk_lens), self.Hkv, self.d, self.B, self.tables.shape[1],
                                                   max_seq_len, P.PKV_FP8_E4M3)
            ws = self.prefill_workspace(nbytes)
        a = P.prefill_args(q, out, self.k[layer], self.v[layer], self.tables, self.lens, self.query_start,
                           self.Hkv, self.N, max_seq_len, int(max(chunk_lens)), scale, window, self.B,
                           k_scale=ks, v_scale=vs, workspace=ws)
        P.pkv_paged_prefill(a, stream)
        return out

    def prefill_workspace(self, nbytes: int) -> torch.Tensor:
        """A device scratch buffer of at least nbytes (256-byte aligned by the
        caching allocator), kept for later calls."""
        ws = getattr(self, "_prefill_ws", None)
        if ws is None or ws.numel() < nbytes:
            ws = self._prefill_ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
        return ws

    def snapshot(self):
        return P.pkv_pool_snapshot(self.pool)

    def length(self, sid: int) -> int:
        return P.pkv_seq_length(self.pool, sid)

    def table(self, sid: int):
        return P.pkv_seq_table(self.pool, sid)
