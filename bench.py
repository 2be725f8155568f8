#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

A step is one pass of the whole decode hot path over the batch: reserve one
slot per sequence on the host allocator (copy-on-write copies if any),
upload block tables and lengths, then for every layer write the new token's
K/V (kv_append) and run paged decode attention (partial + reduce).  Steps
are successive decode steps: every sequence grows by one token per step, and
bytes are counted from the lengths of each step.

Default workload: 16 sequences of 32768 tokens, 64 query / 8 KV heads,
d = 128, bf16, 16-token blocks in random physical order, 512-token split-K
partitions (the long-context configuration).  `value` is KV bytes read by
attention per second (decimal GB/s) over the timed steps.  The *_fp8
configurations keep the same batch in an 8-bit E4M3 cache (bf16 tokens and
queries; KV bytes count the codes and the per-token scales).

Before any timing, the first decode step (same path and inputs as the
timed ones) is checked against the oracle on a few sequences (every query
head; allocator state and those sequences' pool bytes exactly, outputs
within the tolerance); the result is the line's `parity` record, and a
mismatch ends the run with status 3.  The default run also reports the
32-layer step (256 sequences, MHA) under `full_step`: ms per step, decode
tokens/s, KV GB/s and the partial kernel's rate, validated the same way.

Prints one JSON line.  Options: --gpus N (only 1 is supported), --steps K
(default 100 for the long one-layer batches, else 20), --warmup W,
--config NAME, --no-cpu-baseline (also skips the validation),
--no-full-step, --cpu-seconds S.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: KV GB/s read and % of HBM peak; decode tokens/s"
HBM_PEAK_GBS = 8000.0
# the decode kernels' sources: the kernels, and the header with the wave's cell decoding
KERNEL_SRCS = [os.path.join(ROOT, "paged_kv_cache_08_amd", "csrc", f)
               for f in ("kernels.hip", "kernels.hpp", "device_util.hpp")]
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def kernel_hash() -> str:
    h = hashlib.sha256()
    for src in KERNEL_SRCS:
        with open(src, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 100 for a one-layer batch of sequences of 4,096 tokens or more, "
                         "so that a short host stall weighs little; else 20)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="long_context")
    ap.add_argument("--partition", type=int, default=0)
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window: attend to the last W positions and release older blocks each step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--separate-append", action="store_true",
                    help="append the step's new K/V with kv_append_last before each layer's decode instead of "
                         "in the decode kernel")
    ap.add_argument("--flush", action="store_true",
                    help="write a 1 GiB buffer before every decode step, outside its timing, to evict L2 and the "
                         "MALL; value and step time then come from events around each step")
    ap.add_argument("--table-stream", choices=["auto", "side", "main"], default="auto",
                    help="stream of each step's table upload: a side stream with events, or the main stream; "
                         "auto: the side stream for a multi-layer step, the main stream for one layer")
    ap.add_argument("--no-full-step", action="store_true",
                    help="leave out the 32-layer step that the default (long-context) run also reports")
    ap.add_argument("--torch-events", action="store_true",
                    help="time and order the streams with torch's events (recorded with the system-scope fence) "
                         "instead of fence-free HIP events")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB device copies (known bytes) for counter scaling")
    return ap.parse_args()


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class _Hip:
    """The HIP runtime that torch has loaded (found among the process's
    mappings, so the same library instance and device state)."""
    lib = None

    @classmethod
    def get(cls):
        if cls.lib is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            h = ctypes.CDLL(path)
            vp, u = ctypes.c_void_p, ctypes.c_uint
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), u]
            h.hipEventRecord.argtypes = [vp, vp]
            h.hipStreamWaitEvent.argtypes = [vp, vp, u]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            for f in (h.hipEventCreateWithFlags, h.hipEventRecord, h.hipStreamWaitEvent, h.hipEventElapsedTime):
                f.restype = ctypes.c_int
            cls.lib = h
        return cls.lib


class Event:
    """A stream event with the part of torch.cuda.Event's interface the
    bench uses.  By default a HIP event recorded without the system-scope
    fence (hipEventDisableSystemFence): a fenced event writes back and
    invalidates the caches at its marker, which leaves the GPU idle for a
    few microseconds, and the bench's events order and time work on one
    device only.  `use_torch` (--torch-events) takes torch's events."""
    use_torch = False
    _DISABLE_TIMING = 0x2
    _NO_SYSTEM_FENCE = 0x20000000

    def __init__(self, enable_timing: bool = False):
        import torch
        if Event.use_torch:
            self.t = torch.cuda.Event(enable_timing=enable_timing)
            return
        import ctypes
        self.t = None
        self.ev = ctypes.c_void_p()
        flags = self._NO_SYSTEM_FENCE | (0 if enable_timing else self._DISABLE_TIMING)
        self._check(_Hip.get().hipEventCreateWithFlags(ctypes.byref(self.ev), flags), "hipEventCreateWithFlags")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    @staticmethod
    def _handle(stream):
        import torch
        return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream

    def record(self, stream=None):
        if self.t is not None:
            return self.t.record(stream) if stream is not None else self.t.record()
        self._check(_Hip.get().hipEventRecord(self.ev, self._handle(stream)), "hipEventRecord")

    def wait_on(self, stream):
        """Make `stream` wait for this event."""
        if self.t is not None:
            return stream.wait_event(self.t)
        self._check(_Hip.get().hipStreamWaitEvent(self._handle(stream), self.ev, 0), "hipStreamWaitEvent")

    def elapsed_time(self, end: "Event") -> float:
        """Milliseconds from this event to `end` (both completed)."""
        if self.t is not None:
            return self.t.elapsed_time(end.t)
        import ctypes
        ms = ctypes.c_float()
        self._check(_Hip.get().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev), "hipEventElapsedTime")
        return ms.value


def copy_calibration(reps: int = 5, nbytes: int = 1 << 30) -> None:
    """Plain device-to-device copies of a known size: each launch reads and
    writes exactly `nbytes`, so counter readings for it give the scale from
    counter units to bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": reps}), flush=True)


class DecodeBench:
    """Builds the batch through the library, then runs timed decode steps.

    The part of step i that does not depend on the step's data — the host
    slot reservation and the block-table upload — runs on a second stream
    while step i-1's attention still runs on the main stream, as a serving
    loop can do, since block placement does not depend on token values.  The
    copy-on-write copies, the new K/V append (written by the decode call's
    partial kernel where the library fuses it, pkv_decode_fuses_append, else
    and with --separate-append by kv_append_last before the call) and
    attention stay on the main stream, in step order.  Device tables are double-buffered (step i uses
    buffer i % 2): the side stream waits until the step that last read its
    buffer has finished, and the main stream waits for the upload."""

    def __init__(self, wl, steps_total: int, partition: int = 0, device="cuda", window: int = 0,
                 fused_append: bool = True, table_stream: str = "auto"):
        import numpy as np
        import torch
        from paged_kv_cache_08_amd import pkv as P
        from paged_kv_cache_08_amd.engine import PagedDecodeEngine

        self.P, self.torch, self.np = P, torch, np
        self.wl = wl
        self.fused_append = fused_append
        self.window = window
        self.dev = torch.device(device)
        self.layers = wl.layers
        self.eng = PagedDecodeEngine(wl.layers, wl.Hkv, wl.d, wl.num_blocks, wl.cache_dtype, init_perm=wl.perm,
                                     device=device, partition=partition)
        # prefill every sequence to n - 1 tokens, layer by layer so the logical
        # tensors of one layer at a time are resident
        setup_log = self.eng.run_script(wl.setup_ops, None)    # allocator only
        for layer in range(wl.layers):
            _, k, v = wl.tensors(layer, device=device)
            offs = wl.offsets
            for (kind, sid, slots, cow), op in zip(setup_log, [o for o in wl.setup_ops if o[0] == "extend"]):
                assert not cow
                _, _, cnt, src, pos = op
                rows = torch.arange(offs[src] + pos, offs[src] + pos + cnt, device=self.dev)
                dslots = torch.from_numpy(np.ascontiguousarray(slots)).to(self.dev)
                P.pkv_kv_append(self.eng.pool, layer, k.index_select(0, rows), v.index_select(0, rows), dslots)
            del k, v
        torch.cuda.synchronize()
        self.ids = list(wl.seq_ids)
        # numpy forms for the per-step host work, which a short step's kernels
        # (about 70 us for 128 sequences) would otherwise wait for
        self.ids_np = np.asarray(self.ids, dtype=np.int64)
        self.lengths = np.asarray([int(n) - 1 for n in wl.lengths], dtype=np.int64)   # current lengths
        self.max_len = int(self.lengths.max()) + steps_total
        self.max_blocks = -(-self.max_len // wl.block)
        self.tables = [torch.empty((len(self.ids), self.max_blocks), dtype=torch.int32, device=self.dev)
                       for _ in range(2)]
        self.lens = [torch.empty((len(self.ids),), dtype=torch.int32, device=self.dev) for _ in range(2)]
        self.eng.host_lens = np.zeros(len(self.ids), dtype=np.int32)
        self.main = torch.cuda.current_stream()
        self.main_ptr = self.main.cuda_stream     # passed to each call: no stream query per launch
        # The side stream overlaps the upload with the previous step's layers, but the cross-stream wait
        # leaves a gap of about 11 us; in line the upload costs about 6 us.  One layer has nothing to
        # overlap it with.
        if table_stream == "auto":
            table_stream = "side" if wl.layers > 1 else "main"
        self.table_stream = table_stream
        self.side = torch.cuda.Stream() if table_stream == "side" else self.main   # default priority
        self.ready = [Event() for _ in range(2)]
        self.done = [Event() for _ in range(2)]
        for e in self.done:
            e.record(self.main)
        # per-step inputs: new K/V per layer and the step's queries
        g = torch.Generator(device=self.dev)
        g.manual_seed(wl.seed * 7919 + 1)
        dt = self.eng.qdtype
        S = len(self.ids)
        self.knew = [torch.randn((steps_total, S, wl.Hkv, wl.d), generator=g, device=self.dev).to(dt)
                     for _ in range(wl.layers)]
        self.vnew = [torch.randn((steps_total, S, wl.Hkv, wl.d), generator=g, device=self.dev).to(dt)
                     for _ in range(wl.layers)]
        self.q = [torch.randn((S, wl.Hq, wl.d), generator=g, device=self.dev).to(dt) for _ in range(wl.layers)]
        self.out = [torch.empty_like(self.q[l]) for l in range(wl.layers)]
        self.args = []
        for b in range(2):
            self.eng.tables, self.eng.lens = self.tables[b], self.lens[b]
            self.args.append([self.eng.decode_args(l, self.q[l], self.out[l], self.max_len, window=window)
                              for l in range(wl.layers)])
        if fused_append:              # only where the decode call writes the tokens in its partial kernel
            P.set_new_token(self.args[0][0], self.knew[0][0], self.vnew[0][0])
            self.fused_append = P.pkv_decode_fuses_append(self.args[0][0])
            P.set_new_token(self.args[0][0], None, None)
        torch.cuda.synchronize()      # the side stream's first step reads the inputs made above
        self.step_idx = 0
        self.kv_bytes = []            # attention KV bytes of each step (all layers)
        self.events = []              # (k3 start, k3 end, KV bytes) of the timed partial launches
        self.timed_steps = 0          # steps run with record_events
        self.step_events = []         # (step start, step end) when the caches are flushed
        self.flush = None

    def enable_flush(self, nbytes: int = 1 << 30):
        """Before each step, write nbytes on the main stream (a fill kernel),
        more than L2 and the 256 MB MALL together hold."""
        self.flush = self.torch.empty(nbytes, dtype=self.torch.uint8, device=self.dev)

    def step(self, record_events: bool):
        P, torch = self.P, self.torch
        j = self.step_idx
        b = j % 2
        side = self.side
        if side is not self.main:
            self.done[b].wait_on(side)       # the step that last used these tables has finished
        if self.flush is not None:
            self.flush.fill_(j & 0xFF)
        slots, cow = P.pkv_append_slots(self.eng.pool, self.ids_np)
        self.lengths += 1
        if self.window:                  # a block that has just left the window goes back to the pool
            B = self.wl.block
            for sid, n in zip(self.ids, self.lengths.tolist()):
                start = n - self.window
                if start > 0 and start % B == 0:
                    P.pkv_seq_release_before(self.eng.pool, sid, start)
        P.pkv_sync_tables(self.eng.pool, self.ids_np, self.tables[b], self.lens[b], self.eng.host_lens, side)
        if side is not self.main:
            self.ready[b].record(side)
            self.ready[b].wait_on(self.main)
        if self.flush is not None and record_events:
            s0 = Event(enable_timing=True)
            s0.record(self.main)
        ms = self.main_ptr
        if cow:
            P.pkv_copy_blocks(self.eng.pool, cow, ms)
        # A timing event costs the stream about 5 us, so a step times one
        # partial-kernel launch (layers in turn); a one-layer step (well
        # under a millisecond) every fourth step.
        timed = -1
        if record_events:
            if self.layers > 1 or self.timed_steps % 4 == 0:
                timed = j % self.layers
            self.timed_steps += 1
        for l in range(self.layers):
            a = self.args[b][l]
            if self.fused_append:       # the partial kernel writes the step's new token itself
                P.set_new_token(a, self.knew[l][j], self.vnew[l][j])
            else:                       # (the call would run the append kernel first: do it here,
                                        #  outside the timed partial launch)
                P.pkv_kv_append_last(self.eng.pool, l, self.knew[l][j], self.vnew[l][j], self.tables[b], self.lens[b],
                                     stream=ms)
            if l == timed:
                e0 = Event(enable_timing=True)
                e1 = Event(enable_timing=True)
                e0.record()
            P.pkv_paged_decode_partial(a, ms)
            if l == timed:
                e1.record()
                self.events.append((e0, e1, self.attended_bytes(l)))
            P.pkv_paged_decode_reduce(a, ms)
        if side is not self.main:
            self.done[b].record(self.main)
        if self.flush is not None and record_events:
            s1 = Event(enable_timing=True)
            s1.record(self.main)
            self.step_events.append((s0, s1))
        self.kv_bytes.append(self.attended_bytes(0) * self.layers)
        self.step_idx += 1

    def unique_bytes(self) -> int:
        """KV bytes of the distinct pool slots one layer's decode reads at the
        current lengths: a block shared by several sequences counts once."""
        np = self.np
        B = self.wl.block
        slots = []
        for sid, n in zip(self.ids, self.lengths.tolist()):
            table = np.asarray(self.P.pkv_seq_table(self.eng.pool, sid), dtype=np.int64)
            t = np.arange(max(0, n - self.window) if self.window else 0, n)
            slots.append(table[t // B] * B + t % B)
        unique = int(np.unique(np.concatenate(slots)).size) if slots else 0
        return unique * self.wl.Hkv * self.wl.kv_bytes_per_token_head()

    def attended_bytes(self, layer: int) -> int:
        """KV bytes one layer's partial kernel reads at the current lengths."""
        wl = self.wl
        n = self.lengths
        attended = int((self.np.minimum(n, self.window) if self.window else n).sum())
        return attended * wl.Hkv * wl.kv_bytes_per_token_head()


class PrefillBench:
    """Chunked prefill: the setup writes every sequence's context and chunk
    through the library; a step writes the chunk's K/V again (kv_append, the
    same slots) and runs the prefill attention over it, per layer."""

    def __init__(self, wl, device="cuda", window: int = 0):
        import numpy as np
        import torch
        from paged_kv_cache_08_amd import pkv as P
        from paged_kv_cache_08_amd.engine import PagedDecodeEngine

        self.P, self.torch, self.wl, self.window = P, torch, wl, window
        self.dev = torch.device(device)
        self.eng = PagedDecodeEngine(wl.layers, wl.Hkv, wl.d, wl.num_blocks, wl.cache_dtype, init_perm=wl.perm,
                                     device=device)
        log = self.eng.run_script(wl.setup_ops + wl.step_ops, None)          # allocator only
        offs = wl.offsets
        self.k, self.v, self.q, self.chunk_slots = [], [], [], None
        chunk_rows, chunk_slots = [], []
        for layer in range(wl.layers):
            _, k, v = wl.tensors(layer, device=device)
            for (kind, sid, slots, cow), op in zip(log, [o for o in wl.setup_ops + wl.step_ops if o[0] == "extend"]):
                _, _, cnt, src, pos = op
                rows = torch.arange(offs[src] + pos, offs[src] + pos + cnt, device=self.dev)
                dslots = torch.from_numpy(np.ascontiguousarray(slots)).to(self.dev)
                P.pkv_kv_append(self.eng.pool, layer, k.index_select(0, rows), v.index_select(0, rows), dslots)
                if layer == 0 and op in wl.step_ops:
                    chunk_rows.append(rows)
                    chunk_slots.append(dslots)
            rows = torch.cat(chunk_rows)
            self.k.append(k.index_select(0, rows).contiguous())             # the chunk's new K/V
            self.v.append(v.index_select(0, rows).contiguous())
            self.q.append(wl.prefill_queries(layer, device=device))
            del k, v
        self.chunk_slots = torch.cat(chunk_slots).contiguous()
        self.eng.sync(wl.seq_ids)
        self.out = [torch.empty_like(self.q[l]) for l in range(wl.layers)]
        self.chunks = list(map(int, wl.chunk_lens))
        qs = np.zeros(len(self.chunks) + 1, dtype=np.int32)
        qs[1:] = np.cumsum(self.chunks)
        self.query_start = torch.from_numpy(qs).to(self.dev)
        ws = None
        if self.eng.ks is not None:   # 8-bit cache: the call's bf16 copy of the blocks lives in a workspace
            ws = self.eng.prefill_workspace(P.pkv_prefill_workspace_bytes(
                wl.S, wl.Hkv, wl.d, wl.block, self.eng.tables.shape[1], wl.max_len, P.PKV_FP8_E4M3))
        self.args = [P.prefill_args(self.q[l], self.out[l], self.eng.k[l], self.eng.v[l], self.eng.tables,
                                    self.eng.lens, self.query_start, wl.Hkv, wl.num_blocks, wl.max_len,
                                    max(self.chunks), window=window,
                                    k_scale=None if self.eng.ks is None else self.eng.ks[l],
                                    v_scale=None if self.eng.vs is None else self.eng.vs[l], workspace=ws)
                     for l in range(wl.layers)]
        torch.cuda.synchronize()
        self.events = []

    def step(self, record_events: bool):
        P, torch = self.P, self.torch
        for l in range(self.wl.layers):
            P.pkv_kv_append(self.eng.pool, l, self.k[l], self.v[l], self.chunk_slots)
            if record_events:
                e0 = Event(enable_timing=True)
                e1 = Event(enable_timing=True)
                e0.record()
            P.pkv_paged_prefill(self.args[l])
            if record_events:
                e1.record()
                self.events.append((e0, e1))


def prefill_cpu_baseline(wl, seconds: float, window: int = 0):
    """The oracle's prefill on a bounded sample: the first sequence of the
    batch, one query head per KV head... repeated over its KV heads until the
    time is spent; rate in TFLOP/s of the same causal pairs."""
    import numpy as np
    import workloads
    from oracle import attention as OA
    from oracle.pool import to_f64
    from oracle.replay import Replay
    import torch

    def bits(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    one = workloads.prefill_chunks(wl.lengths[:1] - wl.chunk_lens[:1], wl.chunk_lens[:1], wl.Hq, wl.Hkv, wl.d,
                                   wl.dtype, wl.seed)
    if wl.cache_dtype == "fp8":
        one = workloads.fp8_cache(one)
    q = one.prefill_queries()
    _, k, v = one.tensors()
    rp = Replay(one).run(one.setup_ops + one.step_ops, {0: (bits(k), bits(v))})
    q64 = to_f64(bits(q), one.dtype)
    G = one.Hq // one.Hkv
    m = int(one.chunk_lens[0])
    heads, t = 0, 0.0
    while t < seconds or heads == 0:
        h = (heads * G) % one.Hq                          # one query head of each KV head in turn
        rows = {(i, h) for i in range(m)}
        t0 = time.perf_counter()
        OA.prefill(rp.pool, 0, rp.tables(), rp.lengths(), one.chunk_lens, q64, one.Hq, window=window, rows=rows)
        t += time.perf_counter() - t0
        heads += 1
    flops = one.prefill_flops(window) / one.Hq * heads
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"sequence 0 of the batch ({m} new tokens over {int(one.lengths[0])}), "
                      f"{heads} query heads one at a time, {t:.1f} s", "host": host_info()}


def read_ceiling(nbytes: int, reps: int = 5, tile_bytes: int = 4096):
    """What memory delivers for the decode's access pattern without its
    arithmetic: pkv_read_tiles over a buffer of the launch's KV bytes, as
    tiles of one (block, KV head) (4 KiB in bf16, 2 KiB in 8-bit codes) in a
    seeded random order (gather) and in address order (stream), best over
    16-512 tiles per wave; GB/s from the median of `reps` HIP-event-timed
    launches each."""
    import numpy as np
    import torch
    from paged_kv_cache_08_amd import pkv as P
    tiles = max(1, nbytes // tile_bytes)
    g = torch.Generator(device="cuda")
    g.manual_seed(12345)
    buf = torch.empty(tiles * (tile_bytes // 4), dtype=torch.int32, device="cuda").random_(generator=g)
    perm = np.random.default_rng(12345).permutation(tiles).astype(np.int32)
    order = torch.from_numpy(perm).cuda()
    result = {"kernel": "read_tiles", "bytes": tiles * tile_bytes, "tile_bytes": tile_bytes}
    for mode, o in (("gather", order), ("stream", None)):
        best, best_tpw = 0.0, None
        for tpw in (16, 64, 256, 512):
            sink = torch.empty(-(-tiles // tpw) * 64, dtype=torch.int32, device="cuda")
            for _ in range(2):
                P.pkv_read_tiles(buf, o, tiles, tpw, sink, tile_bytes=tile_bytes)
            ms = []
            for _ in range(reps):
                e0 = Event(enable_timing=True)
                e1 = Event(enable_timing=True)
                e0.record()
                P.pkv_read_tiles(buf, o, tiles, tpw, sink, tile_bytes=tile_bytes)
                e1.record()
                ms.append((e0, e1))
            torch.cuda.synchronize()
            t = sorted(a.elapsed_time(b) for a, b in ms)[reps // 2] / 1e3
            rate = tiles * tile_bytes / t / 1e9
            if rate > best:
                best, best_tpw = rate, tpw
        result[f"{mode}_gbs"] = round(best, 1)
        result[f"{mode}_tiles_per_wave"] = best_tpw
    del buf, order
    torch.cuda.empty_cache()
    return result


def host_info() -> dict:
    """The host the oracle baseline ran on: usable cores, CPU model and the
    BLAS library numpy calls (threadpoolctl's view)."""
    info = {"usable_cores": len(os.sched_getaffinity(0))}
    try:
        with open("/proc/cpuinfo") as f:
            info["cpu_model"] = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        info["cpu_model"] = None
    try:
        from threadpoolctl import threadpool_info
        info["blas"] = [{k: i.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
                        for i in threadpool_info() if i.get("user_api") == "blas"]
    except ImportError:
        info["blas"] = None
    return info


def with_steps(args, wl):
    """args with --steps resolved for workload wl.  A one-layer decode step of
    sequences of at least 4,096 tokens lasts about 0.2-0.4 ms: it takes 100
    steps, so that a short host stall weighs little in the wall time, and 100
    more tokens per sequence change its bytes by under 2.5%.  Every other
    workload takes 20: each step lengthens every sequence by one token, and
    the short-sequence batches' pools hold only a few steps' growth."""
    import copy
    a = copy.copy(args)
    if a.steps is None:
        long_one_layer = wl.chunk is None and wl.layers == 1 and int(min(wl.lengths)) >= 4096
        a.steps = 100 if long_one_layer else 20
    return a


def launch_stats_us(ms):
    """Median, min and max of per-launch HIP event times (ms) in us."""
    v = sorted(ms)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"median": round(med * 1e3, 2), "min": round(v[0] * 1e3, 2), "max": round(v[-1] * 1e3, 2)}


def run_prefill(args, wl):
    import torch
    log(f"setup {wl.description}")
    bench = PrefillBench(wl, window=args.window)
    parity = None
    if not args.no_cpu_baseline:
        log("validating the first step against the oracle")
        parity = validate_prefill_first_step(bench, sorted({0, wl.S - 1}))
    for _ in range(args.warmup):
        bench.step(record_events=False)
    torch.cuda.synchronize()
    log("timed steps")
    gc.collect()
    gc.disable()
    try:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            bench.step(record_events=True)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    finally:
        gc.enable()
    flops_step = wl.prefill_flops(args.window) * wl.layers
    k_ms = [a.elapsed_time(b) for a, b in bench.events]
    k_avg = sum(k_ms) / len(k_ms) / 1e3
    achieved = wl.prefill_flops(args.window) / k_avg / 1e12
    value = flops_step * args.steps / elapsed / 1e12
    peak = 2500.0
    result = {
        "metric": "paged prefill attention: TFLOP/s (causal QK and PV) and prefill tokens/s",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "layers": wl.layers, "S": wl.S,
                   "Hq": wl.Hq, "Hkv": wl.Hkv, "d": wl.d, "block": wl.block, "window": args.window,
                   "kv_cache": wl.cache_dtype, "chunk_mean": float(wl.chunk_lens.mean()), "length_mean": float(wl.lengths.mean())},
        "prefill_tokens_per_s": round(float(wl.chunk_lens.sum()) * args.steps / elapsed, 1),
        "roofline": {"bound": "mfma", "kernel": "prefill_bf16", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "avg_launch_us": round(k_avg * 1e6, 2), "launch_us": launch_stats_us(k_ms),
                     "algorithmic_flops_per_launch": wl.prefill_flops(args.window)},
    }
    if parity is not None:
        result["parity"] = parity
    log(f"timed {args.steps} steps: {value:.1f} TFLOP/s; prefill kernel {k_avg * 1e6:.1f} us")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = prefill_cpu_baseline(wl, args.cpu_seconds, args.window)
    print(json.dumps(result), flush=True)


def _bits(t):
    """Raw bit patterns of a CPU tensor (uint32 for fp32, uint16 for bf16)."""
    import numpy as np
    import torch
    t = t.detach().cpu().contiguous()
    return (t.view(torch.int32).numpy().view(np.uint32) if t.dtype == torch.float32
            else t.view(torch.int16).numpy().view(np.uint16))


def pool_problems(eng, rp, layer, seqs, B, window=0):
    """Compares the library's pool with the oracle's for the batch rows
    `seqs` of one layer: every block those sequences wrote in full, bit for
    bit, and each slot of their partly written edge blocks (every head and
    value; the 8-bit pools' scales too).  Returns the differences found."""
    import numpy as np
    import torch
    problems = []
    tables, lengths = rp.tables(), rp.lengths()
    pool = rp.pool
    pairs = [(pool.K[layer], eng.k[layer]), (pool.V[layer], eng.v[layer])]
    if pool.dtype == "fp8":
        pairs += [(pool.KS[layer], eng.ks[layer]), (pool.VS[layer], eng.vs[layer])]
    for ref, dev in pairs:
        ours = (dev.cpu().numpy() if dev.dtype == torch.uint8 else _bits(dev)).reshape(ref.shape)

        def slot(arr, b, o):                  # token slot o of block b, every head and value
            if arr.ndim == 3:                                            # scales [block][head][slot]
                return arr[b][:, o]
            if arr.ndim == 7:                                            # 8-bit V [block][head][a][u][c][b][w]
                return arr[b][:, :, o // 4, :, :, o % 4]
            if arr.ndim == 6:                                            # V [block][head][u][c][b][w]
                return arr[b][:, o // 4, :, :, o % 4]
            return arr[b][:, :, o]                                       # K [block][head][d/x][slot][x]

        for i in seqs:
            n = lengths[i]
            t0 = max(0, n - window) if window else 0
            whole = [tables[i][j] for j in range(-(-t0 // B), n // B)]  # blocks written in full
            if whole and not np.array_equal(ours[whole], ref[whole]):
                problems.append(f"layer {layer}: pool blocks of batch row {i} differ")
            edge = [t for t in range(t0, n) if t < -(-t0 // B) * B or t >= (n // B) * B]
            for t in edge:
                b, o = tables[i][t // B], t % B
                if not np.array_equal(slot(ours, b, o), slot(ref, b, o)):
                    problems.append(f"layer {layer}: pool slot {t} of batch row {i} differs")
                    break
        del ours
    return problems


def validate_first_step(bench, layers, seqs, atol: float = 2e-2, row_rtol: float = 1e-2):
    """The oracle leg, before anything is timed: runs the first decode step
    (the path and inputs the timed steps use, its new token included) and
    compares it with the oracle on the batch rows `seqs`, every query head,
    in `layers`.  The oracle replays the setup through its own allocator
    and pool (writing only those sequences' tokens) and the step's append,
    then decodes.  Checked: the allocator state bit for bit, the pool bytes
    of those sequences (every written slot, new token included) bit for bit,
    and the outputs within max |err| <= atol and row-normwise <= row_rtol.
    Returns the parity record; exits with status 3 on a mismatch."""
    import numpy as np
    import torch
    from oracle import attention as OA
    from oracle.pool import to_f64
    from oracle.replay import Replay

    wl = bench.wl
    bench.step(record_events=False)
    torch.cuda.synchronize()
    entries = wl.step_ops[0][1]                       # (id, logical sequence, position) per batch row
    srcs = {entries[i][1] for i in seqs}
    rp = Replay(wl, layers=max(layers) + 1)
    vals = {}
    for l in layers:
        _, k, v = wl.tensors(l, device=bench.dev)
        vals[l] = (_bits(k), _bits(v))
        del k, v
    rp.run(wl.setup_ops, vals, sources=srcs)
    del vals
    slots, cow = rp.alloc.append(list(bench.ids))
    for a, b in cow:
        rp.pool.copy_block(a, b)
    sel = np.asarray(seqs)
    for l in layers:
        rp.pool.scatter(l, np.asarray(slots)[sel], _bits(bench.knew[l][0])[sel], _bits(bench.vnew[l][0])[sel])
    if bench.window:
        B = wl.block
        for sid in bench.ids:
            start = rp.alloc.length(sid) - bench.window
            if start > 0 and start % B == 0:
                rp.alloc.release_before(sid, start)
    problems = []
    if bench.eng.snapshot() != tuple(rp.alloc.snapshot()):
        problems.append("allocator state differs")
    tables, lengths = rp.tables(), rp.lengths()
    worst_abs, worst_rel = 0.0, 0.0
    for l in layers:
        problems += pool_problems(bench.eng, rp, l, seqs, wl.block, bench.window)
        q64 = to_f64(_bits(bench.q[l]), wl.dtype)
        heads = {(i, h) for i in seqs for h in range(wl.Hq)}
        ref = OA.decode(rp.pool, l, tables, lengths, q64, wl.Hq, heads=heads, window=bench.window)
        got = bench.out[l].float().cpu().double().numpy()
        g = np.concatenate([got[i] for i in seqs])
        r = np.concatenate([ref[i] for i in seqs])
        if not np.all(np.isfinite(g)):
            problems.append(f"layer {l}: non-finite outputs")
            continue
        err = np.abs(g - r)
        worst_abs = max(worst_abs, float(err.max()))
        worst_rel = max(worst_rel, float((err.max(axis=1) / np.maximum(np.abs(r).max(axis=1), 1e-300)).max()))
    if worst_abs > atol or worst_rel > row_rtol:
        problems.append(f"outputs beyond tolerance: max_abs {worst_abs:.3e}, row_rel {worst_rel:.3e}")
    record = {"checked": "first decode step, before timing, against the oracle",
              "layers": list(layers), "batch_rows": list(map(int, seqs)), "rows": len(seqs) * wl.Hq * len(layers),
              "max_abs": worst_abs, "row_rel": worst_rel, "atol": atol, "row_rtol": row_rtol,
              "allocator": "bit-exact" if "allocator state differs" not in problems else "differs",
              "pool": "checked sequences' slots bit-exact" if not any("pool" in p for p in problems) else "differs",
              "pass": not problems}
    if problems:
        log("VALIDATION FAILED: " + "; ".join(problems[:5]))
        print(json.dumps({"metric": METRIC, "value": None, "parity": record, "errors": problems[:20]}), flush=True)
        sys.exit(3)
    log(f"validated the first step on {record['rows']} rows: max_abs {worst_abs:.3e}, row_rel {worst_rel:.3e}")
    return record


def validate_prefill_first_step(bench, seqs, atol: float = 2e-2, row_rtol: float = 1e-2):
    """The oracle leg of a prefill run, before anything is timed: runs the
    first step (the chunk's append and the prefill kernel, as timed) and
    compares layer 0 with the oracle's prefill on the batch rows `seqs`:
    every query head at the chunk's first and last two positions, its middle,
    and the positions around the first 16-token block, 64-token tile and
    384-row workgroup boundaries.  The oracle replays the setup through its
    own allocator and pool, writing only those sequences' tokens.  Checked:
    the allocator state and those sequences' pool slots bit for bit, and the
    outputs within max |err| <= atol and row-normwise <= row_rtol.  Returns
    the parity record; exits with status 3 on a mismatch."""
    import numpy as np
    import torch
    from oracle import attention as OA
    from oracle.pool import to_f64
    from oracle.replay import Replay

    wl = bench.wl
    bench.step(record_events=False)
    torch.cuda.synchronize()
    sids = {wl.seq_ids[i] for i in seqs}
    srcs = {op[3] for op in wl.setup_ops + wl.step_ops if op[0] == "extend" and op[1] in sids}
    _, k, v = wl.tensors(0, device=bench.dev)
    rp = Replay(wl, layers=1).run(wl.setup_ops + wl.step_ops, {0: (_bits(k), _bits(v))}, sources=srcs)
    del k, v
    problems = []
    if bench.eng.snapshot() != tuple(rp.alloc.snapshot()):
        problems.append("allocator state differs")
    problems += pool_problems(bench.eng, rp, 0, seqs, wl.block)
    G = wl.Hq // wl.Hkv
    starts = np.concatenate([[0], np.cumsum(wl.chunk_lens)])
    rows = []
    for i in seqs:
        m = int(wl.chunk_lens[i])
        pos = {0, 1, m // 2, m - 2, m - 1}
        for b in (16, 64, 384 // G):
            pos |= {b - 1, b}
        rows += [(int(starts[i]) + t, h) for t in sorted(t for t in pos if 0 <= t < m) for h in range(wl.Hq)]
    ref = OA.prefill(rp.pool, 0, rp.tables(), rp.lengths(), wl.chunk_lens, to_f64(_bits(bench.q[0]), wl.dtype),
                     wl.Hq, window=bench.window, rows=set(rows))
    got = bench.out[0].float().cpu().double().numpy()
    g = np.stack([got[r, h] for r, h in rows])
    r = np.stack([ref[r, h] for r, h in rows])
    worst_abs = worst_rel = float("nan")
    if not np.all(np.isfinite(g)):
        problems.append("non-finite outputs")
    else:
        err = np.abs(g - r)
        worst_abs = float(err.max())
        worst_rel = float((err.max(axis=1) / np.maximum(np.abs(r).max(axis=1), 1e-300)).max())
        if worst_abs > atol or worst_rel > row_rtol:
            problems.append(f"outputs beyond tolerance: max_abs {worst_abs:.3e}, row_rel {worst_rel:.3e}")
    record = {"checked": "first prefill step, before timing, against the oracle", "layers": [0],
              "batch_rows": list(map(int, seqs)), "rows": len(rows), "max_abs": worst_abs, "row_rel": worst_rel,
              "atol": atol, "row_rtol": row_rtol,
              "allocator": "bit-exact" if "allocator state differs" not in problems else "differs",
              "pool": "checked sequences' slots bit-exact" if not any("pool" in p for p in problems) else "differs",
              "pass": not problems}
    if problems:
        log("VALIDATION FAILED: " + "; ".join(problems[:5]))
        print(json.dumps({"metric": "paged prefill attention", "value": None, "parity": record,
                          "errors": problems[:20]}), flush=True)
        sys.exit(3)
    log(f"validated the first prefill step on {len(rows)} (row, head) pairs: max_abs {worst_abs:.3e}, "
        f"row_rel {worst_rel:.3e}")
    return record


def cpu_baseline(wl_name: str, seconds: float, window: int = 0):
    """The oracle (unchanged) on a bounded sample of the same workload:
    a few of its sequences, one decode step at a time (allocator append,
    scatter of the new token, gather + fp64 attention), on host cores."""
    import numpy as np
    import torch
    import workloads
    from oracle import attention as OA
    from oracle.pool import to_f64
    from oracle.replay import Replay

    def bits(t):
        t = t.contiguous()
        return (t.view(torch.int32).numpy().view(np.uint32) if t.dtype == torch.float32
                else t.view(torch.int16).numpy().view(np.uint16))

    base = wl_name[:-len("_fp8")] if wl_name.endswith("_fp8") else wl_name
    if base == "long_context":
        wl = workloads.long_context(S=2)
        sample = "2 of the 16 sequences (32768 tokens, all 8 KV / 64 query heads), one layer"
    elif base == "full_step":
        wl = workloads.full_step(S=16, layers=1)
        sample = "16 sequences of the same length distribution, 1 of 32 layers"
    else:
        wl = workloads.CONFIGS[base]()
        sample = "whole batch, one layer"
    if base != wl_name:
        wl = workloads.fp8_cache(wl)
    from oracle.allocator import NoBlocks
    q, k, v = wl.tensors(0, device="cpu")
    kv_bits = {0: (bits(k), bits(v))}
    g = torch.Generator().manual_seed(5)
    q64 = to_f64(bits(q), wl.dtype)
    state = {}

    def restart():
        # the set-up state again (outside the timing): a small pool runs out
        # of free blocks after enough steps of growth
        state["rp"] = Replay(wl, layers=1).run(wl.setup_ops, kv_bits)
        state["lengths"] = [int(n) - 1 for n in wl.lengths]

    restart()

    def run(budget):
        steps, kv, t = 0, 0, 0.0
        while t < budget or steps == 0:
            kn = torch.randn((wl.S, wl.Hkv, wl.d), generator=g).to(q.dtype)
            vn = torch.randn((wl.S, wl.Hkv, wl.d), generator=g).to(q.dtype)
            rp = state["rp"]
            t0 = time.perf_counter()
            try:
                slots, cow = rp.alloc.append(list(wl.seq_ids))
            except NoBlocks:
                restart()
                continue
            for a, b in cow:
                rp.pool.copy_block(a, b)
            rp.pool.scatter(0, slots, bits(kn), bits(vn))
            lengths = state["lengths"] = [n + 1 for n in state["lengths"]]
            if window:
                for sid, n in zip(wl.seq_ids, lengths):
                    rp.alloc.release_before(sid, max(0, n - window))
            OA.decode(rp.pool, 0, rp.tables(), lengths, q64, wl.Hq, window=window)
            t += time.perf_counter() - t0
            kv += sum(min(n, window) if window else n for n in lengths) * wl.Hkv * wl.kv_bytes_per_token_head()
            steps += 1
        return steps, kv, t

    steps, kv, t = run(seconds)
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        with threadpool_limits(limits=1):
            steps1, kv1, t1 = run(seconds / 3)
        single = {"value": kv1 / t1 / 1e9, "cores": 1, "sample": f"{steps1} decode steps, {t1:.1f} s",
                  "tokens_per_s": wl.S * steps1 / t1}
    except ImportError:
        cores, single = 1, None
    result = {"value": kv / t / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
              "sample": f"{sample}; {steps} decode steps, {t:.1f} s", "tokens_per_s": wl.S * steps / t,
              "single_thread": single, "host": host_info()}
    full_layers = workloads.CONFIGS[base]().layers
    if full_layers > 1:
        # The sample times one layer; a step of the whole model runs that many layers, each costing about
        # the same per token (the work is proportional to the KV bytes), so tokens/s divides by the layers.
        result["tokens_per_s_all_layers"] = result["tokens_per_s"] / full_layers
        result["extrapolation"] = f"one-layer sample time x {full_layers} layers per step"
    return result


def load_traffic(workload: str):
    """HBM bytes per launch of the partial kernel, from the committed counter
    summary profiles/decode_partial_<workload>_traffic.md, if it was taken on
    the current kernel source (its `kernel_sha:` line)."""
    path = os.path.join(TRAFFIC_DIR, f"decode_partial_{workload}_traffic.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        line = line.strip().lstrip("-* ").strip()
        if ":" in line and line.startswith(("kernel_sha", "traffic_bytes_per_launch")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_sha") != kernel_hash() or "traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["traffic_bytes_per_launch"])


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the decode path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads

    Event.use_torch = args.torch_events
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    from paged_kv_cache_08_amd import pkv
    if not os.path.exists(pkv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()

    wl = workloads.CONFIGS[args.config]()
    given = args                                  # --steps as given, for the 32-layer step below
    args = with_steps(args, wl)
    if wl.chunk is not None:
        run_prefill(args, wl)
        return
    bench, t = run_decode(args, wl)
    elapsed, value, k3_ms, k3_avg_s, kv_per_launch, achieved = (t[k] for k in (
        "elapsed", "value", "k3_ms", "k3_avg_s", "kv_per_launch", "achieved"))
    logical = bench.attended_bytes(0)              # the last step's bytes per layer, logical and unique
    unique = bench.unique_bytes()
    traffic_bytes = load_traffic(args.config) if not args.window else None
    traffic = None if traffic_bytes is None else round(traffic_bytes / k3_avg_s / 1e9, 2)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description, "kv_cache": wl.cache_dtype,
                   "layers": wl.layers,
                   "S": wl.S, "Hq": wl.Hq, "Hkv": wl.Hkv, "d": wl.d, "block": wl.block,
                   "partition": args.partition or 512, "window": args.window, "cache_flush": args.flush,
                   "append": "fused into the decode kernel" if bench.fused_append else "separate kernel",
                   "table_upload": f"{bench.table_stream} stream",
                   "events": "torch" if Event.use_torch else "HIP, no system fence",
                   "start_lengths_mean": float(wl.lengths.mean())},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        # Blocks shared between sequences (a common prefix) are read by each of them; their unique bytes
        # may stay in the MALL, so such a rate on logical bytes is cache-assisted.
        "kv_bytes_unique_per_layer": unique,
        "value_unique_bytes": round(value * unique / logical, 2),
        "cache_assisted": unique < logical,
        # a model step runs every layer: tokens/s of a one-layer batch is a per-layer rate
        ("decode_tokens_per_s" if wl.layers > 1 else "decode_tokens_per_s_one_layer"):
            round(wl.S * args.steps / elapsed, 1),
        "parity": t["parity"],
        "roofline": {"bound": "hbm", "kernel": "decode_partial", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "traffic_bytes_per_launch": traffic_bytes,
                     "avg_launch_us": round(k3_avg_s * 1e6, 2), "launch_us": launch_stats_us(k3_ms),
                     "launches_timed": len(k3_ms),
                     "algorithmic_bytes_per_launch": int(kv_per_launch)},
    }
    log(f"timed {args.steps} steps: {value:.1f} GB/s; partial kernel {k3_avg_s * 1e6:.1f} us")
    log("read ceiling")
    # tiles as the kernel reads them: one (block, KV head) of K or V, 16 x d values
    tile = 16 * wl.d * {"f32": 4, "bf16": 2, "fp8": 1}[wl.cache_dtype]
    ceiling = read_ceiling(int(kv_per_launch), tile_bytes=tile if tile in (1024, 2048, 4096) else 4096)
    ceiling["decode_frac_of_gather"] = round(achieved / ceiling["gather_gbs"], 4)
    result["read_ceiling"] = ceiling
    log(f"read ceiling: gather {ceiling['gather_gbs']} GB/s, stream {ceiling['stream_gbs']} GB/s")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(args.config, args.cpu_seconds, args.window)
    if args.config == "long_context" and not args.window and not args.no_full_step:
        del bench
        torch.cuda.empty_cache()
        result["full_step"] = full_step_extra(given)
    print(json.dumps(result), flush=True)


def run_decode(args, wl):
    """Set up a decode batch, validate its first step against the oracle
    (unless --no-cpu-baseline), run the warmup steps, then time args.steps
    steps.  Returns the bench and its timings."""
    import torch
    total = args.warmup + args.steps + 1           # + the validated first step
    log(f"setup {wl.description}")
    bench = DecodeBench(wl, total, partition=args.partition, window=args.window,
                        fused_append=not args.separate_append, table_stream=args.table_stream)
    if args.flush:
        bench.enable_flush()
    parity = None
    if args.no_cpu_baseline:
        bench.step(record_events=False)
    else:
        log("validating the first step against the oracle")
        longest = int(max(range(wl.S), key=lambda i: wl.lengths[i]))
        shortest = int(min(range(wl.S), key=lambda i: wl.lengths[i]))
        seqs = sorted({0, wl.S // 2, wl.S - 1, longest, shortest})
        layers = sorted({0, wl.layers - 1})
        parity = validate_first_step(bench, layers, seqs)
    log("warmup")
    for _ in range(args.warmup):
        bench.step(record_events=False)
    torch.cuda.synchronize()
    log("timed steps")
    bench.kv_bytes.clear()
    gc.collect()
    gc.disable()                  # no collector pause inside the timed steps
    try:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            bench.step(record_events=True)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    finally:
        gc.enable()
    if args.flush:      # the flush writes are not part of the step
        elapsed = sum(a.elapsed_time(b) for a, b in bench.step_events) / 1e3
    k3_ms = [a.elapsed_time(b) for a, b, _ in bench.events]
    k3_avg_s = sum(k3_ms) / len(k3_ms) / 1e3
    kv_per_launch = sum(n for _, _, n in bench.events) / len(bench.events)   # bytes of the timed launches
    return bench, {"elapsed": elapsed, "value": sum(bench.kv_bytes) / elapsed / 1e9, "k3_ms": k3_ms,
                   "k3_avg_s": k3_avg_s, "kv_per_launch": kv_per_launch,
                   "achieved": kv_per_launch / k3_avg_s / 1e9, "parity": parity}


def full_step_extra(args):
    """The 32-layer decode step (256 sequences, MHA) in the same run as the
    headline: the metric's decode tokens/s is a model step's rate."""
    import workloads
    wl = workloads.full_step()
    args = with_steps(args, wl)
    bench, t = run_decode(args, wl)
    out = {"workload": wl.name, "description": wl.description, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(t["elapsed"] / args.steps * 1e3, 4),
           "decode_tokens_per_s": round(wl.S * args.steps / t["elapsed"], 1),
           "kv_gbs": round(t["value"], 2), "pct_hbm_peak": round(100 * t["value"] / HBM_PEAK_GBS, 2),
           "append": "fused into the decode kernel" if bench.fused_append else "separate kernel",
           "table_upload": f"{bench.table_stream} stream",
           "partial_kernel": {"avg_launch_us": round(t["k3_avg_s"] * 1e6, 2), "launch_us": launch_stats_us(t["k3_ms"]),
                              "launches_timed": len(t["k3_ms"]), "achieved": round(t["achieved"], 2),
                              "frac": round(t["achieved"] / HBM_PEAK_GBS, 4),
                              "algorithmic_bytes_per_launch": int(t["kv_per_launch"])},
           "parity": t["parity"]}
    log(f"full step: {out['ms_per_step']} ms/step, {out['decode_tokens_per_s']} tokens/s, "
        f"{out['kv_gbs']} GB/s; partial kernel {out['partial_kernel']['avg_launch_us']} us")
    del bench
    return out


if __name__ == "__main__":
    main()
