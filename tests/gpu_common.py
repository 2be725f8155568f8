"""Shared pieces of the GPU parity tests: run a workload through the library
on the GPU, replay it on the oracle, compare."""
import math
import sys

import numpy as np
import pytest
import torch

from helpers import bits
from oracle import attention as OA
from oracle.pool import to_f64
from oracle.replay import Replay

ATOL = 2e-2          # max |gpu - oracle| over all elements
ROW_RTOL = 1e-2      # max over (s, h) of ||gpu - oracle||_inf / ||oracle||_inf


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_bits(t: torch.Tensor) -> np.ndarray:
    return bits(t.detach().cpu())


def run_gpu(wl, k_log, v_log, q=None, layers=(0,), partition=0, scale=None, engine_layers=None):
    """Build the batch on the GPU through the library; optionally decode
    layer 0 with q.  k_log / v_log: {layer: device tensor}."""
    from paged_kv_cache_08_amd.engine import PagedDecodeEngine
    eng = PagedDecodeEngine(engine_layers or (max(layers) + 1), wl.Hkv, wl.d, wl.num_blocks, wl.cache_dtype,
                            init_perm=wl.perm, partition=partition)
    log = eng.run_script(wl.setup_ops + wl.step_ops, wl, k_log, v_log, layers=layers)
    eng.sync(wl.seq_ids)
    out = {}
    if q is not None:
        for l in layers:
            out[l] = eng.decode(l, q[l] if isinstance(q, dict) else q, max_seq_len=wl.max_len, scale=scale)
    torch.cuda.synchronize()
    return eng, log, out


def oracle_replay(wl, k_log, v_log, layers=(0,), extra_ops=()):
    rp = Replay(wl, layers=max(layers) + 1)
    vals = {l: (bits(k_log[l].cpu()), bits(v_log[l].cpu())) for l in layers}
    rp.run(wl.setup_ops + wl.step_ops + list(extra_ops), vals)
    return rp


def check_allocator(eng, rp, log):
    assert eng.snapshot() == tuple(rp.alloc.snapshot())
    assert len(log) == len(rp.log)
    for (kind, ids, slots, cow), (okind, oids, oslots, ocow) in zip(log, rp.log):
        assert kind == okind and list(map(int, slots)) == list(oslots)
        assert cow == [tuple(p) for p in ocow]


def check_pool(eng, rp, layer=0):
    """GPU pool == oracle pool, bit for bit, including NaN poison elsewhere."""
    ok = rp.pool.K[layer]
    gk = gpu_bits(eng.k[layer]).reshape(ok.shape)
    assert np.array_equal(gk, ok), "K pool differs"
    ov = rp.pool.V[layer]
    gv = gpu_bits(eng.v[layer]).reshape(ov.shape)
    assert np.array_equal(gv, ov), "V pool differs"
    if rp.pool.dtype == "fp8":
        for name, o, g in (("K", rp.pool.KS[layer], eng.ks[layer]), ("V", rp.pool.VS[layer], eng.vs[layer])):
            assert np.array_equal(gpu_bits(g).reshape(o.shape), o), f"{name} scales differ"


def compare_out(gpu_out: torch.Tensor, ref: np.ndarray, rows=None):
    """Tolerance check; rows: optional list of (s, h) to compare."""
    g = gpu_out.detach().float().cpu().double().numpy()
    if rows is not None:
        g = np.stack([g[s, h] for s, h in rows])
        ref = np.stack([ref[s, h] for s, h in rows])
    else:
        g = g.reshape(-1, g.shape[-1])
        ref = ref.reshape(-1, ref.shape[-1])
    assert np.all(np.isfinite(g)), "non-finite output"
    err = np.abs(g - ref)
    max_abs = float(err.max())
    row_rel = float((err.max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-300)).max())
    assert max_abs <= ATOL, f"max abs err {max_abs}"
    assert row_rel <= ROW_RTOL, f"row-normwise rel err {row_rel}"
    return max_abs, row_rel


def oracle_out(rp, wl, q, layer=0, rows=None, scale=None, window=0):
    q64 = to_f64(bits(q.cpu()), wl.dtype)
    heads = None if rows is None else set(rows)
    return OA.decode(rp.pool, layer, rp.tables(), rp.lengths(), q64, wl.Hq, scale=scale, heads=heads,
                     window=window)


def step_inputs(wl, k_log):
    """The checked step's new token of each batch row ([S][Hkv][d] views of
    the logical tensors) and the ids, for a workload whose step appends one
    token per sequence in batch order."""
    (kind, entries), = wl.step_ops
    assert kind == "append"
    ids = [e[0] for e in entries]
    assert ids == list(wl.seq_ids)
    rows = torch.tensor([wl.offsets[src] + pos for (_, src, pos) in entries], device=k_log.device)
    return ids, rows


def decode_step(wl, k_log, v_log, q, fused, layers=(0,), engine_layers=None, partition=0, window=0):
    """Run the workload's setup, then its decode step the way a serving loop
    does: host slot reservation, table upload, and per layer the new token's
    K/V plus attention — handed to the decode call (fused: the library
    appends, in its partial kernel where it fuses) or written first by
    kv_append_last.  k_log / v_log / q: {layer: device tensor}; engine layer
    i holds layers[i].  Returns (engine, {layer: out})."""
    from paged_kv_cache_08_amd import pkv as P
    from paged_kv_cache_08_amd.engine import PagedDecodeEngine
    eng = PagedDecodeEngine(engine_layers or len(layers), wl.Hkv, wl.d, wl.num_blocks, wl.cache_dtype,
                            init_perm=wl.perm, partition=partition)
    eng.run_script(wl.setup_ops, wl, {i: k_log[l] for i, l in enumerate(layers)},
                   {i: v_log[l] for i, l in enumerate(layers)}, layers=range(len(layers)))
    ids, rows = step_inputs(wl, k_log[layers[0]])
    new = {i: (k_log[l].index_select(0, rows).contiguous(), v_log[l].index_select(0, rows).contiguous())
           for i, l in enumerate(layers)}
    if fused:
        _, cow = P.pkv_append_slots(eng.pool, ids)
        if cow:
            P.pkv_copy_blocks(eng.pool, cow)
        eng.sync(ids)
    else:
        eng.step_append(ids, new)
    out = {}
    for i, l in enumerate(layers):
        kn, vn = new[i] if fused else (None, None)
        out[l] = eng.decode(i, q[l], max_seq_len=wl.max_len, window=window, k_new=kn, v_new=vn)
    torch.cuda.synchronize()
    return eng, out


def check_same_bits(a, b, what):
    assert np.array_equal(gpu_bits(a), gpu_bits(b)), f"{what} differs"


def check_pool_layer(eng, i, rp, layer):
    """Engine layer i against the oracle pool's layer `layer`, bit for bit."""
    for name, o, g in (("K", rp.pool.K[layer], eng.k[i]), ("V", rp.pool.V[layer], eng.v[i])):
        assert np.array_equal(gpu_bits(g).reshape(o.shape), o), f"{name} pool differs (layer {layer})"
    if rp.pool.dtype == "fp8":
        for name, o, g in (("K", rp.pool.KS[layer], eng.ks[i]), ("V", rp.pool.VS[layer], eng.vs[i])):
            assert np.array_equal(gpu_bits(g).reshape(o.shape), o), f"{name} scales differ (layer {layer})"
