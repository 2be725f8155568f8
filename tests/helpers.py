"""Test-side helpers: tensor <-> bit-pattern views and oracle runs."""
import math

import numpy as np
import torch

from oracle import attention as OA
from oracle.pool import to_f64
from oracle.replay import Replay


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a CPU fp32 / bf16 / uint8 tensor as uint32 /
    uint16 / uint8."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.uint8:
        return t.numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)


def oracle_run(wl, q, k, v, layer=0, heads=None, scale=None, window=0, extra_ops=()):
    """Replay the workload's setup + step (+ extra_ops) on the oracle and
    decode one layer.  Returns (replay, out_f64 [S][Hq][d])."""
    rp = Replay(wl, layers=max(wl.layers, layer + 1))
    rp.run(wl.setup_ops + wl.step_ops + list(extra_ops), values={layer: (bits(k), bits(v))})
    q64 = to_f64(bits(q), wl.dtype)
    out = OA.decode(rp.pool, layer, rp.tables(), rp.lengths(), q64, wl.Hq, scale=scale, heads=heads,
                    window=window)
    return rp, out


def brute_force(wl, q, k, v, scale=None, window=0):
    """Pure-Python loops over the logical (unpaged) tensors: the definition
    softmax(q·K/sqrt(d))·V, query head h reading KV head h // (Hq/Hkv), over
    the last ``window`` tokens when window > 0."""
    G = wl.Hq // wl.Hkv
    d = wl.d
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    qq = q.to(torch.float64).tolist()
    kk = k.to(torch.float64).tolist()
    vv = v.to(torch.float64).tolist()
    offs = [int(x) for x in wl.offsets]
    out = []
    for s in range(wl.S):
        n = int(wl.lengths[s])
        t0 = max(0, n - window) if window > 0 else 0
        rows = []
        for h in range(wl.Hq):
            g = h // G
            sc = []
            for t in range(t0, n):
                kt = kk[offs[s] + t][g]
                sc.append(sum(qq[s][h][j] * kt[j] for j in range(d)) * scale)
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            z = sum(w)
            rows.append([sum(w[t - t0] * vv[offs[s] + t][g][j] for t in range(t0, n)) / z for j in range(d)])
        out.append(rows)
    return np.array(out)
