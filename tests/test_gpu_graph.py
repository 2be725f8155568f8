"""HIP graph capture of the decode call.  A serving loop that replays its
step from a graph needs the decode launches (the partial kernel, with the
step's new token written by it or by the append kernel first, and the
reduce) to be capturable: they take every input by pointer and make no
allocation, copy or memset.  The call is captured once and replayed three
times; between replays the program's own eager kernels write new queries,
and after each replay the same call made eagerly must give the same bits.
The first replay is also checked against the oracle."""
import pytest
import torch

import workloads
from gpu_common import (compare_out, gpu_bits, need_gpu, note, oracle_out, oracle_replay, run_gpu,
                        step_inputs)

pytestmark = pytest.mark.gpu

CASES = {
    # multi-partition rows (reduce), four query heads per KV head, new token written by the partial kernel
    "bf16, fused append": (lambda: workloads.random_small(501, S=6, Hq=16, Hkv=4, d=128, dtype="bf16",
                                                          max_len=1800), True),
    "8-bit cache, fused append": (lambda: workloads.fp8_cache(workloads.random_small(
        502, S=5, Hq=16, Hkv=2, d=128, dtype="bf16", max_len=1300)), True),
    # above 1024 (sequence, KV head) rows the call runs the append kernel first
    "bf16, append kernel first": (lambda: workloads.random_small(503, S=160, Hq=8, Hkv=8, d=64, dtype="bf16",
                                                                 max_len=150), True),
    "bf16, no new token": (lambda: workloads.random_small(504, S=7, Hq=8, Hkv=2, d=128, dtype="bf16",
                                                          max_len=2200), False),
}


@pytest.mark.parametrize("static", [False, True], ids=["caller workspace", "static workspace"])
@pytest.mark.parametrize("case", list(CASES))
def test_decode_replays_from_a_graph(case, static):
    need_gpu()
    from paged_kv_cache_08_amd import pkv as P
    make, with_token = CASES[case]
    wl = make()
    note(f"graph: {case}, {'static' if static else 'caller'} workspace: {wl.description}")
    q, k, v = wl.tensors(device="cuda")
    eng, _, _ = run_gpu(wl, {0: k}, {0: v})
    kn = vn = None
    if with_token:                      # the step's own token again: the fused write is idempotent
        _, rows = step_inputs(wl, k)
        kn, vn = k.index_select(0, rows).contiguous(), v.index_select(0, rows).contiguous()
    call = P.pkv_paged_attention_decode_static if static else P.pkv_paged_attention_decode

    def args(out):
        a = eng.decode_args(0, q, out, wl.max_len)
        P.set_new_token(a, kn, vn)
        if static:
            a.workspace, a.workspace_bytes = None, 0
        return a

    out_eager = torch.empty_like(q)
    a_eager = args(out_eager)
    call(a_eager)                       # eager first: one-time set-up happens outside the capture
    torch.cuda.synchronize()

    out_graph = torch.full_like(q, float("nan"))
    a_graph = args(out_graph)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(a_graph)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    for r in range(3):
        if r:
            q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(q.dtype))   # eager work
        out_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        call(a_eager)
        torch.cuda.synchronize()
        assert (gpu_bits(out_graph) == gpu_bits(out_eager)).all(), f"replay {r} differs from the eager call"
        if r == 0:
            rp = oracle_replay(wl, {0: k}, {0: v})
            e = compare_out(out_graph, oracle_out(rp, wl, q))
            note(f"  replay 0 against the oracle: max_abs={e[0]:.3e} row_rel={e[1]:.3e}")
    del g
