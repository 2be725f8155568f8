"""The C-ABI library loads, exports every declared symbol, and validates
arguments on the host (no GPU work is started here)."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

import paged_kv_cache_08_amd.pkv as P

HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for want in ["pkv_pool_create", "pkv_pool_destroy", "pkv_seq_create", "pkv_seq_fork", "pkv_seq_free",
                 "pkv_seq_extend", "pkv_append_slots", "pkv_sync_tables", "pkv_copy_blocks",
                 "pkv_kv_append", "pkv_decode_workspace_bytes", "pkv_paged_attention_decode",
                 "pkv_paged_decode_partial", "pkv_paged_decode_reduce", "pkv_pool_stats",
                 "pkv_pool_snapshot", "pkv_status_string", "pkv_last_error"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = P.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (pkv_[a-z_0-9]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported
    # the binding covers every declared function
    assert set(declared_functions()) == {n for n, _, _ in P.SIGNATURES}


def test_library_has_gfx950_code_object():
    # the offload bundle embedded in the library names its target
    data = open(P.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_status_strings():
    assert P.pkv_status_string(0) == "PKV_OK"
    assert P.pkv_status_string(-2) == "PKV_ERR_NO_BLOCKS"
    assert P.pkv_status_string(-5) == "PKV_ERR_UNSUPPORTED"


def test_pool_create_validation():
    with pytest.raises(P.PkvError) as e:
        P.pkv_pool_create(1, 8, 100, 16, 10, P.PKV_BF16)     # 200 bytes: not a multiple of 16
    assert e.value.status == P.PKV_ERR_INVALID
    with pytest.raises(P.PkvError):
        P.pkv_pool_create(1, 8, 128, 16, 4, P.PKV_BF16, init_perm=[0, 1, 1, 2])
    with pytest.raises(P.PkvError):
        P.pkv_pool_create(0, 8, 128, 16, 4, P.PKV_BF16)


def test_fp8_pool_create_validation():
    P.pkv_pool_create(1, 8, 128, 16, 10, P.PKV_FP8_E4M3)            # allocator only: fine
    for kw in (dict(head_dim=96), dict(block_size=32)):
        args = dict(num_layers=1, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=10,
                    dtype=P.PKV_FP8_E4M3)
        args.update(kw)
        with pytest.raises(P.PkvError) as e:
            P.pkv_pool_create(**args)
        assert e.value.status == P.PKV_ERR_INVALID
    # caches without scale arrays (pointers are only checked, never read)
    with pytest.raises(P.PkvError) as e:
        P.pkv_pool_create(1, 8, 128, 16, 10, P.PKV_FP8_E4M3, k_cache=[16], v_cache=[16])
    assert "scale" in P.pkv_last_error()
    with pytest.raises(P.PkvError):
        P.pkv_pool_create(1, 8, 128, 16, 10, P.PKV_FP8_E4M3, k_cache=[16], v_cache=[16],
                          k_scale=[16], v_scale=[4])
    P.pkv_pool_create(1, 8, 128, 16, 10, P.PKV_FP8_E4M3, k_cache=[16], v_cache=[16], k_scale=[32], v_scale=[48])


def test_device_calls_rejected_without_caches():
    pool = P.pkv_pool_create(1, 1, 64, 16, 8, P.PKV_F32)
    with pytest.raises(P.PkvError) as e:
        P.pkv_copy_blocks(pool, [(0, 1)], stream=0)
    assert e.value.status == P.PKV_ERR_INVALID
    assert "no device caches" in P.pkv_last_error()


def _args(**kw):
    a = P.pkv_decode_args()
    base = dict(q=16, out=16, k_cache=16, v_cache=16, block_tables=16, seq_lens=16, workspace=0,
                workspace_bytes=0, num_seqs=2, num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                num_blocks=10, max_blocks=4, max_seq_len=64, partition=0, dtype=P.PKV_BF16, scale=0.1,
                kv_dtype=P.PKV_BF16)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("bad,status", [
    (dict(num_q_heads=7), P.PKV_ERR_INVALID),
    (dict(head_dim=96), P.PKV_ERR_UNSUPPORTED),
    (dict(block_size=32), P.PKV_ERR_UNSUPPORTED),
    (dict(partition=48), P.PKV_ERR_INVALID),
    (dict(partition=2048), P.PKV_ERR_INVALID),
    (dict(num_seqs=0), P.PKV_ERR_INVALID),
    (dict(q=0), P.PKV_ERR_INVALID),
    (dict(q=8), P.PKV_ERR_INVALID),                       # misaligned
    (dict(max_seq_len=4096), P.PKV_ERR_INVALID),          # needs a workspace
    (dict(dtype=7), P.PKV_ERR_INVALID),
    (dict(kv_dtype=P.PKV_F32), P.PKV_ERR_INVALID),       # cache type differs from bf16 queries
    (dict(dtype=P.PKV_F32, kv_dtype=P.PKV_FP8_E4M3), P.PKV_ERR_INVALID),
    (dict(kv_dtype=P.PKV_FP8_E4M3), P.PKV_ERR_INVALID),  # no scale arrays
    (dict(kv_dtype=P.PKV_FP8_E4M3, k_scale=16, v_scale=8), P.PKV_ERR_INVALID),   # misaligned
    (dict(kv_dtype=P.PKV_FP8_E4M3, k_scale=16, v_scale=16, head_dim=96), P.PKV_ERR_UNSUPPORTED),
    (dict(k_new=16), P.PKV_ERR_INVALID),                  # fused append: k_new without v_new
    (dict(v_new=16), P.PKV_ERR_INVALID),
    (dict(k_new=24, v_new=16), P.PKV_ERR_INVALID),        # misaligned
])
def test_decode_argument_validation(bad, status):
    with pytest.raises(P.PkvError) as e:
        P.pkv_paged_attention_decode(_args(**bad), stream=0)
    assert e.value.status == status


def test_workspace_bytes():
    assert P.pkv_decode_workspace_bytes(4, 8, 128, 512, 0) == 0
    rows = 16 * 64 * 64
    ml = (rows * 8 + 255) // 256 * 256
    assert P.pkv_decode_workspace_bytes(16, 64, 128, 32768, 512) == ml + rows * 128 * 4


def _prefill_args(**kw):
    a = P.pkv_prefill_args()
    base = dict(q=16, out=16, k_cache=16, v_cache=16, block_tables=16, seq_lens=16, query_start=16, num_seqs=2,
                num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16, num_blocks=10, max_blocks=4,
                max_seq_len=64, max_query_len=32, dtype=P.PKV_BF16, scale=0.1, window=0)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("bad,status", [
    (dict(dtype=P.PKV_F32), P.PKV_ERR_UNSUPPORTED),
    (dict(num_q_heads=7), P.PKV_ERR_INVALID),
    (dict(head_dim=96), P.PKV_ERR_UNSUPPORTED),
    (dict(window=-1), P.PKV_ERR_INVALID),
    (dict(scale=0.0), P.PKV_ERR_INVALID),         # the kernel keeps raw scores: the scale must be > 0
    (dict(scale=-0.1), P.PKV_ERR_INVALID),
    (dict(scale=float("inf")), P.PKV_ERR_INVALID),
    (dict(scale=float("nan")), P.PKV_ERR_INVALID),
    (dict(query_start=0), P.PKV_ERR_INVALID),
    (dict(q=8), P.PKV_ERR_INVALID),                # misaligned
    # an 8-bit cache needs its scales and a 256-byte aligned workspace of the stated size
    (dict(dtype=P.PKV_FP8_E4M3, workspace=256, workspace_bytes=1 << 30), P.PKV_ERR_INVALID),
    (dict(dtype=P.PKV_FP8_E4M3, k_scale=16, v_scale=16), P.PKV_ERR_INVALID),
    (dict(dtype=P.PKV_FP8_E4M3, k_scale=16, v_scale=16, workspace=256, workspace_bytes=1000), P.PKV_ERR_INVALID),
    (dict(dtype=P.PKV_FP8_E4M3, k_scale=16, v_scale=16, workspace=16, workspace_bytes=1 << 30), P.PKV_ERR_INVALID),
])
def test_prefill_argument_validation(bad, status):
    with pytest.raises(P.PkvError) as e:
        P.pkv_paged_prefill(_prefill_args(**bad), stream=0)
    assert e.value.status == status


def test_prefill_workspace_bytes():
    # bf16 needs none; 8-bit: int32 tables [S][max_blocks], then K and V bf16 copies of
    # S * ceil(max_seq_len / B) blocks, each part rounded up to 256 bytes
    assert P.pkv_prefill_workspace_bytes(2, 2, 128, 16, 4, 64, P.PKV_BF16) == 0
    up = lambda x: -(-x // 256) * 256
    S, Hkv, d, B, mb, msl = 3, 2, 128, 16, 7, 100
    copy = up(S * (-(-msl // B)) * Hkv * B * d * 2)
    assert P.pkv_prefill_workspace_bytes(S, Hkv, d, B, mb, msl, P.PKV_FP8_E4M3) == up(S * mb * 4) + 2 * copy
    assert P.pkv_prefill_workspace_bytes(0, Hkv, d, B, mb, msl, P.PKV_FP8_E4M3) == 0


@pytest.mark.parametrize("args", [
    (0, 1 << 20, 0, 16, 1, 16),             # null buffer
    (16, 1 << 20, 0, 16, 1, 0),             # null sink
    (16, 1000, 0, 1, 1, 16),                # buffer smaller than one tile
    (16, 1 << 20, 0, 0, 1, 16),             # no tiles
    (16, 1 << 20, 0, 16, 0, 16),            # tiles_per_wave < 1
    (8, 1 << 20, 0, 16, 1, 16),             # misaligned buffer
    (16, 1 << 20, 0, 1025, 1, 16),          # contiguous read past the buffer (at most 1024 tiles)
])
@pytest.mark.parametrize("tile_bytes", [4096, 1024, 3000])
def test_read_tiles_argument_validation(args, tile_bytes):
    base, nbytes, order, n, tpw, sink = args
    status = P.lib().pkv_read_tiles(base, nbytes, tile_bytes, order, n, tpw, sink, 0)
    assert status == P.PKV_ERR_INVALID


def test_read_tiles_2k_tiles_count_against_the_buffer():
    # 513 tiles of 2 KiB do not fit in 1 MiB; with no device the valid call is not made
    assert P.lib().pkv_read_tiles(16, 1 << 20, 2048, 0, 513, 1, 16, 0) == P.PKV_ERR_INVALID


@pytest.mark.parametrize("kw,fused", [
    (dict(), 0),                                          # nothing to append
    (dict(k_new=16, v_new=16), 1),
    (dict(k_new=16, v_new=16, num_q_heads=64), 1),        # 32 query heads per KV head: every head group
                                                          #   substitutes the token, group 0 stores it
    (dict(k_new=16, v_new=16, num_seqs=513), 0),          # 1026 (sequence, KV head) rows: append kernel first
    (dict(k_new=16, v_new=16, num_seqs=512), 1),          # 1024 rows
    (dict(k_new=16, v_new=16, dtype=P.PKV_F32, kv_dtype=P.PKV_F32), 0),   # fp32 cache: append kernel first
])
def test_decode_fuses_append(kw, fused):
    assert P.lib().pkv_decode_fuses_append(P.ctypes.byref(_args(**kw))) == fused


def test_decode_fuses_append_rejects_bad_args():
    assert P.lib().pkv_decode_fuses_append(P.ctypes.byref(_args(k_new=16))) == P.PKV_ERR_INVALID


def test_static_decode_rejects_batches_beyond_its_workspace():
    # 64 x 64 heads x 128 partitions of d = 128: about 272 MB of workspace, more than the 64 MiB
    a = _args(num_seqs=64, num_q_heads=64, num_kv_heads=8, max_seq_len=65536, max_blocks=4096)
    assert P.lib().pkv_paged_attention_decode_static(P.ctypes.byref(a), None) == P.PKV_ERR_INVALID
    assert "workspace" in P.pkv_last_error()
    # invalid arguments are reported as by the caller-workspace call
    assert P.lib().pkv_paged_attention_decode_static(P.ctypes.byref(_args(num_q_heads=7)), None) == P.PKV_ERR_INVALID
