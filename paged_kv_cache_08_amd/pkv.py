"""Python binding of libpkv (include/pkv.h): same names, argument marshalling only.

Device arrays are passed as torch tensors (their ``data_ptr()``); streams
default to torch's current stream.  Every step runs in the library's own
host code and HIP kernels; if ``libpkv.so`` is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIB selects another build of the library (e.g. a tuning variant)
LIB_PATH = os.environ.get("PKV_LIB") or os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID = -1
PKV_ERR_NO_BLOCKS = -2
PKV_ERR_BAD_SEQ = -3
PKV_ERR_HIP = -4
PKV_ERR_UNSUPPORTED = -5
PKV_F32 = 0
PKV_BF16 = 1
PKV_FP8_E4M3 = 2

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_P = ctypes.POINTER


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{pkv_status_string(status)}: {message}")
        self.status = status


class pkv_pool_desc(ctypes.Structure):
    _fields_ = [("num_layers", _i32), ("num_kv_heads", _i32), ("head_dim", _i32),
                ("block_size", _i32), ("num_blocks", _i32), ("dtype", _i32),
                ("k_cache", _P(_vp)), ("v_cache", _P(_vp)), ("init_perm", _P(_i32)),
                ("k_scale", _P(_vp)), ("v_scale", _P(_vp))]


class pkv_stats(ctypes.Structure):
    _fields_ = [("num_blocks", _i64), ("free_blocks", _i64), ("used_blocks", _i64),
                ("num_seqs", _i64), ("sum_len", _i64), ("sum_ref", _i64), ("tail_waste", _i64)]


class pkv_decode_args(ctypes.Structure):
    _fields_ = [("q", _vp), ("out", _vp), ("k_cache", _vp), ("v_cache", _vp),
                ("block_tables", _vp), ("seq_lens", _vp), ("workspace", _vp),
                ("workspace_bytes", ctypes.c_size_t),
                ("num_seqs", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32),
                ("head_dim", _i32), ("block_size", _i32), ("num_blocks", _i32),
                ("max_blocks", _i32), ("max_seq_len", _i32), ("partition", _i32),
                ("dtype", _i32), ("scale", ctypes.c_float), ("host_seq_lens", _vp),
                ("k_scale", _vp), ("v_scale", _vp), ("kv_dtype", _i32), ("window", _i32),
                ("k_new", _vp), ("v_new", _vp)]


class pkv_decode_plan_info(ctypes.Structure):
    _fields_ = [("cells", _i64), ("listed_cells", _i64), ("head_groups", _i32), ("pipeline_depth", _i32), ("resident_waves", _i32),
                ("partitions_per_wave", _i32), ("work_list", _i32), ("run_cap", _i32),
                ("max_wave_blocks", _i32), ("fused_append", _i32), ("partitions_bound", _i32),
                ("lds_bytes", _i32)]


class pkv_prefill_args(ctypes.Structure):
    _fields_ = [("q", _vp), ("out", _vp), ("k_cache", _vp), ("v_cache", _vp),
                ("block_tables", _vp), ("seq_lens", _vp), ("query_start", _vp),
                ("num_seqs", _i32), ("num_q_heads", _i32), ("num_kv_heads", _i32),
                ("head_dim", _i32), ("block_size", _i32), ("num_blocks", _i32),
                ("max_blocks", _i32), ("max_seq_len", _i32), ("max_query_len", _i32),
                ("dtype", _i32), ("scale", ctypes.c_float), ("window", _i32),
                ("k_scale", _vp), ("v_scale", _vp), ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t)]


_lib = None

# (name, restype, argtypes) of every exported entry point
SIGNATURES = [
    ("pkv_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("pkv_last_error", ctypes.c_char_p, []),
    ("pkv_version", ctypes.c_int, []),
    ("pkv_pool_create", ctypes.c_int, [_P(pkv_pool_desc), _P(_vp)]),
    ("pkv_pool_destroy", ctypes.c_int, [_vp]),
    ("pkv_seq_create", ctypes.c_int, [_vp, _P(_i64)]),
    ("pkv_seq_fork", ctypes.c_int, [_vp, _i64, _P(_i64)]),
    ("pkv_seq_free", ctypes.c_int, [_vp, _i64]),
    ("pkv_seq_release_before", ctypes.c_int, [_vp, _i64, _i32, _P(_i32)]),
    ("pkv_prefix_register", ctypes.c_int, [_vp, _i64, _P(_i32), _i32, ctypes.c_uint64, _P(_i32)]),
    ("pkv_prefix_match", ctypes.c_int, [_vp, _P(_i32), _i32, ctypes.c_uint64, _P(_i64), _P(_i32)]),
    ("pkv_prefix_evict", ctypes.c_int, [_vp, _i32, _P(_i32)]),
    ("pkv_prefix_clear", ctypes.c_int, [_vp, _P(_i32)]),
    ("pkv_prefix_snapshot", ctypes.c_int, [_vp, _P(_i64), _P(_i64), _P(ctypes.c_uint64), _P(_i64), _P(_i32),
                                           _P(_i64), _P(_i32)]),
    ("pkv_seq_extend", ctypes.c_int, [_vp, _i64, _i32, _P(_i32), _P(_i32), _P(_i32)]),
    ("pkv_append_slots", ctypes.c_int, [_vp, _P(_i64), _i32, _P(_i32), _P(_i32), _P(_i32)]),
    ("pkv_seq_length", ctypes.c_int, [_vp, _i64, _P(_i32)]),
    ("pkv_seq_table", ctypes.c_int, [_vp, _i64, _P(_i32), _i32, _P(_i32)]),
    ("pkv_sync_tables", ctypes.c_int, [_vp, _P(_i64), _i32, _vp, _i32, _vp, _vp, _vp]),
    ("pkv_copy_blocks", ctypes.c_int, [_vp, _P(_i32), _i32, _vp]),
    ("pkv_kv_append", ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _i32, _vp]),
    ("pkv_kv_append_last", ctypes.c_int, [_vp, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _vp]),
    ("pkv_pool_stats", ctypes.c_int, [_vp, _P(pkv_stats)]),
    ("pkv_pool_snapshot", ctypes.c_int, [_vp, _P(_i32), _P(_i32), _P(_i64), _P(_i32), _P(_i64),
                                         _P(_i32), _P(_i64), _P(_i64), _P(_i64), _P(_i64)]),
    ("pkv_decode_workspace_bytes", ctypes.c_size_t, [_i32, _i32, _i32, _i32, _i32]),
    ("pkv_paged_attention_decode", ctypes.c_int, [_P(pkv_decode_args), _vp]),
    ("pkv_paged_attention_decode_static", ctypes.c_int, [_P(pkv_decode_args), _vp]),
    ("pkv_paged_decode_partial", ctypes.c_int, [_P(pkv_decode_args), _vp]),
    ("pkv_paged_decode_reduce", ctypes.c_int, [_P(pkv_decode_args), _vp]),
    ("pkv_decode_fuses_append", ctypes.c_int, [_P(pkv_decode_args)]),
    ("pkv_decode_plan", ctypes.c_int, [_P(pkv_decode_args), _P(pkv_decode_plan_info), _P(_i32), _i64]),
    ("pkv_paged_prefill", ctypes.c_int, [_P(pkv_prefill_args), _vp]),
    ("pkv_prefill_workspace_bytes", ctypes.c_size_t, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    ("pkv_read_tiles", ctypes.c_int, [_vp, _i64, _i32, _vp, _i64, _i32, _vp, _vp]),
]


def lib():
    """Load libpkv.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (loads the HIP runtime libpkv links against)
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m paged_kv_cache_08_amd.build` "
                               "or __graft_entry__.build()")
        l = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _check(status: int) -> None:
    if status != PKV_OK:
        raise PkvError(status, lib().pkv_last_error().decode())


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _i32buf(n):
    return np.zeros(max(n, 1), dtype=np.int32)


def _as_i32p(a: np.ndarray):
    return a.ctypes.data_as(_P(_i32))


def _as_i64p(a: np.ndarray):
    return a.ctypes.data_as(_P(_i64))


# ---------------------------------------------------------------------------
def pkv_status_string(status: int) -> str:
    return lib().pkv_status_string(status).decode()


def pkv_last_error() -> str:
    return lib().pkv_last_error().decode()


def pkv_version() -> int:
    return lib().pkv_version()


class PoolHandle:
    """Owns a pkv_pool*; destroyed by pkv_pool_destroy or garbage collection."""

    def __init__(self, ptr: int, desc: dict):
        self.ptr = ptr
        self.desc = desc

    def __del__(self):
        if getattr(self, "ptr", None) and _lib is not None:
            _lib.pkv_pool_destroy(self.ptr)
            self.ptr = None


def pkv_pool_create(num_layers: int, num_kv_heads: int, head_dim: int, block_size: int,
                    num_blocks: int, dtype: int, k_cache: Optional[Sequence] = None,
                    v_cache: Optional[Sequence] = None, init_perm=None,
                    k_scale: Optional[Sequence] = None, v_scale: Optional[Sequence] = None) -> PoolHandle:
    """k_scale / v_scale: per-layer fp32 scale tensors of an 8-bit pool."""
    d = pkv_pool_desc(num_layers, num_kv_heads, head_dim, block_size, num_blocks, dtype)
    keep = []

    def ptrs(ts):
        arr = (_vp * num_layers)(*[_ptr(t) for t in ts])
        keep.append(arr)
        return ctypes.cast(arr, _P(_vp))
    if k_cache is not None:
        d.k_cache = ptrs(k_cache)
        d.v_cache = ptrs(v_cache)
    if k_scale is not None:
        d.k_scale = ptrs(k_scale)
        d.v_scale = ptrs(v_scale)
    if init_perm is not None:
        perm = np.ascontiguousarray(init_perm, dtype=np.int32)
        d.init_perm = _as_i32p(perm)
        keep.append(perm)
    out = _vp()
    _check(lib().pkv_pool_create(ctypes.byref(d), ctypes.byref(out)))
    return PoolHandle(out.value, dict(num_layers=num_layers, num_kv_heads=num_kv_heads,
                                      head_dim=head_dim, block_size=block_size,
                                      num_blocks=num_blocks, dtype=dtype))


def pkv_pool_destroy(pool: PoolHandle) -> None:
    if pool.ptr:
        st = lib().pkv_pool_destroy(pool.ptr)
        pool.ptr = None
        _check(st)


def pkv_seq_create(pool: PoolHandle) -> int:
    out = _i64()
    _check(lib().pkv_seq_create(pool.ptr, ctypes.byref(out)))
    return out.value


def pkv_seq_fork(pool: PoolHandle, parent: int) -> int:
    out = _i64()
    _check(lib().pkv_seq_fork(pool.ptr, parent, ctypes.byref(out)))
    return out.value


def pkv_seq_free(pool: PoolHandle, seq_id: int) -> None:
    _check(lib().pkv_seq_free(pool.ptr, seq_id))


def pkv_seq_release_before(pool: PoolHandle, seq_id: int, pos: int) -> int:
    """Give back the blocks holding only positions < pos; returns how many."""
    out = _i32()
    _check(lib().pkv_seq_release_before(pool.ptr, seq_id, pos, ctypes.byref(out)))
    return out.value


def pkv_prefix_register(pool: PoolHandle, seq_id: int, tokens: Sequence[int], ns: int) -> int:
    """Enter seq_id's full blocks into the prefix cache; returns new entries."""
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    out = _i32()
    _check(lib().pkv_prefix_register(pool.ptr, seq_id, _as_i32p(t) if len(t) else None, len(t), ns,
                                     ctypes.byref(out)))
    return out.value


def pkv_prefix_match(pool: PoolHandle, tokens: Sequence[int], ns: int) -> Tuple[int, int]:
    """New sequence from the cached chain; returns (seq id, matched tokens)."""
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    sid, got = _i64(), _i32()
    _check(lib().pkv_prefix_match(pool.ptr, _as_i32p(t) if len(t) else None, len(t), ns, ctypes.byref(sid),
                                  ctypes.byref(got)))
    return sid.value, got.value


def pkv_prefix_evict(pool: PoolHandle, max_blocks: int) -> int:
    out = _i32()
    _check(lib().pkv_prefix_evict(pool.ptr, max_blocks, ctypes.byref(out)))
    return out.value


def pkv_prefix_clear(pool: PoolHandle) -> int:
    out = _i32()
    _check(lib().pkv_prefix_clear(pool.ptr, ctypes.byref(out)))
    return out.value


def pkv_prefix_snapshot(pool: PoolHandle):
    """[(entry, ns, parent, tokens, block, last_use)] by entry index."""
    n = _i64()
    L = lib()
    _check(L.pkv_prefix_snapshot(pool.ptr, ctypes.byref(n), None, None, None, None, None, None))
    k = n.value
    B = pool.desc["block_size"]
    e = np.zeros(max(k, 1), dtype=np.int64)
    ns = np.zeros(max(k, 1), dtype=np.uint64)
    par = np.zeros(max(k, 1), dtype=np.int64)
    blk = _i32buf(k)
    use = np.zeros(max(k, 1), dtype=np.int64)
    tok = _i32buf(k * B)
    _check(L.pkv_prefix_snapshot(pool.ptr, ctypes.byref(n), _as_i64p(e), ns.ctypes.data_as(_P(ctypes.c_uint64)),
                                 _as_i64p(par), _as_i32p(blk), _as_i64p(use), _as_i32p(tok)))
    return [(int(e[i]), int(ns[i]), int(par[i]), [int(x) for x in tok[i * B:(i + 1) * B]], int(blk[i]), int(use[i]))
            for i in range(k)]


def _pairs(cow: np.ndarray, n: int) -> List[Tuple[int, int]]:
    return [(int(cow[2 * i]), int(cow[2 * i + 1])) for i in range(n)]


def pkv_seq_extend(pool: PoolHandle, seq_id: int, ntok: int):
    """Returns (slots int32[ntok], [(src, dst)] copy-on-write pairs)."""
    slots = _i32buf(ntok)
    cow = _i32buf(2)
    n_cow = _i32()
    _check(lib().pkv_seq_extend(pool.ptr, seq_id, ntok, _as_i32p(slots), _as_i32p(cow), ctypes.byref(n_cow)))
    return slots[:ntok], _pairs(cow, n_cow.value)


def pkv_append_slots(pool: PoolHandle, ids: Sequence[int]):
    """Returns (slots int32[n], [(src, dst)] copy-on-write pairs)."""
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    n = len(ids)
    slots = _i32buf(n)
    cow = _i32buf(2 * n)
    n_cow = _i32()
    _check(lib().pkv_append_slots(pool.ptr, _as_i64p(ids), n, _as_i32p(slots), _as_i32p(cow),
                                  ctypes.byref(n_cow)))
    return slots[:n], _pairs(cow, n_cow.value)


def pkv_seq_length(pool: PoolHandle, seq_id: int) -> int:
    out = _i32()
    _check(lib().pkv_seq_length(pool.ptr, seq_id, ctypes.byref(out)))
    return out.value


def pkv_seq_table(pool: PoolHandle, seq_id: int) -> List[int]:
    nb = _i32()
    _check(lib().pkv_seq_table(pool.ptr, seq_id, None, 0, ctypes.byref(nb)))
    buf = _i32buf(nb.value)
    _check(lib().pkv_seq_table(pool.ptr, seq_id, _as_i32p(buf), nb.value, ctypes.byref(nb)))
    return [int(x) for x in buf[:nb.value]]


def pkv_sync_tables(pool: PoolHandle, ids: Sequence[int], dev_block_tables, dev_seq_lens,
                    host_seq_lens_out: Optional[np.ndarray] = None, stream=None) -> None:
    """dev_block_tables: int32 device tensor [n][max_blocks]; dev_seq_lens int32 [n];
    host_seq_lens_out: optional int32 numpy array [n] receiving the lengths."""
    ids = np.ascontiguousarray(ids, dtype=np.int64)
    max_blocks = dev_block_tables.shape[1]
    hl = 0
    if host_seq_lens_out is not None:
        assert host_seq_lens_out.dtype == np.int32 and host_seq_lens_out.flags.c_contiguous
        assert host_seq_lens_out.shape[0] >= len(ids)
        hl = host_seq_lens_out.ctypes.data
    _check(lib().pkv_sync_tables(pool.ptr, _as_i64p(ids), len(ids), _ptr(dev_block_tables), max_blocks,
                                 _ptr(dev_seq_lens), hl, _stream(stream)))


def pkv_copy_blocks(pool: PoolHandle, pairs: Sequence[Tuple[int, int]], stream=None) -> None:
    flat = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1))
    _check(lib().pkv_copy_blocks(pool.ptr, _as_i32p(flat), len(flat) // 2, _stream(stream)))


def pkv_kv_append(pool: PoolHandle, layer: int, k_new, v_new, dev_slot_mapping, stream=None) -> None:
    """k_new, v_new: device [n][Hkv][d] in the pool dtype; dev_slot_mapping int32 [n]."""
    n = dev_slot_mapping.shape[0]
    _check(lib().pkv_kv_append(pool.ptr, layer, _ptr(k_new), _ptr(v_new), _ptr(dev_slot_mapping), n,
                               _stream(stream)))


def pkv_kv_append_last(pool: PoolHandle, layer: int, k_new, v_new, dev_block_tables, dev_seq_lens,
                       stream=None) -> None:
    """Write token i of k_new/v_new ([n][Hkv][d]) at the last position of row
    i of the uploaded tables (dev_block_tables [n][max_blocks], dev_seq_lens [n])."""
    n = dev_seq_lens.shape[0]
    _check(lib().pkv_kv_append_last(pool.ptr, layer, _ptr(k_new), _ptr(v_new), _ptr(dev_block_tables),
                                    dev_block_tables.shape[1], _ptr(dev_seq_lens), n, _stream(stream)))


def pkv_pool_stats(pool: PoolHandle) -> dict:
    s = pkv_stats()
    _check(lib().pkv_pool_stats(pool.ptr, ctypes.byref(s)))
    return {f: getattr(s, f) for f, _ in pkv_stats._fields_}


def pkv_pool_snapshot(pool: PoolHandle):
    """(free stack bottom..top, refcounts, [(id, len, table)] by id, next_id)."""
    nf, ns, ne, nid = _i64(), _i64(), _i64(), _i64()
    L = lib()
    _check(L.pkv_pool_snapshot(pool.ptr, None, None, None, None, None, None, ctypes.byref(nf),
                               ctypes.byref(ns), ctypes.byref(ne), ctypes.byref(nid)))
    free = _i32buf(nf.value)
    ref = _i32buf(pool.desc["num_blocks"])
    ids = np.zeros(max(ns.value, 1), dtype=np.int64)
    lens = _i32buf(ns.value)
    off = np.zeros(ns.value + 1, dtype=np.int64)
    tabs = _i32buf(ne.value)
    _check(L.pkv_pool_snapshot(pool.ptr, _as_i32p(free), _as_i32p(ref), _as_i64p(ids), _as_i32p(lens),
                               _as_i64p(off), _as_i32p(tabs), ctypes.byref(nf), ctypes.byref(ns),
                               ctypes.byref(ne), ctypes.byref(nid)))
    seqs = [(int(ids[i]), int(lens[i]), [int(x) for x in tabs[off[i]:off[i + 1]]]) for i in range(ns.value)]
    return [int(x) for x in free[:nf.value]], [int(x) for x in ref[:pool.desc["num_blocks"]]], seqs, nid.value


def pkv_decode_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, max_seq_len: int,
                               partition: int = 0) -> int:
    return lib().pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len, partition)


def decode_args(q, out, k_cache, v_cache, block_tables, seq_lens, num_kv_heads: int, num_blocks: int,
                max_seq_len: int, scale: Optional[float] = None, partition: int = 0, workspace=None,
                block_size: int = 16, host_seq_lens: Optional[np.ndarray] = None,
                k_scale=None, v_scale=None, window: int = 0, k_new=None, v_new=None) -> pkv_decode_args:
    """Pack a pkv_decode_args from tensors (q/out [S][Hq][d]).  host_seq_lens:
    optional int32 numpy array [S] (kept alive by the returned object; it is
    read at every call, so it may be updated in place between calls).  The
    cache type follows the cache tensors' dtype (uint8 = 8-bit E4M3 codes,
    which need the layer's k_scale / v_scale tensors).  k_new / v_new
    ([S][Hkv][d]): the step's new token, appended by the partial kernel
    (set_new_token changes them between calls)."""
    import torch
    S, Hq, d = q.shape
    dtype = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16}[q.dtype]
    a = pkv_decode_args()
    a.q, a.out, a.k_cache, a.v_cache = _ptr(q), _ptr(out), _ptr(k_cache), _ptr(v_cache)
    a.block_tables, a.seq_lens = _ptr(block_tables), _ptr(seq_lens)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.num_seqs, a.num_q_heads, a.num_kv_heads, a.head_dim = S, Hq, num_kv_heads, d
    a.block_size, a.num_blocks = block_size, num_blocks
    a.max_blocks = block_tables.shape[1]
    a.max_seq_len = max_seq_len
    a.partition = partition
    a.dtype = dtype
    a.kv_dtype = PKV_FP8_E4M3 if k_cache.dtype == torch.uint8 else dtype
    a.window = window
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    a.scale = 1.0 / math.sqrt(d) if scale is None else scale
    if host_seq_lens is not None:
        assert host_seq_lens.dtype == np.int32 and host_seq_lens.flags.c_contiguous
        a.host_seq_lens = host_seq_lens.ctypes.data
        a._keep = host_seq_lens
    set_new_token(a, k_new, v_new)
    return a


def set_new_token(a: pkv_decode_args, k_new, v_new) -> None:
    """Point the fused append of decode args `a` at k_new / v_new (device
    [S][Hkv][d], contiguous), or switch it off with None."""
    a.k_new, a.v_new = _ptr(k_new), _ptr(v_new)


def pkv_paged_attention_decode(args: pkv_decode_args, stream=None) -> None:
    _check(lib().pkv_paged_attention_decode(ctypes.byref(args), _stream(stream)))


def pkv_paged_attention_decode_static(args: pkv_decode_args, stream=None) -> None:
    """pkv_paged_attention_decode with the library's own 64 MiB device
    workspace (args.workspace is ignored); allocates nothing."""
    _check(lib().pkv_paged_attention_decode_static(ctypes.byref(args), _stream(stream)))


def pkv_paged_decode_partial(args: pkv_decode_args, stream=None) -> None:
    _check(lib().pkv_paged_decode_partial(ctypes.byref(args), _stream(stream)))


def pkv_paged_decode_reduce(args: pkv_decode_args, stream=None) -> None:
    _check(lib().pkv_paged_decode_reduce(ctypes.byref(args), _stream(stream)))


def pkv_decode_fuses_append(args: pkv_decode_args) -> bool:
    """Whether a decode call with `args` writes k_new / v_new in its partial
    kernel (else it runs the append kernel first, or has nothing to append)."""
    status = lib().pkv_decode_fuses_append(ctypes.byref(args))
    if status < 0:
        _check(status)
    return status == 1


def pkv_decode_plan(args: pkv_decode_args, with_cells: bool = True):
    """The partial kernel's launch plan for `args` (nothing runs): the
    pkv_decode_plan_info and, with `with_cells`, an int32 array [cells][3] of
    (sequence, first partition, end partition) per grid cell."""
    info = pkv_decode_plan_info()
    _check(lib().pkv_decode_plan(ctypes.byref(args), ctypes.byref(info), None, 0))
    if not with_cells:
        return info, None
    cells = np.zeros((info.cells, 3), dtype=np.int32)
    _check(lib().pkv_decode_plan(ctypes.byref(args), ctypes.byref(info),
                                 cells.ctypes.data_as(_P(_i32)), info.cells))
    return info, cells


def prefill_args(q, out, k_cache, v_cache, block_tables, seq_lens, query_start, num_kv_heads: int,
                 num_blocks: int, max_seq_len: int, max_query_len: int, scale: Optional[float] = None,
                 window: int = 0, block_size: int = 16, k_scale=None, v_scale=None,
                 workspace=None) -> pkv_prefill_args:
    """Pack a pkv_prefill_args from tensors: q/out [T][Hq][d] bf16,
    query_start int32 [S + 1] (device), seq_lens int32 [S] (device).  An
    8-bit cache (uint8 tensors) also takes its scales and a device
    workspace of pkv_prefill_workspace_bytes() bytes (a uint8 tensor)."""
    import torch
    T, Hq, d = q.shape
    a = pkv_prefill_args()
    a.q, a.out, a.k_cache, a.v_cache = _ptr(q), _ptr(out), _ptr(k_cache), _ptr(v_cache)
    a.block_tables, a.seq_lens, a.query_start = _ptr(block_tables), _ptr(seq_lens), _ptr(query_start)
    a.num_seqs = seq_lens.shape[0]
    a.num_q_heads, a.num_kv_heads, a.head_dim = Hq, num_kv_heads, d
    a.block_size, a.num_blocks = block_size, num_blocks
    a.max_blocks = block_tables.shape[1]
    a.max_seq_len, a.max_query_len = max_seq_len, max_query_len
    a.dtype = PKV_FP8_E4M3 if k_cache.dtype == torch.uint8 else PKV_BF16
    a.scale = 1.0 / math.sqrt(d) if scale is None else scale
    a.window = window
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    if workspace is not None:
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    return a


def pkv_prefill_workspace_bytes(num_seqs: int, num_kv_heads: int, head_dim: int, block_size: int,
                                max_blocks: int, max_seq_len: int, dtype: int) -> int:
    return lib().pkv_prefill_workspace_bytes(num_seqs, num_kv_heads, head_dim, block_size, max_blocks,
                                             max_seq_len, dtype)


def pkv_paged_prefill(args: pkv_prefill_args, stream=None) -> None:
    _check(lib().pkv_paged_prefill(ctypes.byref(args), _stream(stream)))



def pkv_read_tiles(base, order, n_tiles: int, tiles_per_wave: int, sink, stream=None,
                   tile_bytes: int = 4096) -> None:
    """Read-bandwidth calibration: base is a device tensor (any dtype), order
    a device int32 tensor of tile ids or None (contiguous tiles), sink a
    device int32/uint32 tensor of ceil(n_tiles / tiles_per_wave) * 64 entries;
    tiles of tile_bytes (4096, 2048 or 1024)."""
    waves = -(-n_tiles // tiles_per_wave)
    if sink.numel() < waves * 64 or sink.element_size() != 4:
        raise ValueError("sink needs ceil(n_tiles / tiles_per_wave) * 64 32-bit entries")
    if order is not None and order.numel() < n_tiles:
        raise ValueError("order holds fewer than n_tiles ids")
    _check(lib().pkv_read_tiles(_ptr(base), base.numel() * base.element_size(), tile_bytes, _ptr(order), n_tiles,
                                tiles_per_wave, _ptr(sink), _stream(stream)))
