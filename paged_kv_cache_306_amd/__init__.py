"""paged_kv_cache_306_amd -- paged KV-cache decode path for AMD Instinct MI355X (gfx950).

A thin ctypes binding over libpkv.so (C ABI in include/pkv.h).  Every step of the path --
block allocation, cache writes, block copies and decode attention -- runs in the native
library; this module only marshals torch tensors (device memory, streams) into pointers.
If libpkv.so has not been built, importing the functions raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "lib", "PkvError", "CacheDesc", "decode_workspace_bytes", "decode_partition_tokens",
    "decode_schedule", "decode_xcd_grid", "decode_xcd_slot_unit",
    "paged_attention_decode", "paged_attention_decode_noalloc", "reshape_and_cache", "copy_blocks", "BlockAllocator",
    "DecodeStepper", "swap_blocks", "check_slot_mapping", "check_copy_pairs", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ENOMEM, PKV_EHIP = range(5)
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = _lib().pkv_status_string(status).decode() if _LIB is not None else str(status)
        super().__init__(f"{what}: {msg} (status {status})")


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_LIB = None
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)
_pdesc = ctypes.POINTER(CacheDesc)

_SIGNATURES = {
    "pkv_abi_version": (_i32, []),
    "pkv_status_string": (ctypes.c_char_p, [_i32]),
    "pkv_decode_workspace_bytes": (_sz, [_pdesc, _i32, _i32]),
    "pkv_decode_partition_tokens": (_i32, [_pdesc, _i32, _i32]),
    "pkv_decode_single_pass_max": (_i32, []),
    "pkv_decode_xcd_grid": (_i64, [_i64, _i32]),
    "pkv_decode_xcd_slot_unit": (_i64, [_i64, _i64, _i32]),
    "pkv_decode_set_xcd_split": (_i32, [_i32]),
    "pkv_decode_xcd_split": (_i32, []),
    "pkv_decode_schedule": (_i32, [_pdesc, _p, _i32, _i32, _p, _i32]),
    "pkv_decode_schedule_grouped": (_i32, [_pdesc, _p, _p, _i32, _i32, _p, _i32]),
    "pkv_paged_attention_decode_scheduled": (_i32, [_pdesc, _p, _p, _p, _p, _p, _i32, _p, _i32,
                                                    _i32, _f32, _p, _i32, ctypes.c_uint32, _p,
                                                    _sz, _p]),
    "pkv_paged_attention_decode": (_i32, [_pdesc, _p, _p, _p, _p, _p, _i32, _p, _i32, _i32, _f32,
                                          _p, _sz, _p]),
    "pkv_paged_attention_decode_noalloc": (_i32, [_pdesc, _p, _p, _p, _p, _p, _i32, _p, _i32,
                                                  _i32, _f32, _p]),
    "pkv_multi_query_tile": (_i32, []),
    "pkv_multi_query_schedule": (_i32, [_p, _p, _i32, _i32, _p, _i32]),
    "pkv_multi_query_schedule_grouped": (_i32, [_p, _p, _p, _i32, _i32, _p, _i32]),
    "pkv_paged_attention_multi_query": (_i32, [_pdesc, _p, _p, _p, _p, _p, _i32, _p, _p, _i32,
                                               _i32, _i32, _i32, _f32, _p, _i32, _p]),
    "pkv_multi_query_schedule_packed": (_i32, [_p, _p, _p, _i32, _i32, _i32, _i32, _p, _i32]),
    "pkv_paged_attention_multi_query_packed": (_i32, [_pdesc, _p, _p, _p, _p, _p, _i32, _p, _p,
                                                      _i32, _i32, _i32, _i32, _f32, _p, _i32,
                                                      _p]),
    "pkv_reshape_and_cache": (_i32, [_pdesc, _p, _p, _p, _p, _p, _i32, _p]),
    "pkv_check_slot_mapping": (_i32, [_pdesc, _p, _i32]),
    "pkv_copy_blocks": (_i32, [_pdesc, _p, _p, _i32, _p, _i32, _p]),
    "pkv_check_copy_pairs": (_i32, [_pdesc, _p, _i32]),
    "pkv_alloc_create": (_p, [_i32, _i32, _p]),
    "pkv_alloc_destroy": (None, [_p]),
    "pkv_alloc_add_seq": (_i32, [_p, _i64, _i32]),
    "pkv_alloc_fork": (_i32, [_p, _i64, _i64]),
    "pkv_alloc_append_slot": (_i32, [_p, _i64, _pi32, _pi32, _pi32]),
    "pkv_alloc_append_slots": (_i32, [_p, _p, _i32, _p, _p, _pi32, _pi32]),
    "pkv_alloc_append_need": (_i32, [_p, _p, _i32, _pi32]),
    "pkv_alloc_free_seq": (_i32, [_p, _i64]),
    "pkv_alloc_add_seqs": (_i32, [_p, _p, _p, _i32, _pi32]),
    "pkv_alloc_fork_many": (_i32, [_p, _p, _p, _i32, _pi32]),
    "pkv_alloc_free_seqs": (_i32, [_p, _p, _i32, _pi32]),
    "pkv_alloc_block_table": (_i32, [_p, _i64, _p, _i32, _pi32]),
    "pkv_alloc_export": (_i32, [_p, _p, _i32, _i32, _p, _p]),
    "pkv_alloc_seq_len": (_i32, [_p, _i64]),
    "pkv_alloc_num_free": (_i32, [_p]),
    "pkv_alloc_refcount": (_i32, [_p, _i32]),
    "pkv_alloc_wasted_slots": (_i64, [_p]),
    "pkv_alloc_add_seq_cached": (_i32, [_p, _i64, _p, _i32, _pi32]),
    "pkv_alloc_num_cached": (_i32, [_p]),
    "pkv_alloc_move_seqs": (_i32, [_p, _p, _p, _i32, _p, _i32, _pi32]),
    "pkv_swap_blocks": (_i32, [_pdesc, _pdesc, _p, _p, _p, _p, _i32, _p, _i32, _p]),
    "pkv_stepper_index_bytes": (_sz, [_pdesc, _i32, _i32]),
    "pkv_stepper_last_attention": (_i32, [_p]),
    "pkv_stepper_create": (_p, [_p, _pdesc, _i32, _i32, _p]),
    "pkv_stepper_destroy": (None, [_p]),
    "pkv_stepper_step": (_i32, [_p, _p, _i32, _p, _p, _sz, _p, _pi32, _pi32, _pi32, _p]),
    "pkv_stepper_last_index": (_p, [_p]),
    "pkv_stepper_xcd_split": (_i32, [_p]),
    "pkv_stepper_set_xcd_split": (_i32, [_p, _i32]),
    "pkv_stepper_xcd_rates": (_i32, [_p, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_double), _pi32]),
    "pkv_xcd_split_from_stamps": (_i32, [_p, _i64, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_double), _pi32]),
    "pkv_stepper_check": (_i32, [_p, _pdesc, _i32, _i32, _p, _i32, _p, _p, _sz, _pi32]),
}


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_306_amd.build` "
                "(there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def lib():
    """The loaded libpkv.so (ctypes.CDLL), loading it on first use."""
    return _lib()


def _check(status: int, what: str):
    if status != PKV_OK:
        raise PkvError(status, what)


# ----------------------------------------------------------------------------- torch glue
def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _stream_ptr(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def desc_for_pool(k_pool) -> CacheDesc:
    """CacheDesc of a [num_blocks][num_heads][block_size][head_dim] pool tensor."""
    nb, h, bs, d = k_pool.shape
    return CacheDesc(nb, h, bs, d, _dtype_code(k_pool))


def decode_workspace_bytes(desc: CacheDesc, num_seqs: int, max_context_len: int) -> int:
    return int(_lib().pkv_decode_workspace_bytes(ctypes.byref(desc), num_seqs, max_context_len))


def decode_partition_tokens(desc: CacheDesc, num_seqs: int, max_context_len: int) -> int:
    return int(_lib().pkv_decode_partition_tokens(ctypes.byref(desc), num_seqs, max_context_len))


def decode_xcd_grid(units: int, split: int) -> int:
    """Workgroups an attention launch of ``units`` units takes under the XCD split (of 1024;
    0: one per unit), pkv_decode_xcd_grid; -1 for bad arguments."""
    return int(_lib().pkv_decode_xcd_grid(int(units), int(split)))


def xcd_split_from_stamps(stamps):
    """The split the step driver takes from a stamped launch's stamps (uint32 numpy [units][4]:
    duration ticks, XCD | 0x100, tokens, start tick), with the halves' rates and the outcome:
    (split, even, odd, outcome) (pkv_xcd_split_from_stamps)."""
    import numpy as np
    w = np.ascontiguousarray(np.asarray(stamps, dtype=np.uint32))
    e, o, k = ctypes.c_double(), ctypes.c_double(), _i32()
    p = _lib().pkv_xcd_split_from_stamps(w.ctypes.data_as(ctypes.c_void_p), int(w.shape[0]),
                                         ctypes.byref(e), ctypes.byref(o), ctypes.byref(k))
    return int(p), e.value, o.value, k.value


def decode_set_xcd_split(split: int) -> None:
    """Split (of 1024; 0: even) the stand-alone decode calls on the current device deal their
    units with (pkv_decode_set_xcd_split)."""
    _check(_lib().pkv_decode_set_xcd_split(int(split)), "pkv_decode_set_xcd_split")


def decode_xcd_split() -> int:
    """The current device's split for the stand-alone decode calls (pkv_decode_xcd_split)."""
    return int(_lib().pkv_decode_xcd_split())


def decode_xcd_slot_unit(slot: int, units: int, split: int) -> int:
    """The unit workgroup ``slot`` runs under the XCD split, -1 for none
    (pkv_decode_xcd_slot_unit); -2 for bad arguments."""
    return int(_lib().pkv_decode_xcd_slot_unit(int(slot), int(units), int(split)))


PKV_DECODE_SHARED_KV = 1
PKV_STEP_ATTN_DECODE, PKV_STEP_ATTN_MULTI_QUERY = 0, 1   # pkv_stepper_last_attention
# outcome of a stepper's XCD measurement (pkv_stepper_xcd_rates)
PKV_XCD_NONE, PKV_XCD_IN_FLIGHT, PKV_XCD_MEASURED, PKV_XCD_TOO_FEW, PKV_XCD_UNMAPPED, \
    PKV_XCD_FAILED = range(6)


def decode_schedule(desc: CacheDesc, lens, max_context_len: int, group_keys=None):
    """Host-built work items for the given host lengths (int32 numpy array): longest first,
    or with ``group_keys`` grouped by key (sequences sharing a prefix side by side)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    S = int(lens.shape[0])
    part = decode_partition_tokens(desc, S, max_context_len)
    cap = max(1, S * (-(-max(max_context_len, 1) // part) if part else 1))
    items = np.empty(cap, np.int32)
    if group_keys is None:
        n = _lib().pkv_decode_schedule(ctypes.byref(desc), lens.ctypes.data_as(ctypes.c_void_p),
                                       S, int(max_context_len),
                                       items.ctypes.data_as(ctypes.c_void_p), cap)
    else:
        keys = np.ascontiguousarray(np.asarray(group_keys, dtype=np.int32))
        if keys.shape != (S,):
            raise ValueError("one group key per sequence")
        n = _lib().pkv_decode_schedule_grouped(
            ctypes.byref(desc), lens.ctypes.data_as(ctypes.c_void_p),
            keys.ctypes.data_as(ctypes.c_void_p), S, int(max_context_len),
            items.ctypes.data_as(ctypes.c_void_p), cap)
    if n < 0:
        raise PkvError(PKV_EINVAL, "pkv_decode_schedule")
    return items[:n].copy()


def paged_attention_decode(out, q, k_pool, v_pool, block_tables, context_lens, scale: float,
                           max_context_len: int, workspace=None, stream=None, work_items=None,
                           shared_kv: bool = False):
    """out[s, h] = softmax(scale * q[s, h] . K(s, :, h)) V(s, :, h) over the context_lens[s]
    tokens of sequence s, gathered through block_tables (see include/pkv.h).  With
    ``work_items`` (int32 device tensor from decode_schedule) the scheduled entry point runs."""
    import torch
    desc = desc_for_pool(k_pool)
    S = q.shape[0]
    if q.shape != out.shape or q.shape[1:] != (desc.num_heads, desc.head_dim):
        raise ValueError("q/out shape mismatch")
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool/v_pool mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables/context_lens shape mismatch")
    need = decode_workspace_bytes(desc, S, max_context_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (ctypes.byref(desc), _dev(out, "out", k_pool.dtype), _dev(q, "q", k_pool.dtype),
            _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
            _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
            _dev(context_lens, "context_lens", torch.int32), S, int(max_context_len),
            float(scale))
    if work_items is None:
        if shared_kv:
            raise ValueError("shared_kv needs a work list (the scheduled entry point)")
        st = _lib().pkv_paged_attention_decode(*args, ws_ptr, ws_bytes, _stream_ptr(stream))
        _check(st, "pkv_paged_attention_decode")
    else:
        st = _lib().pkv_paged_attention_decode_scheduled(
            *args, _dev(work_items, "work_items", torch.int32), int(work_items.numel()),
            PKV_DECODE_SHARED_KV if shared_kv else 0, ws_ptr, ws_bytes, _stream_ptr(stream))
        _check(st, "pkv_paged_attention_decode_scheduled")
    return out


# bytes of the per-GPU scratch array pkv_paged_attention_decode_noalloc uses (include/pkv.h)
DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20


def paged_attention_decode_noalloc(out, q, k_pool, v_pool, block_tables, context_lens,
                                   scale: float, max_context_len: int, stream=None):
    """paged_attention_decode without a workspace: the split-context partials go to the
    library's per-GPU scratch array, and nothing is allocated (include/pkv.h).  Calls on one
    GPU share that array, so calls on different streams must not overlap."""
    import torch
    desc = desc_for_pool(k_pool)
    S = q.shape[0]
    if q.shape != out.shape or q.shape[1:] != (desc.num_heads, desc.head_dim):
        raise ValueError("q/out shape mismatch")
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool/v_pool mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables/context_lens shape mismatch")
    st = _lib().pkv_paged_attention_decode_noalloc(
        ctypes.byref(desc), _dev(out, "out", k_pool.dtype), _dev(q, "q", k_pool.dtype),
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32), S, int(max_context_len), float(scale),
        _stream_ptr(stream))
    _check(st, "pkv_paged_attention_decode_noalloc")
    return out


def multi_query_tile() -> int:
    """New tokens per workgroup tile of the multi-query kernel."""
    return int(_lib().pkv_multi_query_tile())


def multi_query_schedule(query_start, context_lens, max_context_len: int, group_keys=None):
    """Host-built work items (int32 numpy) for multi-query attention from host copies of
    query_start [S+1] and context_lens [S]: one per (sequence, tile) with new tokens.
    ``group_keys`` (int [S], e.g. the first physical block of each table): sequences with
    equal keys are scheduled side by side, so the prefix blocks they share are read from L2."""
    import numpy as np
    qs = np.ascontiguousarray(np.asarray(query_start, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    S = int(cl.shape[0])
    if qs.shape != (S + 1,):
        raise ValueError("query_start needs num_seqs + 1 entries")
    keys = None
    if group_keys is not None:
        keys = np.ascontiguousarray(np.asarray(group_keys, dtype=np.int32))
        if keys.shape != (S,):
            raise ValueError("group_keys needs num_seqs entries")
    tile = multi_query_tile()
    n = np.diff(qs.astype(np.int64))
    cap = max(1, int(np.sum(np.maximum(-(-n // tile), 0))))
    items = np.empty(cap, np.int32)
    k = _lib().pkv_multi_query_schedule_grouped(
        qs.ctypes.data_as(ctypes.c_void_p), cl.ctypes.data_as(ctypes.c_void_p),
        keys.ctypes.data_as(ctypes.c_void_p) if keys is not None else None, S,
        int(max_context_len), items.ctypes.data_as(ctypes.c_void_p), cap)
    if k < 0:
        raise PkvError(PKV_EINVAL, "pkv_multi_query_schedule_grouped")
    return items[:k].copy()


def paged_attention_multi_query(out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                                scale: float, max_query_len: int, max_context_len: int,
                                work_items=None, stream=None):
    """Several new tokens per sequence: row query_start[s] + i of q attends to positions
    0 .. context_lens[s] - n_s + i of sequence s, read through block_tables (include/pkv.h).
    q/out: [T][H][D]; query_start: int32 device [S+1]; ``work_items``: int32 device tensor from
    multi_query_schedule, or None for the plain grid."""
    import torch
    desc = desc_for_pool(k_pool)
    S = context_lens.shape[0]
    if q.shape != out.shape or q.dim() != 3 or q.shape[1:] != (desc.num_heads, desc.head_dim):
        raise ValueError("q/out shape mismatch")
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool/v_pool mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or query_start.shape != (S + 1,):
        raise ValueError("block_tables/query_start shape mismatch")
    work = (_dev(work_items, "work_items", torch.int32) if work_items is not None
            else ctypes.c_void_p(0))
    st = _lib().pkv_paged_attention_multi_query(
        ctypes.byref(desc), _dev(out, "out", k_pool.dtype), _dev(q, "q", k_pool.dtype),
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32),
        _dev(query_start, "query_start", torch.int32), S, int(q.shape[0]), int(max_query_len),
        int(max_context_len), float(scale), work,
        int(work_items.numel()) if work_items is not None else 0, _stream_ptr(stream))
    _check(st, "pkv_paged_attention_multi_query")
    return out


def multi_query_schedule_packed(query_start, context_lens, block_tables, block_size: int,
                                max_context_len: int):
    """Tiles (int32 numpy [n][4]: first sequence, last sequence, first row of the first one,
    shared keys) that pack the new tokens of consecutive sequences sharing prefix blocks into
    full tiles, from host copies of query_start [S+1], context_lens [S] and block_tables
    [S][max_blocks] (include/pkv.h)."""
    import numpy as np
    qs = np.ascontiguousarray(np.asarray(query_start, dtype=np.int32))
    cl = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    bt = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    S = int(cl.shape[0])
    if qs.shape != (S + 1,):
        raise ValueError("query_start needs num_seqs + 1 entries")
    if bt.ndim != 2 or bt.shape[0] != S or bt.shape[1] < 1:
        raise ValueError("block_tables needs num_seqs rows")
    tile = multi_query_tile()
    n = np.diff(qs.astype(np.int64))
    cap = max(1, int(np.sum(np.maximum(-(-n // tile), 0))))
    tiles = np.empty((cap, 4), np.int32)
    k = _lib().pkv_multi_query_schedule_packed(
        qs.ctypes.data_as(ctypes.c_void_p), cl.ctypes.data_as(ctypes.c_void_p),
        bt.ctypes.data_as(ctypes.c_void_p), int(bt.shape[1]), int(block_size), S,
        int(max_context_len), tiles.ctypes.data_as(ctypes.c_void_p), cap)
    if k < 0:
        raise PkvError(PKV_EINVAL, "pkv_multi_query_schedule_packed")
    return tiles[:k].copy()


def paged_attention_multi_query_packed(out, q, k_pool, v_pool, block_tables, context_lens,
                                       query_start, scale: float, max_query_len: int,
                                       max_context_len: int, tiles, stream=None):
    """paged_attention_multi_query over packed tiles (int32 device tensor [n][4] from
    multi_query_schedule_packed): the same outputs, full tiles where sequences share a
    prompt's blocks."""
    import torch
    desc = desc_for_pool(k_pool)
    S = context_lens.shape[0]
    if q.shape != out.shape or q.dim() != 3 or q.shape[1:] != (desc.num_heads, desc.head_dim):
        raise ValueError("q/out shape mismatch")
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool/v_pool mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or query_start.shape != (S + 1,):
        raise ValueError("block_tables/query_start shape mismatch")
    if tiles.dim() != 2 or tiles.shape[1] != 4:
        raise ValueError("tiles must be [n][4]")
    st = _lib().pkv_paged_attention_multi_query_packed(
        ctypes.byref(desc), _dev(out, "out", k_pool.dtype), _dev(q, "q", k_pool.dtype),
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
        _dev(block_tables, "block_tables", torch.int32), block_tables.shape[1],
        _dev(context_lens, "context_lens", torch.int32),
        _dev(query_start, "query_start", torch.int32), S, int(q.shape[0]), int(max_query_len),
        int(max_context_len), float(scale), _dev(tiles, "tiles", torch.int32),
        int(tiles.shape[0]), _stream_ptr(stream))
    _check(st, "pkv_paged_attention_multi_query_packed")
    return out


def _debug_checks() -> bool:
    """PKV_DEBUG=1: check the preconditions of the device index arrays on a host copy before
    each launch (synchronizes; for debugging)."""
    return os.environ.get("PKV_DEBUG", "") == "1"


def check_slot_mapping(desc: CacheDesc, slots):
    """Raise PkvError unless the in-pool slots (host int32 array) are distinct."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(slots, dtype=np.int32))
    _check(_lib().pkv_check_slot_mapping(ctypes.byref(desc), a.ctypes.data_as(ctypes.c_void_p),
                                         int(a.shape[0])), "pkv_check_slot_mapping")


def check_copy_pairs(desc: CacheDesc, pairs):
    """Raise PkvError unless the in-pool (src, dst) pairs (host int32 [n][2]) have distinct
    destinations that are never also sources."""
    import numpy as np
    a = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    _check(_lib().pkv_check_copy_pairs(ctypes.byref(desc), a.ctypes.data_as(ctypes.c_void_p),
                                       int(a.shape[0])), "pkv_check_copy_pairs")


def reshape_and_cache(k, v, k_pool, v_pool, slot_mapping, stream=None):
    """Write token i's K/V rows into slot slot_mapping[i] of the pools (include/pkv.h)."""
    import torch
    desc = desc_for_pool(k_pool)
    N = k.shape[0]
    if k.shape != (N, desc.num_heads, desc.head_dim) or v.shape != k.shape:
        raise ValueError("k/v shape mismatch")
    if slot_mapping.shape != (N,):
        raise ValueError("slot_mapping shape mismatch")
    if _debug_checks():
        check_slot_mapping(desc, slot_mapping.cpu().numpy())
    st = _lib().pkv_reshape_and_cache(
        ctypes.byref(desc), _dev(k, "k", k_pool.dtype), _dev(v, "v", k_pool.dtype),
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
        _dev(slot_mapping, "slot_mapping", torch.int32), N, _stream_ptr(stream))
    _check(st, "pkv_reshape_and_cache")


def copy_blocks(k_pools, v_pools, pairs, stream=None):
    """pool[dst] = pool[src] for every (src, dst) row of `pairs` (int32 [n][2], device), in
    every layer's K and V pool."""
    import torch
    if len(k_pools) != len(v_pools) or not k_pools:
        raise ValueError("need one K and one V pool per layer")
    desc = desc_for_pool(k_pools[0])
    for p in list(k_pools) + list(v_pools):
        if p.shape != k_pools[0].shape or p.dtype != k_pools[0].dtype:
            raise ValueError("all pools must share one shape and dtype")
    n = pairs.shape[0] if pairs.numel() else 0
    if pairs.numel() and (pairs.dim() != 2 or pairs.shape[1] != 2):
        raise ValueError("pairs must be [n][2]")
    if _debug_checks() and n:
        check_copy_pairs(desc, pairs.cpu().numpy())
    L = len(k_pools)
    kp = (ctypes.c_void_p * L)(*[p.data_ptr() for p in k_pools])
    vp = (ctypes.c_void_p * L)(*[p.data_ptr() for p in v_pools])
    for p in list(k_pools) + list(v_pools):
        _dev(p, "pool")
    pptr = _dev(pairs, "pairs", torch.int32) if n else ctypes.c_void_p(0)
    st = _lib().pkv_copy_blocks(ctypes.byref(desc), kp, vp, L, pptr, n, _stream_ptr(stream))
    _check(st, "pkv_copy_blocks")


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs, stream=None):
    """dst[l][d] = src[l][s] for every (s, d) row of ``pairs`` and every layer l, K and V.
    Pools (lists, one per layer) may be device tensors or pinned host tensors; ``pairs`` an
    int32 [n][2] device or pinned host tensor."""
    import torch
    L = len(src_k)
    if not (len(src_v) == len(dst_k) == len(dst_v) == L) or L == 0:
        raise ValueError("one pool per layer in every list")
    for p in list(src_k) + list(src_v) + list(dst_k) + list(dst_v):
        if not p.is_contiguous():
            raise ValueError("pools must be contiguous")
        if p.shape[1:] != src_k[0].shape[1:] or p.dtype != src_k[0].dtype:
            raise ValueError("pools must share everything but the block count")
        if not (p.is_cuda or p.is_pinned()):
            raise ValueError("pools must be device or pinned host tensors")
    for p in list(src_v):
        if p.shape != src_k[0].shape:
            raise ValueError("source pools must share one shape")
    for p in list(dst_v):
        if p.shape != dst_k[0].shape:
            raise ValueError("destination pools must share one shape")
    if pairs.dtype != torch.int32 or (pairs.numel() and (pairs.dim() != 2 or pairs.shape[1] != 2)):
        raise ValueError("pairs must be int32 [n][2]")
    n = pairs.shape[0] if pairs.numel() else 0
    sd, dd = desc_for_pool(src_k[0]), desc_for_pool(dst_k[0])
    arr = lambda lst: (ctypes.c_void_p * L)(*[t.data_ptr() for t in lst])
    st = _lib().pkv_swap_blocks(ctypes.byref(sd), ctypes.byref(dd), arr(src_k), arr(src_v),
                                arr(dst_k), arr(dst_v), L,
                                ctypes.c_void_p(pairs.data_ptr() if n else 0), n,
                                _stream_ptr(stream))
    _check(st, "pkv_swap_blocks")


# ----------------------------------------------------------------------------- allocator
class BlockAllocator:
    """Host block manager (plain C++ inside libpkv): on-demand blocks, reference counts and
    copy-on-write decisions.  See include/pkv.h for the policy."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        import numpy as np
        self.block_size = block_size
        self.num_blocks = num_blocks
        arr = None
        if free_order is not None:
            arr = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if arr.shape != (num_blocks,):
                raise ValueError("free_order must list every block once")
        ptr = arr.ctypes.data_as(ctypes.c_void_p) if arr is not None else None
        self._h = _lib().pkv_alloc_create(num_blocks, block_size, ptr)
        if not self._h:
            raise PkvError(PKV_EINVAL, "pkv_alloc_create")

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _LIB is not None:
            _LIB.pkv_alloc_destroy(h)

    def add_seq(self, seq: int, length: int):
        _check(_lib().pkv_alloc_add_seq(self._h, seq, length), "pkv_alloc_add_seq")

    def add_seq_cached(self, seq: int, tokens) -> int:
        """New sequence with prompt ``tokens``; shares cached prefix blocks.  Returns the
        number of prompt tokens whose K/V is already in the cache."""
        import numpy as np
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        cached = _i32()
        _check(_lib().pkv_alloc_add_seq_cached(self._h, seq, t.ctypes.data_as(ctypes.c_void_p),
                                               int(t.shape[0]), ctypes.byref(cached)),
               "pkv_alloc_add_seq_cached")
        return cached.value

    def num_cached(self) -> int:
        return int(_lib().pkv_alloc_num_cached(self._h))

    def move_seqs(self, to: "BlockAllocator", seqs):
        """Move sequences to another block manager (swap out / swap in); returns the
        (block here, block there) pairs as int32 numpy [n][2] for swap_blocks."""
        import numpy as np
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        cap = int(sum(len(self.block_table(int(s))) for s in seqs)) if len(seqs) else 0
        pairs = np.empty((max(cap, 1), 2), np.int32)
        npairs = _i32()
        _check(_lib().pkv_alloc_move_seqs(self._h, to._h, seqs.ctypes.data_as(ctypes.c_void_p),
                                          int(seqs.shape[0]),
                                          pairs.ctypes.data_as(ctypes.c_void_p), cap,
                                          ctypes.byref(npairs)), "pkv_alloc_move_seqs")
        return pairs[:npairs.value].copy()

    def fork(self, parent: int, child: int):
        _check(_lib().pkv_alloc_fork(self._h, parent, child), "pkv_alloc_fork")

    def append_slot(self, seq: int):
        slot, src, dst = _i32(), _i32(), _i32()
        _check(_lib().pkv_alloc_append_slot(self._h, seq, ctypes.byref(slot), ctypes.byref(src),
                                            ctypes.byref(dst)), "pkv_alloc_append_slot")
        return slot.value, (None if src.value < 0 else (src.value, dst.value))

    def append_slots(self, seqs):
        """Returns (slots int32 [n], cow_pairs int32 [k][2]) as numpy arrays."""
        import numpy as np
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        n = int(seqs.shape[0])
        slots = np.empty(n, np.int32)
        pairs = np.empty((max(n, 1), 2), np.int32)
        ncow, ndone = _i32(), _i32()
        st = _lib().pkv_alloc_append_slots(self._h, seqs.ctypes.data_as(ctypes.c_void_p), n,
                                           slots.ctypes.data_as(ctypes.c_void_p),
                                           pairs.ctypes.data_as(ctypes.c_void_p),
                                           ctypes.byref(ncow), ctypes.byref(ndone))
        if st != PKV_OK:
            err = PkvError(st, "pkv_alloc_append_slots")
            err.num_done = ndone.value
            raise err
        return slots, pairs[:ncow.value].copy()

    def append_slots_into(self, seqs, slots, pairs) -> int:
        """Like ``append_slots`` but writes into caller arrays (int64 seqs [n], int32 slots
        [n], int32 pairs [n][2], all C-contiguous numpy); returns the number of pairs."""
        n = int(seqs.shape[0])
        ncow, ndone = _i32(), _i32()
        st = _lib().pkv_alloc_append_slots(self._h, seqs.ctypes.data_as(ctypes.c_void_p), n,
                                           slots.ctypes.data_as(ctypes.c_void_p),
                                           pairs.ctypes.data_as(ctypes.c_void_p),
                                           ctypes.byref(ncow), ctypes.byref(ndone))
        if st != PKV_OK:
            err = PkvError(st, "pkv_alloc_append_slots")
            err.num_done = ndone.value
            raise err
        return ncow.value

    def export_into(self, seqs, tables, lens):
        """Like ``export`` but writes into caller arrays (int32 tables [n][max_blocks],
        int32 lens [n], C-contiguous numpy)."""
        n = int(seqs.shape[0])
        _check(_lib().pkv_alloc_export(self._h, seqs.ctypes.data_as(ctypes.c_void_p), n,
                                       tables.shape[1], tables.ctypes.data_as(ctypes.c_void_p),
                                       lens.ctypes.data_as(ctypes.c_void_p)), "pkv_alloc_export")

    def append_need(self, seqs) -> int:
        """Blocks ``append_slots(seqs)`` would take from the pool; nothing changes."""
        import numpy as np
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        need = _i32()
        _check(_lib().pkv_alloc_append_need(self._h, seqs.ctypes.data_as(ctypes.c_void_p),
                                            int(seqs.shape[0]), ctypes.byref(need)),
               "pkv_alloc_append_need")
        return need.value

    def free_seq(self, seq: int):
        _check(_lib().pkv_alloc_free_seq(self._h, seq), "pkv_alloc_free_seq")

    def _batched(self, fn, name, arrays, n):
        done = _i32()
        st = getattr(_lib(), fn)(self._h, *[a.ctypes.data_as(ctypes.c_void_p) for a in arrays],
                                 n, ctypes.byref(done))
        if st != PKV_OK:
            err = PkvError(st, name)
            err.num_done = done.value
            raise err

    def add_seqs(self, seqs, lens):
        """add_seq(seqs[i], lens[i]) for every i in one host call; on an error the calls before
        it stay and the raised PkvError carries ``num_done``."""
        import numpy as np
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        lens = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
        if lens.shape != seqs.shape or seqs.ndim != 1:
            raise ValueError("one length per sequence")
        self._batched("pkv_alloc_add_seqs", "pkv_alloc_add_seqs", (seqs, lens), seqs.shape[0])

    def fork_many(self, parents, children):
        """fork(parents[i], children[i]) for every i in one host call (same error rule)."""
        import numpy as np
        parents = np.ascontiguousarray(np.asarray(parents, dtype=np.int64))
        children = np.ascontiguousarray(np.asarray(children, dtype=np.int64))
        if parents.shape != children.shape or parents.ndim != 1:
            raise ValueError("one parent per child")
        self._batched("pkv_alloc_fork_many", "pkv_alloc_fork_many", (parents, children),
                      parents.shape[0])

    def free_seqs(self, seqs):
        """free_seq(seqs[i]) for every i in one host call (same error rule)."""
        import numpy as np
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        if seqs.ndim != 1:
            raise ValueError("a 1-D list of sequences")
        self._batched("pkv_alloc_free_seqs", "pkv_alloc_free_seqs", (seqs,), seqs.shape[0])

    def block_table(self, seq: int):
        n = _i32()
        _check(_lib().pkv_alloc_block_table(self._h, seq, None, 0, ctypes.byref(n)),
               "pkv_alloc_block_table")
        buf = (ctypes.c_int32 * max(1, n.value))()
        _check(_lib().pkv_alloc_block_table(self._h, seq, buf, n.value, ctypes.byref(n)),
               "pkv_alloc_block_table")
        return list(buf[:n.value])

    def export(self, seqs, max_blocks: int):
        """Dense (tables int32 [n][max_blocks], lens int32 [n]) for the given sequences."""
        import numpy as np
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        n = int(seqs.shape[0])
        tables = np.empty((n, max_blocks), np.int32)
        lens = np.empty(n, np.int32)
        _check(_lib().pkv_alloc_export(self._h, seqs.ctypes.data_as(ctypes.c_void_p), n,
                                       max_blocks, tables.ctypes.data_as(ctypes.c_void_p),
                                       lens.ctypes.data_as(ctypes.c_void_p)), "pkv_alloc_export")
        return tables, lens

    def seq_len(self, seq: int) -> int:
        return int(_lib().pkv_alloc_seq_len(self._h, seq))

    def num_free(self) -> int:
        return int(_lib().pkv_alloc_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(_lib().pkv_alloc_refcount(self._h, block))

    def wasted_slots(self) -> int:
        return int(_lib().pkv_alloc_wasted_slots(self._h))


# ----------------------------------------------------------------------------- step driver
class LayerIO(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("k_pools", ctypes.c_void_p),
                ("v_pools", ctypes.c_void_p), ("q", ctypes.c_void_p), ("k_new", ctypes.c_void_p),
                ("v_new", ctypes.c_void_p), ("out", ctypes.c_void_p), ("scale", ctypes.c_float)]


class DecodeStepper:
    """Native decode-step driver (pkv_stepper_* in include/pkv.h): per call, one slot per
    sequence from the block manager, one prologue kernel that pulls the packed tables /
    lengths / slots / pairs / work list from pinned host memory (and appends layer 0's new K/V
    when nothing is copied), copy_blocks for copy-on-write pairs, then per layer
    reshape_and_cache and decode."""

    def __init__(self, alloc: BlockAllocator, k_pools, v_pools, q, k_new, v_new, out,
                 scale: float, max_seqs: int, max_blocks_per_seq: int, max_context_len: int):
        import torch
        self.alloc = alloc                 # keep the block manager alive
        self.desc = desc_for_pool(k_pools[0])
        L = len(k_pools)
        tensors = [k_pools, v_pools, q, k_new, v_new, out]
        if any(len(t) != L for t in tensors):
            raise ValueError("one tensor per layer in every list")
        for p in list(k_pools) + list(v_pools):
            _dev(p, "pool", k_pools[0].dtype)
            if p.shape != k_pools[0].shape:
                raise ValueError("all pools must share one shape")
        for t in list(q) + list(k_new) + list(v_new) + list(out):
            _dev(t, "q/k_new/v_new/out", k_pools[0].dtype)
            if t.shape[1:] != (self.desc.num_heads, self.desc.head_dim) or t.shape[0] < max_seqs:
                raise ValueError("per-layer tensors must be [>= max_seqs][heads][head_dim]")
        self._keep = tensors
        self._arrs = [(ctypes.c_void_p * L)(*[t.data_ptr() for t in lst]) for lst in tensors]
        self.io = LayerIO(L, *[ctypes.cast(a, ctypes.c_void_p) for a in self._arrs], float(scale))
        dev = k_pools[0].device
        nbytes = int(_lib().pkv_stepper_index_bytes(ctypes.byref(self.desc), max_seqs,
                                                     max_blocks_per_seq))
        self.d_index = torch.empty(max(16, nbytes), dtype=torch.uint8, device=dev)
        self.max_blocks = max_blocks_per_seq
        self.max_seqs = max_seqs
        ws = decode_workspace_bytes(self.desc, max_seqs, max_context_len)
        self.workspace = torch.empty(max(16, ws), dtype=torch.uint8, device=dev)
        self.max_context_len = max_context_len
        self._h = _lib().pkv_stepper_create(alloc._h, ctypes.byref(self.desc), max_seqs,
                                            max_blocks_per_seq, self.d_index.data_ptr())
        if not self._h:
            raise PkvError(PKV_EINVAL, "pkv_stepper_create")
        self._max_len, self._ncow, self._ndone = _i32(), _i32(), _i32()

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _LIB is not None:
            _LIB.pkv_stepper_destroy(h)

    def step(self, seqs, events=None, stream=None):
        """One decode step for the sequences in ``seqs`` (C-contiguous int64 numpy).
        ``events``: optional ctypes array of 2 * num_layers hipEvent_t handles (created with
        timing); the attention launch of layer l records its start into event 2l and its end
        into event 2l+1.  Returns (max_len, num_cow)."""
        n = int(seqs.shape[0])
        st = _lib().pkv_stepper_step(self._h, seqs.ctypes.data_as(ctypes.c_void_p), n,
                                     ctypes.byref(self.io), self.workspace.data_ptr(),
                                     self.workspace.numel(), events,
                                     ctypes.byref(self._max_len), ctypes.byref(self._ncow),
                                     ctypes.byref(self._ndone), _stream_ptr(stream))
        if st != PKV_OK:
            # every error but a refused launch leaves the block manager and pools unchanged
            err = PkvError(st, "pkv_stepper_step")
            err.num_done = self._ndone.value
            raise err
        return self._max_len.value, self._ncow.value

    @property
    def last_attention(self) -> int:
        """Which attention the last step ran: PKV_STEP_ATTN_DECODE, PKV_STEP_ATTN_MULTI_QUERY
        (sequences sharing their first blocks, packed tiles), or -1 (no step with sequences)."""
        return int(_lib().pkv_stepper_last_attention(self._h))

    @property
    def xcd_split(self) -> int:
        """Split (of 1024) the attention launches deal their units to the even XCDs with; 0:
        unit b to workgroup b (pkv_stepper_xcd_split)."""
        return int(_lib().pkv_stepper_xcd_split(self._h))

    def xcd_rates(self):
        """(even, odd, outcome): the halves' tokens per 100 MHz tick of workgroup time from the
        last measurement and its PKV_XCD_* outcome (pkv_stepper_xcd_rates)."""
        e, o, k = ctypes.c_double(), ctypes.c_double(), _i32()
        _check(_lib().pkv_stepper_xcd_rates(self._h, ctypes.byref(e), ctypes.byref(o),
                                             ctypes.byref(k)), "pkv_stepper_xcd_rates")
        return e.value, o.value, k.value

    def set_xcd_split(self, split: int) -> None:
        """Fix the split (0..1023, 0: none), or measure it again on the next step (-1)."""
        _check(_lib().pkv_stepper_set_xcd_split(self._h, int(split)), "pkv_stepper_set_xcd_split")

    def index_views(self, n: int, num_cow: int, num_items: int = 0):
        """Device views of the packed index data of the last step: (tables, lens, slots, pairs)
        and, with num_items, the work items as a fifth view."""
        import torch
        base = int(_lib().pkv_stepper_last_index(self._h))
        off = (base - self.d_index.data_ptr()) // 4
        ints = self.d_index.view(torch.int32)[off:]
        MB = self.max_blocks
        t = ints[:n * MB].view(n, MB)
        lens = ints[n * MB:n * MB + n]
        slots = ints[n * MB + n:n * MB + 2 * n]
        pairs = ints[n * MB + 2 * n:n * MB + 2 * n + 2 * num_cow].view(num_cow, 2)
        if num_items:
            o = n * MB + 2 * n + 2 * num_cow
            return t, lens, slots, pairs, ints[o:o + num_items]
        return t, lens, slots, pairs
