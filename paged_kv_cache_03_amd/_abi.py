"""ctypes binding of libkvstore (include/kvstore.h): same names, marshalling only.

Every function here forwards to the C entry point of the same name.  A status
other than KV_OK raises KVError carrying the status, the library's message and,
for a capacity shortfall, the deficit.  The library must be built
(``python paged_kv_cache_03_amd/build_lib.py``); loading fails loudly if not.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvstore.so")

KV_OK, KV_E_INVALID, KV_E_GEOMETRY, KV_E_CAPACITY = 0, 1, 2, 3
KV_E_STALE, KV_E_SHARED_WRITE, KV_E_UNMAPPED, KV_E_DEVICE, KV_E_UNSUPPORTED = 4, 5, 6, 7, 8
STATUS_NAMES = {0: "OK", 1: "INVALID", 2: "GEOMETRY", 3: "CAPACITY", 4: "STALE", 5: "SHARED_WRITE",
                6: "UNMAPPED", 7: "DEVICE", 8: "UNSUPPORTED"}

KV_PROFILE = {"BF16": 0, "INT8_G64": 1, "FP8_E4M3FN_ROW256": 2, "NVFP4_G16": 3, "K8V4": 4}
KV_DT_BF16, KV_DT_I8, KV_DT_E4M3FN, KV_DT_E2M1X2, KV_DT_F32, KV_DT_U8_E4M3, KV_DT_F16 = range(7)
KV_ROLE_K_CODE, KV_ROLE_K_SCALE, KV_ROLE_V_CODE, KV_ROLE_V_SCALE = range(4)
KV_LAYOUT_PAGE_MAJOR, KV_LAYOUT_HEAD_MAJOR = range(2)
KV_DECODE_SCRATCH_BYTES = 32 << 20      # the static scratch of paged_attn_decode_noalloc

# exported symbols, in header order (the CPU test checks the header declares exactly these)
EXPORTS = ["kv_profile_planes", "kv_profile_planes_ex", "kv_plane_bytes", "kv_pool_create", "kv_pool_destroy", "kv_pool_stats",
           "kv_pool_table_host", "kv_pool_page_refs", "kv_seq_open", "kv_seq_fork", "kv_seq_ensure_mapped",
           "kv_seq_commit", "kv_seq_release", "kv_seq_reserve", "kv_seq_trim", "kv_seq_commit_accepted",
           "kv_seq_reservation", "kv_draft_pool_pages", "kv_replica_page_bytes", "kv_seq_offload",
           "kv_seq_restore", "kv_seq_info", "kv_cow_tail_page", "kv_append",
           "paged_attn_workspace_bytes", "paged_attn_decode", "paged_attn_decode_noalloc", "paged_attn_decode_plan", "paged_attn_decode_run",
           "paged_attn_decode_append_run",
           "paged_attn_verify", "kv_decode_step_graph_create", "kv_step_graph_launch", "kv_step_graph_destroy",
           "paged_attn_supported", "kv_trace_next_kernel", "kv_read_probe",
           "kv_last_error_message"]


class KVPageGeometry(ctypes.Structure):
    _fields_ = [("page_size", ctypes.c_uint32), ("num_kv_heads", ctypes.c_uint32), ("head_dim", ctypes.c_uint32),
                ("num_layers", ctypes.c_uint32), ("max_context", ctypes.c_uint32),
                ("max_concurrency", ctypes.c_uint32), ("num_page_groups", ctypes.c_uint32)]


class KVPlaneDesc(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_uint32), ("role", ctypes.c_uint32), ("dtype", ctypes.c_uint32),
                ("x_extent", ctypes.c_uint32), ("elem_bytes", ctypes.c_uint32), ("layout", ctypes.c_uint32),
                ("base", ctypes.c_void_p)]


class KVError(RuntimeError):
    def __init__(self, status: int, message: str, deficit: int = 0):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status, self.message, self.deficit = status, message, deficit


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python paged_kv_cache_03_amd/build_lib.py`")
    # One HIP runtime per process: torch ships its own libamdhip64 (soname
    # libamdhip64.so.7) and loads it by the unversioned name.  Loading torch
    # first makes the library's libamdhip64.so.7 dependency resolve to that same
    # runtime, so device memory from torch and kernels from here share it.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    u32, i32, vp, sz = ctypes.c_uint32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "kv_profile_planes": (i32, [u32, u32, P(KVPlaneDesc), P(u32)]),
        "kv_profile_planes_ex": (i32, [u32, u32, u32, P(KVPlaneDesc), P(u32)]),
        "kv_plane_bytes": (i32, [P(KVPageGeometry), P(KVPlaneDesc), P(ctypes.c_uint64)]),
        "kv_pool_create": (i32, [P(KVPageGeometry), P(KVPlaneDesc), u32, vp, P(i32), vp, P(vp)]),
        "kv_pool_destroy": (None, [vp]),
        "kv_pool_stats": (i32, [vp, P(u32), P(u32), P(u32)]),
        "kv_pool_table_host": (i32, [vp, P(i32), sz]),
        "kv_pool_page_refs": (i32, [vp, u32, P(u32)]),
        "kv_seq_open": (i32, [vp, u32, vp, P(ctypes.c_uint64)]),
        "kv_seq_fork": (i32, [vp, ctypes.c_uint64, u32, u32, vp, P(ctypes.c_uint64)]),
        "kv_seq_ensure_mapped": (i32, [vp, ctypes.c_uint64, u32, P(u32), vp]),
        "kv_seq_commit": (i32, [vp, ctypes.c_uint64, u32]),
        "kv_seq_release": (i32, [vp, ctypes.c_uint64, vp]),
        "kv_seq_reserve": (i32, [vp, ctypes.c_uint64, u32, P(u32)]),
        "kv_seq_trim": (i32, [vp, ctypes.c_uint64, u32, vp]),
        "kv_seq_commit_accepted": (i32, [vp, ctypes.c_uint64, u32, u32, ctypes.c_int, vp]),
        "kv_seq_reservation": (i32, [vp, ctypes.c_uint64, P(u32)]),
        "kv_draft_pool_pages": (i32, [u32, u32, u32, P(u32)]),
        "kv_replica_page_bytes": (i32, [vp, P(ctypes.c_uint64)]),
        "kv_seq_offload": (i32, [vp, ctypes.c_uint64, vp, sz, P(u32), P(u32), vp]),
        "kv_seq_restore": (i32, [vp, u32, vp, sz, u32, P(u32), vp, P(ctypes.c_uint64)]),
        "kv_seq_info": (i32, [vp, ctypes.c_uint64, P(u32), P(u32), P(u32)]),
        "kv_cow_tail_page": (i32, [vp, ctypes.c_uint64, vp]),
        "kv_append": (i32, [vp, u32, u32, vp, vp, vp, u32, vp, vp, vp]),
        "paged_attn_workspace_bytes": (sz, [vp, u32, u32, u32, u32]),
        "paged_attn_decode": (i32, [vp, u32, u32, u32, vp, vp, u32, vp, ctypes.c_float, vp, vp, sz, vp]),
        "paged_attn_decode_noalloc": (i32, [vp, u32, u32, u32, vp, vp, u32, vp, ctypes.c_float, vp, vp]),
        "paged_attn_decode_plan": (i32, [vp, u32, u32, vp, vp, u32, vp, sz, vp]),
        "paged_attn_decode_run": (i32, [vp, u32, u32, u32, u32, vp, ctypes.c_float, vp, vp, sz, vp]),
        "paged_attn_decode_append_run": (i32, [vp, u32, u32, u32, u32, vp, vp, vp, ctypes.c_float, vp, vp, sz, vp]),
        "paged_attn_verify": (i32, [vp, u32, u32, u32, vp, vp, vp, u32, u32, u32, vp, ctypes.c_float, vp, vp, sz,
                                    vp]),
        "kv_decode_step_graph_create": (i32, [vp, u32, u32, u32, vp, vp, u32, vp, vp, vp, vp, u32, vp,
                                              ctypes.c_float, vp, vp, sz, P(vp)]),
        "kv_step_graph_launch": (i32, [vp, vp]),
        "kv_step_graph_destroy": (None, [vp]),
        "paged_attn_supported": (ctypes.c_int, [vp, u32, u32]),
        "kv_trace_next_kernel": (i32, [vp, vp]),
        "kv_read_probe": (i32, [vp, vp, u32, u32, u32, vp, vp]),
        "kv_last_error_message": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


_lib = _load()


def _check(st: int, deficit: int = 0) -> None:
    if st != KV_OK:
        raise KVError(st, _lib.kv_last_error_message().decode(), deficit)


def kv_last_error_message() -> str:
    return _lib.kv_last_error_message().decode()


def kv_read_probe(d_base: int, d_slice_ids: int, n_slices: int, slice_bytes: int, blocks_per_cu: int, d_sink: int,
                  stream: int) -> None:
    _check(_lib.kv_read_probe(d_base, d_slice_ids, n_slices, slice_bytes, blocks_per_cu, d_sink, stream or None))


def kv_trace_next_kernel(before: int, after: int) -> None:
    """Raw hipEvent_t handles (0, 0 clears)."""
    _check(_lib.kv_trace_next_kernel(before or None, after or None))


def kv_profile_planes(profile: int, head_dim: int, scale_dtype: int | None = None) -> list:
    """The profile's plane schema; scale_dtype KV_DT_F16 for 2-byte INT8-G64 / FP8-row scales."""
    buf = (KVPlaneDesc * 4)()
    n = ctypes.c_uint32(4)
    if scale_dtype is None:
        _check(_lib.kv_profile_planes(profile, head_dim, buf, ctypes.byref(n)))
    else:
        _check(_lib.kv_profile_planes_ex(profile, head_dim, scale_dtype, buf, ctypes.byref(n)))
    return [buf[i] for i in range(n.value)]


def kv_plane_bytes(geo: KVPageGeometry, plane: KVPlaneDesc) -> int:
    out = ctypes.c_uint64()
    _check(_lib.kv_plane_bytes(ctypes.byref(geo), ctypes.byref(plane), ctypes.byref(out)))
    return out.value


def kv_pool_create(geo: KVPageGeometry, planes: list, d_block_tables: int | None, free_order=None,
                   stream: int = 0) -> int:
    arr = (KVPlaneDesc * len(planes))(*planes)
    fo = None
    if free_order is not None:
        fo = (ctypes.c_int32 * len(free_order))(*[int(x) for x in free_order])
    out = ctypes.c_void_p()
    _check(_lib.kv_pool_create(ctypes.byref(geo), arr, len(planes), d_block_tables or None, fo, stream or None,
                               ctypes.byref(out)))
    return out.value


def kv_pool_destroy(pool: int) -> None:
    _lib.kv_pool_destroy(pool)


def kv_pool_stats(pool: int) -> tuple:
    a, r, v = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_uint32()
    _check(_lib.kv_pool_stats(pool, ctypes.byref(a), ctypes.byref(r), ctypes.byref(v)))
    return a.value, r.value, v.value


def kv_pool_table_host(pool: int, n_entries: int):
    buf = (ctypes.c_int32 * n_entries)()
    _check(_lib.kv_pool_table_host(pool, buf, n_entries))
    return list(buf)


def kv_pool_page_refs(pool: int, page_group: int) -> int:
    out = ctypes.c_uint32()
    _check(_lib.kv_pool_page_refs(pool, page_group, ctypes.byref(out)))
    return out.value


def kv_seq_open(pool: int, table_row: int, stream: int = 0) -> int:
    out = ctypes.c_uint64()
    _check(_lib.kv_seq_open(pool, table_row, stream or None, ctypes.byref(out)))
    return out.value


def kv_seq_fork(pool: int, src: int, frontier: int, table_row: int, stream: int = 0) -> int:
    out = ctypes.c_uint64()
    _check(_lib.kv_seq_fork(pool, src, frontier, table_row, stream or None, ctypes.byref(out)))
    return out.value


def kv_seq_ensure_mapped(pool: int, seq: int, tokens: int, stream: int = 0) -> None:
    deficit = ctypes.c_uint32()
    st = _lib.kv_seq_ensure_mapped(pool, seq, tokens, ctypes.byref(deficit), stream or None)
    _check(st, deficit.value)


def kv_seq_commit(pool: int, seq: int, frontier: int) -> None:
    _check(_lib.kv_seq_commit(pool, seq, frontier))


def kv_seq_release(pool: int, seq: int, stream: int = 0) -> None:
    _check(_lib.kv_seq_release(pool, seq, stream or None))


def kv_seq_reserve(pool: int, seq: int, pages: int) -> None:
    deficit = ctypes.c_uint32()
    st = _lib.kv_seq_reserve(pool, seq, pages, ctypes.byref(deficit))
    _check(st, deficit.value)


def kv_seq_trim(pool: int, seq: int, provisional: int, stream: int = 0) -> None:
    _check(_lib.kv_seq_trim(pool, seq, provisional, stream or None))


def kv_seq_commit_accepted(pool: int, seq: int, produced: int, accepted: int, cancelled: bool = False,
                           stream: int = 0) -> None:
    _check(_lib.kv_seq_commit_accepted(pool, seq, produced, accepted, int(bool(cancelled)), stream or None))


def kv_seq_reservation(pool: int, seq: int) -> int:
    out = ctypes.c_uint32()
    _check(_lib.kv_seq_reservation(pool, seq, ctypes.byref(out)))
    return out.value


def kv_draft_pool_pages(main_pages: int, max_concurrency: int, draft_window: int) -> int:
    out = ctypes.c_uint32()
    _check(_lib.kv_draft_pool_pages(main_pages, max_concurrency, draft_window, ctypes.byref(out)))
    return out.value


def kv_replica_page_bytes(pool: int) -> int:
    out = ctypes.c_uint64()
    _check(_lib.kv_replica_page_bytes(pool, ctypes.byref(out)))
    return out.value


def kv_seq_offload(pool: int, seq: int, host: int, host_bytes: int, stream: int = 0) -> tuple:
    n, f = ctypes.c_uint32(), ctypes.c_uint32()
    _check(_lib.kv_seq_offload(pool, seq, host, host_bytes, ctypes.byref(n), ctypes.byref(f), stream or None))
    return n.value, f.value


def kv_seq_restore(pool: int, table_row: int, host: int, host_bytes: int, frontier: int, stream: int = 0) -> int:
    deficit, out = ctypes.c_uint32(), ctypes.c_uint64()
    st = _lib.kv_seq_restore(pool, table_row, host, host_bytes, frontier, ctypes.byref(deficit), stream or None,
                             ctypes.byref(out))
    _check(st, deficit.value)
    return out.value


def kv_seq_info(pool: int, seq: int) -> tuple:
    r, f, m = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_uint32()
    _check(_lib.kv_seq_info(pool, seq, ctypes.byref(r), ctypes.byref(f), ctypes.byref(m)))
    return r.value, f.value, m.value


def kv_cow_tail_page(pool: int, seq: int, stream: int = 0) -> None:
    st = _lib.kv_cow_tail_page(pool, seq, stream or None)
    _check(st, 1 if st == KV_E_CAPACITY else 0)


def kv_append(pool: int, layer: int, B: int, d_table_rows: int, d_pos0: int, d_cu_tokens: int, total_tokens: int,
              d_k: int, d_v: int, stream: int = 0) -> None:
    _check(_lib.kv_append(pool, layer, B, d_table_rows, d_pos0, d_cu_tokens, total_tokens, d_k, d_v,
                          stream or None))


def paged_attn_workspace_bytes(pool: int, B: int, Hq: int, max_seq_len: int, max_q_len: int) -> int:
    return int(_lib.paged_attn_workspace_bytes(pool, B, Hq, max_seq_len, max_q_len))


def paged_attn_supported(pool: int, Hq: int, max_q_len: int) -> bool:
    return bool(_lib.paged_attn_supported(pool, Hq, max_q_len))


def paged_attn_decode(pool: int, layer: int, B: int, Hq: int, d_table_rows: int, d_seq_lens: int,
                      max_seq_len: int, d_q: int, sm_scale: float, d_out: int, d_ws: int, ws_bytes: int,
                      stream: int = 0) -> None:
    _check(_lib.paged_attn_decode(pool, layer, B, Hq, d_table_rows, d_seq_lens, max_seq_len, d_q, sm_scale, d_out,
                                  d_ws or None, ws_bytes, stream or None))


def paged_attn_decode_noalloc(pool: int, layer: int, B: int, Hq: int, d_table_rows: int, d_seq_lens: int,
                              max_seq_len: int, d_q: int, sm_scale: float, d_out: int, stream: int = 0) -> None:
    _check(_lib.paged_attn_decode_noalloc(pool, layer, B, Hq, d_table_rows, d_seq_lens, max_seq_len, d_q, sm_scale,
                                          d_out, stream or None))


def paged_attn_decode_plan(pool: int, B: int, Hq: int, d_table_rows: int, d_seq_lens: int, max_seq_len: int,
                           d_ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check(_lib.paged_attn_decode_plan(pool, B, Hq, d_table_rows, d_seq_lens, max_seq_len, d_ws or None, ws_bytes,
                                       stream or None))


def paged_attn_decode_run(pool: int, layer: int, B: int, Hq: int, max_seq_len: int, d_q: int, sm_scale: float,
                          d_out: int, d_ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check(_lib.paged_attn_decode_run(pool, layer, B, Hq, max_seq_len, d_q, sm_scale, d_out, d_ws or None, ws_bytes,
                                      stream or None))


def paged_attn_decode_append_run(pool: int, layer: int, B: int, Hq: int, max_seq_len: int, d_k: int, d_v: int,
                                 d_q: int, sm_scale: float, d_out: int, d_ws: int, ws_bytes: int,
                                 stream: int = 0) -> None:
    _check(_lib.paged_attn_decode_append_run(pool, layer, B, Hq, max_seq_len, d_k, d_v, d_q, sm_scale, d_out,
                                             d_ws or None, ws_bytes, stream or None))


def paged_attn_verify(pool: int, layer: int, B: int, Hq: int, d_table_rows: int, d_q_pos0: int, d_cu_q: int,
                      total_q: int, max_q_len: int, max_seq_len: int, d_q: int, sm_scale: float, d_out: int,
                      d_ws: int, ws_bytes: int, stream: int = 0) -> None:
    _check(_lib.paged_attn_verify(pool, layer, B, Hq, d_table_rows, d_q_pos0, d_cu_q, total_q, max_q_len,
                                  max_seq_len, d_q, sm_scale, d_out, d_ws or None, ws_bytes, stream or None))


def _ptr_array(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*[int(p) for p in ptrs])


def kv_decode_step_graph_create(pool: int, B: int, Hq: int, max_seq_len: int, d_table_rows: int, d_seq_lens: int,
                                d_q: list, sm_scale: float, d_out: list, d_ws: int, ws_bytes: int,
                                d_k: list | None = None, d_v: list | None = None, d_pos0: int = 0,
                                d_cu_tokens: int = 0, total_tokens: int | None = None) -> int:
    n = len(d_q)
    assert len(d_out) == n and (d_k is None) == (d_v is None) and (d_k is None or len(d_k) == len(d_v) == n)
    qa, oa = _ptr_array(d_q), _ptr_array(d_out)
    ka = _ptr_array(d_k) if d_k is not None else None
    va = _ptr_array(d_v) if d_v is not None else None
    out = ctypes.c_void_p()
    _check(_lib.kv_decode_step_graph_create(pool, B, Hq, max_seq_len, d_table_rows, d_seq_lens, n, ka, va,
                                            d_pos0 or None, d_cu_tokens or None,
                                            B if total_tokens is None else total_tokens, qa, sm_scale, oa, d_ws,
                                            ws_bytes, ctypes.byref(out)))
    return out.value


def kv_step_graph_launch(graph: int, stream: int = 0) -> None:
    _check(_lib.kv_step_graph_launch(graph, stream or None))


def kv_step_graph_destroy(graph: int) -> None:
    _lib.kv_step_graph_destroy(graph)
