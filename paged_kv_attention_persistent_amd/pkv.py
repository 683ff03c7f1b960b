"""ctypes binding of libpkv (include/pkv.h), same entry-point names.

Argument marshalling only: every step of decode attention runs in the HIP
kernels of libpkv.so.  Torch tensors are passed as device pointers
(``data_ptr()``) and torch streams / events as their raw HIP handles.  If the
library is missing, ``lib()`` raises; there is no fallback path.
"""

from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY names another build of the same library to load instead of the
# in-tree one (a sanitizer build, for instance); it must exist like the default.
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_CAPACITY = -3
PKV_ERR_HIP = -4
PKV_ERR_STATE = -5
PKV_ERR_DEVICE_FAULT = -6
PKV_ERR_TIMEOUT = -7

PKV_POLICY_AUTO, PKV_POLICY_NO_SPLIT, PKV_POLICY_SPLIT = 0, 1, 2
PKV_ORDER_CANONICAL, PKV_ORDER_LPT = 0, 1
PKV_SCHEDULE_ATOMIC, PKV_SCHEDULE_STATIC, PKV_SCHEDULE_PAGES, PKV_SCHEDULE_STEAL = 0, 1, 2, 3
PKV_MERGE_FUSED, PKV_MERGE_SEPARATE = 0, 1
PKV_KV_BF16, PKV_KV_F32 = 0, 1
PKV_DEVERR_NONE, PKV_DEVERR_PAGE_OOB, PKV_DEVERR_BAD_ITEM = 0, 1, 2

ITEM_DTYPE = np.dtype([("seq", "<u4"), ("kv_head", "<u2"), ("chunk", "<u2"),
                       ("tok_begin", "<u4"), ("tok_end", "<u4")])


class pkv_config(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("num_q_heads", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("page_size", C.c_int32), ("num_pages", C.c_int32),
                ("max_batch", C.c_int32), ("max_pages_per_seq", C.c_int32),
                ("scale", C.c_float), ("policy", C.c_int32), ("order", C.c_int32),
                ("kv_chunk_tokens", C.c_int32), ("num_cus", C.c_int32),
                ("max_items", C.c_int32), ("wg_per_cu", C.c_int32),
                ("merge_mode", C.c_int32), ("persistent", C.c_int32), ("num_layers", C.c_int32),
                ("timeout_ms", C.c_int32), ("schedule", C.c_int32), ("append", C.c_int32),
                ("kv_dtype", C.c_int32), ("reserved", C.c_int32 * 2)]


class pkv_tensors(C.Structure):
    _fields_ = [("q", C.c_void_p), ("k_pool", C.c_void_p), ("v_pool", C.c_void_p),
                ("block_table", C.c_void_p), ("ctx_lens", C.c_void_p),
                ("out", C.c_void_p), ("lse", C.c_void_p), ("batch", C.c_int32),
                ("block_table_stride", C.c_int32), ("layer_stride_q", C.c_int64),
                ("layer_stride_kv", C.c_int64), ("layer_stride_bt", C.c_int64),
                ("layer_stride_out", C.c_int64), ("layer_stride_lse", C.c_int64),
                ("new_k", C.c_void_p), ("new_v", C.c_void_p), ("layer_stride_new", C.c_int64)]


class pkv_queue_info(C.Structure):
    _fields_ = [("n_items", C.c_int32), ("split", C.c_int32), ("chunk_tokens", C.c_int32),
                ("n_split_rows", C.c_int32), ("n_merge_rows", C.c_int32),
                ("n_partial_slots", C.c_int32), ("launches_per_step", C.c_int32),
                ("reserved", C.c_int32), ("kv_bytes", C.c_uint64),
                ("partial_bytes", C.c_uint64)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_ if f != "reserved"}


class pkv_runtime_info(C.Structure):
    _fields_ = [("error_code", C.c_uint32), ("error_detail", C.c_uint32),
                ("queue_head", C.c_uint32), ("n_items", C.c_uint32),
                ("items_done", C.c_uint32), ("decode_calls", C.c_uint32),
                ("grid", C.c_int32), ("num_cus", C.c_int32), ("loop_out_epoch", C.c_uint32),
                ("loop_alive", C.c_uint32), ("loop_exit_reason", C.c_uint32),
                ("loop_steps_started", C.c_uint32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class pkv_layout(C.Structure):
    _fields_ = [("ctrl_off", C.c_uint64), ("queue_off", C.c_uint64),
                ("n_chunks_off", C.c_uint64), ("part_off_off", C.c_uint64),
                ("row_len_off", C.c_uint64),
                ("merge_rows_off", C.c_uint64), ("items_off", C.c_uint64),
                ("partial_o_off", C.c_uint64), ("partial_lse_off", C.c_uint64),
                ("arrive_off", C.c_uint64), ("cursor_off", C.c_uint64), ("loop_off", C.c_uint64),
                ("loop_mirror_off", C.c_uint64), ("sink_off", C.c_uint64),
                ("total_bytes", C.c_uint64),
                ("max_items", C.c_int32),
                ("reserved", C.c_int32)]


# name -> (restype, argtypes); the exported C ABI, one entry per declaration in pkv.h
SIGNATURES = {
    "pkv_workspace_size": (C.c_int32, [C.POINTER(pkv_config), C.POINTER(C.c_size_t)]),
    "pkv_workspace_layout": (C.c_int32, [C.POINTER(pkv_config), C.POINTER(pkv_layout)]),
    "pkv_create": (C.c_int32, [C.POINTER(pkv_config), C.c_void_p, C.c_size_t, C.c_void_p,
                               C.POINTER(C.c_void_p)]),
    "pkv_build_queue": (C.c_int32, [C.c_void_p, C.POINTER(C.c_int32), C.c_int32,
                                    C.POINTER(pkv_queue_info)]),
    "pkv_build_queue_device": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p]),
    "pkv_decode": (C.c_int32, [C.c_void_p, C.POINTER(pkv_tensors), C.c_void_p]),
    "pkv_set_decode_events": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "pkv_query": (C.c_int32, [C.c_void_p, C.POINTER(pkv_runtime_info)]),
    "pkv_clear_error": (C.c_int32, [C.c_void_p]),
    "pkv_destroy": (C.c_int32, [C.c_void_p]),
    "pkv_status_string": (C.c_char_p, [C.c_int32]),
    "pkv_last_error": (C.c_char_p, [C.c_void_p]),
    "pkv_plan_queue": (C.c_int32, [C.POINTER(pkv_config), C.POINTER(C.c_int32), C.c_int32,
                                   C.c_void_p, C.c_int32, C.POINTER(C.c_int32),
                                   C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                   C.POINTER(pkv_queue_info)]),
    "pkv_debug_gather": (C.c_int32, [C.c_void_p, C.POINTER(pkv_tensors), C.c_int32,
                                     C.c_void_p, C.c_void_p, C.c_void_p]),
    "pkv_queue_read": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_size_t, C.POINTER(C.c_size_t)]),
    "pkv_set_trace": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_int32]),
    "pkv_loop_set_free_pages": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_int32]),
    "pkv_loop_free_pages": (C.c_int32, [C.c_void_p, C.POINTER(C.c_int32)]),
    "pkv_copy_probe": (C.c_int32, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int32, C.c_void_p]),
    "pkv_read_probe": (C.c_int32, [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int32, C.c_void_p]),
    "pkv_decode_noalloc": (C.c_int32, [C.POINTER(pkv_config), C.c_void_p, C.c_int32,
                                       C.POINTER(pkv_tensors), C.c_void_p, C.c_void_p]),
}

_LIB = None


def lib() -> C.CDLL:
    """Load libpkv.so (built in-tree by ``build.py``); raise if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_attention_persistent_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = lib().pkv_status_string(status).decode()
        super().__init__(f"{where}: {msg} ({status}){': ' + detail if detail else ''}")


def _check(status: int, where: str, handle=None) -> None:
    if status != PKV_OK:
        detail = lib().pkv_last_error(handle).decode() if handle else ""
        raise PkvError(status, where, detail)


def make_config(num_q_heads, num_kv_heads, head_dim, num_pages, max_batch, max_pages_per_seq,
                page_size=16, scale=0.0, policy=PKV_POLICY_AUTO, order=PKV_ORDER_CANONICAL,
                kv_chunk_tokens=0, num_cus=0, max_items=0, wg_per_cu=0,
                merge_mode=PKV_MERGE_FUSED, persistent=0, num_layers=0,
                timeout_ms=0, schedule=0, append=0, kv_dtype=PKV_KV_BF16) -> pkv_config:
    cfg = pkv_config()
    cfg.struct_size = C.sizeof(pkv_config)
    cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim = num_q_heads, num_kv_heads, head_dim
    cfg.page_size, cfg.num_pages = page_size, num_pages
    cfg.max_batch, cfg.max_pages_per_seq = max_batch, max_pages_per_seq
    cfg.scale, cfg.policy, cfg.order = scale, policy, order
    cfg.kv_chunk_tokens, cfg.num_cus, cfg.max_items, cfg.wg_per_cu = \
        kv_chunk_tokens, num_cus, max_items, wg_per_cu
    cfg.merge_mode = merge_mode
    cfg.persistent, cfg.num_layers, cfg.timeout_ms = persistent, num_layers, timeout_ms
    cfg.schedule = schedule
    cfg.append = append
    cfg.kv_dtype = kv_dtype
    return cfg


def pkv_workspace_size(cfg: pkv_config) -> int:
    n = C.c_size_t(0)
    _check(lib().pkv_workspace_size(C.byref(cfg), C.byref(n)), "pkv_workspace_size")
    return int(n.value)


def pkv_workspace_layout(cfg: pkv_config) -> pkv_layout:
    lay = pkv_layout()
    _check(lib().pkv_workspace_layout(C.byref(cfg), C.byref(lay)), "pkv_workspace_layout")
    return lay


def _stream_ptr(stream) -> int:
    if stream is None:
        return 0
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def pkv_create(cfg: pkv_config, workspace, stream=None) -> int:
    """workspace: a uint8 device tensor of at least pkv_workspace_size bytes."""
    h = C.c_void_p(0)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().pkv_create(C.byref(cfg), C.c_void_p(workspace.data_ptr()), nbytes,
                            C.c_void_p(_stream_ptr(stream)), C.byref(h)), "pkv_create")
    return h.value


def pkv_build_queue(handle: int, ctx_lens) -> pkv_queue_info:
    arr = np.ascontiguousarray(np.asarray(ctx_lens, dtype=np.int32))
    info = pkv_queue_info()
    ptr = arr.ctypes.data_as(C.POINTER(C.c_int32))
    _check(lib().pkv_build_queue(C.c_void_p(handle), ptr, int(arr.shape[0]), C.byref(info)),
           "pkv_build_queue", C.c_void_p(handle))
    return info


def pkv_build_queue_device(handle: int, ctx_lens_dev, stream=None) -> None:
    _check(lib().pkv_build_queue_device(C.c_void_p(handle), C.c_void_p(ctx_lens_dev.data_ptr()),
                                        int(ctx_lens_dev.numel()), C.c_void_p(_stream_ptr(stream))),
           "pkv_build_queue_device", C.c_void_p(handle))


def make_tensors(q, k_pool, v_pool, block_table, ctx_lens, out, lse, batch=None,
                 block_table_stride=0, layer_strides=None, new_k=None, new_v=None,
                 layer_stride_new=0) -> pkv_tensors:
    """layer_strides: (q, kv, bt, out, lse) element strides for layered tensors;
    new_k / new_v: the newest token's K / V for a loop with append."""
    t = pkv_tensors()
    t.q, t.k_pool, t.v_pool = q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr()
    t.block_table = block_table.data_ptr()
    t.ctx_lens = ctx_lens.data_ptr() if ctx_lens is not None else None
    t.out, t.lse = out.data_ptr(), lse.data_ptr()
    t.batch = int(q.shape[0]) if batch is None else int(batch)
    t.block_table_stride = int(block_table_stride or block_table.shape[-1])
    if layer_strides is not None:
        (t.layer_stride_q, t.layer_stride_kv, t.layer_stride_bt, t.layer_stride_out,
         t.layer_stride_lse) = [int(x) for x in layer_strides]
    if new_k is not None:
        t.new_k, t.new_v = new_k.data_ptr(), new_v.data_ptr()
        t.layer_stride_new = int(layer_stride_new)
    return t


def pkv_decode(handle: int, tensors: pkv_tensors, stream=None) -> None:
    _check(lib().pkv_decode(C.c_void_p(handle), C.byref(tensors), C.c_void_p(_stream_ptr(stream))),
           "pkv_decode", C.c_void_p(handle))


def pkv_set_decode_events(handle: int, before=None, after=None) -> None:
    b = int(before.cuda_event) if before is not None else None
    a = int(after.cuda_event) if after is not None else None
    _check(lib().pkv_set_decode_events(C.c_void_p(handle), C.c_void_p(b), C.c_void_p(a)),
           "pkv_set_decode_events", C.c_void_p(handle))


def pkv_query(handle: int, raise_on_fault: bool = True) -> dict:
    info = pkv_runtime_info()
    st = lib().pkv_query(C.c_void_p(handle), C.byref(info))
    if st != PKV_ERR_DEVICE_FAULT or raise_on_fault:
        _check(st, "pkv_query", C.c_void_p(handle))
    d = info.as_dict()
    d["status"] = st
    return d


def pkv_clear_error(handle: int) -> None:
    _check(lib().pkv_clear_error(C.c_void_p(handle)), "pkv_clear_error", C.c_void_p(handle))


def pkv_destroy(handle: int) -> None:
    _check(lib().pkv_destroy(C.c_void_p(handle)), "pkv_destroy")


def pkv_status_string(status: int) -> str:
    return lib().pkv_status_string(status).decode()


def pkv_plan_queue(cfg: pkv_config, ctx_lens, items_cap: int | None = None):
    """Host-only planning: (items ITEM_DTYPE array, n_chunks, part_off, merge_rows, info)."""
    arr = np.ascontiguousarray(np.asarray(ctx_lens, dtype=np.int32))
    bsz = int(arr.shape[0])
    if items_cap is None:
        items_cap = pkv_workspace_layout(cfg).max_items
    items = np.zeros(max(items_cap, 1), dtype=ITEM_DTYPE)
    n_chunks = np.zeros(max(bsz, 1), dtype=np.int32)
    part_off = np.zeros(bsz + 1, dtype=np.int32)
    merge_rows = np.zeros(max(bsz, 1), dtype=np.int32)
    info = pkv_queue_info()
    P32 = C.POINTER(C.c_int32)
    st = lib().pkv_plan_queue(C.byref(cfg), arr.ctypes.data_as(P32), bsz,
                              items.ctypes.data_as(C.c_void_p), int(items_cap),
                              n_chunks.ctypes.data_as(P32), part_off.ctypes.data_as(P32),
                              merge_rows.ctypes.data_as(P32), C.byref(info))
    _check(st, "pkv_plan_queue")
    return (items[:info.n_items].copy(), n_chunks[:bsz].copy(), part_off,
            merge_rows[:info.n_merge_rows].copy(), info)


def pkv_debug_gather(handle: int, tensors: pkv_tensors, item_index: int, k_out, v_out,
                     stream=None) -> None:
    _check(lib().pkv_debug_gather(C.c_void_p(handle), C.byref(tensors), int(item_index),
                                  C.c_void_p(k_out.data_ptr()), C.c_void_p(v_out.data_ptr()),
                                  C.c_void_p(_stream_ptr(stream))),
           "pkv_debug_gather", C.c_void_p(handle))


def pkv_queue_read(handle: int, capacity: int) -> bytes:
    """The device queue as the decode kernel reads it (see pkv.h)."""
    buf = C.create_string_buffer(int(capacity))
    n = C.c_size_t(0)
    _check(lib().pkv_queue_read(C.c_void_p(handle), buf, int(capacity), C.byref(n)), "pkv_queue_read",
           C.c_void_p(handle))
    return buf.raw[:n.value]


def pkv_loop_set_free_pages(handle: int, pages) -> None:
    arr = np.ascontiguousarray(np.asarray(pages, dtype=np.int32))
    _check(lib().pkv_loop_set_free_pages(C.c_void_p(handle), arr.ctypes.data_as(C.c_void_p), int(arr.size)),
           "pkv_loop_set_free_pages", C.c_void_p(handle))


def pkv_loop_free_pages(handle: int) -> int:
    n = C.c_int32(0)
    _check(lib().pkv_loop_free_pages(C.c_void_p(handle), C.byref(n)), "pkv_loop_free_pages",
           C.c_void_p(handle))
    return int(n.value)


def pkv_set_trace(handle: int, buf=None) -> None:
    """buf: a device int64 tensor of 4 * capacity elements, or None."""
    ptr = buf.data_ptr() if buf is not None else None
    cap = buf.numel() // 4 if buf is not None else 0
    _check(lib().pkv_set_trace(C.c_void_p(handle), C.c_void_p(ptr), int(cap)), "pkv_set_trace",
           C.c_void_p(handle))


def pkv_copy_probe(dst, src, nbytes: int, grid: int = 0, stream=None) -> None:
    _check(lib().pkv_copy_probe(C.c_void_p(dst.data_ptr()), C.c_void_p(src.data_ptr()), int(nbytes),
                                int(grid), C.c_void_p(_stream_ptr(stream))), "pkv_copy_probe")


def pkv_read_probe(src, nbytes: int, sink, grid: int = 0, stream=None) -> None:
    """sink: a device int32 tensor of at least grid * 256 elements."""
    _check(lib().pkv_read_probe(C.c_void_p(src.data_ptr()), int(nbytes), C.c_void_p(sink.data_ptr()),
                                int(grid), C.c_void_p(_stream_ptr(stream))), "pkv_read_probe")


def pkv_decode_noalloc(cfg: pkv_config, ctx_lens_dev, tensors: pkv_tensors, error_word=None,
                       stream=None) -> None:
    """Decode with the library's static scratch (no workspace, no handle)."""
    ew = C.c_void_p(error_word.data_ptr()) if error_word is not None else C.c_void_p(None)
    _check(lib().pkv_decode_noalloc(C.byref(cfg), C.c_void_p(ctx_lens_dev.data_ptr()),
                                    int(ctx_lens_dev.numel()), C.byref(tensors), ew,
                                    C.c_void_p(_stream_ptr(stream))), "pkv_decode_noalloc")


class PagedDecoder:
    """A handle plus its workspace tensor, for one model shape.

    Owns nothing but the handle; the workspace is an ordinary torch tensor
    allocated here and kept alive with the handle.
    """

    def __init__(self, cfg: pkv_config, device="cuda", stream=None):
        import torch
        self.cfg = cfg
        self.layout = pkv_workspace_layout(cfg)
        self.workspace = torch.empty(self.layout.total_bytes, dtype=torch.uint8, device=device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(device)
        self.handle = pkv_create(cfg, self.workspace, self.stream)
        self.info = None

    def build_queue(self, ctx_lens) -> pkv_queue_info:
        self.info = pkv_build_queue(self.handle, ctx_lens)
        return self.info

    def build_queue_device(self, ctx_lens_dev) -> None:
        pkv_build_queue_device(self.handle, ctx_lens_dev, self.stream)

    def decode(self, q, k_pool, v_pool, block_table, ctx_lens, out, lse, stream=None):
        t = make_tensors(q, k_pool, v_pool, block_table, ctx_lens, out, lse)
        pkv_decode(self.handle, t, stream if stream is not None else self.stream)

    def query(self, raise_on_fault=True) -> dict:
        return pkv_query(self.handle, raise_on_fault)

    def region(self, name: str, nbytes: int):
        """A uint8 view of a workspace region (for inspection in tests)."""
        off = getattr(self.layout, name + "_off")
        return self.workspace[off:off + nbytes]

    def close(self):
        if self.handle:
            pkv_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
