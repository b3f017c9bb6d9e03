"""ctypes binding of libwf.so: the C ABI declared in include/wf.h, same names.

Argument marshalling only. Device buffers are passed as raw pointers (torch
tensors are accepted and passed by data_ptr()); streams as hipStream_t
handles (a torch.cuda.Stream, an int, or None for torch's current stream).
Every call that returns a non-zero status raises WfError.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwf.so")

WF_OK = 0
WF_E_INVALID_ARG = 1
WF_E_SHAPE = 2
WF_E_NOT_READY = 3
WF_E_HIP = 4

WF_MASK_WAVEFRONT = 0
WF_MASK_ALL_LIVE = 1

WF_DTYPE_BF16 = 0
WF_DTYPE_FP32 = 1
WF_DTYPE_FP8_E4M3 = 2


class wf_config(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int32),
        ("anchor_chunks", ctypes.c_int32),
        ("history_chunks", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_layers", ctypes.c_int32),
        ("chunk_frames", ctypes.c_int32),
        ("frame_h", ctypes.c_int32),
        ("frame_w", ctypes.c_int32),
        ("page_tokens", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("qk_dtype", ctypes.c_int32),
        ("rope_split", ctypes.c_int32 * 3),
        ("first_round", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("live_mask", ctypes.c_int32),
        ("total_chunks", ctypes.c_int32),
    ]


class WfError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        msg = "%s failed: %s (status %d)" % (where, status_string(status), status)
        if detail:
            msg += ": " + detail
        super().__init__(msg)


_lib = None


def load() -> ctypes.CDLL:
    """Load libwf.so (built in-tree by build.py). Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libwf.so is not built at %s; run __graft_entry__.build() "
                          "(or python -m wavefront_causal_attention_amd.build)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I32, I64 = ctypes.c_int32, ctypes.c_int64
    sig = {
        "wf_pool_bytes": (ctypes.c_int, [ctypes.POINTER(wf_config), ctypes.POINTER(ctypes.c_size_t),
                                         ctypes.POINTER(ctypes.c_size_t)]),
        "wf_pool_create": (ctypes.c_int, [ctypes.POINTER(wf_config), P, ctypes.c_size_t, P,
                                          ctypes.c_size_t, ctypes.POINTER(P)]),
        "wf_pool_create_host_model": (ctypes.c_int, [ctypes.POINTER(wf_config), ctypes.POINTER(P)]),
        "wf_pool_destroy": (None, [P]),
        "wf_kv_publish": (ctypes.c_int, [P, I32, I32, I32, P, P, P, I64, P, P, P, P]),
        "wf_kv_publish_noalloc": (ctypes.c_int, [P, I32, I32, I32, P, P, P, I64, P, P, P, P]),
        "wf_qkv_project_publish": (ctypes.c_int, [P, I32, I32, I32, P, I64, I32, P, P, P, P, P]),
        "wf_qkv_project_publish_w8a8": (ctypes.c_int, [P, I32, I32, I32, P, I64, P, I32, P, P, P, P, P, P]),
        "wf_quantize_rows_fp8": (ctypes.c_int, [P, I64, I32, I64, P, I64, P, P]),
        "wf_attention_round": (ctypes.c_int, [P, I32, I32, I32, P, P, P, I32, P]),
        "wf_round_advance": (ctypes.c_int, [P, P]),
        "wf_round_replayed": (ctypes.c_int, [P]),
        "wf_attention_work_list": (ctypes.c_int, [ctypes.POINTER(wf_config), I32, I32, I32, P, I64,
                                                  ctypes.POINTER(I64)]),
        "wf_round_index": (ctypes.c_int, [P, ctypes.POINTER(I64)]),
        "wf_schedule_chunk_ids": (ctypes.c_int, [P, P]),
        "wf_page_table_host": (ctypes.c_int, [P, P]),
        "wf_ready_mask": (ctypes.c_int, [P, I32, ctypes.POINTER(ctypes.c_uint64)]),
        "wf_geometry": (ctypes.c_int, [P, P]),
        "wf_mfma_calibrate": (ctypes.c_int, [I32, I32, P, P]),
        "wf_stream_copy_calibrate": (ctypes.c_int, [P, P, I64, P]),
        "wf_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "wf_last_error": (ctypes.c_char_p, [P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().wf_status_string(int(status)).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError("expected a tensor, an int address or None, got %r" % type(x))


def _stream(st):
    if st is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(st, int):
        return st
    return st.cuda_stream


def _check(status, where, handle=None):
    if status != WF_OK:
        detail = load().wf_last_error(handle).decode() if handle else ""
        raise WfError(status, where, detail)


def wf_pool_bytes(cfg: wf_config):
    pb, tb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().wf_pool_bytes(ctypes.byref(cfg), ctypes.byref(pb), ctypes.byref(tb)), "wf_pool_bytes")
    return pb.value, tb.value


def wf_pool_create(cfg: wf_config, pool, pool_bytes: int, page_table, table_bytes: int) -> int:
    h = ctypes.c_void_p()
    _check(load().wf_pool_create(ctypes.byref(cfg), _ptr(pool), pool_bytes, _ptr(page_table),
                                 table_bytes, ctypes.byref(h)), "wf_pool_create")
    return h.value


def wf_pool_create_host_model(cfg: wf_config) -> int:
    h = ctypes.c_void_p()
    _check(load().wf_pool_create_host_model(ctypes.byref(cfg), ctypes.byref(h)), "wf_pool_create_host_model")
    return h.value


def wf_mfma_calibrate(blocks, steps, out, stream=None) -> None:
    _check(load().wf_mfma_calibrate(int(blocks), int(steps), _ptr(out), _stream(stream)), "wf_mfma_calibrate")


def wf_stream_copy_calibrate(src, dst, nbytes, stream=None) -> None:
    _check(load().wf_stream_copy_calibrate(_ptr(src), _ptr(dst), int(nbytes), _stream(stream)),
           "wf_stream_copy_calibrate")


def wf_pool_destroy(h: int) -> None:
    load().wf_pool_destroy(h)


def wf_kv_publish(h, layer, slot_first, nslots, q, k, v, row_stride_elems,
                  chunk_t0=None, q_out=None, q_scales=None, stream=None, noalloc=False) -> None:
    """noalloc: call wf_kv_publish_noalloc (same arguments)."""
    t0 = None
    if chunk_t0 is not None:
        arr = (ctypes.c_int32 * len(chunk_t0))(*[int(x) for x in chunk_t0])
        t0 = ctypes.cast(arr, ctypes.c_void_p)
    name = "wf_kv_publish_noalloc" if noalloc else "wf_kv_publish"
    _check(getattr(load(), name)(h, layer, slot_first, nslots, _ptr(q), _ptr(k), _ptr(v),
                                 int(row_stride_elems), t0, _ptr(q_out), _ptr(q_scales),
                                 _stream(stream)), name, h)


def wf_qkv_project_publish(h, layer, slot_first, nslots, x, x_row_stride_elems, hidden, w, bias=None,
                           chunk_t0=None, q_out=None, stream=None) -> None:
    t0 = None
    if chunk_t0 is not None:
        arr = (ctypes.c_int32 * len(chunk_t0))(*[int(v) for v in chunk_t0])
        t0 = ctypes.cast(arr, ctypes.c_void_p)
    _check(load().wf_qkv_project_publish(h, layer, slot_first, nslots, _ptr(x), int(x_row_stride_elems),
                                         int(hidden), _ptr(w), _ptr(bias), t0, _ptr(q_out), _stream(stream)),
           "wf_qkv_project_publish", h)


def wf_qkv_project_publish_w8a8(h, layer, slot_first, nslots, x8, x_row_stride, x_scales, hidden, w8, w_scales,
                                bias=None, chunk_t0=None, q_out=None, stream=None) -> None:
    t0 = None
    if chunk_t0 is not None:
        arr = (ctypes.c_int32 * len(chunk_t0))(*[int(v) for v in chunk_t0])
        t0 = ctypes.cast(arr, ctypes.c_void_p)
    _check(load().wf_qkv_project_publish_w8a8(h, layer, slot_first, nslots, _ptr(x8), int(x_row_stride),
                                              _ptr(x_scales), int(hidden), _ptr(w8), _ptr(w_scales), _ptr(bias),
                                              t0, _ptr(q_out), _stream(stream)),
           "wf_qkv_project_publish_w8a8", h)


def wf_quantize_rows_fp8(x, rows, cols, x_row_stride, codes, code_row_stride, scales, stream=None) -> None:
    _check(load().wf_quantize_rows_fp8(_ptr(x), int(rows), int(cols), int(x_row_stride), _ptr(codes),
                                       int(code_row_stride), _ptr(scales), _stream(stream)),
           "wf_quantize_rows_fp8")


def wf_attention_round(h, layer, slot_first, nslots, q, q_scales, out, out_dtype, stream=None) -> None:
    _check(load().wf_attention_round(h, layer, slot_first, nslots, _ptr(q), _ptr(q_scales),
                                     _ptr(out), int(out_dtype), _stream(stream)),
           "wf_attention_round", h)


def wf_round_advance(h, stream=None) -> None:
    _check(load().wf_round_advance(h, _stream(stream)), "wf_round_advance", h)


def wf_round_replayed(h) -> None:
    _check(load().wf_round_replayed(h), "wf_round_replayed", h)


def wf_round_index(h) -> int:
    k = ctypes.c_int64()
    _check(load().wf_round_index(h, ctypes.byref(k)), "wf_round_index")
    return k.value


def wf_schedule_chunk_ids(h, T: int):
    arr = (ctypes.c_int64 * T)()
    _check(load().wf_schedule_chunk_ids(h, ctypes.cast(arr, ctypes.c_void_p)), "wf_schedule_chunk_ids")
    return list(arr)


def wf_page_table_host(h, n: int):
    arr = (ctypes.c_int32 * n)()
    _check(load().wf_page_table_host(h, ctypes.cast(arr, ctypes.c_void_p)), "wf_page_table_host")
    return list(arr)


def wf_ready_mask(h, layer: int) -> int:
    m = ctypes.c_uint64()
    _check(load().wf_ready_mask(h, layer, ctypes.byref(m)), "wf_ready_mask")
    return m.value


def wf_attention_work_list(cfg, slot_first, nslots, cus_per_xcd):
    """The attention launch order for a slot range: list of (slot, head, qtile) or None (idle)."""
    n = ctypes.c_int64(0)
    _check(load().wf_attention_work_list(ctypes.byref(cfg), slot_first, nslots, cus_per_xcd, None, 0,
                                         ctypes.byref(n)), "wf_attention_work_list")
    arr = (ctypes.c_int32 * n.value)()
    _check(load().wf_attention_work_list(ctypes.byref(cfg), slot_first, nslots, cus_per_xcd,
                                         ctypes.cast(arr, ctypes.c_void_p), n.value, ctypes.byref(n)),
           "wf_attention_work_list")
    # uint32 fields: slot 31..26, head 25..16, query tile 15..0; -1 is padding
    return [None if x == -1 else ((x & 0xFFFFFFFF) >> 26, (x >> 16) & 1023, x & 0xFFFF) for x in arr]


def wf_geometry(h):
    arr = (ctypes.c_int64 * 12)()
    _check(load().wf_geometry(h, ctypes.cast(arr, ctypes.c_void_p)), "wf_geometry")
    keys = ["N", "T", "ppc", "k_off", "v_off", "k_layer_bytes", "v_layer_bytes", "kscale_off",
            "kscale_layer_bytes", "kmean_off", "kmean_layer_bytes", "nblk"]
    return dict(zip(keys, list(arr)))


EXPORTED = [
    "wf_pool_bytes", "wf_pool_create", "wf_pool_create_host_model", "wf_pool_destroy",
    "wf_mfma_calibrate", "wf_stream_copy_calibrate", "wf_kv_publish", "wf_kv_publish_noalloc", "wf_qkv_project_publish", "wf_qkv_project_publish_w8a8", "wf_quantize_rows_fp8",
    "wf_attention_round", "wf_round_advance", "wf_round_replayed", "wf_round_index",
    "wf_attention_work_list",
    "wf_schedule_chunk_ids", "wf_page_table_host", "wf_ready_mask", "wf_geometry",
    "wf_status_string", "wf_last_error",
]
