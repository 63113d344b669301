"""MI355X (gfx950) quantized Mixture-of-Experts FFN block.

A thin ctypes binding of libqmoe.so: every function below has the name of the
C entry point it calls (include/moe.h) and only marshals arguments. Device
buffers are torch tensors on the GPU (torch supplies memory and streams);
every step of the block runs in the library's HIP kernels. There is no CPU
fallback: if the library is missing the import of a function fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

__all__ = [
    "MoeError", "MoeShape", "moe_shape", "moe_layer", "lib",
    "moe_workspace_bytes", "moe_workspace_init", "moe_matrix4_bytes", "moe_matrix8_bytes",
    "moe_expert_blob_bytes", "moe_shared_blob_bytes", "moe_router_blob_bytes",
    "moe_pack_matrix4", "moe_pack_matrix8", "moe_unpack_matrix4", "moe_unpack_matrix8",
    "moe_router_topk", "moe_group_by_expert", "moe_expert_ffn_decode", "moe_expert_ffn_prefill_chunk",
    "moe_combine", "moe_layer_decode", "moe_layer_decode_noalloc", "moe_stack_decode", "moe_layer_prefill",
    "moe_status_string",
    "moe_check_device_error",
    "moe_cache_create", "moe_cache_acquire", "moe_cache_stats", "moe_cache_destroy",
    "moe_cache_create_device", "moe_cache_device_state_bytes", "moe_cache_lookup", "moe_cache_decode",
    "moe_shared_expert_decode", "moe_combine_decode",
    "MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED_SHAPE", "MOE_ERR_WORKSPACE", "MOE_ERR_HIP",
    "MOE_ERR_DEVICE_CHECK", "MOE_F32", "MOE_BF16", "MOE_DEVERR_BAD_SLOT",
]

# the in-tree build; QMOE_LIB names another build of the same sources instead (a sanitizer
# build of the host code, or a variant to compare against)
LIB_PATH = os.environ.get("QMOE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED_SHAPE, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_DEVICE_CHECK = \
    0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16 = 0, 1
MOE_DEVERR_BAD_SLOT = 1
MOE_DEVERR_BAD_EXPERT_ID = 2
MOE_DEVERR_SYNC_TIMEOUT = 4
MOE_SLOT_SKIP = 0xFFFFFFFF


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (%d)" % (where, moe_status_string(status), status))
        self.status = status


class moe_shape(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("d_ff", C.c_int32), ("d_ff_shared", C.c_int32),
                ("n_experts", C.c_int32), ("top_k", C.c_int32), ("group", C.c_int32)]


class moe_layer(C.Structure):
    _fields_ = [("pool", C.c_void_p), ("blob_stride", C.c_uint64), ("n_blobs", C.c_uint64),
                ("slot_table", C.c_void_p), ("router_blob", C.c_void_p), ("shared_blob", C.c_void_p)]


def MoeShape(d_model: int, d_ff: int, d_ff_shared: int, n_experts: int = 128, top_k: int = 8,
             group: int = 64) -> moe_shape:
    return moe_shape(d_model, d_ff, d_ff_shared, n_experts, top_k, group)


def as_shape(s) -> moe_shape:
    """Accepts a moe_shape or any object with the same attribute names."""
    if isinstance(s, moe_shape):
        return s
    return moe_shape(s.d_model, s.d_ff, s.d_ff_shared, s.n_experts, s.top_k, getattr(s, "group", 64))


_lib = None
_P = C.c_void_p


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libqmoe.so is not built (%s); run __graft_entry__.build() or "
                              "python quantized_mixture_experts_bit_amd/build.py" % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        S, Ly = C.POINTER(moe_shape), C.POINTER(moe_layer)
        i32, u64, st = C.c_int32, C.c_uint64, C.c_int
        sig = {
            "moe_workspace_bytes": (C.c_size_t, [S, i32]),
            "moe_workspace_init": (st, [_P, C.c_size_t, _P]),
            "moe_matrix4_bytes": (u64, [i32, i32]),
            "moe_matrix8_bytes": (u64, [i32, i32]),
            "moe_expert_blob_bytes": (u64, [S]),
            "moe_shared_blob_bytes": (u64, [S]),
            "moe_router_blob_bytes": (u64, [S]),
            "moe_pack_matrix4": (st, [_P, _P, _P, i32, i32, _P]),
            "moe_pack_matrix8": (st, [_P, _P, _P, i32, i32, _P]),
            "moe_unpack_matrix4": (st, [_P, i32, i32, _P, _P, _P]),
            "moe_unpack_matrix8": (st, [_P, i32, i32, _P, _P, _P]),
            "moe_router_topk": (st, [S, Ly, _P, st, i32, _P, _P, _P, _P, _P, C.c_size_t, _P]),
            "moe_group_by_expert": (st, [S, _P, i32, _P, _P, _P, _P, _P, C.c_size_t, _P]),
            "moe_expert_ffn_decode": (st, [S, Ly, _P, st, _P, _P, _P, C.c_size_t, _P]),
            "moe_expert_ffn_prefill_chunk": (st, [S, Ly, _P, st, i32, _P, _P, _P, _P, C.c_size_t, _P]),
            "moe_combine": (st, [S, Ly, _P, st, i32, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
            "moe_shared_expert_decode": (st, [S, Ly, _P, st, _P, C.c_size_t, _P]),
            "moe_combine_decode": (st, [S, _P, _P, _P, _P, _P, C.c_size_t, _P]),
            "moe_layer_decode": (st, [S, Ly, _P, st, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
            "moe_layer_decode_noalloc": (st, [S, Ly, _P, st, _P, _P, _P, _P, _P, _P, _P]),
            "moe_stack_decode": (st, [S, Ly, i32, _P, C.POINTER(_P), _P, _P, _P, _P, _P, _P, C.c_size_t, _P]),
            "moe_layer_prefill": (st, [S, Ly, _P, st, i32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       C.c_size_t, _P]),
            "moe_status_string": (C.c_char_p, [st]),
            "moe_check_device_error": (st, [_P, C.POINTER(C.c_uint32)]),
            "moe_cache_create": (st, [i32, i32, i32, u64, _P, _P, _P, C.POINTER(_P)]),
            "moe_cache_device_state_bytes": (u64, [i32, i32, i32]),
            "moe_cache_create_device": (st, [i32, i32, i32, u64, _P, _P, _P, _P, u64, _P, C.POINTER(_P)]),
            "moe_cache_acquire": (st, [_P, i32, _P, i32, _P, _P, _P]),
            "moe_cache_lookup": (st, [_P, i32, _P, i32, _P]),
            "moe_cache_decode": (st, [_P, i32, S, _P, _P, _P, st, _P, _P, _P, _P, _P, _P, _P, _P, C.c_size_t, _P,
                                      _P]),
            "moe_cache_stats": (st, [_P, C.POINTER(u64), C.POINTER(u64), C.POINTER(u64)]),
            "moe_cache_destroy": (st, [_P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


# ------------------------------------------------------------------ marshalling helpers

def _dptr(t) -> Optional[int]:
    """Device pointer of a torch tensor on the GPU (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a GPU tensor, got one on %s" % t.device)
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _hptr(a) -> int:
    """Host pointer of a C-contiguous numpy array."""
    if not a.flags.c_contiguous:
        raise ValueError("expected a C-contiguous host array")
    return a.ctypes.data


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dtype_code(x) -> int:
    import torch
    if x.dtype == torch.bfloat16:
        return MOE_BF16
    if x.dtype == torch.float32:
        return MOE_F32
    raise ValueError("activations must be float32 or bfloat16, got %s" % x.dtype)


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


# ------------------------------------------------------------------ sizes and packing

def moe_workspace_bytes(shape, rows: int) -> int:
    return lib().moe_workspace_bytes(C.byref(as_shape(shape)), rows)


def moe_workspace_init(ws, stream=None) -> None:
    _check(lib().moe_workspace_init(_dptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_workspace_init")


def moe_matrix4_bytes(rows: int, cols: int) -> int:
    return lib().moe_matrix4_bytes(rows, cols)


def moe_matrix8_bytes(rows: int, cols: int) -> int:
    return lib().moe_matrix8_bytes(rows, cols)


def moe_expert_blob_bytes(shape) -> int:
    return lib().moe_expert_blob_bytes(C.byref(as_shape(shape)))


def moe_shared_blob_bytes(shape) -> int:
    return lib().moe_shared_blob_bytes(C.byref(as_shape(shape)))


def moe_router_blob_bytes(shape) -> int:
    return lib().moe_router_blob_bytes(C.byref(as_shape(shape)))


def moe_pack_matrix4(q, s, b, out) -> None:
    rows, cols = q.shape[0], q.shape[1] * 2
    _check(lib().moe_pack_matrix4(_hptr(q), _hptr(s), _hptr(b), rows, cols, _hptr(out)), "moe_pack_matrix4")


def moe_pack_matrix8(q, s, b, out) -> None:
    rows, cols = q.shape
    _check(lib().moe_pack_matrix8(_hptr(q), _hptr(s), _hptr(b), rows, cols, _hptr(out)), "moe_pack_matrix8")


def moe_unpack_matrix4(buf, rows: int, cols: int, q, s, b) -> None:
    _check(lib().moe_unpack_matrix4(_hptr(buf), rows, cols, _hptr(q), _hptr(s), _hptr(b)), "moe_unpack_matrix4")


def moe_unpack_matrix8(buf, rows: int, cols: int, q, s, b) -> None:
    _check(lib().moe_unpack_matrix8(_hptr(buf), rows, cols, _hptr(q), _hptr(s), _hptr(b)), "moe_unpack_matrix8")


# ------------------------------------------------------------------ the block's steps

def moe_router_topk(shape, layer: moe_layer, x, rows: int, logit_offset, topk_idx, topk_w, logits, ws,
                    stream=None) -> None:
    _check(lib().moe_router_topk(C.byref(as_shape(shape)), C.byref(layer), _dptr(x), _dtype_code(x), rows,
                                 _dptr(logit_offset), _dptr(topk_idx), _dptr(topk_w), _dptr(logits), _dptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)), "moe_router_topk")


def moe_group_by_expert(shape, topk_idx, rows: int, count, offset, perm, inv_perm, ws, stream=None) -> None:
    _check(lib().moe_group_by_expert(C.byref(as_shape(shape)), _dptr(topk_idx), rows, _dptr(count), _dptr(offset),
                                     _dptr(perm), _dptr(inv_perm), _dptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)), "moe_group_by_expert")


def moe_expert_ffn_decode(shape, layer: moe_layer, x, topk_idx, expert_out, ws, stream=None) -> None:
    _check(lib().moe_expert_ffn_decode(C.byref(as_shape(shape)), C.byref(layer), _dptr(x), _dtype_code(x),
                                       _dptr(topk_idx), _dptr(expert_out), _dptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream)), "moe_expert_ffn_decode")


def moe_expert_ffn_prefill_chunk(shape, layer: moe_layer, x, rows: int, offset, perm, expert_out, ws,
                                 stream=None) -> None:
    _check(lib().moe_expert_ffn_prefill_chunk(C.byref(as_shape(shape)), C.byref(layer), _dptr(x), _dtype_code(x),
                                              rows, _dptr(offset), _dptr(perm), _dptr(expert_out), _dptr(ws),
                                              ws.numel() * ws.element_size(), _stream(stream)),
           "moe_expert_ffn_prefill_chunk")


def moe_combine(shape, layer: moe_layer, x, rows: int, expert_out, inv_perm, topk_w, y, residual, ws,
                stream=None) -> None:
    _check(lib().moe_combine(C.byref(as_shape(shape)), C.byref(layer), _dptr(x), _dtype_code(x), rows,
                             _dptr(expert_out), _dptr(inv_perm), _dptr(topk_w), _dptr(y), _dptr(residual),
                             _dptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_combine")


def moe_shared_expert_decode(shape, layer: moe_layer, x, ws, stream=None) -> None:
    _check(lib().moe_shared_expert_decode(C.byref(as_shape(shape)), C.byref(layer), _dptr(x), _dtype_code(x),
                                          _dptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_shared_expert_decode")


def moe_combine_decode(shape, expert_out, topk_w, y, residual, ws, stream=None) -> None:
    _check(lib().moe_combine_decode(C.byref(as_shape(shape)), _dptr(expert_out), _dptr(topk_w), _dptr(y),
                                    _dptr(residual), _dptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_combine_decode")


def moe_layer_decode(shape, layer: moe_layer, x, logit_offset, topk_idx, topk_w, expert_out, y, residual, ws,
                     stream=None) -> None:
    _check(lib().moe_layer_decode(C.byref(as_shape(shape)), C.byref(layer), _dptr(x), _dtype_code(x),
                                  _dptr(logit_offset), _dptr(topk_idx), _dptr(topk_w), _dptr(expert_out), _dptr(y),
                                  _dptr(residual), _dptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "moe_layer_decode")


def moe_layer_decode_noalloc(shape, layer: moe_layer, x, logit_offset, topk_idx, topk_w, expert_out, y, residual,
                             stream=None) -> None:
    """moe_layer_decode on the library's static device scratch (no workspace argument)."""
    _check(lib().moe_layer_decode_noalloc(C.byref(as_shape(shape)), C.byref(layer), _dptr(x), _dtype_code(x),
                                          _dptr(logit_offset), _dptr(topk_idx), _dptr(topk_w), _dptr(expert_out),
                                          _dptr(y), _dptr(residual), _stream(stream)), "moe_layer_decode_noalloc")


def moe_stack_decode(shape, layers, x, logit_offsets, topk_idx, topk_w, expert_out, y, x_layers, ws,
                     stream=None) -> None:
    """One bf16 row x through the layers (a sequence of moe_layer), residual in place.
    logit_offsets: None or one device tensor (or None) per layer."""
    n = len(layers)
    arr = (moe_layer * max(n, 1))(*layers)
    offs = None
    if logit_offsets is not None:
        offs = (_P * max(n, 1))(*[_dptr(o) for o in logit_offsets])
    _check(lib().moe_stack_decode(C.byref(as_shape(shape)), arr, n, _dptr(x), offs, _dptr(topk_idx),
                                  _dptr(topk_w), _dptr(expert_out), _dptr(y), _dptr(x_layers), _dptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)), "moe_stack_decode")


def moe_layer_prefill(shape, layer: moe_layer, x, rows: int, logit_offset, topk_idx, topk_w, count, offset, perm,
                      inv_perm, expert_out, y, residual, ws, stream=None) -> None:
    _check(lib().moe_layer_prefill(C.byref(as_shape(shape)), C.byref(layer), _dptr(x), _dtype_code(x), rows,
                                   _dptr(logit_offset), _dptr(topk_idx), _dptr(topk_w), _dptr(count), _dptr(offset),
                                   _dptr(perm), _dptr(inv_perm), _dptr(expert_out), _dptr(y), _dptr(residual),
                                   _dptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "moe_layer_prefill")


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_check_device_error(stream=None) -> int:
    """Synchronises the stream; returns the device error flags (0 if none) and clears them."""
    flags = C.c_uint32(0)
    st = lib().moe_check_device_error(_stream(stream), C.byref(flags))
    if st not in (MOE_OK, MOE_ERR_DEVICE_CHECK):
        raise MoeError(st, "moe_check_device_error")
    return flags.value


# ------------------------------------------------------------------ tiered expert residency

def moe_cache_create(n_layers: int, n_experts: int, slots: int, blob_stride: int = 0, host_pool=None,
                     device_slots=None, slot_tables=None) -> int:
    """Returns the cache handle. host_pool: a pinned host torch uint8 tensor (or None);
    device_slots, slot_tables: GPU tensors, or both None for the policy alone."""
    h = C.c_void_p()
    hp = None if host_pool is None else host_pool.data_ptr()
    _check(lib().moe_cache_create(n_layers, n_experts, slots, blob_stride, hp, _dptr(device_slots),
                                  _dptr(slot_tables), C.byref(h)), "moe_cache_create")
    return h.value


def moe_cache_device_state_bytes(n_layers: int, n_experts: int, slots: int) -> int:
    return int(lib().moe_cache_device_state_bytes(n_layers, n_experts, slots))


def moe_cache_create_device(n_layers: int, n_experts: int, slots: int, blob_stride: int, host_pool, device_slots,
                            slot_tables, device_state, stream=None) -> int:
    """The cache with its policy on the device (see moe.h). host_pool: a pinned host torch
    uint8 tensor; device_slots, slot_tables, device_state: GPU tensors."""
    h = C.c_void_p()
    _check(lib().moe_cache_create_device(n_layers, n_experts, slots, blob_stride, host_pool.data_ptr(),
                                         _dptr(device_slots), _dptr(slot_tables), _dptr(device_state),
                                         device_state.numel() * device_state.element_size(), _stream(stream),
                                         C.byref(h)), "moe_cache_create_device")
    return h.value


def moe_cache_acquire(cache: int, layer: int, idx, slots=None, stream=None) -> int:
    """idx: host int32 numpy array of expert ids; slots: optional int32 numpy array that
    receives their slots. Returns the number of misses."""
    import numpy as np
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    miss = C.c_int32(0)
    _check(lib().moe_cache_acquire(cache, layer, _hptr(idx), idx.size, None if slots is None else _hptr(slots),
                                   C.byref(miss), _stream(stream) if stream is not None or _cuda_ok() else None),
           "moe_cache_acquire")
    return miss.value


def moe_cache_lookup(cache: int, layer: int, idx):
    """The slots of the experts idx (host int32 array) as the cache stands, -1 where not
    resident (nothing is counted or changed)."""
    import numpy as np
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    slots = np.empty(idx.size, dtype=np.int32)
    _check(lib().moe_cache_lookup(cache, layer, _hptr(idx), idx.size, _hptr(slots)), "moe_cache_lookup")
    return slots


def moe_cache_decode(cache: int, layer: int, shape, router_blob, shared_blob, x, logit_offset, topk_idx, topk_w,
                     expert_out, y, residual, pass_tables, ws, stream=None, copy_stream=None) -> None:
    """One decode row of `layer` through the cache (see moe.h); copy_stream: a torch
    stream for the misses' copies (overlapped), or None (serial)."""
    _check(lib().moe_cache_decode(cache, layer, C.byref(as_shape(shape)), _dptr(router_blob), _dptr(shared_blob),
                                  _dptr(x), _dtype_code(x), _dptr(logit_offset), _dptr(topk_idx), _dptr(topk_w),
                                  _dptr(expert_out), _dptr(y), _dptr(residual), _dptr(pass_tables), _dptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream),
                                  None if copy_stream is None else _stream(copy_stream)), "moe_cache_decode")


def moe_cache_stats(cache: int):
    """(hits, misses, bytes copied) since creation."""
    h, m, b = C.c_uint64(0), C.c_uint64(0), C.c_uint64(0)
    _check(lib().moe_cache_stats(cache, C.byref(h), C.byref(m), C.byref(b)), "moe_cache_stats")
    return h.value, m.value, b.value


def moe_cache_destroy(cache: int) -> None:
    _check(lib().moe_cache_destroy(cache), "moe_cache_destroy")


def _cuda_ok() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except ImportError:
        return False
