"""Thin ctypes binding of libclefhead (argument marshalling only).

Every function here has the name of the C entry point it calls and does no
arithmetic of its own; all work of the head runs in the HIP library.  Device
buffers are passed as integer addresses (e.g. ``tensor.data_ptr()``), host
tables as numpy arrays.  Loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libclefhead.so")

CLEF_OK, CLEF_E_ARG, CLEF_E_LENGTH, CLEF_E_SPAN, CLEF_E_ID, CLEF_E_SCHEMA, CLEF_E_NOMEM, CLEF_E_HIP, \
    CLEF_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6, -7, -8
CLEF_BF16, CLEF_F32 = 1, 2
CLEF_PADDED, CLEF_VARLEN = 0, 1
CLEF_HIDDEN_F16 = 0x100
CLEF_PRECISION_BF16, CLEF_PRECISION_F32 = 0, 1
CLEF_NOALLOC_SCRATCH_BYTES = 256 << 20
CLEF_TRACE_POOLED, CLEF_TRACE_LEXICAL, CLEF_TRACE_PRIOR, CLEF_TRACE_MEMORY = 1, 2, 3, 4
CLEF_TRACE_F0, CLEF_TRACE_F, CLEF_TRACE_JCOS, CLEF_TRACE_MLP, CLEF_TRACE_U = 5, 6, 7, 8, 16
CLEF_TRACE_POOL_TABLE, CLEF_TRACE_LEX_TABLE, CLEF_TRACE_IDS = 9, 10, 11
CLEF_DEBUG_ALLOC_LIMIT, CLEF_DEBUG_POISON = 1, 2

EXPORTS = ("clef_head_create", "clef_head_create_sharing", "clef_head_forward", "clef_head_forward_answers",
           "clef_head_forward_noalloc",
           "clef_head_stream_begin", "clef_head_stream_rows", "clef_head_stream_end", "clef_head_stream_cancel",
           "clef_head_destroy", "clef_head_last_error",
           "clef_head_check_batch", "clef_head_span_rows", "clef_head_weight_count", "clef_head_weight_info",
           "clef_head_set_trace", "clef_head_trace", "clef_head_set_profiling", "clef_head_stage_times",
           "clef_head_debug_set")
STAGES = ("rowstats", "pool", "lexical", "memory_gemm", "kv_gemm", "query_proj", "route_dense", "route_attn",
          "field", "score")


class ClefError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libclefhead error {code}: {msg}")
        self.code = code


class clef_head_config(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("width", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("routing_layers", ctypes.c_int32), ("layers", ctypes.c_int32), ("feedforward", ctypes.c_int32),
                ("vocab_size", ctypes.c_int32), ("num_types", ctypes.c_int32), ("ln_eps", ctypes.c_float),
                ("field_cross_attention", ctypes.c_int32), ("precision", ctypes.c_int32)]


class clef_head_weight(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("host_data", ctypes.c_void_p), ("numel", ctypes.c_int64),
                ("dtype", ctypes.c_int32)]


_P = ctypes.c_void_p


class clef_head_batch(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("num_records", ctypes.c_int32), ("max_len", ctypes.c_int32),
                ("hidden", _P), ("key_mask", _P), ("cu_seqlens", _P), ("num_questions", ctypes.c_int32),
                ("num_options", ctypes.c_int32), ("q_offsets", _P), ("q_type", _P), ("q_span", _P),
                ("o_offsets", _P), ("o_span", _P), ("o_ids", _P)]


class clef_head_answers(ctypes.Structure):
    """Device fp32 buffers (addresses, 0 = not written): value, confidence [NQ];
    their 4-decimal copies [NQ]; 4-decimal probabilities [NO]."""
    _fields_ = [("value", _P), ("confidence", _P), ("value_4dp", _P), ("confidence_4dp", _P), ("probs_4dp", _P)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m structured_decision_head_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.clef_head_create.argtypes = [ctypes.POINTER(clef_head_config), ctypes.POINTER(clef_head_weight), ctypes.c_int32,
                                   _P, ctypes.POINTER(_P)]
    L.clef_head_forward.argtypes = [_P, ctypes.POINTER(clef_head_batch), _P, _P, _P, _P]
    L.clef_head_forward_answers.argtypes = [_P, ctypes.POINTER(clef_head_batch), _P, _P, _P,
                                            ctypes.POINTER(clef_head_answers), _P]
    L.clef_head_forward_noalloc.argtypes = [_P, ctypes.POINTER(clef_head_batch), _P, _P, _P, _P]
    L.clef_head_stream_begin.argtypes = [_P, ctypes.POINTER(clef_head_batch), _P]
    L.clef_head_stream_rows.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]
    L.clef_head_stream_end.argtypes = [_P, ctypes.POINTER(clef_head_batch), _P, _P, _P,
                                       ctypes.POINTER(clef_head_answers), _P]
    L.clef_head_stream_cancel.argtypes = [_P]
    L.clef_head_create_sharing.argtypes = [_P, ctypes.POINTER(_P)]
    L.clef_head_destroy.argtypes = [_P]
    L.clef_head_destroy.restype = None
    L.clef_head_last_error.restype = ctypes.c_char_p
    L.clef_head_check_batch.argtypes = [ctypes.POINTER(clef_head_config), ctypes.POINTER(clef_head_batch),
                                        ctypes.POINTER(ctypes.c_int64)]
    L.clef_head_span_rows.argtypes = [ctypes.POINTER(clef_head_config), ctypes.POINTER(clef_head_batch), _P]
    L.clef_head_weight_count.argtypes = [ctypes.POINTER(clef_head_config)]
    L.clef_head_weight_count.restype = ctypes.c_int32
    L.clef_head_weight_info.argtypes = [ctypes.POINTER(clef_head_config), ctypes.c_int32, ctypes.c_char_p,
                                        ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]
    L.clef_head_set_trace.argtypes = [_P, ctypes.c_int32]
    L.clef_head_trace.argtypes = [_P, ctypes.c_int32, _P, ctypes.c_int64]
    L.clef_head_set_profiling.argtypes = [_P, ctypes.c_int32]
    L.clef_head_debug_set.argtypes = [ctypes.c_int32, ctypes.c_int64]
    L.clef_head_stage_times.argtypes = [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    _lib = L
    return L


def _check(rc: int):
    if rc != CLEF_OK:
        raise ClefError(rc, load().clef_head_last_error().decode(errors="replace"))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def make_config(head) -> clef_head_config:
    """From any object with the config attribute names (e.g. synth.HeadConfig)."""
    return clef_head_config(head.hidden_size, head.width, head.heads, head.routing_layers, head.layers,
                            head.feedforward, head.vocab_size, head.num_types, head.ln_eps,
                            int(getattr(head, "field_cross_attention", 0)), int(getattr(head, "precision", 0)))


class BatchArgs:
    """clef_head_batch plus the host arrays it points into (kept alive)."""

    def __init__(self, batch, hidden_ptr: int, layout: int = CLEF_PADDED):
        self._keep = []

        def arr(x, dt):
            a = np.ascontiguousarray(x, dtype=dt)
            self._keep.append(a)
            return a

        s = clef_head_batch()
        # the element type of the hidden rows travels as a flag in the layout
        s.layout = layout | (CLEF_HIDDEN_F16 if getattr(batch, "hidden_dtype", "bf16") == "f16" else 0)
        s.num_records = batch.B
        s.max_len = batch.L if layout == CLEF_PADDED else 0
        s.hidden = hidden_ptr
        s.key_mask = _ptr(arr(batch.key_mask(), np.uint8)) if layout == CLEF_PADDED else None
        s.cu_seqlens = _ptr(arr(batch.cu_seqlens(), np.int32)) if layout == CLEF_VARLEN else None
        s.num_questions = batch.NQ
        s.num_options = batch.NO
        s.q_offsets = _ptr(arr(batch.q_offsets, np.int32))
        s.q_type = _ptr(arr(batch.q_type, np.int32))
        s.q_span = _ptr(arr(batch.q_span, np.int32))
        s.o_offsets = _ptr(arr(batch.o_offsets, np.int32))
        s.o_span = _ptr(arr(batch.o_span, np.int32))
        s.o_ids = _ptr(arr(batch.o_ids, np.int32))
        self.struct = s


def clef_head_weight_count(head) -> int:
    cfg = make_config(head)
    n = load().clef_head_weight_count(ctypes.byref(cfg))
    if n < 0:
        _check(CLEF_E_ARG)
    return n


def clef_head_weight_info(head, i: int):
    cfg = make_config(head)
    name = ctypes.create_string_buffer(256)
    numel, dtype = ctypes.c_int64(), ctypes.c_int32()
    _check(load().clef_head_weight_info(ctypes.byref(cfg), i, name, 256, ctypes.byref(numel), ctypes.byref(dtype)))
    return name.value.decode(), numel.value, dtype.value


def clef_head_check_batch(head, batch_args: BatchArgs) -> int:
    cfg = make_config(head)
    n = ctypes.c_int64()
    _check(load().clef_head_check_batch(ctypes.byref(cfg), ctypes.byref(batch_args.struct), ctypes.byref(n)))
    return n.value


def clef_head_span_rows(head, batch_args: BatchArgs, total: int) -> np.ndarray:
    cfg = make_config(head)
    out = np.zeros((total, 2), np.int32)
    _check(load().clef_head_span_rows(ctypes.byref(cfg), ctypes.byref(batch_args.struct), out.ctypes.data))
    return out


def clef_head_create(head, weights: Dict[str, np.ndarray], table_ptr: int) -> int:
    """Returns the handle as an integer address."""
    cfg = make_config(head)
    items = list(weights.items())
    keep = [np.ascontiguousarray(v) for _, v in items]
    arr = (clef_head_weight * len(items))()
    names = [k.encode() for k, _ in items]
    for i, ((k, _), v) in enumerate(zip(items, keep)):
        arr[i].name = names[i]
        arr[i].host_data = v.ctypes.data
        arr[i].numel = v.size
        arr[i].dtype = CLEF_BF16 if v.dtype == np.uint16 else CLEF_F32 if v.dtype == np.float32 else 0
    h = _P()
    _check(load().clef_head_create(ctypes.byref(cfg), arr, len(items), table_ptr, ctypes.byref(h)))
    return h.value


def clef_head_create_sharing(src: int) -> int:
    """A second handle over src's device weights (own workspace and streams)."""
    h = _P()
    _check(load().clef_head_create_sharing(src, ctypes.byref(h)))
    return h.value


def clef_head_forward(handle: int, batch_args: BatchArgs, logits_ptr: int, probs_ptr: int, argmax_ptr: int,
                      stream_ptr: int = 0):
    _check(load().clef_head_forward(handle, ctypes.byref(batch_args.struct), logits_ptr, probs_ptr, argmax_ptr,
                                    stream_ptr or None))


def clef_head_forward_answers(handle: int, batch_args: BatchArgs, logits_ptr: int, probs_ptr: int, argmax_ptr: int,
                              value_ptr: int = 0, confidence_ptr: int = 0, value_4dp_ptr: int = 0,
                              confidence_4dp_ptr: int = 0, probs_4dp_ptr: int = 0, stream_ptr: int = 0):
    ans = clef_head_answers(value_ptr or None, confidence_ptr or None, value_4dp_ptr or None,
                            confidence_4dp_ptr or None, probs_4dp_ptr or None)
    _check(load().clef_head_forward_answers(handle, ctypes.byref(batch_args.struct), logits_ptr, probs_ptr,
                                            argmax_ptr, ctypes.byref(ans), stream_ptr or None))


def clef_head_forward_noalloc(handle: int, batch_args: BatchArgs, logits_ptr: int, probs_ptr: int, argmax_ptr: int,
                              stream_ptr: int = 0):
    _check(load().clef_head_forward_noalloc(handle, ctypes.byref(batch_args.struct), logits_ptr, probs_ptr,
                                            argmax_ptr, stream_ptr or None))


def clef_head_stream_begin(handle: int, batch_args: BatchArgs, stream_ptr: int = 0):
    _check(load().clef_head_stream_begin(handle, ctypes.byref(batch_args.struct), stream_ptr or None))


def clef_head_stream_rows(handle: int, record: int, row0: int, nrows: int, rows_ptr: int, stream_ptr: int = 0):
    _check(load().clef_head_stream_rows(handle, record, row0, nrows, rows_ptr, stream_ptr or None))


def clef_head_stream_end(handle: int, batch_args: BatchArgs, logits_ptr: int, probs_ptr: int, argmax_ptr: int,
                         stream_ptr: int = 0, answer_ptrs=None):
    """answer_ptrs: optional (value, confidence, value_4dp, confidence_4dp, probs_4dp) device addresses."""
    ans = None
    if answer_ptrs is not None:
        ans = ctypes.byref(clef_head_answers(*[a or None for a in answer_ptrs]))
    _check(load().clef_head_stream_end(handle, ctypes.byref(batch_args.struct), logits_ptr, probs_ptr, argmax_ptr,
                                       ans, stream_ptr or None))


def clef_head_stream_cancel(handle: int):
    _check(load().clef_head_stream_cancel(handle))


def clef_head_destroy(handle: int):
    load().clef_head_destroy(handle)


def clef_head_last_error() -> str:
    return load().clef_head_last_error().decode(errors="replace")


def clef_head_set_trace(handle: int, enable: bool):
    _check(load().clef_head_set_trace(handle, 1 if enable else 0))


def clef_head_trace(handle: int, which: int, out: np.ndarray) -> np.ndarray:
    _check(load().clef_head_trace(handle, which, out.ctypes.data, out.nbytes))
    return out


def clef_head_debug_set(what: int, value: int):
    _check(load().clef_head_debug_set(what, value))


def clef_head_set_profiling(handle: int, enable: bool):
    _check(load().clef_head_set_profiling(handle, 1 if enable else 0))


def clef_head_stage_times(handle: int):
    """(dict stage -> summed ms, number of forwards)."""
    ms = (ctypes.c_double * len(STAGES))()
    n = ctypes.c_int64()
    _check(load().clef_head_stage_times(handle, ms, ctypes.byref(n)))
    return {k: ms[i] for i, k in enumerate(STAGES)}, n.value
