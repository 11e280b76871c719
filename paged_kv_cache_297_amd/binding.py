"""Thin Python binding of libpagedattn (ctypes).

Argument marshalling only: shapes are read off the torch tensors, checked,
and passed with ``data_ptr()`` and the current HIP stream to the C ABI in
``include/pagedattn.h``; every step of the computation runs in the library's
HIP kernels.  The argument order follows the paged-attention op of the page
"BI-V100 PagedAttention V2 implementation" (out, exp_sums, max_logits,
tmp_out, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
seq_lens, block_size, max_seq_len, alibi_slopes, kv_cache_dtype, k_scale,
v_scale).  There is no fallback: without the built library every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

#: The in-tree build; PA_LIB_PATH selects another build of the same library.
LIB_PATH = os.environ.get("PA_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_OK = 0
STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_NULL_POINTER", 2: "PA_ERR_BAD_SHAPE",
                3: "PA_ERR_MISALIGNED", 4: "PA_ERR_UNSUPPORTED", 5: "PA_ERR_HIP",
                6: "PA_ERR_BAD_ARGUMENT"}
DTYPE_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
KV_CODE = {"auto": 0, "fp8": 1, "fp8_e4m3": 1}
MODE_CODE = {"v1": 0, "v2": 1, "auto": 2}
#: pa_kv_layout: "decode" (K [NB, Hkv, D/x, bs, x], V [NB, Hkv, D, bs]) or
#: "block_rows" (K and V [NB, Hkv, bs, D]).
LAYOUT_CODE = {"decode": 0, "block_rows": 1}
#: pa_partial_dtype: tmp_out in float32 (the default) or in the query dtype.
PARTIAL_F32, PARTIAL_OUT = 0, 1

#: Every symbol include/pagedattn.h declares.
EXPORTED_SYMBOLS = (
    "paged_attention_v1", "paged_attention_v2", "paged_attention_auto",
    "paged_attention_partition", "paged_attention_reduce",
    "paged_attention_v1_ex", "paged_attention_v2_ex", "paged_attention_auto_ex",
    "paged_attention_partition_ex", "paged_attention_reduce_ex", "paged_attention_split",
    "pa_split_counters_size", "paged_attention_split_static", "paged_attention_worklist", "paged_attention_auto_ws", "paged_prefill", "pa_partition_size",
    "pa_num_partitions", "pa_should_use_v2", "pa_auto_uses_slots", "pa_device_cu_count",
    "pa_set_timing_events",
    "pa_status_string", "pa_version", "pa_stream_read",
)


class PrefillOptions(ctypes.Structure):
    """pa_prefill_options: causal flag, left / right window (-1: none), soft cap (0: none)."""
    _fields_ = [("causal", ctypes.c_int), ("window_left", ctypes.c_int),
                ("window_right", ctypes.c_int), ("logits_soft_cap", ctypes.c_float)]


class DecodeOptions(ctypes.Structure):
    """pa_decode_options: sliding window (-1: none), logit soft cap (0: none),
    the cache layout (LAYOUT_CODE) and the partial dtype of tmp_out
    (PARTIAL_F32 / PARTIAL_OUT)."""
    _fields_ = [("window_left", ctypes.c_int), ("logits_soft_cap", ctypes.c_float),
                ("kv_layout", ctypes.c_int), ("partial_dtype", ctypes.c_int)]


class PagedAttentionError(RuntimeError):
    """A libpagedattn call returned a status other than PA_OK."""

    def __init__(self, status: int, func: str, message: str):
        super().__init__(f"{func}: {STATUS_NAMES.get(status, status)} ({message})")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_PARTITION_ARGS = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _I, _P, _I, _I, _I, _I,
                   _P, _I, _I, _F, _F, _P]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpagedattn and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libpagedattn is not built ({path} missing); run "
            "`python -m paged_kv_cache_297_amd._build` or __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.paged_attention_v1.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _I, _P, _I, _I, _I,
                                       _P, _I, _I, _F, _F, _P]
    lib.paged_attention_v1.restype = _I
    for name in ("paged_attention_v2", "paged_attention_auto"):
        fn = getattr(lib, name)
        fn.argtypes = _PARTITION_ARGS[:]
        fn.restype = _I
    lib.paged_attention_partition.argtypes = [_I] + _PARTITION_ARGS
    lib.paged_attention_partition.restype = _I
    lib.paged_attention_reduce.argtypes = [_I, _P, _P, _P, _P, _I, _I, _I, _I, _P, _I, _I, _I, _P]
    lib.paged_attention_reduce.restype = _I
    # The *_ex forms: the same arguments with a pa_decode_options pointer
    # before the stream.
    for name in ("paged_attention_v1", "paged_attention_v2", "paged_attention_auto",
                 "paged_attention_partition", "paged_attention_reduce"):
        plain = getattr(lib, name).argtypes
        ex = getattr(lib, name + "_ex")
        ex.argtypes = plain[:-1] + [_P, _P]
        ex.restype = _I
    lib.paged_attention_split.argtypes = _PARTITION_ARGS[:4] + [_P] + _PARTITION_ARGS[4:-1] + [_P, _P]
    lib.paged_attention_split.restype = _I
    lib.paged_attention_worklist.argtypes = lib.paged_attention_split.argtypes[:]
    lib.paged_attention_worklist.restype = _I
    lib.paged_attention_auto_ws.argtypes = lib.paged_attention_split.argtypes[:]
    lib.paged_attention_auto_ws.restype = _I
    lib.paged_attention_split_static.argtypes = lib.paged_attention_v1.argtypes[:-1] + [_P, _P]
    lib.paged_attention_split_static.restype = _I
    lib.paged_prefill.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _I, _P, _P, _I, _I,
                                  _I, _I, _I, _P, _P]
    lib.paged_prefill.restype = _I
    lib.pa_split_counters_size.argtypes = [_I, _I]
    lib.pa_split_counters_size.restype = ctypes.c_size_t
    lib.pa_partition_size.argtypes = []
    lib.pa_partition_size.restype = _I
    lib.pa_num_partitions.argtypes = [_I]
    lib.pa_num_partitions.restype = _I
    lib.pa_should_use_v2.argtypes = [_I, _I, _I, _I]
    lib.pa_should_use_v2.restype = _I
    lib.pa_auto_uses_slots.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _P,
                                       ctypes.POINTER(ctypes.c_int)]
    lib.pa_auto_uses_slots.restype = _I
    lib.pa_device_cu_count.argtypes = [ctypes.POINTER(ctypes.c_int)]
    lib.pa_device_cu_count.restype = _I
    lib.pa_set_timing_events.argtypes = [_P, _P, _P, _P]
    lib.pa_set_timing_events.restype = _I
    lib.pa_stream_read.argtypes = [_P, ctypes.c_size_t, _P, _I, _P]
    lib.pa_stream_read.restype = _I
    lib.pa_status_string.argtypes = [_I]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_version.argtypes = []
    lib.pa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, func: str) -> None:
    if status != PA_OK:
        msg = load_library().pa_status_string(status).decode()
        raise PagedAttentionError(status, func, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _kv_code(kv_cache_dtype: str) -> int:
    if kv_cache_dtype not in KV_CODE:
        raise ValueError(f"kv_cache_dtype must be one of {sorted(KV_CODE)}")
    return KV_CODE[kv_cache_dtype]


def _layout_code(kv_layout: str) -> int:
    if kv_layout not in LAYOUT_CODE:
        raise ValueError(f"kv_layout must be one of {sorted(LAYOUT_CODE)}")
    return LAYOUT_CODE[kv_layout]


def _options(window_left: int, logits_soft_cap: float, kv_layout: str = "decode",
             partial: int = PARTIAL_F32) -> Optional[DecodeOptions]:
    """None when every option is off (the plain entry point is called)."""
    code = _layout_code(kv_layout)
    if int(window_left) == -1 and float(logits_soft_cap) == 0.0 and code == 0 and partial == 0:
        return None
    return DecodeOptions(int(window_left), float(logits_soft_cap), code, int(partial))


def _partial_code(tmp_out: torch.Tensor, query: torch.Tensor) -> int:
    """pa_partial_dtype from the dtype of the caller's tmp_out: float32, or the
    query dtype (the V2 page casts each partial to the tmp_output dtype)."""
    if tmp_out.dtype == torch.float32:
        return PARTIAL_F32
    if tmp_out.dtype == query.dtype:
        return PARTIAL_OUT
    raise TypeError("tmp_out must be float32 or have the query's dtype")


def _call(lib, name: str, args, opts: Optional[DecodeOptions]) -> None:
    """Calls ``name`` (opts None) or ``name``_ex with a pointer to opts."""
    if opts is None:
        _check(getattr(lib, name)(*args), name)
    else:
        _check(getattr(lib, name + "_ex")(*args[:-1], ctypes.addressof(opts), args[-1]),
               name + "_ex")


def _geometry(query, key_cache, value_cache, block_tables, seq_lens, kv_cache_dtype,
              kv_layout="decode"):
    """Checks layouts and returns (num_seqs, num_heads, head_size, num_blocks, Hkv,
    block_size, max_blocks)."""
    for name, t in (("query", query), ("key_cache", key_cache), ("value_cache", value_cache),
                    ("block_tables", block_tables), ("seq_lens", seq_lens)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if query.dtype not in DTYPE_CODE:
        raise TypeError("query must be float32, float16 or bfloat16")
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    num_seqs, num_heads, head_size = query.shape
    if _kv_code(kv_cache_dtype) == 1:
        if key_cache.element_size() != 1 or value_cache.element_size() != 1:
            raise TypeError("an fp8 cache must be a 1-byte tensor (uint8 or float8_e4m3fn)")
        elem = 1
    else:
        if key_cache.dtype != query.dtype or value_cache.dtype != query.dtype:
            raise TypeError("with kv_cache_dtype='auto' the caches must have the query dtype")
        elem = query.element_size()
    x = 16 // elem
    if _layout_code(kv_layout) == 1:
        if key_cache.dim() != 4 or key_cache.shape[3] != head_size:
            raise ValueError("key_cache must be [num_blocks, Hkv, block_size, head_size]")
        nb, hkv, bs, _ = key_cache.shape
        if tuple(value_cache.shape) != tuple(key_cache.shape):
            raise ValueError("value_cache must be [num_blocks, Hkv, block_size, head_size]")
    else:
        nb, hkv, dx, bs, xx = key_cache.shape
        if xx != x or dx * x != head_size:
            raise ValueError(
                f"key_cache must be [num_blocks, Hkv, {head_size}/{x}, block_size, {x}]")
        if tuple(value_cache.shape) != (nb, hkv, head_size, bs):
            raise ValueError("value_cache must be [num_blocks, Hkv, head_size, block_size]")
    if block_tables.dim() != 2 or block_tables.shape[0] != num_seqs or seq_lens.shape != (num_seqs,):
        raise ValueError("block_tables must be [num_seqs, max_blocks] and seq_lens [num_seqs]")
    return num_seqs, num_heads, head_size, nb, hkv, bs, block_tables.shape[1]


def paged_attention_v1(out: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                       value_cache: torch.Tensor, num_kv_heads: int, scale: float,
                       block_tables: torch.Tensor, seq_lens: torch.Tensor, block_size: int,
                       max_seq_len: int, alibi_slopes: Optional[torch.Tensor] = None,
                       kv_cache_dtype: str = "auto", k_scale: float = 1.0, v_scale: float = 1.0,
                       stream=None, window_left: int = -1, logits_soft_cap: float = 0.0,
                       kv_layout: str = "decode") -> None:
    """Whole-sequence paged attention; writes ``out`` in place.  ``window_left`` /
    ``logits_soft_cap`` / ``kv_layout`` are the decode options (-1 / 0 / "decode":
    off)."""
    lib = load_library()
    b, h, d, nb, hkv, bs, mbps = _geometry(query, key_cache, value_cache, block_tables, seq_lens,
                                           kv_cache_dtype, kv_layout)
    if hkv != num_kv_heads or bs != block_size:
        raise ValueError("num_kv_heads / block_size disagree with the cache shape")
    if out.shape != query.shape or out.dtype != query.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like query")
    args = [out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), b, h,
            num_kv_heads, d, float(scale), block_tables.data_ptr(), mbps, seq_lens.data_ptr(), nb,
            block_size, int(max_seq_len), _ptr(alibi_slopes), DTYPE_CODE[query.dtype],
            _kv_code(kv_cache_dtype), float(k_scale), float(v_scale), _stream(stream)]
    _call(lib, "paged_attention_v1", args, _options(window_left, logits_soft_cap, kv_layout))


def _v2_args(out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache, num_kv_heads,
             scale, block_tables, seq_lens, block_size, max_seq_len, alibi_slopes,
             kv_cache_dtype, k_scale, v_scale, stream, kv_layout="decode"):
    b, h, d, nb, hkv, bs, mbps = _geometry(query, key_cache, value_cache, block_tables, seq_lens,
                                           kv_cache_dtype, kv_layout)
    if hkv != num_kv_heads or bs != block_size:
        raise ValueError("num_kv_heads / block_size disagree with the cache shape")
    if out.shape != query.shape or out.dtype != query.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like query")
    for name, t in (("exp_sums", exp_sums), ("max_logits", max_logits)):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous float32 tensor")
    _partial_code(tmp_out, query)
    if not tmp_out.is_contiguous():
        raise TypeError("tmp_out must be contiguous")
    p = exp_sums.shape[2]
    if exp_sums.shape != (b, h, p) or max_logits.shape != (b, h, p) or tmp_out.shape != (b, h, p, d):
        raise ValueError("exp_sums/max_logits must be [B, H, P] and tmp_out [B, H, P, D]")
    if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != h):
        raise ValueError("alibi_slopes must be float32 [num_heads]")
    return [out.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(), tmp_out.data_ptr(),
            query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), b, h, num_kv_heads, d,
            float(scale), block_tables.data_ptr(), mbps, seq_lens.data_ptr(), nb, block_size,
            int(max_seq_len), p, _ptr(alibi_slopes), DTYPE_CODE[query.dtype],
            _kv_code(kv_cache_dtype), float(k_scale), float(v_scale), _stream(stream)]


def paged_attention_v2(out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                       num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
                       alibi_slopes=None, kv_cache_dtype="auto", k_scale=1.0, v_scale=1.0,
                       stream=None, window_left=-1, logits_soft_cap=0.0,
                       kv_layout="decode") -> None:
    """Partitioned paged attention (Phase 1 + Phase 2); writes all four outputs in place."""
    lib = load_library()
    args = _v2_args(out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                    num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
                    alibi_slopes, kv_cache_dtype, k_scale, v_scale, stream, kv_layout)
    _call(lib, "paged_attention_v2", args, _options(window_left, logits_soft_cap, kv_layout,
                                                    _partial_code(tmp_out, query)))


def paged_attention_auto(out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                         num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
                         alibi_slopes=None, kv_cache_dtype="auto", k_scale=1.0, v_scale=1.0,
                         stream=None, window_left=-1, logits_soft_cap=0.0,
                         kv_layout="decode") -> None:
    """Per-sequence v1/v2 choice on the device (pa_should_use_v2 rule)."""
    lib = load_library()
    args = _v2_args(out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                    num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
                    alibi_slopes, kv_cache_dtype, k_scale, v_scale, stream, kv_layout)
    _call(lib, "paged_attention_auto", args, _options(window_left, logits_soft_cap, kv_layout,
                                                      _partial_code(tmp_out, query)))


def split_counters(num_seqs: int, num_heads: int, device="cuda") -> torch.Tensor:
    """A zeroed counters buffer for paged_attention_split (int32 [B, H])."""
    return torch.zeros((num_seqs, num_heads), dtype=torch.int32, device=device)


def _split_args(out, exp_sums, max_logits, tmp_out, counters, query, *rest, opts):
    layout = "block_rows" if opts is not None and opts.kv_layout == 1 else "decode"
    args = _v2_args(out, exp_sums, max_logits, tmp_out, query, *rest, kv_layout=layout)
    b, h = query.shape[0], query.shape[1]
    if counters is not None and (counters.dtype != torch.int32 or not counters.is_contiguous()
                                 or counters.numel() < b * h):
        raise TypeError("counters must be a contiguous int32 tensor of num_seqs * num_heads")
    ptr = None if opts is None else ctypes.addressof(opts)
    cptr = None if counters is None else counters.data_ptr()
    return args[:4] + [cptr] + args[4:-1] + [ptr, args[-1]]


def paged_attention_worklist(out, exp_sums, max_logits, tmp_out, counters, query, key_cache,
                             value_cache, num_kv_heads, scale, block_tables, seq_lens, block_size,
                             max_seq_len, alibi_slopes=None, kv_cache_dtype="auto", k_scale=1.0,
                             v_scale=1.0, stream=None, window_left=-1, logits_soft_cap=0.0,
                             kv_layout="decode") -> None:
    """Work-list decode (one persistent launch, items balanced by memory-load
    cost): writes ``out``; the partial buffers are scratch and ``counters``
    (split_counters) must be zero on entry (it is left zero)."""
    lib = load_library()
    opts = _options(window_left, logits_soft_cap, kv_layout, _partial_code(tmp_out, query))
    args = _split_args(out, exp_sums, max_logits, tmp_out, counters, query, key_cache,
                       value_cache, num_kv_heads, scale, block_tables, seq_lens, block_size,
                       max_seq_len, alibi_slopes, kv_cache_dtype, k_scale, v_scale, stream,
                       opts=opts)
    _check(lib.paged_attention_worklist(*args), "paged_attention_worklist")


def paged_attention_auto_ws(out, exp_sums, max_logits, tmp_out, counters, query, key_cache,
                            value_cache, num_kv_heads, scale, block_tables, seq_lens, block_size,
                            max_seq_len, alibi_slopes=None, kv_cache_dtype="auto", k_scale=1.0,
                            v_scale=1.0, stream=None, window_left=-1, logits_soft_cap=0.0,
                            kv_layout="decode") -> None:
    """Auto decode scheduled for balance when ``counters`` (split_counters) is
    given: the work list or the balanced split by batch shape, the partial
    buffers then being scratch; ``counters=None`` is paged_attention_auto."""
    lib = load_library()
    opts = _options(window_left, logits_soft_cap, kv_layout, _partial_code(tmp_out, query))
    args = _split_args(out, exp_sums, max_logits, tmp_out, counters, query, key_cache,
                       value_cache, num_kv_heads, scale, block_tables, seq_lens, block_size,
                       max_seq_len, alibi_slopes, kv_cache_dtype, k_scale, v_scale, stream,
                       opts=opts)
    _check(lib.paged_attention_auto_ws(*args), "paged_attention_auto_ws")


def paged_attention_split(out, exp_sums, max_logits, tmp_out, counters, query, key_cache,
                          value_cache, num_kv_heads, scale, block_tables, seq_lens, block_size,
                          max_seq_len, alibi_slopes=None, kv_cache_dtype="auto", k_scale=1.0,
                          v_scale=1.0, stream=None, window_left=-1, logits_soft_cap=0.0,
                          kv_layout="decode") -> None:
    """Balanced split decode: writes ``out``; the partial buffers are scratch and
    ``counters`` (split_counters) must be zero on entry (it is left zero)."""
    lib = load_library()
    opts = _options(window_left, logits_soft_cap, kv_layout, _partial_code(tmp_out, query))
    args = _split_args(out, exp_sums, max_logits, tmp_out, counters, query, key_cache,
                       value_cache, num_kv_heads, scale, block_tables, seq_lens, block_size,
                       max_seq_len, alibi_slopes, kv_cache_dtype, k_scale, v_scale, stream,
                       opts=opts)
    _check(lib.paged_attention_split(*args), "paged_attention_split")


#: Bytes of the library's own scratch array (paged_attention_split_static).
SPLIT_STATIC_SCRATCH_BYTES = 64 << 20


def paged_attention_split_static(out, query, key_cache, value_cache, num_kv_heads, scale,
                                 block_tables, seq_lens, block_size, max_seq_len,
                                 alibi_slopes=None, kv_cache_dtype="auto", k_scale=1.0,
                                 v_scale=1.0, stream=None, window_left=-1, logits_soft_cap=0.0,
                                 kv_layout="decode", partials="f32") -> None:
    """Balanced split decode with no scratch arguments: the counters and the
    pieces' partials live in the library's own device array (for callers
    that cannot allocate).  Writes ``out``; ``partials`` ('f32' or 'out')
    picks the partial dtype.  Calls that overlap on one GPU race."""
    lib = load_library()
    b, h, d, nb, hkv, bs, mbps = _geometry(query, key_cache, value_cache, block_tables, seq_lens,
                                           kv_cache_dtype, kv_layout)
    if hkv != num_kv_heads or bs != block_size:
        raise ValueError("num_kv_heads / block_size disagree with the cache shape")
    if out.shape != query.shape or out.dtype != query.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like query")
    if partials not in ("f32", "out"):
        raise ValueError("partials must be 'f32' or 'out'")
    opts = _options(window_left, logits_soft_cap, kv_layout,
                    PARTIAL_F32 if partials == "f32" else PARTIAL_OUT)
    args = [out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(), b, h,
            num_kv_heads, d, float(scale), block_tables.data_ptr(), mbps, seq_lens.data_ptr(), nb,
            block_size, int(max_seq_len), _ptr(alibi_slopes), DTYPE_CODE[query.dtype],
            _kv_code(kv_cache_dtype), float(k_scale), float(v_scale),
            None if opts is None else ctypes.addressof(opts), _stream(stream)]
    _check(lib.paged_attention_split_static(*args), "paged_attention_split_static")


class PreparedCall:
    """A v2 / auto call whose arguments were checked and marshalled once.

    ``__call__`` issues only the C call (on the stream fixed at preparation):
    for tight loops where per-call Python argument handling would dominate,
    e.g. timing.  The tensors must stay alive and unchanged in shape."""

    def __init__(self, mode, out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                 num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
                 alibi_slopes=None, kv_cache_dtype="auto", k_scale=1.0, v_scale=1.0,
                 stream=None, window_left=-1, logits_soft_cap=0.0, counters=None,
                 kv_layout="decode"):
        self.lib = load_library()
        self.name = f"paged_attention_{mode}"
        if mode not in ("v2", "auto", "split", "worklist", "auto_ws"):
            raise ValueError("mode must be 'v2', 'auto', 'split', 'worklist' or 'auto_ws'")
        self.opts = _options(window_left, logits_soft_cap, kv_layout,
                             _partial_code(tmp_out, query))
        self.counters = counters
        if mode in ("split", "worklist", "auto_ws"):
            if counters is None and mode != "auto_ws":
                raise ValueError(f"the {mode} mode needs a counters buffer (split_counters)")
            self.args = _split_args(out, exp_sums, max_logits, tmp_out, counters, query,
                                    key_cache, value_cache, num_kv_heads, scale, block_tables,
                                    seq_lens, block_size, max_seq_len, alibi_slopes,
                                    kv_cache_dtype, k_scale, v_scale, stream, opts=self.opts)
            self.fn = getattr(self.lib, self.name)
            self._keep = (out, exp_sums, max_logits, tmp_out, counters, query, key_cache,
                          value_cache, block_tables, seq_lens, alibi_slopes)
            return
        self.args = _v2_args(out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                             num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
                             alibi_slopes, kv_cache_dtype, k_scale, v_scale, stream, kv_layout)
        if self.opts is None:
            self.fn = getattr(self.lib, self.name)
        else:
            self.name += "_ex"
            self.fn = getattr(self.lib, self.name)
            self.args = self.args[:-1] + [ctypes.addressof(self.opts), self.args[-1]]
        self._keep = (out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                      block_tables, seq_lens, alibi_slopes)

    def __call__(self) -> None:
        st = self.fn(*self.args)
        if st != PA_OK:
            _check(st, self.name)


def paged_attention_partition(mode, out, exp_sums, max_logits, tmp_out, query, key_cache,
                              value_cache, num_kv_heads, scale, block_tables, seq_lens,
                              block_size, max_seq_len, alibi_slopes=None, kv_cache_dtype="auto",
                              k_scale=1.0, v_scale=1.0, stream=None, window_left=-1,
                              logits_soft_cap=0.0, kv_layout="decode") -> None:
    """Phase 1 only (mode 'v1', 'v2' or 'auto')."""
    lib = load_library()
    args = _v2_args(out, exp_sums, max_logits, tmp_out, query, key_cache, value_cache,
                    num_kv_heads, scale, block_tables, seq_lens, block_size, max_seq_len,
                    alibi_slopes, kv_cache_dtype, k_scale, v_scale, stream, kv_layout)
    _call(lib, "paged_attention_partition", [MODE_CODE[mode]] + args,
          _options(window_left, logits_soft_cap, kv_layout, _partial_code(tmp_out, query)))


def paged_attention_reduce(mode, out, exp_sums, max_logits, tmp_out, seq_lens, num_kv_heads,
                           max_seq_len, stream=None, window_left=-1) -> None:
    """Phase 2 only (mode 'v2' or 'auto'; 'v1' does nothing).  ``window_left``
    must be the one the partition phase was given."""
    lib = load_library()
    b, h, d = out.shape
    p = exp_sums.shape[2]
    args = [MODE_CODE[mode], out.data_ptr(), exp_sums.data_ptr(), max_logits.data_ptr(),
            tmp_out.data_ptr(), b, h, num_kv_heads, d, seq_lens.data_ptr(), int(max_seq_len), p,
            DTYPE_CODE[out.dtype], _stream(stream)]
    _call(lib, "paged_attention_reduce", args,
          _options(window_left, 0.0, partial=_partial_code(tmp_out, out)))


def _prefill_args(out, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
                  cu_seq_q, cu_seq_k, max_seq_q, max_seq_k, stream, opts):
    for name, t in (("out", out), ("query", query), ("key_cache", key_cache),
                    ("value_cache", value_cache), ("block_tables", block_tables),
                    ("cu_seq_q", cu_seq_q), ("cu_seq_k", cu_seq_k)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if query.dtype not in DTYPE_CODE:
        raise TypeError("query must be float16 or bfloat16")
    if key_cache.dtype != query.dtype or value_cache.dtype != query.dtype or out.dtype != query.dtype:
        raise TypeError("out and the caches must have the query dtype")
    for name, t in (("block_tables", block_tables), ("cu_seq_q", cu_seq_q), ("cu_seq_k", cu_seq_k)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32")
    total_q, h, d = query.shape
    nb, hkv, bs, dk = key_cache.shape
    if hkv != num_kv_heads or dk != d or tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("caches must be [num_blocks, num_kv_heads, block_size, head_size]")
    if out.shape != query.shape:
        raise ValueError("out must be shaped like query")
    b = block_tables.shape[0]
    if cu_seq_q.shape != (b + 1,) or cu_seq_k.shape != (b + 1,):
        raise ValueError("cu_seq_q / cu_seq_k must be [num_seqs + 1]")
    ptr = None if opts is None else ctypes.addressof(opts)
    return [out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
            total_q, b, h, num_kv_heads, d, float(scale), block_tables.data_ptr(),
            block_tables.shape[1], cu_seq_q.data_ptr(), cu_seq_k.data_ptr(), int(max_seq_q),
            int(max_seq_k), nb, bs, DTYPE_CODE[query.dtype], ptr, _stream(stream)]


def paged_prefill(out, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
                  cu_seq_q, cu_seq_k, max_seq_q, max_seq_k, causal=True, window_left=-1,
                  window_right=-1, logits_soft_cap=0.0, stream=None) -> None:
    """Paged prefill attention (pa_prefill_options from the keyword arguments);
    writes ``out`` in place."""
    lib = load_library()
    opts = PrefillOptions(1 if causal else 0, int(window_left), int(window_right),
                          float(logits_soft_cap))
    args = _prefill_args(out, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
                         cu_seq_q, cu_seq_k, max_seq_q, max_seq_k, stream, opts)
    _check(lib.paged_prefill(*args), "paged_prefill")


class PreparedPrefill:
    """A paged_prefill call marshalled once (see PreparedCall)."""

    def __init__(self, out, query, key_cache, value_cache, num_kv_heads, scale, block_tables,
                 cu_seq_q, cu_seq_k, max_seq_q, max_seq_k, causal=True, window_left=-1,
                 window_right=-1, logits_soft_cap=0.0, stream=None):
        self.lib = load_library()
        self.opts = PrefillOptions(1 if causal else 0, int(window_left), int(window_right),
                                   float(logits_soft_cap))
        self.args = _prefill_args(out, query, key_cache, value_cache, num_kv_heads, scale,
                                  block_tables, cu_seq_q, cu_seq_k, max_seq_q, max_seq_k, stream,
                                  self.opts)
        self._keep = (out, query, key_cache, value_cache, block_tables, cu_seq_q, cu_seq_k)

    def __call__(self) -> None:
        st = self.lib.paged_prefill(*self.args)
        if st != PA_OK:
            _check(st, "paged_prefill")


def partition_size() -> int:
    return load_library().pa_partition_size()


def num_partitions(max_seq_len: int) -> int:
    return load_library().pa_num_partitions(int(max_seq_len))


def should_use_v2(num_seqs: int, num_kv_heads: int, seq_len: int, cu_count: int) -> bool:
    return bool(load_library().pa_should_use_v2(num_seqs, num_kv_heads, seq_len, cu_count))


def auto_uses_slots(num_seqs: int, num_heads: int, num_kv_heads: int, head_size: int,
                    block_size: int, max_seq_len: int, dtype: torch.dtype,
                    kv_cache_dtype: str = "auto", window_left: int = -1,
                    logits_soft_cap: float = 0.0, kv_layout: str = "decode") -> bool:
    """pa_auto_uses_slots: whether the auto call runs this batch shape as the
    persistent slot form (its partial buffers are then scratch)."""
    opts = _options(window_left, logits_soft_cap, kv_layout)
    n = ctypes.c_int(0)
    _check(load_library().pa_auto_uses_slots(
        num_seqs, num_heads, num_kv_heads, head_size, block_size, int(max_seq_len),
        DTYPE_CODE[dtype], _kv_code(kv_cache_dtype),
        ctypes.addressof(opts) if opts is not None else None, ctypes.byref(n)),
        "pa_auto_uses_slots")
    return bool(n.value)


def device_cu_count() -> int:
    n = ctypes.c_int(0)
    _check(load_library().pa_device_cu_count(ctypes.byref(n)), "pa_device_cu_count")
    return n.value


def set_timing_events(partition_start=None, partition_stop=None, reduce_start=None,
                      reduce_stop=None) -> None:
    """Profiling hook: hipEvent_t handles (ints) recorded at the kernels' own
    start / end by later calls from this thread; None pairs switch it off."""
    _check(load_library().pa_set_timing_events(partition_start, partition_stop, reduce_start,
                                               reduce_stop), "pa_set_timing_events")


def stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement hook: streams every byte of ``buf`` (contiguous device
    tensor) once; sink (int32, one word per workgroup) gets each workgroup's
    XOR of the words it read."""
    if not (buf.is_contiguous() and sink.is_contiguous() and sink.dtype == torch.int32):
        raise ValueError("stream_read: contiguous buffer and int32 sink required")
    _check(load_library().pa_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                         sink.data_ptr(), sink.numel(), _stream(stream)),
           "pa_stream_read")


def version() -> str:
    return load_library().pa_version().decode()
