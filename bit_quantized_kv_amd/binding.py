"""Thin ctypes binding of ``libtq.so`` (argument marshalling only).

The functions carry the C names; torch tensors are passed by ``data_ptr()``
and the current HIP stream by its handle.  Every compute step runs in the
library's HIP kernels; there is no fallback path: if the library cannot be
loaded, importing this module raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtq.so")

TQ_FORMAT_TQ4 = 0
TQ_FORMAT_MXFP4 = 1
TQ_FORMAT_TQ4V2 = 2
TQ_OUT_F32 = 0
TQ_OUT_BF16 = 1

# entry points declared in include/tq.h
EXPORTS = (
    "tq_record_bytes", "tq_pool_bytes", "tq_create_cache", "tq_cache_info", "tq_default_key_table",
    "tq_quantize_append", "tq_decode_workspace_bytes", "tq_decode_attention", "tq_free",
    "tq_status_string", "tq_last_error", "tq_calibrate_workspace_bytes", "tq_calibrate_key_tables",
    "tq_select_layers", "tq_multitoken_workspace_bytes", "tq_multitoken_attention", "tq_cascade_workspace_bytes",
    "tq_cascade_decode_attention", "tq_debug_dequantize", "tq_decode_attention_noalloc",
)


class TqError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("key_table", ctypes.POINTER(ctypes.c_float)),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python bit_quantized_kv_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    sz = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "tq_record_bytes": ([ctypes.POINTER(CacheDesc), sz], ctypes.c_int),
        "tq_pool_bytes": ([ctypes.POINTER(CacheDesc), sz], ctypes.c_int),
        "tq_create_cache": ([ctypes.POINTER(CacheDesc), P, ctypes.c_size_t, ctypes.POINTER(P)], ctypes.c_int),
        "tq_cache_info": ([P, ctypes.POINTER(P), sz, ctypes.POINTER(ctypes.c_uint16)], ctypes.c_int),
        "tq_default_key_table": ([ctypes.POINTER(ctypes.c_uint16)], ctypes.c_int),
        "tq_quantize_append": ([P, P, P, P, ctypes.c_int64, P], ctypes.c_int),
        "tq_decode_workspace_bytes": ([P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, sz], ctypes.c_int),
        "tq_decode_attention": ([P, P, P, ctypes.c_int32, P, ctypes.c_int32, P, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_float, P, ctypes.c_size_t, P], ctypes.c_int),
        "tq_calibrate_workspace_bytes": ([ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, sz], ctypes.c_int),
        "tq_calibrate_key_tables": ([P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_float), ctypes.c_int32, P, P, P, P, P,
                                     ctypes.c_size_t, P], ctypes.c_int),
        "tq_select_layers": ([ctypes.POINTER(ctypes.c_double), ctypes.c_int32, ctypes.c_int32,
                              ctypes.POINTER(ctypes.c_uint8)], ctypes.c_int),
        "tq_multitoken_workspace_bytes": ([P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                           ctypes.c_int32, sz], ctypes.c_int),
        "tq_multitoken_attention": ([P, P, P, ctypes.c_int32, P, ctypes.c_int64, ctypes.c_int32, P, ctypes.c_int32,
                                     P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, P,
                                     ctypes.c_size_t, P], ctypes.c_int),
        "tq_cascade_workspace_bytes": ([P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, sz], ctypes.c_int),
        "tq_cascade_decode_attention": ([P, P, P, ctypes.c_int32, P, ctypes.c_int32, P, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_float, P, P, P, P, P, P,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P,
                                         ctypes.c_size_t, P], ctypes.c_int),
        "tq_debug_dequantize": ([P, P, ctypes.c_int32, P, P, P], ctypes.c_int),
        "tq_decode_attention_noalloc": ([P, P, P, ctypes.c_int32, P, ctypes.c_int32, P, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_float, P], ctypes.c_int),
        "tq_free": ([P], None),
        "tq_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "tq_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


LIB = _load()


def _check(status):
    if status != 0:
        raise TqError(status, f"{LIB.tq_status_string(status).decode()}: {LIB.tq_last_error().decode()}")


def _desc(fmt, head_dim, num_kv_heads, num_blocks, key_table=None):
    d = CacheDesc(fmt, head_dim, num_kv_heads, 16, num_blocks, None)
    keep = None
    if key_table is not None:
        keep = (ctypes.c_float * 16)(*[float(x) for x in key_table])
        d.key_table = ctypes.cast(keep, ctypes.POINTER(ctypes.c_float))
    return d, keep


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


# ---- functions with the C names ------------------------------------------------

def tq_record_bytes(fmt, head_dim, num_kv_heads=1, num_blocks=1):
    d, _ = _desc(fmt, head_dim, num_kv_heads, num_blocks)
    out = ctypes.c_size_t()
    _check(LIB.tq_record_bytes(ctypes.byref(d), ctypes.byref(out)))
    return out.value


def tq_pool_bytes(fmt, head_dim, num_kv_heads, num_blocks):
    d, _ = _desc(fmt, head_dim, num_kv_heads, num_blocks)
    out = ctypes.c_size_t()
    _check(LIB.tq_pool_bytes(ctypes.byref(d), ctypes.byref(out)))
    return out.value


def tq_default_key_table():
    """The library's own default key table as fp16 bit patterns (no GPU)."""
    buf = (ctypes.c_uint16 * 16)()
    _check(LIB.tq_default_key_table(buf))
    return list(buf)


def tq_create_cache(fmt, head_dim, num_kv_heads, num_blocks, key_table=None, pool=None):
    """Returns an opaque handle.  ``pool``: a device uint8 tensor of at least
    tq_pool_bytes bytes (kept by the caller) or None (library-owned)."""
    d, keep = _desc(fmt, head_dim, num_kv_heads, num_blocks, key_table)
    h = ctypes.c_void_p()
    nbytes = pool.numel() * pool.element_size() if pool is not None else 0
    _check(LIB.tq_create_cache(ctypes.byref(d), _ptr(pool), nbytes, ctypes.byref(h)))
    del keep
    return h


def tq_cache_info(cache):
    p = ctypes.c_void_p()
    n = ctypes.c_size_t()
    tab = (ctypes.c_uint16 * 16)()
    _check(LIB.tq_cache_info(cache, ctypes.byref(p), ctypes.byref(n), tab))
    return p.value, n.value, list(tab)


def tq_quantize_append(cache, k, v, slot_mapping, stream=None):
    _check(LIB.tq_quantize_append(cache, _ptr(k), _ptr(v), _ptr(slot_mapping), int(slot_mapping.numel()),
                                  _stream(stream)))


def tq_decode_workspace_bytes(cache, batch, num_q_heads, max_context_len):
    out = ctypes.c_size_t()
    _check(LIB.tq_decode_workspace_bytes(cache, batch, num_q_heads, max_context_len, ctypes.byref(out)))
    return out.value


def tq_decode_attention(cache, q, out, block_table, context_lens, max_context_len, softmax_scale,
                        workspace=None, stream=None):
    b, hq, _ = q.shape
    out_dtype = TQ_OUT_BF16 if str(out.dtype) == "torch.bfloat16" else TQ_OUT_F32
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(LIB.tq_decode_attention(cache, _ptr(q), _ptr(out), out_dtype, _ptr(block_table),
                                   int(block_table.shape[1]), _ptr(context_lens), b, hq, int(max_context_len),
                                   float(softmax_scale), _ptr(workspace), wbytes, _stream(stream)))


def tq_decode_attention_noalloc(cache, q, out, block_table, context_lens, max_context_len, softmax_scale,
                                stream=None):
    """tq_decode_attention without a workspace (the library's fixed scratch)."""
    b, hq, _ = q.shape
    out_dtype = TQ_OUT_BF16 if str(out.dtype) == "torch.bfloat16" else TQ_OUT_F32
    _check(LIB.tq_decode_attention_noalloc(cache, _ptr(q), _ptr(out), out_dtype, _ptr(block_table),
                                           int(block_table.shape[1]), _ptr(context_lens), b, hq,
                                           int(max_context_len), float(softmax_scale), _stream(stream)))


def tq_multitoken_workspace_bytes(cache, batch, num_q_heads, num_tokens, max_query_len, max_context_len):
    out = ctypes.c_size_t()
    _check(LIB.tq_multitoken_workspace_bytes(cache, batch, num_q_heads, num_tokens, max_query_len,
                                             max_context_len, ctypes.byref(out)))
    return out.value


def tq_multitoken_attention(cache, q, out, q_start, max_query_len, block_table, context_lens, max_context_len,
                            softmax_scale, workspace=None, stream=None):
    """q: device bf16 [num_tokens, Hq, D]; q_start: device int32 [batch + 1]."""
    n, hq, _ = q.shape
    batch = int(q_start.numel()) - 1
    out_dtype = TQ_OUT_BF16 if str(out.dtype) == "torch.bfloat16" else TQ_OUT_F32
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(LIB.tq_multitoken_attention(cache, _ptr(q), _ptr(out), out_dtype, _ptr(q_start), n, int(max_query_len),
                                       _ptr(block_table), int(block_table.shape[1]), _ptr(context_lens), batch, hq,
                                       int(max_context_len), float(softmax_scale), _ptr(workspace), wbytes,
                                       _stream(stream)))


def tq_cascade_workspace_bytes(cache, batch, num_q_heads, max_context_len, num_groups, max_group_size,
                               max_group_blocks, max_depth):
    out = ctypes.c_size_t()
    _check(LIB.tq_cascade_workspace_bytes(cache, batch, num_q_heads, max_context_len, num_groups, max_group_size,
                                          max_group_blocks, max_depth, ctypes.byref(out)))
    return out.value


def tq_cascade_decode_attention(cache, q, out, block_table, context_lens, max_context_len, softmax_scale, groups,
                                workspace, stream=None):
    """``groups``: a CascadeGroups of device int32 tensors (see cache.py)."""
    b, hq, _ = q.shape
    out_dtype = TQ_OUT_BF16 if str(out.dtype) == "torch.bfloat16" else TQ_OUT_F32
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(LIB.tq_cascade_decode_attention(
        cache, _ptr(q), _ptr(out), out_dtype, _ptr(block_table), int(block_table.shape[1]), _ptr(context_lens), b,
        hq, int(max_context_len), float(softmax_scale), _ptr(groups.seq_prefix_blocks), _ptr(groups.seq_depth),
        _ptr(groups.group_start), _ptr(groups.group_seqs), _ptr(groups.group_blocks), _ptr(groups.group_depth),
        groups.num_groups, groups.max_group_size, groups.max_group_blocks, groups.max_depth, _ptr(workspace),
        wbytes, _stream(stream)))


def tq_calibrate_workspace_bytes(num_layers, rows, head_dim):
    out = ctypes.c_size_t()
    _check(LIB.tq_calibrate_workspace_bytes(num_layers, rows, head_dim, ctypes.byref(out)))
    return out.value


def tq_calibrate_key_tables(k, init_table, max_iters, tables_f16, levels=None, mse=None, updates=None,
                            workspace=None, stream=None):
    """k: device bf16 [layers, rows, head_dim]; outputs are device tensors
    (int16 [layers, 16], float64 [layers, 16], float64 [layers, 2], int32
    [layers]); ``init_table``: 16 floats or None (the default table)."""
    layers, rows, d = k.shape
    keep = None
    tab = None
    if init_table is not None:
        keep = (ctypes.c_float * 16)(*[float(x) for x in init_table])
        tab = ctypes.cast(keep, ctypes.POINTER(ctypes.c_float))
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(LIB.tq_calibrate_key_tables(_ptr(k), layers, rows, d, tab, int(max_iters), _ptr(tables_f16),
                                       _ptr(levels), _ptr(mse), _ptr(updates), _ptr(workspace), wbytes,
                                       _stream(stream)))
    del keep


def tq_select_layers(mse, percent=10):
    """Host-side choice of the layers that get a fitted table: list of bools."""
    n = len(mse)
    arr = (ctypes.c_double * max(n, 1))(*[float(x) for x in mse])
    out = (ctypes.c_uint8 * max(n, 1))()
    _check(LIB.tq_select_layers(arr, n, int(percent), out))
    return [bool(out[i]) for i in range(n)]


def tq_debug_dequantize(cache, block_ids, k_out, v_out, stream=None):
    """Test-only: block_ids device int32 [n]; k_out, v_out device float32
    [n, num_kv_heads, 16, head_dim]."""
    _check(LIB.tq_debug_dequantize(cache, _ptr(block_ids), int(block_ids.numel()), _ptr(k_out), _ptr(v_out),
                                   _stream(stream)))


def tq_free(cache):
    LIB.tq_free(cache)
