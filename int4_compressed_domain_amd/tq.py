"""Thin ctypes binding of libtq.so (include/tq.h). Argument marshalling only: every step of
the path runs in the library's HIP kernels. Tensors are torch tensors; device pointers and
the current HIP stream are passed through unchanged. Errors raise TQError.

The binding never falls back to anything else: if libtq.so is missing, every call raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_ENOSPC, TQ_EDEVICE = 0, -1, -2, -3, -4
CODEC_ABSMAX, CODEC_LLOYDMAX, CODEC_FP16, CODEC_ABSMAX3, CODEC_ABSMAX2 = 0, 1, 2, 3, 4
F32, BF16, F16 = 0, 1, 2

PROBE_LIB_PATH = os.path.join(HERE, "libtq_probe.so")  # measurement aid (include/tq_probe.h)

EXPORTS = ("tq_status_str", "tq_page_bytes", "tq_kv_append", "tq_decode_workspace_size",
           "tq_decode_attn", "tq_append_decode_attn", "tq_decode_attn_sparse_v", "tq_dequant_ref",
           "tq_dense_decode_attn", "tq_decode_attn_hotcold", "tq_decode_attn_noalloc",
           "tq_append_decode_attn_sparse_v")
PROBE_EXPORTS = ("tq_stream_read_probe",)


class TQError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s" % (where, _lib().tq_status_str(status).decode()))


class tq_layout(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("k_codec", ctypes.c_int32), ("v_codec", ctypes.c_int32),
                ("sign_bits", ctypes.c_void_p)]


_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libtq.so is not built (run int4_compressed_domain_amd/build.py): "
                              + LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        LP = ctypes.POINTER(tq_layout)
        L.tq_status_str.argtypes = [ctypes.c_int]
        L.tq_status_str.restype = ctypes.c_char_p
        L.tq_page_bytes.argtypes = [LP]
        L.tq_page_bytes.restype = sz
        L.tq_kv_append.argtypes = [LP, P, P, P, i32, i32, P, P]
        L.tq_decode_workspace_size.argtypes = [LP, i32, i32, i32]
        L.tq_decode_workspace_size.restype = sz
        L.tq_decode_attn.argtypes = [LP, P, P, i32, i32, P, i32, P, i32, f32, i32, P, P, sz, P]
        if hasattr(L, "tq_append_decode_attn"):  # (absent from older builds of the library)
            L.tq_append_decode_attn.argtypes = [LP, P, P, P, i32, P, i32, i32, P, i32, P, i32, f32,
                                                i32, P, P, sz, P]
            L.tq_append_decode_attn.restype = ctypes.c_int
        if hasattr(L, "tq_decode_attn_sparse_v"):  # (absent from older builds of the library)
            L.tq_decode_attn_sparse_v.argtypes = [LP, P, P, i32, i32, P, i32, P, i32, f32, f32, i32,
                                                  P, P, sz, P, P]
            L.tq_decode_attn_sparse_v.restype = ctypes.c_int
        if hasattr(L, "tq_append_decode_attn_sparse_v"):
            L.tq_append_decode_attn_sparse_v.argtypes = [LP, P, P, P, i32, P, i32, i32, P, i32, P, i32,
                                                         f32, f32, i32, P, P, sz, P, P]
            L.tq_append_decode_attn_sparse_v.restype = ctypes.c_int
        L.tq_dequant_ref.argtypes = [LP, P, i32, P, i32, P, i32, i32, i32, P, P, P]
        if hasattr(L, "tq_decode_attn_hotcold"):
            L.tq_decode_attn_hotcold.argtypes = [LP, P, P, i32, i32, P, i32, P, i32, P, P, P, i32, f32,
                                                 i32, P, P, sz, P]
            L.tq_decode_attn_hotcold.restype = ctypes.c_int
        L.tq_dense_decode_attn.argtypes = [LP, P, P, P, i32, i32, P, i32, f32, i32, P, P, sz, P]
        if hasattr(L, "tq_decode_attn_noalloc"):
            L.tq_decode_attn_noalloc.argtypes = [LP, P, P, i32, i32, P, i32, P, i32, f32, i32, P, P]
            L.tq_decode_attn_noalloc.restype = ctypes.c_int
        for name in ("tq_kv_append", "tq_decode_attn", "tq_dequant_ref", "tq_dense_decode_attn"):
            getattr(L, name).restype = ctypes.c_int
        _L = L
    return _L


def lib():
    return _lib()


_PL = None


def probe_lib():
    """libtq_probe.so: the streaming-read probe."""
    global _PL
    if _PL is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError("libtq_probe.so is not built (run int4_compressed_domain_amd/build.py): "
                              + PROBE_LIB_PATH)
        L = ctypes.CDLL(PROBE_LIB_PATH)
        L.tq_stream_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                           ctypes.c_size_t, ctypes.c_void_p]
        L.tq_stream_read_probe.restype = ctypes.c_int
        _PL = L
    return _PL


def make_layout(head_dim, num_q_heads, num_kv_heads, num_pages, sign_bits_ptr, k_codec=0,
                v_codec=0, group_size=32, page_size=16):
    return tq_layout(head_dim, num_q_heads, num_kv_heads, group_size, page_size, num_pages,
                     k_codec, v_codec, sign_bits_ptr)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t):
    import torch
    return {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}[t.dtype]


def _check(rc, where):
    if rc != TQ_OK:
        raise TQError(rc, where)


def tq_page_bytes(layout):
    return _lib().tq_page_bytes(ctypes.byref(layout))


def tq_kv_append(layout, pool, k, v, slot_mapping, stream=None):
    n = k.shape[0] if k is not None else 0
    _check(_lib().tq_kv_append(ctypes.byref(layout), _ptr(pool), _ptr(k), _ptr(v), _dtype_code(k),
                               n, _ptr(slot_mapping), _stream(stream)), "tq_kv_append")


def tq_decode_workspace_size(layout, batch, max_context_len, num_splits=0):
    return _lib().tq_decode_workspace_size(ctypes.byref(layout), batch, max_context_len, num_splits)


def tq_decode_attn(layout, pool, q, block_table, context_lens, max_context_len, attn_scale, out,
                   workspace, num_splits=0, stream=None):
    _check(_lib().tq_decode_attn(
        ctypes.byref(layout), _ptr(pool), _ptr(q), _dtype_code(q), q.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(context_lens), max_context_len, attn_scale, num_splits,
        _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)), "tq_decode_attn")


def tq_decode_attn_noalloc(layout, pool, q, block_table, context_lens, max_context_len, attn_scale,
                           out, num_splits=0, stream=None):
    """tq_decode_attn on the library's own device scratch (no workspace argument)."""
    _check(_lib().tq_decode_attn_noalloc(
        ctypes.byref(layout), _ptr(pool), _ptr(q), _dtype_code(q), q.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(context_lens), max_context_len, attn_scale, num_splits,
        _ptr(out), _stream(stream)), "tq_decode_attn_noalloc")


def tq_append_decode_attn(layout, pool, k_last, v_last, q, block_table, context_lens,
                          max_context_len, attn_scale, out, workspace, num_splits=0, stream=None):
    """Append each sequence's newest token (k_last, v_last: [batch][Hkv][D]), then decode."""
    _check(_lib().tq_append_decode_attn(
        ctypes.byref(layout), _ptr(pool), _ptr(k_last), _ptr(v_last), _dtype_code(k_last),
        _ptr(q), _dtype_code(q), q.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(context_lens), max_context_len, attn_scale, num_splits, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)), "tq_append_decode_attn")


def tq_decode_attn_sparse_v(layout, pool, q, block_table, context_lens, max_context_len,
                            attn_scale, v_threshold, out, workspace, num_splits=0,
                            v_pages_skipped=None, stream=None):
    """tq_decode_attn that skips the values of pages whose weights are all below v_threshold;
    v_pages_skipped: optional int64 device tensor of one element, added to."""
    _check(_lib().tq_decode_attn_sparse_v(
        ctypes.byref(layout), _ptr(pool), _ptr(q), _dtype_code(q), q.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(context_lens), max_context_len, attn_scale, v_threshold,
        num_splits, _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(v_pages_skipped), _stream(stream)), "tq_decode_attn_sparse_v")


def tq_append_decode_attn_sparse_v(layout, pool, k_last, v_last, q, block_table, context_lens,
                                   max_context_len, attn_scale, v_threshold, out, workspace,
                                   num_splits=0, v_pages_skipped=None, stream=None):
    """tq_append_decode_attn with sparse values (tq_decode_attn_sparse_v's threshold)."""
    _check(_lib().tq_append_decode_attn_sparse_v(
        ctypes.byref(layout), _ptr(pool), _ptr(k_last), _ptr(v_last), _dtype_code(k_last),
        _ptr(q), _dtype_code(q), q.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(context_lens), max_context_len, attn_scale, v_threshold, num_splits, _ptr(out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(v_pages_skipped),
        _stream(stream)), "tq_append_decode_attn_sparse_v")


def tq_dequant_ref(layout, pool, block_table, context_lens, max_context_len, k_out, v_out,
                   to_original_basis=1, stream=None):
    _check(_lib().tq_dequant_ref(
        ctypes.byref(layout), _ptr(pool), context_lens.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(context_lens), max_context_len, to_original_basis,
        _dtype_code(k_out), _ptr(k_out), _ptr(v_out), _stream(stream)), "tq_dequant_ref")


def tq_dense_decode_attn(layout, k, v, q, context_lens, max_context_len, attn_scale, out,
                         workspace, num_splits=0, stream=None):
    _check(_lib().tq_dense_decode_attn(
        ctypes.byref(layout), _ptr(k), _ptr(v), _ptr(q), _dtype_code(q), q.shape[0],
        _ptr(context_lens), max_context_len, attn_scale, num_splits, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)), "tq_dense_decode_attn")


def tq_stream_read_probe(buf, sink, stream=None):
    """Read every byte of buf (a device tensor) with the plain streaming kernel."""
    _check(probe_lib().tq_stream_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                            sink.numel() * sink.element_size(), _stream(stream)),
           "tq_stream_read_probe")


def tq_decode_attn_hotcold(layout, pool, q, block_table, cold_lens, max_cold_len, hot_k, hot_v,
                           hot_lens, attn_scale, out, workspace, num_splits=0, stream=None):
    """Decode over the pool's cold tokens and an fp16 tail (hot_k, hot_v: [B][Hkv][cap][D])."""
    _check(_lib().tq_decode_attn_hotcold(
        ctypes.byref(layout), _ptr(pool), _ptr(q), _dtype_code(q), q.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(cold_lens), max_cold_len, _ptr(hot_k), _ptr(hot_v), _ptr(hot_lens),
        hot_k.shape[2], attn_scale, num_splits, _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)), "tq_decode_attn_hotcold")
