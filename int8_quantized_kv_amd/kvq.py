"""ctypes binding of libkvq (argument marshalling only).

Every function here has the name of the C entry point it calls and passes
device pointers (``torch.Tensor.data_ptr()`` or plain integers), sizes and the
current HIP stream through unchanged.  All computation happens in the HIP
kernels of libkvq.so; if the library is missing the import fails loudly.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KVQ_LIBRARY", os.path.join(_HERE, "libkvq.so"))

KVQ_OK = 0
KVQ_ERR_INVALID_ARG = 1
KVQ_ERR_OUT_OF_RANGE = 2
KVQ_ERR_UNSUPPORTED = 3
KVQ_ERR_HIP = 4
KVQ_ERR_WORKSPACE = 5

KVQ_SCALE_PER_TOKEN = 0
KVQ_SCALE_GROUP32 = 1
KVQ_SCALE_PER_TOKEN_BF16 = 2
KVQ_CODES_FP8_E4M3 = 3
KVQ_CODES_FP8_E5M2 = 4
KVQ_SCALE_BLOCK_HEAD = 5
KVQ_SCALE_BLOCK_CHANNEL = 6
KVQ_LAYOUT_CONTIGUOUS = 0
KVQ_LAYOUT_PAGED = 1
KVQ_DT_F32 = 0
KVQ_DT_BF16 = 1

STATUS_NAMES = {0: "OK", 1: "INVALID_ARG", 2: "OUT_OF_RANGE", 3: "UNSUPPORTED", 4: "HIP", 5: "WORKSPACE"}

EXPORTED = ("kvq_append", "kvq_attention_decode", "kvq_append_decode", "kvq_attention_chunk", "kvq_dequant",
            "kvq_workspace_size", "kvq_cache_bytes", "kvq_last_error", "kvq_version",
            "kvq_append_recent", "kvq_attention_decode_recent", "kvq_append_decode_recent", "kvq_dequant_recent",
            "kvq_workspace_size_recent", "kvq_attention_decode_window", "kvq_append_decode_window",
            "kvq_attention_chunk_window", "kvq_workspace_size_window", "kvq_attention_chunk_recent",
            "kvq_workspace_size_chunk_recent", "kvq_stream_read", "kvq_append_decode_noalloc")


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class kvq_cache(ctypes.Structure):
    """Mirror of ``struct kvq_cache`` in include/kvq.h."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("scale_mode", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("k_codes", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
    ]


class kvq_recent(ctypes.Structure):
    """Mirror of ``struct kvq_recent`` in include/kvq.h."""
    _fields_ = [
        ("window", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
    ]


def _hip_runtimes():
    """Distinct libamdhip64 files mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def _load(path: str = LIB_PATH):
    # torch ships its own HIP runtime with the same soname as the system one.
    # Loading torch first makes libkvq bind to that already-loaded runtime, so
    # one process never holds two HIP runtimes (the second one would not see
    # the device).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError(f"libkvq.so not found at {path}; build it with "
                          "`python int8_quantized_kv_amd/build.py`")
    lib = ctypes.CDLL(path)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError("two HIP runtimes are loaded (" + ", ".join(sorted(runtimes)) +
                          "); import torch before loading libkvq")
    P = ctypes.c_void_p
    I = ctypes.c_int32
    CP = ctypes.POINTER(kvq_cache)
    lib.kvq_append.argtypes = [CP, P, P, I, I, P, P]
    lib.kvq_append.restype = I
    lib.kvq_attention_decode.argtypes = [CP, P, P, ctypes.c_float, P, P, ctypes.c_size_t, I, P]
    lib.kvq_attention_decode.restype = I
    lib.kvq_append_decode.argtypes = [CP, P, P, I, P, P, ctypes.c_float, P, P, ctypes.c_size_t, I, P]
    lib.kvq_append_decode.restype = I
    lib.kvq_attention_chunk.argtypes = [CP, P, I, P, I, ctypes.c_float, P, P, ctypes.c_size_t, I, P]
    lib.kvq_attention_chunk.restype = I
    lib.kvq_dequant.argtypes = [CP, I, P, I, P, I, P]
    lib.kvq_dequant.restype = I
    lib.kvq_workspace_size.argtypes = [CP, I, I]
    lib.kvq_workspace_size.restype = ctypes.c_size_t
    lib.kvq_cache_bytes.argtypes = [CP]
    lib.kvq_cache_bytes.restype = ctypes.c_uint64
    RP = ctypes.POINTER(kvq_recent)
    lib.kvq_append_recent.argtypes = [CP, RP, P, P, I, I, P, P]
    lib.kvq_append_recent.restype = I
    lib.kvq_attention_decode_recent.argtypes = [CP, RP, P, P, ctypes.c_float, P, P, ctypes.c_size_t, I, P]
    lib.kvq_attention_decode_recent.restype = I
    lib.kvq_append_decode_recent.argtypes = [CP, RP, P, P, I, P, P, ctypes.c_float, P, P, ctypes.c_size_t, I, P]
    lib.kvq_append_decode_recent.restype = I
    lib.kvq_dequant_recent.argtypes = [CP, RP, I, P, I, P, I, P]
    lib.kvq_dequant_recent.restype = I
    lib.kvq_workspace_size_recent.argtypes = [CP, RP, I]
    lib.kvq_workspace_size_recent.restype = ctypes.c_size_t
    lib.kvq_attention_chunk_recent.argtypes = [CP, RP, P, I, P, ctypes.c_float, P, P, ctypes.c_size_t, I, P]
    lib.kvq_attention_chunk_recent.restype = I
    lib.kvq_workspace_size_chunk_recent.argtypes = [CP, RP, I, I]
    lib.kvq_workspace_size_chunk_recent.restype = ctypes.c_size_t
    F = ctypes.c_float
    lib.kvq_attention_decode_window.argtypes = [CP, P, P, F, I, P, P, ctypes.c_size_t, I, P]
    lib.kvq_attention_decode_window.restype = I
    lib.kvq_append_decode_window.argtypes = [CP, P, P, I, P, P, F, I, P, P, ctypes.c_size_t, I, P]
    lib.kvq_append_decode_window.restype = I
    lib.kvq_attention_chunk_window.argtypes = [CP, P, I, P, F, I, P, P, ctypes.c_size_t, I, P]
    lib.kvq_attention_chunk_window.restype = I
    lib.kvq_workspace_size_window.argtypes = [CP, I, I, I]
    lib.kvq_workspace_size_window.restype = ctypes.c_size_t
    lib.kvq_append_decode_noalloc.argtypes = [CP, P, P, I, P, P, F, P, I, P]
    lib.kvq_append_decode_noalloc.restype = I
    lib.kvq_stream_read.argtypes = [P, ctypes.c_size_t, P, I, I, I, I, P]
    lib.kvq_stream_read.restype = I
    lib.kvq_last_error.argtypes = []
    lib.kvq_last_error.restype = ctypes.c_char_p
    lib.kvq_version.argtypes = []
    lib.kvq_version.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library():
    return _lib


def load_library(path: str):
    """Another build of libkvq (the KVQ_DEBUG one, say) with the same
    prototypes; its calls report errors through its own kvq_last_error."""
    return _load(path)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except Exception:
            pass
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != KVQ_OK:
        raise KvqError(status, kvq_last_error())


def kvq_last_error() -> str:
    return _lib.kvq_last_error().decode()


def kvq_version() -> str:
    return _lib.kvq_version().decode()


def make_cache(batch, num_heads, num_kv_heads, head_dim, k_codes, v_codes, k_scales, v_scales, *,
               layout=KVQ_LAYOUT_CONTIGUOUS, scale_mode=KVQ_SCALE_PER_TOKEN, max_len=0,
               page_size=16, num_pages=0, max_blocks_per_seq=0, block_table=None) -> kvq_cache:
    """Fill a ``kvq_cache`` descriptor from tensors (or raw device pointers)."""
    return kvq_cache(batch, num_heads, num_kv_heads, head_dim, layout, scale_mode, max_len,
                     page_size if layout == KVQ_LAYOUT_PAGED else 0, num_pages, max_blocks_per_seq,
                     _ptr(block_table), _ptr(k_codes), _ptr(v_codes), _ptr(k_scales), _ptr(v_scales))


def kvq_append(cache: kvq_cache, k_new, v_new, in_dtype: int, n_new: int, start_pos, stream=None):
    _check(_lib.kvq_append(ctypes.byref(cache), _ptr(k_new), _ptr(v_new), in_dtype, n_new,
                           _ptr(start_pos), _stream(stream)))


def kvq_attention_decode(cache: kvq_cache, q, seq_lens, attn_scale: float, out, workspace,
                         workspace_bytes: int, max_seq_len_hint: int, stream=None):
    _check(_lib.kvq_attention_decode(ctypes.byref(cache), _ptr(q), _ptr(seq_lens), attn_scale, _ptr(out),
                                     _ptr(workspace), workspace_bytes, max_seq_len_hint, _stream(stream)))


def kvq_append_decode(cache: kvq_cache, k_new, v_new, in_dtype: int, q, seq_lens, attn_scale: float, out,
                      workspace, workspace_bytes: int, max_seq_len_hint: int, stream=None):
    _check(_lib.kvq_append_decode(ctypes.byref(cache), _ptr(k_new), _ptr(v_new), in_dtype, _ptr(q), _ptr(seq_lens),
                                  attn_scale, _ptr(out), _ptr(workspace), workspace_bytes, max_seq_len_hint,
                                  _stream(stream)))


def kvq_attention_chunk(cache: kvq_cache, q, n: int, ctx_lens, causal: bool, attn_scale: float, out,
                        workspace, workspace_bytes: int, max_ctx_len_hint: int, stream=None):
    _check(_lib.kvq_attention_chunk(ctypes.byref(cache), _ptr(q), n, _ptr(ctx_lens), int(bool(causal)),
                                    attn_scale, _ptr(out), _ptr(workspace), workspace_bytes,
                                    max_ctx_len_hint, _stream(stream)))


def kvq_dequant(cache: kvq_cache, which: int, seq_lens, out_dtype: int, out, out_len: int, stream=None):
    _check(_lib.kvq_dequant(ctypes.byref(cache), which, _ptr(seq_lens), out_dtype, _ptr(out), out_len,
                            _stream(stream)))


def kvq_workspace_size(cache: kvq_cache, max_seq_len: int, n_query: int) -> int:
    n = _lib.kvq_workspace_size(ctypes.byref(cache), max_seq_len, n_query)
    if n == 0:
        msg = kvq_last_error()
        if msg:
            raise KvqError(KVQ_ERR_INVALID_ARG, msg)
    return int(n)


def kvq_cache_bytes(cache: kvq_cache) -> int:
    n = _lib.kvq_cache_bytes(ctypes.byref(cache))
    if n == 0:
        raise KvqError(KVQ_ERR_INVALID_ARG, kvq_last_error())
    return int(n)


def make_recent(window: int, capacity: int, k, v) -> kvq_recent:
    """Fill a ``kvq_recent`` descriptor (bf16 rings [B, KVH, capacity, D])."""
    return kvq_recent(window, capacity, _ptr(k), _ptr(v))


def _rp(recent):
    return None if recent is None else ctypes.byref(recent)


def kvq_append_recent(cache: kvq_cache, recent, k_new, v_new, in_dtype: int, n_new: int, start_pos, stream=None):
    _check(_lib.kvq_append_recent(ctypes.byref(cache), _rp(recent), _ptr(k_new), _ptr(v_new), in_dtype, n_new,
                                  _ptr(start_pos), _stream(stream)))


def kvq_attention_decode_recent(cache: kvq_cache, recent, q, seq_lens, attn_scale: float, out, workspace,
                                workspace_bytes: int, max_seq_len_hint: int, stream=None):
    _check(_lib.kvq_attention_decode_recent(ctypes.byref(cache), _rp(recent), _ptr(q), _ptr(seq_lens), attn_scale,
                                            _ptr(out), _ptr(workspace), workspace_bytes, max_seq_len_hint,
                                            _stream(stream)))


def kvq_append_decode_recent(cache: kvq_cache, recent, k_new, v_new, in_dtype: int, q, seq_lens,
                             attn_scale: float, out, workspace, workspace_bytes: int, max_seq_len_hint: int,
                             stream=None):
    _check(_lib.kvq_append_decode_recent(ctypes.byref(cache), _rp(recent), _ptr(k_new), _ptr(v_new), in_dtype,
                                         _ptr(q), _ptr(seq_lens), attn_scale, _ptr(out), _ptr(workspace),
                                         workspace_bytes, max_seq_len_hint, _stream(stream)))


def kvq_dequant_recent(cache: kvq_cache, recent, which: int, seq_lens, out_dtype: int, out, out_len: int,
                       stream=None):
    _check(_lib.kvq_dequant_recent(ctypes.byref(cache), _rp(recent), which, _ptr(seq_lens), out_dtype, _ptr(out),
                                   out_len, _stream(stream)))


def kvq_workspace_size_recent(cache: kvq_cache, recent, max_seq_len: int) -> int:
    n = _lib.kvq_workspace_size_recent(ctypes.byref(cache), _rp(recent), max_seq_len)
    if n == 0 and kvq_last_error():
        raise KvqError(KVQ_ERR_INVALID_ARG, kvq_last_error())
    return n


def kvq_attention_chunk_recent(cache: kvq_cache, recent, q, n: int, ctx_lens, attn_scale: float, out, workspace,
                               workspace_bytes: int, max_ctx_len_hint: int, stream=None):
    _check(_lib.kvq_attention_chunk_recent(ctypes.byref(cache), _rp(recent), _ptr(q), n, _ptr(ctx_lens), attn_scale,
                                           _ptr(out), _ptr(workspace), workspace_bytes, max_ctx_len_hint,
                                           _stream(stream)))


def kvq_workspace_size_chunk_recent(cache: kvq_cache, recent, max_seq_len: int, n_query: int) -> int:
    n = _lib.kvq_workspace_size_chunk_recent(ctypes.byref(cache), _rp(recent), max_seq_len, n_query)
    if n == 0 and kvq_last_error():
        raise KvqError(KVQ_ERR_INVALID_ARG, kvq_last_error())
    return n


def kvq_attention_decode_window(cache: kvq_cache, q, seq_lens, attn_scale: float, window: int, out, workspace,
                                workspace_bytes: int, max_seq_len_hint: int, stream=None):
    _check(_lib.kvq_attention_decode_window(ctypes.byref(cache), _ptr(q), _ptr(seq_lens), attn_scale, window,
                                            _ptr(out), _ptr(workspace), workspace_bytes, max_seq_len_hint,
                                            _stream(stream)))


def kvq_append_decode_window(cache: kvq_cache, k_new, v_new, in_dtype: int, q, seq_lens, attn_scale: float,
                             window: int, out, workspace, workspace_bytes: int, max_seq_len_hint: int, stream=None):
    _check(_lib.kvq_append_decode_window(ctypes.byref(cache), _ptr(k_new), _ptr(v_new), in_dtype, _ptr(q),
                                         _ptr(seq_lens), attn_scale, window, _ptr(out), _ptr(workspace),
                                         workspace_bytes, max_seq_len_hint, _stream(stream)))


def kvq_attention_chunk_window(cache: kvq_cache, q, n: int, ctx_lens, attn_scale: float, window: int, out,
                               workspace, workspace_bytes: int, max_ctx_len_hint: int, stream=None):
    _check(_lib.kvq_attention_chunk_window(ctypes.byref(cache), _ptr(q), n, _ptr(ctx_lens), attn_scale, window,
                                           _ptr(out), _ptr(workspace), workspace_bytes, max_ctx_len_hint,
                                           _stream(stream)))


def kvq_workspace_size_window(cache: kvq_cache, max_seq_len: int, n_query: int, window: int) -> int:
    n = _lib.kvq_workspace_size_window(ctypes.byref(cache), max_seq_len, n_query, window)
    if n == 0 and kvq_last_error():
        raise KvqError(KVQ_ERR_INVALID_ARG, kvq_last_error())
    return n


def kvq_stream_read(src, nbytes: int, sink, workgroups: int, waves_per_wg: int = 8, depth: int = 4,
                    interleave: bool = True, stream=None, nontemporal: bool = False):
    _check(_lib.kvq_stream_read(_ptr(src), nbytes, _ptr(sink), workgroups, waves_per_wg, depth,
                                (1 if interleave else 0) | (2 if nontemporal else 0), _stream(stream)))


def kvq_append_decode_noalloc(cache: kvq_cache, k_new, v_new, in_dtype: int, q, seq_lens, attn_scale: float, out,
                              max_seq_len_hint: int, stream=None):
    _check(_lib.kvq_append_decode_noalloc(ctypes.byref(cache), _ptr(k_new), _ptr(v_new), in_dtype, _ptr(q),
                                          _ptr(seq_lens), attn_scale, _ptr(out), max_seq_len_hint,
                                          _stream(stream)))
