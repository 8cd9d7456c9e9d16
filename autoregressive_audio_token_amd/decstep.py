"""ctypes binding of libdecstep.so (include/decstep.h), same names as the C ABI.

Argument marshalling only: every step of the hot path runs in the HIP kernels.
Pointer arguments accept a torch tensor (its data_ptr()), a plain integer
address, or None (NULL).  Stream arguments accept a torch.cuda.Stream, a raw
hipStream_t integer, or None (torch's current stream when a GPU is present,
else the NULL stream).  A non-zero dec_status raises DecError.

The library is loaded at import; if it has not been built the import fails
(there is no fallback).  DECSTEP_LIB overrides the library path.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("DECSTEP_LIB") or os.path.join(_HERE, "libdecstep.so")

DEC_BF16, DEC_F32 = 0, 1
DEC_OK, DEC_E_NULL, DEC_E_SHAPE, DEC_E_DTYPE = 0, 1, 2, 3
DEC_E_WORKSPACE, DEC_E_UNSUPPORTED, DEC_E_HIP, DEC_E_ALIGN = 4, 5, 6, 7


class DecError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def _load():
    # torch ships its own libamdhip64 under the same soname.  Importing torch first
    # lets the dynamic loader bind this library to that same HIP runtime instance;
    # loading ours first would put two HIP runtimes in one process, and the second
    # one to initialise finds no device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m autoregressive_audio_token_amd.build` "
            "(the HIP library is required: there is no CPU fallback)")
    return ctypes.CDLL(LIB_PATH)


_lib = _load()


class Tuning(ctypes.Structure):
    """dec_tuning: launch-policy overrides of the calling thread (all 0: the defaults)."""
    _fields_ = [(n, ctypes.c_int) for n in (
        "attn_chunk_keys", "attn_schedule", "attn_blocks", "attn_no_halves",
        "attn_no_records", "head_kernel", "head_mfma_cfg")]
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGS = {
    "dec_attn_chunk_keys": (_I, []),
    "dec_attn_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "dec_attn_workspace_init": (_I, [_P, _SZ, _P]),
    "dec_attn_self": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "dec_attn_cross": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "dec_attn_step": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _P,
                           _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "dec_attn_step_append": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P,
                                  _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "dec_attn_step_noalloc": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _I, _P,
                                   _I, _I, _I, _I, _I, _F, _P]),
    "dec_attn_step_ex": (_I, [_P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _I, _I, _P,
                              _I, _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "dec_attn_self_paged": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                                 _P, _SZ, _P]),
    "dec_attn_step_paged": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P,
                                 _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "dec_attn_step_paged_ex": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _I,
                                    _I, _P, _I, _I, _I, _I, _I, _I, _F, _P, _SZ, _P]),
    "dec_sample_topk": (_I, [_P, _I, _I, _I, _I, _P, _I, _P, _P, ctypes.c_int32, _P, _P, _P,
                             _P]),
    "dec_sample_topk_philox": (_I, [_P, _I, _I, _I, _I, _P, _I, ctypes.c_uint64, _P,
                                    ctypes.c_int32, _P, _P, _P, _P]),
    "dec_sample_topk_ex": (_I, [_P, _I, _I, _I, _I, _I, _P, _I, _P, ctypes.c_uint64, _P,
                                ctypes.c_int32, _P, _P, _P, _P]),
    "dec_sample_topk_advance": (_I, [_P, _I, _I, _I, _I, _I, _P, _I, _P, ctypes.c_uint64,
                                     _P, _P, ctypes.c_int32, _P, _P, _P, _P]),
    "dec_kv_append": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "dec_lm_head": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "dec_embed_sum": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "dec_step_advance": (_I, [_P, _P, _I, _P]),
    "dec_probe_read": (_I, [_P, _SZ, _P, _P]),
    "dec_probe_empty": (_I, [_P]),
    "dec_graph_begin": (_I, [_P]),
    "dec_graph_end": (_I, [_P, ctypes.POINTER(_P)]),
    "dec_graph_launch": (_I, [_P, _P]),
    "dec_graph_destroy": (_I, [_P]),
    "dec_tuning_set": (_I, [ctypes.POINTER(Tuning)]),
    "dec_tuning_get": (_I, [ctypes.POINTER(Tuning)]),
    "dec_last_hip_error": (_I, []),
    "dec_strerror": (ctypes.c_char_p, [_I]),
    "dec_order_keys_host": (None, [_P, _P, _SZ]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    if hasattr(x, "data_ptr"):
        return x.data_ptr() or None
    if hasattr(x, "ctypes"):            # numpy array (host pointers for host helpers)
        return x.ctypes.data
    raise TypeError(f"cannot pass {type(x).__name__} as a pointer")


def _stream(s):
    if s is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream or None
        return None
    if isinstance(s, int):
        return s or None
    return s.cuda_stream or None


def _check(status):
    if status != DEC_OK:
        msg = _lib.dec_strerror(status).decode()
        if status == DEC_E_HIP:
            msg += f" (hipError_t {_lib.dec_last_hip_error()})"
        raise DecError(status, msg)


def dtype_code(t):
    """DEC_BF16 / DEC_F32 for a torch dtype or tensor."""
    import torch
    dt = getattr(t, "dtype", t)
    if dt == torch.bfloat16:
        return DEC_BF16
    if dt == torch.float32:
        return DEC_F32
    raise TypeError(f"unsupported element type {dt}")


def dec_attn_chunk_keys():
    return _lib.dec_attn_chunk_keys()


def dec_attn_workspace_bytes(n_layers, B, H, hd, L_cap_self, L_cap_cross):
    return _lib.dec_attn_workspace_bytes(n_layers, B, H, hd, L_cap_self, L_cap_cross)


def dec_attn_workspace_init(workspace, ws_bytes, stream=None):
    _check(_lib.dec_attn_workspace_init(_ptr(workspace), ws_bytes, _stream(stream)))


def dec_attn_self(q, k, v, len, out, n_layers, B, H, L_cap, hd, dtype, scale,
                  workspace, ws_bytes, stream=None):
    _check(_lib.dec_attn_self(_ptr(q), _ptr(k), _ptr(v), _ptr(len), _ptr(out), n_layers, B,
                              H, L_cap, hd, dtype, scale, _ptr(workspace), ws_bytes,
                              _stream(stream)))


def dec_attn_cross(q, k, v, enc_len, out, n_layers, B, H, L_cap, hd, dtype, scale,
                   workspace, ws_bytes, stream=None):
    _check(_lib.dec_attn_cross(_ptr(q), _ptr(k), _ptr(v), _ptr(enc_len), _ptr(out), n_layers,
                               B, H, L_cap, hd, dtype, scale, _ptr(workspace), ws_bytes,
                               _stream(stream)))


def dec_attn_step_append(q_self, k_self, v_self, len, L_cap_self, out_self, k_new, v_new,
                         q_cross, k_cross, v_cross, enc_len, L_cap_cross, out_cross,
                         n_layers, B, H, hd, dtype, scale, workspace, ws_bytes, stream=None):
    _check(_lib.dec_attn_step_append(_ptr(q_self), _ptr(k_self), _ptr(v_self), _ptr(len),
                                     L_cap_self, _ptr(out_self), _ptr(k_new), _ptr(v_new),
                                     _ptr(q_cross), _ptr(k_cross), _ptr(v_cross), _ptr(enc_len),
                                     L_cap_cross, _ptr(out_cross), n_layers, B, H, hd, dtype,
                                     scale, _ptr(workspace), ws_bytes, _stream(stream)))


def dec_attn_step(q_self, k_self, v_self, len, L_cap_self, out_self,
                  q_cross, k_cross, v_cross, enc_len, L_cap_cross, out_cross,
                  n_layers, B, H, hd, dtype, scale, workspace, ws_bytes, stream=None):
    _check(_lib.dec_attn_step(_ptr(q_self), _ptr(k_self), _ptr(v_self), _ptr(len), L_cap_self,
                              _ptr(out_self), _ptr(q_cross), _ptr(k_cross), _ptr(v_cross),
                              _ptr(enc_len), L_cap_cross, _ptr(out_cross), n_layers, B, H, hd,
                              dtype, scale, _ptr(workspace), ws_bytes, _stream(stream)))


def dec_attn_step_noalloc(q_self, k_self, v_self, len, L_cap_self, out_self,
                          q_cross, k_cross, v_cross, enc_len, L_cap_cross, out_cross,
                          n_layers, B, H, hd, dtype, scale, stream=None):
    _check(_lib.dec_attn_step_noalloc(_ptr(q_self), _ptr(k_self), _ptr(v_self), _ptr(len),
                                      L_cap_self, _ptr(out_self), _ptr(q_cross), _ptr(k_cross),
                                      _ptr(v_cross), _ptr(enc_len), L_cap_cross,
                                      _ptr(out_cross), n_layers, B, H, hd, dtype, scale,
                                      _stream(stream)))


def dec_attn_step_ex(q_self, k_self, v_self, len, L_cap_self, out_self, q_cross, k_cross,
                     v_cross, enc_len, cross_mask, mask_words, L_cap_cross, out_cross, n_layers,
                     B, H, hd, dtype, out_dtype, scale, workspace, ws_bytes, stream=None):
    _check(_lib.dec_attn_step_ex(_ptr(q_self), _ptr(k_self), _ptr(v_self), _ptr(len),
                                 L_cap_self, _ptr(out_self), _ptr(q_cross), _ptr(k_cross),
                                 _ptr(v_cross), _ptr(enc_len), _ptr(cross_mask), mask_words,
                                 L_cap_cross, _ptr(out_cross), n_layers, B, H, hd, dtype,
                                 out_dtype, scale, _ptr(workspace), ws_bytes, _stream(stream)))


def dec_attn_self_paged(q, k_pool, v_pool, block_table, len, out, n_layers, B, H, hd,
                        block_size, n_blocks, max_blocks, dtype, scale, workspace, ws_bytes,
                        stream=None):
    _check(_lib.dec_attn_self_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                    _ptr(len), _ptr(out), n_layers, B, H, hd, block_size,
                                    n_blocks, max_blocks, dtype, scale, _ptr(workspace),
                                    ws_bytes, _stream(stream)))


def dec_attn_step_paged_ex(q_self, k_pool, v_pool, block_table, len, block_size, n_blocks,
                           max_blocks, out_self, q_cross, k_cross, v_cross, enc_len, cross_mask,
                           mask_words, L_cap_cross, out_cross, n_layers, B, H, hd, dtype,
                           out_dtype, scale, workspace, ws_bytes, stream=None):
    _check(_lib.dec_attn_step_paged_ex(_ptr(q_self), _ptr(k_pool), _ptr(v_pool),
                                       _ptr(block_table), _ptr(len), block_size, n_blocks,
                                       max_blocks, _ptr(out_self), _ptr(q_cross),
                                       _ptr(k_cross), _ptr(v_cross), _ptr(enc_len),
                                       _ptr(cross_mask), mask_words, L_cap_cross,
                                       _ptr(out_cross), n_layers, B, H, hd, dtype, out_dtype,
                                       scale, _ptr(workspace), ws_bytes, _stream(stream)))


def dec_attn_step_paged(q_self, k_pool, v_pool, block_table, len, block_size, n_blocks,
                        max_blocks, out_self, q_cross, k_cross, v_cross, enc_len, L_cap_cross,
                        out_cross, n_layers, B, H, hd, dtype, scale, workspace, ws_bytes,
                        stream=None):
    _check(_lib.dec_attn_step_paged(_ptr(q_self), _ptr(k_pool), _ptr(v_pool),
                                    _ptr(block_table), _ptr(len), block_size, n_blocks,
                                    max_blocks, _ptr(out_self), _ptr(q_cross), _ptr(k_cross),
                                    _ptr(v_cross), _ptr(enc_len), L_cap_cross, _ptr(out_cross),
                                    n_layers, B, H, hd, dtype, scale, _ptr(workspace),
                                    ws_bytes, _stream(stream)))


def dec_sample_topk(logits, B, n_cb, V_valid, V_stride, temperature, top_k, uniforms, step,
                    fill_token, tokens, topk_idx=None, topk_prob=None, stream=None):
    _check(_lib.dec_sample_topk(_ptr(logits), B, n_cb, V_valid, V_stride, _ptr(temperature),
                                top_k, _ptr(uniforms), _ptr(step), fill_token, _ptr(tokens),
                                _ptr(topk_idx), _ptr(topk_prob), _stream(stream)))


def dec_sample_topk_philox(logits, B, n_cb, V_valid, V_stride, temperature, top_k, seed, step,
                           fill_token, tokens, topk_idx=None, topk_prob=None, stream=None):
    _check(_lib.dec_sample_topk_philox(_ptr(logits), B, n_cb, V_valid, V_stride,
                                       _ptr(temperature), top_k, seed, _ptr(step), fill_token,
                                       _ptr(tokens), _ptr(topk_idx), _ptr(topk_prob),
                                       _stream(stream)))


def dec_sample_topk_advance(logits, logits_dtype, B, n_cb, V_valid, V_stride, temperature,
                            top_k, uniforms, seed, step, len, fill_token, tokens, topk_idx=None,
                            topk_prob=None, stream=None):
    _check(_lib.dec_sample_topk_advance(_ptr(logits), logits_dtype, B, n_cb, V_valid, V_stride,
                                        _ptr(temperature), top_k, _ptr(uniforms), seed,
                                        _ptr(step), _ptr(len), fill_token, _ptr(tokens),
                                        _ptr(topk_idx), _ptr(topk_prob), _stream(stream)))


def dec_sample_topk_ex(logits, logits_dtype, B, n_cb, V_valid, V_stride, temperature, top_k,
                       uniforms, seed, step, fill_token, tokens, topk_idx=None, topk_prob=None,
                       stream=None):
    _check(_lib.dec_sample_topk_ex(_ptr(logits), logits_dtype, B, n_cb, V_valid, V_stride,
                                   _ptr(temperature), top_k, _ptr(uniforms), seed, _ptr(step),
                                   fill_token, _ptr(tokens), _ptr(topk_idx), _ptr(topk_prob),
                                   _stream(stream)))


def dec_kv_append(k_new, v_new, k_cache, v_cache, len, n_layers, B, H, L_cap, hd, dtype,
                  stream=None):
    _check(_lib.dec_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(len),
                              n_layers, B, H, L_cap, hd, dtype, _stream(stream)))


def dec_lm_head(h, W, logits, B, D, n_cb, V_valid, V_stride, stream=None):
    _check(_lib.dec_lm_head(_ptr(h), _ptr(W), _ptr(logits), B, D, n_cb, V_valid, V_stride,
                            _stream(stream)))


def dec_embed_sum(tokens, E, x, B, n_cb, V_emb, D, stream=None):
    _check(_lib.dec_embed_sum(_ptr(tokens), _ptr(E), _ptr(x), B, n_cb, V_emb, D,
                              _stream(stream)))


def dec_step_advance(len, step, B, stream=None):
    _check(_lib.dec_step_advance(_ptr(len), _ptr(step), B, _stream(stream)))


def dec_probe_read(buf, nbytes, sink, stream=None):
    _check(_lib.dec_probe_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))


def dec_probe_empty(stream=None):
    _check(_lib.dec_probe_empty(_stream(stream)))


def dec_graph_begin(stream):
    _check(_lib.dec_graph_begin(_stream(stream)))


def dec_graph_end(stream):
    """Ends capture on ``stream``; returns the executable graph handle (an int)."""
    ex = _P()
    _check(_lib.dec_graph_end(_stream(stream), ctypes.byref(ex)))
    return ex.value


def dec_graph_launch(exec_handle, stream=None):
    _check(_lib.dec_graph_launch(exec_handle, _stream(stream)))


def dec_graph_destroy(exec_handle):
    _check(_lib.dec_graph_destroy(exec_handle))


def dec_tuning_set(**fields):
    """Set the calling thread's overrides (fields of Tuning; unnamed fields are 0).
    No arguments restores the defaults."""
    if not fields:
        _check(_lib.dec_tuning_set(None))
        return
    unknown = set(fields) - {n for n, _ in Tuning._fields_}
    if unknown:
        raise TypeError(f"unknown tuning fields {sorted(unknown)}")
    _check(_lib.dec_tuning_set(ctypes.byref(Tuning(**fields))))


def dec_tuning_get():
    t = Tuning()
    _check(_lib.dec_tuning_get(ctypes.byref(t)))
    return {n: getattr(t, n) for n, _ in Tuning._fields_}


def dec_last_hip_error():
    return _lib.dec_last_hip_error()


def dec_strerror(status):
    return _lib.dec_strerror(status).decode()


def dec_order_keys_host(x, keys, n):
    """x: float32 host array, keys: uint32 host array (numpy), n elements."""
    _lib.dec_order_keys_host(_ptr(x), _ptr(keys), n)


def raw_status(name, *args):
    """Call a dec_* entry point with pre-marshalled arguments; returns the status code
    without raising (used to test the error paths)."""
    return getattr(_lib, name)(*args)
