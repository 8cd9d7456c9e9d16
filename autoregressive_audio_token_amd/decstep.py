"""ctypes binding of libdecstep.so (include/decstep.h), same names as the C ABI.

Argument marshalling only: every step of the hot path runs in the HIP kernels.

Each entry point is declared once below (``_API``): its C parameters in order, and
for every buffer the element type and the shape the header gives it in terms of the
call's integer arguments.  The same declaration sets the ctypes signature and the
checks the binding makes before the call:

* a torch tensor must be on a GPU (the same one for every tensor of the call, and
  the stream's), contiguous, of the element type stated, and hold exactly the
  elements of its shape (a workspace or a probe buffer: at least its byte count);
  a mismatch raises DecError with DEC_E_UNSUPPORTED (device), DEC_E_DTYPE or
  DEC_E_SHAPE (count or layout) and nothing is called;
* a plain integer is passed through as a device address, unchecked; None is NULL
  (the library reports a required NULL as DEC_E_NULL);
* a host array (numpy) is refused for a device pointer.

Integer arguments the header rejects (negative sizes, unknown dtype codes) are left
to the library's own checks, which run before anything is enqueued.  Stream
arguments take a torch.cuda.Stream, a raw hipStream_t integer, or None (torch's
current stream when a GPU is present, else the NULL stream).  A non-zero dec_status
raises DecError.

The library is loaded at import; if it has not been built the import fails (there is
no fallback).  DECSTEP_LIB overrides the library path.
"""
import ctypes
import inspect
import math
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

# ---------------------------------------------------------------------------------
# Declarations.  "name:kind" per C parameter, in order.  Buffer kinds carry a shape,
# kind[d0,d1,...], whose entries are integer parameters of the same call or literals:
#   x     element type named by the call's `dtype` (DEC_BF16 bfloat16, DEC_F32 float32)
#   o     element type named by `out_dtype`;  l  by `logits_dtype`
#   bf16, f32, i32   that element type;  u32 / i64  int32 or uint32 / int64 or uint64
#   bytes            any element type; the shape is a byte count, a lower bound
# Scalars: int (C int), i32 (int32_t), u64 (uint64_t), float, size (size_t), stream.
# A trailing "?" gives the Python parameter a default of None.
# ---------------------------------------------------------------------------------
_ATT = "n_layers:int B:int H:int L_cap:int hd:int dtype:int scale:float " \
       "workspace:bytes[ws_bytes] ws_bytes:size stream:stream?"
_STEP_CROSS = "q_cross:x[n_layers,B,H,hd] k_cross:x[n_layers,B,H,L_cap_cross,hd] " \
              "v_cross:x[n_layers,B,H,L_cap_cross,hd] enc_len:i32[B]"
_PAGED_SELF = "q_self:x[n_layers,B,H,hd] k_pool:x[n_layers,n_blocks,H,block_size,hd] " \
              "v_pool:x[n_layers,n_blocks,H,block_size,hd] block_table:i32[B,max_blocks] " \
              "len:i32[B] block_size:int n_blocks:int max_blocks:int"
_TAIL = "n_layers:int B:int H:int hd:int dtype:int"
_WS = "scale:float workspace:bytes[ws_bytes] ws_bytes:size stream:stream?"
_SAMPLE_OUT = "tokens:i32[B,n_cb] topk_idx:i32[B,n_cb,top_k]? " \
              "topk_prob:f32[B,n_cb,top_k]? stream:stream?"

_API = {
    "dec_attn_workspace_init": "workspace:bytes[ws_bytes] ws_bytes:size stream:stream?",
    "dec_attn_self": "q:x[n_layers,B,H,hd] k:x[n_layers,B,H,L_cap,hd] "
                     "v:x[n_layers,B,H,L_cap,hd] len:i32[B] out:f32[n_layers,B,H,hd] " + _ATT,
    "dec_attn_cross": "q:x[n_layers,B,H,hd] k:x[n_layers,B,H,L_cap,hd] "
                      "v:x[n_layers,B,H,L_cap,hd] enc_len:i32[B] out:f32[n_layers,B,H,hd] "
                      + _ATT,
    "dec_attn_step": "q_self:x[n_layers,B,H,hd] k_self:x[n_layers,B,H,L_cap_self,hd] "
                     "v_self:x[n_layers,B,H,L_cap_self,hd] len:i32[B] L_cap_self:int "
                     "out_self:f32[n_layers,B,H,hd] " + _STEP_CROSS + " L_cap_cross:int "
                     "out_cross:f32[n_layers,B,H,hd] " + _TAIL + " " + _WS,
    "dec_attn_step_append": "q_self:x[n_layers,B,H,hd] k_self:x[n_layers,B,H,L_cap_self,hd] "
                            "v_self:x[n_layers,B,H,L_cap_self,hd] len:i32[B] L_cap_self:int "
                            "out_self:f32[n_layers,B,H,hd] k_new:x[n_layers,B,H,hd] "
                            "v_new:x[n_layers,B,H,hd] " + _STEP_CROSS + " L_cap_cross:int "
                            "out_cross:f32[n_layers,B,H,hd] " + _TAIL + " " + _WS,
    "dec_attn_step_noalloc": "q_self:x[n_layers,B,H,hd] k_self:x[n_layers,B,H,L_cap_self,hd] "
                             "v_self:x[n_layers,B,H,L_cap_self,hd] len:i32[B] L_cap_self:int "
                             "out_self:f32[n_layers,B,H,hd] " + _STEP_CROSS +
                             " L_cap_cross:int out_cross:f32[n_layers,B,H,hd] " + _TAIL +
                             " scale:float stream:stream?",
    "dec_attn_step_ex": "q_self:x[n_layers,B,H,hd] k_self:x[n_layers,B,H,L_cap_self,hd] "
                        "v_self:x[n_layers,B,H,L_cap_self,hd] len:i32[B] L_cap_self:int "
                        "out_self:o[n_layers,B,H,hd] " + _STEP_CROSS +
                        " cross_mask:u32[B,mask_words] mask_words:int L_cap_cross:int "
                        "out_cross:o[n_layers,B,H,hd] " + _TAIL + " out_dtype:int " + _WS,
    "dec_attn_self_paged": "q:x[n_layers,B,H,hd] k_pool:x[n_layers,n_blocks,H,block_size,hd] "
                           "v_pool:x[n_layers,n_blocks,H,block_size,hd] "
                           "block_table:i32[B,max_blocks] len:i32[B] "
                           "out:f32[n_layers,B,H,hd] n_layers:int B:int H:int hd:int "
                           "block_size:int n_blocks:int max_blocks:int dtype:int " + _WS,
    "dec_attn_step_paged": _PAGED_SELF + " out_self:f32[n_layers,B,H,hd] " + _STEP_CROSS +
                           " L_cap_cross:int out_cross:f32[n_layers,B,H,hd] " + _TAIL + " "
                           + _WS,
    "dec_attn_step_paged_ex": _PAGED_SELF + " out_self:o[n_layers,B,H,hd] " + _STEP_CROSS +
                              " cross_mask:u32[B,mask_words] mask_words:int L_cap_cross:int "
                              "out_cross:o[n_layers,B,H,hd] " + _TAIL + " out_dtype:int "
                              + _WS,
    "dec_sample_topk": "logits:f32[B,n_cb,V_stride] B:int n_cb:int V_valid:int V_stride:int "
                       "temperature:f32[B] top_k:int uniforms:f32[B,n_cb] step:i32[B] "
                       "fill_token:i32 " + _SAMPLE_OUT,
    "dec_sample_topk_philox": "logits:f32[B,n_cb,V_stride] B:int n_cb:int V_valid:int "
                              "V_stride:int temperature:f32[B] top_k:int seed:u64 "
                              "step:i32[B] fill_token:i32 " + _SAMPLE_OUT,
    "dec_sample_topk_ex": "logits:l[B,n_cb,V_stride] logits_dtype:int B:int n_cb:int "
                          "V_valid:int V_stride:int temperature:f32[B] top_k:int "
                          "uniforms:f32[B,n_cb] seed:u64 step:i32[B] fill_token:i32 "
                          + _SAMPLE_OUT,
    "dec_sample_topk_advance": "logits:l[B,n_cb,V_stride] logits_dtype:int B:int n_cb:int "
                               "V_valid:int V_stride:int temperature:f32[B] top_k:int "
                               "uniforms:f32[B,n_cb] seed:u64 step:i32[B,n_cb] len:i32[B] "
                               "fill_token:i32 " + _SAMPLE_OUT,
    "dec_kv_append": "k_new:x[n_layers,B,H,hd] v_new:x[n_layers,B,H,hd] "
                     "k_cache:x[n_layers,B,H,L_cap,hd] v_cache:x[n_layers,B,H,L_cap,hd] "
                     "len:i32[B] n_layers:int B:int H:int L_cap:int hd:int dtype:int "
                     "stream:stream?",
    "dec_lm_head": "h:bf16[B,D] W:bf16[n_cb,V_stride,D] logits:f32[B,n_cb,V_stride] B:int "
                   "D:int n_cb:int V_valid:int V_stride:int stream:stream?",
    "dec_embed_sum": "tokens:i32[B,n_cb] E:bf16[n_cb,V_emb,D] x:f32[B,D] B:int n_cb:int "
                     "V_emb:int D:int stream:stream?",
    "dec_step_advance": "len:i32[B] step:i32[B] B:int stream:stream?",
    "dec_philox_uniforms": "seed:u64 step0:int n_steps:int B:int n_cb:int "
                           "out:f32[n_steps,B,n_cb] stream:stream?",
    "dec_probe_read": "buf:bytes[bytes] bytes:size sink:u32[1] stream:stream?",
    "dec_probe_empty": "stream:stream?",
    "dec_probe_clock": "clocks:i64[16] stream:stream?",
    "dec_graph_begin": "stream:stream",
    "dec_graph_launch": "exec_handle:int stream:stream?",
}

_SCALAR_C = {"int": ctypes.c_int, "i32": ctypes.c_int32, "u64": ctypes.c_uint64,
             "float": ctypes.c_float, "size": ctypes.c_size_t, "stream": ctypes.c_void_p}


class _Param:
    __slots__ = ("name", "kind", "dims", "optional")

    def __init__(self, text):
        self.name, kind = text.split(":")
        self.optional = kind.endswith("?")
        kind = kind.rstrip("?")
        self.dims = None
        if "[" in kind:
            kind, dims = kind[:-1].split("[")
            self.dims = tuple(int(d) if d.isdigit() else d for d in dims.split(","))
        self.kind = kind

    @property
    def ctype(self):
        if self.dims is not None or self.name == "exec_handle":
            return ctypes.c_void_p
        return _SCALAR_C[self.kind]


def _parse(spec):
    params = [_Param(t) for t in spec.split()]
    names = {p.name for p in params}
    for p in params:
        for d in p.dims or ():
            assert isinstance(d, int) or d in names, (p.name, d)
    return params


_DECL = {name: _parse(spec) for name, spec in _API.items()}


def _torch_dtypes():
    import torch
    u32 = (torch.int32,) + ((torch.uint32,) if hasattr(torch, "uint32") else ())
    u64 = (torch.int64,) + ((torch.uint64,) if hasattr(torch, "uint64") else ())
    return {"bf16": (torch.bfloat16,), "f32": (torch.float32,), "i32": (torch.int32,),
            "u32": u32, "i64": u64, DEC_BF16: (torch.bfloat16,), DEC_F32: (torch.float32,)}


_DTYPES = _torch_dtypes()
_CODE_ARG = {"x": "dtype", "o": "out_dtype", "l": "logits_dtype"}


def _fail(fn, status, what):
    raise DecError(status, f"{fn}: {what}")


def _buffer(fn, p, value, ints):
    """The pointer for buffer parameter ``p``; checks a tensor's element type, count and
    layout against the declaration (its device is checked with the call's others)."""
    if value is None:
        return None
    if isinstance(value, int):
        return value or None
    if not hasattr(value, "data_ptr"):
        _fail(fn, DEC_E_UNSUPPORTED, f"{p.name}: {type(value).__name__} is not a device "
                                     "tensor (host arrays cannot be passed)")
    factors = [d if isinstance(d, int) else ints[d] for d in p.dims]
    count = math.prod(factors)
    if p.kind == "bytes":
        if count > 0 and value.numel() * value.element_size() < count:
            _fail(fn, DEC_E_SHAPE, f"{p.name} holds {value.numel() * value.element_size()} "
                                   f"bytes, fewer than {count}")
    else:
        code = ints.get(_CODE_ARG.get(p.kind), p.kind)
        allowed = _DTYPES.get(code)
        if allowed is not None and value.dtype not in allowed:
            _fail(fn, DEC_E_DTYPE, f"{p.name} is {value.dtype}, expected "
                                   f"{' or '.join(str(a) for a in allowed)}")
        if min(factors, default=1) > 0 and value.numel() != count:
            shape = ", ".join(f"{d}={ints[d]}" if isinstance(d, str) else str(d)
                              for d in p.dims)
            _fail(fn, DEC_E_SHAPE, f"{p.name} holds {value.numel()} elements, its shape "
                                   f"[{shape}] has {count}")
    if not value.is_contiguous():
        _fail(fn, DEC_E_SHAPE, f"{p.name} is not contiguous (the layouts are row-major)")
    return value.data_ptr() or None


def _device(fn, tensors):
    """The one GPU that every tensor argument of the call lives on (None if none)."""
    device = None
    for name, t in tensors:
        if t.device.type != "cuda":
            _fail(fn, DEC_E_UNSUPPORTED, f"{name} is on {t.device}, not on a GPU")
        if device is None:
            device = t.device
        elif t.device != device:
            _fail(fn, DEC_E_UNSUPPORTED, f"{name} is on {t.device}, other tensors on {device}")
    return device


def _stream(s, device=None):
    import torch
    if s is None:
        if not torch.cuda.is_available():
            return None
        if device is not None and device.index != torch.cuda.current_device():
            raise DecError(DEC_E_UNSUPPORTED, f"tensors on {device} but the current device "
                                              f"is cuda:{torch.cuda.current_device()}")
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(s, int):
        return s or None
    if device is not None and s.device != device:
        raise DecError(DEC_E_UNSUPPORTED, f"stream on {s.device}, tensors on {device}")
    return s.cuda_stream or None


def _check(status):
    if status != DEC_OK:
        msg = _lib.dec_strerror(status).decode()
        if status == DEC_E_HIP:
            msg += f" (hipError_t {_lib.dec_last_hip_error()})"
        raise DecError(status, msg)


def _entry(name, params):
    cfn = getattr(_lib, name)
    cfn.restype = ctypes.c_int
    cfn.argtypes = [p.ctype for p in params]
    scalars = [p.name for p in params if p.dims is None and p.kind != "stream"]

    def call(*args, **kwargs):
        bound = call.__signature__.bind(*args, **kwargs)
        bound.apply_defaults()
        a = bound.arguments
        ints = {n: a[n] for n in scalars}
        c_args = [_buffer(name, p, a[p.name], ints) if p.dims is not None else a[p.name]
                  for p in params]
        device = _device(name, [(p.name, a[p.name]) for p in params
                                if p.dims is not None and hasattr(a[p.name], "data_ptr")])
        for i, p in enumerate(params):
            if p.kind == "stream":
                c_args[i] = _stream(c_args[i], device)
        _check(cfn(*c_args))

    call.__name__ = call.__qualname__ = name
    call.__signature__ = inspect.Signature(
        [inspect.Parameter(p.name, inspect.Parameter.POSITIONAL_OR_KEYWORD,
                           default=None if p.optional else inspect.Parameter.empty)
         for p in params])
    call.__doc__ = f"{name}({', '.join(p.name for p in params)}): include/decstep.h."
    return call


for _name, _params in _DECL.items():
    globals()[_name] = _entry(_name, _params)


# ---------------------------------------------------------------------------------
# Entry points with results other than a status, host-only helpers and test access.
# ---------------------------------------------------------------------------------
class Tuning(ctypes.Structure):
    """dec_tuning: launch-policy overrides of the calling thread (all 0: the defaults)."""
    _fields_ = [(n, ctypes.c_int) for n in (
        "attn_chunk_keys", "attn_schedule", "attn_blocks", "attn_no_halves",
        "attn_no_records", "head_kernel", "head_mfma_cfg")]


_OTHER = {
    "dec_attn_chunk_keys": (ctypes.c_int, []),
    "dec_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int] * 6),
    "dec_graph_end": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]),
    "dec_graph_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "dec_tuning_set": (ctypes.c_int, [ctypes.POINTER(Tuning)]),
    "dec_tuning_get": (ctypes.c_int, [ctypes.POINTER(Tuning)]),
    "dec_last_hip_error": (ctypes.c_int, []),
    "dec_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "dec_order_keys_host": (None, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]),
}
for _name, (_res, _args) in _OTHER.items():
    getattr(_lib, _name).restype = _res
    getattr(_lib, _name).argtypes = _args


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


def dec_graph_end(stream):
    """Ends capture on ``stream``; returns the executable graph handle (an int)."""
    ex = ctypes.c_void_p()
    _check(_lib.dec_graph_end(_stream(stream), ctypes.byref(ex)))
    return ex.value


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
    """x: float32 host array, keys: uint32 host array (numpy), n elements; HOST memory."""
    import numpy as np
    if not (isinstance(x, np.ndarray) and x.dtype == np.float32 and x.flags.c_contiguous
            and isinstance(keys, np.ndarray) and keys.dtype == np.uint32
            and keys.flags.c_contiguous and keys.flags.writeable):
        raise DecError(DEC_E_DTYPE, "dec_order_keys_host: contiguous float32 x and writable "
                                    "uint32 keys (numpy) are required")
    if not 0 <= n <= min(x.size, keys.size):
        raise DecError(DEC_E_SHAPE, f"dec_order_keys_host: n = {n} exceeds the arrays")
    _lib.dec_order_keys_host(x.ctypes.data, keys.ctypes.data, n)


def raw_status(name, *args):
    """Call a dec_* entry point with pre-marshalled arguments (integers as addresses,
    None as NULL); returns the status code without raising.  Tests use it to reach the
    library's own error paths past the binding's checks."""
    return getattr(_lib, name)(*args)
