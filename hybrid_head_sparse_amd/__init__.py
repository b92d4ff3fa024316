"""Python binding of liblychee.so, the gfx950 hybrid-head decode-attention step.

Same names as the C ABI in ``include/lychee.h``; this module only marshals
arguments (torch tensors give device pointers, ``torch.cuda.current_stream()``
gives the stream).  Every step of the computation runs in the HIP kernels of
the library; there is no fallback path, and importing the binding without a
built library raises.

Method (the long-form digest "LycheeDecode: Accelerating Long-Context LLM
Inference via Hybrid-Head Sparse Decoding", section 3.4): per layer,
retrieval KV heads attend to the whole cache (Eq. 1) and refresh their
critical-token set with argsTopK over the GQA-pooled score (Eq. 2); sparse
heads attend only to the inherited set (Eq. 3) and pass it on; layer 0 is all
retrieval.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# LYCHEE_LIB selects another build of the same library (the phase-timestamp
# build liblychee_trace.so, for hybrid_head_sparse_amd.timeline)
LIB_PATH = os.environ.get("LYCHEE_LIB") or os.path.join(_HERE, "liblychee.so")

LYCHEE_OK = 0
LYCHEE_ERR_INVALID_ARG = -1
LYCHEE_ERR_UNSUPPORTED = -2
LYCHEE_ERR_HIP = -3
LYCHEE_ERR_WORKSPACE = -4
LYCHEE_ERR_DEVICE_CHECK = -5
LYCHEE_F32 = 0
LYCHEE_BF16 = 1
SELECT_RULES = {"topk": 0, "ratio": 1, "threshold": 2, "topp": 3, "block": 4}   # LYCHEE_SELECT_*

EXPORTED = (
    "lychee_workspace_bytes", "lychee_create", "lychee_decode_layer", "lychee_decode_layer_select",
    "lychee_dense_decode_layer", "lychee_kv_append", "lychee_correction_attention",
    "lychee_validate_layer", "lychee_set_stream", "lychee_set_profile_events",
    "lychee_check_device_errors", "lychee_destroy", "lychee_status_str", "lychee_last_error",
    "lychee_decode_layer_static",
)


class LycheeError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("k_max", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load liblychee.so (build it with ``python -m hybrid_head_sparse_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m hybrid_head_sparse_amd.build` "
                          "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pd = ctypes.POINTER(Dims)
    sig = {
        "lychee_workspace_bytes": (u64, [pd]),
        "lychee_create": (i32, [pd, vp, u64, vp, ctypes.POINTER(vp)]),
        "lychee_decode_layer": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32]),
        "lychee_decode_layer_select": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, ctypes.c_double]),
        "lychee_dense_decode_layer": (i32, [vp, vp, vp, vp, vp, vp]),
        "lychee_kv_append": (i32, [vp, vp, vp, vp, vp, vp]),
        "lychee_correction_attention": (i32, [vp, vp, vp, vp, vp, i32, vp]),
        "lychee_validate_layer": (i32, [pd, vp, vp, vp, vp, vp, vp, vp, vp, i32]),
        "lychee_set_stream": (i32, [vp, vp]),
        "lychee_set_profile_events": (i32, [vp, vp, vp]),
        "lychee_check_device_errors": (i32, [vp]),
        "lychee_destroy": (None, [vp]),
        "lychee_status_str": (ctypes.c_char_p, [i32]),
        "lychee_last_error": (ctypes.c_char_p, []),
        "lychee_decode_layer_static": (i32, [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if hasattr(lib, "lychee_set_trace"):          # the phase-timestamp build
        lib.lychee_set_trace.restype = i32
        lib.lychee_set_trace.argtypes = [vp, vp, ctypes.c_uint32]
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != LYCHEE_OK:
        lib = load()
        raise LycheeError(status, where, f"{lib.lychee_status_str(status).decode()}: "
                                         f"{lib.lychee_last_error().decode()}")


def make_dims(batch, n_q_heads, n_kv_heads, head_dim, max_ctx, k_max, dtype) -> Dims:
    code = {"f32": LYCHEE_F32, "bf16": LYCHEE_BF16, LYCHEE_F32: LYCHEE_F32, LYCHEE_BF16: LYCHEE_BF16}[dtype]
    return Dims(batch, n_q_heads, n_kv_heads, head_dim, max_ctx, k_max, code)


def workspace_bytes(dims: Dims) -> int:
    n = load().lychee_workspace_bytes(ctypes.byref(dims))
    if n == 0:
        _check(LYCHEE_ERR_INVALID_ARG, "lychee_workspace_bytes")
    return int(n)


def validate_layer(dims: Dims, q, k_cache, v_cache, role_mask, S_in, S_out, out, n_ctx, k) -> int:
    """Pure host-side argument check; pointers are plain integers (or None)."""
    role = np.ascontiguousarray(np.asarray(role_mask, dtype=np.uint8))
    return int(load().lychee_validate_layer(ctypes.byref(dims), q, k_cache, v_cache,
                                            role.ctypes.data_as(ctypes.c_void_p), S_in, S_out, out, n_ctx, int(k)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def decode_layer_static(dims: Dims, q, k_cache, v_cache, role_mask, S_in, S_out, out, n_ctx, k, stream=None):
    """lychee_decode_layer_static: one hybrid layer without a handle or a
    workspace (the library's per-GPU scratch); tensors as for
    Handle.decode_layer, ``stream`` a torch stream (default: the current one)."""
    import torch
    role = np.ascontiguousarray(np.asarray(role_mask, dtype=np.uint8).reshape(-1))
    if role.size != dims.n_kv_heads:
        raise ValueError(f"role_mask has {role.size} entries, expected {dims.n_kv_heads}")
    st = stream if stream is not None else torch.cuda.current_stream()
    _check(load().lychee_decode_layer_static(ctypes.byref(dims), ctypes.c_void_p(st.cuda_stream), _ptr(q),
                                             _ptr(k_cache), _ptr(v_cache), role.ctypes.data_as(ctypes.c_void_p),
                                             _ptr(S_in), _ptr(S_out), _ptr(out), _ptr(n_ctx), int(k)),
           "lychee_decode_layer_static")


class Handle:
    """A library handle plus the device workspace it owns (a torch uint8 tensor).

    Tensor arguments must be contiguous CUDA tensors on the handle's device:
    q [B,Hq,d], k_cache/v_cache [B,Hkv,max_ctx,d] (float32 or bfloat16 as
    given by ``dtype``), S_in/S_out [B,Hkv,k] int32, out [B,Hq,d] float32,
    n_ctx [B] int32.  ``role_mask`` is a host sequence of Hkv flags.
    """

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, max_ctx, k_max, dtype="bf16",
                 device=None, stream=None):
        import torch
        self._torch = torch
        self.device = torch.device(device if device is not None else "cuda")
        self.dims = make_dims(batch, n_q_heads, n_kv_heads, head_dim, max_ctx, k_max, dtype)
        self.tdtype = torch.bfloat16 if self.dims.dtype == LYCHEE_BF16 else torch.float32
        nbytes = workspace_bytes(self.dims)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self._h = ctypes.c_void_p()
        s = self._stream_ptr(stream)
        _check(load().lychee_create(ctypes.byref(self.dims), ctypes.c_void_p(self.workspace.data_ptr()),
                                    nbytes, s, ctypes.byref(self._h)), "lychee_create")

    def _stream_ptr(self, stream):
        torch = self._torch
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        return ctypes.c_void_p(st.cuda_stream)

    def _check_tensor(self, t, name, shape, dtype):
        if t is None:
            raise ValueError(f"{name} is required")
        if t.device != self.device and not (t.device.type == "cuda" and self.device.index is None):
            raise ValueError(f"{name} is on {t.device}, expected {self.device}")
        if t.dtype != dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def _check_common(self, q, k_cache, v_cache, out, n_ctx):
        d = self.dims
        torch = self._torch
        self._check_tensor(q, "q", (d.batch, d.n_q_heads, d.head_dim), self.tdtype)
        kv = (d.batch, d.n_kv_heads, d.max_ctx, d.head_dim)
        self._check_tensor(k_cache, "k_cache", kv, self.tdtype)
        self._check_tensor(v_cache, "v_cache", kv, self.tdtype)
        self._check_tensor(out, "out", (d.batch, d.n_q_heads, d.head_dim), torch.float32)
        self._check_tensor(n_ctx, "n_ctx", (d.batch,), torch.int32)

    def set_stream(self, stream=None):
        _check(load().lychee_set_stream(self._h, self._stream_ptr(stream)), "lychee_set_stream")

    def decode_layer(self, q, k_cache, v_cache, role_mask, S_in, S_out, out, n_ctx, k, rule="topk", param=0.0):
        """One hybrid layer; enqueues on the handle's stream and returns at once.

        ``rule`` picks the retrieval heads' selection ("topk", "ratio" with
        theta = ``param``, "threshold" with tau = ``param``, "topp" with
        p = ``param``, "block" with the block size ``param``); anything but
        "topk" goes through lychee_decode_layer_select."""
        if rule not in SELECT_RULES:
            raise ValueError(f"unknown selection rule {rule!r}; expected one of {sorted(SELECT_RULES)}")
        d = self.dims
        torch = self._torch
        self._check_common(q, k_cache, v_cache, out, n_ctx)
        self._check_tensor(S_out, "S_out", (d.batch, d.n_kv_heads, k), torch.int32)
        if S_in is not None:
            self._check_tensor(S_in, "S_in", (d.batch, d.n_kv_heads, k), torch.int32)
        role = np.ascontiguousarray(np.asarray(role_mask, dtype=np.uint8).reshape(-1))
        if role.size != d.n_kv_heads:
            raise ValueError(f"role_mask has {role.size} entries, expected {d.n_kv_heads}")
        args = (self._h, _ptr(q), _ptr(k_cache), _ptr(v_cache), role.ctypes.data_as(ctypes.c_void_p), _ptr(S_in),
                _ptr(S_out), _ptr(out), _ptr(n_ctx), int(k))
        if rule == "topk":
            _check(load().lychee_decode_layer(*args), "lychee_decode_layer")
        else:
            _check(load().lychee_decode_layer_select(*args, SELECT_RULES[rule], float(param)),
                   "lychee_decode_layer_select")

    def dense_decode_layer(self, q, k_cache, v_cache, out, n_ctx):
        """Dense all-heads decode attention (the baseline)."""
        self._check_common(q, k_cache, v_cache, out, n_ctx)
        _check(load().lychee_dense_decode_layer(self._h, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                                _ptr(n_ctx)), "lychee_dense_decode_layer")

    def kv_append(self, k_new, v_new, k_cache, v_cache, n_ctx):
        """Append one token's K and V rows ([B, Hkv, d]) at position n_ctx[b]
        and grow n_ctx on the device."""
        d = self.dims
        torch = self._torch
        kv = (d.batch, d.n_kv_heads, d.max_ctx, d.head_dim)
        self._check_tensor(k_new, "k_new", (d.batch, d.n_kv_heads, d.head_dim), self.tdtype)
        self._check_tensor(v_new, "v_new", (d.batch, d.n_kv_heads, d.head_dim), self.tdtype)
        self._check_tensor(k_cache, "k_cache", kv, self.tdtype)
        self._check_tensor(v_cache, "v_cache", kv, self.tdtype)
        self._check_tensor(n_ctx, "n_ctx", (d.batch,), torch.int32)
        _check(load().lychee_kv_append(self._h, _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(n_ctx)), "lychee_kv_append")

    def correction_attention(self, q, k_cache, v_cache, n_ctx, out):
        """Cache Correction's attention: q [B, T, Hq, d] (bf16) for the last T
        positions, out [B, T, Hq, d] fp32."""
        d = self.dims
        torch = self._torch
        if q.dim() != 4:
            raise ValueError("q must be [B, T, Hq, d]")
        T = int(q.shape[1])
        kv = (d.batch, d.n_kv_heads, d.max_ctx, d.head_dim)
        self._check_tensor(q, "q", (d.batch, T, d.n_q_heads, d.head_dim), self.tdtype)
        self._check_tensor(k_cache, "k_cache", kv, self.tdtype)
        self._check_tensor(v_cache, "v_cache", kv, self.tdtype)
        self._check_tensor(n_ctx, "n_ctx", (d.batch,), torch.int32)
        self._check_tensor(out, "out", (d.batch, T, d.n_q_heads, d.head_dim), torch.float32)
        _check(load().lychee_correction_attention(self._h, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(n_ctx), T,
                                                  _ptr(out)), "lychee_correction_attention")

    def set_profile_events(self, start=None, stop=None):
        """Record torch.cuda.Event ``start``/``stop`` around each following attention kernel."""
        sp = None if start is None else ctypes.c_void_p(start.cuda_event)
        ep = None if stop is None else ctypes.c_void_p(stop.cuda_event)
        _check(load().lychee_set_profile_events(self._h, sp, ep), "lychee_set_profile_events")

    def set_trace(self, buffer=None, launch: int = 0):
        """Phase timestamps of the following attention launches into the
        uint64 tensor ``buffer`` (trace build only; None stops)."""
        lib = load()
        if not hasattr(lib, "lychee_set_trace"):
            raise RuntimeError("set_trace needs the trace build (LYCHEE_LIB=.../liblychee_trace.so)")
        _check(lib.lychee_set_trace(self._h, _ptr(buffer), int(launch)), "lychee_set_trace")

    def check_device_errors(self):
        _check(load().lychee_check_device_errors(self._h), "lychee_check_device_errors")

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            load().lychee_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
