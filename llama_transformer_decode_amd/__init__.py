"""Python binding of libl2d.so, the MI355X single-token Llama-2 decode library.

Argument marshalling only: every step of the decode runs in the library's HIP
kernels. The library must have been built (``build.py``); importing works
without it, but every call raises if the shared object is missing, and there
is no CPU fallback. PyTorch is used only to hold device buffers and streams
for the entry points that take device pointers.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libl2d.so")

F32 = 0
Q8_0 = 1
Q4_0 = 2  # 4-bit weights in groups of 32 (group_size 32)

OK, EINVAL, EFORMAT, ENOMEM, EHIP = 0, -1, -2, -3, -4

_vp = ctypes.c_void_p


class L2DError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"l2d error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("dim", "hidden_dim", "n_layers", "n_heads", "n_kv_heads", "vocab_size",
                 "seq_len", "dtype", "group_size")] + [
        ("rope_theta", ctypes.c_double), ("norm_eps", ctypes.c_double)]


_WFIELDS = []
for _n in ("emb",):
    _WFIELDS += [(_n, _vp), (_n + "_s", _vp)]
_WFIELDS += [("rms_att", _vp)]
for _n in ("wq", "wk", "wv", "wo"):
    _WFIELDS += [(_n, _vp), (_n + "_s", _vp)]
_WFIELDS += [("rms_ffn", _vp)]
for _n in ("w1", "w2", "w3"):
    _WFIELDS += [(_n, _vp), (_n + "_s", _vp)]
_WFIELDS += [("rms_final", _vp), ("wcls", _vp), ("wcls_s", _vp)]


class Weights(ctypes.Structure):
    _fields_ = _WFIELDS


_lib = None


def lib():
    """The loaded shared library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "l2d_blob_parse": (ctypes.c_int, [_vp, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.POINTER(Config), ctypes.POINTER(Weights)]),
            "l2d_init": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(Weights), _vp,
                                        ctypes.POINTER(_vp)]),
            "l2d_forward": (_vp, [_vp, ctypes.c_int32, ctypes.c_int32]),
            "l2d_forward_greedy": (_vp, [_vp, ctypes.c_int32]),
            "l2d_prefill": (_vp, [_vp, _vp, ctypes.c_int32, ctypes.c_int32]),
            "l2d_profile_prefill": (ctypes.c_int, [_vp, _vp, ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.POINTER(ctypes.c_double)]),
            "l2d_sync": (ctypes.c_int, [_vp]),
            "l2d_last_token": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_int32)]),
            "l2d_read_logits": (ctypes.c_int, [_vp, _vp]),
            "l2d_quantize_q80": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int32, _vp, _vp, _vp]),
            "l2d_reset_kv": (ctypes.c_int, [_vp]),
            "l2d_free": (None, [_vp]),
            "l2d_last_error": (ctypes.c_char_p, [_vp]),
            "l2d_kv_cache": (ctypes.c_int, [_vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp)]),
            "l2d_gemv": (ctypes.c_int, [ctypes.c_int32, _vp, _vp, _vp, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int32, _vp, _vp, _vp]),
            "l2d_gemv_noalloc": (ctypes.c_int, [ctypes.c_int32, _vp, _vp, _vp, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.c_int32, _vp, _vp, _vp]),
            "l2d_gemv_noalloc_max_bytes": (ctypes.c_int64, []),
            "l2d_gemv_profile": (ctypes.c_int, [ctypes.c_int32, _vp, _vp, ctypes.c_int32, _vp,
                                                ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, _vp,
                                                ctypes.c_int32, ctypes.POINTER(ctypes.c_double), _vp]),
            "l2d_trace_layer": (ctypes.c_int, [_vp, ctypes.c_int32]),
            "l2d_trace_read": (ctypes.c_int, [_vp, ctypes.c_int32, _vp, _vp]),
            "l2d_use_graph": (ctypes.c_int, [_vp, ctypes.c_int32]),
            "l2d_prefill_combine": (ctypes.c_int, [_vp, ctypes.c_int32]),
            "l2d_use_persistent": (ctypes.c_int, [_vp, ctypes.c_int32]),
            "l2d_set_sampling": (ctypes.c_int, [_vp, ctypes.c_double, ctypes.c_uint64]),
            "l2d_persistent": (ctypes.c_int, [_vp]),
            "l2d_use_chain": (ctypes.c_int, [_vp, ctypes.c_int32]),
            "l2d_chained": (ctypes.c_int, [_vp]),
            "l2d_test_chain_fault": (ctypes.c_int, [_vp]),
            "l2d_stream": (_vp, [_vp]),
            "l2d_profile_step": (ctypes.c_int, [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.POINTER(ctypes.c_double)]),
            "l2d_stream_plan_check": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.c_int32, ctypes.c_char_p,
                                                     ctypes.c_int32]),
            "l2d_stream_shape": (ctypes.c_int, [_vp, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]),
            "l2d_stream_trace": (ctypes.c_int, [_vp, ctypes.c_int32, ctypes.c_int32, _vp, ctypes.c_int64,
                                                ctypes.POINTER(ctypes.c_int64)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


# every symbol include/l2d.h declares
EXPORTS = ("l2d_blob_parse", "l2d_init", "l2d_forward", "l2d_forward_greedy", "l2d_sync",
           "l2d_last_token", "l2d_read_logits", "l2d_quantize_q80", "l2d_reset_kv", "l2d_free",
           "l2d_last_error", "l2d_kv_cache", "l2d_gemv", "l2d_gemv_noalloc", "l2d_gemv_noalloc_max_bytes",
           "l2d_gemv_profile", "l2d_trace_layer", "l2d_trace_read",
           "l2d_use_graph", "l2d_stream", "l2d_profile_step", "l2d_use_persistent", "l2d_persistent",
           "l2d_set_sampling", "l2d_prefill", "l2d_prefill_combine", "l2d_profile_prefill", "l2d_stream_plan_check",
           "l2d_stream_trace", "l2d_stream_shape", "l2d_use_chain", "l2d_chained",
           "l2d_test_chain_fault")

KERNEL_CLASSES = ("qkv", "attn", "wo", "w13", "w2", "cls", "begin")
PREFILL_CLASSES = ("prep", "qkv", "attn", "wo", "w13", "w2", "start", "cls")


def last_error(ctx=None) -> str:
    m = lib().l2d_last_error(ctx)
    return m.decode() if m else ""


def _check(rc: int, ctx=None):
    if rc != OK:
        raise L2DError(rc, last_error(ctx))


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(_vp)


def blob_parse(blob: np.ndarray, dtype: int, group_size: int = 64):
    """Parse a host blob (uint8 numpy array): returns (Config, Weights)."""
    cfg = Config()
    w = Weights()
    _check(lib().l2d_blob_parse(_np_ptr(blob), blob.size, dtype, group_size,
                                ctypes.byref(cfg), ctypes.byref(w)))
    return cfg, w


def _stream_handle(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # a torch.cuda.Stream


class _DevArray:
    """A raw device pointer described through __cuda_array_interface__ so
    that torch.as_tensor can view it without copying."""

    def __init__(self, ptr: int, shape, typestr: str):
        self.__cuda_array_interface__ = {
            "shape": tuple(shape), "typestr": typestr, "data": (int(ptr), False),
            "version": 2, "strides": None}


def device_view(ptr: int, shape, dtype: str = "<f4"):
    """torch tensor viewing device memory at ptr (not owned)."""
    import torch
    return torch.as_tensor(_DevArray(ptr, shape, dtype), device="cuda")


class Context:
    """A decode context: device weights, KV cache and the captured step."""

    def __init__(self, blob: np.ndarray, dtype: int, group_size: int | None = None, stream=None):
        if group_size is None:
            group_size = 32 if dtype == Q4_0 else 64
        self.cfg, w = blob_parse(blob, dtype, group_size)
        h = _vp()
        _check(lib().l2d_init(ctypes.byref(self.cfg), ctypes.byref(w),
                              _stream_handle(stream), ctypes.byref(h)))
        self._h = h
        c = self.cfg
        self.dim, self.hidden_dim, self.n_layers = c.dim, c.hidden_dim, c.n_layers
        self.n_heads, self.n_kv_heads, self.seq_len = c.n_heads, c.n_kv_heads, c.seq_len
        self.vocab = abs(c.vocab_size)
        self.head_size = c.dim // c.n_heads
        self.kv_dim = c.n_kv_heads * self.head_size
        self.dtype = dtype
        self.group_size = group_size

    def close(self):
        if getattr(self, "_h", None):
            lib().l2d_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    def error(self) -> str:
        return last_error(self._h)

    def forward(self, token: int, pos: int) -> int:
        """Enqueue one step; returns the device address of the logits."""
        p = lib().l2d_forward(self._h, int(token), int(pos))
        if not p:
            raise L2DError(EINVAL, self.error())
        return p

    def forward_greedy(self, pos: int) -> int:
        p = lib().l2d_forward_greedy(self._h, int(pos))
        if not p:
            raise L2DError(EINVAL, self.error())
        return p

    def prefill(self, tokens, pos0: int = 0) -> int:
        """Batched prefill of the prompt tokens at pos0..; returns the device
        address of the last token's logits."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        p = lib().l2d_prefill(self._h, _np_ptr(t), int(t.size), int(pos0))
        if not p:
            raise L2DError(EINVAL, self.error())
        return p

    def prefill_profile(self, tokens, pos0: int = 0) -> dict:
        """Mean kernel seconds per class of one batched prefill."""
        t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        out = (ctypes.c_double * len(PREFILL_CLASSES))()
        _check(lib().l2d_profile_prefill(self._h, _np_ptr(t), int(t.size), int(pos0), out), self._h)
        return {k: out[i] for i, k in enumerate(PREFILL_CLASSES)}

    def sync(self):
        _check(lib().l2d_sync(self._h), self._h)

    def logits(self) -> np.ndarray:
        out = np.empty(self.vocab, dtype=np.float32)
        _check(lib().l2d_read_logits(self._h, _np_ptr(out)), self._h)
        return out

    def last_token(self) -> int:
        t = ctypes.c_int32()
        _check(lib().l2d_last_token(self._h, ctypes.byref(t)), self._h)
        return int(t.value)

    def reset_kv(self):
        _check(lib().l2d_reset_kv(self._h), self._h)

    def kv_cache(self):
        """(key_cache, value_cache) as torch views [n_layers, seq_len, kv_dim]."""
        k, v = _vp(), _vp()
        _check(lib().l2d_kv_cache(self._h, ctypes.byref(k), ctypes.byref(v)), self._h)
        shape = (self.n_layers, self.seq_len, self.kv_dim)
        return device_view(k.value, shape), device_view(v.value, shape)

    def stream_handle(self) -> int:
        return lib().l2d_stream(self._h)

    def kernel_profile(self, token: int, pos: int, reps: int = 3) -> dict:
        """Mean seconds per launch of each kernel class (HIP events)."""
        out = (ctypes.c_double * len(KERNEL_CLASSES))()
        _check(lib().l2d_profile_step(self._h, int(token), int(pos), int(reps), out), self._h)
        return {k: float(out[i]) for i, k in enumerate(KERNEL_CLASSES)}

    def prefill_combine(self, fp32: bool):
        """Q8_0 group combine of the prefill matmuls: fp64 (False, the
        default, bit-identical to token-by-token steps) or fp32 (True)."""
        _check(lib().l2d_prefill_combine(self._h, 1 if fp32 else 0), self._h)

    def use_graph(self, enable: bool):
        _check(lib().l2d_use_graph(self._h, 1 if enable else 0), self._h)

    def set_sampling(self, temperature: float, seed: int = 0):
        """Next-token selection: temperature 0 = argmax, > 0 = a draw from
        softmax(logits / temperature) with the given seed."""
        _check(lib().l2d_set_sampling(self._h, float(temperature), int(seed) & (2**64 - 1)), self._h)

    def use_persistent(self, enable: bool):
        """Run each step as the one persistent step kernel (True; Q8_0 with
        group size 64) or as the captured graph of per-phase kernels (False)."""
        _check(lib().l2d_use_persistent(self._h, 1 if enable else 0), self._h)

    def use_chain(self, enable: bool):
        """Chained launches (True: attention + output projection and w1/w3 +
        w2 in one launch each; Q8_0 with group size 64) or one launch per
        phase (False). Re-captures the step graph."""
        _check(lib().l2d_use_chain(self._h, 1 if enable else 0), self._h)

    def test_chain_fault(self):
        """Test hook: set the chained launches' error word from the host."""
        _check(lib().l2d_test_chain_fault(self._h), self._h)

    @property
    def chained(self) -> bool:
        r = lib().l2d_chained(self._h)
        _check(r if r < 0 else 0, self._h)
        return r == 1

    def stream_shape(self):
        """(workgroups, worker waves per workgroup) of the persistent step kernel."""
        g, w = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().l2d_stream_shape(self._h, ctypes.byref(g), ctypes.byref(w)), self._h)
        return g.value, w.value

    def stream_trace(self, token: int, pos: int, workgroups: int, workers: int):
        """One persistent-kernel step with clock stamps: (control [G][E],
        worker reports [G][W][phases]) in 100 MHz ticks."""
        ev = ctypes.c_int64()
        _check(lib().l2d_stream_trace(self._h, 0, 0, None, 0, ctypes.byref(ev)), self._h)
        E = ev.value
        NP = 4 * self.n_layers + 1
        n = workgroups * (E + workers * NP)
        buf = np.zeros(n, dtype=np.uint64)
        _check(lib().l2d_stream_trace(self._h, int(token), int(pos), _np_ptr(buf), n, ctypes.byref(ev)), self._h)
        ctl = buf[:workgroups * E].reshape(workgroups, E)
        wk = buf[workgroups * E:].reshape(workgroups, workers, NP)
        return ctl, wk

    @property
    def persistent(self) -> bool:
        r = lib().l2d_persistent(self._h)
        _check(r if r < 0 else 0, self._h)
        return r == 1

    def trace_layer(self, layer: int):
        _check(lib().l2d_trace_layer(self._h, int(layer)), self._h)

    def trace(self, slot: int):
        n = self.hidden_dim if slot == 3 else self.dim
        q = np.empty(n, dtype=np.int8)
        s = np.empty(n // self.group_size, dtype=np.float32)
        _check(lib().l2d_trace_read(self._h, slot, _np_ptr(q), _np_ptr(s)), self._h)
        return q, s


def stream_plan_check(header, nwg: int, group_size: int = 64) -> str:
    """Run the persistent step kernel's plan (every worker's weight stream,
    row ownership, attention ranges, LDS size) on the host for a launch of
    nwg workgroups; returns "ok" or raises L2DError naming the first problem.
    header: the seven blob-header fields. Host only: no device is touched."""
    cfg = Config(*header, 1, group_size, 10000.0, 1e-5)
    buf = ctypes.create_string_buffer(512)
    rc = lib().l2d_stream_plan_check(ctypes.byref(cfg), int(nwg), buf, 512)
    msg = buf.value.decode()
    if rc != OK:
        raise L2DError(rc, msg)
    return msg


def quantize_q80(x, gs: int = 64, stream=None):
    """Q8_0-quantise a 1-D fp32 torch CUDA tensor: (codes int8, scales fp32)."""
    import torch
    assert x.is_cuda and x.dtype == torch.float32 and x.is_contiguous()
    n = x.numel()
    q = torch.empty(n, dtype=torch.int8, device=x.device)
    s = torch.empty(max(n // gs, 1) if gs > 0 else 1, dtype=torch.float32, device=x.device)
    st = _stream_handle(stream if stream is not None else torch.cuda.current_stream())
    _check(lib().l2d_quantize_q80(x.data_ptr(), n, gs, q.data_ptr(), s.data_ptr(), st))
    return q, s[: n // gs] if gs > 0 else s


def gemv(dtype: int, W, W_s, x, rows: int, cols: int, gs: int = 64, group_dots=None, stream=None):
    """out = W x with the decode step's GEMV kernel (torch CUDA tensors)."""
    import torch
    out = torch.empty(rows, dtype=torch.float32, device=x.device)
    st = _stream_handle(stream if stream is not None else torch.cuda.current_stream())
    _check(lib().l2d_gemv(dtype, W.data_ptr(), W_s.data_ptr() if W_s is not None else None,
                          x.data_ptr(), rows, cols, gs, out.data_ptr(),
                          group_dots.data_ptr() if group_dots is not None else None, st))
    return out


def gemv_noalloc(dtype: int, W, W_s, x, out, rows: int, cols: int, gs: int = 64, group_dots=None, stream=None):
    """l2d_gemv_noalloc: out = W x into the caller's tensor `out`, with no
    device allocation by the library (torch CUDA tensors)."""
    import torch
    st = _stream_handle(stream if stream is not None else torch.cuda.current_stream())
    _check(lib().l2d_gemv_noalloc(dtype, W.data_ptr(), W_s.data_ptr() if W_s is not None else None,
                                  x.data_ptr(), rows, cols, gs, out.data_ptr(),
                                  group_dots.data_ptr() if group_dots is not None else None, st))
    return out


def gemv_noalloc_max_bytes() -> int:
    """Largest rows x cols of Q8_0 codes l2d_gemv_noalloc takes."""
    return int(lib().l2d_gemv_noalloc_max_bytes())


def gemv_profile(dtype: int, Ws, Ss, x, rows: int, cols: int, gs: int = 32, reps: int = 20, stream=None):
    """Mean kernel seconds of the matvec over reps launches cycling through
    the weight copies Ws (and scale copies Ss, or None for fp32); returns
    (seconds, output of the last launch)."""
    import torch
    out = torch.empty(rows, dtype=torch.float32, device=x.device)
    st = _stream_handle(stream if stream is not None else torch.cuda.current_stream())
    wp = (_vp * len(Ws))(*[w.data_ptr() for w in Ws])
    sp = (_vp * len(Ws))(*[s.data_ptr() for s in Ss]) if Ss is not None else None
    sec = ctypes.c_double(0.0)
    _check(lib().l2d_gemv_profile(dtype, wp, sp, len(Ws), x.data_ptr(), rows, cols, gs,
                                  out.data_ptr(), reps, ctypes.byref(sec), st))
    return sec.value, out
