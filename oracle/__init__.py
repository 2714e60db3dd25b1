"""Python handle on the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE. Only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with
the GPU library and never imports it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

F32 = 0
Q8_0 = 1
Q4_0 = 2


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc: -O2, no fast-math, no fp contraction."""
    src = os.path.join(_HERE, "oracle.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None
_vp = ctypes.c_void_p


def bind(path: str):
    """Load an oracle shared library at path and declare its signatures."""
    lib = ctypes.CDLL(path)
    sig = {
        "or_open": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(_vp)]),
        "or_close": (None, [_vp]),
        "or_reset_kv": (None, [_vp]),
        "or_key_cache": (_vp, [_vp]),
        "or_value_cache": (_vp, [_vp]),
        "or_logits": (_vp, [_vp]),
        "or_residual": (_vp, [_vp]),
        "or_attn_out": (_vp, [_vp]),
        "or_set_threads": (None, [ctypes.c_int]),
        "or_threads": (ctypes.c_int, []),
        "or_quantize": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int, _vp, _vp]),
        "or_group_dots": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, ctypes.c_int, _vp]),
        "or_rope_freqs": (None, [ctypes.c_int64, _vp]),
        "or_rope": (None, [_vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int]),
        "or_argmax": (ctypes.c_int, [_vp, ctypes.c_int64]),
        "or_quantize_q40": (ctypes.c_int, [_vp, ctypes.c_int64, _vp, _vp]),
        "or_group_dots_q40": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, _vp]),
        "or_matvec_q40": (ctypes.c_int, [_vp, _vp, _vp, ctypes.c_int64, ctypes.c_int64, _vp]),
        "or_splitmix64": (ctypes.c_uint64, [ctypes.c_uint64, ctypes.c_uint64]),
        "or_uniform": (ctypes.c_double, [ctypes.c_uint64, ctypes.c_uint64]),
        "or_sample_score": (ctypes.c_float, [ctypes.c_float, ctypes.c_double, ctypes.c_uint64,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]),
        "or_sample": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_double, ctypes.c_uint64,
                                     ctypes.c_int64]),
        "or_trace_layer": (None, [_vp, ctypes.c_int]),
        "or_trace_codes": (_vp, [_vp, ctypes.c_int]),
        "or_trace_scales": (_vp, [_vp, ctypes.c_int]),
        "or_trace_input": (_vp, [_vp, ctypes.c_int]),
        "or_trace_codes_at": (_vp, [_vp, ctypes.c_int, ctypes.c_int]),
        "or_trace_scales_at": (_vp, [_vp, ctypes.c_int, ctypes.c_int]),
        "or_trace_input_at": (_vp, [_vp, ctypes.c_int, ctypes.c_int]),
        "or_forward": (ctypes.c_int, [_vp, ctypes.c_int, ctypes.c_int]),
        "or_matvec_f32": (ctypes.c_int, [_vp, _vp, ctypes.c_int64, ctypes.c_int64, _vp]),
        "or_matvec_q80": (ctypes.c_int, [_vp, _vp, _vp, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int, _vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = bind(_SO)
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_vp)


def set_threads(n: int) -> None:
    _load().or_set_threads(n)


def threads() -> int:
    return int(_load().or_threads())


def quantize(x: np.ndarray, gs: int = 64):
    """Q8_0 quantise an fp32 vector: (codes int8[n], scales fp32[n/gs])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.empty(x.size, dtype=np.int8)
    s = np.empty(x.size // gs if gs > 0 else 0, dtype=np.float32)
    rc = _load().or_quantize(_ptr(x), x.size, gs, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("or_quantize: invalid size/group")
    return q, s


def group_dots(wq: np.ndarray, xq: np.ndarray, gs: int = 64) -> np.ndarray:
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    out = np.empty(wq.size // gs, dtype=np.int32)
    rc = _load().or_group_dots(_ptr(wq), _ptr(xq), wq.size, gs, _ptr(out))
    if rc != 0:
        raise ValueError("or_group_dots: invalid size/group")
    return out


def matvec_f32(W: np.ndarray, x: np.ndarray) -> np.ndarray:
    """out = W x for fp32 W [rows][cols] (fp64 dot, stored fp32)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = W.shape
    out = np.empty(rows, dtype=np.float32)
    if _load().or_matvec_f32(_ptr(W), _ptr(x), rows, cols, _ptr(out)) != 0:
        raise ValueError("or_matvec_f32")
    return out


def matvec_q80(Q: np.ndarray, S: np.ndarray, x: np.ndarray, gs: int = 64) -> np.ndarray:
    """out = W x for Q8_0 W (codes [rows][cols], scales [rows][cols/gs]); x
    (fp32) is quantised first."""
    Q = np.ascontiguousarray(Q, dtype=np.int8)
    S = np.ascontiguousarray(S, dtype=np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = Q.shape
    out = np.empty(rows, dtype=np.float32)
    if _load().or_matvec_q80(_ptr(Q), _ptr(S), _ptr(x), rows, cols, gs, _ptr(out)) != 0:
        raise ValueError("or_matvec_q80")
    return out


def rope_freqs(hs: int) -> np.ndarray:
    out = np.empty(hs // 2, dtype=np.float32)
    _load().or_rope_freqs(hs, _ptr(out))
    return out


def rope(vec: np.ndarray, nheads: int, hs: int, pos: int) -> np.ndarray:
    v = np.array(vec, dtype=np.float32, copy=True)
    _load().or_rope(_ptr(v), nheads, hs, pos)
    return v


def argmax(v: np.ndarray) -> int:
    v = np.ascontiguousarray(v, dtype=np.float32)
    return int(_load().or_argmax(_ptr(v), v.size))


def quantize_q40(x: np.ndarray):
    """4-bit group quantisation (groups of 32): (packed codes uint8[n/2], scales[n/32])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.empty(x.size // 2, np.uint8)
    s = np.empty(max(x.size // 32, 1), np.float32)
    if _load().or_quantize_q40(_ptr(x), x.size, _ptr(q), _ptr(s)) != 0:
        raise ValueError("quantize_q40: n must be a multiple of 32")
    return q, s[:x.size // 32]


def group_dots_q40(wq: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """int32 dots of packed 4-bit weight groups with int8 input groups."""
    wq = np.ascontiguousarray(wq, np.uint8)
    xq = np.ascontiguousarray(xq, np.int8)
    out = np.empty(xq.size // 32, np.int32)
    if _load().or_group_dots_q40(_ptr(wq), _ptr(xq), xq.size, _ptr(out)) != 0:
        raise ValueError("group_dots_q40: cols must be a multiple of 32")
    return out


def matvec_q40(Q: np.ndarray, S: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Q4_0 matvec: packed codes [rows][cols/2], scales [rows][cols/32]."""
    Q = np.ascontiguousarray(Q, np.uint8)
    S = np.ascontiguousarray(S, np.float32)
    x = np.ascontiguousarray(x, np.float32)
    rows = Q.shape[0]
    out = np.empty(rows, np.float32)
    if _load().or_matvec_q40(_ptr(Q), _ptr(S), _ptr(x), rows, x.size, _ptr(out)) != 0:
        raise ValueError("matvec_q40: bad shape")
    return out


def splitmix64(seed: int, k: int) -> int:
    """Output k of the splitmix64 stream seeded with seed."""
    return int(_load().or_splitmix64(seed & (2**64 - 1), k & (2**64 - 1)))


def uniform(seed: int, k: int) -> float:
    """Draw k as a uniform on (0, 1)."""
    return float(_load().or_uniform(seed & (2**64 - 1), k & (2**64 - 1)))


def sample_scores(logits: np.ndarray, temperature: float, seed: int, pos: int) -> np.ndarray:
    """fp32 Gumbel-max scores logit_i / T + g_i of every token (test helper)."""
    f = _load().or_sample_score
    n = logits.size
    return np.array([f(float(logits[i]), temperature, seed & (2**64 - 1), pos, n, i)
                     for i in range(n)], np.float32)


def sample(logits: np.ndarray, temperature: float, seed: int, pos: int) -> int:
    """Token drawn from softmax(logits / temperature) at position pos
    (temperature 0: argmax)."""
    v = np.ascontiguousarray(logits, dtype=np.float32)
    return int(_load().or_sample(_ptr(v), v.size, float(temperature), seed & (2**64 - 1), int(pos)))


class Model:
    """The oracle over a weight blob (numpy uint8, kept alive here)."""

    def __init__(self, blob: np.ndarray, dtype: int, gs: int | None = None):
        if gs is None:
            gs = 32 if dtype == Q4_0 else 64
        self._blob = blob
        h = ctypes.c_void_p()
        rc = _load().or_open(_ptr(blob), blob.size, dtype, gs, ctypes.byref(h))
        if rc != 0:
            raise ValueError(f"or_open failed: {rc}")
        self._h = h
        hdr = np.frombuffer(blob[:28].tobytes(), dtype=np.int32)
        (self.dim, self.hidden_dim, self.n_layers, self.n_heads, self.n_kv_heads,
         vs, self.seq_len) = (int(v) for v in hdr)
        self.vocab = abs(vs)
        self.head_size = self.dim // self.n_heads
        self.kv_dim = self.n_kv_heads * self.head_size
        self.dtype = dtype
        self.gs = gs

    def close(self):
        if self._h:
            _load().or_close(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _view(self, addr, n, dt):
        buf = (ctypes.c_byte * (n * np.dtype(dt).itemsize)).from_address(addr)
        return np.frombuffer(buf, dtype=dt)

    def forward(self, token: int, pos: int) -> np.ndarray:
        rc = _load().or_forward(self._h, int(token), int(pos))
        if rc != 0:
            raise ValueError(f"or_forward failed: {rc}")
        return self._view(_load().or_logits(self._h), self.vocab, np.float32).copy()

    def reset_kv(self):
        _load().or_reset_kv(self._h)

    def key_cache(self) -> np.ndarray:
        n = self.n_layers * self.seq_len * self.kv_dim
        return self._view(_load().or_key_cache(self._h), n, np.float32).reshape(
            self.n_layers, self.seq_len, self.kv_dim)

    def value_cache(self) -> np.ndarray:
        n = self.n_layers * self.seq_len * self.kv_dim
        return self._view(_load().or_value_cache(self._h), n, np.float32).reshape(
            self.n_layers, self.seq_len, self.kv_dim)

    def residual(self) -> np.ndarray:
        return self._view(_load().or_residual(self._h), self.dim, np.float32).copy()

    def attn_out(self) -> np.ndarray:
        """The last layer's attention output of the last forward."""
        return self._view(_load().or_attn_out(self._h), self.dim, np.float32).copy()

    def trace_layer(self, layer: int):
        """Record one layer's quantised matvec inputs on the next forwards
        (-2: every layer, -1: stop)."""
        _load().or_trace_layer(self._h, layer)

    def trace_at(self, layer: int, slot: int):
        """(codes, scales, fp32 input) of `slot` of `layer` recorded while
        every layer is traced (trace_layer(-2))."""
        n = self.hidden_dim if slot == 3 else self.dim
        lib = _load()
        q = self._view(lib.or_trace_codes_at(self._h, layer, slot), n, np.int8).copy()
        s = self._view(lib.or_trace_scales_at(self._h, layer, slot), n // self.gs, np.float32).copy()
        f = self._view(lib.or_trace_input_at(self._h, layer, slot), n, np.float32).copy()
        return q, s, f

    def trace(self, slot: int):
        """(codes, scales, fp32 input) of the traced layer's matvec input `slot`."""
        n = self.hidden_dim if slot == 3 else self.dim
        lib = _load()
        q = self._view(lib.or_trace_codes(self._h, slot), n, np.int8).copy()
        s = self._view(lib.or_trace_scales(self._h, slot), n // self.gs, np.float32).copy()
        f = self._view(lib.or_trace_input(self._h, slot), n, np.float32).copy()
        return q, s, f


def trajectory(model: Model, forced: np.ndarray, n_steps: int, keep_logits: bool = True):
    """Greedy decode with forced prompt ids from pos 0.

    Returns (tokens fed at each pos, argmax at each pos, logits per pos or None).
    The token fed at pos p is forced[p] while p < len(forced), else the argmax
    of pos p-1.
    """
    fed = np.empty(n_steps, dtype=np.int32)
    am = np.empty(n_steps, dtype=np.int32)
    logits = np.empty((n_steps, model.vocab), dtype=np.float32) if keep_logits else None
    tok = int(forced[0])
    for p in range(n_steps):
        if p < len(forced):
            tok = int(forced[p])
        fed[p] = tok
        lg = model.forward(tok, p)
        am[p] = argmax(lg)
        if keep_logits:
            logits[p] = lg
        tok = int(am[p])
    return fed, am, logits
