"""Seeded synthetic inputs for the Llama-2 decode step.

This module builds weight blobs in the llama2.c layout and prompt token ids.
It holds none of the decode step's arithmetic: the CPU oracle and the GPU
library each parse and compute from the bytes it writes, with their own code.
The generator itself is C (``synth.c``), OpenMP-parallel, so a 27 GB fp32
7B-shape blob takes seconds.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")

F32 = 0
Q8_0 = 1
Q4_0 = 2  # 4-bit groups of 32 (gs is always 32)


@dataclass(frozen=True)
class Config:
    name: str
    dim: int
    hidden_dim: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    vocab_size: int  # negative: unshared classifier
    seq_len: int
    seed: int
    dtypes: tuple

    @property
    def head_size(self) -> int:
        return self.dim // self.n_heads

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_size

    @property
    def vocab(self) -> int:
        return abs(self.vocab_size)

    def header(self) -> tuple:
        return (self.dim, self.hidden_dim, self.n_layers, self.n_heads,
                self.n_kv_heads, self.vocab_size, self.seq_len)

    def replace(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


# The five workloads: shapes from the pages' model family (15M / 110M
# TinyStories models, Llama-2 7B and 70B), random weights, one seed each.
CONFIGS = {
    "tiny": Config("tiny", 64, 172, 5, 8, 4, 512, 512, 1, (F32,)),
    "15M": Config("15M", 288, 768, 6, 6, 6, 32000, 256, 2, (F32,)),
    "110M": Config("110M", 768, 2048, 12, 12, 12, 32000, 1024, 3, (F32, Q8_0)),
    "7B": Config("7B", 4096, 11008, 32, 32, 32, -32000, 4096, 4, (F32, Q8_0)),
    "70B": Config("70B", 8192, 28672, 80, 64, 8, -32000, 4096, 5, (Q8_0,)),
    # second full-size workload: the 13B shape (its per-tensor element counts
    # exceed 2^31 over the layers, the range where 32-bit offsets overflow)
    "13B": Config("13B", 5120, 13824, 40, 40, 40, -32000, 4096, 6, (F32, Q8_0)),
}

GS = 64


class _CCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("dim", "hidden_dim", "n_layers", "n_heads", "n_kv_heads",
                 "vocab_size", "seq_len")]


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (host code only)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        lib.synth_blob_bytes.restype = ctypes.c_int64
        lib.synth_blob_bytes.argtypes = [ctypes.POINTER(_CCfg), ctypes.c_int, ctypes.c_int]
        lib.synth_fill_blob.restype = ctypes.c_int
        lib.synth_fill_blob.argtypes = [ctypes.POINTER(_CCfg), ctypes.c_int, ctypes.c_int,
                                        ctypes.c_uint64, ctypes.c_void_p]
        lib.synth_prompt.restype = None
        lib.synth_prompt.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_void_p]
        lib.synth_normal_f32.restype = None
        lib.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64,
                                         ctypes.c_double, ctypes.c_void_p]
        _lib = lib
    return _lib


def _ccfg(cfg) -> _CCfg:
    h = cfg.header() if isinstance(cfg, Config) else tuple(cfg)
    return _CCfg(*h)


def blob_bytes(cfg, dtype: int, gs: int = GS) -> int:
    if dtype == Q4_0:
        gs = 32
    return int(_load().synth_blob_bytes(ctypes.byref(_ccfg(cfg)), dtype, gs))


def make_blob(cfg, dtype: int, seed: int | None = None, gs: int = GS) -> np.ndarray:
    """Return the blob as a uint8 numpy array (header + arrays)."""
    if seed is None:
        seed = cfg.seed
    if dtype == Q4_0:
        gs = 32
    n = blob_bytes(cfg, dtype, gs)
    if n < 0:
        raise ValueError("invalid config for blob")
    out = np.empty(n, dtype=np.uint8)
    rc = _load().synth_fill_blob(ctypes.byref(_ccfg(cfg)), dtype, gs, seed,
                                 out.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("invalid config for blob")
    return out


def prompt(seed: int, n: int, vocab: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_prompt(seed, n, vocab, out.ctypes.data_as(ctypes.c_void_p))
    return out


def normal_f32(seed: int, tid: int, n: int, sd: float = 1.0) -> np.ndarray:
    """n fp32 values, approximately N(0, sd) (Irwin-Hall(4) bell), seeded."""
    out = np.empty(n, dtype=np.float32)
    _load().synth_normal_f32(seed, tid, n, sd, out.ctypes.data_as(ctypes.c_void_p))
    return out


def trajectory_plan(cfg: Config, n_steps: int) -> tuple:
    """(forced prompt ids, total steps) for a workload.

    The 15M-shape run forces 16 uniform prompt ids (seed 1000 + config seed)
    at pos 0..15 and decodes greedily after; the others start from token 1.
    """
    if cfg.name == "15M":
        return prompt(1000 + cfg.seed, 16, cfg.vocab), n_steps
    return np.array([1], dtype=np.int32), n_steps
