"""Numpy views of a weight blob, parsed independently of the oracle and the
GPU library, for the brute-force reference and for building twin models.

Layout: seven int32 (dim, hidden_dim, n_layers, n_heads, n_kv_heads,
vocab_size, seq_len), then E, rms_att, wq, wk, wv, wo, rms_ffn, w1, w2, w3,
rms_final, freq_cis_real, freq_cis_imag, and wcls when vocab_size < 0. A
Q8_0 matrix is int8 codes[n] followed by fp32 scales[n/gs]; a Q4_0 matrix
(dtype 2) is packed 4-bit codes[n/2] followed by fp32 scales[n/32].
"""
from __future__ import annotations

import numpy as np

MATS = ("emb", "wq", "wk", "wv", "wo", "w1", "w2", "w3", "wcls")


def layout(hdr, dtype: int, gs: int = 64):
    d, h, L, nh, nkv, vs, S = hdr
    V = abs(vs)
    hs = d // nh
    kvd = nkv * hs
    parts = [("emb", (V, d)), ("rms_att", (L, d)), ("wq", (L, d, d)), ("wk", (L, kvd, d)),
             ("wv", (L, kvd, d)), ("wo", (L, d, d)), ("rms_ffn", (L, d)), ("w1", (L, h, d)),
             ("w2", (L, d, h)), ("w3", (L, h, d)), ("rms_final", (d,)),
             ("freq_re", (S, hs // 2)), ("freq_im", (S, hs // 2))]
    if vs < 0:
        parts.append(("wcls", (V, d)))
    out = []
    off = 28
    for name, shape in parts:
        n = int(np.prod(shape))
        if dtype == 1 and name in MATS:
            out.append((name, "q", off, shape))
            off += n
            sshape = shape[:-1] + (shape[-1] // gs,)
            out.append((name, "s", off, sshape))
            off += 4 * (n // gs)
        elif dtype == 2 and name in MATS:
            out.append((name, "p", off, shape[:-1] + (shape[-1] // 2,)))
            off += n // 2
            out.append((name, "s", off, shape[:-1] + (shape[-1] // 32,)))
            off += 4 * (n // 32)
        else:
            out.append((name, "f", off, shape))
            off += 4 * n
    return out, off


def view(blob: np.ndarray, dtype: int, gs: int = 64) -> dict:
    hdr = tuple(int(v) for v in np.frombuffer(blob[:28].tobytes(), dtype=np.int32))
    parts, total = layout(hdr, dtype, gs)
    assert total == blob.size, (total, blob.size)
    w = {"hdr": hdr}
    for name, kind, off, shape in parts:
        n = int(np.prod(shape))
        if kind == "q":
            w[name + ".q"] = blob[off:off + n].view(np.int8).reshape(shape)
        elif kind == "p":
            w[name + ".p"] = blob[off:off + n].reshape(shape)
        else:
            w[name + ("." + kind if kind == "s" else "")] = \
                blob[off:off + 4 * n].view(np.float32).reshape(shape)
    if hdr[5] > 0:
        for k in ("q", "p", "s"):
            if "emb." + k in w:
                w["wcls." + k] = w["emb." + k]
        if "emb" in w:
            w["wcls"] = w["emb"]
    return w


def assemble(hdr, dtype: int, arrays: dict, gs: int = 64) -> np.ndarray:
    """Write a blob from named arrays (same names as view())."""
    parts, total = layout(hdr, dtype, gs)
    blob = np.empty(total, dtype=np.uint8)
    blob[:28] = np.frombuffer(np.array(hdr, dtype=np.int32).tobytes(), dtype=np.uint8)
    for name, kind, off, shape in parts:
        key = name + ("." + kind if kind in ("q", "s") else "")
        a = arrays[key]
        raw = np.ascontiguousarray(a, dtype=np.int8 if kind == "q" else np.float32)
        assert raw.shape == tuple(shape), (key, raw.shape, shape)
        b = raw.view(np.uint8).reshape(-1)
        blob[off:off + b.size] = b
    return blob
