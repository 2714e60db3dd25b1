"""Full-sequence, non-cached numpy reference of the Llama-2 decoder.

A second, independent implementation used only to pin the oracle. It runs all
T positions at once as matrix products with a causal mask (no KV cache, no
per-position loop in attention), in fp64, rounding to fp32 at the same points
where the model stores a tensor, so that its fp32 activations, and hence its
Q8_0 activation codes, match a correct cached decoder up to the last bit of a
stored value.

Same readings as the oracle: RMSNorm eps 1e-5 inside the root; RoPE on
interleaved pairs with freq_j = fp32(10000^(-2j/hs)) and an fp32 angle; score
scale 1/sqrt(hs); query head h reads kv head h // (n_heads/n_kv_heads);
SwiGLU silu(w1 x) * w3 x; Q8_0 activations quantised per group as the
gitcode porting guide's quantize listing (float max, float division by 127,
round half away from zero). Q4_0 models (dtype 2): 4-bit weight codes
unpacked from their 16-byte groups, inputs quantised to Q8_0 with groups of
32, the same exact integer group dots.
"""
from __future__ import annotations

import numpy as np

from blobview import view

f32 = np.float32
f64 = np.float64


def quantize_rows(x: np.ndarray, gs: int):
    """Q8_0 codes and scales of each row of x (fp32), group size gs."""
    x = np.ascontiguousarray(x, dtype=f32)
    T, n = x.shape
    xg = x.reshape(T, n // gs, gs)
    wmax = np.abs(xg).max(axis=2)                       # fp32 max, exact
    scale = (wmax / f32(127.0)).astype(f32)             # fp32 division, correctly rounded
    safe = np.where(scale == 0, f32(1.0), scale).astype(f32)
    r = (xg / safe[..., None]).astype(f32)              # fp32 quotient
    rd = r.astype(f64)
    q = np.sign(rd) * np.floor(np.abs(rd) + 0.5)        # half away from zero, exact in fp64
    q = np.where(scale[..., None] == 0, 0.0, q)
    return q.astype(np.int8).reshape(T, n), scale


def unpack_q4(P: np.ndarray) -> np.ndarray:
    """4-bit codes in [-8, 7] of packed groups (..., n/2) -> (..., n): byte b
    of a 16-byte group holds code b + 8 (low nibble) and code b + 16 + 8."""
    g = P.reshape(P.shape[:-1] + (P.shape[-1] // 16, 16)).astype(np.int16)
    codes = np.concatenate([(g & 15) - 8, (g >> 4) - 8], axis=-1)
    return codes.reshape(P.shape[:-1] + (P.shape[-1] * 2,)).astype(np.int8)


def matmul(xs: np.ndarray, w: dict, name: str, layer, dtype: int, gs: int):
    """rows of xs (T, cols) times the matrix name[layer]^T -> (T, rows) fp32."""
    if dtype == 0:
        W = w[name] if layer is None else w[name][layer]
        return (xs.astype(f64) @ W.astype(f64).T).astype(f32), None
    if dtype == 2:
        Q = unpack_q4(w[name + ".p"] if layer is None else w[name + ".p"][layer])
        gs = 32
    else:
        Q = w[name + ".q"] if layer is None else w[name + ".q"][layer]
    S = w[name + ".s"] if layer is None else w[name + ".s"][layer]
    rows, cols = Q.shape
    ng = cols // gs
    xq, xsc = quantize_rows(xs, gs)
    Qg = Q.reshape(rows, ng, gs).astype(np.int64)
    Xg = xq.reshape(-1, ng, gs).astype(np.int64)
    out = np.zeros((xs.shape[0], rows), dtype=f64)
    for g in range(ng):
        dots = Xg[:, g, :] @ Qg[:, g, :].T                 # (T, rows) exact integers
        out += dots.astype(f64) * S[:, g].astype(f64)[None, :] * xsc[:, g].astype(f64)[:, None]
    return out.astype(f32), (xq, xsc)


def rmsnorm(x: np.ndarray, g: np.ndarray) -> np.ndarray:
    xd = x.astype(f64)
    r = 1.0 / np.sqrt((xd * xd).mean(axis=1, keepdims=True) + 1e-5)
    return (g.astype(f64)[None, :] * (xd * r)).astype(f32)


def rope(x: np.ndarray, nheads: int, hs: int, positions: np.ndarray) -> np.ndarray:
    T = x.shape[0]
    j = np.arange(hs // 2)
    freq = np.array([f32(10000.0 ** (-(2.0 * jj) / hs)) for jj in j], dtype=f32)
    ang = (positions.astype(f32)[:, None] * freq[None, :]).astype(f32)  # fp32 product
    c = np.cos(ang.astype(f64)).astype(f32).astype(f64)
    s = np.sin(ang.astype(f64)).astype(f32).astype(f64)
    xv = x.reshape(T, nheads, hs // 2, 2).astype(f64)
    a, b = xv[..., 0], xv[..., 1]
    out = np.empty_like(xv)
    out[..., 0] = a * c[:, None, :] - b * s[:, None, :]
    out[..., 1] = a * s[:, None, :] + b * c[:, None, :]
    return out.reshape(T, nheads * hs).astype(f32)


def forward_all(blob: np.ndarray, dtype: int, tokens, gs: int = 64, trace_layer=None):
    """Logits (T, V) for tokens fed at positions 0..T-1, causal, no KV cache.

    With trace_layer set (Q8_0), also returns the quantised inputs of that
    layer's four matvecs, as (codes (T, n), scales (T, n/gs)) per slot.
    """
    w = view(blob, dtype, gs)
    d, h, L, nh, nkv, vs, S = w["hdr"]
    hs = d // nh
    kvd = nkv * hs
    kvmul = nh // nkv
    tokens = np.asarray(tokens, dtype=np.int64)
    T = tokens.size
    pos = np.arange(T)
    if dtype == 0:
        x = w["emb"][tokens].astype(f32)
    elif dtype == 2:
        q = unpack_q4(w["emb.p"][tokens]).astype(f64)
        s = np.repeat(w["emb.s"][tokens].astype(f64), 32, axis=1)
        x = (q * s).astype(f32)
    else:
        q = w["emb.q"][tokens].astype(f64)
        s = np.repeat(w["emb.s"][tokens].astype(f64), gs, axis=1)
        x = (q * s).astype(f32)
    traces = {}
    causal = np.tril(np.ones((T, T), dtype=bool))
    for l in range(L):
        xb = rmsnorm(x, w["rms_att"][l])
        qv, t0 = matmul(xb, w, "wq", l, dtype, gs)
        kv, _ = matmul(xb, w, "wk", l, dtype, gs)
        vv, _ = matmul(xb, w, "wv", l, dtype, gs)
        qv = rope(qv, nh, hs, pos)
        kv = rope(kv, nkv, hs, pos)
        o = np.empty((T, d), dtype=f32)
        for hd in range(nh):
            g = hd // kvmul
            Qh = qv[:, hd * hs:(hd + 1) * hs].astype(f64)
            Kh = kv[:, g * hs:(g + 1) * hs].astype(f64)
            Vh = vv[:, g * hs:(g + 1) * hs].astype(f64)
            sc = (Qh @ Kh.T) / np.sqrt(float(hs))
            sc = np.where(causal, sc, -np.inf)
            sc = sc - sc.max(axis=1, keepdims=True)
            e = np.exp(sc)
            a = e / e.sum(axis=1, keepdims=True)
            o[:, hd * hs:(hd + 1) * hs] = (a @ Vh).astype(f32)
        y, t1 = matmul(o, w, "wo", l, dtype, gs)
        x = (x.astype(f64) + y.astype(f64)).astype(f32)
        xb = rmsnorm(x, w["rms_ffn"][l])
        h1, t2 = matmul(xb, w, "w1", l, dtype, gs)
        h3, _ = matmul(xb, w, "w3", l, dtype, gs)
        z = h1.astype(f64)
        hb = (z / (1.0 + np.exp(-z)) * h3.astype(f64)).astype(f32)
        y, t3 = matmul(hb, w, "w2", l, dtype, gs)
        x = (x.astype(f64) + y.astype(f64)).astype(f32)
        if trace_layer == l:
            traces = {0: t0, 1: t1, 2: t2, 3: t3}
    xb = rmsnorm(x, w["rms_final"])
    logits, _ = matmul(xb, w, "wcls", None, dtype, gs)
    if trace_layer is not None:
        return logits, traces
    return logits
