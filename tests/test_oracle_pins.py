"""Pins of the CPU oracle to facts other than itself.

Each test checks the oracle against something the pages or the mathematics
fix: the quantize listing worked by hand and in exact rationals, closed forms
of RMSNorm / RoPE / softmax, the exact equivalence of GQA with repeated-head
MHA, the tied-classifier rule, and an independent full-sequence non-cached
fp64 recomputation of the whole decoder (tests/bruteforce.py).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from blobview import assemble, view
import bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# small shapes (oracle finishes in well under a second)
TINY = synth.CONFIGS["tiny"]
TINY_Q8 = synth.Config("tinyq8", 128, 256, 3, 4, 2, 320, 64, 11, (synth.Q8_0,))
TINY_Q8_UNSHARED = TINY_Q8.replace(name="tinyq8u", vocab_size=-320, seed=12)
TINY_Q4 = synth.Config("tinyq4", 128, 256, 3, 4, 2, 320, 64, 21, (synth.Q4_0,))
TINY_Q4_UNSHARED = TINY_Q4.replace(name="tinyq4u", vocab_size=-320, seed=22)


def _ulp(x):
    return np.spacing(np.abs(np.float32(x))).astype(np.float64)


# ------------------------------------------------------------- Q8_0 quantise

def test_quantize_handworked_golden():
    g = json.load(open(os.path.join(GOLDEN, "q80_handworked.json")))
    gs = g["gs"]
    x = np.zeros(gs * len(g["groups"]), dtype=np.float32)
    want_q = np.zeros_like(x, dtype=np.int8)
    want_s = np.zeros(len(g["groups"]), dtype=np.float32)
    for gi, grp in enumerate(g["groups"]):
        for k, v in grp["x"].items():
            x[gi * gs + int(k)] = v
        for k, v in grp["codes"].items():
            want_q[gi * gs + int(k)] = v
        want_s[gi] = grp["scale"]
    q, s = oracle.quantize(x, gs)
    np.testing.assert_array_equal(s, want_s)
    np.testing.assert_array_equal(q, want_q)


def _exact_quantize(xg):
    """Exact rational evaluation of the listing's steps for one group of
    fp32 values: fp32(wmax/127) and fp32(x/scale) are the correctly rounded
    quotients, then rounding half away from zero."""
    wmax = max(abs(float(v)) for v in xg)
    scale = _round_f32(Fraction(wmax) / 127)
    codes = []
    for v in xg:
        if scale == 0:
            codes.append(0)
            continue
        r = _round_f32(Fraction(float(v)) / Fraction(float(scale)))
        fr = Fraction(float(r))
        a = abs(fr)
        n = int(a)  # floor
        if a - n >= Fraction(1, 2):
            n += 1
        codes.append(n if fr >= 0 else -n)
    return codes, scale


def _round_f32(fr: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even)."""
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    lo = np.float32(float(a))  # float(a) is the nearest double; check neighbours exactly
    cands = [lo, np.nextafter(lo, np.float32(np.inf)), np.nextafter(lo, np.float32(0))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - a),
                                     int(np.frombuffer(np.float32(c).tobytes(), np.uint32)[0]) & 1))
    return np.float32(sign * best)


def test_quantize_exact_rational_bruteforce():
    rng = np.random.default_rng(7)
    gs = 64
    groups = [
        rng.standard_normal(gs).astype(np.float32),
        (rng.standard_normal(gs) * 1e-20).astype(np.float32),
        (rng.standard_normal(gs) * 3e4).astype(np.float32),
        rng.integers(-1000, 1000, gs).astype(np.float32) / np.float32(8),
        np.full(gs, 0.75, dtype=np.float32),
    ]
    x = np.concatenate(groups)
    q, s = oracle.quantize(x, gs)
    for gi, xg in enumerate(groups):
        codes, scale = _exact_quantize(xg)
        assert s[gi] == scale, (gi, s[gi], scale)
        np.testing.assert_array_equal(q[gi * gs:(gi + 1) * gs], np.array(codes, dtype=np.int8))


def test_quantize_invariants():
    rng = np.random.default_rng(3)
    gs = 64
    x = (rng.standard_normal(gs * 500) * rng.uniform(1e-3, 10, gs * 500)).astype(np.float32)
    q, s = oracle.quantize(x, gs)
    xg = x.reshape(-1, gs)
    qg = q.reshape(-1, gs).astype(np.int64)
    assert np.abs(qg).max() <= 127
    wmax = np.abs(xg).max(axis=1)
    np.testing.assert_array_equal(s, (wmax / np.float32(127)).astype(np.float32))
    # the element of largest magnitude maps to +-127
    arg = np.abs(xg).argmax(axis=1)
    np.testing.assert_array_equal(np.abs(qg[np.arange(len(arg)), arg]), 127)
    # dequantisation error within half a step (+ fp32 rounding slack)
    err = np.abs(xg.astype(np.float64) - qg * s[:, None].astype(np.float64))
    bound = s[:, None].astype(np.float64) * (0.5 + 1e-6) + _ulp(xg)
    assert (err <= bound).all()


def test_quantize_zero_group_and_bad_sizes():
    q, s = oracle.quantize(np.zeros(128, np.float32), 64)
    assert (q == 0).all() and (s == 0).all()
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros(100, np.float32), 64)


def test_quantize_is_not_half_to_even():
    # 2.5 must go to 3 (C round), numpy's rint gives 2
    x = np.zeros(64, np.float32)
    x[0], x[1], x[2] = 127.0, 2.5, -2.5
    q, _ = oracle.quantize(x, 64)
    assert q[1] == 3 and q[2] == -3


# ------------------------------------------------------------- group dots

def test_group_dots_closed_forms():
    gs = 64
    ones = np.ones(gs, np.int8)
    assert oracle.group_dots(ones, ones, gs)[0] == gs
    m = np.full(gs, 127, np.int8)
    assert oracle.group_dots(m, m, gs)[0] == 127 * 127 * gs
    assert oracle.group_dots(m, -m, gs)[0] == -127 * 127 * gs
    alt = np.array([1, -1] * (gs // 2), np.int8)
    assert oracle.group_dots(alt, ones, gs)[0] == 0
    ramp = (np.arange(gs) - 32).astype(np.int8)
    # sum_{k=-32}^{31} k^2 = 2*sum_{1}^{31} k^2 + 32^2
    assert oracle.group_dots(ramp, ramp, gs)[0] == 2 * (31 * 32 * 63 // 6) + 32 * 32
    # several groups are independent
    w = np.concatenate([ones, m, alt])
    x = np.concatenate([ones, m, ones])
    np.testing.assert_array_equal(oracle.group_dots(w, x, gs), [gs, 127 * 127 * gs, 0])


# ------------------------------------------------------------- RoPE closed forms

def test_rope_pos0_identity():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(8 * 16).astype(np.float32)
    np.testing.assert_array_equal(oracle.rope(v, 8, 16, 0), v)


def test_rope_unit_pair_gives_cos_sin():
    hs = 16
    freqs = oracle.rope_freqs(hs)
    for j in range(hs // 2):
        assert abs(float(freqs[j]) - 10000.0 ** (-2.0 * j / hs)) <= float(_ulp(freqs[j]))
    for pos in (1, 7, 300, 4095):
        v = np.zeros(hs, np.float32)
        v[0::2] = 1.0
        r = oracle.rope(v, 1, hs, pos)
        for j in range(hs // 2):
            ang = float(np.float32(np.float32(pos) * freqs[j]))
            # rotating (1, 0) gives exactly the fp32 cosine / sine of the fp32 angle
            assert r[2 * j] == np.float32(math.cos(ang))
            assert r[2 * j + 1] == np.float32(math.sin(ang))


def test_rope_preserves_pair_norms_and_relative_position():
    rng = np.random.default_rng(2)
    hs = 32
    q = rng.standard_normal(hs).astype(np.float32)
    k = rng.standard_normal(hs).astype(np.float32)
    for pos in (3, 100):
        r = oracle.rope(q, 1, hs, pos).astype(np.float64)
        n0 = q.astype(np.float64).reshape(-1, 2)
        n1 = r.reshape(-1, 2)
        np.testing.assert_allclose((n1 ** 2).sum(1), (n0 ** 2).sum(1), rtol=1e-6)
    # <R_m q, R_n k> depends on n - m only (small positions keep fp32 angles exact enough)
    d1 = float(np.dot(oracle.rope(q, 1, hs, 5).astype(np.float64), oracle.rope(k, 1, hs, 2)))
    d2 = float(np.dot(oracle.rope(q, 1, hs, 9).astype(np.float64), oracle.rope(k, 1, hs, 6)))
    assert abs(d1 - d2) < 1e-4
    # the rotation has the sign of a counter-clockwise turn: (1, 0) -> (cos, +sin)
    e = np.zeros(hs, np.float32)
    e[0] = 1.0
    assert oracle.rope(e, 1, hs, 1)[1] > 0


# ------------------------------------------------------------- argmax

def test_argmax_ties_lowest_index():
    v = np.array([0.5, 2.0, -1.0, 2.0, 2.0], np.float32)
    assert oracle.argmax(v) == 1
    assert oracle.argmax(np.zeros(7, np.float32)) == 0


# ------------------------------------------------------------- whole decoder

def _blob(cfg, dtype):
    return synth.make_blob(cfg, dtype)


def _traj(model, n):
    fed, am, lg = oracle.trajectory(model, np.array([1], np.int32), n)
    return fed, am, lg


@pytest.mark.parametrize("cfg,dtype,n", [
    (TINY, synth.F32, 64),
    (TINY_Q8, synth.Q8_0, 48),
    (TINY_Q8_UNSHARED, synth.Q8_0, 24),
    (TINY_Q4, synth.Q4_0, 40),
    (TINY_Q4_UNSHARED, synth.Q4_0, 24),
])
def test_oracle_matches_full_sequence_bruteforce(cfg, dtype, n):
    """Cached decode == non-cached causal recomputation at every position."""
    blob = _blob(cfg, dtype)
    m = oracle.Model(blob, dtype)
    fed, am, lg = _traj(m, n)
    ref = bruteforce.forward_all(blob, dtype, fed)
    np.testing.assert_allclose(lg, ref, rtol=1e-5, atol=2e-6 if dtype == 0 else 2e-5)
    np.testing.assert_array_equal(am, ref.argmax(axis=1))


def test_oracle_15m_shape_bruteforce_prefix():
    cfg = synth.CONFIGS["15M"]
    blob = _blob(cfg, synth.F32)
    m = oracle.Model(blob, synth.F32)
    forced, _ = synth.trajectory_plan(cfg, 8)
    fed, am, lg = oracle.trajectory(m, forced, 8)
    np.testing.assert_array_equal(fed, forced[:8])
    ref = bruteforce.forward_all(blob, synth.F32, fed)
    np.testing.assert_allclose(lg, ref, rtol=1e-5, atol=2e-6)


def test_q8_activation_codes_match_bruteforce():
    blob = _blob(TINY_Q8, synth.Q8_0)
    m = oracle.Model(blob, synth.Q8_0)
    layer = 1
    m.trace_layer(layer)
    fed = np.array([1, 5, 9, 200, 3], np.int32)
    per_pos = []
    for p, t in enumerate(fed):
        m.forward(int(t), p)
        per_pos.append([m.trace(s) for s in range(4)])
    _, traces = bruteforce.forward_all(blob, synth.Q8_0, fed, trace_layer=layer)
    for slot in range(4):
        bq, bs = traces[slot]
        for p in range(len(fed)):
            q, s, f = per_pos[p][slot]
            np.testing.assert_array_equal(s, bs[p])
            np.testing.assert_array_equal(q, bq[p])


def test_gqa_equals_mha_with_repeated_kv_heads():
    """A GQA model and the MHA model whose k/v weight rows repeat each kv head
    kv_mul times compute the same logits, bit for bit."""
    cfg = TINY  # 8 heads, 4 kv heads, head_size 8
    blob = _blob(cfg, synth.F32)
    w = view(blob, synth.F32)
    d, h, L, nh, nkv, vs, S = w["hdr"]
    hs = d // nh
    kvmul = nh // nkv

    def rep(a):  # (L, nkv*hs, d) -> (L, nh*hs, d), kv head g feeds heads g*kvmul..
        a = a.reshape(L, nkv, hs, d)
        return np.repeat(a, kvmul, axis=1).reshape(L, nh * hs, d)

    arrays = {k: v for k, v in w.items() if k not in ("hdr", "wcls")}
    arrays["wk"] = rep(w["wk"])
    arrays["wv"] = rep(w["wv"])
    arrays["freq_re"] = w["freq_re"]
    arrays["freq_im"] = w["freq_im"]
    hdr = (d, h, L, nh, nh, vs, S)
    mha_blob = assemble(hdr, synth.F32, arrays)
    a = oracle.Model(blob, synth.F32)
    b = oracle.Model(mha_blob, synth.F32)
    for p, t in enumerate([1, 7, 300, 2]):
        np.testing.assert_array_equal(a.forward(t, p), b.forward(t, p))


def test_shared_and_unshared_classifier_agree():
    """vocab_size > 0 ties the classifier to the embedding; an unshared blob
    whose classifier array is a copy of the embedding gives the same logits."""
    blob = _blob(TINY, synth.F32)
    w = view(blob, synth.F32)
    d, h, L, nh, nkv, vs, S = w["hdr"]
    arrays = {k: v for k, v in w.items() if k != "hdr"}
    arrays["wcls"] = w["emb"].copy()
    unshared = assemble((d, h, L, nh, nkv, -vs, S), synth.F32, arrays)
    assert unshared.size == blob.size + 4 * vs * d
    a = oracle.Model(blob, synth.F32)
    b = oracle.Model(unshared, synth.F32)
    for p, t in enumerate([1, 4, 9]):
        np.testing.assert_array_equal(a.forward(t, p), b.forward(t, p))
    # and a different classifier array changes them
    arrays["wcls"] = -w["emb"]
    neg = oracle.Model(assemble((d, h, L, nh, nkv, -vs, S), synth.F32, arrays), synth.F32)
    np.testing.assert_array_equal(neg.forward(1, 0), -oracle.Model(blob, synth.F32).forward(1, 0))


def test_legacy_freq_tables_are_skipped():
    """The generator fills the legacy freq_cis tables with NaN: finite logits
    prove they are skipped, and the size check rejects a blob without them."""
    for cfg, dt in ((TINY, synth.F32), (TINY_Q8_UNSHARED, synth.Q8_0)):
        blob = _blob(cfg, dt)
        w = view(blob, dt)
        assert np.isnan(w["freq_re"]).all() and np.isnan(w["freq_im"]).all()
        m = oracle.Model(blob, dt)
        assert np.isfinite(m.forward(1, 0)).all()
        with pytest.raises(ValueError):
            oracle.Model(blob[:-4], dt)
        with pytest.raises(ValueError):
            oracle.Model(np.concatenate([blob, np.zeros(4, np.uint8)]), dt)


def test_attention_pos0_is_v_and_equal_keys_give_mean_v():
    """At pos 0 softmax has one term, so the attention output is v exactly.
    With every cached key equal, the weights are uniform and o is the mean
    of the cached values."""
    cfg = TINY.replace(n_layers=1, name="tiny1")
    blob = _blob(cfg, synth.F32)
    m = oracle.Model(blob, synth.F32)
    m.forward(5, 0)
    kvmul = cfg.n_heads // cfg.n_kv_heads
    hs = cfg.head_size
    v0 = m.value_cache()[0, 0].copy()
    o = m.attn_out()
    for hd in range(cfg.n_heads):
        g = hd // kvmul
        np.testing.assert_array_equal(o[hd * hs:(hd + 1) * hs], v0[g * hs:(g + 1) * hs])
    # equal keys: run pos P once to learn k_P, copy it to slots 0..P-1, rerun
    P = 6
    m.forward(5, P)
    kc, vc = m.key_cache(), m.value_cache()
    kc[0, :P] = kc[0, P]
    rng = np.random.default_rng(0)
    vc[0, :P] = rng.standard_normal((P, cfg.kv_dim)).astype(np.float32)
    m.forward(5, P)  # layer 0's k at pos P depends only on (token, pos)
    o = m.attn_out().astype(np.float64)
    mean_v = vc[0, :P + 1].astype(np.float64).mean(axis=0)
    for hd in range(cfg.n_heads):
        g = hd // kvmul
        np.testing.assert_allclose(o[hd * hs:(hd + 1) * hs], mean_v[g * hs:(g + 1) * hs],
                                   rtol=1e-6, atol=1e-7)


def test_rmsnorm_closed_form_through_embedding():
    """x = c * ones: RMSNorm gives g * c / sqrt(c^2 + eps). Checked through a
    one-layer model whose weights are zero except the embedding row: the
    attention and FFN blocks then add nothing, so the logits are
    E . rmsnorm(x) with x = c * ones."""
    cfg = TINY.replace(n_layers=1, name="tinyc")
    blob = _blob(cfg, synth.F32)
    w = view(blob, synth.F32)
    arrays = {k: v.copy() for k, v in w.items() if k not in ("hdr", "wcls")}
    for k in ("wq", "wk", "wv", "wo", "w1", "w2", "w3"):
        arrays[k][:] = 0
    c = np.float32(0.37)
    arrays["emb"][3] = c
    gains = np.linspace(0.5, 1.5, cfg.dim).astype(np.float32)
    arrays["rms_final"] = gains
    b = assemble(w["hdr"], synth.F32, arrays)
    m = oracle.Model(b, synth.F32)
    lg = m.forward(3, 0).astype(np.float64)
    y = gains.astype(np.float64) * float(c) / math.sqrt(float(c) ** 2 + 1e-5)
    want = arrays["emb"].astype(np.float64) @ y
    np.testing.assert_allclose(lg, want, rtol=1e-6, atol=1e-7)


def test_thread_count_does_not_change_results():
    blob = _blob(TINY_Q8, synth.Q8_0)
    outs = []
    for n in (1, 3):
        oracle.set_threads(n)
        m = oracle.Model(blob, synth.Q8_0)
        outs.append(np.stack([m.forward(t, p) for p, t in enumerate([1, 2, 3])]))
    oracle.set_threads(os.cpu_count() or 1)
    np.testing.assert_array_equal(outs[0], outs[1])


def test_bad_token_pos_rejected():
    m = oracle.Model(_blob(TINY, synth.F32), synth.F32)
    for t, p in ((-1, 0), (512, 0), (0, -1), (0, 512)):
        with pytest.raises(ValueError):
            m.forward(t, p)


# ------------------------------------------------------------- blob sizes vs the pages

def test_blob_sizes_match_pages_table():
    g = json.load(open(os.path.join(GOLDEN, "page_sizes.json")))
    for row in g["rows"]:
        cfg = synth.CONFIGS[row["model"]]
        fp = synth.blob_bytes(cfg, synth.F32)
        assert abs(fp / row["fp32_bytes"] - 1) < g["rel_tol_bytes"], (row, fp)
        for gs in (128, 256):  # the hub page's default group sizes
            q8 = synth.blob_bytes(cfg, synth.Q8_0, gs)
            assert abs(q8 / row["int8_bytes"] - 1) < g["rel_tol_bytes"], (row, gs, q8)
            assert abs((fp / q8) / row["ratio"] - 1) < g["rel_tol_ratio"], (row, gs, fp / q8)
