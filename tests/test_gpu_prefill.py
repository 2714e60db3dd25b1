"""Batched prompt prefill (int8 MFMA matmuls for Q8_0, fp64 MFMA for fp32
weights, causal attention over token blocks) against the oracle's
token-by-token decode, through the C ABI: the K/V cache rows the prefill
writes, the last token's logits and argmax, and the decode that continues
from it on the device.

Small models cover group sizes 64, 128 and 256, GQA ratios 1, 2, 4 and 8,
head sizes 8 to 128, ragged token counts, prompts longer than one 512-token
chunk and prefill in two calls at pos0 > 0; the 7B shape runs at full size
in both dtypes. Head sizes that are multiples of 16 take the matrix-core
attention kernel (blocks of 16 (token, query head) rows); the others take
the vector kernel, which L2D_PREFILL_ATTN_VALU=1 also selects for every
shape, so both kernels are checked at every GQA ratio. Q8_0 is
bit-identical by construction (same exact group dots, same fp64 order); fp32
sums the same exact products in another fp64 order, like the decode step's
fp32 GEMV, and is held to the logits tolerance. The Q8_0 prefill with its
group combine in fp32 is checked where its arithmetic alone decides (layer
0); see its test for why not beyond."""
import gc
import os

import numpy as np
import pytest

import llama_transformer_decode_amd as l2d
import oracle
import synth
from gpu_util import Stats, log, need_gpu

pytestmark = pytest.mark.gpu

TINY_Q8 = synth.Config("tinyq8", 128, 256, 3, 4, 2, 320, 64, 11, (synth.Q8_0,))
GQA8_Q8 = synth.Config("gqa8q8", 256, 512, 2, 8, 1, 320, 96, 12, (synth.Q8_0,))
GQA8_H128 = synth.Config("gqa8h128", 1024, 512, 2, 8, 1, 320, 96, 14, (synth.Q8_0,))  # head size 128, G = 8
GQA4_H64 = synth.Config("gqa4h64", 512, 512, 2, 8, 2, 320, 96, 15, (synth.Q8_0,))  # head size 64, G = 4
GQA4_H32 = synth.Config("gqa4h32", 256, 512, 2, 8, 2, 320, 80, 16, (synth.Q8_0,))  # head size 32, G = 4
MHA_H64 = synth.Config("mhah64", 256, 512, 2, 4, 4, 320, 80, 17, (synth.Q8_0,))  # head size 64, G = 1


def _check_cache(ctx, orc, lo: int, hi: int, st: Stats):
    kc, vc = ctx.kv_cache()
    st.add("k", kc[:, lo:hi].cpu().numpy(), orc.key_cache()[:, lo:hi])
    st.add("v", vc[:, lo:hi].cpu().numpy(), orc.value_cache()[:, lo:hi])


def _run(cfg, gs: int, calls, cont: int = 6, dtype: int = synth.Q8_0, valu: bool = False,
         combine32: bool = False):
    """calls: list of (start, n) prefill calls over one prompt; then `cont`
    greedy decode steps on the device, teacher-checked against the oracle.
    valu: run the prefill with the vector attention kernel for every shape
    (L2D_PREFILL_ATTN_VALU=1, read at each prefill launch).
    combine32: the Q8_0 matmuls combine group dots in fp32."""
    torch = need_gpu()
    if valu:
        os.environ["L2D_PREFILL_ATTN_VALU"] = "1"
    try:
        return _run_inner(cfg, gs, calls, cont, dtype, torch, combine32)
    finally:
        os.environ.pop("L2D_PREFILL_ATTN_VALU", None)


def _run_inner(cfg, gs, calls, cont, dtype, torch, combine32=False):
    total = sum(n for _, n in calls)
    tokens = synth.prompt(cfg.seed + 500, total, abs(cfg.vocab))
    blob = synth.make_blob(cfg, dtype, gs=gs)
    orc = oracle.Model(blob, dtype, gs=gs)
    cache_st, logit_st = Stats(), Stats()
    with l2d.Context(blob, dtype, group_size=gs) as ctx:
        if combine32:
            ctx.prefill_combine(True)
        for start, n in calls:
            log(f"  {cfg.name} dt{dtype} gs{gs}{' fp32 combine' if combine32 else ''}: "
                f"prefill {n} tokens at pos {start}")
            ctx.prefill(tokens[start:start + n], start)
            for i in range(n):
                ref = orc.forward(int(tokens[start + i]), start + i)
            logit_st.add(start + n - 1, ctx.logits(), ref, ctx.last_token())
        _check_cache(ctx, orc, 0, total, cache_st)
        # continue: the first step takes the prefill's pick on the device
        fed = int(np.argmax(ref))
        for j in range(cont):
            p = total + j
            if p >= cfg.seq_len:
                break
            if j == 0:
                ctx.forward_greedy(p)
            else:
                ctx.forward(fed, p)
            r = orc.forward(fed, p)
            logit_st.add(p, ctx.logits(), r, ctx.last_token())
            fed = int(np.argmax(r))
    orc.close()
    torch.cuda.synchronize()
    log(f"  cache rows: {cache_st.summary()}")
    log(f"  logits: {logit_st.summary()}")
    cache_st.assert_ok()
    logit_st.assert_ok()
    return cache_st, logit_st


@pytest.mark.parametrize("cfg,gs,calls", [
    (TINY_Q8, 64, [(0, 41)]),            # G = 2: blocks of 2 tokens, ragged
    (TINY_Q8, 128, [(0, 37)]),           # two 64-value MFMA parts per group
    (TINY_Q8, 64, [(0, 1)]),             # a single token
    (GQA8_Q8, 64, [(0, 50)]),            # G = 8: one token per block
    (GQA8_Q8, 256, [(0, 33), (33, 20)]),  # four parts per group; second call at pos 33
    (GQA8_H128, 64, [(0, 45), (45, 20)]),  # the 70B attention shape: head size 128, G = 8
    (GQA4_H64, 64, [(0, 38), (38, 21)]),  # G = 4 on the matrix cores: 4 tokens x 4 heads per block
    (GQA4_H32, 64, [(0, 29), (29, 18)]),  # G = 4, head size 32
], ids=["tiny-g2-gs64", "tiny-gs128", "tiny-one-token", "gqa8-gs64", "gqa8-gs256-two-calls", "gqa8-hs128-two-calls",
        "gqa4-hs64-two-calls", "gqa4-hs32-two-calls"])
def test_prefill_small(cfg, gs, calls):
    cache_st, _ = _run(cfg, gs, calls)
    assert cache_st.exact / cache_st.n > 0.99


@pytest.mark.parametrize("cfg,calls", [
    (MHA_H64, [(0, 33), (33, 14)]),       # G = 1: blocks of 4 tokens
    (TINY_Q8, [(0, 41)]),                 # G = 2: blocks of 2 tokens
    (GQA4_H64, [(0, 38), (38, 21)]),      # G = 4: one token of 4 heads per block
    (GQA8_H128, [(0, 45), (45, 20)]),     # G = 8: one token per block
], ids=["g1-hs64", "g2-hs32", "g4-hs64", "g8-hs128"])
def test_prefill_vector_attention(cfg, calls):
    """The vector attention kernel at every GQA ratio, on shapes the
    matrix-core kernel would otherwise take (L2D_PREFILL_ATTN_VALU=1)."""
    cache_st, _ = _run(cfg, 64, calls, valu=True)
    assert cache_st.exact / cache_st.n > 0.99


@pytest.mark.parametrize("cfg,gs,n", [
    (TINY_Q8, 64, 41),
    (GQA8_Q8, 256, 53),
    (GQA8_H128, 64, 65),
    (synth.CONFIGS["110M"], 64, 300),
], ids=["tiny-gs64", "gqa8-gs256", "gqa8-hs128", "110m-300"])
def test_prefill_fp32_combine(cfg, gs, n):
    """Q8_0 matmuls with the group combine in fp32 (l2d_prefill_combine).
    Layer 0's inputs are exact (dequantised embedding rows), so its K/V
    cache rows differ from the oracle's only by the combine: within 1e-5
    relative (fp32 accumulation over at most 4096 / gs groups). Later layers
    quantise inputs that already differ in low bits; a code that then rounds
    the other way at a near tie moves everything after it, so the end-to-end
    difference is logged, not held to the logits tolerance."""
    torch = need_gpu()
    tokens = synth.prompt(cfg.seed + 500, n, abs(cfg.vocab))
    blob = synth.make_blob(cfg, synth.Q8_0, gs=gs)
    orc = oracle.Model(blob, synth.Q8_0, gs=gs)
    with l2d.Context(blob, synth.Q8_0, group_size=gs) as ctx:
        ctx.prefill_combine(True)
        ctx.prefill(tokens, 0)
        for i in range(n):
            ref = orc.forward(int(tokens[i]), i)
        kc, vc = ctx.kv_cache()
        for name, g, o in (("k", kc, orc.key_cache()), ("v", vc, orc.value_cache())):
            g0 = g[0, :n].cpu().numpy().astype(np.float64)
            o0 = o[0, :n].astype(np.float64)
            d = np.abs(g0 - o0)
            assert (d <= 1e-6 + 1e-5 * np.abs(o0)).all(), (name, float(d.max()))
        st = Stats()
        _check_cache(ctx, orc, 0, n, st)
        lg = np.abs(ctx.logits().astype(np.float64) - ref).max()
        log(f"  {cfg.name} gs{gs} fp32 combine, {n} tokens: layer 0 K/V within 1e-5 relative; "
            f"all layers {st.summary()}; last logits max|d| {lg:.3g}")
    orc.close()
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,calls", [
    ("tiny", [(0, 45)]),                  # head size 8, G = 2
    ("15M", [(0, 100), (100, 60)]),       # head size 48, second call at pos 100
    ("110M", [(0, 520)]),                 # a full 512-token chunk, then 8
])
def test_prefill_fp32(name, calls):
    cfg = synth.CONFIGS[name]
    cache_st, _ = _run(cfg, 64, calls, cont=4, dtype=synth.F32)
    assert cache_st.exact / cache_st.n > 0.9


def test_prefill_110m_two_chunks_and_two_calls():
    """601 tokens: one call of 250, then 351 at pos 250 (a 512-token chunk
    boundary falls inside neither; the first call is one chunk), and a
    single call of 601 tokens (a full 512-token chunk, then a ragged 89)."""
    cfg = synth.CONFIGS["110M"]
    _run(cfg, 64, [(0, 250), (250, 351)], cont=4)
    _run(cfg, 64, [(0, 601)], cont=4)


def test_prefill_matches_own_decode_bitwise():
    """The prefill and the device's own token-by-token steps leave the same
    cache rows and logits (both follow the oracle's arithmetic)."""
    torch = need_gpu()
    cfg = synth.CONFIGS["110M"]
    blob = synth.make_blob(cfg, synth.Q8_0)
    tokens = synth.prompt(77, 96, cfg.vocab)
    with l2d.Context(blob, synth.Q8_0) as a, l2d.Context(blob, synth.Q8_0) as b:
        a.prefill(tokens, 0)
        for i, t in enumerate(tokens):
            b.forward(int(t), i)
        la, lb = a.logits(), b.logits()
        ka, va = a.kv_cache()
        kb, vb = b.kv_cache()
        dk = (ka[:, :96] - kb[:, :96]).abs().max().item()
        dv = (va[:, :96] - vb[:, :96]).abs().max().item()
        same = float((ka[:, :96] == kb[:, :96]).float().mean().item())
        log(f"  prefill vs decode: max|dK| {dk:.3g} max|dV| {dv:.3g} K identical {same:.5f}, "
            f"logits max|d| {np.abs(la - lb).max():.3g}")
        assert dk <= 1e-5 and dv <= 1e-5
        assert np.abs(la.astype(np.float64) - lb).max() <= 1e-4
        assert a.last_token() == b.last_token() or np.sort(lb)[-1] - np.sort(lb)[-2] <= 1e-3
    torch.cuda.synchronize()


def test_prefill_errors():
    need_gpu()
    blob = synth.make_blob(TINY_Q8, synth.Q8_0)
    with l2d.Context(blob, synth.Q8_0) as ctx:
        with pytest.raises(l2d.L2DError):
            ctx.prefill([], 0)
        with pytest.raises(l2d.L2DError):
            ctx.prefill([1, 2, 3], TINY_Q8.seq_len - 2)   # past the end of the cache
        with pytest.raises(l2d.L2DError):
            ctx.prefill([1, TINY_Q8.vocab], 0)           # token out of range
        with pytest.raises(l2d.L2DError):
            ctx.prefill([1, 2], -1)
        ctx.prefill([1, 2], 0)                           # still usable afterwards
    blob32 = synth.make_blob(TINY_Q8, synth.Q8_0, gs=32)
    with l2d.Context(blob32, synth.Q8_0, group_size=32) as ctx:
        with pytest.raises(l2d.L2DError):
            ctx.prefill([1, 2], 0)                       # group size 32: not built


def test_prefill_7b_q8_full_size():
    """7B Q8_0: 64 prompt tokens, then 24 more at pos 64; every layer's cache
    rows and the last logits of each call against the oracle."""
    torch = need_gpu()
    cfg = synth.CONFIGS["7B"]
    try:
        _run(cfg, 64, [(0, 64), (64, 24)], cont=2)
    finally:
        gc.collect()
        torch.cuda.empty_cache()


def test_prefill_7b_fp32_full_size():
    """7B fp32: 20 prompt tokens, then 8 more at pos 20."""
    torch = need_gpu()
    cfg = synth.CONFIGS["7B"]
    try:
        _run(cfg, 64, [(0, 20), (20, 8)], cont=1, dtype=synth.F32)
    finally:
        gc.collect()
        torch.cuda.empty_cache()
