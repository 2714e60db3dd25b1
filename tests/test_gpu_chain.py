"""Chained launches (attention + output projection, w1/w3 + w2 in one launch
each) against the kernel-by-kernel step and the oracle.

The chained launches run the same per-phase arithmetic in the same order:
only where the second phase's workgroups start (they follow the first
phase's in the grid, prefetch their weights and wait on the first phase's
flags) and where the w2 input's codes sit (one group per 128-byte line)
change. So the
logits must equal the kernel-by-kernel step's bit for bit at every step,
and every step must meet the oracle's logits tolerance and argmax rule.
Shapes cover one, two, four and eight query heads per kv head (eight: two
attention workgroups per kv head of four heads each), head sizes 32, 64 and
128, an odd vocabulary, the 110M, 7B, 13B and 70B shapes, switching the
mode back and forth on one context (each switch re-captures the graph),
deep positions over injected caches, and decoding with the token taken on
the device.
"""
import gc

import numpy as np
import pytest

import llama_transformer_decode_amd as l2d
import oracle
import synth
from gpu_util import Stats, log, need_gpu

pytestmark = pytest.mark.gpu

TINY_Q8 = synth.Config("tinyq8", 128, 256, 3, 4, 2, 320, 64, 11, (synth.Q8_0,))      # hs 32, G 2
GQA4_Q8 = synth.Config("gsq8", 256, 512, 2, 8, 2, 320, 48, 13, (synth.Q8_0,))        # hs 32, G 4
GQA8_H128 = synth.Config("gqa8h128", 1024, 512, 2, 8, 1, 320, 96, 14, (synth.Q8_0,))  # hs 128, G 8
ODD_V = synth.Config("oddv", 128, 192, 2, 4, 4, 321, 40, 15, (synth.Q8_0,))          # hs 32, G 1, odd vocab


def _chain_vs_phase(cfg, steps, label):
    """Oracle-fed trajectory through both modes on one context: chained and
    kernel-by-kernel (the default), bit for bit, and the chained run against
    the oracle at every step."""
    need_gpu()
    blob = synth.make_blob(cfg, synth.Q8_0)
    orc = oracle.Model(blob, synth.Q8_0)
    with l2d.Context(blob, synth.Q8_0) as ctx:
        assert not ctx.chained, f"{label}: chained launches are off by default"
        ctx.use_chain(True)
        assert ctx.chained
        st = Stats()
        chained, fed = [], []
        tok = 1
        for p in range(steps):
            ctx.forward(tok, p)
            r = orc.forward(tok, p)
            g = ctx.logits()
            st.add(p, g, r, ctx.last_token())
            chained.append(g)
            fed.append(tok)
            tok = int(np.argmax(r))
        log(f"  [{label}] chained vs oracle: {st.summary()}")
        st.assert_ok()
        ctx.reset_kv()
        ctx.use_chain(False)
        assert not ctx.chained
        for p, t in enumerate(fed):
            ctx.forward(t, p)
            g = ctx.logits()
            assert np.array_equal(g, chained[p]), (
                f"{label} pos {p}: chained logits differ from the kernel-by-kernel step "
                f"(max |d| {float(np.abs(g - chained[p]).max()):.3g})")
        # and back: the re-captured chained graph continues the same cache
        ctx.reset_kv()
        ctx.use_chain(True)
        assert ctx.chained
        for p, t in enumerate(fed[:8]):
            ctx.forward(t, p)
            assert np.array_equal(ctx.logits(), chained[p]), f"{label} pos {p}: after re-enabling"
        log(f"  [{label}] {steps} steps bit-identical to the kernel-by-kernel step")
    orc.close()


@pytest.mark.parametrize("cfg,steps", [
    (TINY_Q8, 64), (GQA4_Q8, 48), (GQA8_H128, 96), (ODD_V, 40),
], ids=["tiny_g2_hs32", "gqa4_hs32", "gqa8_hs128", "odd_vocab"])
def test_chain_small(cfg, steps):
    _chain_vs_phase(cfg, steps, cfg.name)


def test_chain_110m():
    """110M Q8_0 (head size 64, one query head per kv head): 256 steps."""
    _chain_vs_phase(synth.CONFIGS["110M"], 256, "110M")


def test_chain_greedy_on_device():
    """Greedy decoding with the token taken on the device (the step-start
    kernel reads the previous classifier's argmax): the chained and the
    kernel-by-kernel step pick the same tokens."""
    need_gpu()
    cfg = TINY_Q8
    blob = synth.make_blob(cfg, synth.Q8_0)
    toks = {}
    with l2d.Context(blob, synth.Q8_0) as ctx:
        for chain in (True, False):
            ctx.use_chain(chain)
            ctx.reset_kv()
            ctx.forward(1, 0)
            out = []
            for p in range(1, 48):
                ctx.forward_greedy(p)
                out.append(ctx.last_token())
            toks[chain] = out
    assert toks[True] == toks[False]


def test_chain_availability():
    """Available (off by default) for Q8_0 with group size 64; not for fp32
    or other group sizes (those run kernel by kernel only)."""
    need_gpu()
    blob = synth.make_blob(synth.CONFIGS["tiny"], synth.F32)
    with l2d.Context(blob, synth.F32) as ctx:
        assert not ctx.chained
        with pytest.raises(l2d.L2DError):
            ctx.use_chain(True)
        ctx.use_chain(False)
    blob = synth.make_blob(TINY_Q8, synth.Q8_0, gs=32)
    with l2d.Context(blob, synth.Q8_0, group_size=32) as ctx:
        assert not ctx.chained
        with pytest.raises(l2d.L2DError):
            ctx.use_chain(True)
    blob = synth.make_blob(TINY_Q8, synth.Q8_0)
    with l2d.Context(blob, synth.Q8_0) as ctx:
        assert not ctx.chained
        ctx.use_chain(True)
        assert ctx.chained
        t = ctx.kernel_profile(1, 5, reps=2)
        # chained: class 1 = attention + output matvec, class 3 = w1/w3 + w2
        assert t["attn"] > 0 and t["w13"] > 0 and t["wo"] == 0 and t["w2"] == 0


def test_chain_7b_full_size():
    """7B Q8_0 at full size: pos 0..3 teacher-forced, then deep positions 512
    and 2048 over identical injected caches; chained and kernel-by-kernel
    logits bit for bit, and the chained step against the oracle."""
    torch = need_gpu()
    from test_gpu_decode import _fill_kv_both
    cfg = synth.CONFIGS["7B"]
    blob = synth.make_blob(cfg, synth.Q8_0)
    orc = oracle.Model(blob, synth.Q8_0)
    ctx = l2d.Context(blob, synth.Q8_0)
    try:
        tok = 1
        for p in [0, 1, 2, 3, 512, 2048]:
            if p > 3:
                _fill_kv_both(ctx, orc, p, seed=77 + p)
            r = orc.forward(tok, p)
            out = {}
            for chain in (True, False):
                ctx.use_chain(chain)
                ctx.forward(tok, p)
                out[chain] = ctx.logits()
            st = Stats()
            st.add(p, out[True], r)
            log(f"  7B pos {p} chained: {st.summary()}")
            st.assert_ok()
            assert np.array_equal(out[True], out[False]), f"pos {p}: chained differs from kernel-by-kernel"
            tok = int(np.argmax(r))
    finally:
        ctx.close()
        orc.close()
        del blob
        gc.collect()
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name,deep", [("13B", 4095), ("70B", 4095)])
def test_chain_large_shapes_bitwise(name, deep):
    """13B (dim 5120: two input chunks per thread in the output projection,
    four in w2) and 70B (eight query heads per kv head in attention
    workgroups of four; w2's input of 28672 codes loaded in batches from the
    one-group-per-line layout) at full size: pos 0..2, then a deep position
    over a random cache, chained against kernel by kernel, bit for bit (the
    kernel-by-kernel step meets the oracle in the decode tests)."""
    torch = need_gpu()
    cfg = synth.CONFIGS[name]
    blob = synth.make_blob(cfg, synth.Q8_0)
    ctx = l2d.Context(blob, synth.Q8_0)
    del blob
    gc.collect()
    try:
        tok = 1
        for p in [0, 1, 2, deep]:
            if p == deep:
                kc, vc = ctx.kv_cache()
                g = torch.Generator(device="cuda").manual_seed(p)
                kc[:, :p].normal_(generator=g)
                vc[:, :p].normal_(generator=g)
                torch.cuda.synchronize()
            out = {}
            for chain in (True, False):
                ctx.use_chain(chain)
                assert ctx.chained == chain
                ctx.forward(tok, p)
                out[chain] = ctx.logits()
            log(f"  {name} pos {p}: chained vs kernel by kernel max |d| "
                f"{float(np.abs(out[True] - out[False]).max()):.3g}")
            assert np.array_equal(out[True], out[False]), f"{name} pos {p}: chained differs from kernel-by-kernel"
            tok = int(np.argmax(out[False]))
    finally:
        ctx.close()
        gc.collect()
        torch.cuda.empty_cache()


def test_chain_fault_reported_and_cleared():
    """The failure path of the bounded waits, forced from the host (no kernel
    is made to hang or fault): with the error word set before a chained
    step, its waits give up wherever their flags are not yet set, the next
    synchronisation reports L2D_EHIP, and the step after that is valid
    again (equal to the kernel-by-kernel step's logits, and to the oracle's
    within tolerance)."""
    need_gpu()
    cfg = TINY_Q8
    blob = synth.make_blob(cfg, synth.Q8_0)
    orc = oracle.Model(blob, synth.Q8_0)
    with l2d.Context(blob, synth.Q8_0) as ctx:
        ctx.use_chain(True)
        tok = 1
        for p in range(4):
            ctx.forward(tok, p)
            r = orc.forward(tok, p)
            tok = int(np.argmax(r))
        ctx.sync()
        ctx.test_chain_fault()
        ctx.forward(tok, 4)
        with pytest.raises(l2d.L2DError) as e:
            ctx.sync()
        assert "gave up" in str(e.value)
        ctx.sync()  # the word is clear again
        # the same step again, chained and then kernel by kernel
        ctx.forward(tok, 4)
        chained = ctx.logits()
        ctx.use_chain(False)
        ctx.forward(tok, 4)
        assert np.array_equal(chained, ctx.logits())
        st = Stats()
        st.add(4, chained, orc.forward(tok, 4))
        st.assert_ok()
    orc.close()
