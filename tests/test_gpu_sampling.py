"""On-device temperature sampling fused into the classifier (mht18 essay,
section 3.2), against the oracle's sampler on the same logits and draws.

The GPU compares fp32 scores logit / T + g with g from fp64 logs; the
oracle's logs come from the C library, so a score may differ by one fp32
ulp. The drawn token must equal the oracle's wherever the oracle's top-2
score margin exceeds a few ulps; elsewhere it must be one of the tied top
scores.
"""
import numpy as np
import pytest

import llama_transformer_decode_amd as l2d
import oracle
import synth
from gpu_util import Stats, log, need_gpu

pytestmark = pytest.mark.gpu

T, SEED = 0.8, 20240917


def _check_pick(gpu_tok, ref_logits, pos, where):
    sc = oracle.sample_scores(ref_logits, T, SEED, pos)
    order = np.argsort(sc)[::-1]
    top, second = float(sc[order[0]]), float(sc[order[1]])
    margin = top - second
    if margin > 8 * np.spacing(np.float32(abs(top))):
        assert gpu_tok == int(order[0]), (where, pos, gpu_tok, int(order[0]), margin)
        return 1
    assert sc[gpu_tok] >= top - 8 * np.spacing(np.float32(abs(top))), (where, pos, gpu_tok)
    return 0


@pytest.mark.parametrize("name,dtype", [("15M", synth.F32), ("110M", synth.Q8_0)])
def test_teacher_forced_sampling_matches_oracle(name, dtype):
    need_gpu()
    cfg = synth.CONFIGS[name]
    blob = synth.make_blob(cfg, dtype)
    orc = oracle.Model(blob, dtype)
    steps = 128
    unique = 0
    with l2d.Context(blob, dtype) as ctx:
        ctx.set_sampling(T, SEED)
        tok = 1
        st = Stats()
        for p in range(steps):
            r = orc.forward(tok, p)
            ctx.forward(tok, p)
            g = ctx.logits()
            st.add(p, g, r)
            gtok = ctx.last_token()
            unique += _check_pick(gtok, r, p, name)
            tok = oracle.sample(r, T, SEED, p)
        st.assert_ok()
    orc.close()
    log(f"  {name} dt{dtype}: {st.summary()}, sampled picks compared exactly {unique}/{steps}")
    assert unique >= steps - 2


def test_on_device_sampled_chain_equals_host_loop():
    """forward_greedy with sampling on: the device feeds its own draws; the
    host loop feeds the oracle's draws from the oracle's logits."""
    need_gpu()
    cfg = synth.CONFIGS["15M"]
    blob = synth.make_blob(cfg, synth.F32)
    orc = oracle.Model(blob, synth.F32)
    n = 120
    want = []
    tok = 1
    for p in range(n):
        r = orc.forward(tok, p)
        tok = oracle.sample(r, T, SEED, p)
        want.append(tok)
    orc.close()
    with l2d.Context(blob, synth.F32) as ctx:
        ctx.set_sampling(T, SEED)
        ctx.forward(1, 0)
        got = [ctx.last_token()]
        for p in range(1, n):
            ctx.forward_greedy(p)
            got.append(ctx.last_token())
    np.testing.assert_array_equal(np.array(got), np.array(want))
    # a draw, not the argmax: the chain differs from greedy decoding
    assert len(set(got)) > 5


def test_zero_temperature_is_greedy_and_bad_temperature_rejected():
    need_gpu()
    cfg = synth.CONFIGS["tiny"]
    blob = synth.make_blob(cfg, synth.F32)
    with l2d.Context(blob, synth.F32) as ctx:
        ctx.set_sampling(0.0, 5)
        ctx.forward(1, 0)
        assert ctx.last_token() == int(np.argmax(ctx.logits()))
        for bad in (-1.0, float("nan"), float("inf")):
            with pytest.raises(l2d.L2DError):
                ctx.set_sampling(bad, 1)


@pytest.mark.parametrize("dtype", [synth.Q8_0, synth.F32])
def test_sampled_chain_after_batched_prefill(dtype):
    """A 40-token prompt through the batched prefill with sampling on, then
    the device's own sampled continuation: equals the host loop feeding the
    prompt and then the oracle's draws (the prefill's last step draws the
    first generated token exactly as a single-token step would)."""
    need_gpu()
    cfg = synth.CONFIGS["110M"]
    blob = synth.make_blob(cfg, dtype)
    orc = oracle.Model(blob, dtype)
    prompt = synth.prompt(31, 40, cfg.vocab)
    n = 24
    want = []
    for p, t in enumerate(prompt):
        r = orc.forward(int(t), p)
    tok = oracle.sample(r, T, SEED, len(prompt) - 1)
    want.append(tok)
    for p in range(len(prompt), len(prompt) + n - 1):
        r = orc.forward(tok, p)
        tok = oracle.sample(r, T, SEED, p)
        want.append(tok)
    orc.close()
    with l2d.Context(blob, dtype) as ctx:
        ctx.set_sampling(T, SEED)
        ctx.prefill(prompt, 0)
        got = [ctx.last_token()]
        for p in range(len(prompt), len(prompt) + n - 1):
            ctx.forward_greedy(p)
            got.append(ctx.last_token())
    np.testing.assert_array_equal(np.array(got), np.array(want))


def test_q4_0_sampled_chain_equals_host_loop():
    """Sampling on top of the 4-bit decode step (110M, Q4_0)."""
    need_gpu()
    cfg = synth.CONFIGS["110M"]
    blob = synth.make_blob(cfg, synth.Q4_0)
    orc = oracle.Model(blob, synth.Q4_0)
    n = 64
    want = []
    tok = 1
    for p in range(n):
        r = orc.forward(tok, p)
        tok = oracle.sample(r, T, SEED, p)
        want.append(tok)
    orc.close()
    with l2d.Context(blob, synth.Q4_0) as ctx:
        ctx.set_sampling(T, SEED)
        ctx.forward(1, 0)
        got = [ctx.last_token()]
        for p in range(1, n):
            ctx.forward_greedy(p)
            got.append(ctx.last_token())
    np.testing.assert_array_equal(np.array(got), np.array(want))
