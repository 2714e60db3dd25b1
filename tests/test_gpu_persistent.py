"""The persistent step kernel (one cooperative launch per decode step).

Parity with the oracle in this mode is covered by test_gpu_decode.py (every
decode check runs in both modes); these tests cover what is specific to the
mode: availability, switching, idempotent repeats, and agreement with the
per-phase kernels.
"""
import numpy as np
import pytest

import llama_transformer_decode_amd as l2d
import oracle
import synth
from gpu_util import PERSISTENT_SKIP, Stats, log, need_gpu, set_mode

pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason=PERSISTENT_SKIP)]


@pytest.mark.parametrize("name,dtype", [("tiny", synth.F32), ("110M", synth.F32), ("110M", synth.Q8_0)])
def test_persistent_is_the_default(name, dtype):
    need_gpu()
    blob = synth.make_blob(synth.CONFIGS[name], dtype)
    with l2d.Context(blob, dtype) as ctx:
        assert ctx.persistent, "the step kernel should be available on this device"
        ctx.use_persistent(False)
        assert not ctx.persistent
        ctx.use_persistent(True)
        assert ctx.persistent


def test_unsupported_group_size_falls_back():
    """Q8_0 with group size 32: the step kernel is not built for it; the
    per-phase kernels run, and asking for the step kernel is an error."""
    need_gpu()
    cfg = synth.CONFIGS["110M"]
    blob = synth.make_blob(cfg, synth.Q8_0, gs=32)
    orc = oracle.Model(blob, synth.Q8_0, gs=32)
    with l2d.Context(blob, synth.Q8_0, group_size=32) as ctx:
        assert not ctx.persistent
        with pytest.raises(l2d.L2DError):
            ctx.use_persistent(True)
        r = orc.forward(1, 0)
        ctx.forward(1, 0)
        st = Stats()
        st.add(0, ctx.logits(), r, ctx.last_token())
        st.assert_ok()
    orc.close()


@pytest.mark.parametrize("dtype", [synth.F32, synth.Q8_0])
def test_repeat_is_bitwise_idempotent(dtype):
    need_gpu()
    blob = synth.make_blob(synth.CONFIGS["110M"], dtype)
    with l2d.Context(blob, dtype) as ctx:
        set_mode(ctx, "persistent")
        for p, t in enumerate([1, 50, 7, 9000, 31000]):
            ctx.forward(t, p)
        first = ctx.logits()
        tok = ctx.last_token()
        for _ in range(3):
            ctx.forward(31000, 4)
            np.testing.assert_array_equal(ctx.logits(), first)
            assert ctx.last_token() == tok


@pytest.mark.parametrize("name,dtype", [("15M", synth.F32), ("110M", synth.Q8_0)])
def test_modes_agree_closely(name, dtype):
    """Same inputs through both modes: only the fp64 summation order of the
    attention merge differs, so the logits agree to a few fp32 ulps."""
    need_gpu()
    blob = synth.make_blob(synth.CONFIGS[name], dtype)
    outs = {}
    with l2d.Context(blob, dtype) as ctx:
        for mode in ("persistent", "graph"):
            set_mode(ctx, mode)
            ctx.reset_kv()
            seq = []
            for p, t in enumerate([1, 300, 5000, 12, 31000, 77, 8]):
                ctx.forward(t, p)
                seq.append(ctx.logits())
            outs[mode] = np.stack(seq)
    d = np.abs(outs["persistent"].astype(np.float64) - outs["graph"].astype(np.float64))
    scale = np.maximum(np.abs(outs["graph"]).astype(np.float64), 1.0)
    log(f"  {name} dt{dtype}: max |persistent - graph| = {d.max():.3g}, "
        f"identical {np.mean(outs['persistent'] == outs['graph']):.4f}")
    assert (d <= 1e-5 * scale).all()


def test_greedy_chain_matches_oracle_trajectory():
    """On-device greedy decoding for 200 steps in the persistent mode equals
    the oracle's greedy trajectory wherever its top-2 margins are clear."""
    need_gpu()
    cfg = synth.CONFIGS["15M"]
    blob = synth.make_blob(cfg, synth.F32)
    orc = oracle.Model(blob, synth.F32)
    fed, am, _ = oracle.trajectory(orc, np.array([1], np.int32), 200, keep_logits=False)
    with l2d.Context(blob, synth.F32) as ctx:
        set_mode(ctx, "persistent")
        ctx.forward(1, 0)
        toks = [ctx.last_token()]
        for p in range(1, 200):
            ctx.forward_greedy(p)
            toks.append(ctx.last_token())
    orc.close()
    np.testing.assert_array_equal(np.array(toks), am)
