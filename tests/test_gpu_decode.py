"""End-to-end GPU parity of the decode step against the oracle.

Both sides read the same seeded blob. Decoding is teacher-forced: the
oracle's greedy trajectory (and, for the 15M shape, its forced prompt) is fed
to both, so one near-tie cannot fork the two runs; the GPU's own fused argmax
is checked at every step whose oracle top-2 margin exceeds 1e-3. Logits must
satisfy |gpu - oracle| <= 1e-3 + 1e-4 |oracle| everywhere.

Full-size workloads run the lengths the workloads state: the 7B Q8_0 model
decodes pos 0..2048 and the 7B fp32 model pos 0..255, teacher-forced by the
oracle's greedy trajectory computed in the same pass (one oracle step per
position); the 70B Q8_0 model decodes pos 0..63 and then one step at each of
pos 1024, 2048 and 4095 whose cache slots 0..pos-1 hold the same synthetic
keys and values on both sides (the KV-cache hook), so long-context GQA
attention, its position split and its merge are checked at the real shapes
and launch configuration. The 13B shape and the 4-bit 7B step run a few
steps plus injected deep positions.
"""
import gc
import time

import numpy as np
import pytest

import llama_transformer_decode_amd as l2d
import oracle
import synth
from gpu_util import MODES, decode_and_compare, log, need_gpu, set_mode

pytestmark = pytest.mark.gpu

TINY_Q8 = synth.Config("tinyq8", 128, 256, 3, 4, 2, 320, 64, 11, (synth.Q8_0,))
TINY_Q4 = synth.Config("tinyq4", 128, 256, 3, 4, 2, 320, 64, 21, (synth.Q4_0,))


def _trajectory(cfg, dtype, n):
    blob = synth.make_blob(cfg, dtype)
    orc = oracle.Model(blob, dtype)
    forced, _ = synth.trajectory_plan(cfg, n)
    fed, _, _ = oracle.trajectory(orc, forced, n, keep_logits=False)
    orc.reset_kv()
    return blob, orc, fed


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name,dtype,steps", [
    ("tiny", synth.F32, 256),
    ("15M", synth.F32, 256),
    ("tinyq8", synth.Q8_0, 64),
    ("tinyq4", synth.Q4_0, 64),
])
def test_decode_small(name, dtype, steps, mode):
    need_gpu()
    cfg = {"tinyq8": TINY_Q8, "tinyq4": TINY_Q4}.get(name) or synth.CONFIGS[name]
    blob, orc, fed = _trajectory(cfg, dtype, steps)
    with l2d.Context(blob, dtype) as ctx:
        set_mode(ctx, mode)
        st = decode_and_compare(ctx, orc, fed, label=f"{name} dt{dtype} {mode}")
    st.assert_ok()


GS_Q8 = synth.Config("gsq8", 256, 512, 2, 8, 2, 320, 48, 13, (synth.Q8_0,))


@pytest.mark.parametrize("gs", [16, 32, 128, 256])
def test_decode_q8_group_sizes(gs):
    """Q8_0 at every group size the decode step takes besides 64: tile
    shapes change with the group size (down to one-row tiles handed out in
    pairs to the RoPE and SwiGLU epilogues at 128 and 256)."""
    need_gpu()
    cfg = GS_Q8
    blob = synth.make_blob(cfg, synth.Q8_0, gs=gs)
    orc = oracle.Model(blob, synth.Q8_0, gs=gs)
    forced, _ = synth.trajectory_plan(cfg, 40)
    fed, _, _ = oracle.trajectory(orc, forced, 40, keep_logits=False)
    orc.reset_kv()
    with l2d.Context(blob, synth.Q8_0, group_size=gs) as ctx:
        set_mode(ctx, "graph")
        st = decode_and_compare(ctx, orc, fed, label=f"gsq8 gs{gs}")
    orc.close()
    st.assert_ok()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("dtype", [synth.F32, synth.Q8_0])
def test_decode_110m_full_trajectory(dtype, mode):
    need_gpu()
    cfg = synth.CONFIGS["110M"]
    blob, orc, fed = _trajectory(cfg, dtype, cfg.seq_len)
    with l2d.Context(blob, dtype) as ctx:
        set_mode(ctx, mode)
        st = decode_and_compare(ctx, orc, fed, label=f"110M dt{dtype} {mode}")
    st.assert_ok()


def test_graph_and_eager_agree_and_repeat_bitwise():
    """The captured graph and kernel-by-kernel launches give identical bits,
    and re-running a (token, pos) is idempotent (same cache slot, same bits)."""
    need_gpu()
    cfg = synth.CONFIGS["15M"]
    blob = synth.make_blob(cfg, synth.F32)
    with l2d.Context(blob, synth.F32) as ctx:
        ctx.use_persistent(False)
        outs = []
        for graph in (True, False):
            ctx.reset_kv()
            ctx.use_graph(graph)
            for p, t in enumerate([1, 50, 7, 9000]):
                ctx.forward(t, p)
            outs.append(ctx.logits())
        np.testing.assert_array_equal(outs[0], outs[1])
        ctx.use_graph(True)
        ctx.forward(9000, 3)
        np.testing.assert_array_equal(ctx.logits(), outs[0])


@pytest.mark.parametrize("mode", MODES)
def test_greedy_on_device_matches_host_loop(mode):
    need_gpu()
    cfg = synth.CONFIGS["tiny"]
    blob = synth.make_blob(cfg, synth.F32)
    orc = oracle.Model(blob, synth.F32)
    fed, am, _ = oracle.trajectory(orc, np.array([1], np.int32), 40, keep_logits=False)
    with l2d.Context(blob, synth.F32) as ctx:
        set_mode(ctx, mode)
        ctx.forward(1, 0)
        toks = [ctx.last_token()]
        for p in range(1, 40):
            ctx.forward_greedy(p)
            toks.append(ctx.last_token())
    np.testing.assert_array_equal(np.array(toks), am)


def test_bad_arguments_return_errors():
    need_gpu()
    cfg = synth.CONFIGS["tiny"]
    blob = synth.make_blob(cfg, synth.F32)
    with l2d.Context(blob, synth.F32) as ctx:
        for t, p in ((-1, 0), (512, 0), (0, -1), (0, 512)):
            with pytest.raises(l2d.L2DError):
                ctx.forward(t, p)
        with pytest.raises(l2d.L2DError):
            ctx.forward_greedy(5)  # previous step was not at pos 4
        ctx.forward(1, 0)
        assert np.isfinite(ctx.logits()).all()


@pytest.mark.parametrize("chain", [False, True], ids=["per_phase", "chained"])
def test_q8_activation_codes_match_oracle(chain):
    """Per-layer quantised matvec inputs: codes equal the oracle's except
    where the oracle's |x|/scale lies within 1e-3 of k + 1/2; scales equal
    within 1e-5 relative. Also with chained launches, whose output
    projection and w2 take their inputs after a wait, the latter from the
    one-group-per-line codes."""
    need_gpu()
    cfg = synth.CONFIGS["110M"]
    blob = synth.make_blob(cfg, synth.Q8_0)
    orc = oracle.Model(blob, synth.Q8_0)
    fed = [1, 300, 5000, 12, 31999]
    layer = 7
    orc.trace_layer(layer)
    n_ties = n_codes = 0
    with l2d.Context(blob, synth.Q8_0) as ctx:
        ctx.use_chain(chain)
        ctx.trace_layer(layer)
        for p, t in enumerate(fed):
            ctx.forward(t, p)
            ctx.sync()
            orc.forward(t, p)
            for slot in range(4):
                gq, gsc = ctx.trace(slot)
                oq, osc, of = orc.trace(slot)
                np.testing.assert_allclose(gsc, osc, rtol=1e-5, atol=0)
                diff = gq != oq
                if diff.any():
                    ratio = np.abs(of.astype(np.float64)) / np.repeat(osc.astype(np.float64), 64)
                    near = np.abs(ratio - np.floor(ratio) - 0.5) < 1e-3
                    assert (near[diff]).all(), (p, slot, np.nonzero(diff & ~near)[0][:5])
                    n_ties += int(diff.sum())
                n_codes += gq.size
    log(f"  codes compared {n_codes}, differing at near-ties {n_ties}")


def _fill_kv_both(ctx, orc, P, seed):
    """Place identical synthetic keys/values in slots 0..P-1 of every layer."""
    import torch
    L, kvd = ctx.n_layers, ctx.kv_dim
    kc_o, vc_o = orc.key_cache(), orc.value_cache()
    kc_g, vc_g = ctx.kv_cache()
    for l in range(L):
        k = synth.normal_f32(seed, 2 * l, P * kvd, 1.0).reshape(P, kvd)
        v = synth.normal_f32(seed, 2 * l + 1, P * kvd, 1.0).reshape(P, kvd)
        kc_o[l, :P] = k
        vc_o[l, :P] = v
        kc_g[l, :P].copy_(torch.from_numpy(k))
        vc_g[l, :P].copy_(torch.from_numpy(v))
    torch.cuda.synchronize()


def _full_size(name, dtype, deep_positions, steps=3):
    torch = need_gpu()
    cfg = synth.CONFIGS[name]
    t = time.time()
    blob = synth.make_blob(cfg, dtype)
    log(f"  {name} dt{dtype}: blob {blob.size / 1e9:.2f} GB in {time.time() - t:.1f}s")
    orc = oracle.Model(blob, dtype)
    t = time.time()
    ctx = l2d.Context(blob, dtype)
    log(f"  init (upload + graph) {time.time() - t:.1f}s")
    from gpu_util import Stats
    # the graph always; the persistent step kernel where the model has it (Q8_0
    # with group size 64): an unavailable mode is left out, not the test
    modes = ["graph"]
    try:
        ctx.use_persistent(True)
        modes.append("stream")
    except l2d.L2DError:
        pass
    ctx.use_persistent(False)

    def check(p, r, what):
        # each mode rewrites cache slot p from the same inputs before using it
        for mode in modes:
            set_mode(ctx, mode)
            ctx.forward(fed[-1], p)
            st = Stats()
            st.add(p, ctx.logits(), r, ctx.last_token())
            log(f"  {what} {p} {mode}: {st.summary()}")
            st.assert_ok()

    try:
        fed = [1]
        for p in range(steps):
            r = orc.forward(fed[-1], p)
            check(p, r, "pos")
            fed.append(int(np.argmax(r)))
        for P in deep_positions:
            _fill_kv_both(ctx, orc, P, seed=77 + P)
            r = orc.forward(fed[-1], P)
            check(P, r, "deep pos")
    finally:
        ctx.close()
        orc.close()
        del blob
        gc.collect()
        torch.cuda.empty_cache()


def _long_trajectory(name, dtype, n_steps, deep_positions=(), modes=("graph",), max_flips=3):
    """Teacher-forced greedy decode of pos 0..n_steps-1 at full size: at each
    pos the oracle's step gives the logits to compare and, by its argmax, the
    token both sides take next (one oracle pass; the GPU step is enqueued
    before the oracle's so the two overlap). Then one step at each deep
    position over identical synthetic cache slots 0..pos-1.

    Q8_0 activation codes may round to the neighbouring code where the
    oracle's |x| / scale is within 1e-3 of k + 1/2 (near ties); one such
    flip moves that step's logits past the tolerance and then every later
    step through the cache. A step outside the tolerance is therefore
    audited: both sides re-run it with every layer's quantised inputs traced,
    and it passes only if the first differing input differs at near ties
    alone; the oracle's cache then replaces the device's and the run goes
    on. At most max_flips such steps per run."""
    torch = need_gpu()
    from gpu_util import Stats, copy_cache_from_oracle, near_tie_audit
    cfg = synth.CONFIGS[name]
    t = time.time()
    blob = synth.make_blob(cfg, dtype)
    log(f"  {name} dt{dtype}: blob {blob.size / 1e9:.2f} GB in {time.time() - t:.1f}s")
    orc = oracle.Model(blob, dtype)
    ctx = l2d.Context(blob, dtype)
    try:
        for mode in modes:
            set_mode(ctx, mode)
            ctx.reset_kv()
            orc.reset_kv()
            st = Stats()
            tok = 1
            flips = []
            t0 = t1 = time.time()
            for p in range(n_steps):
                ctx.forward(tok, p)
                r = orc.forward(tok, p)
                nbad = len(st.bad)
                st.add(p, ctx.logits(), r, ctx.last_token())
                if len(st.bad) > nbad and dtype != synth.F32 and len(flips) < max_flips:
                    # a step outside the tolerance: allowed only when its first
                    # differing quantised input differs at near ties (the two
                    # sides' fp64 sums may round one fp32 ulp apart); then
                    # both sides continue from the oracle's cache
                    layer, slot, nd, ok = near_tie_audit(ctx, orc, tok, p, cfg.n_layers)
                    log(f"  [{name} dt{dtype} {mode}] pos {p}: first differing input layer {layer} slot {slot}, "
                        f"{nd} codes, near ties only: {ok}")
                    if ok:
                        del st.bad[nbad:]
                        flips.append((p, layer, slot, nd))
                        copy_cache_from_oracle(ctx, orc, p)
                tok = int(np.argmax(r))
                if time.time() - t1 > 30:
                    log(f"  [{name} dt{dtype} {mode}] pos {p} ({time.time() - t0:.0f}s): {st.summary()}")
                    t1 = time.time()
            log(f"  [{name} dt{dtype} {mode}] pos 0..{n_steps - 1}: {st.summary()}; "
                f"near-tie steps (pos, layer, slot, codes): {flips}")
            st.assert_ok()
            assert st.steps == n_steps and st.argmax_checked > 0
            for P in deep_positions:
                _fill_kv_both(ctx, orc, P, seed=77 + P)
                r = orc.forward(tok, P)
                ctx.forward(tok, P)
                sd = Stats()
                sd.add(P, ctx.logits(), r, ctx.last_token())
                log(f"  [{name} dt{dtype} {mode}] deep pos {P}: {sd.summary()}")
                sd.assert_ok()
    finally:
        ctx.close()
        orc.close()
        del blob
        gc.collect()
        torch.cuda.empty_cache()


def test_decode_7b_fp32_trajectory():
    """7B fp32: pos 0..255 (the logits tolerance after 256 steps), then deep
    positions 512 and 2048 over injected caches."""
    _long_trajectory("7B", synth.F32, 256, [512, 2048])


def test_decode_7b_q8_trajectory():
    """7B Q8_0: pos 0..2048, the decode length of the workload."""
    _long_trajectory("7B", synth.Q8_0, 2049)


def test_decode_7b_q4_full_size():
    _full_size("7B", synth.Q4_0, [512, 2048])


def test_decode_110m_q4_trajectory():
    """110M with 4-bit weights, 512 teacher-forced steps (graph replay)."""
    need_gpu()
    cfg = synth.CONFIGS["110M"]
    blob, orc, fed = _trajectory(cfg, synth.Q4_0, 512)
    with l2d.Context(blob, synth.Q4_0) as ctx:
        set_mode(ctx, "graph")
        st = decode_and_compare(ctx, orc, fed, label="110M Q4_0 graph")
    st.assert_ok()


def test_decode_13b_q8_full_size():
    _full_size("13B", synth.Q8_0, [4095], steps=2)


def test_decode_13b_fp32_full_size():
    _full_size("13B", synth.F32, [1024], steps=2)


def test_decode_70b_q8_trajectory():
    """70B Q8_0 (GQA, 8 query heads per kv head): pos 0..63, then pos 1024,
    2048 and 4095 over injected caches."""
    _long_trajectory("70B", synth.Q8_0, 64, [1024, 2048, 4095])
