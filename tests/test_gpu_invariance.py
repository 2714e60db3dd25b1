"""Launch-shape invariance of the decode step, through the C ABI: how the
work is laid out on the GPU must not change a single bit of the result.

- Attention: the query heads that share a kv head may be spread over 1, 2,
  4 or 8 workgroups (each head's computation and the merge order over
  position ranges are the same), so logits and the sampled tokens must be
  bit-identical.
- Matvecs: 1 to 4 workgroups per CU change which wave streams which rows,
  not how any row is summed, nor how the SwiGLU output is quantised for the
  w2 matvec (one group at a time, by whichever wave completes it).

- Attention split count: 1 or 3 workgroups per CU cut the positions of
  each kv head into different ranges, so the fp64 merge sums in another
  order. Logits then agree to rounding, not bit for bit: they are held to
  the logits tolerance against the default split at every step, and the
  argmax must agree wherever the top-2 margin exceeds the tie margin.

These settings are read when a context is created (environment variables of
the library), so each run builds its own context."""
import os

import numpy as np
import pytest

import llama_transformer_decode_amd as l2d
import synth
from gpu_util import ATOL, MARGIN, RTOL, log, need_gpu

pytestmark = pytest.mark.gpu

GQA8_Q8 = synth.Config("gqa8q8", 256, 512, 2, 8, 1, 320, 96, 12, (synth.Q8_0,))


def _run(blob, dtype, steps: int, env: dict) -> tuple:
    saved = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        with l2d.Context(blob, dtype) as ctx:
            ctx.forward(1, 0)
            logits, toks = [ctx.logits().copy()], [ctx.last_token()]
            for p in range(1, steps):
                ctx.forward_greedy(p)
                logits.append(ctx.logits().copy())
                toks.append(ctx.last_token())
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return np.stack(logits), toks


@pytest.mark.parametrize("dtype", [synth.Q8_0, synth.F32], ids=["q8_0", "fp32"])
def test_attention_head_split_bitwise(dtype):
    """8 query heads per kv head: 1, 2, 4 and 8 workgroups per kv head."""
    torch = need_gpu()
    blob = synth.make_blob(GQA8_Q8, dtype)
    ref_l, ref_t = _run(blob, dtype, 40, {"L2D_ATTN_GSPLIT": "1"})
    for gsplit in ("2", "4", "8"):
        lg, tk = _run(blob, dtype, 40, {"L2D_ATTN_GSPLIT": gsplit})
        diff = np.abs(lg.astype(np.float64) - ref_l).max()
        log(f"  gsplit {gsplit}: max |d logits| {diff:.3g}, tokens equal {tk == ref_t}")
        assert np.array_equal(lg, ref_l) and tk == ref_t
    torch.cuda.synchronize()


def test_gemv_grid_bitwise():
    """110M Q8_0: 1, 2, 3 and 4 matvec workgroups per CU."""
    torch = need_gpu()
    cfg = synth.CONFIGS["110M"]
    blob = synth.make_blob(cfg, synth.Q8_0)
    ref_l, ref_t = _run(blob, synth.Q8_0, 24, {"L2D_GEMV_WG_PER_CU": "2"})
    for per_cu in ("1", "3", "4"):
        lg, tk = _run(blob, synth.Q8_0, 24, {"L2D_GEMV_WG_PER_CU": per_cu})
        diff = np.abs(lg.astype(np.float64) - ref_l).max()
        log(f"  {per_cu} workgroups per CU: max |d logits| {diff:.3g}, tokens equal {tk == ref_t}")
        assert np.array_equal(lg, ref_l) and tk == ref_t
    torch.cuda.synchronize()


def _run_fed(blob, dtype, tokens, env: dict) -> np.ndarray:
    saved = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        with l2d.Context(blob, dtype) as ctx:
            out = []
            for p, t in enumerate(tokens):
                ctx.forward(int(t), p)
                out.append(ctx.logits().copy())
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return np.stack(out)


def test_attention_split_count_agrees():
    """110M Q8_0, a fixed token sequence to pos 700: 1 and 3 (default)
    attention workgroups per CU, i.e. 21 and 32 splits per kv head (the
    latter capped by the context's sub-chunk count), 11 and 22 active
    position ranges at pos 700."""
    torch = need_gpu()
    cfg = synth.CONFIGS["110M"]
    blob = synth.make_blob(cfg, synth.Q8_0)
    tokens = synth.prompt(5, 701, cfg.vocab)
    ref = _run_fed(blob, synth.Q8_0, tokens, {"L2D_ATTN_WG_PER_CU": "3"}).astype(np.float64)
    top2 = np.sort(ref, axis=1)[:, -2:]
    decided = top2[:, 1] - top2[:, 0] > MARGIN
    for per_cu in ("1",):
        lg = _run_fed(blob, synth.Q8_0, tokens, {"L2D_ATTN_WG_PER_CU": per_cu}).astype(np.float64)
        diff = np.abs(lg - ref)
        log(f"  {per_cu} workgroups per CU: max |d logits| {diff.max():.3g}")
        assert (diff <= ATOL + RTOL * np.abs(ref)).all()
        assert (np.argmax(lg, axis=1) == np.argmax(ref, axis=1))[decided].all()
    torch.cuda.synchronize()
