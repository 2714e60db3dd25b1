"""Helpers for the GPU parity tests: run the HIP path and the oracle on the
same seeded inputs and compare them element by element."""
from __future__ import annotations

import os
import sys
import time

import numpy as np
import pytest

# fp32 logits tolerance: |gpu - oracle| <= ATOL + RTOL * |oracle| for every
# vocab entry at every step
ATOL = 1e-3
RTOL = 1e-4
# argmax must agree wherever the oracle's top-2 margin exceeds this
MARGIN = 1e-3


_PROGRESS = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")


def log(*a):
    """Progress line to stderr and, when a gpurun_out/ folder exists at the
    repository root, to gpurun_out/gpu_tests_progress.log (pytest captures
    stderr; the file shows a long test's steps while it runs)."""
    msg = " ".join(str(x) for x in a)
    print(msg, file=sys.stderr, flush=True)
    if os.path.isdir(_PROGRESS):
        with open(os.path.join(_PROGRESS, "gpu_tests_progress.log"), "a") as f:
            f.write(msg + "\n")


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


MODES = ("persistent", "graph", "stream")

# The first persistent step kernel (one 512-thread workgroup per CU, fp32 and
# Q8_0) faulted on its first MI355X run (tiny fp32 model, first step) and
# the cause was not found; that kernel was removed. Its cases stay skipped.
# The step kernel the library has now ("stream": worker waves streaming the
# weights, control waves running barriers, prologues, epilogues and
# attention) is a new design, Q8_0 with group size 64 only.
PERSISTENT_SKIP = ("first persistent step kernel: memory access fault on its first run (tiny fp32, step 0), "
                   "cause not found; the kernel was removed")


def set_mode(ctx, mode: str):
    """persistent: the removed first step kernel (skipped); graph: the
    captured graph of per-phase kernels; stream: the persistent step kernel
    (skips where the model is not Q8_0 with group size 64)."""
    if mode == "persistent":
        pytest.skip(PERSISTENT_SKIP)
    elif mode == "stream":
        try:
            ctx.use_persistent(True)
        except Exception as e:  # noqa: BLE001 - the library's error names the reason
            pytest.skip(f"persistent step kernel not available: {e}")
    else:
        ctx.use_persistent(False)
        ctx.use_graph(True)


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in fp32 units-in-the-last-place (same sign assumed mostly)."""
    ai = a.astype(np.float32).view(np.int32).astype(np.int64)
    bi = b.astype(np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


class Stats:
    def __init__(self):
        self.max_abs = 0.0
        self.max_rel = 0.0
        self.n = 0
        self.exact = 0
        self.steps = 0
        self.argmax_checked = 0
        self.argmax_same = 0
        self.bad = []

    def add(self, pos, gpu, ref, gpu_tok=None):
        d = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
        self.max_abs = max(self.max_abs, float(d.max()))
        self.max_rel = max(self.max_rel, float((d / np.maximum(np.abs(ref), 1e-30)).max()))
        self.n += gpu.size
        self.exact += int((gpu == ref).sum())
        self.steps += 1
        ok = d <= ATOL + RTOL * np.abs(ref.astype(np.float64))
        if not ok.all():
            self.bad.append((pos, int((~ok).sum()), float(d.max())))
        if gpu_tok is not None:
            top2 = np.partition(ref, -2)[-2:]
            margin = float(top2[1] - top2[0])
            if margin > MARGIN:
                self.argmax_checked += 1
                want = int(np.argmax(ref))
                if gpu_tok == want:
                    self.argmax_same += 1
                else:
                    self.bad.append((pos, "argmax", gpu_tok, want, margin))

    def summary(self) -> str:
        return (f"steps={self.steps} max|d|={self.max_abs:.3g} max rel={self.max_rel:.3g} "
                f"bit-exact={self.exact / max(self.n, 1):.6f} "
                f"argmax {self.argmax_same}/{self.argmax_checked}")

    def assert_ok(self):
        assert not self.bad, f"{self.summary()} failures (first 5): {self.bad[:5]}"


def decode_and_compare(ctx, orc, fed: np.ndarray, start: int = 0, label: str = "") -> Stats:
    """Teacher-forced decode: both sides take fed[p] at pos start+p."""
    st = Stats()
    t0 = time.time()
    for i, tok in enumerate(fed):
        p = start + i
        ctx.forward(int(tok), p)
        g = ctx.logits()
        gt = ctx.last_token()
        r = orc.forward(int(tok), p)
        st.add(p, g, r, gt)
        if time.time() - t0 > 20:
            log(f"  [{label}] pos {p}: {st.summary()}")
            t0 = time.time()
    log(f"  [{label}] {st.summary()}")
    return st


# Q8_0 activation codes may differ from the oracle's where the oracle's
# |x| / scale lies within this distance of k + 1/2: the two sides sum in
# different fp64 orders, and a value one fp32 ulp away from the oracle's can
# round to the neighbouring code
NEAR_TIE = 1e-3


def near_tie_audit(ctx, orc, tok: int, pos: int, n_layers: int):
    """Re-run step pos on both sides with the quantised matvec inputs
    traced (the oracle every layer in one pass, the device one layer per
    pass), compared in layer and slot order up to the first input whose
    codes or scales differ. Returns (layer, slot, n_codes_differing, ok):
    ok when every differing code sits at a near tie of the oracle's value
    and every scale agrees within 1e-5 relative; (None, None, 0, False)
    when nothing differs. Re-running a (token, pos) rewrites the same cache
    slot with the same values on both sides."""
    try:
        orc.trace_layer(-2)  # one oracle pass records every layer
        orc.forward(tok, pos)
        for layer in range(n_layers):
            ctx.trace_layer(layer)
            ctx.forward(tok, pos)
            ctx.sync()
            for slot in range(4):
                gq, gsc = ctx.trace(slot)
                oq, osc, of = orc.trace_at(layer, slot)
                diff = gq != oq
                sdiff = gsc != osc
                if not diff.any() and not sdiff.any():
                    continue
                gs = gq.size // gsc.size
                ok = bool(np.all(np.abs(gsc.astype(np.float64) - osc) <= 1e-5 * np.abs(osc.astype(np.float64))))
                if diff.any():
                    sc = np.repeat(osc.astype(np.float64), gs)
                    ratio = np.abs(of.astype(np.float64)) / np.where(sc > 0, sc, 1.0)
                    near = np.abs(ratio - np.floor(ratio) - 0.5) < NEAR_TIE
                    ok = ok and bool(near[diff].all())
                return layer, slot, int(diff.sum()), ok
        return None, None, 0, False
    finally:
        ctx.trace_layer(-1)
        orc.trace_layer(-1)


def copy_cache_from_oracle(ctx, orc, upto: int):
    """Overwrite the device KV cache slots 0..upto of every layer with the
    oracle's (after a near-tie code flip, so that later steps start from the
    same state on both sides)."""
    import torch
    kc_o, vc_o = orc.key_cache(), orc.value_cache()
    kc_g, vc_g = ctx.kv_cache()
    for l in range(kc_o.shape[0]):
        kc_g[l, :upto + 1].copy_(torch.from_numpy(np.ascontiguousarray(kc_o[l, :upto + 1])))
        vc_g[l, :upto + 1].copy_(torch.from_numpy(np.ascontiguousarray(vc_o[l, :upto + 1])))
    torch.cuda.synchronize()
