"""Helpers for the GPU parity tests: run the HIP path and the oracle on the
same seeded inputs and compare them element by element."""
from __future__ import annotations

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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


MODES = ("persistent", "graph")

# The persistent step kernel faulted on its first MI355X run (tiny fp32
# model, first step) and the cause is not found; it stays off and its cases
# are skipped until a cause is shown and fixed.
PERSISTENT_SKIP = "persistent step kernel disabled: memory access fault on first run, cause not yet found"


def set_mode(ctx, mode: str):
    """persistent: the whole step as one kernel; graph: the captured graph
    of per-phase kernels. Skips when the persistent kernel is unavailable."""
    if mode == "persistent":
        pytest.skip(PERSISTENT_SKIP)
        try:
            ctx.use_persistent(True)
        except Exception as e:  # noqa: BLE001 - the library's error names the reason
            pytest.skip(f"persistent step kernel unavailable: {e}")
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
