"""The seeded input generator: deterministic, thread-count independent, with
the shapes and value distributions the workloads call for."""
import numpy as np

import oracle
import synth
from blobview import view


def test_blob_deterministic_and_thread_independent():
    cfg = synth.CONFIGS["tiny"]
    oracle.set_threads(1)
    a = synth.make_blob(cfg, synth.F32)
    oracle.set_threads(4)
    b = synth.make_blob(cfg, synth.F32)
    np.testing.assert_array_equal(a, b)
    c = synth.make_blob(cfg, synth.F32, seed=cfg.seed + 1)
    assert (a[28:] != c[28:]).any()


def test_value_distributions():
    cfg = synth.CONFIGS["110M"]
    w = view(synth.make_blob(cfg, synth.F32), synth.F32)
    x = w["w1"].astype(np.float64).ravel()
    assert abs(x.mean()) < 1e-4 and abs(x.std() - 0.02) < 2e-4
    # normal, not a bounded bell: kurtosis 3, tail mass beyond 3 sd near
    # 0.27%, largest of 1.6 M draws beyond 4.5 sd
    z = x / 0.02
    assert abs((z ** 4).mean() - 3.0) < 0.05
    assert abs((np.abs(z) > 3).mean() - 0.0027) < 0.0005
    assert 4.5 < np.abs(z).max() < 6.8
    assert (w["rms_att"] == 1).all() and (w["rms_ffn"] == 1).all() and (w["rms_final"] == 1).all()
    wq = view(synth.make_blob(cfg, synth.Q8_0), synth.Q8_0)
    q = wq["w1.q"].astype(np.int64).ravel()
    assert q.min() >= -127 and q.max() <= 127
    deq = (wq["w1.q"].reshape(-1, 64).astype(np.float64) * wq["w1.s"].reshape(-1, 1)).ravel()
    assert abs(deq.std() - 0.02) < 1e-3


def test_blob_sizes_and_header():
    for cfg in synth.CONFIGS.values():
        for dt in cfg.dtypes:
            n = synth.blob_bytes(cfg, dt)
            assert n > 0
    cfg = synth.CONFIGS["7B"]
    assert synth.blob_bytes(cfg, synth.F32) == 26_955_759_644
    assert synth.blob_bytes(cfg, synth.Q8_0) == 7_162_445_852
    blob = synth.make_blob(synth.CONFIGS["tiny"], synth.F32)
    assert tuple(np.frombuffer(blob[:28].tobytes(), np.int32)) == synth.CONFIGS["tiny"].header()


def test_invalid_configs_rejected():
    bad = synth.CONFIGS["tiny"].replace(dim=60)  # 60 % 8 heads != 0
    assert synth.blob_bytes(bad, synth.F32) < 0
    assert synth.blob_bytes(synth.CONFIGS["tiny"], synth.Q8_0) < 0  # 172 % 64 != 0


def test_prompt_ids_in_range():
    p = synth.prompt(1002, 16, 32000)
    assert p.min() >= 0 and p.max() < 32000 and len(set(p.tolist())) > 10
