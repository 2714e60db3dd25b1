"""Host logic of bench.py (no GPU): kernel-name shortening, the rocprofv3
CSV summaries and the rule that a committed summary counts only while the
decode kernels' sources are unchanged."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_short_kernel_name():
    assert bench.short_kernel_name("void l2d::gemv_kernel<1, 1, 3, 2, 4, 1, 2, false>(l2d::GemvParams)") == \
        "gemv_kernel<1,1,3,2,4,1,2>"
    assert bench.short_kernel_name("void l2d::attention_kernel<4, 128>(l2d::AttnParams)") == "attention_kernel<4,128>"
    # the test-hook instance keeps its flag
    assert bench.short_kernel_name("void l2d::gemv_kernel<1, 0, 0, 2, 4, 1, 2, true>(l2d::GemvParams)") == \
        "gemv_kernel<1,0,0,2,4,1,2,true>"
    assert bench.kernel_role("gemv_kernel<1,1,3,2,4,1,2>").startswith("Q8_0 w1/w3")
    assert bench.kernel_role("attention_kernel<1,128>").startswith("attention")


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summaries_from_csv(tmp_path):
    w13 = "void l2d::gemv_kernel<1, 1, 3, 2, 4, 1, 2, false>(l2d::GemvParams)"
    copy = "__amd_rocclr_copyBuffer"
    _write(str(tmp_path / "st" / "h" / "run_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [[w13, 4, 88000, 22000, 50, 21000, 23000, 1], [copy, 1, 500, 500, 1, 500, 500, 0]])
    out = tmp_path / "stats.txt"
    bench.summarize_stats(str(tmp_path / "st"), str(out), "T", "cmd")
    f = bench.read_summary(str(out))
    assert float(f["avg_ns_gemv_kernel<1,1,3,2,4,1,2>"]) == 22000.0
    assert f["sources_sha256"] == bench.sources_digest()

    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # the copy moves 1 GiB each way: FETCH_SIZE reads half, WRITE_SIZE all
    _write(str(tmp_path / "pf" / "run_counter_collection.csv"), hdr,
           [[1, copy, "FETCH_SIZE", 524288.0], [2, w13, "FETCH_SIZE", 47000.0], [3, w13, "FETCH_SIZE", 47002.0]])
    _write(str(tmp_path / "pw" / "run_counter_collection.csv"), hdr,
           [[1, copy, "WRITE_SIZE", 1048576.0], [2, w13, "WRITE_SIZE", 431.0], [3, w13, "WRITE_SIZE", 431.0]])
    tout = tmp_path / "traffic.txt"
    bench.summarize_traffic(str(tmp_path / "pf"), str(tmp_path / "pw"), str(tout), "T", ["a", "b"])
    t = bench.read_summary(str(tout))
    assert float(t["hbm_bytes_w13"]) == pytest.approx((2.0 * 47001.0 + 431.0) * 1024, rel=1e-9)


def test_committed_profile_needs_matching_sources(tmp_path, monkeypatch):
    st = tmp_path / "k.txt"
    st.write_text("sources_sha256: " + "0" * 64 + "\navg_ns_gemv_kernel<1,1,3,2,4,1,2>: 22000.0\n")
    monkeypatch.setattr(bench, "STATS_FILE", str(st))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.committed_profile("gemv_kernel<1,1,3,2,4,1,2>") is None
    st.write_text(f"sources_sha256: {bench.sources_digest()}\navg_ns_gemv_kernel<1,1,3,2,4,1,2>: 22000.0\n")
    assert bench.committed_profile("gemv_kernel<1,1,3,2,4,1,2>") == {"avg_us": 22.0}


def test_step_bytes_match_the_survey_figures():
    import synth
    b = bench.step_bytes(synth.CONFIGS["7B"], 1, 512)
    assert b["w13"] == 2 * 11008 * 4096 * 1.0625 == 95813632
    assert b["total"] == pytest.approx(7.56e9, rel=2e-3)
    assert bench.step_bytes(synth.CONFIGS["7B"], 0, 512)["total"] == pytest.approx(26.97e9, rel=2e-3)


class _FakeTraceCtx:
    """Two workgroups, a 5-layer model: every event of phase p at a fixed
    offset from its phase start, phases 10 us apart (clock of 100 MHz)."""

    L = 5

    def stream_shape(self):
        return 2, 4

    def stream_trace(self, token, pos, nwg, nwk):
        import numpy as np
        NP = 4 * self.L + 1
        E = 1 + 6 * NP
        ctl = np.zeros((nwg, E), np.uint64)
        for b in range(nwg):
            ctl[b, 0] = 1000
            for p in range(NP):
                t0 = 1000 + 1000 * p + 10 * b
                # start, flags seen +1 us, ready +3, workers +8, published +9, attention +9.5
                for i, dt in zip(range(1, 7), (0, 100, 300, 800, 900, 950)):
                    ctl[b, i + 6 * p] = t0 + dt
        return ctl, np.zeros((nwg, nwk, NP), np.uint64)


def test_stream_trace_summary():
    cfg = type("C", (), {"n_layers": _FakeTraceCtx.L})()
    tr = bench.stream_trace(_FakeTraceCtx(), cfg, 1, 3)
    for n in ("qkv", "wo", "w13", "w2"):
        assert tr[n]["wait_us"] == pytest.approx(1.0)
        assert tr[n]["prologue_us"] == pytest.approx(2.0)
        assert tr[n]["workers_us"] == pytest.approx(5.0)
        assert tr[n]["epilogue_us"] == pytest.approx(1.0)
        assert tr[n]["publish_spread_us"] == pytest.approx(0.05)
    assert tr["qkv"]["attention_us"] == pytest.approx(0.5)
    assert "attention_us" not in tr["wo"]
    assert tr["per_layer_us"] == pytest.approx(40.0)
    text = bench.format_stream_trace(tr, "title", "python bench.py")
    assert "per_layer_us: 40.00" in text and text.startswith("title\n=====")
