"""Decode-step benchmark of the MI355X Llama-2 decode library.

One step = one pass of the whole decode step (embedding, every layer's
RMSNorm, q/k/v matvec, RoPE, KV-cache write, GQA attention, output matvec,
SwiGLU FFN, residuals, final norm, classifier and argmax) for one token at
batch 1, replayed as the captured HIP graph. Weights are random N(0, 0.02)
of the 7B shape (synthetic, seeded), resident in HBM before timing starts.

The cache is filled by a real greedy decode from pos 0 (on device, no host
round trip). At each reported position the step is replayed K times at that
same position (re-running (token, pos) rewrites the same cache slot with the
same values), timed with HIP events on the context's stream between two
synchronisations.

Each position is timed in TRIALS trials of K replays (default 3); a
trial's rate is K / (its event-timed seconds) and every figure is the
median trial. The GPU clocks (rocm-smi) are recorded before and after.

Prints one JSON line. value = tokens/s of the Q8_0 step at the headline
position. Under "detail" ride along: per-position, fp32 and Q4_0 (4-bit
weights) figures, the step with sampling on, the step as one persistent
kernel launch ("stream"), the 70B-shape Q8_0 step (GQA, 8 kv heads) at
pos 1, 2048 and 4095, the batched prefill of a 512-token prompt (int8
MFMA for Q8_0, fp64 MFMA for fp32) and the Q4_0 matvec on the step's
matrix shapes. cpu_baseline is the oracle on the host cores (threads =
physical cores), with per-config rates and one-core rates of the small
configs under its "per_config".

The same file turns rocprofv3 CSV output into the text summaries kept
under profiles/ (--summarize-stats, --summarize-traffic).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
CSRC = os.path.join(ROOT, "llama_transformer_decode_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_7B_decode_step_q8_0.txt")
STATS_FILE = os.path.join(ROOT, "profiles", "kernels_7B_decode_step.txt")
# the sources the step's decode kernels are built from: a committed summary
# counts only while their digest is the one it records
STEP_SOURCES = ("gemv_core.hpp", "gemv.hip", "attn_decode.hpp", "attn.hip", "attn_core.hpp", "device.hpp",
                "step.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_bytes(cfg, dtype: int, pos: int, gs: int = 64) -> dict:
    """Algorithmic HBM bytes of one step at pos: every matvec weight once
    (with Q8_0 scales), one embedding row, the KV rows read (slots 0..pos)
    and the k/v slot written."""
    d, h, L, V = cfg.dim, cfg.hidden_dim, cfg.n_layers, cfg.vocab
    kvd = cfg.kv_dim
    # bytes per weight: fp32 4; Q8_0 code byte + scale share; Q4_0 half a
    # byte + a 4-byte scale per 32
    bpp = 4.0 if dtype == 0 else 1.0 + 4.0 / gs if dtype == 1 else 0.5 + 4.0 / 32
    qkv = (d + 2 * kvd) * d * bpp
    wo = d * d * bpp
    w13 = 2 * h * d * bpp
    w2 = d * h * bpp
    cls = V * d * bpp
    emb_row = d * bpp
    kv_read = 2 * (pos + 1) * kvd * 4
    kv_write = 2 * kvd * 4
    total = L * (qkv + wo + w13 + w2 + kv_read + kv_write) + cls + emb_row
    return {"total": total, "qkv": qkv, "wo": wo, "w13": w13, "w2": w2, "cls": cls,
            "attn": kv_read}


def time_replays(ctx, token: int, pos: int, steps: int, warmup: int, torch, trials: int = 1) -> dict:
    """Seconds per step at (token, pos): `warmup` untimed replays, then
    `trials` trials of `steps` replays, each timed with HIP events on the
    context's stream between two synchronisations. Returns the median
    trial and every trial."""
    stream = torch.cuda.ExternalStream(ctx.stream_handle())
    for _ in range(warmup):
        ctx.forward(token, pos)
    ctx.sync()
    torch.cuda.synchronize()
    per = []
    for _ in range(trials):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            ctx.forward(token, pos)
        end.record(stream)
        ctx.sync()
        torch.cuda.synchronize()
        per.append(start.elapsed_time(end) / 1e3 / steps)
    return {"sec": statistics.median(per), "trials_ms": [t * 1e3 for t in per]}


def kernel_times(ctx, token: int, pos: int, reps: int) -> dict:
    """Average duration (s) of each kernel class of the step, from HIP events
    stamped at every kernel's own start and end on the context's stream
    (kernel-by-kernel launches, same kernels and grids as the graph)."""
    return ctx.kernel_profile(token, pos, reps)


def sources_digest() -> str:
    h = hashlib.sha256()
    for f in STEP_SOURCES:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def read_summary(path: str) -> dict:
    """key: value lines of a committed profile summary"""
    fields = {}
    try:
        for line in open(path):
            m = re.match(r"^([a-z_0-9<>,]+): (.*)$", line.strip())
            if m:
                fields[m.group(1)] = m.group(2)
    except OSError:
        pass
    return fields


def committed_profile(kernel: str) -> dict | None:
    """Average duration (rocprofv3 kernel trace) and HBM bytes per launch
    (FETCH_SIZE / WRITE_SIZE, copy-calibrated) of one decode-step kernel
    from the committed summaries, each only while the sources match."""
    dig = sources_digest()
    out = {}
    st = read_summary(STATS_FILE)
    if st.get("sources_sha256") == dig and f"avg_ns_{kernel}" in st:
        out["avg_us"] = float(st[f"avg_ns_{kernel}"]) / 1e3
    tr = read_summary(TRAFFIC_FILE)
    if tr.get("sources_sha256") == dig:
        for k, v in tr.items():
            if k.startswith("hbm_bytes_"):
                out.setdefault("traffic", {})[k[len("hbm_bytes_"):]] = float(v)
    return out or None


def gpu_clocks() -> dict:
    """Current GPU clocks as rocm-smi reports them (sclk, mclk, fclk, ...)."""
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=30)
    except (OSError, subprocess.TimeoutExpired) as e:
        return {"error": str(e)}
    out = {}
    for line in r.stdout.splitlines():
        m = re.search(r"(\w+) clock level: \d+: \(?(\d+)\s*Mhz\)?", line, re.I)
        if m:
            out[m.group(1).lower() + "_mhz"] = int(m.group(2))
    if not out:
        out["raw"] = " | ".join(x.strip() for x in r.stdout.splitlines() if "clock" in x.lower())[:400]
    return out


def cpu_info() -> dict:
    """Host CPU model and physical core count (lscpu)."""
    info = {}
    try:
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=30)
        for line in r.stdout.splitlines():
            k, _, v = line.partition(":")
            if k.strip() == "Model name":
                info["model"] = v.strip()
        r = subprocess.run(["lscpu", "-p=core,socket"], capture_output=True, text=True, timeout=30)
        cores = {l for l in r.stdout.splitlines() if l and not l.startswith("#")}
        info["physical_cores"] = len(cores)
        info["logical_cpus"] = os.cpu_count()
    except (OSError, subprocess.TimeoutExpired) as e:
        info["error"] = str(e)
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except OSError:
        pass
    return info


def gemv_q40_rates(cfg, torch, l2d, reps: int = 20) -> dict:
    """The Q4_0 matvec (4-bit weights, groups of 32) on the step's matrix
    shapes: mean kernel duration (HIP events stamped at each kernel's start
    and end) and algorithmic GB/s (packed nibbles, fp32 scales, the fp32
    input and output once). Every shape cycles through
    enough distinct weight copies (>= 1 GiB together) that no launch finds
    its matrix in the 256 MB last-level cache. Weights are seeded random
    bytes and scales (every nibble pattern is valid Q4_0 data)."""
    d, h, V, kvd = cfg.dim, cfg.hidden_dim, cfg.vocab, cfg.kv_dim
    shapes = {"qkv": (d + 2 * kvd, d), "wo": (d, d), "w13": (2 * h, d), "w2": (d, h), "cls": (V, d)}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4040)
    out = {}
    for name, (rows, cols) in shapes.items():
        nbytes = rows * cols // 2 + rows * (cols // 32) * 4
        copies = max(2, -(-(1 << 30) // nbytes))
        Ws = [torch.randint(0, 256, (rows * cols // 2,), dtype=torch.uint8, device="cuda", generator=gen)
              for _ in range(copies)]
        Ss = [(torch.rand(rows * (cols // 32), device="cuda", generator=gen) - 0.5) * 3e-3
              for _ in range(copies)]
        x = torch.randn(cols, device="cuda", generator=gen)
        l2d.gemv_profile(l2d.Q4_0, Ws, Ss, x, rows, cols, 32, reps=copies)  # warm-up
        sec, _ = l2d.gemv_profile(l2d.Q4_0, Ws, Ss, x, rows, cols, 32, reps=max(reps, copies))
        alg = nbytes + cols * 4 + rows * 4
        out[name] = {"rows": rows, "cols": cols, "avg_us": sec * 1e6, "gbs": alg / sec / 1e9,
                     "alg_bytes": alg}
        log(f"[bench] q4_0 gemv {name} {rows}x{cols}: {sec * 1e6:.1f} us, {alg / sec / 1e9:.0f} GB/s")
        del Ws, Ss
        torch.cuda.empty_cache()
    return out


PEAK_INT8_TOPS = 5000.0  # MI355X dense int8 MFMA, 5.0 POP/s


def prefill_rates(cfg, ctx, torch, synth, n: int = 512, reps: int = 3) -> dict:
    """Batched prefill of an n-token prompt at pos 0: tokens/s over reps
    timed calls (HIP events on the context's stream), and the mean kernel
    time of each class from one kernel-stamped pass. The matmuls' rate is
    their multiply-adds (2 * rows * cols * n ops) per second: int8 MFMA ops
    for Q8_0, fp64 MFMA flops for fp32 weights."""
    toks = synth.prompt(4242, n, abs(cfg.vocab))
    stream = torch.cuda.ExternalStream(ctx.stream_handle())
    ctx.prefill(toks, 0)
    ctx.sync()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        ctx.prefill(toks, 0)
    e1.record(stream)
    ctx.sync()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    prof = ctx.prefill_profile(toks, 0)
    d, h, kvd = cfg.dim, cfg.hidden_dim, cfg.kv_dim
    shapes = {"qkv": (d + 2 * kvd, d), "wo": (d, d), "w13": (2 * h, d), "w2": (d, h)}
    kern = {}
    for k, v in prof.items():
        kern[k] = {"avg_us": v * 1e6}
        if k in shapes and v > 0:
            N, K = shapes[k]
            kern[k]["tops"] = 2.0 * N * K * n / v / 1e12
    out = {"tokens": n, "ms": sec * 1e3, "tok_s": n / sec, "kernels": kern}
    log(f"[bench] prefill of {n} tokens: {sec * 1e3:.2f} ms, {n / sec:.0f} tok/s; " +
        ", ".join(f"{k} {v['avg_us']:.1f}us" + (f" {v['tops']:.1f}TOP/s" if 'tops' in v else "")
                  for k, v in kern.items()))
    return out


def decode_to(ctx, positions, torch, fill=True):
    """Greedy decode from pos 0 through max(positions); returns the token fed
    at each requested position. Without fill the cache stays zero and the
    replays run at the requested positions directly (same bytes moved)."""
    if not fill:
        return {p: 1 for p in positions}
    last = max(positions)
    fed = {}
    ctx.forward(1, 0)
    if 0 in positions:
        fed[0] = 1
    for p in range(1, last + 1):
        if p in positions:
            ctx.sync()
            fed[p] = ctx.last_token()
            ctx.forward(fed[p], p)
        else:
            ctx.forward_greedy(p)
    ctx.sync()
    return fed


def bench_dtype(cfg, dtype, positions, steps, warmup, trials, torch, l2d, synth, fill=True, keep_blob=False):
    t = time.time()
    blob = synth.make_blob(cfg, dtype)
    log(f"[bench] {cfg.name} dtype={('fp32', 'q8_0', 'q4_0')[dtype]}: blob {blob.size / 1e9:.2f} GB "
        f"generated in {time.time() - t:.1f}s")
    t = time.time()
    ctx = l2d.Context(blob, dtype)
    if not keep_blob:
        del blob
        blob = None
    log(f"[bench] upload + graph capture {time.time() - t:.1f}s")
    t = time.time()
    fed = decode_to(ctx, positions, torch, fill)
    if fill:
        log(f"[bench] greedy decode 0..{max(positions)} in {time.time() - t:.1f}s")
    res = {}
    for p in positions:
        tr = time_replays(ctx, fed[p], p, steps, warmup, torch, trials)
        sec = tr["sec"]
        b = step_bytes(cfg, dtype, p)
        res[p] = {"tok_s": 1.0 / sec, "ms": sec * 1e3, "trials_ms": tr["trials_ms"],
                  "step_gbs": b["total"] / sec / 1e9, "step_bytes": b["total"]}
        log(f"[bench]   pos {p}: {sec * 1e3:.3f} ms/step (median of {trials}: "
            f"{', '.join(f'{x:.3f}' for x in tr['trials_ms'])}), {1 / sec:.1f} tok/s, "
            f"{b['total'] / sec / 1e9:.0f} GB/s algorithmic")
    return ctx, fed, res, blob


def kernel_detail(ctx, cfg, dtype, token, pos, reps):
    kt = kernel_times(ctx, token, pos, reps)
    b = step_bytes(cfg, dtype, pos)
    kern = {}
    for k, sec in kt.items():
        kb = b.get(k)
        kern[k] = {"avg_us": sec * 1e6}
        if kb:
            kern[k]["gbs"] = kb / sec / 1e9
            kern[k]["alg_bytes"] = kb
    log(f"[bench] {cfg.name} {('fp32', 'q8_0', 'q4_0')[dtype]} kernels at pos {pos}: " +
        ", ".join(f"{k} {v['avg_us']:.1f}us" + (f" {v['gbs']:.0f}GB/s" if 'gbs' in v else "")
                  for k, v in kern.items()))
    return kt, kern


def stream_trace(ctx, cfg, token: int, pos: int) -> dict:
    """One step of the persistent step kernel with its clock stamps
    (l2d_stream_trace, 100 MHz): per matvec phase, the medians over
    workgroups (averaged over layers 2 .. L-3) of the wait for the phase's
    inputs (other workgroups' progress flags), the prologue (input into LDS),
    the workers' part after the input is ready, the epilogue with the flag
    store, and (q/k/v) the attention items; the latency from the last
    producer's flag to the median consumer seeing it; the spread of the
    producers' flag stores; and the step's span per layer."""
    import numpy as np
    nwg, nwk = ctx.stream_shape()
    ctl, _ = ctx.stream_trace(token, pos, nwg, nwk)
    c = ctl.astype(np.int64)
    c = c - c[:, 0].min()
    L = cfg.n_layers
    names = ["qkv", "wo", "w13", "w2"]
    ev = lambda p, i: c[:, i + 6 * p]
    out = {}
    layers = range(2, L - 2)
    for k, n in enumerate(names):
        row = {"wait_us": [], "prologue_us": [], "workers_us": [], "epilogue_us": [], "attention_us": [],
               "flag_latency_us": [], "publish_spread_us": []}
        for l in layers:
            p = 4 * l + k
            row["wait_us"].append(np.median(ev(p, 2) - ev(p, 1)))
            row["prologue_us"].append(np.median(ev(p, 3) - ev(p, 2)))
            row["workers_us"].append(np.median(ev(p, 4) - ev(p, 3)))
            row["epilogue_us"].append(np.median(ev(p, 5) - ev(p, 4)))
            if k == 0:
                row["attention_us"].append(np.median(ev(p, 6) - ev(p, 5)))
            prev = ev(p - 1, 5) if k != 1 else ev(p - 1, 6)
            row["flag_latency_us"].append(np.median(ev(p, 2)) - prev.max())
            row["publish_spread_us"].append(ev(p, 5).max() - np.median(ev(p, 5)))
        out[n] = {kk: float(np.mean(v)) / 100.0 for kk, v in row.items() if v}
    per_layer = [np.median(ev(4 * (l + 1), 1) - ev(4 * l, 1)) for l in layers]
    out["per_layer_us"] = float(np.mean(per_layer)) / 100.0
    out["step_us"] = float(c[:, :1 + 6 * (4 * L + 1)].max()) / 100.0
    return out


def format_stream_trace(tr: dict, title: str, command: str) -> str:
    lines = [title, "=" * len(title), "", "Command (repo root on the GPU machine):", "  " + command, "",
             "Per-layer medians over workgroups (layers 2 .. L-3), microseconds:", "",
             f"{'phase':<6} {'wait':>7} {'prologue':>9} {'workers':>8} {'epilogue':>9} {'attention':>10} "
             f"{'flag->seen':>11} {'pub spread':>11}"]
    for n in ("qkv", "wo", "w13", "w2"):
        r = tr[n]
        att = f"{r['attention_us']:.2f}" if "attention_us" in r else "-"
        lines.append(f"{n:<6} {r['wait_us']:7.2f} {r['prologue_us']:9.2f} {r['workers_us']:8.2f} "
                     f"{r['epilogue_us']:9.2f} {att:>10} {r['flag_latency_us']:11.2f} {r['publish_spread_us']:11.2f}")
    lines += ["", f"per_layer_us: {tr['per_layer_us']:.2f}", f"step_us: {tr['step_us']:.1f}", ""]
    return "\n".join(lines)


def time_oracle(m, budget_s: float, seq_len: int, min_steps: int = 2) -> tuple:
    """Greedy decode from pos 0 with the oracle for about budget_s seconds
    (a short model that reaches seq_len starts over from pos 0 with an empty
    cache)."""
    import numpy as np
    m.reset_kv()
    t0 = time.time()
    n = 0
    tok = 1
    while n < min_steps or time.time() - t0 < budget_s:
        pos = n % seq_len
        if pos == 0 and n > 0:
            m.reset_kv()
            tok = 1
        lg = m.forward(tok, pos)
        tok = int(np.argmax(lg))
        n += 1
    return n, time.time() - t0


def cpu_baseline(cfg, dtype, budget_s: float, synth, per_config: bool, big_blobs: dict,
                 configs=("tiny", "15M", "110M", "7B", "70B")) -> dict:
    """The oracle, untuned, on this host's cores (threads = physical cores
    unless the affinity mask allows fewer): greedy decode from pos 0 for
    about budget_s seconds at the headline config; with per_config, a short
    sample of every config and dtype (one core as well for the small
    ones)."""
    import oracle
    info = cpu_info()
    want = info.get("physical_cores") or os.cpu_count()
    if info.get("affinity_cpus"):
        want = min(want, info["affinity_cpus"])
    oracle.set_threads(int(want))
    blob = big_blobs.get((cfg.name, dtype))
    if blob is None:
        blob = synth.make_blob(cfg, dtype)
    m = oracle.Model(blob, dtype)
    n, dt = time_oracle(m, budget_s, cfg.seq_len)
    cores = oracle.threads()
    m.close()
    dname = {0: "fp32", 1: "Q8_0", 2: "Q4_0"}
    out = {"value": n / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": f"{n} greedy decode steps of the {cfg.name}-shape {dname[dtype]} model from pos 0 "
                     f"({dt:.1f}s, {cores} threads)",
           "cpu": info}
    if per_config:
        rows = {}
        for name in configs:
            c = synth.CONFIGS[name]
            for d in c.dtypes:
                if name == cfg.name and d == dtype:
                    rows[f"{name} {dname[d]}"] = {"threads": cores, "tok_s": n / dt, "steps": n}
                    continue
                b = big_blobs.get((name, d))
                if b is None:
                    if name == "70B":
                        continue  # only when the 70B blob is in host memory already
                    b = synth.make_blob(c, d)
                mm = oracle.Model(b, d)
                small = name in ("tiny", "15M", "110M")
                for th in ((1, cores) if small else (cores,)):
                    oracle.set_threads(th)
                    k, t = time_oracle(mm, 2.0 if small else 4.0, c.seq_len, 2 if small else 1)
                    rows[f"{name} {dname[d]}" + (" 1 core" if th == 1 else "")] = {
                        "threads": th, "tok_s": k / t, "steps": k}
                    log(f"[bench] oracle {name} {dname[d]} {th} threads: {k / t:.2f} tok/s ({k} steps)")
                oracle.set_threads(cores)
                mm.close()
                del b
        out["per_config"] = rows
    return out


def summarize_stats(src: str, out_path: str, title: str, command: str):
    """Text summary of a rocprofv3 --kernel-trace --stats CSV run: calls and
    durations of every kernel, with the step role of each instance."""
    files = sorted(glob.glob(os.path.join(src, "**", "*kernel_stats.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {src}")
    rows = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            k = short_kernel_name(r["Name"])
            calls, total = int(r["Calls"]), float(r["TotalDurationNs"])
            a = rows.setdefault(k, {"calls": 0, "total": 0.0, "min": float("inf"), "max": 0.0})
            a["calls"] += calls
            a["total"] += total
            a["min"] = min(a["min"], float(r["MinNs"]))
            a["max"] = max(a["max"], float(r["MaxNs"]))
    lines = [title, "=" * len(title), "", "Command (repo root on the GPU machine, TMPDIR=/tmp):", "  " + command,
             f"Source: {', '.join(os.path.basename(f) for f in files)} (ns). Summarised by: python bench.py "
             "--summarize-stats <dir> --out <file>.", "",
             f"{'Name':42s} {'Role':46s} {'Calls':>8s} {'AverageNs':>11s} {'MinNs':>9s} {'MaxNs':>9s}"]
    for k, a in sorted(rows.items(), key=lambda kv: -kv[1]["total"]):
        lines.append(f"{k:42s} {kernel_role(k):46s} {a['calls']:8d} {a['total'] / a['calls']:11.1f} "
                     f"{a['min']:9.0f} {a['max']:9.0f}")
    lines += ["", f"sources_sha256: {sources_digest()}"]
    for k, a in rows.items():
        lines.append(f"avg_ns_{k.replace(' ', '')}: {a['total'] / a['calls']:.1f}")
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def short_kernel_name(name: str) -> str:
    """'void l2d::gemv_kernel<1, 1, 3, 2, 4, 1, 2, false>(l2d::GemvParams)'
    -> 'gemv_kernel<1,1,3,2,4,1,2>' (the trailing test-hook flag dropped
    when false)"""
    n = re.sub(r"^void\s+", "", name.strip())
    n = re.sub(r"\(.*\)$", "", n).replace("l2d::", "").replace(" ", "")
    n = n.replace(",false>", ">")
    return n


_ROLES = [
    (r"gemv_kernel<1,1,3,", "Q8_0 w1/w3 + SwiGLU + group quantisation"),
    (r"gemv_kernel<1,1,2,", "Q8_0 q/k/v + RoPE + KV write"),
    (r"gemv_kernel<1,2,1,", "Q8_0 w2 (codes input) + residual"),
    (r"gemv_kernel<1,0,1,", "Q8_0 wo + residual"),
    (r"gemv_kernel<1,1,4,", "Q8_0 classifier + argmax"),
    (r"gemv_kernel<0,1,3,", "fp32 w1/w3 + SwiGLU"),
    (r"gemv_kernel<0,1,2,", "fp32 q/k/v + RoPE + KV write"),
    (r"gemv_kernel<0,0,1,", "fp32 w2 / wo + residual"),
    (r"gemv_kernel<0,1,4,", "fp32 classifier + argmax"),
    (r"gemv_kernel<2,1,3,", "Q4_0 w1/w3 + SwiGLU + group quantisation"),
    (r"gemv_kernel<2,1,2,", "Q4_0 q/k/v + RoPE + KV write"),
    (r"gemv_kernel<2,2,1,", "Q4_0 w2 (codes input) + residual"),
    (r"gemv_kernel<2,0,1,", "Q4_0 wo + residual"),
    (r"gemv_kernel<2,1,4,", "Q4_0 classifier + argmax"),
    (r"gemv_kernel<2,0,0,", "Q4_0 plain matvec (step shapes)"),
    (r"attention_kernel", "attention (splits merged in-kernel)"),
    (r"attn_wo_kernel", "chained: attention, then Q8_0 wo + residual"),
    (r"ffn_kernel", "chained: Q8_0 w1/w3 + SwiGLU, then w2 + residual"),
    (r"begin_step_kernel", "step start: embedding row, RoPE table"),
    (r"stream_step_kernel", "whole step, one persistent launch"),
    (r"prefill", "batched prefill"),
    (r"copyBuffer|elementwise|fill", "calibration / torch"),
]


def kernel_role(k: str) -> str:
    for pat, role in _ROLES:
        if re.search(pat, k):
            return role
    return ""


def summarize_traffic(fetch_dir: str, write_dir: str, out_path: str, title: str, commands: list,
                      cfg_name: str = "7B", pos: int = 512):
    """HBM bytes per launch of each kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), scaled by the factors the
    same counters read for the run's plain 1 GiB device copy
    (--calibrate-copy), against the kernel's algorithmic bytes."""
    import synth

    def load(d, counter):
        files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
        if not files:
            raise SystemExit(f"no *counter_collection.csv under {d}")
        per = {}
        for f in files:
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                per.setdefault(short_kernel_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return per

    fe, wr = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copy = [k for k in fe if k == "__amd_rocclr_copyBuffer"]
    gib_kib = float(1 << 20)
    rf = gib_kib / sum(fe[copy[0]]) if copy else 1.0
    copyw = [k for k in wr if k == "__amd_rocclr_copyBuffer"]
    wf = gib_kib / sum(wr[copyw[0]]) if copyw else 1.0
    cfg = synth.CONFIGS[cfg_name]
    b = step_bytes(cfg, 1, pos)
    alg = {"w13": b["w13"], "qkv": b["qkv"], "w2": b["w2"], "wo": b["wo"], "cls": b["cls"],
           "attn": b["attn"] + 2 * cfg.kv_dim * 4}
    key_of = {"gemv_kernel<1,1,3,": "w13", "gemv_kernel<1,1,2,": "qkv", "gemv_kernel<1,2,1,": "w2",
              "gemv_kernel<1,0,1,": "wo", "gemv_kernel<1,1,4,": "cls", "attention_kernel": "attn"}
    lines = [title, "=" * len(title), "", "Commands (repo root on the GPU machine, TMPDIR=/tmp):"]
    lines += ["  " + c for c in commands]
    lines += ["Figures: mean Counter_Value (KiB) over the dispatches of each kernel. Summarised by: python bench.py "
              "--summarize-traffic <fetch dir> <write dir> --out <file>.", "",
              f"Calibration (plain device copy of 1 GiB, --calibrate-copy): FETCH_SIZE reads "
              f"{1 / rf:.3f}x the bytes read, WRITE_SIZE {1 / wf:.3f}x the bytes written",
              f"  => read factor {rf:.3f}, write factor {wf:.3f}; HBM bytes/launch = (rf * FETCH + wf * WRITE) * 1024",
              "", f"{'kernel':34s} {'dispatches':>10s} {'FETCH KiB':>11s} {'WRITE KiB':>10s} "
                  f"{'HBM bytes/launch':>17s} {'algorithmic':>12s} {'ratio':>6s}"]
    keys = []
    for k in sorted(fe, key=lambda k: -statistics.mean(fe[k])):
        if "copyBuffer" in k:
            continue
        f_ = statistics.mean(fe[k])
        w_ = statistics.mean(wr.get(k, [0.0]))
        hb = (rf * f_ + wf * w_) * 1024
        role = next((v for p_, v in key_of.items() if k.startswith(p_)), None)
        a = alg.get(role) if role else None
        lines.append(f"{k:34s} {len(fe[k]):10d} {f_:11.1f} {w_:10.1f} {hb:17.0f} "
                     f"{(f'{a:12.0f}' if a else ' ' * 12)} {(f'{hb / a:6.3f}' if a else '')}")
        if role:
            keys.append((role, hb))
    lines += ["", f"sources_sha256: {sources_digest()}"]
    for role, hb in keys:
        lines.append(f"hbm_bytes_{role}: {hb:.0f}")
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--trials", type=int, default=3)
    ap.add_argument("--config", default="7B")
    ap.add_argument("--positions", default="1,512,2048")
    ap.add_argument("--headline-pos", type=int, default=512)
    ap.add_argument("--dtypes", default="q8_0,fp32,q4_0")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-oracle-configs", action="store_true",
                    help="time the oracle on the headline config only")
    ap.add_argument("--no-fill", action="store_true",
                    help="skip the greedy decode that fills the cache (profiling runs)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the batched prefill measurement")
    ap.add_argument("--prefill-tokens", type=int, default=512)
    ap.add_argument("--no-q4-gemv", action="store_true",
                    help="skip the Q4_0 matvec measurement")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the persistent step kernel measurement")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the chained-launch step measurement")
    ap.add_argument("--stream-trace-out", metavar="FILE",
                    help="also write the persistent kernel's per-phase trace summary to FILE")
    ap.add_argument("--no-70b", action="store_true", help="skip the 70B-shape Q8_0 step")
    ap.add_argument("--no-clocks", action="store_true",
                    help="do not run rocm-smi for the clocks (profiled runs)")
    ap.add_argument("--positions-70b", default="1,2048,4095")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--summarize-stats", metavar="DIR",
                    help="write the text summary of a rocprofv3 --stats CSV run and exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM traffic summary of two rocprofv3 --pmc CSV runs and exit")
    ap.add_argument("--out", help="summary file (with --summarize-*)")
    ap.add_argument("--title", default="")
    ap.add_argument("--command", action="append", default=[],
                    help="command line(s) that produced the profile (with --summarize-*)")
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.out, args.title, " && ".join(args.command))
        return
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1], args.out, args.title,
                          args.command)
        return
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 "
              "(the multi-GPU split is described in the design notes, not built)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import llama_transformer_decode_amd as l2d
    import synth

    torch.cuda.set_device(0)
    clocks_before = {} if args.no_clocks else gpu_clocks()
    if args.calibrate_copy:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 1 GiB read + 1 GiB written")
        del a, b
    cfg = synth.CONFIGS[args.config]
    positions = sorted({int(p) for p in args.positions.split(",")} | {args.headline_pos})
    codes = {"fp32": 0, "q8_0": 1, "q4_0": 2}
    names = {v: k for k, v in codes.items()}
    dtypes = [codes[d.strip()] for d in args.dtypes.split(",")]
    detail = {}
    head = None
    big_blobs = {}
    for dt in dtypes:
        name = names[dt]
        ctx, fed, res, _ = bench_dtype(cfg, dt, positions, args.steps, args.warmup, args.trials, torch, l2d,
                                       synth, not args.no_fill)
        hp = args.headline_pos
        kt, kern = kernel_detail(ctx, cfg, dt, fed[hp], hp, args.kernel_reps)
        detail[name] = {"per_pos": {str(p): res[p] for p in positions}, "kernels": kern}
        # the same step with next-token sampling on (T = 0.8, fused into the
        # classifier) at the headline position
        ctx.set_sampling(0.8, 12345)
        tr = time_replays(ctx, fed[hp], hp, args.steps, args.warmup, torch, args.trials)
        ctx.set_sampling(0.0, 0)
        detail[name]["sampling_t0.8"] = {"ms": tr["sec"] * 1e3, "tok_s": 1.0 / tr["sec"]}
        log(f"[bench]   pos {hp} with sampling T=0.8: {tr['sec'] * 1e3:.3f} ms/step, {1 / tr['sec']:.1f} tok/s")
        if dt == 1 and not args.no_stream:
            # the whole step as one persistent launch (same arithmetic)
            try:
                ctx.use_persistent(True)
                st = {}
                for p in positions:
                    tr = time_replays(ctx, fed[p], p, args.steps, args.warmup, torch, args.trials)
                    st[str(p)] = {"tok_s": 1.0 / tr["sec"], "ms": tr["sec"] * 1e3, "trials_ms": tr["trials_ms"]}
                    log(f"[bench]   stream kernel pos {p}: {tr['sec'] * 1e3:.3f} ms/step, {1 / tr['sec']:.1f} tok/s")
                detail["q8_0_stream"] = {"per_pos": st}
                tr = stream_trace(ctx, cfg, fed[hp], hp)
                detail["q8_0_stream"]["trace_pos"] = hp
                detail["q8_0_stream"]["trace"] = tr
                log(f"[bench]   stream kernel trace at pos {hp}: {tr['per_layer_us']:.1f} us per layer; " +
                    "; ".join(f"{n} wait {tr[n]['wait_us']:.1f} prologue {tr[n]['prologue_us']:.1f} "
                              f"workers {tr[n]['workers_us']:.1f}" for n in ("qkv", "wo", "w13", "w2")))
                if args.stream_trace_out:
                    with open(args.stream_trace_out, "w") as f:
                        f.write(format_stream_trace(
                            tr, f"Persistent step kernel phases, {cfg.name}-shape Llama-2 decode step, Q8_0 GS=64, "
                                f"batch 1, pos {hp} (l2d_stream_trace clock stamps)",
                            "python bench.py " + " ".join(sys.argv[1:])))
                ctx.use_persistent(False)
            except l2d.L2DError as e:
                detail["q8_0_stream"] = {"unavailable": str(e)}
        if dt == 1 and not args.no_chain:
            # chained launches (attention + output projection, w1/w3 + w2 in
            # one launch each; same arithmetic, off by default)
            try:
                ctx.use_chain(True)
                ch = {}
                for p in positions:
                    tr = time_replays(ctx, fed[p], p, args.steps, args.warmup, torch, args.trials)
                    ch[str(p)] = {"tok_s": 1.0 / tr["sec"], "ms": tr["sec"] * 1e3, "trials_ms": tr["trials_ms"]}
                    log(f"[bench]   chained launches pos {p}: {tr['sec'] * 1e3:.3f} ms/step, {1 / tr['sec']:.1f} tok/s")
                kc = kernel_times(ctx, fed[hp], hp, args.kernel_reps)
                detail["q8_0_chained"] = {
                    "per_pos": ch,
                    "kernels_us": {"qkv": kc["qkv"] * 1e6, "attn+wo": kc["attn"] * 1e6,
                                   "w13+w2": kc["w13"] * 1e6, "cls": kc["cls"] * 1e6}}
                log(f"[bench]   chained launches at pos {hp}: qkv {kc['qkv'] * 1e6:.1f}us, attention + wo "
                    f"{kc['attn'] * 1e6:.1f}us, w1/w3 + w2 {kc['w13'] * 1e6:.1f}us")
                ctx.use_chain(False)
            except l2d.L2DError as e:
                detail["q8_0_chained"] = {"unavailable": str(e)}
        if not args.no_prefill and dt != 2:  # no batched prefill for 4-bit weights
            detail["prefill_" + name] = prefill_rates(cfg, ctx, torch, synth, args.prefill_tokens)
            if dt == 1:
                # the same prefill with the group combine in fp32
                ctx.prefill_combine(True)
                detail["prefill_q8_0_fp32_combine"] = prefill_rates(cfg, ctx, torch, synth, args.prefill_tokens)
                ctx.prefill_combine(False)
        if head is None:
            head = (dt, res[hp], kt, step_bytes(cfg, dt, hp))
        ctx.close()
        del ctx
        torch.cuda.empty_cache()

    if not args.no_70b:
        # 70B-shape Q8_0 (64 query heads over 8 kv heads) at deep positions;
        # the cache is not filled by a decode (same bytes moved per step)
        c70 = synth.CONFIGS["70B"]
        p70 = sorted({int(p) for p in args.positions_70b.split(",")})
        ctx, fed, res, blob70 = bench_dtype(c70, 1, p70, max(5, args.steps // 5), 2, args.trials, torch, l2d,
                                            synth, fill=False, keep_blob=not args.no_cpu_baseline)
        _, kern70 = kernel_detail(ctx, c70, 1, fed[p70[-1]], p70[-1], 3)
        detail["70B_q8_0"] = {"per_pos": {str(p): res[p] for p in p70}, "kernels_at_pos": p70[-1],
                              "kernels": kern70, "cache": "zero-filled (no decode), same bytes per step"}
        if blob70 is not None:
            big_blobs[("70B", 1)] = blob70
        ctx.close()
        del ctx
        torch.cuda.empty_cache()

    dt, r, kt, b = head
    w13 = b["w13"] / kt["w13"] / 1e9
    prof = committed_profile("gemv_kernel<1,1,3,2,4,1,2>") if dt == 1 and cfg.name == "7B" else None
    roof = {"bound": "hbm", "kernel": "gemv w1/w3 + SwiGLU (gemv_kernel<1,1,3,2,4,1,2>)",
            "achieved": w13, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": w13 / PEAK_HBM_GBS,
            "traffic": None,
            "basis": f"algorithmic bytes {b['w13']:.0f} per launch / mean launch duration from HIP events "
                     f"stamped at each launch's start and end on the context's stream "
                     f"({args.kernel_reps} kernel-by-kernel steps at pos {args.headline_pos})",
            "avg_us": kt["w13"] * 1e6}
    if prof:
        if "avg_us" in prof:
            roof["profile_avg_us"] = prof["avg_us"]
            roof["profile_frac"] = b["w13"] / (prof["avg_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS
            roof["profile_file"] = os.path.relpath(STATS_FILE, ROOT)
        if "traffic" in prof:
            roof["traffic"] = prof["traffic"].get("w13")
            roof["traffic_by_kernel"] = prof["traffic"]
            roof["traffic_file"] = os.path.relpath(TRAFFIC_FILE, ROOT)
    out = {
        "metric": "decode tokens/sec at batch 1 + achieved HBM GB/s vs peak (7B-shape Q8_0 & fp32)",
        "value": r["tok_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "trials": args.trials,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "f32 (fp64 accumulate)", 1: "int8xint8->int32, fp32/fp64",
                  2: "int4xint8->int32, fp32/fp64"}[dt],
        "data": "synthetic: seeded random weights of the 7B shape (fp32: N(0, 0.02) by Box-Muller; "
                "Q8_0: random codes, one +-127 per group, scales giving sd 0.02)",
        "config": {"workload": f"{cfg.name}-shape Llama-2 decode step, "
                               f"{('fp32', 'Q8_0 GS=64', 'Q4_0 GS=32')[dt]}, batch 1, pos {args.headline_pos}",
                   "global_batch": 1, "seq_len": cfg.seq_len, "pos": args.headline_pos,
                   "parallelism": "single GPU"},
        "hbm_step_gbs": r["step_gbs"],
        "hbm_step_frac": r["step_gbs"] / PEAK_HBM_GBS,
        "roofline": roof,
        "clocks": {"before": clocks_before, "after": {} if args.no_clocks else gpu_clocks()},
        "detail": detail,
    }
    if not args.no_q4_gemv:
        detail["q4_0_gemv"] = gemv_q40_rates(cfg, torch, l2d)
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores")
        out["cpu_baseline"] = cpu_baseline(cfg, dt, args.cpu_seconds, synth, not args.no_oracle_configs,
                                           big_blobs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
