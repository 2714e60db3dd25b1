"""GPU parity of the individual kernels against the oracle, through the C ABI:
the Q8_0 quantiser (bit-exact codes and scales), the fp32 GEMV (fp64
accumulation: at most one fp32 ulp from the oracle), and the Q8_0 GEMV
(exact int32 group dots; outputs at most one ulp away), and the Q4_0 GEMV
(same bar: exact group dots against 4-bit weights, one ulp on outputs)."""
import numpy as np
import pytest

import llama_transformer_decode_amd as l2d
import oracle
import synth
from gpu_util import log, need_gpu, ulp_diff

pytestmark = pytest.mark.gpu


def _adversarial(n, gs, rng):
    """Values whose quotient x/scale sits exactly on k + 1/2, within a few
    ulp of it under a scale other than 1, zero groups, +-max, tiny and huge
    magnitudes."""
    x = rng.standard_normal(n).astype(np.float32)
    g = x.reshape(-1, gs)
    ng = g.shape[0]
    for i in range(0, ng, 7):      # exact ties: wmax 127 -> scale 1, values k + 0.5
        g[i] = (rng.integers(-127, 127, gs) + 0.5).astype(np.float32)
        g[i, 0] = 127.0
    for i in range(1, ng, 11):     # all-zero group
        g[i] = 0.0
    for i in range(2, ng, 13):     # +-max only
        g[i] = 0.0
        g[i, 3] = -3.0
    for i in range(3, ng, 17):     # tiny magnitudes
        g[i] *= np.float32(1e-30)
    for i in range(4, ng, 19):     # huge magnitudes
        g[i] *= np.float32(1e30)
    for i in range(5, ng, 23):     # near ties: x / scale within 3 ulp of k + 1/2, scale not 1
        m = np.float32(rng.uniform(0.5, 3.0))
        sc = np.float32(m / np.float32(127.0))
        k = rng.integers(-126, 126, gs).astype(np.float64)
        base = ((k + 0.5) * np.float64(sc)).astype(np.float32)
        step = rng.integers(-3, 4, gs).astype(np.float32)
        g[i] = base + step * np.spacing(base)
        g[i, 0] = m
    return g.reshape(-1)


@pytest.mark.parametrize("gs", [16, 32, 64, 128, 256])
def test_quantize_q80_bitexact(gs):
    torch = need_gpu()
    rng = np.random.default_rng(gs)
    for n in (gs, gs * 3, 1_000_000 // gs * gs, 4096):
        for kind in ("normal", "adversarial"):
            x = (rng.standard_normal(n).astype(np.float32) if kind == "normal"
                 else _adversarial(n, gs, rng))
            q, s = l2d.quantize_q80(torch.from_numpy(x).cuda(), gs)
            torch.cuda.synchronize()
            rq, rs = oracle.quantize(x, gs)
            np.testing.assert_array_equal(s.cpu().numpy(), rs)
            np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_quantize_q80_errors():
    need_gpu()
    with pytest.raises(l2d.L2DError):
        l2d.lib() and l2d._check(l2d.lib().l2d_quantize_q80(None, 100, 64, None, None, None))
    with pytest.raises(l2d.L2DError):
        l2d._check(l2d.lib().l2d_quantize_q80(None, 64, 0, None, None, None))
    assert l2d.lib().l2d_quantize_q80(None, 0, 64, None, None, None) == 0


F32_SHAPES = [(2, 4), (6, 172), (34, 288), (770, 768), (4096, 4096), (12288, 4096),
              (4096, 11008), (32000, 4096)]
Q8_SHAPES = [(2, 64), (6, 192), (34, 768), (130, 2048), (4096, 4096), (12288, 4096),
             (4096, 11008), (32000, 4096), (1280, 8192), (8192, 3584)]


def _report(name, g, r):
    u = ulp_diff(g, r)
    log(f"  {name}: exact {np.mean(u == 0):.5f}, max ulp {int(u.max())}")
    return u


@pytest.mark.parametrize("rows,cols", F32_SHAPES)
def test_gemv_f32_vs_oracle(rows, cols):
    torch = need_gpu()
    W = synth.normal_f32(rows * 7 + cols, 1, rows * cols, 0.02).reshape(rows, cols)
    x = synth.normal_f32(rows * 7 + cols, 2, cols, 1.0)
    out = l2d.gemv(l2d.F32, torch.from_numpy(W).cuda(), None, torch.from_numpy(x).cuda(),
                   rows, cols)
    g = out.cpu().numpy()
    r = oracle.matvec_f32(W, x)
    u = _report(f"f32 {rows}x{cols}", g, r)
    assert u.max() <= 1
    assert np.mean(u == 0) > 0.99


@pytest.mark.parametrize("rows,cols", Q8_SHAPES)
def test_gemv_q80_vs_oracle(rows, cols):
    torch = need_gpu()
    gs = 64
    rng = np.random.default_rng(rows + cols)
    Q = rng.integers(-127, 128, (rows, cols)).astype(np.int8)
    S = (rng.uniform(0.5, 1.5, (rows, cols // gs)) * 3e-4).astype(np.float32)
    x = synth.normal_f32(rows + 3 * cols, 3, cols, 1.0)
    gd = torch.zeros(rows * (cols // gs), dtype=torch.int32, device="cuda")
    out = l2d.gemv(l2d.Q8_0, torch.from_numpy(Q).cuda(), torch.from_numpy(S).cuda(),
                   torch.from_numpy(x).cuda(), rows, cols, gs, group_dots=gd)
    g = out.cpu().numpy()
    r = oracle.matvec_q80(Q, S, x, gs)
    # exact int32 group dots against the oracle's, for the activation codes
    # the oracle computes (the kernel quantises x itself; codes are bit-exact)
    xq, _ = oracle.quantize(x, gs)
    dots = gd.cpu().numpy().reshape(rows, cols // gs)
    for i in range(0, rows, max(1, rows // 64)):
        np.testing.assert_array_equal(dots[i], oracle.group_dots(Q[i], xq, gs))
    u = _report(f"q8 {rows}x{cols}", g, r)
    assert u.max() <= 1
    assert np.mean(u == 0) > 0.99


def test_gemv_q80_extreme_codes():
    """All codes +-127 (largest group dots, 64*127^2) and a zero input."""
    torch = need_gpu()
    rows, cols, gs = 64, 4096, 64
    Q = np.where(np.arange(rows * cols).reshape(rows, cols) % 3 == 0, -127, 127).astype(np.int8)
    S = np.full((rows, cols // gs), 1e-3, np.float32)
    x = np.full(cols, 2.5, np.float32)
    gd = torch.zeros(rows * (cols // gs), dtype=torch.int32, device="cuda")
    out = l2d.gemv(l2d.Q8_0, torch.from_numpy(Q).cuda(), torch.from_numpy(S).cuda(),
                   torch.from_numpy(x).cuda(), rows, cols, gs, group_dots=gd)
    xq, _ = oracle.quantize(x, gs)
    assert (xq == 127).all()
    dots = gd.cpu().numpy().reshape(rows, cols // gs)
    for i in range(rows):
        np.testing.assert_array_equal(dots[i], oracle.group_dots(Q[i], xq, gs))
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.matvec_q80(Q, S, x, gs))
    z = l2d.gemv(l2d.Q8_0, torch.from_numpy(Q).cuda(), torch.from_numpy(S).cuda(),
                 torch.zeros(cols, device="cuda"), rows, cols, gs)
    assert (z.cpu().numpy() == 0).all()


def test_gemv_rejects_bad_shapes():
    torch = need_gpu()
    W = torch.zeros(12, device="cuda")
    x = torch.zeros(4, device="cuda")
    with pytest.raises(l2d.L2DError):
        l2d.gemv(l2d.F32, W, None, x, 3, 4)  # odd rows
    with pytest.raises(l2d.L2DError):
        l2d.gemv(l2d.Q8_0, W, W, x, 2, 48, 64)  # gs does not divide cols


# Q4_0: small ragged shapes (group counts not a multiple of the 64- and
# 128-group chunks), the 7B and 13B matvec shapes (q/k/v fused, w1/w3 fused,
# w2, classifier) and the longest accepted input
Q4_SHAPES = [(2, 32), (6, 96), (34, 768), (130, 2080), (258, 4128), (4096, 4096), (12288, 4096),
             (22016, 4096), (4096, 11008), (32000, 4096), (15360, 5120), (5120, 13824), (2, 65536)]


def _q40_weights(rows, cols, rng):
    """Quantised normal weights for small shapes, random bytes and scales
    for large ones (every nibble pattern is valid Q4_0 data)."""
    if rows * cols <= 1 << 22:
        W = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
        q, s = oracle.quantize_q40(W.reshape(-1))
        return q.reshape(rows, cols // 2), s.reshape(rows, cols // 32)
    Q = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    S = (rng.uniform(-1.5, 1.5, (rows, cols // 32)) * 3e-3).astype(np.float32)
    return Q, S


@pytest.mark.parametrize("rows,cols", Q4_SHAPES)
def test_gemv_q40_vs_oracle(rows, cols):
    torch = need_gpu()
    log(f"  q4 gemv {rows}x{cols}")
    rng = np.random.default_rng(rows * 3 + cols)
    Q, S = _q40_weights(rows, cols, rng)
    x = synth.normal_f32(rows + 5 * cols, 4, cols, 1.0)
    gd = torch.zeros(rows * (cols // 32), dtype=torch.int32, device="cuda")
    out = l2d.gemv(l2d.Q4_0, torch.from_numpy(Q).cuda(), torch.from_numpy(S).cuda(),
                   torch.from_numpy(x).cuda(), rows, cols, 32, group_dots=gd)
    g = out.cpu().numpy()
    r = oracle.matvec_q40(Q, S, x)
    xq, _ = oracle.quantize(x, 32)
    dots = gd.cpu().numpy().reshape(rows, cols // 32)
    for i in sorted(set(range(0, rows, max(1, rows // 64))) | {rows - 1}):
        np.testing.assert_array_equal(dots[i], oracle.group_dots_q40(Q[i], xq))
    u = _report(f"q4 {rows}x{cols}", g, r)
    assert u.max() <= 1
    assert np.mean(u == 0) > 0.99


def test_gemv_q40_extreme_codes():
    """Codes -8 and 7 only against inputs at +-127 (largest group dots,
    32 * 8 * 127), an all-zero input and an adversarial one."""
    torch = need_gpu()
    rows, cols = 64, 4096
    lo_hi = np.where(np.arange(rows * cols // 2).reshape(rows, cols // 2) % 3 == 0, 0x00, 0xFF)
    Q = lo_hi.astype(np.uint8)
    Q[::5] = 0x0F  # low nibbles 7, high nibbles -8
    S = np.full((rows, cols // 32), -1e-3, np.float32)
    for x in (np.full(cols, 2.5, np.float32),
              np.where(np.arange(cols) % 2 == 0, 3.0, -3.0).astype(np.float32),
              _adversarial(cols, 32, np.random.default_rng(5))):
        gd = torch.zeros(rows * (cols // 32), dtype=torch.int32, device="cuda")
        out = l2d.gemv(l2d.Q4_0, torch.from_numpy(Q).cuda(), torch.from_numpy(S).cuda(),
                       torch.from_numpy(x).cuda(), rows, cols, 32, group_dots=gd)
        xq, _ = oracle.quantize(x, 32)
        dots = gd.cpu().numpy().reshape(rows, cols // 32)
        for i in range(rows):
            np.testing.assert_array_equal(dots[i], oracle.group_dots_q40(Q[i], xq))
        u = ulp_diff(out.cpu().numpy(), oracle.matvec_q40(Q, S, x))
        assert u.max() <= 1
    assert np.abs(dots).max() <= 32 * 8 * 127
    z = l2d.gemv(l2d.Q4_0, torch.from_numpy(Q).cuda(), torch.from_numpy(S).cuda(),
                 torch.zeros(cols, device="cuda"), rows, cols, 32)
    assert (z.cpu().numpy() == 0).all()


def test_gemv_q40_rejects_bad_shapes():
    torch = need_gpu()
    W = torch.zeros(64, dtype=torch.uint8, device="cuda")
    S = torch.zeros(8, device="cuda")
    x = torch.zeros(64, device="cuda")
    with pytest.raises(l2d.L2DError):
        l2d.gemv(l2d.Q4_0, W, S, x, 2, 64, 64)  # group size other than 32
    with pytest.raises(l2d.L2DError):
        l2d.gemv(l2d.Q4_0, W, S, x, 2, 48, 32)  # 32 does not divide cols
    with pytest.raises(l2d.L2DError):
        l2d.gemv(l2d.Q4_0, W, None, x, 2, 64, 32)  # no scales


def test_gemv_profile_matches_gemv():
    """The timed entry point runs the same kernel: same output as l2d_gemv on
    the last copy, a positive mean duration; Q8_0 is refused (its codes need
    the device layout)."""
    torch = need_gpu()
    rows, cols = 512, 4096
    rng = np.random.default_rng(9)
    Ws, Ss = [], []
    for _ in range(3):
        Q, S = _q40_weights(rows, cols, rng)
        Ws.append(torch.from_numpy(Q).cuda())
        Ss.append(torch.from_numpy(S).cuda())
    x = torch.from_numpy(synth.normal_f32(1, 9, cols, 1.0)).cuda()
    sec, out = l2d.gemv_profile(l2d.Q4_0, Ws, Ss, x, rows, cols, 32, reps=5)  # last launch uses copy 1
    ref = l2d.gemv(l2d.Q4_0, Ws[1], Ss[1], x, rows, cols, 32)
    np.testing.assert_array_equal(out.cpu().numpy(), ref.cpu().numpy())
    assert 0 < sec < 1e-2
    Wf = [torch.from_numpy(synth.normal_f32(2, 10, rows * cols, 0.02)).cuda()]
    sec, out = l2d.gemv_profile(l2d.F32, Wf, None, x, rows, cols, 1, reps=2)
    np.testing.assert_array_equal(out.cpu().numpy(), l2d.gemv(l2d.F32, Wf[0], None, x, rows, cols).cpu().numpy())
    with pytest.raises(l2d.L2DError):
        l2d.gemv_profile(l2d.Q8_0, Wf, Ss[:1], x, rows, cols, 64, reps=1)
