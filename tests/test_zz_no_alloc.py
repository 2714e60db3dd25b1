"""l2d_gemv_noalloc (the matvec entry point that allocates no device memory:
its Q8_0 re-layout goes to the library's fixed scratch array) against
l2d_gemv, which allocates a temporary buffer for the same re-layout. Both
run the same kernels, so outputs and int32 group dots must agree bit for
bit. Two calls in a row, the second smaller, show that the shared array's
leftover contents never leak into a result; the largest size the array
takes runs, one code more is refused on the host."""
import numpy as np
import pytest

import llama_transformer_decode_amd as l2d
from gpu_util import log, need_gpu

pytestmark = pytest.mark.gpu


def _q8_case(torch, rows, cols, gs, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    W = torch.randint(-127, 128, (rows * cols,), dtype=torch.int16, device="cuda", generator=g).to(torch.int8)
    S = (torch.rand(rows * (cols // gs), device="cuda", generator=g) + 0.5) * 1e-3
    x = torch.randn(cols, device="cuda", generator=g)
    return W, S, x


def _both(torch, dtype, W, S, x, rows, cols, gs, dots):
    gd_ref = torch.empty(rows * (cols // gs), dtype=torch.int32, device="cuda") if dots else None
    ref = l2d.gemv(dtype, W, S, x, rows, cols, gs, group_dots=gd_ref)
    out = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    gd = torch.full((rows * (cols // gs),), -1, dtype=torch.int32, device="cuda") if dots else None
    l2d.gemv_noalloc(dtype, W, S, x, out, rows, cols, gs, group_dots=gd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), ref.cpu().numpy())
    if dots:
        np.testing.assert_array_equal(gd.cpu().numpy(), gd_ref.cpu().numpy())


def test_noalloc_q8_two_calls_second_smaller():
    torch = need_gpu()
    for rows, cols, seed in ((1024, 4096, 1), (96, 1024, 2)):
        log(f"  gemv_noalloc Q8_0 {rows}x{cols} gs64")
        W, S, x = _q8_case(torch, rows, cols, 64, seed)
        _both(torch, l2d.Q8_0, W, S, x, rows, cols, 64, dots=True)


def test_noalloc_q8_group_sizes_and_largest():
    torch = need_gpu()
    cap = l2d.gemv_noalloc_max_bytes()
    assert cap == 32 << 20
    for rows, cols, gs in ((64, 2048, 32), (130, 768, 256), (cap // 8192, 8192, 64)):
        log(f"  gemv_noalloc Q8_0 {rows}x{cols} gs{gs}")
        W, S, x = _q8_case(torch, rows, cols, gs, rows + cols)
        _both(torch, l2d.Q8_0, W, S, x, rows, cols, gs, dots=True)


def test_noalloc_refuses_beyond_scratch():
    torch = need_gpu()
    cap = l2d.gemv_noalloc_max_bytes()
    rows, cols = cap // 4096 + 2, 4096  # even rows, two rows past the array
    W = torch.zeros(rows * cols, dtype=torch.int8, device="cuda")
    S = torch.zeros(rows * (cols // 64), dtype=torch.float32, device="cuda")
    x = torch.zeros(cols, dtype=torch.float32, device="cuda")
    out = torch.zeros(rows, dtype=torch.float32, device="cuda")
    with pytest.raises(l2d.L2DError, match="scratch"):
        l2d.gemv_noalloc(l2d.Q8_0, W, S, x, out, rows, cols, 64)


def test_noalloc_fp32_and_q4_pass_through():
    torch = need_gpu()
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    rows, cols = 256, 1024
    W = torch.randn(rows * cols, device="cuda", generator=g) * 0.02
    x = torch.randn(cols, device="cuda", generator=g)
    _both(torch, l2d.F32, W, None, x, rows, cols, 64, dots=False)
    Wq = torch.randint(0, 256, (rows * cols // 2,), dtype=torch.uint8, device="cuda", generator=g)
    Sq = (torch.rand(rows * (cols // 32), device="cuda", generator=g) - 0.5) * 3e-3
    _both(torch, l2d.Q4_0, Wq, Sq, x, rows, cols, 32, dots=True)
