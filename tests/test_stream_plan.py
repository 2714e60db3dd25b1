"""Host check of the persistent step kernel's plan (no GPU): the functions
the kernel computes its addresses with, run over every wave of a launch —
each worker's weight stream in phase order with every code and scale load
inside its array, every row of every matrix streamed exactly once, the
workgroups' row ranges tiling each matrix, the attention position ranges
covering 0..pos exactly for every pos, the partial slots inside their
allocation, and the LDS within a CU's 160 KiB."""
import pytest

import llama_transformer_decode_amd as l2d
import synth

SMALL = [
    synth.Config("tinyq8", 128, 256, 3, 4, 2, 320, 64, 11, (synth.Q8_0,)),
    synth.Config("gsq8", 256, 512, 2, 8, 2, 320, 48, 13, (synth.Q8_0,)),
    synth.Config("gqa8h128", 1024, 512, 2, 8, 1, 320, 96, 14, (synth.Q8_0,)),
    synth.Config("odd_vocab", 128, 192, 2, 4, 4, 321, 40, 15, (synth.Q8_0,)),
]


@pytest.mark.parametrize("name", ["110M", "7B", "13B", "70B"])
@pytest.mark.parametrize("nwg", [256, 304, 80])
def test_plan_full_size(name, nwg):
    assert l2d.stream_plan_check(synth.CONFIGS[name].header(), nwg) == "ok"


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
@pytest.mark.parametrize("nwg", [256, 7, 3])
def test_plan_small(cfg, nwg):
    assert l2d.stream_plan_check(cfg.header(), nwg) == "ok"


def test_plan_rejects_what_the_kernel_does_not_take():
    with pytest.raises(l2d.L2DError):
        l2d.stream_plan_check(synth.CONFIGS["7B"].header(), 256, group_size=32)
    with pytest.raises(l2d.L2DError):  # one workgroup cannot hold a row result per classifier row in LDS
        l2d.stream_plan_check(synth.CONFIGS["7B"].header(), 1)
