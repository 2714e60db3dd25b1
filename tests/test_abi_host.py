"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol include/l2d.h declares, and its blob parser accepts exactly the
layouts the header describes and rejects the rest with the right codes."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import llama_transformer_decode_amd as l2d
import synth
from blobview import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "l2d.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(l2d_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    declared = _declared()
    assert len(declared) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", l2d.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(l2d_\w+)", out))
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    assert set(declared) == set(l2d.EXPORTS)
    lib = l2d.lib()
    for s in declared:
        assert getattr(lib, s) is not None


def _addr(p):
    return p if isinstance(p, int) else (p or 0)


@pytest.mark.parametrize("cfgname,dtype", [("tiny", 0), ("15M", 0), ("110M", 1)])
def test_blob_parse_offsets(cfgname, dtype):
    cfg = synth.CONFIGS[cfgname]
    if cfgname == "110M":
        cfg = cfg.replace(n_layers=2, vocab_size=-1024)  # smaller, unshared
    blob = synth.make_blob(cfg, dtype)
    c, w = l2d.blob_parse(blob, dtype, 64)
    assert (c.dim, c.hidden_dim, c.n_layers, c.n_heads, c.n_kv_heads, c.vocab_size,
            c.seq_len) == cfg.header()
    assert c.dtype == dtype and c.rope_theta == 10000.0 and c.norm_eps == 1e-5
    base = blob.ctypes.data
    parts, total = layout(cfg.header(), dtype, 64)
    assert total == blob.size
    want = {}
    for name, kind, off, shape in parts:
        want[name + ("_s" if kind == "s" else "")] = base + off
    names = {"emb": "emb", "rms_att": "rms_att", "wq": "wq", "wk": "wk", "wv": "wv", "wo": "wo",
             "rms_ffn": "rms_ffn", "w1": "w1", "w2": "w2", "w3": "w3", "rms_final": "rms_final"}
    for fld, key in names.items():
        assert _addr(getattr(w, fld)) == want[key], fld
        if dtype == 1 and fld not in ("rms_att", "rms_ffn", "rms_final"):
            assert _addr(getattr(w, fld + "_s")) == want[key + "_s"], fld
    if cfg.vocab_size > 0:
        assert _addr(w.wcls) == _addr(w.emb)
    else:
        assert _addr(w.wcls) == want["wcls"]


def test_blob_parse_rejects():
    cfg = synth.CONFIGS["tiny"]
    blob = synth.make_blob(cfg, 0)
    with pytest.raises(l2d.L2DError) as e:
        l2d.blob_parse(blob[:-4], 0)
    assert e.value.code == l2d.EFORMAT
    with pytest.raises(l2d.L2DError) as e:
        l2d.blob_parse(np.concatenate([blob, np.zeros(4, np.uint8)]), 0)
    assert e.value.code == l2d.EFORMAT
    with pytest.raises(l2d.L2DError) as e:
        l2d.blob_parse(blob, 1, 64)  # 172 % 64 != 0
    assert e.value.code == l2d.EINVAL
    with pytest.raises(l2d.L2DError) as e:
        l2d.blob_parse(blob, 7)
    assert e.value.code == l2d.EINVAL
    bad = blob.copy()
    bad[0:4] = np.frombuffer(np.int32(60).tobytes(), np.uint8)  # dim 60 % 8 heads
    with pytest.raises(l2d.L2DError) as e:
        l2d.blob_parse(bad, 0)
    assert e.value.code == l2d.EINVAL
    assert "n_heads" in l2d.last_error()
    bad = blob.copy()
    bad[16:20] = np.frombuffer(np.int32(3).tobytes(), np.uint8)  # 8 heads % 3 kv heads
    with pytest.raises(l2d.L2DError):
        l2d.blob_parse(bad, 0)
    with pytest.raises(l2d.L2DError) as e:
        l2d.blob_parse(blob[:20], 0)
    assert e.value.code == l2d.EINVAL


def test_blob_parse_70b_header_64bit_offsets():
    """The 70B header implies ~73 GB; parse a header-only view with a fake
    size to exercise 64-bit size arithmetic without allocating it."""
    cfg = synth.CONFIGS["70B"]
    n = synth.blob_bytes(cfg, 1)
    assert n > 2 ** 36
    hdr = np.frombuffer(np.array(cfg.header(), np.int32).tobytes(), np.uint8).copy()
    c, w = l2d.Config(), l2d.Weights()
    # a 28-byte buffer that claims to be n bytes long: the parser must compute
    # the exact size in 64 bits and accept it without touching the arrays
    rc = l2d.lib().l2d_blob_parse(hdr.ctypes.data_as(ctypes.c_void_p), n, 1, 64,
                                  ctypes.byref(c), ctypes.byref(w))
    assert rc == 0
    base = hdr.ctypes.data
    parts, total = layout(cfg.header(), 1, 64)
    assert total == n
    off = {name + ("_s" if kind == "s" else ""): o for name, kind, o, _ in parts}
    assert w.w2 - base == off["w2"] and w.wcls_s - base == off["wcls_s"]
    assert off["wcls_s"] > 2 ** 32
    rc = l2d.lib().l2d_blob_parse(hdr.ctypes.data_as(ctypes.c_void_p), n + 1, 1, 64,
                                  ctypes.byref(c), ctypes.byref(w))
    assert rc == l2d.EFORMAT
