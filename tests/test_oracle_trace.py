"""The oracle's trace of quantised matvec inputs (test infrastructure for
the near-tie audit of long GPU trajectories): recording every layer in one
pass gives each layer exactly what recording that layer alone gives, and
tracing changes no logit."""
import numpy as np

import oracle
import synth

CFG = synth.Config("traceq8", 128, 256, 3, 4, 2, 320, 64, 11, (synth.Q8_0,))


def test_trace_all_layers_equals_one_layer_at_a_time():
    blob = synth.make_blob(CFG, synth.Q8_0)
    m = oracle.Model(blob, synth.Q8_0)
    toks = [1, 7, 300, 12]
    plain = [m.forward(t, p).copy() for p, t in enumerate(toks)]
    m.reset_kv()
    m.trace_layer(-2)
    for p, t in enumerate(toks):
        np.testing.assert_array_equal(m.forward(t, p), plain[p])
    every = {(l, s): m.trace_at(l, s) for l in range(CFG.n_layers) for s in range(4)}
    last = len(toks) - 1
    for l in range(CFG.n_layers):
        m.trace_layer(l)
        m.forward(toks[last], last)  # same (token, pos): same cache slot, same values
        for s in range(4):
            q, sc, f = m.trace(s)
            eq, esc, ef = every[(l, s)]
            np.testing.assert_array_equal(q, eq)
            np.testing.assert_array_equal(sc, esc)
            np.testing.assert_array_equal(f, ef)
            # the recorded codes are the quantiser's codes of the recorded input
            rq, rs = oracle.quantize(f, 64)
            np.testing.assert_array_equal(q, rq)
            np.testing.assert_array_equal(sc, rs)
    m.trace_layer(-1)
    m.close()
