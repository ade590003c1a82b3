"""The CPU oracle against what the pages and mathematics fix (runs without a GPU)."""
import numpy as np
import pytest

import oracle
from oracle import oracle_np
from attention_sink_softmax_amd import inputs

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_tiny_workload_brute_force(oracle_lib):
    """The tiny workload (L=512, 4 query heads / 1 KV head, window 128, fp32 data): the C
    oracle and the numpy eager form agree to 1e-12 relative, on the fp32 source data and on
    its bf16-rounded copy."""
    w = inputs.TINY
    d = inputs.prefill_inputs(w)
    for q, k, v in ((d["q32"], d["k32"], d["v32"]),
                    (d["q"], d["k"], d["v"])):
        got = oracle.prefill(q, k, v, d["sink"], w.mode, w.window, w.scale, lib=oracle_lib)
        if q.dtype == np.uint16:
            q, k, v = (inputs.bf16_to_f32(x) for x in (q, k, v))
        ref = oracle_np.prefill(q, k, v, d["sink"], w.mode, w.window, w.scale)
        assert np.max(np.abs(got - ref) / (np.abs(ref) + 1e-30)) < 1e-12 or \
            np.max(np.abs(got - ref)) < 1e-14


def test_rows_mode_matches_full(oracle_lib):
    w = inputs.TINY
    d = inputs.prefill_inputs(w)
    full = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], w.mode, w.window, w.scale, lib=oracle_lib)
    rows = np.array([[0, 0, 0], [0, 3, 511], [0, 2, 127], [0, 1, 128], [0, 0, 300]])
    got = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], w.mode, w.window, w.scale, rows=rows,
                         lib=oracle_lib)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(got[r], full[b, h, i])


def test_bad_arguments_rejected(oracle_lib):
    q = np.zeros((1, 3, 4, 8), np.float32)
    k = np.zeros((1, 2, 4, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, k, None, oracle.GLOBAL, 0, 1.0, lib=oracle_lib)  # 3 % 2 != 0
    q = np.zeros((1, 2, 4, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, k, None, oracle.SWA, 0, 1.0, lib=oracle_lib)  # window 0
