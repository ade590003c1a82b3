"""Prefill kernel parity against the CPU oracle (needs an MI355X and the built library)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import assert_parity, dev_bf16, dev_f32, errors, host_f32

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def run_prefill(mode, window, d, sink=True, scale=None):
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    s = dev_f32(d["sink"]) if sink else None
    out = sa.prefill(mode, window, q, k, v, s, scale=scale)
    torch.cuda.synchronize()
    return host_f32(out)


def small_inputs(B, Hq, Hkv, L, seed):
    w = inputs.Workload("t", "prefill", 0, B, Hq, Hkv, seqlen=L, seed=seed)
    return inputs.prefill_inputs(w)


def test_tiny_workload():
    """L=512, 4 query heads / 1 KV head, window 128, fp32 N(0,1) data with a per-head sink."""
    w = inputs.TINY
    d = inputs.prefill_inputs(w)
    print(f"[case] tiny workload {w}", flush=True)
    got = run_prefill(w.mode, w.window, d)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], w.mode, w.window, w.scale)
    assert_parity(got, ref, "tiny vs oracle on the bf16-rounded inputs")
    # the workload's own fp32 data (before rounding to bf16): the same bar holds
    ref32 = oracle.prefill(d["q32"], d["k32"], d["v32"], d["sink"], w.mode, w.window, w.scale)
    assert_parity(got, ref32, "tiny vs oracle on the fp32 source data")


CASES = [
    # B, Hq, Hkv, L, mode, W, sink
    (1, 8, 1, 200, oracle.GLOBAL, 0, True),
    (2, 16, 2, 333, oracle.SWA, 128, True),
    (1, 4, 4, 97, oracle.GLOBAL, 0, False),
    (1, 6, 3, 130, oracle.SWA, 1, True),
    (1, 8, 8, 65, oracle.SWA, 2, True),
    (1, 16, 1, 300, oracle.SWA, 127, True),
    (1, 16, 1, 300, oracle.SWA, 129, True),
    (1, 8, 2, 257, oracle.SWA, 1000, True),
    (1, 4, 1, 1, oracle.GLOBAL, 0, True),
    (1, 4, 1, 31, oracle.SWA, 128, False),
    (3, 12, 3, 150, oracle.GLOBAL, 0, True),
    (1, 64, 8, 160, oracle.SWA, 128, True),
    (1, 64, 4, 130, oracle.GLOBAL, 0, True),
    (1, 32, 1, 64, oracle.SWA, 64, True),
    (1, 3, 1, 70, oracle.SWA, 33, True),
    # global mode with 8 or 16 query heads per KV head (the pipelined causal kernel):
    # 1, 2, 3 and 4+ key tiles, ragged ends, batches, with and without a sink
    (2, 16, 2, 1, oracle.GLOBAL, 0, True),
    (1, 16, 1, 33, oracle.GLOBAL, 0, False),
    (1, 8, 1, 64, oracle.GLOBAL, 0, True),
    (1, 8, 1, 65, oracle.GLOBAL, 0, True),
    (1, 32, 2, 129, oracle.GLOBAL, 0, True),
    (1, 16, 2, 191, oracle.GLOBAL, 0, True),
    (1, 16, 2, 192, oracle.GLOBAL, 0, False),
    (1, 16, 2, 193, oracle.GLOBAL, 0, True),
    (2, 8, 1, 517, oracle.GLOBAL, 0, True),
    # sliding window with a group of 8 or 16 and W <= 128 (the ring kernel): workgroups that
    # walk runs of 3 and 4 blocks with a short last run, sub-block 1 of the ring's first
    # band, single-block runs, windows 1 and 100
    (8, 64, 8, 300, oracle.SWA, 128, True),
    (4, 64, 8, 1000, oracle.SWA, 100, True),
    (1, 8, 1, 20, oracle.SWA, 128, True),
    (2, 16, 1, 97, oracle.SWA, 1, True),
    (1, 8, 1, 200, oracle.SWA, 16, False),
    (33, 64, 8, 70, oracle.SWA, 128, True),  # 264 (sequence, KV head) units: one run each
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_L{}_m{}_W{}_s{}".format(*c))
def test_prefill_small(case):
    B, Hq, Hkv, L, mode, W, sink = case
    print(f"[case] {case}", flush=True)
    d = small_inputs(B, Hq, Hkv, L, seed=sum(case[:6]))
    got = run_prefill(mode, W, d, sink)
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["sink"] if sink else None, mode, W, 192 ** -0.5)
    assert_parity(got, ref, str(case))


def test_sink_extremes():
    """+inf sink -> zero rows; -inf sink == no sink (bitwise); huge finite sink -> ~0."""
    d = small_inputs(1, 8, 2, 90, seed=7)
    sink = np.array([np.inf, 0.0, -np.inf, 3.0, 1e30, -1e30, 6.0, np.inf], np.float32)
    d["sink"] = sink
    print("[case] sink extremes", flush=True)
    got = run_prefill(oracle.SWA, 16, d)
    ref = oracle.prefill(d["q"], d["k"], d["v"], sink.astype(np.float64), oracle.SWA, 16, 192 ** -0.5)
    assert np.all(got[:, 0] == 0) and np.all(got[:, 7] == 0)
    assert_parity(got, ref, "sink extremes")
    d2 = dict(d, sink=np.full(8, -np.inf, np.float32))
    a = run_prefill(oracle.SWA, 16, d2)
    b = run_prefill(oracle.SWA, 16, d2, sink=False)
    assert np.array_equal(a, b)


def test_growing_max_rescales():
    """Logits that keep growing along the sequence force the lazy rescale many times.  The
    attention becomes nearly one-hot, so outputs approach single value rows; V is scaled by
    1/4 to keep them inside the range where the absolute bound is not dominated by the bf16
    rounding of the output itself (half an ulp is 0.016 for values in [4, 8))."""
    B, Hq, Hkv, L = 1, 16, 2, 700
    d = small_inputs(B, Hq, Hkv, L, seed=12)
    k = inputs.bf16_to_f32(d["k"])
    k *= (1.0 + np.arange(L, dtype=np.float32) / 40.0)[None, None, :, None]  # key norms grow ~18x
    d["k"] = inputs.bf16_bits(k)
    d["v"] = inputs.bf16_bits(inputs.bf16_to_f32(d["v"]) * 0.25)
    for mode, W in ((oracle.GLOBAL, 0), (oracle.SWA, 128)):
        # with a sink (every row starts from its sink logit) and without one (every row
        # starts with no reference, so its first visible keys force the first rescale)
        for sink in (True, False):
            got = run_prefill(mode, W, d, sink=sink)
            ref = oracle.prefill(d["q"], d["k"], d["v"], d["sink"] if sink else None, mode, W, 192 ** -0.5)
            assert_parity(got, ref, f"growing logits mode={mode} sink={sink}")


def test_wide_window_equals_global_bitwise():
    d = small_inputs(1, 8, 2, 200, seed=8)
    ga = run_prefill(oracle.GLOBAL, 0, d)
    for W in (200, 201, 4096):
        assert np.array_equal(run_prefill(oracle.SWA, W, d), ga), W


def test_deterministic():
    d = small_inputs(2, 16, 2, 190, seed=9)
    a = run_prefill(oracle.GLOBAL, 0, d)
    b = run_prefill(oracle.GLOBAL, 0, d)
    assert np.array_equal(a, b)


def test_worked_example_through_kernel():
    """The paper-notes §4.3 example end to end: 128 window keys, every logit exactly 2
    (scale 1/8, q[0] = k[0] = 4), sink 4, V = identity so the output row is the weights."""
    g = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))
    L, W = 300, 128
    q = np.zeros((1, 1, L, 192), np.float32)
    k = np.zeros((1, 1, L, 192), np.float32)
    v = np.zeros((1, 1, L, 128), np.float32)
    q[..., 0] = 4.0
    k[..., 0] = 4.0
    for j in range(L):
        v[0, 0, j, j % 128] = 1.0
    d = {"q": inputs.bf16_bits(q), "k": inputs.bf16_bits(k), "v": inputs.bf16_bits(v),
         "sink": np.array([g["sink"]], np.float32)}
    out = run_prefill(oracle.SWA, W, d, scale=0.125)
    x = math.exp(g["logit"] - g["sink"])
    per_key = x / (1 + 128 * x)
    # bf16 bound: the probability enters the value product rounded to bf16 and the output is
    # rounded again, each within half an ulp (2^-8 relative)
    tol = 2 ** -7
    rows = out[0, 0, 127:]  # every row with a full window
    assert np.all(np.abs(rows - per_key) <= per_key * tol)
    mass = rows.sum(axis=-1)
    assert np.all(np.abs(mass - g["printed"]["window_mass"]["value"]) <= g["printed"]["window_mass"]["half_ulp"] + 128 * per_key * tol)
    assert np.all(np.abs(mass - 128 * per_key) <= 128 * per_key * tol)
    # early rows see fewer keys: row i has i+1 keys, each weight x / (1 + (i+1) x)
    for i in (0, 5, 100):
        want = x / (1 + (i + 1) * x)
        assert np.all(np.abs(out[0, 0, i, :i + 1] - want) <= want * tol)


def sampled_rows(Hq, L, seed, n_first, n_last, n_rand):
    rng = np.random.default_rng(seed)
    pos = np.unique(np.concatenate([np.arange(n_first), np.arange(L - n_last, L),
                                    rng.integers(0, L, n_rand)]))
    return np.array([(0, h, i) for h in range(Hq) for i in pos], np.int64)


@pytest.mark.parametrize("name", ["swa_prefill_L32768", "ga_prefill_L32768"])
def test_full_size_sampled(name):
    """The benchmark workloads at full size, compared on sampled rows of every head."""
    w = inputs.WORKLOADS[name]
    print(f"[case] full size {name}", flush=True)
    d = inputs.prefill_inputs(w)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    out = sa.prefill(w.mode, w.window, q, k, v, dev_f32(d["sink"]))
    torch.cuda.synchronize()
    if w.mode == oracle.SWA:
        rows = sampled_rows(w.hq, w.seqlen, 17, 160, 128, 256)
    else:
        rows = inputs.ga_parity_rows(w)  # 512 rows per head: the first 128, the last 128, 256 seeded
    idx = torch.from_numpy(rows).to("cuda")
    got = host_f32(out[idx[:, 0], idx[:, 1], idx[:, 2]])
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], w.mode, w.window, w.scale, rows=rows)
    assert_parity(got, ref, f"{name} sampled {len(rows)} rows")
    assert torch.isfinite(out.float()).all().item()
