"""Chunked prefill over a cached prefix (the model card's serving set-up prefills long prompts
in chunks) against the oracle's chunk rows, which are the prefill definition's rows at the
chunk's positions."""
import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import assert_parity, dev_bf16, dev_f32, host_f32

pytestmark = pytest.mark.gpu

SCALE = 192 ** -0.5


def seq_data(B, Hq, Hkv, L, seed):
    w = inputs.Workload("t", "prefill", 0, B, Hq, Hkv, seqlen=L, seed=seed)
    return inputs.prefill_inputs(w)


def gpu_chunk(mode, W, q_chunk, k, v, sink):
    out = sa.prefill_chunk(mode, W, dev_bf16(q_chunk), dev_bf16(k), dev_bf16(v), dev_f32(sink))
    torch.cuda.synchronize()
    return host_f32(out)


@pytest.mark.parametrize("mode,W,Hq,Hkv,Lk,Lq", [
    (oracle.GLOBAL, 0, 64, 4, 1000, 1),      # one new token (a decode step through the prefill path)
    (oracle.GLOBAL, 0, 64, 4, 1000, 37),     # chunk start not on a 32-position boundary
    (oracle.GLOBAL, 0, 64, 4, 1000, 333),
    (oracle.GLOBAL, 0, 16, 2, 577, 577),     # no prefix: plain prefill
    (oracle.GLOBAL, 0, 8, 4, 900, 200),      # group of 2 (general kernel, two heads per wave)
    (oracle.GLOBAL, 0, 4, 4, 700, 65),       # group of 1
    (oracle.SWA, 128, 64, 8, 1000, 37),
    (oracle.SWA, 128, 64, 8, 1000, 129),
    (oracle.SWA, 100, 16, 2, 800, 300),
    (oracle.SWA, 1, 8, 2, 300, 64),
])
def test_chunk_matches_oracle(mode, W, Hq, Hkv, Lk, Lq):
    print(f"[case] chunk mode={mode} W={W} Hq={Hq} Hkv={Hkv} Lk={Lk} Lq={Lq}", flush=True)
    d = seq_data(2, Hq, Hkv, Lk, seed=Lk + Lq + Hq)
    qc = np.ascontiguousarray(d["q"][:, :, Lk - Lq:])
    got = gpu_chunk(mode, W, qc, d["k"], d["v"], d["sink"])
    ref = oracle.prefill_chunk(qc, d["k"], d["v"], d["sink"], mode, W, SCALE)
    assert_parity(got, ref, f"chunk Lk={Lk} Lq={Lq}")


def test_chunks_stitch_to_prefill():
    """Three chunks (700 + 700 + 600 tokens) give the rows of one prefill over 2000 tokens."""
    Hq, Hkv, L = 64, 4, 2000
    d = seq_data(1, Hq, Hkv, L, seed=3)
    full = host_f32(sa.prefill(oracle.GLOBAL, 0, dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]),
                               dev_f32(d["sink"])))
    start = 0
    for n in (700, 700, 600):
        end = start + n
        qc = np.ascontiguousarray(d["q"][:, :, start:end])
        kc = np.ascontiguousarray(d["k"][:, :, :end])
        vc = np.ascontiguousarray(d["v"][:, :, :end])
        got = gpu_chunk(oracle.GLOBAL, 0, qc, kc, vc, d["sink"])
        assert_parity(got, full[:, :, start:end], f"chunk {start}..{end} vs full prefill")
        start = end


def test_ga_second_half_at_32k_sampled():
    """The GA workload's last 16384 positions as one chunk after a 16384-token prefix, sampled
    rows of every head against the oracle."""
    w = inputs.GA_PREFILL
    print("[case] GA chunk 16K at 32K", flush=True)
    d = inputs.prefill_inputs(w)
    Lq = 16384
    qc = np.ascontiguousarray(d["q"][:, :, w.seqlen - Lq:])
    out = sa.prefill_chunk(w.mode, w.window, dev_bf16(qc), dev_bf16(d["k"]), dev_bf16(d["v"]), dev_f32(d["sink"]))
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    pos = np.unique(np.concatenate([np.arange(8), np.arange(Lq - 8, Lq), rng.integers(0, Lq, 16)]))
    rows = np.array([(0, h, r) for h in range(w.hq) for r in pos], np.int64)
    idx = torch.from_numpy(rows).to("cuda")
    got = host_f32(out[idx[:, 0], idx[:, 1], idx[:, 2]])
    ref = oracle.prefill_chunk(qc, d["k"], d["v"], d["sink"], w.mode, w.window, w.scale, rows=rows)
    assert_parity(got, ref, f"GA chunk sampled {len(rows)} rows")
    assert torch.isfinite(out.float()).all().item()
