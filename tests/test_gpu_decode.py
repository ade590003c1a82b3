"""Decode kernels (ring and paged caches, split-KV merge) against the CPU oracle."""
import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import assert_parity, dev_bf16, dev_f32, dev_i32, host_f32

pytestmark = pytest.mark.gpu

SCALE = 192 ** -0.5


def gpu_decode(mode, window, layout, q, k, v, lens, max_len, sink, bt=None):
    out = sa.decode(mode, window, dev_bf16(q), layout, dev_bf16(k), dev_bf16(v), dev_i32(lens), max_len,
                    dev_f32(sink), None if bt is None else dev_i32(bt))
    torch.cuda.synchronize()
    return host_f32(out)


def seq_data(B, Hq, Hkv, L, seed):
    w = inputs.Workload("t", "prefill", 0, B, Hq, Hkv, seqlen=L, seed=seed)
    return inputs.prefill_inputs(w)


@pytest.mark.parametrize("W,Hq,Hkv", [(128, 16, 2), (64, 8, 1), (200, 64, 8), (1, 4, 4), (128, 32, 1)])
def test_ring_matches_prefill_last_row(W, Hq, Hkv):
    """Ring decode at length n equals the prefill row n-1 of the sequence it was built from."""
    lens = np.array([1, 50, W - 1 if W > 1 else 1, W, 3 * W + 7, 1000], np.int32)
    B, L = len(lens), int(lens.max())
    print(f"[case] ring W={W} Hq={Hq} Hkv={Hkv} lens={lens.tolist()}", flush=True)
    d = seq_data(B, Hq, Hkv, L, seed=W + Hq)
    kr = np.zeros((B, Hkv, W, 192), np.uint16)
    vr = np.zeros((B, Hkv, W, 128), np.uint16)
    for b in range(B):
        k1, v1 = inputs.ring_from_sequence(d["k"][b:b + 1], d["v"][b:b + 1], int(lens[b]), W)
        kr[b], vr[b] = k1[0], v1[0]
    qn = np.stack([d["q"][b, :, lens[b] - 1] for b in range(B)])
    got = gpu_decode(oracle.SWA, W, sa.KV_RING, qn, kr, vr, lens, L, d["sink"])
    ref = oracle.decode(qn, kr, vr, lens, d["sink"], oracle.SWA, W, SCALE, oracle.RING)
    assert_parity(got, ref, f"ring W={W}")
    rows = np.array([(b, h, lens[b] - 1) for b in range(B) for h in range(Hq)])
    pre = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], oracle.SWA, W, SCALE, rows=rows)
    assert_parity(got.reshape(-1, 128), pre, f"ring W={W} vs prefill rows")


@pytest.mark.parametrize("mode,W,ps,Hq,Hkv,perm", [
    (oracle.GLOBAL, 0, 64, 64, 4, True),
    (oracle.GLOBAL, 0, 16, 16, 2, True),
    (oracle.GLOBAL, 0, 128, 32, 1, False),
    (oracle.SWA, 128, 64, 64, 8, True),
    (oracle.SWA, 100, 32, 8, 2, True),
    (oracle.GLOBAL, 0, 64, 4, 4, True),
])
def test_paged(mode, W, ps, Hq, Hkv, perm):
    lens = np.array([1, 63, 64, 65, 1000, 5000, 4097], np.int32)
    B, L = len(lens), int(lens.max())
    print(f"[case] paged mode={mode} W={W} ps={ps} Hq={Hq} Hkv={Hkv} perm={perm}", flush=True)
    d = seq_data(B, Hq, Hkv, L, seed=ps + Hq + mode)
    mp = (L + ps - 1) // ps
    kp, vp, bt = inputs.pages_from_sequence(d["k"], d["v"], L, ps, B * mp + 5, seed=ps, permute=perm)
    qn = np.stack([d["q"][b, :, lens[b] - 1] for b in range(B)])
    got = gpu_decode(mode, W, sa.KV_PAGED, qn, kp, vp, lens, L, d["sink"], bt)
    ref = oracle.decode(qn, kp, vp, lens, d["sink"], mode, W, SCALE, oracle.PAGED, bt)
    assert_parity(got, ref, "paged")
    rows = np.array([(b, h, lens[b] - 1) for b in range(B) for h in range(Hq)])
    pre = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], mode, W, SCALE, rows=rows)
    assert_parity(got.reshape(-1, 128), pre, "paged vs prefill rows")


def growing_keys(d, rate):
    """Key norms that grow along the sequence (1 + position / rate) and V scaled by 1/4, as in
    the prefill test of growing logits: the scores of later slices exceed the lazy-rescale
    threshold again and again, and the nearly one-hot outputs stay where the absolute bound
    is not dominated by the output's own bf16 rounding."""
    k = inputs.bf16_to_f32(d["k"])
    k *= (1.0 + np.arange(k.shape[2], dtype=np.float32) / rate)[None, None, :, None]
    d["k"] = inputs.bf16_bits(k)
    d["v"] = inputs.bf16_bits(inputs.bf16_to_f32(d["v"]) * 0.25)
    return d


@pytest.mark.parametrize("q_len", [1, 4])
def test_growing_scores_rescale(q_len):
    """Paged decode with one and with four new tokens (16 and 64 columns per workgroup) while
    the column maxima keep growing within each wave's slices and across splits."""
    lens = np.array([700, 5000, 4097], np.int32)
    B, L, Hq, Hkv, ps = len(lens), 5000, 64, 4, 64
    print(f"[case] growing scores q_len={q_len}", flush=True)
    d = growing_keys(seq_data(B, Hq, Hkv, L, seed=31 + q_len), 200.0)
    kp, vp, bt = inputs.pages_from_sequence(d["k"], d["v"], L, ps, B * (L // ps + 1) + 3, seed=4)
    q = np.zeros((B, Hq, q_len, 192), np.uint16)
    for b in range(B):
        q[b] = d["q"][b, :, lens[b] - q_len:lens[b]]
    if q_len == 1:
        got = gpu_decode(oracle.GLOBAL, 0, sa.KV_PAGED, q[:, :, 0], kp, vp, lens, L, d["sink"], bt)[:, :, None]
    else:
        out = sa.decode_multi(oracle.GLOBAL, 0, dev_bf16(q), sa.KV_PAGED, dev_bf16(kp), dev_bf16(vp), dev_i32(lens), L,
                              dev_f32(d["sink"]), dev_i32(bt))
        torch.cuda.synchronize()
        got = host_f32(out)
    rows = np.array([(b, h, lens[b] - q_len + t) for b in range(B) for h in range(Hq) for t in range(q_len)])
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], oracle.GLOBAL, 0, SCALE, rows=rows)
    assert_parity(got.reshape(-1, 128), ref, f"growing scores q_len={q_len}")


def test_growing_scores_ring():
    """Ring decode (W = 128) with growing key norms: each wave's single slice grows past the
    threshold and the waves' records merge across different references."""
    W, Hq, Hkv = 128, 16, 2
    lens = np.array([128, 300, 1000], np.int32)
    B, L = len(lens), int(lens.max())
    d = growing_keys(seq_data(B, Hq, Hkv, L, seed=41), 20.0)
    kr = np.zeros((B, Hkv, W, 192), np.uint16)
    vr = np.zeros((B, Hkv, W, 128), np.uint16)
    for b in range(B):
        k1, v1 = inputs.ring_from_sequence(d["k"][b:b + 1], d["v"][b:b + 1], int(lens[b]), W)
        kr[b], vr[b] = k1[0], v1[0]
    qn = np.stack([d["q"][b, :, lens[b] - 1] for b in range(B)])
    got = gpu_decode(oracle.SWA, W, sa.KV_RING, qn, kr, vr, lens, L, d["sink"])
    rows = np.array([(b, h, lens[b] - 1) for b in range(B) for h in range(Hq)])
    ref = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], oracle.SWA, W, SCALE, rows=rows)
    assert_parity(got.reshape(-1, 128), ref, "growing scores ring")


@pytest.mark.parametrize("scale", [0.125, 0.4])
def test_nondefault_scale(scale):
    """Logit scales other than 1/sqrt(192), with growing key norms so that the rescale is taken:
    the scale enters the exponent's FMA and the lazy-rescale threshold (m + 8) / c.  A ring
    (single-slice kernel) and a paged cache split over several workgroups (merge kernel)."""
    print(f"[case] decode scale={scale}", flush=True)
    W, Hq, Hkv = 128, 16, 2
    lens = np.array([128, 300, 1000], np.int32)
    B, L = len(lens), int(lens.max())
    d = growing_keys(seq_data(B, Hq, Hkv, L, seed=51), 100.0)
    kr = np.zeros((B, Hkv, W, 192), np.uint16)
    vr = np.zeros((B, Hkv, W, 128), np.uint16)
    for b in range(B):
        k1, v1 = inputs.ring_from_sequence(d["k"][b:b + 1], d["v"][b:b + 1], int(lens[b]), W)
        kr[b], vr[b] = k1[0], v1[0]
    qn = np.stack([d["q"][b, :, lens[b] - 1] for b in range(B)])
    out = sa.decode(oracle.SWA, W, dev_bf16(qn), sa.KV_RING, dev_bf16(kr), dev_bf16(vr), dev_i32(lens), L,
                    dev_f32(d["sink"]), scale=scale)
    torch.cuda.synchronize()
    ref = oracle.decode(qn, kr, vr, lens, d["sink"], oracle.SWA, W, scale, oracle.RING)
    assert_parity(host_f32(out), ref, f"ring scale={scale}")
    lens2 = np.array([700, 5000, 4097], np.int32)
    L2, Hq2, Hkv2, ps = 5000, 64, 4, 64
    d2 = growing_keys(seq_data(len(lens2), Hq2, Hkv2, L2, seed=52), 400.0)
    kp, vp, bt = inputs.pages_from_sequence(d2["k"], d2["v"], L2, ps, len(lens2) * (L2 // ps + 1) + 3, seed=6)
    qn2 = np.stack([d2["q"][b, :, lens2[b] - 1] for b in range(len(lens2))])
    out2 = sa.decode(oracle.GLOBAL, 0, dev_bf16(qn2), sa.KV_PAGED, dev_bf16(kp), dev_bf16(vp), dev_i32(lens2), L2,
                     dev_f32(d2["sink"]), dev_i32(bt), scale=scale)
    torch.cuda.synchronize()
    ref2 = oracle.decode(qn2, kp, vp, lens2, d2["sink"], oracle.GLOBAL, 0, scale, oracle.PAGED, bt)
    assert_parity(host_f32(out2), ref2, f"paged scale={scale}")


def test_contiguous_equals_permuted_pages():
    lens = np.array([3000, 2048], np.int32)
    d = seq_data(2, 16, 2, 3000, seed=5)
    outs = []
    for perm in (False, True):
        kp, vp, bt = inputs.pages_from_sequence(d["k"], d["v"], 3000, 64, 2 * 47 + 3, seed=1, permute=perm)
        qn = np.stack([d["q"][b, :, lens[b] - 1] for b in range(2)])
        outs.append(gpu_decode(oracle.GLOBAL, 0, sa.KV_PAGED, qn, kp, vp, lens, 3000, d["sink"], bt))
    assert np.array_equal(outs[0], outs[1])


def test_edge_lengths_and_bad_pages():
    """seq_len 0 -> zero row; seq_len above max_seq_len -> NaN row; a page id outside the pool
    -> NaN row for that sequence only; sink +inf -> zero row; no sink -> plain softmax."""
    B, Hq, Hkv, ps = 5, 16, 2, 64
    d = seq_data(B, Hq, Hkv, 600, seed=3)
    kp, vp, bt = inputs.pages_from_sequence(d["k"], d["v"], 600, ps, B * 10, seed=2)
    lens = np.array([600, 0, 700, 600, 300], np.int32)
    bt = bt.copy()
    bt[3, 4] = 10 ** 6
    bt[3, 5] = -1
    qn = np.ascontiguousarray(d["q"][:, :, 299])
    sink = d["sink"].copy()
    sink[1] = np.inf
    got = gpu_decode(oracle.GLOBAL, 0, sa.KV_PAGED, qn, kp, vp, lens, 600, sink, bt)
    assert np.all(got[1] == 0)
    assert np.all(np.isnan(got[2])) and np.all(np.isnan(got[3]))
    ok = [0, 4]
    ref = oracle.decode(qn[ok], kp, vp, lens[ok], sink, oracle.GLOBAL, 0, SCALE, oracle.PAGED, bt[ok])
    assert_parity(got[ok], ref, "edge lengths")
    assert np.all(got[ok][:, 1] == 0)
    nos = gpu_decode(oracle.GLOBAL, 0, sa.KV_PAGED, qn[ok], kp, vp, lens[ok], 600, None, bt[ok])
    ref2 = oracle.decode(qn[ok], kp, vp, lens[ok], None, oracle.GLOBAL, 0, SCALE, oracle.PAGED, bt[ok])
    assert_parity(nos, ref2, "no sink")


def test_swa_decode_workload_full():
    """128 sequences, lengths U[4096, 65536], 128-slot rings, 64/8 heads: every output row."""
    w = inputs.SWA_DECODE
    print(f"[case] {w.name}", flush=True)
    d = inputs.decode_ring_inputs(w)
    got = gpu_decode(w.mode, w.window, sa.KV_RING, d["q"], d["k"], d["v"], d["seq_lens"], int(d["seq_lens"].max()),
                     d["sink"])
    ref = oracle.decode(d["q"], d["k"], d["v"], d["seq_lens"], d["sink"], w.mode, w.window, w.scale, oracle.RING)
    assert_parity(got, ref, w.name)


def test_ga_decode_workload_full():
    """8 sequences at 256K in 64-token pages with a permuted table, 64/4 heads: every row."""
    w = inputs.GA_DECODE
    print(f"[case] {w.name}", flush=True)
    d = inputs.decode_paged_inputs(w)
    got = gpu_decode(w.mode, w.window, sa.KV_PAGED, d["q"], d["k"], d["v"], d["seq_lens"], w.ctx_hi, d["sink"],
                     d["block_table"])
    ref = oracle.decode(d["q"], d["k"], d["v"], d["seq_lens"], d["sink"], w.mode, w.window, w.scale, oracle.PAGED,
                        d["block_table"])
    assert_parity(got, ref, w.name)
