"""Decode of q_len new tokens per sequence at once (the parallel verification of drafted
tokens, "MiMo-V2-Flash 模型架构深度拆解" CH 4.4) against the CPU oracle and against the
last q_len rows of a prefill over the same sequence."""
import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import assert_parity, dev_bf16, dev_f32, dev_i32, host_f32

pytestmark = pytest.mark.gpu

SCALE = 192 ** -0.5


def gpu_multi(mode, window, layout, q, k, v, lens, max_len, sink, bt=None):
    out = sa.decode_multi(mode, window, dev_bf16(q), layout, dev_bf16(k), dev_bf16(v), dev_i32(lens), max_len,
                          dev_f32(sink), None if bt is None else dev_i32(bt))
    torch.cuda.synchronize()
    return host_f32(out)


def seq_data(B, Hq, Hkv, L, seed):
    w = inputs.Workload("t", "prefill", 0, B, Hq, Hkv, seqlen=L, seed=seed)
    return inputs.prefill_inputs(w)


def drafted_queries(q_seq, lens, q_len):
    """q [B,Hq,q_len,192] holding positions lens-q_len .. lens-1 of each sequence (zeros for
    positions below 0)."""
    B, Hq = q_seq.shape[:2]
    qm = np.zeros((B, Hq, q_len, q_seq.shape[3]), np.uint16)
    for b in range(B):
        for t in range(q_len):
            i = int(lens[b]) - q_len + t
            if i >= 0:
                qm[b, :, t] = q_seq[b, :, i]
    return qm


@pytest.mark.parametrize("mode,W,ps,Hq,Hkv,q_len,perm", [
    (oracle.GLOBAL, 0, 64, 64, 4, 4, True),     # 16 heads x 4 tokens: 64 columns, one workgroup
    (oracle.GLOBAL, 0, 16, 16, 2, 2, True),     # 16 columns
    (oracle.GLOBAL, 0, 64, 64, 4, 7, True),     # 112 columns: two workgroups, the second ragged
    (oracle.GLOBAL, 0, 128, 32, 1, 5, False),   # 160 columns, three workgroups
    (oracle.GLOBAL, 0, 64, 4, 4, 3, True),      # one head per KV head
    (oracle.SWA, 128, 64, 64, 8, 4, True),      # 32 columns
    (oracle.SWA, 100, 32, 8, 2, 3, True),       # window not a multiple of the slice
    (oracle.SWA, 1, 16, 8, 2, 4, True),         # each token sees only itself
    (oracle.GLOBAL, 0, 48, 16, 4, 1, True),     # pages of 48 keys (general paged path)
    (oracle.SWA, 128, 48, 16, 2, 4, True),
])
def test_paged_multi(mode, W, ps, Hq, Hkv, q_len, perm):
    lens = np.array([1, 2, q_len, 63, 64, 65, 1000, 5000, 4097], np.int32)
    B, L = len(lens), int(lens.max())
    print(f"[case] multi mode={mode} W={W} ps={ps} Hq={Hq} Hkv={Hkv} q_len={q_len} perm={perm}", flush=True)
    d = seq_data(B, Hq, Hkv, L, seed=ps + Hq + mode + q_len)
    mp = (L + ps - 1) // ps
    kp, vp, bt = inputs.pages_from_sequence(d["k"], d["v"], L, ps, B * mp + 5, seed=ps, permute=perm)
    qm = drafted_queries(d["q"], lens, q_len)
    got = gpu_multi(mode, W, sa.KV_PAGED, qm, kp, vp, lens, L, d["sink"], bt)
    ref = oracle.decode(qm, kp, vp, lens, d["sink"], mode, W, SCALE, oracle.PAGED, bt)
    assert_parity(got, ref, "multi vs oracle decode")
    # the same rows from the prefill oracle; positions below 0 are zero rows
    valid = [(b, t) for b in range(B) for t in range(q_len) if lens[b] - q_len + t >= 0]
    rows = np.array([(b, h, lens[b] - q_len + t) for b, t in valid for h in range(Hq)])
    pre = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], mode, W, SCALE, rows=rows)
    g = np.stack([got[b, h, t] for b, t in valid for h in range(Hq)])
    assert_parity(g, pre, "multi vs prefill rows")
    for b in range(B):
        for t in range(q_len):
            if lens[b] - q_len + t < 0:
                assert np.all(got[b, :, t] == 0)


def test_max_q_len():
    """q_len = 256 (the largest accepted) with one head per KV head: 256 columns per KV head."""
    Hq = Hkv = 2
    lens = np.array([300, 256, 1000], np.int32)
    B, L = len(lens), int(lens.max())
    d = seq_data(B, Hq, Hkv, L, seed=77)
    kp, vp, bt = inputs.pages_from_sequence(d["k"], d["v"], L, 64, B * 16 + 1, seed=3, permute=True)
    qm = drafted_queries(d["q"], lens, 256)
    got = gpu_multi(oracle.GLOBAL, 0, sa.KV_PAGED, qm, kp, vp, lens, L, d["sink"], bt)
    ref = oracle.decode(qm, kp, vp, lens, d["sink"], oracle.GLOBAL, 0, SCALE, oracle.PAGED, bt)
    assert_parity(got, ref, "q_len 256")


@pytest.mark.parametrize("layout", [sa.KV_RING, sa.KV_PAGED])
def test_q_len_one_equals_decode(layout):
    """q_len = 1 through the multi-token entry point is bit-identical to one-token decode."""
    B, Hq, Hkv, W = 6, 64, 8, 128
    lens = np.array([1, 127, 128, 129, 3000, 700], np.int32)
    L = int(lens.max())
    d = seq_data(B, Hq, Hkv, L, seed=11)
    qn = np.stack([d["q"][b, :, lens[b] - 1] for b in range(B)])
    if layout == sa.KV_RING:
        kc = np.zeros((B, Hkv, W, 192), np.uint16)
        vc = np.zeros((B, Hkv, W, 128), np.uint16)
        for b in range(B):
            k1, v1 = inputs.ring_from_sequence(d["k"][b:b + 1], d["v"][b:b + 1], int(lens[b]), W)
            kc[b], vc[b] = k1[0], v1[0]
        bt = None
    else:
        kc, vc, bt = inputs.pages_from_sequence(d["k"], d["v"], L, 64, B * 47 + 2, seed=4, permute=True)
    args = (dev_bf16(kc), dev_bf16(vc), dev_i32(lens), L, dev_f32(d["sink"]), None if bt is None else dev_i32(bt))
    one = sa.decode(oracle.SWA, W, dev_bf16(qn), layout, *args)
    multi = sa.decode_multi(oracle.SWA, W, dev_bf16(qn[:, :, None]), layout, *args)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), multi[:, :, 0].view(torch.int16))


def test_multi_edge_cases():
    """seq_len 0 -> zero rows; above max_seq_len or a bad page -> NaN rows for that sequence
    only; sink +inf -> zero rows; no sink -> plain softmax."""
    B, Hq, Hkv, ps, q_len = 5, 16, 2, 64, 3
    d = seq_data(B, Hq, Hkv, 600, seed=9)
    kp, vp, bt = inputs.pages_from_sequence(d["k"], d["v"], 600, ps, B * 10, seed=2)
    lens = np.array([600, 0, 700, 600, 300], np.int32)
    bt = bt.copy()
    bt[3, 4] = 10 ** 6
    qm = drafted_queries(d["q"], np.array([600, 0, 600, 600, 300]), q_len)
    sink = d["sink"].copy()
    sink[1] = np.inf
    got = gpu_multi(oracle.GLOBAL, 0, sa.KV_PAGED, qm, kp, vp, lens, 600, sink, bt)
    assert np.all(got[1] == 0)
    assert np.all(np.isnan(got[2])) and np.all(np.isnan(got[3]))
    ok = [0, 4]
    ref = oracle.decode(qm[ok], kp, vp, lens[ok], sink, oracle.GLOBAL, 0, SCALE, oracle.PAGED, bt[ok])
    assert_parity(got[ok], ref, "multi edge lengths")
    assert np.all(got[ok][:, 1] == 0)
    nos = gpu_multi(oracle.GLOBAL, 0, sa.KV_PAGED, qm[ok], kp, vp, lens[ok], 600, None, bt[ok])
    ref2 = oracle.decode(qm[ok], kp, vp, lens[ok], None, oracle.GLOBAL, 0, SCALE, oracle.PAGED, bt[ok])
    assert_parity(nos, ref2, "multi no sink")


def test_ga_verify_workload_sampled():
    """8 sequences at 256K, 4 new tokens each, 64/4 heads, in the launch configuration the
    benchmark times; the oracle checks every row of sequences 0 and 7."""
    w = inputs.GA_VERIFY
    print(f"[case] {w.name}", flush=True)
    d = inputs.decode_paged_inputs(w)
    got = gpu_multi(w.mode, w.window, sa.KV_PAGED, d["q"], d["k"], d["v"], d["seq_lens"], w.ctx_hi, d["sink"],
                    d["block_table"])
    ok = [0, 7]
    ref = oracle.decode(d["q"][ok], d["k"], d["v"], d["seq_lens"][ok], d["sink"], w.mode, w.window, w.scale,
                        oracle.PAGED, d["block_table"][ok])
    assert_parity(got[ok], ref, w.name)
    assert np.all(np.isfinite(got))


def test_q_shape_checked_before_launch():
    """A q whose token axis does not match q_len is refused by the binding (ValueError) before
    any launch: the library only receives a pointer and would read past the end of q."""
    B, Hq, Hkv, ps = 2, 16, 1, 64
    k = torch.zeros((4, Hkv, ps, 192), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((4, Hkv, ps, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, 2), dtype=torch.int32, device="cuda")
    lens = torch.full((B,), 100, dtype=torch.int32, device="cuda")
    q1 = torch.zeros((B, Hq, 1, 192), dtype=torch.bfloat16, device="cuda")
    out4 = torch.empty((B, Hq, 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        sa.sinkattn_decode_multi(sa.GLOBAL, 0, 4, q1, sa.KV_PAGED, k, v, lens, 100, None, out4, None, bt)
    with pytest.raises(ValueError):
        sa.sinkattn_decode_ex(sa.GLOBAL, 0, 4, q1, sa.KV_PAGED, k, v, lens, 100, None, out4, None, bt)
    k8 = torch.zeros((4, Hkv, ps, 192), dtype=torch.uint8, device="cuda")
    v8 = torch.zeros((4, Hkv, ps, 128), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        sa.sinkattn_decode_fp8(sa.GLOBAL, 0, 4, q1, k8, v8, lens, 100, None, 1.0, 1.0, out4, None, bt)
    with pytest.raises(ValueError):
        sa.sinkattn_decode_multi(sa.GLOBAL, 0, 4, q1[:, :, 0], sa.KV_PAGED, k, v, lens, 100, None, out4, None, bt)


@pytest.mark.parametrize("B,Hq,Hkv,q_len,L,nsplit", [
    (128, 16, 4, 1, 1600, 1),   # 512 (sequence, KV head) units: one split over up to 1600 keys
    (100, 16, 4, 1, 1600, 2),   # two splits of 896 keys
    (64, 64, 4, 8, 2000, 1),    # 128 columns per KV head in two column chunks, one split
])
def test_many_sequences_long_single_split(B, Hq, Hkv, q_len, L, nsplit):
    """Enough sequences that the plan keeps one (or two) splits per unit over key ranges longer
    than the unsplit limit of 1024: the split kernel then walks the whole range and writes the
    final output itself (the sink added in its epilogue).  Inputs are drawn for the decoded
    tokens only."""
    need = sa.sinkattn_decode_multi_workspace_bytes(oracle.GLOBAL, 0, B, Hq, Hkv, q_len, L)
    assert need == (0 if nsplit == 1 else B * Hq * q_len * nsplit * 132 * 4), need
    print(f"[case] many sequences B={B} Hq={Hq} Hkv={Hkv} q_len={q_len} L={L} nsplit={nsplit}", flush=True)
    rng = np.random.default_rng(B + q_len)
    lens = rng.integers(L // 2, L + 1, size=B).astype(np.int32)
    lens[0], lens[1], lens[2] = L, 1024, 1025
    ps = 64
    k = inputs.normal((B, Hkv, L, 192), 60 + B, 1)
    v = inputs.normal((B, Hkv, L, 128), 60 + B, 2)
    q = inputs.normal((B, Hq, q_len, 192), 60 + B, 0)
    sink = inputs.sink_values(Hq, 60 + B)
    kp, vp, bt = inputs.pages_from_sequence(k, v, L, ps, B * ((L + ps - 1) // ps) + 3, seed=B, permute=True)
    del k, v
    got = gpu_multi(oracle.GLOBAL, 0, sa.KV_PAGED, q, kp, vp, lens, L, sink, bt)
    ref = oracle.decode(q, kp, vp, lens, sink, oracle.GLOBAL, 0, SCALE, oracle.PAGED, bt)
    assert_parity(got, ref, f"many sequences B={B} q_len={q_len}")
