"""Verification of drafted tokens whose keys and values are held beside the cache
(sinkattn_decode_verify): the main model checks the drafts in one parallel pass
("MiMo-V2-Flash 模型架构深度拆解", CH 4.4) and rejects those after the first mismatch (paper
notes §6.4), so a sliding-window ring must not be written before acceptance.  Against the
oracle's decode with keys beside the cache and against the prefill rows of the whole
sequence; the ring is checked to be unchanged."""
import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import assert_parity, dev_bf16, dev_f32, dev_i32, host_f32

pytestmark = pytest.mark.gpu

SCALE = 192 ** -0.5


def split_sequence(d, lens, q_len, W=None, ps=None, n_pages=None, seed=0):
    """Drafts (q, k_new, v_new) at positions lens - q_len .. lens - 1, and a cache of the
    committed positions: a ring of the last W (slot p mod W) or permuted pages whose other
    slots hold data nobody may read."""
    B, Hq = d["q"].shape[:2]
    Hkv = d["k"].shape[1]
    qm = np.zeros((B, Hq, q_len, 192), np.uint16)
    kn = np.zeros((B, Hkv, q_len, 192), np.uint16)
    vn = np.zeros((B, Hkv, q_len, 128), np.uint16)
    for b in range(B):
        nc = int(lens[b]) - q_len
        for t in range(q_len):
            if nc + t >= 0:
                qm[b, :, t] = d["q"][b, :, nc + t]
                kn[b, :, t] = d["k"][b, :, nc + t]
                vn[b, :, t] = d["v"][b, :, nc + t]
    if W is not None:
        kr = inputs.normal((B, Hkv, W, 192), seed, 7)  # slots never written hold noise
        vr = inputs.normal((B, Hkv, W, 128), seed, 8)
        for b in range(B):
            nc = int(lens[b]) - q_len
            for j in range(max(0, nc - W), max(0, nc)):
                kr[b, :, j % W] = d["k"][b, :, j]
                vr[b, :, j % W] = d["v"][b, :, j]
        return qm, kn, vn, kr, vr, None
    mp = int(np.max(lens) + ps - 1) // ps
    bt = np.random.default_rng(seed).permutation(n_pages)[:B * mp].reshape(B, mp).astype(np.int32)
    kp = inputs.normal((n_pages, Hkv, ps, 192), seed, 9)
    vp = inputs.normal((n_pages, Hkv, ps, 128), seed, 10)
    for b in range(B):
        nc = int(lens[b]) - q_len
        for j in range(max(0, nc)):
            kp[bt[b, j // ps], :, j % ps] = d["k"][b, :, j]
            vp[bt[b, j // ps], :, j % ps] = d["v"][b, :, j]
    return qm, kn, vn, kp, vp, bt


def check_rows(got, d, lens, q_len, mode, W, what):
    B, Hq = got.shape[:2]
    valid = [(b, t) for b in range(B) for t in range(q_len) if lens[b] - q_len + t >= 0]
    rows = np.array([(b, h, lens[b] - q_len + t) for b, t in valid for h in range(Hq)])
    pre = oracle.prefill(d["q"], d["k"], d["v"], d["sink"], mode, W, SCALE, rows=rows)
    assert_parity(np.stack([got[b, h, t] for b, t in valid for h in range(Hq)]), pre, what + " vs prefill rows")
    for b in range(B):
        for t in range(q_len):
            if lens[b] - q_len + t < 0:
                assert np.all(got[b, :, t] == 0)


@pytest.mark.parametrize("W,Hq,Hkv,q_len", [(128, 64, 8, 4), (128, 16, 2, 1), (128, 8, 1, 7), (100, 16, 2, 3),
                                            (1, 8, 2, 4), (33, 32, 2, 16)])
def test_ring_verify(W, Hq, Hkv, q_len):
    lens = np.array([1, 2, q_len, W - 1, W, W + 1, W + q_len, 700, 5000], np.int32)
    lens = np.maximum(lens, 1)
    B, L = len(lens), int(lens.max())
    print(f"[case] ring verify W={W} Hq={Hq} Hkv={Hkv} q_len={q_len}", flush=True)
    d = inputs.prefill_inputs(inputs.Workload("t", "prefill", 1, B, Hq, Hkv, seqlen=L, seed=W + q_len))
    qm, kn, vn, kr, vr, _ = split_sequence(d, lens, q_len, W=W, seed=q_len)
    k_ring, v_ring = dev_bf16(kr), dev_bf16(vr)
    k_before, v_before = k_ring.clone(), v_ring.clone()
    out = sa.decode_verify(sa.SWA, W, dev_bf16(qm), sa.KV_RING, k_ring, v_ring, dev_bf16(kn), dev_bf16(vn),
                           dev_i32(lens), L, dev_f32(d["sink"]))
    torch.cuda.synchronize()
    got = host_f32(out)
    ref = oracle.decode(qm, kr, vr, lens, d["sink"], oracle.SWA, W, SCALE, oracle.RING, k_new=kn, v_new=vn)
    assert_parity(got, ref, "ring verify vs oracle")
    check_rows(got, d, lens, q_len, oracle.SWA, W, "ring verify")
    assert torch.equal(k_ring, k_before) and torch.equal(v_ring, v_before), "the ring was written"


@pytest.mark.parametrize("mode,W,ps,q_len", [(oracle.GLOBAL, 0, 64, 4), (oracle.GLOBAL, 0, 48, 2),
                                             (oracle.SWA, 128, 64, 4), (oracle.SWA, 100, 16, 5)])
def test_paged_verify(mode, W, ps, q_len):
    lens = np.array([1, q_len, 63, 64, 65, 1000, 5000, 4097], np.int32)
    B, L, Hq, Hkv = len(lens), int(lens.max()), 64, 4
    print(f"[case] paged verify mode={mode} W={W} ps={ps} q_len={q_len}", flush=True)
    d = inputs.prefill_inputs(inputs.Workload("t", "prefill", mode, B, Hq, Hkv, seqlen=L, seed=ps + q_len))
    npg = B * ((L + ps - 1) // ps) + 7
    qm, kn, vn, kp, vp, bt = split_sequence(d, lens, q_len, ps=ps, n_pages=npg, seed=ps)
    out = sa.decode_verify(mode, W, dev_bf16(qm), sa.KV_PAGED, dev_bf16(kp), dev_bf16(vp), dev_bf16(kn),
                           dev_bf16(vn), dev_i32(lens), L, dev_f32(d["sink"]), dev_i32(bt))
    torch.cuda.synchronize()
    got = host_f32(out)
    ref = oracle.decode(qm, kp, vp, lens, d["sink"], mode, W, SCALE, oracle.PAGED, bt, k_new=kn, v_new=vn)
    assert_parity(got, ref, "paged verify vs oracle")
    check_rows(got, d, lens, q_len, mode, W, "paged verify")


def test_ring_verify_one_token_is_ring_decode():
    """q_len = 1 beside the ring equals ring decode after writing the token into its slot."""
    lens = np.array([5, 127, 128, 129, 4000], np.int32)
    B, L, Hq, Hkv, W = len(lens), int(lens.max()), 64, 8, 128
    d = inputs.prefill_inputs(inputs.Workload("t", "prefill", 1, B, Hq, Hkv, seqlen=L, seed=21))
    qm, kn, vn, kr, vr, _ = split_sequence(d, lens, 1, W=W, seed=21)
    got = host_f32(sa.decode_verify(sa.SWA, W, dev_bf16(qm), sa.KV_RING, dev_bf16(kr), dev_bf16(vr), dev_bf16(kn),
                                    dev_bf16(vn), dev_i32(lens), L, dev_f32(d["sink"])))
    for b in range(B):
        kr[b, :, (lens[b] - 1) % W] = kn[b, :, 0]
        vr[b, :, (lens[b] - 1) % W] = vn[b, :, 0]
    want = host_f32(sa.decode(sa.SWA, W, dev_bf16(qm[:, :, 0]), sa.KV_RING, dev_bf16(kr), dev_bf16(vr),
                              dev_i32(lens), L, dev_f32(d["sink"])))
    torch.cuda.synchronize()
    assert_parity(got[:, :, 0], want.astype(np.float64), "verify q_len=1 vs ring decode")


def test_swa_verify_workload():
    """The sliding-window decode workload (128 rings of 128 slots, lengths U{4096..65536}) with
    4 drafted tokens per sequence beside the rings: every row against the oracle."""
    w = inputs.SWA_VERIFY
    print(f"[case] {w.name}", flush=True)
    dd = inputs.decode_ring_verify_inputs(w)
    lens, L = dd["seq_lens"], w.ctx_hi
    out = sa.decode_verify(w.mode, w.window, dev_bf16(dd["q"]), sa.KV_RING, dev_bf16(dd["k"]), dev_bf16(dd["v"]),
                           dev_bf16(dd["k_new"]), dev_bf16(dd["v_new"]), dev_i32(lens), L, dev_f32(dd["sink"]))
    torch.cuda.synchronize()
    got = host_f32(out)
    ref = oracle.decode(dd["q"], dd["k"], dd["v"], lens, dd["sink"], w.mode, w.window, w.scale, oracle.RING,
                        k_new=dd["k_new"], v_new=dd["v_new"])
    assert_parity(got, ref, f"{w.name} all rows")


def test_verify_argument_errors():
    B, Hq, Hkv, W = 2, 16, 2, 128
    q = torch.zeros((B, Hq, 4, 192), dtype=torch.bfloat16, device="cuda")
    kr = torch.zeros((B, Hkv, W, 192), dtype=torch.bfloat16, device="cuda")
    vr = torch.zeros((B, Hkv, W, 128), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((B, Hkv, 4, 192), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((B,), 200, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # v_new of the wrong shape
        sa.sinkattn_decode_verify(sa.SWA, W, 4, q, sa.KV_RING, kr, vr, kn, kn, lens, 200, None, out, None)
    with pytest.raises(sa.SinkAttnError) as e:  # a ring in global mode
        sa.sinkattn_decode_verify(sa.GLOBAL, W, 4, q, sa.KV_RING, kr, vr, kn, kn[..., :128].contiguous(), lens, 200,
                                  None, out, None)
    assert e.value.status == 3
