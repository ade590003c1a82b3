"""Race check: every attention kernel, run a second time with its workgroups taking their work
in reverse order (SINKATTN_GRID_ORDER=reversed), so that the work runs in another order and
next to other neighbours, must give bit-identical outputs; a race on LDS or on the split
partials would show as a difference.  Small prefill and decode cases of every kernel path."""
import os

import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import assert_parity, dev_bf16, dev_f32, dev_i32, host_f32

pytestmark = pytest.mark.gpu

SCALE = 192 ** -0.5


def both_orders(fn):
    os.environ.pop("SINKATTN_GRID_ORDER", None)
    a = fn()
    os.environ["SINKATTN_GRID_ORDER"] = "reversed"
    try:
        b = fn()
    finally:
        os.environ.pop("SINKATTN_GRID_ORDER", None)
    return a, b


@pytest.mark.parametrize("mode,W,Hq,Hkv,L", [(oracle.GLOBAL, 0, 64, 4, 700), (oracle.SWA, 128, 64, 8, 900),
                                             (oracle.GLOBAL, 0, 8, 4, 333), (oracle.SWA, 100, 16, 2, 517)])
def test_prefill_grid_order(mode, W, Hq, Hkv, L):
    print(f"[case] grid order prefill mode={mode} W={W} Hq={Hq} Hkv={Hkv} L={L}", flush=True)
    d = inputs.prefill_inputs(inputs.Workload("t", "prefill", mode, 2, Hq, Hkv, seqlen=L, seed=L + Hq))
    q, k, v, s = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]), dev_f32(d["sink"])

    def run():
        out = sa.prefill(mode, W, q, k, v, s)
        torch.cuda.synchronize()
        return host_f32(out)

    a, b = both_orders(run)
    assert np.array_equal(a, b), "prefill output depends on the workgroup order"
    assert_parity(b, oracle.prefill(d["q"], d["k"], d["v"], d["sink"], mode, W, SCALE), "reversed order vs oracle")


@pytest.mark.parametrize("layout,mode,W,q_len,L", [(sa.KV_RING, oracle.SWA, 128, 1, 3000),
                                                   (sa.KV_PAGED, oracle.GLOBAL, 0, 1, 20000),
                                                   (sa.KV_PAGED, oracle.GLOBAL, 0, 4, 9000),
                                                   (sa.KV_PAGED, oracle.SWA, 128, 3, 5000)])
def test_decode_grid_order(layout, mode, W, q_len, L):
    print(f"[case] grid order decode layout={layout} mode={mode} q_len={q_len} L={L}", flush=True)
    B, Hq, Hkv, ps = 4, 64, 4 if mode == oracle.GLOBAL else 8, 64
    d = inputs.prefill_inputs(inputs.Workload("t", "prefill", mode, B, Hq, Hkv, seqlen=L, seed=q_len + L))
    lens = np.array([L, L // 2, 77, L - 5], np.int32)
    qm = np.stack([np.stack([d["q"][b, :, lens[b] - q_len + t] for t in range(q_len)], axis=1) for b in range(B)])
    if layout == sa.KV_RING:
        kc = np.zeros((B, Hkv, W, 192), np.uint16)
        vc = np.zeros((B, Hkv, W, 128), np.uint16)
        for b in range(B):
            for j in range(max(0, lens[b] - W), lens[b]):
                kc[b, :, j % W] = d["k"][b, :, j]
                vc[b, :, j % W] = d["v"][b, :, j]
        bt = None
    else:
        kc, vc, bt = inputs.pages_from_sequence(d["k"], d["v"], L, ps, B * (L // ps + 1) + 3, seed=L)
    qd, kd, vd, ld, sd = dev_bf16(qm), dev_bf16(kc), dev_bf16(vc), dev_i32(lens), dev_f32(d["sink"])
    btd = None if bt is None else dev_i32(bt)

    def run():
        out = sa.decode_multi(mode, W, qd, layout, kd, vd, ld, L, sd, btd)
        torch.cuda.synchronize()
        return host_f32(out)

    a, b = both_orders(run)
    assert np.array_equal(a, b), "decode output depends on the workgroup order"
    ref = oracle.decode(qm, kc, vc, lens, d["sink"], mode, W, SCALE,
                        oracle.RING if layout == sa.KV_RING else oracle.PAGED, bt)
    assert_parity(b, ref, "reversed order vs oracle")


@pytest.mark.parametrize("mode,W,Hq,Hkv,L,B", [(oracle.GLOBAL, 0, 16, 4, 333, 2), (oracle.SWA, 128, 16, 2, 517, 1)])
def test_backward_grid_order(mode, W, Hq, Hkv, L, B):
    """The dK/dV kernel's two waves per key group exchange P through LDS and both backward
    kernels share quadruple- and triple-buffered tiles: the gradients must not depend on the
    workgroup order."""
    print(f"[case] grid order backward mode={mode} W={W} Hq={Hq} Hkv={Hkv} L={L} B={B}", flush=True)
    d = inputs.prefill_inputs(inputs.Workload("t", "prefill", mode, B, Hq, Hkv, seqlen=L, seed=L + 7))
    dout = inputs.normal((B, Hq, L, 128), L, 5)
    q, k, v, s = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]), dev_f32(d["sink"])
    out = torch.empty((B, Hq, L, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    ws = torch.empty(sa.sinkattn_prefill_chunk_workspace_bytes(B, L, Hq, Hkv, L), dtype=torch.uint8, device="cuda")
    sa.sinkattn_prefill_ex(mode, W, q, k, v, s, out, ws, lse=lse)
    do = dev_bf16(dout)

    def run():
        g = sa.prefill_backward(mode, W, q, k, v, s, out, do, lse)
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in g]

    a, b = both_orders(run)
    for name, x, y in zip(("dq", "dk", "dv", "dsink"), a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), f"{name} depends on the workgroup order"
    ref = oracle.prefill_backward(d["q"], d["k"], d["v"], d["sink"], dout, mode, W, SCALE)
    for name, x, r in zip(("dq", "dk", "dv"), b, ref):
        rel = np.linalg.norm(x - r) / np.linalg.norm(r)
        assert rel <= 5e-3, f"{name}: rel-L2 {rel:.3e} against the oracle"


def test_decode_step_grid_order():
    """The one-kernel decode step writes each ring's new slot from one wave and reads it back
    from registers and LDS: the output and the rings must not depend on the workgroup order."""
    print("[case] grid order fused decode step B=16 W=128", flush=True)
    B, Hq, Hkv, W = 16, 64, 8, 128
    lens = np.array([1, 5, 127, 128, 129, 300, 4000, 65536] * 2, np.int32)
    q = inputs.normal((B, Hq, 1, 192), 95, 0)
    kn = inputs.normal((B, Hkv, 1, 192), 95, 1)
    vn = inputs.normal((B, Hkv, 1, 128), 95, 2)
    kc = inputs.normal((B, Hkv, W, 192), 96, 1)
    vc = inputs.normal((B, Hkv, W, 128), 96, 2)
    sink = dev_f32(inputs.sink_values(Hq, 97))
    qd, knd, vnd, ld = dev_bf16(q), dev_bf16(kn), dev_bf16(vn), dev_i32(lens)

    def run():
        kcd, vcd = dev_bf16(kc), dev_bf16(vc)
        out = torch.empty((B, Hq, 1, 128), dtype=torch.bfloat16, device="cuda")
        sa.sinkattn_decode_step(sa.SWA_ROPE_THETA, W, qd, knd, vnd, kcd, vcd, ld, int(lens.max()), sink, out)
        torch.cuda.synchronize()
        return [t.view(torch.int16).cpu().numpy() for t in (out, kcd, vcd)]

    a, b = both_orders(run)
    for name, x, y in zip(("output", "k ring", "v ring"), a, b):
        assert np.array_equal(x, y), f"decode step {name} depends on the workgroup order"


@pytest.mark.parametrize("q_len,Hq,Hkv", [(4, 64, 8), (1, 16, 2)])
def test_ring_verify_grid_order(q_len, Hq, Hkv):
    """Drafts beside a ring take the single-buffer kernel with K in registers and up to two
    slices per wave: the output must not depend on the workgroup order."""
    print(f"[case] grid order ring verify q_len={q_len} Hq={Hq} Hkv={Hkv}", flush=True)
    W = 128
    lens = np.array([1, 3, 127, 128, 131, 132, 500, 4096], np.int32)
    B = len(lens)
    q = dev_bf16(inputs.normal((B, Hq, q_len, 192), 98, 0))
    kn = dev_bf16(inputs.normal((B, Hkv, q_len, 192), 98, 1))
    vn = dev_bf16(inputs.normal((B, Hkv, q_len, 128), 98, 2))
    kr = dev_bf16(inputs.normal((B, Hkv, W, 192), 98, 3))
    vr = dev_bf16(inputs.normal((B, Hkv, W, 128), 98, 4))
    sink, ld = dev_f32(inputs.sink_values(Hq, 99)), dev_i32(lens)

    def run():
        out = sa.decode_verify(sa.SWA, W, q, sa.KV_RING, kr, vr, kn, vn, ld, int(lens.max()), sink)
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy()

    a, b = both_orders(run)
    assert np.array_equal(a, b), "ring verify output depends on the workgroup order"
