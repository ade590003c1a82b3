"""Library calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library allocates nothing, never synchronises and launches only kernels on the caller's
stream, so its calls can be captured.  Each case runs the call eagerly, captures the same
call on the same buffers, and replays the graph several times with eager work (the output
overwritten, host synchronisations) between the replays; every replay must reproduce the
eager output bit for bit.  Before the last replay the inputs are changed in place, and the
replay must then equal an eager call on the new inputs: the graph reads the buffers' current
contents.  Parity of the eager calls themselves with the oracle is covered by the other GPU
tests."""
import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import dev_bf16, dev_f32, dev_i32

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).cpu().numpy()


def check_replays(call, outs, change_inputs):
    """call() launches into outs; change_inputs() rewrites the input buffers in place."""
    call()
    torch.cuda.synchronize()
    want = [bits(o) for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert np.array_equal(bits(o), w), f"replay {rep} differs from the eager call"
    change_inputs()
    torch.cuda.synchronize()
    call()
    torch.cuda.synchronize()
    want2 = [bits(o) for o in outs]
    assert any(not np.array_equal(a, b) for a, b in zip(want, want2)), "the input change did not change the output"
    for o in outs:
        o.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for o, w in zip(outs, want2):
        assert np.array_equal(bits(o), w), "replay after the input change differs from the eager call"


def test_graph_decode_noalloc_paged_verify():
    """Split decode with merge, 4 drafted tokens per sequence, paged cache, partials in the
    library's scratch array."""
    B, Hq, Hkv, L, ps, q_len = 3, 64, 4, 9000, 64, 4
    print(f"[case] graph noalloc decode B={B} Hq={Hq} Hkv={Hkv} L={L} q_len={q_len}", flush=True)
    w = inputs.Workload("t", "prefill", 0, B, Hq, Hkv, seqlen=L, seed=80)
    d = inputs.prefill_inputs(w)
    lens = np.linspace(L // 3, L, B).astype(np.int32)
    mp = (L + ps - 1) // ps
    kp, vp, bt = inputs.pages_from_sequence(d["k"], d["v"], L, ps, B * mp + 3, seed=80, permute=True)
    qm = np.zeros((B, Hq, q_len, 192), np.uint16)
    for b in range(B):
        for t in range(q_len):
            qm[b, :, t] = d["q"][b, :, lens[b] - q_len + t]
    q, k, v, lg, sk, btg = dev_bf16(qm), dev_bf16(kp), dev_bf16(vp), dev_i32(lens), dev_f32(d["sink"]), dev_i32(bt)
    out = torch.empty((B, Hq, q_len, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, q_len), dtype=torch.float32, device="cuda")
    q2 = dev_bf16(inputs.normal((B, Hq, q_len, 192), 81, 0))

    def call():
        sa.sinkattn_decode_ex_noalloc(oracle.GLOBAL, 0, q_len, q, sa.KV_PAGED, k, v, lg, L, sk, out, btg, lse=lse,
                                      out_scale=0.75)

    check_replays(call, [out, lse], lambda: q.copy_(q2))


def test_graph_fused_decode_step_ring():
    """The whole sliding-window decode step (RoPE, ring write, attention) in one kernel: a
    replay writes the same ring slot with the same rotated key and value, so it is
    idempotent."""
    B, Hq, Hkv, W = 10, 64, 8, 128
    print(f"[case] graph fused decode step B={B} Hq={Hq} Hkv={Hkv} W={W}", flush=True)
    lens = np.array([1, 2, 64, 127, 128, 129, 200, 4096, 0, 65536], np.int32)
    q = dev_bf16(inputs.normal((B, Hq, 1, 192), 82, 0))
    kn = dev_bf16(inputs.normal((B, Hkv, 1, 192), 82, 1))
    vn = dev_bf16(inputs.normal((B, Hkv, 1, 128), 82, 2))
    kc = dev_bf16(inputs.normal((B, Hkv, W, 192), 83, 1))
    vc = dev_bf16(inputs.normal((B, Hkv, W, 128), 83, 2))
    lg, sk = dev_i32(lens), dev_f32(inputs.sink_values(Hq, 84))
    out = torch.empty((B, Hq, 1, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
    kn2 = dev_bf16(inputs.normal((B, Hkv, 1, 192), 85, 1))

    def call():
        sa.sinkattn_decode_step(sa.SWA_ROPE_THETA, W, q, kn, vn, kc, vc, lg, int(lens.max()), sk, out, lse=lse)

    check_replays(call, [out, lse], lambda: kn.copy_(kn2))


def test_graph_prefill_causal_with_workspace():
    """Causal prefill (the V^T pre-pass and the pipelined kernel) with a caller's workspace."""
    B, Hq, Hkv, L = 2, 16, 1, 517
    print(f"[case] graph prefill B={B} Hq={Hq} Hkv={Hkv} L={L}", flush=True)
    w = inputs.Workload("t", "prefill", 0, B, Hq, Hkv, seqlen=L, seed=86)
    d = inputs.prefill_inputs(w)
    q, k, v, sk = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]), dev_f32(d["sink"])
    out = torch.empty((B, Hq, L, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    ws = sa.prefill_workspace(q, k)
    v2 = dev_bf16(inputs.normal((B, Hkv, L, 128), 87, 2))

    def call():
        sa.sinkattn_prefill_ex(oracle.GLOBAL, 0, q, k, v, sk, out, ws, lse=lse)

    check_replays(call, [out, lse], lambda: v.copy_(v2))
