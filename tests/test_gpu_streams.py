"""Concurrent calls: the library keeps no mutable state between calls (apart from the no-alloc
scratch array, which is not used here), so calls on different streams, issued from one host
thread or from several, must give exactly what the same calls give one after another.  Each
concurrent call has its own outputs and workspace."""
import threading

import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import dev_bf16, dev_f32, dev_i32

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16).cpu().numpy()


def make_calls():
    """Three independent calls (GA prefill, SWA prefill on the ring kernel, paged split
    decode), each a function of an output buffer."""
    w = inputs.Workload("t", "prefill", 0, 2, 16, 1, seqlen=700, seed=90)
    d = inputs.prefill_inputs(w)
    q, k, v, sk = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"]), dev_f32(d["sink"])
    w2 = inputs.Workload("t", "prefill", 1, 4, 64, 8, seqlen=1000, seed=91)
    d2 = inputs.prefill_inputs(w2)
    q2, k2, v2, sk2 = dev_bf16(d2["q"]), dev_bf16(d2["k"]), dev_bf16(d2["v"]), dev_f32(d2["sink"])
    B, Hq, Hkv, L, ps = 3, 64, 4, 6000, 64
    w3 = inputs.Workload("t", "prefill", 0, B, Hq, Hkv, seqlen=L, seed=92)
    d3 = inputs.prefill_inputs(w3)
    lens = np.linspace(L // 2, L, B).astype(np.int32)
    kp, vp, bt = inputs.pages_from_sequence(d3["k"], d3["v"], L, ps, B * (L // ps + 1), seed=92, permute=True)
    q3 = np.stack([d3["q"][b, :, lens[b] - 1] for b in range(B)])[:, :, None, :]
    q3d, kpd, vpd, lg, sk3, btg = dev_bf16(q3), dev_bf16(kp), dev_bf16(vp), dev_i32(lens), dev_f32(d3["sink"]), dev_i32(bt)

    def ga_prefill(out):
        ws = sa.prefill_workspace(q, k)
        return lambda: sa.sinkattn_prefill_ex(oracle.GLOBAL, 0, q, k, v, sk, out, ws)

    def swa_prefill(out):
        ws = sa.prefill_workspace(q2, k2)
        return lambda: sa.sinkattn_prefill_ex(oracle.SWA, 128, q2, k2, v2, sk2, out, ws)

    def decode(out):
        need = sa.sinkattn_decode_multi_workspace_bytes(oracle.GLOBAL, 0, B, Hq, Hkv, 1, L)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
        return lambda: sa.sinkattn_decode_ex(oracle.GLOBAL, 0, 1, q3d, sa.KV_PAGED, kpd, vpd, lg, L, sk3, out, ws, btg)

    shapes = [(2, 16, 700, 128), (4, 64, 1000, 128), (B, Hq, 1, 128)]
    return [ga_prefill, swa_prefill, decode], shapes


def serial_results(makers, shapes):
    res = []
    for mk, shp in zip(makers, shapes):
        out = torch.empty(shp, dtype=torch.bfloat16, device="cuda")
        mk(out)()
        torch.cuda.synchronize()
        res.append(bits(out))
    return res


def test_calls_on_concurrent_streams_match_serial():
    print("[case] three calls on three streams from one thread", flush=True)
    makers, shapes = make_calls()
    want = serial_results(makers, shapes)
    streams = [torch.cuda.Stream() for _ in makers]
    for rep in range(3):
        outs = [torch.full(shp, float("nan"), dtype=torch.bfloat16, device="cuda") for shp in shapes]
        calls = [mk(o) for mk, o in zip(makers, outs)]
        torch.cuda.synchronize()
        for s, c in zip(streams, calls):
            with torch.cuda.stream(s):
                c()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert np.array_equal(bits(o), w), f"call {i} differs on concurrent streams (round {rep})"


def test_calls_from_concurrent_threads_match_serial():
    print("[case] three host threads, each with its own stream, four calls each", flush=True)
    makers, shapes = make_calls()
    want = serial_results(makers, shapes)
    outs = [[torch.full(shp, float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
            for shp in shapes]
    calls = [[mk(o) for o in os_] for mk, os_ in zip(makers, outs)]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for c in calls[i]:
                    c()
            s.synchronize()
        except Exception as e:  # reported on the main thread
            errors.append((i, e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(calls))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (os_, w) in enumerate(zip(outs, want)):
        for j, o in enumerate(os_):
            assert np.array_equal(bits(o), w), f"call {i}, repetition {j} differs when issued from threads"
