"""Decode from an 8-bit (E4M3) paged KV cache against the oracle, which decodes the same
codes from the format's definition (the pages size the cache with one byte per element)."""
import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import assert_parity, dev_bf16, dev_f32, dev_i32, host_f32

pytestmark = pytest.mark.gpu

SCALE = 192 ** -0.5


def dev_u8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to("cuda")


def fp8_cache(B, Hkv, L, ps, seed, k_scale, v_scale, perm=True):
    """Contiguous sequences drawn N(0,1), stored as codes of value / scale, scattered into a
    permuted page pool."""
    k = inputs.normal_e4m3((B, Hkv, L, 192), seed, 1, k_scale)
    v = inputs.normal_e4m3((B, Hkv, L, 128), seed, 2, v_scale)
    mp = (L + ps - 1) // ps
    return inputs.pages_from_sequence(k, v, L, ps, B * mp + 3, seed=seed, permute=perm)


def gpu_fp8(mode, W, q, kp, vp, lens, max_len, sink, ks, vs, bt):
    out = sa.decode_fp8(mode, W, dev_bf16(q), dev_u8(kp), dev_u8(vp), dev_i32(lens), max_len, ks, vs, dev_i32(bt),
                        dev_f32(sink))
    torch.cuda.synchronize()
    return host_f32(out.contiguous())


@pytest.mark.parametrize("mode,W,Hq,Hkv,ps,q_len,ks,vs", [
    (oracle.GLOBAL, 0, 64, 4, 64, 1, 2.0 ** -6, 2.0 ** -6),
    (oracle.GLOBAL, 0, 64, 4, 32, 4, 0.37, 1.9),       # scales that are not powers of two
    (oracle.GLOBAL, 0, 16, 2, 128, 1, 0.05, 0.05),
    (oracle.GLOBAL, 0, 32, 1, 64, 3, 0.02, 0.03),      # 96 columns: two workgroups per KV head
    (oracle.SWA, 128, 64, 8, 64, 1, 0.02, 0.02),
    (oracle.SWA, 100, 8, 2, 32, 4, 0.02, 0.02),
    (oracle.GLOBAL, 0, 4, 4, 64, 1, 1.0, 1.0),         # codes taken as the values themselves
])
def test_fp8_paged(mode, W, Hq, Hkv, ps, q_len, ks, vs):
    lens = np.array([1, 2, 63, 64, 65, 1000, 5000, 4097], np.int32)
    B, L = len(lens), int(lens.max())
    print(f"[case] fp8 mode={mode} W={W} Hq={Hq} Hkv={Hkv} ps={ps} q_len={q_len} scales={ks},{vs}", flush=True)
    kp, vp, bt = fp8_cache(B, Hkv, L, ps, seed=ps + Hq + q_len, k_scale=ks, v_scale=vs)
    q = inputs.normal((B, Hq, q_len, 192), 5 + ps, 0)
    sink = inputs.sink_values(Hq, 7)
    got = gpu_fp8(mode, W, q, kp, vp, lens, L, sink, ks, vs, bt)
    ref = oracle.decode(q, kp, vp, lens, sink, mode, W, SCALE, oracle.PAGED, bt, kv_scales=(ks, vs))
    assert_parity(got, ref, "fp8 paged decode")


def test_fp8_edges():
    """seq_len 0 -> zero rows; above max_seq_len or a page id outside the pool -> NaN rows for
    that sequence only; sink +inf -> zero rows; no sink -> plain softmax."""
    B, Hq, Hkv, ps, L = 5, 16, 2, 64, 600
    kp, vp, bt = fp8_cache(B, Hkv, L, ps, seed=11, k_scale=0.02, v_scale=0.02)
    bt = bt.copy()
    bt[3, 2] = 10 ** 6
    lens = np.array([600, 0, 700, 600, 300], np.int32)
    q = inputs.normal((B, Hq, 192), 12, 0)
    sink = inputs.sink_values(Hq, 13).copy()
    sink[1] = np.inf
    got = gpu_fp8(oracle.GLOBAL, 0, q, kp, vp, lens, L, sink, 0.02, 0.02, bt)
    assert np.all(got[1] == 0)
    assert np.all(np.isnan(got[2])) and np.all(np.isnan(got[3]))
    ok = [0, 4]
    ref = oracle.decode(q[ok], kp, vp, lens[ok], sink, oracle.GLOBAL, 0, SCALE, oracle.PAGED, bt[ok],
                        kv_scales=(0.02, 0.02))
    assert_parity(got[ok], ref, "fp8 edges")
    assert np.all(got[ok][:, 1] == 0)
    nos = gpu_fp8(oracle.GLOBAL, 0, q[ok], kp, vp, lens[ok], L, None, 0.02, 0.02, bt[ok])
    ref2 = oracle.decode(q[ok], kp, vp, lens[ok], None, oracle.GLOBAL, 0, SCALE, oracle.PAGED, bt[ok],
                         kv_scales=(0.02, 0.02))
    assert_parity(nos, ref2, "fp8 no sink")


def test_ga_decode_fp8_workload_sampled():
    """8 sequences at 256K in 64-token E4M3 pages with a permuted table, 64/4 heads, in the
    launch configuration the benchmark times; every row of sequences 0 and 7."""
    w = inputs.GA_DECODE_FP8
    print(f"[case] {w.name}", flush=True)
    d = inputs.decode_paged_inputs(w)
    ks, vs = d["kv_scales"]
    got = gpu_fp8(w.mode, w.window, d["q"], d["k"], d["v"], d["seq_lens"], w.ctx_hi, d["sink"], ks, vs,
                  d["block_table"])
    assert np.all(np.isfinite(got))
    ok = [0, 7]
    ref = oracle.decode(d["q"][ok], d["k"], d["v"], d["seq_lens"][ok], d["sink"], w.mode, w.window, w.scale,
                        oracle.PAGED, d["block_table"][ok], kv_scales=(ks, vs))
    assert_parity(got[ok], ref, w.name)
