"""sinkattn_decode_ex_noalloc, the decode entry point that allocates nothing, against
sinkattn_decode_ex (same arguments plus a caller's workspace) and the oracle: two calls in a
row on the library's scratch array, the second smaller, so stale partials of the first call
would show; and a call whose partials exceed the scratch array is refused on the host."""
import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import assert_parity, dev_bf16, dev_f32, dev_i32, host_f32

pytestmark = pytest.mark.gpu

SCALE = 192 ** -0.5


def case(B, Hq, Hkv, L, ps, q_len, mode, W, seed, kv_fp8=False):
    w = inputs.Workload("t", "prefill", 0, B, Hq, Hkv, seqlen=L, seed=seed)
    d = inputs.prefill_inputs(w)
    lens = np.linspace(max(1, L // 3), L, B).astype(np.int32)
    mp = (L + ps - 1) // ps
    kp, vp, bt = inputs.pages_from_sequence(d["k"], d["v"], L, ps, B * mp + 3, seed=seed, permute=True)
    if kv_fp8:
        kp, vp = oracle.e4m3_encode(kp, 0.05), oracle.e4m3_encode(vp, 0.05)
    qm = np.zeros((B, Hq, q_len, 192), np.uint16)
    for b in range(B):
        for t in range(q_len):
            qm[b, :, t] = d["q"][b, :, lens[b] - q_len + t]
    return d, lens, kp, vp, bt, qm


def run_both(mode, W, q_len, d, lens, kp, vp, bt, qm, kv_fp8):
    B, Hq = qm.shape[:2]
    L = int(lens.max())
    cache = (lambda x: torch.from_numpy(x).to("cuda")) if kv_fp8 else dev_bf16
    args = dict(kv_fp8=kv_fp8, k_scale=0.05 if kv_fp8 else 1.0, v_scale=0.05 if kv_fp8 else 1.0, out_scale=0.75)
    q, k, v, lg, sk, btg = dev_bf16(qm), cache(kp), cache(vp), dev_i32(lens), dev_f32(d["sink"]), dev_i32(bt)
    out_a = torch.empty((B, Hq, q_len, 128), dtype=torch.bfloat16, device="cuda")
    out_b = torch.empty_like(out_a)
    lse_a = torch.empty((B, Hq, q_len), dtype=torch.float32, device="cuda")
    lse_b = torch.empty_like(lse_a)
    need = sa.sinkattn_decode_multi_workspace_bytes(mode, W, B, Hq, kp.shape[1], q_len, L)
    assert 0 < need <= sa.NOALLOC_SCRATCH_BYTES, need  # the split path, which uses the scratch
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    sa.sinkattn_decode_ex_noalloc(mode, W, q_len, q, sa.KV_PAGED, k, v, lg, L, sk, out_a, btg, lse=lse_a, **args)
    sa.sinkattn_decode_ex(mode, W, q_len, q, sa.KV_PAGED, k, v, lg, L, sk, out_b, ws, btg, lse=lse_b, **args)
    torch.cuda.synchronize()
    return host_f32(out_a), host_f32(out_b), lse_a.cpu().numpy(), lse_b.cpu().numpy()


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_noalloc_matches_workspace_entry(kv_fp8):
    # first call: 64 query heads / 4 KV heads, 4 drafted tokens, 9000 keys; second: 16 / 2
    # heads, one token, fewer keys and sequences
    for n, (B, Hq, Hkv, L, q_len, mode, W) in enumerate(((3, 64, 4, 9000, 4, oracle.GLOBAL, 0),
                                                         (2, 16, 2, 3000, 1, oracle.SWA, 1500))):
        print(f"[case] noalloc call {n} fp8={kv_fp8} B={B} Hq={Hq} Hkv={Hkv} L={L} q_len={q_len}", flush=True)
        d, lens, kp, vp, bt, qm = case(B, Hq, Hkv, L, 64, q_len, mode, W, seed=70 + n, kv_fp8=kv_fp8)
        got, want, lse_got, lse_want = run_both(mode, W, q_len, d, lens, kp, vp, bt, qm, kv_fp8)
        assert np.array_equal(got, want), "no-alloc output differs from the workspace entry point"
        assert np.array_equal(lse_got, lse_want), "no-alloc log-sum-exp differs"
        ref, ref_lse = oracle.decode(qm, kp, vp, lens, d["sink"], mode, W, SCALE, oracle.PAGED, bt,
                                     kv_scales=(0.05, 0.05) if kv_fp8 else None, return_lse=True)
        assert_parity(got, 0.75 * ref, f"no-alloc call {n} vs oracle")
        assert np.allclose(lse_got, ref_lse, rtol=1e-5, atol=1e-5)


def test_noalloc_refuses_partials_beyond_scratch():
    """8 sequences of 256K with 16 drafted tokens need 69 MB of partials: refused before any launch."""
    B, Hq, Hkv, ps, L, q_len = 8, 64, 4, 64, 262144, 16
    need = sa.sinkattn_decode_multi_workspace_bytes(sa.GLOBAL, 0, B, Hq, Hkv, q_len, L)
    assert need > sa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, q_len, 192), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, Hkv, ps, 192), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((2, Hkv, ps, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, L // ps), dtype=torch.int32, device="cuda")
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, q_len, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sa.SinkAttnError) as e:
        sa.sinkattn_decode_ex_noalloc(sa.GLOBAL, 0, q_len, q, sa.KV_PAGED, k, v, lens, L, None, out, bt)
    assert e.value.status == 5
