"""The steps on either side of the attention against the oracle: partial RoPE, writing new
tokens into ring and paged caches (bf16 and E4M3), and the epilogue options (output scale,
per-row log-sum-exp) of prefill and decode; then one whole decode step, RoPE -> append ->
attention, against the same chain on the oracle."""
import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import assert_parity, dev_bf16, dev_f32, dev_i32, host_f32

pytestmark = pytest.mark.gpu

SCALE = 192 ** -0.5
LSE_ATOL = 1e-3  # float32 sums of float32 exponentials against the fp64 oracle


def host_bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_lse(got, ref, what):
    got = np.asarray(got, np.float64)
    same_inf = (np.isinf(ref) & (got == ref))
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(got - ref))
    print(f"[lse] {what}: max_abs={np.nanmax(err):.3e}", flush=True)
    assert np.all(np.isfinite(ref) | same_inf), f"{what}: infinite rows differ"
    assert np.nanmax(err) <= LSE_ATOL, f"{what}: lse max_abs {np.nanmax(err):.3e}"


@pytest.mark.parametrize("theta,pos_kind", [(sa.SWA_ROPE_THETA, "pos0"), (sa.GA_ROPE_THETA, "pos0_far"),
                                            (sa.GA_ROPE_THETA, "seq_lens")])
def test_rope(theta, pos_kind):
    B, H, rows = 3, 64, 100
    x = inputs.normal((B, H, rows, 192), 31, 0)
    xd = dev_bf16(x)
    if pos_kind == "seq_lens":
        lens = np.array([100, 5000, 262144], np.int32)
        sa.sinkattn_rope(theta, xd, seq_lens=dev_i32(lens))
        pos = (lens[:, None] - rows + np.arange(rows)[None, :])[:, None, :]
    else:
        p0 = 0 if pos_kind == "pos0" else 262144 - rows
        sa.sinkattn_rope(theta, xd, pos0=p0)
        pos = np.broadcast_to(p0 + np.arange(rows), (B, 1, rows))
    torch.cuda.synchronize()
    got = host_f32(xd)
    ref = oracle.rope(x, np.broadcast_to(pos, (B, H, rows)), theta)
    assert np.array_equal(host_bits(xd)[..., 64:], x[..., 64:]), "trailing 128 dimensions changed"
    assert_parity(got, ref, f"rope {pos_kind}")


@pytest.mark.parametrize("layout,fp8", [(sa.KV_RING, False), (sa.KV_PAGED, False), (sa.KV_PAGED, True),
                                        (sa.KV_RING, True)])
@pytest.mark.parametrize("n_new", [1, 4, 200])
def test_kv_append(layout, fp8, n_new):
    B, Hkv, W, ps = 3, 8, 128, 64
    lens = np.array([n_new, 1000, 5000], np.int32) if n_new > 1 else np.array([1, 129, 5000], np.int32)
    lens[0] = max(1, n_new - 2)  # fewer tokens than new rows: the first positions are skipped
    kn = inputs.normal((B, Hkv, n_new, 192), 40 + n_new, 1)
    vn = inputs.normal((B, Hkv, n_new, 128), 40 + n_new, 2)
    cdt = np.uint8 if fp8 else np.uint16
    scales = (0.05, 0.03) if fp8 else None
    rng = np.random.default_rng(41)
    if layout == sa.KV_RING:
        kc = rng.integers(0, 255, (B, Hkv, W, 192)).astype(cdt)
        vc = rng.integers(0, 255, (B, Hkv, W, 128)).astype(cdt)
        bt = None
    else:
        mp = (int(lens.max()) + ps - 1) // ps
        npg = B * mp + 4
        kc = rng.integers(0, 255, (npg, Hkv, ps, 192)).astype(cdt)
        vc = rng.integers(0, 255, (npg, Hkv, ps, 128)).astype(cdt)
        bt = inputs.page_table(B, mp, npg, 42, True)
    kd = torch.from_numpy(kc.view(np.int16) if not fp8 else kc).to("cuda")
    vd = torch.from_numpy(vc.view(np.int16) if not fp8 else vc).to("cuda")
    if not fp8:
        kd, vd = kd.view(torch.bfloat16), vd.view(torch.bfloat16)
    sa.sinkattn_kv_append(layout, kd, vd, dev_bf16(kn), dev_bf16(vn), dev_i32(lens), window=W,
                          block_table=None if bt is None else dev_i32(bt), kv_fp8=fp8,
                          k_scale=scales[0] if fp8 else 1.0, v_scale=scales[1] if fp8 else 1.0)
    torch.cuda.synchronize()
    oracle.kv_append(kc, vc, oracle.RING if layout == sa.KV_RING else oracle.PAGED, kn, vn, lens, window=W,
                     block_table=bt, fp8_scales=scales)
    gk = kd.view(torch.uint8).cpu().numpy() if fp8 else host_bits(kd)
    gv = vd.view(torch.uint8).cpu().numpy() if fp8 else host_bits(vd)
    assert np.array_equal(gk, kc) and np.array_equal(gv, vc), "cache contents differ from the oracle's append"


@pytest.mark.parametrize("mode,W,Hq,Hkv,Lk,Lq", [(oracle.GLOBAL, 0, 64, 4, 700, 700), (oracle.SWA, 128, 64, 8, 900, 77),
                                                 (oracle.GLOBAL, 0, 8, 4, 300, 300), (oracle.SWA, 128, 64, 8, 300, 300)])
def test_prefill_epilogue(mode, W, Hq, Hkv, Lk, Lq):
    w = inputs.Workload("t", "prefill", 0, 1, Hq, Hkv, seqlen=Lk, seed=50 + Lq)
    d = inputs.prefill_inputs(w)
    sink = d["sink"].copy()
    sink[1] = np.inf
    sink[2] = -np.inf
    qc = np.ascontiguousarray(d["q"][:, :, Lk - Lq:])
    q, k, v = dev_bf16(qc), dev_bf16(d["k"]), dev_bf16(d["v"])
    out = torch.empty((1, Hq, Lq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, Hq, Lq), dtype=torch.float32, device="cuda")
    ws = torch.empty(sa.sinkattn_prefill_chunk_workspace_bytes(1, Lq, Hq, Hkv, Lk), dtype=torch.uint8, device="cuda")
    sa.sinkattn_prefill_ex(mode, W, q, k, v, dev_f32(sink), out, ws, out_scale=0.707, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.prefill_chunk(qc, d["k"], d["v"], sink, mode, W, SCALE, return_lse=True)
    assert_parity(host_f32(out), 0.707 * ref, "prefill out_scale")
    check_lse(lse.cpu().numpy(), ref_lse, "prefill")


@pytest.mark.parametrize("fp8,q_len,long", [(False, 1, False), (False, 4, True), (True, 1, True), (True, 3, False)])
def test_decode_epilogue(fp8, q_len, long):
    """lse and out_scale through the single-split epilogue (short contexts) and the merge
    kernel (long ones), with rows before their sequence, sink +inf and no-sink heads."""
    B, Hq, Hkv, ps = 4, 64, 4, 64
    L = 20000 if long else 900
    lens = np.array([1, 2, L, L // 3], np.int32)
    kseq = inputs.normal_e4m3((B, Hkv, L, 192), 60, 1, 0.02) if fp8 else inputs.normal((B, Hkv, L, 192), 60, 1)
    vseq = inputs.normal_e4m3((B, Hkv, L, 128), 60, 2, 0.02) if fp8 else inputs.normal((B, Hkv, L, 128), 60, 2)
    mp = (L + ps - 1) // ps
    kp, vp, bt = inputs.pages_from_sequence(kseq, vseq, L, ps, B * mp + 3, seed=61)
    q = inputs.normal((B, Hq, q_len, 192), 62, 0)
    sink = inputs.sink_values(Hq, 63).copy()
    sink[5] = np.inf
    sink[6] = -np.inf
    tdev = (lambda a: torch.from_numpy(a).to("cuda")) if fp8 else dev_bf16
    out = torch.empty((B, Hq, q_len, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, q_len), dtype=torch.float32, device="cuda")
    ws = sa.decode_multi_workspace(oracle.GLOBAL, 0, B, Hq, Hkv, q_len, L, "cuda")
    sa.sinkattn_decode_ex(oracle.GLOBAL, 0, q_len, dev_bf16(q), sa.KV_PAGED, tdev(kp), tdev(vp), dev_i32(lens), L,
                          dev_f32(sink), out, ws, dev_i32(bt), kv_fp8=fp8, k_scale=0.02, v_scale=0.02, out_scale=0.5,
                          lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(q, kp, vp, lens, sink, oracle.GLOBAL, 0, SCALE, oracle.PAGED, bt,
                                 kv_scales=(0.02, 0.02) if fp8 else None, return_lse=True)
    assert_parity(host_f32(out), 0.5 * ref, "decode out_scale")
    check_lse(lse.cpu().numpy(), ref_lse, f"decode fp8={fp8} long={long}")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("fp8", [False, True])
def test_decode_step_chain(fp8, fused):
    """One decode step of 2 new tokens on 256 + 2 positions: RoPE on q and the new keys, append
    into pages (separate kernels, or the fused prologue), attention with the value scale and
    lse -- against the oracle's chain."""
    B, Hq, Hkv, ps, n_old, n_new = 2, 16, 2, 32, 256, 2
    theta = sa.GA_ROPE_THETA
    ks = vs = 0.03
    L = n_old + n_new
    kseq = inputs.normal((B, Hkv, n_old, 192), 70, 1)
    vseq = inputs.normal((B, Hkv, n_old, 128), 70, 2)
    pos_old = np.broadcast_to(np.arange(n_old), (B, Hkv, n_old))
    krot_old = inputs.bf16_bits(oracle.rope(kseq, pos_old, theta).astype(np.float32))
    if fp8:
        kstore, vstore = oracle.e4m3_encode(krot_old, ks), oracle.e4m3_encode(vseq, vs)
    else:
        kstore, vstore = krot_old, vseq
    mp = (L + ps - 1) // ps
    # room for the new tokens: the table covers L positions, the last two still empty
    pad = ((0, 0), (0, 0), (0, n_new), (0, 0))
    kp, vp, bt = inputs.pages_from_sequence(np.pad(kstore, pad), np.pad(vstore, pad), L, ps, B * mp + 1, seed=71)
    kp = np.ascontiguousarray(kp)
    vp = np.ascontiguousarray(vp)
    q = inputs.normal((B, Hq, n_new, 192), 72, 0)
    kn = inputs.normal((B, Hkv, n_new, 192), 72, 1)
    vn = inputs.normal((B, Hkv, n_new, 128), 72, 2)
    lens = np.full(B, L, np.int32)
    sink = inputs.sink_values(Hq, 73)
    # GPU chain
    tdev = (lambda a: torch.from_numpy(a).to("cuda")) if fp8 else dev_bf16
    kpd, vpd = tdev(kp), tdev(vp)
    qd, knd, vnd, lensd, btd = dev_bf16(q), dev_bf16(kn), dev_bf16(vn), dev_i32(lens), dev_i32(bt)
    if fused:
        sa.sinkattn_decode_prologue(theta, sa.KV_PAGED, qd, qd, knd, vnd, kpd, vpd, lensd, block_table=btd, kv_fp8=fp8,
                                    k_scale=ks, v_scale=vs)
    else:
        sa.sinkattn_rope(theta, qd, seq_lens=lensd)
        sa.sinkattn_rope(theta, knd, seq_lens=lensd)
        sa.sinkattn_kv_append(sa.KV_PAGED, kpd, vpd, knd, vnd, lensd, block_table=btd, kv_fp8=fp8, k_scale=ks,
                              v_scale=vs)
    out = torch.empty((B, Hq, n_new, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, n_new), dtype=torch.float32, device="cuda")
    sa.sinkattn_decode_ex(oracle.GLOBAL, 0, n_new, qd, sa.KV_PAGED, kpd, vpd, lensd, L, dev_f32(sink), out, None, btd,
                          kv_fp8=fp8, k_scale=ks, v_scale=vs, out_scale=0.707, lse=lse)
    torch.cuda.synchronize()
    # oracle chain: the rotated rows are rounded to bf16 as the GPU stores them
    pos_new = lens[:, None, None] - n_new + np.arange(n_new)[None, None, :]
    qr = inputs.bf16_bits(oracle.rope(q, np.broadcast_to(pos_new, q.shape[:3]), theta).astype(np.float32))
    knr = inputs.bf16_bits(oracle.rope(kn, np.broadcast_to(pos_new, kn.shape[:3]), theta).astype(np.float32))
    oracle.kv_append(kp, vp, oracle.PAGED, knr, vn, lens, block_table=bt, fp8_scales=(ks, vs) if fp8 else None)
    ref, ref_lse = oracle.decode(qr, kp, vp, lens, sink, oracle.GLOBAL, 0, SCALE, oracle.PAGED, bt,
                                 kv_scales=(ks, vs) if fp8 else None, return_lse=True)
    assert_parity(host_f32(out), 0.707 * ref, f"decode step chain fp8={fp8}")
    check_lse(lse.cpu().numpy(), ref_lse, f"decode step chain fp8={fp8}")


@pytest.mark.parametrize("layout,fp8", [(sa.KV_RING, False), (sa.KV_PAGED, False), (sa.KV_PAGED, True),
                                        (sa.KV_RING, True)])
@pytest.mark.parametrize("n_new,in_place", [(1, True), (4, False), (130, True)])
def test_fused_prologue_is_separate_kernels(layout, fp8, n_new, in_place):
    """The fused prologue gives, bit for bit, the rotated queries and the cache contents of
    sinkattn_rope (q), sinkattn_rope (k) and sinkattn_kv_append in turn, and leaves k_new as it
    was; rings (W = 128, a call longer than the ring) and pages, bf16 and E4M3."""
    B, Hq, Hkv, W, ps = 3, 64, 8, 128, 64
    theta = sa.SWA_ROPE_THETA if layout == sa.KV_RING else sa.GA_ROPE_THETA
    lens = np.array([max(1, n_new - 2), 1000, 20000], np.int32)
    q = inputs.normal((B, Hq, n_new, 192), 80 + n_new, 0)
    kn = inputs.normal((B, Hkv, n_new, 192), 80 + n_new, 1)
    vn = inputs.normal((B, Hkv, n_new, 128), 80 + n_new, 2)
    cdt = np.uint8 if fp8 else np.uint16
    rng = np.random.default_rng(81)
    if layout == sa.KV_RING:
        shape_k, shape_v, bt = (B, Hkv, W, 192), (B, Hkv, W, 128), None
    else:
        mp = (int(lens.max()) + ps - 1) // ps
        npg = B * mp + 4
        shape_k, shape_v = (npg, Hkv, ps, 192), (npg, Hkv, ps, 128)
        bt = dev_i32(inputs.page_table(B, mp, npg, 82, True))
    kc = rng.integers(0, 255, shape_k).astype(cdt)
    vc = rng.integers(0, 255, shape_v).astype(cdt)

    def dev_cache(c):
        t = torch.from_numpy(c.view(np.int16) if not fp8 else c).to("cuda")
        return t if fp8 else t.view(torch.bfloat16)

    def raw(t):
        return t.view(torch.uint8).cpu().numpy() if fp8 else host_bits(t)

    kw = dict(window=W, block_table=bt, kv_fp8=fp8, k_scale=0.05 if fp8 else 1.0, v_scale=0.03 if fp8 else 1.0)
    lensd = dev_i32(lens)
    # separate kernels
    qa, ka, va = dev_bf16(q), dev_bf16(kn), dev_bf16(vn)
    kca, vca = dev_cache(kc), dev_cache(vc)
    sa.sinkattn_rope(theta, qa, seq_lens=lensd)
    sa.sinkattn_rope(theta, ka, seq_lens=lensd)
    sa.sinkattn_kv_append(layout, kca, vca, ka, va, lensd, **kw)
    # fused
    qb, kb, vb = dev_bf16(q), dev_bf16(kn), dev_bf16(vn)
    kcb, vcb = dev_cache(kc), dev_cache(vc)
    qo = qb if in_place else torch.empty_like(qb)
    sa.sinkattn_decode_prologue(theta, layout, qb, qo, kb, vb, kcb, vcb, lensd, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qo), host_bits(qa)), "rotated queries differ"
    assert np.array_equal(raw(kcb), raw(kca)) and np.array_equal(raw(vcb), raw(vca)), "cache contents differ"
    assert np.array_equal(host_bits(kb), kn), "k_new was modified"
    if not in_place:
        assert np.array_equal(host_bits(qb), q), "q_in was modified"


@pytest.mark.parametrize("out_scale,with_lse", [(1.0, False), (0.707, True)])
def test_fused_decode_step(out_scale, with_lse):
    """sinkattn_decode_step (RoPE, ring write and attention in one kernel) gives, bit for bit,
    the output, log-sum-exp and ring contents of sinkattn_decode_prologue followed by
    sinkattn_decode_ex, leaves its inputs unchanged, and matches the oracle's chain.  Lengths
    cover a first token, a ring not yet full, exactly full, wrapped, and an empty sequence."""
    B, Hq, Hkv, W = 10, 64, 8, 128
    theta = sa.SWA_ROPE_THETA
    lens = np.array([1, 2, 64, 127, 128, 129, 200, 4096, 0, 65536], np.int32)
    ml = int(lens.max())
    q = inputs.normal((B, Hq, 1, 192), 90, 0)
    kn = inputs.normal((B, Hkv, 1, 192), 90, 1)
    vn = inputs.normal((B, Hkv, 1, 128), 90, 2)
    kc = inputs.normal((B, Hkv, W, 192), 91, 1)
    vc = inputs.normal((B, Hkv, W, 128), 91, 2)
    sink = inputs.sink_values(Hq, 92)
    lensd, sinkd = dev_i32(lens), dev_f32(sink)
    # separate kernels
    qa, ka, va, kca, vca = dev_bf16(q), dev_bf16(kn), dev_bf16(vn), dev_bf16(kc), dev_bf16(vc)
    qr = torch.empty_like(qa)
    sa.sinkattn_decode_prologue(theta, sa.KV_RING, qa, qr, ka, va, kca, vca, lensd, window=W)
    out_a = torch.empty((B, Hq, 1, 128), dtype=torch.bfloat16, device="cuda")
    lse_a = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda") if with_lse else None
    sa.sinkattn_decode_ex(oracle.SWA, W, 1, qr, sa.KV_RING, kca, vca, lensd, ml, sinkd, out_a, None,
                          out_scale=out_scale, lse=lse_a)
    # one kernel
    qb, kb, vb, kcb, vcb = dev_bf16(q), dev_bf16(kn), dev_bf16(vn), dev_bf16(kc), dev_bf16(vc)
    out_b = torch.empty((B, Hq, 1, 128), dtype=torch.bfloat16, device="cuda")
    lse_b = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda") if with_lse else None
    sa.sinkattn_decode_step(theta, W, qb, kb, vb, kcb, vcb, lensd, ml, sinkd, out_b, out_scale=out_scale, lse=lse_b)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out_b), host_bits(out_a)), "output differs from prologue + decode"
    if with_lse:
        assert np.array_equal(lse_b.cpu().numpy().view(np.uint32), lse_a.cpu().numpy().view(np.uint32))
    assert np.array_equal(host_bits(kcb), host_bits(kca)) and np.array_equal(host_bits(vcb), host_bits(vca)), \
        "ring contents differ from the prologue's"
    for t, ref, name in ((qb, q, "q_in"), (kb, kn, "k_new"), (vb, vn, "v_new")):
        assert np.array_equal(host_bits(t), ref), f"{name} was modified"
    # the oracle's chain: rotated rows rounded to bf16 as the GPU stores them
    pos = (lens - 1)[:, None, None]
    qo = inputs.bf16_bits(oracle.rope(q, np.broadcast_to(pos, q.shape[:3]), theta).astype(np.float32))
    kno = inputs.bf16_bits(oracle.rope(kn, np.broadcast_to(pos, kn.shape[:3]), theta).astype(np.float32))
    kco, vco = kc.copy(), vc.copy()
    oracle.kv_append(kco, vco, oracle.RING, kno, vn, lens, window=W)
    ref, ref_lse = oracle.decode(qo, kco, vco, lens, sink, oracle.SWA, W, SCALE, oracle.RING, return_lse=True)
    assert_parity(host_f32(out_b), out_scale * ref, "fused decode step vs oracle chain")
    if with_lse:
        check_lse(lse_b.cpu().numpy(), ref_lse, "fused decode step")
