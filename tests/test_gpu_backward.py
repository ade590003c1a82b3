"""Backward of prefill attention (gradients of q, k, v and of the sink) against the oracle.

Tolerance: the products run in bf16 with float32 accumulation, and the weights P and the
score gradients dS enter them rounded to bf16 (relative error 2^-9 each).  Gradients sum
many such terms (dk and dv over every query row and head of the group), so their size grows
with the sequence; the bar is relative: rel-L2 <= 5e-3 and every element within
2e-2 * max(1, max |reference|).  The sink gradient, a float32 sum over all rows of a head,
is bounded by the scale of its summands (see run())."""
import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import dev_bf16, dev_f32, errors

pytestmark = pytest.mark.gpu

SCALE = 192 ** -0.5


def assert_grad(got, ref, what):
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    max_abs, rel = errors(got, ref)
    bound = 2e-2 * max(1.0, float(np.max(np.abs(ref))))
    print(f"[grad] {what}: max_abs={max_abs:.3e} (bound {bound:.3e}) rel_l2={rel:.3e}", flush=True)
    assert max_abs <= bound and rel <= 5e-3, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"


def run(mode, W, Hq, Hkv, L, B=1, sink_kind="sink", seed=0, scale=SCALE):
    w = inputs.Workload("t", "prefill", 0, B, Hq, Hkv, seqlen=L, seed=seed)
    d = inputs.prefill_inputs(w)
    dout = inputs.normal((B, Hq, L, 128), seed, 5)
    sink = None
    if sink_kind != "none":
        sink = d["sink"].copy()
        if sink_kind == "extremes":
            sink[0] = np.inf
            sink[1] = -np.inf
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    s = dev_f32(sink)
    out = torch.empty((B, Hq, L, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    ws = torch.empty(sa.sinkattn_prefill_chunk_workspace_bytes(B, L, Hq, Hkv, L), dtype=torch.uint8, device="cuda")
    sa.sinkattn_prefill_ex(mode, W, q, k, v, s, out, ws, lse=lse, scale=scale)
    dq, dk, dv, ds = sa.prefill_backward(mode, W, q, k, v, s, out, dev_bf16(dout), lse, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.prefill_backward(d["q"], d["k"], d["v"], sink, dout, mode, W, scale)
    got = (dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy(), None if ds is None else ds.cpu().numpy())
    bound = None
    if sink is not None:
        # The sink gradient sums -exp(sink - LSE_i) (dO_i . O_i) over rows, with O the stored
        # bf16 output (each element within 2^-9 relative of the exact one, before and after the
        # bf16 weights of the forward's value product): its error is bounded by a small multiple
        # of sum_i exp(sink - LSE_i) |dO_i| |O_i|, a scale of the summands rather than of their
        # (cancelling) sum.  The bar is 2^-6 of that.
        o_ref, lse_ref = oracle.prefill_chunk(d["q"], d["k"], d["v"], sink, mode, W, scale, return_lse=True)
        dof = inputs.bf16_to_f32(dout).astype(np.float64)
        with np.errstate(invalid="ignore"):
            ps = np.where(np.isinf(sink)[None, :, None], 0.0, np.exp(sink[None, :, None] - lse_ref))
        mag = ps * np.linalg.norm(dof, axis=-1) * np.linalg.norm(o_ref, axis=-1)
        bound = 2.0 ** -6 * mag.sum(axis=(0, 2))
    return got, ref, sink, bound


def assert_dsink(g, r, bound):
    err = np.abs(np.asarray(g, np.float64) - r)
    print(f"[grad] dsink: max_abs={err.max():.3e} max(err / bound)={np.max(err / np.maximum(bound, 1e-30)):.3f}",
          flush=True)
    assert np.all(err <= np.maximum(bound, 1e-6)), (err, bound)


@pytest.mark.parametrize("mode,W,Hq,Hkv,L,B,sink_kind", [
    (oracle.GLOBAL, 0, 64, 4, 300, 1, "sink"),
    (oracle.GLOBAL, 0, 16, 4, 129, 2, "extremes"),   # group of 4; sinks of +inf and -inf
    (oracle.GLOBAL, 0, 16, 4, 200, 1, "none"),
    (oracle.SWA, 128, 64, 8, 500, 1, "sink"),
    (oracle.SWA, 100, 16, 2, 257, 1, "sink"),        # window not a multiple of 32; group of 8
    (oracle.SWA, 1, 8, 2, 70, 1, "sink"),            # each row sees only itself
])
def test_backward(mode, W, Hq, Hkv, L, B, sink_kind):
    print(f"[case] backward mode={mode} W={W} Hq={Hq} Hkv={Hkv} L={L} B={B} sink={sink_kind}", flush=True)
    got, ref, sink, bound = run(mode, W, Hq, Hkv, L, B, sink_kind, seed=L + Hq)
    for name, i in (("dq", 0), ("dk", 1), ("dv", 2)):
        assert_grad(got[i], ref[i], name)
    if sink is None:
        assert got[3] is None
    else:
        assert_dsink(got[3], ref[3], bound)


@pytest.mark.parametrize("mode,W,scale", [(oracle.GLOBAL, 0, 0.125), (oracle.SWA, 128, 0.3)])
def test_backward_nondefault_scale(mode, W, scale):
    """A logit scale other than 1/sqrt(192): it enters P's exponent (with the forward's LSE),
    dq and dk (a factor of the scale each), and the pre-pass's -LSE log2(e) is taken from the
    forward at the same scale."""
    print(f"[case] backward mode={mode} W={W} scale={scale}", flush=True)
    got, ref, sink, bound = run(mode, W, 16, 2, 333, 1, "sink", seed=11 + W, scale=scale)
    for name, i in (("dq", 0), ("dk", 1), ("dv", 2)):
        assert_grad(got[i], ref[i], f"scale {scale} {name}")
    assert_dsink(got[3], ref[3], bound)


def test_backward_ga_2k_all_heads():
    """64 query / 4 KV heads over 2048 positions (64 tiles of queries and 16 key blocks)."""
    got, ref, sink, bound = run(oracle.GLOBAL, 0, 64, 4, 2048, 1, "sink", seed=3)
    for name, i in (("dq", 0), ("dk", 1), ("dv", 2)):
        assert_grad(got[i], ref[i], f"2K {name}")
    assert_dsink(got[3], ref[3], bound)


@pytest.mark.parametrize("name", ["ga_prefill_L32768", "swa_prefill_L32768"])
def test_backward_full_size_sampled(name):
    """The benchmark's 32K workloads (64 query heads, dO seeded N(0,1) as the backward
    benchmark draws it), in the launch configuration it times. Sampled entries are checked
    against the oracle, which computes them one by one:
    * dq rows at the first, middle and last positions and at tile edges, over several heads;
    * dk and dv of keys with many rows (sliding window) or with the few rows near the end that
      see them (global: a key at position j is seen by every row after it).
    The sink gradient sums over every row; it is checked at 2K positions above."""
    w = inputs.WORKLOADS[name]
    L = w.seqlen
    print(f"[case] backward full size {name}", flush=True)
    d = inputs.prefill_inputs(w)
    dout = inputs.normal((w.batch, w.hq, L, w.d_v), w.seed, 5)
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    s = dev_f32(d["sink"])
    out = torch.empty((w.batch, w.hq, L, w.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.hq, L), dtype=torch.float32, device="cuda")
    ws = torch.empty(sa.sinkattn_prefill_chunk_workspace_bytes(w.batch, L, w.hq, w.hkv, L), dtype=torch.uint8,
                     device="cuda")
    sa.sinkattn_prefill_ex(w.mode, w.window, q, k, v, s, out, ws, lse=lse)
    dq, dk, dv, _ = sa.prefill_backward(w.mode, w.window, q, k, v, s, out, dev_bf16(dout), lse)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    G = w.hq // w.hkv
    qpos = [0, 31, 32, 63, 64, 127, 128, 4095, 16383, 16384, L - 33, L - 32, L - 1]
    qrows = [(0, int(h), i) for i in qpos for h in rng.choice(w.hq, 2, replace=False)]
    if w.mode == oracle.SWA:
        kpos = [0, 1, 127, 128, 4000, 16384, 30001, L - 129, L - 1]
    else:
        kpos = [L - 1, L - 2, L - 31, L - 32, L - 33, L - 64]
    krows = [(0, int(rng.integers(w.hkv)), j) for j in kpos]
    rq, rk, rv = oracle.prefill_backward_sampled(d["q"], d["k"], d["v"], d["sink"], dout, w.mode, w.window,
                                                  w.scale, qrows, krows)
    idx = torch.tensor(qrows, dtype=torch.long)
    got_q = dq[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy()
    kidx = torch.tensor(krows, dtype=torch.long)
    got_k = dk[kidx[:, 0], kidx[:, 1], kidx[:, 2]].cpu().numpy()
    got_v = dv[kidx[:, 0], kidx[:, 1], kidx[:, 2]].cpu().numpy()
    assert_grad(got_q, rq, f"{name} dq rows")
    assert_grad(got_k, rk, f"{name} dk keys")
    assert_grad(got_v, rv, f"{name} dv keys")


def test_backward_ga_full_size_one_head():
    """The 32K global workload with dO zero except on one query head h: then dk and dv of KV
    head h // 16 are that head's contributions alone, and the oracle can sum them for keys at
    the start and in the middle of the sequence (every later row sees them).  dL/dsink of that
    head is checked against the oracle's full rows: -sum_i exp(sink - LSE_i) dO_i . O_i over
    all 32768 positions (the other heads' dsink is exactly 0: their D_i is 0)."""
    w = inputs.WORKLOADS["ga_prefill_L32768"]
    L, G, h = w.seqlen, w.hq // w.hkv, 37
    g = h // G
    print(f"[case] backward full size, one head h={h}", flush=True)
    d = inputs.prefill_inputs(w)
    dout = np.zeros((w.batch, w.hq, L, w.d_v), np.uint16)
    dout[:, h] = inputs.normal((w.batch, 1, L, w.d_v), w.seed, 6)[:, 0]
    q, k, v = dev_bf16(d["q"]), dev_bf16(d["k"]), dev_bf16(d["v"])
    s = dev_f32(d["sink"])
    out = torch.empty((w.batch, w.hq, L, w.d_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.hq, L), dtype=torch.float32, device="cuda")
    ws = torch.empty(sa.sinkattn_prefill_chunk_workspace_bytes(w.batch, L, w.hq, w.hkv, L), dtype=torch.uint8,
                     device="cuda")
    sa.sinkattn_prefill_ex(w.mode, w.window, q, k, v, s, out, ws, lse=lse)
    dq, dk, dv, dsink = sa.prefill_backward(w.mode, w.window, q, k, v, s, out, dev_bf16(dout), lse)
    torch.cuda.synchronize()
    # the problem of head h alone: one query head over its KV head
    qh = np.ascontiguousarray(d["q"][:, h:h + 1])
    kh = np.ascontiguousarray(d["k"][:, g:g + 1])
    vh = np.ascontiguousarray(d["v"][:, g:g + 1])
    doh = np.ascontiguousarray(dout[:, h:h + 1])
    kpos = [0, 16391]
    _, rk, rv = oracle.prefill_backward_sampled(qh, kh, vh, d["sink"][h:h + 1], doh, w.mode, w.window, w.scale,
                                                np.zeros((0, 3), np.int64), [(0, 0, j) for j in kpos])
    assert_grad(dk[0, g, kpos].cpu().numpy(), rk, "32K dk, keys 0 and 16391, one head")
    assert_grad(dv[0, g, kpos].cpu().numpy(), rv, "32K dv, keys 0 and 16391, one head")
    rows = np.array([(0, 0, i) for i in range(L)], np.int64)
    o_ref, lse_ref = oracle.prefill_chunk(qh, kh, vh, d["sink"][h:h + 1], w.mode, w.window, w.scale, rows=rows,
                                          return_lse=True)
    do_f = inputs.bf16_to_f32(doh[0, 0]).astype(np.float64)
    D = np.sum(do_f * o_ref, axis=1)
    p_sink = np.exp(d["sink"][h] - lse_ref)
    want = -np.sum(p_sink * D)
    bound = 2 ** -6 * np.sum(p_sink * np.linalg.norm(do_f, axis=1) * np.linalg.norm(o_ref, axis=1))
    got = dsink.cpu().numpy()
    print(f"[parity] 32K dsink head {h}: got={got[h]:.6e} want={want:.6e} bound={bound:.3e}", flush=True)
    assert abs(got[h] - want) <= bound
    assert np.all(got[np.arange(w.hq) != h] == 0)
