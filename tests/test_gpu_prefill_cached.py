"""Chunked prefill over a prefix held in a KV cache (sinkattn_prefill_cached): the model
card's serving set-up prefills long prompts in chunks of 16384 tokens over a paged cache.  The
chunk's rows against the oracle's cached-prefix chunk (oracle_decode_side) and the prefill
definition's rows at the chunk's positions; the prefix comes from permuted pages (both modes)
or from a sliding-window ring of its last W positions."""
import numpy as np
import pytest
import torch

import attention_sink_softmax_amd as sa
from attention_sink_softmax_amd import inputs
import oracle
from gpu_util import assert_parity, dev_bf16, dev_f32, dev_i32, host_f32

pytestmark = pytest.mark.gpu

SCALE = 192 ** -0.5


def seq_data(B, Hq, Hkv, L, seed):
    return inputs.prefill_inputs(inputs.Workload("t", "prefill", 0, B, Hq, Hkv, seqlen=L, seed=seed))


def prefix_cache(d, q0, layout, W=None, ps=None, seed=0):
    """The prefix (positions 0 .. q0-1) in a ring of its last W positions or in permuted pages;
    every other slot holds N(0,1) data that must not be read."""
    B, Hkv = d["k"].shape[:2]
    if layout == sa.KV_RING:
        kr = inputs.normal((B, Hkv, W, 192), seed, 7)
        vr = inputs.normal((B, Hkv, W, 128), seed, 8)
        for j in range(max(0, q0 - W), q0):
            kr[:, :, j % W] = d["k"][:, :, j]
            vr[:, :, j % W] = d["v"][:, :, j]
        return kr, vr, None
    mp = max(1, (q0 + ps - 1) // ps)
    npg = B * mp + 5
    bt = np.random.default_rng(seed).permutation(npg)[:B * mp].reshape(B, mp).astype(np.int32)
    kp = inputs.normal((npg, Hkv, ps, 192), seed, 9)
    vp = inputs.normal((npg, Hkv, ps, 128), seed, 10)
    for b in range(B):
        for j in range(q0):
            kp[bt[b, j // ps], :, j % ps] = d["k"][b, :, j]
            vp[bt[b, j // ps], :, j % ps] = d["v"][b, :, j]
    return kp, vp, bt


def run_cached(mode, W, d, kv_len, Lq, layout, kc, vc, bt):
    q0 = kv_len - Lq
    qs = [np.ascontiguousarray(d[n][:, :, q0:kv_len]) for n in ("q", "k", "v")]
    out = sa.prefill_cached(mode, W, kv_len, *(dev_bf16(x) for x in qs), layout, dev_bf16(kc), dev_bf16(vc),
                            dev_f32(d["sink"]), None if bt is None else dev_i32(bt))
    torch.cuda.synchronize()
    return host_f32(out), qs


@pytest.mark.parametrize("mode,W,Hq,Hkv,layout,ps,kv_len,Lq", [
    (oracle.GLOBAL, 0, 64, 4, sa.KV_PAGED, 64, 1000, 333),
    (oracle.GLOBAL, 0, 64, 4, sa.KV_PAGED, 16, 1000, 1),     # one new token
    (oracle.GLOBAL, 0, 16, 2, sa.KV_PAGED, 64, 577, 577),    # no prefix
    (oracle.GLOBAL, 0, 8, 4, sa.KV_PAGED, 48, 900, 200),     # group of 2 (general kernel)
    (oracle.SWA, 128, 64, 8, sa.KV_RING, None, 1000, 37),    # ring prefix, chunk start off the 32-grid
    (oracle.SWA, 128, 64, 8, sa.KV_RING, None, 1000, 129),
    (oracle.SWA, 128, 16, 2, sa.KV_RING, None, 140, 100),    # prefix shorter than the window
    (oracle.SWA, 100, 16, 2, sa.KV_RING, None, 800, 300),    # window not a multiple of 32
    (oracle.SWA, 1, 8, 2, sa.KV_RING, None, 300, 64),
    (oracle.SWA, 128, 64, 8, sa.KV_PAGED, 64, 1000, 333),
    (oracle.SWA, 300, 16, 2, sa.KV_PAGED, 32, 1200, 250),    # window above 128 (general kernel)
])
def test_cached_matches_oracle(mode, W, Hq, Hkv, layout, ps, kv_len, Lq):
    print(f"[case] cached mode={mode} W={W} Hq={Hq} Hkv={Hkv} layout={layout} ps={ps} kv_len={kv_len} Lq={Lq}",
          flush=True)
    d = seq_data(2, Hq, Hkv, kv_len, seed=kv_len + Lq + Hq)
    q0 = kv_len - Lq
    kc, vc, bt = prefix_cache(d, q0, layout, W=W, ps=ps, seed=Lq)
    got, (qc, kch, vch) = run_cached(mode, W, d, kv_len, Lq, layout, kc, vc, bt)
    lens = np.full(2, kv_len, np.int32)
    ref = oracle.prefill_cached(qc, kch, vch, kc, vc, lens, d["sink"], mode, W, SCALE,
                                oracle.RING if layout == sa.KV_RING else oracle.PAGED, bt)
    assert_parity(got, ref, "cached prefix vs oracle")
    pre = oracle.prefill_chunk(qc, d["k"], d["v"], d["sink"], mode, W, SCALE)
    assert_parity(got, pre, "cached prefix vs prefill rows")


def test_bad_prefix_page_gives_nan_rows():
    """A prefix page id outside the pool is never read: the rows that see that page are NaN
    (its values stand in as NaN); rows that share a 32-key block with it may be NaN too; rows
    well past it are finite (sliding window 64: the chunk's later rows no longer see the page)."""
    Hq, Hkv, kv_len, Lq, ps, W = 16, 2, 600, 300, 64, 64
    d = seq_data(1, Hq, Hkv, kv_len, seed=5)
    kp, vp, bt = prefix_cache(d, kv_len - Lq, sa.KV_PAGED, ps=ps, seed=5)
    bt[0, 4] = 10 ** 6  # page 4: positions 256..319, of which 256..299 belong to the prefix
    got, _ = run_cached(oracle.SWA, W, d, kv_len, Lq, sa.KV_PAGED, kp, vp, bt)
    first_key = np.arange(Lq) + (kv_len - Lq) - W + 1  # oldest key each row sees
    assert np.all(np.isnan(got[0][:, first_key <= 299]))
    assert np.all(np.isfinite(got[0][:, first_key > 299 + 32]))


@pytest.mark.parametrize("mode,layout", [(oracle.GLOBAL, sa.KV_PAGED), (oracle.SWA, sa.KV_RING)])
def test_chunk_16k_after_16k_sampled(mode, layout):
    """The 32K workloads' last 16384 positions as one chunk after a 16384-token prefix held in
    64-token permuted pages (global) or in a 128-slot ring (sliding window): sampled rows of
    every head (the first 128, the last 128 and 256 seeded positions of the chunk)."""
    w = inputs.GA_PREFILL if mode == oracle.GLOBAL else inputs.SWA_PREFILL
    print(f"[case] {w.name} as a 16K chunk after a 16K cached prefix", flush=True)
    dd = inputs.prefill_cached_inputs(w, 16384)
    Lq = 16384
    out = sa.prefill_cached(w.mode, w.window, w.seqlen, dev_bf16(dd["q"]), dev_bf16(dd["k"]), dev_bf16(dd["v"]),
                            layout, dev_bf16(dd["k_ring" if layout == sa.KV_RING else "k_pages"]),
                            dev_bf16(dd["v_ring" if layout == sa.KV_RING else "v_pages"]), dev_f32(dd["sink"]),
                            None if layout == sa.KV_RING else dev_i32(dd["block_table"]))
    torch.cuda.synchronize()
    wc = inputs.Workload("chunk", "prefill", w.mode, 1, w.hq, w.hkv, seqlen=Lq, window=w.window, seed=w.seed)
    rows = inputs.ga_parity_rows(wc)
    idx = torch.from_numpy(rows).to("cuda")
    got = host_f32(out[idx[:, 0], idx[:, 1], idx[:, 2]])
    full = inputs.prefill_inputs(w)
    ref = oracle.prefill_chunk(dd["q"], full["k"], full["v"], full["sink"], w.mode, w.window, w.scale, rows=rows)
    assert_parity(got, ref, f"{w.name} 16K chunk sampled {len(rows)} rows")
    assert torch.isfinite(out.float()).all().item()
