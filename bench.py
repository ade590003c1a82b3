"""Benchmark of the sink-attention hot path on one MI355X.

One step runs every kernel of the path once, each on its benchmark workload:
  swa_prefill_L32768   sliding-window prefill, L=32768, 64 query / 8 KV heads, W=128
  ga_prefill_L32768    global causal prefill with sink, L=32768, 64 query / 4 KV heads
  swa_decode_B128_ring sliding-window decode, 128 sequences, 128-slot ring caches
  ga_decode_B8_256K    global decode, 8 sequences x 262144 tokens, 64-token permuted pages
  ga_verify_B8_256K_q4 the same caches with 4 new (drafted) tokens per sequence at once
  ga_decode_..._fp8    the 256K global decode from an 8-bit E4M3 cache (half the bytes)
All inputs are synthetic (seeded N(0,1) bf16, sink ~ U[0,6]) and resident in HBM before
timing starts.  Each call is timed with HIP events recorded on the stream the library
launches on.

`value` is the prefill throughput over both 32K prefill workloads (algorithmic flops of
the two / their summed kernel time); the 256K decode KV-read bandwidth is reported next
to it.  Algorithmic work counts 2*(192+128) flops per (query head, visible key) pair and,
for decode, the K/V bytes of the visible keys.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
METRIC = "prefill attn TFLOP/s (SWA & GA+sink, 32K) + decode KV-read HBM GB/s at 256K"
FLOP_PER_PAIR = 2 * (192 + 128)
CSRC = os.path.join(ROOT, "attention_sink_softmax_amd", "csrc")

# HBM bytes per call read by rocprofv3 FETCH_SIZE and WRITE_SIZE (one pass each), scaled by
# the same counters on a plain 1 GiB device copy (read x 2.0, written x 1.0).  Each entry
# holds the hash of the kernel sources it was measured on; once they change the figure is
# stale and `traffic` is reported as null until the counters are taken again.
TRAFFIC = {
    "ga_prefill_L32768": {"sources": ("prefill.hip", "common.h", "launch.h"),
                          "sha256": "0ad3f48061805f92d070cf996575869849d707cfe07f4d1357aba8ff4ed436e4",
                          "read_GB": 3.5704, "written_GB": 0.5369},
    "swa_prefill_L32768": {"sources": ("prefill.hip", "common.h", "launch.h"),
                           "sha256": "0ad3f48061805f92d070cf996575869849d707cfe07f4d1357aba8ff4ed436e4",
                           "read_GB": 1.0234, "written_GB": 0.5369},
    "ga_decode_B8_256K_paged": {"sources": ("decode.hip", "rope.h", "common.h", "launch.h"),
                                "sha256": "e4ac83f4b6eba6bc677512e1c1646afe51736e2fe76416f4f562c21182fc9ec0",
                                "read_GB": 5.3749, "written_GB": 0.0046},
    "ga_decode_B8_256K_paged_fp8": {"sources": ("decode.hip", "rope.h", "common.h", "launch.h"),
                                    "sha256": "e4ac83f4b6eba6bc677512e1c1646afe51736e2fe76416f4f562c21182fc9ec0",
                                    "read_GB": 2.6906, "written_GB": 0.0046},
}


def sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_gb(workload):
    t = TRAFFIC.get(workload)
    if not t or not t["sha256"] or sources_sha256(t["sources"]) != t["sha256"]:
        return None
    return round(t["read_GB"] + t["written_GB"], 4)


def pairs_prefill(L, mode, W):
    if mode == 1:
        n = min(L, W)
        return n * (n + 1) // 2 + (L - n) * W
    return L * (L + 1) // 2


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help="comma list of workloads to run (profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    import attention_sink_softmax_amd as sa
    from attention_sink_softmax_amd import inputs

    sa.lib()  # fails loudly when the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        return copy_calibration(torch, dev)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    only = set(filter(None, args.only.split(",")))
    runs = {}  # name -> (callable, flops, bytes)

    # --- prefill workloads
    for w in (inputs.SWA_PREFILL, inputs.GA_PREFILL):
        if only and w.name not in only:
            continue
        d = inputs.prefill_inputs(w)
        q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
        sink = torch.from_numpy(d["sink"]).to(dev)
        out = torch.empty((w.batch, w.hq, w.seqlen, w.d_v), dtype=torch.bfloat16, device=dev)
        ws = sa.prefill_workspace(q, k)
        del d
        flops = pairs_prefill(w.seqlen, w.mode, w.window) * w.hq * w.batch * FLOP_PER_PAIR
        nbytes = (q.numel() + k.numel() + v.numel() + out.numel()) * 2

        def call(w=w, q=q, k=k, v=v, sink=sink, out=out, ws=ws):
            sa.sinkattn_prefill(w.mode, w.window, q, k, v, sink, out, ws)

        runs[w.name] = (call, flops, nbytes)

    # --- sliding-window decode: 4 input sets rotate (one set fits the 256 MB Infinity Cache)
    w = inputs.SWA_DECODE
    if not only or w.name in only:
        sets = []
        for r in range(4):
            d = inputs.decode_ring_inputs(w, seed=w.seed * 100 + r)
            lens = d["seq_lens"]
            sets.append(dict(q=up(d["q"]), k=up(d["k"]), v=up(d["v"]), lens=torch.from_numpy(lens).to(dev),
                             maxlen=int(lens.max()), sink=torch.from_numpy(d["sink"]).to(dev)))
        out = torch.empty((w.batch, w.hq, w.d_v), dtype=torch.bfloat16, device=dev)
        ws = sa.decode_workspace(w.mode, w.window, w.batch, w.hq, w.hkv, 65536, dev)
        visible = w.batch * w.window  # every context is longer than the window
        flops = visible * w.hq * FLOP_PER_PAIR
        nbytes = visible * w.hkv * (w.d_qk + w.d_v) * 2
        state = {"i": 0}

        def call(w=w, sets=sets, out=out, ws=ws, state=state):
            s = sets[state["i"] % len(sets)]
            state["i"] += 1
            sa.sinkattn_decode(w.mode, w.window, s["q"], sa.KV_RING, s["k"], s["v"], s["lens"], s["maxlen"],
                               s["sink"], out, ws)

        runs[w.name] = (call, flops, nbytes)

    # --- global decode at 256K, permuted 64-token pages
    w = inputs.GA_DECODE
    if not only or w.name in only:
        d = inputs.decode_paged_inputs(w)
        q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
        bt = torch.from_numpy(d["block_table"]).to(dev)
        lens = torch.from_numpy(d["seq_lens"]).to(dev)
        sink = torch.from_numpy(d["sink"]).to(dev)
        del d
        out = torch.empty((w.batch, w.hq, w.d_v), dtype=torch.bfloat16, device=dev)
        ws = sa.decode_workspace(w.mode, w.window, w.batch, w.hq, w.hkv, w.ctx_hi, dev)
        visible = w.batch * w.ctx_hi
        flops = visible * w.hq * FLOP_PER_PAIR
        nbytes = visible * w.hkv * (w.d_qk + w.d_v) * 2

        def call(w=w, q=q, k=k, v=v, bt=bt, lens=lens, sink=sink, out=out, ws=ws):
            sa.sinkattn_decode(w.mode, w.window, q, sa.KV_PAGED, k, v, lens, w.ctx_hi, sink, out, ws, bt)

        runs[w.name] = (call, flops, nbytes)

    # --- verification of 4 drafted tokens per sequence at 256K (same cache shape as above)
    w = inputs.GA_VERIFY
    if not only or w.name in only:
        d = inputs.decode_paged_inputs(w)
        q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
        bt = torch.from_numpy(d["block_table"]).to(dev)
        lens = torch.from_numpy(d["seq_lens"]).to(dev)
        sink = torch.from_numpy(d["sink"]).to(dev)
        del d
        out = torch.empty((w.batch, w.hq, w.q_len, w.d_v), dtype=torch.bfloat16, device=dev)
        ws = sa.decode_multi_workspace(w.mode, w.window, w.batch, w.hq, w.hkv, w.q_len, w.ctx_hi, dev)
        # token t of q_len sees ctx - q_len + t + 1 keys; the cache is read once for all of them
        flops = sum(w.ctx_hi - w.q_len + t + 1 for t in range(w.q_len)) * w.batch * w.hq * FLOP_PER_PAIR
        nbytes = w.batch * w.ctx_hi * w.hkv * (w.d_qk + w.d_v) * 2

        def call(w=w, q=q, k=k, v=v, bt=bt, lens=lens, sink=sink, out=out, ws=ws):
            sa.sinkattn_decode_multi(w.mode, w.window, w.q_len, q, sa.KV_PAGED, k, v, lens, w.ctx_hi, sink, out, ws,
                                     bt)

        runs[w.name] = (call, flops, nbytes)

    # --- whole decode steps: RoPE of q and the new key, the cache write and the attention; one
    # kernel on the sliding-window rings (4 input sets rotate), the prologue kernel then the
    # attention on the 256K pages
    for w, name in ((inputs.SWA_DECODE, "swa_decode_step_B128_ring"), (inputs.GA_DECODE, "ga_decode_step_B8_256K_paged")):
        if only and name not in only:
            continue
        nsets = 4 if w.layout == "ring" else 1
        sets = []
        for r in range(nsets):
            if w.layout == "ring":
                d = inputs.decode_ring_inputs(w, seed=w.seed * 100 + r)
            else:
                d = inputs.decode_paged_inputs(w)
            ss = w.seed * 1000 + r
            sets.append(dict(q=up(d["q"]).unsqueeze(2), k=up(d["k"]), v=up(d["v"]),
                             kn=up(inputs.normal((w.batch, w.hkv, 1, w.d_qk), ss, 3)),
                             vn=up(inputs.normal((w.batch, w.hkv, 1, w.d_v), ss, 4)),
                             bt=torch.from_numpy(d["block_table"]).to(dev) if w.layout == "paged" else None,
                             lens=torch.from_numpy(d["seq_lens"]).to(dev), sink=torch.from_numpy(d["sink"]).to(dev)))
            del d
        qr = torch.empty_like(sets[0]["q"])
        out = torch.empty((w.batch, w.hq, w.d_v), dtype=torch.bfloat16, device=dev)
        ws = sa.decode_workspace(w.mode, w.window, w.batch, w.hq, w.hkv, w.ctx_hi, dev)
        layout = sa.KV_RING if w.layout == "ring" else sa.KV_PAGED
        theta = sa.SWA_ROPE_THETA if w.mode == 1 else sa.GA_ROPE_THETA
        visible = w.batch * (w.window if w.mode == 1 else w.ctx_hi)
        flops = visible * w.hq * FLOP_PER_PAIR
        # the attention's K/V bytes plus the step's own: q and the new key and value read, the
        # new row written
        nbytes = visible * w.hkv * (w.d_qk + w.d_v) * 2 + w.batch * (w.hq * w.d_qk + 2 * w.hkv * (w.d_qk + w.d_v)) * 2
        state = {"i": 0}

        def call(w=w, sets=sets, qr=qr, out=out, ws=ws, layout=layout, theta=theta, state=state):
            s = sets[state["i"] % len(sets)]
            state["i"] += 1
            if layout == sa.KV_RING:
                sa.sinkattn_decode_step(theta, w.window, s["q"], s["kn"], s["vn"], s["k"], s["v"], s["lens"], w.ctx_hi,
                                        s["sink"], out.view(w.batch, w.hq, 1, w.d_v))
                return
            sa.sinkattn_decode_prologue(theta, layout, s["q"], qr, s["kn"], s["vn"], s["k"], s["v"], s["lens"],
                                        window=w.window, block_table=s["bt"])
            sa.sinkattn_decode(w.mode, w.window, qr[:, :, 0], layout, s["k"], s["v"], s["lens"], w.ctx_hi, s["sink"],
                               out, ws, s["bt"])

        runs[name] = (call, flops, nbytes)

    # --- sliding-window verify: the B = 128 rings with 4 drafted tokens per sequence whose keys
    # and values are held beside the rings (the rings are only read); 4 input sets rotate
    w = inputs.SWA_VERIFY
    if not only or w.name in only:
        sets = []
        for r in range(4):
            d = inputs.decode_ring_verify_inputs(w, seed=w.seed * 100 + r)
            sets.append(dict(q=up(d["q"]), k=up(d["k"]), v=up(d["v"]), kn=up(d["k_new"]), vn=up(d["v_new"]),
                             lens=torch.from_numpy(d["seq_lens"]).to(dev), sink=torch.from_numpy(d["sink"]).to(dev)))
        out = torch.empty((w.batch, w.hq, w.q_len, w.d_v), dtype=torch.bfloat16, device=dev)
        ws = sa.decode_multi_workspace(w.mode, w.window, w.batch, w.hq, w.hkv, w.q_len, w.ctx_hi, dev)
        # draft t sees the W - t - 1 newest ring keys and drafts 0..t (W keys); the ring and the
        # drafts are read once for all four
        flops = w.batch * w.q_len * w.window * w.hq * FLOP_PER_PAIR
        nbytes = w.batch * (w.window - 1 + w.q_len) * w.hkv * (w.d_qk + w.d_v) * 2
        state = {"i": 0}

        def call(w=w, sets=sets, out=out, ws=ws, state=state):
            s = sets[state["i"] % len(sets)]
            state["i"] += 1
            sa.sinkattn_decode_verify(w.mode, w.window, w.q_len, s["q"], sa.KV_RING, s["k"], s["v"], s["kn"], s["vn"],
                                      s["lens"], w.ctx_hi, s["sink"], out, ws)

        runs[w.name] = (call, flops, nbytes)

    # --- chunked prefill over a cached prefix: the 32K prefill workloads' last 16384 positions
    # after a 16384-token prefix in 64-token permuted pages (global) or a 128-slot ring (sliding)
    for w, layout, name in ((inputs.GA_PREFILL, sa.KV_PAGED, "ga_prefill_chunk16K_after16K_paged"),
                            (inputs.SWA_PREFILL, sa.KV_RING, "swa_prefill_chunk16K_after16K_ring")):
        if only and name not in only:
            continue
        Lq = 16384
        d = inputs.prefill_cached_inputs(w, Lq)
        q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
        kc = up(d["k_pages"] if layout == sa.KV_PAGED else d["k_ring"])
        vc = up(d["v_pages"] if layout == sa.KV_PAGED else d["v_ring"])
        bt = torch.from_numpy(d["block_table"]).to(dev) if layout == sa.KV_PAGED else None
        sink = torch.from_numpy(d["sink"]).to(dev)
        del d
        out = torch.empty((w.batch, w.hq, Lq, w.d_v), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(sa.sinkattn_prefill_cached_workspace_bytes(w.mode, w.window, w.batch, Lq, w.hq, w.hkv,
                                                                    w.seqlen), dtype=torch.uint8, device=dev)
        pairs = pairs_prefill(w.seqlen, w.mode, w.window) - pairs_prefill(w.seqlen - Lq, w.mode, w.window)
        flops = pairs * w.hq * w.batch * FLOP_PER_PAIR
        kv_seen = w.seqlen if w.mode == 0 else Lq + w.window - 1
        nbytes = (q.numel() + out.numel()) * 2 + w.batch * w.hkv * kv_seen * (w.d_qk + w.d_v) * 2

        def call(w=w, q=q, k=k, v=v, layout=layout, kc=kc, vc=vc, bt=bt, sink=sink, out=out, ws=ws):
            sa.sinkattn_prefill_cached(w.mode, w.window, w.seqlen, q, k, v, layout, kc, vc, sink, out, ws, bt)

        runs[name] = (call, flops, nbytes)

    # --- backward of the 32K global prefill (q, k, v, sink gradients), from the forward's
    # output and log-sum-exp; dO seeded N(0,1)
    name = "ga_prefill_backward_L32768"
    if only and name in only:
        w = inputs.GA_PREFILL
        d = inputs.prefill_inputs(w)
        q, k, v = up(d["q"]), up(d["k"]), up(d["v"])
        sink = torch.from_numpy(d["sink"]).to(dev)
        del d
        out = torch.empty((w.batch, w.hq, w.seqlen, w.d_v), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.batch, w.hq, w.seqlen), dtype=torch.float32, device=dev)
        sa.sinkattn_prefill_ex(w.mode, w.window, q, k, v, sink, out, sa.prefill_workspace(q, k), lse=lse)
        dout = up(inputs.normal((w.batch, w.hq, w.seqlen, w.d_v), w.seed, 5))
        grads = [torch.empty(q.shape, dtype=torch.float32, device=dev), torch.empty(k.shape, dtype=torch.float32, device=dev),
                 torch.empty(v.shape, dtype=torch.float32, device=dev), torch.empty(w.hq, dtype=torch.float32, device=dev)]
        dd = sa.Dims(w.batch, w.seqlen, w.hq, w.hkv, 192, 128, w.scale)
        wsb = torch.empty(sa.lib().sinkattn_prefill_backward_workspace_bytes(sa.ctypes.byref(dd)), dtype=torch.uint8,
                          device=dev)
        # algorithmic work: S, dP, dV, dK, dQ once each per visible pair
        flops = pairs_prefill(w.seqlen, w.mode, w.window) * w.hq * w.batch * 2 * (3 * 192 + 2 * 128)
        nbytes = (q.numel() + k.numel() + v.numel() + out.numel() + dout.numel()) * 2 + sum(g.numel() * 4 for g in grads)

        def call(w=w, q=q, k=k, v=v, sink=sink, out=out, dout=dout, lse=lse, g=grads, ws=wsb):
            sa.sinkattn_prefill_backward(w.mode, w.window, q, k, v, sink, out, dout, lse, g[0], g[1], g[2], g[3], ws)

        runs[name] = (call, flops, nbytes)

    # --- global decode at 256K from an 8-bit (E4M3) cache: half the bytes of the bf16 cache
    w = inputs.GA_DECODE_FP8
    if not only or w.name in only:
        d = inputs.decode_paged_inputs(w)
        q = up(d["q"])
        k = torch.from_numpy(d["k"]).to(dev)
        v = torch.from_numpy(d["v"]).to(dev)
        bt = torch.from_numpy(d["block_table"]).to(dev)
        lens = torch.from_numpy(d["seq_lens"]).to(dev)
        sink = torch.from_numpy(d["sink"]).to(dev)
        ks, vs = d["kv_scales"]
        del d
        out = torch.empty((w.batch, w.hq, 1, w.d_v), dtype=torch.bfloat16, device=dev)
        ws = sa.decode_multi_workspace(w.mode, w.window, w.batch, w.hq, w.hkv, 1, w.ctx_hi, dev)
        visible = w.batch * w.ctx_hi
        flops = visible * w.hq * FLOP_PER_PAIR
        nbytes = visible * w.hkv * (w.d_qk + w.d_v)  # one byte per element

        def call(w=w, q=q.unsqueeze(2), k=k, v=v, bt=bt, lens=lens, sink=sink, out=out, ws=ws, ks=ks, vs=vs):
            sa.sinkattn_decode_fp8(w.mode, w.window, 1, q, k, v, lens, w.ctx_hi, sink, ks, vs, out, ws, bt)

        runs[w.name] = (call, flops, nbytes)

    names = list(runs)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        for n in names:
            runs[n][0]()
    torch.cuda.synchronize()

    ev = {n: [] for n in names}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for n in names:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            runs[n][0]()
            e1.record(stream)
            ev[n].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    comp = {}
    for n in names:
        ms = [a.elapsed_time(b) for a, b in ev[n]]
        avg = float(np.mean(ms))
        med = float(np.median(ms))
        _, flops, nbytes = runs[n]
        # rates from the median call (a long kernel's median and mean agree within drift)
        comp[n] = {"ms_median": round(med, 5), "ms_avg": round(avg, 5), "ms_min": round(float(np.min(ms)), 5),
                   "ms_max": round(float(np.max(ms)), 5),
                   "tflops": round(flops / (med * 1e-3) / 1e12, 3),
                   "gbps": round(nbytes / (med * 1e-3) / 1e9, 1),
                   "algorithmic_gflop": round(flops / 1e9, 3), "algorithmic_gb": round(nbytes / 1e9, 4)}

    pre = [n for n in ("swa_prefill_L32768", "ga_prefill_L32768") if n in comp]
    value = None
    if pre:
        fl = sum(runs[n][1] for n in pre)
        t = sum(comp[n]["ms_median"] for n in pre) * 1e-3
        value = round(fl / t / 1e12, 3)
    dec = comp.get("ga_decode_B8_256K_paged")

    roofline = None
    if "ga_prefill_L32768" in comp:
        c = comp["ga_prefill_L32768"]
        roofline = {"kernel": "prefill_causal_kernel (ga_prefill_L32768)", "bound": "mfma", "achieved": c["tflops"],
                    "peak": MFMA_PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(c["tflops"] / MFMA_PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic_gb("ga_prefill_L32768"), "traffic_unit": "GB per call (HBM read + written)"}
    roofline_decode = None
    if dec:
        roofline_decode = {"kernel": "decode_split_kernel+decode_merge_kernel (ga_decode_B8_256K_paged)",
                           "bound": "hbm", "achieved": dec["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": round(dec["gbps"] / HBM_PEAK_GBPS, 4),
                           "traffic": traffic_gb("ga_decode_B8_256K_paged"),
                           "traffic_unit": "GB per call (HBM read + written)"}

    swa = comp.get("swa_prefill_L32768")
    roofline_swa = None
    if swa:
        roofline_swa = {"kernel": "prefill_swa_kernel (swa_prefill_L32768)", "bound": "hbm", "achieved": swa["gbps"],
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(swa["gbps"] / HBM_PEAK_GBPS, 4),
                        "traffic": traffic_gb("swa_prefill_L32768"),
                        "traffic_unit": "GB per call (HBM read + written)"}

    dec8 = comp.get("ga_decode_B8_256K_paged_fp8")
    roofline_decode_fp8 = None
    if dec8:
        roofline_decode_fp8 = {"kernel": "decode_split_kernel<fp8>+decode_merge_kernel (ga_decode_B8_256K_paged_fp8)",
                               "bound": "hbm", "achieved": dec8["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                               "frac": round(dec8["gbps"] / HBM_PEAK_GBPS, 4),
                               "traffic": traffic_gb("ga_decode_B8_256K_paged_fp8"),
                               "traffic_unit": "GB per call (HBM read + written)"}

    cpu = None
    if not args.no_cpu_baseline and pre:
        cpu = cpu_baseline()

    step_ms = sum(comp[n]["ms_avg"] for n in names)
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 4), "wall_s_timed": round(wall, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v, sink ~ U[0,6]); no weights",
        "config": {"workload": "sink attention hot path: " + " + ".join(names),
                   "swa_prefill": "B=1 L=32768 Hq=64 Hkv=8 W=128 d_qk=192 d_v=128",
                   "ga_prefill": "B=1 L=32768 Hq=64 Hkv=4 causal+sink d_qk=192 d_v=128",
                   "swa_decode": "B=128 ctx~U[4096,65536] 128-slot ring Hq=64 Hkv=8",
                   "ga_decode": "B=8 ctx=262144 64-token pages, permuted table, Hq=64 Hkv=4",
                   "ga_verify": "as ga_decode with q_len=4 new tokens per sequence",
                   "swa_verify": "as swa_decode with q_len=4 drafted tokens whose K/V are held beside the rings",
                   "prefill_chunk": "the 32K prefills' last 16384 positions after a 16384-token prefix in 64-token "
                                    "permuted pages (GA) or a 128-slot ring (SWA)",
                   "decode_step": "RoPE of q and the new key, cache write and attention: one kernel on "
                                  "swa_decode's rings, the prologue kernel + attention on ga_decode's pages",
                   "ga_decode_fp8": "as ga_decode with an E4M3 cache, per-tensor scales 2^-6"},
        "decode_kv_read_GBps": dec["gbps"] if dec else None,
        "components": comp, "roofline": roofline, "roofline_decode": roofline_decode,
        "roofline_decode_fp8": roofline_decode_fp8, "roofline_swa_prefill": roofline_swa, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def copy_calibration(torch, dev, nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of `nbytes`: it reads and writes exactly `nbytes` each,
    so hardware byte counters read on it give the scale factor for the counters read on the
    attention kernels."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps, "ms": round(ms, 4),
                      "GBps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)
    return 0


def cpu_baseline():
    """The CPU oracle (fp64 plain loops, OpenMP over output rows) timed on the host cores, on
    each workload's own inputs (seeded as the GPU's):
      tiny_swa_L512, swa_prefill_L32768, swa_decode_B128_ring and ga_decode_B8_256K_paged over
      their whole output;
      ga_prefill_L32768 on the fixed sample its parity test checks (every head at the first
      128, the last 128 and 256 seeded positions, 0.34 TFLOP), with the whole call's time
      extrapolated by the ratio of (query head, key) pairs and labelled as such.
    One run each, about 15 s in all on 16 host cores.  Rates are algorithmic flops (640 per
    pair) over the oracle's wall time."""
    import oracle
    from attention_sink_softmax_amd import inputs

    oracle.load()
    threads = oracle.threads()
    out = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    for w in (inputs.TINY, inputs.SWA_PREFILL):
        d = inputs.prefill_inputs(w)
        dt = timed(lambda: oracle.prefill(d["q"], d["k"], d["v"], d["sink"], w.mode, w.window, w.scale))
        fl = pairs_prefill(w.seqlen, w.mode, w.window) * w.hq * w.batch * FLOP_PER_PAIR
        out[w.name] = {"s": round(dt, 3), "gflops": round(fl / dt / 1e9, 2), "sample": "whole output"}
        del d
    w = inputs.GA_PREFILL
    d = inputs.prefill_inputs(w)
    rows = inputs.ga_parity_rows(w)
    dt = timed(lambda: oracle.prefill(d["q"], d["k"], d["v"], d["sink"], w.mode, w.window, w.scale, rows=rows))
    pairs = int(np.sum(rows[:, 2] + 1))
    full = pairs_prefill(w.seqlen, w.mode, w.window) * w.hq
    out[w.name] = {"s": round(dt, 3), "gflops": round(pairs * FLOP_PER_PAIR / dt / 1e9, 2),
                   "sample": f"{len(rows)} rows (every head x 512 positions), {pairs / full:.4f} of the pairs",
                   "extrapolated_full_s": round(dt * full / pairs, 1)}
    del d
    w = inputs.SWA_DECODE
    d = inputs.decode_ring_inputs(w, seed=w.seed * 100)
    dt = timed(lambda: oracle.decode(d["q"], d["k"], d["v"], d["seq_lens"], d["sink"], w.mode, w.window, w.scale,
                                     oracle.RING))
    fl = w.batch * w.window * w.hq * FLOP_PER_PAIR
    out[w.name] = {"s": round(dt, 4), "gflops": round(fl / dt / 1e9, 2), "sample": "whole output"}
    w = inputs.GA_DECODE
    d = inputs.decode_paged_inputs(w)
    dt = timed(lambda: oracle.decode(d["q"], d["k"], d["v"], d["seq_lens"], d["sink"], w.mode, w.window, w.scale,
                                     oracle.PAGED, d["block_table"]))
    fl = w.batch * w.ctx_hi * w.hq * FLOP_PER_PAIR
    out[w.name] = {"s": round(dt, 3), "gflops": round(fl / dt / 1e9, 2), "sample": "whole output"}
    del d
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    tot_fl = sum(v["gflops"] * v["s"] for v in out.values())
    tot_s = sum(v["s"] for v in out.values())
    return {"value": round(tot_fl / tot_s / 1e3, 6), "unit": "TFLOP/s", "cores": threads, "host_cores_visible": cores,
            "kind": "oracle",
            "sample": "tiny, SWA prefill 32K, SWA decode B=128 and GA decode 8x256K over their whole output; GA "
                      "prefill 32K on 64 heads x 512 positions (its full time extrapolated by the pair ratio)",
            "configs": out}


if __name__ == "__main__":
    sys.exit(main())
