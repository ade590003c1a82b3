"""Pins for the CPU oracle: checks against facts the pages and mathematics fix.

Each check takes a loaded oracle library (ctypes handle) and raises AssertionError on a
mismatch.  tests/test_oracle_pins.py runs them against the real oracle;
tests/test_oracle_mutations.py runs them against copies of the oracle with planted
mistakes and expects at least one to fail for every mistake.

Sources:
 * worked example -- "MiMo-V2-Flash Technical Report" paper notes, §4.3 (tests/golden/)
 * sink formula, max including the sink -- "MiMo-V2-Flash 架构 QA", Q3.7 and Q3.8
 * eager concat -> softmax -> drop -- "MiMo-V2-Flash 模型架构深度拆解", CH 10.1
 * masks -- same page, CH 10.3; window of 128 keys -- paper notes §4.3
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import oracle_np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def _sdpa_reference(q, k, v, mode, window, scale, sink=None):
    """torch CPU float64 scaled_dot_product_attention with an explicit mask.  With a sink,
    one extra key (zero k, zero v) is appended whose additive mask entry is the sink, so
    the extra column's logit is exactly the sink (the eager concat form)."""
    qt = torch.from_numpy(np.asarray(q, np.float64))
    kt = torch.from_numpy(np.asarray(k, np.float64))
    vt = torch.from_numpy(np.asarray(v, np.float64))
    B, Hq, L, _ = qt.shape
    G = Hq // kt.shape[1]
    kt = kt.repeat_interleave(G, dim=1)
    vt = vt.repeat_interleave(G, dim=1)
    i = torch.arange(L)[:, None]
    j = torch.arange(L)[None, :]
    keep = j <= i
    if mode == oracle.SWA:
        keep = keep & (j > i - window)
    if sink is None:
        return torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=keep, scale=scale).numpy()
    bias = torch.where(keep, 0.0, -math.inf).to(torch.float64)
    bias = bias[None, None].expand(B, Hq, L, L)
    sink_col = torch.as_tensor(np.asarray(sink, np.float64))[None, :, None, None].expand(B, Hq, L, 1)
    bias = torch.cat([bias, sink_col], dim=-1)
    kz = torch.cat([kt, torch.zeros_like(kt[:, :, :1])], dim=2)
    vz = torch.cat([vt, torch.zeros_like(vt[:, :, :1])], dim=2)
    return torch.nn.functional.scaled_dot_product_attention(qt, kz, vz, attn_mask=bias, scale=scale).numpy()


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    assert np.all(err <= lim), f"{what}: max err {err.max():.3e}"


# ------------------------------------------------------------------ P1 worked example
def worked_example_inputs(n=128, logit=2.0, pos=None, dqk=8, dv=None):
    """One head, SWA window n.  scale 1/8, q[0] = 4 and k_j[0] = 4*logit/2 so every logit is
    `logit` exactly; v_j = e_j (identity) so the output row is the weight vector."""
    dv = n if dv is None else dv
    L = n if pos is None else pos + 1
    q = np.zeros((1, 1, L, dqk), np.float32)
    k = np.zeros((1, 1, L, dqk), np.float32)
    v = np.zeros((1, 1, L, dv), np.float32)
    q[..., 0] = 4.0
    k[..., 0] = 2.0 * logit  # a = (4 * 2*logit) / 8 = logit
    for j in range(L):
        v[0, 0, j, j % dv] = 1.0
    return q, k, v


def pin_worked_example(lib):
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    n, a, s = g["n_keys"], g["logit"], g["sink"]
    q, k, v = worked_example_inputs(n, a, pos=300)
    out = oracle.prefill(q, k, v, np.array([s]), oracle.SWA, n, 0.125, rows=[[0, 0, 300]], lib=lib)[0]
    # the row holds the n window weights (keys 173..300 land in distinct identity columns)
    weights = out[out > 0]
    assert weights.size == n, weights.size
    pr = g["printed"]
    window_mass = out.sum()
    sink_mass = 1.0 - window_mass
    per_key = weights.mean()
    denom = 1.0 / sink_mass  # exp(sink - m) = 1 because m = sink
    for name, val in (("window_mass", window_mass), ("sink_mass", sink_mass),
                      ("weight_per_key", per_key), ("denominator", denom)):
        ref = pr[name]
        assert abs(val - ref["value"]) <= ref["half_ulp"] + 1e-12, (name, val, ref)
    assert np.all(np.abs(weights - per_key) < 1e-15)
    # exact values of the same example (weights equal, so each is e^{a-s} / (1 + n e^{a-s}))
    x = math.exp(a - s)
    assert abs(window_mass - n * x / (1 + n * x)) < 1e-13
    assert abs(per_key - x / (1 + n * x)) < 1e-15


def pin_worked_example_range(lib):
    """Logits spread over [0, 2] keep the window mass within [128/(128+e^4), 0.945424]."""
    lo_q, lo_k, lo_v = worked_example_inputs(128, 0.0, pos=200)
    lo = oracle.prefill(lo_q, lo_k, lo_v, np.array([4.0]), oracle.SWA, 128, 0.125,
                        rows=[[0, 0, 200]], lib=lib)[0].sum()
    assert abs(lo - 128 / (128 + math.exp(4))) < 1e-13, lo
    rng = np.random.default_rng(5)
    q = np.zeros((1, 1, 201, 8), np.float32)
    k = np.zeros((1, 1, 201, 8), np.float32)
    q[..., 0] = 4.0
    k[..., 0] = rng.uniform(0, 4, size=201)  # logits uniform in [0, 2]
    v = np.ones((1, 1, 201, 4), np.float32)
    mass = oracle.prefill(q, k, v, np.array([4.0]), oracle.SWA, 128, 0.125, rows=[[0, 0, 200]], lib=lib)[0, 0]
    assert lo < mass < 0.945424, mass


# ------------------------------------------------------------------ P3 / P4 / P5 library forms
def _tiny(seed, B=2, Hq=4, Hkv=2, L=37, dqk=24, dv=16):
    return (_rand((B, Hq, L, dqk), seed), _rand((B, Hkv, L, dqk), seed + 1),
            _rand((B, Hkv, L, dv), seed + 2))


def pin_no_sink_is_sdpa(lib):
    """sink NULL (and sink = -inf) give standard causal / sliding softmax attention."""
    for mode, W in ((oracle.GLOBAL, 0), (oracle.SWA, 5), (oracle.SWA, 1)):
        q, k, v = _tiny(10 + W)
        ref = _sdpa_reference(q, k, v, mode, W, 0.3)
        got = oracle.prefill(q, k, v, None, mode, W, 0.3, lib=lib)
        _close(got, ref, 1e-11, 1e-13, f"no-sink mode={mode} W={W}")
        got_inf = oracle.prefill(q, k, v, np.full(4, -np.inf), mode, W, 0.3, lib=lib)
        assert np.array_equal(got_inf, got)


def pin_sink_is_eager_concat(lib):
    """Sink attention equals SDPA over the keys plus one virtual key whose logit is the sink
    and whose value is zero (concat -> softmax -> drop)."""
    for mode, W in ((oracle.GLOBAL, 0), (oracle.SWA, 7)):
        q, k, v = _tiny(20 + W)
        sink = np.array([0.0, 1.5, 4.0, -2.0])
        ref = _sdpa_reference(q, k, v, mode, W, 0.3, sink)
        got = oracle.prefill(q, k, v, sink, mode, W, 0.3, lib=lib)
        _close(got, ref, 1e-11, 1e-13, f"sink concat mode={mode}")


def pin_sink_closed_form(lib):
    """O_sink = sigmoid(LSE_i - sink_h) * O_std with LSE the log-sum-exp of the visible
    logits (the sink scales every visible weight by one common factor)."""
    q, k, v = _tiny(31, B=1, Hq=4, Hkv=1, L=45, dqk=12, dv=10)
    sink = np.array([3.0, 0.5, 6.0, -1.0])
    W = 9
    std = _sdpa_reference(q, k, v, oracle.SWA, W, 0.5)
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(k.astype(np.float64)).repeat_interleave(4, dim=1)
    logits = (qt @ kt.transpose(-1, -2)) * 0.5
    i = torch.arange(45)[:, None]
    j = torch.arange(45)[None, :]
    logits = logits.masked_fill(~((j <= i) & (j > i - W)), -math.inf)
    lse = torch.logsumexp(logits, dim=-1).numpy()  # [1,4,45]
    factor = 1.0 / (1.0 + np.exp(sink[None, :, None] - lse))
    got = oracle.prefill(q, k, v, sink, oracle.SWA, W, 0.5, lib=lib)
    _close(got, std * factor[..., None], 1e-11, 1e-13, "closed form")


# ------------------------------------------------------------------ P6 / P7 / masks
def pin_wide_window_is_global(lib):
    q, k, v = _tiny(40, L=33)
    sink = np.array([1.0, 2.0, 3.0, 4.0])
    ga = oracle.prefill(q, k, v, sink, oracle.GLOBAL, 0, 0.2, lib=lib)
    for W in (33, 34, 1000):
        sw = oracle.prefill(q, k, v, sink, oracle.SWA, W, 0.2, lib=lib)
        assert np.array_equal(sw, ga), W
    sw32 = oracle.prefill(q, k, v, sink, oracle.SWA, 32, 0.2, lib=lib)
    assert not np.allclose(sw32[:, :, 32], ga[:, :, 32])  # the last row loses key 0


def pin_mass_below_one(lib):
    """With a finite sink the visible weights sum to strictly between 0 and 1; a +inf sink
    takes all the mass (output exactly 0).  v = 1 makes every output entry the weight sum."""
    q, _, _ = _tiny(50)
    k = _rand((2, 2, 37, 24), 51)
    v = np.ones((2, 2, 37, 3), np.float32)
    sink = np.array([0.0, 3.0, -5.0, 20.0])
    out = oracle.prefill(q, k, v, sink, oracle.SWA, 6, 0.3, lib=lib)
    assert np.all(out > 0) and np.all(out < 1)
    nos = oracle.prefill(q, k, v, None, oracle.SWA, 6, 0.3, lib=lib)
    _close(nos, np.ones_like(nos), 1e-14, 0, "no-sink weights sum to 1")
    inf = oracle.prefill(q, k, v, np.array([np.inf, 0, np.inf, 1.0]), oracle.SWA, 6, 0.3, lib=lib)
    assert np.all(inf[:, 0] == 0) and np.all(inf[:, 2] == 0) and np.all(inf[:, 1] > 0)


def pin_window_is_slice(lib):
    """Sliding row i equals global attention of the same query over the slice of the W most
    recent keys (positions i-W+1 .. i, the query's own included)."""
    q, k, v = _tiny(60, B=1, Hq=2, Hkv=1, L=40)
    sink = np.array([2.0, -1.0])
    for W in (1, 2, 7, 16):
        full = oracle.prefill(q, k, v, sink, oracle.SWA, W, 0.25, lib=lib)
        for i in (0, W - 1, W, 25, 39):
            lo = max(0, i - W + 1)
            qs = np.ascontiguousarray(q[:, :, lo:i + 1])
            ks = np.ascontiguousarray(k[:, :, lo:i + 1])
            vs = np.ascontiguousarray(v[:, :, lo:i + 1])
            sl = oracle.prefill(qs, ks, vs, sink, oracle.GLOBAL, 0, 0.25, lib=lib)
            _close(full[:, :, i], sl[:, :, i - lo], 1e-13, 1e-15, f"slice W={W} i={i}")


def pin_gqa_grouping(lib):
    """Query head h reads KV head h // (Hq/Hkv)."""
    q, k, v = _tiny(70, B=1, Hq=6, Hkv=3, L=20)
    sink = np.array([0.5, 1.0, 1.5, 2.0, 2.5, 3.0])
    full = oracle.prefill(q, k, v, sink, oracle.GLOBAL, 0, 0.3, lib=lib)
    for h in range(6):
        g = h // 2
        one = oracle.prefill(np.ascontiguousarray(q[:, h:h + 1]), np.ascontiguousarray(k[:, g:g + 1]),
                             np.ascontiguousarray(v[:, g:g + 1]), sink[h:h + 1], oracle.GLOBAL, 0, 0.3,
                             lib=lib)
        assert np.array_equal(full[:, h:h + 1], one), h


# ------------------------------------------------------------------ P8 brute force
def pin_brute_force(lib, cases=None):
    cases = cases or [(1, 4, 1, 50, 16, 8, oracle.SWA, W) for W in (1, 2, 127, 128, 129, 60)] + \
        [(2, 4, 2, 33, 24, 16, oracle.GLOBAL, 0), (1, 8, 2, 70, 20, 12, oracle.SWA, 9)]
    for n, (B, Hq, Hkv, L, dqk, dv, mode, W) in enumerate(cases):
        q = _rand((B, Hq, L, dqk), 100 + n)
        k = _rand((B, Hkv, L, dqk), 200 + n)
        v = _rand((B, Hkv, L, dv), 300 + n)
        sink = np.random.default_rng(400 + n).uniform(0, 6, Hq)
        ref = oracle_np.prefill(q, k, v, sink, mode, W, 0.17)
        got = oracle.prefill(q, k, v, sink, mode, W, 0.17, lib=lib)
        _close(got, ref, 1e-12, 1e-14, f"brute force case {n}")


# ------------------------------------------------------------------ P10 decode
def pin_decode_matches_prefill(lib):
    """decode at length n equals prefill row n-1, through a ring, an identity page table and
    a permuted page table (the caches are built from one contiguous sequence)."""
    from attention_sink_softmax_amd import inputs

    B, Hq, Hkv, dqk, dv, L = 2, 4, 2, 16, 8, 150
    q = _rand((B, Hq, L, dqk), 500)
    k = _rand((B, Hkv, L, dqk), 501)
    v = _rand((B, Hkv, L, dv), 502)
    sink = np.array([4.0, 0.0, 2.0, 5.0])
    for mode, W in ((oracle.SWA, 16), (oracle.SWA, 128), (oracle.GLOBAL, 0)):
        pre = oracle.prefill(q, k, v, sink, mode, W, 0.3, lib=lib)
        for n in (1, 5, 16, 17, 129, 150):
            lens = np.full(B, n, np.int32)
            qn = np.ascontiguousarray(q[:, :, n - 1])
            want = pre[:, :, n - 1]
            if mode == oracle.SWA:
                kr, vr = inputs.ring_from_sequence(k, v, n, W)
                got = oracle.decode(qn, kr, vr, lens, sink, mode, W, 0.3, oracle.RING, lib=lib)
                _close(got, want, 1e-12, 1e-14, f"ring W={W} n={n}")
            for perm in (False, True):
                kp, vp, bt = inputs.pages_from_sequence(k, v, n, 8, 2 * 19 + 3, 9, perm)
                got = oracle.decode(qn, kp, vp, lens, sink, mode, W, 0.3, oracle.PAGED, bt, lib=lib)
                _close(got, want, 1e-12, 1e-14, f"paged perm={perm} mode={mode} n={n}")


def pin_decode_mixed_lengths(lib):
    """Sequences of different lengths in one paged call each match their own prefill row."""
    from attention_sink_softmax_amd import inputs

    B, Hq, Hkv, dqk, dv, L = 3, 4, 1, 8, 8, 90
    q = _rand((B, Hq, L, dqk), 600)
    k = _rand((B, Hkv, L, dqk), 601)
    v = _rand((B, Hkv, L, dv), 602)
    sink = np.array([1.0, 2.0, 3.0, 4.0])
    lens = np.array([90, 1, 47], np.int32)
    pre = oracle.prefill(q, k, v, sink, oracle.GLOBAL, 0, 0.3, lib=lib)
    kp, vp, bt = inputs.pages_from_sequence(k, v, 90, 16, 20, 3, True)
    qn = np.stack([q[b, :, lens[b] - 1] for b in range(B)])
    got = oracle.decode(qn, kp, vp, lens, sink, oracle.GLOBAL, 0, 0.3, oracle.PAGED, bt, lib=lib)
    for b in range(B):
        _close(got[b], pre[b, :, lens[b] - 1], 1e-12, 1e-14, f"mixed b={b}")


def pin_decode_multi_matches_prefill(lib):
    """q_len new tokens per sequence (the parallel verification of drafted tokens, deep-dive
    CH 4.4) equal the last q_len rows of the prefill over the same sequence; positions below
    0 (n < q_len) give zero rows; q_len = 1 with a 4-D query equals the 3-D decode."""
    from attention_sink_softmax_amd import inputs

    B, Hq, Hkv, dqk, dv, L = 3, 4, 2, 16, 8, 70
    q = _rand((B, Hq, L, dqk), 700)
    k = _rand((B, Hkv, L, dqk), 701)
    v = _rand((B, Hkv, L, dv), 702)
    sink = np.array([3.0, 0.5, 1.5, 6.0])
    for mode, W in ((oracle.SWA, 5), (oracle.GLOBAL, 0)):
        pre = oracle.prefill(q, k, v, sink, mode, W, 0.3, lib=lib)
        for q_len in (1, 2, 4, 7):
            lens = np.array([70, 3, 41], np.int32)
            kp, vp, bt = inputs.pages_from_sequence(k, v, L, 8, 40, 9, True)
            qm = np.zeros((B, Hq, q_len, dqk), np.float32)
            want = np.zeros((B, Hq, q_len, dv))
            for b in range(B):
                for t in range(q_len):
                    i = int(lens[b]) - q_len + t
                    if i >= 0:
                        qm[b, :, t] = q[b, :, i]
                        want[b, :, t] = pre[b, :, i]
            got = oracle.decode(qm, kp, vp, lens, sink, mode, W, 0.3, oracle.PAGED, bt, lib=lib)
            _close(got, want, 1e-12, 1e-14, f"multi mode={mode} q_len={q_len}")
            if q_len == 1:
                got3 = oracle.decode(qm[:, :, 0], kp, vp, lens, sink, mode, W, 0.3, oracle.PAGED, bt, lib=lib)
                assert np.array_equal(got3, got[:, :, 0]), "q_len = 1 differs from one-token decode"


def pin_decode_side_matches_prefill(lib):
    """q_len new tokens whose keys and values are held beside the cache (the cache holds only
    the committed positions) give the last q_len prefill rows: a ring of W slots (sliding
    mode, the ring holding the last W committed positions, slots rotated), and permuted pages
    in both modes (pages past the committed length hold other data, never read).  Lengths
    below q_len give zero rows before position 0; q_len = 1 with a ring equals the one-token
    ring decode of the sequence with the token written into the ring."""
    B, Hq, Hkv, dqk, dv, L, W = 3, 4, 2, 16, 8, 60, 9
    q = _rand((B, Hq, L, dqk), 1300)
    k = _rand((B, Hkv, L, dqk), 1301)
    v = _rand((B, Hkv, L, dv), 1302)
    sink = np.array([1.0, 0.0, 3.0, 2.0])
    pre = {oracle.SWA: oracle.prefill(q, k, v, sink, oracle.SWA, W, 0.3, lib=lib),
           oracle.GLOBAL: oracle.prefill(q, k, v, sink, oracle.GLOBAL, 0, 0.3, lib=lib)}
    for q_len in (1, 2, 4, 7):
        lens = np.array([L, 31, max(1, q_len - 2)], np.int32)
        qm = np.zeros((B, Hq, q_len, dqk), np.float32)
        kn = np.zeros((B, Hkv, q_len, dqk), np.float32)
        vn = np.zeros((B, Hkv, q_len, dv), np.float32)
        kr = np.zeros((B, Hkv, W, dqk), np.float32)
        vr = np.zeros((B, Hkv, W, dv), np.float32)
        kpd = np.full((B * 8 + 3, Hkv, 8, dqk), 7.0, np.float32)  # data nobody may read
        vpd = np.full((B * 8 + 3, Hkv, 8, dv), 7.0, np.float32)
        bt = np.random.default_rng(1303 + q_len).permutation(B * 8 + 3)[:B * 8].reshape(B, 8).astype(np.int32)
        for b in range(B):
            nc = int(lens[b]) - q_len
            for t in range(q_len):
                if nc + t >= 0:
                    qm[b, :, t] = q[b, :, nc + t]
                    kn[b, :, t] = k[b, :, nc + t]
                    vn[b, :, t] = v[b, :, nc + t]
            for j in range(max(0, nc - W), max(0, nc)):
                kr[b, :, j % W] = k[b, :, j]
                vr[b, :, j % W] = v[b, :, j]
            for j in range(max(0, nc)):
                kpd[bt[b, j // 8], :, j % 8] = k[b, :, j]
                vpd[bt[b, j // 8], :, j % 8] = v[b, :, j]
        got = oracle.decode(qm, kr, vr, lens, sink, oracle.SWA, W, 0.3, oracle.RING, lib=lib, k_new=kn, v_new=vn)
        cases = [(oracle.SWA, got)]
        for mode, Wm in ((oracle.SWA, W), (oracle.GLOBAL, 0)):
            cases.append((mode, oracle.decode(qm, kpd, vpd, lens, sink, mode, Wm, 0.3, oracle.PAGED, bt, lib=lib,
                                              k_new=kn, v_new=vn)))
        for mode, out in cases:
            for b in range(B):
                for t in range(q_len):
                    i = int(lens[b]) - q_len + t
                    if i < 0:
                        assert np.all(out[b, :, t] == 0), (q_len, b, t)
                    else:
                        _close(out[b, :, t], pre[mode][b, :, i], 1e-12, 1e-14, f"side q_len={q_len} mode={mode} b={b}")
    # q_len = 1 beside a ring = one-token ring decode with the token written in
    lens = np.array([L, 31, 5], np.int32)
    kr = np.zeros((B, Hkv, W, dqk), np.float32)
    vr = np.zeros((B, Hkv, W, dv), np.float32)
    for b in range(B):
        for j in range(max(0, lens[b] - W), lens[b]):
            kr[b, :, j % W] = k[b, :, j]
            vr[b, :, j % W] = v[b, :, j]
    qn = np.stack([q[b, :, lens[b] - 1] for b in range(B)])
    ref = oracle.decode(qn, kr, vr, lens, sink, oracle.SWA, W, 0.3, oracle.RING, lib=lib)
    kn = np.stack([k[b, :, lens[b] - 1] for b in range(B)])[:, :, None]
    vn = np.stack([v[b, :, lens[b] - 1] for b in range(B)])[:, :, None]
    got = oracle.decode(qn[:, :, None], kr, vr, lens, sink, oracle.SWA, W, 0.3, oracle.RING, lib=lib,
                        k_new=np.ascontiguousarray(kn), v_new=np.ascontiguousarray(vn))[:, :, 0]
    _close(got, ref, 1e-12, 1e-14, "side q_len=1 vs ring decode")


def pin_prefill_cached_is_prefill_rows(lib):
    """A chunk of Lq tokens after a prefix held in permuted pages (both modes) or, in sliding
    mode, in a ring of the prefix's last W positions gives exactly the prefill rows of those
    positions; pages and slots outside the prefix hold data nobody may read."""
    B, Hq, Hkv, dqk, dv, L, W, ps = 2, 4, 2, 16, 8, 150, 11, 16
    q = _rand((B, Hq, L, dqk), 1400)
    k = _rand((B, Hkv, L, dqk), 1401)
    v = _rand((B, Hkv, L, dv), 1402)
    sink = np.array([0.5, 2.0, -1.0, 3.0])
    pre = {oracle.SWA: oracle.prefill(q, k, v, sink, oracle.SWA, W, 0.3, lib=lib),
           oracle.GLOBAL: oracle.prefill(q, k, v, sink, oracle.GLOBAL, 0, 0.3, lib=lib)}
    npg = B * (L // ps + 1) + 3
    bt = np.random.default_rng(1403).permutation(npg)[:B * (L // ps + 1)].reshape(B, -1).astype(np.int32)
    for kv_len, Lq in ((150, 1), (150, 60), (97, 90), (40, 40), (33, 7)):
        q0 = kv_len - Lq
        lens = np.full(B, kv_len, np.int32)
        kp = np.full((npg, Hkv, ps, dqk), 9.0, np.float32)
        vp = np.full((npg, Hkv, ps, dv), 9.0, np.float32)
        kr = np.full((B, Hkv, W, dqk), 9.0, np.float32)
        vr = np.full((B, Hkv, W, dv), 9.0, np.float32)
        for b in range(B):
            for j in range(q0):
                kp[bt[b, j // ps], :, j % ps] = k[b, :, j]
                vp[bt[b, j // ps], :, j % ps] = v[b, :, j]
            for j in range(max(0, q0 - W), q0):
                kr[b, :, j % W] = k[b, :, j]
                vr[b, :, j % W] = v[b, :, j]
        qc = np.ascontiguousarray(q[:, :, q0:kv_len])
        kc = np.ascontiguousarray(k[:, :, q0:kv_len])
        vc = np.ascontiguousarray(v[:, :, q0:kv_len])
        runs = [(oracle.SWA, oracle.RING, kr, vr, None)] + \
            [(mode, oracle.PAGED, kp, vp, bt) for mode in (oracle.SWA, oracle.GLOBAL)]
        for mode, layout, kc_, vc_, btx in runs:
            got = oracle.prefill_cached(qc, kc, vc, kc_, vc_, lens, sink, mode, W if mode == oracle.SWA else 0, 0.3,
                                        layout, btx, lib=lib)
            _close(got, pre[mode][:, :, q0:kv_len], 1e-12, 1e-14, f"cached prefix kv_len={kv_len} Lq={Lq} "
                                                                   f"mode={mode} layout={layout}")


def pin_prefill_chunk_is_prefill_rows(lib):
    """A chunk of Lq new tokens after a prefix of Lk - Lq tokens gives exactly the prefill rows
    Lk - Lq .. Lk - 1 of the whole sequence (model card serving set-up: chunked prefill)."""
    B, Hq, Hkv, dqk, dv, Lk = 2, 4, 2, 16, 8, 90
    q = _rand((B, Hq, Lk, dqk), 800)
    k = _rand((B, Hkv, Lk, dqk), 801)
    v = _rand((B, Hkv, Lk, dv), 802)
    sink = np.array([2.0, 0.0, 4.0, 1.0])
    for mode, W in ((oracle.SWA, 7), (oracle.GLOBAL, 0)):
        pre = oracle.prefill(q, k, v, sink, mode, W, 0.3, lib=lib)
        for Lq in (1, 13, 64, 90):
            qc = np.ascontiguousarray(q[:, :, Lk - Lq:])
            got = oracle.prefill_chunk(qc, k, v, sink, mode, W, 0.3, lib=lib)
            assert np.array_equal(got, pre[:, :, Lk - Lq:]), f"chunk mode={mode} Lq={Lq}"
        got = oracle.prefill_chunk(np.ascontiguousarray(q[:, :, :0]), k, v, sink, mode, W, 0.3, lib=lib)
        assert got.shape == (B, Hq, 0, dv)


def pin_e4m3_codes(lib):
    """The 8-bit cache format: all 256 E4M3 codes against torch's float8_e4m3fn decoding (a
    library routine), plus the format's landmarks (largest finite 448, smallest subnormal 2^-9,
    smallest normal 2^-6, 1.0 and its negative, the two NaN codes)."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        got = oracle.e4m3_value(c, lib=lib)
        assert (math.isnan(got) and math.isnan(ref[c])) or got == ref[c], f"code {c}: {got} vs {ref[c]}"
    assert oracle.e4m3_value(0x7E, lib=lib) == 448.0 and oracle.e4m3_value(0xFE, lib=lib) == -448.0
    assert oracle.e4m3_value(0x01, lib=lib) == 2.0 ** -9 and oracle.e4m3_value(0x08, lib=lib) == 2.0 ** -6
    assert oracle.e4m3_value(0x38, lib=lib) == 1.0 and oracle.e4m3_value(0xB8, lib=lib) == -1.0
    assert math.isnan(oracle.e4m3_value(0x7F, lib=lib)) and math.isnan(oracle.e4m3_value(0xFF, lib=lib))


def pin_e4m3_encode(lib):
    """The encoder that writes an 8-bit cache, against the format itself: every finite code
    survives value -> encode at several scales (powers of two and not); the midpoint of two
    neighbouring codes goes to the even one and points just off it to the nearer one;
    magnitudes above 448 * scale clamp to 0x7E / 0xFE; the sign of zero is kept.  Then
    against torch's float8_e4m3fn conversion (a library routine) on every bf16 value up to
    448 in magnitude, at scales 1 and 0.5."""
    val = {c: oracle.e4m3_value(c, lib=lib) for c in range(256)}
    finite = [c for c in range(256) if not math.isnan(val[c])]
    for s in (1.0, 0.5, 2.0 ** -6, 0.02, 0.37, 1.9):
        x = np.array([val[c] * s for c in finite], np.float32)
        got = oracle.e4m3_encode(x, s, lib=lib)
        bad = [(finite[i], int(got[i])) for i in range(len(finite)) if got[i] != finite[i]]
        assert not bad, f"round trip at scale {s}: {bad[:5]}"
    for sign in (0, 0x80):
        for c in range(0x00, 0x7E):  # neighbours c, c + 1, both finite
            lo, hi = val[c | sign], val[(c + 1) | sign]
            mid = (lo + hi) / 2  # exact in float32 (one more mantissa bit)
            even = c if c % 2 == 0 else c + 1
            got = oracle.e4m3_encode(np.array([mid, np.nextafter(np.float32(mid), np.float32(lo)),
                                               np.nextafter(np.float32(mid), np.float32(hi))], np.float32), 1.0,
                                     lib=lib)
            assert list(got) == [even | sign, c | sign, (c + 1) | sign], (hex(c | sign), list(map(hex, got)))
    for s in (1.0, 0.02):
        big = np.array([448.0001, 464.0, 500.0, 1e6, np.inf], np.float32) * np.float32(s)
        assert np.all(oracle.e4m3_encode(big, s, lib=lib) == 0x7E)
        assert np.all(oracle.e4m3_encode(-big, s, lib=lib) == 0xFE)
    z = oracle.e4m3_encode(np.array([0.0, -0.0, 1e-6, -1e-6, 2.0 ** -11, -(2.0 ** -11)], np.float32), 1.0, lib=lib)
    assert list(z) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80], list(map(hex, z))
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    xf = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    for s in (1.0, 0.5):
        with np.errstate(invalid="ignore", over="ignore"):
            keep = np.isfinite(xf) & (np.abs(xf / np.float32(s)) <= 448)
        want = torch.from_numpy(xf[keep] / np.float32(s)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        got = oracle.e4m3_encode(bits[keep], s, lib=lib)
        assert np.array_equal(got, want), f"torch float8_e4m3fn at scale {s}: {int((got != want).sum())} differ"


def pin_fp8_decode_is_decode_of_values(lib):
    """Decode from an 8-bit cache equals decode from a float32 cache holding the values the
    codes stand for (scale * code value, exact in float32 for these scales), both layouts."""
    from attention_sink_softmax_amd import inputs

    B, Hq, Hkv, dqk, dv, L = 2, 4, 2, 16, 8, 100
    rng = np.random.default_rng(900)
    k8 = rng.integers(0, 256, size=(B, Hkv, L, dqk), dtype=np.uint8)
    v8 = rng.integers(0, 256, size=(B, Hkv, L, dv), dtype=np.uint8)
    k8[(k8 & 0x7F) == 0x7F] = 0x38  # no NaN codes
    v8[(v8 & 0x7F) == 0x7F] = 0x30
    dec = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    ks, vs = 0.125, 2.0
    kf = (dec[k8] * ks).astype(np.float32)
    vf = (dec[v8] * vs).astype(np.float32)
    q = _rand((B, Hq, 3, dqk), 901)
    sink = np.array([1.0, 0.0, 3.0, 2.0])
    lens = np.array([100, 41], np.int32)
    for mode, W in ((oracle.GLOBAL, 0), (oracle.SWA, 9)):
        kp8, vp8, bt = inputs.pages_from_sequence(k8, v8, L, 16, 20, 5, True)
        kpf, vpf, _ = inputs.pages_from_sequence(kf, vf, L, 16, 20, 5, True)
        got = oracle.decode(q, kp8, vp8, lens, sink, mode, W, 0.3, oracle.PAGED, bt, lib=lib, kv_scales=(ks, vs))
        want = oracle.decode(q, kpf, vpf, lens, sink, mode, W, 0.3, oracle.PAGED, bt, lib=lib)
        _close(got, want, 1e-12, 1e-14, f"fp8 decode mode={mode}")


def pin_lse(lib):
    """Each row's log-sum-exp (the log of the sink softmax denominator) against scipy's
    logsumexp over the eager form's S+1 columns; with a sink of -inf (no sink) it is the
    plain softmax's; LSE(sink) = logaddexp(LSE(no sink), sink); an empty row (a decode
    position before the sequence) has LSE = sink."""
    B, Hq, Hkv, L, dqk, dv = 1, 4, 2, 40, 16, 8
    q = _rand((B, Hq, L, dqk), 1000)
    k = _rand((B, Hkv, L, dqk), 1001)
    v = _rand((B, Hkv, L, dv), 1002)
    sink = np.array([0.5, 3.0, -1.0, 6.0])
    for mode, W in ((oracle.GLOBAL, 0), (oracle.SWA, 5)):
        out, lse = oracle.prefill_chunk(q, k, v, sink, mode, W, 0.4, lib=lib, return_lse=True)
        _, ref = oracle_np.prefill(q, k, v, sink, mode, W, 0.4, return_lse=True)
        _close(lse, ref, 1e-12, 1e-13, f"lse mode={mode}")
        # scipy's logsumexp over the visible logits and the sink as one more column
        from scipy.special import logsumexp
        logits = 0.4 * np.einsum("bhid,bhjd->bhij", q.astype(np.float64), np.repeat(k, 2, axis=1).astype(np.float64))
        logits = np.where(oracle_np.mask_matrix(L, mode, W), logits, -np.inf)
        col = np.broadcast_to(sink[None, :, None, None], (B, Hq, L, 1))
        _close(lse, logsumexp(np.concatenate([logits, col], axis=-1), axis=-1), 1e-12, 1e-13, f"lse scipy mode={mode}")
        _, lse0 = oracle.prefill_chunk(q, k, v, None, mode, W, 0.4, lib=lib, return_lse=True)
        _, ref0 = oracle_np.prefill(q, k, v, None, mode, W, 0.4, return_lse=True)
        _close(lse0, ref0, 1e-12, 1e-13, f"lse no sink mode={mode}")
        _close(lse, np.logaddexp(lse0, sink[None, :, None]), 1e-12, 1e-13, f"lse sink relation mode={mode}")
    # decode rows before the sequence start: empty visible set
    from attention_sink_softmax_amd import inputs
    kp, vp, bt = inputs.pages_from_sequence(k, v, L, 8, 6, 3, True)
    qd = np.ascontiguousarray(q[:, :, :3])
    lens = np.array([1], np.int32)
    _, lsed = oracle.decode(qd, kp, vp, lens, sink, oracle.GLOBAL, 0, 0.4, oracle.PAGED, bt, lib=lib, return_lse=True)
    assert np.array_equal(lsed[0, :, 0], sink) and np.array_equal(lsed[0, :, 1], sink)
    _, lsen = oracle.decode(qd, kp, vp, lens, None, oracle.GLOBAL, 0, 0.4, oracle.PAGED, bt, lib=lib, return_lse=True)
    assert np.all(np.isneginf(lsen[0, :, :2]))


def pin_rope(lib):
    """Partial RoPE: the pages' angle pos * theta^(-2i/64) for pair i, seen on unit vectors
    (dimension i turns towards i + 32); position 0 is the identity; the 128 trailing
    dimensions are untouched; every pair keeps its length; the rotated dot product depends on
    the position difference only (q at m, k at n equals q at m - n, k at 0)."""
    rng = np.random.default_rng(1100)
    for theta in (oracle.SWA_ROPE_THETA, oracle.GA_ROPE_THETA):
        eye = np.eye(192, dtype=np.float32)[:64]
        for pos in (0, 1, 7, 131071, 262143):
            out = oracle.rope(eye, np.full(64, pos), theta, lib=lib)
            for i in (0, 1, 13, 31):
                ang = pos * theta ** (-2.0 * i / 64)
                want = np.zeros(192)
                want[i], want[i + 32] = math.cos(ang), math.sin(ang)
                assert np.allclose(out[i], want, rtol=0, atol=1e-12), (theta, pos, i)
                want2 = np.zeros(192)
                want2[i + 32], want2[i] = math.cos(ang), -math.sin(ang)
                assert np.allclose(out[i + 32], want2, rtol=0, atol=1e-12), (theta, pos, i, "partner")
        x = rng.standard_normal((50, 192)).astype(np.float32)
        assert np.array_equal(oracle.rope(x, np.zeros(50), theta, lib=lib), x.astype(np.float64))
        pos = rng.integers(0, 262144, 50)
        out = oracle.rope(x, pos, theta, lib=lib)
        assert np.array_equal(out[:, 64:], x[:, 64:].astype(np.float64))
        n_in = x[:, :32].astype(np.float64) ** 2 + x[:, 32:64].astype(np.float64) ** 2
        assert np.allclose(out[:, :32] ** 2 + out[:, 32:64] ** 2, n_in, rtol=1e-12, atol=0)
        qv, kv = x[:25], x[25:]
        m, n = pos[:25], rng.integers(0, 262144, 25)
        lhs = np.sum(oracle.rope(qv, m, theta, lib=lib)[:, :64] * oracle.rope(kv, n, theta, lib=lib)[:, :64], axis=1)
        rhs = np.sum(oracle.rope(qv, m - n, theta, lib=lib)[:, :64] * kv[:, :64].astype(np.float64), axis=1)
        assert np.allclose(lhs, rhs, rtol=1e-9, atol=1e-9), "relative-position property"


def pin_append_then_decode_is_prefill(lib):
    """Tokens appended one step at a time into a ring and into pages, then decoded, give the
    prefill rows of the whole sequence (both modes for pages; the ring in sliding mode)."""
    B, Hq, Hkv, dqk, dv, L, W, ps = 2, 4, 2, 16, 8, 45, 6, 8
    q = _rand((B, Hq, L, dqk), 1200)
    k = _rand((B, Hkv, L, dqk), 1201)
    v = _rand((B, Hkv, L, dv), 1202)
    sink = np.array([1.0, 2.0, 0.5, 4.0])
    kr = np.zeros((B, Hkv, W, dqk), np.float32)
    vr = np.zeros((B, Hkv, W, dv), np.float32)
    bt = np.random.default_rng(1203).permutation(B * 6 + 2)[:B * 6].reshape(B, 6).astype(np.int32)
    kp = np.zeros((B * 6 + 2, Hkv, ps, dqk), np.float32)
    vp = np.zeros((B * 6 + 2, Hkv, ps, dv), np.float32)
    pre_swa = oracle.prefill(q, k, v, sink, oracle.SWA, W, 0.3, lib=lib)
    pre_ga = oracle.prefill(q, k, v, sink, oracle.GLOBAL, 0, 0.3, lib=lib)
    n = 0
    for step in (3, 1, 1, 7, 1, 20, 12):  # new tokens per step; the first steps act as prefill
        lens = np.full(B, n + step, np.int32)
        oracle.kv_append(kr, vr, oracle.RING, k[:, :, n:n + step], v[:, :, n:n + step], lens, window=W)
        oracle.kv_append(kp, vp, oracle.PAGED, k[:, :, n:n + step], v[:, :, n:n + step], lens, block_table=bt)
        n += step
        qn = np.ascontiguousarray(q[:, :, n - 1])
        got = oracle.decode(qn, kr, vr, lens, sink, oracle.SWA, W, 0.3, oracle.RING, lib=lib)
        _close(got, pre_swa[:, :, n - 1], 1e-12, 1e-14, f"ring after append n={n}")
        for mode, Wm, pre in ((oracle.SWA, W, pre_swa), (oracle.GLOBAL, 0, pre_ga)):
            got = oracle.decode(qn, kp, vp, lens, sink, mode, Wm, 0.3, oracle.PAGED, bt, lib=lib)
            _close(got, pre[:, :, n - 1], 1e-12, 1e-14, f"pages after append n={n} mode={mode}")


def pin_fp8_append_then_decode_is_prefill(lib):
    """Tokens appended one step at a time into an 8-bit paged cache, then decoded with the
    cache's scales, give the prefill rows over the values the cache holds: K and V replaced by
    scale * value(code), each code being the encoder's code of the element at that scale."""
    B, Hq, Hkv, dqk, dv, L, ps = 2, 4, 2, 16, 8, 45, 8
    q = _rand((B, Hq, L, dqk), 1210)
    k = _rand((B, Hkv, L, dqk), 1211)
    v = _rand((B, Hkv, L, dv), 1212)
    sink = np.array([1.0, 2.0, 0.5, 4.0])
    ks, vs = 0.02, 0.37
    dec = np.array([oracle.e4m3_value(c, lib=lib) for c in range(256)])
    # the values the cache holds, rounded to float32 for the prefill oracle (relative 2^-24)
    kq = (dec[oracle.e4m3_encode(k, ks, lib=lib)] * ks).astype(np.float32)
    vq = (dec[oracle.e4m3_encode(v, vs, lib=lib)] * vs).astype(np.float32)
    assert np.allclose(kq, k, rtol=2 ** -4, atol=ks * 2 ** -10) and not np.array_equal(kq, k)
    bt = np.random.default_rng(1213).permutation(B * 6 + 2)[:B * 6].reshape(B, 6).astype(np.int32)
    kp = np.zeros((B * 6 + 2, Hkv, ps, dqk), np.uint8)
    vp = np.zeros((B * 6 + 2, Hkv, ps, dv), np.uint8)
    pre = {mode: oracle.prefill(q, kq, vq, sink, mode, Wm, 0.3, lib=lib) for mode, Wm in ((oracle.SWA, 6),
                                                                                           (oracle.GLOBAL, 0))}
    n = 0
    for step in (3, 1, 9, 1, 20, 11):
        lens = np.full(B, n + step, np.int32)
        oracle.kv_append(kp, vp, oracle.PAGED, k[:, :, n:n + step], v[:, :, n:n + step], lens, block_table=bt,
                         fp8_scales=(ks, vs), lib=lib)
        n += step
        qn = np.ascontiguousarray(q[:, :, n - 1])
        for mode, Wm in ((oracle.SWA, 6), (oracle.GLOBAL, 0)):
            got = oracle.decode(qn, kp, vp, lens, sink, mode, Wm, 0.3, oracle.PAGED, bt, lib=lib, kv_scales=(ks, vs))
            _close(got, pre[mode][:, :, n - 1], 1e-5, 1e-6, f"8-bit pages after append n={n} mode={mode}")


def pin_backward_autograd(lib):
    """Gradients of sum(dO * O) against torch autograd through the eager form (concat the sink
    column -> softmax -> drop -> times V), fp64 on the CPU, with and without a sink, both
    modes, grouped heads."""
    B, Hq, Hkv, L, dqk, dv = 2, 4, 2, 37, 16, 8
    q = _rand((B, Hq, L, dqk), 1300)
    k = _rand((B, Hkv, L, dqk), 1301)
    v = _rand((B, Hkv, L, dv), 1302)
    do = _rand((B, Hq, L, dv), 1303)
    for sink_val in (np.array([0.5, 3.0, -1.0, 2.0]), None):
        for mode, W in ((oracle.GLOBAL, 0), (oracle.SWA, 6)):
            got = oracle.prefill_backward(q, k, v, sink_val, do, mode, W, 0.35, lib=lib)
            tq = torch.from_numpy(q.astype(np.float64)).requires_grad_()
            tk = torch.from_numpy(k.astype(np.float64)).requires_grad_()
            tv = torch.from_numpy(v.astype(np.float64)).requires_grad_()
            ts = None if sink_val is None else torch.from_numpy(sink_val).requires_grad_()
            G = Hq // Hkv
            kx, vx = tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1)
            sc = (tq @ kx.transpose(-1, -2)) * 0.35
            keep = torch.from_numpy(oracle_np.mask_matrix(L, mode, W))
            sc = sc.masked_fill(~keep, float("-inf"))
            if ts is not None:
                sc = torch.cat([sc, ts.view(1, Hq, 1, 1).expand(B, Hq, L, 1)], dim=-1)
            pr = torch.softmax(sc, dim=-1)
            if ts is not None:
                pr = pr[..., :-1]
            out = pr @ vx
            (out * torch.from_numpy(do.astype(np.float64))).sum().backward()
            _close(got[0], tq.grad.numpy(), 1e-10, 1e-12, f"dq sink={sink_val is not None} mode={mode}")
            _close(got[1], tk.grad.numpy(), 1e-10, 1e-12, f"dk sink={sink_val is not None} mode={mode}")
            _close(got[2], tv.grad.numpy(), 1e-10, 1e-12, f"dv sink={sink_val is not None} mode={mode}")
            if ts is not None:
                _close(got[3], ts.grad.numpy(), 1e-10, 1e-12, f"dsink mode={mode}")
            else:
                assert got[3] is None


def pin_backward_finite_differences(lib):
    """dL/dsink and a few dq, dk, dv entries against central differences of the forward oracle
    (L = sum(dO * O), step 1e-5, fp64)."""
    B, Hq, Hkv, L, dqk, dv = 1, 2, 1, 12, 8, 4
    q = _rand((B, Hq, L, dqk), 1400).astype(np.float64)
    k = _rand((B, Hkv, L, dqk), 1401).astype(np.float64)
    v = _rand((B, Hkv, L, dv), 1402).astype(np.float64)
    do = _rand((B, Hq, L, dv), 1403).astype(np.float64)
    sink = np.array([1.5, -0.5])

    def loss(q_, k_, v_, s_):
        return float(np.sum(oracle_np.prefill(q_, k_, v_, s_, oracle.SWA, 5, 0.3) * do))

    dq, dk, dvv, ds = oracle.prefill_backward(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32), sink,
                                              do.astype(np.float32), oracle.SWA, 5, 0.3, lib=lib)
    h = 1e-5
    for hh in range(Hq):
        sp, sm = sink.copy(), sink.copy()
        sp[hh] += h
        sm[hh] -= h
        num = (loss(q, k, v, sp) - loss(q, k, v, sm)) / (2 * h)
        assert abs(num - ds[hh]) < 1e-6 * max(1.0, abs(num)), f"dsink[{hh}] {ds[hh]} vs {num}"
    q32, k32, v32 = (x.astype(np.float32).astype(np.float64) for x in (q, k, v))
    for arr, grad, idx in ((q32, dq, (0, 1, 7, 3)), (k32, dk, (0, 0, 4, 5)), (v32, dvv, (0, 0, 9, 2))):
        xp, xm = arr.copy(), arr.copy()
        xp[idx] += h
        xm[idx] -= h
        args_p = [q32, k32, v32]
        args_m = [q32, k32, v32]
        which = 0 if arr is q32 else 1 if arr is k32 else 2
        args_p[which], args_m[which] = xp, xm
        num = (loss(*args_p, sink) - loss(*args_m, sink)) / (2 * h)
        assert abs(num - grad[idx]) < 1e-6 * max(1.0, abs(num)), f"grad {which} {idx}: {grad[idx]} vs {num}"


def pin_backward_sampled_is_backward(lib):
    """The sampled gradients (chosen dq rows, dk and dv of chosen keys) equal the entries of the
    full backward, both modes, grouped heads, first, middle and last rows and keys."""
    B, Hq, Hkv, L, dqk, dv = 2, 6, 2, 41, 16, 8
    q = _rand((B, Hq, L, dqk), 1500)
    k = _rand((B, Hkv, L, dqk), 1501)
    v = _rand((B, Hkv, L, dv), 1502)
    do = _rand((B, Hq, L, dv), 1503)
    sink = np.array([0.5, 3.0, -1.0, 2.0, np.inf, -np.inf])
    for mode, W in ((oracle.GLOBAL, 0), (oracle.SWA, 7)):
        dq, dk, dvv, _ = oracle.prefill_backward(q, k, v, sink, do, mode, W, 0.3, lib=lib)
        qr = [(b, h, i) for b in range(B) for h in range(Hq) for i in (0, 6, 20, L - 1)]
        kr = [(b, g, j) for b in range(B) for g in range(Hkv) for j in (0, 6, 33, L - 1)]
        sq, sk, sv = oracle.prefill_backward_sampled(q, k, v, sink, do, mode, W, 0.3, qr, kr, lib=lib)
        for n, (b, h, i) in enumerate(qr):
            _close(sq[n], dq[b, h, i], 1e-12, 1e-14, f"dq row {(b, h, i)} mode={mode}")
        for n, (b, g, j) in enumerate(kr):
            _close(sk[n], dk[b, g, j], 1e-12, 1e-14, f"dk key {(b, g, j)} mode={mode}")
            _close(sv[n], dvv[b, g, j], 1e-12, 1e-14, f"dv key {(b, g, j)} mode={mode}")


ALL_PINS = [
    pin_worked_example, pin_worked_example_range, pin_no_sink_is_sdpa, pin_sink_is_eager_concat,
    pin_sink_closed_form, pin_wide_window_is_global, pin_mass_below_one, pin_window_is_slice,
    pin_gqa_grouping, pin_brute_force, pin_decode_matches_prefill, pin_decode_mixed_lengths,
    pin_decode_multi_matches_prefill, pin_decode_side_matches_prefill, pin_prefill_cached_is_prefill_rows,
    pin_prefill_chunk_is_prefill_rows, pin_e4m3_codes, pin_e4m3_encode,
    pin_fp8_decode_is_decode_of_values, pin_lse, pin_rope, pin_append_then_decode_is_prefill,
    pin_fp8_append_then_decode_is_prefill,
    pin_backward_autograd, pin_backward_finite_differences, pin_backward_sampled_is_backward,
]
