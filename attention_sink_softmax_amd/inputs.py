"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds the workload catalogue and the random-input generators. It does
no attention arithmetic: it draws Gaussian and uniform numbers, rounds them to
bfloat16 bit patterns, and builds KV-cache layouts (ring slots, page tables) by
plain indexing. Both the GPU path and the CPU oracle consume what it returns.

Workload shapes follow the model configuration printed on the architecture
deep-dive page ("MiMo-V2-Flash 模型架构深度拆解", CH 8.1 config table and CH 10.3):
64 query heads, 8 KV heads in sliding-window layers and 4 in global layers,
head_dim 192 for q/k, 128 for v, window 128, and the 32K native / 256K extended
context named on the model-card page (§1).

Value distributions: q, k, v ~ N(0, 1); per-query-head sink ~ U[0, 6] (the paper
notes page, §4.3, reports learned sinks spanning 0 to 6 across heads).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

MODE_GLOBAL = 0
MODE_SWA = 1

_CHUNK = 1 << 22


# --------------------------------------------------------------------------- bf16 bits
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits.

    Inputs must be finite (the generators only produce finite values)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill_normal(n: int, seed: int, stream: int, bf16: bool) -> np.ndarray:
    """n draws of N(0,1); chunk c uses the generator seeded by (seed, stream, c), so the
    values do not depend on how many threads produced them."""
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c: int) -> None:
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = np.random.default_rng([seed, stream, c])
        tmp = g.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = bf16_bits(tmp) if bf16 else tmp

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def e4m3_codes(x: np.ndarray, scale: float) -> np.ndarray:
    """Codes of x / scale in the OCP 8-bit E4M3 format (round to nearest even, clamped to the
    largest finite value 448), as uint8, by torch's float8_e4m3fn conversion."""
    import torch

    y = np.clip(np.asarray(x, np.float32) / np.float32(scale), -448.0, 448.0)
    return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def normal_e4m3(shape, seed: int, stream: int, scale: float) -> np.ndarray:
    """Seeded N(0,1) draws stored as E4M3 codes of value / scale (uint8), chunk by chunk."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint8)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c: int) -> None:
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = np.random.default_rng([seed, stream, c])
        out[lo:hi] = e4m3_codes(g.standard_normal(hi - lo, dtype=np.float32), scale)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def normal(shape, seed: int, stream: int, bf16: bool = True) -> np.ndarray:
    """Seeded N(0,1) tensor: uint16 bf16 bits when bf16, else float32."""
    n = int(np.prod(shape))
    return _fill_normal(n, seed, stream, bf16).reshape(shape)


def sink_values(hq: int, seed: int, lo: float = 0.0, hi: float = 6.0) -> np.ndarray:
    """Per-query-head sink, float32 [hq] ~ U[lo, hi]."""
    g = np.random.default_rng([seed, 99])
    return g.uniform(lo, hi, size=hq).astype(np.float32)


# --------------------------------------------------------------------------- catalogue
@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" | "decode"
    mode: int            # MODE_GLOBAL | MODE_SWA
    batch: int
    hq: int
    hkv: int
    seqlen: int = 0      # prefill length L
    window: int = 128
    d_qk: int = 192
    d_v: int = 128
    seed: int = 0
    fp32_source: bool = False  # tiny case: fp32 data, the GPU gets bf16-rounded copies
    # decode only
    layout: str = ""     # "ring" | "paged"
    ctx_lo: int = 0
    ctx_hi: int = 0
    page_size: int = 64
    q_len: int = 1       # new tokens per sequence (q_len > 1: drafted tokens verified together)
    kv_fp8: bool = False  # 8-bit E4M3 cache with per-tensor scales (decode only)
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return float(self.d_qk) ** -0.5


TINY = Workload("tiny_swa_L512", "prefill", MODE_SWA, 1, 4, 1, seqlen=512, window=128, seed=0,
                fp32_source=True)
SWA_PREFILL = Workload("swa_prefill_L32768", "prefill", MODE_SWA, 1, 64, 8, seqlen=32768,
                       window=128, seed=1)
GA_PREFILL = Workload("ga_prefill_L32768", "prefill", MODE_GLOBAL, 1, 64, 4, seqlen=32768,
                      window=0, seed=2)
SWA_DECODE = Workload("swa_decode_B128_ring", "decode", MODE_SWA, 128, 64, 8, window=128, seed=3,
                      layout="ring", ctx_lo=4096, ctx_hi=65536)
GA_DECODE = Workload("ga_decode_B8_256K_paged", "decode", MODE_GLOBAL, 8, 64, 4, window=0, seed=4,
                     layout="paged", ctx_lo=262144, ctx_hi=262144, page_size=64)
# verification of 4 drafted tokens per sequence (the multi-token-prediction step) at 256K
GA_VERIFY = Workload("ga_verify_B8_256K_q4_paged", "decode", MODE_GLOBAL, 8, 64, 4, window=0, seed=5,
                     layout="paged", ctx_lo=262144, ctx_hi=262144, page_size=64, q_len=4)

# the global decode workload with the cache in 8-bit floating point (one byte per element, as
# the pages size it), K and V stored as codes of value / 2^-6
GA_DECODE_FP8 = Workload("ga_decode_B8_256K_paged_fp8", "decode", MODE_GLOBAL, 8, 64, 4, window=0, seed=6,
                         layout="paged", ctx_lo=262144, ctx_hi=262144, page_size=64, kv_fp8=True)
FP8_KV_SCALE = 2.0 ** -6

# the sliding-window decode workload with 4 drafted tokens per sequence, their keys and values
# held beside the rings (the rings hold the committed positions only)
SWA_VERIFY = Workload("swa_verify_B128_ring_q4", "decode", MODE_SWA, 128, 64, 8, window=128, seed=7,
                      layout="ring", ctx_lo=4096, ctx_hi=65536, q_len=4)

WORKLOADS = {w.name: w for w in (TINY, SWA_PREFILL, GA_PREFILL, SWA_DECODE, GA_DECODE, GA_VERIFY, GA_DECODE_FP8,
                                 SWA_VERIFY)}


# --------------------------------------------------------------------------- prefill
def prefill_inputs(w: Workload, seed: int | None = None, seqlen: int | None = None,
                   batch: int | None = None, sink: bool = True) -> dict:
    """q [B,Hq,L,dqk], k [B,Hkv,L,dqk], v [B,Hkv,L,dv] and sink [Hq].

    Returns bf16 bit arrays under q/k/v (what the GPU receives) and, for the fp32-sourced
    tiny case, the original float32 arrays under q32/k32/v32."""
    s = w.seed if seed is None else seed
    L = w.seqlen if seqlen is None else seqlen
    B = w.batch if batch is None else batch
    out = {}
    shapes = {"q": (B, w.hq, L, w.d_qk), "k": (B, w.hkv, L, w.d_qk), "v": (B, w.hkv, L, w.d_v)}
    for i, (nm, shp) in enumerate(shapes.items()):
        if w.fp32_source:
            x = normal(shp, s, i, bf16=False)
            out[nm + "32"] = x
            out[nm] = bf16_bits(x)
        else:
            out[nm] = normal(shp, s, i, bf16=True)
    out["sink"] = sink_values(w.hq, s) if sink else None
    return out


def ga_parity_rows(w: Workload, n_first: int = 128, n_last: int = 128, n_rand: int = 256) -> np.ndarray:
    """The rows of a long causal prefill that are checked against the oracle and that the
    oracle is timed on: for every query head of sequence 0, the first 128 positions, the last
    128 and 256 more drawn without replacement, uniformly from the rest (seeded by the
    workload).  int64 [Hq * 512, 3] of (b, h, i)."""
    L = w.seqlen
    g = np.random.default_rng([w.seed, 11])
    mid = np.sort(g.choice(np.arange(n_first, L - n_last), size=n_rand, replace=False))
    pos = np.concatenate([np.arange(n_first), mid, np.arange(L - n_last, L)])
    return np.array([(0, h, i) for h in range(w.hq) for i in pos], np.int64)


def prefill_cached_inputs(w: Workload, Lq: int, page_size: int = 64) -> dict:
    """A prefill workload's last Lq positions as a chunk after a prefix held in a cache: q, k, v
    of the chunk [B,H,Lq,d]; the prefix (positions 0 .. L-Lq-1) in seeded, permuted pages
    (k_pages, v_pages [P,Hkv,page,d], block_table [B,max_pages], pool of twice the pages needed)
    and in rings of its last `window` positions (k_ring, v_ring [B,Hkv,W,d]); sink."""
    d = prefill_inputs(w)
    L, q0 = w.seqlen, w.seqlen - Lq
    out = {n: np.ascontiguousarray(d[n][:, :, q0:]) for n in ("q", "k", "v")}
    out["sink"] = d["sink"]
    mp = max(1, (q0 + page_size - 1) // page_size)
    out["block_table"] = page_table(w.batch, mp, 2 * w.batch * mp, w.seed + 100)
    P = 2 * w.batch * mp
    kp = np.zeros((P, w.hkv, page_size, w.d_qk), np.uint16)
    vp = np.zeros((P, w.hkv, page_size, w.d_v), np.uint16)
    for b in range(w.batch):
        for i in range(mp):
            j0, j1 = i * page_size, min(q0, (i + 1) * page_size)
            pg = out["block_table"][b, i]
            kp[pg, :, :j1 - j0] = d["k"][b, :, j0:j1]
            vp[pg, :, :j1 - j0] = d["v"][b, :, j0:j1]
    out["k_pages"], out["v_pages"] = kp, vp
    W = max(1, w.window)
    kr = np.zeros((w.batch, w.hkv, W, w.d_qk), np.uint16)
    vr = np.zeros((w.batch, w.hkv, W, w.d_v), np.uint16)
    for j in range(max(0, q0 - W), q0):
        kr[:, :, j % W] = d["k"][:, :, j]
        vr[:, :, j % W] = d["v"][:, :, j]
    out["k_ring"], out["v_ring"] = kr, vr
    return out


# --------------------------------------------------------------------------- decode
def decode_seq_lens(w: Workload, seed: int | None = None, batch: int | None = None) -> np.ndarray:
    s = w.seed if seed is None else seed
    B = w.batch if batch is None else batch
    if w.ctx_lo == w.ctx_hi:
        return np.full(B, w.ctx_lo, dtype=np.int32)
    g = np.random.default_rng([s, 7])
    return g.integers(w.ctx_lo, w.ctx_hi, size=B, endpoint=True).astype(np.int32)


def decode_ring_inputs(w: Workload, seed: int | None = None, batch: int | None = None,
                       seq_lens: np.ndarray | None = None) -> dict:
    """Ring caches of `window` slots per (sequence, KV head): k [B,Hkv,W,dqk],
    v [B,Hkv,W,dv]; the slot of position p is p mod W. Slots hold N(0,1) bf16 data
    (the content of the W most recent positions)."""
    s = w.seed if seed is None else seed
    B = w.batch if batch is None else batch
    W = w.window
    lens = decode_seq_lens(w, s, B) if seq_lens is None else np.asarray(seq_lens, np.int32)
    return {
        "q": normal((B, w.hq, w.d_qk), s, 0),
        "k": normal((B, w.hkv, W, w.d_qk), s, 1),
        "v": normal((B, w.hkv, W, w.d_v), s, 2),
        "seq_lens": lens,
        "sink": sink_values(w.hq, s),
    }


def decode_ring_verify_inputs(w: Workload, seed: int | None = None) -> dict:
    """Rings of the committed positions and q_len drafted tokens beside them: q [B,Hq,q_len,dqk],
    k_new [B,Hkv,q_len,dqk], v_new [B,Hkv,q_len,dv] (bf16 bits), ring caches k [B,Hkv,W,dqk],
    v [B,Hkv,W,dv] filled with N(0,1) data (the slots stand for the last W committed positions),
    seq_lens (committed + q_len) and sink."""
    s = w.seed if seed is None else seed
    lens = decode_seq_lens(w, s)
    B = w.batch
    return {"q": normal((B, w.hq, w.q_len, w.d_qk), s, 0), "k": normal((B, w.hkv, w.window, w.d_qk), s, 1),
            "v": normal((B, w.hkv, w.window, w.d_v), s, 2), "k_new": normal((B, w.hkv, w.q_len, w.d_qk), s, 3),
            "v_new": normal((B, w.hkv, w.q_len, w.d_v), s, 4), "seq_lens": lens, "sink": sink_values(w.hq, s)}


def page_table(batch: int, pages_per_seq: int, num_pages: int, seed: int, permute: bool = True) -> np.ndarray:
    """int32 [batch, pages_per_seq] drawing distinct pool pages; a random permutation of
    the pool when permute, else the identity (contiguous) order."""
    need = batch * pages_per_seq
    if need > num_pages:
        raise ValueError("pool too small for the page table")
    ids = np.random.default_rng([seed, 11]).permutation(num_pages) if permute else np.arange(num_pages)
    return ids[:need].astype(np.int32).reshape(batch, pages_per_seq)


def decode_paged_inputs(w: Workload, seed: int | None = None, batch: int | None = None,
                        ctx: int | None = None, num_pages: int | None = None,
                        permute: bool = True) -> dict:
    """Paged caches: pool k [P,Hkv,page,dqk], v [P,Hkv,page,dv], block_table [B,max_pages];
    q [B,Hq,dqk], or [B,Hq,q_len,dqk] when the workload has q_len > 1."""
    s = w.seed if seed is None else seed
    B = w.batch if batch is None else batch
    n = w.ctx_hi if ctx is None else ctx
    ps = w.page_size
    max_pages = (n + ps - 1) // ps
    P = B * max_pages if num_pages is None else num_pages
    return {
        "q": normal((B, w.hq, w.d_qk) if w.q_len == 1 else (B, w.hq, w.q_len, w.d_qk), s, 0),
        "k": normal_e4m3((P, w.hkv, ps, w.d_qk), s, 1, FP8_KV_SCALE) if w.kv_fp8 else normal((P, w.hkv, ps, w.d_qk), s, 1),
        "v": normal_e4m3((P, w.hkv, ps, w.d_v), s, 2, FP8_KV_SCALE) if w.kv_fp8 else normal((P, w.hkv, ps, w.d_v), s, 2),
        "kv_scales": (FP8_KV_SCALE, FP8_KV_SCALE) if w.kv_fp8 else None,
        "block_table": page_table(B, max_pages, P, s, permute),
        "seq_lens": np.full(B, n, dtype=np.int32),
        "sink": sink_values(w.hq, s),
    }


def ring_from_sequence(k_seq: np.ndarray, v_seq: np.ndarray, n: int, window: int):
    """Build ring caches [B,Hkv,W,d] from contiguous [B,Hkv,>=n,d] sequences holding
    positions 0..n-1: slot p mod W holds position p for the last min(n, W) positions;
    unused slots are zero."""
    B, H, _, dk = k_seq.shape
    dv = v_seq.shape[-1]
    kr = np.zeros((B, H, window, dk), k_seq.dtype)
    vr = np.zeros((B, H, window, dv), v_seq.dtype)
    for p in range(max(0, n - window), n):
        kr[:, :, p % window] = k_seq[:, :, p]
        vr[:, :, p % window] = v_seq[:, :, p]
    return kr, vr


def pages_from_sequence(k_seq: np.ndarray, v_seq: np.ndarray, n: int, page_size: int,
                        num_pages: int, seed: int, permute: bool = True):
    """Scatter contiguous [B,Hkv,>=n,d] sequences into a page pool [P,Hkv,page,d] through a
    (permuted) block table; returns (k_pool, v_pool, block_table). Unused slots are zero."""
    B, H, _, dk = k_seq.shape
    dv = v_seq.shape[-1]
    max_pages = (n + page_size - 1) // page_size
    bt = page_table(B, max_pages, num_pages, seed, permute)
    kp = np.zeros((num_pages, H, page_size, dk), k_seq.dtype)
    vp = np.zeros((num_pages, H, page_size, dv), v_seq.dtype)
    for b in range(B):
        for pg in range(max_pages):
            lo = pg * page_size
            hi = min(n, lo + page_size)
            kp[bt[b, pg], :, : hi - lo] = k_seq[b, :, lo:hi]
            vp[bt[b, pg], :, : hi - lo] = v_seq[b, :, lo:hi]
    return kp, vp, bt
