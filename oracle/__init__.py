"""CPU oracle for sink attention.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The library (attention_sink_softmax_amd) never does, and this package never
imports the library: the two share no code.  The arithmetic lives in oracle.c (fp64,
plain loops, OpenMP over output rows) and, for tiny brute-force checks, oracle_np.py.

Parity status: every function here, the E4M3 encoder included, is pinned by
tests/test_oracle_pins.py against the
worked example of the paper-notes page (§4.3), torch's CPU scaled_dot_product_attention
in float64, closed forms and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

GLOBAL = 0
SWA = 1
RING = 0
PAGED = 1
F32 = 0
BF16 = 1

_lib = None


def build(src: str = SRC, out: str = LIB, extra: tuple = ()) -> str:
    """Compile oracle.c with gcc (-O2, OpenMP) into a shared library."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str = LIB):
    """Load (building first if absent) the compiled oracle and declare its signatures."""
    global _lib
    if path == LIB and _lib is not None:
        return _lib
    if not os.path.exists(path) or (path == LIB and os.path.getmtime(path) < os.path.getmtime(SRC)):
        build(out=path)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_prefill.restype = I
    lib.oracle_prefill.argtypes = [I, I, I, I, I, I, I, I, ctypes.c_double, I, P, P, P, P,
                                   ctypes.c_int64, P, P]
    lib.oracle_prefill_chunk.restype = I
    lib.oracle_prefill_chunk.argtypes = [I, I, I, I, I, I, I, I, I, ctypes.c_double, I, P, P, P, P, ctypes.c_int64, P,
                                         P, P]
    lib.oracle_decode_fp8.restype = I
    lib.oracle_decode_fp8.argtypes = [I, I, I, I, I, I, I, I, I, ctypes.c_double, I, P, P, P, ctypes.c_double,
                                      ctypes.c_double, P, I, I, I, P, P, P, P]
    lib.oracle_prefill_backward.restype = I
    lib.oracle_prefill_backward.argtypes = [I, I, I, I, I, I, I, I, ctypes.c_double, I, P, P, P, P, P, P, P, P, P]
    lib.oracle_prefill_backward_sampled.restype = I
    lib.oracle_prefill_backward_sampled.argtypes = [I, I, I, I, I, I, I, I, ctypes.c_double, I, P, P, P, P, P, I, P, P,
                                                    I, P, P, P]
    lib.oracle_rope.restype = I
    lib.oracle_rope.argtypes = [ctypes.c_int64, I, I, ctypes.c_double, I, P, P, P]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
    lib.oracle_e4m3_encode.restype = I
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_int64, P, ctypes.c_double, P]
    lib.oracle_decode.restype = I
    lib.oracle_decode.argtypes = [I, I, I, I, I, I, I, I, I, ctypes.c_double, I, P, P, P, P, I, I, I,
                                  P, P, P, P]
    lib.oracle_decode_side.restype = I
    lib.oracle_decode_side.argtypes = [I, I, I, I, I, I, I, I, I, ctypes.c_double, I, P, P, P, P, I, I, I,
                                       P, P, P, P, P, P]
    lib.oracle_threads.restype = I
    lib.oracle_threads.argtypes = []
    if path == LIB:
        _lib = lib
    return lib


def _arr(x, dtype):
    """Contiguous array and its storage flag: uint16 -> bf16 bits, else float32."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), BF16
    return np.ascontiguousarray(x, dtype=np.float32), F32


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def prefill(q, k, v, sink, mode: int, window: int, scale: float, rows=None, lib=None) -> np.ndarray:
    """q [B,Hq,L,dqk], k [B,Hkv,L,dqk], v [B,Hkv,L,dv]: all float32, or all uint16 bf16 bits.
    sink: [Hq] floats or None.  rows: optional int array [n,3] of (b, h, i).
    Returns float64 [B,Hq,L,dv] (rows None) or [n,dv]."""
    lib = lib or load()
    qa, dt = _arr(q, None)
    ka, dt2 = _arr(k, None)
    va, dt3 = _arr(v, None)
    if not (dt == dt2 == dt3):
        raise TypeError("q, k, v must share one storage type")
    B, Hq, L, dqk = qa.shape
    Hkv, dv = ka.shape[1], va.shape[3]
    if ka.shape != (B, Hkv, L, dqk) or va.shape != (B, Hkv, L, dv):
        raise ValueError("shape mismatch")
    s = None if sink is None else np.ascontiguousarray(sink, dtype=np.float64)
    if rows is None:
        out = np.empty((B, Hq, L, dv), np.float64)
        n, rp = 0, None
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        out = np.empty((r.shape[0], dv), np.float64)
        n, rp = r.shape[0], r
    rc = lib.oracle_prefill(mode, window, B, L, Hq, Hkv, dqk, dv, scale, dt, _ptr(qa), _ptr(ka),
                            _ptr(va), _ptr(s), n, _ptr(rp), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    return out


def prefill_chunk(q, k, v, sink, mode: int, window: int, scale: float, rows=None, lib=None, return_lse=False):
    """Chunked prefill: q [B,Hq,Lq,dqk] holds positions Lk-Lq .. Lk-1 of sequences whose keys
    and values k [B,Hkv,Lk,dqk], v [B,Hkv,Lk,dv] cover positions 0 .. Lk-1.  rows: optional
    (b, h, r) triplets (r = chunk row).  Returns float64 [B,Hq,Lq,dv] or [nrows,dv], and with
    return_lse also each row's log-sum-exp ([B,Hq,Lq] or [nrows])."""
    lib = lib or load()
    qa, dt = _arr(q, None)
    ka, _ = _arr(k, None)
    va, _ = _arr(v, None)
    B, Hq, Lq, dqk = qa.shape
    Hkv, Lk, dv = ka.shape[1], ka.shape[2], va.shape[3]
    s = None if sink is None else np.ascontiguousarray(sink, dtype=np.float64)
    if rows is None:
        rp, n = None, 0
        out = np.empty((B, Hq, Lq, dv), np.float64)
    else:
        rp = np.ascontiguousarray(rows, dtype=np.int64)
        n = rp.shape[0]
        out = np.empty((n, dv), np.float64)
    lse = np.empty(out.shape[:-1], np.float64)
    rc = lib.oracle_prefill_chunk(mode, window, B, Lq, Lk, Hq, Hkv, dqk, dv, scale, dt, _ptr(qa), _ptr(ka), _ptr(va),
                                  _ptr(s), n, _ptr(rp), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_prefill_chunk rejected its arguments")
    return (out, lse) if return_lse else out


def decode(q, k, v, seq_lens, sink, mode: int, window: int, scale: float, layout: int,
           block_table=None, lib=None, kv_scales=None, return_lse=False, k_new=None, v_new=None):
    """q [B,Hq,dqk] (one new token per sequence) or [B,Hq,q_len,dqk] (q_len new tokens at
    positions seq_lens-q_len .. seq_lens-1); RING: k [B,Hkv,W,dqk], v [B,Hkv,W,dv];
    PAGED: k [P,Hkv,page,dqk], v [P,Hkv,page,dv] with block_table [B,max_pages].
    Returns float64 [B,Hq,dv] or [B,Hq,q_len,dv], matching q.
    uint8 k and v are E4M3 codes of an 8-bit cache; kv_scales = (k_scale, v_scale) then
    gives the per-tensor scales (element = scale * code value).  With return_lse also each
    row's log-sum-exp, shaped like the output without its last axis.
    k_new [B,Hkv,q_len,dqk], v_new [B,Hkv,q_len,dv] (same dtype as q): the new tokens' keys and
    values held beside the cache, which then holds the positions before seq_lens - q_len only
    (RING caches too, any q_len)."""
    lib = lib or load()
    qa, dt = _arr(q, None)
    fp8 = np.asarray(k).dtype == np.uint8
    if fp8:
        ka = np.ascontiguousarray(k, dtype=np.uint8)
        va = np.ascontiguousarray(v, dtype=np.uint8)
    else:
        ka, _ = _arr(k, None)
        va, _ = _arr(v, None)
    B, Hq, dqk = qa.shape[0], qa.shape[1], qa.shape[-1]
    q_len = qa.shape[2] if qa.ndim == 4 else 1
    Hkv, dv = ka.shape[1], va.shape[3]
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    s = None if sink is None else np.ascontiguousarray(sink, dtype=np.float64)
    if layout == PAGED:
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        ps, mp, npg = ka.shape[2], bt.shape[1], ka.shape[0]
    else:
        bt, ps, mp, npg = None, 0, 0, 0
    out = np.empty(qa.shape[:-1] + (dv,), np.float64)
    lse = np.empty(out.shape[:-1], np.float64)
    if k_new is not None:
        if fp8:
            raise TypeError("keys beside the cache need a cache of the queries' dtype")
        kn, dtk = _arr(k_new, None)
        vn, dtv = _arr(v_new, None)
        if not (dtk == dtv == dt) or kn.shape != (B, Hkv, q_len, dqk) or vn.shape != (B, Hkv, q_len, dv):
            raise ValueError("k_new / v_new must be [B,Hkv,q_len,d] in the queries' dtype")
        rc = lib.oracle_decode_side(mode, window, layout, B, Hq, Hkv, dqk, dv, q_len, scale, dt, _ptr(qa), _ptr(ka),
                                    _ptr(va), _ptr(bt), ps, mp, npg, _ptr(lens), _ptr(kn), _ptr(vn), _ptr(s),
                                    _ptr(out), _ptr(lse))
    elif fp8:
        ks, vs = kv_scales if kv_scales is not None else (1.0, 1.0)
        rc = lib.oracle_decode_fp8(mode, window, layout, B, Hq, Hkv, dqk, dv, q_len, scale, dt, _ptr(qa), _ptr(ka),
                                   _ptr(va), ks, vs, _ptr(bt), ps, mp, npg, _ptr(lens), _ptr(s), _ptr(out),
                                   _ptr(lse))
    else:
        rc = lib.oracle_decode(mode, window, layout, B, Hq, Hkv, dqk, dv, q_len, scale, dt, _ptr(qa), _ptr(ka),
                               _ptr(va), _ptr(bt), ps, mp, npg, _ptr(lens), _ptr(s), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return (out, lse) if return_lse else out


def prefill_cached(q, k_chunk, v_chunk, k_cache, v_cache, kv_lens, sink, mode: int, window: int, scale: float,
                   layout: int, block_table=None, lib=None, return_lse=False):
    """Chunked prefill over a cached prefix: q [B,Hq,Lq,dqk] are positions kv_lens[b] - Lq ..
    kv_lens[b] - 1 of each sequence, k_chunk [B,Hkv,Lq,dqk] and v_chunk [B,Hkv,Lq,dv] their keys
    and values; the prefix (positions before kv_lens - Lq) is read from a RING (sliding mode,
    its last `window` positions) or a PAGED cache.  The same definition as decode with the new
    tokens beside the cache, with Lq new tokens (oracle_decode_side)."""
    return decode(q, k_cache, v_cache, kv_lens, sink, mode, window, scale, layout, block_table, lib=lib,
                  return_lse=return_lse, k_new=k_chunk, v_new=v_chunk)


def prefill_backward(q, k, v, sink, dout, mode: int, window: int, scale: float, lib=None):
    """Gradients of prefill attention: q [B,Hq,L,dqk], k, v [B,Hkv,L,.], sink [Hq] or None,
    dout [B,Hq,L,dv] (same dtype as q).  Returns float64 (dq, dk, dv, dsink or None)."""
    lib = lib or load()
    qa, dt = _arr(q, None)
    ka, _ = _arr(k, None)
    va, _ = _arr(v, None)
    da, _ = _arr(dout, None)
    B, Hq, L, dqk = qa.shape
    Hkv, dv = ka.shape[1], va.shape[3]
    s = None if sink is None else np.ascontiguousarray(sink, dtype=np.float64)
    dq = np.empty(qa.shape, np.float64)
    dk = np.empty(ka.shape, np.float64)
    dvv = np.empty(va.shape, np.float64)
    ds = None if sink is None else np.empty(Hq, np.float64)
    rc = lib.oracle_prefill_backward(mode, window, B, L, Hq, Hkv, dqk, dv, scale, dt, _ptr(qa), _ptr(ka), _ptr(va),
                                     _ptr(s), _ptr(da), _ptr(dq), _ptr(dk), _ptr(dvv), _ptr(ds))
    if rc != 0:
        raise ValueError("oracle_prefill_backward rejected its arguments")
    return dq, dk, dvv, ds


def prefill_backward_sampled(q, k, v, sink, dout, mode: int, window: int, scale: float, qrows, krows, lib=None):
    """Entries of the prefill gradients of a large problem, by the same definitions as
    prefill_backward: dq of the rows qrows [(b, h, i), ...] and dk, dv of the keys
    krows [(b, KV head, j), ...].  Returns float64 (dq [nq, dqk], dk [nk, dqk], dv [nk, dv])."""
    lib = lib or load()
    qa, dt = _arr(q, None)
    ka, _ = _arr(k, None)
    va, _ = _arr(v, None)
    da, _ = _arr(dout, None)
    B, Hq, L, dqk = qa.shape
    Hkv, dv = ka.shape[1], va.shape[3]
    s = None if sink is None else np.ascontiguousarray(sink, dtype=np.float64)
    qr = np.ascontiguousarray(np.asarray(qrows, np.int64).reshape(-1, 3))
    kr = np.ascontiguousarray(np.asarray(krows, np.int64).reshape(-1, 3))
    dq = np.empty((qr.shape[0], dqk), np.float64)
    dk = np.empty((kr.shape[0], dqk), np.float64)
    dvv = np.empty((kr.shape[0], dv), np.float64)
    rc = lib.oracle_prefill_backward_sampled(mode, window, B, L, Hq, Hkv, dqk, dv, scale, dt, _ptr(qa), _ptr(ka),
                                             _ptr(va), _ptr(s), _ptr(da), qr.shape[0], _ptr(qr), _ptr(dq),
                                             kr.shape[0], _ptr(kr), _ptr(dk), _ptr(dvv))
    if rc != 0:
        raise ValueError("oracle_prefill_backward_sampled rejected its arguments")
    return dq, dk, dvv


SWA_ROPE_THETA = 10000.0     # sliding-window layers (deep-dive CH 3.5)
GA_ROPE_THETA = 5000000.0    # global layers
ROPE_DIMS = 64               # rotated leading dimensions of the 192 (partial_rotary_factor 0.334)


def rope(x, positions, theta: float, rot: int = ROPE_DIMS, lib=None) -> np.ndarray:
    """Partial RoPE of x [..., dim] (uint16 bf16 bits or float) at integer positions shaped like
    x without its last axis.  Returns float64 like x."""
    lib = lib or load()
    xa, dt = _arr(x, None)
    pa = np.ascontiguousarray(np.broadcast_to(np.asarray(positions, np.int64), xa.shape[:-1]))
    out = np.empty(xa.shape, np.float64)
    rows = int(np.prod(xa.shape[:-1]))
    if lib.oracle_rope(rows, xa.shape[-1], rot, theta, dt, _ptr(xa), _ptr(pa), _ptr(out)) != 0:
        raise ValueError("oracle_rope rejected its arguments")
    return out


def e4m3_encode(x, scale: float, lib=None) -> np.ndarray:
    """E4M3 codes (uint8, shaped like x) of x / scale, by oracle.c's encoder: the quotient in
    float32, clamped to +-448, rounded to the nearest code with ties to even, the sign kept.
    x: float32, or uint16 bf16 bits (widened to float32 exactly)."""
    lib = lib or load()
    xa = np.asarray(x)
    if xa.dtype == np.uint16:
        xa = (xa.astype(np.uint32) << np.uint32(16)).view(np.float32)
    xa = np.ascontiguousarray(xa, dtype=np.float32)
    out = np.empty(xa.shape, np.uint8)
    if lib.oracle_e4m3_encode(xa.size, _ptr(xa), float(scale), _ptr(out)) != 0:
        raise ValueError("oracle_e4m3_encode rejected its arguments")
    return out


def kv_append(k_cache, v_cache, layout: int, k_new, v_new, seq_lens, window: int = 0, block_table=None,
              fp8_scales=None, lib=None):
    """Write n new tokens per sequence into a cache (in place): token t of sequence b, at
    position seq_lens[b] - n + t, goes to ring slot pos mod window (the last `window`
    positions only) or to page block_table[b][pos // page] at offset pos mod page.
    k_new [B,Hkv,n,dqk], v_new [B,Hkv,n,dv]; positions below 0 and page ids outside the pool
    are skipped.  Plain indexing; with fp8_scales = (k_scale, v_scale) the caches hold E4M3
    codes and the new rows are encoded by e4m3_encode first."""
    if fp8_scales is not None:
        k_new, v_new = e4m3_encode(k_new, fp8_scales[0], lib), e4m3_encode(v_new, fp8_scales[1], lib)
    B, Hkv, n = k_new.shape[:3]
    for b in range(B):
        for t in range(n):
            pos = int(seq_lens[b]) - n + t
            if pos < 0:
                continue
            if layout == RING:
                if pos < int(seq_lens[b]) - window:
                    continue
                k_cache[b, :, pos % window] = k_new[b, :, t]
                v_cache[b, :, pos % window] = v_new[b, :, t]
            else:
                ps = k_cache.shape[2]
                page = int(block_table[b, pos // ps])
                if not 0 <= page < k_cache.shape[0]:
                    continue
                k_cache[page, :, pos % ps] = k_new[b, :, t]
                v_cache[page, :, pos % ps] = v_new[b, :, t]


def e4m3_value(code: int, lib=None) -> float:
    return (lib or load()).oracle_e4m3_value(code)


def threads() -> int:
    return load().oracle_threads()
