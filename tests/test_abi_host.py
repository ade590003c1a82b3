"""The C-ABI library on the host: it loads, exports what include/sinkattn.h declares, plans
the decode workspace, and rejects bad arguments before touching any device.

No call here reaches a kernel launch: every call has an argument error that the host-side
checks report first (pointer values are never dereferenced by those checks)."""
import ctypes
import os
import re

import pytest

import attention_sink_softmax_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sinkattn.h")

OK, E_NULL, E_SHAPE, E_UNSUP, E_ALIGN, E_WS = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def L():
    test_lib = os.environ.get("SINKATTN_TEST_LIB")  # a differently built library (the sanitizer run)
    if test_lib:
        sa._lib = sa.lib(test_lib)
        return sa._lib
    if not os.path.exists(sa.LIB_PATH):
        from attention_sink_softmax_amd import build
        build.build()
    return sa.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*\s*|size_t\s+|int\s+)(sinkattn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(sa.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(7):
        assert sa.sinkattn_status_string(s)
    assert sa.sinkattn_status_string(99) == "unknown status"


def dims(B=1, Lq=64, hq=64, hkv=8, dqk=192, dv=128, scale=192 ** -0.5):
    return sa.Dims(B, Lq, hq, hkv, dqk, dv, scale)


A = 0x10000  # a 16-byte aligned fake address (never dereferenced)


def prefill(L, mode=1, window=128, d=None, q=A, k=A, v=A, sink=None, out=A, ws=A, wsb=1 << 40):
    d = d or dims()
    return L.sinkattn_prefill(mode, window, ctypes.byref(d), q, k, v, sink, out, ws, wsb, None)


def test_prefill_argument_errors(L):
    assert L.sinkattn_prefill(1, 128, None, A, A, A, None, A, A, 1 << 40, None) == E_NULL
    assert prefill(L, mode=2) == E_UNSUP
    assert prefill(L, d=dims(dqk=128)) == E_UNSUP
    assert prefill(L, d=dims(dv=192)) == E_UNSUP
    assert prefill(L, d=dims(hq=64, hkv=6)) == E_SHAPE
    assert prefill(L, d=dims(hkv=0)) == E_SHAPE
    assert prefill(L, d=dims(B=-1)) == E_SHAPE
    assert prefill(L, d=dims(Lq=-1)) == E_SHAPE
    assert prefill(L, mode=1, window=0) == E_SHAPE
    assert prefill(L, d=dims(scale=float("nan"))) == E_SHAPE
    assert prefill(L, q=None) == E_NULL
    assert prefill(L, out=None) == E_NULL
    assert prefill(L, k=A + 8) == E_ALIGN
    assert prefill(L, sink=A + 4) == E_ALIGN
    assert prefill(L, ws=None) == E_WS
    assert prefill(L, wsb=1000) == E_WS
    assert prefill(L, ws=A + 8) == E_ALIGN
    assert prefill(L, d=dims(scale=-0.1)) == E_SHAPE
    assert prefill(L, d=dims(scale=0.0)) == E_SHAPE
    assert prefill(L, d=dims(Lq=6_000_000)) == E_SHAPE  # 32-bit row offsets
    # empty work is a no-op success, even with NULL tensors
    assert prefill(L, d=dims(Lq=0), q=None, k=None, v=None, out=None) == OK
    assert prefill(L, d=dims(B=0), q=None, k=None, v=None, out=None) == OK


def kv(layout=1, k=A, v=A, bt=A, ps=64, mp=4096, npg=32768):
    return sa.KVDesc(layout, k, v, bt, ps, mp, npg)


def decode(L, mode=0, window=0, d=None, q=A, desc=None, lens=A, maxlen=262144, sink=None, out=A, ws=A,
           wsb=1 << 30):
    d = d or dims(B=8, hq=64, hkv=4)
    desc = desc if desc is not None else kv()
    return L.sinkattn_decode(mode, window, ctypes.byref(d), q, ctypes.byref(desc), lens, maxlen, sink, out, ws, wsb,
                             None)


def test_decode_argument_errors(L):
    assert decode(L, desc=kv(layout=0)) == E_UNSUP          # ring needs sliding mode
    assert decode(L, desc=kv(layout=5)) == E_UNSUP
    assert decode(L, maxlen=0) == E_SHAPE
    assert decode(L, maxlen=262145) == E_SHAPE              # beyond max_pages * page_size
    assert decode(L, desc=kv(ps=0)) == E_SHAPE
    assert decode(L, desc=kv(npg=0)) == E_SHAPE
    assert decode(L, q=None) == E_NULL
    assert decode(L, lens=None) == E_NULL
    assert decode(L, desc=kv(bt=None)) == E_NULL
    assert decode(L, desc=kv(k=None)) == E_NULL
    assert decode(L, out=A + 2) == E_ALIGN
    assert decode(L, desc=kv(bt=A + 4)) == E_ALIGN
    assert decode(L, ws=None) == E_WS
    assert decode(L, wsb=100) == E_WS
    assert decode(L, ws=A + 8) == E_ALIGN
    assert decode(L, d=dims(B=8, hq=64, hkv=4, dqk=64)) == E_UNSUP
    assert decode(L, mode=1, window=0, desc=kv(layout=0)) == E_SHAPE
    assert L.sinkattn_decode(0, 0, ctypes.byref(dims()), A, None, A, 1, None, A, A, 0, None) == E_NULL
    # batch 0 is a no-op
    assert decode(L, d=dims(B=0, hq=64, hkv=4), q=None, out=None) == OK


def decode_multi(L, q_len=4, mode=0, window=0, d=None, q=A, desc=None, lens=A, maxlen=262144, sink=None, out=A,
                 ws=A, wsb=1 << 30):
    d = d or dims(B=8, hq=64, hkv=4)
    desc = desc if desc is not None else kv()
    return L.sinkattn_decode_multi(mode, window, ctypes.byref(d), q_len, q, ctypes.byref(desc), lens, maxlen, sink,
                                   out, ws, wsb, None)


def test_decode_multi_argument_errors(L):
    assert decode_multi(L, q_len=0) == E_SHAPE
    assert decode_multi(L, q_len=-3) == E_SHAPE
    assert decode_multi(L, q_len=257) == E_SHAPE
    # a ring keeps only the last W keys, which the earlier drafted tokens would need to go past
    assert decode_multi(L, q_len=2, mode=1, window=128, desc=kv(layout=0)) == E_UNSUP
    assert decode_multi(L, q_len=1, mode=0, desc=kv(layout=0)) == E_UNSUP
    assert decode_multi(L, maxlen=262145) == E_SHAPE
    assert decode_multi(L, q=None) == E_NULL
    assert decode_multi(L, out=A + 2) == E_ALIGN
    assert decode_multi(L, ws=None) == E_WS
    assert decode_multi(L, wsb=100) == E_WS
    assert L.sinkattn_decode_multi(0, 0, ctypes.byref(dims()), 4, A, None, A, 1, None, A, A, 0, None) == E_NULL
    assert decode_multi(L, d=dims(B=0, hq=64, hkv=4), q=None, out=None) == OK


def test_decode_multi_workspace_plan(L):
    # q_len = 1 plans exactly as one-token decode
    for args in ((0, 0, 8, 64, 4, 262144), (1, 128, 128, 64, 8, 65536), (0, 0, 1, 64, 4, 5000)):
        assert sa.sinkattn_decode_multi_workspace_bytes(*args[:5], 1, args[5]) == \
            sa.sinkattn_decode_workspace_bytes(*args)
    # 256K global, four drafted tokens: one workgroup covers all 16 heads x 4 tokens of a KV
    # head, so the split is the same 16 x 16384 keys (512 workgroups) and the partials grow
    # by q_len
    assert sa.sinkattn_decode_multi_workspace_bytes(0, 0, 8, 64, 4, 4, 262144) == 8 * 64 * 4 * 16 * 132 * 4
    assert sa.sinkattn_decode_multi_workspace_bytes(1, 128, 128, 64, 8, 4, 65536) == 0
    with pytest.raises(sa.SinkAttnError):
        sa.sinkattn_decode_multi_workspace_bytes(0, 0, 8, 64, 4, 0, 262144)
    with pytest.raises(sa.SinkAttnError):
        sa.sinkattn_decode_multi_workspace_bytes(0, 0, 8, 64, 4, 257, 262144)


def test_prefill_chunk_argument_errors(L):
    def chunk(kv_len, d=None, ws=A, wsb=1 << 40, q=A):
        d = d or dims(Lq=64)
        return L.sinkattn_prefill_chunk(1, 128, ctypes.byref(d), kv_len, q, A, A, None, A, ws, wsb, None)
    assert chunk(63) == E_SHAPE                   # fewer keys than new tokens
    assert chunk(6_000_000) == E_SHAPE            # 32-bit row offsets over the keys
    assert chunk(100_000, wsb=1000) == E_WS       # the V^T copy covers every key
    assert chunk(100_000, q=None) == E_NULL
    assert chunk(100_000, d=dims(Lq=0), q=None) == OK
    assert L.sinkattn_prefill_chunk(1, 128, None, 10, A, A, A, None, A, A, 1 << 40, None) == E_NULL


def test_prefill_chunk_workspace_size(L):
    assert sa.sinkattn_prefill_chunk_workspace_bytes(1, 16384, 64, 4, 32768) == 4 * 128 * 32768 * 2
    assert sa.sinkattn_prefill_chunk_workspace_bytes(2, 1, 4, 1, 65) == 2 * 128 * 128 * 2
    assert sa.sinkattn_prefill_chunk_workspace_bytes(1, 100, 4, 1, 100) == sa.sinkattn_prefill_workspace_bytes(1, 100, 4, 1)
    with pytest.raises(sa.SinkAttnError):
        sa.sinkattn_prefill_chunk_workspace_bytes(1, 101, 4, 1, 100)


def test_decode_fp8_argument_errors(L):
    def fp8(desc=None, ks=0.5, vs=0.5, q=A):
        d = dims(B=8, hq=64, hkv=4)
        desc = desc if desc is not None else kv()
        return L.sinkattn_decode_fp8(0, 0, ctypes.byref(d), 1, q, ctypes.byref(desc), A, 262144, None, ks, vs, A, A,
                                     1 << 30, None)
    assert fp8(desc=kv(layout=0)) == E_UNSUP               # paged caches only
    assert fp8(desc=kv(ps=48, mp=6000)) == E_UNSUP        # pages of a multiple of 32 keys
    assert fp8(ks=0.0) == E_SHAPE
    assert fp8(vs=-1.0) == E_SHAPE
    assert fp8(ks=float("nan")) == E_SHAPE
    assert fp8(ks=float("inf")) == E_SHAPE
    assert fp8(q=None) == E_NULL
    assert L.sinkattn_decode_fp8(0, 0, ctypes.byref(dims()), 1, A, None, A, 1, None, 1.0, 1.0, A, A, 0, None) == E_NULL


def test_rope_argument_errors(L):
    assert L.sinkattn_rope(0.0, 1, 64, 10, A, None, 0, None) == E_SHAPE
    assert L.sinkattn_rope(float("inf"), 1, 64, 10, A, None, 0, None) == E_SHAPE
    assert L.sinkattn_rope(1e4, -1, 64, 10, A, None, 0, None) == E_SHAPE
    assert L.sinkattn_rope(1e4, 1, 64, 10, None, None, 0, None) == E_NULL
    assert L.sinkattn_rope(1e4, 1, 64, 10, A + 2, None, 0, None) == E_ALIGN
    assert L.sinkattn_rope(1e4, 1, 64, 0, None, None, 0, None) == OK


def test_kv_append_argument_errors(L):
    def app(desc=None, window=128, n=1, fp8=0, ks=1.0, vs=1.0, kn=A, lens=A):
        desc = desc if desc is not None else kv()
        return L.sinkattn_kv_append(ctypes.byref(desc), window, 2, 4, n, kn, A, lens, fp8, ks, vs, None)
    assert L.sinkattn_kv_append(None, 128, 1, 4, 1, A, A, A, 0, 1.0, 1.0, None) == E_NULL
    assert app(desc=kv(layout=7)) == E_UNSUP
    assert app(desc=kv(layout=0), window=0) == E_SHAPE
    assert app(desc=kv(ps=0)) == E_SHAPE
    assert app(fp8=1, ks=0.0) == E_SHAPE
    assert app(kn=None) == E_NULL
    assert app(lens=None) == E_NULL
    assert app(desc=kv(bt=None)) == E_NULL
    assert app(kn=A + 8) == E_ALIGN
    assert app(n=0, kn=None) == OK


def test_epilogue_argument_errors(L):
    ep = sa.Epilogue(float("nan"), None)
    d = dims(Lq=64)
    assert L.sinkattn_prefill_ex(1, 128, ctypes.byref(d), 64, A, A, A, None, ctypes.byref(ep), A, A, 1 << 40,
                                 None) == E_SHAPE
    ep = sa.Epilogue(0.7, A + 2)
    assert L.sinkattn_prefill_ex(1, 128, ctypes.byref(d), 64, A, A, A, None, ctypes.byref(ep), A, A, 1 << 40,
                                 None) == E_ALIGN
    d2 = dims(B=8, hq=64, hkv=4)
    desc = kv()
    ep = sa.Epilogue(float("inf"), None)
    assert L.sinkattn_decode_ex(0, 0, ctypes.byref(d2), 1, A, ctypes.byref(desc), 0, 1.0, 1.0, A, 262144, None,
                                ctypes.byref(ep), A, A, 1 << 30, None) == E_SHAPE
    ep = sa.Epilogue(0.707, A + 4)  # 4-byte aligned lse is fine; the null q is reported next
    assert L.sinkattn_decode_ex(0, 0, ctypes.byref(d2), 1, None, ctypes.byref(desc), 0, 1.0, 1.0, A, 262144, None,
                                ctypes.byref(ep), A, A, 1 << 30, None) == E_NULL
    assert L.sinkattn_decode_ex(0, 0, ctypes.byref(d2), 1, A, ctypes.byref(desc), 1, 0.0, 1.0, A, 262144, None,
                                None, A, A, 1 << 30, None) == E_SHAPE


def test_prefill_workspace_size(L):
    # a transposed copy of V, rows padded to 64 keys
    assert sa.sinkattn_prefill_workspace_bytes(1, 32768, 64, 8) == 8 * 128 * 32768 * 2
    assert sa.sinkattn_prefill_workspace_bytes(2, 65, 4, 1) == 2 * 128 * 128 * 2
    assert sa.sinkattn_prefill_workspace_bytes(1, 0, 4, 1) == 0


def test_decode_workspace_plan(L):
    # 256K global decode: 8 sequences x 4 KV heads, split into 16 pieces of 16384 keys (512
    # workgroups)
    n = sa.sinkattn_decode_workspace_bytes(0, 0, 8, 64, 4, 262144)
    assert n == 8 * 64 * 16 * 132 * 4
    # a split never exceeds 16384 keys (the kernel holds the page ids of at most 128 slices per
    # wave): more sequences keep 16 splits of 16384 keys rather than longer splits
    for B in (16, 64):
        assert sa.sinkattn_decode_workspace_bytes(0, 0, B, 64, 4, 262144) == B * 64 * 16 * 132 * 4
    # few (sequence, KV head) pairs: short splits, here 512 of 512 keys
    assert sa.sinkattn_decode_workspace_bytes(0, 0, 1, 16, 1, 262144) == 16 * 512 * 132 * 4
    # sliding ring decode: one split per (sequence, KV head), no workspace
    assert sa.sinkattn_decode_workspace_bytes(1, 128, 128, 64, 8, 65536) == 0
    assert sa.sinkattn_decode_workspace_bytes(1, 128, 1, 64, 8, 100) == 0
    # short global context: single split
    assert sa.sinkattn_decode_workspace_bytes(0, 0, 1, 64, 4, 100) == 0
    with pytest.raises(sa.SinkAttnError):
        sa.sinkattn_decode_workspace_bytes(0, 0, 1, 64, 3, 100)
    with pytest.raises(sa.SinkAttnError):
        sa.sinkattn_decode_workspace_bytes(0, 0, 1, 64, 4, 0)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(sa.LibraryMissing):
        sa.lib(str(tmp_path / "nope.so"))


def backward(L, mode=0, window=0, d=None, q=A, k=A, v=A, sink=None, out=A, dout=A, lse=A, dq=A, dk=A, dv=A,
             dsink=None, ws=A, wsb=1 << 40):
    d = d or dims(hq=64, hkv=4)
    return L.sinkattn_prefill_backward(mode, window, ctypes.byref(d), q, k, v, sink, out, dout, lse, dq, dk, dv, dsink,
                                       ws, wsb, None)


def test_backward_argument_errors(L):
    d = dims(hq=64, hkv=4)
    need = L.sinkattn_prefill_backward_workspace_bytes(ctypes.byref(d))
    assert need == 4 * (2 * 64 * 64 + 64 * ((64 + 15) // 16))  # D and -LSE log2(e) per row + sink-gradient partials
    # empty work is a no-op success, even with NULL tensors
    assert backward(L, d=dims(B=0, hq=64, hkv=4), q=None, k=None, v=None, out=None, dout=None, lse=None, dq=None,
                    dk=None, dv=None, ws=None, wsb=0) == OK
    assert backward(L, d=dims(hq=64, hkv=4, dqk=128)) == E_UNSUP        # head size
    assert backward(L, d=dims(hq=12, hkv=4)) == E_UNSUP                 # group of 3: not a multiple of 4
    assert backward(L, d=dims(hq=64, hkv=5)) == E_SHAPE                 # 64 % 5
    assert backward(L, mode=1, window=0) == E_SHAPE                     # window 0
    assert backward(L, q=None) == E_NULL
    assert backward(L, lse=None) == E_NULL
    assert backward(L, sink=A, dsink=None) == E_NULL                    # a sink needs its gradient
    assert backward(L, dq=A + 4) == E_ALIGN
    assert backward(L, sink=A, dsink=A + 8) == E_ALIGN
    assert backward(L, ws=None) == E_WS
    assert backward(L, wsb=need - 1) == E_WS


def test_decode_verify_argument_errors(L):
    def ver(mode=1, window=128, desc=None, q_len=4, kn=A, vn=A, ml=65536):
        d = dims(B=128, hq=64, hkv=8)
        desc = desc if desc is not None else kv(layout=0, bt=None)
        return L.sinkattn_decode_verify(mode, window, ctypes.byref(d), q_len, A, ctypes.byref(desc), kn, vn, A, ml,
                                        None, None, A, A, 1 << 30, None)
    assert ver(kn=None) == E_NULL
    assert ver(vn=None) == E_NULL
    assert ver(mode=0, window=0) == E_UNSUP           # a ring in global mode
    assert ver(q_len=0) == E_SHAPE
    assert ver(q_len=257) == E_SHAPE
    assert ver(kn=A + 4) == E_ALIGN
    assert ver(desc=kv(layout=1, ps=64, mp=2)) == E_SHAPE   # the table must cover the committed positions
    # pages covering the committed positions only (the drafts are beside the cache): accepted
    # as far as the host checks go (the workspace is too small, so nothing is launched)
    d = dims(B=8, hq=64, hkv=4)
    desc = kv(layout=1, ps=64, mp=4096)
    assert L.sinkattn_decode_verify(0, 0, ctypes.byref(d), 4, A, ctypes.byref(desc), A, A, A, 262144 + 4, None, None,
                                    A, A, 0, None) == E_WS


def test_prefill_cached_argument_errors(L):
    def cached(mode=0, window=0, kv_len=1000, desc=None, d=None, ws=A, wsb=1 << 40, q=A):
        d = d or dims(Lq=300, hq=64, hkv=4)
        desc = desc if desc is not None else kv(layout=1, ps=64, mp=16)
        return L.sinkattn_prefill_cached(mode, window, ctypes.byref(d), kv_len, q, A, A, ctypes.byref(desc), None, None,
                                         A, ws, wsb, None)
    assert cached(kv_len=299) == E_SHAPE                       # fewer keys than chunk tokens
    assert cached(desc=kv(layout=0, bt=None)) == E_UNSUP       # a ring in global mode
    assert cached(desc=kv(layout=1, ps=64, mp=10)) == E_SHAPE  # the table does not cover the 700-token prefix
    assert cached(wsb=1000) == E_WS
    assert cached(q=None) == E_NULL
    assert cached(desc=kv(layout=1, ps=64, mp=16, bt=None)) == E_NULL
    assert cached(d=dims(Lq=0, hq=64, hkv=4), q=None) == OK
    assert L.sinkattn_prefill_cached(0, 0, ctypes.byref(dims()), 100, A, A, A, None, None, None, A, A, 1 << 40,
                                     None) == E_NULL


def test_prefill_cached_workspace_size(L):
    # global: all kv_len rows gathered (K + V) and their V^T copy
    assert sa.sinkattn_prefill_cached_workspace_bytes(0, 0, 1, 16384, 64, 4, 32768) == 4 * 32768 * (384 + 256 + 256)
    # sliding window: the chunk and the window - 1 positions before it
    rows = 16384 + 127
    assert sa.sinkattn_prefill_cached_workspace_bytes(1, 128, 1, 16384, 64, 8, 32768) == \
        8 * rows * (384 + 256) + 8 * 128 * ((rows + 63) // 64 * 64) * 2


def test_decode_prologue_argument_errors(L):
    def pro(theta=1e4, d=None, n=1, q_in=A, q_out=A, desc=None, fp8=0, ks=1.0, window=128):
        d = d or dims(B=2, hq=64, hkv=8)
        desc = desc if desc is not None else kv(layout=0, bt=None)
        return L.sinkattn_decode_prologue(theta, window, ctypes.byref(d), n, q_in, q_out, A, A, ctypes.byref(desc),
                                          fp8, ks, 1.0, A, None)
    assert L.sinkattn_decode_prologue(1e4, 128, None, 1, A, A, A, A, None, 0, 1.0, 1.0, A, None) == E_NULL
    assert pro(theta=0.0) == E_SHAPE
    assert pro(theta=float("nan")) == E_SHAPE
    assert pro(d=dims(B=2, hq=64, hkv=8, dqk=128)) == E_UNSUP
    assert pro(d=dims(B=2, hq=60, hkv=8)) == E_SHAPE
    assert pro(window=0) == E_SHAPE
    assert pro(fp8=1, ks=0.0) == E_SHAPE
    assert pro(q_in=None) == E_NULL
    assert pro(q_out=A + 8) == E_ALIGN
    assert pro(n=0, q_in=None) == OK


def test_decode_step_argument_errors(L):
    def step(theta=1e4, window=128, d=None, desc=None, kn=A, vn=A, q=A, ml=65536, ep=None):
        d = d or dims(B=128, hq=64, hkv=8)
        desc = desc if desc is not None else kv(layout=0, bt=None)
        return L.sinkattn_decode_step(theta, window, ctypes.byref(d), q, kn, vn, ctypes.byref(desc), A, ml, None,
                                      ep, A, None)
    assert L.sinkattn_decode_step(1e4, 128, None, A, A, A, None, A, 100, None, None, A, None) == E_NULL
    assert step(theta=0.0) == E_SHAPE
    assert step(theta=float("inf")) == E_SHAPE
    assert step(window=0) == E_SHAPE
    assert step(desc=kv(layout=1, ps=64, mp=4096)) == E_UNSUP      # pages: prologue + decode instead
    assert step(window=256) == E_UNSUP                             # more than 128 visible slots
    assert step(d=dims(B=8, hq=64, hkv=2)) == E_UNSUP              # 32 query heads per KV head
    assert step(kn=None) == E_NULL
    assert step(vn=None) == E_NULL
    assert step(q=None) == E_NULL
    assert step(vn=A + 4) == E_ALIGN
    assert step(ml=0) == E_SHAPE
    assert step(d=dims(B=0, hq=64, hkv=8), q=None) == OK
