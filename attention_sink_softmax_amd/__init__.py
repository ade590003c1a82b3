"""Python binding of libsinkattn.so: sink-bias softmax attention on MI355X (gfx950).

The functions named like the C ABI (sinkattn_prefill, sinkattn_prefill_workspace_bytes,
sinkattn_decode, sinkattn_decode_workspace_bytes, sinkattn_status_string) only marshal
arguments: they
check that torch tensors have the dtype, device, contiguity and shapes the C ABI
documents, then pass raw device pointers, sizes and the current HIP stream.  Every step
of the computation runs in the library's HIP kernels; there is no fallback.  If the
library has not been built, the first call raises LibraryMissing.

`prefill` and `decode` are conveniences that allocate the output and the workspace with
torch and call the C-ABI functions.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsinkattn.so")

GLOBAL = 0
SWA = 1
KV_RING = 0
KV_PAGED = 1
D_QK = 192
D_V = 128

STATUS = {0: "SINKATTN_OK", 1: "SINKATTN_E_NULL", 2: "SINKATTN_E_SHAPE", 3: "SINKATTN_E_UNSUPPORTED",
          4: "SINKATTN_E_ALIGN", 5: "SINKATTN_E_WORKSPACE", 6: "SINKATTN_E_DEVICE"}


class LibraryMissing(ImportError):
    pass


class SinkAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32), ("hq", ctypes.c_int32),
                ("hkv", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class KVDesc(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


class Epilogue(ctypes.Structure):
    _fields_ = [("out_scale", ctypes.c_float), ("lse", ctypes.c_void_p)]


EXPORTS = ("sinkattn_prefill", "sinkattn_prefill_workspace_bytes", "sinkattn_prefill_chunk",
           "sinkattn_prefill_chunk_workspace_bytes", "sinkattn_prefill_ex", "sinkattn_decode",
           "sinkattn_decode_workspace_bytes", "sinkattn_decode_multi", "sinkattn_decode_multi_workspace_bytes",
           "sinkattn_decode_fp8", "sinkattn_decode_ex", "sinkattn_decode_ex_noalloc", "sinkattn_decode_verify",
           "sinkattn_prefill_cached", "sinkattn_prefill_cached_workspace_bytes", "sinkattn_decode_prologue",
           "sinkattn_decode_step", "sinkattn_rope",
           "sinkattn_kv_append",
           "sinkattn_prefill_backward", "sinkattn_prefill_backward_workspace_bytes",
           "sinkattn_status_string")

_lib = None


def lib(path: str = LIB_PATH):
    """Load libsinkattn.so and declare its C signatures (raises LibraryMissing if absent)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise LibraryMissing(f"{path} is not built; run `python -m attention_sink_softmax_amd.build`")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L.sinkattn_prefill.restype = I
    L.sinkattn_prefill.argtypes = [I, I, ctypes.POINTER(Dims), P, P, P, P, P, P, ctypes.c_size_t, P]
    L.sinkattn_prefill_workspace_bytes.restype = ctypes.c_size_t
    L.sinkattn_prefill_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
    L.sinkattn_prefill_chunk.restype = I
    L.sinkattn_prefill_chunk.argtypes = [I, I, ctypes.POINTER(Dims), ctypes.c_int32, P, P, P, P, P, P,
                                         ctypes.c_size_t, P]
    L.sinkattn_prefill_chunk_workspace_bytes.restype = ctypes.c_size_t
    L.sinkattn_prefill_chunk_workspace_bytes.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32]
    L.sinkattn_decode_workspace_bytes.restype = ctypes.c_size_t
    L.sinkattn_decode_workspace_bytes.argtypes = [I, I, ctypes.POINTER(Dims), ctypes.c_int32]
    L.sinkattn_decode.restype = I
    L.sinkattn_decode.argtypes = [I, I, ctypes.POINTER(Dims), P, ctypes.POINTER(KVDesc), P, ctypes.c_int32,
                                  P, P, P, ctypes.c_size_t, P]
    L.sinkattn_decode_multi_workspace_bytes.restype = ctypes.c_size_t
    L.sinkattn_decode_multi_workspace_bytes.argtypes = [I, I, ctypes.POINTER(Dims), ctypes.c_int32, ctypes.c_int32]
    L.sinkattn_decode_multi.restype = I
    L.sinkattn_decode_multi.argtypes = [I, I, ctypes.POINTER(Dims), ctypes.c_int32, P, ctypes.POINTER(KVDesc), P,
                                        ctypes.c_int32, P, P, P, ctypes.c_size_t, P]
    L.sinkattn_decode_fp8.restype = I
    L.sinkattn_decode_fp8.argtypes = [I, I, ctypes.POINTER(Dims), ctypes.c_int32, P, ctypes.POINTER(KVDesc), P,
                                      ctypes.c_int32, P, ctypes.c_float, ctypes.c_float, P, P, ctypes.c_size_t, P]
    L.sinkattn_prefill_ex.restype = I
    L.sinkattn_prefill_ex.argtypes = [I, I, ctypes.POINTER(Dims), ctypes.c_int32, P, P, P, P, ctypes.POINTER(Epilogue),
                                      P, P, ctypes.c_size_t, P]
    L.sinkattn_decode_ex.restype = I
    L.sinkattn_decode_ex.argtypes = [I, I, ctypes.POINTER(Dims), ctypes.c_int32, P, ctypes.POINTER(KVDesc), I,
                                     ctypes.c_float, ctypes.c_float, P, ctypes.c_int32, P, ctypes.POINTER(Epilogue), P,
                                     P, ctypes.c_size_t, P]
    L.sinkattn_decode_prologue.restype = I
    L.sinkattn_decode_prologue.argtypes = [ctypes.c_double, I, ctypes.POINTER(Dims), ctypes.c_int32, P, P, P, P,
                                           ctypes.POINTER(KVDesc), I, ctypes.c_float, ctypes.c_float, P, P]
    L.sinkattn_decode_step.restype = I
    L.sinkattn_decode_step.argtypes = [ctypes.c_double, I, ctypes.POINTER(Dims), P, P, P, ctypes.POINTER(KVDesc), P,
                                       ctypes.c_int32, P, ctypes.POINTER(Epilogue), P, P]
    L.sinkattn_prefill_cached_workspace_bytes.restype = ctypes.c_size_t
    L.sinkattn_prefill_cached_workspace_bytes.argtypes = [I, I, ctypes.POINTER(Dims), ctypes.c_int32]
    L.sinkattn_prefill_cached.restype = I
    L.sinkattn_prefill_cached.argtypes = [I, I, ctypes.POINTER(Dims), ctypes.c_int32, P, P, P, ctypes.POINTER(KVDesc),
                                          P, ctypes.POINTER(Epilogue), P, P, ctypes.c_size_t, P]
    L.sinkattn_decode_verify.restype = I
    L.sinkattn_decode_verify.argtypes = [I, I, ctypes.POINTER(Dims), ctypes.c_int32, P, ctypes.POINTER(KVDesc), P, P,
                                         P, ctypes.c_int32, P, ctypes.POINTER(Epilogue), P, P, ctypes.c_size_t, P]
    L.sinkattn_decode_ex_noalloc.restype = I
    L.sinkattn_decode_ex_noalloc.argtypes = [I, I, ctypes.POINTER(Dims), ctypes.c_int32, P, ctypes.POINTER(KVDesc), I,
                                             ctypes.c_float, ctypes.c_float, P, ctypes.c_int32, P,
                                             ctypes.POINTER(Epilogue), P, P]
    L.sinkattn_prefill_backward.restype = I
    L.sinkattn_prefill_backward.argtypes = [I, I, ctypes.POINTER(Dims), P, P, P, P, P, P, P, P, P, P, P, P,
                                            ctypes.c_size_t, P]
    L.sinkattn_prefill_backward_workspace_bytes.restype = ctypes.c_size_t
    L.sinkattn_prefill_backward_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
    L.sinkattn_rope.restype = I
    L.sinkattn_rope.argtypes = [ctypes.c_double, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, ctypes.c_int32,
                                P]
    L.sinkattn_kv_append.restype = I
    L.sinkattn_kv_append.argtypes = [ctypes.POINTER(KVDesc), I, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P,
                                     P, I, ctypes.c_float, ctypes.c_float, P]
    L.sinkattn_status_string.restype = ctypes.c_char_p
    L.sinkattn_status_string.argtypes = [I]
    if path == LIB_PATH:
        _lib = L
    return L


def sinkattn_status_string(status: int) -> str:
    return lib().sinkattn_status_string(status).decode()


def _raise(rc: int):
    if rc != 0:
        raise SinkAttnError(rc, sinkattn_status_string(rc))


# ---------------------------------------------------------------------------- marshalling
def _dev_tensor(t, name, dtype, shape=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _stream_ptr(stream, device):
    import torch

    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def sinkattn_prefill_workspace_bytes(batch: int, seqlen: int, hq: int, hkv: int, d_qk: int = D_QK,
                                     d_v: int = D_V) -> int:
    d = Dims(batch, seqlen, hq, hkv, d_qk, d_v, d_qk ** -0.5)
    n = lib().sinkattn_prefill_workspace_bytes(ctypes.byref(d))
    if n == ctypes.c_size_t(-1).value:
        raise SinkAttnError(2, "invalid sizes")
    return n


def sinkattn_prefill(mode: int, window: int, q, k, v, sink, out, workspace, scale: float | None = None,
                     stream=None) -> None:
    """q bf16 [B,Hq,L,192], k bf16 [B,Hkv,L,192], v bf16 [B,Hkv,L,128], sink float32 [Hq] or
    None, out bf16 [B,Hq,L,128] (written), workspace: a GPU tensor of at least
    sinkattn_prefill_workspace_bytes(...) bytes.  Enqueued on `stream` (default: current)."""
    import torch

    B, Hq, L, dqk = q.shape
    Hkv = k.shape[1]
    _dev_tensor(q, "q", torch.bfloat16)
    _dev_tensor(k, "k", torch.bfloat16, (B, Hkv, L, dqk))
    _dev_tensor(v, "v", torch.bfloat16, (B, Hkv, L, v.shape[3]))
    _dev_tensor(out, "out", torch.bfloat16, (B, Hq, L, v.shape[3]))
    if sink is not None:
        _dev_tensor(sink, "sink", torch.float32, (Hq,))
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _dev_tensor(workspace, "workspace", workspace.dtype)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    for t in (k, v, out, sink, workspace):
        if t is not None and t.device != q.device:
            raise ValueError("all tensors must be on one device")
    d = Dims(B, L, Hq, Hkv, dqk, v.shape[3], dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q.device):
        rc = lib().sinkattn_prefill(mode, window, ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(out),
                                    ws_ptr, ws_bytes, _stream_ptr(stream, q.device))
    _raise(rc)


def sinkattn_prefill_chunk_workspace_bytes(batch: int, seqlen: int, hq: int, hkv: int, kv_len: int,
                                           d_qk: int = D_QK, d_v: int = D_V) -> int:
    d = Dims(batch, seqlen, hq, hkv, d_qk, d_v, d_qk ** -0.5)
    n = lib().sinkattn_prefill_chunk_workspace_bytes(ctypes.byref(d), kv_len)
    if n == ctypes.c_size_t(-1).value:
        raise SinkAttnError(2, "invalid sizes")
    return n


def sinkattn_prefill_chunk(mode: int, window: int, q, k, v, sink, out, workspace, scale: float | None = None,
                           stream=None) -> None:
    """Chunked prefill: q bf16 [B,Hq,Lq,192] holds positions kv_len-Lq .. kv_len-1; k bf16
    [B,Hkv,kv_len,192] and v bf16 [B,Hkv,kv_len,128] hold the prefix and the chunk; out bf16
    [B,Hq,Lq,128]; workspace of at least sinkattn_prefill_chunk_workspace_bytes(...) bytes."""
    import torch

    B, Hq, Lq, dqk = q.shape
    Hkv, kv_len = k.shape[1], k.shape[2]
    _dev_tensor(q, "q", torch.bfloat16)
    _dev_tensor(k, "k", torch.bfloat16, (B, Hkv, kv_len, dqk))
    _dev_tensor(v, "v", torch.bfloat16, (B, Hkv, kv_len, v.shape[3]))
    _dev_tensor(out, "out", torch.bfloat16, (B, Hq, Lq, v.shape[3]))
    if sink is not None:
        _dev_tensor(sink, "sink", torch.float32, (Hq,))
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _dev_tensor(workspace, "workspace", workspace.dtype)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    for t in (k, v, out, sink, workspace):
        if t is not None and t.device != q.device:
            raise ValueError("all tensors must be on one device")
    d = Dims(B, Lq, Hq, Hkv, dqk, v.shape[3], dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q.device):
        rc = lib().sinkattn_prefill_chunk(mode, window, ctypes.byref(d), kv_len, _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(sink), _ptr(out), ws_ptr, ws_bytes, _stream_ptr(stream, q.device))
    _raise(rc)


def sinkattn_decode_workspace_bytes(mode: int, window: int, batch: int, hq: int, hkv: int, max_seq_len: int,
                                    d_qk: int = D_QK, d_v: int = D_V) -> int:
    d = Dims(batch, 0, hq, hkv, d_qk, d_v, d_qk ** -0.5)
    n = lib().sinkattn_decode_workspace_bytes(mode, window, ctypes.byref(d), max_seq_len)
    if n == ctypes.c_size_t(-1).value:
        raise SinkAttnError(2, "invalid sizes")
    return n


def sinkattn_decode_multi_workspace_bytes(mode: int, window: int, batch: int, hq: int, hkv: int, q_len: int,
                                          max_seq_len: int, d_qk: int = D_QK, d_v: int = D_V) -> int:
    d = Dims(batch, 0, hq, hkv, d_qk, d_v, d_qk ** -0.5)
    n = lib().sinkattn_decode_multi_workspace_bytes(mode, window, ctypes.byref(d), q_len, max_seq_len)
    if n == ctypes.c_size_t(-1).value:
        raise SinkAttnError(2, "invalid sizes")
    return n


def _decode_args(q, q_len, layout, window, k_cache, v_cache, seq_lens, sink, out, workspace, block_table,
                 kv_fp8=False):
    """Checks the decode tensors and builds the cache descriptor (q is [B,Hq,q_len,192] here)."""
    import torch

    cdt = torch.uint8 if kv_fp8 else torch.bfloat16
    if q.dim() != 4:
        raise ValueError(f"q must be [B,Hq,q_len,192], got shape {tuple(q.shape)}")
    B, Hq, _, dqk = q.shape
    Hkv = k_cache.shape[1]
    dv = v_cache.shape[3]
    _dev_tensor(q, "q", torch.bfloat16, (B, Hq, q_len, dqk))
    _dev_tensor(out, "out", torch.bfloat16, (B, Hq, q_len, dv))
    _dev_tensor(seq_lens, "seq_lens", torch.int32, (B,))
    if sink is not None:
        _dev_tensor(sink, "sink", torch.float32, (Hq,))
    if layout == KV_RING:
        _dev_tensor(k_cache, "k_cache", cdt, (B, Hkv, window, dqk))
        _dev_tensor(v_cache, "v_cache", cdt, (B, Hkv, window, dv))
        desc = KVDesc(KV_RING, k_cache.data_ptr(), v_cache.data_ptr(), None, 0, 0, 0)
    elif layout == KV_PAGED:
        P, _, ps, _ = k_cache.shape
        _dev_tensor(k_cache, "k_cache", cdt, (P, Hkv, ps, dqk))
        _dev_tensor(v_cache, "v_cache", cdt, (P, Hkv, ps, dv))
        _dev_tensor(block_table, "block_table", torch.int32, (B, block_table.shape[1]))
        desc = KVDesc(KV_PAGED, k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(), ps,
                      block_table.shape[1], P)
    else:
        raise ValueError("layout must be KV_RING or KV_PAGED")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _dev_tensor(workspace, "workspace", workspace.dtype)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    for t in (k_cache, v_cache, out, seq_lens, sink, block_table, workspace):
        if t is not None and t.device != q.device:
            raise ValueError("all tensors must be on one device")
    return B, Hq, Hkv, dqk, dv, desc, ws_ptr, ws_bytes


def sinkattn_decode(mode: int, window: int, q, layout: int, k_cache, v_cache, seq_lens, max_seq_len: int,
                    sink, out, workspace, block_table=None, scale: float | None = None, stream=None) -> None:
    """q bf16 [B,Hq,192]; RING: k_cache [B,Hkv,W,192], v_cache [B,Hkv,W,128];
    PAGED: k_cache [P,Hkv,page,192], v_cache [P,Hkv,page,128], block_table int32 [B,max_pages].
    seq_lens int32 [B] (device), sink float32 [Hq] or None, out bf16 [B,Hq,128],
    workspace uint8 tensor of at least sinkattn_decode_workspace_bytes(...) bytes or None."""
    import torch

    B, Hq, Hkv, dqk, dv, desc, ws_ptr, ws_bytes = _decode_args(q.unsqueeze(2), 1, layout, window, k_cache, v_cache,
                                                               seq_lens, sink, out.unsqueeze(2), workspace,
                                                               block_table)
    d = Dims(B, 0, Hq, Hkv, dqk, dv, dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q.device):
        rc = lib().sinkattn_decode(mode, window, ctypes.byref(d), _ptr(q), ctypes.byref(desc), _ptr(seq_lens),
                                   max_seq_len, _ptr(sink), _ptr(out), ws_ptr, ws_bytes,
                                   _stream_ptr(stream, q.device))
    _raise(rc)


def sinkattn_decode_multi(mode: int, window: int, q_len: int, q, layout: int, k_cache, v_cache, seq_lens,
                          max_seq_len: int, sink, out, workspace, block_table=None, scale: float | None = None,
                          stream=None) -> None:
    """q bf16 [B,Hq,q_len,192], out bf16 [B,Hq,q_len,128]; the q_len new tokens are the last
    q_len positions of each sequence (seq_lens counts them).  Otherwise as sinkattn_decode;
    workspace of at least sinkattn_decode_multi_workspace_bytes(...) bytes or None."""
    import torch

    B, Hq, Hkv, dqk, dv, desc, ws_ptr, ws_bytes = _decode_args(q, q_len, layout, window, k_cache, v_cache, seq_lens,
                                                               sink, out, workspace, block_table)
    d = Dims(B, 0, Hq, Hkv, dqk, dv, dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q.device):
        rc = lib().sinkattn_decode_multi(mode, window, ctypes.byref(d), q_len, _ptr(q), ctypes.byref(desc),
                                         _ptr(seq_lens), max_seq_len, _ptr(sink), _ptr(out), ws_ptr, ws_bytes,
                                         _stream_ptr(stream, q.device))
    _raise(rc)


# ---------------------------------------------------------------------------- conveniences
def prefill_workspace(q, k):
    """A workspace tensor sized for sinkattn_prefill on these q/k shapes."""
    import torch

    B, Hq, L, _ = q.shape
    n = sinkattn_prefill_workspace_bytes(B, L, Hq, k.shape[1])
    return torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)


def prefill(mode: int, window: int, q, k, v, sink=None, scale: float | None = None, stream=None, workspace=None):
    """Allocate out (and the workspace if none is given) with torch and run sinkattn_prefill."""
    import torch

    out = torch.empty((*q.shape[:3], v.shape[3]), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        workspace = prefill_workspace(q, k)
    sinkattn_prefill(mode, window, q, k, v, sink, out, workspace, scale, stream)
    return out


def prefill_chunk(mode: int, window: int, q, k, v, sink=None, scale: float | None = None, stream=None,
                  workspace=None):
    """Allocate out (and the workspace if none is given) and run sinkattn_prefill_chunk."""
    import torch

    out = torch.empty((*q.shape[:3], v.shape[3]), dtype=torch.bfloat16, device=q.device)
    if workspace is None:
        n = sinkattn_prefill_chunk_workspace_bytes(q.shape[0], q.shape[2], q.shape[1], k.shape[1], k.shape[2])
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    sinkattn_prefill_chunk(mode, window, q, k, v, sink, out, workspace, scale, stream)
    return out


def decode_workspace(mode: int, window: int, batch: int, hq: int, hkv: int, max_seq_len: int, device):
    import torch

    n = sinkattn_decode_workspace_bytes(mode, window, batch, hq, hkv, max_seq_len)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device) if n else None


def decode(mode: int, window: int, q, layout: int, k_cache, v_cache, seq_lens, max_seq_len: int, sink=None,
           block_table=None, workspace=None, scale: float | None = None, stream=None):
    """Allocate out (and the workspace if none is given) and run sinkattn_decode."""
    import torch

    B, Hq, _ = q.shape
    if workspace is None:
        workspace = decode_workspace(mode, window, B, Hq, k_cache.shape[1], max_seq_len, q.device)
    out = torch.empty((B, Hq, v_cache.shape[3]), dtype=torch.bfloat16, device=q.device)
    sinkattn_decode(mode, window, q, layout, k_cache, v_cache, seq_lens, max_seq_len, sink, out, workspace,
                    block_table, scale, stream)
    return out


def _epilogue(out_scale, lse, shape, device):
    import torch

    if lse is not None:
        _dev_tensor(lse, "lse", torch.float32, shape)
        if lse.device != device:
            raise ValueError("all tensors must be on one device")
    return Epilogue(out_scale, None if lse is None else lse.data_ptr())


def sinkattn_prefill_ex(mode: int, window: int, q, k, v, sink, out, workspace, out_scale: float = 1.0, lse=None,
                        scale: float | None = None, stream=None) -> None:
    """sinkattn_prefill_chunk (q [B,Hq,Lq,192] after a prefix: k, v hold kv_len = k.shape[2]
    keys) with an epilogue: out = out_scale * attention, lse float32 [B,Hq,Lq] or None."""
    import torch

    B, Hq, Lq, dqk = q.shape
    Hkv, kv_len = k.shape[1], k.shape[2]
    _dev_tensor(q, "q", torch.bfloat16)
    _dev_tensor(k, "k", torch.bfloat16, (B, Hkv, kv_len, dqk))
    _dev_tensor(v, "v", torch.bfloat16, (B, Hkv, kv_len, v.shape[3]))
    _dev_tensor(out, "out", torch.bfloat16, (B, Hq, Lq, v.shape[3]))
    if sink is not None:
        _dev_tensor(sink, "sink", torch.float32, (Hq,))
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _dev_tensor(workspace, "workspace", workspace.dtype)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    for t in (k, v, out, sink, workspace):
        if t is not None and t.device != q.device:
            raise ValueError("all tensors must be on one device")
    ep = _epilogue(out_scale, lse, (B, Hq, Lq), q.device)
    d = Dims(B, Lq, Hq, Hkv, dqk, v.shape[3], dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q.device):
        rc = lib().sinkattn_prefill_ex(mode, window, ctypes.byref(d), kv_len, _ptr(q), _ptr(k), _ptr(v), _ptr(sink),
                                       ctypes.byref(ep), _ptr(out), ws_ptr, ws_bytes, _stream_ptr(stream, q.device))
    _raise(rc)


def sinkattn_decode_ex(mode: int, window: int, q_len: int, q, layout: int, k_cache, v_cache, seq_lens,
                       max_seq_len: int, sink, out, workspace, block_table=None, kv_fp8: bool = False,
                       k_scale: float = 1.0, v_scale: float = 1.0, out_scale: float = 1.0, lse=None,
                       scale: float | None = None, stream=None) -> None:
    """Decode with every option: q bf16 [B,Hq,q_len,192], out bf16 [B,Hq,q_len,128]; caches
    bf16 (kv_fp8 False) or uint8 E4M3 codes (kv_fp8 True, paged); lse float32 [B,Hq,q_len]."""
    import torch

    B, Hq, Hkv, dqk, dv, desc, ws_ptr, ws_bytes = _decode_args(q, q_len, layout, window, k_cache, v_cache, seq_lens,
                                                               sink, out, workspace, block_table, kv_fp8)
    ep = _epilogue(out_scale, lse, (B, Hq, q_len), q.device)
    d = Dims(B, 0, Hq, Hkv, dqk, dv, dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q.device):
        rc = lib().sinkattn_decode_ex(mode, window, ctypes.byref(d), q_len, _ptr(q), ctypes.byref(desc),
                                      1 if kv_fp8 else 0, k_scale, v_scale, _ptr(seq_lens), max_seq_len, _ptr(sink),
                                      ctypes.byref(ep), _ptr(out), ws_ptr, ws_bytes, _stream_ptr(stream, q.device))
    _raise(rc)


def sinkattn_prefill_cached_workspace_bytes(mode: int, window: int, batch: int, seqlen: int, hq: int, hkv: int,
                                            kv_len: int) -> int:
    d = Dims(batch, seqlen, hq, hkv, D_QK, D_V, D_QK ** -0.5)
    n = lib().sinkattn_prefill_cached_workspace_bytes(mode, window, ctypes.byref(d), kv_len)
    if n == ctypes.c_size_t(-1).value:
        raise SinkAttnError(2, "invalid sizes")
    return n


def sinkattn_prefill_cached(mode: int, window: int, kv_len: int, q, k, v, layout: int, k_cache, v_cache, sink, out,
                            workspace, block_table=None, out_scale: float = 1.0, lse=None, scale: float | None = None,
                            stream=None) -> None:
    """Chunked prefill over a cached prefix: q bf16 [B,Hq,Lq,192] at positions kv_len-Lq ..
    kv_len-1, k bf16 [B,Hkv,Lq,192] and v bf16 [B,Hkv,Lq,128] the chunk's keys and values; the
    prefix in a RING ([B,Hkv,W,d], sliding window) or PAGED ([P,Hkv,page,d] + block_table) cache;
    out bf16 [B,Hq,Lq,128]; workspace of sinkattn_prefill_cached_workspace_bytes(...) bytes."""
    import torch

    B, Hq, Lq, dqk = q.shape
    Hkv = k.shape[1]
    _dev_tensor(q, "q", torch.bfloat16)
    _dev_tensor(k, "k", torch.bfloat16, (B, Hkv, Lq, dqk))
    _dev_tensor(v, "v", torch.bfloat16, (B, Hkv, Lq, v.shape[3]))
    _dev_tensor(out, "out", torch.bfloat16, (B, Hq, Lq, v.shape[3]))
    if sink is not None:
        _dev_tensor(sink, "sink", torch.float32, (Hq,))
    if layout == KV_RING:
        W = k_cache.shape[2]
        _dev_tensor(k_cache, "k_cache", torch.bfloat16, (B, Hkv, W, dqk))
        _dev_tensor(v_cache, "v_cache", torch.bfloat16, (B, Hkv, W, v.shape[3]))
        desc = KVDesc(KV_RING, k_cache.data_ptr(), v_cache.data_ptr(), None, 0, 0, 0)
    elif layout == KV_PAGED:
        P, _, ps, _ = k_cache.shape
        _dev_tensor(k_cache, "k_cache", torch.bfloat16, (P, Hkv, ps, dqk))
        _dev_tensor(v_cache, "v_cache", torch.bfloat16, (P, Hkv, ps, v.shape[3]))
        _dev_tensor(block_table, "block_table", torch.int32, (B, block_table.shape[1]))
        desc = KVDesc(KV_PAGED, k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(), ps,
                      block_table.shape[1], P)
    else:
        raise ValueError("layout must be KV_RING or KV_PAGED")
    _dev_tensor(workspace, "workspace", workspace.dtype)
    for t in (k, v, out, sink, k_cache, v_cache, block_table, workspace):
        if t is not None and t.device != q.device:
            raise ValueError("all tensors must be on one device")
    ep = _epilogue(out_scale, lse, (B, Hq, Lq), q.device)
    d = Dims(B, Lq, Hq, Hkv, dqk, v.shape[3], dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q.device):
        rc = lib().sinkattn_prefill_cached(mode, window, ctypes.byref(d), kv_len, _ptr(q), _ptr(k), _ptr(v),
                                           ctypes.byref(desc), _ptr(sink), ctypes.byref(ep), _ptr(out),
                                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           _stream_ptr(stream, q.device))
    _raise(rc)


def prefill_cached(mode: int, window: int, kv_len: int, q, k, v, layout: int, k_cache, v_cache, sink=None,
                   block_table=None, workspace=None, scale: float | None = None, stream=None):
    """Allocate out (and the workspace if none is given) and run sinkattn_prefill_cached."""
    import torch

    B, Hq, Lq, _ = q.shape
    if workspace is None:
        n = sinkattn_prefill_cached_workspace_bytes(mode, window, B, Lq, Hq, k.shape[1], kv_len)
        workspace = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    out = torch.empty((B, Hq, Lq, v.shape[3]), dtype=torch.bfloat16, device=q.device)
    sinkattn_prefill_cached(mode, window, kv_len, q, k, v, layout, k_cache, v_cache, sink, out, workspace,
                            block_table, scale=scale, stream=stream)
    return out


def sinkattn_decode_verify(mode: int, window: int, q_len: int, q, layout: int, k_cache, v_cache, k_new, v_new,
                           seq_lens, max_seq_len: int, sink, out, workspace, block_table=None, out_scale: float = 1.0,
                           lse=None, scale: float | None = None, stream=None) -> None:
    """Drafted tokens checked against a cache that does not hold them: q bf16 [B,Hq,q_len,192],
    k_new bf16 [B,Hkv,q_len,192], v_new bf16 [B,Hkv,q_len,128] (the drafts' keys and values),
    a RING ([B,Hkv,W,d], the last W committed positions) or PAGED cache of the committed
    positions; seq_lens counts the committed tokens plus the q_len drafts.  out bf16
    [B,Hq,q_len,128]; workspace of sinkattn_decode_multi_workspace_bytes(...) bytes or None."""
    import torch

    B, Hq, Hkv, dqk, dv, desc, ws_ptr, ws_bytes = _decode_args(q, q_len, layout, window, k_cache, v_cache, seq_lens,
                                                               sink, out, workspace, block_table)
    _dev_tensor(k_new, "k_new", torch.bfloat16, (B, Hkv, q_len, dqk))
    _dev_tensor(v_new, "v_new", torch.bfloat16, (B, Hkv, q_len, dv))
    for t in (k_new, v_new):
        if t.device != q.device:
            raise ValueError("all tensors must be on one device")
    ep = _epilogue(out_scale, lse, (B, Hq, q_len), q.device)
    d = Dims(B, 0, Hq, Hkv, dqk, dv, dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q.device):
        rc = lib().sinkattn_decode_verify(mode, window, ctypes.byref(d), q_len, _ptr(q), ctypes.byref(desc),
                                          _ptr(k_new), _ptr(v_new), _ptr(seq_lens), max_seq_len, _ptr(sink),
                                          ctypes.byref(ep), _ptr(out), ws_ptr, ws_bytes, _stream_ptr(stream, q.device))
    _raise(rc)


def decode_verify(mode: int, window: int, q, layout: int, k_cache, v_cache, k_new, v_new, seq_lens, max_seq_len: int,
                  sink=None, block_table=None, workspace=None, scale: float | None = None, stream=None):
    """Allocate out (and the workspace if none is given) and run sinkattn_decode_verify."""
    import torch

    B, Hq, q_len, _ = q.shape
    if workspace is None:
        workspace = decode_multi_workspace(mode, window, B, Hq, k_cache.shape[1], q_len, max_seq_len, q.device)
    out = torch.empty((B, Hq, q_len, v_cache.shape[3]), dtype=torch.bfloat16, device=q.device)
    sinkattn_decode_verify(mode, window, q_len, q, layout, k_cache, v_cache, k_new, v_new, seq_lens, max_seq_len,
                           sink, out, workspace, block_table, scale=scale, stream=stream)
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20  # SINKATTN_NOALLOC_SCRATCH_BYTES


def sinkattn_decode_ex_noalloc(mode: int, window: int, q_len: int, q, layout: int, k_cache, v_cache, seq_lens,
                               max_seq_len: int, sink, out, block_table=None, kv_fp8: bool = False,
                               k_scale: float = 1.0, v_scale: float = 1.0, out_scale: float = 1.0, lse=None,
                               scale: float | None = None, stream=None) -> None:
    """sinkattn_decode_ex without a workspace: the split partials go to the library's own
    device scratch array (NOALLOC_SCRATCH_BYTES per GPU), so the call allocates nothing.
    Calls that overlap on one GPU race."""
    import torch

    B, Hq, Hkv, dqk, dv, desc, _, _ = _decode_args(q, q_len, layout, window, k_cache, v_cache, seq_lens, sink, out,
                                                   None, block_table, kv_fp8)
    ep = _epilogue(out_scale, lse, (B, Hq, q_len), q.device)
    d = Dims(B, 0, Hq, Hkv, dqk, dv, dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q.device):
        rc = lib().sinkattn_decode_ex_noalloc(mode, window, ctypes.byref(d), q_len, _ptr(q), ctypes.byref(desc),
                                              1 if kv_fp8 else 0, k_scale, v_scale, _ptr(seq_lens), max_seq_len,
                                              _ptr(sink), ctypes.byref(ep), _ptr(out), _stream_ptr(stream, q.device))
    _raise(rc)


SWA_ROPE_THETA = 10000.0
GA_ROPE_THETA = 5000000.0


def sinkattn_prefill_backward(mode: int, window: int, q, k, v, sink, out, dout, lse, dq, dk, dv, dsink, workspace,
                              scale: float | None = None, stream=None) -> None:
    """Gradients of prefill: q, k, v, out, dout bf16 (shapes as sinkattn_prefill), lse float32
    [B,Hq,L] from sinkattn_prefill_ex; writes dq, dk, dv (float32, shaped like q, k, v) and dsink
    (float32 [Hq], when sink is given)."""
    import torch

    B, Hq, L, dqk = q.shape
    Hkv = k.shape[1]
    for t, name, dt, shp in ((q, "q", torch.bfloat16, None), (k, "k", torch.bfloat16, (B, Hkv, L, dqk)),
                             (v, "v", torch.bfloat16, (B, Hkv, L, 128)), (out, "out", torch.bfloat16, (B, Hq, L, 128)),
                             (dout, "dout", torch.bfloat16, (B, Hq, L, 128)), (lse, "lse", torch.float32, (B, Hq, L)),
                             (dq, "dq", torch.float32, (B, Hq, L, dqk)), (dk, "dk", torch.float32, (B, Hkv, L, dqk)),
                             (dv, "dv", torch.float32, (B, Hkv, L, 128))):
        _dev_tensor(t, name, dt, shp)
    if sink is not None:
        _dev_tensor(sink, "sink", torch.float32, (Hq,))
        _dev_tensor(dsink, "dsink", torch.float32, (Hq,))
    _dev_tensor(workspace, "workspace", workspace.dtype)
    d = Dims(B, L, Hq, Hkv, dqk, 128, dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q.device):
        rc = lib().sinkattn_prefill_backward(mode, window, ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(sink),
                                             _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                             _ptr(dsink) if sink is not None else None, _ptr(workspace),
                                             workspace.numel() * workspace.element_size(), _stream_ptr(stream, q.device))
    _raise(rc)


def prefill_backward(mode: int, window: int, q, k, v, sink, out, dout, lse, scale: float | None = None, stream=None):
    """Allocate the gradients and the workspace and run sinkattn_prefill_backward; returns
    (dq, dk, dv, dsink or None)."""
    import torch

    B, Hq, L, _ = q.shape
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    dsink = torch.empty(Hq, dtype=torch.float32, device=q.device) if sink is not None else None
    dd = Dims(B, L, Hq, k.shape[1], 192, 128, 192 ** -0.5)
    n = lib().sinkattn_prefill_backward_workspace_bytes(ctypes.byref(dd))
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)
    sinkattn_prefill_backward(mode, window, q, k, v, sink, out, dout, lse, dq, dk, dv, dsink, ws, scale, stream)
    return dq, dk, dv, dsink


def sinkattn_rope(theta: float, x, seq_lens=None, pos0: int = 0, stream=None) -> None:
    """Rotate the first 64 of the 192 dimensions of x bf16 [B,H,rows,192] in place; row r of
    sequence b at position seq_lens[b] - rows + r (seq_lens int32 [B] on the device) or
    pos0 + r."""
    import torch

    B, H, rows, d = x.shape
    _dev_tensor(x, "x", torch.bfloat16, (B, H, rows, 192))
    if seq_lens is not None:
        _dev_tensor(seq_lens, "seq_lens", torch.int32, (B,))
    with torch.cuda.device(x.device):
        rc = lib().sinkattn_rope(theta, B, H, rows, _ptr(x), _ptr(seq_lens), pos0, _stream_ptr(stream, x.device))
    _raise(rc)


def sinkattn_kv_append(layout: int, k_cache, v_cache, k_new, v_new, seq_lens, window: int = 0, block_table=None,
                       kv_fp8: bool = False, k_scale: float = 1.0, v_scale: float = 1.0, stream=None) -> None:
    """Write k_new bf16 [B,Hkv,n,192] and v_new bf16 [B,Hkv,n,128] at positions
    seq_lens[b] - n .. seq_lens[b] - 1 into a ring ([B,Hkv,window,d]) or paged
    ([P,Hkv,page,d]) cache, bf16 or uint8 E4M3 codes (kv_fp8)."""
    import torch

    B, Hkv, n, dqk = k_new.shape
    cdt = torch.uint8 if kv_fp8 else torch.bfloat16
    _dev_tensor(k_new, "k_new", torch.bfloat16, (B, Hkv, n, 192))
    _dev_tensor(v_new, "v_new", torch.bfloat16, (B, Hkv, n, 128))
    _dev_tensor(seq_lens, "seq_lens", torch.int32, (B,))
    if layout == KV_RING:
        _dev_tensor(k_cache, "k_cache", cdt, (B, Hkv, window, 192))
        _dev_tensor(v_cache, "v_cache", cdt, (B, Hkv, window, 128))
        desc = KVDesc(KV_RING, k_cache.data_ptr(), v_cache.data_ptr(), None, 0, 0, 0)
    else:
        P, _, ps, _ = k_cache.shape
        _dev_tensor(k_cache, "k_cache", cdt, (P, Hkv, ps, 192))
        _dev_tensor(v_cache, "v_cache", cdt, (P, Hkv, ps, 128))
        _dev_tensor(block_table, "block_table", torch.int32, (B, block_table.shape[1]))
        desc = KVDesc(KV_PAGED, k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(), ps,
                      block_table.shape[1], P)
    with torch.cuda.device(k_new.device):
        rc = lib().sinkattn_kv_append(ctypes.byref(desc), window, B, Hkv, n, _ptr(k_new), _ptr(v_new), _ptr(seq_lens),
                                      1 if kv_fp8 else 0, k_scale, v_scale, _stream_ptr(stream, k_new.device))
    _raise(rc)


def sinkattn_decode_prologue(theta: float, layout: int, q_in, q_out, k_new, v_new, k_cache, v_cache, seq_lens,
                             window: int = 0, block_table=None, kv_fp8: bool = False, k_scale: float = 1.0,
                             v_scale: float = 1.0, stream=None) -> None:
    """RoPE of the new queries q_in bf16 [B,Hq,n,192] into q_out (may be q_in) and of the new keys
    k_new bf16 [B,Hkv,n,192], then the cache write of the rotated keys and v_new bf16
    [B,Hkv,n,128] at positions seq_lens[b] - n .. seq_lens[b] - 1 into a ring ([B,Hkv,window,d])
    or pages ([P,Hkv,page,d]), bf16 or uint8 E4M3 codes (kv_fp8); one kernel."""
    import torch

    B, Hq, n, _ = q_in.shape
    Hkv = k_new.shape[1]
    cdt = torch.uint8 if kv_fp8 else torch.bfloat16
    _dev_tensor(q_in, "q_in", torch.bfloat16, (B, Hq, n, 192))
    _dev_tensor(q_out, "q_out", torch.bfloat16, (B, Hq, n, 192))
    _dev_tensor(k_new, "k_new", torch.bfloat16, (B, Hkv, n, 192))
    _dev_tensor(v_new, "v_new", torch.bfloat16, (B, Hkv, n, 128))
    _dev_tensor(seq_lens, "seq_lens", torch.int32, (B,))
    if layout == KV_RING:
        _dev_tensor(k_cache, "k_cache", cdt, (B, Hkv, window, 192))
        _dev_tensor(v_cache, "v_cache", cdt, (B, Hkv, window, 128))
        desc = KVDesc(KV_RING, k_cache.data_ptr(), v_cache.data_ptr(), None, 0, 0, 0)
    else:
        P, _, ps, _ = k_cache.shape
        _dev_tensor(k_cache, "k_cache", cdt, (P, Hkv, ps, 192))
        _dev_tensor(v_cache, "v_cache", cdt, (P, Hkv, ps, 128))
        _dev_tensor(block_table, "block_table", torch.int32, (B, block_table.shape[1]))
        desc = KVDesc(KV_PAGED, k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(), ps,
                      block_table.shape[1], P)
    for t in (q_out, k_new, v_new, seq_lens, k_cache, v_cache, block_table):
        if t is not None and t.device != q_in.device:
            raise ValueError("all tensors must be on one device")
    d = Dims(B, 0, Hq, Hkv, 192, 128, 192 ** -0.5)
    with torch.cuda.device(q_in.device):
        rc = lib().sinkattn_decode_prologue(theta, window, ctypes.byref(d), n, _ptr(q_in), _ptr(q_out), _ptr(k_new),
                                            _ptr(v_new), ctypes.byref(desc), 1 if kv_fp8 else 0, k_scale, v_scale,
                                            _ptr(seq_lens), _stream_ptr(stream, q_in.device))
    _raise(rc)


def sinkattn_decode_step(theta: float, window: int, q_in, k_new, v_new, k_cache, v_cache, seq_lens, max_seq_len: int,
                         sink, out, out_scale: float = 1.0, lse=None, scale: float | None = None, stream=None) -> None:
    """One sliding-window decode step in one kernel: RoPE of the new token's queries q_in bf16
    [B,Hq,1,192] and key k_new bf16 [B,Hkv,1,192] at position seq_lens[b] - 1, the write of the
    rotated key and v_new bf16 [B,Hkv,1,128] into ring slot (seq_lens[b] - 1) mod window of
    k_cache [B,Hkv,window,192] / v_cache [B,Hkv,window,128] (bf16), and the attention; out bf16
    [B,Hq,1,128], lse float32 [B,Hq,1] or None.  q_in, k_new and v_new are not modified."""
    import torch

    B, Hq, Hkv, dqk, dv, desc, _, _ = _decode_args(q_in, 1, KV_RING, window, k_cache, v_cache, seq_lens, sink, out,
                                                   None, None)
    _dev_tensor(k_new, "k_new", torch.bfloat16, (B, Hkv, 1, dqk))
    _dev_tensor(v_new, "v_new", torch.bfloat16, (B, Hkv, 1, dv))
    for t in (k_new, v_new):
        if t.device != q_in.device:
            raise ValueError("all tensors must be on one device")
    ep = _epilogue(out_scale, lse, (B, Hq, 1), q_in.device)
    d = Dims(B, 0, Hq, Hkv, dqk, dv, dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q_in.device):
        rc = lib().sinkattn_decode_step(theta, window, ctypes.byref(d), _ptr(q_in), _ptr(k_new), _ptr(v_new),
                                        ctypes.byref(desc), _ptr(seq_lens), max_seq_len, _ptr(sink), ctypes.byref(ep),
                                        _ptr(out), _stream_ptr(stream, q_in.device))
    _raise(rc)


def sinkattn_decode_fp8(mode: int, window: int, q_len: int, q, k_cache, v_cache, seq_lens, max_seq_len: int, sink,
                        k_scale: float, v_scale: float, out, workspace, block_table,
                        scale: float | None = None, stream=None) -> None:
    """8-bit paged cache: k_cache uint8 [P,Hkv,page,192], v_cache uint8 [P,Hkv,page,128] of
    E4M3 codes (element = scale * code value), block_table int32 [B,max_pages]; q bf16
    [B,Hq,q_len,192], out bf16 [B,Hq,q_len,128]; workspace of at least
    sinkattn_decode_multi_workspace_bytes(...) bytes or None."""
    import torch

    if q.dim() != 4:
        raise ValueError(f"q must be [B,Hq,q_len,192], got shape {tuple(q.shape)}")
    B, Hq, _, dqk = q.shape
    P, Hkv, ps, _ = k_cache.shape
    dv = v_cache.shape[3]
    _dev_tensor(q, "q", torch.bfloat16, (B, Hq, q_len, dqk))
    _dev_tensor(out, "out", torch.bfloat16, (B, Hq, q_len, dv))
    _dev_tensor(seq_lens, "seq_lens", torch.int32, (B,))
    if sink is not None:
        _dev_tensor(sink, "sink", torch.float32, (Hq,))
    _dev_tensor(k_cache, "k_cache", torch.uint8, (P, Hkv, ps, dqk))
    _dev_tensor(v_cache, "v_cache", torch.uint8, (P, Hkv, ps, dv))
    _dev_tensor(block_table, "block_table", torch.int32, (B, block_table.shape[1]))
    desc = KVDesc(KV_PAGED, k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(), ps, block_table.shape[1], P)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _dev_tensor(workspace, "workspace", workspace.dtype)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    for t in (k_cache, v_cache, out, seq_lens, sink, block_table, workspace):
        if t is not None and t.device != q.device:
            raise ValueError("all tensors must be on one device")
    d = Dims(B, 0, Hq, Hkv, dqk, dv, dqk ** -0.5 if scale is None else scale)
    with torch.cuda.device(q.device):
        rc = lib().sinkattn_decode_fp8(mode, window, ctypes.byref(d), q_len, _ptr(q), ctypes.byref(desc),
                                       _ptr(seq_lens), max_seq_len, _ptr(sink), k_scale, v_scale, _ptr(out), ws_ptr,
                                       ws_bytes, _stream_ptr(stream, q.device))
    _raise(rc)


def decode_fp8(mode: int, window: int, q, k_cache, v_cache, seq_lens, max_seq_len: int, k_scale: float,
               v_scale: float, block_table, sink=None, workspace=None, scale: float | None = None, stream=None):
    """Allocate out (and the workspace) and run sinkattn_decode_fp8; q is [B,Hq,192] (one new
    token) or [B,Hq,q_len,192]."""
    import torch

    one = q.dim() == 3
    q4 = q.unsqueeze(2) if one else q
    B, Hq, q_len, _ = q4.shape
    if workspace is None:
        workspace = decode_multi_workspace(mode, window, B, Hq, k_cache.shape[1], q_len, max_seq_len, q.device)
    out = torch.empty((B, Hq, q_len, v_cache.shape[3]), dtype=torch.bfloat16, device=q.device)
    sinkattn_decode_fp8(mode, window, q_len, q4, k_cache, v_cache, seq_lens, max_seq_len, sink, k_scale, v_scale,
                        out, workspace, block_table, scale, stream)
    return out[:, :, 0] if one else out


def decode_multi_workspace(mode: int, window: int, batch: int, hq: int, hkv: int, q_len: int, max_seq_len: int,
                           device):
    import torch

    n = sinkattn_decode_multi_workspace_bytes(mode, window, batch, hq, hkv, q_len, max_seq_len)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device) if n else None


def decode_multi(mode: int, window: int, q, layout: int, k_cache, v_cache, seq_lens, max_seq_len: int, sink=None,
                 block_table=None, workspace=None, scale: float | None = None, stream=None):
    """Allocate out (and the workspace if none is given) and run sinkattn_decode_multi on
    q [B,Hq,q_len,192]."""
    import torch

    B, Hq, q_len, _ = q.shape
    if workspace is None:
        workspace = decode_multi_workspace(mode, window, B, Hq, k_cache.shape[1], q_len, max_seq_len, q.device)
    out = torch.empty((B, Hq, q_len, v_cache.shape[3]), dtype=torch.bfloat16, device=q.device)
    sinkattn_decode_multi(mode, window, q_len, q, layout, k_cache, v_cache, seq_lens, max_seq_len, sink, out,
                          workspace, block_table, scale, stream)
    return out
