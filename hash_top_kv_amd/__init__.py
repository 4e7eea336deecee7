"""Python binding of libhk: binary-hash KV-cache retrieval decode path for MI355X.

Argument marshalling only.  Every computation runs in the HIP kernels of
``libhk.so``; PyTorch provides device memory and the current stream.  The functions
carry the names of the C entry points declared in ``include/hk.h``.

If ``libhk.so`` has not been built the import fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhk.so")

HK_OK, HK_ERR_INVALID_ARGUMENT, HK_ERR_UNSUPPORTED, HK_ERR_WORKSPACE_TOO_SMALL, HK_ERR_HIP = range(5)
HK_F32, HK_BF16 = 0, 1
HK_HASH_LSH, HK_HASH_MLP, HK_HASH_SIGN = 0, 1, 2


class HkError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {strerror(status)} (status {status})")
        self.status = status


class _Hash(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dtype", ctypes.c_int32), ("d", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("R", ctypes.c_void_p), ("W1", ctypes.c_void_p), ("b1", ctypes.c_void_p),
                ("W2", ctypes.c_void_p), ("b2", ctypes.c_void_p)]


_P, _I, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_SIGNATURES = {
    "hk_strerror": (ctypes.c_char_p, [_I]),
    "hk_encode_keys": (_I, [ctypes.POINTER(_Hash), _P, _I, _I, _I64, _I64, _I64, _P, _P]),
    "hk_encode_query": (_I, [ctypes.POINTER(_Hash), _P, _I, _I, _I, _P, _P]),
    "hk_retrieve_topk_workspace": (_SZ, [_I, _I, _I, _I64, _I, _I, _I]),
    "hk_retrieve_topk": (_I, [_P, _P, _I, _I, _I, _I64, _I64, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "hk_hamming_scan": (_I, [_P, _P, _I, _I, _I, _I64, _I64, _I, _I, _I, _P, _SZ, _P]),
    "hk_topk_select": (_I, [_I, _I, _I, _I64, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "hk_hamming_scan_query": (_I, [ctypes.POINTER(_Hash), _P, _I, _I, _I, _P, _I64, _I64, _I, _I,
                                   _I, _P, _P, _SZ, _P]),
    "hk_window_indices": (_I, [_I64, _I, _I, _P, ctypes.POINTER(ctypes.c_int32), _P]),
    "hk_sparse_decode_workspace": (_SZ, [_I, _I, _I, _I, _I]),
    "hk_sparse_decode": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I64, _P, _I64, _P, _I, _F,
                              _P, _P, _P, _SZ, _P]),
    "hk_lse_merge": (_I, [_P, _P, _I, _I64, _I, _P, _P, _P]),
    "hk_retrieve_attend_workspace": (_SZ, [_I, _I, _I, _I, _I64, _I, _I, _I]),
    "hk_evict_workspace": (_SZ, [_I, _I, _I, _I64, _I, _I]),
    "hk_exact_topk_workspace": (_SZ, [_I, _I, _I64, _I, _I, _I]),
    "hk_retrieve_attend_varlen": (_I, [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I64, _P, _I64,
                                       _I, _I, _I, _F, _P, _P, _P, _P, _P, _SZ, _P]),
    "hk_retrieve_topk_qheads": (_I, [_P, _P, _I, _I, _I, _I, _I64, _I64, _I, _I, _I, _P, _P, _P,
                                     _SZ, _P]),
    "hk_sparse_decode_qheads": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I64, _P, _I64, _P, _I, _F,
                                     _P, _P, _P, _SZ, _P]),
    "hk_exact_topk": (_I, [_P, _P, _I, _I, _I, _I, _I, _I64, _I64, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "hk_topk_intersect": (_I, [_P, _P, _I64, _P, _P, _I64, _I, _P, _P]),
    "hk_evict_select": (_I, [_P, _P, _I, _I, _I, _I64, _I64, _I, _I, _P, _P, _SZ, _P]),
    "hk_evict_replace": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I64, _P, _P, _P, _P, _P]),
    "hk_select_attend": (_I, [_I, _P, _P, _P, _I, _I, _I, _I, _I, _I64, _I64, _I, _I, _I, _F,
                              _P, _P, _P, _P, _P, _SZ, _P]),
    "hk_retrieve_attend": (_I, [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I64, _I64, _I, _I,
                                _I, _F, _P, _P, _P, _P, _P, _SZ, _P]),
    "hk_retrieve_attend_noalloc": (_I, [_P, _P, _I, _P, _P, _P, _I, _I, _I, _I, _I, _I64, _I64,
                                        _I, _I, _I, _F, _P, _P, _P, _P, _P]),
    "hk_decode_step": (_I, [ctypes.POINTER(_Hash), _P, _P, _P, _P, _I, _I, _I, _I, _I64, _I64, _I,
                            _I, _I, _F, _P, _P, _P, _P, _P, _P, _SZ, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libhk.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python hash_top_kv_amd/build.py` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


lib()   # fail at import time if the native library is absent


def strerror(status: int) -> str:
    return lib().hk_strerror(int(status)).decode()


def _check(status: int, where: str):
    if status != HK_OK:
        raise HkError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return HK_F32
    if t.dtype == torch.bfloat16:
        return HK_BF16
    raise TypeError(f"unsupported element type {t.dtype} (float32 or bfloat16)")


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class Hash:
    """Hash parameters on the device: LSH (R [bits, d]), MLP (W1 [256, d], W2 [bits,
    256], optional b1, b2), or SIGN (no parameters: bit j is the sign of element j, bits
    = d = 128; give its element type as dtype).  All tensors share one dtype (float32 or
    bfloat16)."""

    def __init__(self, kind: str, bits: int, R=None, W1=None, W2=None, b1=None, b2=None,
                 dtype=None):
        self.kind = kind
        self.bits = int(bits)
        self.R, self.W1, self.W2, self.b1, self.b2 = R, W1, W2, b1, b2
        if kind == "sign":
            if dtype is None:
                raise ValueError("a sign hash needs its element type (dtype)")
            self.dtype = dtype
            code = HK_HASH_SIGN
        else:
            ref = R if kind == "lsh" else W1
            if ref is None:
                raise ValueError("missing hash weights")
            self.dtype = ref.dtype
            code = HK_HASH_LSH if kind == "lsh" else HK_HASH_MLP
        for name in ("R", "W1", "W2", "b1", "b2"):
            t = getattr(self, name)
            if t is not None:
                _need(t, name, dtype=self.dtype)
        dcode = HK_BF16 if self.dtype == torch.bfloat16 else HK_F32
        self._s = _Hash(code, dcode, 128, self.bits, 256 if kind == "mlp" else 0,
                        _ptr(R), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2))

    @property
    def words(self) -> int:
        return self.bits // 32

    def struct(self) -> _Hash:
        return self._s


def encode_keys(h: Hash, k: torch.Tensor, codes: torch.Tensor, t0: int = 0, t1: int | None = None):
    """hk_encode_keys: codes[b, g, t0:t1] = hash codes of k[b, g, t0:t1].
    k [B, Hkv, cap, 128] (h.dtype), codes [B, Hkv, cap, bits/32] int32 (uint32 bits)."""
    _need(k, "k", dtype=h.dtype)
    B, Hkv, cap, d = k.shape
    _need(codes, "codes", dtype=torch.int32, shape=(B, Hkv, cap, h.words))
    t1 = cap if t1 is None else t1
    _check(lib().hk_encode_keys(ctypes.byref(h.struct()), _ptr(k), B, Hkv, cap, t0, t1,
                                _ptr(codes), _stream()), "hk_encode_keys")
    return codes


def encode_query(h: Hash, q: torch.Tensor, Hkv: int, qcodes: torch.Tensor | None = None):
    """hk_encode_query: codes of the group-mean query of each KV head.
    q [B, Hq, 128] (h.dtype) -> qcodes [B, Hkv, bits/32] int32."""
    _need(q, "q", dtype=h.dtype)
    B, Hq, d = q.shape
    if qcodes is None:
        qcodes = torch.empty((B, Hkv, h.words), dtype=torch.int32, device=q.device)
    _need(qcodes, "qcodes", dtype=torch.int32, shape=(B, Hkv, h.words))
    _check(lib().hk_encode_query(ctypes.byref(h.struct()), _ptr(q), B, Hq, Hkv, _ptr(qcodes),
                                 _stream()), "hk_encode_query")
    return qcodes


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device workspace of nbytes (at least 1).  The calls do not depend on its
    contents on entry; it is zero-filled only so that padding bytes are deterministic."""
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def retrieve_topk_workspace(bits, B, Hkv, n_ctx, n_sink, n_local, k) -> int:
    return int(lib().hk_retrieve_topk_workspace(bits, B, Hkv, n_ctx, n_sink, n_local, k))


def _topk_buffers(B, Hkv, k, device, idx, count, ws, ws_bytes):
    if idx is None:
        idx = torch.empty((B, Hkv, max(k, 1)), dtype=torch.int32, device=device)
    if count is None:
        count = torch.empty((B, Hkv), dtype=torch.int32, device=device)
    if ws is None:
        ws = workspace(ws_bytes, device)
    _need(idx, "idx", dtype=torch.int32)
    if idx.shape[:2] != (B, Hkv) or idx.shape[2] < k:
        raise ValueError("idx must be [B, Hkv, >= k]")
    if idx.shape[2] != max(k, 1) and k > 0:
        raise ValueError("idx rows must have exactly k entries")
    _need(count, "count", dtype=torch.int32, shape=(B, Hkv))
    _need(ws, "ws", dtype=torch.uint8)
    return idx, count, ws


def retrieve_topk(codes: torch.Tensor, qcodes: torch.Tensor, bits: int, n_ctx: int,
                  n_sink: int, n_local: int, k: int, idx=None, count=None, ws=None):
    """hk_retrieve_topk over codes [B, Hkv, cap, bits/32] with qcodes [B, Hkv, bits/32].
    Returns (idx [B, Hkv, k] int32 ascending in the first count entries, count [B, Hkv])."""
    _need(codes, "codes", dtype=torch.int32)
    B, Hkv, cap, W = codes.shape
    _need(qcodes, "qcodes", dtype=torch.int32, shape=(B, Hkv, W))
    wsb = retrieve_topk_workspace(bits, B, Hkv, n_ctx, n_sink, n_local, k)
    idx, count, ws = _topk_buffers(B, Hkv, k, codes.device, idx, count, ws, wsb)
    _check(lib().hk_retrieve_topk(_ptr(codes), _ptr(qcodes), bits, B, Hkv, cap, n_ctx, n_sink,
                                  n_local, k, _ptr(idx), _ptr(count), _ptr(ws), ws.numel(),
                                  _stream()), "hk_retrieve_topk")
    return idx, count


def hamming_scan(codes, qcodes, bits, n_ctx, n_sink, n_local, k, ws):
    """hk_hamming_scan: the scan half of hk_retrieve_topk (distances + histograms in ws)."""
    _need(codes, "codes", dtype=torch.int32)
    B, Hkv, cap, W = codes.shape
    _need(qcodes, "qcodes", dtype=torch.int32, shape=(B, Hkv, W))
    _need(ws, "ws", dtype=torch.uint8)
    _check(lib().hk_hamming_scan(_ptr(codes), _ptr(qcodes), bits, B, Hkv, cap, n_ctx, n_sink,
                                 n_local, k, _ptr(ws), ws.numel(), _stream()), "hk_hamming_scan")


def hamming_scan_query(h: Hash, q, codes, n_ctx, n_sink, n_local, k, ws, qcodes=None):
    """hk_hamming_scan_query: hk_encode_query + hk_hamming_scan in one call (the scan
    hashes the query itself when it is small).  Returns qcodes [B, Hkv, bits/32], the
    codes the scan used."""
    _need(q, "q", dtype=h.dtype)
    _need(codes, "codes", dtype=torch.int32)
    B, Hkv, cap, W = codes.shape
    Hq = q.shape[1]
    if qcodes is None:
        qcodes = torch.empty((B, Hkv, h.words), dtype=torch.int32, device=q.device)
    _need(qcodes, "qcodes", dtype=torch.int32, shape=(B, Hkv, h.words))
    _need(ws, "ws", dtype=torch.uint8)
    _check(lib().hk_hamming_scan_query(ctypes.byref(h.struct()), _ptr(q), B, Hq, Hkv, _ptr(codes),
                                       cap, n_ctx, n_sink, n_local, k, _ptr(qcodes), _ptr(ws),
                                       ws.numel(), _stream()), "hk_hamming_scan_query")
    return qcodes


def topk_select(bits, B, Hkv, n_ctx, n_sink, n_local, k, idx, count, ws):
    """hk_topk_select: the select half of hk_retrieve_topk."""
    _need(idx, "idx", dtype=torch.int32)
    _need(count, "count", dtype=torch.int32, shape=(B, Hkv))
    _need(ws, "ws", dtype=torch.uint8)
    _check(lib().hk_topk_select(bits, B, Hkv, n_ctx, n_sink, n_local, k, _ptr(idx), _ptr(count),
                                _ptr(ws), ws.numel(), _stream()), "hk_topk_select")


def window_size(n_ctx: int, n_sink: int, n_local: int) -> int:
    """Size of the static window, from hk_window_indices with no output list."""
    n = ctypes.c_int32(0)
    _check(lib().hk_window_indices(n_ctx, n_sink, n_local, None, ctypes.byref(n), None),
           "hk_window_indices")
    return int(n.value)


def window_indices(n_ctx: int, n_sink: int, n_local: int, device) -> torch.Tensor:
    """hk_window_indices: int32 [n] tokens [0, min(s, N)) U [max(s, N - w), N)."""
    n_host = window_size(n_ctx, n_sink, n_local)
    idx = torch.empty(max(n_host, 1), dtype=torch.int32, device=device)
    n = ctypes.c_int32(0)
    _check(lib().hk_window_indices(n_ctx, n_sink, n_local, _ptr(idx), ctypes.byref(n), _stream()),
           "hk_window_indices")
    assert n.value == n_host
    return idx[:n.value]


def sparse_decode_workspace(B, Hq, Hkv, max_count, d: int = 128) -> int:
    return int(lib().hk_sparse_decode_workspace(B, Hq, Hkv, d, max_count))


def sparse_decode(q, k, v, idx, max_count: int, count=None, idx_stride=None, scale=None,
                  o=None, lse=None, ws=None):
    """hk_sparse_decode: attention of q [B, Hq, 128] over token lists of k, v
    [B, Hkv, cap, 128].  idx is [B, Hkv, stride] (or a shared 1-D list with
    idx_stride=0); count [B, Hkv] or None (= max_count each).
    Returns (o [B, Hq, 128] float32, lse [B, Hq] float32)."""
    dt = _dtype_code(q)
    _need(q, "q")
    _need(k, "k", dtype=q.dtype)
    _need(v, "v", dtype=q.dtype, shape=k.shape)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    _need(idx, "idx", dtype=torch.int32)
    if idx_stride is None:
        idx_stride = idx.shape[-1] if idx.dim() == 3 else 0
    if count is not None:
        _need(count, "count", dtype=torch.int32, shape=(B, Hkv))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(o, "o", dtype=torch.float32, shape=(B, Hq, d))
    _need(lse, "lse", dtype=torch.float32, shape=(B, Hq))
    wsb = sparse_decode_workspace(B, Hq, Hkv, max_count, d)
    if ws is None:
        ws = workspace(wsb, q.device)
    _need(ws, "ws", dtype=torch.uint8)
    _check(lib().hk_sparse_decode(_ptr(q), _ptr(k), _ptr(v), dt, B, Hq, Hkv, d, cap, _ptr(idx),
                                  idx_stride, _ptr(count), max_count, float(scale), _ptr(o),
                                  _ptr(lse), _ptr(ws), ws.numel(), _stream()), "hk_sparse_decode")
    return o, lse


def lse_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, o=None, lse=None):
    """hk_lse_merge: o_parts [P, rows..., d], lse_parts [P, rows...] float32."""
    _need(o_parts, "o_parts", dtype=torch.float32)
    _need(lse_parts, "lse_parts", dtype=torch.float32)
    P = o_parts.shape[0]
    d = o_parts.shape[-1]
    rows = lse_parts[0].numel()
    if tuple(o_parts.shape[:-1]) != tuple(lse_parts.shape):
        raise ValueError("o_parts must be lse_parts.shape + (d,)")
    if o is None:
        o = torch.empty(o_parts.shape[1:], dtype=torch.float32, device=o_parts.device)
    if lse is None:
        lse = torch.empty(lse_parts.shape[1:], dtype=torch.float32, device=o_parts.device)
    _need(o, "o", dtype=torch.float32, shape=o_parts.shape[1:])
    _need(lse, "lse", dtype=torch.float32, shape=lse_parts.shape[1:])
    _check(lib().hk_lse_merge(_ptr(o_parts), _ptr(lse_parts), P, rows, d, _ptr(o), _ptr(lse),
                              _stream()), "hk_lse_merge")
    return o, lse


def retrieve_attend_workspace(bits, B, Hq, Hkv, n_ctx, n_sink, n_local, k) -> int:
    return int(lib().hk_retrieve_attend_workspace(bits, B, Hq, Hkv, n_ctx, n_sink, n_local, k))


def decode_step(h: Hash, q, codes, k, v, n_ctx, n_sink, n_local, topk, scale=None, qcodes=None,
                idx=None, count=None, o=None, lse=None, ws=None):
    """hk_decode_step: the whole step from the query (query hash, Hamming top-k, attention
    over the selected tokens and the window).  Returns (o [B, Hq, 128], lse [B, Hq], idx,
    count, qcodes)."""
    _need(codes, "codes", dtype=torch.int32)
    B, Hkv, cap, W = codes.shape
    _need(q, "q", dtype=h.dtype)
    _need(k, "k", dtype=h.dtype)
    _need(v, "v", dtype=h.dtype, shape=k.shape)
    Hq, d = q.shape[1], q.shape[2]
    if tuple(k.shape[:3]) != (B, Hkv, cap):
        raise ValueError("k must be [B, Hkv, cap, d] like the codes")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    wsb = retrieve_attend_workspace(h.bits, B, Hq, Hkv, n_ctx, n_sink, n_local, topk)
    idx, count, ws = _topk_buffers(B, Hkv, topk, codes.device, idx, count, ws, wsb)
    if qcodes is None:
        qcodes = torch.empty((B, Hkv, h.words), dtype=torch.int32, device=q.device)
    _need(qcodes, "qcodes", dtype=torch.int32, shape=(B, Hkv, h.words))
    if o is None:
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(o, "o", dtype=torch.float32, shape=(B, Hq, d))
    _need(lse, "lse", dtype=torch.float32, shape=(B, Hq))
    _check(lib().hk_decode_step(ctypes.byref(h.struct()), _ptr(q), _ptr(codes), _ptr(k), _ptr(v),
                                B, Hq, Hkv, d, cap, n_ctx, n_sink, n_local, topk, float(scale),
                                _ptr(qcodes), _ptr(idx), _ptr(count), _ptr(o), _ptr(lse), _ptr(ws),
                                ws.numel(), _stream()), "hk_decode_step")
    return o, lse, idx, count, qcodes


def retrieve_attend(codes, qcodes, bits, q, k, v, n_ctx, n_sink, n_local, topk, scale=None,
                    idx=None, count=None, o=None, lse=None, ws=None):
    """hk_retrieve_attend: Hamming top-k + attention over the selected tokens and the
    sink/local window, merged.  Returns (o [B, Hq, 128], lse [B, Hq], idx, count)."""
    _need(codes, "codes", dtype=torch.int32)
    B, Hkv, cap, W = codes.shape
    _need(qcodes, "qcodes", dtype=torch.int32, shape=(B, Hkv, W))
    dt = _dtype_code(q)
    _need(q, "q")
    _need(k, "k", dtype=q.dtype)
    _need(v, "v", dtype=q.dtype, shape=k.shape)
    Hq, d = q.shape[1], q.shape[2]
    if tuple(k.shape[:3]) != (B, Hkv, cap):
        raise ValueError("k must be [B, Hkv, cap, d] like the codes")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    wsb = retrieve_attend_workspace(bits, B, Hq, Hkv, n_ctx, n_sink, n_local, topk)
    idx, count, ws = _topk_buffers(B, Hkv, topk, codes.device, idx, count, ws, wsb)
    if o is None:
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(o, "o", dtype=torch.float32, shape=(B, Hq, d))
    _need(lse, "lse", dtype=torch.float32, shape=(B, Hq))
    _check(lib().hk_retrieve_attend(_ptr(codes), _ptr(qcodes), bits, _ptr(q), _ptr(k), _ptr(v), dt,
                                    B, Hq, Hkv, d, cap, n_ctx, n_sink, n_local, topk, float(scale),
                                    _ptr(idx), _ptr(count), _ptr(o), _ptr(lse), _ptr(ws),
                                    ws.numel(), _stream()), "hk_retrieve_attend")
    return o, lse, idx, count


def retrieve_attend_noalloc(codes, qcodes, bits, q, k, v, n_ctx, n_sink, n_local, topk,
                            scale=None, idx=None, count=None, o=None, lse=None):
    """hk_retrieve_attend_noalloc: hk_retrieve_attend with the library's own workspace (a
    fixed array on each GPU), for callers that cannot allocate.  Returns (o, lse, idx,
    count); the outputs are allocated here only when not given."""
    _need(codes, "codes", dtype=torch.int32)
    B, Hkv, cap, W = codes.shape
    _need(qcodes, "qcodes", dtype=torch.int32, shape=(B, Hkv, W))
    dt = _dtype_code(q)
    _need(q, "q")
    _need(k, "k", dtype=q.dtype)
    _need(v, "v", dtype=q.dtype, shape=k.shape)
    Hq, d = q.shape[1], q.shape[2]
    if tuple(k.shape[:3]) != (B, Hkv, cap):
        raise ValueError("k must be [B, Hkv, cap, d] like the codes")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if idx is None:
        idx = torch.empty((B, Hkv, max(topk, 1)), dtype=torch.int32, device=codes.device)
    if count is None:
        count = torch.empty((B, Hkv), dtype=torch.int32, device=codes.device)
    if o is None:
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(idx, "idx", dtype=torch.int32)
    _need(count, "count", dtype=torch.int32, shape=(B, Hkv))
    _need(o, "o", dtype=torch.float32, shape=(B, Hq, d))
    _need(lse, "lse", dtype=torch.float32, shape=(B, Hq))
    _check(lib().hk_retrieve_attend_noalloc(
        _ptr(codes), _ptr(qcodes), bits, _ptr(q), _ptr(k), _ptr(v), dt, B, Hq, Hkv, d, cap, n_ctx,
        n_sink, n_local, topk, float(scale), _ptr(idx), _ptr(count), _ptr(o), _ptr(lse),
        _stream()), "hk_retrieve_attend_noalloc")
    return o, lse, idx, count


def retrieve_attend_varlen(codes, qcodes, bits, q, k, v, ctx_len, max_ctx, n_sink, n_local, topk,
                           scale=None, idx=None, count=None, o=None, lse=None, ws=None):
    """hk_retrieve_attend_varlen: as retrieve_attend, with sequence b holding ctx_len[b]
    tokens (int32 device tensor [B], each <= max_ctx)."""
    _need(codes, "codes", dtype=torch.int32)
    B, Hkv, cap, W = codes.shape
    _need(qcodes, "qcodes", dtype=torch.int32, shape=(B, Hkv, W))
    _need(ctx_len, "ctx_len", dtype=torch.int32, shape=(B,))
    dt = _dtype_code(q)
    _need(q, "q")
    _need(k, "k", dtype=q.dtype)
    _need(v, "v", dtype=q.dtype, shape=k.shape)
    Hq, d = q.shape[1], q.shape[2]
    if tuple(k.shape[:3]) != (B, Hkv, cap):
        raise ValueError("k must be [B, Hkv, cap, d] like the codes")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    wsb = retrieve_attend_workspace(bits, B, Hq, Hkv, max_ctx, n_sink, n_local, topk)
    idx, count, ws = _topk_buffers(B, Hkv, topk, codes.device, idx, count, ws, wsb)
    if o is None:
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(o, "o", dtype=torch.float32, shape=(B, Hq, d))
    _need(lse, "lse", dtype=torch.float32, shape=(B, Hq))
    _check(lib().hk_retrieve_attend_varlen(_ptr(codes), _ptr(qcodes), bits, _ptr(q), _ptr(k),
                                           _ptr(v), dt, B, Hq, Hkv, d, cap, _ptr(ctx_len), max_ctx,
                                           n_sink, n_local, topk, float(scale), _ptr(idx),
                                           _ptr(count), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(),
                                           _stream()), "hk_retrieve_attend_varlen")
    return o, lse, idx, count


def select_attend(bits, q, k, v, n_ctx, n_sink, n_local, topk, idx, count, o, lse, ws,
                  scale=None):
    """hk_select_attend: the part of hk_retrieve_attend after hk_hamming_scan (same ws)."""
    dt = _dtype_code(q)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (idx, "idx"), (count, "count"), (o, "o"),
                 (lse, "lse"), (ws, "ws")):
        _need(t, n)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(lib().hk_select_attend(bits, _ptr(q), _ptr(k), _ptr(v), dt, B, Hq, Hkv, d, cap, n_ctx,
                                  n_sink, n_local, topk, float(scale), _ptr(idx), _ptr(count),
                                  _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream()),
           "hk_select_attend")
    return o, lse


def evict_workspace(bits, B, Hkv, n_ctx, n_sink, n_local) -> int:
    return int(lib().hk_evict_workspace(bits, B, Hkv, n_ctx, n_sink, n_local))


def evict_select(codes, qcodes, bits, n_ctx, n_sink, n_local, victim=None, ws=None):
    """hk_evict_select: per head, the candidate farthest from the query code (HashEvict's
    victim), lowest index on ties, -1 without candidates.  Returns victim [B, Hkv] int32."""
    _need(codes, "codes", dtype=torch.int32)
    B, Hkv, cap, W = codes.shape
    _need(qcodes, "qcodes", dtype=torch.int32, shape=(B, Hkv, W))
    if victim is None:
        victim = torch.empty((B, Hkv), dtype=torch.int32, device=codes.device)
    _need(victim, "victim", dtype=torch.int32, shape=(B, Hkv))
    if ws is None:
        ws = workspace(evict_workspace(bits, B, Hkv, n_ctx, n_sink, n_local), codes.device)
    _need(ws, "ws", dtype=torch.uint8)
    _check(lib().hk_evict_select(_ptr(codes), _ptr(qcodes), bits, B, Hkv, cap, n_ctx, n_sink,
                                 n_local, _ptr(victim), _ptr(ws), ws.numel(), _stream()),
           "hk_evict_select")
    return victim


def evict_replace(k_new, v_new, code_new, victim, k, v, codes):
    """hk_evict_replace: the new token's key, value and key code take the victim's slot
    of each head.  k_new, v_new [B, Hkv, 128]; code_new [B, Hkv, bits/32]; victim
    [B, Hkv]; k, v [B, Hkv, cap, 128] and codes [B, Hkv, cap, bits/32] are updated."""
    B, Hkv, cap, d = k.shape
    W = codes.shape[-1]
    _need(k, "k")
    _need(v, "v", dtype=k.dtype, shape=k.shape)
    _need(k_new, "k_new", dtype=k.dtype, shape=(B, Hkv, d))
    _need(v_new, "v_new", dtype=k.dtype, shape=(B, Hkv, d))
    _need(codes, "codes", dtype=torch.int32, shape=(B, Hkv, cap, W))
    _need(code_new, "code_new", dtype=torch.int32, shape=(B, Hkv, W))
    _need(victim, "victim", dtype=torch.int32, shape=(B, Hkv))
    _check(lib().hk_evict_replace(_ptr(k_new), _ptr(v_new), _ptr(code_new), _dtype_code(k), 32 * W,
                                  B, Hkv, d, cap, _ptr(victim), _ptr(k), _ptr(v), _ptr(codes),
                                  _stream()), "hk_evict_replace")


def exact_topk_workspace(B, Hkv, n_ctx, n_sink, n_local, k) -> int:
    return int(lib().hk_exact_topk_workspace(B, Hkv, n_ctx, n_sink, n_local, k))


def exact_topk(q, k, n_ctx, n_sink, n_local, topk, idx=None, count=None, ws=None):
    """hk_exact_topk: per KV head, the top-k candidates by the group's summed logit (the
    exact "oracle top-k"), ascending.  q [B, Hq, 128], k [B, Hkv, cap, 128].  Returns
    (idx [B, Hkv, topk], count [B, Hkv])."""
    _need(q, "q")
    _need(k, "k", dtype=q.dtype)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    wsb = exact_topk_workspace(B, Hkv, n_ctx, n_sink, n_local, topk)
    idx, count, ws = _topk_buffers(B, Hkv, topk, q.device, idx, count, ws, wsb)
    _check(lib().hk_exact_topk(_ptr(q), _ptr(k), _dtype_code(q), B, Hq, Hkv, d, cap, n_ctx,
                               n_sink, n_local, topk, _ptr(idx), _ptr(count), _ptr(ws), ws.numel(),
                               _stream()), "hk_exact_topk")
    return idx, count


def topk_intersect(a, count_a, b, count_b, inter=None):
    """hk_topk_intersect: |A_l n B_l| for the ascending lists a[..., l, :count_a] and
    b[..., l, :count_b] (leading dimensions flattened into lists).  Returns int32 [lists]."""
    for t, n in ((a, "a"), (count_a, "count_a"), (b, "b"), (count_b, "count_b")):
        _need(t, n, dtype=torch.int32)
    n = count_a.numel()
    if count_b.numel() != n or a.numel() != n * a.shape[-1] or b.numel() != n * b.shape[-1]:
        raise ValueError("a, b, count_a and count_b must describe the same number of lists")
    if inter is None:
        inter = torch.empty(n, dtype=torch.int32, device=a.device)
    _need(inter, "inter", dtype=torch.int32, shape=(n,))
    _check(lib().hk_topk_intersect(_ptr(a), _ptr(count_a), a.shape[-1], _ptr(b), _ptr(count_b),
                                   b.shape[-1], n, _ptr(inter), _stream()), "hk_topk_intersect")
    return inter


def retrieve_topk_qheads(codes, qcodes, bits, n_ctx, n_sink, n_local, k, idx=None, count=None,
                         ws=None):
    """hk_retrieve_topk_qheads: one top-k set per query head.  codes [B, Hkv, cap, W],
    qcodes [B, Hq, W] (each query head's own code).  Returns (idx [B, Hq, k], count [B, Hq])."""
    _need(codes, "codes", dtype=torch.int32)
    B, Hkv, cap, W = codes.shape
    _need(qcodes, "qcodes", dtype=torch.int32)
    Hq = qcodes.shape[1]
    if tuple(qcodes.shape) != (B, Hq, W):
        raise ValueError("qcodes must be [B, Hq, bits/32]")
    wsb = retrieve_topk_workspace(bits, B, Hq, n_ctx, n_sink, n_local, k)
    idx, count, ws = _topk_buffers(B, Hq, k, codes.device, idx, count, ws, wsb)
    _check(lib().hk_retrieve_topk_qheads(_ptr(codes), _ptr(qcodes), bits, B, Hq, Hkv, cap, n_ctx,
                                         n_sink, n_local, k, _ptr(idx), _ptr(count), _ptr(ws),
                                         ws.numel(), _stream()), "hk_retrieve_topk_qheads")
    return idx, count


def sparse_decode_qheads(q, k, v, idx, max_count, count=None, scale=None, o=None, lse=None,
                         ws=None):
    """hk_sparse_decode_qheads: query head h attends over its own list idx[b, h, :count]
    with the rows of KV head h // G.  Returns (o [B, Hq, 128], lse [B, Hq])."""
    dt = _dtype_code(q)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    _need(q, "q")
    _need(k, "k", dtype=q.dtype)
    _need(v, "v", dtype=q.dtype, shape=k.shape)
    _need(idx, "idx", dtype=torch.int32)
    if idx.shape[:2] != (B, Hq):
        raise ValueError("idx must be [B, Hq, n]")
    if count is not None:
        _need(count, "count", dtype=torch.int32, shape=(B, Hq))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(sparse_decode_workspace(B, Hq, Hq, max_count, d), q.device)
    _check(lib().hk_sparse_decode_qheads(_ptr(q), _ptr(k), _ptr(v), dt, B, Hq, Hkv, d, cap,
                                         _ptr(idx), idx.shape[-1], _ptr(count), max_count,
                                         float(scale), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(),
                                         _stream()), "hk_sparse_decode_qheads")
    return o, lse
