"""Python binding of libhk_probe.so: the measurement aids of include/hk_probe.h (a plain
streaming read and a plain random-row gather), which the benchmark times beside the decode
path's kernels.  Argument marshalling only; not part of the decode path.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import HkError, _check, _need, _ptr, _stream

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_HERE, "libhk_probe.so")

_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
_SIGNATURES = {
    "hk_read_probe_sink_words": (_SZ, [_SZ]),
    "hk_read_probe": (_I, [_P, _SZ, _P, _P]),
    "hk_gather_probe_sink_words": (_SZ, [_I64, _I]),
    "hk_gather_probe": (_I, [_P, _P, _I64, _P, _I64, _I, _P, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libhk_probe.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with "
                              "`python hash_top_kv_amd/build.py`")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def read_probe(src: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """hk_read_probe: a plain streaming read of src's bytes."""
    if not src.is_cuda or not src.is_contiguous():
        raise HkError(1, "read_probe: src must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    nbytes -= nbytes % 16
    words = int(lib().hk_read_probe_sink_words(nbytes))
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=src.device)
    elif sink.numel() < words:
        raise HkError(1, "read_probe: sink too small")
    _check(lib().hk_read_probe(_ptr(src), nbytes, _ptr(sink), _stream()), "hk_read_probe")
    return sink


def gather_probe(k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, rows_per_block: int = 512,
                 sink: torch.Tensor | None = None) -> torch.Tensor:
    """hk_gather_probe: a plain gather of the 256-byte K and V rows idx.
    k, v: contiguous device tensors viewed as [table_rows][256 bytes]; idx: int32."""
    for t, nm in ((k, "k"), (v, "v"), (idx, "idx")):
        if not t.is_cuda or not t.is_contiguous():
            raise HkError(1, f"gather_probe: {nm} must be a contiguous device tensor")
    _need(idx, "idx", dtype=torch.int32)
    rows = k.numel() * k.element_size() // 256
    if v.numel() * v.element_size() // 256 != rows:
        raise HkError(1, "gather_probe: k and v differ in size")
    n = idx.numel()
    words = int(lib().hk_gather_probe_sink_words(n, rows_per_block))
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=k.device)
    elif sink.numel() < words:
        raise HkError(1, "gather_probe: sink too small")
    _check(lib().hk_gather_probe(_ptr(k), _ptr(v), rows, _ptr(idx), n, rows_per_block,
                                 _ptr(sink), _stream()), "hk_gather_probe")
    return sink
