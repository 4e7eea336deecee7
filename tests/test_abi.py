"""The C ABI without a GPU: libhk.so loads, exports every function include/hk.h
declares (and none of the measurement aids), libhk_probe.so exports those of
include/hk_probe.h, and both reject bad arguments on the host before touching HIP."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hk.h")
PROBE_HEADER = os.path.join(ROOT, "include", "hk_probe.h")


def _declared(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hk_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def hk():
    import hash_top_kv_amd
    return hash_top_kv_amd


@pytest.fixture(scope="module")
def hkp():
    from hash_top_kv_amd import probe
    return probe


def test_header_declares_the_five_calls():
    names = _declared()
    for n in ("hk_encode_keys", "hk_encode_query", "hk_retrieve_topk", "hk_sparse_decode",
              "hk_lse_merge"):
        assert n in names


def test_every_declared_symbol_is_exported(hk):
    L = ctypes.CDLL(hk.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing
    assert set(_declared()) <= set(hk._SIGNATURES), "binding lacks a declared call"


def test_probes_live_in_their_own_library(hk):
    """The measurement aids are declared in hk_probe.h and exported by libhk_probe.so
    only; the decode path's header and library hold the method alone."""
    from hash_top_kv_amd import probe
    names = _declared(PROBE_HEADER)
    assert names and not set(names) & set(_declared())
    Lp = ctypes.CDLL(probe.PROBE_LIB_PATH)
    assert all(hasattr(Lp, n) for n in names)
    assert set(names) <= set(probe._SIGNATURES)
    L = ctypes.CDLL(hk.LIB_PATH)
    assert not any(hasattr(L, n) for n in names)


def test_strerror_covers_every_status(hk):
    msgs = {hk.strerror(s) for s in range(5)}
    assert len(msgs) == 5 and "unknown status" not in msgs
    assert hk.strerror(99) == "unknown status"


def test_host_validation_without_gpu(hk):
    L = hk.lib()
    P = None
    # unsupported code width, negative sizes, context beyond capacity
    assert L.hk_retrieve_topk(P, P, 96, 1, 1, 10, 10, 0, 0, 3, P, P, P, 0, P) == hk.HK_ERR_UNSUPPORTED
    assert L.hk_retrieve_topk(P, P, 128, -1, 1, 10, 10, 0, 0, 3, P, P, P, 0, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_retrieve_topk(P, P, 128, 1, 1, 10, 11, 0, 0, 3, P, P, P, 0, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_retrieve_topk(P, P, 128, 1, 1, 10, 10, 0, 0, -3, P, P, P, 0, P) == hk.HK_ERR_INVALID_ARGUMENT
    # missing buffers, then a workspace that is too small (dummy non-null pointers)
    assert L.hk_retrieve_topk(P, P, 128, 1, 1, 10, 10, 0, 0, 3, P, P, P, 0, P) == hk.HK_ERR_INVALID_ARGUMENT
    dummy = ctypes.c_void_p(0x1000)
    assert L.hk_retrieve_topk(dummy, dummy, 128, 1, 1, 10, 10, 0, 0, 3, dummy, dummy, dummy, 1, P) \
        == hk.HK_ERR_WORKSPACE_TOO_SMALL
    # empty problems are successful no-ops
    assert L.hk_retrieve_topk(P, P, 128, 0, 8, 10, 10, 0, 0, 3, P, P, P, 0, P) == hk.HK_OK
    # hashes
    assert L.hk_encode_keys(None, P, 1, 1, 10, 0, 10, P, P) == hk.HK_ERR_INVALID_ARGUMENT
    h = hk._Hash(hk.HK_HASH_LSH, hk.HK_BF16, 128, 96, 0, dummy, P, P, P, P)
    assert L.hk_encode_keys(ctypes.byref(h), dummy, 1, 1, 10, 0, 10, dummy, P) == hk.HK_ERR_UNSUPPORTED
    h = hk._Hash(hk.HK_HASH_MLP, hk.HK_BF16, 128, 128, 128, P, dummy, P, dummy, P)
    assert L.hk_encode_keys(ctypes.byref(h), dummy, 1, 1, 10, 0, 10, dummy, P) == hk.HK_ERR_UNSUPPORTED
    h = hk._Hash(hk.HK_HASH_LSH, hk.HK_BF16, 64, 128, 0, dummy, P, P, P, P)
    assert L.hk_encode_keys(ctypes.byref(h), dummy, 1, 1, 10, 0, 10, dummy, P) == hk.HK_ERR_UNSUPPORTED
    h = hk._Hash(hk.HK_HASH_LSH, hk.HK_BF16, 128, 128, 0, P, P, P, P, P)
    assert L.hk_encode_keys(ctypes.byref(h), dummy, 1, 1, 10, 0, 10, dummy, P) == hk.HK_ERR_INVALID_ARGUMENT
    h = hk._Hash(hk.HK_HASH_LSH, hk.HK_BF16, 128, 128, 0, dummy, P, P, P, P)
    assert L.hk_encode_keys(ctypes.byref(h), dummy, 1, 1, 10, 5, 11, dummy, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_encode_keys(ctypes.byref(h), dummy, 1, 1, 10, 5, 4, dummy, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_encode_keys(ctypes.byref(h), dummy, 1, 1, 10, 5, 5, dummy, P) == hk.HK_OK
    assert L.hk_encode_query(ctypes.byref(h), dummy, 1, 30, 4, dummy, P) == hk.HK_ERR_INVALID_ARGUMENT
    # attention
    f = ctypes.c_float(0.1)
    assert L.hk_sparse_decode(dummy, dummy, dummy, hk.HK_BF16, 1, 36, 4, 128, 10, dummy, 4, P, 4, f,
                              dummy, dummy, dummy, 1 << 30, P) == hk.HK_ERR_UNSUPPORTED   # G = 9
    assert L.hk_sparse_decode(dummy, dummy, dummy, hk.HK_BF16, 1, 30, 4, 128, 10, dummy, 4, P, 4, f,
                              dummy, dummy, dummy, 1 << 30, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_sparse_decode(dummy, dummy, dummy, hk.HK_BF16, 1, 8, 4, 64, 10, dummy, 4, P, 4, f,
                              dummy, dummy, dummy, 1 << 30, P) == hk.HK_ERR_UNSUPPORTED   # d = 64
    assert L.hk_sparse_decode(dummy, dummy, dummy, 7, 1, 8, 4, 128, 10, dummy, 4, P, 4, f,
                              dummy, dummy, dummy, 1 << 30, P) == hk.HK_ERR_UNSUPPORTED
    need = L.hk_sparse_decode_workspace(64, 32, 8, 128, 4000)
    assert need > 0
    assert L.hk_sparse_decode(dummy, dummy, dummy, hk.HK_BF16, 64, 32, 8, 128, 10, dummy, 4, P, 4000,
                              f, dummy, dummy, dummy, need - 1, P) == hk.HK_ERR_WORKSPACE_TOO_SMALL
    assert L.hk_lse_merge(dummy, dummy, 0, 4, 128, dummy, dummy, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_lse_merge(dummy, dummy, 2, -1, 128, dummy, dummy, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_lse_merge(P, P, 2, 0, 128, P, P, P) == hk.HK_OK
    # misaligned vector operands
    odd = ctypes.c_void_p(0x1004)
    h = hk._Hash(hk.HK_HASH_LSH, hk.HK_BF16, 128, 128, 0, odd, P, P, P, P)
    assert L.hk_encode_keys(ctypes.byref(h), dummy, 1, 1, 10, 0, 10, dummy, P) == hk.HK_ERR_UNSUPPORTED
    h = hk._Hash(hk.HK_HASH_LSH, hk.HK_BF16, 128, 128, 0, dummy, P, P, P, P)
    assert L.hk_encode_keys(ctypes.byref(h), odd, 1, 1, 10, 0, 10, dummy, P) == hk.HK_ERR_UNSUPPORTED
    assert L.hk_encode_keys(ctypes.byref(h), dummy, 1, 1, 10, 0, 10, odd, P) == hk.HK_ERR_UNSUPPORTED
    assert L.hk_encode_query(ctypes.byref(h), odd, 1, 8, 4, dummy, P) == hk.HK_ERR_UNSUPPORTED
    wsz = L.hk_retrieve_topk_workspace(128, 1, 1, 10, 0, 0, 3)
    assert L.hk_retrieve_topk(odd, dummy, 128, 1, 1, 10, 10, 0, 0, 3, dummy, dummy, dummy, wsz, P) \
        == hk.HK_ERR_UNSUPPORTED
    assert L.hk_sparse_decode(dummy, odd, dummy, hk.HK_BF16, 1, 8, 4, 128, 10, dummy, 4, P, 4, f,
                              dummy, dummy, dummy, 1 << 30, P) == hk.HK_ERR_UNSUPPORTED
    # sign hash: 128 bits only, no weights needed
    hs = hk._Hash(hk.HK_HASH_SIGN, hk.HK_BF16, 128, 64, 0, P, P, P, P, P)
    assert L.hk_encode_keys(ctypes.byref(hs), dummy, 1, 1, 10, 0, 10, dummy, P) == hk.HK_ERR_UNSUPPORTED
    hs = hk._Hash(hk.HK_HASH_SIGN, hk.HK_BF16, 128, 128, 0, P, P, P, P, P)
    assert L.hk_encode_keys(ctypes.byref(hs), dummy, 1, 1, 10, 5, 5, dummy, P) == hk.HK_OK
    assert L.hk_encode_query(ctypes.byref(hs), dummy, 1, 30, 4, dummy, P) == hk.HK_ERR_INVALID_ARGUMENT
    # eviction: bad width / sizes, missing buffers, small workspace, misaligned rows
    assert L.hk_evict_select(P, P, 96, 1, 1, 10, 10, 0, 0, P, P, 0, P) == hk.HK_ERR_UNSUPPORTED
    assert L.hk_evict_select(P, P, 128, 1, 1, 10, 11, 0, 0, P, P, 0, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_evict_select(P, P, 128, 1, 1, 10, 10, 0, 0, P, P, 0, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_evict_select(dummy, dummy, 128, 1, 1, 5000, 5000, 0, 0, dummy, dummy, 1, P) \
        == hk.HK_ERR_WORKSPACE_TOO_SMALL
    assert L.hk_evict_select(odd, dummy, 128, 1, 1, 5000, 5000, 0, 0, dummy, dummy, 1 << 20, P) \
        == hk.HK_ERR_UNSUPPORTED
    assert L.hk_evict_select(P, P, 128, 0, 4, 10, 10, 0, 0, P, P, 0, P) == hk.HK_OK
    assert L.hk_evict_workspace(64, 4, 4, 262144, 4, 64) == 16 * 128 * 8
    assert L.hk_evict_replace(dummy, dummy, dummy, hk.HK_BF16, 128, 1, 1, 64, 10, dummy, dummy,
                              dummy, dummy, P) == hk.HK_ERR_UNSUPPORTED
    assert L.hk_evict_replace(dummy, dummy, P, hk.HK_BF16, 128, 1, 1, 128, 10, dummy, dummy,
                              dummy, dummy, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_evict_replace(odd, dummy, dummy, hk.HK_BF16, 128, 1, 1, 128, 10, dummy, dummy,
                              dummy, dummy, P) == hk.HK_ERR_UNSUPPORTED
    assert L.hk_evict_replace(P, P, P, hk.HK_BF16, 128, 0, 1, 128, 10, P, P, P, P, P) == hk.HK_OK
    # exact top-k and list intersection
    assert L.hk_exact_topk(dummy, dummy, hk.HK_BF16, 1, 8, 4, 64, 10, 10, 0, 0, 3, dummy, dummy,
                           dummy, 1 << 20, P) == hk.HK_ERR_UNSUPPORTED
    assert L.hk_exact_topk(dummy, dummy, hk.HK_BF16, 1, 7, 4, 128, 10, 10, 0, 0, 3, dummy, dummy,
                           dummy, 1 << 20, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_exact_topk(dummy, dummy, hk.HK_BF16, 1, 8, 4, 128, 5000, 5000, 0, 0, 3, dummy,
                           dummy, dummy, 1, P) == hk.HK_ERR_WORKSPACE_TOO_SMALL
    assert L.hk_exact_topk(dummy, odd, hk.HK_BF16, 1, 8, 4, 128, 5000, 5000, 0, 0, 3, dummy,
                           dummy, dummy, 1 << 30, P) == hk.HK_ERR_UNSUPPORTED
    assert L.hk_exact_topk(P, P, hk.HK_BF16, 0, 8, 4, 128, 10, 10, 0, 0, 3, P, P, P, 0, P) == hk.HK_OK
    assert L.hk_exact_topk_workspace(1, 8, 5000, 0, 0, 3) >= 8 * 5000 * 4
    assert L.hk_topk_intersect(dummy, dummy, 4, dummy, dummy, 4, -1, dummy, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_topk_intersect(P, dummy, 4, dummy, dummy, 4, 3, dummy, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_topk_intersect(P, P, 4, P, P, 4, 0, P, P) == hk.HK_OK
    # variable lengths: the lengths array is required
    assert L.hk_retrieve_attend_varlen(dummy, dummy, 128, dummy, dummy, dummy, hk.HK_BF16, 1, 8, 4,
                                       128, 10, P, 10, 0, 0, 3, f, dummy, dummy, dummy, dummy,
                                       dummy, 1 << 30, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_retrieve_attend_varlen(dummy, dummy, 128, dummy, dummy, dummy, hk.HK_BF16, 1, 8, 4,
                                       128, 10, dummy, 11, 0, 0, 3, f, dummy, dummy, dummy, dummy,
                                       dummy, 1 << 30, P) == hk.HK_ERR_INVALID_ARGUMENT
    # per-query-head retrieval and attention
    assert L.hk_retrieve_topk_qheads(P, P, 128, 1, 6, 4, 10, 10, 0, 0, 3, P, P, P, 0, P) \
        == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_retrieve_topk_qheads(P, P, 128, 1, 36, 4, 10, 10, 0, 0, 3, P, P, P, 0, P) \
        == hk.HK_ERR_UNSUPPORTED
    assert L.hk_retrieve_topk_qheads(dummy, dummy, 128, 1, 8, 4, 5000, 5000, 0, 0, 3, dummy,
                                     dummy, dummy, 1, P) == hk.HK_ERR_WORKSPACE_TOO_SMALL
    assert L.hk_retrieve_topk_qheads(P, P, 128, 0, 8, 4, 10, 10, 0, 0, 3, P, P, P, 0, P) == hk.HK_OK
    assert L.hk_sparse_decode_qheads(dummy, dummy, dummy, hk.HK_BF16, 1, 30, 4, 128, 10, dummy, 4,
                                     P, 4, f, dummy, dummy, dummy, 1 << 30, P) == hk.HK_ERR_INVALID_ARGUMENT
    assert L.hk_sparse_decode_qheads(dummy, odd, dummy, hk.HK_BF16, 1, 8, 4, 128, 10, dummy, 4,
                                     P, 4, f, dummy, dummy, dummy, 1 << 30, P) == hk.HK_ERR_UNSUPPORTED
    n = ctypes.c_int32(-1)
    assert L.hk_window_indices(100, 4, 64, P, ctypes.byref(n), P) == hk.HK_OK and n.value == 68
    assert L.hk_window_indices(-1, 4, 64, P, ctypes.byref(n), P) == hk.HK_ERR_INVALID_ARGUMENT


def test_read_probe_host_checks(hkp):
    """The read probe rejects sizes that are not whole 16-byte vectors and missing
    pointers on the host; zero bytes enqueue nothing."""
    L = hkp.lib()
    assert L.hk_read_probe_sink_words(1 << 30) == (1 << 30) // 32768
    assert L.hk_read_probe_sink_words(16) == 1
    assert L.hk_read_probe(None, 24, None, None) == 1          # not a multiple of 16
    assert L.hk_read_probe(None, 32, None, None) == 1          # NULL src / sink
    assert L.hk_read_probe(None, 0, None, None) == 0           # nothing to read
    assert L.hk_read_probe(ctypes.c_void_p(0x1008), 32, ctypes.c_void_p(0x2000), None) == 2


def test_gather_probe_host_checks(hkp):
    """The gather probe rejects bad workgroup sizes, negative counts and missing pointers
    on the host; an empty list enqueues nothing."""
    L = hkp.lib()
    P = ctypes.c_void_p(0x1000)
    assert L.hk_gather_probe_sink_words(1000, 512) == 2
    assert L.hk_gather_probe_sink_words(1024, 512) == 2
    assert L.hk_gather_probe_sink_words(1000, 500) == 0            # not a multiple of 16
    assert L.hk_gather_probe_sink_words(1000, 8192) == 0           # above 4096
    assert L.hk_gather_probe(P, P, 10, P, 5, 500, P, None) == 1    # rows per workgroup
    assert L.hk_gather_probe(P, P, 10, P, -1, 512, P, None) == 1   # negative count
    assert L.hk_gather_probe(P, P, 0, P, 5, 512, P, None) == 1     # empty table
    assert L.hk_gather_probe(None, P, 10, P, 5, 512, P, None) == 1
    assert L.hk_gather_probe(P, P, 10, None, 5, 512, P, None) == 1
    assert L.hk_gather_probe(P, P, 10, P, 0, 512, None, None) == 0  # nothing to read
    assert L.hk_gather_probe(ctypes.c_void_p(0x1008), P, 10, P, 5, 512, P, None) == 2


def test_workspace_sizes_grow_with_the_problem(hk):
    a = hk.retrieve_topk_workspace(128, 1, 8, 100000, 4, 64, 100)
    b = hk.retrieve_topk_workspace(128, 1, 8, 200000, 4, 64, 100)
    c = hk.retrieve_topk_workspace(128, 2, 8, 200000, 4, 64, 100)
    assert 0 < a < b < c
    assert hk.retrieve_topk_workspace(128, 1, 8, 100000, 4, 64, 100) >= 8 * 99932   # a byte per candidate
    assert hk.sparse_decode_workspace(1, 1, 1, 0) == 0 or hk.sparse_decode_workspace(1, 1, 1, 0) >= 0
    assert hk.sparse_decode_workspace(16, 32, 8, 2622) >= hk.sparse_decode_workspace(16, 32, 8, 100)


def test_noalloc_rejects_problems_beyond_its_array(hk):
    """hk_retrieve_attend_noalloc checks on the host that the fused step's workspace fits
    the library's 64 MiB array; a larger problem returns WORKSPACE_TOO_SMALL before any HIP
    call (none is possible here)."""
    L = hk.lib()
    d = ctypes.c_void_p(0x1000)
    f = ctypes.c_float(0.1)
    big = hk.retrieve_attend_workspace(128, 64, 8, 8, 1 << 20, 0, 0, 1024)
    assert big > (64 << 20)
    assert L.hk_retrieve_attend_noalloc(d, d, 128, d, d, d, hk.HK_BF16, 64, 8, 8, 128, 1 << 20,
                                        1 << 20, 0, 0, 1024, f, d, d, d, d, None) \
        == hk.HK_ERR_WORKSPACE_TOO_SMALL
    # argument errors come first, as for hk_retrieve_attend
    assert L.hk_retrieve_attend_noalloc(d, d, 96, d, d, d, hk.HK_BF16, 1, 8, 8, 128, 100, 100, 0, 0,
                                        10, f, d, d, d, d, None) == hk.HK_ERR_UNSUPPORTED
    assert L.hk_retrieve_attend_noalloc(d, d, 128, d, d, d, hk.HK_BF16, 1, 8, 8, 128, 100, 101, 0,
                                        0, 10, f, d, d, d, d, None) == hk.HK_ERR_INVALID_ARGUMENT
