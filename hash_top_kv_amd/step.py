"""One decode step of binary-hash retrieval attention over a resident KV cache.

Sequences the C entry points with preallocated buffers (no allocation per step, so a
step can be captured in a HIP graph):

    hk_decode_step   (hk_encode_query + hk_retrieve_attend in one call: a small scan hashes the
                      query itself, and small heads run the whole step in one workgroup)
or, through the separate calls (DecodeStep.unfused):
    hk_encode_query -> hk_retrieve_topk -> hk_sparse_decode (top-k list)
                    -> hk_sparse_decode (sink + local window) -> hk_lse_merge

Spotlight Attention (summary, Approach): query hashed, Hamming top-k over the cached
key codes, attention over the selected tokens only.  RetrievalAttention (elamur
summary: Summary; atlas summary: Approach): static window attended separately and
merged by exact log-sum-exp rescaling.
"""
from __future__ import annotations

import math

import torch

from . import (Hash, decode_step, encode_query, evict_replace, evict_select, evict_workspace,
               hamming_scan, hamming_scan_query, lse_merge, retrieve_attend_varlen,
               retrieve_attend_workspace, retrieve_topk_qheads, retrieve_topk_workspace,
               select_attend, sparse_decode, sparse_decode_qheads, sparse_decode_workspace,
               window_indices, workspace, _check, _ptr, _stream, lib)


class DecodeStep:
    def __init__(self, K: torch.Tensor, V: torch.Tensor, codes: torch.Tensor, bits: int,
                 n_ctx: int, n_sink: int, n_local: int, k: int, Hq: int,
                 hash: Hash | None = None):
        self.K, self.V, self.codes, self.bits, self.hash = K, V, codes, bits, hash
        B, Hkv, cap, d = K.shape
        self.B, self.Hkv, self.cap, self.d, self.Hq = B, Hkv, cap, d, Hq
        self.n_ctx, self.n_sink, self.n_local, self.k = n_ctx, n_sink, n_local, k
        dev = K.device
        self.keff = max(0, min(k, n_ctx - n_sink - n_local))
        self.idx = torch.zeros((B, Hkv, max(k, 1)), dtype=torch.int32, device=dev)
        self.count = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
        self.win = window_indices(n_ctx, n_sink, n_local, dev)
        self.n_win = int(self.win.numel())
        self.ws_r = workspace(retrieve_topk_workspace(bits, B, Hkv, n_ctx, n_sink, n_local, k), dev)
        wd = max(sparse_decode_workspace(B, Hq, Hkv, self.keff, d),
                 sparse_decode_workspace(B, Hq, Hkv, self.n_win, d))
        self.ws_d = workspace(wd, dev)
        self.ws_f = workspace(retrieve_attend_workspace(bits, B, Hq, Hkv, n_ctx, n_sink, n_local,
                                                        k), dev)
        self.o_parts = torch.empty((2, B, Hq, d), dtype=torch.float32, device=dev)
        self.lse_parts = torch.empty((2, B, Hq), dtype=torch.float32, device=dev)
        self.o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        self.qcodes = torch.empty((B, Hkv, bits // 32), dtype=torch.int32, device=dev)
        self.scale = 1.0 / math.sqrt(d)

    def retrieve(self, qcodes: torch.Tensor):
        L = lib()
        _check(L.hk_retrieve_topk(_ptr(self.codes), _ptr(qcodes), self.bits, self.B, self.Hkv,
                                  self.cap, self.n_ctx, self.n_sink, self.n_local, self.k,
                                  _ptr(self.idx), _ptr(self.count), _ptr(self.ws_r),
                                  self.ws_r.numel(), _stream()), "hk_retrieve_topk")

    def __call__(self, q: torch.Tensor, qcodes: torch.Tensor | None = None):
        """Returns (o [B, Hq, d], lse [B, Hq]).  Without qcodes: hk_decode_step (the query
        hash and the retrieval-attention step in one call; small heads run it in one
        workgroup each).  With qcodes given the query is not hashed: hk_hamming_scan, then
        hk_select_attend (selection, attention over the selected tokens and the window,
        merge)."""
        if qcodes is None:
            decode_step(self.hash, q, self.codes, self.K, self.V, self.n_ctx, self.n_sink,
                        self.n_local, self.k, scale=self.scale, qcodes=self.qcodes, idx=self.idx,
                        count=self.count, o=self.o, lse=self.lse, ws=self.ws_f)
            return self.o, self.lse
        self.scan(qcodes)
        return self.select_attend(q)

    # The parts of a fused step, in order (hk_retrieve_attend = scan + select_attend).
    def encode(self, q):
        return encode_query(self.hash, q, self.Hkv, self.qcodes)

    def scan_query(self, q):
        return hamming_scan_query(self.hash, q, self.codes, self.n_ctx, self.n_sink, self.n_local,
                                  self.k, self.ws_f, self.qcodes)

    def scan(self, qcodes):
        hamming_scan(self.codes, qcodes, self.bits, self.n_ctx, self.n_sink, self.n_local,
                     self.k, self.ws_f)

    def select_attend(self, q):
        select_attend(self.bits, q, self.K, self.V, self.n_ctx, self.n_sink, self.n_local,
                      self.k, self.idx, self.count, self.o, self.lse, self.ws_f, scale=self.scale)
        return self.o, self.lse

    def unfused(self, q: torch.Tensor, qcodes: torch.Tensor | None = None):
        """The same step through the separate calls: hk_encode_query, hk_retrieve_topk,
        hk_sparse_decode over the top-k list and over the window, hk_lse_merge."""
        if qcodes is None:
            qcodes = encode_query(self.hash, q, self.Hkv, self.qcodes)
        self.retrieve(qcodes)
        sparse_decode(q, self.K, self.V, self.idx, self.keff, count=self.count,
                      scale=self.scale, o=self.o_parts[0], lse=self.lse_parts[0], ws=self.ws_d)
        if self.n_win == 0:
            return self.o_parts[0], self.lse_parts[0]
        sparse_decode(q, self.K, self.V, self.win, self.n_win, idx_stride=0, scale=self.scale,
                      o=self.o_parts[1], lse=self.lse_parts[1], ws=self.ws_d)
        return lse_merge(self.o_parts, self.lse_parts, self.o, self.lse)


class EvictStep:
    """One HashEvict decode step over a fixed-budget cache (HashEvict: Abstract):

        hk_encode_query (the query)  -> hk_evict_select (victim per KV head)
        hk_encode_query (the new key, G = 1) -> hk_evict_replace (into the victim's slot)
        hk_sparse_decode over all n_ctx cached tokens

    Buffers are allocated once; a head without candidates evicts nothing and does not
    cache the current token."""

    def __init__(self, K: torch.Tensor, V: torch.Tensor, codes: torch.Tensor, bits: int,
                 n_ctx: int, n_sink: int, n_local: int, Hq: int, hash: Hash):
        self.K, self.V, self.codes, self.bits, self.hash = K, V, codes, bits, hash
        B, Hkv, cap, d = K.shape
        self.B, self.Hkv, self.cap, self.d, self.Hq = B, Hkv, cap, d, Hq
        self.n_ctx, self.n_sink, self.n_local = n_ctx, n_sink, n_local
        dev = K.device
        W = bits // 32
        self.qcodes = torch.empty((B, Hkv, W), dtype=torch.int32, device=dev)
        self.code_new = torch.empty((B, Hkv, W), dtype=torch.int32, device=dev)
        self.victim = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        self.ws_e = workspace(evict_workspace(bits, B, Hkv, n_ctx, n_sink, n_local), dev)
        self.every = torch.arange(max(n_ctx, 1), dtype=torch.int32, device=dev)
        self.ws_d = workspace(sparse_decode_workspace(B, Hq, Hkv, n_ctx, d), dev)
        self.o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        self.scale = 1.0 / math.sqrt(d)

    def select(self, q):
        encode_query(self.hash, q, self.Hkv, self.qcodes)
        return evict_select(self.codes, self.qcodes, self.bits, self.n_ctx, self.n_sink,
                            self.n_local, self.victim, self.ws_e)

    def replace(self, k_new, v_new):
        encode_query(self.hash, k_new, self.Hkv, self.code_new)
        evict_replace(k_new, v_new, self.code_new, self.victim, self.K, self.V, self.codes)

    def attend(self, q):
        return sparse_decode(q, self.K, self.V, self.every, self.n_ctx, idx_stride=0,
                             scale=self.scale, o=self.o, lse=self.lse, ws=self.ws_d)

    def __call__(self, q, k_new, v_new):
        """Returns (o [B, Hq, d], lse [B, Hq], victim [B, Hkv])."""
        self.select(q)
        self.replace(k_new, v_new)
        o, lse = self.attend(q)
        return o, lse, self.victim


class QHeadStep:
    """The decode step with one selection per query head (RetrievalAttention's GQA
    choice, elamur summary: Summary):

        hk_encode_query with Hkv = Hq (each query head's own code)
        -> hk_retrieve_topk_qheads -> hk_sparse_decode_qheads (each head over its list)
        -> hk_sparse_decode over the sink + local window -> hk_lse_merge
    """

    def __init__(self, K, V, codes, bits, n_ctx, n_sink, n_local, k, Hq, hash: Hash):
        self.K, self.V, self.codes, self.bits, self.hash = K, V, codes, bits, hash
        B, Hkv, cap, d = K.shape
        self.B, self.Hkv, self.cap, self.d, self.Hq = B, Hkv, cap, d, Hq
        self.n_ctx, self.n_sink, self.n_local, self.k = n_ctx, n_sink, n_local, k
        dev = K.device
        self.keff = max(0, min(k, n_ctx - n_sink - n_local))
        W = bits // 32
        self.qcodes = torch.empty((B, Hq, W), dtype=torch.int32, device=dev)
        self.idx = torch.zeros((B, Hq, max(k, 1)), dtype=torch.int32, device=dev)
        self.count = torch.zeros((B, Hq), dtype=torch.int32, device=dev)
        self.win = window_indices(n_ctx, n_sink, n_local, dev)
        self.n_win = int(self.win.numel())
        self.ws_r = workspace(retrieve_topk_workspace(bits, B, Hq, n_ctx, n_sink, n_local, k), dev)
        self.ws_q = workspace(sparse_decode_workspace(B, Hq, Hq, self.keff, d), dev)
        self.ws_w = workspace(sparse_decode_workspace(B, Hq, Hkv, self.n_win, d), dev)
        self.o_parts = torch.empty((2, B, Hq, d), dtype=torch.float32, device=dev)
        self.lse_parts = torch.empty((2, B, Hq), dtype=torch.float32, device=dev)
        self.o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        self.scale = 1.0 / math.sqrt(d)

    def encode(self, q):
        return encode_query(self.hash, q, self.Hq, self.qcodes)

    def retrieve(self, qcodes):
        retrieve_topk_qheads(self.codes, qcodes, self.bits, self.n_ctx, self.n_sink, self.n_local,
                             self.k, self.idx, self.count, self.ws_r)

    def attend(self, q):
        sparse_decode_qheads(q, self.K, self.V, self.idx, self.keff, count=self.count,
                             scale=self.scale, o=self.o_parts[0], lse=self.lse_parts[0], ws=self.ws_q)
        if self.n_win == 0:
            return self.o_parts[0], self.lse_parts[0]
        sparse_decode(q, self.K, self.V, self.win, self.n_win, idx_stride=0, scale=self.scale,
                      o=self.o_parts[1], lse=self.lse_parts[1], ws=self.ws_w)
        return lse_merge(self.o_parts, self.lse_parts, self.o, self.lse)

    def __call__(self, q, qcodes=None):
        """Returns (o [B, Hq, d], lse [B, Hq]); with qcodes [B, Hq, W] given the query is
        not hashed."""
        if qcodes is None:
            qcodes = self.encode(q)
        self.retrieve(qcodes)
        return self.attend(q)


class VarlenDecodeStep:
    """The decode step for a batch of sequences of their own lengths (ctx_len [B] int32 on
    the device, each <= max_ctx): hk_encode_query, then hk_retrieve_attend_varlen
    (scan, select and attend with each sequence's own candidates, budget and window)."""

    def __init__(self, K, V, codes, bits, ctx_len, max_ctx, n_sink, n_local, k, Hq,
                 hash: Hash | None = None):
        self.K, self.V, self.codes, self.bits, self.hash = K, V, codes, bits, hash
        B, Hkv, cap, d = K.shape
        self.B, self.Hkv, self.cap, self.d, self.Hq = B, Hkv, cap, d, Hq
        self.ctx_len, self.max_ctx = ctx_len, max_ctx
        self.n_sink, self.n_local, self.k = n_sink, n_local, k
        dev = K.device
        self.idx = torch.zeros((B, Hkv, max(k, 1)), dtype=torch.int32, device=dev)
        self.count = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
        self.ws = workspace(retrieve_attend_workspace(bits, B, Hq, Hkv, max_ctx, n_sink, n_local,
                                                      k), dev)
        self.o = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        self.qcodes = torch.empty((B, Hkv, bits // 32), dtype=torch.int32, device=dev)
        self.scale = 1.0 / math.sqrt(d)

    def __call__(self, q, qcodes=None):
        if qcodes is None:
            qcodes = encode_query(self.hash, q, self.Hkv, self.qcodes)
        retrieve_attend_varlen(self.codes, qcodes, self.bits, q, self.K, self.V, self.ctx_len,
                               self.max_ctx, self.n_sink, self.n_local, self.k, scale=self.scale,
                               idx=self.idx, count=self.count, o=self.o, lse=self.lse, ws=self.ws)
        return self.o, self.lse
