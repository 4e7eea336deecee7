"""CPU oracle for the binary-hash KV-cache retrieval decode step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links this
package: only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library (no kernels, headers, helpers or
constant tables); the two meet only in the seeded inputs of ``synth``.

Plain NumPy in float64, written from the definitions on the pages, one function per
step, without blocking, fusion or reordering:

* encode        sign-bit codes of a Gaussian projection ("binarized Gaussian
                projections", HashEvict: Abstract; "angular LSH", Spotlight Attention:
                Experimental setup / Builds on) or of a two-layer MLP ("sign of an MLP
                output", Spotlight Attention: Approach).
* hamming       Hamming distance between the query code and every cached key code
                (HashEvict: Abstract; "bitwise hashing retrieval", Spotlight Attention:
                Key results).
* select_topk   the per-head top-k tokens by hash distance (Spotlight Attention:
                summary and Key results, top-2% retrieval), ties broken by
                (distance ascending, token index ascending).
* attend        exact softmax attention restricted to a token set ("partial
                attention", RetrievalAttention (elamur summary): Summary).
* lse_merge     exact log-sum-exp combination of partial attentions
                (RetrievalAttention (atlas summary): Approach).

Readings of points the pages leave open (bit order, zero sign, GQA query, budgets,
window, hidden rounding, empty sets) are stated at each function.  Every function is
pinned by the ``-m "not gpu"`` tests against brute force, closed forms, invariants and
library special cases; no function here is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "widen", "round_bf16", "gelu", "prepare_hash", "project", "pack_bits", "unpack_bits",
    "encode", "group_mean_query", "encode_query", "candidate_range", "window_indices",
    "hamming", "select_topk", "attend", "sparse_attention", "lse_merge", "decode_step",
    "decode_step_qheads",
    "near_zero_mask", "evict_victim", "evict_step", "exact_topk", "exact_topk_group", "iou",
]

NEAR_ZERO = 1e-3   # |pre-sign value| below which a code bit may legitimately differ


# ---------------------------------------------------------------------------------
# Input widening.  Every input converts exactly to float64: float32 directly, bf16
# (carried as uint16 bit patterns) by placing the 16 bits above 16 zero bits.
# ---------------------------------------------------------------------------------
def widen(x, dtype: str) -> np.ndarray:
    """Exact float64 value of stored inputs ('f32' float32 array or 'bf16' uint16 bits)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, returned as float64.

    bf16 has float32's 8-bit exponent and 7 stored fraction bits.  For normal values
    this keeps the top 7 of float64's 52 fraction bits with round-half-even; below the
    bf16 normal range the grid is the subnormal spacing 2**-133.  Overflow to bf16
    infinity is not needed by the workloads and is rejected.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_bf16: non-finite input")
    if np.any(np.abs(x) >= 3.3895313892515355e38):
        raise ValueError("round_bf16: beyond the bf16 range")
    bits = np.ascontiguousarray(x).view(np.uint64)
    drop = np.uint64(45)
    lsb = (bits >> drop) & np.uint64(1)
    half_minus_one = np.uint64((1 << 44) - 1)
    rounded = ((bits + half_minus_one + lsb) >> drop) << drop
    out = rounded.view(np.float64).copy()
    tiny = np.abs(x) < 2.0 ** -126
    if np.any(tiny):
        step = 2.0 ** -133
        out[tiny] = np.round(x[tiny] / step) * step   # numpy rounds half to even
    return out


def gelu(a) -> np.ndarray:
    """GELU in its exact erf form, a * Phi(a) = a/2 * (1 + erf(a / sqrt 2))."""
    a = np.asarray(a, dtype=np.float64)
    return 0.5 * a * (1.0 + _erf(a / math.sqrt(2.0)))


# ---------------------------------------------------------------------------------
# Hash encoders (S1 keys, S2 queries)
# ---------------------------------------------------------------------------------
def prepare_hash(h: dict) -> dict:
    """Float64 view of hash parameters given in storage form.

    LSH: R [bits, d], row j gives bit j.  MLP: W1 [hidden, d], W2 [bits, hidden] in the
    [out, in] orientation, optional biases b1 [hidden], b2 [bits].  The hidden
    activation is rounded to bf16 when the hash's dtype is bf16 (a bf16 model keeps its
    activations in bf16); pre-activations and the output are never rounded.
    """
    dt = h["dtype"]
    out = {"kind": h["kind"], "bits": int(h["bits"]), "round_hidden": dt == "bf16"}
    if h["kind"] == "lsh":
        out["R"] = widen(h["R"], dt)
    elif h["kind"] == "mlp":
        out["W1"] = widen(h["W1"], dt)
        out["W2"] = widen(h["W2"], dt)
        out["b1"] = widen(h["b1"], dt) if h.get("b1") is not None else None
        out["b2"] = widen(h["b2"], dt) if h.get("b2") is not None else None
    elif h["kind"] != "sign":
        raise ValueError(h["kind"])
    return out


def project(x, hp: dict) -> np.ndarray:
    """Pre-sign values y for rows x [n, d] (float64).

    LSH (HashEvict: Abstract, "binarized Gaussian projections"): y = R x.
    MLP (Spotlight Attention: Approach, "sign of an MLP output"): y = W2 rho(GELU(W1 x
    + b1)) + b2, with rho the bf16 rounding of the hidden layer when it is bf16.
    SIGN (Self-Indexing KVCache: Abstract, "sign-based 1-bit" keys): y = x.
    """
    x = np.asarray(x, dtype=np.float64)
    if hp["kind"] == "sign":
        return x.copy()
    if hp["kind"] == "lsh":
        return x @ hp["R"].T
    a = x @ hp["W1"].T
    if hp.get("b1") is not None:
        a = a + hp["b1"]
    hidden = gelu(a)
    if hp["round_hidden"]:
        hidden = round_bf16(hidden)
    y = hidden @ hp["W2"].T
    if hp.get("b2") is not None:
        y = y + hp["b2"]
    return y


def pack_bits(bits) -> np.ndarray:
    """Pack boolean bits [..., b] into uint32 words [..., b/32].

    Bit j goes to word j // 32 at bit position j % 32 (least significant first); words
    are in increasing order and stored little-endian.
    """
    bits = np.asarray(bits, dtype=bool)
    nb = bits.shape[-1]
    if nb % 32:
        raise ValueError("bit count must be a multiple of 32")
    words = np.zeros(bits.shape[:-1] + (nb // 32,), dtype=np.uint64)
    for j in range(nb):
        words[..., j // 32] |= bits[..., j].astype(np.uint64) << np.uint64(j % 32)
    return words.astype(np.uint32)


def unpack_bits(words, nbits: int) -> np.ndarray:
    """Inverse of pack_bits."""
    words = np.asarray(words, dtype=np.uint32)
    out = np.zeros(words.shape[:-1] + (nbits,), dtype=bool)
    for j in range(nbits):
        out[..., j] = ((words[..., j // 32] >> np.uint32(j % 32)) & np.uint32(1)) == 1
    return out


def encode(x, hp: dict):
    """Codes of rows x [n, d]: bit j = [y_j > 0] (zero and NaN give 0).

    Returns (codes [n, bits/32] uint32, y [n, bits] float64) so that a checker can
    exempt bits whose pre-sign value is near zero.
    """
    y = project(x, hp)
    return pack_bits(y > 0.0), y


def near_zero_mask(y) -> np.ndarray:
    """Bits whose float64 pre-sign value satisfies |y| < 1e-3, packed like codes."""
    return pack_bits(np.abs(np.asarray(y)) < NEAR_ZERO)


def group_mean_query(q, Hkv: int) -> np.ndarray:
    """q [B, Hq, d] -> the mean query of each KV head's group [B, Hkv, d] (float64).

    One selection per KV head is shared by its G = Hq/Hkv query heads.  Its code is the
    code of the group-mean query: sum_g q_g . k = G * mean(q) . k, so the mean ranks
    keys by the group's summed logit.  Query head h belongs to KV head h // G.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    G = Hq // Hkv
    return q.reshape(B, Hkv, G, d).mean(axis=2)


def encode_query(q, hp: dict, Hkv: int):
    """Query codes [B, Hkv, bits/32] of the group-mean queries, plus their y."""
    qbar = group_mean_query(q, Hkv)
    B = qbar.shape[0]
    codes, y = encode(qbar.reshape(B * Hkv, -1), hp)
    return codes.reshape(B, Hkv, -1), y.reshape(B, Hkv, -1)


# ---------------------------------------------------------------------------------
# Token sets
# ---------------------------------------------------------------------------------
def candidate_range(n_ctx: int, n_sink: int, n_local: int) -> np.ndarray:
    """Tokens that compete in retrieval: [n_sink, n_ctx - n_local), empty if inverted.

    Sink and local-window tokens are attended separately (RetrievalAttention (elamur
    summary): Summary, tokens kept by fixed patterns), so the retrieved set and the
    window are disjoint and their merge is attention over the union.
    """
    lo, hi = n_sink, n_ctx - n_local
    return np.arange(lo, hi, dtype=np.int64) if lo < hi else np.zeros(0, dtype=np.int64)


def window_indices(n_ctx: int, n_sink: int, n_local: int) -> np.ndarray:
    """Static window [0, min(s, N)) U [max(s, N - w), N) in ascending order."""
    sink = np.arange(0, min(n_sink, n_ctx), dtype=np.int64)
    local = np.arange(max(n_sink, n_ctx - n_local), n_ctx, dtype=np.int64)
    return np.concatenate([sink, local])


# ---------------------------------------------------------------------------------
# Retrieval (S3, S4)
# ---------------------------------------------------------------------------------
def hamming(codes, qcode) -> np.ndarray:
    """D_j = number of differing bits between qcode [W] and each code [n, W]."""
    codes = np.asarray(codes, dtype=np.uint32)
    qcode = np.asarray(qcode, dtype=np.uint32)
    return np.bitwise_count(np.bitwise_xor(codes, qcode[None, :])).sum(axis=-1).astype(np.int64)


def select_topk(codes, qcode, n_ctx: int, n_sink: int, n_local: int, k: int) -> np.ndarray:
    """The k_eff = min(k, |C|) candidates nearest to qcode, in ascending token order.

    codes [>= n_ctx, W] of one (batch, KV head).  Candidates are ordered by (Hamming
    distance ascending, token index ascending), which makes the set unique; the first
    k_eff are kept and returned sorted by token index.
    """
    cand = candidate_range(n_ctx, n_sink, n_local)
    keff = max(0, min(int(k), cand.size))
    if keff == 0:
        return np.zeros(0, dtype=np.int64)
    dist = hamming(np.asarray(codes)[cand], qcode)
    order = np.argsort(dist, kind="stable")        # equal distances keep index order
    return np.sort(cand[order[:keff]])


# ---------------------------------------------------------------------------------
# Attention (S5, S6) and merge (S7)
# ---------------------------------------------------------------------------------
def attend(q, k_rows, v_rows, scale: float):
    """Exact softmax attention of one query over the given rows.

    l_j = scale * q . k_j; o = sum_j softmax(l)_j v_j; lse = ln sum_j exp(l_j).  An
    empty set gives o = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k_rows = np.asarray(k_rows, dtype=np.float64)
    v_rows = np.asarray(v_rows, dtype=np.float64)
    if k_rows.shape[0] == 0:
        return np.zeros(q.shape[-1]), -np.inf
    logits = (k_rows @ q) * scale
    m = logits.max()
    p = np.exp(logits - m)
    s = p.sum()
    return (p @ v_rows) / s, m + math.log(s)


def sparse_attention(q, K, V, idx_lists, scale: float):
    """Attention of every query head of one sequence over its KV head's token list.

    q [Hq, d]; K, V [Hkv, N, d] (float64); idx_lists[h_kv] = token indices.  Query head
    h uses KV head h // G (contiguous GQA groups) and its own query vector.
    """
    Hq = q.shape[0]
    Hkv = K.shape[0]
    G = Hq // Hkv
    o = np.zeros((Hq, q.shape[1]))
    lse = np.zeros(Hq)
    for h in range(Hq):
        kv = h // G
        idx = np.asarray(idx_lists[kv], dtype=np.int64)
        o[h], lse[h] = attend(q[h], K[kv][idx], V[kv][idx], scale)
    return o, lse


def lse_merge(o_parts, lse_parts):
    """Combine partial attentions (o_p, lse_p) of disjoint token sets exactly.

    m = max lse_p; o = sum_p e^(lse_p - m) o_p / sum_p e^(lse_p - m);
    lse = m + ln sum_p e^(lse_p - m).  Parts with lse = -inf (empty sets) contribute
    nothing; if every part is empty, o = 0 and lse = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    live = lse_parts > -np.inf
    if not np.any(live):
        return np.zeros(o_parts.shape[-1]), -np.inf
    m = lse_parts[live].max()
    w = np.exp(lse_parts[live] - m)
    return (w @ o_parts[live]) / w.sum(), m + math.log(w.sum())


def decode_step(q, K, V, key_codes, hp: dict, n_ctx: int, n_sink: int, n_local: int,
                k: int, scale: float | None = None, qcodes=None):
    """One decode step of one batch: query code, retrieval, two partials, merge.

    q [Hq, d], K, V [Hkv, >= n_ctx, d] float64, key_codes [Hkv, >= n_ctx, W].  When
    ``qcodes`` [Hkv, W] is given it replaces the query encoding (workloads whose codes
    are given directly).  Returns dict(o [Hq, d], lse [Hq], idx list per KV head,
    qcodes, qy).
    """
    Hq, d = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qy = None
    if qcodes is None:
        qc, qy = encode_query(q[None], hp, Hkv)
        qcodes, qy = qc[0], qy[0]
    idx_lists = [select_topk(key_codes[h], qcodes[h], n_ctx, n_sink, n_local, k)
                 for h in range(Hkv)]
    win = window_indices(n_ctx, n_sink, n_local)
    o1, l1 = sparse_attention(q, K, V, idx_lists, scale)
    o2, l2 = sparse_attention(q, K, V, [win] * Hkv, scale)
    o = np.zeros((Hq, d))
    lse = np.zeros(Hq)
    for h in range(Hq):
        o[h], lse[h] = lse_merge(np.stack([o1[h], o2[h]]), np.array([l1[h], l2[h]]))
    return {"o": o, "lse": lse, "idx": idx_lists, "qcodes": qcodes, "qy": qy,
            "o_topk": o1, "lse_topk": l1, "o_win": o2, "lse_win": l2, "G": G}


def decode_step_qheads(q, K, V, key_codes, hp: dict, n_ctx: int, n_sink: int, n_local: int,
                       k: int, scale: float | None = None, qcodes=None):
    """The decode step with one selection per query head (RetrievalAttention (elamur
    summary): Summary, an index per query head): query head h hashes its own query,
    selects the top-k of KV head h // G's codes by Hamming distance, attends over them
    and over the window, and the two partials are merged.

    q [Hq, d], K, V [Hkv, >= n_ctx, d], key_codes [Hkv, >= n_ctx, W]; ``qcodes`` [Hq, W]
    replaces the query hash when given.  Returns dict(o, lse, idx per query head, qcodes).
    """
    Hq, d = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if qcodes is None:
        qcodes, _ = encode(q, hp)
    win = window_indices(n_ctx, n_sink, n_local)
    o = np.zeros((Hq, d))
    lse = np.zeros(Hq)
    idx = []
    for h in range(Hq):
        kv = h // G
        sel = select_topk(key_codes[kv], qcodes[h], n_ctx, n_sink, n_local, k)
        idx.append(sel)
        o1, l1 = attend(q[h], K[kv][sel], V[kv][sel], scale)
        o2, l2 = attend(q[h], K[kv][win], V[kv][win], scale)
        o[h], lse[h] = lse_merge(np.stack([o1, o2]), np.array([l1, l2]))
    return {"o": o, "lse": lse, "idx": idx, "qcodes": qcodes}


# ---------------------------------------------------------------------------------
# Adjacent steps
# ---------------------------------------------------------------------------------
def evict_victim(codes, qcode, n_ctx: int, n_sink: int, n_local: int) -> int:
    """HashEvict's victim: the candidate most cosine-dissimilar to the query, i.e. the
    largest Hamming distance between the codes (HashEvict: Abstract).  Ties go to the
    lowest token index; -1 when there is no candidate."""
    cand = candidate_range(n_ctx, n_sink, n_local)
    if cand.size == 0:
        return -1
    dist = hamming(np.asarray(codes)[cand], qcode)
    return int(cand[int(np.argmax(dist))])        # argmax returns the first maximum


def evict_step(q, K, V, key_codes, qcodes, k_new, v_new, code_new, n_ctx: int,
               n_sink: int, n_local: int, scale: float | None = None):
    """One HashEvict decode step of one batch (HashEvict: Abstract): per KV head, the
    victim (evict_victim) has its key, value and key code replaced by the current
    token's, then every query head attends over all n_ctx cached tokens.  A head with no
    candidate evicts nothing and does not cache the current token.

    q [Hq, d]; K, V [Hkv, >= n_ctx, d] float64; key_codes [Hkv, >= n_ctx, W]; qcodes
    [Hkv, W]; k_new, v_new [Hkv, d]; code_new [Hkv, W].  The inputs are not modified.
    Returns dict(victim [Hkv], K, V, codes (updated copies), o [Hq, d], lse [Hq]).
    """
    Hq, d = q.shape
    Hkv = K.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    K, V = np.array(K, dtype=np.float64), np.array(V, dtype=np.float64)
    codes = np.array(key_codes, dtype=np.uint32)
    victim = np.full(Hkv, -1, dtype=np.int64)
    for h in range(Hkv):
        j = evict_victim(codes[h], qcodes[h], n_ctx, n_sink, n_local)
        victim[h] = j
        if j >= 0:
            K[h, j], V[h, j], codes[h, j] = k_new[h], v_new[h], code_new[h]
    every = np.arange(n_ctx, dtype=np.int64)
    o, lse = sparse_attention(q, K, V, [every] * Hkv, scale)
    return {"victim": victim, "K": K, "V": V, "codes": codes, "o": o, "lse": lse}


def iou(a, b) -> float:
    """Retrieval IoU of two token sets (Spotlight Attention: Key results): |A n B| /
    |A u B|; two empty sets give 1."""
    sa, sb = set(np.asarray(a).tolist()), set(np.asarray(b).tolist())
    union = len(sa | sb)
    return 1.0 if union == 0 else len(sa & sb) / union


def exact_topk_group(q_rows, K, n_ctx: int, n_sink: int, n_local: int, k: int) -> np.ndarray:
    """Exact top-k of one (batch, KV head) by the group's summed logit sum_g q_g . k_j over
    the candidates [n_sink, n_ctx - n_local): the exact counterpart of the hash
    retrieval, whose group-mean query ranks keys the same way.  q_rows [G, d], K [>= n_ctx,
    d].  Ascending token order."""
    cand = candidate_range(n_ctx, n_sink, n_local)
    if cand.size == 0:
        return np.zeros(0, dtype=np.int64)
    qsum = np.asarray(q_rows, dtype=np.float64).sum(axis=0)
    return exact_topk(qsum, np.asarray(K, dtype=np.float64)[cand], k, first=int(cand[0]))


def exact_topk(q, k_rows, k: int, first: int = 0) -> np.ndarray:
    """Exact top-k tokens by the logit q . k_j (the pages' "oracle top-k" / Flat
    search), ties to the lower index, ascending token order.  k_rows are the rows of
    tokens first, first+1, ..."""
    s = np.asarray(k_rows, dtype=np.float64) @ np.asarray(q, dtype=np.float64)
    keff = max(0, min(int(k), s.size))
    order = np.argsort(-s, kind="stable")
    return np.sort(order[:keff]) + first
