"""Pins of the oracle's restricted softmax attention and log-sum-exp merge."""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle


def _rand_head(rng, n, d=128):
    return rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))


def test_all_tokens_equal_dense_attention_library():
    """k = N with no window is dense attention; compare with SciPy's softmax and
    logsumexp over all logits."""
    rng = np.random.default_rng(31)
    for n in (1, 2, 17, 500):
        q, K, V = _rand_head(rng, n)
        scale = 1 / math.sqrt(128)
        logits = K @ q * scale
        o, lse = oracle.attend(q, K[np.arange(n)], V[np.arange(n)], scale)
        assert np.allclose(o, softmax(logits) @ V, rtol=0, atol=1e-12)
        assert abs(lse - logsumexp(logits)) < 1e-12


def test_two_token_closed_form_pins_scale():
    """q = sqrt(d) ln3 e0, k0 = e0, k1 = 0: logits (ln 3, 0) at scale 1/sqrt(d), so
    weights are 3/4 and 1/4 and lse = ln 4."""
    d = 128
    q = np.zeros(d)
    q[0] = math.sqrt(d) * math.log(3)
    K = np.zeros((2, d))
    K[0, 0] = 1.0
    V = np.zeros((2, d))
    V[0, :] = 1.0
    V[1, :] = -3.0
    o, lse = oracle.attend(q, K, V, 1 / math.sqrt(d))
    assert np.allclose(o, 0.75 * 1.0 + 0.25 * -3.0, atol=1e-14)
    assert abs(lse - math.log(4)) < 1e-14


def test_single_token_and_identical_keys():
    rng = np.random.default_rng(32)
    q, K, V = _rand_head(rng, 40)
    scale = 0.0883883
    o, lse = oracle.attend(q, K[7:8], V[7:8], scale)
    assert np.array_equal(o, V[7]) and abs(lse - scale * float(K[7] @ q)) < 1e-12
    Ks = np.repeat(K[:1], 40, axis=0)
    o, lse = oracle.attend(q, Ks, V, scale)
    assert np.allclose(o, V.mean(axis=0), atol=1e-12)
    assert abs(lse - (scale * float(K[0] @ q) + math.log(40))) < 1e-12


def test_empty_set():
    o, lse = oracle.attend(np.ones(128), np.zeros((0, 128)), np.zeros((0, 128)), 0.1)
    assert lse == -np.inf and np.array_equal(o, np.zeros(128))


def test_permutation_invariance():
    rng = np.random.default_rng(33)
    q, K, V = _rand_head(rng, 64)
    idx = rng.choice(64, 20, replace=False)
    o1, l1 = oracle.attend(q, K[idx], V[idx], 0.1)
    p = rng.permutation(idx)
    o2, l2 = oracle.attend(q, K[p], V[p], 0.1)
    assert np.allclose(o1, o2, atol=1e-13) and abs(l1 - l2) < 1e-13


def test_gqa_head_mapping():
    """Query head h reads KV head h // G: with one token per KV head, o_h = V[h//G]."""
    rng = np.random.default_rng(34)
    Hq, Hkv, d = 8, 2, 128
    q = rng.standard_normal((Hq, d))
    K = rng.standard_normal((Hkv, 5, d))
    V = rng.standard_normal((Hkv, 5, d))
    o, lse = oracle.sparse_attention(q, K, V, [[3], [1]], 0.1)
    for h in range(Hq):
        kv, j = (0, 3) if h < 4 else (1, 1)
        assert np.array_equal(o[h], V[kv, j])
        assert abs(lse[h] - 0.1 * float(K[kv, j] @ q[h])) < 1e-12


@pytest.mark.parametrize("P", [2, 3, 5, 8])
def test_merge_of_any_split_equals_unsplit(P):
    rng = np.random.default_rng(40 + P)
    q, K, V = _rand_head(rng, 300)
    full_o, full_l = oracle.attend(q, K, V, 0.09)
    for _ in range(20):
        part_of = rng.integers(0, P, size=300)
        parts = [np.flatnonzero(part_of == p) for p in range(P)]
        parts.append(np.zeros(0, dtype=np.int64))            # an empty part
        res = [oracle.attend(q, K[ix], V[ix], 0.09) for ix in parts]
        o, l = oracle.lse_merge(np.stack([r[0] for r in res]), np.array([r[1] for r in res]))
        assert np.allclose(o, full_o, atol=1e-12) and abs(l - full_l) < 1e-12


def test_merge_two_singletons_closed_form():
    """Two single-token parts with lse 0 and ln 3 weigh 1/4 and 3/4."""
    o, l = oracle.lse_merge(np.array([[2.0] * 4, [-2.0] * 4]), np.array([0.0, math.log(3)]))
    assert np.allclose(o, 0.25 * 2 - 0.75 * 2, atol=1e-15) and abs(l - math.log(4)) < 1e-15


def test_merge_neg_inf_parts():
    o, l = oracle.lse_merge(np.array([[1.0, 2.0], [9.0, 9.0]]), np.array([0.5, -np.inf]))
    assert np.array_equal(o, [1.0, 2.0]) and l == 0.5
    o, l = oracle.lse_merge(np.ones((3, 4)), np.full(3, -np.inf))
    assert l == -np.inf and np.array_equal(o, np.zeros(4))


def test_decode_step_with_full_budget_is_dense_attention():
    """With k >= |candidates| the retrieved set and the window cover [0, N) exactly
    once, so the merged result is dense attention over the whole context."""
    rng = np.random.default_rng(50)
    Hq, Hkv, N, d = 4, 2, 200, 128
    q = rng.standard_normal((Hq, d))
    K = rng.standard_normal((Hkv, N, d))
    V = rng.standard_normal((Hkv, N, d))
    hp = oracle.prepare_hash({"kind": "lsh", "bits": 64, "dtype": "f32",
                              "R": rng.standard_normal((64, d)).astype(np.float32)})
    codes = np.stack([oracle.encode(K[h], hp)[0] for h in range(Hkv)])
    r = oracle.decode_step(q, K, V, codes, hp, N, 4, 16, k=1000)
    scale = 1 / math.sqrt(d)
    for h in range(Hq):
        logits = K[h // 2] @ q[h] * scale
        assert np.allclose(r["o"][h], softmax(logits) @ V[h // 2], atol=1e-12)
        assert abs(r["lse"][h] - logsumexp(logits)) < 1e-12
    # with a small budget, the step equals attention over window U top-k
    r = oracle.decode_step(q, K, V, codes, hp, N, 4, 16, k=10)
    for h in range(Hq):
        sel = np.concatenate([r["idx"][h // 2], oracle.window_indices(N, 4, 16)])
        logits = K[h // 2][sel] @ q[h] * scale
        assert np.allclose(r["o"][h], softmax(logits) @ V[h // 2][sel], atol=1e-12)
        assert abs(r["lse"][h] - logsumexp(logits)) < 1e-12


def test_exact_topk_brute_force():
    rng = np.random.default_rng(51)
    q = rng.standard_normal(16)
    K = rng.standard_normal((30, 16))
    K[5] = K[9]                                               # a tie
    s = K @ q
    want = sorted(sorted(range(30), key=lambda j: (-s[j], j))[:7])
    assert oracle.exact_topk(q, K, 7).tolist() == want
    assert oracle.exact_topk(q, K, 7, first=4).tolist() == [w + 4 for w in want]


def test_exact_topk_group_brute_force():
    """Group ranking by the summed logit, over the candidate range only, with ties."""
    rng = np.random.default_rng(53)
    G, d, N, s, w = 3, 8, 40, 3, 5
    qs = rng.standard_normal((G, d))
    pool = rng.standard_normal((4, d))
    K = pool[rng.integers(0, 4, size=N)]                      # many exact ties
    for k in (0, 1, 6, N - s - w, N + 3):
        score = {j: sum(float(np.dot(qs[g], K[j])) for g in range(G)) for j in range(s, N - w)}
        want = sorted(sorted(score, key=lambda j: (-score[j], j))[:k])
        assert oracle.exact_topk_group(qs, K, N, s, w, k).tolist() == want
    assert oracle.exact_topk_group(qs, K, 7, 4, 4, 3).size == 0


def test_iou_definition():
    assert oracle.iou([1, 2, 3], [2, 3, 4]) == 2 / 4
    assert oracle.iou([], []) == 1.0
    assert oracle.iou([5], []) == 0.0
    rng = np.random.default_rng(55)
    for _ in range(20):
        a = rng.choice(100, size=int(rng.integers(0, 30)), replace=False)
        b = rng.choice(100, size=int(rng.integers(0, 30)), replace=False)
        inter = sum(1 for x in a if x in list(b))
        union = len(a) + len(b) - inter
        assert oracle.iou(a, b) == (1.0 if union == 0 else inter / union)


def test_decode_step_qheads_is_per_head_hamming_topk_then_softmax():
    """Per-query-head selection against a separate construction: each query head's own
    code (its sign pattern under R), its top-k by (bit-count distance, index) over its
    KV head (h // G) built with Python sets of bits, and scipy's softmax over the union
    with the window.  With G = 1 it coincides with the per-KV-head step."""
    rng = np.random.default_rng(57)
    Hq, Hkv, N, d, s, w, k = 6, 2, 150, 16, 3, 10, 9
    q = rng.standard_normal((Hq, d))
    K = rng.standard_normal((Hkv, N, d))
    V = rng.standard_normal((Hkv, N, d))
    R = rng.standard_normal((64, d)).astype(np.float32)
    hp = oracle.prepare_hash({"kind": "lsh", "bits": 64, "dtype": "f32", "R": R})
    codes = np.stack([oracle.encode(K[h], hp)[0] for h in range(Hkv)])
    r = oracle.decode_step_qheads(q, K, V, codes, hp, N, s, w, k)
    scale = 1 / math.sqrt(d)
    win = list(range(s)) + list(range(N - w, N))
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        qbits = {j for j in range(64) if float(np.dot(R[j].astype(np.float64), q[h])) > 0}
        dist = {}
        for t in range(s, N - w):
            kbits = {j for j in range(64) if float(np.dot(R[j].astype(np.float64), K[kv, t])) > 0}
            dist[t] = len(qbits ^ kbits)
        want = sorted(sorted(dist, key=lambda t: (dist[t], t))[:k])
        assert r["idx"][h].tolist() == want
        sel = want + win
        logits = K[kv][sel] @ q[h] * scale
        assert np.allclose(r["o"][h], softmax(logits) @ V[kv][sel], atol=1e-12)
        assert abs(r["lse"][h] - logsumexp(logits)) < 1e-12
    # G = 1: the same as the per-KV-head step
    r1 = oracle.decode_step_qheads(q[:Hkv], K, V, codes, hp, N, s, w, k)
    r2 = oracle.decode_step(q[:Hkv], K, V, codes, hp, N, s, w, k)
    assert np.allclose(r1["o"], r2["o"], atol=1e-12) and np.allclose(r1["lse"], r2["lse"], atol=1e-12)
