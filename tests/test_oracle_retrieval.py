"""Pins of the oracle's Hamming distance, bit packing and top-k selection.

Each check is independent of the oracle's own code path: Python big-integer bit
counting, NumPy's packbits, sorting with an explicit (distance, index) key, and the
closed form of planted near neighbours.
"""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _as_int(words):
    return sum(int(w) << (32 * i) for i, w in enumerate(words))


def test_golden_hamming_cases():
    n = 0
    for line in open(os.path.join(GOLDEN, "hamming_cases.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        bits, a, b, dist = [f.strip() for f in line.split("|")]
        wa = np.array([int(x, 16) for x in a.split()], dtype=np.uint32)
        wb = np.array([int(x, 16) for x in b.split()], dtype=np.uint32)
        assert wa.size * 32 == int(bits)
        assert oracle.hamming(wa[None], wb)[0] == int(dist)
        n += 1
    assert n == 12


@pytest.mark.parametrize("bits", [64, 128])
def test_hamming_brute_force(bits):
    rng = np.random.default_rng(11)
    W = bits // 32
    a = rng.integers(0, 2 ** 32, size=(10000, W), dtype=np.uint32)
    # bias some pairs to be close so small distances are exercised too
    b = a.copy()
    flips = rng.integers(0, 2 ** 32, size=(10000, W), dtype=np.uint32)
    b[::2] ^= flips[::2] & rng.integers(0, 2 ** 32, size=(5000, W), dtype=np.uint32) \
        & rng.integers(0, 2 ** 32, size=(5000, W), dtype=np.uint32)
    b[1::2] = rng.integers(0, 2 ** 32, size=(5000, W), dtype=np.uint32)
    for i in range(0, 10000, 7):
        want = bin(_as_int(a[i]) ^ _as_int(b[i])).count("1")
        assert oracle.hamming(a[i][None], b[i])[0] == want


@pytest.mark.parametrize("bits", [64, 128])
def test_pack_matches_numpy_packbits(bits):
    rng = np.random.default_rng(3)
    x = rng.random((500, bits)) < 0.5
    want = np.packbits(x, axis=1, bitorder="little").view("<u4")
    got = oracle.pack_bits(x)
    assert got.dtype == np.uint32 and np.array_equal(got, want)
    assert np.array_equal(oracle.unpack_bits(got, bits), x)
    # bit j alone -> word j // 32 has value 1 << (j % 32)
    for j in (0, 1, 31, 32, 63, bits - 1):
        e = np.zeros(bits, dtype=bool)
        e[j] = True
        w = oracle.pack_bits(e)
        assert _as_int(w) == 1 << j


@pytest.mark.parametrize("bits", [64, 128])
def test_hamming_metric_properties(bits):
    rng = np.random.default_rng(5)
    W = bits // 32
    c = rng.integers(0, 2 ** 32, size=(300, W), dtype=np.uint32)
    for i in range(100):
        x, y, z = c[i], c[i + 100], c[i + 200]
        assert oracle.hamming(x[None], x)[0] == 0
        assert oracle.hamming(x[None], ~x)[0] == bits
        dxy = oracle.hamming(x[None], y)[0]
        assert dxy == oracle.hamming(y[None], x)[0]
        assert dxy <= oracle.hamming(x[None], z)[0] + oracle.hamming(z[None], y)[0]


def _brute_select(dist_of, n_ctx, s, w, k):
    cand = [j for j in range(n_ctx) if s <= j < n_ctx - w]
    chosen = sorted(cand, key=lambda j: (dist_of[j], j))[:max(0, k)]
    return sorted(chosen)


@pytest.mark.parametrize("bits", [64, 128])
def test_select_brute_force_with_ties(bits):
    rng = np.random.default_rng(17)
    W = bits // 32
    for trial in range(60):
        n_ctx = int(rng.integers(1, 70))
        s = int(rng.integers(0, 6))
        w = int(rng.integers(0, 12))
        pool = rng.integers(0, 2 ** 32, size=(4, W), dtype=np.uint32)   # few codes -> ties
        codes = pool[rng.integers(0, 4, size=n_ctx + 3)]
        q = rng.integers(0, 2 ** 32, size=W, dtype=np.uint32)
        dist_of = [bin(_as_int(codes[j]) ^ _as_int(q)).count("1") for j in range(n_ctx)]
        ncand = max(0, n_ctx - s - w)
        for k in sorted({0, 1, max(0, ncand - 1), ncand, ncand + 5}):
            got = oracle.select_topk(codes, q, n_ctx, s, w, k)
            assert got.tolist() == _brute_select(dist_of, n_ctx, s, w, k), (n_ctx, s, w, k)


def test_select_invariants():
    rng = np.random.default_rng(23)
    codes = rng.integers(0, 2 ** 32, size=(3000, 4), dtype=np.uint32)
    q = rng.integers(0, 2 ** 32, size=4, dtype=np.uint32)
    n_ctx, s, w, k = 2900, 4, 64, 61
    idx = oracle.select_topk(codes, q, n_ctx, s, w, k)
    cand = np.arange(s, n_ctx - w)
    dist = np.array([bin(_as_int(codes[j]) ^ _as_int(q)).count("1") for j in cand])
    sel = np.isin(cand, idx)
    assert idx.size == k and np.all(np.diff(idx) > 0)
    T = dist[sel].max()
    assert np.all(dist[~sel] >= T)
    tied = cand[dist == T]
    taken = np.isin(tied, idx)
    # within the threshold distance, the chosen ones are exactly the lowest indices
    assert np.all(taken[:taken.sum()]) and not np.any(taken[taken.sum():])


def test_select_empty_and_degenerate():
    codes = np.zeros((10, 4), dtype=np.uint32)
    q = np.zeros(4, dtype=np.uint32)
    assert oracle.select_topk(codes, q, 10, 4, 6, 5).size == 0       # n_ctx == s + w
    assert oracle.select_topk(codes, q, 10, 8, 6, 5).size == 0       # s + w > n_ctx
    assert oracle.select_topk(codes, q, 10, 0, 0, 0).size == 0       # k = 0
    # all distances equal: the lowest indices win
    assert oracle.select_topk(codes, q, 10, 2, 1, 3).tolist() == [2, 3, 4]
    assert oracle.select_topk(codes, q, 10, 0, 0, 50).tolist() == list(range(10))


def _planted_expected(pos, delta, k):
    order = sorted(range(len(pos)), key=lambda i: (int(delta[i]), int(pos[i])))
    return sorted(int(pos[i]) for i in order[:k])


@pytest.mark.parametrize("N,k", [(65536, 300), (524288, 1024)])
def test_select_planted_closed_form(N, k):
    """Uniform background codes lie at distance ~64 +- 6 from the query code; the
    planted ones at 0..8.  So the top-k is the planted list ordered by (delta, pos)."""
    wl = synth.scaled(synth.WORKLOADS[2], N=N, k=k)
    g = synth.make_given_codes(wl, heads=[(0, 3)])
    idx = oracle.select_topk(g["codes"][0, 3], g["qcodes"][0, 3], N, 0, 0, k)
    want = _planted_expected(g["planted_pos"][0, 3], g["planted_delta"][0, 3], k)
    assert idx.tolist() == want
    # the planted distances are what the generator claims
    d = oracle.hamming(g["codes"][0, 3][g["planted_pos"][0, 3]], g["qcodes"][0, 3])
    assert np.array_equal(d, g["planted_delta"][0, 3])


def test_golden_budgets():
    for line in open(os.path.join(GOLDEN, "budgets.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        n, pct, k = (int(x) for x in line.split())
        assert synth.budget_percent(n, pct) == k
    assert synth.WORKLOADS[0].k == 82 and synth.WORKLOADS[3].k == 2622


def test_window_and_candidates_partition_context():
    for n_ctx, s, w in [(100, 4, 64), (60, 4, 64), (10, 0, 0), (5, 8, 2), (68, 4, 64), (0, 4, 4)]:
        win = oracle.window_indices(n_ctx, s, w)
        cand = oracle.candidate_range(n_ctx, s, w)
        allt = np.sort(np.concatenate([win, cand]))
        assert allt.tolist() == list(range(n_ctx)), (n_ctx, s, w)


def test_evict_victim_brute_force():
    rng = np.random.default_rng(29)
    for _ in range(40):
        n = int(rng.integers(1, 50))
        pool = rng.integers(0, 2 ** 32, size=(3, 2), dtype=np.uint32)
        codes = pool[rng.integers(0, 3, size=n)]
        q = rng.integers(0, 2 ** 32, size=2, dtype=np.uint32)
        s, w = int(rng.integers(0, 4)), int(rng.integers(0, 4))
        cand = [j for j in range(n) if s <= j < n - w]
        want = -1
        if cand:
            dist = {j: bin(_as_int(codes[j]) ^ _as_int(q)).count("1") for j in cand}
            want = sorted(cand, key=lambda j: (-dist[j], j))[0]
        assert oracle.evict_victim(codes, q, n, s, w) == want


def test_evict_step_is_slot_replacement_then_full_softmax():
    """The eviction step against a separate construction: the victim chosen by brute
    force over (distance desc, index asc), the cache rebuilt as Python lists with the
    victim's entries replaced, and attention from scipy's softmax / logsumexp over every
    cached token."""
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(31)
    for n, s, w, Hkv, G in [(40, 2, 5, 2, 3), (9, 4, 5, 1, 2), (30, 0, 0, 3, 1)]:
        d, W = 8, 2
        K = rng.standard_normal((Hkv, n, d))
        V = rng.standard_normal((Hkv, n, d))
        codes = rng.integers(0, 4, size=(Hkv, n, W)).astype(np.uint32)   # many ties
        qcodes = rng.integers(0, 4, size=(Hkv, W)).astype(np.uint32)
        q = rng.standard_normal((Hkv * G, d))
        k_new, v_new = rng.standard_normal((Hkv, d)), rng.standard_normal((Hkv, d))
        code_new = rng.integers(0, 2 ** 32, size=(Hkv, W), dtype=np.uint32)
        K0, codes0 = K.copy(), codes.copy()
        got = oracle.evict_step(q, K, V, codes, qcodes, k_new, v_new, code_new, n, s, w, 0.5)
        assert np.array_equal(K, K0) and np.array_equal(codes, codes0)   # inputs untouched
        for h in range(Hkv):
            cand = [j for j in range(n) if s <= j < n - w]
            want = -1
            if cand:
                dist = {j: sum(bin(int(codes[h, j, x]) ^ int(qcodes[h, x])).count("1")
                               for x in range(W)) for j in cand}
                want = sorted(cand, key=lambda j: (-dist[j], j))[0]
            assert got["victim"][h] == want
            krows, vrows, crows = list(K[h]), list(V[h]), list(codes[h])
            if want >= 0:
                krows[want], vrows[want], crows[want] = k_new[h], v_new[h], code_new[h]
            assert np.array_equal(got["K"][h], np.array(krows))
            assert np.array_equal(got["V"][h], np.array(vrows))
            assert np.array_equal(got["codes"][h], np.array(crows))
            for g in range(G):
                logits = 0.5 * (np.array(krows) @ q[h * G + g])
                assert np.allclose(got["o"][h * G + g], softmax(logits) @ np.array(vrows),
                                   atol=1e-12, rtol=0)
                assert abs(got["lse"][h * G + g] - logsumexp(logits)) < 1e-12
