"""Parity of the exact ("oracle") top-k by logit and of the list intersection behind the
retrieval IoU with the CPU oracle.

The GPU ranks by fp32 logits, the oracle by fp64 ones, so a token whose logit lies
within the fp32 rounding band of the k-th largest may go either way: the random cases
check that every token clearly above the threshold is selected, none clearly below is,
and the count is exact.  The pooled cases (K rows drawn from a few distinct rows, so
logits tie exactly and are far apart otherwise) have a unique answer and are compared
entry by entry, ties going to the lower token."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import say

pytestmark = pytest.mark.gpu

hk = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global hk
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hash_top_kv_amd
    hk = hash_top_kv_amd


def _inputs(dtype, B, Hkv, G, N, pool, seed):
    wl = synth.scaled(synth.WORKLOADS[1], B=B, Hkv=Hkv, Hq=Hkv * G, N=N, dtype=dtype)
    kv = synth.make_kv(wl, "k")
    Kn = kv["K"]
    if pool:
        rng = np.random.default_rng(seed)
        for b in range(B):
            for h in range(Hkv):
                rows = Kn[b, h, rng.choice(N, pool, replace=False)].copy()
                Kn[b, h] = rows[rng.integers(0, pool, size=N)]
    q = synth.make_q(wl, replica=seed)
    return Kn, q


EXACT_CASES = [
    # dtype, B, Hkv, G, N, s, w, k, pool
    ("bf16", 2, 2, 4, 5000, 4, 64, 100, 0),
    ("bf16", 1, 3, 7, 70001, 4, 512, 1401, 0),     # many chunks, ragged tail
    ("f32", 1, 2, 1, 4096, 4, 64, 82, 0),
    ("bf16", 2, 2, 3, 6000, 4, 64, 300, 5),        # exact ties, unique answer
    ("f32", 1, 2, 2, 3000, 0, 0, 700, 3),
    ("bf16", 1, 2, 1, 100, 4, 64, 82, 0),           # k >= candidates
    ("bf16", 1, 2, 1, 60, 4, 64, 82, 0),            # no candidates
    ("bf16", 1, 2, 1, 1000, 4, 64, 0, 0),           # k = 0
]


@pytest.mark.parametrize("case", EXACT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_exact_topk_matches_oracle(case):
    dtype, B, Hkv, G, N, s, w, k, pool = case
    say(f"exact_topk {case}")
    Kn, qn = _inputs(dtype, B, Hkv, G, N, pool, 3)
    K = synth.to_device(Kn, dtype)
    q = synth.to_device(qn, dtype)
    idx, count = hk.exact_topk(q, K, N, s, w, k)
    torch.cuda.synchronize()
    idx, count = idx.cpu().numpy(), count.cpu().numpy()
    Kw, qw = oracle.widen(Kn, dtype), oracle.widen(qn, dtype)
    cand = oracle.candidate_range(N, s, w)
    keff = max(0, min(k, cand.size))
    for b in range(B):
        for h in range(Hkv):
            assert count[b, h] == keff
            got = idx[b, h, :keff]
            assert np.all(np.diff(got) > 0) and (keff == 0 or (got[0] >= s and got[-1] < N - w))
            qg = qw[b, h * G:(h + 1) * G]
            want = oracle.exact_topk_group(qg, Kw[b, h], N, s, w, k)
            if pool or keff == cand.size or keff == 0:
                assert np.array_equal(got, want), (b, h)
                continue
            score = Kw[b, h][cand] @ qg.sum(axis=0)
            band = 1e-5 * (np.abs(Kw[b, h][cand]) @ np.abs(qg).sum(axis=0))   # fp32 error scale
            kth = np.sort(score)[::-1][keff - 1]
            sel = np.zeros(N, bool)
            sel[got] = True
            sure_in = cand[score > kth + band]
            sure_out = cand[score < kth - band]
            assert sel[sure_in].all() and not sel[sure_out].any(), (b, h)
            say(f"  head {b},{h}: {len(np.setxor1d(got, want)) // 2} swaps inside the rounding band")


def test_topk_intersect_matches_sets():
    rng = np.random.default_rng(61)
    L, sa, sb = 37, 50, 64
    a = np.zeros((L, sa), np.int32)
    b = np.zeros((L, sb), np.int32)
    ca = rng.integers(0, sa + 1, size=L).astype(np.int32)
    cb = rng.integers(0, sb + 1, size=L).astype(np.int32)
    ca[0], cb[1] = 0, 0                                        # empty lists
    ca[2] = sa + 9                                             # clamped to the stride
    for l in range(L):
        a[l, :min(ca[l], sa)] = np.sort(rng.choice(200, min(ca[l], sa), replace=False))
        b[l, :cb[l]] = np.sort(rng.choice(200, cb[l], replace=False))
    inter = hk.topk_intersect(*(torch.from_numpy(x).cuda() for x in (a, ca, b, cb)))
    torch.cuda.synchronize()
    inter = inter.cpu().numpy()
    for l in range(L):
        A, Bs = set(a[l, :min(ca[l], sa)].tolist()), set(b[l, :cb[l]].tolist())
        assert inter[l] == len(A & Bs)
        union = len(A | Bs)
        iou = 1.0 if union == 0 else inter[l] / union
        assert iou == oracle.iou(list(A), list(Bs))
