"""Parity of the per-query-head selection variant (hk_retrieve_topk_qheads,
hk_sparse_decode_qheads and the step built on them) with the CPU oracle: indices
bit-exact, attention within the bf16 / fp32 bounds."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import codes_tensor, compare_codes, np_u32, say

pytestmark = pytest.mark.gpu

hk = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global hk
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hash_top_kv_amd
    hk = hash_top_kv_amd


QH_CASES = [
    # bits, B, Hkv, G, N, s, w, k, pool
    (128, 2, 2, 4, 5000, 4, 64, 100, 0),
    (64, 1, 4, 7, 9001, 4, 512, 181, 0),
    (128, 1, 2, 8, 70000, 4, 64, 1400, 0),     # many chunks per head
    (128, 2, 1, 3, 4100, 0, 0, 500, 3),        # heavy ties
    (64, 1, 3, 1, 3333, 4, 64, 77, 0),         # G = 1
    (128, 1, 2, 2, 100, 4, 64, 82, 0),         # k >= candidates
    (128, 1, 2, 2, 60, 4, 64, 82, 0),          # no candidates
]


@pytest.mark.parametrize("case", QH_CASES, ids=lambda c: "-".join(map(str, c)))
def test_retrieve_topk_qheads_matches_oracle(case):
    bits, B, Hkv, G, N, s, w, k, pool = case
    say(f"retrieve_topk_qheads {case}")
    W = bits // 32
    Hq = Hkv * G
    rng = np.random.default_rng(N + G)
    if pool:
        table = rng.integers(0, 2 ** 32, size=(pool, W), dtype=np.uint32)
        codes = table[rng.integers(0, pool, size=(B, Hkv, N))]
        qc = table[rng.integers(0, pool, size=(B, Hq))]
    else:
        codes = rng.integers(0, 2 ** 32, size=(B, Hkv, N, W), dtype=np.uint32)
        qc = rng.integers(0, 2 ** 32, size=(B, Hq, W), dtype=np.uint32)
        # near neighbours of some query heads so small distances occur
        for b in range(B):
            for h in range(0, Hq, 2):
                pos = rng.choice(N, min(N, 50), replace=False)
                codes[b, h // G, pos] = qc[b, h] ^ (rng.random((len(pos), W)) < 0.05).astype(np.uint32)
    idx, count = hk.retrieve_topk_qheads(codes_tensor(codes), codes_tensor(qc), bits, N, s, w, k)
    torch.cuda.synchronize()
    idx, count = idx.cpu().numpy(), count.cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            want = oracle.select_topk(codes[b, h // G], qc[b, h], N, s, w, k)
            assert count[b, h] == want.size
            assert np.array_equal(idx[b, h, :want.size], want), (b, h)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sparse_decode_qheads_matches_oracle(dtype):
    B, Hkv, G, N = 2, 2, 3, 900
    Hq = Hkv * G
    wl = synth.scaled(synth.WORKLOADS[1], B=B, Hkv=Hkv, Hq=Hq, N=N, dtype=dtype)
    kv = synth.make_kv(wl)
    qn = synth.make_q(wl)
    rng = np.random.default_rng(71)
    L = 300
    counts = rng.integers(0, L + 1, size=(B, Hq)).astype(np.int32)
    counts[0, 1] = 0                                        # an empty list
    counts[1, 2] = L
    lists = np.zeros((B, Hq, L), np.int32)
    for b in range(B):
        for h in range(Hq):
            lists[b, h, :counts[b, h]] = np.sort(rng.choice(N, counts[b, h], replace=False))
    K, V = synth.to_device(kv["K"], dtype), synth.to_device(kv["V"], dtype)
    q = synth.to_device(qn, dtype)
    o, lse = hk.sparse_decode_qheads(q, K, V, torch.from_numpy(lists).cuda(), L,
                                     count=torch.from_numpy(counts).cuda())
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    Kw, Vw, qw = (oracle.widen(x, dtype) for x in (kv["K"], kv["V"], qn))
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for b in range(B):
        for h in range(Hq):
            sel = lists[b, h, :counts[b, h]]
            ro, rl = oracle.attend(qw[b, h], Kw[b, h // G][sel], Vw[b, h // G][sel], 1 / np.sqrt(128))
            assert np.max(np.abs(o[b, h] - ro)) <= tol
            assert (rl == -np.inf and lse[b, h] == -np.inf) or abs(lse[b, h] - rl) <= tol


@pytest.mark.parametrize("case", [("mlp", 128, "bf16", 4), ("lsh", 64, "bf16", 7), ("lsh", 128, "f32", 2)],
                         ids=lambda c: "-".join(map(str, c)))
def test_qhead_step_matches_oracle(case):
    kind, bits, dtype, G = case
    B, Hkv, N, s, w = 2, 2, 6000, 4, 64
    k = synth.budget_percent(N, 2)
    say(f"qhead step {case}")
    wl = synth.scaled(synth.WORKLOADS[4], B=B, Hkv=Hkv, Hq=Hkv * G, N=N, dtype=dtype,
                      hashes=(synth.HashSpec(kind, bits),), n_sink=s, n_local=w, k=k)
    kv = synth.make_kv(wl)
    qn = synth.make_q(wl)
    hnp = synth.make_hash(wl, wl.hashes[0])
    h = hk.Hash(kind, bits, **synth.hash_to_device(hnp))
    hp = oracle.prepare_hash(hnp)
    K, V = synth.to_device(kv["K"], dtype), synth.to_device(kv["V"], dtype)
    codes = torch.empty((B, Hkv, N, bits // 32), dtype=torch.int32, device="cuda")
    hk.encode_keys(h, K, codes)
    from hash_top_kv_amd.step import QHeadStep
    step = QHeadStep(K, V, codes, bits, N, s, w, k, Hkv * G, h)
    o, lse = step(synth.to_device(qn, dtype))
    torch.cuda.synchronize()
    qc = np_u32(step.qcodes)
    ref_q, yq = oracle.encode(oracle.widen(qn, dtype).reshape(B * Hkv * G, -1), hp)
    compare_codes(qc.reshape(B * Hkv * G, -1), ref_q, yq)
    cc = np_u32(codes)
    idx, count = step.idx.cpu().numpy(), step.count.cpu().numpy()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for b in range(B):
        ref = oracle.decode_step_qheads(oracle.widen(qn[b], dtype), oracle.widen(kv["K"][b], dtype),
                                        oracle.widen(kv["V"][b], dtype), cc[b], hp, N, s, w, k,
                                        qcodes=qc[b])
        for hq in range(Hkv * G):
            assert np.array_equal(idx[b, hq, :count[b, hq]], ref["idx"][hq])
        assert np.max(np.abs(o[b] - ref["o"])) <= tol
        assert np.max(np.abs(lse[b] - ref["lse"])) <= tol
