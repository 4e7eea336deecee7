"""Parity of each HIP entry point with the CPU oracle at small sizes that still span
several workgroup tiles and ragged tails, plus the degenerate cases."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import codes_tensor, compare_codes, np_u32, say

pytestmark = pytest.mark.gpu

hk = None
hkp = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global hk, hkp
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hash_top_kv_amd
    from hash_top_kv_amd import probe
    hk = hash_top_kv_amd
    hkp = probe


# ----------------------------------------------------------------- retrieval
RETRIEVE_CASES = [
    # bits, B, Hkv, N, s, w, k, pool (number of distinct codes -> ties)
    (128, 1, 1, 4096, 4, 64, 82, 0),
    (128, 2, 3, 5000, 4, 64, 100, 6),       # heavy ties
    (64, 2, 2, 9001, 4, 512, 181, 0),
    (64, 1, 4, 3333, 0, 0, 77, 3),
    (128, 3, 2, 70000, 4, 64, 1400, 0),     # many chunks per head
    (128, 1, 2, 100, 4, 64, 82, 0),         # k >= candidates
    (128, 1, 2, 60, 4, 64, 82, 0),          # n_ctx < s + w: no candidates
    (128, 1, 2, 1000, 4, 64, 0, 0),         # k = 0
    (64, 1, 1, 1, 0, 0, 5, 0),              # single token
    (128, 2, 2, 4100, 4, 0, 4096, 2),       # k = C, two distinct codes
    (128, 1, 8, 300001, 4, 64, 6001, 0),    # >= 2M tokens: 8 codes per thread
    (64, 2, 4, 600000, 4, 512, 3000, 0),    # 8 codes per thread, 64-bit
    (128, 1, 8, 540000, 0, 0, 1024, 9),     # > 256 chunks per head (second threshold
                                            # window for 128-bit codes), heavy ties
    (64, 1, 2, 1100000, 0, 0, 500, 0),      # > 512 chunks per head (64-bit codes)
    (64, 16, 8, 70000, 4, 64, 700, 0),      # 4480 chunks: 4 chunks per emit workgroup,
                                            # the last group of each head 3 chunks
    (64, 32, 8, 70000, 0, 0, 1400, 5),      # 8960 chunks: 8 per emit workgroup, ties
]


@pytest.mark.parametrize("case", RETRIEVE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_retrieve_topk_bit_exact(case):
    bits, B, Hkv, N, s, w, k, pool = case
    say(f"retrieve {case}")
    W = bits // 32
    rng = np.random.default_rng(N * 31 + k)
    cap = N + 37                                           # capacity beyond the context
    if pool:
        table = rng.integers(0, 2 ** 32, size=(pool, W), dtype=np.uint32)
        codes = table[rng.integers(0, pool, size=(B, Hkv, cap))]
    else:
        codes = rng.integers(0, 2 ** 32, size=(B, Hkv, cap, W), dtype=np.uint32)
    qc = rng.integers(0, 2 ** 32, size=(B, Hkv, W), dtype=np.uint32)
    idx, count = hk.retrieve_topk(codes_tensor(codes), codes_tensor(qc), bits, N, s, w, k)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    count = count.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            want = oracle.select_topk(codes[b, h], qc[b, h], N, s, w, k)
            assert count[b, h] == want.size
            assert np.array_equal(idx[b, h, :want.size], want), (b, h)


@pytest.mark.parametrize("bits", [64, 128])
def test_retrieve_ties_at_the_largest_distance(bits):
    """Most codes are the complement of the query code (distance = bits, a bin the
    per-chunk histograms leave out): the threshold lands on it and the tie quota is
    taken in index order."""
    rng = np.random.default_rng(bits)
    W = bits // 32
    B, Hkv, N, k = 1, 3, 20000, 700
    qc = rng.integers(0, 2 ** 32, size=(B, Hkv, W), dtype=np.uint32)
    codes = np.broadcast_to(~qc[:, :, None, :], (B, Hkv, N, W)).copy()
    few = rng.choice(N, size=150, replace=False)
    codes[:, :, few] = rng.integers(0, 2 ** 32, size=(B, Hkv, few.size, W), dtype=np.uint32)
    idx, count = hk.retrieve_topk(codes_tensor(codes), codes_tensor(qc), bits, N, 0, 0, k)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for h in range(Hkv):
        want = oracle.select_topk(codes[0, h], qc[0, h], N, 0, 0, k)
        assert np.array_equal(idx[0, h], want), h


def test_retrieve_split_halves_equal_whole_and_workspace_reuse():
    """The two halves equal the whole call, and one workspace serves many calls: each
    call leaves its counters at zero (inputs differ between the calls)."""
    rng = np.random.default_rng(2)
    wsb = hk.retrieve_topk_workspace(128, 2, 2, 20000, 4, 64, 400)
    ws = hk.workspace(wsb)
    for trial in range(3):
        codes = rng.integers(0, 2 ** 32, size=(2, 2, 20000, 4), dtype=np.uint32)
        qc = rng.integers(0, 2 ** 32, size=(2, 2, 4), dtype=np.uint32)
        c, q = codes_tensor(codes), codes_tensor(qc)
        idx1, cnt1 = hk.retrieve_topk(c, q, 128, 20000, 4, 64, 400, ws=ws)
        idx2 = torch.full((2, 2, 400), -7, dtype=torch.int32, device="cuda")
        cnt2 = torch.zeros((2, 2), dtype=torch.int32, device="cuda")
        hk.hamming_scan(c, q, 128, 20000, 4, 64, 400, ws)
        hk.topk_select(128, 2, 2, 20000, 4, 64, 400, idx2, cnt2, ws)
        torch.cuda.synchronize()
        assert torch.equal(idx1, idx2) and torch.equal(cnt1, cnt2)
        assert (idx2 >= 0).all()                                 # every slot written
        for b in range(2):
            for h in range(2):
                want = oracle.select_topk(codes[b, h], qc[b, h], 20000, 4, 64, 400)
                assert np.array_equal(idx1[b, h].cpu().numpy(), want)


@pytest.mark.parametrize("shape", [(2, 8, 2, [700, 2000]), (3, 8, 8, [1024, 3, 0])],
                         ids=["merge-kernel", "merge-in-gather"])
def test_sparse_decode_workspace_reuse(shape):
    B, Hq, Hkv, counts = shape
    K, V, Q, idx, cnt, idx_np, cnt_np, maxc = _attention_case("bf16", B, Hq, Hkv, 3000, counts, 21)
    ws = hk.workspace(hk.sparse_decode_workspace(B, Hq, Hkv, maxc))
    outs = [hk.sparse_decode(Q, K, V, idx, maxc, count=cnt, ws=ws) for _ in range(3)]
    torch.cuda.synchronize()
    for o, lse in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_retrieve_is_deterministic():
    rng = np.random.default_rng(3)
    table = rng.integers(0, 2 ** 32, size=(5, 4), dtype=np.uint32)
    codes = table[rng.integers(0, 5, size=(1, 4, 50000))]
    qc = rng.integers(0, 2 ** 32, size=(1, 4, 4), dtype=np.uint32)
    c, q = codes_tensor(codes), codes_tensor(qc)
    a = hk.retrieve_topk(c, q, 128, 50000, 4, 64, 1000)[0].clone()
    b = hk.retrieve_topk(c, q, 128, 50000, 4, 64, 1000)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_retrieve_planted_closed_form():
    wl = synth.scaled(synth.WORKLOADS[2], N=100000, Hkv=2, Hq=2, k=300)
    g = synth.make_given_codes(wl)
    idx, count = hk.retrieve_topk(codes_tensor(g["codes"]), codes_tensor(g["qcodes"]), 128,
                                  wl.N, 0, 0, wl.k)
    idx = idx.cpu().numpy()
    for h in range(2):
        pos, dl = g["planted_pos"][0, h], g["planted_delta"][0, h]
        want = sorted(int(pos[i]) for i in sorted(range(len(pos)), key=lambda i: (dl[i], pos[i]))[:wl.k])
        assert idx[0, h].tolist() == want


def test_window_indices():
    for n, s, w in [(4096, 4, 64), (60, 4, 64), (131072, 4, 512), (3, 4, 64), (10, 0, 0)]:
        got = hk.window_indices(n, s, w, "cuda").cpu().numpy()
        assert np.array_equal(got, oracle.window_indices(n, s, w)), (n, s, w)


# ----------------------------------------------------------------- attention
def _attention_case(dtype, B, Hq, Hkv, cap, counts, seed, stride0=False):
    rng = np.random.default_rng(seed)
    d = 128
    Kf = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32) * 1.5
    Vf = rng.standard_normal((B, Hkv, cap, d)).astype(np.float32)
    Qf = rng.standard_normal((B, Hq, d)).astype(np.float32) * 1.5
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    K = torch.from_numpy(Kf).to(tdt).cuda()
    V = torch.from_numpy(Vf).to(tdt).cuda()
    Q = torch.from_numpy(Qf).to(tdt).cuda()
    maxc = max(counts)
    if stride0:
        lst = np.sort(rng.choice(cap, size=maxc, replace=False)).astype(np.int32)
        idx_np = np.broadcast_to(lst, (B, Hkv, maxc))
        idx = torch.from_numpy(lst).cuda()
        cnt = None
    else:
        idx_np = np.zeros((B, Hkv, max(maxc, 1)), dtype=np.int32)
        cnt_np = np.zeros((B, Hkv), dtype=np.int32)
        for b in range(B):
            for h in range(Hkv):
                c = counts[(b * Hkv + h) % len(counts)]
                idx_np[b, h, :c] = np.sort(rng.choice(cap, size=c, replace=False))
                cnt_np[b, h] = c
        idx = torch.from_numpy(idx_np).cuda()
        cnt = torch.from_numpy(cnt_np).cuda()
    return K, V, Q, idx, cnt, idx_np, (cnt.cpu().numpy() if cnt is not None else None), maxc


ATT_CASES = [
    # dtype, B, Hq, Hkv, cap, counts
    ("f32", 1, 1, 1, 4096, [82]),
    ("f32", 2, 8, 2, 3000, [1, 0, 700, 2000]),
    ("bf16", 1, 32, 8, 5000, [656, 1, 300, 0, 1999, 17, 64, 655]),
    ("bf16", 2, 28, 4, 9000, [5243, 100, 3, 4000]),
    ("bf16", 3, 8, 8, 2000, [1024]),
    ("bf16", 1, 16, 8, 500, [0]),
    ("f32", 1, 6, 2, 9000, [8000, 33]),
    ("bf16", 2, 5, 1, 800, [130, 129]),
]


@pytest.mark.parametrize("case", ATT_CASES, ids=lambda c: f"{c[0]}-B{c[1]}-Hq{c[2]}-Hkv{c[3]}")
def test_sparse_decode_matches_oracle(case):
    dtype, B, Hq, Hkv, cap, counts = case
    say(f"sparse_decode {case}")
    K, V, Q, idx, cnt, idx_np, cnt_np, maxc = _attention_case(dtype, B, Hq, Hkv, cap, counts, 7)
    o, lse = hk.sparse_decode(Q, K, V, idx, maxc, count=cnt)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    Kd, Vd, Qd = (x.cpu().to(torch.float64).numpy() for x in (K, V, Q))
    tol = 1e-5 if dtype == "f32" else 2e-2
    scale = 1 / math.sqrt(128)
    for b in range(B):
        lists = [idx_np[b, h, :cnt_np[b, h]] for h in range(Hkv)]
        ro, rl = oracle.sparse_attention(Qd[b], Kd[b], Vd[b], lists, scale)
        say(f"  batch {b}: max |o - oracle| = {np.max(np.abs(o[b] - ro)):.2e}")
        assert np.max(np.abs(o[b] - ro)) <= tol
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(lse[b]))
        assert np.all(lse[b][~fin] == -np.inf)
        if fin.any():
            assert np.max(np.abs(lse[b][fin] - rl[fin])) <= tol


def test_sparse_decode_shared_list_stride0():
    K, V, Q, idx, cnt, idx_np, _, maxc = _attention_case("bf16", 2, 8, 4, 3000, [68], 9, stride0=True)
    o, lse = hk.sparse_decode(Q, K, V, idx, maxc, idx_stride=0)
    torch.cuda.synchronize()
    Kd, Vd, Qd = (x.cpu().to(torch.float64).numpy() for x in (K, V, Q))
    for b in range(2):
        ro, rl = oracle.sparse_attention(Qd[b], Kd[b], Vd[b], [idx_np[b, h] for h in range(4)],
                                         1 / math.sqrt(128))
        assert np.max(np.abs(o[b].cpu().numpy() - ro)) <= 2e-2
        assert np.max(np.abs(lse[b].cpu().numpy() - rl)) <= 2e-2


@pytest.mark.parametrize("P,d", [(1, 128), (5, 128), (37, 128), (64, 128), (65, 128), (200, 128),
                                 (5, 96)], ids=lambda v: str(v))
def test_lse_merge_matches_oracle(P, d):
    """Both merge kernels: up to 64 parts of d = 128 (one workgroup per row, wavefronts
    over parts), and the general one."""
    rng = np.random.default_rng(11 + P + d)
    rows = 300
    o_parts = rng.standard_normal((P, rows, d)).astype(np.float32)
    lse_parts = (rng.standard_normal((P, rows)) * 4).astype(np.float32)
    lse_parts[rng.random((P, rows)) < 0.3] = -np.inf
    lse_parts[:, 7] = -np.inf                                # an all-empty row
    o, lse = hk.lse_merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda())
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    for r in range(rows):
        ro, rl = oracle.lse_merge(o_parts[:, r].astype(np.float64), lse_parts[:, r].astype(np.float64))
        assert np.max(np.abs(o[r] - ro)) <= 1e-5
        assert (rl == -np.inf and lse[r] == -np.inf) or abs(lse[r] - rl) <= 1e-5


# ----------------------------------------------------------------- encoders
def _hash_case(kind, bits, dtype, seed, identity=False, bias=False):
    rng = np.random.default_rng(seed)
    d = 128
    if kind == "lsh":
        if identity:
            R = np.zeros((bits, d), np.float32)
            R[np.arange(bits), rng.permutation(d)[:bits]] = 1.0
        else:
            R = rng.standard_normal((bits, d)).astype(np.float32)
        h = {"kind": "lsh", "bits": bits, "dtype": dtype,
             "R": R if dtype == "f32" else synth.to_bf16_bits(R)}
    else:
        if identity:
            W1 = np.zeros((256, d), np.float32)
            W1[np.arange(128), rng.permutation(d)] = 1.0
            W2 = np.zeros((bits, 256), np.float32)
            W2[np.arange(bits), rng.permutation(128)[:bits]] = 1.0
        else:
            W1 = (rng.standard_normal((256, d)) / math.sqrt(d)).astype(np.float32)
            W2 = (rng.standard_normal((bits, 256)) / 16).astype(np.float32)
        cv = (lambda a: a) if dtype == "f32" else synth.to_bf16_bits
        h = {"kind": "mlp", "bits": bits, "dtype": dtype, "W1": cv(W1), "W2": cv(W2)}
        if bias:
            h["b1"] = cv((rng.standard_normal(256) * 0.3).astype(np.float32))
            h["b2"] = cv((rng.standard_normal(bits) * 0.1).astype(np.float32))
    return h


# (kind, bits, dtype, identity weights, biases)
ENC_CASES = [
    ("lsh", 128, "f32", False, False), ("lsh", 64, "f32", False, False),
    ("mlp", 128, "f32", False, False), ("mlp", 128, "f32", False, True),
    ("lsh", 128, "bf16", True, False), ("lsh", 64, "bf16", True, False),
    ("mlp", 128, "bf16", True, False), ("mlp", 64, "bf16", True, False),
    ("lsh", 128, "bf16", False, False), ("lsh", 64, "bf16", False, False),
    ("mlp", 128, "bf16", False, False), ("mlp", 64, "bf16", False, False),
    ("mlp", 128, "bf16", False, True), ("mlp", 64, "bf16", False, True),
]


@pytest.mark.parametrize("case", ENC_CASES, ids=lambda c: "-".join(map(str, c)))
def test_encode_keys_matches_oracle(case):
    kind, bits, dtype, identity, bias = case
    say(f"encode_keys {case}")
    B, Hkv, cap = 2, 3, 1111
    t0, t1 = 5, 1071                                         # ragged range inside the cache
    wl = synth.scaled(synth.WORKLOADS[1], B=B, Hkv=Hkv, Hq=Hkv, N=cap, dtype=dtype)
    kv = synth.make_kv(wl, "k")
    hnp = _hash_case(kind, bits, dtype, 5, identity, bias)
    h = hk.Hash(kind, bits, **synth.hash_to_device(hnp))
    K = synth.to_device(kv["K"], dtype)
    sentinel = 0x5A5A5A5A
    codes = torch.full((B, Hkv, cap, bits // 32), sentinel, dtype=torch.int32, device="cuda")
    hk.encode_keys(h, K, codes, t0, t1)
    torch.cuda.synchronize()
    got = np_u32(codes)
    hp = oracle.prepare_hash(hnp)
    flips = 0
    for b in range(B):
        for g in range(Hkv):
            ref, y = oracle.encode(oracle.widen(kv["K"][b, g, t0:t1], dtype), hp)
            n = compare_codes(got[b, g, t0:t1], ref, y)
            if identity:
                assert n == 0
            flips += n
            assert np.all(got[b, g, :t0] == sentinel) and np.all(got[b, g, t1:] == sentinel)
    say(f"  exempt bits that differ: {flips}")


@pytest.mark.parametrize("case", [("lsh", 128, "f32", False), ("mlp", 128, "bf16", False),
                                  ("lsh", 64, "bf16", False), ("mlp", 64, "f32", False),
                                  ("mlp", 128, "bf16", True), ("mlp", 64, "f32", True)],
                         ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("G", [1, 4, 7])
def test_encode_query_matches_oracle(case, G):
    kind, bits, dtype, bias = case
    Hkv, B = 4, 3
    wl = synth.scaled(synth.WORKLOADS[1], B=B, Hkv=Hkv, Hq=Hkv * G, dtype=dtype)
    q = synth.make_q(wl)
    hnp = _hash_case(kind, bits, dtype, 6, bias=bias)
    h = hk.Hash(kind, bits, **synth.hash_to_device(hnp))
    qc = hk.encode_query(h, synth.to_device(q, dtype), Hkv)
    torch.cuda.synchronize()
    ref, y = oracle.encode_query(oracle.widen(q, dtype), oracle.prepare_hash(hnp), Hkv)
    compare_codes(np_u32(qc), ref, y)


def test_encode_keys_append_one_token():
    dtype, bits = "bf16", 128
    wl = synth.scaled(synth.WORKLOADS[1], B=2, Hkv=2, Hq=2, N=300, dtype=dtype)
    kv = synth.make_kv(wl, "k")
    hnp = _hash_case("mlp", bits, dtype, 8)
    h = hk.Hash("mlp", bits, **synth.hash_to_device(hnp))
    K = synth.to_device(kv["K"], dtype)
    codes = torch.zeros((2, 2, 300, 4), dtype=torch.int32, device="cuda")
    hk.encode_keys(h, K, codes, 0, 299)
    hk.encode_keys(h, K, codes, 299, 300)
    torch.cuda.synchronize()
    got = np_u32(codes)
    hp = oracle.prepare_hash(hnp)
    for b in range(2):
        for g in range(2):
            ref, y = oracle.encode(oracle.widen(kv["K"][b, g], dtype), hp)
            compare_codes(got[b, g], ref, y)


# (kind, bits, dtype, biases, G, N): small scans hash the query inside the scan; the
# last case has more than 512 scan workgroups and runs the query encoder, then the scan.
SCANQ_CASES = [
    ("lsh", 128, "f32", False, 1, 4096), ("mlp", 128, "f32", True, 4, 5000),
    ("mlp", 64, "f32", False, 8, 3000), ("sign", 128, "bf16", False, 3, 4000),
    ("sign", 128, "f32", False, 2, 2500), ("lsh", 64, "bf16", False, 2, 6000),
    ("lsh", 128, "bf16", False, 7, 3333), ("mlp", 128, "bf16", True, 4, 7000),
    ("mlp", 64, "bf16", False, 5, 4100), ("mlp", 128, "bf16", False, 4, 300000),
]


@pytest.mark.parametrize("case", SCANQ_CASES, ids=lambda c: "-".join(map(str, c)))
def test_hamming_scan_query_matches_encode_then_scan(case):
    """hk_hamming_scan_query against hk_encode_query + hk_hamming_scan on the same inputs:
    fp32 and sign hashes (and every hash on the two-kernel path) give the same query codes
    bit for bit and the same selection; bf16 LSH/MLP codes computed inside the scan agree
    with the oracle outside the near-zero exemption, and the selection is the oracle's
    top-k of the codes the scan reports."""
    kind, bits, dtype, bias, G, N = case
    say(f"hamming_scan_query {case}")
    B, Hkv = 2, 2
    wl = synth.scaled(synth.WORKLOADS[1], B=B, Hkv=Hkv, Hq=Hkv * G, N=N, dtype=dtype)
    q = synth.to_device(synth.make_q(wl), dtype)
    if kind == "sign":
        hnp = {"kind": "sign", "bits": 128, "dtype": dtype}
        h = hk.Hash("sign", 128, dtype=q.dtype)
    else:
        hnp = _hash_case(kind, bits, dtype, 11, bias=bias)
        h = hk.Hash(kind, bits, **synth.hash_to_device(hnp))
    rng = np.random.default_rng(3)
    W = bits // 32
    codes = codes_tensor(rng.integers(0, 2 ** 32, size=(B, Hkv, N, W), dtype=np.uint32))
    n_sink, n_local, k = 4, 64, max(1, N // 100)
    nbytes = hk.retrieve_topk_workspace(bits, B, Hkv, N, n_sink, n_local, k)
    ws1, ws2 = hk.workspace(nbytes), hk.workspace(nbytes)
    idx1 = torch.zeros((B, Hkv, k), dtype=torch.int32, device="cuda")
    idx2 = torch.zeros_like(idx1)
    cnt1 = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    cnt2 = torch.zeros_like(cnt1)
    qref = hk.encode_query(h, q, Hkv)
    hk.hamming_scan(codes, qref, bits, N, n_sink, n_local, k, ws1)
    hk.topk_select(bits, B, Hkv, N, n_sink, n_local, k, idx1, cnt1, ws1)
    qc = hk.hamming_scan_query(h, q, codes, N, n_sink, n_local, k, ws2)
    hk.topk_select(bits, B, Hkv, N, n_sink, n_local, k, idx2, cnt2, ws2)
    torch.cuda.synchronize()
    same = dtype == "f32" or kind == "sign" or N >= 300000
    if same:
        assert np.array_equal(np_u32(qc), np_u32(qref))
        assert torch.equal(idx1, idx2) and torch.equal(cnt1, cnt2)
    else:
        ref, y = oracle.encode_query(oracle.widen(synth.make_q(wl), dtype), oracle.prepare_hash(hnp), Hkv)
        n = compare_codes(np_u32(qc), ref, y)
        say(f"  exempt bits that differ from the oracle: {n}")
        _check_all_selections(codes, qc, idx2, cnt2, N, n_sink, n_local, k)


# (kind, bits, dtype, G, N, n_sink, n_local, k, codes): G = 1 heads of at most 4096
# candidates run the whole step in one workgroup; the others (G > 1, or longer heads)
# the scan-and-select+attend kernels.  codes: "rand", or "far" (every code the complement
# of its head's query code: all at distance bits, so T = bits with the whole quota).
DECODE_CASES = [
    ("lsh", 128, "f32", 1, 4096, 4, 64, 82, "rand"), ("lsh", 128, "f32", 1, 1500, 0, 0, 1500, "rand"),
    ("mlp", 128, "bf16", 1, 3000, 4, 64, 300, "rand"), ("lsh", 64, "bf16", 1, 4164, 4, 64, 1, "rand"),
    ("sign", 128, "f32", 1, 900, 4, 64, 0, "rand"), ("lsh", 128, "f32", 1, 100, 4, 64, 50, "rand"),
    ("mlp", 64, "f32", 1, 2500, 4, 64, 40, "far"), ("lsh", 128, "bf16", 1, 60, 4, 64, 10, "rand"),
    ("mlp", 128, "bf16", 4, 6000, 4, 64, 120, "rand"), ("lsh", 128, "f32", 1, 9000, 4, 64, 90, "rand"),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(map(str, c)))
def test_decode_step_matches_scan_then_select_attend(case):
    """hk_decode_step against hk_hamming_scan_query + hk_select_attend on the same
    inputs: the same query codes and the same idx and count bit for bit, o and lse
    within the dtype's bound (the one-workgroup path attends over the selection and the
    window in one pass, the other merges two partials)."""
    kind, bits, dtype, G, N, n_sink, n_local, k, mode = case
    say(f"decode_step {case}")
    B, Hkv = 2, 2
    wl = synth.scaled(synth.WORKLOADS[1], B=B, Hkv=Hkv, Hq=Hkv * G, N=N, dtype=dtype,
                      n_sink=n_sink, n_local=n_local, k=k)
    q = synth.to_device(synth.make_q(wl), dtype)
    kv = synth.make_kv(wl)
    K, V = synth.to_device(kv["K"], dtype), synth.to_device(kv["V"], dtype)
    if kind == "sign":
        h = hk.Hash("sign", 128, dtype=q.dtype)
    else:
        h = hk.Hash(kind, bits, **synth.hash_to_device(_hash_case(kind, bits, dtype, 12)))
    W = bits // 32
    qc0 = hk.encode_query(h, q, Hkv)
    torch.cuda.synchronize()
    if mode == "far":
        codes_np = np.broadcast_to(~np_u32(qc0)[:, :, None, :], (B, Hkv, N, W)).copy()
    else:
        codes_np = np.random.default_rng(5).integers(0, 2 ** 32, size=(B, Hkv, N, W), dtype=np.uint32)
    codes = codes_tensor(codes_np)
    nb = hk.retrieve_attend_workspace(bits, B, Hkv * G, Hkv, N, n_sink, n_local, k)
    ws1, ws2 = hk.workspace(nb), hk.workspace(nb)
    kk = max(k, 1)
    idx1 = torch.full((B, Hkv, kk), -7, dtype=torch.int32, device="cuda")
    idx2 = idx1.clone()
    cnt1 = torch.zeros((B, Hkv), dtype=torch.int32, device="cuda")
    cnt2 = cnt1.clone()
    o1 = torch.empty((B, Hkv * G, 128), dtype=torch.float32, device="cuda")
    l1 = torch.empty((B, Hkv * G), dtype=torch.float32, device="cuda")
    qc1 = hk.hamming_scan_query(h, q, codes, N, n_sink, n_local, k, ws1)
    hk.select_attend(bits, q, K, V, N, n_sink, n_local, k, idx1, cnt1, o1, l1, ws1)
    o2, l2, _, _, qc2 = hk.decode_step(h, q, codes, K, V, N, n_sink, n_local, k, idx=idx2,
                                       count=cnt2, ws=ws2)
    torch.cuda.synchronize()
    assert np.array_equal(np_u32(qc1), np_u32(qc2))
    assert torch.equal(cnt1, cnt2)
    keff = int(cnt1[0, 0])
    assert torch.equal(idx1[..., :keff], idx2[..., :keff])
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert float((o1 - o2).abs().max()) <= tol
    fin = torch.isfinite(l1)
    assert torch.equal(fin, torch.isfinite(l2))
    if bool(fin.any()):
        assert float((l1[fin] - l2[fin]).abs().max()) <= tol
    if mode == "far" and keff:
        # every candidate at distance bits: the first k_eff candidates in index order
        want = np.arange(n_sink, n_sink + keff)
        assert np.array_equal(idx2[0, 0, :keff].cpu().numpy(), want)


def _check_all_selections(codes, qcodes, idx, count, N, n_sink, n_local, k):
    codes, qcodes = np_u32(codes), np_u32(qcodes)
    idx, count = idx.cpu().numpy(), count.cpu().numpy()
    for b in range(codes.shape[0]):
        for g in range(codes.shape[1]):
            want = oracle.select_topk(codes[b, g], qcodes[b, g], N, n_sink, n_local, k)
            assert count[b, g] == want.size and np.array_equal(idx[b, g, :want.size], want), (b, g)


def test_invalid_arguments_enqueue_nothing():
    c = torch.zeros((1, 1, 10, 4), dtype=torch.int32, device="cuda")
    q = torch.zeros((1, 1, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(hk.HkError) as e:
        hk.retrieve_topk(c, q, 96, 10, 0, 0, 3)
    assert e.value.status == hk.HK_ERR_UNSUPPORTED
    with pytest.raises(hk.HkError) as e:
        hk.retrieve_topk(c, q, 128, 11, 0, 0, 3)              # n_ctx > cap
    assert e.value.status == hk.HK_ERR_INVALID_ARGUMENT
    ws = torch.empty(1, dtype=torch.uint8, device="cuda")
    with pytest.raises(hk.HkError) as e:
        hk.retrieve_topk(c, q, 128, 10, 0, 0, 3, ws=ws)
    assert e.value.status == hk.HK_ERR_WORKSPACE_TOO_SMALL


# ----------------------------------------------------------------- fused step
FUSED_CASES = [
    # bits, dtype, B, Hq, Hkv, N, s, w, k, pool
    (128, "f32", 1, 1, 1, 4096, 4, 64, 82, 0),
    (128, "bf16", 2, 8, 2, 20000, 4, 64, 400, 5),
    (64, "bf16", 1, 7, 1, 9000, 4, 512, 181, 0),
    (128, "bf16", 1, 4, 4, 60, 4, 64, 82, 0),       # no candidates: the window only
    (128, "bf16", 2, 4, 2, 1000, 0, 0, 50, 0),      # no window
    (128, "bf16", 1, 4, 2, 1000, 4, 64, 0, 0),      # k = 0: the window only
    (128, "bf16", 1, 2, 2, 0, 4, 64, 10, 0),        # empty context
    (128, "f32", 2, 16, 2, 70000, 4, 512, 1400, 0), # several window slices, G = 8
    # heads whose bin counts just fit in LDS (64 chunks x 64 bins, 32 x 128) and one
    # chunk more, which read them from memory
    (64, "bf16", 1, 2, 2, 65536 + 68, 4, 64, 1300, 3),
    (64, "bf16", 1, 2, 2, 65536 + 69, 4, 64, 1300, 0),
    (128, "bf16", 1, 4, 2, 32768 + 68, 4, 64, 655, 4),
    (128, "bf16", 1, 4, 2, 32768 + 69, 4, 64, 655, 0),
    # pool < 0: a share of -pool/10 of the tokens at distance `bits` (the complement of
    # the query code, not counted in the histograms), so that T = bits
    (128, "bf16", 1, 4, 2, 5000, 4, 64, 100, -10),
    (64, "bf16", 2, 2, 2, 9000, 4, 64, 5000, -6),
    (128, "bf16", 1, 4, 2, 70000 + 68, 4, 64, 40000, -6),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "-".join(map(str, c)))
def test_retrieve_attend_matches_oracle_and_unfused(case):
    bits, dtype, B, Hq, Hkv, N, s, w, k, pool = case
    say(f"retrieve_attend {case}")
    W = bits // 32
    rng = np.random.default_rng(N + k + 7)
    cap = N + 5
    if pool > 0:
        table = rng.integers(0, 2 ** 32, size=(pool, W), dtype=np.uint32)
        codes = table[rng.integers(0, pool, size=(B, Hkv, cap))]
    else:
        codes = rng.integers(0, 2 ** 32, size=(B, Hkv, cap, W), dtype=np.uint32)
    qc = rng.integers(0, 2 ** 32, size=(B, Hkv, W), dtype=np.uint32)
    if pool < 0:
        far = rng.random((B, Hkv, cap)) < -pool / 10
        codes = np.where(far[..., None], ~qc[:, :, None, :], codes)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    K = torch.from_numpy(rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32) * 1.5).to(tdt).cuda()
    V = torch.from_numpy(rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32)).to(tdt).cuda()
    Q = torch.from_numpy(rng.standard_normal((B, Hq, 128)).astype(np.float32) * 1.5).to(tdt).cuda()
    c, q = codes_tensor(codes), codes_tensor(qc)
    o, lse, idx, cnt = hk.retrieve_attend(c, q, bits, Q, K, V, N, s, w, k)
    torch.cuda.synchronize()
    o, lse, idx, cnt = o.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    Kd, Vd, Qd = (x.cpu().to(torch.float64).numpy() for x in (K, V, Q))
    G = Hq // Hkv
    tol = 1e-5 if dtype == "f32" else 2e-2
    scale = 1 / math.sqrt(128)
    win = oracle.window_indices(N, s, w)
    worst = 0.0
    for b in range(B):
        for h in range(Hkv):
            sel = oracle.select_topk(codes[b, h], qc[b, h], N, s, w, k)
            assert cnt[b, h] == sel.size and np.array_equal(idx[b, h, :sel.size], sel)
            for g in range(G):
                hq = h * G + g
                o1, l1 = oracle.attend(Qd[b, hq], Kd[b, h][sel], Vd[b, h][sel], scale)
                o2, l2 = oracle.attend(Qd[b, hq], Kd[b, h][win], Vd[b, h][win], scale)
                ro, rl = oracle.lse_merge(np.stack([o1, o2]), np.array([l1, l2]))
                assert np.max(np.abs(o[b, hq] - ro)) <= tol
                assert (rl == -np.inf and lse[b, hq] == -np.inf) or abs(lse[b, hq] - rl) <= tol
                worst = max(worst, float(np.max(np.abs(o[b, hq] - ro))))
    say(f"  max |o - oracle| = {worst:.2e}")
    # the unfused calls give the same result
    if N > 0:
        from hash_top_kv_amd.step import DecodeStep
        st = DecodeStep(K, V, c, bits, N, s, w, k, Hq)
        o2, l2 = st.unfused(Q, q)
        torch.cuda.synchronize()
        # bf16 paths round the softmax weights to bf16 before the P.V product, against
        # running maxima that differ between the two schedules
        assert np.allclose(o2.cpu().numpy(), o, atol=tol, rtol=0)
        l2 = l2.cpu().numpy()
        fin = np.isfinite(lse)
        assert np.array_equal(fin, np.isfinite(l2)) and np.allclose(l2[fin], lse[fin], atol=tol, rtol=0)


# ----------------------------------------------------------------- sign codes
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sign_codes_keys_queries_and_step(dtype):
    """SIGN hash (bit j = sign of element j): key codes bit-exact, query codes of the
    group mean within the near-zero exemption, and a whole decode step against the
    oracle."""
    B, Hkv, G, N = 2, 2, 3, 5000
    wl = synth.scaled(synth.WORKLOADS[1], B=B, Hkv=Hkv, Hq=Hkv * G, N=N, dtype=dtype,
                      hashes=(synth.HashSpec("sign", 128),), k=100, n_sink=4, n_local=64)
    kv = synth.make_kv(wl)
    qn = synth.make_q(wl)
    K, V = synth.to_device(kv["K"], dtype), synth.to_device(kv["V"], dtype)
    h = hk.Hash("sign", 128, dtype=K.dtype)
    hp = oracle.prepare_hash(synth.make_hash(wl, wl.hashes[0]))
    codes = torch.full((B, Hkv, N, 4), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    hk.encode_keys(h, K, codes, 3, N)
    Q = synth.to_device(qn, dtype)
    qc = hk.encode_query(h, Q, Hkv)
    torch.cuda.synchronize()
    got = np_u32(codes)
    for b in range(B):
        for g in range(Hkv):
            ref, _ = oracle.encode(oracle.widen(kv["K"][b, g, 3:], dtype), hp)
            assert np.array_equal(got[b, g, 3:], ref)
            assert np.all(got[b, g, :3] == 0x5A5A5A5A)
    ref_q, yq = oracle.encode_query(oracle.widen(qn, dtype), hp, Hkv)
    compare_codes(np_u32(qc), ref_q, yq)
    hk.encode_keys(h, K, codes, 0, 3)
    from hash_top_kv_amd.step import DecodeStep
    st = DecodeStep(K, V, codes, 128, N, 4, 64, wl.k, wl.Hq, h)
    o, lse = st(Q)
    torch.cuda.synchronize()
    cc = np_u32(codes)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for b in range(B):
        ref = oracle.decode_step(oracle.widen(qn[b], dtype), oracle.widen(kv["K"][b], dtype),
                                 oracle.widen(kv["V"][b], dtype), cc[b], hp, N, 4, 64, wl.k,
                                 qcodes=np_u32(qc)[b])
        for g in range(Hkv):
            assert np.array_equal(st.idx[b, g, :st.keff].cpu().numpy(), ref["idx"][g])
        assert np.max(np.abs(o[b].cpu().numpy() - ref["o"])) <= tol
        assert np.max(np.abs(lse[b].cpu().numpy() - ref["lse"])) <= tol


# ----------------------------------------------------------------- variable lengths
VARLEN_CASES = [
    # bits, dtype, Hq, Hkv, cap, lengths, s, w, k
    (128, "bf16", 8, 2, 9000, (9000, 4711, 70, 0, 2049, 8999), 4, 64, 180),
    (64, "bf16", 7, 1, 30000, (30000, 12345, 68, 1), 4, 512, 600),
    (128, "f32", 4, 4, 5000, (5000, 3000), 4, 64, 100),
    (128, "bf16", 4, 2, 3000, (3000, 3000, 3000), 0, 0, 60),     # equal lengths, no window
    # enough chunks for several per workgroup, so shorter sequences spread fewer chunks
    (128, "bf16", 8, 2, 50000, (50000, 31000, 12000, 47000, 5000, 2000), 4, 64, 100),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: "-".join(map(str, c[:5])) + f"-B{len(c[5])}")
def test_retrieve_attend_varlen_matches_oracle_per_sequence(case):
    """Each sequence of a variable-length batch gives what the oracle gives for that
    sequence alone with its own n_ctx (selection bit-exact, attention within the bound),
    including sequences with no candidates and an empty one."""
    bits, dtype, Hq, Hkv, cap, lengths, s, w, k = case
    say(f"retrieve_attend_varlen {case}")
    B, W = len(lengths), bits // 32
    rng = np.random.default_rng(cap + B)
    codes = rng.integers(0, 2 ** 32, size=(B, Hkv, cap, W), dtype=np.uint32)
    qc = rng.integers(0, 2 ** 32, size=(B, Hkv, W), dtype=np.uint32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    K = torch.from_numpy(rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32) * 1.5).to(tdt).cuda()
    V = torch.from_numpy(rng.standard_normal((B, Hkv, cap, 128)).astype(np.float32)).to(tdt).cuda()
    Q = torch.from_numpy(rng.standard_normal((B, Hq, 128)).astype(np.float32) * 1.5).to(tdt).cuda()
    ctx = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    o, lse, idx, cnt = hk.retrieve_attend_varlen(codes_tensor(codes), codes_tensor(qc), bits, Q, K, V,
                                                 ctx, max(lengths), s, w, k)
    torch.cuda.synchronize()
    o, lse, idx, cnt = o.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    Kd, Vd, Qd = (x.cpu().to(torch.float64).numpy() for x in (K, V, Q))
    G = Hq // Hkv
    tol = 1e-5 if dtype == "f32" else 2e-2
    scale = 1 / math.sqrt(128)
    for b, n in enumerate(lengths):
        win = oracle.window_indices(n, s, w)
        for h in range(Hkv):
            sel = oracle.select_topk(codes[b, h], qc[b, h], n, s, w, k)
            assert cnt[b, h] == sel.size and np.array_equal(idx[b, h, :sel.size], sel), (b, h)
            for g in range(G):
                hq = h * G + g
                o1, l1 = oracle.attend(Qd[b, hq], Kd[b, h][sel], Vd[b, h][sel], scale)
                o2, l2 = oracle.attend(Qd[b, hq], Kd[b, h][win], Vd[b, h][win], scale)
                ro, rl = oracle.lse_merge(np.stack([o1, o2]), np.array([l1, l2]))
                assert np.max(np.abs(o[b, hq] - ro)) <= tol, (b, hq)
                assert (rl == -np.inf and lse[b, hq] == -np.inf) or abs(lse[b, hq] - rl) <= tol
    if len(set(lengths)) == 1:
        # equal lengths: the same as the uniform call, bit for bit
        o2, l2, i2, c2 = hk.retrieve_attend(codes_tensor(codes), codes_tensor(qc), bits, Q, K, V,
                                            lengths[0], s, w, k)
        torch.cuda.synchronize()
        assert np.array_equal(o2.cpu().numpy(), o) and np.array_equal(l2.cpu().numpy(), lse)
        assert np.array_equal(c2.cpu().numpy(), cnt)


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 3 * (1 << 20) + 16 * 7, 64 << 20])
def test_read_probe_reads_every_byte(nbytes):
    """The measurement probe reads the whole buffer: the XOR of its per-workgroup words is
    the XOR of every 32-bit word of the buffer."""
    say(f"read_probe {nbytes} bytes")
    rng = np.random.default_rng(nbytes % 1000)
    data = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    x = torch.from_numpy(data.view(np.int32)).cuda()
    sink = hkp.read_probe(x)
    torch.cuda.synchronize()
    words = int(hkp.lib().hk_read_probe_sink_words(nbytes))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)[:words])
    assert got == np.bitwise_xor.reduce(data)


@pytest.mark.parametrize("rpb", [16, 512, 4096])
def test_gather_probe_reads_every_row(rpb):
    """The gather probe reads the K and V row of every list entry, duplicates and
    out-of-range entries (row 0) included: the XOR of its sink equals the XOR of those
    rows' words."""
    say(f"gather_probe rows_per_block={rpb}")
    rng = np.random.default_rng(rpb)
    rows = 5000
    Kw = rng.integers(0, 2 ** 32, size=(rows, 64), dtype=np.uint32)
    Vw = rng.integers(0, 2 ** 32, size=(rows, 64), dtype=np.uint32)
    idx = rng.integers(0, rows, size=9001).astype(np.int32)
    idx[::97] = idx[3]                                     # duplicates
    idx[5], idx[77], idx[-1] = -3, rows, 2 ** 31 - 1       # outside the table: row 0
    k = torch.from_numpy(Kw.view(np.int32)).cuda()
    v = torch.from_numpy(Vw.view(np.int32)).cuda()
    sink = hkp.gather_probe(k, v, torch.from_numpy(idx).cuda(), rpb)
    torch.cuda.synchronize()
    words = int(hkp.lib().hk_gather_probe_sink_words(idx.size, rpb))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)[:words])
    eff = np.where((idx >= 0) & (idx < rows), idx, 0)
    want = np.bitwise_xor.reduce(Kw[eff].ravel()) ^ np.bitwise_xor.reduce(Vw[eff].ravel())
    assert got == want


def test_retrieve_attend_fp32_two_chunk_groups():
    """fp32 K/V at the batch-16 x 131072 shape (8 KV heads, 32 query heads, sink 4 + local
    512, top-2%), where the fused step runs two chunk groups per workgroup: sampled heads
    against the oracle (top-k bit for bit, attention within the fp32 bound).  Inputs are
    drawn on the device."""
    B, Hkv, G, N, s, w, k = 16, 8, 4, 131072, 4, 512, 2621
    Hq = Hkv * G
    say("retrieve_attend fp32, 16 x 8 x 131072, two chunk groups per workgroup")
    gen = torch.Generator(device="cuda").manual_seed(123)
    K = torch.randn((B, Hkv, N, 128), generator=gen, device="cuda")
    V = torch.randn((B, Hkv, N, 128), generator=gen, device="cuda")
    q = torch.randn((B, Hq, 128), generator=gen, device="cuda")
    codes = torch.randint(-2 ** 31, 2 ** 31 - 1, (B, Hkv, N, 4), generator=gen, device="cuda",
                          dtype=torch.int32)
    qc = torch.randint(-2 ** 31, 2 ** 31 - 1, (B, Hkv, 4), generator=gen, device="cuda",
                       dtype=torch.int32)
    o, lse, idx, count = hk.retrieve_attend(codes, qc, 128, q, K, V, N, s, w, k)
    torch.cuda.synchronize()
    o, lse, idx, count = (t.cpu().numpy() for t in (o, lse, idx, count))
    scale = 1 / np.sqrt(128)
    win = oracle.window_indices(N, s, w)
    for b, g in [(0, 0), (15, 7), (9, 3)]:
        cc = np_u32(codes[b, g])
        want = oracle.select_topk(cc, np_u32(qc[b, g]), N, s, w, k)
        assert count[b, g] == want.size and np.array_equal(idx[b, g, :want.size], want), (b, g)
        Kf = K[b, g].double().cpu().numpy()
        Vf = V[b, g].double().cpu().numpy()
        for h in range(G):
            qh = q[b, g * G + h].double().cpu().numpy()
            o1, l1 = oracle.attend(qh, Kf[want], Vf[want], scale)
            o2, l2 = oracle.attend(qh, Kf[win], Vf[win], scale)
            ro, rl = oracle.lse_merge(np.stack([o1, o2]), np.array([l1, l2]))
            assert np.max(np.abs(o[b, g * G + h] - ro)) <= 1e-5 and abs(lse[b, g * G + h] - rl) <= 1e-5
    del K, V
    torch.cuda.empty_cache()

