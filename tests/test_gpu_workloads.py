"""Parity at the five workloads' full sizes, in the launch configurations the
benchmark uses: every (batch, KV head)'s selection against the oracle's top-k of the
GPU's own codes, and the whole step on sampled (batch, KV head) pairs the oracle
computes one by one.

For each workload:
  * key codes: the whole cache is encoded on the GPU; sampled heads are compared with
    the oracle bit for bit, except bits whose oracle pre-sign value is below 1e-3
    (counted and reported);
  * retrieval: the sampled heads' cache codes are replaced by the oracle's codes, so
    both sides rank identical codes; the GPU's top-k must equal the oracle's exactly;
  * the decode step (query code, retrieval, top-k attention, window attention, merge):
    outputs within 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs) of the oracle.  When the
    query code has near-zero bits, every assignment of them is a correct code; the
    GPU's selection must match the oracle's selection for one of them.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import codes_tensor, compare_codes, np_u32, say

pytestmark = pytest.mark.gpu

hk = None
_CACHE = {}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global hk
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hash_top_kv_amd
    hk = hash_top_kv_amd
    yield
    _CACHE.clear()
    torch.cuda.empty_cache()


def _inputs(wid):
    """Generated inputs of a workload, on host and device (cached per module)."""
    if wid in _CACHE:
        return _CACHE[wid]
    _CACHE.clear()
    torch.cuda.empty_cache()
    wl = synth.WORKLOADS[wid]
    say(f"generating workload {wid}: {wl.name}")
    kv = synth.make_kv(wl)
    d = {"wl": wl, "kv": kv, "q": synth.make_q(wl),
         "K": synth.to_device(kv["K"], wl.dtype), "V": synth.to_device(kv["V"], wl.dtype)}
    d["Q"] = synth.to_device(d["q"], wl.dtype)
    _CACHE[wid] = d
    return d


def _sample_heads(wl, n=3):
    pairs = [(0, 0), (wl.B - 1, wl.Hkv - 1), (wl.B // 2, wl.Hkv // 2)]
    return list(dict.fromkeys(pairs))[:n]


def _oracle_head_step(qg, Kf, Vf, key_codes, qcode, wl, scale):
    """Oracle step of one (batch, KV head): top-k + window attention of its G query
    heads, merged.  qg [G, d], Kf/Vf [N, d] float64."""
    idx = oracle.select_topk(key_codes, qcode, wl.N, wl.n_sink, wl.n_local, wl.k)
    win = oracle.window_indices(wl.N, wl.n_sink, wl.n_local)
    o = np.zeros((qg.shape[0], qg.shape[1]))
    lse = np.zeros(qg.shape[0])
    for g in range(qg.shape[0]):
        o1, l1 = oracle.attend(qg[g], Kf[idx], Vf[idx], scale)
        o2, l2 = oracle.attend(qg[g], Kf[win], Vf[win], scale)
        o[g], lse[g] = oracle.lse_merge(np.stack([o1, o2]), np.array([l1, l2]))
    return idx, o, lse


def _check_head_step(gpu_idx, gpu_o, gpu_lse, qg, Kf, Vf, key_codes, qcode_ref, qy, wl, tol):
    scale = 1 / math.sqrt(wl.d)
    exempt_bits = [j for j in range(qy.size) if abs(qy[j]) < oracle.NEAR_ZERO][:4]
    variants = []
    for flips in itertools.product([0, 1], repeat=len(exempt_bits)):
        qc = qcode_ref.copy()
        for j, f in zip(exempt_bits, flips):
            if f:
                qc[j // 32] ^= np.uint32(1 << (j % 32))
        variants.append(_oracle_head_step(qg, Kf, Vf, key_codes, qc, wl, scale))
    match = [v for v in variants if np.array_equal(v[0], gpu_idx)]
    assert match, "GPU top-k matches no correct selection"
    _, ro, rl = match[0]
    err_o = float(np.max(np.abs(gpu_o - ro)))
    err_l = float(np.max(np.abs(gpu_lse - rl)))
    assert err_o <= tol and err_l <= tol, (err_o, err_l)
    return err_o, err_l


def _check_all_heads(codes, qcodes, idx, count, wl, lengths=None):
    """Every (batch, KV head) at full size: given the GPU's own key and query codes, the
    GPU's selection (count, ascending indices, ties to the lower index) must equal the
    oracle's top-k of those codes.  lengths: per-sequence context lengths, else wl.N."""
    codes, qcodes = np_u32(codes), np_u32(qcodes)
    idx, count = idx.cpu().numpy(), count.cpu().numpy()
    for b in range(wl.B):
        n = wl.N if lengths is None else lengths[b]
        for g in range(wl.Hkv):
            want = oracle.select_topk(codes[b, g, :n], qcodes[b, g], n, wl.n_sink, wl.n_local, wl.k)
            assert count[b, g] == want.size, (b, g)
            assert np.array_equal(idx[b, g, :want.size], want), (b, g)
    say(f"  all {wl.B * wl.Hkv} (batch, KV head) selections equal the oracle's on the GPU's codes")


def _encode_and_check(wl, spec, hidx, sample):
    d = _inputs(wl.wid)
    hnp = synth.make_hash(wl, spec, hidx)
    h = hk.Hash(spec.kind, spec.bits, dtype=d["K"].dtype, **synth.hash_to_device(hnp))
    codes = torch.zeros((wl.B, wl.Hkv, wl.N, spec.words), dtype=torch.int32, device="cuda")
    hk.encode_keys(h, d["K"], codes)
    torch.cuda.synchronize()
    hp = oracle.prepare_hash(hnp)
    ref_codes = {}
    flips = 0
    for b, g in sample:
        ref, y = oracle.encode(oracle.widen(d["kv"]["K"][b, g], wl.dtype), hp)
        flips += compare_codes(np_u32(codes[b, g]), ref, y)
        ref_codes[(b, g)] = ref
    say(f"  {spec.kind}-{spec.bits}: {len(sample)} heads x {wl.N} keys, exempt bits differing: {flips}")
    return h, hnp, hp, codes, ref_codes


def _run_workload(wid, hidx=0, spec=None, k=None):
    wl = synth.WORKLOADS[wid] if k is None else synth.scaled(synth.WORKLOADS[wid], k=k)
    spec = spec or wl.hashes[hidx]
    sample = _sample_heads(wl)
    d = _inputs(wid)
    h, hnp, hp, codes, ref_codes = _encode_and_check(wl, spec, hidx, sample)
    # identical codes on both sides for the sampled heads
    for (b, g), ref in ref_codes.items():
        codes[b, g] = codes_tensor(ref)
    from hash_top_kv_amd.step import DecodeStep
    step = DecodeStep(d["K"], d["V"], codes, spec.bits, wl.N, wl.n_sink, wl.n_local, wl.k, wl.Hq, h)
    o, lse = step(d["Q"])
    torch.cuda.synchronize()
    _check_all_heads(codes, step.qcodes, step.idx, step.count, wl)
    gq = np_u32(step.qcodes)
    qref, qy = oracle.encode_query(oracle.widen(d["q"], wl.dtype), hp, wl.Hkv)
    compare_codes(gq, qref, qy)
    # retrieval with identical query codes too: bit-exact top-k
    idx_same, cnt_same = hk.retrieve_topk(codes, codes_tensor(qref), spec.bits, wl.N, wl.n_sink,
                                          wl.n_local, wl.k)
    idx_same = idx_same.cpu().numpy()
    G = wl.G
    tol = 1e-5 if wl.dtype == "f32" else 2e-2
    gidx = step.idx.cpu().numpy()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    for b, g in sample:
        want = oracle.select_topk(ref_codes[(b, g)], qref[b, g], wl.N, wl.n_sink, wl.n_local, wl.k)
        assert np.array_equal(idx_same[b, g, :want.size], want), (b, g)
        Kf = oracle.widen(d["kv"]["K"][b, g], wl.dtype)
        Vf = oracle.widen(d["kv"]["V"][b, g], wl.dtype)
        qg = oracle.widen(d["q"][b, g * G:(g + 1) * G], wl.dtype)
        e = _check_head_step(gidx[b, g, :step.keff], o[b, g * G:(g + 1) * G], lse[b, g * G:(g + 1) * G],
                             qg, Kf, Vf, ref_codes[(b, g)], qref[b, g], qy[b, g], wl, tol)
        say(f"  head {(b, g)}: max|do| {e[0]:.2e} max|dlse| {e[1]:.2e}")


def test_workload0_single_head_fp32_lsh128():
    _run_workload(0)


def test_workload1_llama3_8b_mlp128():
    _run_workload(1)


def test_workload3_batch16_131072_mlp128():
    _run_workload(3)


def test_workload3_large_budget():
    """The batch-16 workload with k = 40000: two chunk groups per workgroup, each group
    selecting about 5000 tokens, more than the workgroup's list holds at once."""
    _run_workload(3, k=40000)


def test_workload3_sign_codes():
    """Sign codes (bit j = sign of element j) at full size: keys and query codes bit for
    bit, the step on sampled heads."""
    _run_workload(3, spec=synth.HashSpec("sign", 128))


def test_workload3_per_sequence_lengths():
    """The batch-16 workload with the benchmark's per-sequence lengths (131072 down to
    69632): each sampled sequence against the oracle's step at its own length."""
    wl = synth.WORKLOADS[3]
    spec = wl.hashes[0]
    sample = _sample_heads(wl)
    d = _inputs(3)
    h, hnp, hp, codes, ref_codes = _encode_and_check(wl, spec, 0, sample)
    for (b, g), ref in ref_codes.items():
        codes[b, g] = codes_tensor(ref)
    lengths = [wl.N - (b * wl.N) // (2 * wl.B) for b in range(wl.B)]
    ctx_len = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    from hash_top_kv_amd.step import VarlenDecodeStep
    step = VarlenDecodeStep(d["K"], d["V"], codes, spec.bits, ctx_len, wl.N, wl.n_sink,
                            wl.n_local, wl.k, wl.Hq, h)
    o, lse = step(d["Q"])
    torch.cuda.synchronize()
    _check_all_heads(codes, step.qcodes, step.idx, step.count, wl, lengths)
    qref, qy = oracle.encode_query(oracle.widen(d["q"], wl.dtype), hp, wl.Hkv)
    compare_codes(np_u32(step.qcodes), qref, qy)
    gidx, gcnt = step.idx.cpu().numpy(), step.count.cpu().numpy()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    G = wl.G
    for b, g in sample:
        n = lengths[b]
        wb = synth.scaled(wl, N=n)
        keff = max(0, min(wl.k, n - wl.n_sink - wl.n_local))
        assert gcnt[b, g] == keff, (b, g)
        Kf = oracle.widen(d["kv"]["K"][b, g], wl.dtype)
        Vf = oracle.widen(d["kv"]["V"][b, g], wl.dtype)
        qg = oracle.widen(d["q"][b, g * G:(g + 1) * G], wl.dtype)
        e = _check_head_step(gidx[b, g, :keff], o[b, g * G:(g + 1) * G], lse[b, g * G:(g + 1) * G],
                             qg, Kf, Vf, ref_codes[(b, g)][:n], qref[b, g], qy[b, g], wb, 2e-2)
        say(f"  sequence {b} (n = {n}), head {g}: max|do| {e[0]:.2e} max|dlse| {e[1]:.2e}")


def test_workload4_qwen_lsh64():
    _run_workload(4, 0)


def test_workload4_qwen_mlp128():
    _run_workload(4, 1)


def test_workload4_sign_codes():
    """Sign codes at full size on the GQA 7:1 workload."""
    _run_workload(4, spec=synth.HashSpec("sign", 128))


def test_workload4_per_query_head_step():
    """Per-query-head selection at full size (28 query heads over 4 KV heads x 262144
    LSH-64 codes, top-5243 each), as the benchmark's --qheads step runs it: every query
    head of one sequence against the oracle, indices bit for bit given identical codes."""
    wl = synth.WORKLOADS[4]
    spec = wl.hashes[0]
    d = _inputs(4)
    hnp = synth.make_hash(wl, spec, 0)
    h = hk.Hash(spec.kind, spec.bits, **synth.hash_to_device(hnp))
    codes = torch.empty((wl.B, wl.Hkv, wl.N, spec.words), dtype=torch.int32, device="cuda")
    hk.encode_keys(h, d["K"], codes)
    from hash_top_kv_amd.step import QHeadStep
    step = QHeadStep(d["K"], d["V"], codes, spec.bits, wl.N, wl.n_sink, wl.n_local, wl.k,
                     wl.Hq, h)
    o, lse = step(d["Q"])
    torch.cuda.synchronize()
    b = wl.B - 1
    qc = np_u32(step.qcodes)
    hp = oracle.prepare_hash(hnp)
    ref_q, yq = oracle.encode(oracle.widen(d["q"][b], wl.dtype), hp)
    compare_codes(qc[b], ref_q, yq)
    ref = oracle.decode_step_qheads(oracle.widen(d["q"][b], wl.dtype),
                                    oracle.widen(d["kv"]["K"][b], wl.dtype),
                                    oracle.widen(d["kv"]["V"][b], wl.dtype), np_u32(codes[b]), hp,
                                    wl.N, wl.n_sink, wl.n_local, wl.k, qcodes=qc[b])
    idx, count = step.idx.cpu().numpy(), step.count.cpu().numpy()
    for hq in range(wl.Hq):
        assert count[b, hq] == ref["idx"][hq].size
        assert np.array_equal(idx[b, hq, :count[b, hq]], ref["idx"][hq]), hq
    err_o = float(np.max(np.abs(o[b].cpu().numpy() - ref["o"])))
    err_l = float(np.max(np.abs(lse[b].cpu().numpy() - ref["lse"])))
    assert err_o <= 2e-2 and err_l <= 2e-2, (err_o, err_l)
    say(f"  sequence {b}: {wl.Hq} query heads, max|do| {err_o:.2e} max|dlse| {err_l:.2e}")


def test_workload4_exact_topk():
    """The exact top-k by logit at full size (4 x 4 x 262144 keys, top-5243), sampled
    heads: the count exact, every token clearly above the k-th logit selected and none
    clearly below (fp32 against fp64 logits)."""
    wl = synth.WORKLOADS[4]
    d = _inputs(4)
    idx, count = hk.exact_topk(d["Q"], d["K"], wl.N, wl.n_sink, wl.n_local, wl.k)
    torch.cuda.synchronize()
    idx, count = idx.cpu().numpy(), count.cpu().numpy()
    cand = oracle.candidate_range(wl.N, wl.n_sink, wl.n_local)
    keff = min(wl.k, cand.size)
    G = wl.G
    for b, g in _sample_heads(wl):
        assert count[b, g] == keff
        got = idx[b, g, :keff]
        assert np.all(np.diff(got) > 0) and got[0] >= wl.n_sink and got[-1] < wl.N - wl.n_local
        Kw = oracle.widen(d["kv"]["K"][b, g], wl.dtype)
        qg = oracle.widen(d["q"][b, g * G:(g + 1) * G], wl.dtype)
        want = oracle.exact_topk_group(qg, Kw, wl.N, wl.n_sink, wl.n_local, wl.k)
        score = Kw[cand] @ qg.sum(axis=0)
        band = 1e-5 * (np.abs(Kw[cand]) @ np.abs(qg).sum(axis=0))
        kth = np.sort(score)[::-1][keff - 1]
        sel = np.zeros(wl.N, bool)
        sel[got] = True
        assert sel[cand[score > kth + band]].all() and not sel[cand[score < kth - band]].any()
        say(f"  head {(b, g)}: {len(np.setxor1d(got, want)) // 2} swaps inside the rounding band")


@pytest.mark.parametrize("hidx", [0, 1])
def test_workload4_prefill_encode_sampled_rows(hidx):
    """The key encode of all 4 x 4 x 262144 keys (the prefill), sampled rows."""
    wl = synth.WORKLOADS[4]
    spec = wl.hashes[hidx]
    d = _inputs(4)
    hnp = synth.make_hash(wl, spec, hidx)
    h = hk.Hash(spec.kind, spec.bits, **synth.hash_to_device(hnp))
    codes = torch.zeros((wl.B, wl.Hkv, wl.N, spec.words), dtype=torch.int32, device="cuda")
    hk.encode_keys(h, d["K"], codes)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    rows = rng.integers(0, wl.B * wl.Hkv * wl.N, size=30000)
    flatK = d["kv"]["K"].reshape(-1, wl.d)
    ref, y = oracle.encode(oracle.widen(flatK[rows], wl.dtype), oracle.prepare_hash(hnp))
    got = np_u32(codes).reshape(-1, spec.words)[rows]
    n = compare_codes(got, ref, y)
    say(f"  {spec.kind}-{spec.bits}: 30000 sampled rows, exempt bits differing: {n}")


def test_workload2_fused_step_512k_planted():
    """The 512K retrieval step as the benchmark runs it: hk_hamming_scan, then
    hk_select_attend on the same workspace."""
    wl = synth.WORKLOADS[2]
    d = _inputs(2)
    g = synth.make_given_codes(wl)
    codes, qc = codes_tensor(g["codes"]), codes_tensor(g["qcodes"])
    B, Hkv, k = wl.B, wl.Hkv, wl.k
    ws = hk.workspace(hk.retrieve_attend_workspace(128, B, wl.Hq, Hkv, wl.N, 0, 0, k))
    idx = torch.empty((B, Hkv, k), dtype=torch.int32, device="cuda")
    count = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    o = torch.empty((B, wl.Hq, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, wl.Hq), dtype=torch.float32, device="cuda")
    hk.hamming_scan(codes, qc, 128, wl.N, 0, 0, k, ws)
    hk.select_attend(128, d["Q"], d["K"], d["V"], wl.N, 0, 0, k, idx, count, o, lse, ws)
    torch.cuda.synchronize()
    idx, count, o, lse = (t.cpu().numpy() for t in (idx, count, o, lse))
    for h in range(Hkv):
        pos, dl = g["planted_pos"][0, h], g["planted_delta"][0, h]
        closed = np.sort(pos[np.lexsort((pos, dl))[:k]])
        assert count[0, h] == k and np.array_equal(idx[0, h], closed), h
        Kf = oracle.widen(d["kv"]["K"][0, h][closed], wl.dtype)
        Vf = oracle.widen(d["kv"]["V"][0, h][closed], wl.dtype)
        ro, rl = oracle.attend(oracle.widen(d["q"][0, h], wl.dtype), Kf, Vf, 1 / math.sqrt(128))
        assert np.max(np.abs(o[0, h] - ro)) <= 2e-2 and abs(lse[0, h] - rl) <= 2e-2


def test_workload2_retrieval_512k_planted():
    wl = synth.WORKLOADS[2]
    d = _inputs(2)
    g = synth.make_given_codes(wl)
    codes, qc = codes_tensor(g["codes"]), codes_tensor(g["qcodes"])
    idx, count = hk.retrieve_topk(codes, qc, 128, wl.N, 0, 0, wl.k)
    o, lse = hk.sparse_decode(d["Q"], d["K"], d["V"], idx, wl.k, count=count)
    torch.cuda.synchronize()
    idx, o, lse = idx.cpu().numpy(), o.cpu().numpy(), lse.cpu().numpy()
    for h in range(wl.Hkv):
        pos, dl = g["planted_pos"][0, h], g["planted_delta"][0, h]
        closed = np.sort(pos[np.lexsort((pos, dl))[:wl.k]])
        assert np.array_equal(idx[0, h], closed), h
        assert np.array_equal(idx[0, h], oracle.select_topk(g["codes"][0, h], g["qcodes"][0, h],
                                                            wl.N, 0, 0, wl.k))
        Kf = oracle.widen(d["kv"]["K"][0, h][closed], wl.dtype)
        Vf = oracle.widen(d["kv"]["V"][0, h][closed], wl.dtype)
        ro, rl = oracle.attend(oracle.widen(d["q"][0, h], wl.dtype), Kf, Vf, 1 / math.sqrt(128))
        assert np.max(np.abs(o[0, h] - ro)) <= 2e-2 and abs(lse[0, h] - rl) <= 2e-2
