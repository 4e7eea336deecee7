"""Parity of HashEvict's eviction step (hk_evict_select, hk_evict_replace and the step
that uses them) with the CPU oracle: victims and cache updates bit-exact, attention
within the bf16 / fp32 bounds."""
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


def _codes(rng, B, Hkv, cap, W, pool):
    if pool:
        table = rng.integers(0, 2 ** 32, size=(pool, W), dtype=np.uint32)
        return table[rng.integers(0, pool, size=(B, Hkv, cap))]
    return rng.integers(0, 2 ** 32, size=(B, Hkv, cap, W), dtype=np.uint32)


EVICT_CASES = [
    # bits, B, Hkv, cap, n_ctx, s, w, pool (distinct codes -> ties at the maximum)
    (128, 2, 3, 5100, 5000, 4, 64, 0),
    (64, 2, 2, 9001, 9001, 4, 512, 0),
    (128, 1, 4, 4100, 4100, 0, 0, 3),           # heavy ties: lowest index must win
    (64, 3, 1, 70000, 69999, 4, 64, 5),         # many chunks, ragged tail
    (128, 1, 2, 100, 68, 4, 64, 0),             # no candidates: -1
    (64, 1, 2, 70, 69, 4, 64, 0),               # one candidate
    (128, 1, 1, 1, 1, 0, 0, 0),                 # one token
    (128, 2, 2, 64, 0, 0, 0, 0),                # empty context
]


@pytest.mark.parametrize("case", EVICT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_evict_select_matches_oracle(case):
    bits, B, Hkv, cap, n_ctx, s, w, pool = case
    say(f"evict_select {case}")
    W = bits // 32
    rng = np.random.default_rng(cap + 7 * B + Hkv)
    codes = _codes(rng, B, Hkv, cap, W, pool)
    q = rng.integers(0, 2 ** 32, size=(B, Hkv, W), dtype=np.uint32)
    if pool == 0 and n_ctx > s + w + 10:
        # plant the farthest code (the complement of the query) at three places; the
        # lowest of them is the victim
        for b in range(B):
            for h in range(Hkv):
                for j in sorted(rng.choice(np.arange(s, n_ctx - w), 3, replace=False)):
                    codes[b, h, j] = ~q[b, h]
    victim = hk.evict_select(codes_tensor(codes), codes_tensor(q), bits, n_ctx, s, w)
    torch.cuda.synchronize()
    got = victim.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            assert got[b, h] == oracle.evict_victim(codes[b, h], q[b, h], n_ctx, s, w), (b, h)


def test_evict_select_full_size():
    """Four sequences x 4 KV heads x 262144 cached 64-bit codes, as the step would run on
    a Qwen2.5-7B-shaped layer; every head's victim checked."""
    B, Hkv, N, W = 4, 4, 262144, 2
    rng = np.random.default_rng(41)
    codes = rng.integers(0, 2 ** 32, size=(B, Hkv, N, W), dtype=np.uint32)
    q = rng.integers(0, 2 ** 32, size=(B, Hkv, W), dtype=np.uint32)
    victim = hk.evict_select(codes_tensor(codes), codes_tensor(q), 64, N, 4, 64)
    torch.cuda.synchronize()
    got = victim.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            assert got[b, h] == oracle.evict_victim(codes[b, h], q[b, h], N, 4, 64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_evict_replace_writes_only_the_victim_slot(dtype):
    B, Hkv, cap, W = 2, 3, 777, 4
    rng = np.random.default_rng(43)
    wl = synth.scaled(synth.WORKLOADS[1], B=B, Hkv=Hkv, Hq=Hkv, N=cap, dtype=dtype)
    kv = synth.make_kv(wl)
    K, V = synth.to_device(kv["K"], dtype), synth.to_device(kv["V"], dtype)
    codes_np = rng.integers(0, 2 ** 32, size=(B, Hkv, cap, W), dtype=np.uint32)
    codes = codes_tensor(codes_np)
    k_new = torch.randn((B, Hkv, 128), device="cuda").to(K.dtype)
    v_new = torch.randn((B, Hkv, 128), device="cuda").to(K.dtype)
    code_new_np = rng.integers(0, 2 ** 32, size=(B, Hkv, W), dtype=np.uint32)
    victim_np = np.array([[5, -1, cap - 1], [0, cap, 400]], dtype=np.int32)   # -1, cap: no-ops
    K0, V0 = K.clone(), V.clone()
    hk.evict_replace(k_new, v_new, codes_tensor(code_new_np), torch.from_numpy(victim_np).cuda(),
                     K, V, codes)
    torch.cuda.synchronize()
    Kw, Vw, cw = K0.clone(), V0.clone(), codes_np.copy()
    for b in range(B):
        for h in range(Hkv):
            j = int(victim_np[b, h])
            if 0 <= j < cap:
                Kw[b, h, j], Vw[b, h, j], cw[b, h, j] = k_new[b, h], v_new[b, h], code_new_np[b, h]
    assert torch.equal(K, Kw) and torch.equal(V, Vw)
    assert np.array_equal(np_u32(codes), cw)


@pytest.mark.parametrize("case", [("lsh", 64, "bf16"), ("mlp", 128, "bf16"), ("lsh", 128, "f32")],
                         ids=lambda c: "-".join(map(str, c)))
def test_evict_step_matches_oracle(case):
    """Two consecutive steps of hash -> victim -> replace -> attention over the whole
    cache, against oracle.evict_step fed with the GPU's query codes (codes are compared
    separately, with the near-zero exemption)."""
    kind, bits, dtype = case
    B, Hkv, G, N, s, w = 2, 2, 3, 3000, 4, 64
    say(f"evict step {case}")
    wl = synth.scaled(synth.WORKLOADS[4], B=B, Hkv=Hkv, Hq=Hkv * G, N=N, dtype=dtype,
                      hashes=(synth.HashSpec(kind, bits),), n_sink=s, n_local=w)
    kv = synth.make_kv(wl)
    hnp = synth.make_hash(wl, wl.hashes[0])
    h = hk.Hash(kind, bits, **synth.hash_to_device(hnp))
    hp = oracle.prepare_hash(hnp)
    K, V = synth.to_device(kv["K"], dtype), synth.to_device(kv["V"], dtype)
    codes = torch.empty((B, Hkv, N, bits // 32), dtype=torch.int32, device="cuda")
    hk.encode_keys(h, K, codes)
    Kc = oracle.widen(kv["K"], dtype)
    Vc = oracle.widen(kv["V"], dtype)
    cc = np_u32(codes)
    from hash_top_kv_amd.step import EvictStep
    step = EvictStep(K, V, codes, bits, N, s, w, Hkv * G, h)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for it in range(2):
        q_np = synth.make_q(wl, replica=it + 1)
        new = synth.make_kv(synth.scaled(wl, N=1, wid=90 + it))
        q = synth.to_device(q_np, dtype)
        k_new = synth.to_device(new["K"][:, :, 0], dtype)
        v_new = synth.to_device(new["V"][:, :, 0], dtype)
        o, lse, victim = step(q, k_new, v_new)
        torch.cuda.synchronize()
        qc = np_u32(step.qcodes)
        cn = np_u32(step.code_new)
        ref_q, yq = oracle.encode_query(oracle.widen(q_np, dtype), hp, Hkv)
        compare_codes(qc, ref_q, yq)
        ref_n, yn = oracle.encode(oracle.widen(new["K"][:, :, 0], dtype).reshape(B * Hkv, -1), hp)
        compare_codes(cn.reshape(B * Hkv, -1), ref_n, yn)
        for b in range(B):
            ref = oracle.evict_step(oracle.widen(q_np[b], dtype), Kc[b], Vc[b], cc[b], qc[b],
                                    oracle.widen(new["K"][b, :, 0], dtype),
                                    oracle.widen(new["V"][b, :, 0], dtype), cn[b], N, s, w)
            assert np.array_equal(victim[b].cpu().numpy(), ref["victim"])
            assert np.max(np.abs(o[b].cpu().numpy() - ref["o"])) <= tol
            assert np.max(np.abs(lse[b].cpu().numpy() - ref["lse"])) <= tol
            Kc[b], Vc[b], cc[b] = ref["K"], ref["V"], ref["codes"]
        # the device cache now equals the oracle's updated cache
        assert np.array_equal(np_u32(codes), cc)
        assert np.array_equal(K.float().cpu().numpy().astype(np.float64), Kc)
