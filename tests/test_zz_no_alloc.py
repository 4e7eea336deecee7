"""hk_retrieve_attend_noalloc (the library's own workspace) against hk_retrieve_attend with a
caller workspace, on two calls in a row, the second with a smaller problem: the same
kernels run in both, so indices, counts, outputs and log-sum-exps must be identical."""
import math

import numpy as np
import pytest
import torch

import synth
from helpers import codes_tensor, say

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, N, bits, seed):
    """Seeded inputs: random codes (with a few repeated codes, so distances tie), a query
    code per KV head, bf16 queries and K/V drawn as in the workloads' two-cone picture."""
    rng = np.random.default_rng(seed)
    W = bits // 32
    pool = rng.integers(0, 2 ** 32, size=(B, Hkv, 64, W), dtype=np.uint32)
    pick = rng.integers(0, 64, size=(B, Hkv, N))
    codes = np.take_along_axis(pool, pick[..., None].repeat(W, axis=-1), axis=2)
    fresh = rng.random((B, Hkv, N)) < 0.5
    codes[fresh] = rng.integers(0, 2 ** 32, size=(int(fresh.sum()), W), dtype=np.uint32)
    qcodes = rng.integers(0, 2 ** 32, size=(B, Hkv, W), dtype=np.uint32)
    wl = synth.Workload(wid=300 + seed, name="no-alloc case", B=B, Hq=Hq, Hkv=Hkv, N=N,
                        dtype="bf16", hashes=(), k=1, n_sink=0, n_local=0)
    kv = synth.make_kv(wl)
    q = synth.make_q(wl)
    return (codes_tensor(codes), codes_tensor(qcodes), synth.to_device(q, "bf16"),
            synth.to_device(kv["K"], "bf16"), synth.to_device(kv["V"], "bf16"))


@pytest.fixture(scope="module")
def hk():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import hash_top_kv_amd
    return hash_top_kv_amd


def test_noalloc_matches_workspace_call_twice(hk):
    cases = [  # B, Hq, Hkv, N, bits, s, w, k  -- the second call is smaller
        (2, 16, 4, 40000, 128, 4, 64, 800),
        (1, 7, 1, 9001, 64, 4, 16, 150),
    ]
    for n, (B, Hq, Hkv, N, bits, s, w, k) in enumerate(cases):
        say(f"no-alloc call {n}: B={B} Hq={Hq} Hkv={Hkv} N={N} bits={bits} k={k}")
        codes, qcodes, q, K, V = _case(B, Hq, Hkv, N, bits, seed=n)
        o1, l1, i1, c1 = hk.retrieve_attend_noalloc(codes, qcodes, bits, q, K, V, N, s, w, k)
        o2, l2, i2, c2 = hk.retrieve_attend(codes, qcodes, bits, q, K, V, N, s, w, k)
        torch.cuda.synchronize()
        c1n, c2n = c1.cpu().numpy(), c2.cpu().numpy()
        assert np.array_equal(c1n, c2n)
        assert (c1n == min(k, N - s - w)).all()
        i1n, i2n = i1.cpu().numpy(), i2.cpu().numpy()
        for b in range(B):
            for h in range(Hkv):
                assert np.array_equal(i1n[b, h, :c1n[b, h]], i2n[b, h, :c2n[b, h]])
        assert np.array_equal(o1.cpu().numpy(), o2.cpu().numpy())
        assert np.array_equal(l1.cpu().numpy(), l2.cpu().numpy())
        assert np.isfinite(l1.cpu().numpy()).all()
