"""The decode step captured in a HIP graph and replayed: every replay, with eager work
and synchronisations between replays, must reproduce the eager results bit for bit (the
kernels are deterministic and the step allocates nothing)."""
import numpy as np
import pytest
import torch

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


@pytest.mark.parametrize("variant", ["fused", "unfused", "qheads", "varlen"])
def test_graph_replays_equal_eager(variant):
    from hash_top_kv_amd.step import DecodeStep, QHeadStep, VarlenDecodeStep
    say(f"graph replay, {variant} step")
    wl = synth.scaled(synth.WORKLOADS[1], B=2, Hq=8, Hkv=2, N=20000, k=400)
    spec = wl.hashes[0]
    kv = synth.make_kv(wl)
    K, V = synth.to_device(kv["K"], wl.dtype), synth.to_device(kv["V"], wl.dtype)
    h = hk.Hash(spec.kind, spec.bits, **synth.hash_to_device(synth.make_hash(wl, spec)))
    codes = torch.empty((wl.B, wl.Hkv, wl.N, spec.words), dtype=torch.int32, device="cuda")
    hk.encode_keys(h, K, codes)
    Qs = [synth.to_device(synth.make_q(wl, replica=r), wl.dtype) for r in range(3)]
    if variant == "qheads":
        mk = lambda: QHeadStep(K, V, codes, spec.bits, wl.N, wl.n_sink, wl.n_local, wl.k, wl.Hq, h)
    elif variant == "varlen":
        ctx_len = torch.tensor([wl.N, wl.N // 3], dtype=torch.int32, device="cuda")
        mk = lambda: VarlenDecodeStep(K, V, codes, spec.bits, ctx_len, wl.N, wl.n_sink,
                                      wl.n_local, wl.k, wl.Hq, h)
    else:
        mk = lambda: DecodeStep(K, V, codes, spec.bits, wl.N, wl.n_sink, wl.n_local, wl.k, wl.Hq, h)
    steps = [mk(), mk(), mk()]

    def run(st, q):
        return st.unfused(q) if variant == "unfused" else st(q)

    def snapshot(st, out):
        return [t.clone() for t in out] + [st.idx.clone(), st.count.clone()]

    eager = []
    for st, q in zip(steps[:2], Qs[:2]):
        eager.append(snapshot(st, run(st, q)))
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        outs = [run(st, q) for st, q in zip(steps[:2], Qs[:2])]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = [run(st, q) for st, q in zip(steps[:2], Qs[:2])]
    for rep in range(4):
        # eager work between replays: another step, a torch op, a synchronisation
        for st in steps[:2]:
            st.o.fill_(float("nan"))
            st.idx.fill_(-7)
        run(steps[2], Qs[2])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for st, out, ref in zip(steps[:2], outs, eager):
            got = snapshot(st, out)
            for a, b in zip(got, ref):
                assert torch.equal(a, b), f"replay {rep} differs from the eager step"
