"""The seeded generators: reproducible, per-head independent, shaped as described."""
import numpy as np

import synth


def test_workload_shapes():
    w = synth.WORKLOADS
    assert (w[1].Hq, w[1].Hkv, w[1].G, w[1].N) == (32, 8, 4, 32768)
    assert (w[4].Hq, w[4].Hkv, w[4].G) == (28, 4, 7)
    assert [h.bits for h in w[4].hashes] == [64, 128]
    assert (w[3].n_sink, w[3].n_local, w[0].n_sink, w[0].n_local) == (4, 512, 4, 64)


def test_generation_is_reproducible_and_per_head():
    wl = synth.scaled(synth.WORKLOADS[1], B=2, N=64)
    a = synth.make_kv(wl)
    b = synth.make_kv(wl, heads=[(1, 3)])
    assert a["K"].dtype == np.uint16 and a["K"].shape == (2, 8, 64, 128)
    assert np.array_equal(a["K"][1, 3], b["K"][1, 3]) and np.array_equal(a["V"][1, 3], b["V"][1, 3])
    assert not np.array_equal(a["K"][1, 3], a["K"][1, 2])
    q1, q2 = synth.make_q(wl), synth.make_q(wl)
    assert np.array_equal(q1, q2) and not np.array_equal(q1, synth.make_q(wl, replica=1))


def test_two_cone_geometry():
    wl = synth.scaled(synth.WORKLOADS[0], N=2000)
    k = synth.make_kv(wl, "k")["K"][0, 0].astype(np.float64)
    q = synth.make_q(wl)[0, 0].astype(np.float64)
    uk = k.mean(axis=0) / np.linalg.norm(k.mean(axis=0))
    assert abs(np.linalg.norm(k.mean(axis=0)) - 4.0) < 0.1     # keys sit around 4 u_k
    assert abs(np.mean(np.sum(k * k, axis=1)) - (16 + 0.25 * 128)) < 1.5
    cos = float(q @ uk) / np.linalg.norm(q)
    assert abs(cos) < 0.5                                       # query off the key cone


def test_hash_params_and_planted_codes():
    wl = synth.WORKLOADS[4]
    lsh = synth.make_hash(wl, wl.hashes[0], 0)
    mlp = synth.make_hash(wl, wl.hashes[1], 1)
    assert lsh["R"].shape == (64, 128) and lsh["R"].dtype == np.uint16
    assert mlp["W1"].shape == (256, 128) and mlp["W2"].shape == (128, 256)
    w1 = synth.bf16_bits_to_f32(mlp["W1"])
    assert abs(w1.std() - 1 / np.sqrt(128)) < 0.005
    g = synth.make_given_codes(synth.scaled(synth.WORKLOADS[2], N=10000), heads=[(0, 1)])
    assert g["planted_pos"].shape[-1] == 100
    assert len(set(g["planted_pos"][0, 1].tolist())) == 100
    assert g["planted_delta"][0, 1].min() >= 0 and g["planted_delta"][0, 1].max() <= 8
