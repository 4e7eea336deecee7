"""Pins of the oracle's hash encoders (LSH and MLP), GELU and bf16 rounding."""
import math
import os

import numpy as np
import pytest
import torch
from scipy.optimize import brentq

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lsh(R, dtype="f32"):
    return oracle.prepare_hash({"kind": "lsh", "bits": R.shape[0], "dtype": dtype,
                                "R": np.asarray(R, dtype=np.float32)})


def _mlp(W1, W2, dtype="f32", round_hidden=None):
    hp = oracle.prepare_hash({"kind": "mlp", "bits": W2.shape[0], "dtype": dtype,
                              "W1": np.asarray(W1, np.float32), "W2": np.asarray(W2, np.float32)}
                             if dtype == "f32" else
                             {"kind": "mlp", "bits": W2.shape[0], "dtype": dtype,
                              "W1": synth.to_bf16_bits(W1), "W2": synth.to_bf16_bits(W2)})
    if round_hidden is not None:
        hp["round_hidden"] = round_hidden
    return hp


def _unit_pair(rng, d, theta):
    basis, _ = np.linalg.qr(rng.standard_normal((d, 2)))
    a, b = basis[:, 0], basis[:, 1]
    return a, math.cos(theta) * a + math.sin(theta) * b


def test_lsh_collision_rate_tracks_angle():
    """Sign random projections agree on a bit with probability 1 - theta/pi."""
    rng = np.random.default_rng(7)
    d, bits, draws = 128, 128, 200
    rows = [l.split() for l in open(os.path.join(GOLDEN, "lsh_collision.txt"))
            if l.strip() and not l.startswith("#")]
    for t_over_pi, p in ((float(a), float(b)) for a, b in rows):
        theta = t_over_pi * math.pi
        agree = 0
        for _ in range(draws):
            x, y = _unit_pair(rng, d, theta)
            hp = _lsh(rng.standard_normal((bits, d)).astype(np.float32))
            cx, _ = oracle.encode(x[None], hp)
            cy, _ = oracle.encode(y[None], hp)
            agree += bits - int(oracle.hamming(cx, cy[0])[0])
        n = bits * draws
        sigma = math.sqrt(max(p * (1 - p), 1.0 / n) / n)
        assert abs(agree / n - p) <= 4 * sigma + 1e-12, (t_over_pi, agree / n, p)


def test_lsh_scale_and_negation():
    rng = np.random.default_rng(8)
    hp = _lsh(rng.standard_normal((128, 128)).astype(np.float32))
    x = rng.standard_normal((50, 128))
    c, y = oracle.encode(x, hp)
    c2, _ = oracle.encode(3.7 * x, hp)
    assert np.array_equal(c, c2)
    cn, _ = oracle.encode(-x, hp)
    nz = oracle.pack_bits(y != 0)
    assert np.array_equal(cn & nz, (~c) & nz)


def test_lsh_orientation_row_j_gives_bit_j():
    """R [bits, d], row j is the projection of bit j: with R a permutation matrix,
    bit j = [x[perm[j]] > 0].  A transposed R would give x[perm^-1[j]]."""
    rng = np.random.default_rng(9)
    perm = rng.permutation(128)
    R = np.zeros((128, 128), dtype=np.float32)
    R[np.arange(128), perm] = 1.0
    x = rng.standard_normal((20, 128))
    c, _ = oracle.encode(x, _lsh(R))
    assert np.array_equal(oracle.unpack_bits(c, 128), x[:, perm] > 0)
    R64 = R[:64]                                    # a 64-bit projection
    c64, _ = oracle.encode(x, _lsh(R64))
    assert c64.shape == (20, 2)
    assert np.array_equal(oracle.unpack_bits(c64, 64), x[:, perm[:64]] > 0)


def test_zero_and_sign_conventions():
    hp = _lsh(np.eye(128, dtype=np.float32)[:64])
    x = np.zeros((1, 128))
    x[0, 1] = 1.0
    x[0, 2] = -1.0
    c, _ = oracle.encode(x, hp)
    assert _bits(c[0], 64) == {1}                  # +0, -0 and negatives give 0
    x[0, 0] = -0.0
    assert _bits(oracle.encode(x, hp)[0][0], 64) == {1}


def _bits(words, nb):
    return {j for j in range(nb) if (int(words[j // 32]) >> (j % 32)) & 1}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mlp_identity_weights_reduce_to_sign_code(dtype):
    """W1 = [P1; 0], W2 = [P2 0]: y_j = rho(GELU(x[P1[P2[j]]])), and GELU keeps the
    sign, so the code is sign(x) permuted -- the sign-based 1-bit code of the
    Self-Indexing KVCache page (Abstract)."""
    rng = np.random.default_rng(10)
    p1, p2 = rng.permutation(128), rng.permutation(128)
    W1 = np.zeros((256, 128), np.float32)
    W1[np.arange(128), p1] = 1.0
    W2 = np.zeros((128, 256), np.float32)
    W2[np.arange(128), p2] = 1.0
    x = rng.standard_normal((40, 128))
    c, y = oracle.encode(x, _mlp(W1, W2, dtype))
    assert np.array_equal(oracle.unpack_bits(c, 128), x[:, p1[p2]] > 0)
    cl, _ = oracle.encode(x[:, p1[p2]], _lsh(np.eye(128, dtype=np.float32)))
    assert np.array_equal(c, cl)


def test_gelu_against_math_erf_and_identities():
    grid = np.linspace(-6, 6, 2401)
    want = np.array([v * 0.5 * (1 + math.erf(v / math.sqrt(2))) for v in grid])
    assert np.max(np.abs(oracle.gelu(grid) - want)) < 1e-15
    # x*Phi(x) - (-x)*Phi(-x) = x ; GELU(0) = 0 ; GELU(-1) = -0.15865525393145707
    assert np.max(np.abs(oracle.gelu(grid) - oracle.gelu(-grid) - grid)) < 1e-14
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.gelu(np.array([-1.0]))[0] + 0.15865525393145707) < 1e-15


def test_mlp_uses_gelu_not_relu():
    """y = h0 + h1 with a0 = -1 (GELU -0.1587, ReLU 0) and a1 = 0.1 (GELU 0.0540):
    the GELU form gives y < 0, a ReLU would give y > 0."""
    W1 = np.zeros((256, 128), np.float32)
    W1[0, 0] = W1[1, 1] = 1.0
    W2 = np.zeros((128, 256), np.float32)
    W2[0, 0] = W2[0, 1] = 1.0
    x = np.zeros((1, 128))
    x[0, 0], x[0, 1] = -1.0, 0.1
    c, y = oracle.encode(x, _mlp(W1, W2, "f32"))
    assert abs(y[0, 0] - (-0.15865525393145707 + 0.1 * 0.5 * (1 + math.erf(0.1 / math.sqrt(2))))) < 1e-15
    assert not (int(c[0, 0]) & 1)


def test_round_bf16_against_torch_and_ties():
    rng = np.random.default_rng(12)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x32.astype(np.float64)), want)
    # ties to even, exactly at the midpoint
    assert oracle.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert oracle.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # direct rounding from float64: just above the midpoint goes up (a float32 detour
    # would land on the tie and round down to 1.0)
    assert oracle.round_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(np.array([-(1.0 + 2.0 ** -8 + 2.0 ** -40)]))[0] == -(1.0 + 2.0 ** -7)
    # the bf16 subnormal grid
    assert oracle.round_bf16(np.array([3 * 2.0 ** -134]))[0] == 2.0 ** -132


def test_mlp_hidden_is_rounded_after_gelu():
    """h0 = GELU(a0) = 1.0060 and h1 = GELU(a1) = 1.0050 both round to bf16 1.0078125,
    so y = rho(h0) - rho(h1) = 0 (bit 0) when the hidden layer is bf16, and y = 0.001
    (bit 1) when it is not."""
    a0 = brentq(lambda a: oracle.gelu(np.array([a]))[0] - 1.0060, 0.5, 2.0, xtol=1e-15)
    a1 = brentq(lambda a: oracle.gelu(np.array([a]))[0] - 1.0050, 0.5, 2.0, xtol=1e-15)
    W1 = np.zeros((256, 128), np.float32)
    W1[0, 0] = W1[1, 1] = 1.0
    W2 = np.zeros((128, 256), np.float32)
    W2[0, 0], W2[0, 1] = 1.0, -1.0
    x = np.zeros((1, 128))
    x[0, 0], x[0, 1] = a0, a1
    c_r, y_r = oracle.encode(x, _mlp(W1, W2, "f32", round_hidden=True))
    c_n, y_n = oracle.encode(x, _mlp(W1, W2, "f32", round_hidden=False))
    assert y_r[0, 0] == 0.0 and not (int(c_r[0, 0]) & 1)
    assert abs(y_n[0, 0] - 0.001) < 1e-12 and (int(c_n[0, 0]) & 1)
    # a bf16 hash turns the rounding on
    assert _mlp(W1, W2, "bf16")["round_hidden"] and not _mlp(W1, W2, "f32")["round_hidden"]


def test_mlp_biases_enter_before_gelu_and_before_sign():
    W1 = np.zeros((256, 128), np.float32)
    W1[0, 0] = 1.0
    W2 = np.zeros((128, 256), np.float32)
    W2[0, 0] = 1.0
    hp = oracle.prepare_hash({"kind": "mlp", "bits": 128, "dtype": "f32", "W1": W1, "W2": W2,
                              "b1": np.full(256, 2.0, np.float32),
                              "b2": np.full(128, -0.5, np.float32)})
    x = np.zeros((1, 128))
    x[0, 0] = -1.0                        # a = -1 + 2 = 1, GELU(1) = 0.8413, y = 0.3413
    _, y = oracle.encode(x, hp)
    assert abs(y[0, 0] - (1.0 * 0.5 * (1 + math.erf(1 / math.sqrt(2))) - 0.5)) < 1e-15
    assert abs(y[0, 1] + 0.5) < 1e-15     # row with W2 = 0: just b2
    # hidden units with zero pre-activation weights still see b1: GELU(2) * W2 = 0 here


def test_group_mean_query_code():
    """The KV head's query code is the code of the mean of its G query heads; for LSH
    (scale free) that is the code of the sum, and G identical heads give that head's
    own code.  Query head h belongs to KV head h // G."""
    rng = np.random.default_rng(13)
    hp = _lsh(rng.standard_normal((128, 128)).astype(np.float32))
    q = rng.standard_normal((2, 8, 128))
    codes, y = oracle.encode_query(q, hp, Hkv=2)
    for b in range(2):
        for h in range(2):
            c_sum, _ = oracle.encode(q[b, 4 * h:4 * h + 4].sum(axis=0)[None], hp)
            assert np.array_equal(codes[b, h], c_sum[0])
    same = np.repeat(q[:, :1], 8, axis=1)
    c_same, _ = oracle.encode_query(same, hp, Hkv=4)
    c_one, _ = oracle.encode(q[:, 0], hp)
    for h in range(4):
        assert np.array_equal(c_same[:, h], c_one)


def test_near_zero_mask():
    y = np.array([[0.5, -2e-4, 9e-4, -1e-3, 1.5e-3] + [1.0] * 59])
    m = oracle.near_zero_mask(y)
    assert _bits(m[0], 64) == {1, 2}


def test_widen_bf16_is_exact():
    vals = np.array([1.0, -2.5, 0.0078125, 3.0e38, 1.0e-38], dtype=np.float32)
    u = synth.to_bf16_bits(vals)
    got = oracle.widen(u, "bf16")
    want = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, want)


def test_sign_hash_is_the_sign_of_each_element():
    """SIGN codes (identity projection) against bit-by-bit signs, with zero, negative
    zero and NaN giving 0, and against LSH with R = I."""
    rng = np.random.default_rng(91)
    x = rng.standard_normal((50, 128))
    x[0, :5] = [0.0, -0.0, np.nan, 1e-30, -1e-30]
    hp = oracle.prepare_hash({"kind": "sign", "bits": 128, "dtype": "f32"})
    codes, y = oracle.encode(x, hp)
    for r in range(50):
        for j in range(128):
            want = 1 if (x[r, j] == x[r, j] and x[r, j] > 0) else 0
            assert (int(codes[r, j // 32]) >> (j % 32)) & 1 == want
    lsh = oracle.prepare_hash({"kind": "lsh", "bits": 128, "dtype": "f32",
                               "R": np.eye(128, dtype=np.float32)})
    assert np.array_equal(oracle.encode(x[1:], lsh)[0], codes[1:])
