"""Seeded synthetic inputs for the binary-hash KV-cache retrieval decode step.

This module is shared by the tests, the benchmark and the CPU oracle's callers.  It
holds the shapes of the five synthetic workloads and the random draws that fill them,
and none of the method's arithmetic: no hashing, no distances, no selection and no
attention.  Hash parameters (the Gaussian projection of angular LSH, the weights of
the two-layer hash MLP) are random draws too, so they are produced here and passed as
inputs to both the HIP path and the oracle.

Workload geometry ("two narrow cones"): Spotlight Attention (Problem) and
RetrievalAttention (Key points: query-key distribution gap) both describe queries and
keys as occupying different, nearly orthogonal regions.  Keys of one KV head are
``4*u_k + 0.5*z`` and queries ``4*u_q + 0.5*z`` with ``u_k``, ``u_q`` random unit
vectors and ``z ~ N(0, I)``; values are ``N(0, 1)``.

Every tensor comes from its own NumPy PCG64 stream keyed by
``SeedSequence([0x484B, workload_id, tensor_id, b, head, (replica)])`` so that
generation can run per head, in parallel, and is reproducible bit for bit.

Rounding recipe: draws are made in float32 (R, W1, W2 in float64, then rounded to
float32); bf16 tensors are the float32 values rounded to nearest-even by PyTorch's CPU
conversion.  bf16 tensors are returned as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED_TAG = 0x484B

# tensor ids inside the seed key
T_HASH, T_UK, T_K, T_UQ, T_Q, T_V, T_CODES, T_PLANT, T_QCODE = range(9)

D_HEAD = 128
HIDDEN = 256


@dataclass(frozen=True)
class HashSpec:
    kind: str          # "lsh" or "mlp"
    bits: int          # 64 or 128
    hidden: int = HIDDEN

    @property
    def words(self) -> int:
        return self.bits // 32


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    dtype: str                 # "f32" or "bf16" (K, V, Q and hash weights)
    hashes: tuple = ()         # HashSpec(s); empty when codes are given directly
    k: int = 0
    n_sink: int = 0
    n_local: int = 0
    codes_given: bool = False  # uniform random codes + planted near neighbours
    planted_radius: int = 8
    d: int = D_HEAD
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def cap(self) -> int:
        return self.N


def budget_percent(n: int, pct: int) -> int:
    """ceil(pct% of n) in integer arithmetic: the per-head retrieval budget."""
    return (pct * n + 99) // 100


WORKLOADS = {
    0: Workload(0, "single-head d128 N4096 fp32 LSH-128", B=1, Hq=1, Hkv=1, N=4096,
                dtype="f32", hashes=(HashSpec("lsh", 128),), k=budget_percent(4096, 2),
                n_sink=4, n_local=64),
    1: Workload(1, "Llama-3-8B layer 32q/8kv N32768 bf16 MLP-128", B=1, Hq=32, Hkv=8,
                N=32768, dtype="bf16", hashes=(HashSpec("mlp", 128),),
                k=budget_percent(32768, 2), n_sink=4, n_local=64),
    2: Workload(2, "retrieval 8kv x 524288 tok 128-bit codes top-1024", B=1, Hq=8, Hkv=8,
                N=524288, dtype="bf16", hashes=(), k=1024, n_sink=0, n_local=0,
                codes_given=True),
    3: Workload(3, "batch16 x 131072 tok 32q/8kv bf16 MLP-128", B=16, Hq=32, Hkv=8,
                N=131072, dtype="bf16", hashes=(HashSpec("mlp", 128),),
                k=budget_percent(131072, 2), n_sink=4, n_local=512),
    4: Workload(4, "Qwen2.5-7B layer 28q/4kv batch4 x 262144 tok bf16 LSH-64 | MLP-128",
                B=4, Hq=28, Hkv=4, N=262144, dtype="bf16",
                hashes=(HashSpec("lsh", 64), HashSpec("mlp", 128)),
                k=budget_percent(262144, 2), n_sink=4, n_local=64),
}


def scaled(wl: Workload, **over) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    fields = dict(wid=wl.wid, name=wl.name + " (scaled)", B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv,
                  N=wl.N, dtype=wl.dtype, hashes=wl.hashes, k=wl.k, n_sink=wl.n_sink,
                  n_local=wl.n_local, codes_given=wl.codes_given,
                  planted_radius=wl.planted_radius, d=wl.d)
    fields.update(over)
    return Workload(**fields)


def rng_for(wid: int, tensor: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [SEED_TAG, wid, tensor, *[int(i) for i in ids]])))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (round to nearest even), via PyTorch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for input bookkeeping only)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return x32 if dtype == "f32" else to_bf16_bits(x32)


def unit_vector(rng: np.random.Generator, d: int) -> np.ndarray:
    z = rng.standard_normal(d)
    return z / np.linalg.norm(z)


def _cone_rows(wl, tensor_u, tensor_z, b, h, n, out):
    u = unit_vector(rng_for(wl.wid, tensor_u, b, h), wl.d).astype(np.float32)
    z = rng_for(wl.wid, tensor_z, b, h).standard_normal((n, wl.d), dtype=np.float32)
    x = np.float32(4.0) * u[None, :] + np.float32(0.5) * z
    out[...] = _store(x, wl.dtype)


def _normal_rows(wl, tensor, b, h, n, out):
    z = rng_for(wl.wid, tensor, b, h).standard_normal((n, wl.d), dtype=np.float32)
    out[...] = _store(z, wl.dtype)


def _storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def make_kv(wl: Workload, which: str = "kv", heads=None):
    """K and/or V, shape [B, Hkv, N, d] (float32 or bf16 bits).

    ``heads`` optionally restricts generation to a list of (b, h) pairs (the rest of
    the array stays zero); the values of a generated head never depend on the others.
    """
    dt = _storage_dtype(wl.dtype)
    out = {}
    jobs = []
    pairs = heads if heads is not None else [(b, h) for b in range(wl.B) for h in range(wl.Hkv)]
    if "k" in which:
        out["K"] = np.zeros((wl.B, wl.Hkv, wl.N, wl.d), dtype=dt)
        jobs += [(_cone_rows, (wl, T_UK, T_K, b, h, wl.N, out["K"][b, h])) for b, h in pairs]
    if "v" in which:
        out["V"] = np.zeros((wl.B, wl.Hkv, wl.N, wl.d), dtype=dt)
        jobs += [(_normal_rows, (wl, T_V, b, h, wl.N, out["V"][b, h])) for b, h in pairs]
    with ThreadPoolExecutor(_workers()) as ex:
        for f in [ex.submit(fn, *args) for fn, args in jobs]:
            f.result()
    return out


def make_q(wl: Workload, replica: int = 0) -> np.ndarray:
    """Queries of one decode step, shape [B, Hq, d]."""
    dt = _storage_dtype(wl.dtype)
    q = np.zeros((wl.B, wl.Hq, wl.d), dtype=dt)
    for b in range(wl.B):
        for h in range(wl.Hq):
            ids = (b, h) if replica == 0 else (b, h, replica)
            u = unit_vector(rng_for(wl.wid, T_UQ, *ids), wl.d).astype(np.float32)
            z = rng_for(wl.wid, T_Q, *ids).standard_normal((1, wl.d), dtype=np.float32)
            q[b, h] = _store(np.float32(4.0) * u[None, :] + np.float32(0.5) * z, wl.dtype)[0]
    return q


def make_hash(wl: Workload, spec: HashSpec, index: int = 0) -> dict:
    """Random hash parameters in the workload dtype.

    LSH: R [bits, d] ~ N(0, 1).  MLP: W1 [hidden, d] ~ N(0, 1/d), W2 [bits, hidden]
    ~ N(0, 1/hidden), no biases.  SIGN: none (bits = d).  Values are returned in storage
    form (float32 or bf16 bits) together with the spec.
    """
    rng = rng_for(wl.wid, T_HASH, index)
    out = {"kind": spec.kind, "bits": spec.bits, "hidden": spec.hidden, "dtype": wl.dtype}
    if spec.kind == "lsh":
        r = rng.standard_normal((spec.bits, wl.d)).astype(np.float32)
        out["R"] = _store(r, wl.dtype)
    elif spec.kind == "mlp":
        w1 = (rng.standard_normal((spec.hidden, wl.d)) / math.sqrt(wl.d)).astype(np.float32)
        w2 = (rng.standard_normal((spec.bits, spec.hidden)) / math.sqrt(spec.hidden)).astype(np.float32)
        out["W1"] = _store(w1, wl.dtype)
        out["W2"] = _store(w2, wl.dtype)
    elif spec.kind != "sign":              # the identity: no parameters
        raise ValueError(spec.kind)
    return out


def make_given_codes(wl: Workload, bits: int = 128, replica: int = 0, heads=None):
    """Uniform random cached codes with planted near neighbours of the query code.

    Returns dict(codes [B,Hkv,N,W] u32, qcodes [B,Hkv,W] u32, planted_pos [B,Hkv,P]
    int64, planted_delta [B,Hkv,P] int64).  P = ceil(1% of N) planted tokens per head
    at uniform distinct positions; planted token i copies the query code with
    ``delta_i ~ U{0..radius}`` distinct uniformly chosen bits flipped.
    """
    W = bits // 32
    P = budget_percent(wl.N, 1)
    codes = np.zeros((wl.B, wl.Hkv, wl.N, W), dtype=np.uint32)
    qcodes = np.zeros((wl.B, wl.Hkv, W), dtype=np.uint32)
    ppos = np.zeros((wl.B, wl.Hkv, P), dtype=np.int64)
    pdel = np.zeros((wl.B, wl.Hkv, P), dtype=np.int64)
    pairs = heads if heads is not None else [(b, h) for b in range(wl.B) for h in range(wl.Hkv)]

    def one(b, h):
        ids = (b, h) if replica == 0 else (b, h, replica)
        codes[b, h] = rng_for(wl.wid, T_CODES, *ids).integers(
            0, 2 ** 32, size=(wl.N, W), dtype=np.uint32)
        qc = rng_for(wl.wid, T_QCODE, *ids).integers(0, 2 ** 32, size=W, dtype=np.uint32)
        qcodes[b, h] = qc
        r = rng_for(wl.wid, T_PLANT, *ids)
        pos = r.choice(wl.N, size=P, replace=False)
        delta = r.integers(0, wl.planted_radius + 1, size=P)
        order = np.argsort(r.random((P, bits)), axis=1)          # random bit permutation
        flip = np.zeros((P, bits), dtype=bool)
        rows = np.arange(P)[:, None]
        sel = np.arange(bits)[None, :] < delta[:, None]
        flip[np.broadcast_to(rows, (P, bits))[sel], order[sel]] = True
        masks = np.packbits(flip, axis=1, bitorder="little").view("<u4").astype(np.uint32)
        codes[b, h, pos] = qc[None, :] ^ masks
        ppos[b, h] = pos
        pdel[b, h] = delta

    with ThreadPoolExecutor(_workers()) as ex:
        for f in [ex.submit(one, b, h) for b, h in pairs]:
            f.result()
    return {"codes": codes, "qcodes": qcodes, "planted_pos": ppos, "planted_delta": pdel}


def describe(wl: Workload) -> dict:
    return {"workload": wl.name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "N": wl.N,
            "d": wl.d, "dtype": wl.dtype, "k": wl.k, "n_sink": wl.n_sink,
            "n_local": wl.n_local,
            "hashes": [f"{h.kind}-{h.bits}" for h in wl.hashes] or ["given-128"]}


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    """Upload a generated array: float32 as is, bf16 bit patterns as torch.bfloat16,
    uint32 codes as int32 (same bits)."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(device)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)


def hash_to_device(h: dict, device="cuda") -> dict:
    """Hash parameter tensors of make_hash() on the device (keys R / W1 / W2)."""
    return {k: to_device(h[k], h["dtype"], device) for k in ("R", "W1", "W2", "b1", "b2")
            if h.get(k) is not None}
