"""Seeded synthetic inputs for the linear-recurrence scans.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds no arithmetic of the scans themselves: it only draws random tensors
with the shapes and value distributions of the five workloads and rounds them
to the I/O precision.  Both the CPU oracle and the GPU path consume exactly the
arrays produced here.

Recipe (one stream per tensor):
    rng = numpy.random.default_rng(SeedSequence([seed, cfg_id, tensor_id]))
    draw in float64 -> round to float32 (RNE) -> round to bfloat16 (RNE) for
    tensors whose I/O type is bf16.  ``A`` and ``Dskip`` are always float32.

Distributions (per workload, see ``CONFIGS``):
    diag       a ~ U(0.90, 0.999), b ~ N(0, 1), float32
    selective  x, B, C ~ N(0, 1); dt = softplus(N(-4, 1)); A[d, n] = -(n + 1);
               Dskip ~ N(0, 1)
    ssd        x, B, C ~ N(0, 1); dt = softplus(N(-4, 1));
               A_h = -exp(U(0, ln 16)); Dskip ~ N(0, 1); dy ~ N(0, 1)
    gla        q, k ~ N(0, 1)/sqrt(K); v ~ N(0, 1); g = sigmoid(N(3, 1))
    rotlru     r ~ U(0.90, 0.999), theta ~ U(-pi, pi), u ~ N(0, 1)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SEED = 2026

# Full-size workloads.  Index = the workload id used in the seed sequence.
CONFIGS = {
    1: dict(kind="diag", io="f32", B=1, L=1024, D=256),
    2: dict(kind="selective", io="bf16", B=8, L=4096, D=2048, N=16, disc="zoh"),
    3: dict(kind="ssd", io="bf16", B=8, L=2048, H=32, P=64, G=1, N=128, chunk=256),
    4: dict(kind="gla", io="bf16", B=8, L=4096, H=16, K=128, V=128, chunk=64),
    5: dict(kind="ssd_bwd", io="bf16", B=4, L=8192, H=32, P=64, G=1, N=128,
            chunk=256, seg=256),
    # rotational LRU on the diagonal workload's shape (D/2 = 128 channel pairs)
    6: dict(kind="rotlru", io="f32", B=1, L=1024, D=256),
}

NAMES = {
    1: "diag_rglru_fp32_B1_D256_L1024",
    2: "mamba1_selective_zoh_bf16_B8_D2048_N16_L4096",
    3: "mamba2_ssd_bf16_B8_H32_P64_N128_L2048",
    4: "gla_bf16_B8_H16_K128_V128_L4096",
    5: "ssd_fwd_bwd_ckpt_bf16_B4_H32_P64_N128_L8192_seg256",
    6: "rotlru_fp32_B1_D256_L1024",
}

_CHUNK = 1 << 22  # elements per draw call; keeps peak host memory bounded


def round_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> float32, round-to-nearest-even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64/float32 -> float32 array holding bf16-representable values."""
    return bits_to_f32(bf16_bits(round_f32(x)))


@dataclass
class Tensor:
    """One generated tensor: float32 values and the I/O type they stand for."""
    name: str
    values: np.ndarray          # float32, already rounded to ``io``
    io: str                     # "f32" or "bf16"

    def bits(self) -> np.ndarray:
        assert self.io == "bf16"
        return bf16_bits(self.values)


@dataclass
class Inputs:
    cfg_id: int
    params: dict
    tensors: dict = field(default_factory=dict)

    def __getitem__(self, k):
        return self.tensors[k].values

    def t(self, k) -> Tensor:
        return self.tensors[k]

    def f64(self, k) -> np.ndarray:
        return self.tensors[k].values.astype(np.float64)


class _Stream:
    def __init__(self, seed, cfg_id, tensor_id):
        self.rng = np.random.default_rng(np.random.SeedSequence([seed, cfg_id, tensor_id]))

    def normal(self, shape, mean=0.0, std=1.0):
        n = int(np.prod(shape))
        out = np.empty(n, dtype=np.float32)
        for i in range(0, n, _CHUNK):
            m = min(_CHUNK, n - i)
            out[i:i + m] = round_f32(mean + std * self.rng.standard_normal(m))
        return out.reshape(shape)

    def uniform(self, shape, lo, hi):
        n = int(np.prod(shape))
        out = np.empty(n, dtype=np.float32)
        for i in range(0, n, _CHUNK):
            m = min(_CHUNK, n - i)
            out[i:i + m] = round_f32(self.rng.uniform(lo, hi, m))
        return out.reshape(shape)

    def softplus_normal(self, shape, mean, std):
        n = int(np.prod(shape))
        out = np.empty(n, dtype=np.float32)
        for i in range(0, n, _CHUNK):
            m = min(_CHUNK, n - i)
            z = mean + std * self.rng.standard_normal(m)
            out[i:i + m] = round_f32(np.logaddexp(0.0, z))
        return out.reshape(shape)

    def sigmoid_normal(self, shape, mean, std):
        n = int(np.prod(shape))
        out = np.empty(n, dtype=np.float32)
        for i in range(0, n, _CHUNK):
            m = min(_CHUNK, n - i)
            z = mean + std * self.rng.standard_normal(m)
            out[i:i + m] = round_f32(1.0 / (1.0 + np.exp(-z)))
        return out.reshape(shape)


def _io_round(x32: np.ndarray, io: str) -> np.ndarray:
    return round_bf16(x32) if io == "bf16" else x32


def make(cfg_id: int, seed: int = SEED, **over) -> Inputs:
    """Generate the inputs of workload ``cfg_id``; keyword overrides change
    shapes (e.g. ``L=65``) or the I/O type (``io="f32"``) while keeping the
    value distributions.  ``grads=True`` adds a seeded upstream gradient of
    the outputs (dh, dy or do, N(0, 1)) for backward cases."""
    p = dict(CONFIGS[cfg_id])
    p.update(over)
    io = p["io"]
    out = Inputs(cfg_id, p)
    kind = p["kind"]

    def put(name, arr, tio):
        out.tensors[name] = Tensor(name, np.ascontiguousarray(_io_round(arr, tio)), tio)

    if kind == "diag":
        B, L, D = p["B"], p["L"], p["D"]
        put("a", _Stream(seed, cfg_id, 0).uniform((B, L, D), 0.90, 0.999), io)
        put("b", _Stream(seed, cfg_id, 1).normal((B, L, D)), io)
        if p.get("grads"):
            put("dh", _Stream(seed, cfg_id, 2).normal((B, L, D)), io)
    elif kind == "rotlru":
        B, L, D = p["B"], p["L"], p["D"]
        put("r", _Stream(seed, cfg_id, 0).uniform((B, L, D // 2), 0.90, 0.999), io)
        put("theta", _Stream(seed, cfg_id, 1).uniform((B, L, D // 2), -math.pi, math.pi), io)
        put("u", _Stream(seed, cfg_id, 2).normal((B, L, D)), io)
        if p.get("grads"):
            put("dh", _Stream(seed, cfg_id, 3).normal((B, L, D)), io)
    elif kind == "selective":
        B, L, D, N = p["B"], p["L"], p["D"], p["N"]
        put("x", _Stream(seed, cfg_id, 0).normal((B, L, D)), io)
        put("dt", _Stream(seed, cfg_id, 1).softplus_normal((B, L, D), -4.0, 1.0), io)
        A = -np.broadcast_to(np.arange(1, N + 1, dtype=np.float32), (D, N))
        put("A", np.ascontiguousarray(A), "f32")
        put("B", _Stream(seed, cfg_id, 3).normal((B, L, N)), io)
        put("C", _Stream(seed, cfg_id, 4).normal((B, L, N)), io)
        put("Dskip", _Stream(seed, cfg_id, 5).normal((D,)), "f32")
        if p.get("grads"):
            put("dy", _Stream(seed, cfg_id, 6).normal((B, L, D)), io)
    elif kind in ("ssd", "ssd_bwd"):
        B, L, H, P, G, N = p["B"], p["L"], p["H"], p["P"], p["G"], p["N"]
        put("x", _Stream(seed, cfg_id, 0).normal((B, L, H, P)), io)
        put("dt", _Stream(seed, cfg_id, 1).softplus_normal((B, L, H), -4.0, 1.0), io)
        u = _Stream(seed, cfg_id, 2).uniform((H,), 0.0, math.log(16.0)).astype(np.float64)
        put("A", round_f32(-np.exp(u)), "f32")
        put("B", _Stream(seed, cfg_id, 3).normal((B, L, G, N)), io)
        put("C", _Stream(seed, cfg_id, 4).normal((B, L, G, N)), io)
        put("Dskip", _Stream(seed, cfg_id, 5).normal((H,)), "f32")
        if kind == "ssd_bwd":
            put("dy", _Stream(seed, cfg_id, 6).normal((B, L, H, P)), io)
    elif kind == "gla":
        B, L, H, K, V = p["B"], p["L"], p["H"], p["K"], p["V"]
        s = 1.0 / math.sqrt(K)
        put("q", _Stream(seed, cfg_id, 0).normal((B, L, H, K), 0.0, s), io)
        put("k", _Stream(seed, cfg_id, 1).normal((B, L, H, K), 0.0, s), io)
        put("v", _Stream(seed, cfg_id, 2).normal((B, L, H, V)), io)
        put("g", _Stream(seed, cfg_id, 3).sigmoid_normal((B, L, H), 3.0, 1.0), io)
        if p.get("grads"):
            put("do", _Stream(seed, cfg_id, 4).normal((B, L, H, V)), io)
    else:
        raise ValueError(kind)
    return out


def state_normal(shape, cfg_id: int, tensor_id: int = 20, seed: int = SEED,
                 std: float = 1.0) -> np.ndarray:
    """A seeded float32 tensor for optional fp32 state inputs (h0, S0,
    dh_last) used by parity cases."""
    return _Stream(seed, cfg_id, tensor_id).normal(shape, 0.0, std)


def softplus_normal(shape, cfg_id: int, mean: float, std: float = 1.0, tensor_id: int = 30,
                    seed: int = SEED, io: str = "f32") -> np.ndarray:
    """A seeded step tensor softplus(N(mean, std)) rounded to ``io``, for
    parity cases whose steps are far from the workloads' (e.g. mean = -9:
    steps near 1e-4)."""
    return _io_round(_Stream(seed, cfg_id, tensor_id).softplus_normal(shape, mean, std), io)
