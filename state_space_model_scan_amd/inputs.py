"""Seeded synthetic inputs for the selective-scan forward workloads.

This module only draws random numbers and stores them in the io dtype; it holds
none of the operator's arithmetic.  Both the oracle side and the HIP side get
their inputs from here and nowhere else.

Workloads (shapes and distributions follow the page's selective_scan_fn
argument list: u/delta/z (batch, dim, seqlen), A (dim, dstate), B/C fixed
(dim, dstate), time-varying (batch, dstate, seqlen) or grouped
(batch, groups, dstate, seqlen), D/delta_bias (dim,)):

  tiny        b=1  d=16   l=64    n=4   fp32  varying B/C (g=1)  seed 0
  mamba130m   b=4  d=1536 l=2048  n=16  bf16  varying B/C (g=1)  seed 1
  mamba2p8b   b=8  d=5120 l=2048  n=16  bf16  grouped B/C g=4    seed 2
              A = -exp(N(0, 0.5))
  longseq     b=1  d=2560 l=65536 n=16  fp32  varying B/C, no z,  seed 3
              raw delta ~ N(-3, 0.5)
  convfixed   b=16 d=2048 l=4096  n=16  bf16  fixed B/C (d, n), conv prologue
              (width 4, weight ~ N(0, 0.5), bias ~ N(0, 1), silu), seed 4

Unless a workload says otherwise: u (or the conv input x), z, B, C, D ~ N(0, 1);
raw delta ~ N(-2, 0.5); delta_bias ~ U(-0.1, 0.1); softplus on;
A[d, s] = -(s + 1); D, z, delta_bias present; last_state requested.
N(mu, sigma) names the standard deviation.

Draw order from ``numpy.random.default_rng(seed)``, all in float32:
u (or x), delta, z, B, C, D, delta_bias, A-noise, conv weight, conv bias.
Large tensors are drawn in fixed chunks of CHUNK values, in order.
bf16 storage rounds the float32 draw to nearest, ties to even.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional

import numpy as np

CHUNK = 1 << 24

F32, BF16, F16 = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    dim: int
    seqlen: int
    dstate: int
    io_dtype: int             # F32 or BF16
    bc_kind: str              # "varying" or "fixed"
    ngroups: int = 1
    has_z: bool = True
    has_D: bool = True
    has_bias: bool = True
    softplus: bool = True
    delta_mean: float = -2.0
    delta_std: float = 0.5
    A_mode: str = "s4d"        # "s4d": A = -(s+1);  "lognormal": A = -exp(N(0, 0.5))
    conv: bool = False
    seed: int = 0

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.seqlen

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 16, 64, 4, F32, "varying", seed=0),
    "mamba130m": Workload("mamba130m", 4, 1536, 2048, 16, BF16, "varying", seed=1),
    "mamba2p8b": Workload("mamba2p8b", 8, 5120, 2048, 16, BF16, "varying", ngroups=4,
                          A_mode="lognormal", seed=2),
    "longseq": Workload("longseq", 1, 2560, 65536, 16, F32, "varying", has_z=False,
                        delta_mean=-3.0, seed=3),
    "convfixed": Workload("convfixed", 16, 2048, 4096, 16, BF16, "fixed", conv=True, seed=4),
}


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    """One decode step: selective_state_update against a cached fp32 state
    (batch, dim, dstate) and causal_conv1d_update against a conv cache
    (batch, dim, conv_state_len) with conv_tokens new tokens."""
    name: str
    batch: int
    dim: int
    dstate: int
    io_dtype: int
    ngroups: int = 1
    has_z: bool = True
    has_D: bool = True
    has_bias: bool = True
    softplus: bool = True
    conv_width: int = 4
    conv_state_len: int = 3
    conv_tokens: int = 1
    seed: int = 0

    @property
    def channels(self) -> int:
        return self.batch * self.dim

    def scaled(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


# decode2p8b: the Mamba-2.8B-shaped layer of mamba2p8b (d=5120, n=16, g=4,
# bf16) at a decode batch of 1024, whose 335 MB state exceeds the 256 MB
# last-level cache, so a step streams the state from HBM.
DECODE_WORKLOADS: Dict[str, DecodeWorkload] = {
    "decode_tiny": DecodeWorkload("decode_tiny", 2, 16, 4, F32, seed=10),
    "decode2p8b": DecodeWorkload("decode2p8b", 1024, 5120, 16, BF16, ngroups=4, seed=12),
}


@dataclasses.dataclass(frozen=True)
class SsdWorkload:
    """The Mamba-2 chunked scan: x, z (batch, seqlen, nheads, headdim), dt
    (batch, seqlen, nheads), B, C (batch, seqlen, ngroups, dstate), A, dt_bias
    (nheads), D (nheads) or (nheads, headdim), states (batch, nheads, headdim,
    dstate)."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    io_dtype: int = 1
    has_z: bool = True
    has_D: bool = True
    D_per_channel: bool = False
    has_bias: bool = True
    softplus: bool = True
    init_state: bool = False
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    @property
    def elements(self) -> int:
        return self.batch * self.seqlen * self.nheads * self.headdim

    def scaled(self, **kw) -> "SsdWorkload":
        return dataclasses.replace(self, **kw)


# ssd2p7b: a Mamba-2 2.7B-shaped layer (d_inner 5120 = 80 heads of 64, dstate
# 128, one B/C group) at batch 8 and 2048 tokens, bf16.
SSD_WORKLOADS: Dict[str, "SsdWorkload"] = {
    "ssd_tiny": SsdWorkload("ssd_tiny", 1, 100, 4, 64, 32, 2, init_state=True, seed=20),
    "ssd2p7b": SsdWorkload("ssd2p7b", 8, 2048, 80, 64, 128, 1, seed=22),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bits."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy: nearest, ties to even);
    return the bits."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(h, dtype=np.uint16).view(np.float16).astype(np.float32)


def io_bits_to_f64(a: np.ndarray, io_dtype: int) -> np.ndarray:
    """The values of stored io bits (any io dtype) as float64."""
    if io_dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    if io_dtype == F16:
        return f16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _normal(rng: np.random.Generator, shape, mean=0.0, std=1.0) -> np.ndarray:
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.float32)
    for i in range(0, total, CHUNK):
        j = min(total, i + CHUNK)
        out[i:j] = rng.standard_normal(j - i, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    if mean != 0.0:
        out += np.float32(mean)
    return out.reshape(shape)


def _uniform(rng: np.random.Generator, shape, lo, hi) -> np.ndarray:
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def _store(a: np.ndarray, io_dtype: int) -> np.ndarray:
    if io_dtype == BF16:
        return f32_to_bf16_bits(a)
    if io_dtype == F16:
        return f32_to_f16_bits(a)
    return np.ascontiguousarray(a, dtype=np.float32)


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every tensor of workload ``w``.

    io tensors come back as their stored bits (uint16 for bf16, float32 for fp32);
    parameters (A, D, delta_bias, conv weight/bias) are float32.  Absent optional
    tensors are ``None``.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    b, d, l, n, g = w.batch, w.dim, w.seqlen, w.dstate, w.ngroups
    io = w.io_dtype
    t: Dict[str, Optional[np.ndarray]] = {}
    first = _store(_normal(rng, (b, d, l)), io)
    if w.conv:
        t["conv_x"], t["u"] = first, None
    else:
        t["u"], t["conv_x"] = first, None
    t["delta"] = _store(_normal(rng, (b, d, l), w.delta_mean, w.delta_std), io)
    t["z"] = _store(_normal(rng, (b, d, l)), io) if w.has_z else None
    bc_shape = (d, n) if w.bc_kind == "fixed" else (b, g, n, l)
    t["B"] = _store(_normal(rng, bc_shape), io)
    t["C"] = _store(_normal(rng, bc_shape), io)
    t["D"] = _normal(rng, (d,)) if w.has_D else None
    t["delta_bias"] = _uniform(rng, (d,), -0.1, 0.1) if w.has_bias else None
    if w.A_mode == "lognormal":
        t["A"] = (-np.exp(_normal(rng, (d, n), 0.0, 0.5).astype(np.float64))).astype(np.float32)
    else:
        t["A"] = np.ascontiguousarray(
            np.broadcast_to(-(np.arange(n, dtype=np.float32) + 1.0), (d, n)))
    if w.conv:
        t["conv_weight"] = _normal(rng, (d, 4), 0.0, 0.5)
        t["conv_bias"] = _normal(rng, (d,))
    else:
        t["conv_weight"] = t["conv_bias"] = None
    return t


@dataclasses.dataclass(frozen=True)
class ComplexWorkload:
    """The selective scan with complex A (the page's section 4.1: A may be real
    or complex): u, delta, z (batch, dim, seqlen) real; A (dim, dstate, 2)
    float32 (real, imaginary) pairs; B, C complex io pairs, fixed
    (dim, dstate, 2) or varying (batch, ngroups, dstate, seqlen, 2)."""
    name: str
    batch: int
    dim: int
    seqlen: int
    dstate: int
    io_dtype: int
    bc_kind: str = "varying"     # "varying" or "fixed" (both B and C)
    ngroups: int = 1
    has_z: bool = True
    has_D: bool = True
    has_bias: bool = True
    softplus: bool = True
    delta_mean: float = -2.0
    delta_std: float = 0.5
    A_imag: str = "lin"          # "lin": Im A[d, s] = pi * s;  "normal": Im A ~ N(0, 3)
    init_state: bool = False
    seed: int = 0

    @property
    def elements(self) -> int:
        return self.batch * self.dim * self.seqlen

    def scaled(self, **kw) -> "ComplexWorkload":
        return dataclasses.replace(self, **kw)


# mamba2p8b_complex: the Mamba-2.8B-shaped layer of mamba2p8b (b=8, d=5120,
# l=2048, n=16, g=4, bf16) with complex A, B and C.
COMPLEX_WORKLOADS: Dict[str, ComplexWorkload] = {
    "complex_tiny": ComplexWorkload("complex_tiny", 2, 24, 100, 16, F32, ngroups=2, init_state=True,
                                    seed=30),
    "mamba2p8b_complex": ComplexWorkload("mamba2p8b_complex", 8, 5120, 2048, 16, BF16, ngroups=4,
                                         seed=32),
}


def make_complex_inputs(w: ComplexWorkload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every tensor of complex-A workload ``w``, in this order: u,
    delta (N(delta_mean, delta_std)), z, B, C (each component N(0, 1)), D,
    delta_bias (U(-0.1, 0.1)), Re A = -exp(N(0, 0.5)), Im A (pi * s, or
    N(0, 3) drawn here), initial state (batch, dim, dstate, 2) N(0, 1) when
    the workload has one.  Same storage rules as ``make_inputs``."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    b, d, l, n, g = w.batch, w.dim, w.seqlen, w.dstate, w.ngroups
    io = w.io_dtype
    t: Dict[str, Optional[np.ndarray]] = {}
    t["u"] = _store(_normal(rng, (b, d, l)), io)
    t["delta"] = _store(_normal(rng, (b, d, l), w.delta_mean, w.delta_std), io)
    t["z"] = _store(_normal(rng, (b, d, l)), io) if w.has_z else None
    bc_shape = (d, n, 2) if w.bc_kind == "fixed" else (b, g, n, l, 2)
    t["B"] = _store(_normal(rng, bc_shape), io)
    t["C"] = _store(_normal(rng, bc_shape), io)
    t["D"] = _normal(rng, (d,)) if w.has_D else None
    t["delta_bias"] = _uniform(rng, (d,), -0.1, 0.1) if w.has_bias else None
    A = np.empty((d, n, 2), dtype=np.float32)
    A[..., 0] = (-np.exp(_normal(rng, (d, n), 0.0, 0.5).astype(np.float64))).astype(np.float32)
    if w.A_imag == "normal":
        A[..., 1] = _normal(rng, (d, n), 0.0, 3.0)
    else:
        A[..., 1] = (np.pi * np.arange(n, dtype=np.float64)).astype(np.float32)
    t["A"] = A
    t["initial_state"] = _normal(rng, (b, d, n, 2)) if w.init_state else None
    return t


def make_dout(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """The output gradient of the backward: N(0, 1) of shape (batch, dim,
    seqlen) in the io dtype, from its own stream (seed + 1000)."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 1000)
    return _store(_normal(rng, (w.batch, w.dim, w.seqlen)), w.io_dtype)


def sha256(a: Optional[np.ndarray]) -> Optional[str]:
    if a is None:
        return None
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


def sample_rows(w: Workload, count: int, seed: int = 1234) -> np.ndarray:
    """A fixed spread of row ids (b*dim + d) for spot checks at full size:
    the first and last rows, group and block boundaries, plus random rows."""
    total = w.batch * w.dim
    rng = np.random.default_rng(seed)
    fixed = {0, 1, 63, 64, 65, w.dim - 1, w.dim, total - 1, total - 64}
    per_group = w.dim // w.ngroups
    for gi in range(w.ngroups):
        fixed.update({gi * per_group, gi * per_group + per_group - 1})
    fixed = {r for r in fixed if 0 <= r < total}
    extra = rng.choice(total, size=min(total, max(0, count - len(fixed))), replace=False)
    return np.array(sorted(fixed.union(int(r) for r in extra)), dtype=np.int64)


def make_decode_inputs(w: DecodeWorkload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every tensor of decode workload ``w``, in this order:
    x, dt (N(-2, 0.5)), z, B, C (b, g, n), D, dt_bias (U(-0.1, 0.1)), A
    (-exp(N(0, 0.5))), state (b, d, n) fp32 N(0, 1), conv x (b, d, conv_tokens),
    conv state (b, d, conv_state_len), conv weight (N(0, 0.5)), conv bias,
    cache_seqlens (b,) int32 uniform in [0, 4096).  Same storage rules as
    ``make_inputs``."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    b, d, n, g = w.batch, w.dim, w.dstate, w.ngroups
    io = w.io_dtype
    t: Dict[str, Optional[np.ndarray]] = {}
    t["x"] = _store(_normal(rng, (b, d)), io)
    t["dt"] = _store(_normal(rng, (b, d), -2.0, 0.5), io)
    t["z"] = _store(_normal(rng, (b, d)), io) if w.has_z else None
    t["B"] = _store(_normal(rng, (b, g, n)), io)
    t["C"] = _store(_normal(rng, (b, g, n)), io)
    t["D"] = _normal(rng, (d,)) if w.has_D else None
    t["dt_bias"] = _uniform(rng, (d,), -0.1, 0.1) if w.has_bias else None
    t["A"] = (-np.exp(_normal(rng, (d, n), 0.0, 0.5).astype(np.float64))).astype(np.float32)
    t["state"] = _normal(rng, (b, d, n))
    t["conv_x"] = _store(_normal(rng, (b, d, w.conv_tokens)), io)
    t["conv_state"] = _store(_normal(rng, (b, d, w.conv_state_len)), io)
    t["conv_weight"] = _normal(rng, (d, w.conv_width), 0.0, 0.5)
    t["conv_bias"] = _normal(rng, (d,))
    t["cache_seqlens"] = rng.integers(0, 4096, size=(b,), dtype=np.int32)
    return t


def make_ssd_inputs(w: SsdWorkload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every tensor of the Mamba-2 workload ``w``, in this order:
    x, dt (N(-3, 0.5): with softplus and the bias a step near 0.05), z, B, C,
    D (N(0, 1), per head or per channel), dt_bias (U(-0.1, 0.1)), A
    (-U(1, 16) per head), initial states (N(0, 1), when the workload has
    them).  Same storage rules as ``make_inputs``."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    b, l, h, p, n, g = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    io = w.io_dtype
    t: Dict[str, Optional[np.ndarray]] = {}
    t["x"] = _store(_normal(rng, (b, l, h, p)), io)
    t["dt"] = _store(_normal(rng, (b, l, h), -3.0, 0.5), io)
    t["z"] = _store(_normal(rng, (b, l, h, p)), io) if w.has_z else None
    t["B"] = _store(_normal(rng, (b, l, g, n)), io)
    t["C"] = _store(_normal(rng, (b, l, g, n)), io)
    if w.has_D:
        t["D"] = _normal(rng, (h, p) if w.D_per_channel else (h,))
    else:
        t["D"] = None
    t["dt_bias"] = _uniform(rng, (h,), -0.1, 0.1) if w.has_bias else None
    t["A"] = -_uniform(rng, (h,), 1.0, 16.0)
    t["initial_states"] = _normal(rng, (b, h, p, n)) if w.init_state else None
    return t
