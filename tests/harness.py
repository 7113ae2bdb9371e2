"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI, run the oracle on the same bits, compare.

Tolerance (per element): |gpu - ref| <= tol * (1 + |ref|), with
  out:        tol = 1e-4 for fp32 io, 2e-2 for bf16 io, 5e-3 for fp16 io;
  last_state: tol = 1e-4 in every io dtype -- the state is fp32 throughout
              and is never rounded to the io dtype.
"""
from __future__ import annotations

import sys
from typing import Dict, Optional

import numpy as np

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import BF16, F16, F32, Workload

# fp16: ten half-units in the last place of binary16 (2^-11), as 2e-2 is
# about ten for bf16 (2^-9)
TOL = {F32: 1e-4, BF16: 2e-2, F16: 5e-3}
# the fp32 state, in every io dtype
TOL_STATE = 1e-4


def log(msg: str) -> None:
    """Name the case on stdout before a GPU step, flushed."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a: Optional[np.ndarray], io_dtype: int = F32, param: bool = False):
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if not param and a.dtype == np.uint16 and io_dtype in (BF16, F16):
        t = t.view(torch.bfloat16 if io_dtype == BF16 else torch.float16)
    return t.cuda()


def run_gpu(w: Workload, t: Dict[str, np.ndarray], *, last: bool = True,
            init: Optional[np.ndarray] = None, poison: bool = True, seq_segments: int = 0):
    """Run ssm_scan_fwd on the workload's inputs.  Returns (out (b*d, l) float64,
    last_state (b*d, n) float64 or None)."""
    import torch
    from state_space_model_scan_amd import binding
    io = w.io_dtype
    delta = to_dev(t["delta"], io)
    out = torch.empty_like(delta)
    if poison:
        out.fill_(float("nan"))
    last_t = None
    if last:
        last_t = torch.full((w.batch, w.dim, w.dstate), float("nan"), dtype=torch.float32, device="cuda")
    B, C = to_dev(t["B"], io), to_dev(t["C"], io)
    kw = {}
    if w.conv:
        kw = dict(conv_x=to_dev(t["conv_x"], io), conv_weight=to_dev(t["conv_weight"], param=True),
                  conv_bias=to_dev(t["conv_bias"], param=True))
    binding.ssm_scan_fwd(to_dev(t["u"], io), delta, to_dev(t["A"], param=True), B, C,
                         to_dev(t["D"], param=True), to_dev(t["z"], io),
                         to_dev(t["delta_bias"], param=True), w.softplus, out=out,
                         last_state=last_t,
                         initial_state=None if init is None else to_dev(init.astype(np.float32), param=True),
                         seq_segments=seq_segments, **kw)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64).reshape(w.batch * w.dim, w.seqlen)
    ls = None if last_t is None else last_t.cpu().numpy().astype(np.float64).reshape(w.batch * w.dim, w.dstate)
    return o, ls


def run_oracle(w: Workload, t: Dict[str, np.ndarray], rows=None, init=None, nthreads=0):
    bk = orc.BC_FIXED if t["B"].ndim == 2 else orc.BC_VARYING
    ck = orc.BC_FIXED if t["C"].ndim == 2 else orc.BC_VARYING
    return orc.selective_scan(
        t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], w.softplus,
        io_dtype=w.io_dtype, ngroups=w.ngroups, B_kind=bk, C_kind=ck,
        initial_state=None if init is None else init.astype(np.float32).astype(np.float64),
        conv_x=t.get("conv_x"), conv_weight=t.get("conv_weight"), conv_bias=t.get("conv_bias"),
        conv_act=orc.ACT_SILU, rows=rows, nthreads=nthreads,
        shape=(w.batch, w.dim, w.seqlen))


def max_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    if gpu.size == 0:
        return 0.0
    if not np.all(np.isfinite(gpu)):
        return float("inf")
    return float(np.max(np.abs(gpu - ref) / (1.0 + np.abs(ref))))


def _io_values(a: np.ndarray, io_dtype: int) -> np.ndarray:
    """Stored io bits as float64 values."""
    if a.dtype == np.uint16:
        if io_dtype == BF16:
            return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return a.view(np.float16).astype(np.float64)
    return a.astype(np.float64)


def conv_flip_slack(w: Workload, t: Dict[str, np.ndarray]) -> Optional[np.ndarray]:
    """Allowance on last_state for the fused conv prologue with a 16-bit io
    dtype, (batch*dim, dstate) float64, or None when there is nothing to allow.

    The prologue rounds u = silu(conv(x)) to the io dtype: a rounding
    decision taken by floating point.  The kernel takes it from an fp32
    evaluation, the oracle from float64; where the float64 value lies within
    the fp32 evaluation's error bound of a rounding midpoint, either rounding
    is a correct one, and they differ by one io ulp.  The bound used for the
    fp32 evaluation is generous: 12 eps32 times the sum of the conv terms'
    magnitudes (an FMA chain), scaled by silu's slope (at most 1.1), plus
    12 eps32 of the output (exp2, reciprocal and product).  last_state is
    linear in u, x_T = sum_t prod_{tau > t} dA_tau * delta'_t B_t u_t + ...,
    so a flip at timestep t moves x_T[s] by at most
        |delta'_t B_t[s]| * ulp(u_t) * exp(A[d,s] * sum_{tau > t} delta'_tau);
    the allowance is that sum over the ambiguous timesteps of each row.
    Everything here comes from the inputs and the oracle, none from the GPU."""
    if not w.conv or w.io_dtype == F32:
        return None
    mant = 8 if w.io_dtype == BF16 else 11                 # significant bits of the io dtype
    eps32 = 2.0 ** -24
    rows_all, l, n = w.batch * w.dim, w.seqlen, w.dstate
    slack = np.zeros((rows_all, n))
    xbits = t["conv_x"].reshape(rows_all, l)
    dbits = t["delta"].reshape(rows_all, l)
    for r0 in range(0, rows_all, 2048):                      # blocks of rows bound the memory
        rr = np.arange(r0, min(rows_all, r0 + 2048), dtype=np.int64)
        d_of = rr % w.dim
        v = orc.causal_conv1d(t["conv_x"], t["conv_weight"], t["conv_bias"], orc.ACT_SILU,
                              io_dtype=w.io_dtype, rows=rr, nthreads=16)   # unrounded
        x = _io_values(xbits[rr], w.io_dtype)
        wt = np.abs(t["conv_weight"].astype(np.float64))[d_of]            # (k, 4)
        mag = np.repeat(np.abs(t["conv_bias"].astype(np.float64))[d_of][:, None], l, axis=1)
        for k in range(4):
            sh = 3 - k
            mag[:, sh:] += wt[:, k:k + 1] * np.abs(x[:, :l - sh])
        err = 1.1 * 12 * eps32 * mag + 12 * eps32 * np.abs(v)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(v), 1e-300))) - (mant - 1))
        u = np.round(v / ulp) * ulp                          # round to nearest, ties to even
        amb = (ulp / 2 - np.abs(v - u)) <= err
        ri, ti = np.nonzero(amb)
        if ri.size == 0:
            continue
        dvar = _io_values(dbits[rr], w.io_dtype) + t["delta_bias"].astype(np.float64)[d_of][:, None]
        dt = np.logaddexp(0.0, dvar) if w.softplus else dvar
        suffix = dt.sum(1, keepdims=True) - np.cumsum(dt, axis=1)     # sum over tau > t
        rows = rr[ri]
        d_idx, b_idx = rows % w.dim, rows // w.dim
        if t["B"].ndim == 2:
            Bv = _io_values(t["B"], w.io_dtype)[d_idx]                       # (k, n)
        else:
            g = d_idx // (w.dim // t["B"].shape[1])
            Bv = _io_values(t["B"], w.io_dtype)[b_idx, g, :, ti]            # (k, n)
        A = t["A"].astype(np.float64)[d_idx]                                  # (k, n)
        contrib = (np.abs(dt[ri, ti] * ulp[ri, ti])[:, None] * np.abs(Bv)
                   * np.exp(A * suffix[ri, ti][:, None]))
        np.add.at(slack, rows, contrib)
    return slack


def check(w: Workload, gpu, ref, last_gpu=None, last_ref=None, what="", last_slack=None):
    """Per-element bars; last_slack (same shape as last_state) adds an
    allowance where a rounding decision is not determined (conv_flip_slack)."""
    tol = TOL[w.io_dtype]
    e = max_err(gpu, ref)
    assert e <= tol, f"{what} out: max normalised error {e:.3e} > {tol:.0e}"
    if last_gpu is not None:
        if last_slack is None:
            el = max_err(last_gpu, last_ref)
        else:
            assert np.all(np.isfinite(last_gpu)), f"{what} last_state not finite"
            el = float(np.max(np.maximum(np.abs(last_gpu - last_ref) - last_slack, 0.0) / (1.0 + np.abs(last_ref))))
        assert el <= TOL_STATE, f"{what} last_state: max normalised error {el:.3e} > {TOL_STATE:.0e}"
        return e, el
    return e, None
