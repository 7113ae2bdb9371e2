"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI, run the oracle on the same bits, compare.

Tolerance (per element, for out and last_state):
    |gpu - ref| <= tol * (1 + |ref|),  tol = 1e-4 for fp32 io, 2e-2 for bf16 io,
    5e-3 for fp16 io.
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


def check(w: Workload, gpu, ref, last_gpu=None, last_ref=None, what=""):
    tol = TOL[w.io_dtype]
    e = max_err(gpu, ref)
    assert e <= tol, f"{what} out: max normalised error {e:.3e} > {tol:.0e}"
    if last_gpu is not None:
        # the state is fp32 in every workload: hold last_state to the tighter
        # bound when the io is fp32, and to the io bound otherwise
        el = max_err(last_gpu, last_ref)
        assert el <= tol, f"{what} last_state: max normalised error {el:.3e} > {tol:.0e}"
        return e, el
    return e, None
