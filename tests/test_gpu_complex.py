"""GPU parity of ssm_scan_fwd_complex (the selective scan with complex A, the
page's section 4.1: A may be real or complex) against the float64 oracle's
complex scan, element by element, on the same seeded inputs.

Tolerance per element (both pair components): |gpu - ref| <= tol * (1 + |ref|),
for out tol = 1e-4 fp32 io, 2e-2 bf16, 5e-3 fp16; for last_state (fp32 in
every io dtype) 1e-4.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import (BF16, COMPLEX_WORKLOADS, F16, F32, make_complex_inputs,
                                               sample_rows)
from tests.harness import TOL, TOL_STATE, log, max_err, to_dev

pytestmark = pytest.mark.gpu

BASE = COMPLEX_WORKLOADS["complex_tiny"]


def _gpu(w, t, *, last=True):
    import torch
    from state_space_model_scan_amd import binding
    io = w.io_dtype
    delta = to_dev(t["delta"], io)
    out = torch.full_like(delta, float("nan"))
    last_t = None
    if last:
        last_t = torch.full((w.batch, w.dim, w.dstate, 2), float("nan"), dtype=torch.float32, device="cuda")
    init = t.get("initial_state")
    binding.ssm_scan_fwd_complex(
        to_dev(t["u"], io), delta, to_dev(t["A"], param=True), to_dev(t["B"], io), to_dev(t["C"], io),
        to_dev(t["D"], param=True), to_dev(t["z"], io), to_dev(t["delta_bias"], param=True), w.softplus,
        out=out, last_state=last_t, initial_state=None if init is None else to_dev(init, param=True))
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64).reshape(w.batch * w.dim, w.seqlen)
    ls = None if last_t is None else last_t.cpu().numpy().astype(np.float64).reshape(w.batch * w.dim, w.dstate, 2)
    return o, ls


def _oracle(w, t, rows=None):
    kind = orc.BC_FIXED if w.bc_kind == "fixed" else orc.BC_VARYING
    init = t.get("initial_state")
    return orc.selective_scan_complex(
        t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], w.softplus,
        io_dtype=w.io_dtype, ngroups=w.ngroups, B_kind=kind, C_kind=kind,
        initial_state=None if init is None else init.astype(np.float64), rows=rows)


def _check(w, gpu, ref, what):
    tol = TOL[w.io_dtype]
    e = max_err(gpu[0], ref[0])
    assert e <= tol, f"{what} out: max normalised error {e:.3e} > {tol:.0e}"
    if gpu[1] is not None:
        el = max_err(gpu[1], ref[1])
        assert el <= TOL_STATE, f"{what} last_state: max normalised error {el:.3e} > {TOL_STATE:.0e}"
        return e, el
    return e, None


CASES = [
    # (batch, dim, seqlen, dstate, ngroups, io, bc_kind, A_imag, extra)
    (2, 24, 100, 16, 2, F32, "varying", "lin", {}),
    (2, 24, 100, 16, 2, F32, "varying", "normal", {}),
    (1, 40, 257, 5, 1, F32, "fixed", "normal", {}),
    (3, 16, 64, 8, 1, BF16, "varying", "lin", {}),
    (2, 48, 300, 4, 3, BF16, "varying", "normal", dict(has_z=False, init_state=True)),
    (2, 32, 31, 3, 2, F16, "varying", "normal", dict(has_D=False)),
    (1, 20, 1, 16, 1, F32, "varying", "lin", dict(init_state=True)),
    (2, 16, 256, 1, 1, BF16, "fixed", "lin", dict(has_bias=False, softplus=False, delta_mean=0.1,
                                                  delta_std=0.02)),
    (1, 64, 512, 16, 4, F32, "varying", "normal", dict(init_state=True, delta_mean=-4.0)),
    (2, 256, 1024, 16, 2, F16, "varying", "lin", {}),
    (4, 96, 777, 12, 1, BF16, "fixed", "normal", dict(init_state=True)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}d{c[1]}l{c[2]}n{c[3]}g{c[4]}io{c[5]}{c[6]}{c[7]}")
def test_complex_parity(case):
    b, d, l, n, g, io, kind, imag, extra = case
    extra = dict(extra)
    w = BASE.scaled(batch=b, dim=d, seqlen=l, dstate=n, ngroups=g, io_dtype=io, bc_kind=kind, A_imag=imag,
                    init_state=extra.pop("init_state", False), seed=300 + b * 7 + d + l + n, **extra)
    t = make_complex_inputs(w)
    log(f"complex parity {w}")
    e, el = _check(w, _gpu(w, t), _oracle(w, t), str(case[:8]))
    log(f"  max normalised error out {e:.2e} last_state {el:.2e}")


def test_complex_mixed_bc_kinds():
    """B fixed with C varying and the other way round (each tensor has its own
    layout kind)."""
    import torch
    from state_space_model_scan_amd import binding
    w = BASE.scaled(batch=2, dim=24, seqlen=77, dstate=6, ngroups=2, io_dtype=F32, seed=351)
    tv = make_complex_inputs(w)
    tf = make_complex_inputs(w.scaled(bc_kind="fixed"), seed=352)
    for B, C, bk, ck in ((tf["B"], tv["C"], orc.BC_FIXED, orc.BC_VARYING),
                         (tv["B"], tf["C"], orc.BC_VARYING, orc.BC_FIXED)):
        log(f"complex mixed kinds B {bk} C {ck}")
        delta = to_dev(tv["delta"])
        out = torch.full_like(delta, float("nan"))
        last = torch.full((w.batch, w.dim, w.dstate, 2), float("nan"), device="cuda")
        binding.ssm_scan_fwd_complex(to_dev(tv["u"]), delta, to_dev(tv["A"]), to_dev(B), to_dev(C),
                                     to_dev(tv["D"]), to_dev(tv["z"]), to_dev(tv["delta_bias"]), True,
                                     out=out, last_state=last,
                                     initial_state=to_dev(tv["initial_state"]))
        torch.cuda.synchronize()
        ref = orc.selective_scan_complex(tv["u"], tv["delta"], tv["A"], B, C, tv["D"], tv["z"],
                                         tv["delta_bias"], True, io_dtype=F32, ngroups=w.ngroups,
                                         B_kind=bk, C_kind=ck,
                                         initial_state=tv["initial_state"].astype(np.float64))
        got = (out.cpu().numpy().astype(np.float64).reshape(-1, w.seqlen),
               last.cpu().numpy().astype(np.float64).reshape(-1, w.dstate, 2))
        _check(w, got, ref, f"mixed B {bk} C {ck}")


def test_complex_page_signature():
    """selective_scan_fn with a complex64 A, B and C routes to the complex
    scan and returns a complex64 last_state."""
    import torch
    from state_space_model_scan_amd import binding
    w = BASE.scaled(batch=2, dim=24, seqlen=96, dstate=4, ngroups=1, init_state=False, seed=353)
    t = make_complex_inputs(w)
    cplx = lambda a: torch.view_as_complex(torch.from_numpy(np.ascontiguousarray(a))).cuda()  # noqa: E731
    B3 = t["B"][:, 0]          # the 3-D (batch, dstate, seqlen) form, one group
    out, last = binding.selective_scan_fn(
        to_dev(t["u"]), to_dev(t["delta"]), cplx(t["A"]), cplx(B3), cplx(t["C"][:, 0]),
        D=to_dev(t["D"]), z=to_dev(t["z"]), delta_bias=to_dev(t["delta_bias"]), delta_softplus=True,
        return_last_state=True)
    torch.cuda.synchronize()
    assert last.dtype == torch.complex64 and tuple(last.shape) == (2, 24, 4)
    ref = _oracle(w, t)
    got = (out.cpu().numpy().astype(np.float64).reshape(-1, w.seqlen),
           torch.view_as_real(last).cpu().numpy().astype(np.float64).reshape(-1, w.dstate, 2))
    _check(w, got, ref, "selective_scan_fn complex")


def test_complex_real_case_equals_real_kernel():
    """Zero imaginary parts: the complex kernel's output equals the real
    scan's (both HIP paths; each is also checked against its oracle)."""
    import torch
    from state_space_model_scan_amd import binding
    w = BASE.scaled(batch=2, dim=40, seqlen=130, dstate=16, ngroups=2, io_dtype=BF16, seed=354)
    t = make_complex_inputs(w)
    A = t["A"].copy()
    A[..., 1] = 0.0
    B, C = t["B"].copy(), t["C"].copy()
    B[..., 1] = 0
    C[..., 1] = 0
    t2 = dict(t, A=A, B=B, C=C)
    oc, _ = _gpu(w, t2)
    real_out = binding.ssm_scan_fwd(to_dev(t["u"], BF16), to_dev(t["delta"], BF16),
                                    to_dev(np.ascontiguousarray(A[..., 0])),
                                    to_dev(np.ascontiguousarray(B[..., 0]), BF16),
                                    to_dev(np.ascontiguousarray(C[..., 0]), BF16),
                                    to_dev(t["D"]), to_dev(t["z"], BF16), to_dev(t["delta_bias"]), True,
                                    initial_state=to_dev(np.ascontiguousarray(t["initial_state"][..., 0])))
    torch.cuda.synchronize()
    orl = real_out.float().cpu().numpy().astype(np.float64).reshape(-1, w.seqlen)
    e = max_err(oc, orl)
    assert e <= TOL[BF16], e
    _check(w, (oc, None), _oracle(w, t2), "real case")


def test_complex_full_size_sampled_rows():
    """The Mamba-2.8B-shaped layer with complex A, B, C (b=8 d=5120 l=2048
    n=16 g=4, bf16) in the launch bench.py times; the oracle on sampled rows
    (group and block boundaries included)."""
    w = COMPLEX_WORKLOADS["mamba2p8b_complex"]
    t = make_complex_inputs(w)
    rows = sample_rows(w, 48)
    log(f"complex full size {w.name}: {len(rows)} sampled rows")
    o, ls = _gpu(w, t)
    ref = _oracle(w, t, rows=rows)
    e, el = _check(w, (o[rows], ls[rows]), ref, w.name)
    log(f"  max normalised error out {e:.2e} last_state {el:.2e}")


@pytest.mark.parametrize("seqlen,io,kind", [(96, None, "varying"), (100, None, "varying"), (64, F32, "varying"),
                                            (70, F16, "varying"), (66, F32, "fixed")])
def test_complex_mixed_plan_all_rows(seqlen, io, kind):
    """The Mamba-2.8B-shaped width (b=8 d=5120 g=4: 2560 blocks of 16
    channels, 2048 whole waves and 1024 eight-lane waves of 8 channels) on a
    short sequence, whole chunks (96, vector loads) and a ragged one (100,
    element loads), with the layer's bf16 io and with fp16 io (the mixed
    kernel's instances), and with fp32 io, which takes the plain plan, B/C
    varying and fixed (one group: the same 2560 blocks): every row of out
    and last_state against the oracle."""
    w = COMPLEX_WORKLOADS["mamba2p8b_complex"].scaled(seqlen=seqlen, init_state=True, seed=1200 + seqlen)
    if io is not None:
        w = w.scaled(io_dtype=io)
    if kind != w.bc_kind:
        w = w.scaled(bc_kind=kind)
    t = make_complex_inputs(w)
    log(f"complex mixed plan: b={w.batch} d={w.dim} l={w.seqlen} io={w.io_dtype} B/C {w.bc_kind}")
    o, ls = _gpu(w, t)
    e, el = _check(w, (o, ls), _oracle(w, t), f"mixed plan l={seqlen}")
    log(f"  max normalised error out {e:.2e} last_state {el:.2e}")


def test_complex_misaligned_pointers():
    """Every io tensor one element off 16-byte alignment at a sequence length
    divisible by 8: the element-wise loads and stores."""
    import torch
    from state_space_model_scan_amd import binding
    from tests.test_gpu_parity import _offset_view
    w = BASE.scaled(batch=2, dim=24, seqlen=128, dstate=8, io_dtype=BF16, seed=355)
    t = make_complex_inputs(w)
    log("complex misaligned")
    ov = lambda k: _offset_view(t[k], w.io_dtype)  # noqa: E731
    out = _offset_view(np.zeros(t["delta"].shape, dtype=t["delta"].dtype), w.io_dtype)
    last = torch.empty((w.batch, w.dim, w.dstate, 2), dtype=torch.float32, device="cuda")
    binding.ssm_scan_fwd_complex(ov("u"), ov("delta"), to_dev(t["A"], param=True), ov("B"), ov("C"),
                                 to_dev(t["D"], param=True), ov("z"), to_dev(t["delta_bias"], param=True), True,
                                 out=out, last_state=last,
                                 initial_state=to_dev(t["initial_state"], param=True))
    torch.cuda.synchronize()
    got = (out.float().cpu().numpy().astype(np.float64).reshape(-1, w.seqlen),
           last.cpu().numpy().astype(np.float64).reshape(-1, w.dstate, 2))
    _check(w, got, _oracle(w, t), "complex misaligned")
