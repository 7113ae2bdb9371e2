"""GPU parity of the complex-A backward (ssm_scan_bwd_complex) and of the
complex forward's checkpoints, against the float64 oracle, through the C ABI.

The complex forward runs on the GPU with checkpoints, then the backward; the
oracle (oracle.selective_scan_complex_bwd, pinned on the CPU by finite
differences, the real case, conjugation and Euler's identity) computes every
gradient from the same input bits and dout.  Bar, per element and pair
component: |gpu - ref| <= tol * (1 + |ref|), tol 1e-4 for fp32 io, 2e-2 for
bf16 and 5e-3 for fp16 (du, ddelta, dz are stored in the io dtype; dA, dB,
dC, dD, ddelta_bias and dinitial_state in fp32).

The gradients that hold A a_t (ddelta, ddelta_bias, dA) are ill-conditioned
where |Im A| is large: with the default ladder Im A[d, s] = pi s (up to 47
at 16 states) an error of one rounding in delta' or in the phase reaches
them magnified by |A|^2 delta', and a plain binary32 evaluation of the same
definition (oracle.selective_scan_complex_bwd_f32_floor, libm's cexpf and
log1pf) lands near 1e-4 by itself.  For fp32 io their bar is therefore
max(1e-4, 3 x F), F the largest of that evaluation's errors in the three on
the same input: the kernel must be as accurate as straightforward fp32
arithmetic.  F is taken over the three together and given a factor of three
because one binary32 evaluation's error is a single draw of its rounding
(on the base ladder case it is 9.5e-5 for ddelta but 2.2e-5 for their sum
over time, ddelta_bias), and another order of the same sums lands up to
about twice as far.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import (BF16, COMPLEX_WORKLOADS, F16, F32, io_bits_to_f64,
                                               make_complex_inputs, make_dout)
from tests.harness import TOL, TOL_STATE, log, max_err, to_dev

pytestmark = pytest.mark.gpu

BASE = COMPLEX_WORKLOADS["complex_tiny"]


def _kinds(t):
    bk = orc.BC_FIXED if t["B"].ndim == 3 else orc.BC_VARYING
    ck = orc.BC_FIXED if t["C"].ndim == 3 else orc.BC_VARYING
    return bk, ck


def _gpu(w, t, dout, want_dinit=True, ret_ckpt=False, segments=0):
    import torch
    from state_space_model_scan_amd import binding
    io = w.io_dtype
    dev = lambda a: to_dev(a, io)          # noqa: E731
    par = lambda a: to_dev(a, param=True)  # noqa: E731
    ck = torch.full((w.batch, w.dim, binding.checkpoint_count(w.seqlen), w.dstate, 2), float("nan"),
                    dtype=torch.float32, device="cuda")
    u, delta, B, C, z = dev(t["u"]), dev(t["delta"]), dev(t["B"]), dev(t["C"]), dev(t["z"])
    A, D, bias = par(t["A"]), par(t["D"]), par(t["delta_bias"])
    init = t.get("initial_state")
    init_t = None if init is None else par(init.astype(np.float32))
    binding.ssm_scan_fwd_complex(u, delta, A, B, C, D, z, bias, w.softplus, initial_state=init_t,
                                 checkpoints=ck)
    g = binding.ssm_scan_bwd_complex(u, delta, A, B, C, dev(dout), ck, D=D, z=z, delta_bias=bias,
                                     delta_softplus=w.softplus, want_dinitial_state=want_dinit,
                                     seq_segments=segments)
    torch.cuda.synchronize()
    res = {k: (None if v is None else v.float().cpu().numpy().astype(np.float64)) for k, v in g.items()}
    if ret_ckpt:
        res["ckpt"] = ck.cpu().numpy().astype(np.float64)
    return res


def _oracle(w, t, dout):
    bk, ck = _kinds(t)
    init = t.get("initial_state")
    return orc.selective_scan_complex_bwd(
        t["u"], t["delta"], t["A"], t["B"], t["C"], io_bits_to_f64(dout, w.io_dtype), t["D"], t["z"],
        t["delta_bias"], w.softplus, io_dtype=w.io_dtype, ngroups=w.ngroups, B_kind=bk, C_kind=ck,
        initial_state=None if init is None else init.astype(np.float32).astype(np.float64))


FLOOR_FACTOR = 3.0
FLOOR_NAMES = ("ddelta", "ddelta_bias", "dA")


def _floor_bars(w, t, dout, want):
    """fp32 io: the bar of ddelta, ddelta_bias and dA, max(1e-4, 3 x the
    binary32 evaluation's largest max normalised error in the three on this
    input)."""
    if w.io_dtype != F32:
        return {}
    bk, ck = _kinds(t)
    init = t.get("initial_state")
    f = orc.selective_scan_complex_bwd_f32_floor(
        t["u"], t["delta"], t["A"], t["B"], t["C"], io_bits_to_f64(dout, w.io_dtype), t["z"],
        t["delta_bias"], w.softplus, io_dtype=w.io_dtype, ngroups=w.ngroups, B_kind=bk, C_kind=ck,
        initial_state=None if init is None else init.astype(np.float32).astype(np.float64))
    names = [k for k in FLOOR_NAMES if want.get(k) is not None]
    floor = max(max_err(f[k], want[k].reshape(f[k].shape)) for k in names)
    return {k: max(TOL[F32], FLOOR_FACTOR * floor) for k in names}


def _compare(w, got, want, what, names=None, bars=None):
    tol = TOL[w.io_dtype]
    errs = {}
    for k in names or ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dinitial_state"):
        if want.get(k) is None or got.get(k) is None:
            continue
        e = max_err(got[k], want[k].reshape(got[k].shape))
        errs[k] = e
        bar = (bars or {}).get(k, tol)
        assert e <= bar, f"{what} {k}: max normalised error {e:.3e} > {bar:.3e}"
    return errs


def _run(w, what, t=None, segments=0):
    log(f"[cbwd] {what}: b={w.batch} d={w.dim} l={w.seqlen} n={w.dstate} g={w.ngroups} io={w.io_dtype} "
        f"bc={w.bc_kind} z={w.has_z} D={w.has_D} bias={w.has_bias} sp={w.softplus} init={w.init_state} "
        f"Im A={w.A_imag}")
    t = make_complex_inputs(w) if t is None else t
    dout = make_dout(w)
    got = _gpu(w, t, dout, segments=segments)
    want = _oracle(w, t, dout)
    bars = _floor_bars(w, t, dout, want)
    errs = _compare(w, got, want, what, bars=bars)
    log(f"[cbwd]   errors {', '.join(f'{k} {v:.2e}' for k, v in errs.items())}; "
        f"bars {', '.join(f'{k} {v:.2e}' for k, v in bars.items()) or 'io tolerance'}")
    return errs


@pytest.mark.parametrize("io", [F32, BF16, F16])
def test_complex_bwd_base(io):
    _run(BASE.scaled(io_dtype=io, init_state=True, seed=800 + io), f"base io={io}")


@pytest.mark.parametrize("io", [F32, BF16, F16])
def test_complex_bwd_spread_imaginary_parts(io):
    # Im A ~ N(0, 3): well conditioned, so fp32 meets 1e-4 on every gradient
    w = BASE.scaled(io_dtype=io, init_state=True, A_imag="normal", seed=805 + io)
    t = make_complex_inputs(w)
    dout = make_dout(w)
    _compare(w, _gpu(w, t, dout), _oracle(w, t, dout), f"normal Im A io={io}")



@pytest.mark.parametrize("n", [1, 5, 16])
@pytest.mark.parametrize("seqlen", [1, 31, 32, 33, 100])
def test_complex_bwd_sizes(n, seqlen):
    w = BASE.scaled(dstate=n, seqlen=seqlen, io_dtype=F32, A_imag="normal", seed=810 + n * 7 + seqlen)
    _run(w, f"n={n} l={seqlen}")


@pytest.mark.parametrize("bc", ["varying", "fixed", "Bfixed", "Cfixed"])
def test_complex_bwd_bc_layouts(bc):
    w = BASE.scaled(io_dtype=F32, bc_kind="fixed" if bc == "fixed" else "varying", init_state=True,
                    seed=830 + len(bc))
    t = make_complex_inputs(w)
    if bc in ("Bfixed", "Cfixed"):
        fixed = make_complex_inputs(w.scaled(bc_kind="fixed"))
        t[bc[0]] = fixed[bc[0]]
    _run(w, f"bc={bc}", t=t)


@pytest.mark.parametrize("flags", [dict(has_z=False), dict(has_D=False), dict(has_bias=False),
                                   dict(softplus=False, delta_mean=0.1, delta_std=0.02),
                                   dict(has_z=False, has_D=False, has_bias=False)])
def test_complex_bwd_optional_inputs(flags):
    w = BASE.scaled(io_dtype=F32, seed=850 + len(flags), **flags)
    _run(w, f"flags={flags}")


@pytest.mark.parametrize("groups,dim", [(1, 64), (2, 96), (4, 256), (3, 24)])
def test_complex_bwd_groups_and_channel_blocks(groups, dim):
    # 32-channel workgroups: 96 / 2 = 48 channels per group leaves a partial block
    w = BASE.scaled(dim=dim, ngroups=groups, seqlen=70, io_dtype=BF16, A_imag="normal",
                    seed=870 + groups + dim)
    _run(w, f"groups={groups} dim={dim}")


def test_complex_bwd_checkpoints_are_the_forward_states():
    """Entry k of the forward's checkpoints is the state before timestep 32k:
    entry 0 is the initial state, the others are the last states of the
    forward run on the first 32k timesteps (oracle)."""
    w = BASE.scaled(batch=2, dim=24, seqlen=100, dstate=6, io_dtype=F32, init_state=True, seed=880)
    t = make_complex_inputs(w)
    got = _gpu(w, t, make_dout(w), ret_ckpt=True)["ckpt"]
    np.testing.assert_array_equal(got[:, :, 0], t["initial_state"].astype(np.float32).astype(np.float64))
    bk, ck = _kinds(t)
    for k in (1, 2, 3):
        L = 32 * k
        cut = dict(t)
        for key in ("u", "delta", "z"):
            cut[key] = np.ascontiguousarray(t[key][:, :, :L])
        for key in ("B", "C"):
            if t[key].ndim == 5:
                cut[key] = np.ascontiguousarray(t[key][:, :, :, :L])
        _, last = orc.selective_scan_complex(
            cut["u"], cut["delta"], t["A"], cut["B"], cut["C"], t["D"], cut["z"], t["delta_bias"],
            w.softplus, io_dtype=w.io_dtype, ngroups=w.ngroups, B_kind=bk, C_kind=ck,
            initial_state=t["initial_state"].astype(np.float64))
        e = max_err(got[:, :, k].reshape(-1, w.dstate, 2), last)
        assert e <= TOL_STATE, f"checkpoint {k}: {e:.3e}"


def test_complex_bwd_deterministic():
    w = BASE.scaled(batch=2, dim=64, seqlen=96, io_dtype=BF16, seed=890)
    t = make_complex_inputs(w)
    dout = make_dout(w)
    a, b = _gpu(w, t, dout), _gpu(w, t, dout)
    for k, v in a.items():
        if v is not None:
            np.testing.assert_array_equal(v, b[k])


@pytest.mark.parametrize("segments", [2, 3, 7])
@pytest.mark.parametrize("bc", ["varying", "fixed"])
@pytest.mark.parametrize("io", [F32, BF16])
def test_complex_bwd_sequence_split(segments, bc, io):
    """The sequence split forced to 2, 3 and 7 segments (10 chunks of 32 and
    a ragged last chunk: segments of 5, 4 and 2 chunks), every gradient
    against the oracle.  The carry that crosses a boundary still weighs
    about exp(-0.3 * 20) of a gradient after a five-chunk segment, well above
    the bar, so a wrong fold fails.  (Real parts of A near zero on the Im A
    ladder put even the unsplit walk past the fp32 bar: du 3.0e-4 at
    Re A = -0.02, the same with and without the split.)"""
    w = BASE.scaled(batch=2, dim=64, seqlen=300, bc_kind=bc, io_dtype=io, init_state=True,
                    seed=900 + segments + 10 * io + (bc == "fixed"))
    _run(w, f"split segments={segments} bc={bc} io={io}", segments=segments)


def test_complex_bwd_split_one_chunk_per_segment():
    """Every chunk its own segment (9 segments over 270 timesteps), grouped
    time-varying B/C, bf16."""
    w = BASE.scaled(batch=2, dim=128, seqlen=270, ngroups=2, io_dtype=BF16, init_state=True, seed=930)
    _run(w, "one chunk per segment", segments=9)


def test_complex_bwd_split_agrees_with_unsplit():
    """Split (4 segments) and unsplit runs agree to fp32 rounding on every
    gradient: the same sums, reassociated."""
    w = BASE.scaled(batch=2, dim=64, seqlen=512, io_dtype=F32, seed=935)
    t = make_complex_inputs(w)
    dout = make_dout(w)
    a, b = _gpu(w, t, dout, segments=1), _gpu(w, t, dout, segments=4)
    for k, v in a.items():
        if v is not None:
            e = max_err(b[k], v)
            assert e <= 1e-4, f"{k}: split against unsplit {e:.3e}"


def test_complex_bwd_mid_size():
    """A mid-size grouped layer (64-channel groups, several chunks of 32 and
    a ragged last chunk), every gradient on every element."""
    w = BASE.scaled(batch=2, dim=256, seqlen=1000, dstate=16, ngroups=4, io_dtype=BF16, A_imag="normal",
                    init_state=True, seed=895)
    _run(w, "mid size")


def test_complex_bwd_full_size_slices():
    """mamba2p8b_complex (b=8 d=5120 l=2048 n=16 g=4, bf16, complex A/B/C)
    through the GPU in the launch configuration bench.py times; the oracle on
    batch 5 / group 1 (all 1280 channels of the group: complete dB and dC
    sums) and on every batch of channels 0, 3001 and 5119 (dA, dD,
    ddelta_bias)."""
    import torch
    from state_space_model_scan_amd import binding
    w = COMPLEX_WORKLOADS["mamba2p8b_complex"]
    log(f"[cbwd] full size {w.name}")
    t = make_complex_inputs(w)
    dout = make_dout(w)
    g = _gpu(w, t, dout, want_dinit=False)

    bb, gg = 5, 1
    cpg = w.dim // w.ngroups
    ch = slice(gg * cpg, (gg + 1) * cpg)
    sub = w.scaled(batch=1, dim=cpg, ngroups=1)
    ts = dict(t)
    for k in ("u", "delta", "z"):
        ts[k] = np.ascontiguousarray(t[k][bb:bb + 1, ch])
    for k in ("B", "C"):
        ts[k] = np.ascontiguousarray(t[k][bb:bb + 1, gg:gg + 1])
    for k in ("A", "D", "delta_bias"):
        ts[k] = np.ascontiguousarray(t[k][ch])
    want = _oracle(sub, ts, np.ascontiguousarray(dout[bb:bb + 1, ch]))
    got = {k: g[k][bb:bb + 1, ch] for k in ("du", "ddelta", "dz")}
    got["dB"] = g["dB"][bb:bb + 1, gg:gg + 1]
    got["dC"] = g["dC"][bb:bb + 1, gg:gg + 1]
    errs = _compare(w, got, want, f"full size (b={bb}, g={gg})", names=("du", "ddelta", "dz", "dB", "dC"))
    log(f"[cbwd]   slice errors {', '.join(f'{k} {v:.2e}' for k, v in errs.items())}")

    for d in (0, 3001, 5119):
        gi = d // cpg
        one = w.scaled(dim=1, ngroups=1)
        t1 = dict(t)
        for k in ("u", "delta", "z"):
            t1[k] = np.ascontiguousarray(t[k][:, d:d + 1])
        for k in ("B", "C"):
            t1[k] = np.ascontiguousarray(t[k][:, gi:gi + 1])
        for k in ("A", "D", "delta_bias"):
            t1[k] = np.ascontiguousarray(t[k][d:d + 1])
        want1 = _oracle(one, t1, np.ascontiguousarray(dout[:, d:d + 1]))
        got1 = {k: g[k][d:d + 1] for k in ("dA", "dD", "ddelta_bias")}
        errs = _compare(w, got1, want1, f"full size channel {d}", names=("dA", "dD", "ddelta_bias"))
        log(f"[cbwd]   channel {d} errors {', '.join(f'{k} {v:.2e}' for k, v in errs.items())}")
