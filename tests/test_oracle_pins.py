"""Pins for the float64 oracle: closed forms, invariants, brute force and library
routines, each independent of the oracle's own code.

The pages (PaddleNLP Kernel operator-library guide, section 4.1 selective_scan)
print no worked numbers for the scan, so every pin here is mathematics: a
plausible mistake in the oracle (a dropped term, a wrong sign or index, a
transposed operand) changes at least one of these results.
"""
import math

import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits

RTOL = 1e-12


def _close(a, b, tol=RTOL):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"max normalised error {err:.3e} > {tol:.1e}"


def _rand(rng, shape, mean=0.0, std=1.0):
    return (rng.standard_normal(shape) * std + mean).astype(np.float32)


def _softplus_np(v):
    # numpy's logaddexp(0, v) = log(1 + e^v): a library routine, not the oracle's code
    return np.logaddexp(0.0, np.asarray(v, np.float64))


def _silu_np(v):
    v = np.asarray(v, np.float64)
    return v * 0.5 * (1.0 + np.tanh(0.5 * v))   # sigmoid via tanh


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------

def test_softplus_closed_forms():
    assert orc.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    # softplus(log(e - 1)) = 1 and softplus(log 3) = log 4
    assert orc.softplus(math.log(math.e - 1.0)) == pytest.approx(1.0, rel=1e-15)
    assert orc.softplus(math.log(3.0)) == pytest.approx(math.log(4.0), rel=1e-15)
    # softplus(x) - softplus(-x) = x
    for x in (-30.0, -3.7, -0.5, 0.25, 2.0, 19.0, 45.0):
        assert orc.softplus(x) - orc.softplus(-x) == pytest.approx(x, rel=1e-14, abs=1e-300)
    # tails: softplus(x) -> x for large x, -> e^x for very negative x
    assert orc.softplus(60.0) == 60.0
    assert orc.softplus(-60.0) == pytest.approx(math.exp(-60.0), rel=1e-15)


def test_silu_closed_forms():
    assert orc.silu(0.0) == 0.0
    assert orc.silu(math.log(3.0)) == pytest.approx(math.log(3.0) * 0.75, rel=1e-15)
    for x in (-8.0, -1.0, 0.3, 5.0):
        assert orc.silu(x) - orc.silu(-x) == pytest.approx(x, rel=1e-14)


def test_bf16_rounding_pins():
    r = orc.round_bf16
    # exact bf16 values are unchanged
    for v in (1.0, -2.5, 0.0078125, 3.0 * 2.0 ** 100, -(2.0 ** -126), 2.0 ** -133):
        assert r(v) == v
    assert math.copysign(1.0, r(-0.0)) == -1.0 and r(0.0) == 0.0
    # ties go to the even neighbour
    assert r(1.0 + 2.0 ** -8) == 1.0
    assert r(1.0 + 3.0 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert r(-(1.0 + 2.0 ** -8)) == -1.0
    # just off the tie goes to the nearer neighbour
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    # subnormal spacing 2^-133; half of it ties to 0 (even)
    assert r(2.0 ** -134) == 0.0
    assert r(3.0 * 2.0 ** -134) == 2.0 ** -132
    # overflow past the largest finite value (plus half an ulp) goes to inf
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert r(big) == big
    assert math.isinf(r(big + 2.0 ** 119))
    # agreement with an independent bit-level rounding of float32 values
    rng = np.random.default_rng(7)
    f = np.concatenate([_rand(rng, 2000), _rand(rng, 500) * np.float32(1e-30),
                        _rand(rng, 500) * np.float32(1e30)])
    want = bf16_bits_to_f32(f32_to_bf16_bits(f)).astype(np.float64)
    got = np.array([r(float(v)) for v in f])
    np.testing.assert_array_equal(got, want)


# --------------------------------------------------------------------------
# scan: closed forms
# --------------------------------------------------------------------------

def _run(inp, **kw):
    return orc.selective_scan(inp["u"], inp["delta"], inp["A"], inp["B"], inp["C"],
                              inp.get("D"), inp.get("z"), inp.get("delta_bias"),
                              kw.pop("softplus", True), **kw)


def _tiny_inputs(rng, b=2, d=3, l=17, n=4, g=1, fixed=False):
    inp = {
        "u": _rand(rng, (b, d, l)),
        "delta": _rand(rng, (b, d, l), -1.0, 0.7),
        "z": _rand(rng, (b, d, l)),
        "A": -np.exp(_rand(rng, (d, n), 0.0, 0.5)),
        "D": _rand(rng, (d,)),
        "delta_bias": (rng.uniform(-0.1, 0.1, d)).astype(np.float32),
    }
    shp = (d, n) if fixed else (b, g, n, l)
    inp["B"], inp["C"] = _rand(rng, shp), _rand(rng, shp)
    return inp


def _bc(arr, kind_fixed, b, d, s, t, dim, g):
    if kind_fixed:
        return float(arr[d, s])
    return float(arr[b, d // (dim // g), s, t])


def _dt_np(inp, softplus=True):
    dt = inp["delta"].astype(np.float64)
    if inp.get("delta_bias") is not None:
        dt = dt + inp["delta_bias"].astype(np.float64)[None, :, None]
    return _softplus_np(dt) if softplus else dt


def test_A_zero_is_prefix_sum():
    """A = 0: dA = 1, so x_t[s] = sum_{tau<=t} delta'_tau B_tau[s] u_tau."""
    rng = np.random.default_rng(1)
    b, d, l, n = 2, 3, 41, 5
    inp = _tiny_inputs(rng, b, d, l, n)
    inp["A"] = np.zeros((d, n), np.float32)
    out, last = _run(inp)
    dt = _dt_np(inp)
    u = inp["u"].astype(np.float64)
    B = inp["B"].astype(np.float64)[:, 0]   # (b, n, l)
    C = inp["C"].astype(np.float64)[:, 0]
    for bi in range(b):
        for di in range(d):
            incr = dt[bi, di][None, :] * B[bi] * u[bi, di][None, :]   # (n, l)
            x = np.cumsum(incr, axis=1)
            # fsum for the final state as an independent summation
            x_last = np.array([math.fsum(incr[s]) for s in range(n)])
            y = (C[bi] * x).sum(axis=0) + inp["D"][di] * u[bi, di]
            y = y * _silu_np(inp["z"][bi, di])
            _close(out[bi * d + di], y)
            _close(last[bi * d + di], x_last)


def test_constant_decay_is_geometric_series():
    """Constant delta' = c, A[s] = a_s, B, u: x_t = c B u (1 - r^{t+1}) / (1 - r), r = e^{c a}."""
    b, d, l, n = 1, 2, 50, 3
    c = 0.3
    a = np.array([[-0.5, -1.5, -0.05], [-2.0, -0.1, -1.0]], np.float32)
    Bv = np.array([0.7, -1.25, 2.0], np.float32)
    Cv = np.array([1.5, 0.5, -0.75], np.float32)
    uval = np.array([0.8, -1.1], np.float32)
    inp = {
        "u": np.broadcast_to(uval[None, :, None], (b, d, l)).astype(np.float32),
        "delta": np.full((b, d, l), c, np.float32),
        "A": a,
        "B": np.broadcast_to(Bv[None, None, :, None], (b, 1, n, l)).astype(np.float32),
        "C": np.broadcast_to(Cv[None, None, :, None], (b, 1, n, l)).astype(np.float32),
    }
    out, last = _run(inp, softplus=False)
    cc = float(np.float32(c))
    t = np.arange(l, dtype=np.float64)
    for di in range(d):
        r = np.exp(cc * a[di].astype(np.float64))                          # (n,)
        B64, C64 = Bv.astype(np.float64), Cv.astype(np.float64)
        x = cc * B64[:, None] * float(uval[di]) * (1 - r[:, None] ** (t[None, :] + 1)) / (1 - r[:, None])
        y = (C64[:, None] * x).sum(axis=0)
        _close(out[di], y)
        _close(last[di], x[:, -1])


def test_lti_case_is_a_convolution():
    """Fixed B/C, constant delta': y = K * u with K_k = sum_s C_s r_s^k c B_s."""
    rng = np.random.default_rng(3)
    b, d, l, n = 2, 2, 37, 4
    c = 0.2
    inp = {
        "u": _rand(rng, (b, d, l)),
        "delta": np.full((b, d, l), c, np.float32),
        "A": -np.exp(_rand(rng, (d, n), 0.0, 0.5)),
        "B": _rand(rng, (d, n)),
        "C": _rand(rng, (d, n)),
    }
    out, _ = _run(inp, softplus=False, B_kind=orc.BC_FIXED, C_kind=orc.BC_FIXED)
    cc = float(np.float32(c))
    k = np.arange(l, dtype=np.float64)
    for bi in range(b):
        for di in range(d):
            r = np.exp(cc * inp["A"][di].astype(np.float64))
            C64, B64 = inp["C"][di].astype(np.float64), inp["B"][di].astype(np.float64)
            K = (C64[:, None] * (r[:, None] ** k[None, :]) * cc * B64[:, None]).sum(0)
            y = np.convolve(inp["u"][bi, di].astype(np.float64), K)[:l]
            _close(out[bi * d + di], y)


def test_single_step():
    """l = 1: y = sum_s C_s B_s delta' u + D u, gated by silu(z)."""
    rng = np.random.default_rng(4)
    b, d, n = 3, 5, 6
    inp = _tiny_inputs(rng, b, d, 1, n)
    out, last = _run(inp)
    dt = _dt_np(inp)[..., 0]
    for bi in range(b):
        for di in range(d):
            u = float(inp["u"][bi, di, 0])
            Bs = inp["B"][bi, 0, :, 0].astype(np.float64)
            Cs = inp["C"][bi, 0, :, 0].astype(np.float64)
            y = (Cs * Bs).sum() * dt[bi, di] * u + float(inp["D"][di]) * u
            y *= _silu_np(inp["z"][bi, di, 0])
            _close(out[bi * d + di, 0], y)
            _close(last[bi * d + di], Bs * dt[bi, di] * u)


# --------------------------------------------------------------------------
# scan: brute force on tiny inputs (explicit transfer products, O(l^2 n))
# --------------------------------------------------------------------------

def _brute_force(inp, softplus, g=1, fixed_B=False, fixed_C=False, init=None):
    u = inp["u"].astype(np.float64)
    b, d, l = u.shape
    n = inp["A"].shape[1]
    dt = _dt_np(inp, softplus)
    A = inp["A"].astype(np.float64)
    out = np.zeros((b * d, l))
    last = np.zeros((b * d, n))
    for bi in range(b):
        for di in range(d):
            # log of dA for every step; products over (tau, t] as exp of sums
            logdA = dt[bi, di][None, :] * A[di][:, None]          # (n, l)
            for t in range(l):
                y = 0.0
                xs = []
                for s in range(n):
                    acc = 0.0
                    if init is not None:
                        acc += math.exp(logdA[s, : t + 1].sum()) * init[bi, di, s]
                    for tau in range(t + 1):
                        trans = math.exp(logdA[s, tau + 1: t + 1].sum())
                        Bv = _bc(inp["B"], fixed_B, bi, di, s, tau, d, g)
                        acc += trans * dt[bi, di, tau] * Bv * u[bi, di, tau]
                    xs.append(acc)
                    y += _bc(inp["C"], fixed_C, bi, di, s, t, d, g) * acc
                if inp.get("D") is not None:
                    y += float(inp["D"][di]) * u[bi, di, t]
                if inp.get("z") is not None:
                    y *= float(_silu_np(inp["z"][bi, di, t]))
                out[bi * d + di, t] = y
                if t == l - 1:
                    last[bi * d + di] = xs
    return out, last


@pytest.mark.parametrize("fixed", [False, True])
@pytest.mark.parametrize("softplus", [True, False])
def test_brute_force_tiny(fixed, softplus):
    rng = np.random.default_rng(10 + fixed + 2 * softplus)
    b, d, l, n = 2, 4, 13, 3
    inp = _tiny_inputs(rng, b, d, l, n, fixed=fixed)
    if not softplus:
        inp["delta"] = np.abs(inp["delta"]) * np.float32(0.3)
        inp["delta_bias"] = None
    kind = orc.BC_FIXED if fixed else orc.BC_VARYING
    out, last = _run(inp, softplus=softplus, B_kind=kind, C_kind=kind)
    ref, ref_last = _brute_force(inp, softplus, fixed_B=fixed, fixed_C=fixed)
    _close(out, ref, 1e-11)
    _close(last, ref_last, 1e-11)


def test_brute_force_grouped_mixed_kinds_and_initial_state():
    rng = np.random.default_rng(21)
    b, d, l, n, g = 2, 4, 9, 2, 2
    inp = _tiny_inputs(rng, b, d, l, n, g=g)
    inp["C"] = _rand(rng, (d, n))                      # fixed C with grouped varying B
    init = rng.standard_normal((b, d, n))
    out, last = _run(inp, ngroups=g, B_kind=orc.BC_VARYING, C_kind=orc.BC_FIXED,
                     initial_state=init)
    ref, ref_last = _brute_force(inp, True, g=g, fixed_C=True, init=init)
    _close(out, ref, 1e-11)
    _close(last, ref_last, 1e-11)


def test_brute_force_bf16_bits():
    """The oracle reads bf16 bits as the exact values they encode."""
    rng = np.random.default_rng(5)
    b, d, l, n = 1, 3, 11, 4
    inp32 = _tiny_inputs(rng, b, d, l, n)
    inp16 = dict(inp32)
    for k in ("u", "delta", "z", "B", "C"):
        inp16[k] = f32_to_bf16_bits(inp32[k])
        inp32[k] = bf16_bits_to_f32(inp16[k])
    out, last = _run(inp16, io_dtype=orc.BF16)
    ref, ref_last = _brute_force(inp32, True)
    _close(out, ref, 1e-11)
    _close(last, ref_last, 1e-11)


# --------------------------------------------------------------------------
# scan: invariants
# --------------------------------------------------------------------------

def test_linearity_in_u():
    rng = np.random.default_rng(6)
    inp = _tiny_inputs(rng, 2, 3, 29, 4)
    out1, last1 = _run(inp)
    inp2 = dict(inp, u=inp["u"] * np.float32(2.0))
    out2, last2 = _run(inp2)
    _close(out2, 2.0 * out1, 1e-14)
    _close(last2, 2.0 * last1, 1e-14)


def test_D_term_and_gate():
    rng = np.random.default_rng(8)
    inp = _tiny_inputs(rng, 2, 3, 23, 4)
    full, _ = _run(inp)
    noD, _ = _run(dict(inp, D=None))
    nogate, _ = _run(dict(inp, z=None))
    nogate_noD, _ = _run(dict(inp, z=None, D=None))
    b, d, l = inp["u"].shape
    u = inp["u"].astype(np.float64).reshape(b * d, l)
    sz = _silu_np(inp["z"]).reshape(b * d, l)
    Dd = np.tile(inp["D"].astype(np.float64), b)[:, None]
    _close(full - noD, Dd * u * sz, 1e-12)
    _close(full, nogate * sz, 1e-13)
    _close(nogate - nogate_noD, Dd * u, 1e-12)
    zero = _run(dict(inp, z=np.zeros_like(inp["z"])))[0]
    assert np.all(zero == 0.0)


def test_delta_bias_shift():
    rng = np.random.default_rng(9)
    inp = _tiny_inputs(rng, 1, 4, 19, 3)
    inp["delta_bias"] = np.full(4, 0.25, np.float32)     # exact in fp32, exact sum below
    inp["delta"] = (np.round(inp["delta"] * 64) / 64).astype(np.float32)
    a, _ = _run(inp)
    shifted = dict(inp, delta=(inp["delta"] + np.float32(0.25)).astype(np.float32), delta_bias=None)
    b, _ = _run(shifted)
    _close(a, b, 1e-15)


def test_split_continuation():
    """Scan [0, l1), then continue from last_state over [l1, l): same as one scan."""
    rng = np.random.default_rng(11)
    b, d, l, n, l1 = 2, 3, 40, 4, 17
    inp = _tiny_inputs(rng, b, d, l, n)
    full, last = _run(inp)

    def cut(a, lo, hi):
        return None if a is None else np.ascontiguousarray(a[..., lo:hi])

    head = {k: (cut(v, 0, l1) if k in ("u", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    tail = {k: (cut(v, l1, l) if k in ("u", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    o1, s1 = _run(head)
    o2, s2 = _run(tail, initial_state=s1.reshape(b, d, n))
    _close(np.concatenate([o1, o2], axis=1), full, 1e-13)
    _close(s2, last, 1e-13)


def test_one_hot_C_selects_state():
    rng = np.random.default_rng(12)
    b, d, l, n = 1, 2, 15, 4
    inp = _tiny_inputs(rng, b, d, l, n)
    inp["D"] = inp["z"] = None
    ref_all, _ = _brute_force(dict(inp, C=np.ones_like(inp["C"])), True)
    total = np.zeros_like(ref_all)
    for k in range(n):
        C = np.zeros_like(inp["C"])
        C[:, :, k, :] = 1.0
        out_k, _ = _run(dict(inp, C=C))
        total += out_k
    _close(total, ref_all, 1e-11)


def test_grouped_layout_invariants():
    rng = np.random.default_rng(13)
    b, d, l, n, g = 2, 8, 21, 4, 4
    inp = _tiny_inputs(rng, b, d, l, n, g=1)
    base, base_last = _run(inp)
    # g identical groups == one group
    rep = dict(inp, B=np.repeat(inp["B"], g, axis=1), C=np.repeat(inp["C"], g, axis=1))
    out, last = _run(rep, ngroups=g)
    np.testing.assert_array_equal(out, base)
    np.testing.assert_array_equal(last, base_last)
    # fixed B/C == varying B/C tiled along (batch, time)
    Bf, Cf = _rand(rng, (d, n)), _rand(rng, (d, n))
    fx, fx_last = _run(dict(inp, B=Bf, C=Cf), B_kind=orc.BC_FIXED, C_kind=orc.BC_FIXED)
    # a per-channel fixed B is a varying B only when every channel has its own group
    Bv = np.broadcast_to(Bf[None, :, :, None], (b, d, n, l)).astype(np.float32)
    Cv = np.broadcast_to(Cf[None, :, :, None], (b, d, n, l)).astype(np.float32)
    vy, vy_last = _run(dict(inp, B=Bv, C=Cv), ngroups=d)
    np.testing.assert_array_equal(fx, vy)
    np.testing.assert_array_equal(fx_last, vy_last)


def test_group_assignment_convention():
    """Convention (parity unpinned by the pages): channel d uses group d // (dim // g)."""
    rng = np.random.default_rng(14)
    b, d, l, n, g = 1, 8, 7, 2, 4
    inp = _tiny_inputs(rng, b, d, l, n, g=g)
    inp["D"] = None
    for k in range(g):
        B = np.zeros_like(inp["B"])
        B[:, k] = inp["B"][:, k]
        out, _ = _run(dict(inp, B=B), ngroups=g)
        nz = np.flatnonzero(np.abs(out).sum(axis=1) > 0)
        np.testing.assert_array_equal(nz, np.arange(k * (d // g), (k + 1) * (d // g)))


def test_rows_subset_matches_full():
    rng = np.random.default_rng(15)
    inp = _tiny_inputs(rng, 3, 5, 12, 3)
    full, last = _run(inp)
    rows = np.array([14, 0, 7, 3])
    sub, sub_last = _run(inp, rows=rows)
    np.testing.assert_array_equal(sub, full[rows])
    np.testing.assert_array_equal(sub_last, last[rows])
    par, _ = _run(inp, nthreads=3)
    np.testing.assert_array_equal(par, full)


# --------------------------------------------------------------------------
# causal conv
# --------------------------------------------------------------------------

def _conv_inputs(rng, b=2, d=3, l=25, w=4):
    return _rand(rng, (b, d, l)), _rand(rng, (d, w), 0.0, 0.5), _rand(rng, (d,))


def test_conv_matches_numpy_convolve():
    """Cross-correlation with left zero padding: y[t] = sum_k w[k] x[t-(W-1)+k],
    i.e. numpy.convolve(x, w[::-1])[:l]."""
    rng = np.random.default_rng(16)
    x, w, bias = _conv_inputs(rng)
    out = orc.causal_conv1d(x, w, bias, orc.ACT_NONE)
    b, d, l = x.shape
    for bi in range(b):
        for di in range(d):
            ref = np.convolve(x[bi, di].astype(np.float64), w[di, ::-1].astype(np.float64))[:l]
            _close(out[bi * d + di], ref + bias[di], 1e-14)
    act = orc.causal_conv1d(x, w, bias, orc.ACT_SILU)
    _close(act, _silu_np(out), 1e-14)


def test_conv_one_hot_and_constant():
    rng = np.random.default_rng(17)
    x, _, bias = _conv_inputs(rng, l=10)
    d = x.shape[1]
    ident = np.zeros((d, 4), np.float32)
    ident[:, 3] = 1.0
    out = orc.causal_conv1d(x, ident, None).reshape(x.shape)
    np.testing.assert_array_equal(out, x.astype(np.float64))
    delay = np.zeros((d, 4), np.float32)
    delay[:, 0] = 1.0
    out = orc.causal_conv1d(x, delay, bias).reshape(x.shape)
    np.testing.assert_array_equal(out[..., :3], np.broadcast_to(bias[None, :, None], out[..., :3].shape))
    _close(out[..., 3:], x[..., :-3].astype(np.float64) + bias[None, :, None], 1e-15)
    const = np.full(x.shape, 1.5, np.float32)
    w = _rand(rng, (d, 4))
    out = orc.causal_conv1d(const, w, None).reshape(x.shape)
    _close(out[..., 3:], np.broadcast_to(1.5 * w.astype(np.float64).sum(1)[None, :, None], out[..., 3:].shape), 1e-14)
    # symmetric kernels: orientation-free check of padding, bias and activation
    sym = np.array([[0.5, -1.0, -1.0, 0.5]] * d, np.float32)
    out = orc.causal_conv1d(x, sym, bias, orc.ACT_SILU)
    out_flip = orc.causal_conv1d(x, sym[:, ::-1].copy(), bias, orc.ACT_SILU)
    np.testing.assert_array_equal(out, out_flip)


def test_conv_prologue_composition():
    """Fused prologue == conv oracle, rounded to the io dtype, fed as u."""
    rng = np.random.default_rng(18)
    b, d, l, n = 2, 3, 19, 4
    inp = _tiny_inputs(rng, b, d, l, n)
    x, w, cb = _conv_inputs(rng, b, d, l)
    for io in (orc.F32, orc.BF16):
        enc = (lambda a: f32_to_bf16_bits(a)) if io == orc.BF16 else (lambda a: a)
        ii = {k: (enc(v) if k in ("u", "delta", "z", "B", "C") else v) for k, v in inp.items()}
        xx = enc(x)
        fused, fused_last = _run(ii, io_dtype=io, conv_x=xx, conv_weight=w, conv_bias=cb,
                                 conv_act=orc.ACT_SILU)
        conv = orc.causal_conv1d(xx, w, cb, orc.ACT_SILU, io_dtype=io).reshape(b, d, l)
        if io == orc.BF16:
            u = f32_to_bf16_bits(np.array([orc.round_bf16(v) for v in conv.ravel()],
                                          np.float32).reshape(b, d, l))
        else:
            u = conv.astype(np.float32)
        sep, sep_last = _run(dict(ii, u=u), io_dtype=io)
        np.testing.assert_array_equal(fused, sep)
        np.testing.assert_array_equal(fused_last, sep_last)


def test_f32_floor_is_the_same_definition():
    """oracle.selective_scan_f32_floor (the binary32 in-order evaluation that
    sets the slow-decay bar) computes the oracle's definition: on well
    conditioned inputs it agrees with the float64 oracle to fp32 rounding,
    with and without softplus, z and D, for time-varying and fixed B/C."""
    import numpy as np
    from state_space_model_scan_amd.inputs import WORKLOADS, make_inputs
    for kw in (dict(), dict(softplus=False, delta_mean=0.1, delta_std=0.05),
               dict(has_z=False, has_D=False), dict(bc_kind="fixed", dstate=8)):
        w = WORKLOADS["tiny"].scaled(dim=24, seqlen=200, **kw)
        t = make_inputs(w)
        bk = orc.BC_FIXED if t["B"].ndim == 2 else orc.BC_VARYING
        ref, ref_last = orc.selective_scan(
            t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], w.softplus,
            io_dtype=w.io_dtype, B_kind=bk, C_kind=bk)
        f, fl = orc.selective_scan_f32_floor(
            t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"], t["delta_bias"], w.softplus,
            io_dtype=w.io_dtype, B_kind=bk, C_kind=bk)
        assert np.max(np.abs(f - ref) / (1 + np.abs(ref))) < 2e-5, kw
        assert np.max(np.abs(fl - ref_last) / (1 + np.abs(ref_last))) < 2e-5, kw
        # and it is a float32 evaluation: not the float64 result itself
        assert not np.array_equal(f, ref)
