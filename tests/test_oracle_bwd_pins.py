"""Pins for the oracle's selective-scan backward (oracle_selective_scan_bwd).

The backward is the gradient of the forward oracle, which is pinned on its
own (test_oracle_pins.py).  Each pin here checks the gradient against the
forward alone, so a mistake in the adjoint recurrence cannot hide:

  * central finite differences of L = sum(dout * out) through the forward
    oracle, element by element, for every input the backward differentiates
    (u, delta, A, B, C, D, z, delta_bias, initial_state), for the varying and
    the fixed B/C layouts, with and without softplus, groups, the gate, D;
  * Euler's identity for functions homogeneous of degree one: out is linear
    in (u, initial_state) jointly, in C, and (with no initial state and no D)
    in B, so <grad, input> must equal L exactly up to rounding;
  * the bf16-io gradients equal the fp32-io gradients of the same values.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import f32_to_bf16_bits, bf16_bits_to_f32


def _rand(rng, shape, mean=0.0, std=1.0):
    return (rng.standard_normal(shape) * std + mean).astype(np.float32)


def _problem(rng, b=2, d=4, l=6, n=3, g=1, fixed_B=False, fixed_C=False, has_z=True, has_D=True,
             has_bias=True, init=True):
    p = {
        "u": _rand(rng, (b, d, l)),
        "delta": _rand(rng, (b, d, l), -0.5, 0.7),
        "A": -rng.uniform(0.3, 2.5, (d, n)).astype(np.float32),
        "B": _rand(rng, (d, n)) if fixed_B else _rand(rng, (b, g, n, l)),
        "C": _rand(rng, (d, n)) if fixed_C else _rand(rng, (b, g, n, l)),
        "D": _rand(rng, (d,)) if has_D else None,
        "z": _rand(rng, (b, d, l)) if has_z else None,
        "delta_bias": rng.uniform(-0.3, 0.3, d).astype(np.float32) if has_bias else None,
        "initial_state": rng.standard_normal((b, d, n)) if init else None,
    }
    kinds = dict(ngroups=g, B_kind=orc.BC_FIXED if fixed_B else orc.BC_VARYING,
                 C_kind=orc.BC_FIXED if fixed_C else orc.BC_VARYING)
    return p, kinds


def _forward(p, softplus, kinds, io=orc.F32):
    out, _ = orc.selective_scan(p["u"], p["delta"], p["A"], p["B"], p["C"], p["D"], p["z"],
                                p["delta_bias"], softplus, io_dtype=io,
                                initial_state=p["initial_state"], **kinds)
    return out.reshape(p["delta"].shape)


def _backward(p, dout, softplus, kinds, io=orc.F32):
    return orc.selective_scan_bwd(p["u"], p["delta"], p["A"], p["B"], p["C"], dout, p["D"], p["z"],
                                  p["delta_bias"], softplus, io_dtype=io,
                                  initial_state=p["initial_state"], **kinds)


GRAD_OF = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz",
           "delta_bias": "ddelta_bias", "initial_state": "dinitial_state"}


def _finite_difference(p, dout, softplus, kinds, name, h=1e-4):
    """dL/d(p[name]) by central differences; a float32 input moves by its
    float32-rounded step, and the exact step taken is the divisor."""
    base = p[name]
    fd = np.zeros(base.shape)
    for idx in np.ndindex(base.shape):
        vals = []
        steps = []
        for sgn in (1.0, -1.0):
            q = dict(p)
            arr = base.copy()
            arr[idx] = arr[idx] + sgn * h
            steps.append(float(arr[idx]) - float(base[idx]))
            q[name] = arr
            vals.append(float(np.sum(_forward(q, softplus, kinds) * dout)))
        fd[idx] = (vals[0] - vals[1]) / (steps[0] - steps[1])
    return fd


CASES = {
    "varying": dict(),
    "fixed_B": dict(fixed_B=True),
    "fixed_BC": dict(fixed_B=True, fixed_C=True),
    "groups2": dict(d=4, g=2),
    "bare": dict(has_z=False, has_D=False, has_bias=False, init=False),
}


@pytest.mark.parametrize("softplus", [True, False])
@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_matches_finite_differences(case, softplus):
    rng = np.random.default_rng(300 + len(case) + 7 * softplus)
    p, kinds = _problem(rng, **CASES[case])
    if not softplus:   # keep the step positive without softplus
        p["delta"] = (0.2 + 0.3 * np.abs(p["delta"])).astype(np.float32)
    dout = rng.standard_normal(p["delta"].shape)
    g = _backward(p, dout, softplus, kinds)
    for name, gname in GRAD_OF.items():
        if p[name] is None:
            continue
        fd = _finite_difference(p, dout, softplus, kinds, name)
        err = np.max(np.abs(g[gname] - fd)) / (1.0 + np.max(np.abs(fd)))
        assert err <= 1e-6, f"{case} softplus={softplus}: {gname} differs from finite differences by {err:.2e}"


@pytest.mark.parametrize("softplus", [True, False])
def test_backward_euler_identities(softplus):
    rng = np.random.default_rng(320 + softplus)
    p, kinds = _problem(rng, b=2, d=6, l=11, n=4, g=2)
    dout = rng.standard_normal(p["delta"].shape)
    L = float(np.sum(_forward(p, softplus, kinds) * dout))
    g = _backward(p, dout, softplus, kinds)
    # jointly linear in (u, initial_state)
    lin_u = np.sum(g["du"] * p["u"]) + np.sum(g["dinitial_state"] * p["initial_state"])
    assert abs(lin_u - L) <= 1e-11 * (1 + abs(L))
    # linear in C (D off)
    q = dict(p, D=None)
    Lq = float(np.sum(_forward(q, softplus, kinds) * dout))
    gq = _backward(q, dout, softplus, kinds)
    assert abs(np.sum(gq["dC"] * q["C"]) - Lq) <= 1e-11 * (1 + abs(Lq))
    # linear in B (D off, zero initial state)
    r = dict(p, D=None, initial_state=None)
    Lr = float(np.sum(_forward(r, softplus, kinds) * dout))
    gr = _backward(r, dout, softplus, kinds)
    assert abs(np.sum(gr["dB"] * r["B"]) - Lr) <= 1e-11 * (1 + abs(Lr))
    # the D term is linear in D
    assert abs(np.sum(g["dD"] * p["D"]) - (L - Lq)) <= 1e-11 * (1 + abs(L))


def test_backward_bf16_io_equals_f32_io_on_the_same_values():
    rng = np.random.default_rng(330)
    p, kinds = _problem(rng, b=1, d=4, l=9, n=3, g=2)
    pb = dict(p)
    pf = dict(p)
    for k in ("u", "delta", "B", "C", "z"):
        pb[k] = f32_to_bf16_bits(p[k])
        pf[k] = bf16_bits_to_f32(pb[k])
    dout = rng.standard_normal(p["delta"].shape)
    gb = _backward(pb, dout, True, kinds, io=orc.BF16)
    gf = _backward(pf, dout, True, kinds, io=orc.F32)
    for k in GRAD_OF.values():
        np.testing.assert_array_equal(gb[k], gf[k])


def test_backward_initial_state_gradient_closed_form():
    """The initial state reaches out_t through exp(A sum_{k<=t} dt'_k) C_t and
    the gate alone, so its gradient is the sum over t of
    dout_t silu(z_t) C_t exp(A cs_t), with cs_t the running sum of the steps."""
    rng = np.random.default_rng(331)
    p, kinds = _problem(rng, b=2, d=3, l=17, n=4, g=1)
    dout = rng.standard_normal(p["delta"].shape)
    g = _backward(p, dout, True, kinds)
    step = np.logaddexp(0.0, p["delta"].astype(np.float64) + p["delta_bias"].astype(np.float64)[None, :, None])
    cs = np.cumsum(step, axis=2)                                      # (b, d, l)
    zf = p["z"].astype(np.float64)
    gate = dout * zf / (1.0 + np.exp(-zf))                            # (b, d, l)
    decay = np.exp(p["A"].astype(np.float64)[None, :, :, None] * cs[:, :, None, :])   # (b, d, n, l)
    Cm = p["C"][:, 0].astype(np.float64)                              # (b, n, l)
    want = np.einsum("bdl,bdnl,bnl->bdn", gate, decay, Cm)
    np.testing.assert_allclose(g["dinitial_state"], want, rtol=1e-12, atol=1e-13)
