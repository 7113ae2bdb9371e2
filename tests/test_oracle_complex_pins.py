"""Pins for the oracle's complex-A selective scan, each against something
other than the complex code:

  * the real case: zero imaginary parts reproduce the (separately pinned)
    real oracle scan, output and last state;
  * brute force on tiny inputs: every complex state written as a real
    2-vector, its decay exp(delta' A) as the matrix exponential (scipy) of the
    2x2 real block [[Re A, -Im A], [Im A, Re A]] times delta', and the output
    as [Re C, -Im C] applied to the state;
  * a closed form: A = i w, a constant step c and constant B = beta, C =
    gamma, u = 1 give the geometric sum x_t = c beta (1 - q^(t+1)) / (1 - q),
    q = exp(i w c), so y_t = Re(gamma x_t): this fixes the direction of the
    rotation and that C is not conjugated;
  * conjugation: conjugating A, B, C and the initial state leaves the output
    unchanged and conjugates the last state.

The pages (PaddleNLP Kernel operator-library guide, section 4.1) only say
that A may be real or complex; the reading (complex B and C, the real part of
the contraction) is stated in ssm_oracle.c.
"""
import numpy as np
import pytest
import scipy.linalg

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import f32_to_bf16_bits, io_bits_to_f64

TOL = 1e-12


def _close(a, b, tol=TOL):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"max normalised error {err:.3e} > {tol:.1e}"


def _rand(rng, shape, mean=0.0, std=1.0):
    return (rng.standard_normal(shape) * std + mean).astype(np.float32)


def _complex_inputs(rng, b, d, l, n, g, fixed=False):
    u = _rand(rng, (b, d, l))
    dt = _rand(rng, (b, d, l), -1.0, 0.5)
    z = _rand(rng, (b, d, l))
    A = np.stack([-np.exp(_rand(rng, (d, n), 0.0, 0.5)), _rand(rng, (d, n), 0.0, 3.0)], axis=-1)
    shp = (d, n, 2) if fixed else (b, g, n, l, 2)
    B, C = _rand(rng, shp), _rand(rng, shp)
    D = _rand(rng, (d,))
    bias = rng.uniform(-0.1, 0.1, d).astype(np.float32)
    init = rng.standard_normal((b, d, n, 2))
    return u, dt, z, A.astype(np.float32), B, C, D, bias, init


@pytest.mark.parametrize("io", [orc.F32, orc.BF16])
@pytest.mark.parametrize("fixed,g", [(False, 1), (False, 2), (True, 1)])
def test_complex_real_case_equals_real_scan(io, fixed, g):
    rng = np.random.default_rng(40 + g + 3 * fixed + 7 * io)
    b, d, l, n = 2, 4, 13, 5
    u, dt, z, A, B, C, D, bias, init = _complex_inputs(rng, b, d, l, n, g, fixed)
    A[..., 1] = 0.0
    B[..., 1] = 0.0
    C[..., 1] = 0.0
    init[..., 1] = 0.0
    if io == orc.BF16:
        u, dt, z, B, C = (f32_to_bf16_bits(a) for a in (u, dt, z, B, C))
    kind = orc.BC_FIXED if fixed else orc.BC_VARYING
    out_c, last_c = orc.selective_scan_complex(u, dt, A, B, C, D, z, bias, True, io_dtype=io, ngroups=g,
                                               B_kind=kind, C_kind=kind, initial_state=init)
    Br, Cr = np.ascontiguousarray(B[..., 0]), np.ascontiguousarray(C[..., 0])
    out_r, last_r = orc.selective_scan(u, dt, np.ascontiguousarray(A[..., 0]), Br, Cr, D, z, bias, True,
                                       io_dtype=io, ngroups=g, B_kind=kind, C_kind=kind,
                                       initial_state=np.ascontiguousarray(init[..., 0]))
    _close(out_c, out_r)
    _close(last_c[..., 0], last_r)
    assert np.all(last_c[..., 1] == 0.0)


def _brute(u, dt, z, A, B, C, D, bias, init, fixed, softplus):
    """Each complex state as a real 2-vector; decay by the matrix exponential."""
    b, d, l = dt.shape
    n = A.shape[1]
    out = np.zeros((b, d, l))
    last = np.zeros((b, d, n, 2))
    for bb in range(b):
        for dd in range(d):
            v = [np.array(init[bb, dd, s], np.float64) for s in range(n)]
            for t in range(l):
                step = float(dt[bb, dd, t]) + float(bias[dd])
                if softplus:
                    step = np.log1p(np.exp(step))
                y = 0.0
                for s in range(n):
                    ar, ai = float(A[dd, s, 0]), float(A[dd, s, 1])
                    M = np.array([[ar, -ai], [ai, ar]]) * step
                    bv = B[dd, s] if fixed else B[bb, 0, s, t]
                    cv = C[dd, s] if fixed else C[bb, 0, s, t]
                    v[s] = scipy.linalg.expm(M) @ v[s] + step * float(u[bb, dd, t]) * np.array(bv, np.float64)
                    y += float(cv[0]) * v[s][0] - float(cv[1]) * v[s][1]
                y += float(D[dd]) * float(u[bb, dd, t])
                zz = float(z[bb, dd, t])
                out[bb, dd, t] = y * zz / (1.0 + np.exp(-zz))
            for s in range(n):
                last[bb, dd, s] = v[s]
    return out, last


@pytest.mark.parametrize("fixed", [False, True])
@pytest.mark.parametrize("softplus", [True, False])
def test_complex_brute_force_tiny(fixed, softplus):
    rng = np.random.default_rng(50 + fixed + 2 * softplus)
    b, d, l, n = 2, 3, 7, 3
    u, dt, z, A, B, C, D, bias, init = _complex_inputs(rng, b, d, l, n, 1, fixed)
    if not softplus:
        dt = (np.abs(dt) * 0.4).astype(np.float32)
    kind = orc.BC_FIXED if fixed else orc.BC_VARYING
    out, last = orc.selective_scan_complex(u, dt, A, B, C, D, z, bias, softplus, B_kind=kind, C_kind=kind,
                                           initial_state=init)
    want_out, want_last = _brute(u, dt, z, A, B, C, D, bias, init, fixed, softplus)
    _close(out, want_out.reshape(b * d, l), 1e-11)
    _close(last, want_last.reshape(b * d, n, 2), 1e-11)


def test_complex_rotation_closed_form():
    l, c, w = 40, 0.25, 1.7
    beta, gamma = 0.8 - 0.6j, -0.3 + 1.1j
    u = np.ones((1, 1, l), np.float32)
    dt = np.full((1, 1, l), c, np.float32)
    A = np.array([[[0.0, w]]], np.float32)
    B = np.array([[[beta.real, beta.imag]]], np.float32)
    C = np.array([[[gamma.real, gamma.imag]]], np.float32)
    out, last = orc.selective_scan_complex(u, dt, A, B, C, B_kind=orc.BC_FIXED, C_kind=orc.BC_FIXED)
    cb = float(np.float32(c)) * complex(float(np.float32(beta.real)), float(np.float32(beta.imag)))
    gm = complex(float(np.float32(gamma.real)), float(np.float32(gamma.imag)))
    q = np.exp(1j * float(np.float32(w)) * float(np.float32(c)))
    t = np.arange(l)
    x = cb * (1.0 - q ** (t + 1)) / (1.0 - q)
    _close(out[0], (gm * x).real)
    _close(last[0, 0], [x[-1].real, x[-1].imag])


def test_complex_conjugate_symmetry():
    rng = np.random.default_rng(60)
    b, d, l, n = 2, 4, 11, 4
    u, dt, z, A, B, C, D, bias, init = _complex_inputs(rng, b, d, l, n, 2)
    out1, last1 = orc.selective_scan_complex(u, dt, A, B, C, D, z, bias, True, ngroups=2, initial_state=init)
    neg = lambda a: np.concatenate([a[..., :1], -a[..., 1:]], axis=-1)
    out2, last2 = orc.selective_scan_complex(u, dt, neg(A).astype(np.float32), neg(B).astype(np.float32),
                                             neg(C).astype(np.float32), D, z, bias, True, ngroups=2,
                                             initial_state=neg(init))
    _close(out2, out1)
    _close(last2, neg(last1))


def test_complex_bf16_pairs_read_as_stored():
    """bf16 pairs: the oracle reads each half of a pair from its own bits."""
    rng = np.random.default_rng(61)
    b, d, l, n = 1, 2, 9, 3
    u, dt, z, A, B, C, D, bias, init = _complex_inputs(rng, b, d, l, n, 1)
    bits = [f32_to_bf16_bits(a) for a in (u, dt, z, B, C)]
    widened = [io_bits_to_f64(x, orc.BF16).astype(np.float32) for x in bits]
    o16, l16 = orc.selective_scan_complex(*bits[:2], A, bits[3], bits[4], D, bits[2], bias, True,
                                          io_dtype=orc.BF16, initial_state=init)
    o32, l32 = orc.selective_scan_complex(*widened[:2], A, widened[3], widened[4], D, widened[2], bias, True,
                                          io_dtype=orc.F32, initial_state=init)
    _close(o16, o32)
    _close(l16, l32)
