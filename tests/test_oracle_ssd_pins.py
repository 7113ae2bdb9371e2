"""Pins for the oracle's Mamba-2 scan (oracle_ssd_scan): the SSD operators of
the PaddleNLP Kernel operator-library guide (section 4.4: mamba_chunk_scan,
mamba_chunk_scan_combined, chunk_state, state_passing), read as the selective
scan recurrence with a scalar decay per head and a step shared by the head's
channels.  Each pin is independent of the SSD code:

  * the same computation through the selective-scan oracle (which is pinned
    on its own) with the head layout flattened into channels;
  * the quadratic "dual" form, y_t = sum_{tau <= t} (C_t . B_tau) *
    exp(A sum_{tau<k<=t} dt'_k) * dt'_tau * x_tau + C_t . decay(H_0),
    written out in numpy with its own softplus;
  * continuation of a split sequence through the states;
  * D given per head equals D repeated per channel.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import f32_to_bf16_bits, bf16_bits_to_f32

TOL = 1e-12


def _close(a, b, tol=TOL):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"max normalised error {err:.3e} > {tol:.1e}"


def _rand(rng, shape, mean=0.0, std=1.0):
    return (rng.standard_normal(shape) * std + mean).astype(np.float32)


def _inputs(rng, b, l, h, p, n, g, io=orc.F32):
    x = _rand(rng, (b, l, h, p))
    dt = _rand(rng, (b, l, h), -1.5, 0.5)
    z = _rand(rng, (b, l, h, p))
    B = _rand(rng, (b, l, g, n))
    C = _rand(rng, (b, l, g, n))
    A = -rng.uniform(0.5, 4.0, h).astype(np.float32)
    D = _rand(rng, (h,))
    bias = rng.uniform(-0.1, 0.1, h).astype(np.float32)
    init = rng.standard_normal((b, h, p, n))
    if io == orc.BF16:
        x, dt, z, B, C = (f32_to_bf16_bits(a) for a in (x, dt, z, B, C))
    return x, dt, z, B, C, A, D, bias, init


def _as_float(a, io):
    return bf16_bits_to_f32(a).astype(np.float64) if io == orc.BF16 else np.asarray(a, np.float64)


@pytest.mark.parametrize("io", [orc.F32, orc.BF16])
@pytest.mark.parametrize("g", [1, 2])
@pytest.mark.parametrize("softplus", [True, False])
def test_ssd_equals_selective_scan_flattened(io, g, softplus):
    rng = np.random.default_rng(50 + g + 2 * io)
    b, l, h, p, n = 2, 13, 4, 3, 5
    x, dt, z, B, C, A, D, bias, init = _inputs(rng, b, l, h, p, n, g, io)
    out, fin = orc.ssd_scan(x, dt, A, B, C, D, z, bias, softplus, io_dtype=io, initial_states=init)
    # channel d = head * p + element; the head's step, decay, bias and D repeat over p
    u1 = np.ascontiguousarray(x.transpose(0, 2, 3, 1).reshape(b, h * p, l))
    z1 = np.ascontiguousarray(z.transpose(0, 2, 3, 1).reshape(b, h * p, l))
    dt1 = np.ascontiguousarray(np.repeat(dt.transpose(0, 2, 1), p, axis=1))
    A1 = np.ascontiguousarray(np.repeat(A, p)[:, None] * np.ones((1, n), np.float32))
    B1 = np.ascontiguousarray(B.transpose(0, 2, 3, 1))
    C1 = np.ascontiguousarray(C.transpose(0, 2, 3, 1))
    ref, last = orc.selective_scan(u1, dt1, A1, B1, C1, np.repeat(D, p), z1, np.repeat(bias, p),
                                   softplus, io_dtype=io, ngroups=g,
                                   initial_state=init.reshape(b, h * p, n))
    _close(out.transpose(0, 2, 3, 1).reshape(b * h * p, l), ref)
    _close(fin.reshape(b * h * p, n), last)


@pytest.mark.parametrize("softplus", [True, False])
def test_ssd_dual_quadratic_form(softplus):
    """Brute force in the quadratic form, per (b, h)."""
    rng = np.random.default_rng(60)
    b, l, h, p, n, g = 2, 9, 4, 3, 4, 2
    x, dt, z, B, C, A, D, bias, init = _inputs(rng, b, l, h, p, n, g)
    out, fin = orc.ssd_scan(x, dt, A, B, C, D, None, bias, softplus, initial_states=init)
    step = dt.astype(np.float64) + bias.astype(np.float64)[None, None, :]
    if softplus:
        step = np.logaddexp(0.0, step)
    want = np.zeros((b, l, h, p))
    want_fin = np.zeros((b, h, p, n))
    for bb in range(b):
        for hh in range(h):
            gg = hh // (h // g)
            a = float(A[hh])
            cs = np.concatenate([[0.0], np.cumsum(step[bb, :, hh])])   # cs[t+1] = sum_{k<=t} dt'_k
            Bm = B[bb, :, gg, :].astype(np.float64)
            Cm = C[bb, :, gg, :].astype(np.float64)
            X = x[bb, :, hh, :].astype(np.float64)
            for t in range(l):
                acc = np.zeros(p)
                for tau in range(t + 1):
                    w = (Cm[t] @ Bm[tau]) * np.exp(a * (cs[t + 1] - cs[tau + 1])) * step[bb, tau, hh]
                    acc += w * X[tau]
                acc += np.exp(a * cs[t + 1]) * (init[bb, hh] @ Cm[t])
                want[bb, t, hh] = acc + D[hh] * X[t]
            Hf = np.exp(a * cs[l]) * init[bb, hh]
            for tau in range(l):
                Hf += np.exp(a * (cs[l] - cs[tau + 1])) * step[bb, tau, hh] * np.outer(X[tau], Bm[tau])
            want_fin[bb, hh] = Hf
    _close(out, want, 1e-11)
    _close(fin, want_fin, 1e-11)


def test_ssd_split_continuation():
    rng = np.random.default_rng(61)
    b, l, h, p, n, g = 1, 16, 2, 4, 3, 1
    x, dt, z, B, C, A, D, bias, init = _inputs(rng, b, l, h, p, n, g)
    full, fin = orc.ssd_scan(x, dt, A, B, C, D, z, bias, True, initial_states=init)
    k = 7
    o1, f1 = orc.ssd_scan(np.ascontiguousarray(x[:, :k]), np.ascontiguousarray(dt[:, :k]), A,
                          np.ascontiguousarray(B[:, :k]), np.ascontiguousarray(C[:, :k]), D,
                          np.ascontiguousarray(z[:, :k]), bias, True, initial_states=init)
    o2, f2 = orc.ssd_scan(np.ascontiguousarray(x[:, k:]), np.ascontiguousarray(dt[:, k:]), A,
                          np.ascontiguousarray(B[:, k:]), np.ascontiguousarray(C[:, k:]), D,
                          np.ascontiguousarray(z[:, k:]), bias, True, initial_states=f1)
    _close(np.concatenate([o1, o2], axis=1), full)
    _close(f2, fin)


def test_ssd_D_per_head_equals_per_channel():
    rng = np.random.default_rng(62)
    b, l, h, p, n, g = 1, 5, 3, 4, 2, 3
    x, dt, z, B, C, A, D, bias, init = _inputs(rng, b, l, h, p, n, g)
    o1, _ = orc.ssd_scan(x, dt, A, B, C, D, z, bias, True)
    o2, _ = orc.ssd_scan(x, dt, A, B, C, np.repeat(D[:, None], p, axis=1), z, bias, True)
    _close(o1, o2)
    Dc = _rand(rng, (h, p))
    o3, _ = orc.ssd_scan(x, dt, A, B, C, Dc, None, bias, True)
    o4, _ = orc.ssd_scan(x, dt, A, B, C, None, None, bias, True)
    _close(o3 - o4, Dc[None, None] * x.astype(np.float64))
