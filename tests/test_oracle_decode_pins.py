"""Pins for the oracle's single-step decode functions (selective_state_update
and causal_conv1d_update), each against something other than the decode code:

  * decode == prefill: chaining the decode step over a sequence reproduces the
    oracle scan / conv over the whole sequence (those are pinned on their own
    by closed forms, brute force and library routines in the other pin files);
  * closed forms of special cases (A = 0, B = 0, one-hot C, identity kernels);
  * cache invariants: what the conv cache holds after a call, and that the
    ring-buffer mode sees the same history as the shifted cache.

The operators are named in the PaddleNLP Kernel operator-library guide:
selective_state_update in the mamba operator list of section 4.4, and
causal_conv1d_update with its conv_state cache and optional ring buffer
(cache_seqlens) in section 4.2.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import f32_to_bf16_bits, f32_to_f16_bits

TOL = 1e-12


def _close(a, b, tol=TOL):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"max normalised error {err:.3e} > {tol:.1e}"


def _rand(rng, shape, mean=0.0, std=1.0):
    return (rng.standard_normal(shape) * std + mean).astype(np.float32)


def _decode_inputs(rng, b, d, l, n, g, io=orc.F32):
    u = _rand(rng, (b, d, l))
    dt = _rand(rng, (b, d, l), -1.5, 0.5)
    z = _rand(rng, (b, d, l))
    B = _rand(rng, (b, g, n, l))
    C = _rand(rng, (b, g, n, l))
    A = -np.exp(_rand(rng, (d, n), 0.0, 0.5))
    D = _rand(rng, (d,))
    bias = (rng.uniform(-0.1, 0.1, d)).astype(np.float32)
    init = rng.standard_normal((b, d, n))
    if io == orc.BF16:
        u, dt, z, B, C = (f32_to_bf16_bits(a) for a in (u, dt, z, B, C))
    return u, dt, z, B, C, A, D, bias, init


# --------------------------------------------------------------------------
# selective_state_update
# --------------------------------------------------------------------------

@pytest.mark.parametrize("io", [orc.F32, orc.BF16])
@pytest.mark.parametrize("g", [1, 2])
@pytest.mark.parametrize("softplus", [True, False])
def test_state_update_chain_equals_scan(io, g, softplus):
    """l decode steps fed their own state equal one scan of length l started
    from the same state: every output and the final state."""
    rng = np.random.default_rng(11 + 3 * g + io)
    b, d, l, n = 2, 4, 9, 5
    u, dt, z, B, C, A, D, bias, init = _decode_inputs(rng, b, d, l, n, g, io)
    if not softplus:
        dt = dt if io == orc.BF16 else np.abs(dt).astype(np.float32) * 0.3
    ref_out, ref_last = orc.selective_scan(u, dt, A, B, C, D, z, bias, softplus, io_dtype=io,
                                           ngroups=g, initial_state=init)
    ref_out = ref_out.reshape(b, d, l)
    state = init.copy()
    for t in range(l):
        out, state = orc.selective_state_update(
            state, np.ascontiguousarray(u[:, :, t]), np.ascontiguousarray(dt[:, :, t]), A,
            np.ascontiguousarray(B[..., t]), np.ascontiguousarray(C[..., t]), D,
            np.ascontiguousarray(z[:, :, t]), bias, softplus, io_dtype=io)
        _close(out, ref_out[:, :, t])
    _close(state, ref_last.reshape(b, d, n))


def test_state_update_a_zero_is_accumulation():
    """A = 0: the state just accumulates dt'*B*x, and y = C . state."""
    rng = np.random.default_rng(5)
    b, d, n, g = 2, 6, 3, 3
    x, dt = _rand(rng, (b, d)), _rand(rng, (b, d), -1.0, 0.3)
    B, C = _rand(rng, (b, g, n)), _rand(rng, (b, g, n))
    A = np.zeros((d, n), np.float32)
    state = rng.standard_normal((b, d, n))
    out, new = orc.selective_state_update(state, x, dt, A, B, C, None, None, None, False)
    grp = np.arange(d) // (d // g)
    step = dt.astype(np.float64)
    want = state + step[..., None] * B[:, grp, :].astype(np.float64) * x.astype(np.float64)[..., None]
    _close(new, want)
    _close(out, np.einsum("bdn,bdn->bd", C[:, grp, :].astype(np.float64), want))


def test_state_update_zero_step_keeps_state():
    """dt' = 0 (no softplus, bias cancels dt): the state is unchanged and the
    output is C . state + D x, gated."""
    rng = np.random.default_rng(6)
    b, d, n = 1, 4, 4
    x = _rand(rng, (b, d))
    dt = np.full((b, d), 0.25, np.float32)
    bias = np.full((d,), -0.25, np.float32)
    B, C = _rand(rng, (b, 1, n)), _rand(rng, (b, 1, n))
    A, D = -np.ones((d, n), np.float32), _rand(rng, (d,))
    state = rng.standard_normal((b, d, n))
    out, new = orc.selective_state_update(state, x, dt, A, B, C, D, None, bias, False)
    _close(new, state)
    want = np.einsum("bn,bdn->bd", C[:, 0].astype(np.float64), state) + D * x.astype(np.float64)
    _close(out, want)


def test_state_update_one_hot_c_reads_one_state():
    rng = np.random.default_rng(7)
    b, d, n = 2, 3, 6
    x, dt = _rand(rng, (b, d)), _rand(rng, (b, d), -1.0, 0.5)
    B = _rand(rng, (b, 1, n))
    A = -np.exp(_rand(rng, (d, n), 0.0, 0.5))
    state = rng.standard_normal((b, d, n))
    for s in (0, 4):
        C = np.zeros((b, 1, n), np.float32)
        C[:, :, s] = 1.0
        out, new = orc.selective_state_update(state, x, dt, A, B, C, None, None, None, True)
        _close(out, new[:, :, s])


def test_state_update_groups_broadcast():
    """ngroups identical groups give the one-group result."""
    rng = np.random.default_rng(8)
    b, d, n = 2, 8, 4
    x, dt, z = _rand(rng, (b, d)), _rand(rng, (b, d)), _rand(rng, (b, d))
    B1, C1 = _rand(rng, (b, 1, n)), _rand(rng, (b, 1, n))
    A = -np.exp(_rand(rng, (d, n), 0.0, 0.5))
    state = rng.standard_normal((b, d, n))
    o1, s1 = orc.selective_state_update(state, x, dt, A, B1, C1, None, z, None, True)
    o4, s4 = orc.selective_state_update(state, x, dt, A, np.repeat(B1, 4, axis=1),
                                        np.repeat(C1, 4, axis=1), None, z, None, True)
    _close(o4, o1)
    _close(s4, s1)


# --------------------------------------------------------------------------
# causal_conv1d_update
# --------------------------------------------------------------------------

@pytest.mark.parametrize("io", [orc.F32, orc.BF16, orc.F16])
@pytest.mark.parametrize("act", [orc.ACT_NONE, orc.ACT_SILU])
@pytest.mark.parametrize("width", [2, 4])
def test_conv_update_chain_equals_conv(io, act, width):
    """Token-by-token updates from an all-zero cache reproduce the causal conv
    of the whole sequence, in both cache modes; the shifted cache ends holding
    the last state_len inputs bit for bit."""
    rng = np.random.default_rng(20 + width + 2 * io)
    b, d, l = 2, 3, 11
    x = _rand(rng, (b, d, l))
    if io == orc.BF16:
        x = f32_to_bf16_bits(x)
    elif io == orc.F16:
        x = f32_to_f16_bits(x)
    w = _rand(rng, (d, width), 0.0, 0.5)
    bias = _rand(rng, (d,))
    ref = orc.causal_conv1d(x, w, bias, act, io_dtype=io).reshape(b, d, l)
    S = width - 1 + 2
    dtype = x.dtype
    shift = np.zeros((b, d, S), dtype)
    ring = np.zeros((b, d, S), dtype)
    pos = np.zeros((b,), np.int32)
    for t in range(l):
        xt = np.ascontiguousarray(x[:, :, t:t + 1])
        o1, shift = orc.causal_conv1d_update(xt, shift, w, bias, act, io_dtype=io)
        o2, ring = orc.causal_conv1d_update(xt, ring, w, bias, act, pos, io_dtype=io)
        pos = pos + 1
        _close(o1[:, :, 0], ref[:, :, t])
        _close(o2[:, :, 0], ref[:, :, t])
    assert np.array_equal(shift, x[:, :, l - S:])
    # the ring buffer holds the same inputs, rotated to slot t % S
    for t in range(l - S, l):
        assert np.array_equal(ring[:, :, t % S], x[:, :, t])


@pytest.mark.parametrize("ring", [False, True])
def test_conv_update_multi_token_equals_single_steps(ring):
    rng = np.random.default_rng(31)
    b, d, width, S, L = 2, 4, 4, 5, 6
    x = _rand(rng, (b, d, L))
    w, bias = _rand(rng, (d, width), 0.0, 0.5), _rand(rng, (d,))
    cache = _rand(rng, (b, d, S))
    pos = np.array([3, 7], np.int32) if ring else None
    many, st_many = orc.causal_conv1d_update(x, cache, w, bias, orc.ACT_SILU, pos)
    st = cache.copy()
    for t in range(L):
        p = None if pos is None else (pos + t).astype(np.int32)
        o, st = orc.causal_conv1d_update(np.ascontiguousarray(x[:, :, t:t + 1]), st, w, bias,
                                         orc.ACT_SILU, p)
        _close(o[:, :, 0], many[:, :, t])
    assert np.array_equal(st, st_many)


def test_conv_update_identity_kernel_and_history():
    """A one-hot kernel on the oldest tap returns the input width-1 steps back,
    which for the first new token is the cache's last width-1 entries."""
    rng = np.random.default_rng(32)
    b, d, width, S, L = 1, 2, 4, 3, 5
    x = _rand(rng, (b, d, L))
    cache = _rand(rng, (b, d, S))
    w = np.zeros((d, width), np.float32)
    w[:, 0] = 1.0
    out, new = orc.causal_conv1d_update(x, cache, w, None, orc.ACT_NONE)
    hist = np.concatenate([cache, x], axis=2).astype(np.float64)
    for t in range(L):
        _close(out[:, :, t], hist[:, :, S + t - (width - 1)])
    assert np.array_equal(new, np.concatenate([cache, x], axis=2)[:, :, L:])
    w[:, 0] = 0.0
    w[:, -1] = 1.0   # current sample
    out, _ = orc.causal_conv1d_update(x, cache, w, None, orc.ACT_NONE)
    _close(out, x)


def test_conv_update_ring_reads_the_slots_before_the_position():
    """Ring mode with a filled cache: the window of the first token is the
    width-1 slots before position p, circularly."""
    rng = np.random.default_rng(33)
    b, d, width, S = 3, 2, 4, 5
    cache = _rand(rng, (b, d, S))
    x = _rand(rng, (b, d, 1))
    w = _rand(rng, (d, width), 0.0, 0.5)
    pos = np.array([0, 2, 9], np.int32)
    out, new = orc.causal_conv1d_update(x, cache, w, None, orc.ACT_NONE, pos)
    for bb in range(b):
        p = int(pos[bb])
        win = [cache[bb, :, (p - (width - 1) + k) % S] for k in range(width - 1)] + [x[bb, :, 0]]
        want = sum(w[:, k].astype(np.float64) * np.asarray(win[k], np.float64) for k in range(width))
        _close(out[bb, :, 0], want)
        expect = cache[bb].copy()
        expect[:, p % S] = x[bb, :, 0]
        assert np.array_equal(new[bb], expect)
