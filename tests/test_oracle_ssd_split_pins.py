"""Pins for the oracle's split chunk-scan operators (oracle_ssd_chunk_state,
oracle_ssd_state_passing, oracle_ssd_chunk_scan): the three parts of
mamba_chunk_scan_combined that section 4.4 of the PaddleNLP Kernel
operator-library guide names.  Each pin goes through the separately pinned
oracle_ssd_scan (or numpy), never through the split code:

  * composition: chunk_state -> state_passing -> chunk_scan gives
    oracle_ssd_scan's output and final state, for chunk sizes from one token
    to more than the sequence, with initial states, the step range, packed
    sequences and D per channel;
  * chunk_state: a chunk's end state is oracle_ssd_scan run on that chunk's
    tokens alone from a zero state, and its factor is exp(A * the chunk's
    summed steps) with the softplus written out in numpy; a sequence start
    at any of the chunk's tokens, the first included, makes the factor 0;
  * state_passing is affine: the carried states split into the part from
    the initial state and the part from the chunk states;
  * chunk_scan started from the true states at the chunk boundaries (the
    final states of oracle_ssd_scan on each prefix) gives oracle_ssd_scan's
    outputs.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits

TOL = 1e-11


def _close(a, b, tol=TOL):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"max normalised error {err:.3e} > {tol:.1e}"


def _rand(rng, shape, mean=0.0, std=1.0):
    return (rng.standard_normal(shape) * std + mean).astype(np.float32)


def _inputs(rng, b, l, h, p, n, g, io=orc.F32, d_per_channel=False):
    x = _rand(rng, (b, l, h, p))
    dt = _rand(rng, (b, l, h), -1.5, 0.5)
    z = _rand(rng, (b, l, h, p))
    B = _rand(rng, (b, l, g, n))
    C = _rand(rng, (b, l, g, n))
    A = -rng.uniform(0.5, 3.0, h).astype(np.float32)
    D = _rand(rng, (h, p) if d_per_channel else (h,))
    bias = rng.uniform(-0.1, 0.1, h).astype(np.float32)
    init = rng.standard_normal((b, h, p, n))
    if io == orc.BF16:
        x, dt, z, B, C = (f32_to_bf16_bits(a) for a in (x, dt, z, B, C))
    return dict(x=x, dt=dt, z=z, B=B, C=C, A=A, D=D, bias=bias, init=init)


SEQ = np.array([[0, 0, 0, 1, 1, 1, 1, 1, 2, 2, 3, 3, 3], [5, 5, 5, 5, 5, 5, 5, 5, 5, 5, 5, 6, 6]], np.int32)


@pytest.mark.parametrize("chunk", [1, 4, 5, 13, 20])
@pytest.mark.parametrize("opts", ["plain", "init", "limit", "seq", "bf16_all"])
def test_composition_is_the_scan(chunk, opts):
    rng = np.random.default_rng(900 + chunk + 31 * len(opts))
    io = orc.BF16 if opts == "bf16_all" else orc.F32
    t = _inputs(rng, 2, 13, 3, 4, 5, 1 if opts != "bf16_all" else 3, io, d_per_channel=opts == "bf16_all")
    kw = dict(io_dtype=io)
    if opts in ("limit", "bf16_all"):
        kw["dt_limit"] = (0.15, 0.4)
    if opts in ("seq", "bf16_all"):
        kw["seq_idx"] = SEQ
    init = t["init"] if opts in ("init", "seq", "bf16_all") else None
    out, fin = orc.ssd_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["z"], t["bias"], True,
                            initial_states=init, **kw)
    states, decays = orc.ssd_chunk_state(t["x"], t["dt"], t["A"], t["B"], chunk, t["bias"], True, **kw)
    carried, fin2 = orc.ssd_state_passing(states, decays, init)
    out3, fin3 = orc.ssd_chunk_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], carried, chunk, t["D"], t["z"],
                                    t["bias"], True, **kw)
    _close(out3, out)
    _close(fin2, fin)
    _close(fin3, fin)


def _softplus(v):
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def test_chunk_state_is_the_chunk_alone_from_zero():
    rng = np.random.default_rng(930)
    t = _inputs(rng, 2, 13, 3, 4, 5, 1)
    chunk = 5
    states, decays = orc.ssd_chunk_state(t["x"], t["dt"], t["A"], t["B"], chunk, t["bias"], True)
    for c in range(3):
        sl = slice(c * chunk, min(13, (c + 1) * chunk))
        sub = {k: np.ascontiguousarray(t[k][:, sl]) for k in ("x", "dt", "z", "B", "C")}
        _, fin = orc.ssd_scan(sub["x"], sub["dt"], t["A"], sub["B"], sub["C"], None, None, t["bias"], True)
        _close(states[c], fin)
        steps = _softplus(t["dt"][:, sl].astype(np.float64) + t["bias"].astype(np.float64))
        _close(decays[c], np.exp(t["A"].astype(np.float64) * steps.sum(axis=1)))


def test_chunk_state_factor_is_zero_where_a_sequence_starts():
    rng = np.random.default_rng(940)
    t = _inputs(rng, 1, 12, 2, 3, 4, 1)
    chunk = 4
    # sequence starts at token 4 (first token of chunk 1) and token 10 (inside chunk 2)
    sid = np.array([[0, 0, 0, 0, 1, 1, 1, 1, 1, 1, 2, 2]], np.int32)
    _, decays = orc.ssd_chunk_state(t["x"], t["dt"], t["A"], t["B"], chunk, t["bias"], True, seq_idx=sid)
    assert np.all(decays[0] > 0)
    assert np.all(decays[1] == 0.0) and np.all(decays[2] == 0.0)
    _, dec_plain = orc.ssd_chunk_state(t["x"], t["dt"], t["A"], t["B"], chunk, t["bias"], True)
    _close(decays[0], dec_plain[0])


def test_state_passing_is_affine():
    rng = np.random.default_rng(950)
    nc, b, h, p, n = 5, 2, 3, 2, 4
    states = rng.standard_normal((nc, b, h, p, n))
    decays = rng.uniform(0.0, 1.0, (nc, b, h))
    decays[2, 0, 1] = 0.0
    init = rng.standard_normal((b, h, p, n))
    car, fin = orc.ssd_state_passing(states, decays, init)
    car_s, fin_s = orc.ssd_state_passing(states, decays, None)
    car_i, fin_i = orc.ssd_state_passing(np.zeros_like(states), decays, init)
    _close(car, car_s + car_i)
    _close(fin, fin_s + fin_i)
    _close(car[0], init)
    # behind a zero factor nothing of the initial state is left
    assert np.all(car_i[3:, 0, 1] == 0.0)


def test_chunk_scan_from_the_true_boundary_states():
    rng = np.random.default_rng(960)
    t = _inputs(rng, 2, 13, 3, 4, 5, 1)
    chunk = 4
    nc = 4
    carried = np.empty((nc, 2, 3, 4, 5))
    carried[0] = t["init"]
    for c in range(1, nc):
        pre = {k: np.ascontiguousarray(t[k][:, :c * chunk]) for k in ("x", "dt", "B", "C")}
        _, carried[c] = orc.ssd_scan(pre["x"], pre["dt"], t["A"], pre["B"], pre["C"], None, None, t["bias"], True,
                                     initial_states=t["init"])
    out, fin = orc.ssd_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["z"], t["bias"], True,
                            initial_states=t["init"])
    out2, fin2 = orc.ssd_chunk_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], carried, chunk, t["D"], t["z"],
                                    t["bias"], True)
    _close(out2, out)
    _close(fin2, fin)
