"""Pins for the oracle's fp16 io (IEEE binary16): decoding and rounding
against numpy's float16 (an independent implementation, round to nearest,
ties to even), and the scan on fp16 io equal to the scan on fp32 io of the
same values."""
import numpy as np

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import WORKLOADS, f16_bits_to_f32, f32_to_f16_bits, make_inputs


def test_decode_every_bit_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_bits_to_double(int(b)) for b in bits])
    finite = np.isfinite(want)
    np.testing.assert_array_equal(got[finite], want[finite])
    assert np.all(np.isinf(got[np.isinf(want)]))
    assert np.all(np.isnan(got[np.isnan(want)]))


def test_rounding_matches_numpy():
    rng = np.random.default_rng(700)
    # wide magnitudes, subnormals, exact ties between neighbours, overflow
    v = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 6, 4000),
        (np.arange(1, 2000) + 0.5) * 2.0 ** -24,                     # subnormal ties
        (1024 + np.arange(0, 1000) + 0.5) * 2.0 ** -10,              # ties in [1, 2)
        np.array([65504.0, 65519.0, 65520.0, 70000.0, -65520.0, 2.0 ** -25, 2.0 ** -26, 0.0, -0.0]),
    ])
    want = v.astype(np.float16).astype(np.float64)     # numpy rounds from double directly
    got = np.array([orc.round_f16(x) for x in v])
    np.testing.assert_array_equal(got, want)


def test_scan_f16_io_equals_f32_io_of_the_same_values():
    w = WORKLOADS["tiny"].scaled(batch=2, dim=8, seqlen=40, dstate=4, ngroups=2)
    t = make_inputs(w)
    t16 = dict(t)
    t32 = dict(t)
    for k in ("u", "delta", "z", "B", "C"):
        t16[k] = f32_to_f16_bits(t[k])
        t32[k] = f16_bits_to_f32(t16[k])
    init = np.random.default_rng(701).standard_normal((2, 8, 4))
    args = dict(ngroups=2, initial_state=init)
    o16, l16 = orc.selective_scan(t16["u"], t16["delta"], t["A"], t16["B"], t16["C"], t["D"], t16["z"],
                                  t["delta_bias"], True, io_dtype=orc.F16, **args)
    o32, l32 = orc.selective_scan(t32["u"], t32["delta"], t["A"], t32["B"], t32["C"], t["D"], t32["z"],
                                  t["delta_bias"], True, io_dtype=orc.F32, **args)
    np.testing.assert_array_equal(o16, o32)
    np.testing.assert_array_equal(l16, l32)
    # the fused conv prologue rounds u to fp16
    cw = np.random.default_rng(702).standard_normal((8, 4)).astype(np.float32)
    cb = np.random.default_rng(703).standard_normal(8).astype(np.float32)
    oc, _ = orc.selective_scan(None, t16["delta"], t["A"], t16["B"], t16["C"], None, None, None, True,
                               io_dtype=orc.F16, ngroups=2, conv_x=t16["u"], conv_weight=cw, conv_bias=cb)
    u = orc.causal_conv1d(t16["u"], cw, cb, orc.ACT_SILU, io_dtype=orc.F16)
    u16 = np.array([orc.round_f16(x) for x in u.ravel()]).reshape(2, 8, 40)
    ou, _ = orc.selective_scan(f32_to_f16_bits(u16.astype(np.float32)), t16["delta"], t["A"], t16["B"], t16["C"],
                               None, None, None, True, io_dtype=orc.F16, ngroups=2)
    np.testing.assert_array_equal(oc, ou)
