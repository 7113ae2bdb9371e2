"""Pins for the oracle's causal_conv1d with its optional inputs
(oracle_causal_conv1d_ex): seq_idx, initial_states and the final states of
causal_conv1d_fn (PaddleNLP Kernel operator-library guide, section 4.2).
Each pin goes through the plain conv oracle (pinned in test_oracle_pins.py)
and numpy slicing only:

  * no optional input: the plain conv;
  * initial states: the plain conv of the inputs with the initial states
    prepended, its first width-1 outputs dropped;
  * final states: the last width-1 values of that prepended sequence,
    bit for bit (also when seqlen < width-1);
  * split continuation: final states of a prefix fed as initial states of
    the rest reproduce the whole sequence;
  * seq_idx: equal ids change nothing; packed sequences give, segment by
    segment, the plain conv of each segment alone.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import f32_to_bf16_bits, bf16_bits_to_f32


def _x(rng, shape, io):
    a = rng.standard_normal(shape).astype(np.float32)
    return f32_to_bf16_bits(a) if io == orc.BF16 else a


def _plain(x, w, bias, act, io):
    b, d, l = x.shape
    out = orc.causal_conv1d(x, w, bias, act, io_dtype=io)
    return out.reshape(b, d, l)


def _vals(a, io):
    return bf16_bits_to_f32(a).astype(np.float64) if io == orc.BF16 else a.astype(np.float64)


@pytest.mark.parametrize("io", [orc.F32, orc.BF16])
@pytest.mark.parametrize("width", [2, 3, 4])
def test_no_options_is_the_plain_conv(io, width):
    rng = np.random.default_rng(400 + width + io)
    x = _x(rng, (2, 3, 17), io)
    w = rng.standard_normal((3, width)).astype(np.float32)
    bias = rng.standard_normal(3).astype(np.float32)
    out, fin = orc.causal_conv1d_ex(x, w, bias, orc.ACT_SILU, io_dtype=io)
    np.testing.assert_array_equal(out, _plain(x, w, bias, orc.ACT_SILU, io))
    assert fin is None


@pytest.mark.parametrize("io", [orc.F32, orc.BF16])
@pytest.mark.parametrize("seqlen", [1, 2, 3, 9])
def test_initial_and_final_states(io, seqlen):
    rng = np.random.default_rng(410 + seqlen + io)
    b, d, W = 2, 3, 4
    x = _x(rng, (b, d, seqlen), io)
    init = _x(rng, (b, d, W - 1), io)
    w = rng.standard_normal((d, W)).astype(np.float32)
    bias = rng.standard_normal(d).astype(np.float32)
    out, fin = orc.causal_conv1d_ex(x, w, bias, orc.ACT_NONE, io_dtype=io, initial_states=init,
                                    want_final=True)
    ext = np.ascontiguousarray(np.concatenate([init, x], axis=2))
    want = _plain(ext, w, bias, orc.ACT_NONE, io)[:, :, W - 1:]
    np.testing.assert_allclose(out, want, rtol=1e-15, atol=1e-15)
    np.testing.assert_array_equal(fin, _vals(ext[:, :, -(W - 1):], io))
    # without initial states the final states are the last inputs, zero-padded
    _, fin0 = orc.causal_conv1d_ex(x, w, bias, orc.ACT_NONE, io_dtype=io, want_final=True)
    pad = np.concatenate([np.zeros((b, d, W - 1)), _vals(x, io)], axis=2)
    np.testing.assert_array_equal(fin0, pad[:, :, -(W - 1):])


def test_split_continuation_through_states():
    rng = np.random.default_rng(420)
    b, d, l, W = 1, 4, 23, 4
    x = _x(rng, (b, d, l), orc.F32)
    w = rng.standard_normal((d, W)).astype(np.float32)
    full, fin = orc.causal_conv1d_ex(x, w, None, orc.ACT_SILU, want_final=True)
    for k in (1, 2, 5, 11):
        o1, f1 = orc.causal_conv1d_ex(np.ascontiguousarray(x[:, :, :k]), w, None, orc.ACT_SILU,
                                      want_final=True)
        o2, f2 = orc.causal_conv1d_ex(np.ascontiguousarray(x[:, :, k:]), w, None, orc.ACT_SILU,
                                      initial_states=f1.astype(np.float32), want_final=True)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), full, rtol=1e-15, atol=1e-15)
        np.testing.assert_array_equal(f2, fin)


@pytest.mark.parametrize("io", [orc.F32, orc.BF16])
def test_seq_idx_packed_sequences(io):
    rng = np.random.default_rng(430 + io)
    b, d, W = 2, 3, 4
    lens = [[5, 1, 7, 3], [2, 14]]
    l = 16
    x = _x(rng, (b, d, l), io)
    w = rng.standard_normal((d, W)).astype(np.float32)
    bias = rng.standard_normal(d).astype(np.float32)
    seq = np.zeros((b, l), np.int32)
    for bb, ls in enumerate(lens):
        seq[bb] = np.repeat(np.arange(len(ls)), ls)
    out, _ = orc.causal_conv1d_ex(x, w, bias, orc.ACT_SILU, io_dtype=io, seq_idx=seq)
    for bb, ls in enumerate(lens):
        start = 0
        for n in ls:
            seg = np.ascontiguousarray(x[bb:bb + 1, :, start:start + n])
            want = _plain(seg, w, bias, orc.ACT_SILU, io)
            np.testing.assert_allclose(out[bb:bb + 1, :, start:start + n], want, rtol=1e-15, atol=1e-15)
            start += n
    # one id everywhere changes nothing
    same, _ = orc.causal_conv1d_ex(x, w, bias, orc.ACT_SILU, io_dtype=io,
                                   seq_idx=np.full((b, l), 7, np.int32))
    np.testing.assert_array_equal(same, _plain(x, w, bias, orc.ACT_SILU, io))
