"""GPU parity of causal_conv1d_fwd_ex (seq_idx, initial_states, final states
of causal_conv1d_fn) against the float64 oracle, through the C ABI.

out: |gpu - ref| <= tol * (1 + |ref|) (tol 1e-4 fp32 io, 2e-2 bf16 io);
final states are copies of inputs and must match bit for bit.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import BF16, F32, WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits
from tests.harness import TOL, log, max_err, to_dev

pytestmark = pytest.mark.gpu


def _draw(seed, b, d, l, io):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, d, l)).astype(np.float32)
    init = rng.standard_normal((b, d, 3)).astype(np.float32)
    w = (rng.standard_normal((d, 4)) * 0.5).astype(np.float32)
    bias = rng.standard_normal(d).astype(np.float32)
    if io == BF16:
        x, init = f32_to_bf16_bits(x), f32_to_bf16_bits(init)
    return x, init, w, bias


def _gpu(x, w, bias, io, act, seq=None, init=None, want_final=False):
    import torch
    from state_space_model_scan_amd import binding
    xt = to_dev(x, io)
    fin = None
    if want_final:
        fin = torch.full((x.shape[0], x.shape[1], 3), float("nan"), device="cuda").to(xt.dtype)
    out = binding.causal_conv1d_fwd_ex(xt, to_dev(w, param=True), to_dev(bias, param=True),
                                       seq_idx=None if seq is None else to_dev(seq, param=True),
                                       initial_states=None if init is None else to_dev(init, io),
                                       final_states=fin, act=act)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    f = None if fin is None else fin.float().cpu().numpy().astype(np.float64)
    return o, f


def _vals(a, io):
    return bf16_bits_to_f32(a).astype(np.float64) if io == BF16 else a.astype(np.float64)


@pytest.mark.parametrize("io", [F32, BF16])
@pytest.mark.parametrize("seqlen", [1, 2, 3, 7, 8, 9, 64, 1000])
def test_conv_states(io, seqlen):
    log(f"[conv_ex] states io={io} l={seqlen}")
    x, init, w, bias = _draw(600 + seqlen + io, 2, 24, seqlen, io)
    for use_init in (True, False):
        got, fin = _gpu(x, w, bias, io, orc.ACT_SILU, init=init if use_init else None, want_final=True)
        ref, rfin = orc.causal_conv1d_ex(x, w, bias, orc.ACT_SILU, io_dtype=io,
                                         initial_states=init if use_init else None, want_final=True)
        e = max_err(got, ref)
        assert e <= TOL[io], f"out {e:.3e}"
        np.testing.assert_array_equal(fin, rfin)


@pytest.mark.parametrize("io", [F32, BF16])
@pytest.mark.parametrize("seqlen", [13, 256, 1001])
def test_conv_seq_idx(io, seqlen):
    log(f"[conv_ex] seq_idx io={io} l={seqlen}")
    x, _, w, bias = _draw(620 + seqlen + io, 3, 16, seqlen, io)
    rng = np.random.default_rng(621 + seqlen)
    seq = np.zeros((3, seqlen), np.int32)
    for b in range(3):
        cuts = np.sort(rng.choice(np.arange(1, seqlen), size=min(seqlen - 1, 5 + b * 7), replace=False))
        seq[b] = np.searchsorted(cuts, np.arange(seqlen), side="right")
    got, _ = _gpu(x, w, bias, io, orc.ACT_NONE, seq=seq)
    ref, _ = orc.causal_conv1d_ex(x, w, bias, orc.ACT_NONE, io_dtype=io, seq_idx=seq)
    e = max_err(got, ref)
    assert e <= TOL[io], f"out {e:.3e}"


def test_conv_continuation_on_device():
    """final states of a prefix fed as initial states of the rest reproduce
    the whole sequence (bf16, odd split)."""
    io = BF16
    x, _, w, bias = _draw(640, 2, 32, 300, io)
    full, ffin = _gpu(x, w, bias, io, orc.ACT_SILU, want_final=True)
    k = 131
    o1, f1 = _gpu(np.ascontiguousarray(x[:, :, :k]), w, bias, io, orc.ACT_SILU, want_final=True)
    o2, f2 = _gpu(np.ascontiguousarray(x[:, :, k:]), w, bias, io, orc.ACT_SILU,
                  init=f32_to_bf16_bits(f1.astype(np.float32)), want_final=True)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=2), full)
    np.testing.assert_array_equal(f2, ffin)


def test_conv_seq_idx_full_size_batch_slice():
    """convfixed's conv input (b=16 d=2048 l=4096 bf16) with packed
    sequences through the GPU; the oracle on batch rows 0 and 15."""
    w_ = WORKLOADS["convfixed"]
    log(f"[conv_ex] full size {w_.name}")
    rng = np.random.default_rng(650)
    b, d, l = w_.batch, w_.dim, w_.seqlen
    x = f32_to_bf16_bits(rng.standard_normal((b, d, l), dtype=np.float32))
    w = (rng.standard_normal((d, 4)) * 0.5).astype(np.float32)
    bias = rng.standard_normal(d).astype(np.float32)
    seq = np.zeros((b, l), np.int32)
    for bb in range(b):
        cuts = np.sort(rng.choice(np.arange(1, l), size=40, replace=False))
        seq[bb] = np.searchsorted(cuts, np.arange(l), side="right")
    got, _ = _gpu(x, w, bias, BF16, orc.ACT_SILU, seq=seq)
    for bb in (0, b - 1):
        ref, _ = orc.causal_conv1d_ex(np.ascontiguousarray(x[bb:bb + 1]), w, bias, orc.ACT_SILU, io_dtype=BF16,
                                      seq_idx=np.ascontiguousarray(seq[bb:bb + 1]))
        e = max_err(got[bb:bb + 1], ref)
        assert e <= TOL[BF16], f"batch row {bb}: {e:.3e}"
