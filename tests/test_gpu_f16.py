"""GPU parity of the fp16-io paths (ssm_scan_fwd, causal_conv1d_fwd,
causal_conv1d_fwd_ex) against the float64 oracle on the same fp16 bits.
Bar: |gpu - ref| <= 5e-3 * (1 + |ref|) per element (ten binary16 half-ulps)."""
import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import F16, WORKLOADS, f32_to_f16_bits, make_inputs, sample_rows
from tests.harness import TOL, check, conv_flip_slack, log, max_err, run_gpu, run_oracle, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(2, 64, 100, 16), (1, 128, 33, 16), (2, 48, 257, 5), (1, 32, 64, 1)])
@pytest.mark.parametrize("bc", ["varying", "fixed"])
def test_scan_f16(shape, bc):
    b, d, l, n = shape
    w = WORKLOADS["tiny"].scaled(batch=b, dim=d, seqlen=l, dstate=n, io_dtype=F16, bc_kind=bc,
                                 ngroups=2 if bc == "varying" else 1, seed=710 + l + n)
    log(f"[f16] scan {shape} {bc}")
    t = make_inputs(w)
    init = np.random.default_rng(711).standard_normal((b, d, n))
    out, last = run_gpu(w, t, init=init)
    ref, ref_last = run_oracle(w, t, init=init)
    check(w, out, ref, last, ref_last, what=f"f16 {shape} {bc}")


def test_scan_f16_conv_prologue():
    w = WORKLOADS["convfixed"].scaled(batch=2, dim=64, seqlen=300, io_dtype=F16, seed=720)
    log("[f16] scan + conv prologue")
    t = make_inputs(w)
    out, last = run_gpu(w, t)
    ref, ref_last = run_oracle(w, t)
    check(w, out, ref, last, ref_last, what="f16 conv prologue", last_slack=conv_flip_slack(w, t))


def test_scan_f16_mamba130m_sampled_rows():
    w = WORKLOADS["mamba130m"].scaled(io_dtype=F16)
    log("[f16] mamba130m shape")
    t = make_inputs(w)
    out, last = run_gpu(w, t)
    rows = sample_rows(w, 48)
    ref, ref_last = run_oracle(w, t, rows=rows)
    check(w, out[rows], ref, last[rows], ref_last, what="f16 mamba130m")


@pytest.mark.parametrize("seqlen", [1, 5, 64, 1000])
def test_conv_f16(seqlen):
    import torch
    from state_space_model_scan_amd import binding
    log(f"[f16] conv l={seqlen}")
    rng = np.random.default_rng(730 + seqlen)
    b, d = 2, 40
    x = f32_to_f16_bits(rng.standard_normal((b, d, seqlen)).astype(np.float32))
    init = f32_to_f16_bits(rng.standard_normal((b, d, 3)).astype(np.float32))
    wt = (rng.standard_normal((d, 4)) * 0.5).astype(np.float32)
    bias = rng.standard_normal(d).astype(np.float32)
    xt = to_dev(x, F16)
    out = binding.causal_conv1d_fwd(xt, to_dev(wt, param=True), to_dev(bias, param=True), act=orc.ACT_SILU)
    fin = torch.empty((b, d, 3), dtype=torch.float16, device="cuda")
    out2 = binding.causal_conv1d_fwd_ex(xt, to_dev(wt, param=True), to_dev(bias, param=True),
                                        initial_states=to_dev(init, F16), final_states=fin, act=orc.ACT_SILU)
    torch.cuda.synchronize()
    ref = orc.causal_conv1d(x, wt, bias, orc.ACT_SILU, io_dtype=orc.F16).reshape(b, d, seqlen)
    e = max_err(out.float().cpu().numpy().astype(np.float64), ref)
    assert e <= TOL[F16], f"conv {e:.3e}"
    ref2, rfin = orc.causal_conv1d_ex(x, wt, bias, orc.ACT_SILU, io_dtype=orc.F16, initial_states=init,
                                      want_final=True)
    e2 = max_err(out2.float().cpu().numpy().astype(np.float64), ref2)
    assert e2 <= TOL[F16], f"conv_ex {e2:.3e}"
    np.testing.assert_array_equal(fin.float().cpu().numpy().astype(np.float64), rfin)
