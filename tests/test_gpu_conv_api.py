"""GPU checks of the standalone conv, fused-vs-unfused equality, and the
page-signature wrappers."""
import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import BF16, F32, WORKLOADS, make_inputs
from tests.harness import TOL, check, log, max_err, run_gpu, run_oracle, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("io", [F32, BF16])
@pytest.mark.parametrize("act", [orc.ACT_NONE, orc.ACT_SILU])
@pytest.mark.parametrize("shape", [(2, 64, 256), (1, 3, 1), (2, 5, 13), (1, 70, 4099)])
def test_conv_matches_oracle(io, act, shape):
    import torch
    from state_space_model_scan_amd import binding
    rng = np.random.default_rng(sum(shape) + act + 2 * io)
    b, d, l = shape
    xf = rng.standard_normal(shape).astype(np.float32)
    from state_space_model_scan_amd.inputs import f32_to_bf16_bits
    x = f32_to_bf16_bits(xf) if io == BF16 else xf
    w = (rng.standard_normal((d, 4)) * 0.5).astype(np.float32)
    bias = rng.standard_normal(d).astype(np.float32)
    log(f"[conv] io={io} act={act} shape={shape}")
    out = binding.causal_conv1d_fwd(to_dev(x, io), to_dev(w, param=True), to_dev(bias, param=True), act=act)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64).reshape(b * d, l)
    ref = orc.causal_conv1d(x, w, bias, act, io_dtype=io)
    # one fp32 evaluation (error a few ulp of sum |w x| + |bias|, scaled by the
    # activation's slope <= 1.1) then one rounding to the io dtype
    if io == F32:
        mag = orc.causal_conv1d(np.abs(xf), np.abs(w), np.abs(bias), orc.ACT_NONE, io_dtype=F32)
        bound = 8 * 2.0 ** -24 * mag + 1e-30
    else:
        mag = orc.causal_conv1d(f32_to_bf16_bits(np.abs(xf)), np.abs(w), np.abs(bias), orc.ACT_NONE, io_dtype=BF16)
        bound = 8 * 2.0 ** -24 * mag + 2.0 ** -8 * np.abs(ref) + 1e-30
    worst = np.max(np.abs(got - ref) / bound)
    assert worst <= 1.0, f"conv error exceeds its fp32 evaluation bound by {worst:.2f}x"
    assert max_err(got, ref) <= TOL[io]


@pytest.mark.parametrize("io", [F32, BF16])
def test_fused_equals_unfused_bitwise(io):
    """u is rounded to the io dtype in both paths, so fused and unfused agree exactly."""
    import torch
    from state_space_model_scan_amd import binding
    w = WORKLOADS["convfixed"].scaled(batch=2, dim=128, seqlen=520, io_dtype=io)
    t = make_inputs(w)
    log(f"[conv] fused vs unfused io={io}")
    fused, fused_last = run_gpu(w, t)
    u = binding.causal_conv1d_fwd(to_dev(t["conv_x"], io), to_dev(t["conv_weight"], param=True),
                                  to_dev(t["conv_bias"], param=True), act=1)
    torch.cuda.synchronize()
    raw = u.cpu()
    u_np = raw.view(torch.int16).numpy().view(np.uint16) if io == BF16 else raw.numpy()
    t2 = dict(t, u=u_np, conv_x=None, conv_weight=None, conv_bias=None)
    w2 = w.scaled(conv=False)
    unfused, unfused_last = run_gpu(w2, t2)
    np.testing.assert_array_equal(fused, unfused)
    np.testing.assert_array_equal(fused_last, unfused_last)


def test_page_signature_wrappers():
    """selective_scan_fn with 3-D B/C, non-contiguous inputs, return_last_state."""
    import torch
    from state_space_model_scan_amd import selective_scan_fn, conv1d_selective_scan_fn
    w = WORKLOADS["tiny"].scaled(dim=64, seqlen=100, dstate=16)
    t = make_inputs(w)
    ref, ref_last = run_oracle(w, t)
    u = to_dev(t["u"]); delta = to_dev(t["delta"]); z = to_dev(t["z"])
    # non-contiguous views with last stride != 1
    u_nc = u.transpose(1, 2).contiguous().transpose(1, 2)
    B3 = to_dev(t["B"][:, 0]); C3 = to_dev(t["C"][:, 0])
    log("[api] selective_scan_fn")
    out, last = selective_scan_fn(u_nc, delta, to_dev(t["A"], param=True), B3, C3,
                                  to_dev(t["D"], param=True), z, to_dev(t["delta_bias"], param=True),
                                  delta_softplus=True, return_last_state=True)
    torch.cuda.synchronize()
    check(w, out.double().cpu().numpy().reshape(-1, w.seqlen), ref,
          last.double().cpu().numpy().reshape(-1, w.dstate), ref_last, what="selective_scan_fn")
    only = selective_scan_fn(u, delta, to_dev(t["A"], param=True), B3, C3, delta_softplus=True)
    torch.cuda.synchronize()
    assert only.shape == u.shape
    wc = WORKLOADS["convfixed"].scaled(batch=1, dim=64, seqlen=64)
    tc = make_inputs(wc)
    refc, refc_last = run_oracle(wc, tc)
    outc, lastc = conv1d_selective_scan_fn(
        to_dev(tc["conv_x"], BF16), to_dev(tc["conv_weight"], param=True), to_dev(tc["conv_bias"], param=True),
        to_dev(tc["delta"], BF16), to_dev(tc["A"], param=True), to_dev(tc["B"], BF16), to_dev(tc["C"], BF16),
        to_dev(tc["D"], param=True), to_dev(tc["z"], BF16), to_dev(tc["delta_bias"], param=True),
        delta_softplus=True, return_last_state=True, activation="swish")
    torch.cuda.synchronize()
    check(wc, outc.double().cpu().numpy().reshape(-1, wc.seqlen), refc,
          lastc.double().cpu().numpy().reshape(-1, wc.dstate), refc_last, what="conv1d_selective_scan_fn")
    with pytest.raises(NotImplementedError):
        conv1d_selective_scan_fn(to_dev(tc["conv_x"], BF16), to_dev(tc["conv_weight"], param=True), None,
                                 to_dev(tc["delta"], BF16), to_dev(tc["A"], param=True),
                                 to_dev(tc["B"], BF16), to_dev(tc["C"], BF16), activation="relu")
