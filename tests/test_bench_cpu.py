"""Host-side checks of bench.py (no GPU): it refuses more than one GPU before
touching the device, its algorithmic byte and operation counts are the ones
the roofline is stated with, and the input digest names the inputs."""
import importlib.util
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_algorithmic_counts_of_the_measured_workloads():
    from state_space_model_scan_amd.inputs import COMPLEX_WORKLOADS, WORKLOADS
    b = _bench()
    w = WORKLOADS["mamba2p8b"]
    e = w.batch * w.dim * w.seqlen
    # u, delta, z, out in bf16; B, C (b, g, n, l) bf16; A fp32; D, bias fp32;
    # last_state fp32
    want = (4 * e * 2 + 2 * w.batch * w.ngroups * w.dstate * w.seqlen * 2
            + w.dim * w.dstate * 4 + 2 * w.dim * 4 + w.batch * w.dim * w.dstate * 4)
    assert b.algorithmic_bytes(w) == want == 678273024
    # per (timestep, state) 4 plain ops + one exp weighing 2 slots; per
    # element 10 plain + 4 transcendentals weighing 2 each
    assert b.TRANS_WEIGHT == 2
    assert b.algorithmic_alu_ops(w) == e * (6 * w.dstate + 18)
    # one plain fp32 wave-instruction per clock per CU: 256 x 64 lanes x 2.4 GHz
    assert abs(b.ALU_PEAK_TOPS - 39.3216) < 1e-9
    wc = COMPLEX_WORKLOADS["mamba2p8b_complex"]
    want_c = (4 * e * 2 + 2 * wc.batch * wc.ngroups * wc.dstate * wc.seqlen * 2 * 2
              + wc.dim * wc.dstate * 8 + 2 * wc.dim * 4 + wc.batch * wc.dim * wc.dstate * 8)
    assert b.complex_algorithmic_bytes(wc) == want_c == 685416448
    assert b.complex_algorithmic_alu_ops(wc) == e * (19 * wc.dstate + 18)


def test_sixteen_bit_io_counts_two_bytes():
    from state_space_model_scan_amd.inputs import F16, WORKLOADS
    b = _bench()
    w = WORKLOADS["mamba2p8b"]
    assert b.algorithmic_bytes(w.scaled(io_dtype=F16)) == b.algorithmic_bytes(w)
    assert b.io_bytes(0) == 4 and b.io_bytes(1) == 2 and b.io_bytes(2) == 2
    assert b.dtype_label(1) == "bf16-io/fp32"


def test_inputs_digest_names_the_inputs():
    from state_space_model_scan_amd.inputs import WORKLOADS, make_inputs
    b = _bench()
    w = WORKLOADS["tiny"]
    t1, t2 = make_inputs(w), make_inputs(w)
    assert b.inputs_digest(t1) == b.inputs_digest(t2)
    t2["delta"] = t2["delta"].copy()
    t2["delta"].flat[5] = np.float32(t2["delta"].flat[5] + 1.0)
    assert b.inputs_digest(t1) != b.inputs_digest(t2)
    assert b.inputs_digest(make_inputs(w, seed=1)) != b.inputs_digest(t1)
