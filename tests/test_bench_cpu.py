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
    assert b.algorithmic_alu_ops(w) == e * (8 * w.dstate + 26)
    wc = COMPLEX_WORKLOADS["mamba2p8b_complex"]
    want_c = (4 * e * 2 + 2 * wc.batch * wc.ngroups * wc.dstate * wc.seqlen * 2 * 2
              + wc.dim * wc.dstate * 8 + 2 * wc.dim * 4 + wc.batch * wc.dim * wc.dstate * 8)
    assert b.complex_algorithmic_bytes(wc) == want_c == 685416448
    assert b.complex_algorithmic_alu_ops(wc) == e * (25 * wc.dstate + 26)


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
