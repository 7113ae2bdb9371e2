"""Benchmark of the selective-scan forward (ssm_scan_fwd) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one ssm_scan_fwd call over the whole workload (discretisation,
recurrence, contraction, D skip, gate, last_state -- and the conv prologue for
the workload that has one), with every input already resident in HBM.  W
untimed steps, then K steps timed between two device synchronisations.  Prints
one JSON line.

Default workload: mamba2p8b (b=8, d=5120, l=2048, n=16, g=4, bf16 io, fp32
state), the Mamba-2.8B-shaped layer the throughput target is quoted on.

Roofline of the scan kernel (the only kernel of that workload), the metric's
own: bound "hbm", achieved = algorithmic bytes (every input read once, every
output written once) / launch time, against 8 TB/s.  The ALU figures sit
beside it as flat keys (alu_*), from the rates `--microbench` measures:
  * one plain fp32 VALU wave-instruction per clock per compute unit (4 SIMDs
    x 16 lanes; the build turns packed FP32 off), so the peak is 256 CUs x 64
    lanes x 2.4 GHz = 39.3 T lane-ops/s;
  * v_exp_f32 (and log, rcp) at half that rate, so a transcendental weighs 2.
  The method needs, per (timestep, state), 4 plain ops (delta'*A, delta'u*B,
  state FMA, C.x FMA) and one exp; per element 10 plain ops and 4
  transcendentals (softplus: exp, log; silu: exp, rcp): ops = E * (6 n + 18).
The launch time is measured live with HIP events on the stream the kernel runs
on.  `traffic` (HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE,
scaled by the same counters on a copy of known size) is read from
profiles/traffic_<workload>.json when that file was taken from the current
kernel source, else null.

cpu_baseline: the float64 oracle (test infrastructure) timed on this host's
cores over a bounded sample of the workload's rows, scaled to elements/s,
with a single-thread figure on a slice of those rows beside it.  Before the
warm-up, 20 launches each follow a 512 MiB write that evicts the caches
(outside their timed pair): roofline.kernel_avg_ms_cold_caches.
config.inputs_sha256 digests every input tensor.

Standalone conv (--conv): a step is one causal_conv1d_fwd (width 4, silu) on
the conv workload's input; the roofline is HBM (x read and out written once,
plus the weights).

Complex-A workloads (--workload mamba2p8b_complex): a step is one
ssm_scan_fwd_complex call (complex A, B and C; real u, delta, z, out).  The
value is elements/s; the roofline is ALU with 19 weighted ops per (timestep,
state) -- 13 plain ops and exp2, sine and cosine weighted 2 -- plus the 18 per
element of the real scan, and the HBM rate beside it.

Decode workloads (--workload decode2p8b): a step is one decode step of one
layer, causal_conv1d_update (one new token against the conv cache) then
ssm_state_update (one timestep against the cached fp32 state), both in place.
The value is channel-steps/s (b*d per step); the roofline is HBM for the
state update, the dominant kernel: the state read and written once, x, dt,
z, out, B, C once, A/D/dt_bias once (d*n*4 + 2*d*4 bytes, shared by the
batch), against 8 TB/s.

Backward (--backward, with a selective-scan workload): a step is one
ssm_scan_bwd call (every input gradient: du, ddelta, dz, dA, dB, dC, dD,
d(delta_bias)) from the checkpoints a forward call wrote before timing.  The
value is elements/s (b*d*l).  The roofline is the VALU rate (bwd_alu_ops per
step over the step's event time, which brackets the backward kernel and the
short partial-sum kernels after it), with the HBM rate of the algorithmic
bytes beside it.

Mamba-2 workloads (--workload ssd2p7b): a step is one ssd_scan_fwd call.
The value is elements/s (b*l*h*p).  The roofline is HBM (x, z, out, dt, B, C
read or written once, plus the small per-head vectors), with the matrix-core
rate beside it: the chunked form's minimal work per (chunk, head) is
Q^2 n / 2 + Q^2 p / 2 + 2 Q p n multiply-adds (causal halves of C B^T and
M X, then C S^T and the state update), against 2.5 PFLOP/s bf16.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "selective-scan fwd elements/s (b·d·l) and HBM GB/s as % of MI355X peak"
HBM_PEAK_GBS = 8000.0
# one plain fp32 VALU wave-instruction per clock per CU (measured 0.94 at 8
# waves per SIMD by --microbench; packed FP32 is off): 39.32 T lane-ops/s
ALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
TRANS_WEIGHT = 2     # v_exp_f32 / v_log_f32 / v_rcp_f32 issue at half the plain rate (--microbench)


def io_bytes(io_dtype: int) -> int:
    """Bytes of one io element: fp32 4, bf16 and fp16 2."""
    return 4 if io_dtype == 0 else 2


def dtype_label(io_dtype: int) -> str:
    """io dtype and arithmetic: the state and every operation are fp32."""
    return {0: "fp32", 1: "bf16-io/fp32", 2: "fp16-io/fp32"}[io_dtype]
CSRC = os.path.join(ROOT, "state_space_model_scan_amd", "csrc")
KERNEL_SRCS = ("scan_kernel.h", "device_util.h", "scan_bf16.hip", "scan_f32.hip", "ssm_scan.hip")
DECODE_SRCS = ("decode.hip", "device_util.h")
SSD_SRCS = ("ssd.hip", "device_util.h")
BWD_SRCS = ("bwd.hip", "device_util.h")
CBWD_SRCS = ("bwd_complex.hip", "complex_util.h", "device_util.h")
COMPLEX_SRCS = ("scan_complex.hip", "complex_util.h", "scan_kernel.h", "device_util.h")
CONV_SRCS = ("ssm_scan.hip", "device_util.h")
MFMA_BF16_PEAK_TFLOPS = 2500.0


def algorithmic_bytes(w) -> int:
    """Every input read once, every output written once (the fused minimum for
    the conv workload: the conv input replaces u, u never touches memory)."""
    es = io_bytes(w.io_dtype)
    E = w.elements
    n = w.dstate
    io_tensors = 2 + (1 if w.has_z else 0) + 1          # u or conv x, delta, z, out
    total = io_tensors * E * es
    bc = 2 * (w.dim * n if w.bc_kind == "fixed" else w.batch * w.ngroups * n * w.seqlen) * es
    params = w.dim * n * 4 + (w.dim * 4 if w.has_D else 0) + (w.dim * 4 if w.has_bias else 0)
    if w.conv:
        params += w.dim * 4 * 4 + w.dim * 4
    last = w.batch * w.dim * n * 4
    return total + bc + params + last


def algorithmic_alu_ops(w) -> float:
    """Per (timestep, state) 4 plain + 1 exp, per element 10 plain + 4
    transcendentals; a transcendental weighs TRANS_WEIGHT plain slots."""
    return float(w.elements) * ((4 + TRANS_WEIGHT) * w.dstate + 10 + 4 * TRANS_WEIGHT)


def settle(step, seconds: float = 0.2) -> None:
    """Untimed launches for a fixed wall time before any measurement, so the
    GPU's clocks have ramped up under load however few warm-up steps are
    asked for (with 5, the first timed launches ran 15-25% slow)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


def kernel_sha(srcs=KERNEL_SRCS) -> str:
    h = hashlib.sha256()
    for name in srcs:
        h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def load_traffic(name: str, srcs=KERNEL_SRCS):
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sha256") != kernel_sha(srcs):
        return None
    return rec.get("traffic_bytes")


def decode_state_update_bytes(w) -> int:
    es = io_bytes(w.io_dtype)
    bd = w.batch * w.dim
    state = 2 * bd * w.dstate * 4
    vecs = (3 + (1 if w.has_z else 0)) * bd * es            # x, dt, out (+ z)
    bc = 2 * w.batch * w.ngroups * w.dstate * es
    params = w.dim * w.dstate * 4 + (w.dim * 4 if w.has_D else 0) + (w.dim * 4 if w.has_bias else 0)
    return state + vecs + bc + params


def decode_conv_update_bytes(w) -> int:
    es = io_bytes(w.io_dtype)
    bd = w.batch * w.dim
    return (2 * bd * w.conv_tokens * es + 2 * bd * w.conv_state_len * es
            + w.dim * w.conv_width * 4 + w.dim * 4)


def cpu_model() -> str:
    """The host CPU's model string (Linux), or the platform's processor name."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def inputs_digest(t) -> str:
    """SHA-256 over every input tensor's bytes, in name order (absent ones
    skipped): names the exact synthetic inputs the line was measured on."""
    h = hashlib.sha256()
    for k in sorted(t):
        if t[k] is not None:
            h.update(k.encode())
            h.update(np.ascontiguousarray(t[k]).view(np.uint8))
    return h.hexdigest()


def cpu_baseline(w, t, budget_s: float):
    """Oracle throughput on a bounded sample of rows (all host threads)."""
    from oracle import oracle as orc
    from tests.harness import run_oracle
    threads = orc.max_threads()
    total_rows = w.batch * w.dim
    rng = np.random.default_rng(0)
    # calibrate (the first call also loads the oracle library): grow the probe
    # until it takes a measurable time, then size the sample for ~budget_s
    n = min(total_rows, max(threads, 16))
    while True:
        probe = np.sort(rng.choice(total_rows, size=n, replace=False))
        t0 = time.perf_counter()
        run_oracle(w, t, rows=probe, nthreads=threads)
        dt = time.perf_counter() - t0
        if dt >= 0.5 or n == total_rows:
            break
        n = min(total_rows, 4 * n)
    per_row = dt / len(probe)
    nrows = int(min(total_rows, max(len(probe), budget_s / max(per_row, 1e-9))))
    rows = np.sort(rng.choice(total_rows, size=nrows, replace=False))
    t0 = time.perf_counter()
    run_oracle(w, t, rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    # one thread on a slice of the same rows, as a per-core figure
    one = rows[: max(1, min(len(rows), int(len(rows) * 2.0 / max(dt * threads, 1e-9))))]
    t1 = time.perf_counter()
    run_oracle(w, t, rows=one, nthreads=1)
    dt1 = time.perf_counter() - t1
    return {"value": nrows * w.seqlen / dt, "unit": "elements/s", "cores": threads,
            "single_thread_value": len(one) * w.seqlen / dt1,
            "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{nrows} of {total_rows} (b,d) rows x full seqlen {w.seqlen}, "
                      f"{dt:.1f} s float64 on {threads} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="mamba2p8b")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch one 512 MiB device copy (for rocprofv3 counter scaling)")
    ap.add_argument("--conv", action="store_true",
                    help="time the standalone causal_conv1d_fwd on the conv workload's input")
    ap.add_argument("--backward", action="store_true",
                    help="time ssm_scan_bwd (all gradients) on the selective-scan workload")
    ap.add_argument("--split", action="store_true",
                    help="Mamba-2 workload: time ssd_chunk_state, ssd_state_passing and ssd_chunk_scan in turn")
    ap.add_argument("--chunk-size", type=int, default=256,
                    help="chunk size of --split (a multiple of 64; 256 is the usual Mamba-2 value)")
    ap.add_argument("--microbench", action="store_true",
                    help="measure the VALU, transcendental, LDS and copy rates the ALU ceilings use")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the operator shards with no communication along batch and channels", file=sys.stderr)
        sys.exit(2)

    if args.microbench:
        return microbench_main(args)
    import torch
    from state_space_model_scan_amd import _lib, binding
    from state_space_model_scan_amd.inputs import BF16, DECODE_WORKLOADS, WORKLOADS, make_inputs
    if args.workload in DECODE_WORKLOADS:
        return decode_main(args)
    from state_space_model_scan_amd.inputs import SSD_WORKLOADS
    if args.workload in SSD_WORKLOADS:
        return ssd_main(args)
    from state_space_model_scan_amd.inputs import COMPLEX_WORKLOADS
    if args.backward:
        return complex_bwd_main(args) if args.workload in COMPLEX_WORKLOADS else bwd_main(args)
    if args.conv:
        return conv_main(args)
    if args.workload in COMPLEX_WORKLOADS:
        return complex_main(args)

    def to_dev(a, io_dtype, param=False):
        x = torch.from_numpy(np.ascontiguousarray(a))
        if not param and io_dtype == BF16 and a.dtype == np.uint16:
            x = x.view(torch.bfloat16)
        return x.cuda()

    _lib.lib()  # fail loudly when the HIP library is missing
    w = WORKLOADS[args.workload]
    t = make_inputs(w)
    io = w.io_dtype
    dev = {k: (to_dev(v, io, param=k in ("A", "D", "delta_bias", "conv_weight", "conv_bias"))
               if v is not None else None) for k, v in t.items()}
    out = torch.empty_like(dev["delta"])
    last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device="cuda")
    conv = {}
    if w.conv:
        conv = dict(conv_x=dev["conv_x"], conv_weight=dev["conv_weight"], conv_bias=dev["conv_bias"])

    def step():
        binding.ssm_scan_fwd(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"],
                             dev["delta_bias"], w.softplus, out=out, last_state=last, **conv)

    plan = binding.ssm_scan_plan(dev["u"], dev["delta"], dev["A"], dev["B"], dev["C"], dev["D"], dev["z"],
                                 dev["delta_bias"], w.softplus, out=out, last_state=last, **conv)
    if plan["segments"] > 1:
        kernel = "scan_kernel (state pass + full pass)"
    elif plan["eight_lane_waves"]:
        kernel = "scan_mix_kernel"
    else:
        kernel = "scan_kernel"

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    # the clocks settle under load whatever W is: 0.2 s of untimed launches
    settle(step)
    # launches from cold caches: each after a 512 MiB write (outside the timed
    # pair) that evicts L2 and the last-level cache
    evict = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold_ms = []
    for i in range(20):
        evict.fill_(i & 0xff)
        s_ev, e_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_ev.record(stream)
        step()
        e_ev.record(stream)
        torch.cuda.synchronize()
        cold_ms.append(s_ev.elapsed_time(e_ev))
    del evict

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_launch_s = float(np.mean(launch_ms)) / 1e3
    ms_per_step = wall * 1e3 / args.steps
    elems = w.elements
    value = elems * args.steps / wall

    abytes = algorithmic_bytes(w)
    aops = algorithmic_alu_ops(w)
    alu_tops = aops / avg_launch_s / 1e12
    hbm_gbs = abytes / avg_launch_s / 1e9
    traffic = load_traffic(w.name)
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_label(io),
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: b={w.batch} d={w.dim} l={w.seqlen} n={w.dstate} g={w.ngroups} "
                        f"B/C {w.bc_kind}, {dtype_label(io)} (io/state), "
                        f"{'conv prologue, ' if w.conv else ''}{'z gate' if w.has_z else 'no z'}",
            "io_dtype": {0: "fp32", 1: "bf16", 2: "fp16"}[io],
            "state_dtype": "fp32",
            "elements_per_step": elems,
            "inputs_sha256": inputs_digest(t),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": hbm_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": hbm_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes": abytes,
            "kernel": kernel,
            "plan": plan,
            "kernel_avg_ms": avg_launch_s * 1e3,
            "kernel_median_ms": float(np.median(launch_ms)),
            "kernel_min_ms": float(np.min(launch_ms)),
            "kernel_avg_ms_cold_caches": float(np.mean(cold_ms)),
            "alu_achieved_tops": alu_tops,
            "alu_peak_tops": ALU_PEAK_TOPS,
            "alu_frac": alu_tops / ALU_PEAK_TOPS,
            "alu_ops_per_element": (4 + TRANS_WEIGHT) * w.dstate + 10 + 4 * TRANS_WEIGHT,
            "alu_trans_weight": TRANS_WEIGHT,
        },
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, t, args.cpu_budget)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)



def complex_algorithmic_bytes(w) -> int:
    """Every input read once and every output written once: u, delta, z, out
    (b, d, l) io; complex B, C (pairs) io; A (d, n, 2), D, delta_bias fp32;
    last_state (b, d, n, 2) fp32."""
    es = 2 if w.io_dtype in (1, 2) else 4
    e = w.batch * w.dim * w.seqlen
    vecs = (3 + (1 if w.has_z else 0)) * e * es
    per_bc = (w.dim * w.dstate * 2 if w.bc_kind == "fixed"
              else w.batch * w.ngroups * w.dstate * w.seqlen * 2) * es
    params = w.dim * w.dstate * 8 + (w.dim * 4 if w.has_D else 0) + (w.dim * 4 if w.has_bias else 0)
    return vecs + 2 * per_bc + params + w.batch * w.dim * w.dstate * 8


def complex_algorithmic_alu_ops(w) -> float:
    """Per (timestep, state): delta' times Re A and Im A, the fraction of the
    phase, the decay's two products, B's two products with delta' u, four
    FMAs of the complex state update and two of Re(C.x) (13 plain ops), plus
    exp2, sine and cosine, each weighted TRANS_WEIGHT; per element the 10
    plain ops and 4 transcendentals of the real scan (softplus, gate, D)."""
    return float(w.elements) * ((13 + 3 * TRANS_WEIGHT) * w.dstate + 10 + 4 * TRANS_WEIGHT)


def complex_main(args):
    """One ssm_scan_fwd_complex launch per timed step."""
    import torch
    from state_space_model_scan_amd import _lib, binding
    from state_space_model_scan_amd.inputs import BF16, COMPLEX_WORKLOADS, F16, make_complex_inputs

    _lib.lib()
    w = COMPLEX_WORKLOADS[args.workload]
    t = make_complex_inputs(w)
    io = w.io_dtype

    def dev(a, param=False):
        if a is None:
            return None
        x = torch.from_numpy(np.ascontiguousarray(a))
        if not param and io in (BF16, F16) and a.dtype == np.uint16:
            x = x.view(torch.bfloat16 if io == BF16 else torch.float16)
        return x.cuda()

    u, delta, z, B, C = dev(t["u"]), dev(t["delta"]), dev(t["z"]), dev(t["B"]), dev(t["C"])
    A, D, bias = dev(t["A"], True), dev(t["D"], True), dev(t["delta_bias"], True)
    init = dev(t["initial_state"], True)
    out = torch.empty_like(delta)
    last = torch.empty((w.batch, w.dim, w.dstate, 2), dtype=torch.float32, device="cuda")

    def step():
        binding.ssm_scan_fwd_complex(u, delta, A, B, C, D, z, bias, w.softplus, out=out, last_state=last,
                                     initial_state=init)

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)]
    avg_launch_s = float(np.mean(launch_ms)) / 1e3
    abytes = complex_algorithmic_bytes(w)
    alu_tops = complex_algorithmic_alu_ops(w) / avg_launch_s / 1e12
    hbm_gbs = abytes / avg_launch_s / 1e9
    iot = {0: "fp32", 1: "bf16", 2: "fp16"}[io]
    rec = {
        "metric": METRIC, "value": w.elements * args.steps / wall, "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: b={w.batch} d={w.dim} l={w.seqlen} n={w.dstate} g={w.ngroups} "
                               f"complex A/B/C, B/C {w.bc_kind}, {iot} io, fp32 complex state"
                               f"{', z gate' if w.has_z else ''}",
                   "io_dtype": iot, "elements_per_step": w.elements},
        "roofline": {
            "bound": "alu", "achieved": alu_tops, "peak": ALU_PEAK_TOPS,
            "unit": "T fp32 VALU lane-ops/s (transcendental weighted 2)", "frac": alu_tops / ALU_PEAK_TOPS,
            "traffic": load_traffic(w.name, COMPLEX_SRCS),
            "kernel_avg_ms": avg_launch_s * 1e3, "kernel_median_ms": float(np.median(launch_ms)),
            "kernel_min_ms": float(np.min(launch_ms)),
            "hbm": {"achieved_GBs": hbm_gbs, "peak_GBs": HBM_PEAK_GBS, "frac": hbm_gbs / HBM_PEAK_GBS,
                    "algorithmic_bytes": abytes},
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = complex_cpu_baseline(w, t, args.cpu_budget)
    print(json.dumps(rec), flush=True)


def complex_cpu_baseline(w, t, budget_s: float):
    """The oracle's complex scan on a bounded sample of rows (all host threads)."""
    from oracle import oracle as orc
    threads = orc.max_threads()
    total_rows = w.batch * w.dim
    rng = np.random.default_rng(0)
    kind = orc.BC_FIXED if w.bc_kind == "fixed" else orc.BC_VARYING
    init = None if t["initial_state"] is None else t["initial_state"].astype(np.float64)

    def run(rows):
        orc.selective_scan_complex(t["u"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["z"],
                                   t["delta_bias"], w.softplus, io_dtype=w.io_dtype, ngroups=w.ngroups,
                                   B_kind=kind, C_kind=kind, initial_state=init, rows=rows,
                                   nthreads=threads)

    n = min(total_rows, max(threads, 16))
    while True:
        probe = np.sort(rng.choice(total_rows, size=n, replace=False))
        t0 = time.perf_counter()
        run(probe)
        dt = time.perf_counter() - t0
        if dt >= 0.5 or n == total_rows:
            break
        n = min(total_rows, 4 * n)
    nrows = int(min(total_rows, max(len(probe), budget_s / max(dt / len(probe), 1e-9))))
    rows = np.sort(rng.choice(total_rows, size=nrows, replace=False))
    t0 = time.perf_counter()
    run(rows)
    dt = time.perf_counter() - t0
    return {"value": nrows * w.seqlen / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "sample": f"{nrows} of {total_rows} (b,d) rows x full seqlen {w.seqlen}, "
                      f"{dt:.1f} s float64 complex scan on {threads} threads"}


def conv_main(args):
    """One standalone causal_conv1d_fwd per timed step (width 4, silu) on the
    conv input of the workload (convfixed by default: b=16 d=2048 l=4096
    bf16).  HBM-bound: x read once and out written once, plus the weights."""
    import torch
    from state_space_model_scan_amd import _lib, binding
    from state_space_model_scan_amd.inputs import BF16, F16, WORKLOADS, make_inputs

    _lib.lib()
    name = args.workload if args.workload != "mamba2p8b" else "convfixed"
    w = WORKLOADS[name]
    if not w.conv:
        raise SystemExit(f"--conv needs a workload with the conv prologue, not {name}")
    t = make_inputs(w)
    io = w.io_dtype
    x = torch.from_numpy(t["conv_x"])
    if io in (BF16, F16):
        x = x.view(torch.bfloat16 if io == BF16 else torch.float16)
    x = x.cuda()
    wt = torch.from_numpy(t["conv_weight"]).cuda()
    bias = torch.from_numpy(t["conv_bias"]).cuda()
    out = torch.empty_like(x)

    def step():
        binding.causal_conv1d_fwd(x, wt, bias, out=out, act=_lib.SSM_ACT_SILU)

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s_.elapsed_time(e_) for s_, e_ in zip(starts, ends)]
    avg_s = float(np.mean(launch_ms)) / 1e3
    es = 2 if io in (BF16, F16) else 4
    abytes = 2 * w.elements * es + w.dim * 4 * 4 + w.dim * 4
    gbs = abytes / avg_s / 1e9
    rec = {
        "metric": METRIC, "value": w.elements * args.steps / wall, "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"causal_conv1d_fwd on {w.name}'s input: b={w.batch} d={w.dim} l={w.seqlen} "
                               f"width 4, silu, {'bf16' if io == BF16 else 'fp16' if io == F16 else 'fp32'} io",
                   "elements_per_step": w.elements},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": load_traffic(f"conv_{w.name}", CONV_SRCS),
                     "kernel": "conv_kernel",
                     "kernel_avg_ms": avg_s * 1e3, "kernel_median_ms": float(np.median(launch_ms)),
                     "algorithmic_bytes": abytes},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def decode_main(args):
    """One decode step per timed step: conv update, then state update."""
    import torch
    from state_space_model_scan_amd import _lib, binding
    from state_space_model_scan_amd.inputs import BF16, DECODE_WORKLOADS, make_decode_inputs

    _lib.lib()
    w = DECODE_WORKLOADS[args.workload]
    t = make_decode_inputs(w)
    io = w.io_dtype

    def dev(a, param=False):
        x = torch.from_numpy(np.ascontiguousarray(a))
        if not param and io == BF16 and a.dtype == np.uint16:
            x = x.view(torch.bfloat16)
        return x.cuda()

    x, dt = dev(t["x"]), dev(t["dt"])
    z = dev(t["z"]) if t["z"] is not None else None
    B, C = dev(t["B"]), dev(t["C"])
    A = dev(t["A"], True)
    D = dev(t["D"], True) if t["D"] is not None else None
    bias = dev(t["dt_bias"], True) if t["dt_bias"] is not None else None
    state = dev(t["state"], True)
    conv_x, conv_state = dev(t["conv_x"]), dev(t["conv_state"])
    cw, cb = dev(t["conv_weight"], True), dev(t["conv_bias"], True)
    u = torch.empty_like(conv_x)
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    def conv_step():
        binding.causal_conv1d_update(conv_x, conv_state, cw, cb, "silu", None, out=u)

    def state_step():
        binding.selective_state_update(state, x, dt, A, B, C, D, z, bias, w.softplus, out=out)

    settle(lambda: (conv_step(), state_step()))
    for _ in range(args.warmup):
        conv_step()
        state_step()
    torch.cuda.synchronize()
    cs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ss = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    se = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        cs[i].record(stream)
        conv_step()
        ce[i].record(stream)
        ss[i].record(stream)
        state_step()
        se[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    conv_ms = [a.elapsed_time(b) for a, b in zip(cs, ce)]
    su_ms = [a.elapsed_time(b) for a, b in zip(ss, se)]
    su_s = float(np.mean(su_ms)) / 1e3
    conv_s = float(np.mean(conv_ms)) / 1e3
    su_bytes = decode_state_update_bytes(w)
    cv_bytes = decode_conv_update_bytes(w)
    su_gbs = su_bytes / su_s / 1e9
    rec = {
        "metric": "decode step (conv update + selective_state_update) channel-steps/s (b·d)",
        "value": w.channels * args.steps / wall,
        "unit": "channel-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: b={w.batch} d={w.dim} n={w.dstate} g={w.ngroups} "
                        f"{'bf16' if io == BF16 else 'fp32'} io, fp32 state, conv width {w.conv_width} "
                        f"cache {w.conv_state_len}, {w.conv_tokens} token(s)",
            "io_dtype": "bf16" if io == BF16 else "fp32",
            "channels_per_step": w.channels,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": su_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": su_gbs / HBM_PEAK_GBS,
            "traffic": load_traffic(w.name, DECODE_SRCS),
            "kernel": "state_update_kernel",
            "kernel_avg_ms": su_s * 1e3,
            "kernel_median_ms": float(np.median(su_ms)),
            "algorithmic_bytes": su_bytes,
            "conv_update": {"avg_ms": conv_s * 1e3, "algorithmic_bytes": cv_bytes,
                            "GBs": cv_bytes / conv_s / 1e9},
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = decode_cpu_baseline(w, t, args.cpu_budget)
    print(json.dumps(rec), flush=True)


def decode_cpu_baseline(w, t, budget_s: float):
    """The oracle's state update (single-threaded C) on a batch slice."""
    from oracle import oracle as orc
    nb = min(w.batch, 16)
    while True:
        sl = slice(0, nb)
        t0 = time.perf_counter()
        orc.selective_state_update(t["state"][sl].astype(np.float64), t["x"][sl], t["dt"][sl], t["A"],
                                   t["B"][sl], t["C"][sl], t["D"], t["z"][sl] if t["z"] is not None else None,
                                   t["dt_bias"], w.softplus, io_dtype=w.io_dtype)
        dt = time.perf_counter() - t0
        if dt >= min(budget_s, 2.0) or nb == w.batch:
            break
        nb = min(w.batch, nb * 4)
    return {"value": nb * w.dim / dt, "unit": "channel-steps/s", "cores": 1, "kind": "oracle",
            "sample": f"state update of {nb} of {w.batch} batch rows (d={w.dim}, n={w.dstate}), "
                      f"{dt:.2f} s float64 on 1 thread"}



def ssd_bytes(w) -> int:
    es = 2
    xs = w.batch * w.seqlen * w.nheads * w.headdim * es
    total = xs * (3 if w.has_z else 2)                     # x, out (+ z)
    total += w.batch * w.seqlen * w.nheads * es             # dt
    total += 2 * w.batch * w.seqlen * w.ngroups * w.dstate * es   # B, C
    total += w.nheads * 4 * 3                               # A, D, dt_bias
    states = w.batch * w.nheads * w.headdim * w.dstate * 4
    total += states                                         # final states written
    if w.init_state:
        total += states                                     # initial states read
    return total


def ssd_flops(w, Q=64) -> float:
    chunks = -(-w.seqlen // Q)
    n, p = w.dstate, w.headdim
    macs = Q * Q * n / 2 + Q * Q * p / 2 + 2 * Q * p * n
    return 2.0 * macs * chunks * w.batch * w.nheads


def ssd_main(args):
    import torch
    from state_space_model_scan_amd import _lib, binding
    from state_space_model_scan_amd.inputs import SSD_WORKLOADS, make_ssd_inputs

    _lib.lib()
    w = SSD_WORKLOADS[args.workload]
    t = make_ssd_inputs(w)

    def dev(a, param=False):
        if a is None:
            return None
        x = torch.from_numpy(np.ascontiguousarray(a))
        if not param and a.dtype == np.uint16:
            x = x.view(torch.bfloat16)
        return x.cuda()

    x, dt, z, B, C = dev(t["x"]), dev(t["dt"]), dev(t["z"]), dev(t["B"]), dev(t["C"])
    A, D, bias, init = dev(t["A"], True), dev(t["D"], True), dev(t["dt_bias"], True), dev(t["initial_states"], True)
    out = torch.empty_like(x)
    fin = torch.empty((w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device="cuda")

    need = binding.ssd_scan_workspace_size(x, dt, A, B, C, D, z, bias, w.softplus, initial_states=init,
                                           out=out, final_states=fin)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def step():
        binding.ssd_scan_fwd(x, dt, A, B, C, D, z, bias, w.softplus, initial_states=init, out=out,
                             final_states=fin, workspace=ws)

    split_bytes = 0
    if args.split:
        # the three operators in turn, into preallocated states / carried
        # states; their extra traffic is the fp32 chunk states written by
        # chunk_state, read and carried by state_passing, read by chunk_scan
        nc = -(-w.seqlen // args.chunk_size)
        states = torch.empty((nc, w.batch, w.nheads, w.headdim, w.dstate), dtype=torch.float32, device="cuda")
        decays = torch.empty((nc, w.batch, w.nheads), dtype=torch.float32, device="cuda")
        carried = torch.empty_like(states)
        fin_pass = torch.empty_like(fin)
        split_bytes = 4 * states.numel() * 4 + 2 * decays.numel() * 4

        def step():   # noqa: F811
            binding.ssd_chunk_state(x, dt, A, B, args.chunk_size, bias, w.softplus, states=states, decays=decays)
            binding.ssd_state_passing(states, decays, init, carried=carried, final_states=fin_pass)
            binding.ssd_chunk_scan(x, dt, A, B, C, carried, args.chunk_size, D, z, bias, w.softplus, out=out,
                                   final_states=fin)

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    k_s = float(np.mean(ms)) / 1e3
    nbytes = ssd_bytes(w) + w.batch * w.nheads * w.headdim * w.dstate * 4   # + final states
    gbs = nbytes / k_s / 1e9
    tflops = ssd_flops(w) / k_s / 1e12
    if args.split:
        kernel = (f"ssd_chunk_state + ssd_state_passing + ssd_chunk_scan at chunk {args.chunk_size} (the step's "
                  f"events bracket the three; the chunk states add {split_bytes / 1e6:.0f} MB of traffic beyond "
                  f"the algorithmic bytes)")
    else:
        kernel = "ssd_kernel (state pass + full pass)" if need else "ssd_kernel"
    rec = {
        "metric": "Mamba-2 chunked scan elements/s (b·l·h·p)",
        "value": w.elements * args.steps / wall,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: b={w.batch} l={w.seqlen} h={w.nheads} p={w.headdim} n={w.dstate} "
                        f"g={w.ngroups}, bf16 io, fp32 state, chunk 64"
                        + (f", split operators at chunk_size {args.chunk_size}" if args.split else ""),
            "elements_per_step": w.elements,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": None if args.split else load_traffic(w.name, SSD_SRCS),
            "kernel": kernel,
            "workspace_bytes": 0 if args.split else need,
            "kernel_avg_ms": k_s * 1e3,
            "kernel_median_ms": float(np.median(ms)),
            "algorithmic_bytes": nbytes,
            "mfma": {"achieved_TFLOPs": tflops, "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                     "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "algorithmic_flops": ssd_flops(w)},
        },
        "cpu_baseline": None if args.no_cpu_baseline else ssd_cpu_baseline(w, t, args.cpu_budget),
    }
    print(json.dumps(rec), flush=True)


def ssd_cpu_baseline(w, t, budget_s: float):
    """The oracle's sequential Mamba-2 scan (all host threads) on a batch slice."""
    from oracle import oracle as orc
    nb = 1
    threads = orc.max_threads()
    while True:
        sl = slice(0, nb)
        t0 = time.perf_counter()
        orc.ssd_scan(t["x"][sl], t["dt"][sl], t["A"], t["B"][sl], t["C"][sl], t["D"],
                     None if t["z"] is None else t["z"][sl], t["dt_bias"], w.softplus, io_dtype=w.io_dtype,
                     nthreads=threads)
        dt = time.perf_counter() - t0
        if dt >= min(budget_s, 4.0) or nb == w.batch:
            break
        nb = min(w.batch, nb * 2)
    return {"value": nb * w.seqlen * w.nheads * w.headdim / dt, "unit": "elements/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{nb} of {w.batch} batch rows x all {w.nheads} heads x {w.seqlen} tokens, "
                      f"{dt:.1f} s float64 on {threads} threads"}


def bwd_bytes(w) -> int:
    """Backward minimum: u, delta, z, dout, B, C and the checkpoints read once;
    du, ddelta, dz (io) and dA, dB, dC, dD, d(delta_bias) (fp32) written once."""
    es = io_bytes(w.io_dtype)
    E = w.elements
    n = w.dstate
    zed = 1 if w.has_z else 0
    bcn = w.dim * n if w.bc_kind == "fixed" else w.batch * w.ngroups * n * w.seqlen
    nck = -(-w.seqlen // 32)
    reads = (3 + zed) * E * es + 2 * bcn * es + w.batch * w.dim * nck * n * 4 + w.dim * n * 4 + 2 * w.dim * 4
    writes = (2 + zed) * E * es + 2 * bcn * 4 + w.dim * n * 4 + 2 * w.dim * 4
    return reads + writes


def bwd_alu_ops(w) -> float:
    """Per (timestep, state): the forward re-run (delta'*A, delta'u*B, the
    state FMA, C.x for dz: 4 plain, and one exp weighted TRANS_WEIGHT), the
    adjoint (h FMA, carry multiply, a*x, h*a*x, dA FMA, h*B, A*hax FMA with
    u*hB, the two sums over states, dB and dC products and their sums over
    channels) = 14, plus the sum of C.x over states = 1.  Per element:
    softplus (exp, log), its derivative (exp, rcp), silu and its derivative
    (exp, rcp) -- six transcendentals -- and about 16 plain ops."""
    return float(w.elements) * ((19 + TRANS_WEIGHT) * w.dstate + 16 + 6 * TRANS_WEIGHT)


def bwd_main(args):
    import torch
    from state_space_model_scan_amd import _lib, binding
    from state_space_model_scan_amd.inputs import BF16, WORKLOADS, make_dout, make_inputs

    _lib.lib()
    w = WORKLOADS[args.workload]
    if w.conv:
        raise SystemExit("the backward covers the scan; pick a workload without the conv prologue")
    t = make_inputs(w)
    dout_np = make_dout(w)
    io = w.io_dtype

    def dev(a, param=False):
        if a is None:
            return None
        x = torch.from_numpy(np.ascontiguousarray(a))
        if not param and io == BF16 and a.dtype == np.uint16:
            x = x.view(torch.bfloat16)
        return x.cuda()

    u, delta, z, B, C = dev(t["u"]), dev(t["delta"]), dev(t["z"]), dev(t["B"]), dev(t["C"])
    A, D, bias = dev(t["A"], True), dev(t["D"], True), dev(t["delta_bias"], True)
    dout = dev(dout_np)
    ck = torch.empty((w.batch, w.dim, binding.checkpoint_count(w.seqlen), w.dstate), dtype=torch.float32,
                     device="cuda")
    binding.ssm_scan_fwd(u, delta, A, B, C, D, z, bias, w.softplus, checkpoints=ck)

    def step():
        binding.ssm_scan_bwd(u, delta, A, B, C, dout, ck, D=D, z=z, delta_bias=bias,
                             delta_softplus=w.softplus)

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    k_s = float(np.mean(ms)) / 1e3
    ops = bwd_alu_ops(w)
    tops = ops / k_s / 1e12
    nbytes = bwd_bytes(w)
    gbs = nbytes / k_s / 1e9
    rec = {
        "metric": "selective-scan bwd elements/s (b·d·l), all input gradients",
        "value": w.elements * args.steps / wall,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name} backward: b={w.batch} d={w.dim} l={w.seqlen} n={w.dstate} g={w.ngroups} "
                        f"B/C {w.bc_kind}, {'bf16' if io == BF16 else 'fp32'} io, fp32 state, checkpoints "
                        f"every 32 timesteps from the forward",
            "elements_per_step": w.elements,
        },
        "roofline": {
            "bound": "alu",
            "achieved": tops,
            "peak": ALU_PEAK_TOPS,
            "unit": "T fp32 VALU lane-ops/s (transcendental weighted 2)",
            "frac": tops / ALU_PEAK_TOPS,
            "traffic": load_traffic(f"{w.name}_bwd", BWD_SRCS),
            "kernel": "scan_bwd_kernel (+ the sequence split's carry pass and the partial-sum kernels: the "
                      "step's events bracket all of them)",
            "kernel_avg_ms": k_s * 1e3,
            "kernel_median_ms": float(np.median(ms)),
            "hbm": {"achieved_GBs": gbs, "peak_GBs": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS,
                    "algorithmic_bytes": nbytes},
        },
        "cpu_baseline": None if args.no_cpu_baseline else bwd_cpu_baseline(w, t, dout_np, args.cpu_budget),
    }
    print(json.dumps(rec), flush=True)


def bwd_cpu_baseline(w, t, dout, budget_s: float):
    """The oracle's backward (one thread: it has no parallel loop) on the first
    channels of batch 0's first group, grown until it takes about budget_s."""
    from oracle import oracle as orc
    cpg = w.dim // w.ngroups
    nch = 8
    while True:
        ch = slice(0, nch)
        sub = {k: v for k, v in t.items()}
        for k in ("u", "delta", "z"):
            sub[k] = None if t[k] is None else np.ascontiguousarray(t[k][0:1, ch])
        for k in ("B", "C"):
            sub[k] = np.ascontiguousarray(t[k][ch] if t[k].ndim == 2 else t[k][0:1, 0:1])
        for k in ("A", "D", "delta_bias"):
            sub[k] = None if t[k] is None else np.ascontiguousarray(t[k][ch])
        d64 = dout[0:1, ch]
        d64 = (d64.astype(np.uint32) << 16).view(np.float32) if d64.dtype == np.uint16 else d64
        t0 = time.perf_counter()
        orc.selective_scan_bwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], d64.astype(np.float64),
                               sub["D"], sub["z"], sub["delta_bias"], w.softplus, io_dtype=w.io_dtype,
                               ngroups=1, B_kind=orc.BC_FIXED if t["B"].ndim == 2 else orc.BC_VARYING,
                               C_kind=orc.BC_FIXED if t["C"].ndim == 2 else orc.BC_VARYING)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or nch >= cpg:
            break
        nch = min(cpg, nch * 4)
    return {"value": nch * w.seqlen / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{nch} channels of batch 0 x full seqlen {w.seqlen} (backward), {dt:.1f} s float64 "
                      f"on 1 thread"}



def complex_bwd_bytes(w) -> int:
    """Complex backward minimum: u, delta, z, dout (io), complex B, C (io
    pairs) and the complex checkpoints (fp32 pairs) read once; du, ddelta, dz
    (io) and dA, dB, dC (fp32 pairs), dD, d(delta_bias) (fp32) written once."""
    es = io_bytes(w.io_dtype)
    E = w.elements
    n = w.dstate
    zed = 1 if w.has_z else 0
    bcn = 2 * (w.dim * n if w.bc_kind == "fixed" else w.batch * w.ngroups * n * w.seqlen)
    nck = -(-w.seqlen // 32)
    reads = ((3 + zed) * E * es + 2 * bcn * es + w.batch * w.dim * nck * n * 8 + w.dim * n * 8
             + 2 * w.dim * 4)
    writes = (2 + zed) * E * es + 2 * bcn * 4 + w.dim * n * 8 + 2 * w.dim * 4
    return reads + writes


def complex_bwd_alu_ops(w) -> float:
    """Per (timestep, state): the forward re-run (delta' times Re A and Im A,
    the phase's fraction, the decay's two products, delta'u B (2), the
    complex state update (4): 11 plain ops and exp2, sine, cosine); the
    adjoint (Re(C x) 2, h += dy conj C 2, dy conj x 2, h conj x 4, A a 4,
    Re(h conj B) 2, the delta' term 3, the du term 1, dA 6, dB 2, the carry
    conj(a) h 4, the three sums over states 3 and the four sums of dB/dC over
    channels 4: 39).  Per element: softplus, its derivative, silu and its
    derivative (seven transcendentals) and about 20 plain ops.  The kernel
    also recomputes a_t and x_t in its backward walk; those are not counted."""
    return float(w.elements) * ((50 + 3 * TRANS_WEIGHT) * w.dstate + 20 + 7 * TRANS_WEIGHT)


def complex_bwd_main(args):
    """One ssm_scan_bwd_complex call (every gradient) per timed step, from
    the checkpoints of one ssm_scan_fwd_complex run before the timed region."""
    import torch
    from state_space_model_scan_amd import _lib, binding
    from state_space_model_scan_amd.inputs import BF16, COMPLEX_WORKLOADS, F16, make_complex_inputs, make_dout

    _lib.lib()
    w = COMPLEX_WORKLOADS[args.workload]
    t = make_complex_inputs(w)
    dout_np = make_dout(w)
    io = w.io_dtype

    def dev(a, param=False):
        if a is None:
            return None
        x = torch.from_numpy(np.ascontiguousarray(a))
        if not param and io in (BF16, F16) and a.dtype == np.uint16:
            x = x.view(torch.bfloat16 if io == BF16 else torch.float16)
        return x.cuda()

    u, delta, z, B, C = dev(t["u"]), dev(t["delta"]), dev(t["z"]), dev(t["B"]), dev(t["C"])
    A, D, bias = dev(t["A"], True), dev(t["D"], True), dev(t["delta_bias"], True)
    init = dev(t["initial_state"], True)
    dout = dev(dout_np)
    ck = torch.empty((w.batch, w.dim, binding.checkpoint_count(w.seqlen), w.dstate, 2), dtype=torch.float32,
                     device="cuda")
    binding.ssm_scan_fwd_complex(u, delta, A, B, C, D, z, bias, w.softplus, initial_state=init, checkpoints=ck)

    def step():
        binding.ssm_scan_bwd_complex(u, delta, A, B, C, dout, ck, D=D, z=z, delta_bias=bias,
                                     delta_softplus=w.softplus)

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
    settle(step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    k_s = float(np.mean(ms)) / 1e3
    tops = complex_bwd_alu_ops(w) / k_s / 1e12
    nbytes = complex_bwd_bytes(w)
    gbs = nbytes / k_s / 1e9
    iot = {0: "fp32", 1: "bf16", 2: "fp16"}[io]
    rec = {
        "metric": "complex-A selective-scan bwd elements/s (b·d·l), all input gradients",
        "value": w.elements * args.steps / wall, "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name} backward: b={w.batch} d={w.dim} l={w.seqlen} n={w.dstate} "
                               f"g={w.ngroups} complex A/B/C, B/C {w.bc_kind}, {iot} io, fp32 complex state, "
                               f"checkpoints every 32 timesteps from the forward",
                   "io_dtype": iot, "elements_per_step": w.elements},
        "roofline": {
            "bound": "alu", "achieved": tops, "peak": ALU_PEAK_TOPS,
            "unit": "T fp32 VALU lane-ops/s (transcendental weighted 2)", "frac": tops / ALU_PEAK_TOPS,
            "traffic": load_traffic(f"{w.name}_bwd", CBWD_SRCS),
            "kernel": "cbwd_kernel (+ cbwd_sum_kernel, the partial sums: the step's events bracket both)",
            "kernel_avg_ms": k_s * 1e3, "kernel_median_ms": float(np.median(ms)),
            "hbm": {"achieved_GBs": gbs, "peak_GBs": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS,
                    "algorithmic_bytes": nbytes},
        },
        "cpu_baseline": (None if args.no_cpu_baseline
                         else complex_bwd_cpu_baseline(w, t, dout_np, args.cpu_budget)),
    }
    print(json.dumps(rec), flush=True)


def complex_bwd_cpu_baseline(w, t, dout, budget_s: float):
    """The oracle's complex backward (one thread) on the first channels of
    batch 0's first group, grown until it takes about budget_s / 4."""
    from oracle import oracle as orc
    from state_space_model_scan_amd.inputs import io_bits_to_f64
    cpg = w.dim // w.ngroups
    nch = 8
    fixed = w.bc_kind == "fixed"
    while True:
        ch = slice(0, nch)
        sub = {}
        for k in ("u", "delta", "z"):
            sub[k] = None if t[k] is None else np.ascontiguousarray(t[k][0:1, ch])
        for k in ("B", "C"):
            sub[k] = np.ascontiguousarray(t[k][ch] if fixed else t[k][0:1, 0:1])
        for k in ("A", "D", "delta_bias"):
            sub[k] = None if t[k] is None else np.ascontiguousarray(t[k][ch])
        init = None if t["initial_state"] is None else t["initial_state"][0:1, ch].astype(np.float64)
        d64 = io_bits_to_f64(np.ascontiguousarray(dout[0:1, ch]), w.io_dtype)
        t0 = time.perf_counter()
        orc.selective_scan_complex_bwd(sub["u"], sub["delta"], sub["A"], sub["B"], sub["C"], d64, sub["D"],
                                       sub["z"], sub["delta_bias"], w.softplus, io_dtype=w.io_dtype, ngroups=1,
                                       B_kind=orc.BC_FIXED if fixed else orc.BC_VARYING,
                                       C_kind=orc.BC_FIXED if fixed else orc.BC_VARYING, initial_state=init)
        dt = time.perf_counter() - t0
        if dt >= budget_s / 4 or nch >= cpg:
            break
        nch = min(cpg, nch * 4)
    return {"value": nch * w.seqlen / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"{nch} channels of batch 0 x full seqlen {w.seqlen} (complex backward), {dt:.1f} s "
                      f"float64 on 1 thread"}


# ---------------------------------------------------------------------------
# --microbench: the chip rates behind the ALU ceilings (include/ssmmicro.h)
# ---------------------------------------------------------------------------

# probe -> (kind, VALU wave-instructions per loop iteration, transcendental
# wave-instructions per iteration, LDS bytes per iteration per wave)
MB_PROBES = {
    "fma": (0, 128, 0, 0),
    "exp": (1, 0, 128, 0),
    "sin": (8, 0, 128, 0),
    "mix": (2, 136, 32, 0),
    "mix_mfma": (9, 104, 32, 0),
    "dpp": (3, 128, 0, 0),
    "lds_read_b128_broadcast": (4, 0, 0, 16 * 64 * 16),
    "lds_read_b128_linear": (5, 0, 0, 16 * 64 * 16),
    "lds_write_b32": (6, 0, 0, 16 * 64 * 4),
}
NOMINAL_CLK_HZ = 2.4e9
NUM_CU = 256


def microbench_main(args):
    """Instruction rates per compute unit and clock at k waves per SIMD, and
    the device copy bandwidth.  Rates use the nominal 2.4 GHz clock; the
    shader clock measured inside the probe (s_memtime against the 100 MHz
    s_memrealtime) is reported beside them."""
    import ctypes

    import torch
    from state_space_model_scan_amd import _build
    lib = ctypes.CDLL(_build.MICRO_LIB)
    lib.ssm_microbench.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    clk = torch.zeros(4, dtype=torch.int64, device="cuda")

    def run(kind, blocks, iters, buf, reps=5):
        rc = lib.ssm_microbench(kind, blocks, iters, ctypes.c_void_p(buf.data_ptr()),
                                ctypes.c_void_p(clk.data_ptr()), sp)
        if rc != 0:
            raise RuntimeError(f"ssm_microbench({kind}) returned {rc}")
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            lib.ssm_microbench(kind, blocks, iters, ctypes.c_void_p(buf.data_ptr()),
                               ctypes.c_void_p(clk.data_ptr()), sp)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b)
            best = ms if best is None else min(best, ms)
        c = clk.cpu().tolist()
        real = (c[3] - c[1]) / 100e6
        shader_hz = (c[2] - c[0]) / real if real > 0 else None
        return best / 1e3, shader_hz

    res = {"nominal_clock_GHz": NOMINAL_CLK_HZ / 1e9, "compute_units": NUM_CU, "probes": {}}
    for name, (kind, valu, trans, lds) in MB_PROBES.items():
        rows = {}
        for k in (1, 2, 3, 4, 8):
            blocks = NUM_CU * k
            iters = max(64, 2048 // k)
            buf = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            t, hz = run(kind, blocks, iters, buf)
            waves = blocks * 4
            cu_clk = t * NUM_CU * NOMINAL_CLK_HZ
            row = {"ms": t * 1e3, "shader_clock_GHz": None if hz is None else hz / 1e9}
            if valu:
                row["valu_per_cu_clk"] = waves * iters * valu / cu_clk
            if trans:
                row["trans_per_cu_clk"] = waves * iters * trans / cu_clk
            if lds:
                row["lds_bytes_per_cu_clk"] = waves * iters * lds / cu_clk
            rows[f"{k}_waves_per_simd"] = row
        res["probes"][name] = rows
    # device copy: 1 GiB read + 1 GiB written
    blocks, iters = NUM_CU * 8, 128
    nbytes = blocks * 256 * iters * 16
    buf = torch.empty(2 * nbytes // 4, dtype=torch.float32, device="cuda")
    t, _ = run(7, blocks, iters, buf)
    res["copy"] = {"bytes_read": nbytes, "bytes_written": nbytes, "ms": t * 1e3,
                   "GBs": 2 * nbytes / t / 1e9, "frac_of_8TBs": 2 * nbytes / t / 1e9 / HBM_PEAK_GBS}
    print(json.dumps({"microbench": res}), flush=True)


if __name__ == "__main__":
    main()
