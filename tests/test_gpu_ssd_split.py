"""GPU parity of the split chunk-scan operators (ssd_chunk_state,
ssd_state_passing, ssd_chunk_scan) against the float64 oracle's split
operators (oracle.ssd_chunk_state / ssd_state_passing / ssd_chunk_scan,
pinned on the CPU through the sequential scan), through the C ABI.

Each operator is checked on its own, from the same inputs the oracle gets
(state_passing and chunk_scan from the oracle's chunk states and carried
states, rounded to float32), and the three composed on the GPU are checked
against ssd_scan_fwd with the same segmentation: the same kernels and the
same fp32 fma per carried state, so out and the state after chunk_scan's
last chunk must be identical bits.

Bars, per element, |gpu - ref| <= tol * (1 + |ref|): out at the bf16 io
tolerance 2e-2 (as ssd_scan_fwd); the fp32 states (chunk states, carried,
final) at STATE_TOL = 1e-4, the bar of every fp32 state (measured: about
3e-6; the state products take bf16 head + tail operands, about 16
significant bits); decays and state_passing (fp32 exponentials and fmas
only) at 1e-5.
"""
import numpy as np
import pytest

from oracle import oracle as orc
from state_space_model_scan_amd.inputs import BF16, SSD_WORKLOADS, make_ssd_inputs
from tests.harness import TOL, log, max_err, to_dev

pytestmark = pytest.mark.gpu

STATE_TOL = 1e-4
EXACT_TOL = 1e-5
SEQ_CUTS = [[5, 64, 70, 71, 128, 200, 255], [1, 2, 127, 129, 192, 256, 299]]


def _packed_ids(cuts, seqlen):
    sid = np.zeros((len(cuts), seqlen), np.int32)
    for b, cs in enumerate(cuts):
        for c in cs:
            if c < seqlen:
                sid[b, c:] += 1
    return sid


def _case(n=64, seqlen=300, init=True, seed=0, **kw):
    w = SSD_WORKLOADS["ssd_tiny"].scaled(batch=2, seqlen=seqlen, nheads=4, dstate=n, ngroups=2,
                                         init_state=init, seed=seed, **kw)
    return w, make_ssd_inputs(w)


def _dev(t, seq_idx):
    import torch
    d = {k: to_dev(t[k], BF16) for k in ("x", "dt", "B", "C", "z")}
    for k in ("A", "D", "dt_bias", "initial_states"):
        d[k] = to_dev(t[k], param=True)
    d["seq_idx"] = None if seq_idx is None else torch.from_numpy(seq_idx).to("cuda")
    return d


def _np(a):
    return a.float().cpu().numpy().astype(np.float64)


OPTS = {"plain": {}, "seq": {"seq": True}, "limit": {"limit": (0.05, 0.3)}}


def _opts(name, w):
    o = OPTS[name]
    sid = _packed_ids(SEQ_CUTS, w.seqlen) if o.get("seq") else None
    return sid, o.get("limit")


@pytest.mark.parametrize("opt", sorted(OPTS))
@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("n", [32, 128])
def test_chunk_state(n, chunk, opt):
    import torch
    from state_space_model_scan_amd import binding
    w, t = _case(n=n, seed=600 + n + chunk)
    sid, lim = _opts(opt, w)
    log(f"[ssd-split] chunk_state n={n} chunk={chunk} {opt}")
    d = _dev(t, sid)
    st, dc = binding.ssd_chunk_state(d["x"], d["dt"], d["A"], d["B"], chunk, d["dt_bias"], w.softplus,
                                     seq_idx=d["seq_idx"], dt_limit=lim)
    torch.cuda.synchronize()
    rs, rd = orc.ssd_chunk_state(t["x"], t["dt"], t["A"], t["B"], chunk, t["dt_bias"], w.softplus,
                                 io_dtype=BF16, dt_limit=lim, seq_idx=sid)
    es, ed = max_err(_np(st), rs), max_err(_np(dc), rd)
    log(f"[ssd-split]   states {es:.2e} decays {ed:.2e}")
    assert es <= STATE_TOL, f"states {es:.3e}"
    assert ed <= EXACT_TOL, f"decays {ed:.3e}"
    if sid is not None:   # a sequence start inside a chunk makes its factor exactly 0
        assert np.array_equal(_np(dc) == 0.0, rd == 0.0)


@pytest.mark.parametrize("init", [True, False])
def test_state_passing(init):
    import torch
    from state_space_model_scan_amd import binding
    w, t = _case(n=128, seqlen=700, init=init, seed=640 + init)
    log(f"[ssd-split] state_passing init={init}")
    rs, rd = orc.ssd_chunk_state(t["x"], t["dt"], t["A"], t["B"], 64, t["dt_bias"], w.softplus, io_dtype=BF16)
    rs32, rd32 = rs.astype(np.float32), rd.astype(np.float32)
    init32 = None if t["initial_states"] is None else t["initial_states"].astype(np.float32)
    car, fin = binding.ssd_state_passing(torch.from_numpy(rs32).cuda(), torch.from_numpy(rd32).cuda(),
                                         None if init32 is None else torch.from_numpy(init32).cuda())
    torch.cuda.synchronize()
    rc, rf = orc.ssd_state_passing(rs32, rd32, init32)
    ec, ef = max_err(_np(car), rc), max_err(_np(fin), rf)
    log(f"[ssd-split]   carried {ec:.2e} final {ef:.2e}")
    assert ec <= EXACT_TOL and ef <= EXACT_TOL, (ec, ef)


@pytest.mark.parametrize("opt", sorted(OPTS))
@pytest.mark.parametrize("chunk", [64, 192])
@pytest.mark.parametrize("n", [64, 128])
def test_chunk_scan(n, chunk, opt):
    import torch
    from state_space_model_scan_amd import binding
    w, t = _case(n=n, seed=660 + n + chunk)
    sid, lim = _opts(opt, w)
    log(f"[ssd-split] chunk_scan n={n} chunk={chunk} {opt}")
    rs, rd = orc.ssd_chunk_state(t["x"], t["dt"], t["A"], t["B"], chunk, t["dt_bias"], w.softplus,
                                 io_dtype=BF16, dt_limit=lim, seq_idx=sid)
    rc, _ = orc.ssd_state_passing(rs, rd, t["initial_states"])
    rc32 = rc.astype(np.float32)
    d = _dev(t, sid)
    fin = torch.full((w.batch, w.nheads, w.headdim, w.dstate), float("nan"), device="cuda")
    out = binding.ssd_chunk_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], torch.from_numpy(rc32).cuda(), chunk,
                                 d["D"], d["z"], d["dt_bias"], w.softplus, seq_idx=d["seq_idx"], dt_limit=lim,
                                 final_states=fin)
    torch.cuda.synchronize()
    ro, rf = orc.ssd_chunk_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], rc32, chunk, t["D"], t["z"], t["dt_bias"],
                                w.softplus, io_dtype=BF16, dt_limit=lim, seq_idx=sid)
    eo, ef = max_err(_np(out), ro), max_err(_np(fin), rf)
    log(f"[ssd-split]   out {eo:.2e} final {ef:.2e}")
    assert eo <= TOL[BF16], f"out {eo:.3e}"
    assert ef <= STATE_TOL, f"final {ef:.3e}"


def _composed(w, d, chunk, sid_t, lim):
    import torch
    from state_space_model_scan_amd import binding
    st, dc = binding.ssd_chunk_state(d["x"], d["dt"], d["A"], d["B"], chunk, d["dt_bias"], w.softplus,
                                     seq_idx=sid_t, dt_limit=lim)
    car, fin = binding.ssd_state_passing(st, dc, d["initial_states"])
    fin2 = torch.empty_like(fin)
    out = binding.ssd_chunk_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], car, chunk, d["D"], d["z"],
                                 d["dt_bias"], w.softplus, seq_idx=sid_t, dt_limit=lim, final_states=fin2)
    return out, fin, fin2


@pytest.mark.parametrize("opt", sorted(OPTS))
@pytest.mark.parametrize("chunk,segments", [(64, 5), (128, 3), (192, 2), (320, 1)])
def test_composition_is_ssd_scan_fwd_bit_for_bit(chunk, segments, opt):
    """chunk_state -> state_passing -> chunk_scan on the GPU equals
    ssd_scan_fwd cut into the same segments (300 tokens: 5 chunks of 64)."""
    import torch
    from state_space_model_scan_amd import binding
    w, t = _case(n=128, seed=700 + chunk)
    sid, lim = _opts(opt, w)
    log(f"[ssd-split] composition chunk={chunk} segments={segments} {opt}")
    d = _dev(t, sid)
    out, fin, fin2 = _composed(w, d, chunk, d["seq_idx"], lim)
    ref_fin = torch.empty_like(fin)
    ws = torch.empty(16 << 20, dtype=torch.uint8, device="cuda")
    ref = binding.ssd_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], d["dt_bias"], w.softplus,
                               initial_states=d["initial_states"], final_states=ref_fin, seq_idx=d["seq_idx"],
                               dt_limit=lim, workspace=ws, seq_segments=segments)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(fin2, ref_fin)
    # state_passing's last state is P E-folded, not walked: equal to rounding
    ef = max_err(_np(fin), _np(ref_fin))
    assert ef <= STATE_TOL, f"state_passing final {ef:.3e}"


def test_full_size_composition():
    """ssd2p7b (b=8 l=2048 h=80 p=64 n=128): chunk size 1024 composed equals
    ssd_scan_fwd's own two-segment plan bit for bit; chunk size 256 (the
    Mamba-2 default chunk) composed matches the oracle on three heads."""
    import torch
    from state_space_model_scan_amd import binding
    from tests.test_gpu_ssd import _oracle
    w = SSD_WORKLOADS["ssd2p7b"]
    log(f"[ssd-split] full size {w.name}")
    t = make_ssd_inputs(w)
    d = _dev(t, None)
    out, _, fin2 = _composed(w, d, 1024, None, None)
    ref_fin = torch.empty_like(fin2)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    ref = binding.ssd_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], d["dt_bias"], w.softplus,
                               initial_states=d["initial_states"], final_states=ref_fin, workspace=ws,
                               seq_segments=2)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(fin2, ref_fin)
    out, fin, _ = _composed(w, d, 256, None, None)
    torch.cuda.synchronize()
    heads = [0, 41, 79]
    ro, rf = _oracle(w, t, heads)
    eo = max_err(_np(out)[:, :, heads], ro)
    ef = max_err(_np(fin)[:, heads], rf)
    log(f"[ssd-split]   chunk 256: out {eo:.2e} final {ef:.2e}")
    assert eo <= TOL[BF16] and ef <= STATE_TOL, (eo, ef)


@pytest.mark.parametrize("seqlen,chunk", [(1, 64), (64, 64), (65, 64), (129, 256), (256, 128)])
def test_split_edges(seqlen, chunk):
    """One token, whole and ragged last chunks, a single chunk longer than
    the sequence, no initial state: each operator against the oracle and the
    composition against ssd_scan_fwd with the matching segments."""
    import torch
    from state_space_model_scan_amd import binding
    w, t = _case(n=32, seqlen=seqlen, init=False, seed=720 + seqlen + chunk)
    log(f"[ssd-split] edge l={seqlen} chunk={chunk}")
    d = _dev(t, None)
    st, dc = binding.ssd_chunk_state(d["x"], d["dt"], d["A"], d["B"], chunk, d["dt_bias"], w.softplus)
    torch.cuda.synchronize()
    rs, rd = orc.ssd_chunk_state(t["x"], t["dt"], t["A"], t["B"], chunk, t["dt_bias"], w.softplus, io_dtype=BF16)
    assert st.shape[0] == rs.shape[0] == -(-seqlen // chunk)
    assert max_err(_np(st), rs) <= STATE_TOL and max_err(_np(dc), rd) <= EXACT_TOL
    out, fin, fin2 = _composed(w, d, chunk, None, None)
    ref_fin = torch.empty_like(fin)
    ws = torch.empty(16 << 20, dtype=torch.uint8, device="cuda")
    nseg = -(-seqlen // chunk)
    ref = binding.ssd_scan_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["z"], d["dt_bias"], w.softplus,
                               final_states=ref_fin, workspace=ws, seq_segments=nseg)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(fin2, ref_fin)
    ro, rf = orc.ssd_scan(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["z"], t["dt_bias"], w.softplus,
                          io_dtype=BF16)
    assert max_err(_np(out), ro) <= TOL[BF16] and max_err(_np(fin), rf) <= STATE_TOL
