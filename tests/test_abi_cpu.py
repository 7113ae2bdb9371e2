"""C-ABI checks that need no GPU: the library loads, exports every function
include/ssmscan.h declares, and rejects bad arguments on the host (status
codes 1-3) before any HIP call.  No compute entry point is called with valid
arguments here."""
import ctypes
import os
import re

import pytest

from state_space_model_scan_amd import _lib
from state_space_model_scan_amd._lib import ScanArgs, SsdArgs, StateUpdateArgs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssmscan.h")

FAKE = 0x1000  # a non-null pointer value; validation never dereferences it


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_header_symbols():
    L = _lib.lib()
    funcs = _header_functions()
    assert set(funcs) == set(_lib.EXPORTS), funcs
    for name in funcs:
        assert hasattr(L, name), f"{name} not exported"
    assert L.ssm_abi_version() == 13


def test_status_strings():
    L = _lib.lib()
    for code in range(7):
        assert L.ssm_status_str(code)
    assert L.ssm_status_str(99) == b"unknown status"


def _good_args(**kw):
    a = ScanArgs()
    a.batch, a.dim, a.seqlen, a.dstate, a.ngroups = 2, 64, 128, 16, 1
    a.io_dtype = _lib.SSM_BF16
    a.u = a.delta = a.A = a.B = a.C = a.out = FAKE
    a.B_kind = a.C_kind = _lib.SSM_BC_VARYING
    a.delta_softplus = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _validate(a):
    return _lib.lib().ssm_scan_validate(ctypes.byref(a))


def test_valid_arguments_pass():
    assert _validate(_good_args()) == _lib.SSM_OK
    assert _validate(_good_args(u=None, conv_x=FAKE, conv_weight=FAKE, conv_width=4,
                                conv_act=_lib.SSM_ACT_SILU)) == _lib.SSM_OK
    assert _validate(_good_args(ngroups=4, dim=256)) == _lib.SSM_OK
    assert _validate(_good_args(dstate=1)) == _lib.SSM_OK


@pytest.mark.parametrize("field", ["delta", "A", "B", "C", "out", "u"])
def test_null_required_pointer(field):
    assert _validate(_good_args(**{field: None})) == _lib.SSM_ERR_NULL


def test_null_conv_input():
    a = _good_args(u=None, conv_weight=FAKE, conv_width=4)
    assert _validate(a) == _lib.SSM_ERR_NULL


@pytest.mark.parametrize("field,val", [("batch", 0), ("dim", -1), ("seqlen", 0), ("dstate", 0),
                                       ("ngroups", 0), ("ngroups", 3), ("seq_segments", -1)])
def test_bad_shapes(field, val):
    assert _validate(_good_args(**{field: val})) == _lib.SSM_ERR_SHAPE


def test_overflowing_sizes():
    assert _validate(_good_args(batch=1 << 40, dim=1 << 20, seqlen=1 << 20)) == _lib.SSM_ERR_SHAPE


@pytest.mark.parametrize("kw", [dict(io_dtype=3), dict(dstate=17), dict(B_kind=2), dict(C_kind=-1),
                                dict(delta_softplus=2),
                                dict(conv_weight=FAKE, conv_x=FAKE, conv_width=3),
                                dict(conv_weight=FAKE, conv_x=FAKE, conv_width=4, conv_act=7)])
def test_unsupported(kw):
    assert _validate(_good_args(**kw)) == _lib.SSM_ERR_UNSUPPORTED


def test_fwd_rejects_before_any_hip_call():
    """Invalid arguments return their status from ssm_scan_fwd itself, without
    touching HIP (this runs on a machine with no GPU)."""
    L = _lib.lib()
    assert L.ssm_scan_fwd(ctypes.byref(_good_args(delta=None)), None) == _lib.SSM_ERR_NULL
    assert L.ssm_scan_fwd(ctypes.byref(_good_args(dstate=33)), None) == _lib.SSM_ERR_UNSUPPORTED
    assert L.ssm_scan_fwd(None, None) == _lib.SSM_ERR_NULL
    size = ctypes.c_size_t(0)
    assert L.ssm_scan_workspace_size(ctypes.byref(_good_args(seqlen=0)), ctypes.byref(size)) == _lib.SSM_ERR_SHAPE


def test_missing_workspace_is_rejected_before_any_launch():
    """The library allocates nothing: when its plan needs scratch (a sequence
    split) and the caller passes no workspace, or too little, ssm_scan_fwd
    returns SSM_ERR_WORKSPACE before it enqueues anything.  The pointers here
    are not dereferenceable, so any memory access would crash the test."""
    L = _lib.lib()
    for kw in (dict(batch=1, dim=64, seqlen=4096), dict(seq_segments=2),
               dict(batch=1, dim=2560, seqlen=65536, B_kind=_lib.SSM_BC_VARYING)):
        a = _good_args(**kw)
        need = ctypes.c_size_t(0)
        assert L.ssm_scan_workspace_size(ctypes.byref(a), ctypes.byref(need)) == _lib.SSM_OK
        assert need.value > 0, kw
        assert L.ssm_scan_fwd(ctypes.byref(a), None) == _lib.SSM_ERR_WORKSPACE
        a.workspace, a.workspace_bytes = FAKE, need.value - 1
        assert L.ssm_scan_fwd(ctypes.byref(a), None) == _lib.SSM_ERR_WORKSPACE
    # a plan with no split needs no scratch at all (the Mamba-2.8B layer)
    need = ctypes.c_size_t(1)
    a = _good_args(batch=8, dim=5120, ngroups=4, seqlen=2048)
    assert L.ssm_scan_workspace_size(ctypes.byref(a), ctypes.byref(need)) == _lib.SSM_OK
    assert need.value == 0


def test_noalloc_rejects_before_any_hip_call():
    """ssm_scan_fwd_noalloc validates like ssm_scan_fwd and rejects a plan
    whose scratch exceeds its built-in buffer with SSM_ERR_SCRATCH, before
    any HIP call (this runs on a machine with no GPU)."""
    L = _lib.lib()
    assert L.ssm_scan_fwd_noalloc(None, None) == _lib.SSM_ERR_NULL
    assert L.ssm_scan_fwd_noalloc(ctypes.byref(_good_args(delta=None)), None) == _lib.SSM_ERR_NULL
    assert L.ssm_scan_fwd_noalloc(ctypes.byref(_good_args(dstate=33)), None) == _lib.SSM_ERR_UNSUPPORTED
    big = _good_args(batch=1, dim=4096, seqlen=1 << 16, seq_segments=200)
    need = ctypes.c_size_t(0)
    assert L.ssm_scan_workspace_size(ctypes.byref(big), ctypes.byref(need)) == _lib.SSM_OK
    assert need.value > _lib.SSM_NOALLOC_SCRATCH_BYTES
    assert L.ssm_scan_fwd_noalloc(ctypes.byref(big), None) == _lib.SSM_ERR_SCRATCH
    assert b"no-allocation" in L.ssm_status_str(_lib.SSM_ERR_SCRATCH)


def test_conv_validation():
    L = _lib.lib()
    v = L.causal_conv1d_validate
    assert v(FAKE, FAKE, FAKE, 2, 8, 16, 4, _lib.SSM_F32, _lib.SSM_ACT_SILU) == _lib.SSM_OK
    assert v(None, FAKE, FAKE, 2, 8, 16, 4, _lib.SSM_F32, 0) == _lib.SSM_ERR_NULL
    assert v(FAKE, FAKE, FAKE, 0, 8, 16, 4, _lib.SSM_F32, 0) == _lib.SSM_ERR_SHAPE
    assert v(FAKE, FAKE, FAKE, 2, 8, 16, 5, _lib.SSM_F32, 0) == _lib.SSM_ERR_UNSUPPORTED
    assert v(FAKE, FAKE, FAKE, 2, 8, 16, 4, 9, 0) == _lib.SSM_ERR_UNSUPPORTED
    assert v(FAKE, FAKE, FAKE, 2, 8, 16, 4, _lib.SSM_BF16, 3) == _lib.SSM_ERR_UNSUPPORTED
    assert L.causal_conv1d_fwd(None, FAKE, None, FAKE, 2, 8, 16, 4, 0, 0, None) == _lib.SSM_ERR_NULL


def test_python_binding_errors():
    import torch
    from state_space_model_scan_amd import binding
    with pytest.raises(NotImplementedError):
        binding._act_code("gelu")
    assert binding._act_code("swish") == binding._act_code("silu") == _lib.SSM_ACT_SILU
    assert binding._act_code(None) == _lib.SSM_ACT_NONE
    with pytest.raises(ValueError):
        binding._bc_kind(torch.zeros(2, 3, 4, 5, 6), "B")
    assert binding._bc_kind(torch.zeros(4, 16), "B") == (_lib.SSM_BC_FIXED, 0)
    assert binding._bc_kind(torch.zeros(2, 16, 8), "B") == (_lib.SSM_BC_VARYING, 1)
    assert binding._bc_kind(torch.zeros(2, 4, 16, 8), "B") == (_lib.SSM_BC_VARYING, 4)


# --------------------------------------------------------------------------
# decode entry points
# --------------------------------------------------------------------------

def _good_su(**kw):
    a = StateUpdateArgs()
    a.batch, a.dim, a.dstate, a.ngroups = 4, 64, 16, 2
    a.io_dtype = _lib.SSM_BF16
    a.state = a.x = a.dt = a.A = a.B = a.C = a.out = FAKE
    a.dt_softplus = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _su(a):
    return _lib.lib().ssm_state_update_validate(ctypes.byref(a))


def test_state_update_validation():
    L = _lib.lib()
    assert _su(_good_su()) == _lib.SSM_OK
    assert _su(_good_su(dstate=1, ngroups=1)) == _lib.SSM_OK
    assert _su(_good_su(D=FAKE, z=FAKE, dt_bias=FAKE)) == _lib.SSM_OK
    for field in ("state", "x", "dt", "A", "B", "C", "out"):
        assert _su(_good_su(**{field: None})) == _lib.SSM_ERR_NULL, field
    for field, val in (("batch", 0), ("dim", -3), ("dstate", 0), ("ngroups", 0), ("ngroups", 3)):
        assert _su(_good_su(**{field: val})) == _lib.SSM_ERR_SHAPE, (field, val)
    assert _su(_good_su(batch=1 << 40, dim=1 << 22)) == _lib.SSM_ERR_SHAPE
    for kw in (dict(io_dtype=5), dict(dstate=17), dict(dt_softplus=3)):
        assert _su(_good_su(**kw)) == _lib.SSM_ERR_UNSUPPORTED, kw
    assert L.ssm_state_update_validate(None) == _lib.SSM_ERR_NULL
    # the compute entry point returns the same status before any HIP call
    assert L.ssm_state_update(ctypes.byref(_good_su(out=None)), None) == _lib.SSM_ERR_NULL
    assert L.ssm_state_update(None, None) == _lib.SSM_ERR_NULL


def test_conv_update_validation():
    L = _lib.lib()
    v = L.causal_conv1d_update_validate
    F32, BF16 = _lib.SSM_F32, _lib.SSM_BF16
    # x, conv_state, weight, out, batch, dim, seqlen, state_len, width, io, act
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 3, 4, BF16, 1) == _lib.SSM_OK
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 5, 7, 2, F32, 0) == _lib.SSM_OK
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 256, 4, F32, 0) == _lib.SSM_OK
    for i in range(4):
        ptrs = [FAKE] * 4
        ptrs[i] = None
        assert v(*ptrs, 2, 8, 1, 3, 4, F32, 0) == _lib.SSM_ERR_NULL
    assert v(FAKE, FAKE, FAKE, FAKE, 0, 8, 1, 3, 4, F32, 0) == _lib.SSM_ERR_SHAPE
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 0, 3, 4, F32, 0) == _lib.SSM_ERR_SHAPE
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 2, 4, F32, 0) == _lib.SSM_ERR_SHAPE    # cache < width-1
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 257, 4, F32, 0) == _lib.SSM_ERR_UNSUPPORTED
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 3, 5, F32, 0) == _lib.SSM_ERR_UNSUPPORTED
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 3, 1, F32, 0) == _lib.SSM_ERR_UNSUPPORTED
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 3, 4, 7, 0) == _lib.SSM_ERR_UNSUPPORTED
    assert v(FAKE, FAKE, FAKE, FAKE, 2, 8, 1, 3, 4, F32, 2) == _lib.SSM_ERR_UNSUPPORTED
    assert L.causal_conv1d_update(None, FAKE, FAKE, None, None, FAKE, 2, 8, 1, 3, 4, F32, 0,
                                  None) == _lib.SSM_ERR_NULL


def test_decode_binding_errors():
    import torch
    from state_space_model_scan_amd import binding
    st = torch.zeros(2, 4, 8)
    x = torch.zeros(2, 4)
    with pytest.raises(ValueError):   # state must be contiguous float32
        binding.selective_state_update(st.transpose(1, 2), x, x, torch.zeros(4, 8),
                                       torch.zeros(2, 8), torch.zeros(2, 8))
    with pytest.raises(ValueError):   # mismatched B/C groups
        binding.selective_state_update(st, x, x, torch.zeros(4, 8), torch.zeros(2, 2, 8),
                                       torch.zeros(2, 4, 8))
    with pytest.raises(ValueError):   # cache_seqlens must be int32
        binding.causal_conv1d_update(x, torch.zeros(2, 4, 3), torch.zeros(4, 4),
                                     cache_seqlens=torch.zeros(2, dtype=torch.int64))
    with pytest.raises(NotImplementedError):
        binding.causal_conv1d_update(x, torch.zeros(2, 4, 3), torch.zeros(4, 4), activation="relu")


def _good_ssd(**kw):
    a = SsdArgs()
    a.batch, a.seqlen, a.nheads, a.headdim, a.dstate, a.ngroups = 2, 128, 8, 64, 128, 2
    a.io_dtype = _lib.SSM_BF16
    a.x = a.dt = a.A = a.B = a.C = a.out = 0x1000
    a.dt_softplus = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_ssd_validation():
    L = _lib.lib()
    v = lambda a: L.ssd_scan_validate(ctypes.byref(a))
    assert v(_good_ssd()) == _lib.SSM_OK
    assert v(_good_ssd(dstate=32, ngroups=1, z=0x2000, D=0x3000, D_per_channel=1)) == _lib.SSM_OK
    for field in ("x", "dt", "A", "B", "C", "out"):
        assert v(_good_ssd(**{field: None})) == _lib.SSM_ERR_NULL, field
    for field, val in (("batch", 0), ("seqlen", -1), ("nheads", 0), ("ngroups", 3), ("dstate", 0)):
        assert v(_good_ssd(**{field: val})) == _lib.SSM_ERR_SHAPE, (field, val)
    for kw in (dict(io_dtype=_lib.SSM_F32), dict(headdim=32), dict(dstate=16), dict(dstate=96),
               dict(dt_softplus=2), dict(D_per_channel=5), dict(x=0x1002), dict(z=0x1008)):
        assert v(_good_ssd(**kw)) == _lib.SSM_ERR_UNSUPPORTED, kw
    assert L.ssd_scan_fwd(ctypes.byref(_good_ssd(B=None)), None) == _lib.SSM_ERR_NULL
    assert L.ssd_scan_validate(None) == _lib.SSM_ERR_NULL
    # the step range and the split
    assert v(_good_ssd(dt_limit=1, dt_min=0.001, dt_max=0.1)) == _lib.SSM_OK
    assert v(_good_ssd(dt_limit=1, dt_min=0.5, dt_max=0.5)) == _lib.SSM_OK
    assert v(_good_ssd(dt_limit=1, dt_min=0.2, dt_max=0.1)) == _lib.SSM_ERR_SHAPE
    assert v(_good_ssd(dt_limit=1, dt_min=float("nan"), dt_max=0.1)) == _lib.SSM_ERR_SHAPE
    assert v(_good_ssd(dt_limit=0, dt_min=0.2, dt_max=0.1)) == _lib.SSM_OK   # range unused
    assert v(_good_ssd(dt_limit=2)) == _lib.SSM_ERR_UNSUPPORTED
    assert v(_good_ssd(seq_segments=-1)) == _lib.SSM_ERR_SHAPE
    assert v(_good_ssd(seq_idx=0x4000)) == _lib.SSM_OK


def test_ssd_split_needs_workspace_before_any_launch():
    """A forced split needs scratch: without it, or with too little, the call
    returns SSM_ERR_WORKSPACE before anything is enqueued (the pointers are
    not dereferenceable)."""
    L = _lib.lib()
    a = _good_ssd(seqlen=1024, seq_segments=4)
    need = ctypes.c_size_t(0)
    assert L.ssd_scan_workspace_size(ctypes.byref(a), ctypes.byref(need)) == _lib.SSM_OK
    # three carried (headdim x dstate) fp32 states and decays per (batch, head)
    assert need.value >= 3 * 2 * 8 * 64 * 128 * 4 + 3 * 2 * 8 * 4
    assert L.ssd_scan_fwd(ctypes.byref(a), None) == _lib.SSM_ERR_WORKSPACE
    a.workspace, a.workspace_bytes = 0x5000, need.value - 1
    assert L.ssd_scan_fwd(ctypes.byref(a), None) == _lib.SSM_ERR_WORKSPACE
    one = _good_ssd(seqlen=1024, seq_segments=1)
    assert L.ssd_scan_workspace_size(ctypes.byref(one), ctypes.byref(need)) == _lib.SSM_OK
    assert need.value == 0
    # more segments than chunks: one per chunk
    few = _good_ssd(seqlen=100, seq_segments=9)
    assert L.ssd_scan_workspace_size(ctypes.byref(few), ctypes.byref(need)) == _lib.SSM_OK
    assert need.value >= 1 * 2 * 8 * 64 * 128 * 4


def test_ssd_split_operator_validation():
    """ssd_chunk_state / ssd_state_passing / ssd_chunk_scan reject bad
    arguments before any launch (the device pointers are never touched)."""
    L = _lib.lib()
    st, dc, car = 0x6000, 0x7000, 0x8000
    cs = lambda a, k=128, s=st, d=dc: L.ssd_chunk_state_validate(ctypes.byref(a), k, s, d)  # noqa: E731
    sc = lambda a, k=128, c=car: L.ssd_chunk_scan_validate(ctypes.byref(a), k, c)             # noqa: E731
    assert cs(_good_ssd()) == _lib.SSM_OK
    assert sc(_good_ssd()) == _lib.SSM_OK
    # chunk_state reads neither C nor out
    assert cs(_good_ssd(C=None, out=None)) == _lib.SSM_OK
    assert sc(_good_ssd(C=None)) == _lib.SSM_ERR_NULL
    assert sc(_good_ssd(out=None)) == _lib.SSM_ERR_NULL
    for k in (0, -64, 32, 100):
        assert cs(_good_ssd(), k) == _lib.SSM_ERR_UNSUPPORTED, k
        assert sc(_good_ssd(), k) == _lib.SSM_ERR_UNSUPPORTED, k
    assert cs(_good_ssd(), 64, s=None) == _lib.SSM_ERR_NULL
    assert cs(_good_ssd(), 64, d=None) == _lib.SSM_ERR_NULL
    assert sc(_good_ssd(), 64, c=None) == _lib.SSM_ERR_NULL
    for kw in (dict(io_dtype=_lib.SSM_F32), dict(headdim=32), dict(dstate=96), dict(x=0x1002)):
        assert cs(_good_ssd(**kw)) == _lib.SSM_ERR_UNSUPPORTED, kw
        assert sc(_good_ssd(**kw)) == _lib.SSM_ERR_UNSUPPORTED, kw
    assert sc(_good_ssd(z=0x1008)) == _lib.SSM_ERR_UNSUPPORTED
    assert cs(_good_ssd(ngroups=3)) == _lib.SSM_ERR_SHAPE
    assert cs(_good_ssd(dt_limit=1, dt_min=0.2, dt_max=0.1)) == _lib.SSM_ERR_SHAPE
    assert L.ssd_chunk_state(ctypes.byref(_good_ssd(B=None)), 64, st, dc, None) == _lib.SSM_ERR_NULL
    assert L.ssd_chunk_scan(ctypes.byref(_good_ssd()), 96, car, None) == _lib.SSM_ERR_UNSUPPORTED
    sp = L.ssd_state_passing_validate
    assert sp(4, 2, 8, 64, 128, st, dc, car) == _lib.SSM_OK
    assert sp(0, 2, 8, 64, 128, st, dc, car) == _lib.SSM_ERR_SHAPE
    assert sp(4, 2, -8, 64, 128, st, dc, car) == _lib.SSM_ERR_SHAPE
    for args in ((None, dc, car), (st, None, car), (st, dc, None)):
        assert sp(4, 2, 8, 64, 128, *args) == _lib.SSM_ERR_NULL
    assert L.ssd_state_passing(4, 2, 8, 64, 128, st, dc, None, None, None, None) == _lib.SSM_ERR_NULL


def _good_bwd(**kw):
    a = _lib.BwdArgs()
    a.batch, a.dim, a.seqlen, a.dstate, a.ngroups = 2, 64, 100, 16, 2
    a.io_dtype = _lib.SSM_BF16
    a.u = a.delta = a.A = a.B = a.C = a.checkpoints = a.dout = FAKE
    a.du = a.ddelta = a.dA = a.dB = a.dC = FAKE
    a.B_kind = a.C_kind = _lib.SSM_BC_VARYING
    a.delta_softplus = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_bwd_validation():
    L = _lib.lib()
    v = lambda a: L.ssm_scan_bwd_validate(ctypes.byref(a))
    assert v(_good_bwd()) == _lib.SSM_OK
    assert v(_good_bwd(z=FAKE, dz=FAKE, D=FAKE, dD=FAKE, delta_bias=FAKE, ddelta_bias=FAKE,
                       B_kind=_lib.SSM_BC_FIXED)) == _lib.SSM_OK
    for field in ("u", "delta", "A", "B", "C", "checkpoints", "dout", "du", "ddelta", "dA", "dB", "dC"):
        assert v(_good_bwd(**{field: None})) == _lib.SSM_ERR_NULL, field
    # an optional input asks for its gradient
    for inp, grad in (("z", "dz"), ("D", "dD"), ("delta_bias", "ddelta_bias")):
        assert v(_good_bwd(**{inp: FAKE})) == _lib.SSM_ERR_NULL, inp
    for field, val in (("batch", 0), ("dim", -1), ("seqlen", 0), ("dstate", 0), ("ngroups", 3)):
        assert v(_good_bwd(**{field: val})) == _lib.SSM_ERR_SHAPE, (field, val)
    for kw in (dict(io_dtype=7), dict(dstate=17), dict(B_kind=5), dict(delta_softplus=3)):
        assert v(_good_bwd(**kw)) == _lib.SSM_ERR_UNSUPPORTED, kw
    assert v(_good_bwd(batch=1 << 40, dim=1 << 20)) == _lib.SSM_ERR_SHAPE
    assert L.ssm_scan_bwd_validate(None) == _lib.SSM_ERR_NULL
    # rejected before any HIP call: usable without a GPU
    assert L.ssm_scan_bwd(ctypes.byref(_good_bwd(dout=None)), None) == _lib.SSM_ERR_NULL
    need = ctypes.c_size_t(0)
    assert L.ssm_scan_bwd_workspace_size(ctypes.byref(_good_bwd()), ctypes.byref(need)) == _lib.SSM_OK
    # partial dB/dC per 48-channel workgroup, dA per batch, dD and ddelta_bias per batch
    nblk = (64 // 2 + 47) // 48
    up = lambda e: (e * 4 + 255) // 256 * 256
    assert need.value == 2 * up(2 * 2 * nblk * 16 * 100) + up(2 * 64 * 16) + 2 * up(2 * 64)
    # a sequence split (100 timesteps: 4 chunks) keeps dA, dD, ddelta_bias per
    # (segment, batch) and adds each segment's carry and sum of delta'
    for segs, ns in ((2, 2), (3, 2), (4, 4), (1000, 4)):
        assert L.ssm_scan_bwd_workspace_size(ctypes.byref(_good_bwd(seq_segments=segs)),
                                             ctypes.byref(need)) == _lib.SSM_OK
        assert need.value == (2 * up(2 * 2 * nblk * 16 * 100) + up(ns * 2 * 64 * 16) + 2 * up(ns * 2 * 64)
                              + up(ns * 2 * 64 * 16) + up(ns * 2 * 64)), segs
    assert v(_good_bwd(seq_segments=-1)) == _lib.SSM_ERR_SHAPE
    # the backward always needs scratch, and allocates none itself
    a = _good_bwd()
    assert L.ssm_scan_bwd(ctypes.byref(a), None) == _lib.SSM_ERR_WORKSPACE
    L.ssm_scan_bwd_workspace_size(ctypes.byref(a), ctypes.byref(need))
    a.workspace, a.workspace_bytes = FAKE, need.value - 1
    assert L.ssm_scan_bwd(ctypes.byref(a), None) == _lib.SSM_ERR_WORKSPACE


def test_bwd_binding_errors():
    import torch
    from state_space_model_scan_amd import binding
    b, d, l, n = 1, 4, 10, 3
    u = torch.zeros(b, d, l)
    A = torch.zeros(d, n)
    B = torch.zeros(b, 1, n, l)
    ck = torch.zeros(b, d, 1, n)
    with pytest.raises(ValueError, match="checkpoints must have shape"):
        binding.ssm_scan_bwd(u, u, A, B, B, u, torch.zeros(b, d, 2, n))
    with pytest.raises(ValueError, match="io dtype"):
        binding.ssm_scan_bwd(u, u, A, B, B, u.to(torch.bfloat16), ck)
    with pytest.raises(ValueError, match="checkpoints must have shape"):
        binding.ssm_scan_fwd(u, u, A, B, B, checkpoints=torch.zeros(b, d, 2, n))


def _good_conv(**kw):
    a = _lib.ConvArgs()
    a.batch, a.dim, a.seqlen, a.width = 2, 8, 33, 4
    a.io_dtype, a.act = _lib.SSM_BF16, _lib.SSM_ACT_SILU
    a.x = a.weight = a.out = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_conv_ex_validation():
    L = _lib.lib()
    v = lambda a: L.causal_conv1d_ex_validate(ctypes.byref(a))
    assert v(_good_conv()) == _lib.SSM_OK
    assert v(_good_conv(initial_states=FAKE, final_states=FAKE, bias=FAKE)) == _lib.SSM_OK
    assert v(_good_conv(seq_idx=FAKE)) == _lib.SSM_OK
    for field in ("x", "weight", "out"):
        assert v(_good_conv(**{field: None})) == _lib.SSM_ERR_NULL, field
    assert v(_good_conv(seqlen=0)) == _lib.SSM_ERR_SHAPE
    assert v(_good_conv(width=3)) == _lib.SSM_ERR_UNSUPPORTED
    # the page: seq_idx excludes initial_states and the final states
    assert v(_good_conv(seq_idx=FAKE, initial_states=FAKE)) == _lib.SSM_ERR_UNSUPPORTED
    assert v(_good_conv(seq_idx=FAKE, final_states=FAKE)) == _lib.SSM_ERR_UNSUPPORTED
    assert L.causal_conv1d_ex_validate(None) == _lib.SSM_ERR_NULL
    assert L.causal_conv1d_fwd_ex(ctypes.byref(_good_conv(x=None)), None) == _lib.SSM_ERR_NULL


def test_conv_fn_binding_errors():
    import torch
    from state_space_model_scan_amd import binding
    x = torch.zeros(1, 2, 8)
    w = torch.zeros(2, 4)
    with pytest.raises(ValueError, match="seq_idx cannot be used"):
        binding.causal_conv1d_fn(x, w, seq_idx=torch.zeros(1, 8, dtype=torch.int32), return_final_states=True)
    with pytest.raises(ValueError, match="seq_idx must be int32"):
        binding.causal_conv1d_fwd_ex(x, w, seq_idx=torch.zeros(1, 8, dtype=torch.int64))
    with pytest.raises(ValueError, match="initial_states must be"):
        binding.causal_conv1d_fwd_ex(x, w, initial_states=torch.zeros(1, 2, 4))
    with pytest.raises(NotImplementedError):
        binding.causal_conv1d_fn(x, w, activation="relu")


def test_fp16_io_is_taken_by_all_but_the_mamba2_scan():
    L = _lib.lib()
    assert _validate(_good_args(io_dtype=_lib.SSM_F16)) == _lib.SSM_OK
    assert L.causal_conv1d_validate(FAKE, FAKE, FAKE, 1, 4, 8, 4, _lib.SSM_F16, 0) == _lib.SSM_OK
    assert L.causal_conv1d_ex_validate(ctypes.byref(_good_conv(io_dtype=_lib.SSM_F16))) == _lib.SSM_OK
    assert L.ssm_scan_bwd_validate(ctypes.byref(_good_bwd(io_dtype=_lib.SSM_F16))) == _lib.SSM_OK
    assert L.ssd_scan_validate(ctypes.byref(_good_ssd(io_dtype=_lib.SSM_F16))) == _lib.SSM_ERR_UNSUPPORTED


def test_complex_validation():
    """ssm_scan_fwd_complex: the real scan's checks, plus no conv prologue,
    no checkpoints and a required u; rejected before any HIP call."""
    L = _lib.lib()
    v = lambda a: L.ssm_scan_complex_validate(ctypes.byref(a))  # noqa: E731
    assert v(_good_args()) == _lib.SSM_OK
    assert v(_good_args(io_dtype=_lib.SSM_F16, dstate=3, B_kind=_lib.SSM_BC_FIXED)) == _lib.SSM_OK
    assert v(_good_args(u=None)) == _lib.SSM_ERR_NULL
    assert v(_good_args(A=None)) == _lib.SSM_ERR_NULL
    assert v(_good_args(ngroups=3)) == _lib.SSM_ERR_SHAPE
    assert v(_good_args(dstate=17)) == _lib.SSM_ERR_UNSUPPORTED
    assert v(_good_args(conv_weight=FAKE, conv_x=FAKE, conv_width=4)) == _lib.SSM_ERR_UNSUPPORTED
    assert v(_good_args(checkpoints=FAKE)) == _lib.SSM_OK   # the backward's saved states
    assert L.ssm_scan_complex_validate(None) == _lib.SSM_ERR_NULL
    assert L.ssm_scan_fwd_complex(ctypes.byref(_good_args(delta=None)), None) == _lib.SSM_ERR_NULL
    assert L.ssm_scan_fwd_complex(ctypes.byref(_good_args(conv_weight=FAKE, conv_x=FAKE, conv_width=4)),
                                  None) == _lib.SSM_ERR_UNSUPPORTED


def test_complex_binding_errors():
    import torch
    from state_space_model_scan_amd import binding
    u = torch.zeros(1, 4, 8)
    A = torch.zeros(4, 2, dtype=torch.complex64)
    Bv = torch.zeros(1, 2, 8, dtype=torch.complex64)
    with pytest.raises(ValueError, match="pair"):
        binding.ssm_scan_fwd_complex(u, u, A, torch.zeros(1, 2, 8, 3), Bv)
    with pytest.raises(ValueError, match="A must be"):
        binding.ssm_scan_fwd_complex(u, u, torch.zeros(4, 2), Bv, Bv)
    with pytest.raises(ValueError, match="io dtype"):
        binding.ssm_scan_fwd_complex(u, u, A, torch.zeros(1, 2, 8, 2, dtype=torch.bfloat16), Bv)


def test_plan_query():
    """ssm_scan_plan reports the plan ssm_scan_fwd takes.  Without a GPU the
    occupancy query fails, so the mixed plan is never chosen here."""
    L = _lib.lib()
    def plan(**kw):
        p = _lib.ScanPlan()
        assert L.ssm_scan_plan(ctypes.byref(_good_args(**kw)), ctypes.byref(p)) == _lib.SSM_OK
        return p
    p = plan(batch=8, dim=5120, ngroups=4, seqlen=2048)
    assert (p.segments, p.waves, p.lanes_per_channel, p.eight_lane_waves, p.workspace_bytes) == (1, 2560, 4, 0, 0)
    p = plan(batch=1, dim=2560, seqlen=65536)
    assert p.segments == 38 and p.waves == 160 and p.workspace_bytes > 0   # 6080 waves: <= 6 per SIMD
    need = ctypes.c_size_t(0)
    assert L.ssm_scan_workspace_size(ctypes.byref(_good_args(batch=1, dim=2560, seqlen=65536)),
                                     ctypes.byref(need)) == _lib.SSM_OK
    assert need.value == p.workspace_bytes
    assert plan(seq_segments=3, seqlen=960).segments == 3
    assert plan(seq_segments=3).segments == 2   # whole chunks of 32: 64 + 64
    assert plan(dstate=8).lanes_per_channel == 2 and plan(dstate=8).waves == 2 * 2
    assert L.ssm_scan_plan(ctypes.byref(_good_args(delta=None)), ctypes.byref(_lib.ScanPlan())) == _lib.SSM_ERR_NULL
    assert L.ssm_scan_plan(ctypes.byref(_good_args()), None) == _lib.SSM_ERR_NULL


def test_complex_bwd_validation():
    """ssm_scan_bwd_complex: the real backward's checks, any sequence split,
    and the workspace required before anything is enqueued (more segments,
    more partial sums)."""
    L = _lib.lib()
    v = lambda a: L.ssm_scan_bwd_complex_validate(ctypes.byref(a))  # noqa: E731
    assert v(_good_bwd()) == _lib.SSM_OK
    assert v(_good_bwd(seq_segments=1)) == _lib.SSM_OK
    assert v(_good_bwd(seq_segments=3)) == _lib.SSM_OK
    assert v(_good_bwd(seq_segments=-1)) == _lib.SSM_ERR_SHAPE
    sizes = []
    for k in (1, 3):
        need = ctypes.c_size_t(0)
        assert L.ssm_scan_bwd_complex_workspace_size(ctypes.byref(_good_bwd(seq_segments=k)),
                                                     ctypes.byref(need)) == _lib.SSM_OK
        sizes.append(need.value)
    assert sizes[1] > sizes[0]
    assert v(_good_bwd(checkpoints=None)) == _lib.SSM_ERR_NULL
    assert v(_good_bwd(dstate=17)) == _lib.SSM_ERR_UNSUPPORTED
    assert L.ssm_scan_bwd_complex_validate(None) == _lib.SSM_ERR_NULL
    a = _good_bwd()
    need = ctypes.c_size_t(0)
    assert L.ssm_scan_bwd_complex_workspace_size(ctypes.byref(a), ctypes.byref(need)) == _lib.SSM_OK
    assert need.value > 0
    assert L.ssm_scan_bwd_complex(ctypes.byref(a), None) == _lib.SSM_ERR_WORKSPACE
    a.workspace, a.workspace_bytes = FAKE, need.value - 1
    assert L.ssm_scan_bwd_complex(ctypes.byref(a), None) == _lib.SSM_ERR_WORKSPACE
