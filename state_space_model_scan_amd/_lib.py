"""ctypes view of libssmscan.so (include/ssmscan.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libssmscan.so")

SSM_F32, SSM_BF16, SSM_F16 = 0, 1, 2
SSM_BC_FIXED, SSM_BC_VARYING = 0, 1
SSM_ACT_NONE, SSM_ACT_SILU = 0, 1
SSM_OK, SSM_ERR_NULL, SSM_ERR_SHAPE, SSM_ERR_UNSUPPORTED, SSM_ERR_HIP, SSM_ERR_WORKSPACE, SSM_ERR_SCRATCH = range(7)
SSM_NOALLOC_SCRATCH_BYTES = 8 << 20
SSM_MAX_DSTATE = 16
SSM_CONV_WIDTH = 4
SSM_MAX_CONV_STATE = 256
SSD_HEADDIM = 64
SSD_CHUNK = 64
SSM_CKPT_INTERVAL = 32

# Every symbol include/ssmscan.h declares.
EXPORTS = (
    "ssm_scan_fwd", "ssm_scan_validate", "ssm_scan_workspace_size", "ssm_scan_fwd_noalloc", "ssm_scan_plan",
    "ssm_scan_fwd_complex", "ssm_scan_complex_validate",
    "causal_conv1d_fwd", "causal_conv1d_validate", "causal_conv1d_fwd_ex", "causal_conv1d_ex_validate",
    "ssm_state_update", "ssm_state_update_validate",
    "causal_conv1d_update", "causal_conv1d_update_validate",
    "ssd_scan_fwd", "ssd_scan_validate", "ssd_scan_workspace_size",
    "ssd_chunk_state", "ssd_chunk_state_validate", "ssd_state_passing", "ssd_state_passing_validate",
    "ssd_chunk_scan", "ssd_chunk_scan_validate",
    "ssm_scan_bwd", "ssm_scan_bwd_validate", "ssm_scan_bwd_workspace_size",
    "ssm_scan_bwd_complex", "ssm_scan_bwd_complex_validate", "ssm_scan_bwd_complex_workspace_size",
    "ssm_status_str", "ssm_last_hip_error", "ssm_abi_version",
)

_vp = ctypes.c_void_p


class ScanPlan(ctypes.Structure):
    """ssm_scan_plan_t"""
    _fields_ = [("segments", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("lanes_per_channel", ctypes.c_int32), ("eight_lane_waves", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


class ScanArgs(ctypes.Structure):
    """Mirror of ssm_scan_args_t."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("u", _vp), ("delta", _vp), ("A", _vp),
        ("B", _vp), ("B_kind", ctypes.c_int32),
        ("C", _vp), ("C_kind", ctypes.c_int32),
        ("D", _vp), ("delta_bias", _vp), ("z", _vp),
        ("delta_softplus", ctypes.c_int32),
        ("out", _vp), ("last_state", _vp), ("initial_state", _vp),
        ("conv_x", _vp), ("conv_weight", _vp), ("conv_bias", _vp),
        ("conv_width", ctypes.c_int32), ("conv_act", ctypes.c_int32),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("checkpoints", _vp),
        ("seq_segments", ctypes.c_int32),
    ]


class ConvArgs(ctypes.Structure):
    """Mirror of causal_conv1d_args_t."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("width", ctypes.c_int32), ("io_dtype", ctypes.c_int32), ("act", ctypes.c_int32),
        ("x", _vp), ("weight", _vp), ("bias", _vp), ("seq_idx", _vp), ("initial_states", _vp),
        ("out", _vp), ("final_states", _vp),
    ]


class BwdArgs(ctypes.Structure):
    """Mirror of ssm_scan_bwd_args_t."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("seqlen", ctypes.c_int64),
        ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("u", _vp), ("delta", _vp), ("A", _vp),
        ("B", _vp), ("B_kind", ctypes.c_int32),
        ("C", _vp), ("C_kind", ctypes.c_int32),
        ("D", _vp), ("delta_bias", _vp), ("z", _vp),
        ("delta_softplus", ctypes.c_int32),
        ("checkpoints", _vp), ("dout", _vp),
        ("du", _vp), ("ddelta", _vp), ("dz", _vp), ("dA", _vp), ("dB", _vp), ("dC", _vp),
        ("dD", _vp), ("ddelta_bias", _vp), ("dinitial_state", _vp),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("seq_segments", ctypes.c_int32),
    ]


class StateUpdateArgs(ctypes.Structure):
    """Mirror of ssm_state_update_args_t."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
        ("ngroups", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("state", _vp), ("x", _vp), ("dt", _vp), ("A", _vp), ("B", _vp), ("C", _vp),
        ("D", _vp), ("dt_bias", _vp), ("z", _vp),
        ("dt_softplus", ctypes.c_int32),
        ("out", _vp),
    ]


class SsdArgs(ctypes.Structure):
    """Mirror of ssd_scan_args_t."""
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
        ("io_dtype", ctypes.c_int32),
        ("x", _vp), ("dt", _vp), ("A", _vp), ("B", _vp), ("C", _vp),
        ("D", _vp), ("D_per_channel", ctypes.c_int32),
        ("z", _vp), ("dt_bias", _vp), ("dt_softplus", ctypes.c_int32),
        ("initial_states", _vp), ("out", _vp), ("final_states", _vp),
        ("dt_limit", ctypes.c_int32), ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float),
        ("seq_idx", _vp), ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("seq_segments", ctypes.c_int32),
    ]


class SsmError(ValueError):
    """A non-zero status from libssmscan."""

    def __init__(self, status: int, text: str):
        super().__init__(f"libssmscan status {status}: {text}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libssmscan.so; raises with a clear message when it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python -m state_space_model_scan_amd._build`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.ssm_scan_fwd.argtypes = [ctypes.POINTER(ScanArgs), _vp]
        L.ssm_scan_fwd.restype = ctypes.c_int
        L.ssm_scan_fwd_noalloc.argtypes = [ctypes.POINTER(ScanArgs), _vp]
        L.ssm_scan_fwd_noalloc.restype = ctypes.c_int
        L.ssm_scan_validate.argtypes = [ctypes.POINTER(ScanArgs)]
        L.ssm_scan_validate.restype = ctypes.c_int
        L.ssm_scan_workspace_size.argtypes = [ctypes.POINTER(ScanArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.ssm_scan_workspace_size.restype = ctypes.c_int
        L.ssm_scan_plan.argtypes = [ctypes.POINTER(ScanArgs), ctypes.POINTER(ScanPlan)]
        L.ssm_scan_plan.restype = ctypes.c_int
        L.ssm_scan_fwd_complex.argtypes = [ctypes.POINTER(ScanArgs), _vp]
        L.ssm_scan_fwd_complex.restype = ctypes.c_int
        L.ssm_scan_complex_validate.argtypes = [ctypes.POINTER(ScanArgs)]
        L.ssm_scan_complex_validate.restype = ctypes.c_int
        L.causal_conv1d_fwd.argtypes = [_vp, _vp, _vp, _vp, i64, i64, i64, i32, i32, i32, _vp]
        L.causal_conv1d_fwd.restype = ctypes.c_int
        L.causal_conv1d_validate.argtypes = [_vp, _vp, _vp, i64, i64, i64, i32, i32, i32]
        L.causal_conv1d_validate.restype = ctypes.c_int
        L.ssm_state_update.argtypes = [ctypes.POINTER(StateUpdateArgs), _vp]
        L.ssm_state_update.restype = ctypes.c_int
        L.ssm_state_update_validate.argtypes = [ctypes.POINTER(StateUpdateArgs)]
        L.ssm_state_update_validate.restype = ctypes.c_int
        L.causal_conv1d_update.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, i64, i64, i64, i64,
                                           i32, i32, i32, _vp]
        L.causal_conv1d_update.restype = ctypes.c_int
        L.causal_conv1d_update_validate.argtypes = [_vp, _vp, _vp, _vp, i64, i64, i64, i64,
                                                    i32, i32, i32]
        L.causal_conv1d_update_validate.restype = ctypes.c_int
        L.ssd_scan_fwd.argtypes = [ctypes.POINTER(SsdArgs), _vp]
        L.ssd_scan_fwd.restype = ctypes.c_int
        L.ssd_scan_validate.argtypes = [ctypes.POINTER(SsdArgs)]
        L.ssd_scan_validate.restype = ctypes.c_int
        L.ssd_scan_workspace_size.argtypes = [ctypes.POINTER(SsdArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.ssd_scan_workspace_size.restype = ctypes.c_int
        i64 = ctypes.c_int64
        L.ssd_chunk_state.argtypes = [ctypes.POINTER(SsdArgs), i64, _vp, _vp, _vp]
        L.ssd_chunk_state.restype = ctypes.c_int
        L.ssd_chunk_state_validate.argtypes = [ctypes.POINTER(SsdArgs), i64, _vp, _vp]
        L.ssd_chunk_state_validate.restype = ctypes.c_int
        L.ssd_state_passing.argtypes = [i64, i64, i64, i64, i64, _vp, _vp, _vp, _vp, _vp, _vp]
        L.ssd_state_passing.restype = ctypes.c_int
        L.ssd_state_passing_validate.argtypes = [i64, i64, i64, i64, i64, _vp, _vp, _vp]
        L.ssd_state_passing_validate.restype = ctypes.c_int
        L.ssd_chunk_scan.argtypes = [ctypes.POINTER(SsdArgs), i64, _vp, _vp]
        L.ssd_chunk_scan.restype = ctypes.c_int
        L.ssd_chunk_scan_validate.argtypes = [ctypes.POINTER(SsdArgs), i64, _vp]
        L.ssd_chunk_scan_validate.restype = ctypes.c_int
        L.causal_conv1d_fwd_ex.argtypes = [ctypes.POINTER(ConvArgs), _vp]
        L.causal_conv1d_fwd_ex.restype = ctypes.c_int
        L.causal_conv1d_ex_validate.argtypes = [ctypes.POINTER(ConvArgs)]
        L.causal_conv1d_ex_validate.restype = ctypes.c_int
        L.ssm_scan_bwd.argtypes = [ctypes.POINTER(BwdArgs), _vp]
        L.ssm_scan_bwd.restype = ctypes.c_int
        L.ssm_scan_bwd_validate.argtypes = [ctypes.POINTER(BwdArgs)]
        L.ssm_scan_bwd_validate.restype = ctypes.c_int
        L.ssm_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(BwdArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.ssm_scan_bwd_workspace_size.restype = ctypes.c_int
        L.ssm_scan_bwd_complex.argtypes = [ctypes.POINTER(BwdArgs), _vp]
        L.ssm_scan_bwd_complex.restype = ctypes.c_int
        L.ssm_scan_bwd_complex_validate.argtypes = [ctypes.POINTER(BwdArgs)]
        L.ssm_scan_bwd_complex_validate.restype = ctypes.c_int
        L.ssm_scan_bwd_complex_workspace_size.argtypes = [ctypes.POINTER(BwdArgs), ctypes.POINTER(ctypes.c_size_t)]
        L.ssm_scan_bwd_complex_workspace_size.restype = ctypes.c_int
        L.ssm_status_str.argtypes = [ctypes.c_int]
        L.ssm_status_str.restype = ctypes.c_char_p
        L.ssm_last_hip_error.argtypes = []
        L.ssm_last_hip_error.restype = ctypes.c_int
        L.ssm_abi_version.argtypes = []
        L.ssm_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != SSM_OK:
        text = lib().ssm_status_str(status).decode()
        if status == SSM_ERR_HIP:
            text += f" (hipError_t {lib().ssm_last_hip_error()})"
        raise SsmError(status, text)
