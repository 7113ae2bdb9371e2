"""Python binding of libssmscan.so.  Argument marshalling only: every step of
the operator runs in the HIP kernels behind the C ABI; torch provides device
memory and the current stream.

``ssm_scan_fwd`` / ``causal_conv1d_fwd`` mirror the C entry points.
``selective_scan_fn`` / ``causal_conv1d_fn`` keep the signatures the page
gives (PaddleNLP Kernel operator-library guide, sections 4.1 and 4.2),
forward only: tensors whose last stride is not 1 are made contiguous, a 3-D
B/C (batch, dstate, seqlen) is the grouped form with one group, and an
activation other than None / "silu" / "swish" raises NotImplementedError.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple, Union

import torch

from . import _lib
from ._lib import BwdArgs, ConvArgs, ScanArgs, check

_IO = {torch.float32: _lib.SSM_F32, torch.bfloat16: _lib.SSM_BF16, torch.float16: _lib.SSM_F16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dense(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if t is None:
        return None
    return t if t.is_contiguous() else t.contiguous()


def _stream(device: torch.device, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


# Every wrapper checks each tensor against the sizes that delta (or x) and A
# fix before it hands a pointer to the library: the kernels index their
# buffers with those sizes, so a wrong shape, dtype or device would be an
# access outside a buffer, not an error.

def _spec(t: Optional[torch.Tensor], name: str, shape, dtype, dev: torch.device) -> None:
    """Raise ValueError unless t (when given) has this shape and dtype and
    lives on dev."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != dev:
        raise ValueError(f"{name} must be on {dev} with the other tensors, got {t.device}")


def _out_spec(t: Optional[torch.Tensor], name: str, shape, dtype, dev: torch.device) -> None:
    """_spec for a tensor the library writes in place: also contiguous (the
    kernels write it as a dense row-major array)."""
    _spec(t, name, shape, dtype, dev)
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} is written in place and must be contiguous")


def _on_gpu(dev: torch.device) -> None:
    if dev.type != "cuda":
        raise ValueError(f"the operator runs on the GPU: tensors must be on a cuda device, got {dev}")


def _io_of(t: torch.Tensor, name: str, ndim: int) -> int:
    io = _IO.get(t.dtype)
    if io is None:
        raise ValueError(f"io dtype must be float32, bfloat16 or float16, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return io


def _workspace_spec(ws: torch.Tensor, dev: torch.device) -> None:
    if ws.device != dev or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {dev}")


def _conv_params_spec(weight: torch.Tensor, bias: Optional[torch.Tensor], dim: int,
                      dev: torch.device) -> None:
    if weight.dim() != 2:
        raise ValueError(f"conv weight must be (dim, width), got shape {tuple(weight.shape)}")
    _spec(weight, "weight", (dim, weight.shape[1]), torch.float32, dev)
    _spec(bias, "bias", (dim,), torch.float32, dev)


def _bc_shape(t: torch.Tensor, kind: int, ngroups: int, batch: int, dim: int, dstate: int,
              seqlen: int, tail=()) -> tuple:
    """The shape a B or C of this kind must have (tail: the pair axis)."""
    if kind == _lib.SSM_BC_FIXED:
        return (dim, dstate) + tail
    if t.dim() == 3 + len(tail):
        return (batch, dstate, seqlen) + tail
    return (batch, ngroups, dstate, seqlen) + tail


def _bc_kind(t: torch.Tensor, name: str) -> Tuple[int, int]:
    """(kind, ngroups) of a B or C tensor from its rank."""
    if t.dim() == 2:
        return _lib.SSM_BC_FIXED, 0
    if t.dim() == 3:
        return _lib.SSM_BC_VARYING, 1
    if t.dim() == 4:
        return _lib.SSM_BC_VARYING, t.shape[1]
    raise ValueError(f"{name} must be (dim, dstate), (batch, dstate, seqlen) or "
                     f"(batch, groups, dstate, seqlen); got shape {tuple(t.shape)}")


def _act_code(activation) -> int:
    if activation is None:
        return _lib.SSM_ACT_NONE
    if activation in ("silu", "swish"):
        return _lib.SSM_ACT_SILU
    raise NotImplementedError("activation must be None, silu, or swish")


def _scan_args(u, delta, A, B, C, D, z, delta_bias, delta_softplus, out, last_state, initial_state,
               conv_x, conv_weight, conv_bias, conv_act, checkpoints, seq_segments):
    """ssm_scan_args_t for the tensors (made contiguous where needed); returns
    (args, out, tensors kept alive until the call is enqueued)."""
    delta = _dense(delta)
    io = _io_of(delta, "delta", 3)
    batch, dim, seqlen = delta.shape
    if A.dim() != 2 or A.shape[0] != dim:
        raise ValueError(f"A must be (dim, dstate) with dim {dim}, got shape {tuple(A.shape)}")
    dstate = A.shape[1]
    B, C = _dense(B), _dense(C)
    bk, bg = _bc_kind(B, "B")
    ck, cg = _bc_kind(C, "C")
    if bk == _lib.SSM_BC_VARYING and ck == _lib.SSM_BC_VARYING and bg != cg:
        raise ValueError("B and C must have the same number of groups")
    ngroups = max(bg, cg, 1)
    for name, t in (("u", u), ("z", z), ("B", B), ("C", C), ("conv_x", conv_x)):
        if t is not None and t.dtype != delta.dtype:
            raise ValueError(f"{name} must have the io dtype {delta.dtype}, got {t.dtype}")
    for name, t in (("A", A), ("D", D), ("delta_bias", delta_bias), ("initial_state", initial_state),
                    ("conv_weight", conv_weight), ("conv_bias", conv_bias)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32, got {t.dtype}")
    dev, f32, bld, bdn = delta.device, torch.float32, (batch, dim, seqlen), (batch, dim, dstate)
    for name, t in (("u", u), ("z", z), ("conv_x", conv_x)):
        _spec(t, name, bld, delta.dtype, dev)
    _spec(A, "A", (dim, dstate), f32, dev)
    _spec(B, "B", _bc_shape(B, bk, ngroups, batch, dim, dstate, seqlen), delta.dtype, dev)
    _spec(C, "C", _bc_shape(C, ck, ngroups, batch, dim, dstate, seqlen), delta.dtype, dev)
    for name, t in (("D", D), ("delta_bias", delta_bias), ("conv_bias", conv_bias)):
        _spec(t, name, (dim,), f32, dev)
    _spec(initial_state, "initial_state", bdn, f32, dev)
    if conv_weight is not None:
        if conv_weight.dim() != 2:
            raise ValueError(f"conv_weight must be (dim, width), got shape {tuple(conv_weight.shape)}")
        _spec(conv_weight, "conv_weight", (dim, conv_weight.shape[1]), f32, dev)
        if conv_x is None:
            raise ValueError("the conv prologue needs conv_x")
    elif u is None:
        raise ValueError("u is required without the conv prologue")
    _out_spec(out, "out", bld, delta.dtype, dev)
    _out_spec(last_state, "last_state", bdn, f32, dev)
    if checkpoints is not None:
        _out_spec(checkpoints, "checkpoints", (batch, dim, checkpoint_count(seqlen), dstate), f32, dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty_like(delta)
    args = ScanArgs()
    args.batch, args.dim, args.seqlen, args.dstate, args.ngroups = batch, dim, seqlen, dstate, ngroups
    args.io_dtype = io
    u, A, D, z, delta_bias = _dense(u), _dense(A), _dense(D), _dense(z), _dense(delta_bias)
    initial_state, conv_x = _dense(initial_state), _dense(conv_x)
    conv_weight, conv_bias = _dense(conv_weight), _dense(conv_bias)
    args.u, args.delta, args.A = _ptr(u), _ptr(delta), _ptr(A)
    args.B, args.B_kind, args.C, args.C_kind = _ptr(B), bk, _ptr(C), ck
    args.D, args.delta_bias, args.z = _ptr(D), _ptr(delta_bias), _ptr(z)
    args.delta_softplus = int(bool(delta_softplus))
    args.out, args.last_state, args.initial_state = _ptr(out), _ptr(last_state), _ptr(initial_state)
    args.conv_x, args.conv_weight, args.conv_bias = _ptr(conv_x), _ptr(conv_weight), _ptr(conv_bias)
    args.conv_width = 0 if conv_weight is None else conv_weight.shape[1]
    args.conv_act = conv_act
    args.seq_segments = int(seq_segments)
    if checkpoints is not None:
        args.checkpoints = _ptr(checkpoints)
    keep = (u, delta, A, B, C, D, z, delta_bias, initial_state, conv_x, conv_weight, conv_bias)
    return args, out, keep


def ssm_scan_fwd(u: Optional[torch.Tensor], delta: torch.Tensor, A: torch.Tensor,
                 B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                 z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                 delta_softplus: bool = False, out: Optional[torch.Tensor] = None,
                 last_state: Optional[torch.Tensor] = None,
                 initial_state: Optional[torch.Tensor] = None,
                 conv_x: Optional[torch.Tensor] = None, conv_weight: Optional[torch.Tensor] = None,
                 conv_bias: Optional[torch.Tensor] = None, conv_act: int = _lib.SSM_ACT_SILU,
                 workspace: Optional[torch.Tensor] = None, stream=None,
                 checkpoints: Optional[torch.Tensor] = None, seq_segments: int = 0) -> torch.Tensor:
    """Enqueue ssm_scan_fwd on the current stream; returns ``out``.

    Shapes as in include/ssmscan.h.  ``out`` (same dtype as delta) and
    ``last_state`` (float32, optional) are written in place; ``out`` is
    allocated when not given.  With ``conv_weight`` the conv prologue computes
    u from ``conv_x`` and ``u`` may be None.  ``checkpoints`` (float32,
    (batch, dim, ceil(seqlen / 32), dstate), optional) receives the states the
    backward starts its chunks from.  ``seq_segments`` (0: the library's
    choice) asks for a sequence split into that many parallel segments.  The
    scratch the plan needs is allocated here (torch) unless ``workspace`` is
    given.
    """
    args, out, keep = _scan_args(u, delta, A, B, C, D, z, delta_bias, delta_softplus, out, last_state,
                                 initial_state, conv_x, conv_weight, conv_bias, conv_act, checkpoints,
                                 seq_segments)
    L = _lib.lib()
    if workspace is None:
        need = ctypes.c_size_t(0)
        check(L.ssm_scan_workspace_size(ctypes.byref(args), ctypes.byref(need)))
        if need.value:
            workspace = torch.empty(need.value, dtype=torch.uint8, device=delta.device)
    if workspace is not None:
        _workspace_spec(workspace, delta.device)
        args.workspace, args.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    check(L.ssm_scan_fwd(ctypes.byref(args), _stream(delta.device, stream)))
    return out


def ssm_scan_plan(u: Optional[torch.Tensor], delta: torch.Tensor, A: torch.Tensor,
                  B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                  z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                  delta_softplus: bool = False, out: Optional[torch.Tensor] = None,
                  last_state: Optional[torch.Tensor] = None,
                  initial_state: Optional[torch.Tensor] = None,
                  conv_x: Optional[torch.Tensor] = None, conv_weight: Optional[torch.Tensor] = None,
                  conv_bias: Optional[torch.Tensor] = None, conv_act: int = _lib.SSM_ACT_SILU,
                  checkpoints: Optional[torch.Tensor] = None, seq_segments: int = 0) -> dict:
    """The plan ssm_scan_fwd takes for these tensors (ssm_scan_plan): a dict
    of segments, waves, lanes_per_channel, eight_lane_waves and
    workspace_bytes.  ``out`` should be the tensor the call will write (its
    alignment is part of the plan)."""
    args, out, keep = _scan_args(u, delta, A, B, C, D, z, delta_bias, delta_softplus, out, last_state,
                                 initial_state, conv_x, conv_weight, conv_bias, conv_act, checkpoints,
                                 seq_segments)
    plan = _lib.ScanPlan()
    check(_lib.lib().ssm_scan_plan(ctypes.byref(args), ctypes.byref(plan)))
    return {k: getattr(plan, k) for k, _ in _lib.ScanPlan._fields_}


def ssm_scan_fwd_noalloc(u: Optional[torch.Tensor], delta: torch.Tensor, A: torch.Tensor,
                         B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                         z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                         delta_softplus: bool = False, out: Optional[torch.Tensor] = None,
                         last_state: Optional[torch.Tensor] = None,
                         initial_state: Optional[torch.Tensor] = None,
                         conv_x: Optional[torch.Tensor] = None, conv_weight: Optional[torch.Tensor] = None,
                         conv_bias: Optional[torch.Tensor] = None, conv_act: int = _lib.SSM_ACT_SILU,
                         stream=None, checkpoints: Optional[torch.Tensor] = None,
                         seq_segments: int = 0) -> torch.Tensor:
    """Enqueue ssm_scan_fwd_noalloc: ssm_scan_fwd with the plan's scratch in
    the library's built-in per-device buffer (nothing allocated for it).
    ``out`` must be given: a missing output would be an allocation."""
    if out is None:
        raise ValueError("ssm_scan_fwd_noalloc needs a caller-allocated out")
    args, out, keep = _scan_args(u, delta, A, B, C, D, z, delta_bias, delta_softplus, out, last_state,
                                 initial_state, conv_x, conv_weight, conv_bias, conv_act, checkpoints,
                                 seq_segments)
    check(_lib.lib().ssm_scan_fwd_noalloc(ctypes.byref(args), _stream(delta.device, stream)))
    return out


def _pairs(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    """A complex tensor as its (real, imaginary) pairs; other tensors as given."""
    if t is None:
        return None
    return torch.view_as_real(t) if t.is_complex() else t


def _bc_kind_complex(t: torch.Tensor, name: str) -> Tuple[int, int]:
    """(kind, ngroups) of a complex B or C given as pairs (trailing axis 2)."""
    if t.shape[-1] != 2:
        raise ValueError(f"{name} must be complex or end in a (real, imaginary) pair axis")
    kind, g = _bc_kind(t[..., 0], name)
    return kind, g


def ssm_scan_fwd_complex(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor,
                         B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                         z: Optional[torch.Tensor] = None,
                         delta_bias: Optional[torch.Tensor] = None,
                         delta_softplus: bool = False, out: Optional[torch.Tensor] = None,
                         last_state: Optional[torch.Tensor] = None,
                         initial_state: Optional[torch.Tensor] = None,
                         stream=None, checkpoints: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Enqueue ssm_scan_fwd_complex on the current stream; returns ``out``.

    A is complex64 (dim, dstate) or float32 pairs (dim, dstate, 2).  B and C
    are complex64 (fp32 io) or io-dtype pairs: fixed (dim, dstate, 2), varying
    (batch, dstate, seqlen, 2) or (batch, groups, dstate, seqlen, 2).
    ``last_state`` / ``initial_state`` are complex64 or float32 pairs
    (batch, dim, dstate, 2).  u, delta, z and out are real, as in ssm_scan_fwd.
    """
    delta = _dense(delta)
    io = _io_of(delta, "delta", 3)
    batch, dim, seqlen = delta.shape
    A, B, C = _pairs(A), _pairs(B), _pairs(C)
    initial_state = _pairs(initial_state)
    if last_state is not None:
        last_state = _pairs(last_state)
        if not last_state.is_contiguous():
            raise ValueError("last_state must be contiguous")
    if A.dim() != 3 or A.shape[-1] != 2 or A.shape[0] != dim:
        raise ValueError(f"A must be complex (dim, dstate) or float32 pairs (dim, dstate, 2) with dim {dim}")
    dstate = A.shape[1]
    if B.dim() == 4:
        B = B.unsqueeze(1)
    if C.dim() == 4:
        C = C.unsqueeze(1)
    B, C = _dense(B), _dense(C)
    bk, bg = _bc_kind_complex(B, "B")
    ck, cg = _bc_kind_complex(C, "C")
    if bk == _lib.SSM_BC_VARYING and ck == _lib.SSM_BC_VARYING and bg != cg:
        raise ValueError("B and C must have the same number of groups")
    ngroups = max(bg, cg, 1)
    for name, t in (("u", u), ("z", z), ("B", B), ("C", C)):
        if t is not None and t.dtype != delta.dtype:
            raise ValueError(f"{name} must have the io dtype {delta.dtype} (as pairs), got {t.dtype}")
    for name, t in (("A", A), ("D", D), ("delta_bias", delta_bias), ("initial_state", initial_state),
                    ("last_state", last_state)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 (complex64 for A and the states), got {t.dtype}")
    if u is None:
        raise ValueError("u is required")
    dev, f32, bld, bdn2 = delta.device, torch.float32, (batch, dim, seqlen), (batch, dim, dstate, 2)
    _spec(u, "u", bld, delta.dtype, dev)
    _spec(z, "z", bld, delta.dtype, dev)
    _spec(A, "A", (dim, dstate, 2), f32, dev)
    _spec(B, "B", _bc_shape(B, bk, ngroups, batch, dim, dstate, seqlen, (2,)), delta.dtype, dev)
    _spec(C, "C", _bc_shape(C, ck, ngroups, batch, dim, dstate, seqlen, (2,)), delta.dtype, dev)
    _spec(D, "D", (dim,), f32, dev)
    _spec(delta_bias, "delta_bias", (dim,), f32, dev)
    _spec(initial_state, "initial_state", bdn2, f32, dev)
    _out_spec(out, "out", bld, delta.dtype, dev)
    _out_spec(last_state, "last_state", bdn2, f32, dev)
    if checkpoints is not None:
        _out_spec(checkpoints, "checkpoints", (batch, dim, checkpoint_count(seqlen), dstate, 2), f32, dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty_like(delta)
    args = ScanArgs()
    args.batch, args.dim, args.seqlen, args.dstate, args.ngroups = batch, dim, seqlen, dstate, ngroups
    args.io_dtype = io
    u, A, D, z, delta_bias = _dense(u), _dense(A), _dense(D), _dense(z), _dense(delta_bias)
    initial_state = _dense(initial_state)
    args.u, args.delta, args.A = _ptr(u), _ptr(delta), _ptr(A)
    args.B, args.B_kind, args.C, args.C_kind = _ptr(B), bk, _ptr(C), ck
    args.D, args.delta_bias, args.z = _ptr(D), _ptr(delta_bias), _ptr(z)
    args.delta_softplus = int(bool(delta_softplus))
    args.out, args.last_state, args.initial_state = _ptr(out), _ptr(last_state), _ptr(initial_state)
    args.checkpoints = _ptr(checkpoints)
    check(_lib.lib().ssm_scan_fwd_complex(ctypes.byref(args), _stream(delta.device, stream)))
    return out


def checkpoint_count(seqlen: int) -> int:
    """Saved states per channel: one every SSM_CKPT_INTERVAL timesteps."""
    return (seqlen + _lib.SSM_CKPT_INTERVAL - 1) // _lib.SSM_CKPT_INTERVAL


def ssm_scan_bwd(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                 C: torch.Tensor, dout: torch.Tensor, checkpoints: torch.Tensor,
                 D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                 delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
                 want_dinitial_state: bool = False, workspace: Optional[torch.Tensor] = None,
                 seq_segments: int = 0, stream=None) -> dict:
    """Enqueue ssm_scan_bwd; returns the gradients in a dict.

    Inputs as for ``ssm_scan_fwd`` (B/C 2-D fixed or 4-D grouped), ``dout`` in
    the io dtype and the ``checkpoints`` that forward call wrote.  du, ddelta
    and dz come back in the io dtype; dA, dB, dC, dD, ddelta_bias and
    dinitial_state in float32 (dB/dC in B's/C's layout).  ``seq_segments``
    caps the sequence split (0: the library's choice).
    """
    delta = _dense(delta)
    io = _io_of(delta, "delta", 3)
    batch, dim, seqlen = delta.shape
    if A.dim() != 2 or A.shape[0] != dim:
        raise ValueError(f"A must be (dim, dstate) with dim {dim}, got shape {tuple(A.shape)}")
    dstate = A.shape[1]
    u, B, C, z, dout = _dense(u), _dense(B), _dense(C), _dense(z), _dense(dout)
    bk, bg = _bc_kind(B, "B")
    ck, cg = _bc_kind(C, "C")
    if bk == _lib.SSM_BC_VARYING and ck == _lib.SSM_BC_VARYING and bg != cg:
        raise ValueError("B and C must have the same number of groups")
    ngroups = max(bg, cg, 1)
    for name, t in (("u", u), ("z", z), ("B", B), ("C", C), ("dout", dout)):
        if t is not None and t.dtype != delta.dtype:
            raise ValueError(f"{name} must have the io dtype {delta.dtype}, got {t.dtype}")
    for name, t in (("A", A), ("D", D), ("delta_bias", delta_bias), ("checkpoints", checkpoints)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32, got {t.dtype}")
    dev, bld = delta.device, (batch, dim, seqlen)
    for name, t in (("u", u), ("dout", dout), ("z", z)):
        _spec(t, name, bld, delta.dtype, dev)
    _spec(A, "A", (dim, dstate), torch.float32, dev)
    _spec(B, "B", _bc_shape(B, bk, ngroups, batch, dim, dstate, seqlen), delta.dtype, dev)
    _spec(C, "C", _bc_shape(C, ck, ngroups, batch, dim, dstate, seqlen), delta.dtype, dev)
    _spec(D, "D", (dim,), torch.float32, dev)
    _spec(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    _spec(checkpoints, "checkpoints", (batch, dim, checkpoint_count(seqlen), dstate), torch.float32, dev)
    if workspace is not None:
        _workspace_spec(workspace, dev)
    _on_gpu(dev)
    A, D, delta_bias, checkpoints = _dense(A), _dense(D), _dense(delta_bias), _dense(checkpoints)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {
        "du": torch.empty_like(delta), "ddelta": torch.empty_like(delta),
        "dz": None if z is None else torch.empty_like(delta),
        "dA": torch.empty((dim, dstate), **f32),
        "dB": torch.empty(B.shape, **f32), "dC": torch.empty(C.shape, **f32),
        "dD": None if D is None else torch.empty((dim,), **f32),
        "ddelta_bias": None if delta_bias is None else torch.empty((dim,), **f32),
        "dinitial_state": torch.empty((batch, dim, dstate), **f32) if want_dinitial_state else None,
    }
    args = BwdArgs()
    args.batch, args.dim, args.seqlen, args.dstate, args.ngroups = batch, dim, seqlen, dstate, ngroups
    args.io_dtype = io
    args.u, args.delta, args.A = _ptr(u), _ptr(delta), _ptr(A)
    args.B, args.B_kind, args.C, args.C_kind = _ptr(B), bk, _ptr(C), ck
    args.D, args.delta_bias, args.z = _ptr(D), _ptr(delta_bias), _ptr(z)
    args.delta_softplus = int(bool(delta_softplus))
    args.checkpoints, args.dout = _ptr(checkpoints), _ptr(dout)
    args.seq_segments = int(seq_segments)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dinitial_state"):
        setattr(args, k, _ptr(g[k]))
    L = _lib.lib()
    if workspace is None:
        need = ctypes.c_size_t(0)
        check(L.ssm_scan_bwd_workspace_size(ctypes.byref(args), ctypes.byref(need)))
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
    args.workspace, args.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    check(L.ssm_scan_bwd(ctypes.byref(args), _stream(dev, stream)))
    return g


def ssm_scan_bwd_complex(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                         C: torch.Tensor, dout: torch.Tensor, checkpoints: torch.Tensor,
                         D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                         delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
                         want_dinitial_state: bool = False, workspace: Optional[torch.Tensor] = None,
                         seq_segments: int = 0, stream=None) -> dict:
    """Enqueue ssm_scan_bwd_complex; returns the gradients in a dict.

    Inputs as for ``ssm_scan_fwd_complex`` (A complex64 or float32 pairs
    (dim, dstate, 2); B/C complex64 or io-dtype pairs, fixed (dim, dstate, 2)
    or grouped (batch, groups, dstate, seqlen, 2)), ``dout`` in the io dtype
    and the ``checkpoints`` (batch, dim, nck, dstate, 2) float32 that forward
    call wrote.  du, ddelta, dz come back in the io dtype; dD, ddelta_bias in
    float32; dA, dB, dC and dinitial_state as float32 (real, imaginary)
    pairs in A's, B's, C's and the state's layouts (``torch.view_as_complex``
    turns them into complex64).  ``seq_segments`` caps the sequence split
    (0: the library's choice)."""
    delta = _dense(delta)
    io = _io_of(delta, "delta", 3)
    batch, dim, seqlen = delta.shape
    A, B, C = _pairs(A), _pairs(B), _pairs(C)
    if A.dim() != 3 or A.shape[-1] != 2 or A.shape[0] != dim:
        raise ValueError(f"A must be complex (dim, dstate) or float32 pairs (dim, dstate, 2) with dim {dim}")
    dstate = A.shape[1]
    if B.dim() == 4:
        B = B.unsqueeze(1)
    if C.dim() == 4:
        C = C.unsqueeze(1)
    u, B, C, z, dout, A = _dense(u), _dense(B), _dense(C), _dense(z), _dense(dout), _dense(A)
    bk, bg = _bc_kind_complex(B, "B")
    ck, cg = _bc_kind_complex(C, "C")
    if bk == _lib.SSM_BC_VARYING and ck == _lib.SSM_BC_VARYING and bg != cg:
        raise ValueError("B and C must have the same number of groups")
    ngroups = max(bg, cg, 1)
    for name, t in (("u", u), ("z", z), ("B", B), ("C", C), ("dout", dout)):
        if t is not None and t.dtype != delta.dtype:
            raise ValueError(f"{name} must have the io dtype {delta.dtype} (as pairs), got {t.dtype}")
    dev, f32, bld = delta.device, torch.float32, (batch, dim, seqlen)
    for name, t in (("u", u), ("dout", dout), ("z", z)):
        _spec(t, name, bld, delta.dtype, dev)
    _spec(A, "A", (dim, dstate, 2), f32, dev)
    _spec(B, "B", _bc_shape(B, bk, ngroups, batch, dim, dstate, seqlen, (2,)), delta.dtype, dev)
    _spec(C, "C", _bc_shape(C, ck, ngroups, batch, dim, dstate, seqlen, (2,)), delta.dtype, dev)
    _spec(D, "D", (dim,), f32, dev)
    _spec(delta_bias, "delta_bias", (dim,), f32, dev)
    _spec(checkpoints, "checkpoints", (batch, dim, checkpoint_count(seqlen), dstate, 2), f32, dev)
    if workspace is not None:
        _workspace_spec(workspace, dev)
    _on_gpu(dev)
    D, delta_bias, checkpoints = _dense(D), _dense(delta_bias), _dense(checkpoints)
    g = {
        "du": torch.empty_like(delta), "ddelta": torch.empty_like(delta),
        "dz": None if z is None else torch.empty_like(delta),
        "dA": torch.empty((dim, dstate, 2), dtype=f32, device=dev),
        "dB": torch.empty(B.shape, dtype=f32, device=dev), "dC": torch.empty(C.shape, dtype=f32, device=dev),
        "dD": None if D is None else torch.empty((dim,), dtype=f32, device=dev),
        "ddelta_bias": None if delta_bias is None else torch.empty((dim,), dtype=f32, device=dev),
        "dinitial_state": (torch.empty((batch, dim, dstate, 2), dtype=f32, device=dev)
                           if want_dinitial_state else None),
    }
    args = BwdArgs()
    args.batch, args.dim, args.seqlen, args.dstate, args.ngroups = batch, dim, seqlen, dstate, ngroups
    args.io_dtype = io
    args.u, args.delta, args.A = _ptr(u), _ptr(delta), _ptr(A)
    args.B, args.B_kind, args.C, args.C_kind = _ptr(B), bk, _ptr(C), ck
    args.D, args.delta_bias, args.z = _ptr(D), _ptr(delta_bias), _ptr(z)
    args.delta_softplus = int(bool(delta_softplus))
    args.checkpoints, args.dout = _ptr(checkpoints), _ptr(dout)
    args.seq_segments = int(seq_segments)
    for k in ("du", "ddelta", "dz", "dA", "dB", "dC", "dD", "ddelta_bias", "dinitial_state"):
        setattr(args, k, _ptr(g[k]))
    L = _lib.lib()
    if workspace is None:
        need = ctypes.c_size_t(0)
        check(L.ssm_scan_bwd_complex_workspace_size(ctypes.byref(args), ctypes.byref(need)))
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
    args.workspace, args.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    check(L.ssm_scan_bwd_complex(ctypes.byref(args), _stream(dev, stream)))
    return g


def causal_conv1d_fwd(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, act: int = _lib.SSM_ACT_NONE,
                      stream=None) -> torch.Tensor:
    """Enqueue causal_conv1d_fwd on the current stream; returns ``out``."""
    x = _dense(x)
    io = _io_of(x, "x", 3)
    weight, bias = _dense(weight), _dense(bias)
    if weight.dtype != torch.float32 or (bias is not None and bias.dtype != torch.float32):
        raise ValueError("conv weight and bias must be float32")
    batch, dim, seqlen = x.shape
    _conv_params_spec(weight, bias, dim, x.device)
    _out_spec(out, "out", (batch, dim, seqlen), x.dtype, x.device)
    _on_gpu(x.device)
    if out is None:
        out = torch.empty_like(x)
    check(_lib.lib().causal_conv1d_fwd(_ptr(x), _ptr(weight), _ptr(bias), _ptr(out),
                                       batch, dim, seqlen, weight.shape[1], io, act,
                                       _stream(x.device, stream)))
    return out


def selective_scan_fn(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                      delta_softplus=False, return_last_state=False
                      ) -> Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]]:
    """Forward of selective_scan_fn with the page's signature and returns.
    A complex A (section 4.1: real or complex) runs ssm_scan_fwd_complex;
    its B and C are then complex too (complex64, or io-dtype pairs), and
    last_state is complex64."""
    if A.is_complex():
        last = None
        if return_last_state:
            last = torch.empty((delta.shape[0], delta.shape[1], A.shape[1]), dtype=torch.complex64,
                               device=delta.device)
        out = ssm_scan_fwd_complex(u, delta, A, B, C, D, z, delta_bias, delta_softplus,
                                   last_state=last)
        return (out, last) if return_last_state else out
    if B.dim() == 3:
        B = B.unsqueeze(1)
    if C.dim() == 3:
        C = C.unsqueeze(1)
    last = None
    if return_last_state:
        last = torch.empty((delta.shape[0], delta.shape[1], A.shape[1]), dtype=torch.float32,
                           device=delta.device)
    out = ssm_scan_fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, last_state=last)
    return (out, last) if return_last_state else out


def causal_conv1d_fwd_ex(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                         seq_idx: Optional[torch.Tensor] = None,
                         initial_states: Optional[torch.Tensor] = None,
                         final_states: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None, act: int = _lib.SSM_ACT_NONE,
                         stream=None) -> torch.Tensor:
    """Enqueue causal_conv1d_fwd_ex; returns ``out``.  ``final_states``
    (batch, dim, width-1) in the io dtype is written when given."""
    x = _dense(x)
    io = _io_of(x, "x", 3)
    weight, bias = _dense(weight), _dense(bias)
    if weight.dtype != torch.float32 or (bias is not None and bias.dtype != torch.float32):
        raise ValueError("conv weight and bias must be float32")
    batch, dim, seqlen = x.shape
    _conv_params_spec(weight, bias, dim, x.device)
    width = weight.shape[1]
    if seq_idx is not None:
        seq_idx = _dense(seq_idx)
        if seq_idx.dtype != torch.int32 or tuple(seq_idx.shape) != (batch, seqlen):
            raise ValueError(f"seq_idx must be int32 of shape {(batch, seqlen)}")
    for name, t in (("initial_states", initial_states), ("final_states", final_states)):
        if t is not None and (t.dtype != x.dtype or tuple(t.shape) != (batch, dim, width - 1)
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous {x.dtype} tensor of shape {(batch, dim, width - 1)}")
    for name, t in (("seq_idx", seq_idx), ("initial_states", initial_states), ("final_states", final_states)):
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} must be on {x.device} with the other tensors, got {t.device}")
    _out_spec(out, "out", (batch, dim, seqlen), x.dtype, x.device)
    _on_gpu(x.device)
    if out is None:
        out = torch.empty_like(x)
    a = ConvArgs()
    a.batch, a.dim, a.seqlen, a.width, a.io_dtype, a.act = batch, dim, seqlen, width, io, act
    a.x, a.weight, a.bias, a.seq_idx = _ptr(x), _ptr(weight), _ptr(bias), _ptr(seq_idx)
    a.initial_states, a.out, a.final_states = _ptr(initial_states), _ptr(out), _ptr(final_states)
    check(_lib.lib().causal_conv1d_fwd_ex(ctypes.byref(a), _stream(x.device, stream)))
    return out


def causal_conv1d_fn(x, weight, bias=None, seq_idx=None, initial_states=None, return_final_states=False,
                     final_states_out=None, activation=None):
    """causal_conv1d_fn with the page's signature (section 4.2): returns out,
    or (out, final_states) with return_final_states.  seq_idx cannot be used
    with initial_states or return_final_states."""
    act = _act_code(activation)
    if seq_idx is not None and (initial_states is not None or return_final_states):
        raise ValueError("seq_idx cannot be used with initial_states or return_final_states")
    if seq_idx is None and initial_states is None and not return_final_states:
        return causal_conv1d_fwd(x, weight, bias, act=act)
    fin = None
    if return_final_states:
        fin = final_states_out
        if fin is None:
            fin = torch.empty((x.shape[0], x.shape[1], weight.shape[1] - 1), dtype=x.dtype, device=x.device)
    out = causal_conv1d_fwd_ex(x, weight, bias, seq_idx=seq_idx, initial_states=initial_states,
                               final_states=fin, act=act)
    return (out, fin) if return_final_states else out


def conv1d_selective_scan_fn(x, conv_weight, conv_bias, delta, A, B, C, D=None, z=None,
                             delta_bias=None, delta_softplus=False, return_last_state=False,
                             activation="silu"):
    """causal_conv1d_fn followed by selective_scan_fn, fused into one pass:
    u = causal_conv1d_fn(x, conv_weight, conv_bias, activation) is computed in
    registers (rounded to the io dtype exactly as the stored conv output) and
    never written to memory."""
    if B.dim() == 3:
        B = B.unsqueeze(1)
    if C.dim() == 3:
        C = C.unsqueeze(1)
    last = None
    if return_last_state:
        last = torch.empty((delta.shape[0], delta.shape[1], A.shape[1]), dtype=torch.float32,
                           device=delta.device)
    out = ssm_scan_fwd(None, delta, A, B, C, D, z, delta_bias, delta_softplus, last_state=last,
                       conv_x=x, conv_weight=conv_weight, conv_bias=conv_bias,
                       conv_act=_act_code(activation))
    return (out, last) if return_last_state else out


# ---------------------------------------------------------------------------
# single-step decode
# ---------------------------------------------------------------------------

def selective_state_update(state: torch.Tensor, x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor,
                           B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                           z: Optional[torch.Tensor] = None, dt_bias: Optional[torch.Tensor] = None,
                           dt_softplus: bool = False, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """One decode step (ssm_state_update): updates ``state`` (batch, dim, dstate)
    float32 in place and returns ``out`` (batch, dim).  x, dt, z: (batch, dim);
    A: (dim, dstate); B, C: (batch, dstate) or (batch, ngroups, dstate);
    D, dt_bias: (dim,).  ``state`` must be contiguous: it is written in place."""
    if not state.is_contiguous() or state.dtype != torch.float32 or state.dim() != 3:
        raise ValueError("state must be a contiguous float32 (batch, dim, dstate) tensor")
    x, dt = _dense(x), _dense(dt)
    io = _IO.get(x.dtype)
    if io is None:
        raise ValueError(f"io dtype must be float32, bfloat16 or float16, got {x.dtype}")
    if B.dim() == 2:
        B = B.unsqueeze(1)
    if C.dim() == 2:
        C = C.unsqueeze(1)
    if B.dim() != 3 or C.dim() != 3 or B.shape[1] != C.shape[1]:
        raise ValueError("B and C must be (batch, dstate) or (batch, ngroups, dstate) with equal groups")
    B, C, A, D, z, dt_bias = _dense(B), _dense(C), _dense(A), _dense(D), _dense(z), _dense(dt_bias)
    for name, t in (("dt", dt), ("z", z), ("B", B), ("C", C)):
        if t is not None and t.dtype != x.dtype:
            raise ValueError(f"{name} must have the io dtype {x.dtype}, got {t.dtype}")
    for name, t in (("A", A), ("D", D), ("dt_bias", dt_bias)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32, got {t.dtype}")
    batch, dim, dstate = state.shape
    dev, G = state.device, B.shape[1]
    for name, t in (("x", x), ("dt", dt), ("z", z)):
        _spec(t, name, (batch, dim), x.dtype, dev)
    _spec(A, "A", (dim, dstate), torch.float32, dev)
    _spec(B, "B", (batch, G, dstate), x.dtype, dev)
    _spec(C, "C", (batch, G, dstate), x.dtype, dev)
    _spec(D, "D", (dim,), torch.float32, dev)
    _spec(dt_bias, "dt_bias", (dim,), torch.float32, dev)
    _out_spec(out, "out", (batch, dim), x.dtype, dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty_like(x)
    a = _lib.StateUpdateArgs()
    a.batch, a.dim, a.dstate, a.ngroups = batch, dim, dstate, B.shape[1]
    a.io_dtype = io
    a.state, a.x, a.dt, a.A, a.B, a.C = _ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C)
    a.D, a.dt_bias, a.z = _ptr(D), _ptr(dt_bias), _ptr(z)
    a.dt_softplus = int(bool(dt_softplus))
    a.out = _ptr(out)
    check(_lib.lib().ssm_state_update(ctypes.byref(a), _stream(state.device, stream)))
    return out


def causal_conv1d_update(x: torch.Tensor, conv_state: torch.Tensor, weight: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, activation=None,
                         cache_seqlens: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Conv over new tokens against a cache (causal_conv1d_update): x is
    (batch, dim) or (batch, dim, seqlen); conv_state (batch, dim, state_len) is
    updated in place; cache_seqlens (batch,) int32 selects ring-buffer mode.
    Returns ``out`` shaped like x."""
    if not conv_state.is_contiguous() or conv_state.dim() != 3:
        raise ValueError("conv_state must be a contiguous (batch, dim, state_len) tensor")
    act = _act_code(activation)
    squeeze = x.dim() == 2
    x_shape = tuple(x.shape)
    x = _dense(x.unsqueeze(-1) if squeeze else x)
    if x.dim() != 3:
        raise ValueError(f"x must be (batch, dim) or (batch, dim, seqlen), got shape {x_shape}")
    io = _IO.get(x.dtype)
    if io is None or conv_state.dtype != x.dtype:
        raise ValueError("x and conv_state must share the io dtype (float32 or bfloat16)")
    weight, bias = _dense(weight), _dense(bias)
    if weight.dtype != torch.float32 or (bias is not None and bias.dtype != torch.float32):
        raise ValueError("conv weight and bias must be float32")
    if cache_seqlens is not None:
        if cache_seqlens.dtype != torch.int32:
            raise ValueError("cache_seqlens must be int32")
        cache_seqlens = _dense(cache_seqlens)
    batch, dim, seqlen = x.shape
    dev = x.device
    _spec(conv_state, "conv_state", (batch, dim, conv_state.shape[2]), x.dtype, dev)
    _conv_params_spec(weight, bias, dim, dev)
    _spec(cache_seqlens, "cache_seqlens", (batch,), torch.int32, dev)
    _out_spec(out, "out", x_shape, x.dtype, dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty_like(x)
    elif squeeze:
        out = out.unsqueeze(-1)
    check(_lib.lib().causal_conv1d_update(
        _ptr(x), _ptr(conv_state), _ptr(weight), _ptr(bias), _ptr(cache_seqlens), _ptr(out),
        batch, dim, seqlen, conv_state.shape[2], weight.shape[1], io, act,
        _stream(x.device, stream)))
    return out.squeeze(-1) if squeeze else out


# ---------------------------------------------------------------------------
# Mamba-2 chunked scan
# ---------------------------------------------------------------------------

def _ssd_args(x, dt, A, B, C, D, z, dt_bias, dt_softplus, initial_states, out, final_states, seq_idx,
              dt_limit, workspace, seq_segments, need_out=True):
    """ssd_scan_args_t for the tensors (checked; made contiguous where
    needed); returns (args, out, tensors kept alive until the call)."""
    x, dt, B, C = _dense(x), _dense(dt), _dense(B), _dense(C)
    if x.dtype != torch.bfloat16:
        raise ValueError(f"ssd_scan_fwd takes bfloat16 io, got {x.dtype}")
    for name, t in (("dt", dt), ("B", B), ("C", C), ("z", z)):
        if t is not None and t.dtype != x.dtype:
            raise ValueError(f"{name} must have the io dtype {x.dtype}, got {t.dtype}")
    A, D, z, dt_bias, initial_states = _dense(A), _dense(D), _dense(z), _dense(dt_bias), _dense(initial_states)
    for name, t in (("A", A), ("D", D), ("dt_bias", dt_bias), ("initial_states", initial_states)):
        if t is not None and t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32, got {t.dtype}")
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be (batch, seqlen, nheads, headdim) and B (batch, seqlen, ngroups, dstate)")
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    dev, f32 = x.device, torch.float32
    _spec(z, "z", x.shape, x.dtype, dev)
    _spec(dt, "dt", (batch, seqlen, nheads), x.dtype, dev)
    _spec(B, "B", (batch, seqlen, ngroups, dstate), x.dtype, dev)
    _spec(C, "C", (batch, seqlen, ngroups, dstate), x.dtype, dev)
    _spec(A, "A", (nheads,), f32, dev)
    _spec(dt_bias, "dt_bias", (nheads,), f32, dev)
    if D is not None:
        _spec(D, "D", (nheads,) if D.dim() == 1 else (nheads, headdim), f32, dev)
    _spec(initial_states, "initial_states", (batch, nheads, headdim, dstate), f32, dev)
    if seq_idx is not None:
        seq_idx = _dense(seq_idx)
        _spec(seq_idx, "seq_idx", (batch, seqlen), torch.int32, dev)
    _out_spec(out, "out", x.shape, x.dtype, dev)
    _out_spec(final_states, "final_states", (batch, nheads, headdim, dstate), f32, dev)
    if workspace is not None:
        _workspace_spec(workspace, dev)
    _on_gpu(dev)
    if out is None and need_out:
        out = torch.empty_like(x)
    a = _lib.SsdArgs()
    a.batch, a.seqlen, a.nheads, a.headdim = batch, seqlen, nheads, headdim
    a.dstate, a.ngroups = dstate, ngroups
    a.io_dtype = _lib.SSM_BF16
    a.x, a.dt, a.A, a.B, a.C = _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C)
    a.D = _ptr(D)
    a.D_per_channel = int(D is not None and D.dim() == 2)
    a.z, a.dt_bias = _ptr(z), _ptr(dt_bias)
    a.dt_softplus = int(bool(dt_softplus))
    a.initial_states, a.out, a.final_states = _ptr(initial_states), _ptr(out), _ptr(final_states)
    if dt_limit is not None:
        a.dt_limit, a.dt_min, a.dt_max = 1, float(dt_limit[0]), float(dt_limit[1])
    a.seq_idx = _ptr(seq_idx)
    a.seq_segments = int(seq_segments)
    return a, out, (x, dt, A, B, C, D, z, dt_bias, initial_states, seq_idx)


def ssd_scan_fwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                 C: torch.Tensor, D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                 dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = False,
                 initial_states: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 final_states: Optional[torch.Tensor] = None, seq_idx: Optional[torch.Tensor] = None,
                 dt_limit: Optional[Tuple[float, float]] = None, workspace: Optional[torch.Tensor] = None,
                 seq_segments: int = 0, stream=None) -> torch.Tensor:
    """Enqueue ssd_scan_fwd; returns ``out`` (batch, seqlen, nheads, headdim).

    x, z: (batch, seqlen, nheads, headdim) bf16; dt: (batch, seqlen, nheads) bf16;
    A, dt_bias: (nheads,) float32; B, C: (batch, seqlen, ngroups, dstate) bf16;
    D: (nheads,) or (nheads, headdim) float32; initial_states / final_states:
    (batch, nheads, headdim, dstate) float32; seq_idx: (batch, seqlen) int32
    sequence ids, non-decreasing along seqlen; dt_limit: (dt_min, dt_max), the
    step's clamp after softplus.  The scratch of a sequence split is allocated
    here (torch) unless ``workspace`` is given; ``seq_segments`` (0: the
    library's choice) asks for that many segments."""
    a, out, keep = _ssd_args(x, dt, A, B, C, D, z, dt_bias, dt_softplus, initial_states, out, final_states,
                             seq_idx, dt_limit, workspace, seq_segments)
    dev = out.device
    L = _lib.lib()
    if workspace is None:
        need = ctypes.c_size_t(0)
        check(L.ssd_scan_workspace_size(ctypes.byref(a), ctypes.byref(need)))
        if need.value:
            workspace = torch.empty(need.value, dtype=torch.uint8, device=dev)
    if workspace is not None:
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    check(L.ssd_scan_fwd(ctypes.byref(a), _stream(dev, stream)))
    return out


def _nchunks(seqlen: int, chunk_size: int) -> int:
    if chunk_size <= 0 or chunk_size % _lib.SSD_CHUNK != 0:
        raise ValueError(f"chunk_size must be a positive multiple of {_lib.SSD_CHUNK}, got {chunk_size}")
    return -(-seqlen // chunk_size)


def ssd_chunk_state(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, chunk_size: int,
                    dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = False,
                    seq_idx: Optional[torch.Tensor] = None, dt_limit: Optional[Tuple[float, float]] = None,
                    states: Optional[torch.Tensor] = None, decays: Optional[torch.Tensor] = None,
                    stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Enqueue ssd_chunk_state: per chunk of ``chunk_size`` tokens its end
    state from zero, ``states`` (nchunks, batch, nheads, headdim, dstate)
    float32, and the factor of the state entering it, ``decays`` (nchunks,
    batch, nheads) float32.  Inputs as ``ssd_scan_fwd``."""
    a, _, keep = _ssd_args(x, dt, A, B, None, None, None, dt_bias, dt_softplus, None, None, None, seq_idx,
                           dt_limit, None, 0, need_out=False)
    batch, seqlen, nheads, headdim = x.shape
    dstate = B.shape[3]
    nc = _nchunks(seqlen, chunk_size)
    dev, f32 = x.device, torch.float32
    _out_spec(states, "states", (nc, batch, nheads, headdim, dstate), f32, dev)
    _out_spec(decays, "decays", (nc, batch, nheads), f32, dev)
    if states is None:
        states = torch.empty((nc, batch, nheads, headdim, dstate), dtype=f32, device=dev)
    if decays is None:
        decays = torch.empty((nc, batch, nheads), dtype=f32, device=dev)
    check(_lib.lib().ssd_chunk_state(ctypes.byref(a), chunk_size, _ptr(states), _ptr(decays),
                                     _stream(dev, stream)))
    return states, decays


def ssd_state_passing(states: torch.Tensor, decays: torch.Tensor, initial_states: Optional[torch.Tensor] = None,
                      carried: Optional[torch.Tensor] = None, final_states: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Enqueue ssd_state_passing: ``carried`` (the state entering every
    chunk, the shape of ``states``) and ``final_states`` (batch, nheads,
    headdim, dstate), both float32."""
    states, decays, initial_states = _dense(states), _dense(decays), _dense(initial_states)
    if states.dim() != 5:
        raise ValueError("states must be (nchunks, batch, nheads, headdim, dstate)")
    nc, batch, nheads, headdim, dstate = states.shape
    dev, f32 = states.device, torch.float32
    _spec(states, "states", states.shape, f32, dev)
    _spec(decays, "decays", (nc, batch, nheads), f32, dev)
    _spec(initial_states, "initial_states", (batch, nheads, headdim, dstate), f32, dev)
    _out_spec(carried, "carried", states.shape, f32, dev)
    _out_spec(final_states, "final_states", (batch, nheads, headdim, dstate), f32, dev)
    _on_gpu(dev)
    if carried is None:
        carried = torch.empty_like(states)
    if final_states is None:
        final_states = torch.empty((batch, nheads, headdim, dstate), dtype=f32, device=dev)
    check(_lib.lib().ssd_state_passing(nc, batch, nheads, headdim, dstate, _ptr(states), _ptr(decays),
                                       _ptr(initial_states), _ptr(carried), _ptr(final_states),
                                       _stream(dev, stream)))
    return carried, final_states


def ssd_chunk_scan(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                   carried: torch.Tensor, chunk_size: int, D: Optional[torch.Tensor] = None,
                   z: Optional[torch.Tensor] = None, dt_bias: Optional[torch.Tensor] = None,
                   dt_softplus: bool = False, seq_idx: Optional[torch.Tensor] = None,
                   dt_limit: Optional[Tuple[float, float]] = None, out: Optional[torch.Tensor] = None,
                   final_states: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Enqueue ssd_chunk_scan: every chunk's outputs from ``carried``
    (nchunks, batch, nheads, headdim, dstate) float32; returns ``out``.  The
    state after the last chunk goes to ``final_states`` when given."""
    a, out, keep = _ssd_args(x, dt, A, B, C, D, z, dt_bias, dt_softplus, None, out, final_states, seq_idx,
                             dt_limit, None, 0)
    batch, seqlen, nheads, headdim = x.shape
    dstate = B.shape[3]
    nc = _nchunks(seqlen, chunk_size)
    carried = _dense(carried)
    _spec(carried, "carried", (nc, batch, nheads, headdim, dstate), torch.float32, x.device)
    check(_lib.lib().ssd_chunk_scan(ctypes.byref(a), chunk_size, _ptr(carried), _stream(x.device, stream)))
    return out


def ssd_scan_workspace_size(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=False,
                            initial_states=None, out=None, final_states=None, seq_idx=None,
                            dt_limit=None, seq_segments=0) -> int:
    """Scratch bytes ssd_scan_fwd needs for these tensors (0 without a
    sequence split)."""
    a, _, keep = _ssd_args(x, dt, A, B, C, D, z, dt_bias, dt_softplus, initial_states, out, final_states,
                           seq_idx, dt_limit, None, seq_segments)
    need = ctypes.c_size_t(0)
    check(_lib.lib().ssd_scan_workspace_size(ctypes.byref(a), ctypes.byref(need)))
    return need.value
