"""ctypes front end of the float64 CPU oracle (``ssm_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product package.

What the oracle computes is documented in ``ssm_oracle.c`` (the pages: the
PaddleNLP Kernel operator-library guide, sections 4.1 selective_scan and 4.2
causal_conv1d).  This module only marshals numpy arrays: io tensors are passed
as their stored bits (float32 arrays, or uint16 arrays holding bf16 bits), and
results come back as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssm_oracle.c")
LIB = os.path.join(HERE, "libssm_oracle.so")

F32, BF16, F16 = 0, 1, 2
BC_FIXED, BC_VARYING = 0, 1
ACT_NONE, ACT_SILU = 0, 1

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP over rows)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def use_library(path: Optional[str]) -> None:
    """Point this module at another build of the oracle source (None: the
    default build).  Used only by the mutation test, which plants mistakes in
    a copy of the source to show the pins catch them."""
    global _lib, _lib_path
    _lib, _lib_path = None, path


_lib_path: Optional[str] = None


def _load():
    global _lib
    if _lib is None:
        if _lib_path is None:
            build()
        lib = ctypes.CDLL(_lib_path or LIB)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_selective_scan.argtypes = [
            i64, i64, i64, i64, i64, i32,
            p, p, p, p, i32, p, i32, p, p, p, i32, p,
            p, p, p, i32, i32,
            p, i64, p, p, i32]
        lib.oracle_selective_scan.restype = i32
        lib.oracle_selective_scan_f32_floor.argtypes = [
            i64, i64, i64, i64, i64, i32,
            p, p, p, p, i32, p, i32, p, p, p, i32, p, p, i32]
        lib.oracle_selective_scan_f32_floor.restype = i32
        lib.oracle_causal_conv1d.argtypes = [
            i64, i64, i64, i32, i32, p, p, p, i32, p, i64, p, i32]
        lib.oracle_causal_conv1d.restype = i32
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_double
        lib.oracle_softplus.argtypes = [ctypes.c_double]
        lib.oracle_softplus.restype = ctypes.c_double
        lib.oracle_silu.argtypes = [ctypes.c_double]
        lib.oracle_silu.restype = ctypes.c_double
        lib.oracle_selective_state_update.argtypes = [
            i64, i64, i64, i64, i32, p, p, p, p, p, p, p, p, p, i32, p, p]
        lib.oracle_selective_state_update.restype = i32
        lib.oracle_causal_conv1d_update.argtypes = [
            i64, i64, i64, i32, i64, i32, p, p, p, p, i32, p, p, p]
        lib.oracle_causal_conv1d_update.restype = i32
        lib.oracle_ssd_scan.argtypes = [
            i64, i64, i64, i64, i64, i64, i32, p, p, p, p, p, p, i32, p, p, i32, p, p, p,
            i32, ctypes.c_double, ctypes.c_double, p, i32]
        lib.oracle_ssd_scan.restype = i32
        d = ctypes.c_double
        lib.oracle_ssd_chunk_state.argtypes = [i64, i64, i64, i64, i64, i64, i32, i64, p, p, p, p, p, i32,
                                               i32, d, d, p, p, p]
        lib.oracle_ssd_chunk_state.restype = i32
        lib.oracle_ssd_state_passing.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p]
        lib.oracle_ssd_state_passing.restype = i32
        lib.oracle_ssd_chunk_scan.argtypes = [i64, i64, i64, i64, i64, i64, i32, i64, p, p, p, p, p, p, i32,
                                              p, p, i32, i32, d, d, p, p, p, p]
        lib.oracle_ssd_chunk_scan.restype = i32
        lib.oracle_selective_scan_bwd.argtypes = [
            i64, i64, i64, i64, i64, i32, p, p, p, p, i32, p, i32, p, p, p, i32, p, p,
            p, p, p, p, p, p, p, p, p]
        lib.oracle_selective_scan_bwd.restype = i32
        lib.oracle_selective_scan_complex_bwd.argtypes = [
            i64, i64, i64, i64, i64, i32, p, p, p, p, i32, p, i32, p, p, p, i32, p, p,
            p, p, p, p, p, p, p, p, p]
        lib.oracle_selective_scan_complex_bwd.restype = i32
        lib.oracle_selective_scan_complex_bwd_f32_floor.argtypes = [
            i64, i64, i64, i64, i64, i32, p, p, p, p, i32, p, i32, p, p, i32, p, p, p, p, p]
        lib.oracle_selective_scan_complex_bwd_f32_floor.restype = i32
        lib.oracle_causal_conv1d_ex.argtypes = [i64, i64, i64, i32, i32, p, p, p, i32, p, p, p, p]
        lib.oracle_causal_conv1d_ex.restype = i32
        lib.oracle_round_f16.argtypes = [ctypes.c_double]
        lib.oracle_round_f16.restype = ctypes.c_double
        lib.oracle_f16_bits_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_bits_to_double.restype = ctypes.c_double
        lib.oracle_selective_scan_complex.argtypes = [
            i64, i64, i64, i64, i64, i32,
            p, p, p, p, i32, p, i32, p, p, p, i32, p,
            p, i64, p, p, i32]
        lib.oracle_selective_scan_complex.restype = i32
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i32
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _io(a: Optional[np.ndarray], dtype: int):
    """Check an io tensor holds the stored bits of the stated dtype."""
    if a is None:
        return None
    want = np.uint16 if dtype in (BF16, F16) else np.float32
    if a.dtype != want:
        raise TypeError(f"io tensor must be {want.__name__}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _f32(a: Optional[np.ndarray]):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def round_bf16(v: float) -> float:
    return float(_load().oracle_round_bf16(float(v)))


def round_f16(v: float) -> float:
    return float(_load().oracle_round_f16(float(v)))


def f16_bits_to_double(h: int) -> float:
    return float(_load().oracle_f16_bits_to_double(int(h)))


def softplus(v: float) -> float:
    return float(_load().oracle_softplus(float(v)))


def silu(v: float) -> float:
    return float(_load().oracle_silu(float(v)))


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                   delta_softplus=False, *, io_dtype=F32, ngroups=1,
                   B_kind=BC_VARYING, C_kind=BC_VARYING, initial_state=None,
                   conv_x=None, conv_weight=None, conv_bias=None, conv_act=ACT_SILU,
                   rows=None, nthreads=0, shape=None):
    """Oracle selective scan.

    u, delta, z: (batch, dim, seqlen) io bits; A: (dim, dstate) float32;
    B/C: (dim, dstate) when fixed, (batch, ngroups, dstate, seqlen) when varying;
    D, delta_bias: (dim,) float32; initial_state: (batch, dim, dstate) float64.
    With conv_weight given, u is ignored and computed from conv_x.
    rows: optional int64 array of row ids b*dim + d.
    Returns (out (nrows, seqlen) float64, last_state (nrows, dstate) float64).
    """
    lib = _load()
    delta = _io(delta, io_dtype)
    batch, dim, seqlen = shape if shape is not None else delta.shape
    A = _f32(A)
    dstate = A.shape[1]
    u = _io(u, io_dtype)
    B = _io(B, io_dtype)
    C = _io(C, io_dtype)
    z = _io(z, io_dtype)
    conv_x = _io(conv_x, io_dtype)
    D, delta_bias = _f32(D), _f32(delta_bias)
    conv_weight, conv_bias = _f32(conv_weight), _f32(conv_bias)
    init = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = batch * dim if rows_a is None else rows_a.shape[0]
    out = np.empty((nrows, seqlen), dtype=np.float64)
    last = np.empty((nrows, dstate), dtype=np.float64)
    width = 0 if conv_weight is None else conv_weight.shape[1]
    rc = lib.oracle_selective_scan(
        batch, dim, seqlen, dstate, ngroups, io_dtype,
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), B_kind, _ptr(C), C_kind,
        _ptr(D), _ptr(delta_bias), _ptr(z), int(bool(delta_softplus)), _ptr(init),
        _ptr(conv_x), _ptr(conv_weight), _ptr(conv_bias), width, conv_act,
        _ptr(rows_a), nrows, _ptr(out), _ptr(last), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_selective_scan failed with status {rc}")
    return out, last


def selective_scan_f32_floor(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                             delta_softplus=False, *, io_dtype=F32, ngroups=1,
                             B_kind=BC_VARYING, C_kind=BC_VARYING, nthreads=0):
    """The selective scan evaluated in binary32, in order (see ``ssm_oracle.c``):
    not a reference, but the rounding floor of a plain fp32 evaluation, used
    to set the bar of inputs no fp32 evaluation can meet at fp32 tolerance.
    Returns (out (batch*dim, seqlen), last_state (batch*dim, dstate)) float64."""
    lib = _load()
    delta = _io(delta, io_dtype)
    batch, dim, seqlen = delta.shape
    A = _f32(A)
    dstate = A.shape[1]
    u, B, C, z = _io(u, io_dtype), _io(B, io_dtype), _io(C, io_dtype), _io(z, io_dtype)
    D, delta_bias = _f32(D), _f32(delta_bias)
    out = np.empty((batch * dim, seqlen), dtype=np.float64)
    last = np.empty((batch * dim, dstate), dtype=np.float64)
    rc = lib.oracle_selective_scan_f32_floor(
        batch, dim, seqlen, dstate, ngroups, io_dtype, _ptr(u), _ptr(delta), _ptr(A),
        _ptr(B), B_kind, _ptr(C), C_kind, _ptr(D), _ptr(delta_bias), _ptr(z),
        int(bool(delta_softplus)), _ptr(out), _ptr(last), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_selective_scan_f32_floor failed with status {rc}")
    return out, last


def selective_scan_complex(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                           delta_softplus=False, *, io_dtype=F32, ngroups=1,
                           B_kind=BC_VARYING, C_kind=BC_VARYING, initial_state=None,
                           rows=None, nthreads=0):
    """Oracle selective scan with complex A (see ``ssm_oracle.c``).

    u, delta, z: (batch, dim, seqlen) io bits; A: (dim, dstate, 2) float32
    (real, imaginary) pairs; B/C: io bits with a trailing pair axis,
    (dim, dstate, 2) fixed or (batch, ngroups, dstate, seqlen, 2) varying;
    initial_state: (batch, dim, dstate, 2) float64 or None.
    Returns (out (nrows, seqlen) float64, last_state (nrows, dstate, 2) float64).
    """
    lib = _load()
    delta = _io(delta, io_dtype)
    batch, dim, seqlen = delta.shape
    A = _f32(A)
    if A.ndim != 3 or A.shape[2] != 2:
        raise ValueError("A must be (dim, dstate, 2) pairs")
    dstate = A.shape[1]
    u, z = _io(u, io_dtype), _io(z, io_dtype)
    B, C = _io(B, io_dtype), _io(C, io_dtype)
    for name, t in (("B", B), ("C", C)):
        if t.shape[-1] != 2:
            raise ValueError(f"{name} must end in a (real, imaginary) pair axis")
    D, delta_bias = _f32(D), _f32(delta_bias)
    init = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = batch * dim if rows_a is None else rows_a.shape[0]
    out = np.empty((nrows, seqlen), dtype=np.float64)
    last = np.empty((nrows, dstate, 2), dtype=np.float64)
    rc = lib.oracle_selective_scan_complex(
        batch, dim, seqlen, dstate, ngroups, io_dtype,
        _ptr(u), _ptr(delta), _ptr(A), _ptr(B), B_kind, _ptr(C), C_kind,
        _ptr(D), _ptr(delta_bias), _ptr(z), int(bool(delta_softplus)), _ptr(init),
        _ptr(rows_a), nrows, _ptr(out), _ptr(last), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_selective_scan_complex failed with status {rc}")
    return out, last


def causal_conv1d(x, weight, bias=None, act=ACT_NONE, *, io_dtype=F32, rows=None,
                  nthreads=0):
    """Oracle causal depthwise conv: x (batch, dim, seqlen) io bits, weight
    (dim, width) float32, bias (dim,) float32.  Returns (nrows, seqlen) float64
    (not rounded to the io dtype)."""
    lib = _load()
    x = _io(x, io_dtype)
    batch, dim, seqlen = x.shape
    weight, bias = _f32(weight), _f32(bias)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = batch * dim if rows_a is None else rows_a.shape[0]
    out = np.empty((nrows, seqlen), dtype=np.float64)
    rc = lib.oracle_causal_conv1d(batch, dim, seqlen, weight.shape[1], io_dtype,
                                  _ptr(x), _ptr(weight), _ptr(bias), act,
                                  _ptr(rows_a), nrows, _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_causal_conv1d failed with status {rc}")
    return out


def selective_state_update(state, x, dt, A, B, C, D=None, z=None, dt_bias=None,
                           dt_softplus=False, *, io_dtype=F32):
    """Oracle single decode step against a cached state.

    state: (batch, dim, dstate) float (the cached fp32 state, widened);
    x, dt, z: (batch, dim) io bits; A: (dim, dstate) float32;
    B, C: (batch, ngroups, dstate) io bits; D, dt_bias: (dim,) float32.
    Returns (out (batch, dim) float64, new state (batch, dim, dstate) float64).
    """
    lib = _load()
    x, dt, z = _io(x, io_dtype), _io(dt, io_dtype), _io(z, io_dtype)
    B, C = _io(B, io_dtype), _io(C, io_dtype)
    A, D, dt_bias = _f32(A), _f32(D), _f32(dt_bias)
    st = np.ascontiguousarray(state, dtype=np.float64)
    batch, dim = x.shape
    dstate = A.shape[1]
    ngroups = B.shape[1]
    out = np.empty((batch, dim), dtype=np.float64)
    new = np.empty((batch, dim, dstate), dtype=np.float64)
    rc = lib.oracle_selective_state_update(
        batch, dim, dstate, ngroups, io_dtype, _ptr(st), _ptr(x), _ptr(dt), _ptr(A),
        _ptr(B), _ptr(C), _ptr(D), _ptr(dt_bias), _ptr(z), int(bool(dt_softplus)),
        _ptr(out), _ptr(new))
    if rc != 0:
        raise ValueError(f"oracle_selective_state_update failed with status {rc}")
    return out, new


def causal_conv1d_update(x, conv_state, weight, bias=None, act=ACT_NONE, cache_seqlens=None,
                         *, io_dtype=F32):
    """Oracle conv continued from a cache of earlier inputs.

    x: (batch, dim, seqlen) io bits; conv_state: (batch, dim, state_len) io bits
    (not modified); weight (dim, width) float32; bias (dim,) float32;
    cache_seqlens: None (shift mode) or (batch,) int32 ring-buffer positions.
    Returns (out (batch, dim, seqlen) float64, new conv_state (io bits)).
    """
    lib = _load()
    x, conv_state = _io(x, io_dtype), _io(conv_state, io_dtype)
    batch, dim, seqlen = x.shape
    state_len = conv_state.shape[2]
    weight, bias = _f32(weight), _f32(bias)
    cs = None if cache_seqlens is None else np.ascontiguousarray(cache_seqlens, dtype=np.int32)
    out = np.empty((batch, dim, seqlen), dtype=np.float64)
    new = np.empty_like(conv_state)
    rc = lib.oracle_causal_conv1d_update(
        batch, dim, seqlen, weight.shape[1], state_len, io_dtype, _ptr(x), _ptr(conv_state),
        _ptr(weight), _ptr(bias), act, _ptr(cs), _ptr(out), _ptr(new))
    if rc != 0:
        raise ValueError(f"oracle_causal_conv1d_update failed with status {rc}")
    return out, new


def ssd_scan(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus=False, *,
             io_dtype=F32, initial_states=None, dt_limit=None, seq_idx=None, nthreads=0):
    """Oracle Mamba-2 scan (scalar decay per head), sequential in time.

    x, z: (batch, seqlen, nheads, headdim) io bits; dt: (batch, seqlen, nheads)
    io bits; A, dt_bias: (nheads,) float32; B, C: (batch, seqlen, ngroups,
    dstate) io bits; D: (nheads,) or (nheads, headdim) float32;
    initial_states: (batch, nheads, headdim, dstate) float; dt_limit: None or
    (dt_min, dt_max), the step's clamp after softplus; seq_idx: None or
    (batch, seqlen) int32 sequence ids (the state restarts where they change).
    Returns (out (batch, seqlen, nheads, headdim) float64,
             final_states (batch, nheads, headdim, dstate) float64).
    """
    lib = _load()
    x, dt, z = _io(x, io_dtype), _io(dt, io_dtype), _io(z, io_dtype)
    B, C = _io(B, io_dtype), _io(C, io_dtype)
    A, D, dt_bias = _f32(A), _f32(D), _f32(dt_bias)
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    init = None if initial_states is None else np.ascontiguousarray(initial_states, dtype=np.float64)
    sid = None if seq_idx is None else np.ascontiguousarray(seq_idx, dtype=np.int32)
    if sid is not None and sid.shape != (batch, seqlen):
        raise ValueError("seq_idx must be (batch, seqlen)")
    lim = (0.0, 0.0) if dt_limit is None else (float(dt_limit[0]), float(dt_limit[1]))
    out = np.empty(x.shape, dtype=np.float64)
    fin = np.empty((batch, nheads, headdim, dstate), dtype=np.float64)
    rc = lib.oracle_ssd_scan(batch, seqlen, nheads, headdim, dstate, ngroups, io_dtype,
                             _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                             int(D is not None and D.ndim == 2), _ptr(z), _ptr(dt_bias),
                             int(bool(dt_softplus)), _ptr(init), _ptr(out), _ptr(fin),
                             int(dt_limit is not None), lim[0], lim[1], _ptr(sid), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_ssd_scan failed with status {rc}")
    return out, fin


def _ssd_common(x, dt, B, dt_limit, seq_idx, io_dtype):
    x, dt, B = _io(x, io_dtype), _io(dt, io_dtype), _io(B, io_dtype)
    batch, seqlen, nheads, headdim = x.shape
    sid = None if seq_idx is None else np.ascontiguousarray(seq_idx, dtype=np.int32)
    if sid is not None and sid.shape != (batch, seqlen):
        raise ValueError("seq_idx must be (batch, seqlen)")
    lim = (0.0, 0.0) if dt_limit is None else (float(dt_limit[0]), float(dt_limit[1]))
    return x, dt, B, sid, lim


def ssd_chunk_state(x, dt, A, B, chunk_size, dt_bias=None, dt_softplus=False, *, io_dtype=F32,
                    dt_limit=None, seq_idx=None):
    """Oracle chunk_state: per chunk of chunk_size tokens its end state from
    a zero state and the factor P of the state entering it (0 where the
    state restarts inside it).  Inputs as ``ssd_scan``.  Returns
    (states (nchunks, batch, nheads, headdim, dstate), decays (nchunks,
    batch, nheads)), float64."""
    lib = _load()
    x, dt, B, sid, lim = _ssd_common(x, dt, B, dt_limit, seq_idx, io_dtype)
    A, dt_bias = _f32(A), _f32(dt_bias)
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    nc = -(-seqlen // chunk_size)
    states = np.empty((nc, batch, nheads, headdim, dstate))
    decays = np.empty((nc, batch, nheads))
    rc = lib.oracle_ssd_chunk_state(batch, seqlen, nheads, headdim, dstate, ngroups, io_dtype, chunk_size,
                                    _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(dt_bias), int(bool(dt_softplus)),
                                    int(dt_limit is not None), lim[0], lim[1], _ptr(sid), _ptr(states),
                                    _ptr(decays))
    if rc != 0:
        raise ValueError(f"oracle_ssd_chunk_state failed with status {rc}")
    return states, decays


def ssd_state_passing(states, decays, initial_states=None):
    """Oracle state_passing: carried[c] = the state entering chunk c
    (S_0 = initial_states or zero, S_{c+1} = decays[c] S_c + states[c]) and
    the final state.  Returns (carried (nchunks, batch, nheads, headdim,
    dstate), final (batch, nheads, headdim, dstate)), float64."""
    lib = _load()
    states = np.ascontiguousarray(states, dtype=np.float64)
    decays = np.ascontiguousarray(decays, dtype=np.float64)
    nc, batch, nheads, headdim, dstate = states.shape
    init = None if initial_states is None else np.ascontiguousarray(initial_states, dtype=np.float64)
    carried = np.empty(states.shape)
    fin = np.empty(states.shape[1:])
    rc = lib.oracle_ssd_state_passing(nc, batch, nheads, headdim, dstate, _ptr(states), _ptr(decays),
                                      _ptr(init), _ptr(carried), _ptr(fin))
    if rc != 0:
        raise ValueError(f"oracle_ssd_state_passing failed with status {rc}")
    return carried, fin


def ssd_chunk_scan(x, dt, A, B, C, carried, chunk_size, D=None, z=None, dt_bias=None, dt_softplus=False, *,
                   io_dtype=F32, dt_limit=None, seq_idx=None):
    """Oracle chunk scan: every chunk's outputs from the recurrence started
    at carried[c].  Returns (out (batch, seqlen, nheads, headdim), the state
    after the last chunk (batch, nheads, headdim, dstate)), float64."""
    lib = _load()
    x, dt, B, sid, lim = _ssd_common(x, dt, B, dt_limit, seq_idx, io_dtype)
    C, z = _io(C, io_dtype), _io(z, io_dtype)
    A, D, dt_bias = _f32(A), _f32(D), _f32(dt_bias)
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    carried = np.ascontiguousarray(carried, dtype=np.float64)
    out = np.empty(x.shape)
    fin = np.empty((batch, nheads, headdim, dstate))
    rc = lib.oracle_ssd_chunk_scan(batch, seqlen, nheads, headdim, dstate, ngroups, io_dtype, chunk_size,
                                   _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                   int(D is not None and D.ndim == 2), _ptr(z), _ptr(dt_bias),
                                   int(bool(dt_softplus)), int(dt_limit is not None), lim[0], lim[1], _ptr(sid),
                                   _ptr(carried), _ptr(out), _ptr(fin))
    if rc != 0:
        raise ValueError(f"oracle_ssd_chunk_scan failed with status {rc}")
    return out, fin


def selective_scan_bwd(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None,
                       delta_softplus=False, *, io_dtype=F32, ngroups=1, B_kind=BC_VARYING,
                       C_kind=BC_VARYING, initial_state=None):
    """Oracle gradients of the selective-scan forward (no conv prologue).

    Inputs as in ``selective_scan``; dout: (batch, dim, seqlen) float.
    Returns a dict of float64 arrays: du, ddelta, dA, dB, dC, and dD, dz,
    ddelta_bias, dinitial_state when the corresponding input is given.
    """
    lib = _load()
    delta = _io(delta, io_dtype)
    batch, dim, seqlen = delta.shape
    A = _f32(A)
    dstate = A.shape[1]
    u, B, C, z = _io(u, io_dtype), _io(B, io_dtype), _io(C, io_dtype), _io(z, io_dtype)
    D, delta_bias = _f32(D), _f32(delta_bias)
    init = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    dout = np.ascontiguousarray(dout, dtype=np.float64)
    out = {
        "du": np.empty((batch, dim, seqlen)), "ddelta": np.empty((batch, dim, seqlen)),
        "dA": np.empty((dim, dstate)), "dB": np.empty(B.shape), "dC": np.empty(C.shape),
        "dD": None if D is None else np.empty((dim,)),
        "dz": None if z is None else np.empty((batch, dim, seqlen)),
        "ddelta_bias": None if delta_bias is None else np.empty((dim,)),
        "dinitial_state": np.empty((batch, dim, dstate)),
    }
    rc = lib.oracle_selective_scan_bwd(
        batch, dim, seqlen, dstate, ngroups, io_dtype, _ptr(u), _ptr(delta), _ptr(A),
        _ptr(B), B_kind, _ptr(C), C_kind, _ptr(D), _ptr(delta_bias), _ptr(z),
        int(bool(delta_softplus)), _ptr(init), _ptr(dout),
        _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
        _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["ddelta_bias"]), _ptr(out["dinitial_state"]))
    if rc != 0:
        raise ValueError(f"oracle_selective_scan_bwd failed with status {rc}")
    return out


def selective_scan_complex_bwd(u, delta, A, B, C, dout, D=None, z=None, delta_bias=None,
                               delta_softplus=False, *, io_dtype=F32, ngroups=1, B_kind=BC_VARYING,
                               C_kind=BC_VARYING, initial_state=None):
    """Oracle gradients of the complex-A forward (``selective_scan_complex``).

    Inputs as there; dout: (batch, dim, seqlen) float.  Returns a dict of
    float64 arrays: du, ddelta, dz, dD, ddelta_bias as in the real backward;
    dA (dim, dstate, 2), dB / dC in B's / C's layout and dinitial_state
    (batch, dim, dstate, 2), each the gradient of the real and the
    imaginary part.
    """
    lib = _load()
    delta = _io(delta, io_dtype)
    batch, dim, seqlen = delta.shape
    A = _f32(A)
    if A.ndim != 3 or A.shape[2] != 2:
        raise ValueError("A must be (dim, dstate, 2) pairs")
    dstate = A.shape[1]
    u, B, C, z = _io(u, io_dtype), _io(B, io_dtype), _io(C, io_dtype), _io(z, io_dtype)
    D, delta_bias = _f32(D), _f32(delta_bias)
    init = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    dout = np.ascontiguousarray(dout, dtype=np.float64)
    out = {
        "du": np.empty((batch, dim, seqlen)), "ddelta": np.empty((batch, dim, seqlen)),
        "dA": np.empty((dim, dstate, 2)), "dB": np.empty(B.shape), "dC": np.empty(C.shape),
        "dD": None if D is None else np.empty((dim,)),
        "dz": None if z is None else np.empty((batch, dim, seqlen)),
        "ddelta_bias": None if delta_bias is None else np.empty((dim,)),
        "dinitial_state": np.empty((batch, dim, dstate, 2)),
    }
    rc = lib.oracle_selective_scan_complex_bwd(
        batch, dim, seqlen, dstate, ngroups, io_dtype, _ptr(u), _ptr(delta), _ptr(A),
        _ptr(B), B_kind, _ptr(C), C_kind, _ptr(D), _ptr(delta_bias), _ptr(z),
        int(bool(delta_softplus)), _ptr(init), _ptr(dout),
        _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
        _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["ddelta_bias"]), _ptr(out["dinitial_state"]))
    if rc != 0:
        raise ValueError(f"oracle_selective_scan_complex_bwd failed with status {rc}")
    return out


def selective_scan_complex_bwd_f32_floor(u, delta, A, B, C, dout, z=None, delta_bias=None,
                                         delta_softplus=False, *, io_dtype=F32, ngroups=1,
                                         B_kind=BC_VARYING, C_kind=BC_VARYING, initial_state=None):
    """The complex backward's step gradient evaluated in binary32 in time
    order (see ``ssm_oracle.c``): a dict of ddelta (batch, dim, seqlen),
    ddelta_bias (dim) and dA (dim, dstate, 2) as float64 arrays.  Test
    infrastructure: it sets the bar where fp32 cannot meet the fp32
    tolerance."""
    lib = _load()
    delta = _io(delta, io_dtype)
    batch, dim, seqlen = delta.shape
    A = _f32(A)
    dstate = A.shape[1]
    u, B, C, z = _io(u, io_dtype), _io(B, io_dtype), _io(C, io_dtype), _io(z, io_dtype)
    delta_bias = _f32(delta_bias)
    init = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    dout = np.ascontiguousarray(dout, dtype=np.float64)
    out = {"ddelta": np.empty((batch, dim, seqlen)), "ddelta_bias": np.empty((dim,)),
           "dA": np.empty((dim, dstate, 2))}
    rc = lib.oracle_selective_scan_complex_bwd_f32_floor(
        batch, dim, seqlen, dstate, ngroups, io_dtype, _ptr(u), _ptr(delta), _ptr(A),
        _ptr(B), B_kind, _ptr(C), C_kind, _ptr(delta_bias), _ptr(z), int(bool(delta_softplus)),
        _ptr(init), _ptr(dout), _ptr(out["ddelta"]), _ptr(out["ddelta_bias"]), _ptr(out["dA"]))
    if rc != 0:
        raise ValueError(f"oracle_selective_scan_complex_bwd_f32_floor failed with status {rc}")
    return out


def causal_conv1d_ex(x, weight, bias=None, act=ACT_NONE, *, io_dtype=F32, seq_idx=None,
                     initial_states=None, want_final=False):
    """Oracle causal_conv1d with seq_idx / initial_states / final states.

    x: (batch, dim, seqlen) io bits; weight (dim, width) float32; seq_idx
    (batch, seqlen) int32; initial_states (batch, dim, width-1) io bits.
    Returns (out (batch, dim, seqlen) float64, final_states (batch, dim,
    width-1) float64 or None).
    """
    lib = _load()
    x = _io(x, io_dtype)
    batch, dim, seqlen = x.shape
    weight = _f32(weight)
    width = weight.shape[1]
    bias = _f32(bias)
    init = _io(initial_states, io_dtype)
    sq = None if seq_idx is None else np.ascontiguousarray(seq_idx, dtype=np.int32)
    out = np.empty((batch, dim, seqlen))
    fin = np.empty((batch, dim, width - 1)) if want_final else None
    rc = lib.oracle_causal_conv1d_ex(batch, dim, seqlen, width, io_dtype, _ptr(x), _ptr(weight), _ptr(bias),
                                     act, _ptr(sq), _ptr(init), _ptr(out), _ptr(fin))
    if rc != 0:
        raise ValueError(f"oracle_causal_conv1d_ex failed with status {rc}")
    return out, fin
