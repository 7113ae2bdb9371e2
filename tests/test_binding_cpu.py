"""The Python wrappers reject tensors that do not match the sizes delta (or
x) and A fix, a wrong dtype, an in-place output that is not contiguous and a
tensor off the GPU -- with ValueError, before anything reaches the library.
CPU tensors only: every call here stops in the wrapper (the last check of a
well-formed call is the device check)."""
import pytest
import torch

from state_space_model_scan_amd import binding

b, d, l, n, G = 2, 8, 12, 4, 2
bf, f32 = torch.bfloat16, torch.float32


def _scan(**kw):
    t = dict(u=torch.zeros(b, d, l, dtype=bf), delta=torch.zeros(b, d, l, dtype=bf),
             A=torch.zeros(d, n), B=torch.zeros(b, G, n, l, dtype=bf), C=torch.zeros(b, G, n, l, dtype=bf),
             D=torch.zeros(d), z=torch.zeros(b, d, l, dtype=bf), delta_bias=torch.zeros(d))
    t.update(kw)
    return t


def test_well_formed_scan_stops_at_the_device_check():
    with pytest.raises(ValueError, match="cuda device"):
        binding.ssm_scan_fwd(**_scan())
    with pytest.raises(ValueError, match="cuda device"):
        binding.ssm_scan_fwd(**_scan(B=torch.zeros(d, n, dtype=bf), C=torch.zeros(b, n, l, dtype=bf)))
    with pytest.raises(ValueError, match="cuda device"):
        binding.ssm_scan_fwd_noalloc(**_scan(), out=torch.zeros(b, d, l, dtype=bf))


@pytest.mark.parametrize("field,bad,msg", [
    ("u", torch.zeros(b, d, l - 1, dtype=bf), "u must have shape"),
    ("z", torch.zeros(b, d + 1, l, dtype=bf), "z must have shape"),
    ("A", torch.zeros(d - 1, n), "A must be"),
    ("A", torch.zeros(d, n, dtype=torch.float64), "A must be float32"),
    ("B", torch.zeros(b, G, n - 1, l, dtype=bf), "B must have shape"),
    ("B", torch.zeros(b, G, n, l + 4, dtype=bf), "B must have shape"),
    ("C", torch.zeros(b + 1, G, n, l, dtype=bf), "C must have shape"),
    ("C", torch.zeros(d + 1, n, dtype=bf), "C must have shape"),
    ("D", torch.zeros(d + 1), "D must have shape"),
    ("delta_bias", torch.zeros(d, 1), "delta_bias must have shape"),
    ("delta", torch.zeros(b, d, l, dtype=torch.int32), "io dtype"),
    ("delta", torch.zeros(d, l, dtype=bf), "delta must have 3 dimensions"),
])
def test_scan_input_rejections(field, bad, msg):
    with pytest.raises(ValueError, match=msg):
        binding.ssm_scan_fwd(**_scan(**{field: bad}))


def test_scan_output_rejections():
    t = _scan()
    with pytest.raises(ValueError, match="last_state must have shape"):
        binding.ssm_scan_fwd(**t, last_state=torch.zeros(b, d))
    with pytest.raises(ValueError, match="last_state must be torch.float32"):
        binding.ssm_scan_fwd(**t, last_state=torch.zeros(b, d, n, dtype=bf))
    with pytest.raises(ValueError, match="last_state is written in place"):
        binding.ssm_scan_fwd(**t, last_state=torch.zeros(b, n, d).transpose(1, 2))
    with pytest.raises(ValueError, match="out is written in place"):
        binding.ssm_scan_fwd(**t, out=torch.zeros(b, l, d, dtype=bf).transpose(1, 2))
    with pytest.raises(ValueError, match="out must have shape"):
        binding.ssm_scan_fwd(**t, out=torch.zeros(b, d, l - 1, dtype=bf))
    with pytest.raises(ValueError, match="initial_state must have shape"):
        binding.ssm_scan_fwd(**t, initial_state=torch.zeros(b, d, n + 1))
    with pytest.raises(ValueError, match="checkpoints must have shape"):
        binding.ssm_scan_fwd(**t, checkpoints=torch.zeros(b, d, 2, n))
    with pytest.raises(ValueError, match="needs a caller-allocated out"):
        binding.ssm_scan_fwd_noalloc(**t)


def test_scan_mixed_devices_are_rejected():
    if not torch.cuda.is_available():
        meta = torch.zeros(d, device="meta")
    else:
        meta = torch.zeros(d, device="cuda")
    with pytest.raises(ValueError, match="must be on cpu"):
        binding.ssm_scan_fwd(**_scan(D=meta))


def test_conv_prologue_rejections():
    t = _scan(u=None)
    x = torch.zeros(b, d, l, dtype=bf)
    with pytest.raises(ValueError, match="conv_weight must have shape"):
        binding.ssm_scan_fwd(**t, conv_x=x, conv_weight=torch.zeros(d + 1, 4))
    with pytest.raises(ValueError, match="conv_bias must have shape"):
        binding.ssm_scan_fwd(**t, conv_x=x, conv_weight=torch.zeros(d, 4), conv_bias=torch.zeros(1))
    with pytest.raises(ValueError, match="conv_x must have shape"):
        binding.ssm_scan_fwd(**t, conv_x=x[:, :, :-1], conv_weight=torch.zeros(d, 4))
    with pytest.raises(ValueError, match="needs conv_x"):
        binding.ssm_scan_fwd(**t, conv_weight=torch.zeros(d, 4))
    with pytest.raises(ValueError, match="u is required"):
        binding.ssm_scan_fwd(**t)
    with pytest.raises(ValueError, match="cuda device"):
        binding.conv1d_selective_scan_fn(x, torch.zeros(d, 4), torch.zeros(d), t["delta"], t["A"],
                                         t["B"], t["C"])


def test_complex_rejections():
    c64 = torch.complex64
    u = torch.zeros(b, d, l)
    A = torch.zeros(d, n, dtype=c64)
    Bv = torch.zeros(b, G, n, l, dtype=c64)
    with pytest.raises(ValueError, match="cuda device"):
        binding.ssm_scan_fwd_complex(u, u, A, Bv, Bv)
    with pytest.raises(ValueError, match="B must have shape"):
        binding.ssm_scan_fwd_complex(u, u, A, torch.zeros(b, G, n, l - 1, dtype=c64), Bv)
    with pytest.raises(ValueError, match="A must be"):
        binding.ssm_scan_fwd_complex(u, u, torch.zeros(d + 1, n, dtype=c64), Bv, Bv)
    with pytest.raises(ValueError, match="last_state must have shape"):
        binding.ssm_scan_fwd_complex(u, u, A, Bv, Bv, last_state=torch.zeros(b, d, n + 1, dtype=c64))
    with pytest.raises(ValueError, match="initial_state must have shape"):
        binding.ssm_scan_fwd_complex(u, u, A, Bv, Bv, initial_state=torch.zeros(b, d, 1, dtype=c64))
    with pytest.raises(ValueError, match="z must have shape"):
        binding.ssm_scan_fwd_complex(u, u, A, Bv, Bv, z=torch.zeros(b, d, l + 1))
    with pytest.raises(ValueError, match="u is required"):
        binding.ssm_scan_fwd_complex(None, u, A, Bv, Bv)


def test_bwd_rejections():
    t = _scan()
    ck = torch.zeros(b, d, binding.checkpoint_count(l), n)
    args = (t["u"], t["delta"], t["A"], t["B"], t["C"])
    with pytest.raises(ValueError, match="cuda device"):
        binding.ssm_scan_bwd(*args, t["delta"], ck)
    with pytest.raises(ValueError, match="dout must have shape"):
        binding.ssm_scan_bwd(*args, t["delta"][:, :, :-1], ck)
    with pytest.raises(ValueError, match="z must have shape"):
        binding.ssm_scan_bwd(*args, t["delta"], ck, z=torch.zeros(b, d, 1, dtype=bf))
    with pytest.raises(ValueError, match="A must be"):
        binding.ssm_scan_bwd(t["u"], t["delta"], torch.zeros(d + 2, n), t["B"], t["C"], t["delta"], ck)


def test_conv_rejections():
    x = torch.zeros(b, d, l, dtype=bf)
    w = torch.zeros(d, 4)
    with pytest.raises(ValueError, match="cuda device"):
        binding.causal_conv1d_fwd(x, w)
    with pytest.raises(ValueError, match="weight must have shape"):
        binding.causal_conv1d_fwd(x, torch.zeros(d - 1, 4))
    with pytest.raises(ValueError, match="bias must have shape"):
        binding.causal_conv1d_fwd(x, w, torch.zeros(d + 1))
    with pytest.raises(ValueError, match="out is written in place"):
        binding.causal_conv1d_fwd(x, w, out=torch.zeros(b, l, d, dtype=bf).transpose(1, 2))
    with pytest.raises(ValueError, match="cuda device"):
        binding.causal_conv1d_fwd_ex(x, w, final_states=torch.zeros(b, d, 3, dtype=bf))
    with pytest.raises(ValueError, match="out must have shape"):
        binding.causal_conv1d_fwd_ex(x, w, out=torch.zeros(b, d, 1, dtype=bf))


def test_decode_rejections():
    st = torch.zeros(b, d, n)
    x = torch.zeros(b, d, dtype=bf)
    A = torch.zeros(d, n)
    Bd = torch.zeros(b, G, n, dtype=bf)
    with pytest.raises(ValueError, match="cuda device"):
        binding.selective_state_update(st, x, x, A, Bd, Bd)
    with pytest.raises(ValueError, match="dt must have shape"):
        binding.selective_state_update(st, x, torch.zeros(b, d + 1, dtype=bf), A, Bd, Bd)
    with pytest.raises(ValueError, match="B must have shape"):
        binding.selective_state_update(st, x, x, A, torch.zeros(b, G, n + 1, dtype=bf), torch.zeros(b, G, n + 1, dtype=bf))
    with pytest.raises(ValueError, match="A must have shape"):
        binding.selective_state_update(st, x, x, torch.zeros(d, n - 1), Bd, Bd)
    with pytest.raises(ValueError, match="out is written in place"):
        binding.selective_state_update(st, x, x, A, Bd, Bd, out=torch.zeros(d, b, dtype=bf).t())
    cs = torch.zeros(b, d, 3, dtype=bf)
    with pytest.raises(ValueError, match="cuda device"):
        binding.causal_conv1d_update(x, cs, torch.zeros(d, 4))
    with pytest.raises(ValueError, match="conv_state must have shape"):
        binding.causal_conv1d_update(x, torch.zeros(b + 1, d, 3, dtype=bf), torch.zeros(d, 4))
    with pytest.raises(ValueError, match="cache_seqlens must have shape"):
        binding.causal_conv1d_update(x, cs, torch.zeros(d, 4), cache_seqlens=torch.zeros(b + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="out must have shape"):
        binding.causal_conv1d_update(x, cs, torch.zeros(d, 4), out=torch.zeros(b, d, 1, dtype=bf))


def test_ssd_rejections():
    h, p, nn, g = 4, 8, 16, 1
    x = torch.zeros(b, l, h, p, dtype=bf)
    dt = torch.zeros(b, l, h, dtype=bf)
    A = torch.zeros(h)
    B = torch.zeros(b, l, g, nn, dtype=bf)
    with pytest.raises(ValueError, match="cuda device"):
        binding.ssd_scan_fwd(x, dt, A, B, B)
    with pytest.raises(ValueError, match="dt must have shape"):
        binding.ssd_scan_fwd(x, dt[:, :-1], A, B, B)
    with pytest.raises(ValueError, match="C must have shape"):
        binding.ssd_scan_fwd(x, dt, A, B, torch.zeros(b, l, g, nn + 1, dtype=bf))
    with pytest.raises(ValueError, match="D must have shape"):
        binding.ssd_scan_fwd(x, dt, A, B, B, D=torch.zeros(h, p + 1))
    with pytest.raises(ValueError, match="final_states must have shape"):
        binding.ssd_scan_fwd(x, dt, A, B, B, final_states=torch.zeros(b, h, p, nn - 1))
    with pytest.raises(ValueError, match="final_states is written in place"):
        binding.ssd_scan_fwd(x, dt, A, B, B, final_states=torch.zeros(b, h, nn, p).transpose(2, 3))
