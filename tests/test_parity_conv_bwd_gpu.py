"""ssm_scan_bwd_conv (the gradient of the scan behind the Mamba block's x
branch: through the scan, then SiLU and the causal width-4 convolution)
against the fp64 oracle's chain rule (needs MI355X). Shapes cover ragged
lengths across the convolution's chunks and register blocks, ragged channel
counts, N from 1 to 16, both dtypes, the optional parts, empty inputs and
bitwise determinism."""
import numpy as np
import pytest

import oracle
import selective_state_space_16_amd as ssm
import workloads as W
from gpu_util import check_grads, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

KEYS = ("dx_raw", "dconv_w", "dconv_b", "dconv_state", "ddelta_raw", "ddt_bias", "dz", "dA", "dBt", "dCt", "dDskip",
        "dstate_in")


def _cfg(name, batch, L, D, N=16, dtype="f32", gate=True, dskip="uniform", state_in=0.3, seed=93):
    return W.ScanConfig(name, batch, L, D, N, dtype, gate=gate, dskip=dskip, state_in=state_in, seed=seed)


def gpu_scan_bwd_conv(inp, grads):
    import torch
    dev = {k: to_dev(v) for k, v in inp.items()}
    g = ssm.ssm_scan_bwd_conv(dev["x_raw"], dev["conv_w"], dev["delta_raw"], dev.get("dt_bias"), dev["A"], dev["Bt"],
                              dev["Ct"], to_dev(grads["dy"]), conv_b=dev.get("conv_b"),
                              conv_state=dev.get("conv_state"), Dskip=dev.get("Dskip"), z=dev.get("z"),
                              state_in=dev.get("state_in"), dstate=to_dev(grads.get("dstate")))
    torch.cuda.synchronize()
    return {k: (None if v is None else to_f64(v)) for k, v in g.items()}


def _run(cfg, conv_state=True, conv_b=True):
    say(f"case {cfg} conv_state={conv_state} conv_b={conv_b}")
    inp = W.scan_inputs(cfg, raw_delta=True, conv=True)
    if not conv_state:
        inp["conv_state"] = None
    if not conv_b:
        inp["conv_b"] = None
    grads = W.grad_inputs(cfg)
    got = gpu_scan_bwd_conv(inp, grads)
    ref = oracle.get().scan_bwd_conv(inp, grads["dy"], grads["dstate"], cfg.dtype)
    if not conv_state:
        ref["dconv_state"] = None
    if not conv_b:
        ref["dconv_b"] = None
    check_grads(got, ref, cfg.dtype, KEYS)
    return got


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 200])
def test_bwd_conv(dtype, D):
    _run(_cfg(f"bwdconv_{D}", 2, 300, D, 16, dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_conv_no_state_no_bias(dtype):
    _run(_cfg("bwdconv_bare", 2, 150, 64, 16, dtype), conv_state=False, conv_b=False)


@pytest.mark.parametrize("N", [1, 4, 8])
def test_bwd_conv_state_sizes(N):
    _run(_cfg(f"bwdconv_N{N}", 2, 130, 96, N, "f32"))


@pytest.mark.parametrize("L", [1, 2, 3, 17, 33, 1025])
def test_bwd_conv_ragged_lengths(L):
    """Shorter than the window, one past a register block, and several chunks
    with a ragged tail."""
    _run(_cfg(f"bwdconv_L{L}", 2, L, 37, 16, "f32"))


@pytest.mark.parametrize("gate,dskip", [(False, "uniform"), (True, "none"), (False, "none")])
def test_bwd_conv_optional_parts(gate, dskip):
    _run(_cfg("bwdconv_opt", 1, 200, 64, 16, "bf16", gate=gate, dskip=dskip, state_in=None))


def test_bwd_conv_small_layer_whole():
    """The small layer (2 x 2048 x 1536, float32), every gradient."""
    _run(W.SCAN_CONFIGS["c1"])


def test_bwd_conv_deterministic():
    cfg = _cfg("bwdconv_det", 2, 700, 128, 16, "bf16")
    inp = W.scan_inputs(cfg, raw_delta=True, conv=True)
    grads = W.grad_inputs(cfg)
    a = gpu_scan_bwd_conv(inp, grads)
    b = gpu_scan_bwd_conv(inp, grads)
    for k in KEYS:
        assert (a[k] is None and b[k] is None) or np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("batch,L", [(0, 50), (2, 0)])
def test_bwd_conv_empty(batch, L):
    """No token: zero gradients of the taps, bias and earlier raw tokens."""
    import torch
    D, N = 64, 16
    x = torch.zeros((batch, L, D), device="cuda")
    A = -torch.ones((D, N), device="cuda")
    bt = torch.zeros((batch, L, N), device="cuda")
    w = torch.ones((D, 4), device="cuda")
    cb = torch.ones((D,), device="cuda")
    cs = torch.ones((batch, D, 3), device="cuda")
    out = {"dconv_w": torch.full((D, 4), 7.0, device="cuda"), "dconv_b": torch.full((D,), 7.0, device="cuda"),
           "dconv_state": torch.full((batch, D, 3), 7.0, device="cuda")}
    g = ssm.ssm_scan_bwd_conv(x, w, x, None, A, bt, bt, x, conv_b=cb, conv_state=cs, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g["dconv_w"]) == 0 and torch.count_nonzero(g["dconv_b"]) == 0
    assert torch.count_nonzero(g["dconv_state"]) == 0
