"""Gradient of the scan (ssm_scan_bwd) against the fp64 oracle's reverse-mode
gradient (needs MI355X). The loss is sum(dy * y) + sum(dstate * state_out);
the states are recomputed from 32-token chunks ("Notas sobre Mamba", section
"A varredura paralela ciente do hardware"). Shapes cover several chunks with
a ragged last chunk, channel blocks cut short (with whole waves past the last
channel), every state size, every option on and off, the empty cases, the
small-layer workload whole, and sampled channels of the large-layer workload."""
import numpy as np
import pytest

import oracle
import selective_state_space_16_amd as ssm
import workloads as W
from gpu_util import check_grads, gpu_scan_bwd, oracle_scan_bwd, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _cfg(name, batch, L, D, N=16, dtype="f32", gate=True, dskip="uniform", state_in=0.3, seed=80):
    return W.ScanConfig(name, batch, L, D, N, dtype, gate=gate, dskip=dskip, state_in=state_in, seed=seed)


def _run(cfg, dstate=True, **kw):
    say(f"case {cfg} dstate={'given' if dstate else 'NULL'}")
    inp = W.scan_inputs(cfg)
    grads = W.grad_inputs(cfg, dstate=dstate)
    got = gpu_scan_bwd(inp, grads, **kw)
    ref = oracle_scan_bwd(inp, grads, cfg.dtype)
    check_grads(got, ref, cfg.dtype)
    return got


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 200])
def test_bwd_chunks(dtype, D):
    """4 chunks, the last 4 tokens long; D = 200 leaves a short channel block."""
    _run(_cfg(f"bwd_{D}", 2, 100, D, 16, dtype))


@pytest.mark.parametrize("N", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_state_sizes(N, dtype):
    _run(_cfg(f"bwd_N{N}", 2, 77, 300, N, dtype))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_no_options(dtype):
    """No gate, no skip term, zero start, no gradient of the final state."""
    _run(_cfg("bwd_plain", 1, 130, 96, 16, dtype, gate=False, dskip="none", state_in=None), dstate=False)


@pytest.mark.parametrize("L", [1, 7, 31, 32, 33, 64, 257])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_ragged_lengths(L, dtype):
    """Chunks of 1 to 32 tokens and blocks of 1 to 8; with bfloat16 the
    chunk's activations are staged in LDS only up to its last token."""
    _run(_cfg(f"bwd_L{L}", 1, L, 128, 16, dtype, seed=81))


def test_bwd_skip_without_its_gradient():
    """Dskip given, dDskip not asked for: the call leaves it out."""
    cfg = _cfg("bwd_nodD", 1, 40, 64)
    inp, grads = W.scan_inputs(cfg), W.grad_inputs(cfg)
    got = gpu_scan_bwd(inp, grads, want_dskip=False)
    ref = oracle_scan_bwd(inp, grads, "f32")
    assert got["dDskip"] is None
    ref["dDskip"] = None
    check_grads(got, ref, "f32")


def test_bwd_dstate_in_aliases_dstate():
    cfg = _cfg("bwd_alias", 2, 90, 64)
    inp, grads = W.scan_inputs(cfg), W.grad_inputs(cfg)
    got = gpu_scan_bwd(inp, grads, dstate_alias=True)
    check_grads(got, oracle_scan_bwd(inp, grads, "f32"), "f32")


def test_bwd_deterministic():
    """Every sum runs in a fixed order: equal inputs give equal bits."""
    cfg = _cfg("bwd_det", 2, 300, 256, 16, "bf16")
    inp, grads = W.scan_inputs(cfg), W.grad_inputs(cfg)
    a = gpu_scan_bwd(inp, grads)
    b = gpu_scan_bwd(inp, grads)
    for k, v in a.items():
        if v is not None:
            assert np.array_equal(v, b[k]), k


@pytest.mark.parametrize("batch,L", [(2, 0), (0, 5)])
def test_bwd_empty(batch, L):
    """No tokens: dA and dDskip are zero and dstate_in is dstate."""
    import torch
    D, N = 64, 16
    say(f"case empty batch={batch} L={L}")
    f = lambda *s: torch.randn(*s, device="cuda")
    x = f(batch, L, D)
    out = {"dA": torch.full((D, N), 7.0, device="cuda"), "dDskip": torch.full((D,), 7.0, device="cuda"),
           "dstate_in": torch.full((batch, D, N), 7.0, device="cuda")}
    dstate = f(batch, D, N)
    g = ssm.ssm_scan_bwd(x, f(batch, L, D), -torch.rand(D, N, device="cuda"), f(batch, L, N), f(batch, L, N),
                         f(batch, L, D), Dskip=f(D), z=f(batch, L, D), dstate=dstate, out=out)
    torch.cuda.synchronize()
    assert torch.all(g["dA"] == 0) and torch.all(g["dDskip"] == 0)
    assert torch.equal(g["dstate_in"], dstate)


def test_bwd_small_layer_whole():
    """The small-layer workload (batch 2, 2048 tokens, 1536 channels, N 16,
    float32, gate and skip on), every gradient whole."""
    cfg = W.SCAN_CONFIGS["c1"]
    _run(dataclass_replace(cfg, state_in=0.3))


def test_bwd_large_layer_sampled():
    """The large-layer workload (batch 8, 4096 tokens, 5120 channels, N 16,
    bfloat16) run whole on the GPU; the per-channel gradients (dx, ddelta,
    dz, dA, dDskip, dstate_in) checked on sampled channels, which the oracle
    computes exactly from those channels alone. dBt and dCt sum over all
    channels and are checked whole on the small layer."""
    import torch
    cfg = W.SCAN_CONFIGS["c2"]
    sel = np.array([0, 1, 63, 64, 127, 128, 129, 64 * 40 + 5, 64 * 40 + 60, cfg.D - 2, cfg.D - 1])
    say(f"case {cfg.name} full size, sampled channels {list(sel)}")
    part = W.scan_inputs(cfg, channels=sel)
    gpart = W.grad_inputs(cfg, channels=sel)
    fill = W.fill_scan_device(cfg, "cuda")
    whole = W.scan_inputs(cfg, 0, 0)  # A, Dskip, state_in for every channel
    sel_t = torch.as_tensor(sel, device="cuda")
    for k in ("x", "delta", "z"):
        fill[k][:, :, sel_t] = to_dev(part[k])
    fill["Bt"], fill["Ct"] = to_dev(part["Bt"]), to_dev(part["Ct"])
    dy = torch.randn((cfg.batch, cfg.L, cfg.D), device="cuda").to(torch.bfloat16)
    dy[:, :, sel_t] = to_dev(gpart["dy"])
    dstate = to_dev(W.grad_inputs(cfg, 0, 0)["dstate"])
    g = ssm.ssm_scan_bwd(fill["x"], fill["delta"], to_dev(whole["A"]), fill["Bt"], fill["Ct"], dy,
                         Dskip=to_dev(whole["Dskip"]), z=fill["z"], state_in=to_dev(whole["state_in"]),
                         dstate=dstate)
    torch.cuda.synchronize()
    ref = oracle_scan_bwd(part, gpart, cfg.dtype)
    got = {"dx": to_f64(g["dx"][:, :, sel_t]), "ddelta": to_f64(g["ddelta"][:, :, sel_t]),
           "dz": to_f64(g["dz"][:, :, sel_t]), "dA": to_f64(g["dA"][sel_t]), "dDskip": to_f64(g["dDskip"][sel_t]),
           "dstate_in": to_f64(g["dstate_in"][:, sel_t])}
    check_grads(got, ref, cfg.dtype, keys=("dx", "ddelta", "dz", "dA", "dDskip", "dstate_in"))


def dataclass_replace(cfg, **kw):
    import dataclasses
    return dataclasses.replace(cfg, **kw)


def _run_raw(cfg, bias=True, want_dbias=True):
    say(f"case {cfg} raw delta, dt_bias={'given' if bias else 'NULL'}")
    inp = W.scan_inputs(cfg, raw_delta=True)
    if not bias:
        inp["dt_bias"] = None
    grads = W.grad_inputs(cfg)
    got = gpu_scan_bwd(inp, grads, raw=True, want_dbias=want_dbias)
    ref = oracle.get().scan_bwd_dt(inp, grads["dy"], grads["dstate"], cfg.dtype)
    if not want_dbias:
        assert got["ddt_bias"] is None
        ref["ddt_bias"] = None
    check_grads(got, ref, cfg.dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bias", [True, False])
def test_bwd_raw_delta(dtype, bias):
    """ssm_scan_bwd_dt: the step size activated in the kernel, softplus(raw + bias)."""
    _run_raw(_cfg("bwd_raw", 2, 100, 200, 16, dtype), bias=bias)


@pytest.mark.parametrize("N", [1, 4, 8])
def test_bwd_raw_delta_state_sizes(N):
    _run_raw(_cfg(f"bwd_raw_N{N}", 1, 77, 130, N, "f32"))


def test_bwd_raw_delta_without_bias_gradient():
    _run_raw(_cfg("bwd_raw_nob", 1, 40, 64, 16, "bf16"), want_dbias=False)


def test_bwd_raw_delta_small_layer_whole():
    """The small-layer workload with its step size given before the activation."""
    _run_raw(dataclass_replace(W.SCAN_CONFIGS["c1"], state_in=0.3))


def _run_trap(cfg, prev=True):
    say(f"case {cfg} trapezoidal, x_prev/B_prev={'given' if prev else 'NULL'}")
    inp = W.scan_inputs(cfg, trap=True)
    if not prev:
        inp["x_prev"] = inp["B_prev"] = None
    grads = W.grad_inputs(cfg)
    got = gpu_scan_bwd(inp, grads, trap=True)
    ref = oracle.get().scan_bwd_trap(inp, grads["dy"], grads["dstate"], cfg.dtype)
    check_grads(got, ref, cfg.dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("prev", [True, False])
def test_bwd_trap(dtype, prev):
    """ssm_scan_bwd_trap: 4 chunks with a ragged tail, a short channel block,
    with and without the token before the first."""
    _run_trap(_cfg("bwd_trap", 2, 100, 200, 16, dtype), prev=prev)


@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_bwd_trap_state_sizes(N):
    _run_trap(_cfg(f"bwd_trap_N{N}", 2, 77, 130, N, "f32"))


@pytest.mark.parametrize("L", [1, 31, 33, 257])
def test_bwd_trap_ragged_lengths(L):
    _run_trap(_cfg(f"bwd_trap_L{L}", 1, L, 64, 16, "f32", seed=82))


def test_bwd_trap_no_options():
    _run_trap(_cfg("bwd_trap_plain", 1, 70, 64, 16, "f32", gate=False, dskip="none", state_in=None), prev=False)


def test_bwd_trap_small_layer_whole():
    """The small-layer workload with the trapezoidal rule, every gradient whole."""
    _run_trap(dataclass_replace(W.SCAN_CONFIGS["c1"], state_in=0.3))


def test_bwd_million_token_sampled():
    """The million-token workload (1 x 1,048,576 x 1536, N 16, bfloat16,
    carried-in state): 32,768 chunks, the largest gradient grid here, run whole
    on the GPU; the per-channel gradients checked on sampled channels against
    the oracle over the whole sequence."""
    import torch
    cfg = W.SCAN_CONFIGS["c3"]
    sel = np.array([0, 700, cfg.D - 1])
    say(f"case {cfg.name} full size, sampled channels {list(sel)}")
    part = W.scan_inputs(cfg, channels=sel)
    gpart = W.grad_inputs(cfg, channels=sel)
    fill = W.fill_scan_device(cfg, "cuda")
    whole = W.scan_inputs(cfg, 0, 0)
    sel_t = torch.as_tensor(sel, device="cuda")
    for k in ("x", "delta", "z"):
        fill[k][:, :, sel_t] = to_dev(part[k])
    fill["Bt"], fill["Ct"] = to_dev(part["Bt"]), to_dev(part["Ct"])
    dy = torch.randn((cfg.batch, cfg.L, cfg.D), device="cuda").to(torch.bfloat16)
    dy[:, :, sel_t] = to_dev(gpart["dy"])
    dstate = to_dev(W.grad_inputs(cfg, 0, 0)["dstate"])
    g = ssm.ssm_scan_bwd(fill["x"], fill["delta"], to_dev(whole["A"]), fill["Bt"], fill["Ct"], dy,
                         Dskip=to_dev(whole["Dskip"]), z=fill["z"], state_in=to_dev(whole["state_in"]),
                         dstate=dstate)
    torch.cuda.synchronize()
    del fill, dy
    ref = oracle_scan_bwd(part, gpart, cfg.dtype)
    got = {"dx": to_f64(g["dx"][:, :, sel_t]), "ddelta": to_f64(g["ddelta"][:, :, sel_t]),
           "dz": to_f64(g["dz"][:, :, sel_t]), "dA": to_f64(g["dA"][sel_t]), "dDskip": to_f64(g["dDskip"][sel_t]),
           "dstate_in": to_f64(g["dstate_in"][:, sel_t])}
    check_grads(got, ref, cfg.dtype, keys=("dx", "ddelta", "dz", "dA", "dDskip", "dstate_in"))


@pytest.mark.parametrize("D,N", [(1, 16), (3, 16), (63, 16), (129, 2), (5, 1)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_ragged_channels(D, N, dtype):
    """Channel counts that leave most lanes of the last block idle, including
    whole waves past the last channel (with bfloat16 they read the staged rows
    of the last existing channel)."""
    _run(_cfg(f"bwd_D{D}_N{N}", 2, 45, D, N, dtype, seed=83))


@pytest.mark.parametrize("D", [1, 63])
def test_bwd_trap_ragged_channels(D):
    _run_trap(_cfg(f"bwd_trap_D{D}", 2, 45, D, 16, "bf16", seed=84))
