"""GPU path against the fp64 oracle on the same seeded inputs (needs MI355X).

Small and medium cases compare every output on the seeded numpy streams; the
full-size workloads (large layer, million tokens, 1000 decode steps) compare
every output too, in the launch configuration the bench times, on inputs
drawn on the device with the same recipe (seeded torch draws) and copied back
as stored values for the oracle."""
import numpy as np
import pytest

import workloads as W
from gpu_util import (TOL, check, check_sum, device_scan_blocks, errors, gpu_scan, oracle_scan, say,
                      to_dev, to_f64, to_host)

pytestmark = pytest.mark.gpu


def _cfg(name, batch, L, D, N=16, dtype="f32", gate=True, dskip="uniform", state_in=None, seed=11):
    return W.ScanConfig(name, batch, L, D, N, dtype, gate=gate, dskip=dskip, state_in=state_in, seed=seed)


def _run_full(cfg, want_state=None):
    say(f"case {cfg}")
    inp = W.scan_inputs(cfg)
    want_state = (cfg.state_in is not None) if want_state is None else want_state
    y, st = gpu_scan(inp, want_state=True)
    yr, sr = oracle_scan(inp, cfg.dtype)
    check(y, yr, cfg.dtype, "y")
    check(st, sr, cfg.dtype, "state_out")
    return y, yr


def test_c0_tiny_f32():
    _run_full(W.SCAN_CONFIGS["c0"])


def test_c1_small_layer_f32():
    _run_full(W.SCAN_CONFIGS["c1"])


@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_state_sizes(N, dtype):
    _run_full(_cfg(f"N{N}", 2, 333, 130, N, dtype, gate=True, state_in=0.5, seed=20 + N))


@pytest.mark.parametrize("L", [1, 2, 7, 63, 64, 65, 129, 1000, 4097])
def test_ragged_lengths(L):
    _run_full(_cfg(f"L{L}", 1, L, 96, 16, "f32", gate=True, state_in=0.3, seed=40))


@pytest.mark.parametrize("D", [1, 3, 63, 64, 65, 200])
def test_ragged_channels(D):
    _run_full(_cfg(f"D{D}", 3, 300, D, 16, "f32", gate=True, state_in=0.3, seed=50))


@pytest.mark.parametrize("L", [1, 7, 65, 1000, 4097])
def test_ragged_lengths_bf16(L):
    """bfloat16 tiles of 64 tokens: the last tile of a sequence runs past L."""
    _run_full(_cfg(f"L{L}b", 1, L, 96, 16, "bf16", gate=True, state_in=0.3, seed=41))


@pytest.mark.parametrize("D,dtype", [(4, "f32"), (68, "f32"), (132, "f32"), (8, "bf16"), (56, "bf16"),
                                     (72, "bf16"), (200, "bf16"), (264, "bf16")])
def test_partial_channel_columns(D, dtype):
    """Widths that are whole 16-byte pieces but not whole 64-channel tile
    columns: the last column's loads clamp to the row and its extra channels
    are never stored."""
    _run_full(_cfg(f"D{D}{dtype}", 2, 777, D, 16, dtype, gate=True, state_in=0.3, seed=51))


@pytest.mark.parametrize("gate,dskip,state", [(False, "none", None), (True, "none", None),
                                              (False, "uniform", 1.0), (True, "one", 0.1)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_optional_parts(gate, dskip, state, dtype):
    _run_full(_cfg("opt", 2, 700, 100, 16, dtype, gate=gate, dskip=dskip, state_in=state, seed=60))


def test_c2_twin_bf16():
    """Large-layer recipe at reduced width: every output compared."""
    _run_full(_cfg("c2_twin", 2, 4096, 320, 16, "bf16", gate=True, seed=2))


def test_c3_twin_bf16():
    """Million-token recipe at reduced length and width: carried-in and final state."""
    _run_full(_cfg("c3_twin", 1, 131072, 128, 16, "bf16", gate=True, state_in=0.1, seed=3))


def _run_full_size(cfg, chans, seed):
    """The workload at full size, in the launch configuration the bench times
    (one call, a workspace given, inputs resident on the device): inputs drawn
    on the device with the workload's recipe (seeded), every output and every
    final-state value compared with the oracle on the same stored values,
    `chans` channels of one batch row at a time."""
    import torch
    import oracle
    import selective_state_space_16_amd as ssm
    say(f"case {cfg.name} full size, every output (device-drawn inputs, seed {seed})")
    dev = W.fill_scan_device(cfg, "cuda", seed=seed)
    whole = W.scan_inputs(cfg, 0, 0)  # A, Dskip, state_in for every channel
    dev["A"], dev["Dskip"], dev["state_in"] = to_dev(whole["A"]), to_dev(whole["Dskip"]), to_dev(whole["state_in"])
    st_out = torch.empty((cfg.batch, cfg.D, cfg.N), dtype=torch.float32, device="cuda")
    ws = ssm.new_workspace(ssm.ssm_scan_workspace_bytes(cfg.batch, cfg.L, cfg.D, cfg.N,
                                                        0 if cfg.dtype == "f32" else 1))
    y = ssm.ssm_scan_fwd(dev["x"], dev["delta"], dev["A"], dev["Bt"], dev["Ct"], Dskip=dev["Dskip"], z=dev["z"],
                         state_in=dev["state_in"], state_out=st_out, workspace=ws)
    torch.cuda.synchronize()
    assert ssm.ssm_scan_workspace_status(ws) == 0, "a look-back wait gave up"
    ey, es, secs = oracle.scan_compare(device_scan_blocks(dev, y, st_out, chans), cfg.dtype)
    say(f"  oracle: {secs:.1f}s on {oracle.get().threads()} threads")
    assert ey.count == cfg.batch * cfg.L * cfg.D and es.count == cfg.batch * cfg.D * cfg.N
    check_sum(ey, cfg.dtype, "y (every output)")
    check_sum(es, cfg.dtype, "state_out (every value)")


def test_c2_full_size_every_output():
    _run_full_size(W.SCAN_CONFIGS["c2"], chans=5120, seed=202)


def test_c3_full_size_every_output():
    """The million-token workload: all 24 tile columns (cut into stripes that
    run at the same time) and the final state of every channel."""
    _run_full_size(W.SCAN_CONFIGS["c3"], chans=64, seed=303)


def test_c4_decode_1000_steps_every_channel():
    """The decode workload: (256, 5120, 16) float32 state updated in place for
    1000 steps with device-drawn tokens (seeded); y of every channel at every
    step and the whole final state against 1000 oracle steps on the same
    stored values."""
    import torch
    import oracle
    import selective_state_space_16_amd as ssm
    cfg = W.STEP_CONFIG
    steps = cfg.steps
    say(f"case {cfg.name}: {steps} steps, every channel")
    base = W.step_inputs(cfg)
    state = to_dev(base["state"])
    A, Dskip = to_dev(base["A"]), to_dev(base["Dskip"])
    fill = W.fill_step_device(cfg, steps, "cuda", seed=404)
    ys = torch.empty((steps, cfg.batch, cfg.D), dtype=fill["x"].dtype, device="cuda")
    for s in range(steps):
        ssm.ssm_step(fill["x"][s], fill["delta"][s], A, fill["Bt"][s], fill["Ct"][s], state,
                     Dskip=Dskip, z=fill["z"][s], y=ys[s])
    torch.cuda.synchronize()
    o = oracle.get()
    st64 = np.ascontiguousarray(base["state"], dtype=np.float64)
    ey = oracle.ErrorSum()
    for s in range(steps):
        tk = {k: to_host(fill[k][s]) for k in ("x", "delta", "z", "Bt", "Ct")}
        ey.add(to_f64(ys[s]), o.step(tk, base["A"], base["Dskip"], st64, cfg.dtype))
    es = oracle.ErrorSum()
    es.add(to_f64(state), st64)
    assert ey.count == steps * cfg.batch * cfg.D
    check_sum(ey, cfg.dtype, "y, every channel of every step")
    check_sum(es, cfg.dtype, "final state, every value")


@pytest.mark.parametrize("N", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [1, 37, 64, 300])
def test_step_every_output(N, dtype, D):
    """Decode step on small shapes: every output and the whole state, 20 steps."""
    import torch
    import oracle
    import selective_state_space_16_amd as ssm
    cfg = W.StepConfig("step_small", 5, D, N, dtype, gate=(D != 64), dskip="uniform" if D != 37 else "none",
                       state_std=1.0, steps=20, seed=70 + N)
    say(f"case {cfg}")
    base = W.step_inputs(cfg)
    state = to_dev(base["state"])
    A = to_dev(base["A"])
    Dskip = to_dev(base["Dskip"])
    st64 = base["state"].astype(np.float64)
    o = oracle.get()
    for s in range(cfg.steps):
        tk = W.step_token_inputs(cfg, s)
        y = ssm.ssm_step(to_dev(tk["x"]), to_dev(tk["delta"]), A, to_dev(tk["Bt"]), to_dev(tk["Ct"]), state,
                         Dskip=Dskip, z=to_dev(tk["z"]))
        yr = o.step(tk, base["A"], base["Dskip"], st64, dtype)
        torch.cuda.synchronize()
        check(to_f64(y), yr, dtype, f"y step {s}")
    check(to_f64(state), st64, dtype, "state")


def test_step_more_row_groups_than_grid_rows():
    """Decode step with more batch-row groups than one launch row of blocks can
    hold (the kernel strides over them): batch 140001 (odd), D 3, N 2, fp32."""
    import torch
    import oracle
    import selective_state_space_16_amd as ssm
    cfg = W.StepConfig("step_tall", 140001, 3, 2, "f32", gate=True, dskip="uniform",
                       state_std=1.0, steps=2, seed=91)
    say(f"case {cfg}")
    base = W.step_inputs(cfg)
    state = to_dev(base["state"])
    A = to_dev(base["A"])
    Dskip = to_dev(base["Dskip"])
    st64 = base["state"].astype(np.float64)
    o = oracle.get()
    for s in range(cfg.steps):
        tk = W.step_token_inputs(cfg, s)
        y = ssm.ssm_step(to_dev(tk["x"]), to_dev(tk["delta"]), A, to_dev(tk["Bt"]), to_dev(tk["Ct"]), state,
                         Dskip=Dskip, z=to_dev(tk["z"]))
        yr = o.step(tk, base["A"], base["Dskip"], st64, "f32")
        torch.cuda.synchronize()
        check(to_f64(y), yr, "f32", f"y step {s}")
    check(to_f64(state), st64, "f32", "state")
