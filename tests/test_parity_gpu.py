"""GPU path against the fp64 oracle on the same seeded inputs (needs MI355X).

Small and medium cases compare every output; the full-size workloads compare
sampled channels (all tokens, all batch rows) in the launch configuration the
bench times, with the other channels filled by torch draws of the same
distributions."""
import numpy as np
import pytest

import workloads as W
from gpu_util import TOL, check, errors, gpu_scan, oracle_scan, say, to_dev, to_f64

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


def _run_sampled(cfg, sel):
    """Full-size launch; compare the `sel` channels of y and of the final state."""
    import torch
    say(f"case {cfg.name} full size, sampled channels {list(sel)}")
    part = W.scan_inputs(cfg, channels=sel)
    fill = W.fill_scan_device(cfg, "cuda")
    whole = W.scan_inputs(cfg, 0, 0)  # A, Dskip, state_in for every channel
    sel_t = torch.as_tensor(sel, device="cuda")
    for k in ("x", "delta", "z"):
        if fill[k] is not None:
            fill[k][:, :, sel_t] = to_dev(part[k])
    fill["Bt"], fill["Ct"] = to_dev(part["Bt"]), to_dev(part["Ct"])
    import selective_state_space_16_amd as ssm
    A, Dskip = to_dev(whole["A"]), to_dev(whole["Dskip"])
    st_in = to_dev(whole["state_in"])
    st_out = torch.empty((cfg.batch, cfg.D, cfg.N), dtype=torch.float32, device="cuda")
    y = ssm.ssm_scan_fwd(fill["x"], fill["delta"], A, fill["Bt"], fill["Ct"], Dskip=Dskip, z=fill["z"],
                         state_in=st_in, state_out=st_out)
    torch.cuda.synchronize()
    yg = to_f64(y[:, :, sel_t])
    sg = to_f64(st_out[:, sel_t])
    del fill, y
    yr, sr = oracle_scan(part, cfg.dtype)
    check(yg, yr, cfg.dtype, "y (sampled)")
    check(sg, sr, cfg.dtype, "state_out (sampled)")


def test_c2_full_size_sampled():
    cfg = W.SCAN_CONFIGS["c2"]
    _run_sampled(cfg, np.array([0, 1, 37, 63, 64 * 40 + 5, 64 * 40 + 60, cfg.D - 2, cfg.D - 1]))


def test_c3_full_size_sampled():
    cfg = W.SCAN_CONFIGS["c3"]
    _run_sampled(cfg, np.array([64 * 7 + 0, 64 * 7 + 9, 64 * 7 + 33, 64 * 7 + 63]))


def test_c4_decode_1000_steps_sampled():
    """The decode workload: (256, 5120, 16) float32 state updated in place for
    1000 steps; sampled channels checked against 1000 oracle steps (y of
    every step and the final state)."""
    import torch
    import oracle
    import selective_state_space_16_amd as ssm
    cfg = W.STEP_CONFIG
    steps = cfg.steps
    sel = np.array([0, 5, 64 * 33 + 2, 64 * 33 + 61, cfg.D - 1])
    say(f"case {cfg.name}: {steps} steps, sampled channels {list(sel)}")
    base = W.step_inputs(cfg)
    state = to_dev(base["state"])
    A, Dskip = to_dev(base["A"]), to_dev(base["Dskip"])
    fill = W.fill_step_device(cfg, steps, "cuda")
    sel_t = torch.as_tensor(sel, device="cuda")
    toks = []
    for s in range(steps):
        tk = W.step_token_inputs(cfg, s, channels=sel)
        toks.append(tk)
        for k in ("x", "delta", "z"):
            fill[k][s][:, sel_t] = to_dev(tk[k])
        fill["Bt"][s] = to_dev(tk["Bt"])
        fill["Ct"][s] = to_dev(tk["Ct"])
    ys = torch.empty((steps, cfg.batch, len(sel)), dtype=torch.float32, device="cuda")
    y = torch.empty((cfg.batch, cfg.D), dtype=fill["x"].dtype, device="cuda")
    for s in range(steps):
        ssm.ssm_step(fill["x"][s], fill["delta"][s], A, fill["Bt"][s], fill["Ct"][s], state,
                     Dskip=Dskip, z=fill["z"][s], y=y)
        ys[s] = y[:, sel_t].float()
    torch.cuda.synchronize()
    o = oracle.get()
    st64 = np.ascontiguousarray(base["state"][:, sel], dtype=np.float64)
    yref = np.empty((steps, cfg.batch, len(sel)))
    for s in range(steps):
        yref[s] = o.step(toks[s], base["A"][sel], base["Dskip"][sel], st64, cfg.dtype)
    check(to_f64(ys), yref, cfg.dtype, "y, all steps (sampled)")
    check(to_f64(state[:, sel_t]), st64, cfg.dtype, "final state (sampled)")


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
