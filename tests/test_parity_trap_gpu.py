"""The exponential-trapezoidal rule (ssm_scan_fwd_trap, ssm_step_trap; "Notas
sobre Mamba", section "Recorrência trapezoidal") against the fp64 oracle's
trapezoidal scan and step (needs MI355X). Shapes cover the LDS-tiled scan,
stripes cut from long columns (the look-back composes the kernel's shifted
state), the fallback scan, ragged lengths, every state size, resumption with
the previous token, lam = 1 against the plain scan, and the decode step."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import check, gpu_scan, gpu_scan_trap, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _cfg(name, batch, L, D, N=16, dtype="f32", gate=True, dskip="uniform", state_in=None, seed=70):
    return W.ScanConfig(name, batch, L, D, N, dtype, gate=gate, dskip=dskip, state_in=state_in, seed=seed)


def _run(cfg, prev=True):
    say(f"case {cfg} x_prev/B_prev={'given' if prev else 'NULL'}")
    inp = W.scan_inputs(cfg, trap=True)
    y, st = gpu_scan_trap(inp, prev=prev)
    ref = dict(inp) if prev else dict(inp, x_prev=None, B_prev=None)
    yr, sr = oracle.get().scan_trap(ref, cfg.dtype)
    check(y, yr, cfg.dtype, "y")
    check(st, sr, cfg.dtype, "state_out")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [96, 200])
def test_trap_tiled(dtype, D):
    _run(_cfg(f"trap_{D}", 2, 777, D, 16, dtype, state_in=0.3))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_trap_no_earlier_token(dtype):
    _run(_cfg("trap_noprev", 2, 300, 64, 16, dtype, state_in=0.2), prev=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_trap_no_options(dtype):
    _run(_cfg("trap_plain", 1, 500, 128, 16, dtype, gate=False, dskip="none"), prev=False)


@pytest.mark.parametrize("D,dtype", [(63, "f32"), (100, "bf16"), (130, "bf16")])
def test_trap_fallback_shapes(D, dtype):
    """Channel counts that are not whole 16-byte pieces take the chunked scan."""
    _run(_cfg(f"trap_fb{D}", 2, 500, D, 16, dtype, state_in=0.3))


@pytest.mark.parametrize("N", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_trap_state_sizes(N, dtype):
    _run(_cfg(f"trap_N{N}", 2, 333, 128, N, dtype, state_in=0.5))


@pytest.mark.parametrize("L", [1, 2, 63, 64, 65, 4097])
def test_trap_ragged_lengths_bf16(L):
    _run(_cfg(f"trap_L{L}", 1, L, 96, 16, "bf16", state_in=0.3))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_trap_cut_columns(dtype):
    """Few channel columns and a long sequence: every column is cut into stripes,
    whose summaries the look-back composes."""
    _run(_cfg("trap_cut", 1, 131072 if dtype == "bf16" else 40000, 128, 16, dtype, state_in=0.1, seed=3))


def test_trap_c1_layer_f32():
    c = W.SCAN_CONFIGS["c1"]
    _run(_cfg("trap_c1", c.batch, c.L, c.D, c.N, c.dtype, gate=c.gate, dskip=c.dskip, state_in=c.state_in,
              seed=c.seed))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [128, 100])
def test_trap_lambda_one_equals_scan(dtype, D):
    """lam = 1 turns the rule into the exponential-Euler scan: the kernels then
    compute exactly what ssm_scan_fwd computes, bit for bit."""
    cfg = _cfg("trap_lam1", 2, 1000, D, 16, dtype, state_in=0.3)
    say(f"case {cfg}")
    inp = W.scan_inputs(cfg, trap=True)
    inp["lam"] = W._store(np.ones(inp["x"].shape), dtype)
    y1, s1 = gpu_scan_trap(inp)
    y2, s2 = gpu_scan(inp)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_trap_resume(dtype):
    """A sequence scanned in two calls, the second given the first's state and
    its last token, equals one call (to the tolerance: the cut moves stripes)."""
    cfg = _cfg("trap_resume", 2, 3000, 128, 16, dtype, state_in=0.2)
    say(f"case {cfg}")
    full = W.scan_inputs(cfg, trap=True)
    y, st = gpu_scan_trap(full)
    m = 1234
    p1 = W.scan_inputs(cfg, 0, m, trap=True)
    y1, s1 = gpu_scan_trap(p1)
    p2 = W.scan_inputs(cfg, m, cfg.L, trap=True)
    p2["state_in"] = s1.astype(np.float32)
    y2, s2 = gpu_scan_trap(p2)
    check(np.concatenate([y1, y2], 1), y, dtype, "two calls vs one (y)")
    check(s2, st, dtype, "two calls vs one (state)")


@pytest.mark.parametrize("N", [1, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [37, 300])
def test_step_trap_every_output(N, dtype, D):
    """Decode steps with the trapezoidal rule, each given the previous token:
    every output and the whole state over 10 steps (the first with no earlier
    token)."""
    import torch
    import selective_state_space_16_amd as ssm
    cfg = W.StepConfig("step_trap", 5, D, N, dtype, gate=True, dskip="uniform", state_std=1.0, steps=10, seed=75 + N)
    say(f"case {cfg}")
    base = W.step_inputs(cfg)
    state, A, Dskip = to_dev(base["state"]), to_dev(base["A"]), to_dev(base["Dskip"])
    st64 = base["state"].astype(np.float64)
    o = oracle.get()
    prev = None
    for s in range(cfg.steps):
        tk = W.step_token_inputs(cfg, s, trap=True)
        xp, bp = (None, None) if prev is None else (prev["x"], prev["Bt"])
        y = ssm.ssm_step_trap(to_dev(tk["x"]), to_dev(tk["delta"]), to_dev(tk["lam"]), A, to_dev(tk["Bt"]),
                              to_dev(tk["Ct"]), state, Dskip=Dskip, z=to_dev(tk["z"]), x_prev=to_dev(xp),
                              B_prev=to_dev(bp))
        yr = o.step_trap(dict(tk, x_prev=xp, B_prev=bp), base["A"], base["Dskip"], st64, dtype)
        torch.cuda.synchronize()
        check(to_f64(y), yr, dtype, f"y step {s}")
        prev = tk
    check(to_f64(state), st64, dtype, "state")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_trap_fold_equals_scan(dtype):
    """L trapezoidal decode steps, each given the previous token, equal one scan."""
    import torch
    import selective_state_space_16_amd as ssm
    cfg = _cfg("fold_trap", 2, 150, 70, 16, dtype, state_in=0.4)
    say(f"case {cfg}")
    inp = W.scan_inputs(cfg, trap=True)
    y, st = gpu_scan_trap(inp)
    dev = {k: to_dev(v) for k, v in inp.items()}
    state = dev["state_in"].clone()
    xp, bp = dev["x_prev"], dev["B_prev"]
    ys = []
    for t in range(cfg.L):
        xt, bt = dev["x"][:, t].contiguous(), dev["Bt"][:, t].contiguous()
        yt = ssm.ssm_step_trap(xt, dev["delta"][:, t].contiguous(), dev["lam"][:, t].contiguous(), dev["A"], bt,
                               dev["Ct"][:, t].contiguous(), state, Dskip=dev["Dskip"],
                               z=dev["z"][:, t].contiguous(), x_prev=xp, B_prev=bp)
        ys.append(to_f64(yt))
        xp, bp = xt, bt
    torch.cuda.synchronize()
    check(np.stack(ys, 1), y, dtype, "fold of steps vs scan (y)")
    check(to_f64(state), st, dtype, "fold of steps vs scan (state)")
