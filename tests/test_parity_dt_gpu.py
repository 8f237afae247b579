"""The entry points that take the step size before its activation
(ssm_scan_fwd_dt, ssm_step_dt: delta = softplus(delta_raw + dt_bias[d]))
against the fp64 oracle's activation followed by its scan or step (needs
MI355X). Shapes cover the LDS-tiled scan (channel counts that are whole
16-byte pieces), the fallback scan, ragged lengths and channel counts, cut
columns, and the decode step."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import check, gpu_scan_dt, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _cfg(name, batch, L, D, N=16, dtype="f32", gate=True, dskip="uniform", state_in=None, seed=90):
    return W.ScanConfig(name, batch, L, D, N, dtype, gate=gate, dskip=dskip, state_in=state_in, seed=seed)


def _run(cfg, bias=True):
    say(f"case {cfg} dt_bias={'given' if bias else 'NULL'}")
    inp = W.scan_inputs(cfg, raw_delta=True)
    y, st = gpu_scan_dt(inp, dt_bias=bias)
    ref_inp = dict(inp) if bias else dict(inp, dt_bias=None)
    yr, sr = oracle.get().scan_dt(ref_inp, cfg.dtype)
    check(y, yr, cfg.dtype, "y")
    check(st, sr, cfg.dtype, "state_out")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [96, 200])
def test_scan_dt_tiled(dtype, D):
    _run(_cfg(f"dt_{D}", 2, 777, D, 16, dtype, state_in=0.3))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_dt_no_bias(dtype):
    _run(_cfg("dt_nobias", 2, 300, 64, 16, dtype, state_in=0.2), bias=False)


@pytest.mark.parametrize("D,dtype", [(63, "f32"), (100, "bf16"), (130, "bf16")])
def test_scan_dt_fallback_shapes(D, dtype):
    """Channel counts that are not whole 16-byte pieces take the fallback scan."""
    _run(_cfg(f"dt_fb{D}", 2, 500, D, 16, dtype, state_in=0.3))


@pytest.mark.parametrize("N", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_dt_state_sizes(N, dtype):
    _run(_cfg(f"dt_N{N}", 2, 333, 128, N, dtype, state_in=0.5))


@pytest.mark.parametrize("L", [1, 65, 4097])
def test_scan_dt_ragged_lengths_bf16(L):
    _run(_cfg(f"dt_L{L}", 1, L, 96, 16, "bf16", state_in=0.3))


def test_scan_dt_cut_columns_bf16():
    """Few channel columns and a long sequence: every column is cut into stripes."""
    _run(_cfg("dt_c3twin", 1, 131072, 128, 16, "bf16", state_in=0.1, seed=3))


def test_scan_dt_c1_layer_f32():
    _run(W.SCAN_CONFIGS["c1"])


@pytest.mark.parametrize("N", [1, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [37, 300])
def test_step_dt_every_output(N, dtype, D):
    """Decode steps with the raw step size: every output and the whole state, 10 steps."""
    import torch
    import selective_state_space_16_amd as ssm
    cfg = W.StepConfig("step_dt", 5, D, N, dtype, gate=True, dskip="uniform", state_std=1.0, steps=10, seed=95 + N)
    say(f"case {cfg}")
    base = W.step_inputs(cfg)
    state, A, Dskip, bias = to_dev(base["state"]), to_dev(base["A"]), to_dev(base["Dskip"]), to_dev(base["dt_bias"])
    st64 = base["state"].astype(np.float64)
    o = oracle.get()
    for s in range(cfg.steps):
        tk = W.step_token_inputs(cfg, s, raw_delta=True)
        y = ssm.ssm_step_dt(to_dev(tk["x"]), to_dev(tk["delta_raw"]), bias, A, to_dev(tk["Bt"]), to_dev(tk["Ct"]),
                            state, Dskip=Dskip, z=to_dev(tk["z"]))
        yr = o.step_dt(tk, base["A"], base["Dskip"], base["dt_bias"], st64, dtype)
        torch.cuda.synchronize()
        check(to_f64(y), yr, dtype, f"y step {s}")
    check(to_f64(state), st64, dtype, "state")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_dt_fold_equals_scan_dt(dtype):
    """L decode steps with the raw step size equal one scan with it."""
    import torch
    import selective_state_space_16_amd as ssm
    cfg = _cfg("fold_dt", 2, 150, 70, 16, dtype, state_in=0.4)
    say(f"case {cfg}")
    inp = W.scan_inputs(cfg, raw_delta=True)
    y, st = gpu_scan_dt(inp)
    dev = {k: to_dev(v) for k, v in inp.items()}
    state = dev["state_in"].clone()
    ys = []
    for t in range(cfg.L):
        yt = ssm.ssm_step_dt(dev["x"][:, t].contiguous(), dev["delta_raw"][:, t].contiguous(), dev["dt_bias"],
                             dev["A"], dev["Bt"][:, t].contiguous(), dev["Ct"][:, t].contiguous(), state,
                             Dskip=dev["Dskip"], z=dev["z"][:, t].contiguous())
        ys.append(to_f64(yt))
    torch.cuda.synchronize()
    check(np.stack(ys, 1), y, dtype, "fold of steps vs scan (y)")
    check(to_f64(state), st, dtype, "fold of steps vs scan (state)")


# -- the activation on its own ------------------------------------------------
# With a zero carried-in state, x = 1, Bt = 1, Ct = (1, 0, ..., 0), no skip
# term and no gate, the first state of a channel after a token is exactly its
# activated step size, and so is y; A = -2e38 (A log2(e) still finite) makes
# dA = 0 in the scan for every step size the sweep gives (the smallest,
# softplus(-80) ~ 1.8e-35, still sends delta A below -5000), so no earlier
# token leaks in (the step starts from a zero state anyway). This reads
# the kernels' softplus(delta_raw + dt_bias) value by value.

def _act_raw(shape, dtype, seed):
    """Raw step sizes whose activated argument u = raw + bias sweeps the range a
    projection can give, with fine sweeps where exp(-|u|) falls below the
    float32 rounding of 1 + e and around u = 0."""
    rng = np.random.default_rng(seed)
    D = shape[-1]
    bias = rng.uniform(-1.0, 1.0, D).astype(np.float32)
    n = int(np.prod(shape))
    parts = [np.linspace(-80.0, 40.0, n // 4), np.linspace(-19.0, -13.0, n // 4),
             np.linspace(-1.0, 1.0, n // 4)]
    parts.append(rng.normal(-4.0, 3.0, n - sum(len(p) for p in parts)))
    u = np.concatenate(parts)
    rng.shuffle(u)
    raw = W._store(u.reshape(shape) - bias.astype(np.float64), dtype)
    return raw, bias


def _act_check(got, raw, bias, dtype):
    """got: float64 copy of the kernel's activated step sizes."""
    raw64 = W.storage_to_f64(raw, dtype)
    ref = oracle.get().softplus_bias64(raw64, bias.astype(np.float64))
    u = raw64 + bias.astype(np.float64)
    # float32 evaluation: u = raw + bias rounds (relative error |u| 2^-24 in
    # exp(u)), exp and log cost a few ulps
    tol = (8.0 + 4.0 * np.abs(u)) * 2.0 ** -24 * np.abs(ref)
    # bfloat16: the value is then rounded to 8 significant bits, half an ulp
    half = 0.5 * 2.0 ** (np.floor(np.log2(np.abs(ref))) - 7) if dtype == "bf16" else 0.0 * ref
    excess = np.abs(got - ref) - half  # error beyond the storage rounding
    worst = int(np.argmax(excess / tol))
    say(f"  activation: max (err - storage rounding)/tol {excess.flat[worst] / tol.flat[worst]:.3f} at "
        f"u={u.flat[worst]:.6g} (got {got.flat[worst]:.9g}, ref {ref.flat[worst]:.9g}); "
        f"max rel err {np.max(np.abs(got - ref) / ref):.3e}")
    assert np.all(excess <= tol), "activated step sizes beyond the float32 error bound"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [96, 128])
def test_scan_dt_activation_values(dtype, D):
    import torch
    import selective_state_space_16_amd as ssm
    batch, L, N = 2, 700, 16
    say(f"case scan activation values batch={batch} L={L} D={D} N={N} {dtype}")
    raw, bias = _act_raw((batch, L, D), dtype, seed=D)
    one = W._store(np.ones((batch, L, D)), dtype)
    Bt = W._store(np.ones((batch, L, N)), dtype)
    Ct = W._store(np.eye(N)[0][None, None, :].repeat(L, 1).repeat(batch, 0), dtype)
    A = np.full((D, N), -2e38, np.float32)
    dev = [to_dev(v) for v in (one, raw, bias, A, Bt, Ct)]
    ws = ssm.new_workspace(ssm.ssm_scan_workspace_bytes(batch, L, D, N, 0 if dtype == "f32" else 1))
    y = ssm.ssm_scan_fwd_dt(*dev, workspace=ws)
    torch.cuda.synchronize()
    assert ssm.workspace_error(ws) == 0
    _act_check(to_f64(y), raw, bias, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_dt_activation_values(dtype):
    import torch
    import selective_state_space_16_amd as ssm
    batch, D, N = 64, 4096, 16
    say(f"case step activation values batch={batch} D={D} N={N} {dtype}")
    raw, bias = _act_raw((batch, D), dtype, seed=7)
    one = W._store(np.ones((batch, D)), dtype)
    Bt = W._store(np.ones((batch, N)), dtype)
    Ct = W._store(np.eye(N)[0][None, :].repeat(batch, 0), dtype)
    A = np.full((D, N), -1.0, np.float32)
    state = torch.zeros((batch, D, N), dtype=torch.float32, device="cuda")
    y = ssm.ssm_step_dt(to_dev(one), to_dev(raw), to_dev(bias), to_dev(A), to_dev(Bt), to_dev(Ct), state)
    torch.cuda.synchronize()
    _act_check(to_f64(y), raw, bias, dtype)
    _act_check(to_f64(state[:, :, 0]), raw, bias, dtype)
