"""Early mode of the tiled scan on cut columns (needs MI355X). Long stripes (or
any, with SSM_STRIPE_EARLY=1) run the scan from a zero start first, writing y;
after the look-back a second walk from the carried-in state rewrites y only
until that state's decayed contribution is below the output's rounding.
Against the fp64 oracle: stops that come after a tile or two (fast decays),
never (slow decays), each form of the step size and the x branch, the
trapezoidal rule, and inputs where the stop must not be taken (a positive A, a
negative delta). The million-token workload itself takes early mode by default
and is compared at full size in test_parity_gpu.py."""
import numpy as np
import pytest

import oracle
import selective_state_space_16_amd as ssm
import workloads as W
from gpu_util import TOL, check, errors, gpu_scan, gpu_scan_dt, gpu_scan_trap, oracle_scan, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture
def early(monkeypatch):
    monkeypatch.setenv("SSM_STRIPE_EARLY", "1")


def _cfg(name, L=32768, D=128, dtype="bf16", state_in=0.5, seed=71, batch=1):
    # two tile columns: each is cut into 64 stripes of a few hundred tokens
    return W.ScanConfig(name, batch, L, D, 16, dtype, gate=True, dskip="uniform", state_in=state_in, seed=seed)


def _both_orders(run, inp, ref, dtype, monkeypatch):
    """Early mode and the two-pass order on the same inputs, each against the
    oracle: early mode within the relative tolerance, and its largest error at
    most twice the two-pass order's (or the absolute tolerance). Inputs with
    scaled step sizes have larger outputs than the recipe's, so the two-pass
    order's own error is the bar for the largest one."""
    monkeypatch.setenv("SSM_STRIPE_EARLY", "0")
    two = run(inp)
    monkeypatch.setenv("SSM_STRIPE_EARLY", "1")
    got = run(inp)
    tol = TOL[dtype]
    for what, g, t, r in (("y", got[0], two[0], ref[0]), ("state_out", got[1], two[1], ref[1])):
        rel, mx = errors(g, r)
        rel_t, mx_t = errors(t, r)
        say(f"  {what}: early relL2={rel:.3e} maxabs={mx:.3e} | two-pass relL2={rel_t:.3e} maxabs={mx_t:.3e}")
        assert np.all(np.isfinite(g)), what + ": non-finite output"
        assert rel <= tol["rel"], f"{what}: relL2 {rel:.3e} > {tol['rel']}"
        bound = max(tol["maxabs"] if tol["maxabs"] is not None else 0.0, 2.0 * mx_t)
        if tol["maxabs"] is not None or mx_t > 0:
            assert mx <= bound, f"{what}: maxabs {mx:.3e} > {bound:.3e}"


def _scale_delta(inp, dtype, k):
    """delta times k, stored again in the activation dtype (faster decays)."""
    d = W.storage_to_f64(inp["delta"], dtype) * k
    inp["delta"] = d.astype(np.float32) if dtype == "f32" else W.bf16_bits_from_f64(d)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_early_fast_decay_stops_early(dtype, monkeypatch):
    """delta 100 times the recipe's: the carried-in state has decayed below
    rounding after a few tiles of each stripe."""
    cfg = _cfg(f"early_fast_{dtype}", dtype=dtype)
    say(f"case {cfg} delta x100")
    inp = W.scan_inputs(cfg)
    _scale_delta(inp, dtype, 100.0)
    _both_orders(gpu_scan, inp, oracle_scan(inp, dtype), dtype, monkeypatch)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_early_slow_decay_walks_whole_stripes(dtype, early):
    """The recipe's delta on stripes of a few hundred tokens: the slowest
    channels keep the carried-in state above rounding to each stripe's end."""
    cfg = _cfg(f"early_slow_{dtype}", L=20000, dtype=dtype, seed=72)
    say(f"case {cfg}")
    inp = W.scan_inputs(cfg)
    y, st = gpu_scan(inp)
    yr, sr = oracle_scan(inp, dtype)
    check(y, yr, dtype, "y")
    check(st, sr, dtype, "state_out")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_early_softplus_delta(dtype, monkeypatch):
    """The step size given before its activation, its bias raised so that the
    stops come early."""
    cfg = _cfg(f"early_dt_{dtype}", dtype=dtype, seed=73)
    say(f"case {cfg} dt_bias + 4")
    inp = W.scan_inputs(cfg, raw_delta=True)
    inp["dt_bias"] = (inp["dt_bias"] + 4.0).astype(np.float32)
    _both_orders(gpu_scan_dt, inp, oracle.get().scan_dt(inp, dtype), dtype, monkeypatch)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_early_x_branch(dtype, monkeypatch):
    """The x branch ahead of the scan: pass 2 re-runs each stripe's halo and
    convolution from the raw x of the tokens before it."""
    import torch
    cfg = _cfg(f"early_conv_{dtype}", dtype=dtype, seed=74)
    say(f"case {cfg} conv, dt_bias + 4")
    inp = W.scan_inputs(cfg, raw_delta=True, conv=True)
    inp["dt_bias"] = (inp["dt_bias"] + 4.0).astype(np.float32)

    def run(inp):
        dev = {k: to_dev(v) for k, v in inp.items()}
        st = torch.empty((cfg.batch, cfg.D, cfg.N), dtype=torch.float32, device="cuda")
        y = ssm.ssm_scan_fwd_conv(dev["x_raw"], dev["conv_w"], dev["delta_raw"], dev["dt_bias"], dev["A"],
                                  dev["Bt"], dev["Ct"], conv_b=dev["conv_b"], conv_state=dev["conv_state"],
                                  Dskip=dev["Dskip"], z=dev["z"], state_in=dev["state_in"], state_out=st)
        torch.cuda.synchronize()
        return to_f64(y), to_f64(st)

    _both_orders(run, inp, oracle.get().scan_conv(inp, dtype), dtype, monkeypatch)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_early_trapezoidal(dtype, monkeypatch):
    cfg = _cfg(f"early_trap_{dtype}", dtype=dtype, seed=75)
    say(f"case {cfg} trapezoidal, delta x100")
    inp = W.scan_inputs(cfg, trap=True)
    _scale_delta(inp, dtype, 100.0)
    _both_orders(gpu_scan_trap, inp, oracle.get().scan_trap(inp, dtype), dtype, monkeypatch)


def test_early_positive_A_never_stops(monkeypatch):
    """One state per channel with A > 0: its lanes never vote to stop."""
    cfg = _cfg("early_posA", L=8192, dtype="f32", seed=76)
    say(f"case {cfg} A[:, 0] = +0.001, delta x20")
    inp = W.scan_inputs(cfg)
    _scale_delta(inp, "f32", 20.0)
    inp["A"] = inp["A"].copy()
    inp["A"][:, 0] = 0.001  # grows by about e^3 over the sequence
    _both_orders(gpu_scan, inp, oracle_scan(inp, "f32"), "f32", monkeypatch)


def test_early_negative_delta_never_stops(monkeypatch):
    """A negative delta late in each stripe would bring the carried-in state
    back: lanes that see one in the first walk never vote to stop."""
    cfg = _cfg("early_negdelta", L=8192, dtype="f32", seed=77)
    say(f"case {cfg} delta x50, a negative delta every 96 tokens")
    inp = W.scan_inputs(cfg)
    _scale_delta(inp, "f32", 50.0)
    inp["delta"][:, 95::96, :] = -0.3
    _both_orders(gpu_scan, inp, oracle_scan(inp, "f32"), "f32", monkeypatch)


def test_early_agrees_with_two_pass_mode(monkeypatch):
    """The million-token recipe at reduced width, both orders: each matches the
    oracle, and the two agree to the output's rounding."""
    cfg = W.ScanConfig("early_twin", 1, 262144, 128, 16, "bf16", gate=True, dskip="uniform", state_in=0.1, seed=3)
    say(f"case {cfg} early and two-pass")
    inp = W.scan_inputs(cfg)
    monkeypatch.setenv("SSM_STRIPE_EARLY", "1")
    ye, se = gpu_scan(inp)
    monkeypatch.setenv("SSM_STRIPE_EARLY", "0")
    yt, stt = gpu_scan(inp)
    yr, sr = oracle_scan(inp, "bf16")
    check(ye, yr, "bf16", "y (early)")
    check(se, sr, "bf16", "state_out (early)")
    check(yt, yr, "bf16", "y (two-pass)")
    check(ye, yt, "bf16", "y (early vs two-pass)")


def test_early_deterministic(early):
    cfg = _cfg("early_det", seed=78)
    inp = W.scan_inputs(cfg)
    _scale_delta(inp, "bf16", 10.0)
    ya, sa = gpu_scan(inp)
    yb, sb = gpu_scan(inp)
    assert np.array_equal(ya, yb) and np.array_equal(sa, sb)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_early_ragged_shapes(dtype, monkeypatch):
    """Two batch rows, a channel count that leaves the last tile column part
    empty (its lanes past D vote on clamped data), and a length that leaves a
    ragged last tile in the last stripe."""
    cfg = _cfg(f"early_ragged_{dtype}", L=24000 - 37, D=200, dtype=dtype, seed=79, batch=2)
    say(f"case {cfg} delta x30")
    inp = W.scan_inputs(cfg)
    _scale_delta(inp, dtype, 30.0)
    _both_orders(gpu_scan, inp, oracle_scan(inp, dtype), dtype, monkeypatch)


def test_early_graph_replay(early):
    """Early mode captured into a graph: replays, with eager calls of another
    size between them, equal the eager call bit for bit."""
    import torch
    cfg = _cfg("early_graph", seed=80)
    say(f"case {cfg} graph replay, delta x30")
    inp = W.scan_inputs(cfg)
    _scale_delta(inp, "bf16", 30.0)
    d = {k: to_dev(v) for k, v in inp.items()}
    other = {k: to_dev(v) for k, v in W.scan_inputs(_cfg("early_graph_other", L=5000, D=64, seed=81)).items()}
    ws = ssm.new_workspace(max(ssm.ssm_scan_workspace_bytes(1, cfg.L, cfg.D, 16, 1),
                               ssm.ssm_scan_workspace_bytes(1, 5000, 64, 16, 1)))

    def run(v, y=None, st=None, stream=None):
        y = torch.empty_like(v["x"]) if y is None else y
        st = torch.empty_like(v["state_in"]) if st is None else st
        ssm.ssm_scan_fwd(v["x"], v["delta"], v["A"], v["Bt"], v["Ct"], Dskip=v["Dskip"], z=v["z"],
                         state_in=v["state_in"], state_out=st, y=y, workspace=ws, stream=stream)
        return y, st

    y_ref, st_ref = run(d)
    torch.cuda.synchronize()
    assert ssm.workspace_error(ws) == 0
    y_g, st_g = torch.empty_like(y_ref), torch.empty_like(st_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(d, y_g, st_g, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        y_g.fill_(float("nan"))
        st_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert ssm.workspace_error(ws) == 0
        assert torch.equal(y_g, y_ref), f"y differs on replay {rep}"
        assert torch.equal(st_g, st_ref), f"state differs on replay {rep}"
        run(other)
        torch.cuda.synchronize()


def test_early_two_stripes(monkeypatch):
    """The fewest stripes a cut column has: 256 tile columns (32 per list) are
    cut into two, so the last stripe's look-back reads stripe 0's end state
    directly, with no pairs in between."""
    cfg = _cfg("early_two_stripes", L=1024, D=16384, dtype="bf16", seed=82)
    say(f"case {cfg} delta x30")
    inp = W.scan_inputs(cfg)
    _scale_delta(inp, "bf16", 30.0)
    _both_orders(gpu_scan, inp, oracle_scan(inp, "bf16"), "bf16", monkeypatch)


def test_early_state_in_place(early):
    """state_out given as state_in's own memory: the last stripe writes the
    final state (before its second walk) only after its look-back, which
    follows stripe 0's read of state_in through the records."""
    cfg = _cfg("early_inplace", seed=83)
    say(f"case {cfg} state_out = state_in, delta x30")
    inp = W.scan_inputs(cfg)
    _scale_delta(inp, "bf16", 30.0)
    y, st = gpu_scan(inp, state_alias=True)
    yr, sr = oracle_scan(inp, "bf16")
    check(y, yr, "bf16", "y")
    check(st, sr, "bf16", "state_out (in place)")
