"""ssm_scan_fwd_conv (the scan behind the Mamba block's x branch: SiLU of a
causal width-4 convolution of x_raw per channel, with the step size given
before its activation) against the fp64 oracle's convolution, activation and
scan (needs MI355X). Shapes cover the LDS-tiled scan (the convolution runs on
each landed tile, with the previous tile's raw rows as its halo), the fallback
scan (a per-lane window), ragged lengths and channel counts, cut columns
(stripes whose halo comes from the tokens before them), resumption from the
raw x of an earlier piece, and the optional parts."""
import os

import numpy as np
import pytest

import oracle
import selective_state_space_16_amd as ssm
import workloads as W
from gpu_util import check, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _cfg(name, batch, L, D, N=16, dtype="f32", gate=True, dskip="uniform", state_in=None, seed=91):
    return W.ScanConfig(name, batch, L, D, N, dtype, gate=gate, dskip=dskip, state_in=state_in, seed=seed)


def gpu_scan_conv(inp, state_out=True):
    """ssm_scan_fwd_conv on stored inputs; returns (y64, state64 or None)."""
    import torch
    dev = {k: to_dev(v) for k, v in inp.items()}
    batch, L, D = dev["x_raw"].shape
    N = dev["A"].shape[1]
    st = torch.empty((batch, D, N), dtype=torch.float32, device="cuda") if state_out else None
    ws = ssm.new_workspace(ssm.ssm_scan_workspace_bytes(batch, L, D, N,
                                                        0 if dev["x_raw"].dtype == torch.float32 else 1))
    y = ssm.ssm_scan_fwd_conv(dev["x_raw"], dev["conv_w"], dev["delta_raw"], dev.get("dt_bias"), dev["A"], dev["Bt"],
                              dev["Ct"], conv_b=dev.get("conv_b"), conv_state=dev.get("conv_state"),
                              Dskip=dev.get("Dskip"), z=dev.get("z"), state_in=dev.get("state_in"), state_out=st,
                              workspace=ws)
    torch.cuda.synchronize()
    assert ssm.workspace_error(ws) == 0, "a look-back wait gave up"
    return to_f64(y), None if st is None else to_f64(st)


def _inputs(cfg, t0=0, t1=None, conv_state=True, conv_b=True):
    inp = W.scan_inputs(cfg, t0, t1, raw_delta=True, conv=True)
    if not conv_state:
        inp["conv_state"] = None
    if not conv_b:
        inp["conv_b"] = None
    return inp


def _run(cfg, **kw):
    say(f"case {cfg} {kw}")
    inp = _inputs(cfg, **kw)
    y, st = gpu_scan_conv(inp)
    yr, sr = oracle.get().scan_conv(inp, cfg.dtype)
    check(y, yr, cfg.dtype, "y")
    check(st, sr, cfg.dtype, "state_out")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [96, 200])
def test_scan_conv_tiled(dtype, D):
    _run(_cfg(f"conv_{D}", 2, 777, D, 16, dtype, state_in=0.3))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_conv_no_state_no_bias(dtype):
    """conv_state NULL (zeros before token 0) and conv_b NULL (zero bias)."""
    _run(_cfg("conv_bare", 2, 300, 64, 16, dtype, state_in=0.2), conv_state=False, conv_b=False)


@pytest.mark.parametrize("D,dtype", [(63, "f32"), (100, "bf16"), (130, "bf16")])
def test_scan_conv_fallback_shapes(D, dtype):
    """Channel counts that are not whole 16-byte pieces take the fallback scan."""
    _run(_cfg(f"conv_fb{D}", 2, 500, D, 16, dtype, state_in=0.3))


@pytest.mark.parametrize("N", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_conv_state_sizes(N, dtype):
    _run(_cfg(f"conv_N{N}", 2, 333, 128, N, dtype, state_in=0.5))


@pytest.mark.parametrize("L", [1, 2, 3, 4, 65, 4097])
def test_scan_conv_ragged_lengths_bf16(L):
    """Lengths shorter than the window, one past a tile, and a ragged tail."""
    _run(_cfg(f"conv_L{L}", 1, L, 96, 16, "bf16", state_in=0.3))


@pytest.mark.parametrize("gate,dskip", [(False, "uniform"), (True, "none"), (False, "none")])
def test_scan_conv_optional_parts(gate, dskip):
    _run(_cfg("conv_opt", 2, 400, 128, 16, "bf16", gate=gate, dskip=dskip, state_in=0.2))


def test_scan_conv_cut_columns_bf16():
    """Few channel columns and a long sequence: every column is cut into
    stripes, and each stripe's first tile takes its halo from the three tokens
    before the stripe, in both passes."""
    _run(_cfg("conv_c3twin", 1, 131072, 128, 16, "bf16", state_in=0.1, seed=3))


def test_scan_conv_c1_layer_f32():
    _run(W.SCAN_CONFIGS["c1"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_conv_fallback_chunks(dtype, monkeypatch):
    """The fallback scan cut into chunks: each chunk starts its window from the
    three tokens before it."""
    monkeypatch.setenv("SSM_SCAN_IMPL", "twopass")
    _run(_cfg("conv_twopass", 2, 3000, 128, 16, dtype, state_in=0.3))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_conv_resume(dtype):
    """Two calls, the second given the first's final state and its last three
    raw tokens as conv_state, match the oracle over the whole sequence."""
    cfg = _cfg("conv_resume", 2, 1500, 128, 16, dtype, state_in=0.3)
    say(f"case {cfg} resume at 700")
    whole = _inputs(cfg)
    first = _inputs(cfg, 0, 700)
    y1, s1 = gpu_scan_conv(first)
    second = _inputs(cfg, 700, 1500)
    assert np.array_equal(second["conv_state"], np.ascontiguousarray(first["x_raw"][:, -3:].transpose(0, 2, 1)))
    second["state_in"] = s1.astype(np.float32)
    y2, s2 = gpu_scan_conv(second)
    yr, sr = oracle.get().scan_conv(whole, dtype)
    check(np.concatenate([y1, y2], axis=1), yr, dtype, "y")
    check(s2, sr, dtype, "state_out")


def test_scan_conv_deterministic():
    """Two calls on the same inputs give the same bits."""
    cfg = _cfg("conv_det", 1, 20000, 128, 16, "bf16", state_in=0.1)
    inp = _inputs(cfg)
    ya, sa = gpu_scan_conv(inp)
    yb, sb = gpu_scan_conv(inp)
    assert np.array_equal(ya, yb) and np.array_equal(sa, sb)


def test_scan_conv_stripe_and_fallback_agree():
    """The tiled scan and the fallback round the convolved x the same way: on
    float32 inputs they agree to float32 rounding of the recurrence."""
    cfg = _cfg("conv_paths", 1, 600, 128, 16, "f32", state_in=0.3)
    inp = _inputs(cfg)
    y1, s1 = gpu_scan_conv(inp)
    os.environ["SSM_SCAN_IMPL"] = "twopass"
    try:
        y2, s2 = gpu_scan_conv(inp)
    finally:
        del os.environ["SSM_SCAN_IMPL"]
    assert np.allclose(y1, y2, rtol=1e-5, atol=1e-5) and np.allclose(s1, s2, rtol=1e-5, atol=1e-5)


# -- the decode step ----------------------------------------------------------

@pytest.mark.parametrize("N", [1, 16])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [37, 300])
def test_step_conv_every_output(N, dtype, D):
    """One step of five sequences against the oracle's scan over that one
    token (y and state), and the window it leaves: the last two earlier raw
    tokens and this token's raw x, bit for bit."""
    import torch
    cfg = _cfg(f"step_conv_{N}_{D}", 5, 1, D, N, dtype, state_in=1.0)
    say(f"case {cfg}")
    inp = _inputs(cfg)
    yr, sr = oracle.get().scan_conv(inp, dtype)
    dev = {k: to_dev(v) for k, v in inp.items()}
    state = dev["state_in"].clone()
    window = dev["conv_state"].clone()
    y = ssm.ssm_step_conv(dev["x_raw"][:, 0].contiguous(), dev["conv_w"], window, dev["delta_raw"][:, 0].contiguous(),
                          dev["dt_bias"], dev["A"], dev["Bt"][:, 0].contiguous(), dev["Ct"][:, 0].contiguous(), state,
                          conv_b=dev["conv_b"], Dskip=dev["Dskip"], z=dev["z"][:, 0].contiguous())
    torch.cuda.synchronize()
    check(to_f64(y)[:, None, :], yr, dtype, "y")
    check(to_f64(state), sr, dtype, "state")
    want = np.concatenate([inp["conv_state"][:, :, 1:], inp["x_raw"][:, 0][:, :, None]], axis=2)
    got = window.cpu()
    got = got.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else got.numpy()
    assert np.array_equal(got, want), "conv_state after the step"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_conv_fold_equals_scan_conv(dtype):
    """T decode steps from the scan's conv_state and state_in give the scan's
    y and final state, and leave the last three raw tokens as the window."""
    import torch
    cfg = _cfg("fold_conv", 2, 150, 70, 16, dtype, state_in=0.4)
    say(f"case {cfg}")
    inp = _inputs(cfg)
    y, st = gpu_scan_conv(inp)
    dev = {k: to_dev(v) for k, v in inp.items()}
    state = dev["state_in"].clone()
    window = dev["conv_state"].clone()
    ys = []
    for t in range(cfg.L):
        yt = ssm.ssm_step_conv(dev["x_raw"][:, t].contiguous(), dev["conv_w"], window,
                               dev["delta_raw"][:, t].contiguous(), dev["dt_bias"], dev["A"],
                               dev["Bt"][:, t].contiguous(), dev["Ct"][:, t].contiguous(), state, conv_b=dev["conv_b"],
                               Dskip=dev["Dskip"], z=dev["z"][:, t].contiguous())
        ys.append(to_f64(yt))
    torch.cuda.synchronize()
    check(np.stack(ys, 1), y, dtype, "fold of steps vs scan (y)")
    check(to_f64(state), st, dtype, "fold of steps vs scan (state)")
    assert torch.equal(window, dev["x_raw"][:, -3:].transpose(1, 2).contiguous()), "window after the steps"


# -- capture into a HIP graph -------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_conv_graph_replay(dtype):
    """ssm_scan_fwd_conv with a workspace, captured into a graph on a shape
    whose columns are cut into stripes: four replays, each followed by eager
    calls of another size on the same workspace, equal the eager call bit for
    bit (y and final state)."""
    import torch
    cfg = _cfg("conv_graph", 2, 2048, 1536, 16, dtype, state_in=0.3, seed=94)
    say(f"case {cfg} graph replay")
    d = {k: to_dev(v) for k, v in _inputs(cfg).items()}
    other = _cfg("conv_graph_other", 2, 700, 96, 16, dtype, state_in=0.3, seed=95)
    o = {k: to_dev(v) for k, v in _inputs(other).items()}
    code = 0 if dtype == "f32" else 1
    ws = ssm.new_workspace(max(ssm.ssm_scan_workspace_bytes(2, 2048, 1536, 16, code),
                               ssm.ssm_scan_workspace_bytes(2, 700, 96, 16, code)))

    def run(inp, y=None, st=None, stream=None):
        if y is None:
            y = torch.empty_like(inp["x_raw"])
        if st is None:
            st = torch.empty_like(inp["state_in"])
        ssm.ssm_scan_fwd_conv(inp["x_raw"], inp["conv_w"], inp["delta_raw"], inp["dt_bias"], inp["A"], inp["Bt"],
                              inp["Ct"], conv_b=inp["conv_b"], conv_state=inp["conv_state"], Dskip=inp["Dskip"],
                              z=inp["z"], state_in=inp["state_in"], state_out=st, y=y, workspace=ws, stream=stream)
        return y, st

    y_ref, st_ref = run(d)
    torch.cuda.synchronize()
    assert ssm.workspace_error(ws) == 0
    y_g, st_g = torch.empty_like(y_ref), torch.empty_like(st_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(d, y_g, st_g, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(4):
        y_g.fill_(float("nan"))
        st_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert ssm.workspace_error(ws) == 0
        assert torch.equal(y_g, y_ref), f"y differs on replay {rep}"
        assert torch.equal(st_g, st_ref), f"state differs on replay {rep}"
        run(o)  # eager work of another size on the same workspace
        run(d)
        torch.cuda.synchronize()
        assert ssm.workspace_error(ws) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_conv_graph_replay(dtype):
    """Decode steps with the x branch captured into a graph: every replay (with
    eager scans between replays) equals the same steps launched eagerly, bit
    for bit, in y, the state and the window of raw tokens."""
    import torch
    cfg = _cfg("step_conv_graph", 3, 6, 200, 16, dtype, state_in=0.5, seed=96)
    say(f"case {cfg} graph replay")
    dev = {k: to_dev(v) for k, v in _inputs(cfg).items()}
    toks = [{k: dev[k][:, t].contiguous() for k in ("x_raw", "delta_raw", "Bt", "Ct", "z")} for t in range(cfg.L)]
    st_g, st_e = dev["state_in"].clone(), dev["state_in"].clone()
    win_g, win_e = dev["conv_state"].clone(), dev["conv_state"].clone()
    y_g, y_e = torch.empty_like(toks[0]["x_raw"]), torch.empty_like(toks[0]["x_raw"])

    def steps(state, window, y):
        for tk in toks:
            ssm.ssm_step_conv(tk["x_raw"], dev["conv_w"], window, tk["delta_raw"], dev["dt_bias"], dev["A"], tk["Bt"],
                              tk["Ct"], state, conv_b=dev["conv_b"], Dskip=dev["Dskip"], z=tk["z"], y=y,
                              stream=torch.cuda.current_stream())

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps(st_g, win_g, y_g)
    torch.cuda.synchronize()
    st_g.copy_(dev["state_in"])
    win_g.copy_(dev["conv_state"])
    for rep in range(4):
        graph.replay()
        steps(st_e, win_e, y_e)
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"y differs on replay {rep}"
        assert torch.equal(st_g, st_e), f"state differs on replay {rep}"
        assert torch.equal(win_g, win_e), f"window differs on replay {rep}"
        gpu_scan_conv(_inputs(_cfg("conv_between", 1, 50, 40, 16, dtype, seed=97 + rep)))
        torch.cuda.synchronize()
