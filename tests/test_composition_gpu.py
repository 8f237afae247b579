"""Invariants of the GPU path itself (needs MI355X): split-and-resume equals one
call, a fold of decode steps equals the scan, repeated runs are bit-identical,
delta = 0 keeps the state, in-place state, and the empty cases."""
import numpy as np
import pytest

import selective_state_space_16_amd as ssm
import workloads as W
from gpu_util import check, gpu_scan, oracle_scan, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _inp(L=900, D=96, dtype="f32", state=0.4, seed=80, batch=2):
    return W.scan_inputs(W.ScanConfig("comp", batch, L, D, 16, dtype, gate=True, dskip="uniform",
                                      state_in=state, seed=seed))


def _slice(inp, t0, t1):
    return {k: (v[:, t0:t1] if k in ("x", "delta", "z", "Bt", "Ct") and v is not None else v)
            for k, v in inp.items()}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L1", [1, 64, 333, 899])
def test_split_and_resume(dtype, L1):
    """scan(L) == scan(L1) then scan(L - L1) from the first call's state."""
    say(f"case split dtype={dtype} L1={L1}")
    inp = _inp(dtype=dtype)
    y, st = gpu_scan(inp)
    a = _slice(inp, 0, L1)
    y1, s1 = gpu_scan(a)
    b = _slice(inp, L1, inp["x"].shape[1])
    b["state_in"] = s1.astype(np.float32)
    y2, s2 = gpu_scan(b)
    check(np.concatenate([y1, y2], 1), y, dtype, "y split vs whole")
    check(s2, st, dtype, "state split vs whole")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_fold_equals_scan(dtype):
    import torch
    say(f"case fold dtype={dtype}")
    inp = _inp(L=200, D=70, dtype=dtype)
    y, st = gpu_scan(inp)
    dev = {k: to_dev(v) for k, v in inp.items()}
    state = dev["state_in"].clone()
    ys = []
    for t in range(200):
        yt = ssm.ssm_step(dev["x"][:, t].contiguous(), dev["delta"][:, t].contiguous(), dev["A"],
                          dev["Bt"][:, t].contiguous(), dev["Ct"][:, t].contiguous(), state,
                          Dskip=dev["Dskip"], z=dev["z"][:, t].contiguous())
        ys.append(to_f64(yt))
    torch.cuda.synchronize()
    check(np.stack(ys, 1), y, dtype, "fold of steps vs scan (y)")
    check(to_f64(state), st, dtype, "fold of steps vs scan (state)")


@pytest.mark.parametrize("cfg", ["c0", "c1"])
def test_bitwise_deterministic(cfg):
    say(f"case determinism {cfg}")
    inp = W.scan_inputs(W.SCAN_CONFIGS[cfg])
    y1, _ = gpu_scan(inp, want_state=False)
    y2, _ = gpu_scan(inp, want_state=False)
    assert np.array_equal(y1, y2)


def test_zero_delta_keeps_state_bitwise():
    say("case delta = 0")
    inp = _inp(L=1000, D=64, state=1.0)
    inp["delta"] = np.zeros_like(inp["delta"])
    y, st = gpu_scan(inp)
    assert np.array_equal(st, inp["state_in"].astype(np.float64))
    yr, _ = oracle_scan(inp, "f32")
    check(y, yr, "f32", "y with delta = 0")


def test_state_in_place():
    say("case state_out aliases state_in")
    inp = _inp(L=500, D=80)
    y, st = gpu_scan(inp)
    y2, st2 = gpu_scan(inp, state_alias=True)
    assert np.array_equal(y, y2) and np.array_equal(st, st2)


def test_empty_and_zero_length():
    import torch
    say("case empty")
    A = torch.full((64, 16), -1.0, device="cuda")
    x = torch.zeros((0, 5, 64), device="cuda")
    Bt = torch.zeros((0, 5, 16), device="cuda")
    ssm.ssm_scan_fwd(x, x, A, Bt, Bt)
    # L = 0: state_out receives state_in (or zeros)
    x = torch.zeros((2, 0, 64), device="cuda")
    Bt = torch.zeros((2, 0, 16), device="cuda")
    sin = torch.randn((2, 64, 16), device="cuda")
    sout = torch.full((2, 64, 16), 7.0, device="cuda")
    ssm.ssm_scan_fwd(x, x, A, Bt, Bt, state_in=sin, state_out=sout)
    torch.cuda.synchronize()
    assert torch.equal(sin, sout)
    ssm.ssm_scan_fwd(x, x, A, Bt, Bt, state_out=sout)
    torch.cuda.synchronize()
    assert not sout.any()


def test_lookback_many_chunks_one_column():
    """One channel block and thousands of chunks: long chains of cross-workgroup
    carries (every chunk depends on all earlier ones)."""
    say("case look-back stress: 1 x 200000 x 16")
    inp = _inp(L=200_000, D=16, dtype="f32", state=0.5, seed=81, batch=1)
    y, st = gpu_scan(inp)
    yr, sr = oracle_scan(inp, "f32")
    check(y, yr, "f32", "y")
    check(st, sr, "f32", "state_out")


def test_workspace_reuse_across_sizes():
    """A workspace reused by calls of different sizes without clearing."""
    import torch
    say("case workspace reuse")
    big = _inp(L=5000, D=96, seed=82)
    small = _inp(L=700, D=40, seed=83)
    nbytes = max(ssm.ssm_scan_workspace_bytes(2, 5000, 96, 16, 0), ssm.ssm_scan_workspace_bytes(2, 700, 40, 16, 0))
    ws = ssm.new_workspace(nbytes)
    for inp in (big, small, big, small):
        dev = {k: to_dev(v) for k, v in inp.items()}
        st = torch.empty_like(dev["state_in"])
        y = ssm.ssm_scan_fwd(dev["x"], dev["delta"], dev["A"], dev["Bt"], dev["Ct"], Dskip=dev["Dskip"],
                             z=dev["z"], state_in=dev["state_in"], state_out=st, workspace=ws)
        torch.cuda.synchronize()
        assert ssm.workspace_error(ws) == 0
        yr, sr = oracle_scan(inp, "f32")
        check(to_f64(y), yr, "f32", "y")
        check(to_f64(st), sr, "f32", "state_out")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_graph_replay(dtype):
    """Decode steps captured into a HIP graph: every replay (with eager scans and
    synchronisations between replays) equals the same steps launched eagerly,
    bit for bit, in y and in the state."""
    import torch
    say(f"case graph replay dtype={dtype}")
    inp = _inp(L=6, D=200, dtype=dtype, batch=3)
    dev = {k: to_dev(v) for k, v in inp.items()}
    tok = lambda k, t: dev[k][:, t].contiguous()
    toks = [{k: tok(k, t) for k in ("x", "delta", "Bt", "Ct", "z")} for t in range(6)]
    st_g = dev["state_in"].clone()
    st_e = dev["state_in"].clone()
    y_g = torch.empty_like(toks[0]["x"])
    y_e = torch.empty_like(toks[0]["x"])

    def steps(state, y):
        for tk in toks:
            ssm.ssm_step(tk["x"], tk["delta"], dev["A"], tk["Bt"], tk["Ct"], state, Dskip=dev["Dskip"],
                         z=tk["z"], y=y, stream=torch.cuda.current_stream())

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        steps(st_g, y_g)
    torch.cuda.synchronize()
    st_g.copy_(dev["state_in"])
    for rep in range(4):
        graph.replay()
        steps(st_e, y_e)
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"y differs on replay {rep}"
        assert torch.equal(st_g, st_e), f"state differs on replay {rep}"
        gpu_scan(_inp(L=50, D=40, dtype=dtype, seed=81 + rep))  # eager work between replays
        torch.cuda.synchronize()
