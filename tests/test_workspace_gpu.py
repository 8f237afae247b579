"""The scan's workspace on the GPU (needs MI355X): a scan captured into a HIP
graph replays like eager calls, and a wait that gives up poisons what depends
on it and is reported, without leaving anything behind for the next call.

The give-up is forced from the host: the header's error word is set to the tag
the next call will take, so every wait of that call gives up before its first
poll and every kernel exits normally."""
import numpy as np
import pytest

import selective_state_space_16_amd as ssm
import workloads as W
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu

HDR_ERROR, HDR_EPOCH, HDR_DONE = 0, 1, 2  # 32-bit words of the workspace header


def _inputs(dtype, L=2048, D=1536, batch=2, seed=90):
    # the small-model layer's shape: every tile column is cut into stripes
    cfg = W.ScanConfig("ws", batch, L, D, 16, dtype, gate=True, dskip="uniform", state_in=0.3, seed=seed)
    return {k: to_dev(v) for k, v in W.scan_inputs(cfg).items()}


def _run(d, ws, y=None, st=None, stream=None):
    import torch
    if y is None:
        y = torch.empty_like(d["x"])
    if st is None:
        st = torch.empty_like(d["state_in"])
    ssm.ssm_scan_fwd(d["x"], d["delta"], d["A"], d["Bt"], d["Ct"], Dskip=d["Dskip"], z=d["z"],
                     state_in=d["state_in"], state_out=st, y=y, workspace=ws, stream=stream)
    return y, st


def _header(ws):
    return ws[:16].view(__import__("torch").int32).cpu().numpy().astype(np.int64) & 0xFFFFFFFF


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_graph_replay(dtype):
    """ssm_scan_fwd with a workspace, captured into a graph: four replays,
    each followed by eager scans of other sizes on the same workspace, equal
    the eager call on the same inputs bit for bit (y and final state)."""
    import torch
    say(f"case scan graph replay dtype={dtype}")
    d = _inputs(dtype)
    other = _inputs(dtype, L=700, D=96, seed=91)
    nbytes = max(ssm.ssm_scan_workspace_bytes(2, 2048, 1536, 16, 0 if dtype == "f32" else 1),
                 ssm.ssm_scan_workspace_bytes(2, 700, 96, 16, 0 if dtype == "f32" else 1))
    ws = ssm.new_workspace(nbytes)
    y_ref, st_ref = _run(d, ws)  # eager reference (also warms up the library)
    torch.cuda.synchronize()
    assert ssm.ssm_scan_workspace_status(ws) == 0
    y_g, st_g = torch.empty_like(y_ref), torch.empty_like(st_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(d, ws, y_g, st_g, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(4):
        y_g.fill_(float("nan"))
        st_g.fill_(float("nan"))
        e0 = int(_header(ws)[HDR_EPOCH])
        graph.replay()
        torch.cuda.synchronize()
        h = _header(ws)
        assert h[HDR_EPOCH] == (e0 + 1) & 0xFFFFFFFF and h[HDR_DONE] == 0, f"header after replay {rep}: {h[:3]}"
        assert ssm.ssm_scan_workspace_status(ws) == 0
        assert torch.equal(y_g, y_ref), f"y differs on replay {rep}"
        assert torch.equal(st_g, st_ref), f"state differs on replay {rep}"
        _run(other, ws)  # eager work of another size on the same workspace
        _run(d, ws)
        torch.cuda.synchronize()
        assert ssm.ssm_scan_workspace_status(ws) == 0


@pytest.mark.parametrize("early", ["0", "1"])
def test_giveup_poisons_and_is_reported(early, monkeypatch):
    """A call whose waits give up: the first stripe of every column (which
    waits for nothing) is exact, every later token is NaN, the final state is
    NaN, the status reports SSM_ERR_TIMEOUT; the next call on the same
    workspace is exact and reports SSM_OK. In early mode too, where the later
    stripes have written y from a zero start before their wait: the walk from
    the NaN state never stops early, so it overwrites all of it."""
    import torch
    monkeypatch.setenv("SSM_STRIPE_EARLY", early)
    say(f"case forced give-up early={early}")
    d = _inputs("f32")
    ws = ssm.new_workspace(ssm.ssm_scan_workspace_bytes(2, 2048, 1536, 16, 0))
    y_ref, st_ref = _run(d, ws)
    torch.cuda.synchronize()
    assert ssm.ssm_scan_workspace_status(ws) == 0
    nxt = (int(_header(ws)[HDR_EPOCH]) + 1) & 0xFFFFFFFF
    nxt = nxt if nxt != 0 else 1
    ws[:16].view(torch.int32)[HDR_ERROR] = nxt - (1 << 32) if nxt >= (1 << 31) else nxt
    y, st = _run(d, ws)
    torch.cuda.synchronize()
    assert ssm.ssm_scan_workspace_status(ws) == ssm.SSM_ERR_TIMEOUT
    nan_tok = torch.isnan(y).any(dim=2).any(dim=0).cpu().numpy()
    first = int(np.argmax(nan_tok)) if nan_tok.any() else -1
    say(f"  first poisoned token {first} of {y.shape[1]}")
    assert 0 < first < y.shape[1], "the cut columns' later stripes must be poisoned"
    assert torch.equal(y[:, :first], y_ref[:, :first]), "the first stripes must be exact"
    assert torch.isnan(y[:, first:]).all(), "every token after the first stripe depends on a wait"
    assert torch.isnan(st).all()
    # the next call starts afresh
    y2, st2 = _run(d, ws)
    torch.cuda.synchronize()
    assert ssm.ssm_scan_workspace_status(ws) == 0
    assert torch.equal(y2, y_ref) and torch.equal(st2, st_ref)


def test_binding_owned_workspace_on_another_stream():
    """With no workspace given, the binding allocates and clears one on the
    current stream; a launch on another stream waits for that, and the result
    equals the same call on the current stream."""
    import torch
    say("case binding workspace on a side stream")
    d = _inputs("f32", L=1500, D=512, seed=92)
    y_ref = ssm.ssm_scan_fwd(d["x"], d["delta"], d["A"], d["Bt"], d["Ct"], Dskip=d["Dskip"], z=d["z"],
                             state_in=d["state_in"])
    side = torch.cuda.Stream()
    y = ssm.ssm_scan_fwd(d["x"], d["delta"], d["A"], d["Bt"], d["Ct"], Dskip=d["Dskip"], z=d["z"],
                         state_in=d["state_in"], stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
