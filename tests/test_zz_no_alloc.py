"""ssm_scan_fwd_noalloc on the GPU (needs MI355X): the scan with the library's
static workspace equals ssm_scan_fwd with a workspace of its own, bit for bit,
on calls in a row of shrinking size (the array keeps the last call's words),
on the chunked scan's shapes, and when captured into a graph and replayed."""
import pytest

import selective_state_space_16_amd as ssm
import workloads as W
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _dev(batch, L, D, dtype, seed, state=0.3):
    cfg = W.ScanConfig("noalloc", batch, L, D, 16, dtype, gate=True, dskip="uniform", state_in=state, seed=seed)
    return {k: to_dev(v) for k, v in W.scan_inputs(cfg).items()}


def _both(d):
    """(y, state) from ssm_scan_fwd with its own workspace, and from the
    no-allocation entry point."""
    import torch
    st_a, st_b = torch.empty_like(d["state_in"]), torch.empty_like(d["state_in"])
    y_a = ssm.ssm_scan_fwd(d["x"], d["delta"], d["A"], d["Bt"], d["Ct"], Dskip=d["Dskip"], z=d["z"],
                           state_in=d["state_in"], state_out=st_a)
    y_b = torch.empty_like(d["x"])
    ssm.ssm_scan_fwd_noalloc(d["x"], d["delta"], d["A"], d["Bt"], d["Ct"], y_b, Dskip=d["Dskip"], z=d["z"],
                             state_in=d["state_in"], state_out=st_b)
    torch.cuda.synchronize()
    return (y_a, st_a), (y_b, st_b)


@pytest.mark.parametrize("dtype,shapes", [
    ("f32", [(2, 2048, 1536), (1, 700, 96)]),            # every column cut into stripes, then a smaller call
    ("bf16", [(1, 131072, 1536), (2, 1000, 256)]),       # many stripes per column, then a smaller call
    ("f32", [(1, 3000, 63), (1, 200, 5)]),               # the chunked scan (rows not whole 16-byte pieces)
])
def test_noalloc_equals_scan(dtype, shapes):
    import torch
    for k, (batch, L, D) in enumerate(shapes):
        say(f"case noalloc dtype={dtype} shape=({batch}, {L}, {D}, 16) call {k}")
        (y_a, st_a), (y_b, st_b) = _both(_dev(batch, L, D, dtype, seed=70 + k))
        assert torch.isfinite(y_b).all()
        assert torch.equal(y_a, y_b), "y differs from ssm_scan_fwd"
        assert torch.equal(st_a, st_b), "state differs from ssm_scan_fwd"


def test_noalloc_graph_replay():
    """Captured into a graph (nothing to allocate during capture), replayed
    three times with an eager call of another size in between."""
    import torch
    say("case noalloc graph replay")
    d = _dev(2, 2048, 1536, "bf16", seed=75)
    (y_ref, st_ref), _ = _both(d)
    y_g, st_g = torch.empty_like(y_ref), torch.empty_like(st_ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ssm.ssm_scan_fwd_noalloc(d["x"], d["delta"], d["A"], d["Bt"], d["Ct"], y_g, Dskip=d["Dskip"], z=d["z"],
                                 state_in=d["state_in"], state_out=st_g, stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    small = _dev(1, 600, 128, "bf16", seed=76)
    for rep in range(3):
        y_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_ref) and torch.equal(st_g, st_ref), f"replay {rep} differs"
        _both(small)
