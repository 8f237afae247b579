"""Helpers for the GPU parity tests: move stored inputs to the device, run the
library through its binding, compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import selective_state_space_16_amd as ssm
import workloads as W

# Tolerances fixed for this path: float32 activations must match the float64
# oracle to relative L2 1e-5 and max-abs 1e-4; bfloat16 activations with a
# float32 state to relative L2 2e-2 (outputs and final state).
TOL = {"f32": {"rel": 1e-5, "maxabs": 1e-4}, "bf16": {"rel": 2e-2, "maxabs": None}}


def say(*a):
    """Print and flush, so a GPU failure names the case that was running."""
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def to_host(t):
    """A device tensor as the stored numpy array the oracle takes: float32 as
    it is, bfloat16 as its uint16 bit patterns (exact)."""
    import torch
    if t is None:
        return None
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def device_scan_blocks(dev, y, st_out, chans):
    """Blocks of a scan run on the device, for oracle.scan_compare: for every
    batch row and every `chans` channels, the stored inputs of those channels
    over the whole sequence (copied back from the device), and the device's y
    and final state for them in float64."""
    batch, L, D = dev["x"].shape
    for b in range(batch):
        bt, ct = to_host(dev["Bt"][b:b + 1]), to_host(dev["Ct"][b:b + 1])
        for c0 in range(0, D, chans):
            sl = slice(c0, min(D, c0 + chans))
            part = lambda k: None if dev.get(k) is None else to_host(dev[k][b:b + 1, :, sl])
            inp = {"x": part("x"), "delta": part("delta"), "z": part("z"), "Bt": bt, "Ct": ct,
                   "A": to_host(dev["A"][sl]), "Dskip": None if dev.get("Dskip") is None else to_host(dev["Dskip"][sl]),
                   "state_in": None if dev.get("state_in") is None else to_host(dev["state_in"][b:b + 1, sl])}
            yield inp, to_f64(y[b:b + 1, :, sl]), (None if st_out is None else to_f64(st_out[b:b + 1, sl]))


def check_sum(acc, dtype, what):
    """check() for an oracle.ErrorSum accumulated over a whole output."""
    tol = TOL[dtype]
    say(f"  {what}: relL2={acc.rel:.3e} maxabs={acc.maxabs:.3e} over {acc.count} values")
    assert np.isfinite(acc.rel), what + ": non-finite output"
    assert acc.rel <= tol["rel"], f"{what}: relL2 {acc.rel:.3e} > {tol['rel']}"
    if tol["maxabs"] is not None:
        assert acc.maxabs <= tol["maxabs"], f"{what}: maxabs {acc.maxabs:.3e} > {tol['maxabs']}"


def errors(got: np.ndarray, ref: np.ndarray):
    diff = got - ref
    nref = float(np.sqrt(np.sum(ref * ref)))
    rel = float(np.sqrt(np.sum(diff * diff))) / (nref if nref > 0 else 1.0)
    return rel, float(np.abs(diff).max()) if diff.size else 0.0


def check(got, ref, dtype, what):
    rel, mx = errors(got, ref)
    tol = TOL[dtype]
    say(f"  {what}: relL2={rel:.3e} maxabs={mx:.3e}")
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    assert rel <= tol["rel"], f"{what}: relL2 {rel:.3e} > {tol['rel']}"
    if tol["maxabs"] is not None:
        assert mx <= tol["maxabs"], f"{what}: maxabs {mx:.3e} > {tol['maxabs']}"
    return rel, mx


def gpu_scan(inp, want_state=True, state_alias=False):
    """Run ssm_scan_fwd on stored inputs; returns (y64, state64 or None)."""
    import torch
    dev = {k: to_dev(v) for k, v in inp.items()}
    st_out = None
    if want_state:
        if state_alias and dev["state_in"] is not None:
            st_out = dev["state_in"]
        else:
            st_out = torch.empty((dev["x"].shape[0], dev["A"].shape[0], dev["A"].shape[1]),
                                 dtype=torch.float32, device="cuda")
    batch, L, D = dev["x"].shape
    ws = ssm.new_workspace(ssm.ssm_scan_workspace_bytes(batch, L, D, dev["A"].shape[1],
                                                        0 if dev["x"].dtype == torch.float32 else 1))
    y = ssm.ssm_scan_fwd(dev["x"], dev["delta"], dev["A"], dev["Bt"], dev["Ct"], Dskip=dev["Dskip"],
                         z=dev["z"], state_in=dev["state_in"], state_out=st_out, workspace=ws)
    torch.cuda.synchronize()
    assert ssm.workspace_error(ws) == 0, "a look-back wait gave up"
    return to_f64(y), (to_f64(st_out) if st_out is not None else None)


def oracle_scan(inp, dtype):
    return oracle.get().scan(inp, dtype)


def gpu_scan_dt(inp, dt_bias=True):
    """Run ssm_scan_fwd_dt on stored inputs (inp["delta_raw"], inp["dt_bias"]);
    returns (y64, state64). With dt_bias=False the bias argument is NULL."""
    import torch
    dev = {k: to_dev(v) for k, v in inp.items()}
    batch, L, D = dev["x"].shape
    N = dev["A"].shape[1]
    st_out = torch.empty((batch, D, N), dtype=torch.float32, device="cuda")
    ws = ssm.new_workspace(ssm.ssm_scan_workspace_bytes(batch, L, D, N,
                                                        0 if dev["x"].dtype == torch.float32 else 1))
    y = ssm.ssm_scan_fwd_dt(dev["x"], dev["delta_raw"], dev["dt_bias"] if dt_bias else None, dev["A"], dev["Bt"],
                            dev["Ct"], Dskip=dev["Dskip"], z=dev["z"], state_in=dev["state_in"], state_out=st_out,
                            workspace=ws)
    torch.cuda.synchronize()
    assert ssm.workspace_error(ws) == 0, "a look-back wait gave up"
    return to_f64(y), to_f64(st_out)


def gpu_scan_trap(inp, prev=True, want_state=True):
    """Run ssm_scan_fwd_trap on stored inputs (inp["lam"], inp["x_prev"],
    inp["B_prev"]); with prev=False no earlier token is passed. Returns (y64,
    state64 or None)."""
    import torch
    dev = {k: to_dev(v) for k, v in inp.items()}
    batch, L, D = dev["x"].shape
    N = dev["A"].shape[1]
    st_out = torch.empty((batch, D, N), dtype=torch.float32, device="cuda") if want_state else None
    ws = ssm.new_workspace(ssm.ssm_scan_workspace_bytes(batch, L, D, N,
                                                        0 if dev["x"].dtype == torch.float32 else 1))
    y = ssm.ssm_scan_fwd_trap(dev["x"], dev["delta"], dev["lam"], dev["A"], dev["Bt"], dev["Ct"],
                              Dskip=dev["Dskip"], z=dev["z"], x_prev=dev["x_prev"] if prev else None,
                              B_prev=dev["B_prev"] if prev else None, state_in=dev["state_in"], state_out=st_out,
                              workspace=ws)
    torch.cuda.synchronize()
    assert ssm.workspace_error(ws) == 0, "a look-back wait gave up"
    return to_f64(y), (to_f64(st_out) if st_out is not None else None)


def gpu_ssd(inp, want_state=True):
    """Run ssm_ssd_fwd on stored SSD inputs; returns (y64, state64 or None)."""
    import torch
    dev = {k: to_dev(v) for k, v in inp.items()}
    batch, L, H, P = dev["x"].shape
    N = dev["Bt"].shape[3]
    st_out = torch.empty((batch, H, P, N), dtype=torch.float32, device="cuda") if want_state else None
    y = ssm.ssm_ssd_fwd(dev["x"], dev["delta"], dev["A"], dev["Bt"], dev["Ct"], Dskip=dev["Dskip"],
                        state_in=dev["state_in"], state_out=st_out)
    torch.cuda.synchronize()
    return to_f64(y), (to_f64(st_out) if st_out is not None else None)


def gpu_scan_bwd(inp, grads, want_dskip=True, dstate_alias=False, raw=False, want_dbias=True, trap=False):
    """Run ssm_scan_bwd (or, with raw, ssm_scan_bwd_dt on delta_raw and dt_bias)
    on stored inputs and upstream gradients; returns a dict of float64 arrays
    with the oracle's keys (dDskip/dz None when absent)."""
    import torch
    dev = {k: to_dev(v) for k, v in inp.items()}
    dy, dstate = to_dev(grads["dy"]), to_dev(grads.get("dstate"))
    out = {}
    if dstate_alias and dstate is not None:
        out["dstate_in"] = dstate
    if not want_dskip:
        out["dDskip"] = None
    if trap:
        g = ssm.ssm_scan_bwd_trap(dev["x"], dev["delta"], dev["lam"], dev["A"], dev["Bt"], dev["Ct"], dy,
                                  Dskip=dev["Dskip"], z=dev["z"], x_prev=dev.get("x_prev"), B_prev=dev.get("B_prev"),
                                  state_in=dev["state_in"], dstate=dstate, out=out)
    elif raw:
        if not want_dbias:
            out["ddt_bias"] = None
        g = ssm.ssm_scan_bwd_dt(dev["x"], dev["delta_raw"], dev.get("dt_bias"), dev["A"], dev["Bt"], dev["Ct"], dy,
                                Dskip=dev["Dskip"], z=dev["z"], state_in=dev["state_in"], dstate=dstate, out=out)
    else:
        g = ssm.ssm_scan_bwd(dev["x"], dev["delta"], dev["A"], dev["Bt"], dev["Ct"], dy, Dskip=dev["Dskip"],
                             z=dev["z"], state_in=dev["state_in"], dstate=dstate, out=out)
    torch.cuda.synchronize()
    return {k: (None if v is None else to_f64(v)) for k, v in g.items()}


def oracle_scan_bwd(inp, grads, dtype):
    return oracle.get().scan_bwd(inp, grads["dy"], grads.get("dstate"), dtype)


def check_grads(got, ref, dtype, keys=None):
    """Every gradient against the oracle's: relative L2 as for the outputs;
    for float32, max-abs 1e-4 scaled by the largest reference magnitude (the
    parameter gradients are sums over many tokens and channels)."""
    for k in keys or ("dx", "ddelta", "ddelta_raw", "ddt_bias", "dlam", "dz", "dA", "dBt", "dCt", "dDskip",
                      "dx_prev", "dB_prev", "dstate_in"):
        if ref.get(k) is None:
            assert got.get(k) is None, k + " written but not expected"
            continue
        g, r = got[k], ref[k]
        rel, mx = errors(g, r)
        scale = max(1.0, float(np.abs(r).max()) if r.size else 1.0)
        say(f"  {k}: relL2={rel:.3e} maxabs={mx:.3e} (scale {scale:.3g})")
        assert np.all(np.isfinite(g)), k + ": non-finite output"
        assert rel <= TOL[dtype]["rel"], f"{k}: relL2 {rel:.3e} > {TOL[dtype]['rel']}"
        if TOL[dtype]["maxabs"] is not None:
            assert mx <= TOL[dtype]["maxabs"] * scale, f"{k}: maxabs {mx:.3e} > {TOL[dtype]['maxabs']} x {scale:.3g}"
