"""The C ABI on the host: the library loads, exports what include/ssm.h
declares, and rejects bad arguments before any HIP call (CPU only; no
kernel is launched here)."""
import ctypes
import os
import re

import pytest

import selective_state_space_16_amd as ssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssm.h")

P = 0x10000        # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10004      # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_\w+)\s*\(", text)))


def test_header_matches_binding():
    assert declared_functions() == sorted(ssm.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ssm.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and the exported symbols are really in the dynamic symbol table
    out = os.popen("nm -D --defined-only " + ssm.lib_path).read()
    for name in declared_functions():
        assert re.search(r"\sT\s" + name + r"$", out, re.M), name


def test_status_strings_and_version():
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        assert ssm.ssm_status_string(code) and ssm.ssm_status_string(code) != "unknown status"
    assert ssm.ssm_status_string(99) == "unknown status"
    assert "gfx950" in ssm.ssm_version()


def test_workspace_status_without_a_workspace():
    # no workspace, or one too small to hold a header: nothing to report, no HIP call
    assert ssm.lib().ssm_scan_workspace_status(None, 0, None) == 0
    assert ssm.lib().ssm_scan_workspace_status(P, 16, None) == 0
    assert ssm.lib().ssm_scan_workspace_status(MIS, 4096, None) == -5


def noalloc(**kw):
    a = dict(batch=1, L=8, D=64, N=16, dtype=0, x=P, delta=P, A=P, Bt=P, Ct=P, Dskip=None, z=None,
             state_in=None, state_out=None, y=P, stream=None)
    a.update(kw)
    return ssm.lib().ssm_scan_fwd_noalloc(a["batch"], a["L"], a["D"], a["N"], a["dtype"], a["x"], a["delta"],
                                          a["A"], a["Bt"], a["Ct"], a["Dskip"], a["z"], a["state_in"],
                                          a["state_out"], a["y"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=2), -3), (dict(N=3), -4), (dict(x=None), -1), (dict(y=None), -1),
    (dict(x=MIS), -5), (dict(state_out=MIS), -5),
    # the chunked scan (channel rows not whole 16-byte pieces) of a large
    # input needs more workspace than the library's static array
    (dict(batch=64, L=1 << 16, D=63), -6),
])
def test_noalloc_rejects_before_any_hip_call(kw, code):
    assert noalloc(**kw) == code


def test_noalloc_empty_is_ok_without_gpu():
    assert noalloc(batch=0) == 0 and noalloc(D=0) == 0
    # L = 0 with state_out aliasing state_in: nothing to copy
    assert noalloc(L=0, state_in=P, state_out=P) == 0


def test_workspace_bytes():
    assert ssm.ssm_scan_workspace_bytes(1, 256, 64, 16, ssm.SSM_F32) >= 0
    assert ssm.ssm_scan_workspace_bytes(-1, 256, 64, 16, ssm.SSM_F32) == 0
    assert ssm.ssm_scan_workspace_bytes(1, 256, 64, 3, ssm.SSM_F32) == 0
    assert ssm.ssm_scan_workspace_bytes(1, 256, 64, 16, 7) == 0
    assert ssm.ssm_scan_workspace_bytes(0, 256, 64, 16, ssm.SSM_F32) == 0
    # long sequences are split and need chunk summaries: (N+1) floats per chunk and channel
    w = ssm.ssm_scan_workspace_bytes(1, 1 << 20, 1536, 16, ssm.SSM_BF16)
    assert w > 0 and w % 256 == 0


def scan(**kw):
    a = dict(batch=1, L=8, D=64, N=16, dtype=0, x=P, delta=P, A=P, Bt=P, Ct=P, Dskip=None, z=None,
             state_in=None, state_out=None, y=P, ws=None, wsb=0, stream=None)
    a.update(kw)
    return ssm.lib().ssm_scan_fwd(a["batch"], a["L"], a["D"], a["N"], a["dtype"], a["x"], a["delta"],
                                  a["A"], a["Bt"], a["Ct"], a["Dskip"], a["z"], a["state_in"],
                                  a["state_out"], a["y"], a["ws"], a["wsb"], a["stream"])


def step(**kw):
    a = dict(batch=1, D=64, N=16, dtype=0, x=P, delta=P, A=P, Bt=P, Ct=P, Dskip=None, z=None,
             state=P, y=P, stream=None)
    a.update(kw)
    return ssm.lib().ssm_step(a["batch"], a["D"], a["N"], a["dtype"], a["x"], a["delta"], a["A"],
                              a["Bt"], a["Ct"], a["Dskip"], a["z"], a["state"], a["y"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(L=-5), -2), (dict(D=-1), -2), (dict(N=-16), -2),
    (dict(dtype=2), -3), (dict(N=3), -4), (dict(N=32), -4), (dict(N=0), -4),
    (dict(x=None), -1), (dict(delta=None), -1), (dict(A=None), -1), (dict(Bt=None), -1),
    (dict(Ct=None), -1), (dict(y=None), -1),
    (dict(x=MIS), -5), (dict(Ct=MIS), -5), (dict(z=MIS), -5), (dict(Dskip=MIS), -5),
    (dict(state_out=MIS), -5),
    (dict(batch=1 << 40, L=1 << 20, D=1 << 20), -2),
    # a long sequence needs a workspace
    (dict(L=1 << 20, D=64), -6), (dict(L=1 << 20, D=64, ws=P, wsb=16), -6),
])
def test_scan_rejects(kw, code):
    assert scan(**kw) == code


def test_scan_empty_is_ok_without_gpu():
    # nothing to compute: returns before any HIP call
    assert scan(batch=0) == 0
    assert scan(D=0) == 0
    assert scan(L=0) == 0            # no state_out: nothing to write


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=5), -3), (dict(N=5), -4), (dict(state=None), -1),
    (dict(y=None), -1), (dict(state=MIS), -5), (dict(Bt=MIS), -5),
])
def test_step_rejects(kw, code):
    assert step(**kw) == code


def test_step_empty_is_ok_without_gpu():
    assert step(batch=0) == 0
    assert step(D=0) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 8)
    A = torch.zeros(8, 16)
    with pytest.raises((ValueError, TypeError)):
        ssm.ssm_scan_fwd(x, x, A, torch.zeros(1, 4, 16), torch.zeros(1, 4, 16))


def scan_dt(**kw):
    a = dict(batch=1, L=8, D=64, N=16, dtype=0, x=P, delta_raw=P, dt_bias=None, A=P, Bt=P, Ct=P, Dskip=None,
             z=None, state_in=None, state_out=None, y=P, ws=None, wsb=0, stream=None)
    a.update(kw)
    return ssm.lib().ssm_scan_fwd_dt(a["batch"], a["L"], a["D"], a["N"], a["dtype"], a["x"], a["delta_raw"],
                                     a["dt_bias"], a["A"], a["Bt"], a["Ct"], a["Dskip"], a["z"], a["state_in"],
                                     a["state_out"], a["y"], a["ws"], a["wsb"], a["stream"])


def step_dt(**kw):
    a = dict(batch=1, D=64, N=16, dtype=0, x=P, delta_raw=P, dt_bias=None, A=P, Bt=P, Ct=P, Dskip=None,
             z=None, state=P, y=P, stream=None)
    a.update(kw)
    return ssm.lib().ssm_step_dt(a["batch"], a["D"], a["N"], a["dtype"], a["x"], a["delta_raw"], a["dt_bias"],
                                 a["A"], a["Bt"], a["Ct"], a["Dskip"], a["z"], a["state"], a["y"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=2), -3), (dict(N=3), -4), (dict(delta_raw=None), -1),
    (dict(y=None), -1), (dict(dt_bias=MIS), -5), (dict(x=MIS), -5),
    (dict(L=1 << 20, D=64), -6),
])
def test_scan_dt_rejects(kw, code):
    assert scan_dt(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=2), -3), (dict(N=5), -4), (dict(delta_raw=None), -1),
    (dict(state=None), -1), (dict(dt_bias=MIS), -5),
])
def test_step_dt_rejects(kw, code):
    assert step_dt(**kw) == code


def test_dt_entry_points_empty_ok_without_gpu():
    assert scan_dt(batch=0) == 0 and scan_dt(D=0) == 0
    assert step_dt(batch=0) == 0 and step_dt(D=0) == 0


def scan_conv(**kw):
    a = dict(batch=1, L=8, D=64, N=16, dtype=0, x_raw=P, conv_w=P, conv_b=None, conv_state=None, delta_raw=P,
             dt_bias=None, A=P, Bt=P, Ct=P, Dskip=None, z=None, state_in=None, state_out=None, y=P, ws=None, wsb=0,
             stream=None)
    a.update(kw)
    return ssm.lib().ssm_scan_fwd_conv(a["batch"], a["L"], a["D"], a["N"], a["dtype"], a["x_raw"], a["conv_w"],
                                       a["conv_b"], a["conv_state"], a["delta_raw"], a["dt_bias"], a["A"], a["Bt"],
                                       a["Ct"], a["Dskip"], a["z"], a["state_in"], a["state_out"], a["y"], a["ws"],
                                       a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=2), -3), (dict(N=3), -4), (dict(conv_w=None), -1), (dict(x_raw=None), -1),
    (dict(delta_raw=None), -1), (dict(y=None), -1), (dict(conv_w=MIS), -5), (dict(conv_b=MIS), -5),
    (dict(conv_state=MIS), -5), (dict(x_raw=MIS), -5), (dict(L=1 << 20, D=64), -6),
])
def test_scan_conv_rejects(kw, code):
    assert scan_conv(**kw) == code


def step_conv(**kw):
    a = dict(batch=1, D=64, N=16, dtype=0, x_raw=P, conv_w=P, conv_b=None, conv_state=P, delta_raw=P, dt_bias=None,
             A=P, Bt=P, Ct=P, Dskip=None, z=None, state=P, y=P, stream=None)
    a.update(kw)
    return ssm.lib().ssm_step_conv(a["batch"], a["D"], a["N"], a["dtype"], a["x_raw"], a["conv_w"], a["conv_b"],
                                   a["conv_state"], a["delta_raw"], a["dt_bias"], a["A"], a["Bt"], a["Ct"],
                                   a["Dskip"], a["z"], a["state"], a["y"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=2), -3), (dict(N=5), -4), (dict(conv_w=None), -1), (dict(conv_state=None), -1),
    (dict(x_raw=None), -1), (dict(state=None), -1), (dict(conv_w=MIS), -5), (dict(conv_b=MIS), -5),
    (dict(conv_state=MIS), -5),
])
def test_step_conv_rejects(kw, code):
    assert step_conv(**kw) == code


def test_conv_entry_point_empty_ok_without_gpu():
    assert scan_conv(batch=0) == 0 and scan_conv(D=0) == 0 and scan_conv(conv_w=None, L=0) == 0
    assert step_conv(batch=0) == 0 and step_conv(D=0) == 0 and step_conv(conv_state=None, batch=0) == 0


def scan_trap(**kw):
    a = dict(batch=1, L=8, D=64, N=16, dtype=0, x=P, delta=P, lam=P, A=P, Bt=P, Ct=P, Dskip=None, z=None,
             x_prev=None, B_prev=None, state_in=None, state_out=None, y=P, ws=None, wsb=0, stream=None)
    a.update(kw)
    return ssm.lib().ssm_scan_fwd_trap(a["batch"], a["L"], a["D"], a["N"], a["dtype"], a["x"], a["delta"],
                                       a["lam"], a["A"], a["Bt"], a["Ct"], a["Dskip"], a["z"], a["x_prev"],
                                       a["B_prev"], a["state_in"], a["state_out"], a["y"], a["ws"], a["wsb"],
                                       a["stream"])


def step_trap(**kw):
    a = dict(batch=1, D=64, N=16, dtype=0, x=P, delta=P, lam=P, A=P, Bt=P, Ct=P, Dskip=None, z=None,
             x_prev=None, B_prev=None, state=P, y=P, stream=None)
    a.update(kw)
    return ssm.lib().ssm_step_trap(a["batch"], a["D"], a["N"], a["dtype"], a["x"], a["delta"], a["lam"], a["A"],
                                   a["Bt"], a["Ct"], a["Dskip"], a["z"], a["x_prev"], a["B_prev"], a["state"],
                                   a["y"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=2), -3), (dict(N=3), -4), (dict(lam=None), -1), (dict(delta=None), -1),
    (dict(x_prev=P), -1), (dict(B_prev=P), -1), (dict(y=None), -1), (dict(lam=MIS), -5),
    (dict(x_prev=MIS, B_prev=P), -5), (dict(x_prev=P, B_prev=MIS), -5), (dict(L=1 << 20, D=64), -6),
])
def test_scan_trap_rejects(kw, code):
    assert scan_trap(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=2), -3), (dict(N=5), -4), (dict(lam=None), -1), (dict(state=None), -1),
    (dict(x_prev=P), -1), (dict(B_prev=P), -1), (dict(lam=MIS), -5), (dict(x_prev=MIS, B_prev=P), -5),
])
def test_step_trap_rejects(kw, code):
    assert step_trap(**kw) == code


def test_trap_entry_points_empty_ok_without_gpu():
    assert scan_trap(batch=0) == 0 and scan_trap(D=0) == 0 and scan_trap(lam=None, L=0) == 0
    assert step_trap(batch=0) == 0 and step_trap(D=0) == 0


def ssd(**kw):
    a = dict(batch=1, L=8, H=4, P=64, G=1, N=128, dtype=1, x=P, delta=P, A=P, Bt=P, Ct=P, Dskip=None,
             state_in=None, state_out=None, y=P, stream=None)
    a.update(kw)
    return ssm.lib().ssm_ssd_fwd(a["batch"], a["L"], a["H"], a["P"], a["G"], a["N"], a["dtype"], a["x"], a["delta"],
                                 a["A"], a["Bt"], a["Ct"], a["Dskip"], a["state_in"], a["state_out"], a["y"],
                                 a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=3), -3), (dict(dtype=0), -4), (dict(P=32), -4), (dict(N=16), -4),
    (dict(G=3), -2), (dict(G=0), -2), (dict(x=None), -1), (dict(y=None), -1), (dict(Bt=MIS), -5),
    (dict(state_out=MIS), -5),
    # 64 tokens of x or of Bt, Ct would span 4 GiB or more (the kernel's offsets are 32-bit)
    (dict(H=8192 * 64, G=1), -4), (dict(H=1 << 18, G=1 << 18, N=128), -4),
])
def test_ssd_rejects(kw, code):
    assert ssd(**kw) == code


def test_ssd_empty_ok_without_gpu():
    assert ssd(batch=0) == 0 and ssd(H=0) == 0 and ssd(L=0) == 0


def test_ssd_largest_offsets_accepted():
    """The largest H and G * N the 32-bit offsets allow pass the checks (an
    empty batch, so nothing runs)."""
    assert ssd(batch=0, H=8192 * 64 - 1, G=1) == 0
    assert ssd(batch=0, H=(1 << 25) // 128 - 1, G=(1 << 25) // 128 - 1, N=128) == 0


def bwd(**kw):
    a = dict(batch=2, L=100, D=64, N=16, dtype=0, x=P, delta=P, A=P, Bt=P, Ct=P, Dskip=None, z=None,
             state_in=None, dy=P, dstate=None, dx=P, ddelta=P, dA=P, dBt=P, dCt=P, dDskip=None, dz=None,
             dstate_in=None, ws=P, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return ssm.lib().ssm_scan_bwd(a["batch"], a["L"], a["D"], a["N"], a["dtype"], a["x"], a["delta"], a["A"],
                                  a["Bt"], a["Ct"], a["Dskip"], a["z"], a["state_in"], a["dy"], a["dstate"],
                                  a["dx"], a["ddelta"], a["dA"], a["dBt"], a["dCt"], a["dDskip"], a["dz"],
                                  a["dstate_in"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(L=-1), -2), (dict(dtype=2), -3), (dict(N=3), -4), (dict(N=32), -4),
    (dict(dA=None), -1), (dict(z=P, dz=None), -1), (dict(x=None), -1), (dict(dy=None), -1), (dict(dx=None), -1),
    (dict(ddelta=None), -1), (dict(dBt=None), -1), (dict(dCt=None), -1), (dict(dz=MIS, z=P), -5),
    (dict(dstate=MIS), -5), (dict(ws=None), -6), (dict(ws_bytes=100), -6), (dict(ws=MIS), -5),
    (dict(batch=1 << 40, L=1 << 20), -2),
])
def test_scan_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def test_scan_bwd_workspace_bytes():
    f = ssm.ssm_scan_bwd_workspace_bytes
    assert f(0, 10, 64, 16, 0) == 0 and f(1, 0, 64, 16, 0) == 0 and f(1, 10, 0, 16, 0) == 0
    assert f(1, 10, 64, 3, 0) == 0 and f(1, 10, 64, 16, 5) == 0 and f(-1, 10, 64, 16, 0) == 0
    # 4 chunks of 32 tokens; every region a multiple of 256 bytes after a 256-byte header
    n = f(2, 100, 64, 16, 0)
    # states, gradients and dA partials per (batch, chunk, channel, n); dBt, dCt partials
    assert n % 256 == 0 and n >= 256 + 3 * 2 * 4 * 64 * 16 * 4 + 2 * 2 * 100 * 16 * 4
    assert f(2, 100, 64, 16, 1) == n  # the workspace is float32 whatever the activation dtype
    assert f(2, 200, 64, 16, 0) > n


def test_scan_bwd_empty_ok_without_gpu():
    assert bwd(D=0) == 0


def bwd_dt(**kw):
    a = dict(batch=2, L=100, D=64, N=16, dtype=0, x=P, delta=P, dt_bias=None, A=P, Bt=P, Ct=P, Dskip=None, z=None,
             state_in=None, dy=P, dstate=None, dx=P, ddelta=P, ddt_bias=None, dA=P, dBt=P, dCt=P, dDskip=None,
             dz=None, dstate_in=None, ws=P, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return ssm.lib().ssm_scan_bwd_dt(a["batch"], a["L"], a["D"], a["N"], a["dtype"], a["x"], a["delta"],
                                     a["dt_bias"], a["A"], a["Bt"], a["Ct"], a["Dskip"], a["z"], a["state_in"],
                                     a["dy"], a["dstate"], a["dx"], a["ddelta"], a["ddt_bias"], a["dA"], a["dBt"],
                                     a["dCt"], a["dDskip"], a["dz"], a["dstate_in"], a["ws"], a["ws_bytes"],
                                     a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=2), -3), (dict(N=5), -4), (dict(dA=None), -1), (dict(delta=None), -1),
    (dict(ddelta=None), -1), (dict(dt_bias=MIS), -5), (dict(ddt_bias=MIS), -5), (dict(ws_bytes=1), -6),
])
def test_scan_bwd_dt_rejects(kw, code):
    assert bwd_dt(**kw) == code


def test_scan_bwd_dt_empty_ok_without_gpu():
    assert bwd_dt(D=0) == 0


def bwd_conv(**kw):
    a = dict(batch=2, L=100, D=64, N=16, dtype=0, x_raw=P, conv_w=P, conv_b=None, conv_state=None, delta=P,
             dt_bias=None, A=P, Bt=P, Ct=P, Dskip=None, z=None, state_in=None, dy=P, dstate=None, dx_raw=P,
             dconv_w=P, dconv_b=None, dconv_state=None, ddelta=P, ddt_bias=None, dA=P, dBt=P, dCt=P, dDskip=None,
             dz=None, dstate_in=None, ws=P, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return ssm.lib().ssm_scan_bwd_conv(a["batch"], a["L"], a["D"], a["N"], a["dtype"], a["x_raw"], a["conv_w"],
                                       a["conv_b"], a["conv_state"], a["delta"], a["dt_bias"], a["A"], a["Bt"],
                                       a["Ct"], a["Dskip"], a["z"], a["state_in"], a["dy"], a["dstate"], a["dx_raw"],
                                       a["dconv_w"], a["dconv_b"], a["dconv_state"], a["ddelta"], a["ddt_bias"],
                                       a["dA"], a["dBt"], a["dCt"], a["dDskip"], a["dz"], a["dstate_in"], a["ws"],
                                       a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=2), -3), (dict(N=5), -4), (dict(conv_w=None), -1), (dict(dconv_w=None), -1),
    (dict(x_raw=None), -1), (dict(dx_raw=None), -1), (dict(delta=None), -1), (dict(dy=None), -1),
    (dict(dA=None), -1), (dict(conv_w=MIS), -5), (dict(conv_state=MIS), -5), (dict(dconv_state=MIS), -5),
    (dict(x_raw=MIS), -5), (dict(dt_bias=MIS), -5), (dict(ws_bytes=1), -6), (dict(ws=None), -6),
])
def test_scan_bwd_conv_rejects(kw, code):
    assert bwd_conv(**kw) == code


def test_scan_bwd_conv_workspace_bytes():
    f = ssm.lib().ssm_scan_bwd_conv_workspace_bytes
    base = ssm.lib().ssm_scan_bwd_workspace_bytes(2, 100, 64, 16, 1)
    # the scan gradient's, the branch's output and its gradient (bf16), the partial sums
    assert f(2, 100, 64, 16, 1) >= base + 2 * 2 * 100 * 64 * 2
    assert f(0, 100, 64, 16, 1) == 0 and f(2, 0, 64, 16, 1) == 0 and f(2, 100, 64, 3, 1) == 0


def test_scan_bwd_conv_empty_ok_without_gpu():
    assert bwd_conv(D=0) == 0


def bwd_trap(**kw):
    a = dict(batch=2, L=100, D=64, N=16, dtype=0, x=P, delta=P, lam=P, A=P, Bt=P, Ct=P, Dskip=None, z=None,
             x_prev=None, B_prev=None, state_in=None, dy=P, dstate=None, dx=P, ddelta=P, dlam=P, dA=P, dBt=P, dCt=P,
             dDskip=None, dz=None, dx_prev=None, dB_prev=None, dstate_in=None, ws=P, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return ssm.lib().ssm_scan_bwd_trap(*[a[k] for k in (
        "batch", "L", "D", "N", "dtype", "x", "delta", "lam", "A", "Bt", "Ct", "Dskip", "z", "x_prev", "B_prev",
        "state_in", "dy", "dstate", "dx", "ddelta", "dlam", "dA", "dBt", "dCt", "dDskip", "dz", "dx_prev",
        "dB_prev", "dstate_in", "ws", "ws_bytes", "stream")])


@pytest.mark.parametrize("kw,code", [
    (dict(lam=None), -1), (dict(dlam=None), -1), (dict(x_prev=P), -1), (dict(B_prev=P), -1),
    (dict(dx_prev=P), -1), (dict(dB_prev=P), -1), (dict(lam=MIS), -5), (dict(dlam=MIS), -5),
    (dict(x_prev=P, B_prev=MIS), -5), (dict(N=3), -4), (dict(ws=None), -6),
])
def test_scan_bwd_trap_rejects(kw, code):
    assert bwd_trap(**kw) == code


def test_scan_bwd_trap_empty_ok_without_gpu():
    assert bwd_trap(D=0) == 0


def ssd_step(**kw):
    a = dict(batch=2, H=4, P=64, G=1, N=128, dtype=1, x=P, delta=P, A=P, Bt=P, Ct=P, Dskip=None, state=P, y=P,
             stream=None)
    a.update(kw)
    return ssm.lib().ssm_ssd_step(*[a[k] for k in ("batch", "H", "P", "G", "N", "dtype", "x", "delta", "A", "Bt",
                                                    "Ct", "Dskip", "state", "y", "stream")])


@pytest.mark.parametrize("kw,code", [
    (dict(batch=-1), -2), (dict(dtype=4), -3), (dict(P=32), -4), (dict(N=16), -4), (dict(G=3), -2), (dict(G=0), -2),
    (dict(x=None), -1), (dict(state=None), -1), (dict(y=None), -1), (dict(state=MIS), -5), (dict(Dskip=MIS), -5),
])
def test_ssd_step_rejects(kw, code):
    assert ssd_step(**kw) == code


def test_ssd_step_empty_ok_without_gpu():
    assert ssd_step(batch=0) == 0 and ssd_step(H=0) == 0
