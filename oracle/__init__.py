"""fp64 CPU oracle for the selective scan (S6) and its decode step.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the bench's CPU-baseline
leg may import this package; the product path never does. It shares no code
with the HIP library. The arithmetic lives in ``ssm_oracle.c`` (plain C,
float64, libm ``exp``, token loop in order); this module only compiles it with
gcc, upcasts stored inputs exactly to float64 and calls it through ctypes.

Parity is pinned by ``tests/test_oracle_pins.py`` against facts the pages fix
(worked step example, LTI convolution, geometric closed form, delta limits,
brute-force semiseparable sum, scalar-A masked form, step/scan composition;
for the exponential-trapezoidal variant the pages' seeded comparison with the
Euler rule, the classic trapezoidal convolution, second-order convergence on
an ODE with a closed-form solution, an unrolled sum and resumption) and by
``tests/test_oracle_mutants.py`` (each planted mistake fails a pin).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "ssm_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

_DP = ctypes.POINTER(ctypes.c_double)


def build(src: str = SRC, out: str = LIB, force: bool = False) -> str:
    """Compile the oracle with gcc -O2 -fopenmp (no fast-math)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes handle on one compiled oracle library."""

    def __init__(self, lib_path: Optional[str] = None):
        path = lib_path or build()
        self.path = path
        self.lib = ctypes.CDLL(path)
        i64, ci = ctypes.c_int64, ctypes.c_int
        self.lib.oracle_scan.argtypes = [i64, i64, i64, i64] + [_DP] * 10 + [ci]
        self.lib.oracle_scan.restype = ci
        self.lib.oracle_step.argtypes = [i64, i64, i64] + [_DP] * 9 + [ci]
        self.lib.oracle_step.restype = ci
        self.lib.oracle_threads.argtypes = [ci]
        self.lib.oracle_threads.restype = ci
        self.lib.oracle_softplus_bias.argtypes = [i64, i64, _DP, _DP, _DP]
        self.lib.oracle_softplus_bias.restype = ci
        self.lib.oracle_conv_silu.argtypes = [i64, i64, i64] + [_DP] * 5
        self.lib.oracle_conv_silu.restype = ci
        self.lib.oracle_conv_silu_bwd.argtypes = [i64, i64, i64] + [_DP] * 9
        self.lib.oracle_conv_silu_bwd.restype = ci
        self.lib.oracle_scan_trap.argtypes = [i64, i64, i64, i64] + [_DP] * 13 + [ci]
        self.lib.oracle_scan_trap.restype = ci
        self.lib.oracle_step_trap.argtypes = [i64, i64, i64] + [_DP] * 12 + [ci]
        self.lib.oracle_step_trap.restype = ci
        self.lib.oracle_ssd.argtypes = [i64] * 6 + [_DP] * 9 + [ci]
        self.lib.oracle_ssd.restype = ci
        self.lib.oracle_scan_bwd.argtypes = [i64] * 4 + [_DP] * 18
        self.lib.oracle_scan_bwd.restype = ci
        self.lib.oracle_softplus_grad.argtypes = [i64, i64] + [_DP] * 5
        self.lib.oracle_scan_bwd_trap.argtypes = [i64] * 4 + [_DP] * 24
        self.lib.oracle_scan_bwd_trap.restype = ci
        self.lib.oracle_softplus_grad.restype = ci

    def threads(self, nthreads: int = 0) -> int:
        return int(self.lib.oracle_threads(nthreads))

    # -- float64 entry points ------------------------------------------------
    def scan64(self, x, delta, A, Bt, Ct, Dskip=None, z=None, state_in=None,
               want_state: bool = True, nthreads: int = 0):
        """All arguments float64 arrays (see ssm_oracle.c for shapes).
        Returns (y, state_out or None)."""
        x = _c64(x)
        batch, L, D = x.shape
        A = _c64(A)
        N = A.shape[1]
        delta, Bt, Ct = _c64(delta), _c64(Bt), _c64(Ct)
        assert delta.shape == x.shape and A.shape == (D, N)
        assert Bt.shape == (batch, L, N) and Ct.shape == (batch, L, N)
        Dskip = None if Dskip is None else _c64(Dskip)
        z = None if z is None else _c64(z)
        state_in = None if state_in is None else _c64(state_in)
        if z is not None:
            assert z.shape == x.shape
        if state_in is not None:
            assert state_in.shape == (batch, D, N)
        y = np.empty((batch, L, D), dtype=np.float64)
        st = np.empty((batch, D, N), dtype=np.float64) if want_state else None
        rc = self.lib.oracle_scan(batch, L, D, N, _p(x), _p(delta), _p(A), _p(Bt), _p(Ct),
                                  _p(Dskip), _p(z), _p(state_in), _p(st), _p(y), nthreads)
        if rc != 0:
            raise ValueError("oracle_scan rejected sizes")
        return y, st

    def step64(self, x, delta, A, Bt, Ct, Dskip, z, state, nthreads: int = 0):
        """One decode step; `state` (batch, D, N) float64 is updated in place. Returns y."""
        x = _c64(x)
        batch, D = x.shape
        A = _c64(A)
        N = A.shape[1]
        assert state.dtype == np.float64 and state.flags.c_contiguous and state.shape == (batch, D, N)
        delta, Bt, Ct = _c64(delta), _c64(Bt), _c64(Ct)
        Dskip = None if Dskip is None else _c64(Dskip)
        z = None if z is None else _c64(z)
        y = np.empty((batch, D), dtype=np.float64)
        rc = self.lib.oracle_step(batch, D, N, _p(x), _p(delta), _p(A), _p(Bt), _p(Ct),
                                  _p(Dskip), _p(z), _p(state), _p(y), nthreads)
        if rc != 0:
            raise ValueError("oracle_step rejected sizes")
        return y

    def scan_trap64(self, x, delta, lam, A, Bt, Ct, Dskip=None, z=None, x_prev=None, B_prev=None,
                    state_in=None, want_state: bool = True, nthreads: int = 0):
        """Exponential-trapezoidal scan; lam has x's shape, x_prev (batch, D) and
        B_prev (batch, N) are the token before the first (None = none).
        All arrays float64. Returns (y, state_out or None)."""
        x = _c64(x)
        batch, L, D = x.shape
        A = _c64(A)
        N = A.shape[1]
        delta, lam, Bt, Ct = _c64(delta), _c64(lam), _c64(Bt), _c64(Ct)
        assert delta.shape == x.shape and lam.shape == x.shape and A.shape == (D, N)
        assert Bt.shape == (batch, L, N) and Ct.shape == (batch, L, N)
        opt = lambda a, shape: None if a is None else _c64(a).reshape(shape)
        Dskip, z = opt(Dskip, (D,)), opt(z, x.shape)
        x_prev, B_prev = opt(x_prev, (batch, D)), opt(B_prev, (batch, N))
        state_in = opt(state_in, (batch, D, N))
        y = np.empty((batch, L, D), dtype=np.float64)
        st = np.empty((batch, D, N), dtype=np.float64) if want_state else None
        rc = self.lib.oracle_scan_trap(batch, L, D, N, _p(x), _p(delta), _p(lam), _p(A), _p(Bt), _p(Ct),
                                       _p(Dskip), _p(z), _p(x_prev), _p(B_prev), _p(state_in), _p(st),
                                       _p(y), nthreads)
        if rc != 0:
            raise ValueError("oracle_scan_trap rejected sizes")
        return y, st

    def step_trap64(self, x, delta, lam, A, Bt, Ct, Dskip, z, x_prev, B_prev, state, nthreads: int = 0):
        """One exponential-trapezoidal decode step; `state` (batch, D, N) float64
        is updated in place. Returns y."""
        x = _c64(x)
        batch, D = x.shape
        A = _c64(A)
        N = A.shape[1]
        assert state.dtype == np.float64 and state.flags.c_contiguous and state.shape == (batch, D, N)
        delta, lam, Bt, Ct = _c64(delta), _c64(lam), _c64(Bt), _c64(Ct)
        assert lam.shape == x.shape
        opt = lambda a, shape: None if a is None else _c64(a).reshape(shape)
        Dskip, z = opt(Dskip, (D,)), opt(z, x.shape)
        x_prev, B_prev = opt(x_prev, (batch, D)), opt(B_prev, (batch, N))
        y = np.empty((batch, D), dtype=np.float64)
        rc = self.lib.oracle_step_trap(batch, D, N, _p(x), _p(delta), _p(lam), _p(A), _p(Bt), _p(Ct),
                                       _p(Dskip), _p(z), _p(x_prev), _p(B_prev), _p(state), _p(y), nthreads)
        if rc != 0:
            raise ValueError("oracle_step_trap rejected sizes")
        return y

    def ssd64(self, x, delta, A, Bt, Ct, Dskip=None, state_in=None, want_state: bool = True, nthreads: int = 0):
        """Mamba-2 SSD layer on float64 arrays: x (batch, L, H, P), delta (batch, L, H),
        A (H,), Bt/Ct (batch, L, G, N), Dskip (H,), state_in (batch, H, P, N).
        Returns (y, state_out or None)."""
        x = _c64(x)
        batch, L, H, P = x.shape
        Bt, Ct = _c64(Bt), _c64(Ct)
        G, N = Bt.shape[2], Bt.shape[3]
        delta, A = _c64(delta), _c64(A).reshape(H)
        assert delta.shape == (batch, L, H) and Bt.shape == (batch, L, G, N) and Ct.shape == Bt.shape
        Dskip = None if Dskip is None else _c64(Dskip).reshape(H)
        state_in = None if state_in is None else _c64(state_in).reshape(batch, H, P, N)
        y = np.empty((batch, L, H, P), dtype=np.float64)
        st = np.empty((batch, H, P, N), dtype=np.float64) if want_state else None
        rc = self.lib.oracle_ssd(batch, L, H, P, G, N, _p(x), _p(delta), _p(A), _p(Bt), _p(Ct), _p(Dskip),
                                 _p(state_in), _p(st), _p(y), nthreads)
        if rc != 0:
            raise ValueError("oracle_ssd rejected sizes")
        return y, st

    def scan_bwd64(self, x, delta, A, Bt, Ct, Dskip, z, state_in, dy, dstate=None):
        """Gradient of scan64 for the loss sum(dy * y) + sum(dstate * state_out).
        float64 arrays; returns a dict dx, ddelta, dA, dBt, dCt, dDskip (or None),
        dz (or None), dstate_in."""
        x = _c64(x)
        batch, L, D = x.shape
        A = _c64(A)
        N = A.shape[1]
        delta, Bt, Ct, dy = _c64(delta), _c64(Bt), _c64(Ct), _c64(dy)
        assert delta.shape == x.shape and dy.shape == x.shape and Bt.shape == (batch, L, N) and Ct.shape == Bt.shape
        opt = lambda a, shape: None if a is None else _c64(a).reshape(shape)
        Dskip, z = opt(Dskip, (D,)), opt(z, x.shape)
        state_in, dstate = opt(state_in, (batch, D, N)), opt(dstate, (batch, D, N))
        out = {"dx": np.empty_like(x), "ddelta": np.empty_like(x), "dA": np.empty((D, N)),
               "dBt": np.empty((batch, L, N)), "dCt": np.empty((batch, L, N)),
               "dDskip": None if Dskip is None else np.empty(D), "dz": None if z is None else np.empty_like(x),
               "dstate_in": np.empty((batch, D, N))}
        rc = self.lib.oracle_scan_bwd(batch, L, D, N, _p(x), _p(delta), _p(A), _p(Bt), _p(Ct), _p(Dskip), _p(z),
                                      _p(state_in), _p(dy), _p(dstate), _p(out["dx"]), _p(out["ddelta"]),
                                      _p(out["dA"]), _p(out["dBt"]), _p(out["dCt"]), _p(out["dDskip"]),
                                      _p(out["dz"]), _p(out["dstate_in"]))
        if rc != 0:
            raise ValueError("oracle_scan_bwd rejected sizes")
        return out

    def scan_bwd_trap64(self, x, delta, lam, A, Bt, Ct, Dskip, z, x_prev, B_prev, state_in, dy, dstate=None):
        """Gradient of scan_trap64 for the loss sum(dy * y) + sum(dstate * state_out).
        Returns scan_bwd64's dict plus dlam, and dx_prev, dB_prev (None unless
        x_prev and B_prev are given)."""
        x = _c64(x)
        batch, L, D = x.shape
        A = _c64(A)
        N = A.shape[1]
        delta, lam, Bt, Ct, dy = _c64(delta), _c64(lam), _c64(Bt), _c64(Ct), _c64(dy)
        assert delta.shape == x.shape and lam.shape == x.shape and dy.shape == x.shape
        assert Bt.shape == (batch, L, N) and Ct.shape == Bt.shape
        opt = lambda a, shape: None if a is None else _c64(a).reshape(shape)
        Dskip, z = opt(Dskip, (D,)), opt(z, x.shape)
        x_prev, B_prev = opt(x_prev, (batch, D)), opt(B_prev, (batch, N))
        state_in, dstate = opt(state_in, (batch, D, N)), opt(dstate, (batch, D, N))
        prev = x_prev is not None and B_prev is not None
        out = {"dx": np.empty_like(x), "ddelta": np.empty_like(x), "dlam": np.empty_like(x), "dA": np.empty((D, N)),
               "dBt": np.empty((batch, L, N)), "dCt": np.empty((batch, L, N)),
               "dDskip": None if Dskip is None else np.empty(D), "dz": None if z is None else np.empty_like(x),
               "dx_prev": np.empty((batch, D)) if prev else None, "dB_prev": np.empty((batch, N)) if prev else None,
               "dstate_in": np.empty((batch, D, N))}
        rc = self.lib.oracle_scan_bwd_trap(batch, L, D, N, _p(x), _p(delta), _p(lam), _p(A), _p(Bt), _p(Ct),
                                           _p(Dskip), _p(z), _p(x_prev), _p(B_prev), _p(state_in), _p(dy),
                                           _p(dstate), _p(out["dx"]), _p(out["ddelta"]), _p(out["dlam"]),
                                           _p(out["dA"]), _p(out["dBt"]), _p(out["dCt"]), _p(out["dDskip"]),
                                           _p(out["dz"]), _p(out["dx_prev"]), _p(out["dB_prev"]),
                                           _p(out["dstate_in"]))
        if rc != 0:
            raise ValueError("oracle_scan_bwd_trap rejected sizes")
        return out

    def scan_bwd_dt64(self, x, delta_raw, dt_bias, A, Bt, Ct, Dskip, z, state_in, dy, dstate=None):
        """Gradient of the scan whose step size is softplus(delta_raw + dt_bias):
        scan_bwd64 on the activated step, then the chain rule through the
        activation. Returns scan_bwd64's dict with ddelta replaced by
        ddelta_raw, plus ddt_bias (D,)."""
        d64 = self.softplus_bias64(delta_raw, dt_bias)
        out = self.scan_bwd64(x, d64, A, Bt, Ct, Dskip, z, state_in, dy, dstate)
        raw = _c64(delta_raw)
        D = raw.shape[-1]
        bias = None if dt_bias is None else _c64(dt_bias)
        g = out.pop("ddelta")
        graw, gbias = np.empty_like(raw), np.empty(D)
        if self.lib.oracle_softplus_grad(raw.size // D if D else 0, D, _p(raw), _p(bias), _p(g), _p(graw),
                                         _p(gbias)) != 0:
            raise ValueError("oracle_softplus_grad rejected sizes")
        out["ddelta_raw"], out["ddt_bias"] = graw, gbias
        return out

    def softplus_bias64(self, raw, bias=None):
        """softplus(raw + bias[d]) over the last axis (D) of a float64 array."""
        raw = _c64(raw)
        D = raw.shape[-1]
        rows = raw.size // D if D else 0
        bias = None if bias is None else _c64(bias)
        if bias is not None:
            assert bias.shape == (D,)
        out = np.empty_like(raw)
        if self.lib.oracle_softplus_bias(rows, D, _p(raw), _p(bias), _p(out)) != 0:
            raise ValueError("oracle_softplus_bias rejected sizes")
        return out

    def conv_silu64(self, x, w, cb=None, state=None):
        """The x branch ahead of the scan on float64 arrays: x (batch, L, D), taps
        w (D, 4) (tap 3 on the token itself), bias cb (D,) or None, and the raw x
        of the three tokens before token 0, state (batch, D, 3) oldest first, or
        None (zeros). Returns silu(causal depthwise convolution), (batch, L, D)."""
        x = _c64(x)
        batch, L, D = x.shape
        w = _c64(w)
        assert w.shape == (D, 4)
        cb = None if cb is None else _c64(cb)
        state = None if state is None else _c64(state)
        if cb is not None:
            assert cb.shape == (D,)
        if state is not None:
            assert state.shape == (batch, D, 3)
        out = np.empty_like(x)
        if self.lib.oracle_conv_silu(batch, L, D, _p(x), _p(w), _p(cb), _p(state), _p(out)) != 0:
            raise ValueError("oracle_conv_silu rejected sizes")
        return out

    def conv_silu_bwd64(self, x, w, cb, state, gout):
        """Gradient of conv_silu64 for a loss with d loss / d out = gout (float64
        arrays shaped as in conv_silu64). Returns dict gx (batch, L, D), gw (D, 4),
        gb (D,) and gstate (batch, D, 3)."""
        x = _c64(x)
        batch, L, D = x.shape
        w, gout = _c64(w), _c64(gout)
        cb = None if cb is None else _c64(cb)
        state = None if state is None else _c64(state)
        out = {"gx": np.empty_like(x), "gw": np.empty((D, 4)), "gb": np.empty(D), "gstate": np.empty((batch, D, 3))}
        if self.lib.oracle_conv_silu_bwd(batch, L, D, _p(x), _p(w), _p(cb), _p(state), _p(gout), _p(out["gx"]),
                                         _p(out["gw"]), _p(out["gb"]), _p(out["gstate"])) != 0:
            raise ValueError("oracle_conv_silu_bwd rejected sizes")
        return out

    # -- stored-dtype entry points -------------------------------------------
    def scan(self, inp: Dict[str, np.ndarray], dtype: str, nthreads: int = 0):
        """Scan on stored inputs (float32 arrays, or bfloat16 bit patterns as uint16).
        A, Dskip and state_in are float32. Returns float64 (y, state_out)."""
        up = lambda a: None if a is None else upcast(a, dtype)
        return self.scan64(up(inp["x"]), up(inp["delta"]), upcast(inp["A"], "f32"), up(inp["Bt"]),
                           up(inp["Ct"]), None if inp.get("Dskip") is None else upcast(inp["Dskip"], "f32"),
                           up(inp.get("z")),
                           None if inp.get("state_in") is None else upcast(inp["state_in"], "f32"),
                           nthreads=nthreads)

    def scan_dt(self, inp: Dict[str, np.ndarray], dtype: str, nthreads: int = 0):
        """Scan whose step size is given before its activation: inp["delta_raw"]
        (stored dtype) and inp["dt_bias"] (D,) float32 or None."""
        bias = None if inp.get("dt_bias") is None else upcast(inp["dt_bias"], "f32")
        d64 = self.softplus_bias64(upcast(inp["delta_raw"], dtype), bias)
        up = lambda a: None if a is None else upcast(a, dtype)
        return self.scan64(up(inp["x"]), d64, upcast(inp["A"], "f32"), up(inp["Bt"]),
                           up(inp["Ct"]), None if inp.get("Dskip") is None else upcast(inp["Dskip"], "f32"),
                           up(inp.get("z")),
                           None if inp.get("state_in") is None else upcast(inp["state_in"], "f32"),
                           nthreads=nthreads)

    def scan_conv(self, inp: Dict[str, np.ndarray], dtype: str, nthreads: int = 0):
        """Scan behind the Mamba block's x branch: inp["x_raw"] (stored dtype)
        goes through the causal convolution (inp["conv_w"] (D, 4), inp["conv_b"]
        (D,) or None, float32) and SiLU, with inp["conv_state"] (batch, D, 3,
        stored dtype) or None before token 0; the step size is given before its
        activation, as in scan_dt."""
        f32 = lambda a: None if a is None else upcast(a, "f32")
        up = lambda a: None if a is None else upcast(a, dtype)
        x64 = self.conv_silu64(upcast(inp["x_raw"], dtype), f32(inp["conv_w"]), f32(inp.get("conv_b")),
                               up(inp.get("conv_state")))
        d64 = self.softplus_bias64(upcast(inp["delta_raw"], dtype), f32(inp.get("dt_bias")))
        return self.scan64(x64, d64, upcast(inp["A"], "f32"), up(inp["Bt"]), up(inp["Ct"]), f32(inp.get("Dskip")),
                           up(inp.get("z")), f32(inp.get("state_in")), nthreads=nthreads)

    def step_dt(self, tok: Dict[str, np.ndarray], A, Dskip, dt_bias, state64: np.ndarray, dtype: str,
                nthreads: int = 0):
        """Decode step with tok["delta_raw"] and dt_bias (D,) float32 or None."""
        bias = None if dt_bias is None else upcast(dt_bias, "f32")
        d64 = self.softplus_bias64(upcast(tok["delta_raw"], dtype), bias)
        up = lambda a: None if a is None else upcast(a, dtype)
        return self.step64(up(tok["x"]), d64, upcast(A, "f32"), up(tok["Bt"]),
                           up(tok["Ct"]), None if Dskip is None else upcast(Dskip, "f32"),
                           up(tok.get("z")), state64, nthreads=nthreads)

    def step_conv(self, tok: Dict[str, np.ndarray], A, Dskip, dt_bias, conv_w, conv_b, window64: np.ndarray,
                  state64: np.ndarray, dtype: str, nthreads: int = 0):
        """Decode step behind the x branch: tok["x"] is the token's raw x,
        window64 (batch, D, 3) float64 the raw x of the three tokens before it
        (oldest first). x is the branch's convolution and SiLU (conv_silu64 over
        that one token); window64 is shifted in place to end with this token's
        raw x; the step runs as step_dt."""
        f32 = lambda a: None if a is None else upcast(a, "f32")
        raw = upcast(tok["x"], dtype)
        x64 = self.conv_silu64(raw[:, None, :], f32(conv_w), f32(conv_b), window64)[:, 0, :]
        window64[:, :, :2] = window64[:, :, 1:].copy()
        window64[:, :, 2] = raw
        bias = None if dt_bias is None else upcast(dt_bias, "f32")
        d64 = self.softplus_bias64(upcast(tok["delta_raw"], dtype), bias)
        up = lambda a: None if a is None else upcast(a, dtype)
        return self.step64(x64, d64, upcast(A, "f32"), up(tok["Bt"]), up(tok["Ct"]), f32(Dskip), up(tok.get("z")),
                           state64, nthreads=nthreads)

    def scan_trap(self, inp: Dict[str, np.ndarray], dtype: str, nthreads: int = 0):
        """Exponential-trapezoidal scan on stored inputs: inp["lam"] (stored dtype)
        and optional inp["x_prev"], inp["B_prev"] (stored dtype)."""
        up = lambda a: None if a is None else upcast(a, dtype)
        return self.scan_trap64(up(inp["x"]), up(inp["delta"]), up(inp["lam"]), upcast(inp["A"], "f32"),
                                up(inp["Bt"]), up(inp["Ct"]),
                                None if inp.get("Dskip") is None else upcast(inp["Dskip"], "f32"),
                                up(inp.get("z")), up(inp.get("x_prev")), up(inp.get("B_prev")),
                                None if inp.get("state_in") is None else upcast(inp["state_in"], "f32"),
                                nthreads=nthreads)

    def step_trap(self, tok: Dict[str, np.ndarray], A, Dskip, state64: np.ndarray, dtype: str,
                  nthreads: int = 0):
        """Exponential-trapezoidal decode step: tok["lam"], tok["x_prev"], tok["B_prev"]."""
        up = lambda a: None if a is None else upcast(a, dtype)
        return self.step_trap64(up(tok["x"]), up(tok["delta"]), up(tok["lam"]), upcast(A, "f32"), up(tok["Bt"]),
                                up(tok["Ct"]), None if Dskip is None else upcast(Dskip, "f32"),
                                up(tok.get("z")), up(tok.get("x_prev")), up(tok.get("B_prev")), state64,
                                nthreads=nthreads)

    def ssd(self, inp: Dict[str, np.ndarray], dtype: str, nthreads: int = 0):
        """SSD layer on stored inputs (x, delta, Bt, Ct in the stored dtype; A,
        Dskip, state_in float32)."""
        up = lambda a: None if a is None else upcast(a, dtype)
        f32 = lambda a: None if a is None else upcast(a, "f32")
        return self.ssd64(up(inp["x"]), up(inp["delta"]), f32(inp["A"]), up(inp["Bt"]), up(inp["Ct"]),
                          f32(inp.get("Dskip")), f32(inp.get("state_in")), nthreads=nthreads)

    def scan_bwd(self, inp: Dict[str, np.ndarray], dy, dstate, dtype: str):
        """Gradient of the scan on stored inputs; dy in the stored dtype, dstate float32 or None."""
        up = lambda a: None if a is None else upcast(a, dtype)
        f32 = lambda a: None if a is None else upcast(a, "f32")
        return self.scan_bwd64(up(inp["x"]), up(inp["delta"]), f32(inp["A"]), up(inp["Bt"]), up(inp["Ct"]),
                               f32(inp.get("Dskip")), up(inp.get("z")), f32(inp.get("state_in")), up(dy), f32(dstate))

    def scan_bwd_trap(self, inp: Dict[str, np.ndarray], dy, dstate, dtype: str):
        """scan_bwd_trap64 on stored inputs (lam, x_prev, B_prev in the stored dtype)."""
        up = lambda a: None if a is None else upcast(a, dtype)
        f32 = lambda a: None if a is None else upcast(a, "f32")
        return self.scan_bwd_trap64(up(inp["x"]), up(inp["delta"]), up(inp["lam"]), f32(inp["A"]), up(inp["Bt"]),
                                    up(inp["Ct"]), f32(inp.get("Dskip")), up(inp.get("z")), up(inp.get("x_prev")),
                                    up(inp.get("B_prev")), f32(inp.get("state_in")), up(dy), f32(dstate))

    def scan_bwd_conv(self, inp: Dict[str, np.ndarray], dy, dstate, dtype: str):
        """Gradient of scan_conv: the scan's gradient on the branch's output x
        (with the step size before its activation), then back through SiLU and
        the convolution. Keys as scan_bwd_dt's with dx replaced by dx_raw, plus
        dconv_w, dconv_b and dconv_state."""
        f32 = lambda a: None if a is None else upcast(a, "f32")
        up = lambda a: None if a is None else upcast(a, dtype)
        xr, w, cb, cs = up(inp["x_raw"]), f32(inp["conv_w"]), f32(inp.get("conv_b")), up(inp.get("conv_state"))
        x64 = self.conv_silu64(xr, w, cb, cs)
        g = self.scan_bwd_dt64(x64, up(inp["delta_raw"]), f32(inp.get("dt_bias")), f32(inp["A"]), up(inp["Bt"]),
                               up(inp["Ct"]), f32(inp.get("Dskip")), up(inp.get("z")), f32(inp.get("state_in")),
                               upcast(dy, dtype), None if dstate is None else upcast(dstate, "f32"))
        c = self.conv_silu_bwd64(xr, w, cb, cs, g.pop("dx"))
        g["dx_raw"], g["dconv_w"], g["dconv_b"], g["dconv_state"] = c["gx"], c["gw"], c["gb"], c["gstate"]
        return g

    def scan_bwd_dt(self, inp: Dict[str, np.ndarray], dy, dstate, dtype: str):
        """scan_bwd64_dt on stored inputs (delta_raw in the stored dtype, dt_bias float32 or None)."""
        up = lambda a: None if a is None else upcast(a, dtype)
        f32 = lambda a: None if a is None else upcast(a, "f32")
        return self.scan_bwd_dt64(up(inp["x"]), up(inp["delta_raw"]), f32(inp.get("dt_bias")), f32(inp["A"]),
                                  up(inp["Bt"]), up(inp["Ct"]), f32(inp.get("Dskip")), up(inp.get("z")),
                                  f32(inp.get("state_in")), up(dy), f32(dstate))

    def step(self, tok: Dict[str, np.ndarray], A, Dskip, state64: np.ndarray, dtype: str,
             nthreads: int = 0):
        up = lambda a: None if a is None else upcast(a, dtype)
        return self.step64(up(tok["x"]), up(tok["delta"]), upcast(A, "f32"), up(tok["Bt"]),
                           up(tok["Ct"]), None if Dskip is None else upcast(Dskip, "f32"),
                           up(tok.get("z")), state64, nthreads=nthreads)


class ErrorSum:
    """Relative L2 and max-abs error of a large output accumulated piece by
    piece (sums of squares in float64), so that neither the whole reference
    nor the whole device result needs to be held at once. A non-finite value
    in the device result makes the relative error NaN."""

    def __init__(self):
        self.dd = 0.0
        self.rr = 0.0
        self.maxabs = 0.0
        self.count = 0

    def add(self, got: np.ndarray, ref: np.ndarray) -> None:
        d = (np.asarray(got, dtype=np.float64) - ref).ravel()
        r = np.asarray(ref, dtype=np.float64).ravel()
        self.dd += float(np.dot(d, d))
        self.rr += float(np.dot(r, r))
        if d.size:
            self.maxabs = max(self.maxabs, float(np.max(np.abs(d))))
        self.count += r.size

    @property
    def rel(self) -> float:
        return float(np.sqrt(self.dd) / (np.sqrt(self.rr) if self.rr > 0 else 1.0))


def scan_compare(blocks, dtype: str, nthreads: int = 0, rule: str = "scan"):
    """Compare a scan computed elsewhere with the oracle, block by block.
    `blocks` yields (inp, y_got, state_got): `inp` the stored inputs of a part
    of the workload that the oracle can run alone (some batch rows and channels
    over the whole sequence, as Oracle.scan takes them), y_got and state_got
    float64 (state_got None to skip it). `rule` names the oracle function:
    "scan", "scan_dt" (step size before its activation), "scan_conv" (also x
    before the block's convolution and SiLU) or "scan_trap".
    Returns (ErrorSum of y, ErrorSum of the state, seconds spent in the
    oracle)."""
    o = get()
    fn = {"scan": o.scan, "scan_dt": o.scan_dt, "scan_conv": o.scan_conv, "scan_trap": o.scan_trap}[rule]
    ey, es, secs = ErrorSum(), ErrorSum(), 0.0
    for inp, y_got, st_got in blocks:
        t = time.perf_counter()
        yr, sr = fn(inp, dtype, nthreads=nthreads)
        secs += time.perf_counter() - t
        ey.add(y_got, yr)
        if st_got is not None:
            es.add(st_got, sr)
    return ey, es, secs


def upcast(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array: float32, or bfloat16 bits (uint16)."""
    if dtype == "f32" or a.dtype == np.float32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return (np.asarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def _c64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.cast(None, _DP)
    return a.ctypes.data_as(_DP)


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from ``ssm_oracle.c`` (compiled on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def timed_scan(inp, dtype, nthreads: int = 0):
    """Run the scan and return (y, state_out, seconds, threads_used)."""
    o = get()
    t = time.perf_counter()
    y, st = o.scan(inp, dtype, nthreads)
    return y, st, time.perf_counter() - t, o.threads(nthreads)
