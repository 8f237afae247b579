"""Seeded synthetic inputs for the selective scan (S6) and its decode step.

This module is shared by the tests, the bench and the oracle checks. It only
draws random numbers and stores them in the storage dtypes; it holds none of
the scan's arithmetic. Every tensor is drawn in float64 and stored once in its
storage dtype: float32 (round to nearest even) or bfloat16 (float64 -> float32
-> bfloat16, each round to nearest even). bfloat16 arrays are numpy ``uint16``
arrays that hold the raw bit patterns.

Shapes (D fastest everywhere):
  x, delta, z, y : (batch, L, D)       activation dtype
  A              : (D, N)              float32
  Bt, Ct         : (batch, L, N)       activation dtype
  Dskip          : (D,)                float32
  state          : (batch, D, N)       float32

Distributions follow the workloads described for the Mamba selective scan
(Mamba notes, "O mecanismo de seleção (S6)"; Mamba encyclopedia entry,
"como funciona"): A = -exp(A_log) with the S4D-real choice A[d, n] = -(n+1);
delta = softplus(0.5*eps + dt_bias) where dt_bias is the inverse softplus of a
per-channel dt drawn log-uniform in [1e-3, 1e-1]; x, z, Bt, Ct ~ N(0, 1);
Dskip = 1 or U(0.5, 1.5). delta is handed to the scan after the softplus.
For the Mamba-2 SSD layer (x (batch, L, H, P), Bt/Ct (batch, L, G, N)): A_h =
-U(1, 16) per head, delta = softplus(0.5*eps + dt_bias) with dt_bias per head
as above, x, Bt, Ct ~ N(0, 1), Dskip ~ U(0.5, 1.5), bfloat16 activations.
For the exponential-trapezoidal rule ("Recorrência trapezoidal"), the weight
lam = sigmoid(u) with u ~ N(0, 1) per (b, t, d) (the sigmoid of a per-token
projection), and the token before the first, x_prev and B_prev, ~ N(0, 1).
For the x branch ahead of the scan ("O bloco Mamba": a short depthwise causal
convolution of width 4, then SiLU), x_raw is the N(0, 1) draw that x is
otherwise, and the taps (D, 4) and bias (D,) are U(-0.5, 0.5), float32 (the
pages give no initialisation; this is PyTorch's default for a depthwise
Conv1d of width 4, bound 1/sqrt(4)); the raw x of the three tokens before
token 0 ~ N(0, 1).

Random streams: ``numpy.random.default_rng(SeedSequence(seed, spawn_key=key))``
with one key per (tensor kind, batch row, token chunk of 65536, block of 64
channels). Generation is therefore chunked and restartable: any token range
or channel subset can be regenerated without the rest of the tensor.

``fill_scan_device`` / ``fill_step_device`` draw tensors of the same
distributions with torch on the GPU; they fill the channels of very large
workloads that a test computes but does not compare, so that only the
compared channels need the (slower) numpy streams.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "fill_scan_device", "fill_step_device", "ScanConfig", "StepConfig", "SCAN_CONFIGS", "STEP_CONFIG", "DTYPES",
    "scan_inputs", "step_inputs", "step_token_inputs", "bf16_bits_from_f64",
    "storage_to_f64", "scan_bytes", "step_bytes", "trap_extra_bytes", "trap_step_extra_bytes",
    "SsdConfig", "SSD_CONFIGS", "ssd_inputs", "fill_ssd_device", "ssd_bytes", "grad_inputs", "scan_bwd_bytes", "ssd_step_bytes",
]

DTYPES = ("f32", "bf16")
_CHUNK = 65536  # tokens per random stream
_CBLK = 64      # channels per random stream

# stream keys (tensor kinds)
_K_DT, _K_DNOISE, _K_X, _K_Z, _K_B, _K_C, _K_D, _K_STATE, _K_LAM, _K_XPREV, _K_BPREV, _K_AH, _K_DY, _K_DSTATE = \
    range(14)
_K_CONVW, _K_CONVB, _K_CONVSTATE = range(14, 17)


@dataclasses.dataclass(frozen=True)
class ScanConfig:
    """One selective-scan workload: sizes, dtype and which optional parts are on."""
    name: str
    batch: int
    L: int
    D: int
    N: int = 16
    dtype: str = "f32"          # activation dtype of x, delta, z, Bt, Ct, y
    gate: bool = True           # silu(z) gate on
    dskip: str = "uniform"      # "one", "uniform" or "none"
    state_in: Optional[float] = None  # std of the carried-in state, None = zero state
    seed: int = 0

    @property
    def elems(self) -> int:
        return self.batch * self.L * self.D * self.N


@dataclasses.dataclass(frozen=True)
class StepConfig:
    """A decode workload: `steps` consecutive single-token updates of a batch of states."""
    name: str
    batch: int
    D: int
    N: int = 16
    dtype: str = "bf16"
    gate: bool = True
    dskip: str = "uniform"
    state_std: float = 1.0
    steps: int = 1000
    seed: int = 4

    @property
    def elems_per_step(self) -> int:
        return self.batch * self.D * self.N


@dataclasses.dataclass(frozen=True)
class SsdConfig:
    """A Mamba-2 SSD workload: x (batch, L, H, P), Bt/Ct (batch, L, G, N)."""
    name: str
    batch: int
    L: int
    H: int
    P: int = 64
    G: int = 1
    N: int = 128
    dtype: str = "bf16"
    dskip: bool = True
    state_in: Optional[float] = None
    seed: int = 5

    @property
    def elems(self) -> int:
        """State updates per launch: batch * L * H * P * N."""
        return self.batch * self.L * self.H * self.P * self.N


# A Mamba-2 layer with 5120 inner channels as 80 heads of 64, state size 128
# (the pages: the SSD state can grow from 16 to 64, 128 or 256), one group.
SSD_CONFIGS: Dict[str, SsdConfig] = {
    "ssd": SsdConfig("ssd_mamba2_layer_bf16", 8, 4096, 80, 64, 1, 128, "bf16", dskip=True, seed=5),
    # decode: 256 sequences, one token per step, the same layer's heads and state
    "ssd_step": SsdConfig("ssd_decode_step_bf16", 256, 1000, 80, 64, 1, 128, "bf16", dskip=True, state_in=1.0,
                          seed=6),
}


# The five workloads, in order: tiny fp32; small-model layer fp32; large-model
# layer bf16; million-token context bf16 with a carried-in state; decode step.
SCAN_CONFIGS: Dict[str, ScanConfig] = {
    "c0": ScanConfig("c0_tiny_f32", 1, 256, 64, 16, "f32", gate=False, dskip="one", seed=0),
    "c1": ScanConfig("c1_small_layer_f32", 2, 2048, 1536, 16, "f32", gate=True, dskip="uniform", seed=1),
    "c2": ScanConfig("c2_large_layer_bf16", 8, 4096, 5120, 16, "bf16", gate=True, dskip="uniform", seed=2),
    "c3": ScanConfig("c3_million_token_bf16", 1, 1048576, 1536, 16, "bf16", gate=True, dskip="uniform",
                     state_in=0.1, seed=3),
}
STEP_CONFIG = StepConfig("c4_decode_step_bf16", 256, 5120, 16, "bf16", gate=True, dskip="uniform",
                         state_std=1.0, steps=1000, seed=4)


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(int(k) for k in key)))


def bf16_bits_from_f64(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bfloat16 (RNE), returned as uint16 bit patterns."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of a stored tensor (float32, or bfloat16 bits) to float64."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def _store(a64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return a64.astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f64(a64)
    raise ValueError(dtype)


def _softplus(u: np.ndarray) -> np.ndarray:
    return np.maximum(u, 0.0) + np.log1p(np.exp(-np.abs(u)))


def _channel_params(seed: int, D: int, N: int, dskip: str):
    """A (D, N) float32, dt_bias (D,) float64, Dskip (D,) float32 or None."""
    A = np.broadcast_to(-(np.arange(N, dtype=np.float64) + 1.0), (D, N)).astype(np.float32).copy()
    dt = np.exp(_rng(seed, _K_DT).uniform(math.log(1e-3), math.log(1e-1), size=D))
    dt_bias = dt + np.log(-np.expm1(-dt))  # inverse softplus
    if dskip == "one":
        Dskip = np.ones(D, dtype=np.float32)
    elif dskip == "uniform":
        Dskip = _rng(seed, _K_D).uniform(0.5, 1.5, size=D).astype(np.float32)
    elif dskip == "none":
        Dskip = None
    else:
        raise ValueError(dskip)
    return A, dt_bias, Dskip


def _token_block(seed: int, kind: int, b: int, t0: int, t1: int, width: int,
                 cols: Optional[np.ndarray] = None) -> np.ndarray:
    """N(0,1) float64 block of shape (t1-t0, len(cols)) from the per-(chunk,
    channel block) streams; `cols` defaults to all `width` columns."""
    cols = np.arange(width) if cols is None else np.asarray(cols)
    out = np.empty((t1 - t0, len(cols)), dtype=np.float64)
    if t1 == t0 or len(cols) == 0:
        return out
    blocks = np.unique(cols // _CBLK)
    for c in range(t0 // _CHUNK, (t1 - 1) // _CHUNK + 1):
        cs = c * _CHUNK
        lo, hi = max(t0, cs), min(t1, cs + _CHUNK)
        for blk in blocks:
            w = min(_CBLK, width - blk * _CBLK)
            # A stream's draws are a fixed sequence: drawing the first (hi - cs)
            # rows gives the same rows as drawing the whole chunk.
            block = _rng(seed, kind, b, c, blk).standard_normal((hi - cs, w))
            sel = np.nonzero(cols // _CBLK == blk)[0]
            out[lo - t0:hi - t0, sel] = block[lo - cs:, cols[sel] - blk * _CBLK]
    return out


def _sigmoid(u: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * u))


def scan_inputs(cfg: ScanConfig, t0: int = 0, t1: Optional[int] = None,
                channels: Optional[np.ndarray] = None, raw_delta: bool = False,
                trap: bool = False, conv: bool = False) -> Dict[str, np.ndarray]:
    """Inputs of `cfg` for tokens [t0, t1) (default: all), in storage dtypes.

    `channels` selects a subset of the D channels for x, delta, z, A and Dskip
    (used to check sampled channels of very large workloads); Bt and Ct are
    shared by all channels and always returned whole. state_in is returned
    for every batch row and the selected channels when the workload has one.
    The values do not depend on how the token range is split.

    With raw_delta, the step size is also returned before its activation:
    delta_raw = 0.5*eps in the storage dtype and dt_bias (D,) float32, the two
    terms whose softplus is delta.

    With trap, also the exponential-trapezoidal inputs: lam (batch, T, D) and
    the token before t0, x_prev (batch, D) and B_prev (batch, N): token t0 - 1
    of x and Bt when t0 > 0, else draws of their own (the last token of an
    earlier piece of the sequence).

    With conv, also the x branch's inputs: x_raw (the same array as x, taken
    as the convolution's input), conv_w (D, 4) and conv_b (D,) float32, and
    conv_state (batch, D, 3) in the storage dtype, the raw x of tokens t0 - 3
    .. t0 - 1, oldest first (draws of their own before token 0).
    """
    if t1 is None:
        t1 = cfg.L
    assert 0 <= t0 <= t1 <= cfg.L
    A, dt_bias, Dskip = _channel_params(cfg.seed, cfg.D, cfg.N, cfg.dskip)
    sel = np.arange(cfg.D) if channels is None else np.asarray(channels)
    T = t1 - t0
    act = cfg.dtype
    x = np.empty((cfg.batch, T, len(sel)), dtype=np.float32 if act == "f32" else np.uint16)
    dl = np.empty_like(x)
    z = np.empty_like(x) if cfg.gate else None
    Bt = np.empty((cfg.batch, T, cfg.N), dtype=x.dtype)
    Ct = np.empty_like(Bt)
    draw = np.empty_like(x) if raw_delta else None
    for b in range(cfg.batch):
        eps = _token_block(cfg.seed, _K_DNOISE, b, t0, t1, cfg.D, sel)
        dl[b] = _store(_softplus(0.5 * eps + dt_bias[sel][None, :]), act)
        if draw is not None:
            draw[b] = _store(0.5 * eps, act)
        x[b] = _store(_token_block(cfg.seed, _K_X, b, t0, t1, cfg.D, sel), act)
        if z is not None:
            z[b] = _store(_token_block(cfg.seed, _K_Z, b, t0, t1, cfg.D, sel), act)
        Bt[b] = _store(_token_block(cfg.seed, _K_B, b, t0, t1, cfg.N), act)
        Ct[b] = _store(_token_block(cfg.seed, _K_C, b, t0, t1, cfg.N), act)
    out = {"x": x, "delta": dl, "z": z, "A": np.ascontiguousarray(A[sel]), "Bt": Bt, "Ct": Ct,
           "Dskip": None if Dskip is None else np.ascontiguousarray(Dskip[sel]), "state_in": None}
    if cfg.state_in is not None:
        st = _rng(cfg.seed, _K_STATE).standard_normal((cfg.batch, cfg.D, cfg.N)) * cfg.state_in
        out["state_in"] = np.ascontiguousarray(st[:, sel, :].astype(np.float32))
    if draw is not None:
        out["delta_raw"] = draw
        out["dt_bias"] = np.ascontiguousarray(dt_bias[sel].astype(np.float32))
    if trap:
        lam = np.empty_like(x)
        xp = np.empty((cfg.batch, len(sel)), dtype=x.dtype)
        bp = np.empty((cfg.batch, cfg.N), dtype=x.dtype)
        for b in range(cfg.batch):
            lam[b] = _store(_sigmoid(_token_block(cfg.seed, _K_LAM, b, t0, t1, cfg.D, sel)), act)
            if t0 > 0:
                xp[b] = _store(_token_block(cfg.seed, _K_X, b, t0 - 1, t0, cfg.D, sel)[0], act)
                bp[b] = _store(_token_block(cfg.seed, _K_B, b, t0 - 1, t0, cfg.N)[0], act)
            else:
                xp[b] = _store(_token_block(cfg.seed, _K_XPREV, b, 0, 1, cfg.D, sel)[0], act)
                bp[b] = _store(_token_block(cfg.seed, _K_BPREV, b, 0, 1, cfg.N)[0], act)
        out["lam"], out["x_prev"], out["B_prev"] = lam, xp, bp
    if conv:
        w = _rng(cfg.seed, _K_CONVW).uniform(-0.5, 0.5, size=(cfg.D, 4))
        cb = _rng(cfg.seed, _K_CONVB).uniform(-0.5, 0.5, size=cfg.D)
        cs = np.empty((cfg.batch, len(sel), 3), dtype=x.dtype)
        for b in range(cfg.batch):
            before = _token_block(cfg.seed, _K_CONVSTATE, b, 0, 3, cfg.D, sel)  # tokens -3 .. -1
            for j in range(3):
                s_tok = t0 - 3 + j
                if s_tok >= 0:
                    cs[b, :, j] = _store(_token_block(cfg.seed, _K_X, b, s_tok, s_tok + 1, cfg.D, sel)[0], act)
                else:
                    cs[b, :, j] = _store(before[s_tok + 3], act)
        out["x_raw"] = x
        out["conv_w"] = np.ascontiguousarray(w[sel].astype(np.float32))
        out["conv_b"] = np.ascontiguousarray(cb[sel].astype(np.float32))
        out["conv_state"] = cs
    return out


def grad_inputs(cfg: ScanConfig, t0: int = 0, t1: Optional[int] = None, channels: Optional[np.ndarray] = None,
                dstate: bool = True) -> Dict[str, np.ndarray]:
    """Upstream gradients for the scan of `cfg` over tokens [t0, t1): dy
    (batch, T, D) N(0,1) in the storage dtype, and dstate (batch, D, N) N(0,1)
    float32 (None unless `dstate`). Channel selection as in scan_inputs."""
    if t1 is None:
        t1 = cfg.L
    sel = np.arange(cfg.D) if channels is None else np.asarray(channels)
    dy = np.empty((cfg.batch, t1 - t0, len(sel)), dtype=np.float32 if cfg.dtype == "f32" else np.uint16)
    for b in range(cfg.batch):
        dy[b] = _store(_token_block(cfg.seed, _K_DY, b, t0, t1, cfg.D, sel), cfg.dtype)
    out = {"dy": dy, "dstate": None}
    if dstate:
        st = _rng(cfg.seed, _K_DSTATE).standard_normal((cfg.batch, cfg.D, cfg.N))
        out["dstate"] = np.ascontiguousarray(st[:, sel, :].astype(np.float32))
    return out


def step_inputs(cfg: StepConfig, channels: Optional[np.ndarray] = None, conv: bool = False) -> Dict[str, np.ndarray]:
    """Per-workload tensors of a decode run: A, Dskip, dt_bias (float32) and
    the initial state; with conv also the x branch's taps conv_w (D, 4) and
    bias conv_b (D,) (float32) and its initial window conv_state (batch, D, 3)
    in the storage dtype, drawn as in scan_inputs."""
    A, dt_bias, Dskip = _channel_params(cfg.seed, cfg.D, cfg.N, cfg.dskip)
    sel = np.arange(cfg.D) if channels is None else np.asarray(channels)
    st = _rng(cfg.seed, _K_STATE).standard_normal((cfg.batch, cfg.D, cfg.N)) * cfg.state_std
    out = {"A": np.ascontiguousarray(A[sel]),
           "Dskip": None if Dskip is None else np.ascontiguousarray(Dskip[sel]),
           "dt_bias": np.ascontiguousarray(dt_bias[sel].astype(np.float32)),
           "state": np.ascontiguousarray(st[:, sel, :].astype(np.float32))}
    if conv:
        w = _rng(cfg.seed, _K_CONVW).uniform(-0.5, 0.5, size=(cfg.D, 4))
        cb = _rng(cfg.seed, _K_CONVB).uniform(-0.5, 0.5, size=cfg.D)
        cs = _rng(cfg.seed, _K_CONVSTATE).standard_normal((cfg.batch, cfg.D, 3))
        out["conv_w"] = np.ascontiguousarray(w[sel].astype(np.float32))
        out["conv_b"] = np.ascontiguousarray(cb[sel].astype(np.float32))
        out["conv_state"] = np.ascontiguousarray(_store(cs[:, sel, :], cfg.dtype))
    return out


def step_token_inputs(cfg: StepConfig, step: int, channels: Optional[np.ndarray] = None,
                      raw_delta: bool = False, trap: bool = False) -> Dict[str, np.ndarray]:
    """Inputs of decode step `step`: x, delta, z (batch, D) and Bt, Ct (batch, N);
    with raw_delta also delta_raw = 0.5*eps (delta is its softplus plus dt_bias);
    with trap also lam (batch, D) (the previous token's x and Bt are those of
    step - 1)."""
    _A, dt_bias, _D = _channel_params(cfg.seed, cfg.D, cfg.N, cfg.dskip)
    sel = np.arange(cfg.D) if channels is None else np.asarray(channels)
    act = cfg.dtype
    key = 1000 + step  # step s draws "batch row" 1000+s, one token per sequence

    def chan(kind):  # (batch, len(sel)): the batch axis plays the token axis
        return _token_block(cfg.seed, kind, key, 0, cfg.batch, cfg.D, sel)

    eps = chan(_K_DNOISE)
    out = {
        "delta": _store(_softplus(0.5 * eps + dt_bias[sel][None, :]), act),
        "x": _store(chan(_K_X), act),
        "z": _store(chan(_K_Z), act) if cfg.gate else None,
        "Bt": _store(_token_block(cfg.seed, _K_B, key, 0, cfg.batch, cfg.N), act),
        "Ct": _store(_token_block(cfg.seed, _K_C, key, 0, cfg.batch, cfg.N), act),
    }
    if raw_delta:
        out["delta_raw"] = _store(0.5 * eps, act)
    if trap:
        out["lam"] = _store(_sigmoid(chan(_K_LAM)), act)
    return out


def fill_scan_device(cfg: ScanConfig, device, seed: int = 12345, raw_delta: bool = False, trap: bool = False):
    """torch tensors of the full workload `cfg` on `device`, same distributions
    as scan_inputs but drawn with torch (values differ from the numpy streams).
    Returns x, delta, z (or None) and Bt, Ct; A, Dskip and state_in come from
    scan_inputs(cfg, 0, 0)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    act = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    _A, dt_bias, _D = _channel_params(cfg.seed, cfg.D, cfg.N, cfg.dskip)
    bias = torch.tensor(dt_bias, dtype=torch.float32, device=device)
    shape = (cfg.batch, cfg.L, cfg.D)

    def normal(shp):
        return torch.randn(shp, generator=g, device=device, dtype=torch.float32)

    eps = normal(shape).mul_(0.5)
    if raw_delta:  # delta before its activation, and the bias
        delta, extra = eps.to(act), {"delta_raw": None, "dt_bias": bias}
    else:
        delta, extra = torch.nn.functional.softplus(eps.add_(bias)).to(act), {}
    del eps
    out = {"delta": delta, "x": normal(shape).to(act),
           "z": normal(shape).to(act) if cfg.gate else None,
           "Bt": normal((cfg.batch, cfg.L, cfg.N)).to(act), "Ct": normal((cfg.batch, cfg.L, cfg.N)).to(act)}
    if raw_delta:
        out["delta_raw"], out["dt_bias"] = out.pop("delta"), extra["dt_bias"]
    if trap:  # lam = sigmoid(N(0,1)) and the token before the first
        out["lam"] = torch.sigmoid(normal(shape)).to(act)
        out["x_prev"] = normal((cfg.batch, cfg.D)).to(act)
        out["B_prev"] = normal((cfg.batch, cfg.N)).to(act)
    return out


def fill_step_device(cfg: StepConfig, steps: int, device, seed: int = 54321, raw_delta: bool = False,
                     trap: bool = False):
    """torch tensors for `steps` decode steps on `device` (same distributions as
    step_token_inputs, drawn with torch): x, delta, z of shape (steps, batch, D)
    and Bt, Ct of shape (steps, batch, N)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    act = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    _A, dt_bias, _D = _channel_params(cfg.seed, cfg.D, cfg.N, cfg.dskip)
    bias = torch.tensor(dt_bias, dtype=torch.float32, device=device)
    shape = (steps, cfg.batch, cfg.D)

    def normal(shp):
        return torch.randn(shp, generator=g, device=device, dtype=torch.float32)

    eps = normal(shape).mul_(0.5)
    if raw_delta:  # delta before its activation; the bias is step_inputs' dt_bias
        return {"delta_raw": eps.to(act), "x": normal(shape).to(act),
                "z": normal(shape).to(act) if cfg.gate else None,
                "Bt": normal((steps, cfg.batch, cfg.N)).to(act), "Ct": normal((steps, cfg.batch, cfg.N)).to(act)}
    delta = torch.nn.functional.softplus(eps.add_(bias)).to(act)
    del eps
    out = {"delta": delta, "x": normal(shape).to(act), "z": normal(shape).to(act) if cfg.gate else None,
           "Bt": normal((steps, cfg.batch, cfg.N)).to(act), "Ct": normal((steps, cfg.batch, cfg.N)).to(act)}
    if trap:
        out["lam"] = torch.sigmoid(normal(shape)).to(act)
    return out


def _esize(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def scan_bytes(cfg: ScanConfig, state_out: bool = False) -> int:
    """Bytes the scan must move: x, delta, (z) read and y written once per (b,t,d);
    Bt, Ct once per token; A, Dskip once; state_in / state_out when used.
    The (batch, L, D, N) expanded state is never counted: it is never stored."""
    e = _esize(cfg.dtype)
    btd = cfg.batch * cfg.L * cfg.D
    n = btd * e * (3 + (1 if cfg.gate else 0))
    n += 2 * cfg.batch * cfg.L * cfg.N * e
    n += cfg.D * cfg.N * 4 + (cfg.D * 4 if cfg.dskip != "none" else 0)
    if cfg.state_in is not None:
        n += cfg.batch * cfg.D * cfg.N * 4
    if state_out:
        n += cfg.batch * cfg.D * cfg.N * 4
    return n


def scan_bwd_bytes(cfg: ScanConfig) -> int:
    """Bytes the gradient must move: x, delta, dy, (z) read and dx, ddelta, (dz)
    written once per (b,t,d); Bt, Ct read and dBt, dCt (float32) written once
    per token; A, Dskip read and dA, dDskip written once; state_in (when used),
    dstate and dstate_in once."""
    e = _esize(cfg.dtype)
    btd = cfg.batch * cfg.L * cfg.D
    n = btd * e * (5 + (2 if cfg.gate else 0))
    n += cfg.batch * cfg.L * cfg.N * (2 * e + 2 * 4)
    n += 2 * (cfg.D * cfg.N * 4 + (cfg.D * 4 if cfg.dskip != "none" else 0))
    n += cfg.batch * cfg.D * cfg.N * 4 * (3 if cfg.state_in is not None else 2)
    return n


def _ssd_head_params(cfg: SsdConfig):
    """A (H,) float32, dt_bias (H,) float64, Dskip (H,) float32 or None."""
    A = (-_rng(cfg.seed, _K_AH).uniform(1.0, 16.0, size=cfg.H)).astype(np.float32)
    dt = np.exp(_rng(cfg.seed, _K_DT).uniform(math.log(1e-3), math.log(1e-1), size=cfg.H))
    dt_bias = dt + np.log(-np.expm1(-dt))
    Dskip = _rng(cfg.seed, _K_D).uniform(0.5, 1.5, size=cfg.H).astype(np.float32) if cfg.dskip else None
    return A, dt_bias, Dskip


def ssd_inputs(cfg: SsdConfig, t0: int = 0, t1: Optional[int] = None, batches=None, heads=None):
    """SSD inputs of `cfg` for tokens [t0, t1), in storage dtypes; `batches`
    and `heads` select batch rows and heads. Selected heads must share one
    group: Bt and Ct are then that group's (G = 1). The values do not depend on
    the selection or on how the token range is split."""
    if t1 is None:
        t1 = cfg.L
    bsel = np.arange(cfg.batch) if batches is None else np.asarray(batches)
    hsel = np.arange(cfg.H) if heads is None else np.asarray(heads)
    A, dt_bias, Dskip = _ssd_head_params(cfg)
    T, act = t1 - t0, cfg.dtype
    cols = (hsel[:, None] * cfg.P + np.arange(cfg.P)[None, :]).reshape(-1)
    groups = np.arange(cfg.G)
    if heads is not None:
        groups = np.unique(hsel // (cfg.H // cfg.G))
        assert len(groups) == 1, "selected heads must share one group"
    gcols = (groups[:, None] * cfg.N + np.arange(cfg.N)[None, :]).reshape(-1)
    NG = len(groups)
    x = np.empty((len(bsel), T, len(hsel), cfg.P), dtype=np.float32 if act == "f32" else np.uint16)
    dl = np.empty((len(bsel), T, len(hsel)), dtype=x.dtype)
    Bt = np.empty((len(bsel), T, NG, cfg.N), dtype=x.dtype)
    Ct = np.empty_like(Bt)
    for k, b in enumerate(bsel):
        x[k] = _store(_token_block(cfg.seed, _K_X, b, t0, t1, cfg.H * cfg.P, cols), act).reshape(T, len(hsel), cfg.P)
        eps = _token_block(cfg.seed, _K_DNOISE, b, t0, t1, cfg.H, hsel)
        dl[k] = _store(_softplus(0.5 * eps + dt_bias[hsel][None, :]), act)
        Bt[k] = _store(_token_block(cfg.seed, _K_B, b, t0, t1, cfg.G * cfg.N, gcols), act).reshape(T, NG, cfg.N)
        Ct[k] = _store(_token_block(cfg.seed, _K_C, b, t0, t1, cfg.G * cfg.N, gcols), act).reshape(T, NG, cfg.N)
    out = {"x": x, "delta": dl, "A": np.ascontiguousarray(A[hsel]), "Bt": Bt, "Ct": Ct,
           "Dskip": None if Dskip is None else np.ascontiguousarray(Dskip[hsel]), "state_in": None}
    if cfg.state_in is not None:
        st = _rng(cfg.seed, _K_STATE).standard_normal((cfg.batch, cfg.H, cfg.P, cfg.N)) * cfg.state_in
        out["state_in"] = np.ascontiguousarray(st[bsel][:, hsel].astype(np.float32))
    return out


def fill_ssd_device(cfg: SsdConfig, device, seed: int = 777):
    """torch tensors of the full SSD workload on `device`, same distributions as
    ssd_inputs drawn with torch: x, delta, Bt, Ct."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    act = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    _A, dt_bias, _D = _ssd_head_params(cfg)
    bias = torch.tensor(dt_bias, dtype=torch.float32, device=device)

    def normal(shp):
        return torch.randn(shp, generator=g, device=device, dtype=torch.float32)

    return {"x": normal((cfg.batch, cfg.L, cfg.H, cfg.P)).to(act),
            "delta": torch.nn.functional.softplus(normal((cfg.batch, cfg.L, cfg.H)).mul_(0.5).add_(bias)).to(act),
            "Bt": normal((cfg.batch, cfg.L, cfg.G, cfg.N)).to(act),
            "Ct": normal((cfg.batch, cfg.L, cfg.G, cfg.N)).to(act)}


def ssd_step_bytes(cfg: SsdConfig) -> int:
    """Bytes one SSD decode step must move: the (batch, H, P, N) float32 state
    read and written, x read and y written per (b, h, p), delta per (b, h), Bt
    and Ct per (b, g, n), A and Dskip."""
    e = _esize(cfg.dtype)
    n = 2 * cfg.batch * cfg.H * cfg.P * cfg.N * 4 + 2 * cfg.batch * cfg.H * cfg.P * e + cfg.batch * cfg.H * e
    return n + 2 * cfg.batch * cfg.G * cfg.N * e + cfg.H * 4 * (2 if cfg.dskip else 1)


def ssd_bytes(cfg: SsdConfig, state_out: bool = False) -> int:
    """Bytes the SSD layer must move: x read and y written per (b, t, h, p),
    delta per (b, t, h), Bt and Ct per (b, t, g, n), A and Dskip once, the state
    when carried in or out."""
    e = _esize(cfg.dtype)
    n = 2 * cfg.batch * cfg.L * cfg.H * cfg.P * e + cfg.batch * cfg.L * cfg.H * e
    n += 2 * cfg.batch * cfg.L * cfg.G * cfg.N * e + cfg.H * 4 * (2 if cfg.dskip else 1)
    st = cfg.batch * cfg.H * cfg.P * cfg.N * 4
    return n + (st if cfg.state_in is not None else 0) + (st if state_out else 0)


def trap_extra_bytes(cfg: ScanConfig) -> int:
    """What the exponential-trapezoidal scan reads beyond scan_bytes: lam per
    (b, t, d) and the earlier token, x_prev (batch, D) and B_prev (batch, N)."""
    e = _esize(cfg.dtype)
    return cfg.batch * cfg.L * cfg.D * e + cfg.batch * (cfg.D + cfg.N) * e


def trap_step_extra_bytes(cfg: StepConfig) -> int:
    """The same for one decode step: lam and x_prev (batch, D), B_prev (batch, N)."""
    e = _esize(cfg.dtype)
    return cfg.batch * (2 * cfg.D + cfg.N) * e


def step_bytes(cfg: StepConfig) -> int:
    """Bytes one decode step must move: the state read and written, x, delta,
    (z) read and y written per (b,d), Bt and Ct per sequence, A and Dskip."""
    e = _esize(cfg.dtype)
    bd = cfg.batch * cfg.D
    n = 2 * bd * cfg.N * 4
    n += bd * e * (3 + (1 if cfg.gate else 0))
    n += 2 * cfg.batch * cfg.N * e
    n += cfg.D * cfg.N * 4 + (cfg.D * 4 if cfg.dskip != "none" else 0)
    return n
