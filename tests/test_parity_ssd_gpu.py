"""The Mamba-2 SSD layer (ssm_ssd_fwd; "Notas sobre Mamba", section "A forma
dual: atenção mascarada", and "Mamba-2 e State Space Duality (SSD)") against
the fp64 oracle's SSD recurrence (needs MI355X). The kernel computes by chunks
of 64 tokens on the matrix cores; the cases cover several chunks and a ragged
last chunk, both state sizes, heads sharing groups, a carried-in state,
resumption, and the full-size layer: sampled heads on the seeded streams, and
every output on device-drawn inputs."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import check, check_sum, gpu_ssd, say, to_dev, to_f64, to_host

pytestmark = pytest.mark.gpu


def _run(cfg):
    say(f"case {cfg}")
    inp = W.ssd_inputs(cfg)
    y, st = gpu_ssd(inp)
    yr, sr = oracle.get().ssd(inp, cfg.dtype)
    check(y, yr, cfg.dtype, "y")
    check(st, sr, cfg.dtype, "state_out")


@pytest.mark.parametrize("N", [64, 128])
@pytest.mark.parametrize("G", [1, 2])
def test_ssd_small(N, G):
    _run(W.SsdConfig(f"ssd_N{N}_G{G}", 2, 200, 4, 64, G, N, "bf16", dskip=True, state_in=0.5, seed=10 + N + G))


@pytest.mark.parametrize("L", [1, 63, 64, 65, 1000])
def test_ssd_ragged_lengths(L):
    _run(W.SsdConfig(f"ssd_L{L}", 1, L, 3, 64, 1, 128, "bf16", dskip=True, seed=30 + L))


def test_ssd_no_skip_no_state():
    _run(W.SsdConfig("ssd_plain", 2, 300, 2, 64, 1, 64, "bf16", dskip=False, seed=41))


def test_ssd_resume():
    """Two calls, the second from the first's final state, equal one call."""
    cfg = W.SsdConfig("ssd_resume", 2, 500, 2, 64, 1, 128, "bf16", dskip=True, state_in=0.3, seed=42)
    say(f"case {cfg}")
    y, st = gpu_ssd(W.ssd_inputs(cfg))
    m = 200  # not a multiple of the chunk
    y1, s1 = gpu_ssd(W.ssd_inputs(cfg, 0, m))
    p2 = W.ssd_inputs(cfg, m, cfg.L)
    p2["state_in"] = s1.astype(np.float32)
    y2, s2 = gpu_ssd(p2)
    check(np.concatenate([y1, y2], 1), y, "bf16", "two calls vs one (y)")
    check(s2, st, "bf16", "two calls vs one (state)")


def test_ssd_full_layer_sampled_heads():
    """The full Mamba-2 layer workload (8 x 4096 tokens, 80 heads of 64, state
    128): sampled (batch row, head) pairs take the seeded streams and are
    compared with the oracle; the other heads are filled on the GPU."""
    import torch
    import selective_state_space_16_amd as ssm
    cfg = W.SSD_CONFIGS["ssd"]
    say(f"case {cfg}")
    dev = W.fill_ssd_device(cfg, "cuda")
    whole = W.ssd_inputs(cfg, 0, 0)
    A, Dskip = to_dev(whole["A"]), to_dev(whole["Dskip"])
    picks = [(0, 0), (3, 17), (7, 79)]
    subs = {}
    for b, h in picks:
        sub = W.ssd_inputs(cfg, batches=[b], heads=[h])
        subs[(b, h)] = sub
        dev["x"][b, :, h] = to_dev(sub["x"][0, :, 0])
        dev["delta"][b, :, h] = to_dev(sub["delta"][0, :, 0])
        dev["Bt"][b] = to_dev(sub["Bt"][0])  # one group: every head of row b reads it
        dev["Ct"][b] = to_dev(sub["Ct"][0])
    st_out = torch.empty((cfg.batch, cfg.H, cfg.P, cfg.N), dtype=torch.float32, device="cuda")
    y = ssm.ssm_ssd_fwd(dev["x"], dev["delta"], A, dev["Bt"], dev["Ct"], Dskip=Dskip, state_out=st_out)
    torch.cuda.synchronize()
    o = oracle.get()
    for (b, h), sub in subs.items():
        yr, sr = o.ssd(sub, cfg.dtype)
        check(to_f64(y[b, :, h]), yr[0, :, 0], cfg.dtype, f"y (b={b}, h={h})")
        check(to_f64(st_out[b, h]), sr[0, 0], cfg.dtype, f"state_out (b={b}, h={h})")


@pytest.mark.parametrize("G", [1, 80])
def test_ssd_full_layer_every_output(G):
    """The full Mamba-2 layer workload (8 x 4096 tokens, 80 heads of 64, state
    128), in the launch configuration the bench times: inputs drawn on the
    device with the workload's recipe (seeded), copied back as stored values;
    every y and every final-state value against the oracle, one batch row at a
    time. G = 80 gives every head its own B and C."""
    import dataclasses
    import torch
    import selective_state_space_16_amd as ssm
    cfg = dataclasses.replace(W.SSD_CONFIGS["ssd"], G=G)
    say(f"case {cfg}: every output (device-drawn inputs, seed {505 + G})")
    dev = W.fill_ssd_device(cfg, "cuda", seed=505 + G)
    whole = W.ssd_inputs(cfg, 0, 0)
    A, Dskip = to_dev(whole["A"]), to_dev(whole["Dskip"])
    st_out = torch.empty((cfg.batch, cfg.H, cfg.P, cfg.N), dtype=torch.float32, device="cuda")
    y = ssm.ssm_ssd_fwd(dev["x"], dev["delta"], A, dev["Bt"], dev["Ct"], Dskip=Dskip, state_out=st_out)
    torch.cuda.synchronize()
    o = oracle.get()
    ey, es = oracle.ErrorSum(), oracle.ErrorSum()
    for b in range(cfg.batch):
        sub = {k: to_host(dev[k][b:b + 1]) for k in ("x", "delta", "Bt", "Ct")}
        sub["A"], sub["Dskip"] = whole["A"], whole["Dskip"]
        yr, sr = o.ssd(sub, cfg.dtype)
        ey.add(to_f64(y[b:b + 1]), yr)
        es.add(to_f64(st_out[b:b + 1]), sr)
    assert ey.count == cfg.batch * cfg.L * cfg.H * cfg.P and es.count == cfg.batch * cfg.H * cfg.P * cfg.N
    check_sum(ey, cfg.dtype, "y (every output)")
    check_sum(es, cfg.dtype, "state_out (every value)")
