#!/usr/bin/env python3
"""Selective-scan (S6) benchmark on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
a full ssm_scan_fwd call on the workload (default: the million-token context,
batch 1, L 1048576, D 1536, N 16, bfloat16 activations with a float32 state
carried in and out, silu gate), or one ssm_step call for the decode workload. Inputs are resident in HBM before the timed region;
several input/output sets rotate so that the 256 MB Infinity Cache cannot
hold a whole step's working set.

Prints one JSON line: throughput in G(B*L*D*N)-elements/s, the roofline of
the kernel (its algorithmic work per launch over its average launch time,
timed with events around every launch, against the MI355X peak of the unit
that bounds it), the same launch against the HBM peak, and the fp64 oracle
timed on the host cores on a bounded sample of the same workload.

`--copy-calibration BYTES` instead runs a plain device-to-device copy of
BYTES bytes a few times; under `rocprofv3 --pmc FETCH_SIZE` (or WRITE_SIZE) it
gives the factor that turns those counters into HBM bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
# VALU issue slots per second: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (one
# fp32 instruction per lane per slot; packed fp32 is not used).
VALU_PEAK_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12
# Issue slots the recurrence needs per (b, t, d, n) element at the least:
# delta*A (mul), exp (a transcendental, issued at half rate: 2 slots),
# B*(delta*x) (mul), dA*h + dBx (fma), C*h accumulated (fma).
SCAN_SLOTS_PER_ELEM = 6
# The gradient per element at the least: the recurrence again (delta*A, exp
# at 2 slots, B*(delta*x), fma) and the reverse step (G += C*ds, ds*h,
# G*a*h (2), two fmas into d(delta), dA fma, G*(delta*x), dx fma, G *= a).
BWD_SLOTS_PER_ELEM = 15
SCAN_KERNEL = "scan_stripe_kernel"
STEP_KERNEL = "step_kernel"
SSD_KERNEL = "ssd_kernel"
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bfloat16 matrix-core peak
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
# What the source pages claim for the fused selective scan and for the model
# around it, quoted as context only: the pages name no hardware, precision or
# workload for any of them, so none is a target or a baseline here.
PAGE_CLAIMS = {
    "note": "context only; the pages give no hardware, precision or workload for these figures",
    "claims": [
        {"claim": "fused selective scan vs a standard PyTorch implementation", "value": "20-40x faster",
         "source": "Mamba encyclopedia page (tonho.wtf), 'como funciona'"},
        {"claim": "fused selective scan vs FlashAttention-2", "value": "faster from 2K sequence length on",
         "source": "Mamba encyclopedia page (tonho.wtf), 'como funciona'"},
        {"claim": "Mamba inference throughput vs a comparable Transformer", "value": "about 5x",
         "source": "'Notas sobre Mamba' (rodolfoviana.com.br), introduction; encyclopedia entry "
                   "(magik.kayoridolfi.ai)"},
    ],
}


# The sources each measured kernel is built from (besides the shared headers).
KERNEL_SOURCES = {
    "scan": ("ssm_scan_stripe_kernel.h", "ssm_scan_stripe.hip", "ssm_scan_stripe_act.hip", "ssm_scan_stripe_trap.hip",
             "ssm_scan_stripe_conv.hip"),
    "step": ("ssm_step.hip",),
    "ssd": ("ssm_ssd.hip",),
    "ssd_step": ("ssm_ssd_step.hip",),
    "grad": ("ssm_scan_bwd_kernel.h", "ssm_scan_bwd.hip", "ssm_scan_bwd_trap.hip"),
    "conv_grad": ("ssm_scan_bwd_kernel.h", "ssm_scan_bwd.hip", "ssm_scan_bwd_trap.hip", "ssm_conv_bwd.hip"),
}
SHARED_SOURCES = ("ssm_common.h", "ssm_device.h", "ssm_internal.h")


def kernel_family(workload: str) -> str:
    if workload.endswith("_conv_grad"):
        return "conv_grad"
    if workload.endswith("_grad"):
        return "grad"
    base = workload[:-len("_conv")] if workload.endswith("_conv") else workload
    return {"c4": "step", "ssd": "ssd", "ssd_step": "ssd_step"}.get(base, "scan")


def kernel_source_hash(family: str) -> str:
    """sha256 (first 16 hex) of the sources of one kernel family and the shared
    device headers under csrc/."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_16_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[family] + SHARED_SOURCES):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; else None."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_src_sha") != kernel_source_hash(kernel_family(workload)):
        return None
    return rec.get("hbm_bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a):
    import numpy as np
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t):
    """A device tensor as the stored numpy array the oracle takes (bfloat16 as
    its uint16 bit patterns)."""
    import numpy as np
    import torch
    if t is None:
        return None
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def device_blocks(dev, y, st_out, order, chans):
    """(stored inputs, y, final state) of `chans`-channel blocks of batch row 0
    of a scan run on the device, block indices in `order`, for
    oracle.scan_compare. Every block runs over the whole sequence."""
    D = dev["x"].shape[2]
    bt, ct = to_host(dev["Bt"][0:1]), to_host(dev["Ct"][0:1])
    f64 = lambda t: t.detach().float().cpu().numpy().astype("float64")
    for k in order:
        sl = slice(k * chans, min(D, (k + 1) * chans))
        part = lambda key: None if dev.get(key) is None else to_host(dev[key][0:1, :, sl])
        inp = {"x": part("x"), "delta": part("delta"), "delta_raw": part("delta_raw"), "lam": part("lam"),
               "z": part("z"), "Bt": bt, "Ct": ct, "A": to_host(dev["A"][sl]),
               "Dskip": None if dev.get("Dskip") is None else to_host(dev["Dskip"][sl]),
               "dt_bias": None if dev.get("dt_bias") is None else to_host(dev["dt_bias"][sl]),
               "x_raw": part("x") if dev.get("conv_w") is not None else None,
               "conv_w": None if dev.get("conv_w") is None else to_host(dev["conv_w"][sl]),
               "conv_b": None if dev.get("conv_b") is None else to_host(dev["conv_b"][sl]),
               "conv_state": None if dev.get("conv_state") is None else to_host(dev["conv_state"][0:1, sl]),
               "x_prev": None if dev.get("x_prev") is None else to_host(dev["x_prev"][0:1, sl]),
               "B_prev": None if dev.get("B_prev") is None else to_host(dev["B_prev"][0:1]),
               "state_in": None if dev.get("state_in") is None else to_host(dev["state_in"][0:1, sl])}
        yield inp, f64(y[0:1, :, sl]), (None if st_out is None else f64(st_out[0:1, sl]))


def rel_l2(got, ref):
    import numpy as np
    d = got - ref
    return float(np.sqrt((d * d).sum()) / max(np.sqrt((ref * ref).sum()), 1e-300)), float(np.abs(d).max())


def timed(steps, step, stream):
    """Run `steps` steps back to back on `stream`, twice. Returns (ms per step
    over the whole first run, mean ms of one launch in the second), from events
    on that stream: one pair around the first run (nothing else between the
    launches), one pair around every launch of the second (each step is a
    single kernel launch)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, sum(a.elapsed_time(b) for a, b in ev) / steps


def copy_calibration(nbytes):
    """A plain device copy of nbytes, five times: the reference for the HBM
    byte counters (FETCH_SIZE, WRITE_SIZE) of a profiled run."""
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "launches": 5}), flush=True)


def valu_calibration():
    """Issue rates of v_exp_f32, v_fma_f32 and of the scan's mix (four
    multiply-adds per exponential), from the calibration kernels of
    libssm_calib.so at 1, 2, 4 and 8 waves per SIMD: lane instructions per
    second, timed with events around each launch. This is the measurement the
    VALU roofline's cost of two issue slots per exponential rests on."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "selective_state_space_16_amd", "libssm_calib.so"))
    lib.ssm_calib_valu_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.ssm_calib_valu_rate.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    iters = 4096
    stream = torch.cuda.current_stream()
    rows = []
    for op, name, per_step, exps in ((0, "v_exp_f32", 1, 1), (1, "v_fma_f32", 1, 0), (2, "4 fma + 1 exp", 5, 1)):
        for wps in (1, 2, 4, 8):
            blocks = cus * wps  # 4 waves per workgroup, one per SIMD
            out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
            for _ in range(2):  # warm-up
                assert lib.ssm_calib_valu_rate(op, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                               ctypes.c_void_p(stream.cuda_stream)) == 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                lib.ssm_calib_valu_rate(op, blocks, iters, ctypes.c_void_p(out.data_ptr()),
                                        ctypes.c_void_p(stream.cuda_stream))
            e1.record(stream)
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) / 5 * 1e-3
            lane_instr = blocks * 256.0 * iters * 8 * per_step
            rate = lane_instr / sec / 1e12
            rows.append({"op": name, "waves_per_simd": wps, "launch_us": sec * 1e6, "T_lane_instr_per_s": rate,
                         "frac_of_issue_peak": rate / VALU_PEAK_TSLOTS,
                         "slots_per_exp": (None if exps == 0 else None)})
            log(f"[calib] {name:>14}  {wps} waves/SIMD  {sec * 1e6:8.1f} us  {rate:6.2f} T lane-instr/s "
                f"({rate / VALU_PEAK_TSLOTS:.2f} of {VALU_PEAK_TSLOTS:.1f})")
    # slots an exponential costs, from the best rates: issue peak / exp rate,
    # and from the mix: time per step over the time of four fmas
    best = {n: max(r["T_lane_instr_per_s"] for r in rows if r["op"] == n) for n in ("v_exp_f32", "v_fma_f32",
                                                                                    "4 fma + 1 exp")}
    exp_slots = best["v_fma_f32"] / best["v_exp_f32"]
    mix_slots = 5 * best["v_fma_f32"] / best["4 fma + 1 exp"] - 4
    for r in rows:
        r.pop("slots_per_exp")
    print(json.dumps({"valu_calibration": rows, "issue_peak_T_lane_instr_per_s": VALU_PEAK_TSLOTS,
                      "cus": cus, "exp_cost_in_fma_slots_alone": exp_slots,
                      "exp_cost_in_fma_slots_in_the_mix": mix_slots}), flush=True)


def bench_scan(args, name):
    import numpy as np
    import torch
    import selective_state_space_16_amd as ssm
    import workloads as W

    cfg = W.SCAN_CONFIGS[name]
    log(f"[bench] workload {cfg}")
    t0 = time.time()
    # set 0: the seeded numpy streams (checked against the oracle below)
    cv = args.conv  # x before the block's short convolution and SiLU (ssm_scan_fwd_conv)
    sp = args.softplus or cv  # delta handed over before its activation
    tr = args.trap  # exponential-trapezoidal rule
    bw = args.backward  # the gradient (ssm_scan_bwd) in place of the forward scan
    inp = W.scan_inputs(cfg, raw_delta=sp, trap=tr, conv=cv) if name != "c3" else None
    grads = W.grad_inputs(cfg) if (bw and inp is not None) else None
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
    whole = W.scan_inputs(cfg, 0, 0, conv=cv)
    A, Dskip = to_dev(whole["A"]), to_dev(whole["Dskip"])
    st_in = to_dev(whole["state_in"])
    # the convolution's taps, bias and earlier raw tokens (per channel: shared by every set)
    cw, cb, cs = (to_dev(whole["conv_w"]), to_dev(whole["conv_b"]), to_dev(whole["conv_state"])) if cv else \
        (None, None, None)
    sets = []
    if inp is not None:
        keys = ("x", "delta_raw", "dt_bias", "z", "Bt", "Ct") if sp else ("x", "delta", "z", "Bt", "Ct")
        if tr:
            keys += ("lam", "x_prev", "B_prev")
        sets.append({k: to_dev(inp[k]) for k in keys})
        if bw:
            sets[0]["dy"] = to_dev(grads["dy"])
    # further sets: same distributions, drawn on the GPU
    per_set = W.scan_bytes(cfg)
    nsets = max(1, min(args.rotate, int(60e9 // max(per_set, 1))))
    while len(sets) < nsets:
        sets.append(W.fill_scan_device(cfg, "cuda", seed=1000 + len(sets), raw_delta=sp, trap=tr))
        if bw:
            sets[-1]["dy"] = torch.randn(sets[-1]["x"].shape, device="cuda").to(sets[-1]["x"].dtype)
    ys = [torch.empty_like(s["x"]) for s in sets]
    if bw:
        f32 = torch.float32
        ys = [{("dx_raw" if cv else "dx"): torch.empty_like(s["x"]),
               ("ddelta_raw" if sp else "ddelta"): torch.empty_like(s["x"]),
               "dz": torch.empty_like(s["x"]) if s["z"] is not None else None,
               "dA": torch.empty((cfg.D, cfg.N), dtype=f32, device="cuda"),
               "dBt": torch.empty((cfg.batch, cfg.L, cfg.N), dtype=f32, device="cuda"),
               "dCt": torch.empty((cfg.batch, cfg.L, cfg.N), dtype=f32, device="cuda"),
               "dDskip": torch.empty((cfg.D,), dtype=f32, device="cuda") if Dskip is not None else None,
               "dstate_in": torch.empty((cfg.batch, cfg.D, cfg.N), dtype=f32, device="cuda")} for s in sets]
        if sp:
            for o_ in ys:
                o_["ddt_bias"] = torch.empty((cfg.D,), dtype=f32, device="cuda")
        if cv:
            for o_, s_ in zip(ys, sets):
                o_["dconv_w"] = torch.empty((cfg.D, 4), dtype=f32, device="cuda")
                o_["dconv_b"] = torch.empty((cfg.D,), dtype=f32, device="cuda")
                o_["dconv_state"] = torch.empty((cfg.batch, cfg.D, 3), dtype=s_["x"].dtype, device="cuda")
        if tr:
            for o_, s_ in zip(ys, sets):
                o_["dlam"] = torch.empty_like(s_["x"])
                o_["dx_prev"] = torch.empty((cfg.batch, cfg.D), dtype=s_["x"].dtype, device="cuda")
                o_["dB_prev"] = torch.empty((cfg.batch, cfg.N), dtype=f32, device="cuda")
        dstate = to_dev(W.grad_inputs(cfg, 0, 0)["dstate"])
        bws_fn = ssm.lib().ssm_scan_bwd_conv_workspace_bytes if cv else ssm.ssm_scan_bwd_workspace_bytes
        bws = torch.empty(bws_fn(cfg.batch, cfg.L, cfg.D, cfg.N, 0 if cfg.dtype == "f32" else 1),
                          dtype=torch.uint8, device="cuda")
    ws_bytes = ssm.ssm_scan_workspace_bytes(cfg.batch, cfg.L, cfg.D, cfg.N, 0 if cfg.dtype == "f32" else 1)
    ws = ssm.new_workspace(ws_bytes)
    st_out = torch.empty((cfg.batch, cfg.D, cfg.N), dtype=torch.float32, device="cuda") \
        if cfg.state_in is not None else None
    stream = torch.cuda.current_stream()

    def step(i):
        s = sets[i % len(sets)]
        if bw and cv:
            ssm.ssm_scan_bwd_conv(s["x"], cw, s["delta_raw"], s["dt_bias"], A, s["Bt"], s["Ct"], s["dy"], conv_b=cb,
                                  conv_state=cs, Dskip=Dskip, z=s["z"], state_in=st_in, dstate=dstate,
                                  out=ys[i % len(sets)], workspace=bws, stream=stream)
        elif bw and tr:
            ssm.ssm_scan_bwd_trap(s["x"], s["delta"], s["lam"], A, s["Bt"], s["Ct"], s["dy"], Dskip=Dskip, z=s["z"],
                                  x_prev=s["x_prev"], B_prev=s["B_prev"], state_in=st_in, dstate=dstate,
                                  out=ys[i % len(sets)], workspace=bws, stream=stream)
        elif bw and sp:
            ssm.ssm_scan_bwd_dt(s["x"], s["delta_raw"], s["dt_bias"], A, s["Bt"], s["Ct"], s["dy"], Dskip=Dskip,
                                z=s["z"], state_in=st_in, dstate=dstate, out=ys[i % len(sets)], workspace=bws,
                                stream=stream)
        elif bw:
            ssm.ssm_scan_bwd(s["x"], s["delta"], A, s["Bt"], s["Ct"], s["dy"], Dskip=Dskip, z=s["z"],
                             state_in=st_in, dstate=dstate, out=ys[i % len(sets)], workspace=bws, stream=stream)
        elif cv:
            ssm.ssm_scan_fwd_conv(s["x"], cw, s["delta_raw"], s["dt_bias"], A, s["Bt"], s["Ct"], conv_b=cb,
                                  conv_state=cs, Dskip=Dskip, z=s["z"], state_in=st_in, state_out=st_out,
                                  y=ys[i % len(sets)], workspace=ws, stream=stream)
        elif sp:
            ssm.ssm_scan_fwd_dt(s["x"], s["delta_raw"], s["dt_bias"], A, s["Bt"], s["Ct"], Dskip=Dskip, z=s["z"],
                                state_in=st_in, state_out=st_out, y=ys[i % len(sets)], workspace=ws, stream=stream)
        elif tr:
            ssm.ssm_scan_fwd_trap(s["x"], s["delta"], s["lam"], A, s["Bt"], s["Ct"], Dskip=Dskip, z=s["z"],
                                  x_prev=s["x_prev"], B_prev=s["B_prev"], state_in=st_in, state_out=st_out,
                                  y=ys[i % len(sets)], workspace=ws, stream=stream)
        else:
            ssm.ssm_scan_fwd(s["x"], s["delta"], A, s["Bt"], s["Ct"], Dskip=Dskip, z=s["z"], state_in=st_in,
                             state_out=st_out, y=ys[i % len(sets)], workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms, launch_ms = timed(args.steps, step, stream)
    log(f"[bench] {args.steps} steps, {ms * 1e3:.2f} us/step ({launch_ms * 1e3:.2f} us/launch) "
        f"over {len(sets)} rotating sets")
    out = {"cfg": cfg, "ms": ms, "launch_ms": launch_ms, "elems": cfg.elems,
           "bytes": W.scan_bytes(cfg, st_out is not None) + (cfg.D * 4 if sp else 0) +
                    (W.trap_extra_bytes(cfg) if tr else 0) +
                    (cfg.D * 5 * 4 + cfg.batch * cfg.D * 3 * W._esize(cfg.dtype) if cv else 0), "dtype": cfg.dtype,
           "parity": None, "cpu": None}
    if bw:
        out["bytes"] = W.scan_bwd_bytes(cfg) + (2 * cfg.D * 4 if sp else 0)  # dt_bias read, ddt_bias written
        if cv:  # taps and bias read and their gradients written; the earlier raw tokens and their gradient
            out["bytes"] += 2 * cfg.D * 5 * 4 + 2 * cfg.batch * cfg.D * 3 * W._esize(cfg.dtype)
        if tr:  # lam read and dlam written; x_prev, B_prev read and their gradients written
            out["bytes"] += 2 * cfg.batch * cfg.L * cfg.D * W._esize(cfg.dtype) + \
                2 * cfg.batch * (cfg.D * W._esize(cfg.dtype) + cfg.N * 4)
        if inp is not None and not args.no_cpu:
            import oracle
            torch.cuda.synchronize()
            step(0)
            torch.cuda.synchronize()
            got = {k: (v.double().cpu().numpy() if v is not None else None) for k, v in ys[0].items()}
            o = oracle.get()
            reps, tot, ref = 0, 0.0, None
            while reps == 0 or tot < args.cpu_seconds:
                t = time.perf_counter()
                ref = (o.scan_bwd_conv if cv else o.scan_bwd_trap if tr else o.scan_bwd_dt if sp else o.scan_bwd)(
                    inp, grads["dy"], grads["dstate"], cfg.dtype)
                tot += time.perf_counter() - t
                reps += 1
            out["parity"] = {k: dict(zip(("relL2", "maxabs"), rel_l2(got[k], ref[k])))
                             for k in ("dx", "dx_raw", "dconv_w", "dconv_b", "dconv_state", "ddelta", "ddelta_raw",
                                       "ddt_bias", "dlam", "dz", "dA", "dBt", "dCt", "dDskip", "dx_prev", "dB_prev",
                                       "dstate_in")
                             if ref.get(k) is not None}
            out["cpu"] = {"value": cfg.elems * reps / tot / 1e9, "unit": "G(B*L*D*N)-elem/s", "cores": 1,
                          "kind": "oracle",
                          "sample": f"whole workload, {reps} run(s), {tot:.1f}s, fp64 C oracle gradient, one thread"}
        return out
    if inp is None and not args.no_cpu and cfg.batch == 1:
        # The million-token workload: set 0 was drawn on the device. Its
        # result is compared with the oracle on the same stored values, one
        # 64-channel block at a time over the whole sequence (with the final
        # state), blocks spread over the tile columns, until about
        # cpu_seconds of oracle time; that sample also gives the CPU rate.
        import oracle
        torch.cuda.synchronize()
        step(0)
        torch.cuda.synchronize()
        dev = dict(sets[0], A=A, Dskip=Dskip, state_in=st_in, conv_w=cw, conv_b=cb, conv_state=cs)
        nblk = (cfg.D + 63) // 64
        stride = next(k for k in (7, 5, 3, 1) if np.gcd(k, nblk) == 1)
        order = [(k * stride) % nblk for k in range(nblk)]
        rule = "scan_conv" if cv else "scan_dt" if sp else "scan_trap" if tr else "scan"

        def bounded():
            spent = 0.0
            for blk in device_blocks(dev, ys[0], st_out, order, 64):
                if spent >= args.cpu_seconds:
                    return
                t = time.perf_counter()
                yield blk
                spent += time.perf_counter() - t  # the oracle ran between the two yields

        ey, es, secs = oracle.scan_compare(bounded(), cfg.dtype, rule=rule)
        nch = ey.count // cfg.L
        out["parity"] = {"relL2": ey.rel, "maxabs": ey.maxabs, "state_relL2": es.rel,
                         "state_maxabs": es.maxabs, "channels_compared": nch, "channels": cfg.D,
                         "tokens_per_channel": cfg.L, "tol_relL2": 2e-2 if cfg.dtype == "bf16" else 1e-5}
        out["data"] = "synthetic, seeded; drawn on the device with the workload's recipe (workloads/)"
        out["cpu"] = {"value": ey.count * cfg.N / secs / 1e9, "unit": "G(B*L*D*N)-elem/s",
                      "cores": oracle.get().threads(), "kind": "oracle",
                      "sample": f"{nch} of {cfg.D} channels (64-channel blocks from {nch // 64 or 1} tile columns), "
                                f"every one over all {cfg.L} tokens with its final state, {secs:.1f}s, fp64 C oracle, "
                                f"OpenMP over channels"}
        return out
    # parity of the timed configuration on set 0, and the CPU baseline
    if inp is not None and not args.no_cpu:
        import oracle
        torch.cuda.synchronize()
        step(0)
        torch.cuda.synchronize()
        y0 = ys[0].double().cpu().numpy()
        o = oracle.get()
        reps, tot, yr = 0, 0.0, None
        while reps == 0 or tot < args.cpu_seconds:
            t = time.perf_counter()
            yr, _ = o.scan_conv(inp, cfg.dtype) if cv else o.scan_dt(inp, cfg.dtype) if sp else \
                o.scan_trap(inp, cfg.dtype) if tr else o.scan(inp, cfg.dtype)
            tot += time.perf_counter() - t
            reps += 1
        rel, mx = rel_l2(y0, yr)
        out["parity"] = {"relL2": rel, "maxabs": mx}
        out["cpu"] = {"value": cfg.elems * reps / tot / 1e9, "unit": "G(B*L*D*N)-elem/s", "cores": o.threads(),
                      "kind": "oracle",
                      "sample": f"whole workload, {reps} run(s), {tot:.1f}s, fp64 C oracle, OpenMP over (b,d)"}
    return out


def ssd_flops(cfg) -> int:
    """Matrix-core flops the chunked SSD algorithm needs per launch (Q = 64):
    per chunk and head, C B^T and M x on the lower triangle with its diagonal
    (Q (Q + 1) / 2 entries), C H^T and the state update x^T (w o B) in full."""
    Q = 64
    chunks = (cfg.L + Q - 1) // Q
    tri = Q * (Q + 1) // 2
    per = 2 * (tri * cfg.N + tri * cfg.P + Q * cfg.N * cfg.P + cfg.P * Q * cfg.N)
    return cfg.batch * cfg.H * chunks * per


def bench_ssd(args):
    import numpy as np
    import torch
    import selective_state_space_16_amd as ssm
    import workloads as W

    cfg = W.SSD_CONFIGS["ssd"]
    log(f"[bench] workload {cfg}")
    whole = W.ssd_inputs(cfg, 0, 0)
    A, Dskip = to_dev(whole["A"]), to_dev(whole["Dskip"])
    per_set = W.ssd_bytes(cfg)
    nsets = max(1, min(args.rotate, int(60e9 // max(per_set, 1))))
    sets = [W.fill_ssd_device(cfg, "cuda", seed=2000 + k) for k in range(nsets)]
    # set 0: sampled (batch row, head) pairs from the seeded streams, for the parity check
    picks = [(0, 0), (cfg.batch - 1, cfg.H - 1)]
    subs = {}
    for b, h in picks:
        sub = W.ssd_inputs(cfg, batches=[b], heads=[h])
        subs[(b, h)] = sub
        sets[0]["x"][b, :, h] = to_dev(sub["x"][0, :, 0])
        sets[0]["delta"][b, :, h] = to_dev(sub["delta"][0, :, 0])
        sets[0]["Bt"][b] = to_dev(sub["Bt"][0])
        sets[0]["Ct"][b] = to_dev(sub["Ct"][0])
    ys = [torch.empty_like(s_["x"]) for s_ in sets]
    stream = torch.cuda.current_stream()

    def step(i):
        s_ = sets[i % len(sets)]
        ssm.ssm_ssd_fwd(s_["x"], s_["delta"], A, s_["Bt"], s_["Ct"], Dskip=Dskip, y=ys[i % len(sets)], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ms, launch_ms = timed(args.steps, step, stream)
    log(f"[bench] {args.steps} steps, {ms * 1e3:.2f} us/step ({launch_ms * 1e3:.2f} us/launch) "
        f"over {len(sets)} rotating sets")
    out = {"cfg": cfg, "ms": ms, "launch_ms": launch_ms, "elems": cfg.elems, "bytes": W.ssd_bytes(cfg),
           "flops": ssd_flops(cfg), "dtype": cfg.dtype, "parity": None, "cpu": None}
    if not args.no_cpu:
        import oracle
        step(0)
        torch.cuda.synchronize()
        o = oracle.get()
        worst, reps, tot = 0.0, 0, 0.0
        for (b, h), sub in subs.items():
            t = time.perf_counter()
            yr, _ = o.ssd(sub, cfg.dtype)
            tot += time.perf_counter() - t
            reps += 1
            rel, _ = rel_l2(ys[0][b, :, h].double().cpu().numpy(), yr[0, :, 0])
            worst = max(worst, rel)
        out["parity"] = {"relL2_worst_sampled_head": worst, "heads": len(subs)}
        # CPU baseline: the oracle on whole heads, about cpu_seconds of work
        k = 0
        while tot < args.cpu_seconds:
            sub = W.ssd_inputs(cfg, batches=[k % cfg.batch], heads=[(7 * k) % cfg.H])
            t = time.perf_counter()
            o.ssd(sub, cfg.dtype)
            tot += time.perf_counter() - t
            reps += 1
            k += 1
        per_head = cfg.L * cfg.P * cfg.N
        out["cpu"] = {"value": per_head * reps / tot / 1e9, "unit": "G(B*L*H*P*N)-elem/s", "cores": 1,
                      "kind": "oracle",
                      "sample": f"{reps} whole (batch row, head) sequences, {tot:.1f}s, fp64 C oracle "
                                f"(one head per call, so one thread)"}
    return out


def bench_ssd_step(args):
    """The Mamba-2 SSD decode workload: K consecutive ssm_ssd_step calls, one
    token each, on a (256, 80, 64, 128) float32 state resident in HBM, from a
    captured graph as for the S6 decode step."""
    import numpy as np
    import torch
    import dataclasses
    import selective_state_space_16_amd as ssm
    import workloads as W

    cfg = W.SSD_CONFIGS["ssd_step"]
    log(f"[bench] workload {cfg}")
    nsteps = args.steps + args.warmup
    tok = W.fill_ssd_device(dataclasses.replace(cfg, L=nsteps), "cuda")
    # per-step tensors: (step, batch, ...) contiguous
    tok = {k: v.transpose(0, 1).contiguous() for k, v in tok.items()}
    whole = W.ssd_inputs(dataclasses.replace(cfg, L=0, state_in=None), batches=[0])
    A, Dskip = to_dev(whole["A"]), to_dev(whole["Dskip"])
    g = torch.Generator(device="cuda")
    g.manual_seed(4321)
    state = torch.randn((cfg.batch, cfg.H, cfg.P, cfg.N), generator=g, device="cuda")
    y = torch.empty((cfg.batch, cfg.H, cfg.P), dtype=tok["x"].dtype, device="cuda")
    stream = torch.cuda.current_stream()

    def step(s):  # on the current stream (the capture stream inside the graph)
        ssm.ssm_ssd_step(tok["x"][s], tok["delta"][s], A, tok["Bt"][s], tok["Ct"][s], state, Dskip=Dskip, y=y,
                         stream=torch.cuda.current_stream())

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(args.warmup + i)
    graph.replay()  # untimed: first replay uploads the graph
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] {args.steps} SSD decode steps from a graph, {ms * 1e3:.2f} us/step")
    out = {"cfg": cfg, "ms": ms, "launch_ms": ms, "elems": cfg.batch * cfg.H * cfg.P * cfg.N,
           "bytes": W.ssd_step_bytes(cfg), "dtype": cfg.dtype, "parity": None, "cpu": None}
    if not args.no_cpu:
        # parity and the oracle's rate on a bounded sample: 4 batch rows x 8
        # heads, their inputs and state from the seeded streams, for T steps
        import oracle
        T = 16
        bsel, hsel = np.array([0, 1, 128, 255]), np.arange(0, cfg.H, 10)
        part = W.ssd_inputs(dataclasses.replace(cfg, L=T), batches=bsel, heads=hsel)
        st = torch.zeros_like(state[:1]).expand(len(bsel), -1, -1, -1).contiguous()
        st[:, torch.as_tensor(hsel, device="cuda")] = to_dev(part["state_in"])
        d = {k: to_dev(v) for k, v in part.items()}
        hs = torch.as_tensor(hsel, device="cuda")
        ys = []
        for t in range(T):
            xs = torch.zeros((len(bsel), cfg.H, cfg.P), dtype=tok["x"].dtype, device="cuda")
            ds = torch.ones((len(bsel), cfg.H), dtype=tok["x"].dtype, device="cuda")
            xs[:, hs], ds[:, hs] = d["x"][:, t], d["delta"][:, t]
            ys.append(ssm.ssm_ssd_step(xs, ds, A, d["Bt"][:, t].contiguous(), d["Ct"][:, t].contiguous(), st,
                                       Dskip=Dskip)[:, hs])
        torch.cuda.synchronize()
        yg = torch.stack(ys, 1).double().cpu().numpy()
        o = oracle.get()
        t = time.perf_counter()
        yr, _ = o.ssd(part, cfg.dtype, nthreads=1)
        tot = time.perf_counter() - t
        rel, mx = rel_l2(yg, yr)
        out["parity"] = {"relL2": rel, "maxabs": mx}
        out["cpu"] = {"value": len(bsel) * len(hsel) * T * cfg.P * cfg.N / tot / 1e9 / T,
                      "unit": "G(B*H*P*N)-elem/s per step", "cores": 1, "kind": "oracle",
                      "sample": f"{len(bsel)} batch rows x {len(hsel)} heads x {T} steps, {tot:.2f}s, fp64 C oracle"}
    return out


def bench_step(args):
    import numpy as np
    import torch
    import selective_state_space_16_amd as ssm
    import workloads as W

    cfg = W.STEP_CONFIG
    log(f"[bench] workload {cfg}")
    nsteps = args.steps + args.warmup
    cv = args.conv  # x before the block's convolution and SiLU (ssm_step_conv)
    base = W.step_inputs(cfg, conv=cv)
    state = to_dev(base["state"])
    A, Dskip = to_dev(base["A"]), to_dev(base["Dskip"])
    cw, cb, window = (to_dev(base["conv_w"]), to_dev(base["conv_b"]), to_dev(base["conv_state"])) if cv else \
        (None, None, None)
    sp = args.softplus or cv  # delta handed over before its activation
    tr = args.trap  # exponential-trapezoidal rule; step s gets token s - 1 as the earlier token
    fill = W.fill_step_device(cfg, nsteps, "cuda", raw_delta=sp, trap=tr)
    bias = to_dev(base["dt_bias"])
    y = torch.empty((cfg.batch, cfg.D), dtype=fill["x"].dtype, device="cuda")
    stream = torch.cuda.current_stream()

    def step(s):
        if cv:
            ssm.ssm_step_conv(fill["x"][s], cw, window, fill["delta_raw"][s], bias, A, fill["Bt"][s], fill["Ct"][s],
                              state, conv_b=cb, Dskip=Dskip, z=fill["z"][s], y=y, stream=torch.cuda.current_stream())
        elif sp:
            ssm.ssm_step_dt(fill["x"][s], fill["delta_raw"][s], bias, A, fill["Bt"][s], fill["Ct"][s], state,
                            Dskip=Dskip, z=fill["z"][s], y=y, stream=torch.cuda.current_stream())
        elif tr:
            xp, bp = (fill["x"][s - 1], fill["Bt"][s - 1]) if s > 0 else (None, None)
            ssm.ssm_step_trap(fill["x"][s], fill["delta"][s], fill["lam"][s], A, fill["Bt"][s], fill["Ct"][s], state,
                              Dskip=Dskip, z=fill["z"][s], x_prev=xp, B_prev=bp, y=y,
                              stream=torch.cuda.current_stream())
        else:
            ssm.ssm_step(fill["x"][s], fill["delta"][s], A, fill["Bt"][s], fill["Ct"][s], state, Dskip=Dskip,
                         z=fill["z"][s], y=y, stream=torch.cuda.current_stream())

    # A decode loop is launch-bound from Python (the binding's argument checks
    # take about as long as the kernel), so the K timed steps are captured once
    # into a HIP graph, as a serving loop would, and the graph is replayed in
    # the timed region: K kernel launches, one per step, each on its own token.
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    eager_ms, _ = timed(args.steps, lambda i: step(args.warmup + i), stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            step(args.warmup + i)
    graph.replay()  # untimed: first replay uploads the graph
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    launch_ms = ms  # one launch per step, back to back inside the graph
    log(f"[bench] {args.steps} decode steps from a graph, {ms * 1e3:.2f} us/step "
        f"(eager launches from Python: {eager_ms * 1e3:.2f} us/step)")
    out = {"cfg": cfg, "ms": ms, "launch_ms": launch_ms, "elems": cfg.elems_per_step,
           "bytes": W.step_bytes(cfg) + (cfg.D * 4 if sp else 0) + (W.trap_step_extra_bytes(cfg) if tr else 0) +
                    (cfg.D * 5 * 4 + 2 * cfg.batch * cfg.D * 3 * W._esize(cfg.dtype) if cv else 0),
           "dtype": cfg.dtype, "parity": None, "cpu": None}
    if not args.no_cpu:
        import oracle
        o = oracle.get()
        sel = np.arange(0, cfg.D, 16)  # a bounded sample: every 16th channel
        st64 = np.ascontiguousarray(base["state"][:, sel], dtype=np.float64)
        win64 = W.storage_to_f64(base["conv_state"][:, sel], cfg.dtype) if cv else None
        reps, tot, prev = 0, 0.0, None
        while reps == 0 or (tot < args.cpu_seconds and reps < cfg.steps):
            tk = W.step_token_inputs(cfg, reps, channels=sel, raw_delta=sp, trap=tr)
            t = time.perf_counter()
            if cv:
                o.step_conv(tk, base["A"][sel], base["Dskip"][sel], base["dt_bias"][sel], base["conv_w"][sel],
                            base["conv_b"][sel], win64, st64, cfg.dtype)
            elif sp:
                o.step_dt(tk, base["A"][sel], base["Dskip"][sel], base["dt_bias"][sel], st64, cfg.dtype)
            elif tr:
                o.step_trap(dict(tk, x_prev=None if prev is None else prev["x"],
                                 B_prev=None if prev is None else prev["Bt"]),
                            base["A"][sel], base["Dskip"][sel], st64, cfg.dtype)
                prev = tk
            else:
                o.step(tk, base["A"][sel], base["Dskip"][sel], st64, cfg.dtype)
            tot += time.perf_counter() - t
            reps += 1
        out["cpu"] = {"value": cfg.batch * len(sel) * cfg.N * reps / tot / 1e9, "unit": "G(B*D*N)-elem/s",
                      "cores": o.threads(), "kind": "oracle",
                      "sample": f"{reps} decode steps on every 16th channel ({len(sel)} of {cfg.D}), {tot:.1f}s"}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3", choices=["c0", "c1", "c2", "c3", "c4", "ssd", "ssd_step"])
    ap.add_argument("--rotate", type=int, default=4, help="input/output sets cycled through")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline and parity check")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="oracle time for the CPU baseline and parity sample (default: 20)")
    ap.add_argument("--softplus", action="store_true",
                    help="hand delta over before its activation (ssm_scan_fwd_dt / ssm_step_dt)")
    ap.add_argument("--trap", action="store_true",
                    help="the exponential-trapezoidal rule (ssm_scan_fwd_trap / ssm_step_trap)")
    ap.add_argument("--conv", action="store_true",
                    help="x before the Mamba block's short convolution and SiLU, delta before its activation "
                         "(ssm_scan_fwd_conv)")
    ap.add_argument("--backward", action="store_true",
                    help="time the gradient of the scan (ssm_scan_bwd) instead of the forward")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (counter calibration)")
    ap.add_argument("--valu-calibration", action="store_true",
                    help="only measure the VALU issue rates of exp, fma and the scan's mix")
    args = ap.parse_args()
    if sum((args.softplus, args.trap, args.conv)) > 1:
        ap.error("--softplus, --trap and --conv select different entry points; give one")
    if args.conv and (args.workload in ("ssd", "ssd_step") or (args.backward and args.workload == "c4")):
        ap.error("--conv applies to the scan (c0-c3, forward or --backward) and the decode step (c4)")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the selective scan shards across channels and needs no "
              f"collective on this path, so it is measured on a single MI355X (asked for --gpus "
              f"{args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.valu_calibration:
        valu_calibration()
        return

    if args.backward and args.workload in ("c4", "ssd", "ssd_step"):
        ap.error("--backward times the gradient of the scan (plain, --softplus or --trap) on c0-c3")
    if args.workload in ("ssd", "ssd_step") and (args.softplus or args.trap):
        ap.error("--softplus and --trap apply to the S6 scan and step")
    if args.workload == "ssd":
        r = bench_ssd(args)
    elif args.workload == "ssd_step":
        r = bench_ssd_step(args)
    else:
        r = bench_step(args) if args.workload == "c4" else bench_scan(args, args.workload)
    cfg = r["cfg"]
    ms, launch_ms = r["ms"], r["launch_ms"]
    gbs = r["bytes"] / (launch_ms * 1e-3) / 1e9
    traffic = None if (args.softplus or args.trap) else \
        measured_traffic(args.workload + ("_conv" if args.conv else "") + ("_grad" if args.backward else ""))
    kernel = {"c4": STEP_KERNEL, "ssd": SSD_KERNEL, "ssd_step": "ssd_step_kernel"}.get(args.workload, SCAN_KERNEL)
    hbm = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
           "traffic": traffic, "kernel": kernel,
           "algorithmic_bytes_per_launch": r["bytes"], "launch_us": launch_ms * 1e3}
    mfma = None
    if args.workload == "ssd":
        tf = r["flops"] / (launch_ms * 1e-3) / 1e12
        mfma = {"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tf / MFMA_BF16_PEAK_TFLOPS, "kernel": kernel, "algorithmic_flops_per_launch": r["flops"],
                "launch_us": launch_ms * 1e3}
    alu = None
    if args.workload in ("c4", "ssd", "ssd_step"):
        roof = hbm  # the SSD layer needs more time at the HBM peak than at the matrix-core peak
    elif args.backward:
        # the whole gradient call (all its launches), against the VALU peak
        slots = r["elems"] * BWD_SLOTS_PER_ELEM
        tslots = slots / (launch_ms * 1e-3) / 1e12
        hbm["kernel"] = "ssm_scan_bwd (all launches)"
        roof = {"bound": "alu", "achieved": tslots, "peak": VALU_PEAK_TSLOTS, "unit": "T VALU-slots/s",
                "frac": tslots / VALU_PEAK_TSLOTS, "traffic": traffic, "kernel": "ssm_scan_bwd (all launches)",
                "algorithmic_slots_per_launch": slots, "launch_us": launch_ms * 1e3}
    else:
        # The headline is the HBM roofline, the fraction the target is set on;
        # the VALU roofline, which this kernel meets first (it needs more time
        # at the VALU peak than at the HBM peak), is reported beside it.
        slots = r["elems"] * SCAN_SLOTS_PER_ELEM
        tslots = slots / (launch_ms * 1e-3) / 1e12
        alu = {"bound": "alu", "achieved": tslots, "peak": VALU_PEAK_TSLOTS, "unit": "T VALU-slots/s",
               "frac": tslots / VALU_PEAK_TSLOTS, "kernel": SCAN_KERNEL,
               "algorithmic_slots_per_launch": slots, "launch_us": launch_ms * 1e3}
        roof = hbm
    if args.workload == "ssd":
        config = {"workload": cfg.name, "batch": cfg.batch, "L": cfg.L, "H": cfg.H, "P": cfg.P, "G": cfg.G,
                  "N": cfg.N, "dtype": cfg.dtype, "chunk": 64}
        metric = "ssd-layer G(B*L*H*P*N)-elem/s"
    elif args.workload == "ssd_step":
        config = {"workload": cfg.name, "batch": cfg.batch, "H": cfg.H, "P": cfg.P, "G": cfg.G, "N": cfg.N,
                  "dtype": cfg.dtype, "steps_timed": args.steps}
        metric = "ssd-decode-step G(B*H*P*N)-elem/s"
    elif args.workload == "c4":
        config = {"workload": cfg.name, "batch": cfg.batch, "D": cfg.D, "N": cfg.N, "dtype": cfg.dtype,
                  "gate": cfg.gate, "steps_timed": args.steps}
        if args.softplus or args.conv:
            config["delta"] = "raw: softplus(delta_raw + dt_bias) in the kernel"
        if args.conv:
            config["x"] = "raw: SiLU of the causal width-4 depthwise convolution in the kernel, window updated in place"
        if args.trap:
            config["rule"] = "exponential-trapezoidal, lam per token and channel"
        metric = "decode-step G(B*D*N)-elem/s"
    else:
        config = {"workload": cfg.name, "batch": cfg.batch, "L": cfg.L, "D": cfg.D, "N": cfg.N,
                  "dtype": cfg.dtype, "gate": cfg.gate, "state_in": cfg.state_in is not None}
        if args.softplus or args.conv:
            config["delta"] = "raw: softplus(delta_raw + dt_bias) in the kernel"
        if args.conv:
            config["x"] = "raw: SiLU of the causal width-4 depthwise convolution in the kernel"
        if args.trap:
            config["rule"] = "exponential-trapezoidal, lam per token and channel"
        metric = "selective-scan G(B*L*D*N)-elem/s"
        if args.backward:
            config["pass"] = "gradient (ssm_scan_bwd%s), dstate given" % (
                "_conv" if args.conv else "_dt" if args.softplus else "_trap" if args.trap else "")
            metric = "selective-scan gradient G(B*L*D*N)-elem/s"
    line = {
        "metric": metric,
        "value": r["elems"] / (ms * 1e-3) / 1e9,
        "unit": {"c4": "G(B*D*N)-elem/s", "ssd": "G(B*L*H*P*N)-elem/s",
                 "ssd_step": "G(B*H*P*N)-elem/s"}.get(args.workload, "G(B*L*D*N)-elem/s"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": r.get("data", "synthetic (seeded; recipe in workloads/)"),
        "config": config,
        "hbm_gbs_algorithmic": gbs,
        "roofline": roof,
        "roofline_hbm": hbm,
        "roofline_alu": alu,
        "roofline_mfma": mfma,
        "cpu_baseline": r["cpu"],
        "parity": r["parity"],
        "context": PAGE_CLAIMS,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
