"""The seeded input generators: determinism, chunk independence, recipes (CPU)."""
import numpy as np

import workloads as W


def test_deterministic_and_chunk_independent():
    c = W.ScanConfig("t", 2, 300, 40, 16, "bf16", gate=True, dskip="uniform", state_in=0.1, seed=7)
    a = W.scan_inputs(c)
    a2 = W.scan_inputs(c)
    for k in ("x", "delta", "z", "Bt", "Ct", "A", "Dskip", "state_in"):
        assert np.array_equal(a[k], a2[k]), k
    b = W.scan_inputs(c, 100, 250)
    for k in ("x", "delta", "z", "Bt", "Ct"):
        assert np.array_equal(a[k][:, 100:250], b[k]), k
    sel = np.array([3, 17, 39])
    s = W.scan_inputs(c, channels=sel)
    for k in ("x", "delta", "z"):
        assert np.array_equal(a[k][:, :, sel], s[k]), k
    assert np.array_equal(a["state_in"][:, sel], s["state_in"])
    assert np.array_equal(a["A"][sel], s["A"])


def test_recipe_values():
    c = W.ScanConfig("t", 1, 4000, 64, 16, "f32", gate=False, dskip="one", seed=0)
    a = W.scan_inputs(c)
    assert a["z"] is None and a["state_in"] is None
    assert np.array_equal(a["A"], np.broadcast_to(-(np.arange(16) + 1.0), (64, 16)).astype(np.float32))
    assert np.all(a["Dskip"] == 1.0)
    d = a["delta"].astype(np.float64)
    # softplus(0.5 eps + softplus^-1(dt)), dt in [1e-3, 1e-1]: about 2e-4 .. 0.4
    assert d.min() > 1e-4 and d.max() < 0.6
    for k in ("x", "Bt", "Ct"):
        v = a[k].astype(np.float64)
        assert abs(v.mean()) < 0.05 and abs(v.std() - 1) < 0.05, k


def test_bf16_rounding():
    vals = np.array([1.0, -2.5, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 3.0e38, 1e-40])
    bits = W.bf16_bits_from_f64(vals)
    back = W.storage_to_f64(bits, "bf16")
    assert back[0] == 1.0 and back[1] == -2.5
    assert back[2] == 1.0                    # tie rounds to even
    assert back[3] == 1.0 + 2 ** -7          # above the tie rounds up
    assert np.all(np.abs(back[:5] - vals[:5]) <= np.abs(vals[:5]) * 2 ** -8)


def test_byte_counts_match_workloads():
    assert W.scan_bytes(W.SCAN_CONFIGS["c0"]) == 233_728
    assert W.scan_bytes(W.SCAN_CONFIGS["c1"]) == 101_292_032
    assert W.scan_bytes(W.SCAN_CONFIGS["c2"]) == 1_344_622_592
    assert W.scan_bytes(W.SCAN_CONFIGS["c3"], state_out=True) == 12_952_311_808
    assert W.step_bytes(W.STEP_CONFIG) == 178_622_464


def test_step_inputs():
    c = W.StepConfig("t", 4, 32, 16, "bf16", steps=3, seed=9)
    s = W.step_inputs(c)
    assert s["state"].shape == (4, 32, 16) and s["state"].dtype == np.float32
    t0 = W.step_token_inputs(c, 0)
    t1 = W.step_token_inputs(c, 1)
    assert t0["x"].shape == (4, 32) and t0["Bt"].shape == (4, 16)
    assert not np.array_equal(t0["x"], t1["x"])
    assert np.array_equal(W.step_token_inputs(c, 1)["delta"], t1["delta"])
