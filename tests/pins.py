"""Checks that pin the fp64 oracle to facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
when the oracle disagrees. They are run on the real oracle by
``test_oracle_pins.py`` and on deliberately broken copies of it by
``test_oracle_mutants.py`` (every planted mistake must trip at least one pin).

None of these checks re-types the oracle's loop: each compares it with an
independent statement of the same result (a printed worked example, a closed
form, numpy's convolution, an explicit matrix, the masked-matmul dual form,
an invariant).
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    return rows


def _rand_problem(rng, batch, L, D, N, gate=True, skip=True, state=True, s4d=False):
    A = (-(np.arange(N) + 1.0))[None, :].repeat(D, 0) if s4d else -np.exp(rng.normal(size=(D, N)))
    p = dict(
        x=rng.normal(size=(batch, L, D)),
        delta=np.exp(rng.uniform(np.log(1e-3), np.log(0.5), size=(batch, L, D))),
        A=A,
        Bt=rng.normal(size=(batch, L, N)),
        Ct=rng.normal(size=(batch, L, N)),
        Dskip=rng.uniform(0.5, 1.5, size=D) if skip else None,
        z=rng.normal(size=(batch, L, D)) if gate else None,
        state_in=rng.normal(size=(batch, D, N)) if state else None,
    )
    return p


def _scan(o, p, **kw):
    return o.scan64(p["x"], p["delta"], p["A"], p["Bt"], p["Ct"], p.get("Dskip"), p.get("z"),
                    p.get("state_in"), **kw)


# --- P4: the printed single-step example ------------------------------------
def pin_step_example(o):
    """Worked example: A=-1, B=1, h=1, x=1; delta=5 forgets, delta=0.01 holds."""
    for dt, abar, bbar, hnew in _golden_rows("selective_step_example.txt"):
        N = 4
        A = -np.ones((1, N))
        ones = np.ones((1, 1, N))
        # full step: new state
        _, st = o.scan64(np.ones((1, 1, 1)), np.full((1, 1, 1), dt), A, ones, ones, state_in=ones)
        assert np.all(np.round(st, 4) == hnew), (dt, st)
        # exact value of the same quantity: exp(-dt) + dt
        assert abs(st[0, 0, 0] - (math.exp(-dt) + dt)) <= 1e-15 * (1 + dt), st
        # A-bar alone: B = 0 leaves h = A-bar * 1
        _, st0 = o.scan64(np.ones((1, 1, 1)), np.full((1, 1, 1), dt), A, 0 * ones, ones, state_in=ones)
        assert np.all(np.round(st0, 4) == abar), (dt, st0)
        # B-bar alone: h = 0 before the step gives h = B-bar * x
        _, stb = o.scan64(np.ones((1, 1, 1)), np.full((1, 1, 1), dt), A, ones, ones, state_in=0 * ones)
        assert np.all(np.round(stb, 4) == bbar), (dt, stb)
        # the same example through the single-token decode step
        h = np.ones((1, 1, N))
        y = o.step64(np.ones((1, 1)), np.full((1, 1), dt), A, np.ones((1, N)), np.ones((1, N)), None, None, h)
        assert np.all(np.round(h, 4) == hnew), (dt, h)
        assert abs(h[0, 0, 0] - (math.exp(-dt) + dt)) <= 1e-15 * (1 + dt), h
        assert abs(y[0, 0] - N * h[0, 0, 0]) <= 1e-14 * N * (1 + dt), y


# --- P1: time-invariant case equals convolution ------------------------------
def _conv_reference(A_diag, Bbar, C, x, dt):
    abar = np.exp(dt * A_diag)
    L = len(x)
    K = np.array([C @ (abar ** k * Bbar) for k in range(L)])
    return np.convolve(x, K)[:L]


def pin_lti_convolution(o):
    """Constant delta, B, C and no skip, gate or initial state: y = K * x."""
    seed, N, L, dt, printed = _golden_rows("lti_convolution_demo.txt")[0]
    rng = np.random.default_rng(int(seed))
    N, L = int(N), int(L)
    A = -np.exp(rng.normal(size=N))
    B, C = rng.normal(size=N), rng.normal(size=N)
    x = rng.normal(size=L)
    abar = np.exp(dt * A)
    Bbar = (abar - 1.0) / A * B               # the demo's zero-order-hold B-bar
    # Feed B-bar through the exp-Euler input rule: delta * (Bbar / delta) = Bbar.
    y, _ = o.scan64(x[None, :, None], np.full((1, L, 1), dt), A[None, :],
                    np.broadcast_to(Bbar / dt, (1, L, N)), np.broadcast_to(C, (1, L, N)))
    ref = _conv_reference(A, Bbar, C, x, dt)
    err = np.abs(y[0, :, 0] - ref).max()
    # the page printed `printed` for its own float64 run; this oracle gives 1.67e-16
    assert err <= 10 * printed, err
    # several channels, random constant delta per channel, S4D-real A, B-bar = delta*B
    rng = np.random.default_rng(10)
    D, N, L = 5, 16, 200
    A = (-(np.arange(N) + 1.0))[None, :].repeat(D, 0)
    dts = np.exp(rng.uniform(np.log(1e-3), np.log(0.3), size=D))
    B, C = rng.normal(size=N), rng.normal(size=N)
    x = rng.normal(size=(L, D))
    y, _ = o.scan64(x[None], np.broadcast_to(dts, (1, L, D)), A,
                    np.broadcast_to(B, (1, L, N)), np.broadcast_to(C, (1, L, N)))
    for d in range(D):
        ref = _conv_reference(A[d], dts[d] * B, C, x[:, d], dts[d])
        assert np.allclose(y[0, :, d], ref, rtol=1e-12, atol=1e-12), d


# --- P2: N = 1 geometric closed form -----------------------------------------
def pin_geometric(o):
    """N=1, constant delta/B/C, x = 1: h_t = a^(t+1) h0 + b (1 - a^(t+1)) / (1 - a)."""
    for dt, Aval, Bv, Cv, Dv, h0 in [(0.05, -1.0, 0.7, -1.3, 0.9, 0.4), (0.3, -2.5, -1.1, 0.6, 1.2, -2.0),
                                     (1e-3, -0.5, 2.0, 1.0, 0.0, 3.0)]:
        L = 300
        y, st = o.scan64(np.ones((1, L, 1)), np.full((1, L, 1), dt), np.array([[Aval]]),
                         np.full((1, L, 1), Bv), np.full((1, L, 1), Cv), np.array([Dv]),
                         state_in=np.array([[[h0]]]))
        a, b = math.exp(dt * Aval), dt * Bv
        t = np.arange(1, L + 1, dtype=np.float64)
        h = a ** t * h0 + b * (1 - a ** t) / (1 - a)
        assert np.allclose(y[0, :, 0], Cv * h + Dv, rtol=1e-11, atol=1e-12)
        assert abs(st[0, 0, 0] - h[-1]) <= 1e-11 * max(1, abs(h[-1]))


# --- P3: delta limits ---------------------------------------------------------
def pin_delta_limits(o):
    """delta = 0 keeps the state bit for bit; a huge delta resets it to delta*B*x."""
    rng = np.random.default_rng(3)
    p = _rand_problem(rng, 2, 40, 3, 16)
    p["delta"] = np.zeros_like(p["delta"])
    y, st = _scan(o, p)
    assert np.array_equal(st, p["state_in"])
    gate = p["z"] / (1 + np.exp(-p["z"]))
    for b in range(2):
        ref = (np.einsum("tn,dn->td", p["Ct"][b], p["state_in"][b]) + p["Dskip"] * p["x"][b]) * gate[b]
        assert np.allclose(y[b], ref, rtol=1e-13, atol=1e-13)
    # huge delta: A-bar underflows, the new state is delta * B * x
    p = _rand_problem(rng, 1, 5, 4, 8, s4d=True)
    p["delta"] = np.full_like(p["delta"], 60.0)
    _, st = _scan(o, p)
    ref = 60.0 * p["Bt"][0, -1][None, :] * p["x"][0, -1][:, None]
    assert np.allclose(st[0], ref, rtol=1e-14, atol=0)
    # small delta holds: 0.01 * |A| << 1, state moves by O(delta)
    p = _rand_problem(rng, 1, 1, 4, 8, s4d=True, gate=False, skip=False)
    p["delta"] = np.full_like(p["delta"], 1e-6)
    _, st = _scan(o, p)
    assert np.allclose(st, p["state_in"], rtol=1e-4, atol=1e-4)


# --- P5: brute-force semiseparable sum ---------------------------------------
def pin_semiseparable(o):
    """y_j = sum_{i<=j} C_j^T (prod_{k=i+1..j} Abar_k) Bbar_i x_i + C_j^T (prod_{k<=j} Abar_k) h_-1."""
    rng = np.random.default_rng(5)
    for L in range(1, 9):
        p = _rand_problem(rng, 2, L, 3, 5, gate=False, skip=False)
        y, st = _scan(o, p)
        for b in range(2):
            for d in range(3):
                abar = np.exp(p["delta"][b, :, d, None] * p["A"][d][None, :])        # (L, N)
                bbar = p["delta"][b, :, d, None] * p["Bt"][b]                       # (L, N)
                for j in range(L):
                    tot = 0.0
                    for i in range(j + 1):
                        prod = np.ones(5)
                        for k in range(i + 1, j + 1):
                            prod = prod * abar[k]
                        tot += float(np.sum(p["Ct"][b, j] * prod * bbar[i])) * p["x"][b, i, d]
                    prod = np.ones(5)
                    for k in range(0, j + 1):
                        prod = prod * abar[k]
                    tot += float(np.sum(p["Ct"][b, j] * prod * p["state_in"][b, d]))
                    assert abs(y[b, j, d] - tot) <= 1e-12 * (1 + abs(tot)), (L, b, d, j)
                # final state, the same sums without C
                hend = np.zeros(5)
                for i in range(L):
                    prod = np.ones(5)
                    for k in range(i + 1, L):
                        prod = prod * abar[k]
                    hend += prod * bbar[i] * p["x"][b, i, d]
                prod = np.ones(5)
                for k in range(L):
                    prod = prod * abar[k]
                hend += prod * p["state_in"][b, d]
                assert np.allclose(st[b, d], hend, rtol=1e-12, atol=1e-13)


# --- P7: scalar transition equals the masked (quadratic) dual form -----------
def pin_scalar_a_dual(o):
    """A[d, :] constant: y = (Lmask o C B^T) X, as in the SSD check."""
    seed, L, N, P, printed = _golden_rows("ssd_dual_demo.txt")[0]
    rng = np.random.default_rng(int(seed))
    L, N, P = int(L), int(N), int(P)
    a = rng.uniform(0.85, 0.99, size=L)
    B, C = rng.normal(size=(L, N)), rng.normal(size=(L, N))
    X = rng.normal(size=(L, P))
    # quadratic form written from the definition: Lmask_ji = prod_{k=i+1..j} a_k
    Lmask = np.zeros((L, L))
    for j in range(L):
        for i in range(j + 1):
            Lmask[j, i] = np.prod(a[i + 1:j + 1])
    Yq = (Lmask * (C @ B.T)) @ X
    # the same recurrence through the S6 oracle: a_t = exp(delta_t * (-1)),
    # input term delta_t * (B_t / delta_t) * x_t = B_t x_t, channels = P columns.
    dt = -np.log(a)
    y, _ = o.scan64(X[None], np.broadcast_to(dt[:, None], (1, L, P)), -np.ones((P, N)),
                    (B / dt[:, None])[None], C[None])
    err = np.abs(y[0] - Yq).max()
    assert err <= 10 * printed, err  # this oracle: 1.07e-14 against the printed 9.44e-15
    # longer random case, per-channel scalar A and random delta
    rng = np.random.default_rng(7)
    L, N, D = 256, 16, 4
    Ad = -np.exp(rng.normal(size=D))
    delta = np.exp(rng.uniform(np.log(1e-3), np.log(0.2), size=(L, D)))
    B, C = rng.normal(size=(L, N)), rng.normal(size=(L, N))
    x = rng.normal(size=(L, D))
    y, _ = o.scan64(x[None], delta[None], np.repeat(Ad[:, None], N, 1), B[None], C[None])
    for d in range(D):
        cum = np.cumsum(delta[:, d] * Ad[d])               # log of prod_{k<=j} a_k
        Lmask = np.tril(np.exp(cum[:, None] - cum[None, :]))
        ref = (Lmask * (C @ B.T)) @ (delta[:, d] * x[:, d])
        assert np.allclose(y[0, :, d], ref, rtol=1e-10, atol=1e-10), d


# --- P6: composition of steps and of scans -----------------------------------
def pin_composition(o):
    """A fold of single steps equals the scan; scan(L) = scan(L1) then scan(L-L1)."""
    rng = np.random.default_rng(6)
    p = _rand_problem(rng, 2, 37, 5, 16, s4d=True)
    y, st = _scan(o, p)
    state = p["state_in"].copy()
    for t in range(37):
        yt = o.step64(p["x"][:, t], p["delta"][:, t], p["A"], p["Bt"][:, t], p["Ct"][:, t],
                      p["Dskip"], p["z"][:, t], state)
        assert np.array_equal(yt, y[:, t]), t
    assert np.array_equal(state, st)
    for L1 in (0, 1, 17, 36, 37):
        q1 = {k: (v[:, :L1] if k in ("x", "delta", "Bt", "Ct", "z") else v) for k, v in p.items()}
        q2 = {k: (v[:, L1:] if k in ("x", "delta", "Bt", "Ct", "z") else v) for k, v in p.items()}
        y1, s1 = _scan(o, q1)
        q2["state_in"] = s1
        y2, s2 = _scan(o, q2)
        assert np.array_equal(np.concatenate([y1, y2], 1), y), L1
        assert np.array_equal(s2, st), L1


# --- P8: skip, gate, linearity, causality ------------------------------------
def pin_skip_gate(o):
    """B=0 and h0=0 gives y = D x exactly; z = 0 gives 0; the gate is silu(z)."""
    import torch
    rng = np.random.default_rng(8)
    p = _rand_problem(rng, 2, 30, 6, 16, gate=False, state=False)
    p["Bt"] = np.zeros_like(p["Bt"])
    y, st = _scan(o, p)
    assert np.array_equal(y, p["Dskip"] * p["x"])
    assert not st.any()
    # the gate multiplies (C.h + D.x): with B = 0, y = D x silu(z)
    p["z"] = rng.normal(size=p["x"].shape) * 3
    y, _ = _scan(o, p)
    silu = torch.nn.functional.silu(torch.from_numpy(p["z"])).numpy()
    assert np.allclose(y, p["Dskip"] * p["x"] * silu, rtol=1e-14, atol=1e-15)
    p["z"] = np.zeros_like(p["z"])
    p["Bt"] = rng.normal(size=p["Bt"].shape)
    y, _ = _scan(o, p)
    assert not y.any()
    # no skip term: x enters only through B
    p = _rand_problem(rng, 1, 10, 3, 8, gate=False, skip=False, state=False)
    p["Bt"] = np.zeros_like(p["Bt"])
    y, _ = _scan(o, p)
    assert not y.any()


def pin_linearity_causality(o):
    """Gate off: y is linear in (x, h0); nothing at t > t0 changes y[:t0+1]."""
    rng = np.random.default_rng(9)
    p = _rand_problem(rng, 2, 50, 4, 16, gate=False)
    q = dict(p)
    q["x"] = rng.normal(size=p["x"].shape)
    q["state_in"] = rng.normal(size=p["state_in"].shape)
    a, b = 0.7, -1.9
    r = dict(p)
    r["x"] = a * p["x"] + b * q["x"]
    r["state_in"] = a * p["state_in"] + b * q["state_in"]
    yp, sp = _scan(o, p)
    yq, sq = _scan(o, q)
    yr, sr = _scan(o, r)
    assert np.allclose(yr, a * yp + b * yq, rtol=1e-11, atol=1e-11)
    assert np.allclose(sr, a * sp + b * sq, rtol=1e-11, atol=1e-11)
    # causality
    p = _rand_problem(rng, 2, 50, 4, 16)
    y0, _ = _scan(o, p)
    t0 = 20
    for k in ("x", "delta", "Bt", "Ct", "z"):
        pk = dict(p)
        pk[k] = p[k].copy()
        pk[k][:, t0 + 1:] = pk[k][:, t0 + 1:] * 1.5 + 0.25
        yk, _ = _scan(o, pk)
        assert np.array_equal(yk[:, :t0 + 1], y0[:, :t0 + 1]), k
        assert not np.array_equal(yk[:, t0 + 1:], y0[:, t0 + 1:]), k


def pin_entering_state_decay(o):
    """The scan's dependence on its entering state in closed form ("Notas sobre
    Mamba", "O mecanismo de seleção (S6)": each update multiplies the state by
    exp(delta_t A) before adding the input, so the map is affine in h_0). With
    the same inputs, y from h_in minus y from a zero start is, at token t,
    silu(z_t) * sum_n Ct[t, n] exp(A[d, n] * sum_{s<=t} delta_s[d]) h_in[d, n]
    (the readout sees the state after token t's update), and the final states
    differ by exp(A * sum delta) h_in. The stripe scan's early stop (a walk from
    zero whose y stands once this term is below rounding) rests on it."""
    rng = np.random.default_rng(17)
    p = _rand_problem(rng, 2, 300, 5, 16, s4d=True)  # A = -(n+1); gate, skip and entering state on
    q = dict(p)
    q["state_in"] = None
    yp, sp = _scan(o, p)
    yq, sq = _scan(o, q)
    cum = np.cumsum(p["delta"], axis=1)  # inclusive: token t's own step counts
    decay = np.exp(cum[..., None] * p["A"][None, None])  # (batch, L, D, N)
    carried = decay * p["state_in"][:, None]
    z = p["z"]
    want = np.einsum("bln,bldn->bld", p["Ct"], carried) * (z / (1.0 + np.exp(-z)))
    assert np.allclose(yp - yq, want, rtol=1e-9, atol=1e-12)
    assert np.allclose(sp - sq, carried[:, -1], rtol=1e-9, atol=1e-12)
    # and it vanishes: far enough into the sequence the two runs agree to rounding
    assert np.max(np.abs(want[:, -1])) < 1e-3 * np.max(np.abs(want[:, 0]))


def pin_softplus_activation(o):
    """Step-size activation delta = softplus(raw + dt_bias[d]) ("Notas sobre
    Mamba", section "O mecanismo de seleção (S6)"): against closed forms, the
    identity softplus(u) - softplus(-u) = u, numpy's logaddexp(0, u), the
    per-channel broadcast of the bias, and a scan on that activated delta."""
    ln2 = math.log(2.0)
    assert abs(o.softplus_bias64(np.zeros((1, 1)))[0, 0] - ln2) <= 1e-16
    u = np.concatenate([np.linspace(-60, 60, 241), [-700.0, -36.5, -1e-9, 1e-9, 36.5, 700.0]])[None, :]
    sp = o.softplus_bias64(u)
    ref = np.logaddexp(0.0, u)
    assert np.all(np.abs(sp - ref) <= 4e-16 * np.maximum(np.abs(ref), 1e-300) + 1e-300), "softplus vs logaddexp"
    assert np.allclose(sp - o.softplus_bias64(-u), u, rtol=0, atol=1e-13), "softplus(u) - softplus(-u) = u"
    assert abs(o.softplus_bias64(np.array([[-50.0]]))[0, 0] / math.exp(-50.0) - 1.0) < 1e-15, "left tail exp(u)"
    rng = np.random.default_rng(7)
    raw = rng.normal(size=(6, 11)) * 3.0
    bias = rng.normal(size=11)
    got = o.softplus_bias64(raw, bias)
    assert np.allclose(got, np.logaddexp(0.0, raw + bias[None, :]), rtol=1e-15, atol=0), "bias per channel"
    # a scan on the activated step equals the scan with delta given directly
    p = _rand_problem(rng, 2, 9, 5, 4)
    draw = rng.normal(size=p["x"].shape) * 0.5
    db = np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=5))))  # inverse softplus of dt
    d_act = o.softplus_bias64(draw, db)
    assert np.allclose(d_act, np.logaddexp(0.0, draw + db[None, None, :]), rtol=1e-15, atol=0)
    q = dict(p, delta=np.logaddexp(0.0, draw + db[None, None, :]))
    y1, s1 = _scan(o, dict(p, delta=d_act))
    y2, s2 = _scan(o, q)
    assert np.allclose(y1, y2, rtol=1e-13, atol=1e-14) and np.allclose(s1, s2, rtol=1e-13, atol=1e-14)


# --- the x branch ahead of the scan (NEXT-1's convolution) ------------------
def pin_conv_silu(o):
    """Short causal depthwise convolution (4 taps) and SiLU ahead of the scan
    ("Notas sobre Mamba", section "O bloco Mamba"; d_conv = 4 in the Mamba-2
    layer configuration of the SSD production blog post): against numpy's
    convolution per channel, SiLU through the identity sigmoid(u) = (1 +
    tanh(u / 2)) / 2 and printed values, causality with a support of exactly
    4 tokens, and resumption from the raw x of the three tokens before."""
    silu = lambda u: u * 0.5 * (1.0 + np.tanh(0.5 * u))
    rng = np.random.default_rng(11)
    batch, L, D = 2, 13, 5
    x = rng.normal(size=(batch, L, D))
    w = rng.uniform(-0.5, 0.5, size=(D, 4))
    cb = rng.uniform(-0.5, 0.5, size=D)
    st = rng.normal(size=(batch, D, 3))
    for state in (None, st):
        got = o.conv_silu64(x, w, cb, state)
        for b in range(batch):
            for d in range(D):
                head = np.zeros(3) if state is None else state[b, d]
                xpad = np.concatenate([head, x[b, :, d]])
                # cross-correlation: tap 3 on the token itself, tap 0 three tokens back
                u = np.convolve(xpad, w[d, ::-1], mode="valid") + cb[d]
                assert u.shape == (L,)
                assert np.allclose(got[b, :, d], silu(u), rtol=1e-14, atol=1e-15), (state is None, b, d)
    # printed values of silu through the identity tap: silu(1), silu(-1), silu(0)
    ident = np.zeros((1, 4))
    ident[0, 3] = 1.0
    v = o.conv_silu64(np.array([[[1.0], [-1.0], [0.0], [40.0]]]), ident)[0, :, 0]
    assert abs(v[0] - 0.7310585786300049) <= 2e-16 and abs(v[1] + 0.2689414213699951) <= 2e-16
    assert v[2] == 0.0 and abs(v[3] - 40.0) < 1e-15
    # causality and support: a change at token t0 moves outputs t0..t0+3 only
    base = o.conv_silu64(x, w, cb)
    t0 = 5
    x2 = x.copy()
    x2[:, t0, :] += 1.0
    moved = o.conv_silu64(x2, w, cb)
    assert np.array_equal(moved[:, :t0], base[:, :t0]) and np.array_equal(moved[:, t0 + 4:], base[:, t0 + 4:])
    assert np.all(moved[:, t0:t0 + 4] != base[:, t0:t0 + 4])
    # resumption: the second part with the last three raw tokens of the first
    L1 = 7
    first = o.conv_silu64(x[:, :L1], w, cb, st)
    second = o.conv_silu64(x[:, L1:], w, cb, np.ascontiguousarray(x[:, L1 - 3:L1].transpose(0, 2, 1)))
    whole = o.conv_silu64(x, w, cb, st)
    assert np.array_equal(np.concatenate([first, second], axis=1), whole)


def pin_conv_silu_bwd(o):
    """Gradient of the x branch: every element of the gradients of the raw x,
    the taps, the bias and the earlier raw tokens against central differences
    of the loss sum(g * conv_silu(...)), and, through the whole scan, the
    gradients of x_raw and the taps against central differences of the scan's
    loss."""
    rng = np.random.default_rng(12)
    batch, L, D = 2, 7, 3
    x = rng.normal(size=(batch, L, D))
    w = rng.uniform(-0.5, 0.5, size=(D, 4))
    cb = rng.uniform(-0.5, 0.5, size=D)
    st = rng.normal(size=(batch, D, 3))
    g = rng.normal(size=(batch, L, D))
    got = o.conv_silu_bwd64(x, w, cb, st, g)
    loss = lambda xx, ww, bb, ss: float(np.sum(g * o.conv_silu64(xx, ww, bb, ss)))
    eps = 1e-6
    for name, arr, key in (("x", x, "gx"), ("w", w, "gw"), ("b", cb, "gb"), ("state", st, "gstate")):
        for idx in np.ndindex(arr.shape):
            args = {"x": x, "w": w, "b": cb, "state": st}
            hi = {k: v.copy() for k, v in args.items()}
            lo = {k: v.copy() for k, v in args.items()}
            hi[name][idx] += eps
            lo[name][idx] -= eps
            fd = (loss(hi["x"], hi["w"], hi["b"], hi["state"]) - loss(lo["x"], lo["w"], lo["b"], lo["state"])) / (2 * eps)
            assert abs(fd - got[key][idx]) <= 1e-7 * (1 + abs(fd)), (name, idx, fd, got[key][idx])
    # through the scan: inputs as the stored-dtype entry points take them (float32 arrays)
    p = _rand_problem(rng, 1, 6, 3, 4)
    inp = {"x_raw": x[:1, :6].astype(np.float32), "conv_w": w.astype(np.float32), "conv_b": cb.astype(np.float32),
           "conv_state": st[:1].astype(np.float32), "delta_raw": (0.5 * rng.normal(size=(1, 6, 3))).astype(np.float32),
           "dt_bias": rng.normal(size=3).astype(np.float32) * 0.1, "A": p["A"].astype(np.float32),
           "Bt": p["Bt"].astype(np.float32), "Ct": p["Ct"].astype(np.float32),
           "Dskip": p["Dskip"].astype(np.float32), "z": p["z"].astype(np.float32),
           "state_in": p["state_in"].astype(np.float32)}
    dy = rng.normal(size=(1, 6, 3)).astype(np.float32)
    dst = rng.normal(size=(1, 3, 4)).astype(np.float32)
    gr = o.scan_bwd_conv(inp, dy, dst, "f32")

    def scan_loss(q):
        y, sfin = o.scan_conv(q, "f32")
        return float(np.sum(dy.astype(np.float64) * y) + np.sum(dst.astype(np.float64) * sfin))
    for key, gkey in (("x_raw", "dx_raw"), ("conv_w", "dconv_w"), ("conv_state", "dconv_state")):
        for idx in list(np.ndindex(inp[key].shape))[::3]:
            base = inp[key][idx]
            h = 1e-3 * max(1.0, abs(float(base)))
            qa, qb = dict(inp), dict(inp)
            qa[key], qb[key] = inp[key].copy(), inp[key].copy()
            qa[key][idx] = np.float32(base + h)
            qb[key][idx] = np.float32(base - h)
            step = float(qa[key][idx]) - float(qb[key][idx])
            fd = (scan_loss(qa) - scan_loss(qb)) / step
            assert abs(fd - gr[gkey][idx]) <= 1e-4 * (1 + abs(fd)), (key, idx, fd, gr[gkey][idx])


# --- the exponential-trapezoidal variant ------------------------------------
def _trap(o, p, lam, **kw):
    return o.scan_trap64(p["x"], p["delta"], lam, p["A"], p["Bt"], p["Ct"], p.get("Dskip"), p.get("z"),
                         p.get("x_prev"), p.get("B_prev"), p.get("state_in"), **kw)


def _states_one_channel(fn, N, L):
    """h_t[n] for every t and n of a one-channel scan: one run per n with the
    readout vector Ct = e_n, so that y_t = h_t[n] exactly."""
    H = np.empty((L, N))
    for n in range(N):
        C = np.zeros((1, L, N))
        C[0, :, n] = 1.0
        H[:, n] = fn(C)[0][0, :, 0]
    return H


def pin_trap_pages_example(o):
    """The pages' seeded comparison of the two rules ("Notas sobre Mamba",
    section "Recorrência trapezoidal"): lambda = 1 gives the exponential-Euler
    states back, lambda = 1/2 departs from them by the printed 1.50."""
    for seed, L, N, lam, printed in _golden_rows("trapezoid_demo.txt"):
        rng = np.random.default_rng(int(seed))
        L, N = int(L), int(N)
        A = -np.exp(rng.normal(size=N))
        B = rng.normal(size=(L, N))
        x = rng.normal(size=L)
        delta = np.exp(rng.normal(size=L) * 0.3)
        args = (x[None, :, None], delta[None, :, None])
        euler = _states_one_channel(lambda C: o.scan64(*args, A[None, :], B[None], C), N, L)
        trap = _states_one_channel(
            lambda C: o.scan_trap64(*args, np.full((1, L, 1), lam), A[None, :], B[None], C), N, L)
        err = np.abs(trap - euler).max()
        if lam == 1.0:
            assert err <= 10 * printed, err   # rounding order only
        else:
            assert abs(err - printed) < 0.005, err  # the printed three digits


def pin_trap_lambda_one_is_euler(o):
    """lambda = 1 removes the previous-token term: the exponential-Euler scan,
    with every optional part and an earlier input given (which must then be
    ignored)."""
    rng = np.random.default_rng(31)
    p = _rand_problem(rng, 2, 37, 5, 4)
    p["x_prev"], p["B_prev"] = rng.normal(size=(2, 5)), rng.normal(size=(2, 4))
    y1, s1 = _trap(o, p, np.ones_like(p["x"]))
    y2, s2 = _scan(o, p)
    assert np.allclose(y1, y2, rtol=1e-12, atol=1e-13) and np.allclose(s1, s2, rtol=1e-12, atol=1e-13)


def pin_trap_classic_convolution(o):
    """Constant delta, lambda = 1/2, constant B and C, no earlier input: the
    classic trapezoidal rule on the exponential. Unrolled, token t-k enters
    h_t with weight delta/2 for k = 0 and delta * Abar^k for k >= 1, so y is
    numpy's convolution of x with sum_n C_n B_n K_k[n]."""
    rng = np.random.default_rng(12)
    D, N, L = 3, 4, 120
    A = -np.exp(rng.normal(size=(D, N)))
    dts = np.exp(rng.uniform(np.log(1e-2), np.log(0.5), size=D))
    B, C = rng.normal(size=N), rng.normal(size=N)
    x = rng.normal(size=(L, D))
    y, _ = o.scan_trap64(x[None], np.broadcast_to(dts, (1, L, D)), np.full((1, L, D), 0.5), A,
                         np.broadcast_to(B, (1, L, N)), np.broadcast_to(C, (1, L, N)))
    k = np.arange(L)[:, None]
    for d in range(D):
        K = dts[d] * np.exp(dts[d] * A[d])[None, :] ** k      # (L, N): delta * Abar^k
        K[0] = dts[d] / 2.0
        kappa = (K * (C * B)[None, :]).sum(1)
        ref = np.convolve(x[:, d], kappa)[:L]
        assert np.allclose(y[0, :, d], ref, rtol=1e-11, atol=1e-12), d


def pin_trap_second_order(o):
    """The rule integrates h' = a h + x(s) with x(s) = cos(s), h(0) = 0 at
    second order for lambda = 1/2 (error ratio about 4 when the step halves)
    and at first order for lambda = 1 (ratio about 2). Token t sits at time
    (t + 1) * delta, and the input before token 0 is x(0) = 1, passed as the
    earlier token; the exact value is h(T) = (sin T - a cos T + a e^(aT)) / (a^2 + 1)."""
    a, T = -0.7, 4.0
    exact = (math.sin(T) - a * math.cos(T) + a * math.exp(a * T)) / (a * a + 1.0)
    errs = {0.5: [], 1.0: []}
    for L in (40, 80, 160):
        dt = T / L
        x = np.cos(dt * (np.arange(L) + 1.0))[None, :, None]
        ones = np.ones((1, L, 1))
        for lam in errs:
            y, _ = o.scan_trap64(x, ones * dt, ones * lam, np.array([[a]]), ones, ones,
                                 x_prev=np.ones((1, 1)), B_prev=np.ones((1, 1)))
            errs[lam].append(abs(y[0, -1, 0] - exact))
    for lam, order in ((0.5, 4.0), (1.0, 2.0)):
        e = errs[lam]
        for r in (e[0] / e[1], e[1] / e[2]):
            assert abs(r / order - 1.0) < 0.1, (lam, e)


def pin_trap_brute_force(o):
    """Tiny inputs against the unrolled sum: h_t = (prod_{r<=t} Abar_r) h_in +
    sum_{s<=t} (prod_{s<r<=t} Abar_r) (gamma_s v_s + beta_s v_{s-1}), with a
    random lambda per token and channel, an earlier input and every optional
    part."""
    rng = np.random.default_rng(5)
    batch, L, D, N = 2, 6, 3, 2
    p = _rand_problem(rng, batch, L, D, N)
    p["x_prev"], p["B_prev"] = rng.normal(size=(batch, D)), rng.normal(size=(batch, N))
    lam = rng.uniform(0.0, 1.0, size=(batch, L, D))
    y, st = _trap(o, p, lam)
    for b in range(batch):
        for d in range(D):
            abar = np.exp(p["delta"][b, :, d][:, None] * p["A"][d][None, :])       # (L, N)
            v = p["Bt"][b] * p["x"][b, :, d][:, None]                                # (L, N)
            vprev = np.vstack([p["B_prev"][b] * p["x_prev"][b, d], v[:-1]])
            w = (lam[b, :, d] * p["delta"][b, :, d])[:, None] * v +                 ((1.0 - lam[b, :, d]) * p["delta"][b, :, d])[:, None] * abar * vprev
            for t in range(L):
                h = np.prod(abar[:t + 1], axis=0) * p["state_in"][b, d]
                for s_ in range(t + 1):
                    h = h + np.prod(abar[s_ + 1:t + 1], axis=0) * w[s_]
                yt = (p["Ct"][b, t] * h).sum() + p["Dskip"][d] * p["x"][b, t, d]
                g = p["z"][b, t, d]
                yt *= g / (1.0 + math.exp(-g))
                assert abs(y[b, t, d] - yt) <= 1e-12 * (1 + abs(yt)), (b, t, d)
            assert np.allclose(st[b, d], h, rtol=1e-12, atol=1e-13)


def pin_trap_composition(o):
    """Resuming: a scan cut at token m, the second part given the first part's
    final state and its last token as the earlier input, equals one scan; and
    L decode steps, each given the previous token, equal the scan."""
    rng = np.random.default_rng(8)
    batch, L, D, N = 2, 23, 4, 3
    p = _rand_problem(rng, batch, L, D, N)
    p["x_prev"], p["B_prev"] = rng.normal(size=(batch, D)), rng.normal(size=(batch, N))
    lam = rng.uniform(0.0, 1.0, size=(batch, L, D))
    y, st = _trap(o, p, lam)
    m = 9
    cut = lambda a, sl: None if a is None else a[:, sl]
    p1 = dict(p, x=p["x"][:, :m], delta=p["delta"][:, :m], Bt=p["Bt"][:, :m], Ct=p["Ct"][:, :m], z=cut(p["z"], slice(0, m)))
    y1, s1 = _trap(o, p1, lam[:, :m])
    p2 = dict(p, x=p["x"][:, m:], delta=p["delta"][:, m:], Bt=p["Bt"][:, m:], Ct=p["Ct"][:, m:], z=cut(p["z"], slice(m, L)),
              state_in=s1, x_prev=p["x"][:, m - 1], B_prev=p["Bt"][:, m - 1])
    y2, s2 = _trap(o, p2, lam[:, m:])
    assert np.allclose(np.concatenate([y1, y2], 1), y, rtol=1e-12, atol=1e-13)
    assert np.allclose(s2, st, rtol=1e-12, atol=1e-13)
    state = np.ascontiguousarray(p["state_in"], dtype=np.float64).copy()
    xp, bp = p["x_prev"], p["B_prev"]
    for t in range(L):
        yt = o.step_trap64(p["x"][:, t], p["delta"][:, t], lam[:, t], p["A"], p["Bt"][:, t], p["Ct"][:, t],
                           p["Dskip"], p["z"][:, t], xp, bp, state)
        assert np.allclose(yt, y[:, t], rtol=1e-12, atol=1e-13), t
        xp, bp = p["x"][:, t], p["Bt"][:, t]
    assert np.allclose(state, st, rtol=1e-12, atol=1e-13)


# --- the Mamba-2 SSD layer -----------------------------------------------------
def pin_ssd_pages_dual(o):
    """The pages' check of the SSD dual ("Notas sobre Mamba", section "A forma
    dual: atenção mascarada"): the (P, N)-state recurrence of the SSD oracle
    equals the quadratic masked form (Lmask o C B^T) X, to the printed 9.44e-15
    (within 10x, as the rounding order differs)."""
    seed, L, N, P, printed = _golden_rows("ssd_dual_demo.txt")[0]
    rng = np.random.default_rng(int(seed))
    L, N, P = int(L), int(N), int(P)
    a = rng.uniform(0.85, 0.99, size=L)
    B, C = rng.normal(size=(L, N)), rng.normal(size=(L, N))
    X = rng.normal(size=(L, P))
    Lmask = np.zeros((L, L))
    for j in range(L):
        for i in range(j + 1):
            Lmask[j, i] = np.prod(a[i + 1:j + 1])
    Yq = (Lmask * (C @ B.T)) @ X
    # a_t = exp(delta_t * A) with A = -1; the input term delta_t x_t B_t = X_t B_t
    dt = -np.log(a)
    y, _ = o.ssd64((X / dt[:, None])[None, :, None, :], dt[None, :, None], np.array([-1.0]),
                   B[None, :, None, :], C[None, :, None, :])
    err = np.abs(y[0, :, 0, :] - Yq).max()
    assert err <= 10 * printed, err


def pin_ssd_is_scalar_a_s6(o):
    """Head dimension P = 1, one head per channel: the S6 scan with A[d, :]
    equal to the head's scalar (the restriction the SSD layer makes), with the
    skip term and a carried-in state."""
    rng = np.random.default_rng(21)
    batch, L, H, N = 2, 40, 5, 6
    p = _rand_problem(rng, batch, L, H, N, gate=False)
    Ah = -np.exp(rng.normal(size=H))
    p["A"] = np.repeat(Ah[:, None], N, 1)
    y6, s6 = _scan(o, p)
    y, st = o.ssd64(p["x"][..., None], p["delta"], Ah, p["Bt"][:, :, None, :], p["Ct"][:, :, None, :],
                    p["Dskip"], p["state_in"][:, :, None, :])
    assert np.allclose(y[..., 0], y6, rtol=1e-12, atol=1e-13)
    assert np.allclose(st[:, :, 0, :], s6, rtol=1e-12, atol=1e-13)


def pin_ssd_brute_force(o):
    """Tiny inputs with several heads per group against the explicit sum
    y_t[p] = sum_{i<=t} (prod_{i<k<=t} a_k) (C_t . B_i) delta_i x_i[p]
             + (prod_{k<=t} a_k) C_t . S0[p] + D x_t[p]."""
    rng = np.random.default_rng(22)
    batch, L, H, P, G, N = 2, 6, 4, 3, 2, 2
    x = rng.normal(size=(batch, L, H, P))
    dl = np.exp(rng.uniform(np.log(0.05), np.log(1.0), size=(batch, L, H)))
    A = -np.exp(rng.normal(size=H))
    B, C = rng.normal(size=(batch, L, G, N)), rng.normal(size=(batch, L, G, N))
    Dk = rng.uniform(0.5, 1.5, size=H)
    S0 = rng.normal(size=(batch, H, P, N))
    y, st = o.ssd64(x, dl, A, B, C, Dk, S0)
    for b in range(batch):
        for h in range(H):
            g = h // (H // G)
            a = np.exp(dl[b, :, h] * A[h])
            for t in range(L):
                ref = np.prod(a[:t + 1]) * (S0[b, h] @ C[b, t, g]) + Dk[h] * x[b, t, h]
                for i in range(t + 1):
                    ref = ref + np.prod(a[i + 1:t + 1]) * (C[b, t, g] @ B[b, i, g]) * dl[b, i, h] * x[b, i, h]
                assert np.allclose(y[b, t, h], ref, rtol=1e-12, atol=1e-12), (b, t, h)
            fin = np.prod(a) * S0[b, h]
            for i in range(L):
                fin = fin + np.prod(a[i + 1:]) * dl[b, i, h] * np.outer(x[b, i, h], B[b, i, g])
            assert np.allclose(st[b, h], fin, rtol=1e-12, atol=1e-12)


def pin_ssd_resume(o):
    """A sequence cut in two, the second part started from the first part's
    final state, equals one call."""
    rng = np.random.default_rng(23)
    batch, L, H, P, G, N = 2, 29, 4, 5, 2, 3
    x = rng.normal(size=(batch, L, H, P))
    dl = np.exp(rng.uniform(np.log(1e-3), np.log(0.5), size=(batch, L, H)))
    A = -np.exp(rng.normal(size=H))
    B, C = rng.normal(size=(batch, L, G, N)), rng.normal(size=(batch, L, G, N))
    S0 = rng.normal(size=(batch, H, P, N))
    y, st = o.ssd64(x, dl, A, B, C, None, S0)
    m = 11
    y1, s1 = o.ssd64(x[:, :m], dl[:, :m], A, B[:, :m], C[:, :m], None, S0)
    y2, s2 = o.ssd64(x[:, m:], dl[:, m:], A, B[:, m:], C[:, m:], None, s1)
    assert np.allclose(np.concatenate([y1, y2], 1), y, rtol=1e-12, atol=1e-13)
    assert np.allclose(s2, st, rtol=1e-12, atol=1e-13)


# --- the scan's gradient -------------------------------------------------------
def _loss(o, p, dy, dstate):
    y, st = _scan(o, p)
    return float(np.sum(y * dy) + np.sum(st * dstate))


def pin_bwd_finite_differences(o):
    """Every gradient of the backward oracle against central differences of the
    forward oracle's loss sum(dy * y) + sum(dstate * state_out), element by
    element, on a tiny problem with every optional part."""
    rng = np.random.default_rng(41)
    batch, L, D, N = 2, 6, 3, 4
    p = _rand_problem(rng, batch, L, D, N)
    dy, dstate = rng.normal(size=(batch, L, D)), rng.normal(size=(batch, D, N))
    g = o.scan_bwd64(p["x"], p["delta"], p["A"], p["Bt"], p["Ct"], p["Dskip"], p["z"], p["state_in"], dy, dstate)
    names = {"x": "dx", "delta": "ddelta", "A": "dA", "Bt": "dBt", "Ct": "dCt", "Dskip": "dDskip", "z": "dz",
             "state_in": "dstate_in"}
    for k, gk in names.items():
        base = p[k]
        num = np.empty_like(base)
        for i in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[i]))
            q = dict(p)
            q[k] = base.copy()
            q[k][i] = base[i] + eps
            up = _loss(o, q, dy, dstate)
            q[k][i] = base[i] - eps
            dn = _loss(o, q, dy, dstate)
            num[i] = (up - dn) / (2 * eps)
        assert np.allclose(g[gk], num, rtol=1e-6, atol=1e-7), (k, np.abs(g[gk] - num).max())


def pin_bwd_dt_finite_differences(o):
    """The gradient through the step-size activation (delta = softplus(delta_raw
    + dt_bias)): ddelta_raw and ddt_bias against central differences of the
    loss of the forward oracle run on the activated step, and dx against the
    plain gradient at that step; at raw + bias = 0 the factor is sigmoid(0) = 1/2."""
    rng = np.random.default_rng(43)
    batch, L, D, N = 2, 5, 3, 4
    p = _rand_problem(rng, batch, L, D, N)
    raw = rng.normal(scale=1.5, size=(batch, L, D))
    raw[0, 0, 0] = -0.25
    bias = rng.normal(size=D)
    bias[0] = 0.25  # raw + bias = 0 at (0, 0, 0)
    dy, dstate = rng.normal(size=(batch, L, D)), rng.normal(size=(batch, D, N))

    def loss(r, bv):
        return _loss(o, dict(p, delta=o.softplus_bias64(r, bv)), dy, dstate)

    g = o.scan_bwd_dt64(p["x"], raw, bias, p["A"], p["Bt"], p["Ct"], p["Dskip"], p["z"], p["state_in"], dy, dstate)
    for name, base, gk in (("raw", raw, "ddelta_raw"), ("bias", bias, "ddt_bias")):
        num = np.empty_like(base)
        for i in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[i]))
            a, b_ = base.copy(), base.copy()
            a[i] += eps
            b_[i] -= eps
            up = loss(a, bias) if name == "raw" else loss(raw, a)
            dn = loss(b_, bias) if name == "raw" else loss(raw, b_)
            num[i] = (up - dn) / (2 * eps)
        assert np.allclose(g[gk], num, rtol=1e-6, atol=1e-7), (name, np.abs(g[gk] - num).max())
    plain = o.scan_bwd64(p["x"], o.softplus_bias64(raw, bias), p["A"], p["Bt"], p["Ct"], p["Dskip"], p["z"],
                         p["state_in"], dy, dstate)
    assert np.array_equal(g["dx"], plain["dx"]) and np.array_equal(g["dA"], plain["dA"])
    assert g["ddelta_raw"][0, 0, 0] == plain["ddelta"][0, 0, 0] / 2.0


def pin_bwd_trap_finite_differences(o):
    """The trapezoidal rule's gradient: every element of every gradient (dlam,
    dx_prev and dB_prev included) against central differences of the loss of
    the trapezoidal forward oracle, on a tiny problem with every optional part
    and an earlier token; with lam = 1 it equals the Euler gradient, and the
    earlier token gets none."""
    rng = np.random.default_rng(44)
    batch, L, D, N = 2, 5, 3, 4
    p = _rand_problem(rng, batch, L, D, N)
    p["lam"] = rng.uniform(0.0, 1.0, size=(batch, L, D))
    p["x_prev"], p["B_prev"] = rng.normal(size=(batch, D)), rng.normal(size=(batch, N))
    dy, dstate = rng.normal(size=(batch, L, D)), rng.normal(size=(batch, D, N))

    def loss(q):
        y, st = o.scan_trap64(q["x"], q["delta"], q["lam"], q["A"], q["Bt"], q["Ct"], q["Dskip"], q["z"],
                              q["x_prev"], q["B_prev"], q["state_in"])
        return float(np.sum(y * dy) + np.sum(st * dstate))

    def grads(q):
        return o.scan_bwd_trap64(q["x"], q["delta"], q["lam"], q["A"], q["Bt"], q["Ct"], q["Dskip"], q["z"],
                                 q["x_prev"], q["B_prev"], q["state_in"], dy, dstate)

    g = grads(p)
    names = {"x": "dx", "delta": "ddelta", "lam": "dlam", "A": "dA", "Bt": "dBt", "Ct": "dCt", "Dskip": "dDskip",
             "z": "dz", "x_prev": "dx_prev", "B_prev": "dB_prev", "state_in": "dstate_in"}
    for k, gk in names.items():
        base = p[k]
        num = np.empty_like(base)
        for i in np.ndindex(base.shape):
            eps = 1e-6 * max(1.0, abs(base[i]))
            q = dict(p)
            q[k] = base.copy()
            q[k][i] = base[i] + eps
            up = loss(q)
            q[k][i] = base[i] - eps
            num[i] = (up - loss(q)) / (2 * eps)
        assert np.allclose(g[gk], num, rtol=1e-6, atol=1e-7), (k, np.abs(g[gk] - num).max())
    one = grads(dict(p, lam=np.ones_like(p["lam"])))
    euler = o.scan_bwd64(p["x"], p["delta"], p["A"], p["Bt"], p["Ct"], p["Dskip"], p["z"], p["state_in"], dy, dstate)
    for k in ("dx", "ddelta", "dA", "dBt", "dCt", "dDskip", "dz", "dstate_in"):
        assert np.allclose(one[k], euler[k], rtol=1e-12, atol=1e-12), k
    assert not one["dx_prev"].any() and not one["dB_prev"].any()


def pin_bwd_adjoint_identities(o):
    """y is linear in x (zero carried-in state), and, without the skip term,
    in Bt, in Ct and in the carried-in state (x = 0 for the last): for each,
    <dy, J v> = <J^T dy, v> exactly, which pins dx, dBt, dCt and dstate_in to
    rounding at a larger size."""
    rng = np.random.default_rng(42)
    batch, L, D, N = 2, 40, 5, 6
    p = _rand_problem(rng, batch, L, D, N, state=False)
    dy = rng.normal(size=(batch, L, D))
    for k, gk, skip in (("x", "dx", True), ("Bt", "dBt", False), ("Ct", "dCt", False)):
        q = dict(p, Dskip=p["Dskip"] if skip else None)
        g = o.scan_bwd64(q["x"], q["delta"], q["A"], q["Bt"], q["Ct"], q["Dskip"], q["z"], None, dy)
        v = rng.normal(size=p[k].shape)
        q[k] = v
        y, _ = _scan(o, q)
        lhs, rhs = float(np.sum(dy * y)), float(np.sum(g[gk] * v))
        assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs)), (k, lhs, rhs)
    # the carried-in state, with x = 0 (and no skip contribution then)
    q = dict(p, x=np.zeros_like(p["x"]), state_in=rng.normal(size=(batch, D, N)))
    g = o.scan_bwd64(q["x"], q["delta"], q["A"], q["Bt"], q["Ct"], q["Dskip"], q["z"], q["state_in"], dy)
    y, _ = _scan(o, q)
    lhs, rhs = float(np.sum(dy * y)), float(np.sum(g["dstate_in"] * q["state_in"]))
    assert abs(lhs - rhs) <= 1e-10 * (1 + abs(lhs)), (lhs, rhs)


ALL_PINS = [pin_conv_silu, pin_conv_silu_bwd, pin_bwd_trap_finite_differences, pin_bwd_dt_finite_differences, pin_bwd_finite_differences, pin_bwd_adjoint_identities, pin_ssd_pages_dual, pin_ssd_is_scalar_a_s6, pin_ssd_brute_force, pin_ssd_resume,
            pin_trap_pages_example, pin_trap_lambda_one_is_euler, pin_trap_classic_convolution,
            pin_trap_second_order, pin_trap_brute_force, pin_trap_composition, pin_softplus_activation, pin_step_example, pin_lti_convolution, pin_geometric, pin_delta_limits,
            pin_semiseparable, pin_scalar_a_dual, pin_composition, pin_skip_gate,
            pin_linearity_causality, pin_entering_state_decay]
