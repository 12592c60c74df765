"""Pins for the fp64 oracle: each function checks one build of the oracle
(``oracle.oracle.Oracle``) against something other than itself and returns
``(ok, detail)``.  Used by ``test_oracle_pins.py`` on the real oracle and, with
planted mistakes, on mutated builds (every mutant must fail at least one pin).

Page cited (by title): P1 = "Jane Street ML Engineers Map Mamba-2 Recurrent
State Computation to Tensor Cores with cuTile" (disconfirmai.com).
"""
from __future__ import annotations

import json
import os

import numpy as np

from mamba_ssd_scan_chunk_amd.inputs import make_inputs
from oracle import forms
from oracle.oracle import dA_cumsum_ref

HERE = os.path.dirname(os.path.abspath(__file__))
TOL = 1e-12


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.abs(b).max()
    if den == 0:
        return float(np.abs(a).max())
    return float(np.abs(a - b).max() / den)


def _h0(inp, seed=11):
    s = inp.shape
    return np.random.default_rng(seed).standard_normal((s["batch"], s["nheads"], s["dstate"], s["headdim"]))


def pin_semiseparable(o):
    """Brute-force L x L semiseparable matrix (direct decay products) equals the
    recurrence, with groups, skip and an initial state."""
    worst = 0.0
    for (B, L, H, P, N, G, seed) in [(1, 40, 2, 4, 3, 1, 1), (2, 33, 4, 3, 5, 2, 2), (1, 64, 3, 8, 8, 3, 3)]:
        inp = make_inputs(B, L, H, P, N, G, 16, seed=seed, dt_shift=0.5)
        h0 = _h0(inp)
        y, f = o.forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0)
        ys, fs = forms.semiseparable_forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0)
        worst = max(worst, rel(y, ys), rel(f, fs))
    return worst <= TOL, f"max rel err {worst:.3g}"


def pin_zero_decay(o):
    """A = 0: jump formula, state = running sum of dt b x^T (closed form)."""
    inp = make_inputs(2, 37, 3, 5, 4, 1, 8, seed=5, A_override=0.0)
    y, f = o.forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
    yc, fc = forms.zero_decay_closed_form(inp.x, inp.dt, inp.Bm, inp.Cm, inp.D)
    e = max(rel(y, yc), rel(f, fc))
    return e <= TOL, f"max rel err {e:.3g}"


def pin_geometric(o):
    """Scalar constant inputs: geometric series in r = exp(dt A)."""
    L, dt, A, b, c, xv, D = 50, 0.3, -0.7, 1.5, -0.8, 2.0, 0.25
    x = np.full((1, L, 1, 1), xv, np.float32)
    dts = np.full((1, L, 1), dt, np.float32)
    Bm = np.full((1, L, 1, 1), b, np.float32)
    Cm = np.full((1, L, 1, 1), c, np.float32)
    y, f = o.forward(x, dts, np.array([A], np.float32), Bm, Cm, np.array([D], np.float32))
    f64 = lambda v: np.float64(np.float32(v))      # the values the oracle actually sees
    yg, hg = forms.geometric_series(L, f64(dt), f64(A), f64(b), f64(c), f64(xv), f64(D))
    e = max(rel(y[0, :, 0, 0], yg), rel(f.ravel(), [hg]))
    return e <= TOL, f"max rel err {e:.3g}"


def pin_single_token(o):
    """L = 1: y = dt (C.B) x + D x and h = dt B x^T (decay never applies)."""
    inp = make_inputs(2, 1, 3, 4, 5, 1, 1, seed=7)
    y, f = o.forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
    x, dt = inp.x.astype(np.float64), inp.dt.astype(np.float64)
    Bm, Cm, D = inp.Bm.astype(np.float64), inp.Cm.astype(np.float64), inp.D.astype(np.float64)
    cb = np.einsum("bgn,bgn->bg", Cm[:, 0], Bm[:, 0])[:, 0]
    ye = dt[:, 0, :, None] * cb[:, None, None] * x[:, 0] + D[None, :, None] * x[:, 0]
    fe = dt[:, 0, :, None, None] * Bm[:, 0, 0][:, None, :, None] * x[:, 0][:, :, None, :]
    e = max(rel(y[:, 0], ye), rel(f, fe))
    return e <= TOL, f"max rel err {e:.3g}"


def pin_skip_only(o):
    """B = 0 or C = 0: y = D x exactly (bitwise)."""
    inp = make_inputs(1, 20, 2, 3, 4, 1, 4, seed=9)
    ok = True
    for zero in ("Bm", "Cm"):
        args = dict(x=inp.x, dt=inp.dt, A=inp.A, Bm=inp.Bm, Cm=inp.Cm)
        args[zero] = np.zeros_like(args[zero])
        y, _ = o.forward(args["x"], args["dt"], args["A"], args["Bm"], args["Cm"], inp.D)
        ok &= bool(np.array_equal(y, inp.D.astype(np.float64)[None, None, :, None] * inp.x.astype(np.float64)))
    return ok, "y == D x exactly" if ok else "y != D x"


def pin_chunk_invariance(o):
    """The chunked form (cumsum, chunk states, state passing, fused output) at
    every chunk size, ragged ones included, equals the recurrence; Q=1 is the
    recurrence itself and Q=L the full quadratic form."""
    inp = make_inputs(1, 48, 2, 4, 3, 1, 8, seed=13, dt_shift=1.0)
    h0 = _h0(inp)
    y, f = o.forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0)
    worst = 0.0
    for Q in (1, 2, 4, 8, 16, 48, 5, 7, 32):
        r = forms.chunked_forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0, Q=Q)
        worst = max(worst, rel(r["y"], y), rel(r["final"], f))
    return worst <= TOL, f"max rel err {worst:.3g}"


def pin_chunk_intermediates(o):
    """Oracle chunk states (recurrence restarted at zero per chunk) and carried
    states (recurrence read at chunk boundaries) equal the chunked form's S and
    H_in; dA_cumsum_ref equals the chunked form's G."""
    inp = make_inputs(2, 40, 3, 4, 5, 1, 8, seed=17, dt_shift=1.0)
    h0 = _h0(inp)
    worst = 0.0
    for Q in (8, 16, 40):
        r = forms.chunked_forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0, Q=Q)
        S = o.chunk_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, Q)
        Hin, fin = o.carried_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, Q, h0=h0)
        worst = max(worst, rel(S, r["S"]), rel(Hin, r["Hin"]), rel(fin, r["final"]))
        worst = max(worst, rel(dA_cumsum_ref(inp.dt, inp.A, Q), r["G"]))
    return worst <= TOL, f"max rel err {worst:.3g}"


def pin_split_chaining(o):
    """Sequence split: the final state of the first part, fed as the initial
    state of the second part, reproduces the unsplit run."""
    inp = make_inputs(2, 50, 2, 3, 4, 1, 10, seed=19, dt_shift=1.0)
    y, f = o.forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
    k = 23
    y1, f1 = o.forward(inp.x[:, :k], inp.dt[:, :k], inp.A, inp.Bm[:, :k], inp.Cm[:, :k], inp.D)
    y2, f2 = o.forward(inp.x[:, k:], inp.dt[:, k:], inp.A, inp.Bm[:, k:], inp.Cm[:, k:], inp.D, h0=f1)
    e = max(rel(np.concatenate([y1, y2], axis=1), y), rel(f2, f))
    return e <= TOL, f"max rel err {e:.3g}"


def pin_decode_chain(o):
    """Single-token steps (``Oracle.decode_step``, P1 opening paragraph: the
    state is updated once per token) chained from an initial state reproduce
    the brute-force semiseparable form over the whole sequence, token by token
    and in the final state (groups and skip included)."""
    inp = make_inputs(2, 12, 4, 3, 5, 2, 4, seed=41, dt_shift=0.5)
    h0 = _h0(inp)
    ys, fs = forms.semiseparable_forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0)
    st = h0
    worst = 0.0
    for t in range(inp.x.shape[1]):
        y, st = o.decode_step(inp.x[:, t], inp.dt[:, t], inp.A, inp.Bm[:, t], inp.Cm[:, t], inp.D, st)
        worst = max(worst, rel(y, ys[:, t]))
    worst = max(worst, rel(st, fs))
    return worst <= TOL, f"max rel err {worst:.3g}"


def pin_linearity(o):
    """y and the final state are linear in x (with dt, A, B, C, D fixed)."""
    a = make_inputs(1, 30, 2, 4, 3, 1, 6, seed=23)
    b = make_inputs(1, 30, 2, 4, 3, 1, 6, seed=29)
    alpha = 0.75
    # choose values exactly representable so the combined input is exact
    xa = np.round(a.x * 8) / 8
    xb = np.round(b.x * 8) / 8
    xc = (alpha * xa + xb).astype(np.float32)
    args = (a.dt, a.A, a.Bm, a.Cm, a.D)
    ya, fa = o.forward(xa.astype(np.float32), *args)
    yb, fb = o.forward(xb.astype(np.float32), *args)
    yc, fc = o.forward(xc, *args)
    e = max(rel(yc, alpha * ya + yb), rel(fc, alpha * fa + fb))
    return e <= TOL, f"max rel err {e:.3g}"


def pin_causality(o):
    """Changing x at token t leaves y before t bitwise unchanged and changes y_t."""
    inp = make_inputs(1, 30, 2, 3, 4, 1, 6, seed=31)
    y, _ = o.forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
    x2 = inp.x.copy()
    t = 17
    x2[:, t] += 1.0
    y2, _ = o.forward(x2, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
    ok = bool(np.array_equal(y[:, :t], y2[:, :t])) and bool(np.abs(y2[:, t] - y[:, t]).max() > 0)
    return ok, "causal" if ok else "non-causal"


def pin_head_permutation(o):
    """Permuting heads (x, dt, A, D with G = 1) permutes y and final states."""
    inp = make_inputs(2, 25, 5, 3, 4, 1, 5, seed=37)
    perm = np.array([3, 0, 4, 1, 2])
    y, f = o.forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
    yp, fp = o.forward(inp.x[:, :, perm], inp.dt[:, :, perm], inp.A[perm], inp.Bm, inp.Cm, inp.D[perm])
    e = max(rel(yp, y[:, :, perm]), rel(fp, f[:, perm]))
    return e == 0.0, f"max rel err {e:.3g}"


def pin_group_expansion(o):
    """G > 1 equals G = H after replicating each group's B/C to its heads,
    head h using group h // (H/G)."""
    inp = make_inputs(2, 21, 6, 3, 4, 3, 7, seed=41)
    y, f = o.forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
    idx = np.arange(6) // 2
    ye, fe = o.forward(inp.x, inp.dt, inp.A, inp.Bm[:, :, idx], inp.Cm[:, :, idx], inp.D)
    e = max(rel(ye, y), rel(fe, f))
    return e == 0.0, f"max rel err {e:.3g}"


def pin_memoryless(o):
    """Very fast decay (dt*|A| ~ 200): each token forgets the past, so
    y_t = dt_t (C_t.B_t) x_t + D x_t to double precision."""
    inp = make_inputs(1, 20, 2, 3, 4, 1, 4, seed=43, dt_override=20.0, A_override=-10.0)
    y, f = o.forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
    x = inp.x.astype(np.float64)
    cb = np.einsum("btgn,btgn->bt", inp.Cm.astype(np.float64), inp.Bm.astype(np.float64))
    ye = 20.0 * cb[:, :, None, None] * x + inp.D.astype(np.float64)[None, None, :, None] * x
    e = rel(y, ye)
    return e <= TOL, f"max rel err {e:.3g}"


def pin_pairs_and_threads(o):
    """A subset of (b, h) pairs and any thread count give bitwise the same
    values as the full single-threaded run."""
    inp = make_inputs(2, 30, 3, 4, 5, 1, 6, seed=47)
    y1, f1, _ = o.recurrence(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, nthreads=1)
    y4, f4, _ = o.recurrence(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, nthreads=4)
    pairs = [5, 0, 3]
    ys, fs, _ = o.recurrence(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, pairs=pairs, nthreads=2)
    ok = np.array_equal(y1, y4) and np.array_equal(f1, f4)
    ok = ok and np.array_equal(ys, y1[pairs]) and np.array_equal(fs, f1[pairs])
    return bool(ok), "bitwise equal" if ok else "mismatch"


def pin_golden(o):
    """Hand-worked examples stored in tests/golden/hand_examples.json."""
    with open(os.path.join(HERE, "golden", "hand_examples.json")) as fh:
        data = json.load(fh)
    details, ok = [], True
    for ex in data["examples"]:
        f32 = lambda k: np.asarray(ex[k], dtype=np.float32)
        y, f = o.forward(f32("x"), f32("dt"), f32("A"), f32("B"), f32("C"), f32("D"))
        ey = rel(y, np.asarray(ex["y"], np.float64))
        ef = rel(f, np.asarray(ex["final"], np.float64))
        good = max(ey, ef) <= ex["rtol"]
        ok &= good
        details.append(f"{ex['name']}: {max(ey, ef):.3g}")
    return bool(ok), "; ".join(details)


ALL_PINS = [pin_semiseparable, pin_zero_decay, pin_geometric, pin_single_token, pin_skip_only,
            pin_chunk_invariance, pin_chunk_intermediates, pin_split_chaining, pin_decode_chain, pin_linearity,
            pin_causality, pin_head_permutation, pin_group_expansion, pin_memoryless,
            pin_pairs_and_threads, pin_golden]
