"""The fp64 gradient oracle (oracle/backward.py) checked against something
other than itself (CPU only): central finite differences of the brute-force
semiseparable forward (oracle/forms.py), one directional derivative per input
tensor, and planted mistakes in copies of its source, each of which must break
at least one of those checks."""
import os
import types

import numpy as np
import pytest

from mamba_ssd_scan_chunk_amd.inputs import make_inputs
from oracle import backward as bwd_mod
from oracle import forms

NAMES = ["x", "dt", "A", "Bm", "Cm", "D", "h0"]
GRAD = {"x": "dx", "dt": "ddt", "A": "dA", "Bm": "dB", "Cm": "dC", "D": "dD", "h0": "dh0"}


def _problem(seed=3):
    inp = make_inputs(2, 12, 4, 3, 5, 2, 4, seed=seed, dt_shift=0.5)
    rng = np.random.default_rng(seed + 1)
    v = {"x": inp.x, "dt": inp.dt, "A": inp.A, "Bm": inp.Bm, "Cm": inp.Cm, "D": inp.D,
         "h0": rng.standard_normal((2, 4, 5, 3))}
    v = {k: np.asarray(a, dtype=np.float64) for k, a in v.items()}
    dy = rng.standard_normal(inp.x.shape)
    dfin = rng.standard_normal((2, 4, 5, 3))
    return v, dy, dfin


def _loss(v, dy, dfin):
    y, fin = forms.semiseparable_forward(v["x"], v["dt"], v["A"], v["Bm"], v["Cm"], v["D"], v["h0"])
    return float(np.sum(dy * y) + np.sum(dfin * fin))


def fd_errors(backward_fn, seed=3, eps=1e-6):
    """Relative error of <grad, u> against the central difference of the loss
    along a random direction u, for every input tensor."""
    v, dy, dfin = _problem(seed)
    g = backward_fn(v["x"], v["dt"], v["A"], v["Bm"], v["Cm"], v["D"], dy, h0=v["h0"], dfinal=dfin)
    rng = np.random.default_rng(seed + 2)
    errs = {}
    for name in NAMES:
        u = rng.standard_normal(v[name].shape)
        if name == "dt":
            u *= 0.1 * v["dt"]  # keep dt positive
        plus = dict(v); plus[name] = v[name] + eps * u
        minus = dict(v); minus[name] = v[name] - eps * u
        fd = (_loss(plus, dy, dfin) - _loss(minus, dy, dfin)) / (2 * eps)
        an = float(np.sum(g[GRAD[name]] * u))
        errs[name] = abs(fd - an) / max(abs(fd), abs(an), 1e-12)
    return errs


def test_backward_matches_finite_differences():
    for seed in (3, 11):
        errs = fd_errors(bwd_mod.backward, seed=seed)
        assert max(errs.values()) <= 1e-7, errs


def test_backward_without_h0_or_dfinal():
    """No initial state and no final-state gradient: dh0 still follows (the
    gradient w.r.t. a zero initial state), and the defaults agree with zeros."""
    v, dy, dfin = _problem(5)
    z = np.zeros_like(dfin)
    a = bwd_mod.backward(v["x"], v["dt"], v["A"], v["Bm"], v["Cm"], v["D"], dy)
    b = bwd_mod.backward(v["x"], v["dt"], v["A"], v["Bm"], v["Cm"], v["D"], dy, h0=z, dfinal=z)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_backward_terms_compose_ddt_and_dA():
    """The per-token pieces returned with terms=True recompose the pinned ddt
    and dA (ddt = A dlogr + beta, dA = sum over tokens of dt dlogr), and
    asking for them changes no gradient."""
    v, dy, dfin = _problem(7)
    g = bwd_mod.backward(v["x"], v["dt"], v["A"], v["Bm"], v["Cm"], v["D"], dy, h0=v["h0"], dfinal=dfin, terms=True)
    g0 = bwd_mod.backward(v["x"], v["dt"], v["A"], v["Bm"], v["Cm"], v["D"], dy, h0=v["h0"], dfinal=dfin)
    for k in g0:
        assert np.array_equal(g[k], g0[k]), k
    ddt = v["A"][None, None, :] * g["dlogr"] + g["beta"]
    assert np.allclose(ddt, g["ddt"], rtol=1e-12, atol=1e-12 * np.abs(g["ddt"]).max())
    dA = (v["dt"] * g["dlogr"]).sum(axis=(0, 1))
    assert np.allclose(dA, g["dA"], rtol=1e-12, atol=1e-12 * np.abs(g["dA"]).max())


# (text in backward.py, replacement, what the mistake is)
MUTATIONS = [
    ("gst += np.outer(Cm[b, t, g], dy[b, t, h])", "gst += np.outer(Bm[b, t, g], dy[b, t, h])", "C replaced by B in the adjoint"),
    ("gst = r[t] * gst", "gst = gst", "adjoint decay dropped"),
    ("D[h] * dy[b, t, h] + dt[b, t, h] * (Bm[b, t, g] @ gst)", "D[h] * dy[b, t, h] + (Bm[b, t, g] @ gst)", "dt dropped from dx"),
    ("out[\"dB\"][b, t, g] += dt[b, t, h] * gx", "out[\"dB\"][b, t, g] = dt[b, t, h] * gx", "dB not summed over the group's heads"),
    ("out[\"dC\"][b, t, g] += ht @ dy[b, t, h]", "out[\"dC\"][b, t, g] += hprev @ dy[b, t, h]", "dC from the previous state"),
    ("A[h] * r[t] * gh + float(Bm[b, t, g] @ gx)", "r[t] * gh + float(Bm[b, t, g] @ gx)", "A dropped from ddt"),
    ("out[\"dA\"][h] += dt[b, t, h] * r[t] * gh", "out[\"dA\"][h] += r[t] * gh", "dt dropped from dA"),
    ("out[\"dD\"][h] += float(dy[b, t, h] @ x[b, t, h])", "out[\"dD\"][h] += float(dy[b, t, h] @ dy[b, t, h])", "dD from dy alone"),
    ("out[\"dh0\"][b, h] = gst", "out[\"dh0\"][b, h] = gst / r[0]", "dh0 missing the first decay"),
]


@pytest.mark.parametrize("orig,repl,what", MUTATIONS, ids=[m[2] for m in MUTATIONS])
def test_planted_mistake_is_caught(orig, repl, what):
    src = open(bwd_mod.__file__).read()
    assert src.count(orig) == 1, f"mutation anchor not found exactly once: {orig!r}"
    mod = types.ModuleType("backward_mutant")
    exec(compile(src.replace(orig, repl), os.path.basename(bwd_mod.__file__), "exec"), mod.__dict__)
    errs = fd_errors(mod.backward)
    assert max(errs.values()) > 1e-4, f"{what} not caught: {errs}"
