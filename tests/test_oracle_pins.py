"""The fp64 oracle checked against things other than itself (CPU only).

Every pin in ``pins.py`` must hold for the real oracle, and every planted
mistake (a mutated copy of ``oracle/ssd_oracle.c`` compiled on the CPU) must
break at least one pin, which shows the pins are sharp enough to catch a
dropped term, a wrong sign, a wrong index or a swapped operand.
"""
import os

import numpy as np
import pytest

import pins
from mamba_ssd_scan_chunk_amd.inputs import make_inputs
from oracle import oracle as oracle_mod
from oracle.oracle import dA_cumsum_ref


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin_holds(oracle_lib, pin):
    ok, detail = pin(oracle_lib)
    assert ok, f"{pin.__name__}: {detail}"


# (text in ssd_oracle.c, replacement, what the mistake is)
MUTATIONS = [
    ("const double r = exp(dtv * a);", "const double r = exp(-dtv * a);", "decay sign flipped"),
    ("hrow[p] = r * hrow[p] + coef * (double)xt[p];", "hrow[p] = hrow[p] + coef * (double)xt[p];", "decay dropped"),
    ("const double coef = dtv * (double)bt[n];", "const double coef = (double)bt[n];", "dt dropped from the input term"),
    ("const int64_t g = hd / (H / G);", "const int64_t g = hd % G;", "head-to-group map interleaved"),
    ("yt[p] = dskip * (double)xt[p];", "yt[p] = 0.0;", "skip connection dropped"),
    ("const float* ct = j->Cm + ((b * L + t) * G + g) * N;", "const float* ct = j->Bm + ((b * L + t) * G + g) * N;", "C replaced by B"),
    ("for (int64_t e = 0; e < N * P; ++e) h[e] = src[e];", "for (int64_t e = 0; e < N * P; ++e) h[e] = 0.0 * src[e];", "initial state ignored"),
    ("const double dtv = (double)j->dt[(b * L + t) * H + hd];", "const double dtv = (double)j->dt[(b * L + (t > 0 ? t - 1 : 0)) * H + hd];", "dt taken from the previous token"),
    ("const double cn = (double)ct[n];", "const double cn = (double)ct[N - 1 - n];", "C read in reversed state order"),
    ("hrow[p] = r * hrow[p] + coef * (double)xt[p];", "hrow[p] = r * hrow[p] + coef * (double)xt[P - 1 - p];", "x transposed against the state columns"),
    ("if (j->chunk > 0 && t % j->chunk == 0) {", "if (j->chunk > 0 && t % j->chunk == 1) {", "chunk boundary off by one"),
]


@pytest.mark.parametrize("orig,repl,what", MUTATIONS, ids=[m[2] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, orig, repl, what):
    src = open(oracle_mod.SRC_PATH).read()
    assert src.count(orig) == 1, f"mutation anchor not found exactly once: {orig!r}"
    mutated = tmp_path / "ssd_oracle_mut.c"
    mutated.write_text(src.replace(orig, repl))
    lib = oracle_mod.build(str(mutated), str(tmp_path / "libmut.so"))
    o = oracle_mod.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            ok, _ = pin(o)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"planted mistake '{what}' passed every pin"


# ---- dt_bhl_ref: a pure re-layout, pinned by the layout definition in the C
# header (dt_bhl[b,h,c,i] = dt[b,cQ+i,h], 0 past a ragged end) on inputs whose
# values encode their own coordinates, and by its consistency with the pinned
# dA_cumsum_ref (consecutive in-chunk sums differ by A * dt of that position).

def _coded_dt(Bsz, L, H):
    """dt whose value names its coordinates: 1 + b*1e6 + t*1e2 + h (exact in
    fp64 for these sizes; h < 100, t < 1e4)."""
    b = np.arange(Bsz)[:, None, None]
    t = np.arange(L)[None, :, None]
    h = np.arange(H)[None, None, :]
    return (1.0 + b * 1e6 + t * 1e2 + h).astype(np.float64)


def _dt_bhl_layout_ok(fn, Bsz, L, H, Q):
    dt = _coded_dt(Bsz, L, H)
    out = np.asarray(fn(dt, Q), dtype=np.float64)
    nc = -(-L // Q)
    if out.shape != (Bsz, H, nc, Q):
        return False
    for b in range(Bsz):
        for h in range(H):
            for c in range(nc):
                for i in range(Q):
                    t = c * Q + i
                    want = 1.0 + b * 1e6 + t * 1e2 + h if t < L else 0.0
                    if out[b, h, c, i] != want:
                        return False
    return True


DT_BHL_CASES = [(1, 8, 1, 4), (2, 12, 3, 4), (2, 10, 3, 4), (1, 7, 2, 8), (3, 33, 5, 16)]


@pytest.mark.parametrize("case", DT_BHL_CASES, ids=[f"B{c[0]}L{c[1]}H{c[2]}Q{c[3]}" for c in DT_BHL_CASES])
def test_dt_bhl_ref_layout(case):
    """Every element of dt_bhl_ref sits where the header's definition puts it,
    zeros past a ragged end included (L % Q != 0 in three of the cases)."""
    from oracle.oracle import dt_bhl_ref
    assert _dt_bhl_layout_ok(dt_bhl_ref, *case)


def test_dt_bhl_ref_matches_pinned_cumsum():
    """dA_cumsum_ref (pinned against the chunked form) steps by A*dt at every
    valid position: G[i] - G[i-1] = A dt_bhl[i], G[0] = A dt_bhl[0]."""
    from oracle.oracle import dt_bhl_ref
    inp = make_inputs(2, 200, 3, 4, 4, 1, 64, seed=23, dt_shift=1.0)
    for Q in (16, 64, 48):
        G = dA_cumsum_ref(inp.dt, inp.A, Q)
        d = dt_bhl_ref(inp.dt, Q)
        step = np.diff(G, axis=3, prepend=0.0)
        L = inp.dt.shape[1]
        nc = -(-L // Q)
        valid = (np.arange(nc)[:, None] * Q + np.arange(Q)[None, :]) < L
        want = inp.A.astype(np.float64)[None, :, None, None] * d
        assert np.allclose(step[..., valid], want[..., valid], rtol=1e-12, atol=1e-14)


def test_dt_bhl_pin_catches_planted_layouts():
    """Plausible wrong layouts each fail the layout pin."""
    def swapped_axes(dt, Q):  # [B,nc,Q,H] left untransposed
        Bsz, L, H = dt.shape
        nc = -(-L // Q)
        out = np.zeros((Bsz, nc * Q, H))
        out[:, :L] = dt
        return out.reshape(Bsz, nc, Q, H)

    def shifted(dt, Q):  # token off by one inside a chunk
        Bsz, L, H = dt.shape
        nc = -(-L // Q)
        out = np.zeros((Bsz, nc * Q, H))
        out[:, 1:L] = dt[:, :L - 1]
        return out.reshape(Bsz, nc, Q, H).transpose(0, 3, 1, 2)

    def ragged_repeat(dt, Q):  # past-the-end positions repeat the last dt instead of 0
        Bsz, L, H = dt.shape
        nc = -(-L // Q)
        out = np.zeros((Bsz, nc * Q, H))
        out[:, :L] = dt
        out[:, L:] = dt[:, L - 1:L]
        return out.reshape(Bsz, nc, Q, H).transpose(0, 3, 1, 2)

    for bad in (swapped_axes, shifted, ragged_repeat):
        assert not all(_dt_bhl_layout_ok(bad, *c) for c in DT_BHL_CASES), bad.__name__
