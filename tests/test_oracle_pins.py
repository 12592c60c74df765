"""The fp64 oracle checked against things other than itself (CPU only).

Every pin in ``pins.py`` must hold for the real oracle, and every planted
mistake (a mutated copy of ``oracle/ssd_oracle.c`` compiled on the CPU) must
break at least one pin, which shows the pins are sharp enough to catch a
dropped term, a wrong sign, a wrong index or a swapped operand.
"""
import os

import pytest

import pins
from oracle import oracle as oracle_mod


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
