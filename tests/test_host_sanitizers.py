"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The C ABI's host layer (``ssd_api.cpp``: argument validation, shape limits,
  workspace arithmetic) is built with g++ against stand-ins for the device
  launchers that abort if reached, and driven over many random shapes with
  extreme field values by ``sanitize/abi_driver.cpp``: any out-of-bounds
  access, signed overflow, invalid enum load or a launch on invalid arguments
  fails the run.
* The fp64 oracle (``oracle/ssd_oracle.c``, threaded) is built with gcc under
  both sanitizers and run on small problems (all pairs with an initial state;
  a pair subset with chunk bookkeeping); its results must equal the regular
  build's.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from mamba_ssd_scan_chunk_amd.inputs import make_inputs
from oracle import oracle as oracle_mod

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "mamba_ssd_scan_chunk_amd", "csrc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g",
       "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="host compilers not available")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_abi_host_layer_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-I", "/opt/rocm/include", os.path.join(CSRC, "ssd_api.cpp"), os.path.join(CSRC, "tuning.cpp"),
          os.path.join(HERE, "sanitize", "abi_stubs.cpp"),
          os.path.join(HERE, "sanitize", "abi_driver.cpp"), "-L", "/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe, "60000"], env=ENV, timeout=600)
    print(r.stdout)
    assert "0 mismatches" in r.stdout


@pytest.mark.parametrize("variant", ["all_pairs_h0", "pair_subset_chunks", "reset_each_chunk"])
def test_oracle_under_asan_ubsan(tmp_path, variant):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", *SAN, "-pthread", oracle_mod.SRC_PATH, os.path.join(HERE, "sanitize", "oracle_driver.c"),
          "-lm", "-o", exe])
    B, L, H, P, N, G, Q = 2, 77, 4, 8, 6, 2, 16
    inp = make_inputs(B, L, H, P, N, G, Q, seed=29, dt_shift=1.0)
    h0 = np.random.default_rng(30).standard_normal((B, H, N, P))
    fin_path, fout_path = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    with open(fin_path, "wb") as f:
        for a in (inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D):
            f.write(np.ascontiguousarray(a, dtype=np.float32).tobytes())
        f.write(np.ascontiguousarray(h0 if variant == "all_pairs_h0" else np.zeros_like(h0)).tobytes())
    pairs = [] if variant == "all_pairs_h0" else [7, 0, 3, 5]
    chunk = 0 if variant == "all_pairs_h0" else Q
    reset = 1 if variant == "reset_each_chunk" else 0
    _run([exe, fin_path, fout_path, *map(str, (B, L, H, P, N, G, 3, chunk, reset, len(pairs))), *map(str, pairs)],
         env=ENV, timeout=300)
    out = np.fromfile(fout_path, dtype=np.float64)
    o = oracle_mod.get()
    y, fin, bnd = o.recurrence(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D,
                               h0=h0 if variant == "all_pairs_h0" else None, pairs=pairs or None, chunk=chunk,
                               reset_each_chunk=bool(reset), want_boundary=chunk > 0, nthreads=2)
    want = np.concatenate([y.ravel(), fin.ravel()] + ([bnd.ravel()] if bnd is not None else []))
    assert out.shape == want.shape
    assert np.array_equal(out, want)
