"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times (one ssd_forward call).

The oracle recomputes EVERY (batch, head) pair over the whole sequence (once
per workload, threaded over the host cores), and y and the final states are
compared as whole tensors, max|err| / max|ref|, on both precision paths.  The
worst single pair, normalised by its own slice, is printed beside it.  The
chunk cumsum is checked over the whole tensor.
"""
import numpy as np
import pytest
import torch

from gpu_common import TOL_CUMSUM, gpu_forward, oracle, relerr, say, tol_for, upload
from mamba_ssd_scan_chunk_amd import ops
from mamba_ssd_scan_chunk_amd.inputs import WORKLOADS, workload_inputs
from oracle.oracle import dA_cumsum_ref

pytestmark = pytest.mark.gpu

NAMES = list(WORKLOADS)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def cache():
    return {}


def _inputs(cache, name):
    if cache.get("name") != name:
        cache.clear()  # keep one workload (inputs and oracle results) resident at a time
        cache["name"] = name
        cache["inp"] = workload_inputs(name)
    return cache["inp"]


def _oracle_all_pairs(cache, name):
    """y [B*H, L, P] and final states [B*H, N, P] (fp64) of every pair."""
    inp = _inputs(cache, name)
    if "ref" not in cache:
        say(f"  oracle: all {inp.x.shape[0] * inp.x.shape[2]} (batch, head) pairs of {name}")
        yo, fo, _ = oracle().recurrence(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
        cache["ref"] = (yo, fo)
    return cache["ref"]


@pytest.mark.parametrize("name", NAMES)
def test_workload_cumsum(cache, name):
    say(f"workload cumsum {name}")
    inp = _inputs(cache, name)
    t = upload(inp)
    dA, _ = ops.ssd_chunk_cumsum(ops.shape_of(t, inp.chunk), t["dt"], t["A"])
    torch.cuda.synchronize()
    assert relerr(dA, dA_cumsum_ref(inp.dt, inp.A, inp.chunk)) <= TOL_CUMSUM


def _pair_major(t_bl_h_x):
    """[B, L, H, X] -> [B*H, L, X] (the oracle's pair-major layout)."""
    a = t_bl_h_x
    return np.ascontiguousarray(a.transpose(0, 2, 1, 3)).reshape(a.shape[0] * a.shape[2], a.shape[1], a.shape[3])


@pytest.mark.parametrize("mma", ["bf16", "f32"])
@pytest.mark.parametrize("name", NAMES)
def test_workload_forward(cache, name, mma):
    w = WORKLOADS[name]
    inp = _inputs(cache, name)
    y_dtype = "f32" if mma == "f32" else w.in_dtype
    say(f"workload forward {name} mma={mma} y={y_dtype}")
    y, fin = gpu_forward(inp, mma, y_dtype=y_dtype)
    y_np = _pair_major(y.float().cpu().numpy())
    f_np = fin.cpu().numpy().reshape(w.batch * w.nheads, w.dstate, w.headdim)
    del y, fin
    assert np.isfinite(y_np).all() and np.isfinite(f_np).all()
    yo, fo = _oracle_all_pairs(cache, name)
    ey, ef = relerr(y_np, yo), relerr(f_np, fo)
    # worst single (batch, head) pair, each normalised by its own slice (informational)
    pair_y = max(float(np.abs(y_np[s] - yo[s]).max() / max(np.abs(yo[s]).max(), 1e-300)) for s in range(len(yo)))
    pair_f = max(float(np.abs(f_np[s] - fo[s]).max() / max(np.abs(fo[s]).max(), 1e-300)) for s in range(len(fo)))
    say(f"  all {len(yo)} pairs: rel err y {ey:.3g} final {ef:.3g} (worst pair: y {pair_y:.3g} final {pair_f:.3g})")
    assert ey <= tol_for(mma) and ef <= tol_for(mma)
