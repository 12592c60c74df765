"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times (one ssd_forward call).

The oracle recomputes a seeded sample of (batch, head) pairs over the whole
sequence (always the first and the last pair); y and the final state of
those pairs must meet the acceptance bar, each normalised by its own slice.
The chunk cumsum is checked over the whole tensor.
"""
import numpy as np
import pytest
import torch

from gpu_common import TOL_CUMSUM, gpu_forward, oracle, pairs_sample, relerr, say, tol_for, upload
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
    if name not in cache:
        cache.clear()  # keep one workload resident at a time
        cache[name] = workload_inputs(name)
    return cache[name]


@pytest.mark.parametrize("name", NAMES)
def test_workload_cumsum(cache, name):
    say(f"workload cumsum {name}")
    inp = _inputs(cache, name)
    t = upload(inp)
    dA, _ = ops.ssd_chunk_cumsum(ops.shape_of(t, inp.chunk), t["dt"], t["A"])
    torch.cuda.synchronize()
    assert relerr(dA, dA_cumsum_ref(inp.dt, inp.A, inp.chunk)) <= TOL_CUMSUM


@pytest.mark.parametrize("mma", ["bf16", "f32"])
@pytest.mark.parametrize("name", NAMES)
def test_workload_forward(cache, name, mma):
    w = WORKLOADS[name]
    inp = _inputs(cache, name)
    y_dtype = "f32" if mma == "f32" else w.in_dtype
    say(f"workload forward {name} mma={mma} y={y_dtype}")
    y, fin = gpu_forward(inp, mma, y_dtype=y_dtype)
    pairs = pairs_sample(w.batch, w.nheads, 6, seed=w.seed)
    yo, fo, _ = oracle().forward_pairs(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, pairs)
    y_np = y.float().cpu().numpy()
    f_np = fin.cpu().numpy()
    worst_y = worst_f = 0.0
    for s, pr in enumerate(pairs):
        b, h = divmod(pr, w.nheads)
        worst_y = max(worst_y, relerr(y_np[b, :, h, :], yo[s]))
        worst_f = max(worst_f, relerr(f_np[b, h], fo[s]))
    say(f"  pairs {pairs}: rel err y {worst_y:.3g} final {worst_f:.3g}")
    assert worst_y <= tol_for(mma) and worst_f <= tol_for(mma)
    assert np.isfinite(y_np).all()
