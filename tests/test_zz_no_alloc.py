"""ssd_forward_noalloc: the forward with the library's own static device
scratch array as its workspace (for callers that cannot allocate).

Called through the C ABI (the ops binding) and compared with ssd_forward,
which runs the same kernels on a caller-provided workspace: y and the final
states must be bit-identical, on two calls in a row (the second smaller, so
it runs on scratch left over from the first), on both precision paths.
Shapes beyond the scratch array are refused before any launch.
"""
import pytest
import torch

from gpu_common import make_inputs, oracle, relerr, say, tol_for, upload
from mamba_ssd_scan_chunk_amd import ops
from mamba_ssd_scan_chunk_amd._lib import SSDError, load_library

pytestmark = pytest.mark.gpu

# (name, B, L, H, P, N, G, Q): a large call, then a smaller ragged one
CALLS = [("large", 2, 4096, 32, 64, 128, 1, 256), ("small_ragged", 1, 700, 4, 64, 128, 1, 256)]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("mma", ["bf16", "f32"])
def test_noalloc_matches_forward_on_two_calls(mma):
    in_dtype = "bf16" if mma == "bf16" else "f32"
    y_dtype = "bf16" if mma == "bf16" else "f32"
    for k, (name, B, L, H, P, N, G, Q) in enumerate(CALLS):
        say(f"noalloc forward call {k}: {name} {(B, L, H, P, N, G, Q)} mma={mma}")
        inp = make_inputs(B, L, H, P, N, G, Q, in_dtype=in_dtype, seed=60 + k, dt_shift=1.0)
        t = upload(inp)
        sh = ops.shape_of(t, Q)
        h0 = torch.randn((B, H, N, P), device="cuda", generator=torch.Generator(device="cuda").manual_seed(70 + k))
        y1, f1 = ops.ssd_forward_noalloc(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], initial_states=h0,
                                         y_dtype=y_dtype, mma=mma)
        y2, f2 = ops.ssd_forward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], initial_states=h0,
                                 y_dtype=y_dtype, mma=mma)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(f1, f2)
        if k == 1:  # the small call also against the oracle
            yo, fo = oracle().forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D,
                                      h0=h0.double().cpu().numpy())
            assert relerr(y1, yo) <= tol_for(mma) and relerr(f1, fo) <= tol_for(mma)


def test_noalloc_refuses_shapes_beyond_scratch():
    """A shape whose workspace exceeds the scratch array is refused with
    SSD_ERR_SCRATCH before any launch (the pointers are never read)."""
    lib = load_library()
    sh = ops.SSDShape.make(8, 4096, 64, 64, 256, 8, 128)  # ~554 MB of bf16 workspace
    fake = 0x100000
    st = lib.ssd_forward_noalloc(sh, fake, fake, fake, fake, fake, fake, 1, None, fake, 1, None, 0, None)
    assert st == 8
    assert lib.ssd_status_string(st).decode().startswith("SSD_ERR_SCRATCH")
    x = torch.empty((8, 4096, 64, 64), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(SSDError):
        ops.ssd_forward_noalloc(sh, x, torch.empty((8, 4096, 64), device="cuda"), torch.empty(64, device="cuda"),
                                torch.empty((8, 4096, 8, 256), device="cuda", dtype=torch.bfloat16),
                                torch.empty((8, 4096, 8, 256), device="cuda", dtype=torch.bfloat16),
                                torch.empty(64, device="cuda"))
