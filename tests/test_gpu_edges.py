"""GPU edge cases of the one-call forward: sequences shorter than or barely
longer than one chunk, the largest head and state sizes the ABI accepts, and
the degenerate inputs whose results have closed forms (the recurrence with
dt = 0 leaves the state unchanged; B = 0 or C = 0 leaves y = D x)."""
import numpy as np
import pytest
import torch

from gpu_common import gpu_forward, make_inputs, oracle, relerr, say, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _h0(B, H, N, P, seed=5):
    return np.random.default_rng(seed).standard_normal((B, H, N, P)).astype(np.float32)


def _check(inp, mma, h0=None, y_dtype="f32"):
    y, fin = gpu_forward(inp, mma, y_dtype=y_dtype, h0=h0)
    yref, fref = oracle().forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0=h0)
    e1, e2 = relerr(y, yref), relerr(fin, fref)
    say(f"  rel err y {e1:.3g} final {e2:.3g}")
    assert e1 <= tol_for(mma) and e2 <= tol_for(mma)
    return y, fin


# (L, Q, P, N): head-group shapes (P 64, N 128 / 256) and generic ones; L = 1,
# one token short of a chunk, one past it
SHORT = [(1, 256, 64, 128), (255, 256, 64, 128), (257, 256, 64, 128), (1, 128, 64, 256), (129, 128, 64, 256),
         (1, 64, 32, 48), (63, 64, 32, 48), (65, 32, 16, 16)]


@pytest.mark.parametrize("mma", ["f32", "bf16"])
@pytest.mark.parametrize("L,Q,P,N", SHORT, ids=[f"L{s[0]}_q{s[1]}_p{s[2]}_n{s[3]}" for s in SHORT])
def test_short_sequences(L, Q, P, N, mma):
    """Sequences of 1 token, Q - 1 and Q + 1 tokens (one ragged chunk, or one
    full chunk plus a single-token one), with an initial state."""
    say(f"short sequence L={L} Q={Q} P={P} N={N} {mma}")
    inp = make_inputs(2, L, 3, P, N, 1, Q, in_dtype="bf16", seed=21, dt_shift=2.0)
    _check(inp, mma, h0=_h0(2, 3, N, P))


# (P, N, Q): the largest headdim and dstate the ABI accepts (256), with the
# chunk sizes that send them to the head-group or the generic kernels
MAXDIM = [(256, 256, 256), (256, 256, 64), (256, 128, 256), (256, 64, 128), (128, 256, 128), (16, 256, 32),
          (256, 16, 32)]


@pytest.mark.parametrize("mma", ["f32", "bf16"])
@pytest.mark.parametrize("P,N,Q", MAXDIM, ids=[f"p{s[0]}_n{s[1]}_q{s[2]}" for s in MAXDIM])
def test_largest_head_and_state(P, N, Q, mma):
    say(f"largest sizes P={P} N={N} Q={Q} {mma}")
    L = 2 * Q + 5  # two full chunks and a ragged one
    inp = make_inputs(1, L, 2, P, N, 1, Q, in_dtype="bf16", seed=22, dt_shift=3.0)
    _check(inp, mma, h0=_h0(1, 2, N, P, seed=6))


def _zeroed(inp, name):
    arr = getattr(inp, name)
    setattr(inp, name, np.zeros_like(arr))
    if getattr(inp, name + "_bits", None) is not None:
        setattr(inp, name + "_bits", np.zeros_like(getattr(inp, name + "_bits")))
    return inp


@pytest.mark.parametrize("mma", ["f32", "bf16"])
def test_zero_dt_keeps_the_state(mma):
    """dt = 0 everywhere: every decay is exp(0) = 1 and every input term is 0,
    so the final state is the initial state exactly (the recurrence adds
    zeros to it), and y = C^T h0 + D x."""
    say(f"dt = 0 {mma}")
    B, L, H, P, N, Q = 2, 300, 4, 64, 128, 256
    inp = make_inputs(B, L, H, P, N, 1, Q, in_dtype="bf16", seed=23, dt_override=0.0)
    h0 = _h0(B, H, N, P, seed=7)
    y, fin = _check(inp, mma, h0=h0)
    assert np.array_equal(fin.cpu().numpy(), h0)


@pytest.mark.parametrize("which", ["Bm", "Cm"])
@pytest.mark.parametrize("mma", ["f32", "bf16"])
def test_zero_B_or_C_leaves_the_skip(which, mma):
    """B = 0 (nothing enters the state) or C = 0 (nothing is read out), no
    initial state: y = D x, computed by the kernel as 0 + D*x in fp32 and
    rounded once, so it equals that product bit for bit; with B = 0 the final
    state is exactly zero."""
    say(f"{which} = 0 {mma}")
    B, L, H, P, N, Q = 1, 520, 4, 64, 128, 256
    inp = _zeroed(make_inputs(B, L, H, P, N, 1, Q, in_dtype="bf16", seed=24), which)
    for y_dtype in ("f32", "bf16"):
        y, fin = gpu_forward(inp, mma, y_dtype=y_dtype)
        skip = torch.from_numpy(inp.x).cuda() * torch.from_numpy(inp.D).cuda()[None, None, :, None]
        expect = skip if y_dtype == "f32" else skip.to(torch.bfloat16)
        assert torch.equal(y, expect), y_dtype
        if which == "Bm":
            assert not fin.any()
        else:
            fref = oracle().forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)[1]
            assert relerr(fin, fref) <= tol_for(mma)
