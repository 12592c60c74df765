"""GPU parity of the single-token recurrent step (``ssd_decode_step``) against
the fp64 oracle (the recurrence over one token), and its chaining: steps
applied token by token reproduce the chunked forward with the same initial
state.  Acceptance (max|err|/max|ref|): 1e-6 on the fp32 state, 1e-4 on fp32
y (an N-term fp32 sum), 1e-2 on bf16 y (output rounding)."""
import numpy as np
import pytest
import torch

from gpu_common import make_inputs, oracle, relerr, say
from mamba_ssd_scan_chunk_amd import ops

pytestmark = pytest.mark.gpu

TOL_STATE = 1e-6
TOL_Y = {"f32": 1e-4, "bf16": 1e-2}

# (name, B, H, P, N, G)
DEC_SHAPES = [
    ("tiny", 1, 2, 16, 16, 1),
    ("layer_130m", 3, 24, 64, 128, 1),
    ("grouped", 2, 8, 48, 40, 4),   # 12 column groups: 252 of 256 threads hold rows
    ("wide", 1, 3, 256, 256, 1),
    ("odd", 2, 2, 20, 7, 1),        # P, N the chunked calls refuse
    ("p1024", 1, 1, 1024, 8, 1),    # one row group
]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _step_inputs(shape, in_dtype, seed):
    name, B, H, P, N, G = shape
    inp = make_inputs(B, 1, H, P, N, G, 1, in_dtype=in_dtype, seed=seed, dt_shift=1.0)
    t = inp.to_torch("cuda")
    state = np.random.default_rng(seed + 100).standard_normal((B, H, N, P)).astype(np.float32)
    return inp, t, state


@pytest.mark.parametrize("y_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", DEC_SHAPES, ids=[s[0] for s in DEC_SHAPES])
def test_decode_step(shape, in_dtype, y_dtype):
    say(f"decode step {shape} in={in_dtype} y={y_dtype}")
    inp, t, state = _step_inputs(shape, in_dtype, seed=51)
    st = torch.from_numpy(state).cuda()
    y = ops.ssd_decode_step(t["x"][:, 0].contiguous(), t["dt"][:, 0].contiguous(), t["A"],
                            t["Bm"][:, 0].contiguous(), t["Cm"][:, 0].contiguous(), t["D"], st, y_dtype=y_dtype)
    torch.cuda.synchronize()
    yref, sref = oracle().decode_step(inp.x[:, 0], inp.dt[:, 0], inp.A, inp.Bm[:, 0], inp.Cm[:, 0], inp.D,
                                      state.astype(np.float64))
    e_s, e_y = relerr(st, sref), relerr(y.float(), yref)
    say(f"  rel err state {e_s:.3g} y {e_y:.3g}")
    assert e_s <= TOL_STATE and e_y <= TOL_Y[y_dtype]
    if y_dtype == "bf16":
        # y is the fp32 result rounded once, to nearest even
        y32 = ops.ssd_decode_step(t["x"][:, 0].contiguous(), t["dt"][:, 0].contiguous(), t["A"],
                                  t["Bm"][:, 0].contiguous(), t["Cm"][:, 0].contiguous(), t["D"],
                                  torch.from_numpy(state).cuda(), y_dtype="f32")
        torch.cuda.synchronize()
        assert torch.equal(y, y32.to(torch.bfloat16))


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_decode_chain_equals_forward(in_dtype):
    """L single-token steps from an initial state against the chunked forward
    over the same L tokens (fp32 matrix operands) and against the oracle."""
    B, L, H, P, N, G, Q = 2, 64, 4, 64, 32, 2, 32
    say(f"decode chain vs forward in={in_dtype}")
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype=in_dtype, seed=53, dt_shift=2.0)
    t = inp.to_torch("cuda")
    h0 = np.random.default_rng(54).standard_normal((B, H, N, P)).astype(np.float32)
    st = torch.from_numpy(h0).cuda()
    ys = []
    for k in range(L):
        ys.append(ops.ssd_decode_step(t["x"][:, k].contiguous(), t["dt"][:, k].contiguous(), t["A"],
                                      t["Bm"][:, k].contiguous(), t["Cm"][:, k].contiguous(), t["D"], st,
                                      y_dtype="f32"))
    y_dec = torch.stack(ys, dim=1)
    sh = ops.shape_of(t, Q)
    y_fwd, fin = ops.ssd_forward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"],
                                 initial_states=torch.from_numpy(h0).cuda(), y_dtype="f32", mma="f32")
    torch.cuda.synchronize()
    yref, fref = oracle().forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0=h0.astype(np.float64))
    e = {"dec y": relerr(y_dec, yref), "dec final": relerr(st, fref), "fwd vs dec y": relerr(y_fwd, y_dec.double().cpu().numpy()),
         "fwd vs dec final": relerr(fin, st.double().cpu().numpy())}
    say("  " + ", ".join(f"{k} {v:.3g}" for k, v in e.items()))
    assert max(e.values()) <= 1e-4


def test_decode_step_zero_input_decays_state():
    """x = 0: the state only decays, h <- exp(dt A) h (special case of the
    recurrence), to fp32 rounding."""
    B, H, P, N, G = 2, 3, 32, 16, 1
    rng = np.random.default_rng(57)
    x = torch.zeros((B, H, P), device="cuda")
    dt = torch.from_numpy(rng.uniform(0.05, 0.5, (B, H)).astype(np.float32)).cuda()
    A = torch.from_numpy(-rng.uniform(0.5, 4.0, H).astype(np.float32)).cuda()
    Bm = torch.from_numpy(rng.standard_normal((B, G, N)).astype(np.float32)).cuda()
    Cm = torch.from_numpy(rng.standard_normal((B, G, N)).astype(np.float32)).cuda()
    D = torch.from_numpy(rng.standard_normal(H).astype(np.float32)).cuda()
    h = torch.from_numpy(rng.standard_normal((B, H, N, P)).astype(np.float32)).cuda()
    st = h.clone()
    ops.ssd_decode_step(x, dt, A, Bm, Cm, D, st, y_dtype="f32")
    torch.cuda.synchronize()
    r = torch.exp(dt.double() * A.double()[None, :])
    assert relerr(st, (r[:, :, None, None] * h.double()).cpu().numpy()) <= 1e-6
