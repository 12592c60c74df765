"""GPU parity of the gradient call (``ssd_backward``, through the C ABI)
against the fp64 gradient oracle (oracle/backward.py, itself pinned by finite
differences of the brute-force forward), in both matrix-operand modes.

Acceptance: 1e-4 with fp32 matrix operands (the forward's fp32 bar: every
product runs in fp32), 1e-2 with bf16 operands (the forward's bf16 bar), and
2e-2 for ddt and dA with bf16 operands (below).  dx, dB, dC, dD and dinitial: max|gpu - ref| / max|ref| per tensor.
ddt and dA are sums of terms of both signs that can be much larger than the
sum (ddt_t = A q_t - A dt_t beta_t + beta_t with q_t = <g_t, h_t>, dA a sum over
every token), so their error is measured against the size of those terms,
taken from the oracle's per-token pieces: ddt against max_t of
|A| (|dlogr_t| + 2 dt_t |beta_t|) + |beta_t|, and dA_h against
sum_{b,t} dt (|dlogr| + 2 dt |beta|) of its head.

At full size (the 2.7B-layer and grouped workloads) the oracle runs on sampled
(batch, head) slices (dx, ddt, dinitial of those slices; dA of a sampled head
over every row),
and the rest is checked by identities that hold at any size:
  * per token, C_t . dC_t = sum_h dy_t . (y_t - D_h x_t)     (dC_t = sum_h h_t dy_t)
  * per token, B_t . dB_t = sum_h x_t . (dx_t - D_h dy_t)    (both equal sum_h dt_t B_t^T g_t x_t)
  * per (b, h), <dx, x> + <dinitial, h0> = <dy, y> + <dfinal, final>  (the loss is linear in x, h0)
  * dD_h = sum over tokens of dy . x
with y and final from the forward on the same inputs (fp32 matrix operands)."""
import numpy as np
import pytest
import torch

from gpu_common import make_inputs, relerr, say
from mamba_ssd_scan_chunk_amd import ops
from mamba_ssd_scan_chunk_amd.inputs import workload_inputs
from oracle import backward as bwd_oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}
# ddt and dA with bf16 matrix operands, against the size of their terms: each
# term carries several bf16-rounded quantities (chunk and carried states, the
# recomputed outputs y0 and y1, each rounded at 2^-9 relative), so a few 1e-3
# up to ~1e-2 of the term size is this mode's accuracy; a wrong index or sign
# gives errors of order 1 in this norm.
TOL_DECAY_BF16 = 2e-2


def tol_for(key, mma):
    return TOL_DECAY_BF16 if (mma == "bf16" and key in ("ddt", "dA")) else TOL[mma]
KEYS = ["dx", "ddt", "dA", "dB", "dC", "dD", "dh0"]


def grad_errors(g, ref, dt, A, keys=KEYS):
    """Error of each GPU gradient against the oracle's (``ref`` from
    backward(..., terms=True)); ddt and dA scaled by the size of their terms."""
    dt = np.asarray(dt, np.float64)
    aA = np.abs(np.asarray(A, np.float64))[None, None, :]
    dl, be = np.abs(ref["dlogr"]), np.abs(ref["beta"])
    errs = {}
    for k in keys:
        if k == "ddt":
            scale = (aA * (dl + 2 * dt * be) + be).max()
            errs[k] = float(np.abs(g[k].double().cpu().numpy() - ref[k]).max() / scale)
        elif k == "dA":
            scale = (dt * (dl + 2 * dt * be)).sum(axis=(0, 1))
            errs[k] = float((np.abs(g[k].double().cpu().numpy() - ref[k]) / scale).max())
        else:
            errs[k] = relerr(g[k], ref[k])
    return errs


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cuda(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda", dtype)


def run_gpu(inp, dy, h0, dfin, dy_dtype="f32", mma="f32"):
    t = inp.to_torch("cuda")
    sh = ops.shape_of(t, inp.chunk)
    dy_t = _cuda(dy, torch.bfloat16 if dy_dtype == "bf16" else torch.float32)
    g = ops.ssd_backward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], dy_t,
                         initial_states=None if h0 is None else _cuda(h0),
                         dfinal=None if dfin is None else _cuda(dfin), mma=mma)
    torch.cuda.synchronize()
    g["dh0"] = g.pop("dinitial")
    return g, t


# (name, B, L, H, P, N, G, Q)
BWD_SHAPES = [
    ("tiny", 1, 256, 2, 16, 16, 1, 64),
    ("grouped", 2, 256, 4, 32, 48, 2, 64),
    ("ragged", 2, 200, 2, 32, 64, 1, 64),       # last chunk of 8 positions
    ("q256", 1, 640, 2, 64, 128, 1, 256),       # the 2.7B-layer head shape, ragged tail
    ("wide_p", 1, 160, 3, 128, 32, 3, 32),      # P > N
    ("q128_n256", 1, 330, 4, 48, 256, 2, 128),  # dB/dC kernels at chunk 128, N = 256, a 48-wide headdim, ragged
    ("q256_n256", 1, 300, 2, 32, 256, 1, 256),  # chunk 256 with N = 256: dC's state part in its own launch
    # head-group chunk kernels at chunk 128 (the adjoint reads dy, C, B in
    # reversed order in place when they are bf16), ragged
    ("q128_n256_p64", 1, 300, 4, 64, 256, 2, 128),
    ("q128_n128_p128", 1, 200, 2, 128, 128, 1, 128),
    ("one_short_chunk_q128", 1, 100, 2, 64, 128, 1, 128),  # L < Q: 28 of the 128 reversed steps are padding
    # more heads than one 16-head tile of the decay-gradient kernel, the last
    # tile partial, ragged
    ("twenty_heads", 1, 300, 20, 16, 32, 2, 64),
]


@pytest.mark.parametrize("mma", ["f32", "bf16"])
@pytest.mark.parametrize("dy_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", BWD_SHAPES, ids=[s[0] for s in BWD_SHAPES])
def test_backward_matches_oracle(shape, in_dtype, dy_dtype, mma):
    name, B, L, H, P, N, G, Q = shape
    say(f"backward {shape} in={in_dtype} dy={dy_dtype} mma={mma}")
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype=in_dtype, seed=61, dt_shift=2.0)
    rng = np.random.default_rng(62)
    dy = rng.standard_normal(inp.x.shape).astype(np.float32)
    if dy_dtype == "bf16":
        dy = torch.from_numpy(dy).to(torch.bfloat16).float().numpy()  # the values the GPU sees
    h0 = rng.standard_normal((B, H, N, P)).astype(np.float32)
    dfin = rng.standard_normal((B, H, N, P)).astype(np.float32)
    g, _ = run_gpu(inp, dy, h0, dfin, dy_dtype, mma)
    ref = bwd_oracle.backward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, dy, h0=h0, dfinal=dfin, terms=True)
    errs = grad_errors(g, ref, inp.dt, inp.A)
    say("  " + ", ".join(f"{k} {v:.3g}" for k, v in errs.items()))
    for k in KEYS:
        assert errs[k] <= tol_for(k, mma), (k, errs[k])


@pytest.mark.parametrize("shape", [s for s in BWD_SHAPES if s[4] % 64 == 0 and (s[7], s[5]) in
                                   ((256, 128), (128, 256), (128, 128), (256, 64), (128, 64))],
                         ids=lambda s: s[0])
def test_backward_reversed_reading_matches_copies(shape):
    """With bf16 operands, bf16 x, B, C and bf16 dy on the head-group shapes
    the adjoint pass reads dy, C and B in reversed order where they are; the
    same dy values passed as fp32 go through reversed bf16 copies instead.
    The gradients that depend only on the two passes (dx, ddt, dA, dD, the
    initial-state gradient) are bit for bit the same either way."""
    name, B, L, H, P, N, G, Q = shape
    say(f"backward reversed reading vs copies {shape}")
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype="bf16", seed=67, dt_shift=2.0)
    rng = np.random.default_rng(68)
    dy = torch.from_numpy(rng.standard_normal(inp.x.shape).astype(np.float32)).to(torch.bfloat16).float().numpy()
    h0 = rng.standard_normal((B, H, N, P)).astype(np.float32)
    dfin = rng.standard_normal((B, H, N, P)).astype(np.float32)
    g_rev, _ = run_gpu(inp, dy, h0, dfin, "bf16", "bf16")
    g_cpy, _ = run_gpu(inp, dy, h0, dfin, "f32", "bf16")
    for k in ("dx", "ddt", "dA", "dD", "dh0"):
        assert torch.equal(g_rev[k], g_cpy[k]), k


def test_backward_without_initial_or_final():
    """No initial state and no final-state gradient (both NULL through the ABI)."""
    B, L, H, P, N, G, Q = 2, 192, 2, 32, 32, 1, 64
    say("backward without h0 / dfinal")
    inp = make_inputs(B, L, H, P, N, G, Q, seed=63)
    dy = np.random.default_rng(64).standard_normal(inp.x.shape).astype(np.float32)
    g, _ = run_gpu(inp, dy, None, None)
    ref = bwd_oracle.backward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, dy, terms=True)
    errs = grad_errors(g, ref, inp.dt, inp.A)
    say("  " + ", ".join(f"{k} {v:.3g}" for k, v in errs.items()))
    for k in KEYS:
        assert errs[k] <= TOL["f32"], (k, errs[k])


def test_backward_zero_dy_only_final_gradient():
    """dy = 0: only dfinal drives the gradients, so dC = 0 and dD = 0 exactly
    (no term reaches them), and the rest matches the oracle."""
    B, L, H, P, N, G, Q = 1, 128, 2, 16, 32, 1, 32
    say("backward with dy = 0")
    # slow decay (dt ~ softplus(N(0,1) - 4)), so that dfinal still reaches the first token
    inp = make_inputs(B, L, H, P, N, G, Q, seed=65, dt_shift=4.0)
    rng = np.random.default_rng(66)
    dy = np.zeros(inp.x.shape, np.float32)
    dfin = rng.standard_normal((B, H, N, P)).astype(np.float32)
    g, _ = run_gpu(inp, dy, None, dfin)
    assert torch.count_nonzero(g["dC"]) == 0 and torch.count_nonzero(g["dD"]) == 0
    ref = bwd_oracle.backward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, dy, dfinal=dfin, terms=True)
    errs = grad_errors(g, ref, inp.dt, inp.A, keys=("dx", "ddt", "dA", "dB", "dh0"))
    say("  " + ", ".join(f"{k} {v:.3g}" for k, v in errs.items()))
    for k, v in errs.items():
        assert v <= TOL["f32"], (k, v)


def _dot(a, b, dims):
    return (a.double() * b.double()).sum(dim=dims)


def _close(lhs, rhs, scale, tol):
    err = float(((lhs - rhs).abs() / scale.clamp_min(1e-30)).max())
    return err, err <= tol


@pytest.mark.parametrize("mma", ["f32", "bf16"])
@pytest.mark.parametrize("workload", ["mamba2_2p7b_layer", "grouped_n256"])
def test_backward_full_size_sampled_and_identities(workload, mma):
    """Full-size workloads: the 2.7B-layer shape (B=2, L=8192, H=80, P=64,
    N=128, G=1, Q=256) and the grouped one (B=8, L=4096, H=64, P=64, N=256,
    G=8, Q=128), bf16 inputs."""
    inp = workload_inputs(workload)
    B, L, H, P = inp.x.shape
    N, G = inp.Bm.shape[3], inp.Bm.shape[2]
    say(f"backward at {workload} B={B} L={L} H={H} P={P} N={N} G={G} mma={mma}")
    rng = np.random.default_rng(67)
    dy = rng.standard_normal(inp.x.shape).astype(np.float32)
    h0 = rng.standard_normal((B, H, N, P)).astype(np.float32)
    dfin = rng.standard_normal((B, H, N, P)).astype(np.float32)
    g, t = run_gpu(inp, dy, h0, dfin, mma=mma)
    tol = TOL[mma]
    for k in KEYS:
        assert torch.isfinite(g[k]).all(), k
    # forward on the same inputs, fp32 matrix operands
    sh = ops.shape_of(t, inp.chunk)
    y, fin = ops.ssd_forward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], initial_states=_cuda(h0),
                             y_dtype="f32", mma="f32")
    torch.cuda.synchronize()
    x = t["x"].float()
    dy_t, D = _cuda(dy), t["D"].double()
    Bm, Cm = t["Bm"].float(), t["Cm"].float()
    # per token: C . dC = sum_h dy . (y - D x)
    lhs = _dot(Cm, g["dC"], (2, 3))
    ymd = y.double() - D[None, None, :, None] * x.double()
    rhs = (dy_t.double() * ymd).sum(dim=(2, 3))
    scale = (Cm.double().abs() * g["dC"].double().abs()).sum(dim=(2, 3)) + (dy_t.double() * ymd).abs().sum(dim=(2, 3))
    e1, ok1 = _close(lhs, rhs, scale, tol)
    # per token: B . dB = sum_h x . (dx - D dy)
    lhs = _dot(Bm, g["dB"], (2, 3))
    dxm = g["dx"].double() - D[None, None, :, None] * dy_t.double()
    rhs = (x.double() * dxm).sum(dim=(2, 3))
    scale = (Bm.double().abs() * g["dB"].double().abs()).sum(dim=(2, 3)) + (x.double() * dxm).abs().sum(dim=(2, 3))
    e2, ok2 = _close(lhs, rhs, scale, tol)
    # per (b, h): <dx, x> + <dh0, h0> = <dy, y> + <dfinal, final>
    h0_t, dfin_t = _cuda(h0), _cuda(dfin)
    lhs = _dot(g["dx"], x, (1, 3)) + _dot(g["dh0"], h0_t, (2, 3))
    rhs = _dot(dy_t, y, (1, 3)) + _dot(dfin_t, fin, (2, 3))
    scale = ((g["dx"].double() * x.double()).abs().sum(dim=(1, 3)) + (g["dh0"].double() * h0_t.double()).abs().sum(dim=(2, 3))
             + (dy_t.double() * y.double()).abs().sum(dim=(1, 3)) + (dfin_t.double() * fin.double()).abs().sum(dim=(2, 3)))
    e3, ok3 = _close(lhs, rhs, scale, tol)
    # dD = sum over tokens of dy . x
    dD_ref = _dot(dy_t, x, (0, 1, 3))
    e4 = float(((g["dD"].double() - dD_ref).abs() / dD_ref.abs().max()).max())
    say(f"  identities: C.dC {e1:.3g}, B.dB {e2:.3g}, linear in x,h0 {e3:.3g}, dD {e4:.3g}")
    assert ok1 and ok2 and ok3 and e4 <= tol
    # sampled heads against the oracle on their (batch, head) slices
    heads = sorted(set([0, H - 1] + np.random.default_rng(68).choice(H, 1).tolist()))
    for h in heads:
        dA_ref, dA_scale = 0.0, 0.0
        gg = h // (H // G)
        for b in range(B):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
            ref = bwd_oracle.backward(inp.x[sl], inp.dt[sl], inp.A[h:h + 1], inp.Bm[b:b + 1, :, gg:gg + 1],
                                      inp.Cm[b:b + 1, :, gg:gg + 1], inp.D[h:h + 1], dy[sl],
                                      h0=h0[b:b + 1, h:h + 1], dfinal=dfin[b:b + 1, h:h + 1], terms=True)
            dA_ref += ref["dA"][0]
            dts, be = inp.dt[sl].astype(np.float64), np.abs(ref["beta"])
            dA_scale += float((dts * (np.abs(ref["dlogr"]) + 2 * dts * be)).sum())
            gs = {"dx": g["dx"][b:b + 1, :, h:h + 1], "ddt": g["ddt"][b:b + 1, :, h:h + 1],
                  "dh0": g["dh0"][b:b + 1, h:h + 1]}
            errs = grad_errors(gs, ref, inp.dt[sl], inp.A[h:h + 1], keys=("dx", "ddt", "dh0"))
            say(f"  head {h} row {b}: " + ", ".join(f"{k} {v:.3g}" for k, v in errs.items()))
            for k, v in errs.items():
                assert v <= tol_for(k, mma), (h, b, k, v)
        e = abs(float(g["dA"][h]) - dA_ref) / dA_scale
        say(f"  head {h}: dA err {e:.3g} (|dA| / sum of |terms| {abs(dA_ref) / dA_scale:.3g})")
        assert e <= tol_for("dA", mma)
