"""GPU parity: every ABI call against the fp64 oracle on the same seeded inputs.

Small shapes span several tiles and every tail the kernels have (partial
head tile in the cumsum, 16/32-wide P slices, zero-padded state contraction,
32-token chunks, grouped B/C); each kernel is also checked in isolation by
feeding it oracle intermediates.  Acceptance (max|err|/max|ref| per tensor):
1e-6 for the cumsum, 1e-4 for the fp32-MFMA path, 1e-2 for the bf16-operand
path.
"""
import math

import numpy as np
import pytest
import torch

from gpu_common import (TOL_CUMSUM, TOL_PASSING, gpu_forward, make_inputs, oracle, relerr, say, tol_for,
                        upload)
from mamba_ssd_scan_chunk_amd import ops
from mamba_ssd_scan_chunk_amd._lib import SSDError
from oracle.oracle import dA_cumsum_ref, dt_bhl_ref

pytestmark = pytest.mark.gpu

# (name, B, L, H, P, N, G, Q)
SHAPES = [
    ("tiny", 1, 256, 2, 16, 16, 1, 64),
    ("two_chunks", 2, 512, 4, 64, 128, 1, 256),
    ("grouped", 1, 256, 6, 32, 64, 2, 64),
    ("ragged_tiles", 2, 384, 3, 48, 48, 3, 128),
    ("n256", 1, 256, 4, 64, 256, 2, 128),
    ("q32_h20", 1, 96, 20, 32, 32, 4, 32),
    ("p128", 1, 256, 2, 128, 64, 1, 128),
    # ragged last chunk (L % Q != 0): head-group kernels, then generic ones
    ("ragged_q256", 2, 300, 4, 64, 128, 1, 256),
    ("ragged_q128_n256", 1, 130, 4, 64, 256, 2, 128),
    ("ragged_q64", 1, 200, 3, 48, 48, 3, 64),
    ("ragged_q256_n64", 2, 600, 4, 64, 64, 2, 256),
    ("ragged_q64_n128", 2, 300, 4, 64, 128, 2, 64),
    ("q64_n256", 1, 192, 2, 64, 256, 1, 64),
]
MODES = [("f32", "f32"), ("bf16", "f32"), ("f32", "bf16"), ("bf16", "bf16")]  # (input dtype, mma)


def _inp(shape, in_dtype, seed=0, **kw):
    name, B, L, H, P, N, G, Q = shape
    return make_inputs(B, L, H, P, N, G, Q, in_dtype=in_dtype, seed=seed, dt_shift=kw.pop("dt_shift", 1.0), **kw)


def _h0(inp, seed=5, scale=1.0):
    s = inp.shape
    return (scale * np.random.default_rng(seed).standard_normal(
        (s["batch"], s["nheads"], s["dstate"], s["headdim"]))).astype(np.float32)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_chunk_cumsum(shape):
    say(f"chunk_cumsum {shape}")
    inp = _inp(shape, "f32")
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    torch.cuda.synchronize()
    ref = dA_cumsum_ref(inp.dt, inp.A, inp.chunk)
    # positions past a ragged end hold the last valid sum (the ABI's layout
    # convention: missing tokens count as dt = 0)
    name, B, L, H, P, N, G, Q = shape
    nc, q = -(-L // Q), L - (-(-L // Q) - 1) * Q
    ref[:, :, nc - 1, q:] = ref[:, :, nc - 1, q - 1:q]
    assert relerr(dA, ref) <= TOL_CUMSUM
    # all terms share a sign, so the error is also small elementwise
    g = dA.double().cpu().numpy()
    assert (np.abs(g - ref) <= TOL_CUMSUM * np.abs(ref) + 1e-30).all()
    assert np.array_equal(dtb.cpu().numpy(), dt_bhl_ref(inp.dt, inp.chunk).astype(np.float32))
    # dt_bhl is optional
    dA2, none = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"], with_dt=False)
    torch.cuda.synchronize()
    assert none is None and torch.equal(dA2, dA)


@pytest.mark.parametrize("mode", MODES, ids=["-".join(m) for m in MODES])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_chunk_state(shape, mode):
    in_dtype, mma = mode
    say(f"chunk_state {shape} {mode}")
    inp = _inp(shape, in_dtype, seed=1)
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    S = ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, mma=mma)
    torch.cuda.synchronize()
    ref = oracle().chunk_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk)
    e = relerr(S, ref)
    say(f"  rel err {e:.3g}")
    assert e <= tol_for(mma)


@pytest.mark.parametrize("mode", [("f32", "f32"), ("bf16", "f32"), ("f32", "bf16")], ids=["f32-f32", "bf16-f32", "f32-bf16"])
def test_chunk_state_head_sharing(mode):
    """The generic chunk-state kernel serves four heads of a group per block
    (one staged B tile for all four) once the grid still has two blocks per
    compute unit: 8 x 32 chunks x 2 head quads = 512 blocks here, the
    threshold on a 256-unit GPU.  Against the oracle, fp32 and bf16 states."""
    shape = ("head_sharing", 8, 2048, 8, 64, 32, 1, 64)
    in_dtype, mma = mode
    say(f"chunk_state head sharing {shape} {mode}")
    inp = _inp(shape, in_dtype, seed=31)
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    S = ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, mma=mma)
    S16 = ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, mma=mma, states_dtype="bf16")
    torch.cuda.synchronize()
    from mamba_ssd_scan_chunk_amd.inputs import bf16_round
    assert np.array_equal(S16.view(torch.int16).cpu().numpy().view(np.uint16), bf16_round(S.cpu().numpy()))
    ref = oracle().chunk_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk)
    e = relerr(S, ref)
    say(f"  rel err {e:.3g}")
    assert e <= tol_for(mma)


@pytest.mark.parametrize("mode", MODES, ids=["-".join(m) for m in MODES])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_chunk_state_bf16_storage(shape, mode):
    """Chunk states stored as bf16 are the fp32 states of the same call rounded
    to nearest even (the accumulators are the same; only the store differs),
    on every kernel instance, and within the bf16 bound of the oracle."""
    from mamba_ssd_scan_chunk_amd.inputs import bf16_round
    in_dtype, mma = mode
    say(f"chunk_state bf16 storage {shape} {mode}")
    inp = _inp(shape, in_dtype, seed=1)
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    S32 = ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, mma=mma)
    S16 = ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, mma=mma, states_dtype="bf16")
    torch.cuda.synchronize()
    assert S16.dtype == torch.bfloat16
    got = S16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, bf16_round(S32.cpu().numpy()))
    ref = oracle().chunk_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk)
    e = relerr(S16.float(), ref)
    say(f"  rel err {e:.3g}")
    assert e <= tol_for(mma) + 2.0 ** -8


@pytest.mark.parametrize("with_h0", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_state_passing_bf16_chunk_states(shape, with_h0):
    """The state passing over bf16 chunk states widens them exactly and runs
    the same fp32 recurrence: bit-equal to the fp32 call over the widened
    values, for fp32 and bf16 carried states and for the bf16 in-place form;
    within the bf16 bound of the oracle."""
    say(f"state_passing bf16 chunk states {shape} h0={with_h0}")
    inp = _inp(shape, "f32", seed=2, dt_shift=3.0)
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    o = oracle()
    S = o.chunk_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk)
    h0 = _h0(inp) if with_h0 else None
    Hin, fin = o.carried_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk, h0=h0)
    dA, _ = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    S16 = torch.from_numpy(S.astype(np.float32)).cuda().to(torch.bfloat16)
    S16w = S16.float()
    h0_t = None if h0 is None else torch.from_numpy(h0).cuda()
    c_ref32, f_ref = ops.ssd_state_passing(sh, S16w, dA, initial_states=h0_t)
    c_ref16, _ = ops.ssd_state_passing(sh, S16w, dA, initial_states=h0_t, carried_dtype="bf16")
    c32, f1 = ops.ssd_state_passing(sh, S16, dA, initial_states=h0_t, carried_dtype="f32")
    c16, f2 = ops.ssd_state_passing(sh, S16, dA, initial_states=h0_t, carried_dtype="bf16")
    S16b = S16.clone()
    c16i, f3 = ops.ssd_state_passing(sh, S16b, dA, initial_states=h0_t, in_place=True)
    torch.cuda.synchronize()
    assert c16i.data_ptr() == S16b.data_ptr() and c16i.dtype == torch.bfloat16
    assert torch.equal(c32, c_ref32) and torch.equal(c16, c_ref16) and torch.equal(c16i, c_ref16)
    assert torch.equal(f1, f_ref) and torch.equal(f2, f_ref) and torch.equal(f3, f_ref)
    e1, e2 = relerr(c32, Hin), relerr(f1, fin)
    say(f"  rel err carried {e1:.3g} final {e2:.3g}")
    assert e1 <= 2.0 ** -8 and e2 <= 2.0 ** -8


@pytest.mark.parametrize("states_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("nc", [32, 40, 71])
def test_state_passing_long_chains(nc, states_dtype):
    """Few heads and many chunks (fewer than 4 waves per compute unit): the
    state passing then keeps 16 chunk loads per thread in flight; chains of
    two full batches, with a remainder of 8, and with an odd remainder.  The
    carried and final states equal the fp32 recurrence over the same stored
    chunk states bit for bit (fp32 carried, then bf16 carried = its rounding)
    and match the oracle."""
    from mamba_ssd_scan_chunk_amd.inputs import bf16_round
    shape = ("long_chain", 1, 32 * nc, 2, 32, 32, 1, 32)
    say(f"state_passing long chain nc={nc} states {states_dtype}")
    inp = _inp(shape, "f32", seed=3, dt_shift=5.0)
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    o = oracle()
    S = o.chunk_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk)
    h0 = _h0(inp)
    Hin, fin = o.carried_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk, h0=h0)
    dA, _ = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    S_t = torch.from_numpy(S.astype(np.float32)).cuda()
    if states_dtype == "bf16":
        S_t = S_t.to(torch.bfloat16)
    h0_t = torch.from_numpy(h0).cuda()
    c32, f32_ = ops.ssd_state_passing(sh, S_t, dA, initial_states=h0_t, carried_dtype="f32")
    c16, f16_ = ops.ssd_state_passing(sh, S_t, dA, initial_states=h0_t, carried_dtype="bf16")
    torch.cuda.synchronize()
    # the same recurrence run on the host in fp32 with the same fused multiply-adds is not
    # available in NumPy, so the bit-level check is between the two carried dtypes
    got = c16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, bf16_round(c32.cpu().numpy())) and torch.equal(f16_, f32_)
    e1, e2 = relerr(c32, Hin), relerr(f32_, fin)
    say(f"  rel err carried {e1:.3g} final {e2:.3g}")
    bound = TOL_PASSING if states_dtype == "f32" else 2.0 ** -8
    assert e1 <= bound and e2 <= bound


@pytest.mark.parametrize("with_h0", [False, True])
@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_state_passing(shape, in_place, with_h0):
    say(f"state_passing {shape} in_place={in_place} h0={with_h0}")
    inp = _inp(shape, "f32", seed=2, dt_shift=3.0)  # slow decay: carried states matter
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    o = oracle()
    S = o.chunk_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk)
    h0 = _h0(inp) if with_h0 else None
    Hin, fin = o.carried_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk, h0=h0)
    dA, _ = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    S_t = torch.from_numpy(S.astype(np.float32)).cuda()
    h0_t = None if h0 is None else torch.from_numpy(h0).cuda()
    carried, final = ops.ssd_state_passing(sh, S_t, dA, initial_states=h0_t, in_place=in_place)
    torch.cuda.synchronize()
    if in_place:
        assert carried.data_ptr() == S_t.data_ptr()
    e1, e2 = relerr(carried, Hin), relerr(final, fin)
    say(f"  rel err carried {e1:.3g} final {e2:.3g}")
    assert e1 <= TOL_PASSING and e2 <= TOL_PASSING


@pytest.mark.parametrize("with_h0", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_state_passing_bf16_carried(shape, with_h0):
    """bf16 carried states are the fp32 recurrence rounded to nearest even:
    bit-equal to rounding the fp32 variant's carried states, and within the
    bf16 rounding bound of the oracle; the final states stay fp32."""
    from mamba_ssd_scan_chunk_amd.inputs import bf16_round
    say(f"state_passing bf16 carried {shape} h0={with_h0}")
    inp = _inp(shape, "f32", seed=2, dt_shift=3.0)
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    o = oracle()
    S = o.chunk_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk)
    h0 = _h0(inp) if with_h0 else None
    Hin, fin = o.carried_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk, h0=h0)
    dA, _ = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    S_t = torch.from_numpy(S.astype(np.float32)).cuda()
    h0_t = None if h0 is None else torch.from_numpy(h0).cuda()
    c32, f32_ = ops.ssd_state_passing(sh, S_t, dA, initial_states=h0_t)
    c16, f16_ = ops.ssd_state_passing(sh, S_t, dA, initial_states=h0_t, carried_dtype="bf16")
    torch.cuda.synchronize()
    assert c16.dtype == torch.bfloat16
    got = c16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, bf16_round(c32.cpu().numpy()))
    assert torch.equal(f16_, f32_)
    e1, e2 = relerr(c16.float(), Hin), relerr(f16_, fin)
    say(f"  rel err carried(bf16) {e1:.3g} final {e2:.3g}")
    assert e1 <= 2.0 ** -8 and e2 <= TOL_PASSING


@pytest.mark.parametrize("y_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", MODES, ids=["-".join(m) for m in MODES])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_chunk_scan(shape, mode, y_dtype):
    in_dtype, mma = mode
    if mma == "f32" and y_dtype == "bf16":
        pytest.skip("bf16 output rounding alone exceeds the fp32-path bar")
    say(f"chunk_scan {shape} {mode} y={y_dtype}")
    inp = _inp(shape, in_dtype, seed=3, dt_shift=2.0)
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    o = oracle()
    h0 = _h0(inp)
    Hin, _ = o.carried_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk, h0=h0)
    yref, _ = o.forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0=h0)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    car = torch.from_numpy(Hin.astype(np.float32)).cuda()
    y = ops.ssd_chunk_scan(sh, t["x"], t["Bm"], t["Cm"], dtb, dA, car, t["D"], y_dtype=y_dtype, mma=mma)
    torch.cuda.synchronize()
    e = relerr(y, yref)
    say(f"  rel err {e:.3g}")
    assert e <= tol_for(mma)
    # bf16 carried states: on the bf16 path they are the matrix operands the
    # kernel rounds fp32 carried states to, so y is bit-identical; on the fp32
    # path they widen exactly and stay within the bf16 bar
    y16 = ops.ssd_chunk_scan(sh, t["x"], t["Bm"], t["Cm"], dtb, dA, car.to(torch.bfloat16), t["D"],
                             y_dtype=y_dtype, mma=mma)
    torch.cuda.synchronize()
    if mma == "bf16":
        assert torch.equal(y16, y)
    else:
        assert relerr(y16, yref) <= tol_for("bf16")


@pytest.mark.parametrize("mma", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [SHAPES[1], SHAPES[4]], ids=[SHAPES[1][0], SHAPES[4][0]])
def test_bf16_output_rounding_is_rne(shape, mma):
    """The bf16 output is the round-to-nearest-even of the fp32 output of the
    same kernel (same accumulators, only the final conversion differs)."""
    from mamba_ssd_scan_chunk_amd.inputs import bf16_round
    say(f"bf16 output rounding {shape} {mma}")
    inp = _inp(shape, "bf16", seed=12, dt_shift=2.0)
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    S = ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, mma=mma)
    car, _ = ops.ssd_state_passing(sh, S, dA)
    y32 = ops.ssd_chunk_scan(sh, t["x"], t["Bm"], t["Cm"], dtb, dA, car, t["D"], y_dtype="f32", mma=mma)
    y16 = ops.ssd_chunk_scan(sh, t["x"], t["Bm"], t["Cm"], dtb, dA, car, t["D"], y_dtype="bf16", mma=mma)
    torch.cuda.synchronize()
    expect = bf16_round(y32.cpu().numpy())
    got = y16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, expect)


@pytest.mark.parametrize("mode", MODES, ids=["-".join(m) for m in MODES])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_forward(shape, mode):
    in_dtype, mma = mode
    say(f"forward {shape} {mode}")
    inp = _inp(shape, in_dtype, seed=4, dt_shift=2.0)
    h0 = _h0(inp)
    y_dtype = "f32" if mma == "f32" else in_dtype
    y, fin = gpu_forward(inp, mma, y_dtype=y_dtype, h0=h0)
    yref, fref = oracle().forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0=h0)
    e1, e2 = relerr(y, yref), relerr(fin, fref)
    say(f"  rel err y {e1:.3g} final {e2:.3g}")
    assert e1 <= tol_for(mma) and e2 <= tol_for(mma)


@pytest.mark.parametrize("mma", ["f32", "bf16"])
def test_forward_padded_variable_lengths(mma):
    """Sequences of different lengths in one padded batch: a padding token
    with dt = 0 leaves the state unchanged (decay exp(0) = 1, input term 0),
    so setting dt = 0 past each sequence's end gives, for every sequence, the
    outputs of its own tokens and its final state exactly as if it ran alone
    (outputs at padding positions are not meaningful)."""
    lens = [300, 768, 517]
    B, L, H, P, N, G, Q = len(lens), 768, 4, 64, 128, 2, 256
    say(f"padded variable lengths {lens} {mma}")
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype="bf16", seed=16, dt_shift=2.0)
    for b, n in enumerate(lens):
        inp.dt[b, n:] = 0.0
    h0 = _h0(inp)
    y, fin = gpu_forward(inp, mma, y_dtype="f32", h0=h0)
    o = oracle()
    for b, n in enumerate(lens):
        sl = lambda a: np.ascontiguousarray(a[b:b + 1, :n])
        yref, fref = o.forward(sl(inp.x), sl(inp.dt), inp.A, sl(inp.Bm), sl(inp.Cm), inp.D, h0=h0[b:b + 1])
        e1, e2 = relerr(y[b:b + 1, :n], yref), relerr(fin[b:b + 1], fref)
        say(f"  sequence {b} (length {n}): rel err y {e1:.3g} final {e2:.3g}")
        assert e1 <= tol_for(mma) and e2 <= tol_for(mma)


# ---------------------------------------------------------------- numerics stress
STRESS = {
    # carried state dominates: tiny dt, slow A
    "slow_decay": dict(dt_shift=7.0, log_a_range=(math.log(0.1), 0.0)),
    # no decay at all (the jump formula): the state grows over the sequence
    "zero_decay": dict(A_override=0.0),
    # memoryless: exp(G) underflows to exactly 0 within a few tokens
    "fast_decay": dict(dt_shift=-3.0),
}


@pytest.mark.parametrize("mma", ["f32", "bf16"])
@pytest.mark.parametrize("case", list(STRESS), ids=list(STRESS))
def test_forward_stress(case, mma):
    shape = ("stress", 1, 1024, 4, 64, 64, 1, 128)
    say(f"forward stress {case} {mma}")
    kw = dict(STRESS[case])
    inp = _inp(shape, "bf16", seed=6, **kw)
    h0 = _h0(inp)
    y, fin = gpu_forward(inp, mma, y_dtype="f32", h0=h0)
    yref, fref = oracle().forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0=h0)
    e1, e2 = relerr(y, yref), relerr(fin, fref)
    say(f"  rel err y {e1:.3g} final {e2:.3g}")
    assert e1 <= tol_for(mma) and e2 <= tol_for(mma)


@pytest.mark.parametrize("L,k", [(1024, 512), (1000, 333)], ids=["aligned", "ragged"])
@pytest.mark.parametrize("mma", ["f32", "bf16"])
def test_split_chaining(mma, L, k):
    """final states of the first part fed as initial states of the second part
    reproduce the unsplit run (sequence resume), also when the split and the
    ends are not chunk-aligned (every part then has a ragged last chunk)."""
    say(f"split chaining {mma} L={L} k={k}")
    B, H, P, N, G, Q = 2, 4, 64, 128, 1, 256
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype="bf16", seed=8, dt_shift=4.0)
    t = upload(inp)
    sh_full = ops.shape_of(t, Q)
    part = lambda a, lo, hi: a[:, lo:hi].contiguous()
    sh_half = ops.SSDShape.make(B, k, H, P, N, G, Q)
    sh_rest = ops.SSDShape.make(B, L - k, H, P, N, G, Q)
    y_full, f_full = ops.ssd_forward(sh_full, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], y_dtype="f32",
                                     mma=mma)
    y1, f1 = ops.ssd_forward(sh_half, part(t["x"], 0, k), part(t["dt"], 0, k), t["A"], part(t["Bm"], 0, k),
                             part(t["Cm"], 0, k), t["D"], y_dtype="f32", mma=mma)
    y2, f2 = ops.ssd_forward(sh_rest, part(t["x"], k, L), part(t["dt"], k, L), t["A"], part(t["Bm"], k, L),
                             part(t["Cm"], k, L), t["D"], initial_states=f1, y_dtype="f32", mma=mma)
    torch.cuda.synchronize()
    yref, fref = oracle().forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
    y_cat = torch.cat([y1, y2], dim=1)
    assert relerr(y_cat, yref) <= tol_for(mma) and relerr(f2, fref) <= tol_for(mma)
    assert relerr(y_cat, y_full.double().cpu().numpy()) <= tol_for(mma)


# (name, B, L, H, P, N, G, Q): shapes of the bf16 head-group kernels, where the
# one-call forward hands the carried states to the chunk scan as bf16
HG_SHAPES = [
    ("ragged_q256", 2, 300, 6, 64, 128, 2, 256),
    ("q256_n128", 2, 768, 6, 64, 128, 2, 256),
    ("q128_n256", 1, 512, 4, 128, 256, 2, 128),
    ("q128_n128", 2, 384, 3, 64, 128, 1, 128),
    ("q256_n64", 2, 512, 4, 64, 64, 1, 256),
    ("ragged_q128_n64", 1, 300, 4, 128, 64, 2, 128),
    ("generic_q64", 1, 256, 6, 32, 64, 2, 64),  # the generic chunk-scan kernel
]


@pytest.mark.parametrize("y_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", HG_SHAPES, ids=[s[0] for s in HG_SHAPES])
def test_forward_bitwise_equals_split_calls(shape, y_dtype):
    """On the bf16 path the one-call forward stores the chunk states as bf16
    and passes the carried states to the chunk scan rounded to bf16, exactly
    the operand values the chunk scan rounds fp32 carried states to: y and the
    final states must equal the split calls (bf16 chunk states, either carried
    dtype, or the fused state call) bit for bit."""
    say(f"forward vs split calls {shape} y {y_dtype}")
    inp = _inp(shape, "bf16", seed=12, dt_shift=2.0)
    h0 = torch.from_numpy(_h0(inp)).cuda()
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    y_f, fin_f = ops.ssd_forward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], initial_states=h0,
                                 y_dtype=y_dtype, mma="bf16")
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    name, B, L, H, P, N, G, Q = shape
    # the forward's state step is either the two-call path or (N, P multiples
    # of 64) the fused state call; the outputs must equal one of them exactly
    S = ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, mma="bf16", states_dtype="bf16")
    fused_ok = N % 64 == 0 and P % 64 == 0
    for cdt in ["f32", "bf16"]:
        states = [ops.ssd_state_passing(sh, S, dA, initial_states=h0, carried_dtype=cdt)]
        if fused_ok:
            states.append(ops.ssd_chunk_state_passing(sh, t["x"], t["Bm"], dtb, dA, initial_states=h0,
                                                      carried_dtype=cdt))
        match = False
        for car, fin_s in states:
            y_s = ops.ssd_chunk_scan(sh, t["x"], t["Bm"], t["Cm"], dtb, dA, car, t["D"], y_dtype=y_dtype,
                                     mma="bf16")
            torch.cuda.synchronize()
            match = match or (torch.equal(y_f, y_s) and torch.equal(fin_f, fin_s))
        assert match, cdt


# (name, B, L, H, P, N, G, Q): shapes of the fused state path (N, P multiples of 64)
FUSED_SHAPES = [
    ("ragged_q256", 2, 300, 6, 64, 128, 2, 256),
    ("ragged_q64", 1, 100, 2, 64, 64, 1, 64),
    ("q256_n128", 2, 768, 6, 64, 128, 2, 256),
    ("q128_n256", 1, 512, 4, 128, 256, 2, 128),
    ("q128_n128", 2, 384, 3, 64, 128, 1, 128),
    ("q64_n64", 1, 320, 5, 64, 64, 5, 64),
    ("q32_p128", 1, 96, 2, 128, 64, 1, 32),
    ("q64_n128", 1, 256, 4, 64, 128, 2, 64),
    ("ragged_q32_n128", 1, 200, 4, 64, 128, 2, 32),  # two heads per block, ragged last chunk
]


@pytest.mark.parametrize("carried_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_h0", [False, True])
@pytest.mark.parametrize("shape", FUSED_SHAPES, ids=[s[0] for s in FUSED_SHAPES])
def test_chunk_state_passing(shape, with_h0, carried_dtype):
    """Fused state path against the oracle; on the shapes of the head-group
    chunk-state kernel (same fragment order) also bit for bit against the two
    calls it fuses."""
    say(f"chunk_state_passing {shape} h0={with_h0} carried={carried_dtype}")
    name, B, L, H, P, N, G, Q = shape
    inp = _inp(shape, "bf16", seed=13, dt_shift=3.0)
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    o = oracle()
    h0 = _h0(inp) if with_h0 else None
    h0_t = None if h0 is None else torch.from_numpy(h0).cuda()
    Hin, fin = o.carried_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk, h0=h0)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    car, fin_g = ops.ssd_chunk_state_passing(sh, t["x"], t["Bm"], dtb, dA, initial_states=h0_t,
                                             carried_dtype=carried_dtype)
    torch.cuda.synchronize()
    e1, e2 = relerr(car.float(), Hin), relerr(fin_g, fin)
    say(f"  rel err carried {e1:.3g} final {e2:.3g}")
    assert e1 <= tol_for("bf16") and e2 <= tol_for("bf16")
    if (Q, N) in ((256, 128), (128, 256)):
        S = ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, mma="bf16")
        car2, fin2 = ops.ssd_state_passing(sh, S, dA, initial_states=h0_t, carried_dtype=carried_dtype)
        torch.cuda.synchronize()
        assert torch.equal(car, car2) and torch.equal(fin_g, fin2)


# (name, B, L, H, P, N, G, Q): shapes of the fused forward (chunk 128, N 256)
FWD_FUSED_SHAPES = [
    ("one_head_pair", 1, 256, 2, 64, 256, 1, 128),
    ("ragged_g2", 2, 300, 4, 64, 256, 2, 128),
    ("p128", 1, 512, 2, 128, 256, 1, 128),
    ("g8_ragged", 2, 600, 16, 64, 256, 8, 128),
    ("one_short_chunk", 1, 50, 1, 64, 256, 1, 128),
    ("p192_three_slices", 1, 300, 3, 192, 256, 3, 128),
]


@pytest.mark.parametrize("with_h0", [False, True])
@pytest.mark.parametrize("shape", FWD_FUSED_SHAPES, ids=[s[0] for s in FWD_FUSED_SHAPES])
def test_forward_fused_kernel(shape, with_h0, monkeypatch):
    """The fused forward (state walk and chunk output in one kernel, taken with
    the tuning override path=fwd) against the oracle on every element of y
    and the final states; its final states bit for bit those of the fused
    state walk (same operands, same order); its y differs in the last bits
    from both two-kernel compositions (exact per-element decays instead of
    factorized ones), which shows that the fused kernel ran."""
    say(f"forward fused kernel {shape} h0={with_h0}")
    name, B, L, H, P, N, G, Q = shape
    inp = _inp(shape, "bf16", seed=23, dt_shift=3.0)
    h0 = _h0(inp) if with_h0 else None
    monkeypatch.setenv("SSD_TUNE", "path=fwd")
    y, fin = gpu_forward(inp, "bf16", y_dtype="bf16", h0=h0)
    yref, fref = oracle().forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0=h0)
    e1, e2 = relerr(y, yref), relerr(fin, fref)
    say(f"  rel err y {e1:.3g} final {e2:.3g}")
    assert e1 <= tol_for("bf16") and e2 <= tol_for("bf16")
    monkeypatch.setenv("SSD_TUNE", "path=fused")
    y_w, fin_w = gpu_forward(inp, "bf16", y_dtype="bf16", h0=h0)
    monkeypatch.setenv("SSD_TUNE", "path=split")
    y_s, _ = gpu_forward(inp, "bf16", y_dtype="bf16", h0=h0)
    assert torch.equal(fin, fin_w)
    assert not torch.equal(y, y_w) and not torch.equal(y, y_s)


def test_forward_state_path_choice():
    """ssd_forward takes the fused state path when it has at least two blocks
    per compute unit (blocks of 128 state rows where N is a multiple of 128
    and the chunk at most 128 tokens, else 64: 8 x 64 heads x 1 row block =
    512 here), else the two-kernel path; either way y and the final states
    match the oracle, and bit for bit the composition of the ABI calls of the
    path it takes (at chunk 64 the two state paths round differently, so the
    check tells them apart)."""
    shape = ("fwd_path", 8, 256, 64, 64, 128, 8, 64)
    say(f"forward state path choice {shape}")
    name, B, L, H, P, N, G, Q = shape
    inp = _inp(shape, "bf16", seed=15, dt_shift=2.0)
    h0 = _h0(inp)
    y, fin = gpu_forward(inp, "bf16", y_dtype="bf16", h0=h0)
    yref, fref = oracle().forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, h0=h0)
    e1, e2 = relerr(y, yref), relerr(fin, fref)
    say(f"  rel err y {e1:.3g} final {e2:.3g}")
    assert e1 <= tol_for("bf16") and e2 <= tol_for("bf16")
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    h0_t = torch.from_numpy(h0).cuda()
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows = 128 if (N % 128 == 0 and Q <= 128) else 64
    fused = B * H * (N // rows) * (P // 64) >= 2 * cus
    if fused:
        car, fin_s = ops.ssd_chunk_state_passing(sh, t["x"], t["Bm"], dtb, dA, initial_states=h0_t,
                                                 carried_dtype="bf16")
    else:
        S = ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, mma="bf16", states_dtype="bf16")
        car, fin_s = ops.ssd_state_passing(sh, S, dA, initial_states=h0_t, in_place=True)
    y_s = ops.ssd_chunk_scan(sh, t["x"], t["Bm"], t["Cm"], dtb, dA, car, t["D"], y_dtype="bf16", mma="bf16")
    torch.cuda.synchronize()
    say(f"  {cus} compute units: {'fused' if fused else 'two-kernel'} state path expected")
    assert torch.equal(y, y_s) and torch.equal(fin, fin_s)


def test_chunk_state_passing_unsupported_and_no_final():
    say("chunk_state_passing unsupported / no final")
    inp = make_inputs(1, 128, 2, 48, 64, 1, 64, in_dtype="bf16", seed=14)  # P = 48: not a multiple of 64
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    with pytest.raises(SSDError):
        ops.ssd_chunk_state_passing(sh, t["x"], t["Bm"], dtb, dA)
    inp = make_inputs(1, 128, 2, 64, 64, 1, 64, in_dtype="bf16", seed=14)
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    with pytest.raises(SSDError):
        ops.ssd_chunk_state_passing(sh, t["x"], t["Bm"], dtb, dA, mma="f32")
    car, fin = ops.ssd_chunk_state_passing(sh, t["x"], t["Bm"], dtb, dA, want_final=False)
    car2, fin2 = ops.ssd_chunk_state_passing(sh, t["x"], t["Bm"], dtb, dA)
    torch.cuda.synchronize()
    assert fin is None and torch.equal(car, car2)


@pytest.mark.parametrize("mma", ["f32", "bf16"])
def test_deterministic(mma):
    """No atomics: two runs give bitwise identical outputs."""
    say(f"determinism {mma}")
    inp = make_inputs(2, 1024, 8, 64, 128, 2, 256, in_dtype="bf16", seed=9)
    y1, f1 = gpu_forward(inp, mma)
    y2, f2 = gpu_forward(inp, mma)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_errors_raise_through_binding():
    say("errors")
    inp = make_inputs(1, 128, 2, 64, 64, 1, 64, in_dtype="bf16", seed=10)
    t = upload(inp)
    bad = ops.SSDShape.make(1, 128, 2, 64, 64, 1, 16)  # chunk 16 unsupported
    with pytest.raises(ValueError):
        ops.ssd_chunk_cumsum(bad, t["dt"], t["A"], dA_cumsum=torch.empty(1, 2, 8, 64, device="cuda"))
    with pytest.raises(SSDError) as ei:
        ops.ssd_chunk_cumsum(bad, t["dt"], t["A"])
    assert ei.value.code == 4
    with pytest.raises(ValueError):  # dtype mismatch between x and B
        ops.ssd_chunk_state(ops.shape_of(t, 64), t["x"], t["Bm"].float(),
                            torch.empty(1, 2, 2, 64, device="cuda"), torch.empty(1, 2, 2, 64, device="cuda"))


# ---------------------------------------------------------------- packed sequences
# (name, B, H, P, N, G, Q, sequence lengths per row): boundaries at chunk starts,
# inside chunks, sequences shorter than a chunk, one spanning several chunks
PACKED = [
    ("hg_q256", 2, 4, 64, 128, 1, 256, [[256, 100, 1, 155, 300], [812]]),
    ("hg_q128_n256", 1, 4, 64, 256, 2, 128, [[5, 123, 128, 60, 200]]),
    ("generic_q64", 2, 3, 48, 48, 3, 64, [[64, 64, 10, 54, 100], [33, 31, 1, 1, 1, 1, 224]]),
    # whole chunks (the packed instances without ragged-row guards), sequences
    # starting on chunk boundaries and one-token sequences
    ("hg_q256_whole", 2, 4, 64, 128, 1, 256, [[256, 256, 1, 11, 500], [1024]]),
    ("hg_q128_n256_whole", 1, 4, 64, 256, 2, 128, [[128, 1, 127, 256]]),
    # enough chunks that the head-group kernels run two heads per block on a
    # 256-CU device
    ("hg_q256_two_heads", 2, 32, 64, 128, 1, 256, [[256, 300, 1, 467, 512, 512], [2048]]),
]


def _packed_seq_idx(rows, L):
    idx = np.zeros((len(rows), L), dtype=np.int32)
    for b, lens in enumerate(rows):
        assert sum(lens) == L
        idx[b] = np.repeat(np.arange(len(lens), dtype=np.int32), lens)
    return idx


@pytest.mark.parametrize("with_h0", [False, True])
@pytest.mark.parametrize("mma,in_dtype,y_dtype",
                         [("f32", "f32", "f32"), ("bf16", "bf16", "f32"), ("f32", "bf16", "f32"),
                          ("bf16", "bf16", "bf16")],
                         ids=["f32", "bf16", "f32_mma_bf16_in", "bf16_y_bf16"])
@pytest.mark.parametrize("case", PACKED, ids=[c[0] for c in PACKED])
def test_forward_packed_sequences(case, mma, in_dtype, y_dtype, with_h0):
    """Every sequence of a packed row gives the outputs of its own run from a
    zero state (the row's first one from the row's initial state), and the
    final state is that of the row's last sequence."""
    name, B, H, P, N, G, Q, rows = case
    L = sum(rows[0])
    say(f"packed sequences {name} {mma} in={in_dtype} y={y_dtype} h0={with_h0}")
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype=in_dtype, seed=17, dt_shift=2.0)
    t = upload(inp)
    sh = ops.shape_of(t, Q)
    sq = torch.from_numpy(_packed_seq_idx(rows, L)).cuda()
    h0 = _h0(inp) if with_h0 else None
    h0_t = None if h0 is None else torch.from_numpy(h0).cuda()
    # per-sequence states: after every sequence's last token, and after a token
    # inside each sequence longer than 2 (its middle)
    last, probes = [], []
    for b, lens in enumerate(rows):
        s0 = 0
        for k, n in enumerate(lens):
            last.append(b * L + s0 + n - 1)
            probes.append((b, k, s0, n))
            if n > 2:
                last.append(b * L + s0 + n // 2 - 1)
                probes.append((b, k, s0, n // 2))
            s0 += n
    last_t = torch.tensor(last, dtype=torch.int64, device="cuda")
    y, fin, sst = ops.ssd_forward_varlen(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], sq,
                                         initial_states=h0_t, y_dtype=y_dtype, mma=mma, seq_last=last_t)
    torch.cuda.synchronize()
    o = oracle()
    for b, lens in enumerate(rows):
        s0 = 0
        for k, n in enumerate(lens):
            sl = lambda a: np.ascontiguousarray(a[b:b + 1, s0:s0 + n])
            hk = h0[b:b + 1] if (h0 is not None and k == 0) else None
            yref, fref = o.forward(sl(inp.x), sl(inp.dt), inp.A, sl(inp.Bm), sl(inp.Cm), inp.D, h0=hk)
            e = relerr(y[b:b + 1, s0:s0 + n], yref)
            assert e <= tol_for(mma), (b, k, n, e)
            s0 += n
        ef = relerr(fin[b:b + 1], fref)
        say(f"  row {b}: {len(lens)} sequences, final rel err {ef:.3g}")
        assert ef <= tol_for(mma)
    # the states after the requested tokens
    worst = 0.0
    for q, (b, k, s0, n) in enumerate(probes):
        sl = lambda a: np.ascontiguousarray(a[b:b + 1, s0:s0 + n])
        hk = h0[b:b + 1] if (h0 is not None and k == 0) else None
        _, sref = o.forward(sl(inp.x), sl(inp.dt), inp.A, sl(inp.Bm), sl(inp.Cm), inp.D, h0=hk)
        worst = max(worst, relerr(sst[q:q + 1], sref))
    say(f"  {len(probes)} requested states: worst rel err {worst:.3g}")
    assert worst <= tol_for(mma)
    # one sequence per row reproduces the plain forward bit for bit
    one = torch.zeros((B, L), dtype=torch.int32, device="cuda")
    y1, f1 = ops.ssd_forward_varlen(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], one,
                                    initial_states=h0_t, y_dtype=y_dtype, mma=mma)
    y2, f2 = ops.ssd_forward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], initial_states=h0_t,
                             y_dtype=y_dtype, mma=mma)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


@pytest.mark.parametrize("states_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mode", MODES, ids=["-".join(m) for m in MODES])
@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_chunk_cumsum_state(shape, mode, states_dtype):
    """The combined first step (cumulative sums + chunk states, one kernel on
    the head-group shapes) equals ssd_chunk_cumsum then ssd_chunk_state bit
    for bit, and the oracle within the bar."""
    in_dtype, mma = mode
    say(f"chunk_cumsum_state {shape} {mode} states={states_dtype}")
    inp = _inp(shape, in_dtype, seed=2)
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    dA, dtb, S = ops.ssd_chunk_cumsum_state(sh, t["x"], t["Bm"], t["dt"], t["A"], mma=mma, states_dtype=states_dtype)
    dA2, dtb2 = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    S2 = ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb2, dA2, mma=mma, states_dtype=states_dtype)
    torch.cuda.synchronize()
    assert torch.equal(dA, dA2) and torch.equal(dtb, dtb2) and torch.equal(S, S2)
    ref = oracle().chunk_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.chunk)
    # bf16 storage rounds each state to 2^-9 relative, above the fp32 path's bar
    assert relerr(S.float(), ref) <= (tol_for(mma) if states_dtype == "f32" else tol_for("bf16"))
