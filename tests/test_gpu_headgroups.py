"""GPU parity of the head-group kernels with SEVERAL heads per block.

The head-group chunk scan and chunk-state kernels run a block over HG heads of
one B/C group, reusing the group's C.B^T tiles (chunk scan) or B fragments
(chunk states) across them, with the next head's tiles prefetched and
double-buffered while the current one computes.  The launchers take HG as
large as the grid allows while every compute unit still gets a block, so
small problems run HG = 1.  These mid-size shapes are chosen so that, on the
device's compute-unit count, HG >= 2 for every (chunk, dstate) instance of
both kernels (asserted from the launch rule), including the ragged-chunk
instance, a 128-column headdim (two column slices) and packed sequences.
Every (batch, head) pair of y, the final states and the chunk states is
compared with the fp64 oracle.
"""
import numpy as np
import pytest
import torch

from gpu_common import (chunk_state_hg_fused_cap, device_cus, heads_per_block, make_inputs, oracle, relerr, say,
                        tol_for, upload)
from mamba_ssd_scan_chunk_amd import ops

pytestmark = pytest.mark.gpu

# (name, B, L, H, P, N, G, Q)
CASES = [
    ("q256_n128", 2, 4096, 32, 64, 128, 1, 256),
    ("q128_n256", 2, 2048, 16, 64, 256, 2, 128),
    ("q128_n128", 2, 2048, 24, 64, 128, 1, 128),
    ("q256_n64", 2, 2048, 32, 64, 64, 1, 256),
    ("q128_n64", 2, 2048, 32, 64, 64, 2, 128),
    ("ragged_q256_n128", 2, 4000, 32, 64, 128, 1, 256),
    ("ragged_q128_n256", 1, 4000, 32, 64, 256, 2, 128),
    ("p128_q256_n128", 2, 2048, 16, 128, 128, 1, 256),
    ("q64_n128", 1, 2048, 16, 64, 128, 1, 64),
    ("q64_n256", 1, 1024, 32, 64, 256, 2, 64),
]
SCAN_HG = {(128, 64), (128, 128), (128, 256), (256, 64), (256, 128)}   # (Q, N) of the chunk-scan instances
STATE_HG = {(64, 128), (128, 128), (256, 128), (64, 256), (128, 256)}  # (Q, N) of the chunk-state instances


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


_CACHE = {}


def _case(case):
    """Inputs and every oracle result of one case, computed once."""
    name = case[0]
    if _CACHE.get("name") != name:
        _CACHE.clear()
        _, B, L, H, P, N, G, Q = case
        inp = make_inputs(B, L, H, P, N, G, Q, in_dtype="bf16", seed=41, dt_shift=1.0)
        o = oracle()
        say(f"  oracle: {B * H} pairs of {name}")
        yo, fo, bnd = o.recurrence(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, chunk=Q, want_boundary=True)
        S = o.chunk_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, Q)
        _CACHE.update(name=name, inp=inp, yo=yo, fo=fo, S=S)
    return _CACHE


def _pair_major(y):
    y = y.float().cpu().numpy()
    return np.ascontiguousarray(y.transpose(0, 2, 1, 3)).reshape(y.shape[0] * y.shape[2], y.shape[1], y.shape[3])


def _assert_multi_head(case):
    _, B, L, H, P, N, G, Q = case
    cus = device_cus()
    hg_scan = heads_per_block(B, L, H, P, N, G, Q, cus) if (Q, N) in SCAN_HG else None
    hg_state = heads_per_block(B, L, H, P, N, G, Q, cus) if (Q, N) in STATE_HG else None
    hg_state_fused = (heads_per_block(B, L, H, P, N, G, Q, cus, cap=chunk_state_hg_fused_cap(Q, N))
                      if (Q, N) in STATE_HG else None)
    say(f"  {cus} compute units: heads per block chunk_scan {hg_scan}, chunk_state {hg_state} "
        f"(with the cumsum fused: {hg_state_fused})")
    for v in (hg_scan, hg_state, hg_state_fused):
        assert v is None or v >= 2, "shape does not exercise several heads per block on this device"
    assert hg_scan is not None or hg_state is not None


@pytest.mark.parametrize("y_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_headgroup_forward(case, y_dtype):
    """ssd_forward (bf16 operands) on all pairs against the oracle."""
    say(f"head-group forward {case} y={y_dtype}")
    _assert_multi_head(case)
    c = _case(case)
    inp = c["inp"]
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    y, fin = ops.ssd_forward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], y_dtype=y_dtype, mma="bf16")
    torch.cuda.synchronize()
    ey = relerr(_pair_major(y), c["yo"])
    ef = relerr(fin.reshape(-1, fin.shape[2], fin.shape[3]), c["fo"])
    say(f"  rel err y {ey:.3g} final {ef:.3g}")
    assert ey <= tol_for("bf16") and ef <= tol_for("bf16")


@pytest.mark.parametrize("dtypes", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16")],
                         ids=["states_f32-carried_f32", "states_bf16-carried_bf16", "states_f32-carried_bf16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_headgroup_split_calls(case, dtypes):
    """The four split calls (chunk states without the fused cumsum, state
    passing, chunk scan with fp32 or bf16 carried states), all pairs of the
    chunk states, y and the final states against the oracle."""
    states_dtype, carried_dtype = dtypes
    say(f"head-group split calls {case} states={states_dtype} carried={carried_dtype}")
    _assert_multi_head(case)
    c = _case(case)
    inp = c["inp"]
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    S = ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, mma="bf16", states_dtype=states_dtype)
    torch.cuda.synchronize()
    es = relerr(S.float(), c["S"])
    carried, fin = ops.ssd_state_passing(sh, S, dA, carried_dtype=carried_dtype)
    y = ops.ssd_chunk_scan(sh, t["x"], t["Bm"], t["Cm"], dtb, dA, carried, t["D"], y_dtype="f32", mma="bf16")
    torch.cuda.synchronize()
    ey = relerr(_pair_major(y), c["yo"])
    ef = relerr(fin.reshape(-1, fin.shape[2], fin.shape[3]), c["fo"])
    say(f"  rel err chunk states {es:.3g} y {ey:.3g} final {ef:.3g}")
    assert es <= tol_for("bf16") and ey <= tol_for("bf16") and ef <= tol_for("bf16")


PACKED_HG = [
    # (name, B, H, P, N, G, Q, sequence lengths per row)
    ("q256_n128", 2, 32, 64, 128, 1, 256, [[1000, 3, 600, 1, 2492], [4096]]),
    ("q128_n256", 2, 16, 64, 256, 2, 128, [[129, 127, 1792], [7, 2041]]),
]


@pytest.mark.parametrize("case", PACKED_HG, ids=[c[0] for c in PACKED_HG])
def test_headgroup_packed_sequences(case):
    """Packed rows through the head-group chunk scan's packed-sequence
    instance with several heads per block: every sequence against its own
    oracle run from a zero state."""
    name, B, H, P, N, G, Q, rows = case
    L = sum(rows[0])
    say(f"head-group packed sequences {name}")
    cus = device_cus()
    hg = heads_per_block(B, L, H, P, N, G, Q, cus)
    say(f"  chunk_scan heads per block {hg}")
    assert hg >= 2
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype="bf16", seed=43, dt_shift=1.0)
    t = upload(inp)
    sh = ops.shape_of(t, Q)
    idx = np.zeros((B, L), dtype=np.int32)
    for b, lens in enumerate(rows):
        assert sum(lens) == L
        idx[b] = np.repeat(np.arange(len(lens), dtype=np.int32), lens)
    y, fin = ops.ssd_forward_varlen(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"],
                                    torch.from_numpy(idx).cuda(), y_dtype="f32", mma="bf16")
    torch.cuda.synchronize()
    o = oracle()
    worst = 0.0
    for b, lens in enumerate(rows):
        s0 = 0
        for n in lens:
            sl = lambda a: np.ascontiguousarray(a[b:b + 1, s0:s0 + n])
            yref, fref = o.forward(sl(inp.x), sl(inp.dt), inp.A, sl(inp.Bm), sl(inp.Cm), inp.D)
            worst = max(worst, relerr(y[b:b + 1, s0:s0 + n], yref))
            s0 += n
        worst = max(worst, relerr(fin[b:b + 1], fref))
    say(f"  worst rel err over sequences {worst:.3g}")
    assert worst <= tol_for("bf16")


# (name, B, L, H, P, N, G, Q): head counts with odd and even divisors
HG_SWEEP = [
    ("q256_h30", 1, 1024, 30, 64, 128, 1, 256),
    ("ragged_q128_h15", 2, 600, 15, 64, 128, 1, 128),
]


@pytest.mark.parametrize("case", HG_SWEEP, ids=[c[0] for c in HG_SWEEP])
def test_chunk_state_heads_per_block_sweep(case, monkeypatch):
    """Every head count per block that divides the group's heads, forced
    through SSD_TUNE: the chunk-state kernel's head loop runs its heads in
    unrolled pairs plus, for an odd count, one last single step.  Each head's
    state is computed on its own, so every split must give the same bits: the
    chunk states (fp32 and bf16 storage) and the backward with bf16 and with
    fp32 matrix operands, whose adjoint and recomputed chunk states take the
    same override.  The first
    split's chunk states are also checked against the oracle."""
    name, B, L, H, P, N, G, Q = case
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype="bf16", seed=43, dt_shift=1.0)
    t = upload(inp)
    sh = ops.shape_of(t, Q)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    S_ref = oracle().chunk_states_ref(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, Q)
    gen = torch.Generator(device="cuda").manual_seed(5)
    dy = torch.randn(tuple(t["x"].shape), device="cuda", generator=gen).to(t["x"].dtype)
    base = None
    for k in [d for d in range(1, H // G + 1) if (H // G) % d == 0]:
        monkeypatch.setenv("SSD_TUNE", f"state_hg={k}")
        say(f"chunk-state heads per block {name}: {k}")
        states = [ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, mma="bf16", states_dtype=sd) for sd in ("f32", "bf16")]
        grads = [ops.ssd_backward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], dy, mma=m)
                 for m in ("bf16", "f32")]
        torch.cuda.synchronize()
        cur = [s.cpu() for s in states] + [gr[n].cpu() for gr in grads for n in sorted(gr) if gr[n] is not None]
        if base is None:
            base = cur
            es = relerr(states[0], S_ref)
            say(f"  rel err chunk states {es:.3g}")
            assert es <= tol_for("bf16")
        else:
            assert len(cur) == len(base)
            for i, (a, b) in enumerate(zip(base, cur)):
                assert torch.equal(a, b), (k, i)


@pytest.mark.parametrize("case", HG_SWEEP, ids=[c[0] for c in HG_SWEEP])
def test_chunk_scan_heads_per_block_sweep(case, monkeypatch):
    """Every head count per block of the head-group chunk scan, forced through
    SSD_TUNE: a block computes the chunk's C.B^T once and walks its heads with
    the next head's rows prefetched and the per-head tiles double-buffered, and
    each head's y is computed on its own, so every split must give the same
    bits: y and the final states of the forward (bf16 and fp32 matrix
    operands) and the bf16-operand gradients, whose two chunk scans take the
    same override.  The first split's y is also checked against the oracle."""
    name, B, L, H, P, N, G, Q = case
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype="bf16", seed=47, dt_shift=1.0)
    t = upload(inp)
    sh = ops.shape_of(t, Q)
    yo, _, _ = oracle().recurrence(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D, chunk=Q)
    gen = torch.Generator(device="cuda").manual_seed(6)
    dy = torch.randn(tuple(t["x"].shape), device="cuda", generator=gen).to(t["x"].dtype)
    base = None
    for k in [d for d in range(1, H // G + 1) if (H // G) % d == 0]:
        monkeypatch.setenv("SSD_TUNE", f"scan_hg={k}")
        say(f"chunk-scan heads per block {name}: {k}")
        fwd = [ops.ssd_forward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], mma=m, y_dtype=yd)
               for m, yd in (("bf16", "bf16"), ("f32", "f32"))]
        grads = ops.ssd_backward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], dy, mma="bf16")
        torch.cuda.synchronize()
        cur = [v.cpu() for y, fin in fwd for v in (y, fin)] + [grads[n].cpu() for n in sorted(grads) if grads[n] is not None]
        if base is None:
            base = cur
            ey = relerr(_pair_major(fwd[1][0]), yo)
            say(f"  rel err y (fp32 operands) {ey:.3g}")
            assert ey <= tol_for("f32")
        else:
            assert len(cur) == len(base)
            for i, (a, b) in enumerate(zip(base, cur)):
                assert torch.equal(a, b), (k, i)


# sequence lengths per row of the packed sweep, for the two HG_SWEEP shapes
PACKED_SWEEP_ROWS = {"q256_h30": [[300, 1, 467, 256]], "ragged_q128_h15": [[100, 250, 250], [600]]}


@pytest.mark.parametrize("case", HG_SWEEP, ids=[c[0] for c in HG_SWEEP])
def test_packed_heads_per_block_sweep(case, monkeypatch):
    """Packed rows (sequences starting inside chunks, a one-token sequence)
    through the packed-sequence instances of the chunk-state and chunk-scan
    kernels at every head count per block, forced through SSD_TUNE for both:
    y and the final states must be the same bits at every split, with bf16
    and with fp32 matrix operands."""
    name, B, L, H, P, N, G, Q = case
    rows = PACKED_SWEEP_ROWS[name]
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype="bf16", seed=53, dt_shift=1.0)
    t = upload(inp)
    sh = ops.shape_of(t, Q)
    idx = np.zeros((B, L), dtype=np.int32)
    for b, lens in enumerate(rows):
        assert sum(lens) == L
        idx[b] = np.repeat(np.arange(len(lens), dtype=np.int32), lens)
    seq = torch.from_numpy(idx).cuda()
    base = None
    for k in [d for d in range(1, H // G + 1) if (H // G) % d == 0]:
        monkeypatch.setenv("SSD_TUNE", f"scan_hg={k},state_hg={k}")
        say(f"packed heads per block {name}: {k}")
        outs = [ops.ssd_forward_varlen(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], seq, y_dtype="f32", mma=m)
                for m in ("bf16", "f32")]
        torch.cuda.synchronize()
        cur = [v.cpu() for y, fin in outs for v in (y, fin)]
        if base is None:
            base = cur
        else:
            for i, (a, b) in enumerate(zip(base, cur)):
                assert torch.equal(a, b), (k, i)
