"""Guard bands around every output and workspace (device-side bounds check).

Each output tensor is a view into a larger allocation whose bytes before and
after it are filled with a sentinel pattern; after the calls (ragged last
chunk, packed sequences, decode step, gradients) the padding must still hold
the sentinel, byte for byte: no kernel writes outside its outputs.  The
workspaces get the same treatment.  The outputs themselves are also checked
against the fp64 oracle, so the views are known to have been written.
"""
import numpy as np
import pytest
import torch

from gpu_common import make_inputs, oracle, relerr, say, tol_for, upload
from mamba_ssd_scan_chunk_amd import ops

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A  # byte pattern of the guard bands
PAD = 4096        # guard bytes on each side (keeps every view 256-byte aligned)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Guarded:
    """Device tensors carved out of sentinel-filled byte buffers."""

    def __init__(self):
        self.items = []

    def tensor(self, name, shape, dtype):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        buf = torch.full((PAD + n + PAD,), SENTINEL, dtype=torch.uint8, device="cuda")
        view = buf[PAD:PAD + n].view(dtype).view(shape)
        self.items.append((name, buf, n))
        return view

    def workspace(self, name, nbytes):
        buf = torch.full((PAD + nbytes + PAD,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.items.append((name, buf, nbytes))
        return buf[PAD:PAD + nbytes]

    def check(self):
        torch.cuda.synchronize()
        for name, buf, n in self.items:
            head = buf[:PAD].cpu().numpy()
            tail = buf[PAD + n:].cpu().numpy()
            assert (head == SENTINEL).all(), f"{name}: {int((head != SENTINEL).sum())} guard bytes before it written"
            assert (tail == SENTINEL).all(), f"{name}: {int((tail != SENTINEL).sum())} guard bytes after it written"


# (name, B, L, H, P, N, G, Q): ragged last chunks for every kernel family
RAGGED = [
    ("hg_q256_n128", 2, 300, 4, 64, 128, 1, 256),
    ("hg_q128_n256", 1, 130, 4, 64, 256, 2, 128),
    ("hg_q256_n64", 2, 600, 4, 64, 64, 2, 256),
    ("generic_q64", 1, 200, 3, 48, 48, 3, 64),
    ("generic_q32", 1, 77, 20, 32, 32, 4, 32),
]


@pytest.mark.parametrize("mma", ["bf16", "f32"])
@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_guard_forward_and_split_calls(case, mma):
    name, B, L, H, P, N, G, Q = case
    say(f"guard bands: forward + split calls {name} mma={mma}")
    in_dtype = "bf16" if mma == "bf16" else "f32"
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype=in_dtype, seed=3, dt_shift=1.0)
    t = upload(inp)
    sh = ops.shape_of(t, Q)
    nc = -(-L // Q)
    g = Guarded()
    io = t["x"].dtype
    y = g.tensor("y", (B, L, H, P), io)
    fin = g.tensor("final_states", (B, H, N, P), torch.float32)
    ws = g.workspace("workspace", ops.ssd_workspace_bytes(sh))
    ops.ssd_forward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], y=y, final_states=fin, workspace=ws,
                    mma=mma)
    # the split calls, each into guarded outputs (bf16 states and carried states too)
    dA = g.tensor("dA_cumsum", (B, H, nc, Q), torch.float32)
    dtb = g.tensor("dt_bhl", (B, H, nc, Q), torch.float32)
    ops.ssd_chunk_cumsum(sh, t["dt"], t["A"], dA_cumsum=dA, dt_bhl=dtb)
    sdt = torch.bfloat16 if mma == "bf16" else torch.float32
    S = g.tensor("chunk_states", (B, nc, H, N, P), sdt)
    ops.ssd_chunk_state(sh, t["x"], t["Bm"], dtb, dA, states=S, mma=mma)
    carried = g.tensor("carried", (B, nc, H, N, P), sdt)
    fin2 = g.tensor("final_states (split)", (B, H, N, P), torch.float32)
    ops.ssd_state_passing(sh, S, dA, carried=carried, final_states=fin2)
    y2 = g.tensor("y (split)", (B, L, H, P), torch.float32)
    ops.ssd_chunk_scan(sh, t["x"], t["Bm"], t["Cm"], dtb, dA, carried, t["D"], y=y2, mma=mma)
    g.check()
    yo, fo = oracle().forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
    assert relerr(y2, yo) <= tol_for(mma) and relerr(fin2, fo) <= tol_for(mma)
    assert relerr(y, yo) <= tol_for(mma) and relerr(fin, fo) <= tol_for(mma)


def test_guard_fused_state_path():
    B, L, H, P, N, G, Q = 2, 300, 4, 64, 128, 1, 128
    say(f"guard bands: fused state path {(B, L, H, P, N, G, Q)}")
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype="bf16", seed=4, dt_shift=1.0)
    t = upload(inp)
    sh = ops.shape_of(t, Q)
    nc = -(-L // Q)
    dA, dtb = ops.ssd_chunk_cumsum(sh, t["dt"], t["A"])
    g = Guarded()
    carried = g.tensor("carried", (B, nc, H, N, P), torch.bfloat16)
    fin = g.tensor("final_states", (B, H, N, P), torch.float32)
    ops.ssd_chunk_state_passing(sh, t["x"], t["Bm"], dtb, dA, carried=carried, final_states=fin)
    g.check()
    _, fo = oracle().forward(inp.x, inp.dt, inp.A, inp.Bm, inp.Cm, inp.D)
    assert relerr(fin, fo) <= tol_for("bf16")


@pytest.mark.parametrize("mma", ["bf16", "f32"])
def test_guard_packed_sequences(mma):
    B, H, P, N, G, Q = 2, 4, 64, 128, 1, 256
    rows = [[100, 1, 155, 44], [300]]
    L = sum(rows[0])
    say(f"guard bands: packed sequences mma={mma}")
    in_dtype = "bf16" if mma == "bf16" else "f32"
    inp = make_inputs(B, L, H, P, N, G, Q, in_dtype=in_dtype, seed=5, dt_shift=1.0)
    t = upload(inp)
    sh = ops.shape_of(t, Q)
    idx = np.zeros((B, L), dtype=np.int32)
    for b, lens in enumerate(rows):
        idx[b] = np.repeat(np.arange(len(lens), dtype=np.int32), lens)
    last = torch.tensor([99, 100, 255, 299, L + 299], dtype=torch.int64, device="cuda")
    g = Guarded()
    y = g.tensor("y", (B, L, H, P), torch.float32)
    fin = g.tensor("final_states", (B, H, N, P), torch.float32)
    sst = g.tensor("seq_states", (5, H, N, P), torch.float32)
    ws = g.workspace("workspace", int(ops.load_library().ssd_workspace_bytes_varlen(sh)))
    ops.ssd_forward_varlen(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], torch.from_numpy(idx).cuda(),
                           y=y, final_states=fin, seq_last=last, seq_states=sst, workspace=ws, mma=mma)
    g.check()
    # the last sequence of row 1 is the whole row
    yo, fo = oracle().forward(inp.x[1:], inp.dt[1:], inp.A, inp.Bm[1:], inp.Cm[1:], inp.D)
    assert relerr(y[1:], yo) <= tol_for(mma) and relerr(fin[1:], fo) <= tol_for(mma)
    assert relerr(sst[4:], fo) <= tol_for(mma)


def test_guard_decode_step():
    Bn, H, P, N, G = 5, 6, 64, 128, 2
    say("guard bands: decode step")
    rng = np.random.default_rng(6)
    x = rng.standard_normal((Bn, H, P)).astype(np.float32)
    dt = (0.1 + rng.random((Bn, H))).astype(np.float32)
    A = -np.exp(rng.random(H)).astype(np.float32)
    Bm = rng.standard_normal((Bn, G, N)).astype(np.float32)
    Cm = rng.standard_normal((Bn, G, N)).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    s0 = rng.standard_normal((Bn, H, N, P)).astype(np.float32)
    g = Guarded()
    st = g.tensor("state", (Bn, H, N, P), torch.float32)
    st.copy_(torch.from_numpy(s0))
    y = g.tensor("y", (Bn, H, P), torch.float32)
    cu = lambda a: torch.from_numpy(a).cuda()
    ops.ssd_decode_step(cu(x), cu(dt), cu(A), cu(Bm), cu(Cm), cu(D), st, y=y)
    g.check()
    yo, so = oracle().decode_step(x, dt, A, Bm, Cm, D, s0.astype(np.float64))
    assert relerr(y, yo) <= 1e-5 and relerr(st, so) <= 1e-5


@pytest.mark.parametrize("mma", ["bf16", "f32"])
def test_guard_backward(mma):
    B, L, H, P, N, G, Q = 1, 200, 4, 64, 64, 2, 64
    say(f"guard bands: backward mma={mma}")
    inp = make_inputs(B, L, H, P, N, G, Q, seed=7, dt_shift=1.0)
    t = upload(inp)
    sh = ops.shape_of(t, Q)
    dy = torch.randn((B, L, H, P), device="cuda", generator=torch.Generator(device="cuda").manual_seed(8))
    g = Guarded()
    shapes = {"dx": (B, L, H, P), "ddt": (B, L, H), "dA": (H,), "dB": (B, L, G, N), "dC": (B, L, G, N),
              "dD": (H,), "dinitial": (B, H, N, P)}
    out = {k: g.tensor(k, s, torch.float32) for k, s in shapes.items()}
    ws = g.workspace("workspace", ops.ssd_backward_workspace_bytes(sh))
    r = ops.ssd_backward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], dy, workspace=ws, mma=mma, out=out)
    g.check()
    assert all(r[k] is out[k] for k in shapes)
    assert all(torch.isfinite(out[k]).all() for k in shapes)
