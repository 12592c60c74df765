"""The seeded input generator (CPU only)."""
import numpy as np
import torch

from mamba_ssd_scan_chunk_amd.inputs import WORKLOADS, bf16_round, bf16_widen, make_inputs


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    # add exact ties: values halfway between two bf16 numbers
    ties = (bf16_widen(bf16_round(v[:1000])).view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties, np.float32([0.0, -0.0, 1e-30, 65504.0])])
    ours = bf16_round(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_recipe_is_deterministic_and_in_range():
    a = make_inputs(2, 64, 3, 8, 4, 1, 16, seed=5, in_dtype="bf16")
    b = make_inputs(2, 64, 3, 8, 4, 1, 16, seed=5, in_dtype="bf16")
    for k in ("x", "dt", "A", "Bm", "Cm", "D"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert (a.dt > 0).all()
    assert (a.A <= -1.0).all() and (a.A > -16.0).all()
    assert np.array_equal(bf16_widen(a.x_bits), a.x)


def test_workloads_table():
    assert len(WORKLOADS) == 5
    for w in WORKLOADS.values():
        assert w.nheads % w.ngroups == 0
        assert w.seqlen % w.chunk == 0
