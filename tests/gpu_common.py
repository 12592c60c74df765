"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding, run the fp64 oracle on the same seeded inputs, compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

from mamba_ssd_scan_chunk_amd import ops
from mamba_ssd_scan_chunk_amd.inputs import make_inputs  # noqa: F401  (re-exported for tests)
from oracle import oracle as oracle_mod

# Acceptance bars: max|gpu - ref| / max|ref| over the compared tensor.
TOL_F32_MMA = 1e-4
TOL_BF16_MMA = 1e-2
TOL_CUMSUM = 1e-6
TOL_PASSING = 1e-5


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def relerr(gpu, ref) -> float:
    g = gpu.detach().double().cpu().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.isfinite(g).all(), "non-finite GPU output"
    den = np.abs(r).max()
    return float(np.abs(g - r).max() / (den if den > 0 else 1.0))


def tol_for(mma: str) -> float:
    return TOL_F32_MMA if mma == "f32" else TOL_BF16_MMA


def upload(inp):
    t = inp.to_torch("cuda")
    return t


def pairs_sample(B, H, k, seed=0):
    """A seeded sample of (b, h) pair indices b*H+h, always including the first
    and the last pair."""
    total = B * H
    rng = np.random.default_rng(seed)
    extra = rng.choice(total, size=min(k, total), replace=False).tolist()
    return sorted(set([0, total - 1] + extra))


def oracle():
    return oracle_mod.get()


def gpu_forward(inp, mma, y_dtype=None, h0=None, want_final=True):
    t = upload(inp)
    sh = ops.shape_of(t, inp.chunk)
    h0_t = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0, dtype=np.float32)).cuda()
    y, fin = ops.ssd_forward(sh, t["x"], t["dt"], t["A"], t["Bm"], t["Cm"], t["D"], initial_states=h0_t,
                             y_dtype=y_dtype, want_final=want_final, mma=mma)
    torch.cuda.synchronize()
    return y, fin


def device_cus() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def heads_per_block(B, L, H, P, N, G, Q, cus, cap=None):
    """Heads per block the head-group kernels' launchers choose: the largest
    divisor HG of the group's head count H/G (at most `cap`) such that the grid
    (B * nc * G * P/64 blocks per head run) still gives every compute unit one
    block."""
    nc = -(-L // Q)
    hpg = H // G
    base = B * nc * G * (P // 64)
    best = 1
    for k in range(1, hpg + 1):
        if hpg % k or (cap is not None and hpg // k > cap):
            continue
        best = hpg // k
        if base * k >= cus:
            break
    return best


def chunk_state_hg_fused_cap(Q, N):
    """Most heads one block of the chunk-state kernel with the cumulative sum
    fused in can take: its LDS holds the B and x tiles plus 8*Q bytes (sums
    and dt) per head, within 160 KiB."""
    lds = Q * (N + 16) * 2 + Q * (64 + 16) * 2
    return (160 * 1024 - lds) // (8 * Q)
