"""The bench line's algorithmic model (CPU): the bytes and flops per launch that
`roofline.achieved` divides by a measured duration, checked against tensor
inventories written out here from each kernel's inputs and outputs, and the
causal flop counts against a brute-force count of the (i, j <= i) pairs."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mamba_ssd_scan_chunk_amd.inputs import WORKLOADS  # noqa: E402


def nbytes(shape, itemsize):
    return int(np.prod(shape, dtype=np.int64)) * itemsize


def causal_pairs(Q):
    return sum(1 for i in range(Q) for j in range(Q) if j <= i)


def inventory(w, in_b, y_b, car_b, st_b):
    B, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    nc = L // Q
    x, bm, cm = (B, L, H, P), (B, L, G, N), (B, L, G, N)
    bhcq, states, fin = (B, H, nc, Q), (B, nc, H, N, P), (B, H, N, P)
    return {
        # reads dt [B,L,H] and A [H]; writes dA_cumsum and dt_bhl
        "chunk_cumsum": nbytes((B, L, H), 4) + nbytes((H,), 4) + 2 * nbytes(bhcq, 4),
        # reads x, B, dA_cumsum, dt_bhl; writes the chunk states
        "chunk_state": nbytes(x, in_b) + nbytes(bm, in_b) + 2 * nbytes(bhcq, 4) + nbytes(states, st_b),
        # the forward's fused first step: dt and A in, dA_cumsum and dt_bhl out
        "chunk_cumsum_state": nbytes(x, in_b) + nbytes(bm, in_b) + nbytes((B, L, H), 4) + nbytes((H,), 4)
        + 2 * nbytes(bhcq, 4) + nbytes(states, st_b),
        # reads the chunk states and one decay per (b, h, c); writes the carried
        # states and the final states
        "state_passing": nbytes(states, st_b) + nbytes((B, H, nc), 4) + nbytes(states, car_b) + nbytes(fin, 4),
        # reads x, B, C, dA_cumsum, dt_bhl, the carried states and D; writes y
        "chunk_scan": nbytes(x, in_b) + nbytes(bm, in_b) + nbytes(cm, in_b) + 2 * nbytes(bhcq, 4)
        + nbytes(states, car_b) + nbytes((H,), 4) + nbytes(x, y_b),
    }


@pytest.mark.parametrize("name", sorted(WORKLOADS))
@pytest.mark.parametrize("bf16_states", [True, False])
def test_algorithmic_bytes_match_the_tensor_inventory(name, bf16_states):
    w = WORKLOADS[name]
    in_b = 2 if w.in_dtype == "bf16" else 4
    s_b = 2 if bf16_states else 4
    model = bench.algorithmic_costs(w, in_b, in_b, s_b, s_b)
    inv = inventory(w, in_b, in_b, s_b, s_b)
    for k, v in inv.items():
        assert model[k]["bytes"] == v, (k, model[k]["bytes"], v)


def test_headline_chunk_scan_bytes_and_flops():
    """The 2.7B-layer chunk scan with bf16 carried states moves 438.3 MB; its
    flops are C.B^T once per group over the causal pairs, M.X per head over the
    causal pairs, and C.H_in per token."""
    w = WORKLOADS["mamba2_2p7b_layer"]
    model = bench.algorithmic_costs(w, 2, 2, 2, 2)["chunk_scan"]
    assert abs(model["bytes"] / 1e6 - 438.3) < 0.05
    B, L, H, P, N, G, Q = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    nc = L // Q
    pairs = causal_pairs(Q)
    flops = 2 * B * nc * G * pairs * N + 2 * B * nc * H * pairs * P + 2 * B * L * H * N * P
    assert model["flops"] == flops


def test_chunk_state_flops_are_one_product_per_token():
    w = WORKLOADS["mamba2_2p7b_layer"]
    model = bench.algorithmic_costs(w, 2, 2, 2, 2)
    assert model["chunk_state"]["flops"] == 2 * w.batch * w.seqlen * w.nheads * w.dstate * w.headdim
    assert model["chunk_cumsum_state"]["flops"] == model["chunk_state"]["flops"] + 2 * w.batch * w.seqlen * w.nheads
