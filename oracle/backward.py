"""fp64 CPU oracle for the gradients of the Mamba-2 SSD forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  It shares no code
with the HIP library and imports nothing from it.

Page cited (by title): P1 = "Jane Street ML Engineers Map Mamba-2 Recurrent
State Computation to Tensor Cores with cuTile" (disconfirmai.com).  P1 says
the backward pass exists but does not publish it (its closing paragraphs);
what is computed here is the reverse-mode derivative of the same token
recurrence the forward oracle runs (P1 opening and jump-formula paragraphs):

    h_t = r_t h_{t-1} + dt_t B_t x_t^T,   r_t = exp(dt_t A),   y_t = C_t^T h_t + D x_t

For a scalar loss with dL/dy_t = dy_t and dL/dh_{L-1} = dfinal, the adjoint
state g_t = dL/dh_t runs backwards over the tokens,

    g_t = C_t dy_t^T + r_{t+1} g_{t+1}          (g_{L-1} = C_{L-1} dy_{L-1}^T + dfinal)

and each input's derivative is read off the step that uses it:

    dx_t   = D dy_t + dt_t g_t^T B_t
    dB_t   = dt_t g_t x_t            (summed over the heads of the group)
    dC_t   = h_t dy_t                (summed over the heads of the group)
    ddt_t  = A r_t <g_t, h_{t-1}> + B_t^T g_t x_t
    dA     = sum_t dt_t r_t <g_t, h_{t-1}>
    dD     = sum_t dy_t . x_t
    dh0    = r_0 g_0

Plain per-token loops in fp64 (numpy for the N x P state arithmetic), meant
for the small sizes of the tests.  Pinned in ``tests/pins.py`` by central
finite differences of the brute-force semiseparable forward.
"""
from __future__ import annotations

import numpy as np


def backward(x, dt, A, Bm, Cm, D, dy, h0=None, dfinal=None, terms=False):
    """Gradients of L = sum(dy * y) + sum(dfinal * final) w.r.t. every input.

    Shapes: x [B,L,H,P], dt [B,L,H], A [H], Bm/Cm [B,L,G,N], D [H], dy like x,
    h0 and dfinal [B,H,N,P] or None.  Returns a dict of fp64 arrays dx, ddt,
    dA, dB, dC, dD, dh0 with the inputs' shapes.  With ``terms``, also the
    per-token pieces of ddt and dA, both [B,L,H]: "dlogr" = dL/d(dt_t A) =
    r_t <g_t, h_{t-1}> and "beta" = B_t^T g_t x_t (ddt = A dlogr + beta,
    dA = sum dt dlogr); tests use their magnitudes to scale error bars."""
    x, dt, A, Bm, Cm, D, dy = (np.asarray(a, dtype=np.float64) for a in (x, dt, A, Bm, Cm, D, dy))
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    out = {"dx": np.zeros_like(x), "ddt": np.zeros_like(dt), "dA": np.zeros(H), "dB": np.zeros_like(Bm),
           "dC": np.zeros_like(Cm), "dD": np.zeros(H), "dh0": np.zeros((Bsz, H, N, P))}
    dlogr, beta = np.zeros_like(dt), np.zeros_like(dt)
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            # forward states h_{-1} .. h_{L-1}
            hs = np.zeros((L + 1, N, P))
            if h0 is not None:
                hs[0] = np.asarray(h0, dtype=np.float64)[b, h]
            r = np.exp(dt[b, :, h] * A[h])
            for t in range(L):
                hs[t + 1] = r[t] * hs[t] + dt[b, t, h] * np.outer(Bm[b, t, g], x[b, t, h])
            gst = np.zeros((N, P)) if dfinal is None else np.asarray(dfinal, dtype=np.float64)[b, h].copy()
            for t in range(L - 1, -1, -1):
                gst += np.outer(Cm[b, t, g], dy[b, t, h])
                ht, hprev = hs[t + 1], hs[t]
                out["dC"][b, t, g] += ht @ dy[b, t, h]
                out["dx"][b, t, h] = D[h] * dy[b, t, h] + dt[b, t, h] * (Bm[b, t, g] @ gst)
                gx = gst @ x[b, t, h]
                out["dB"][b, t, g] += dt[b, t, h] * gx
                gh = float(np.sum(gst * hprev))
                dlogr[b, t, h], beta[b, t, h] = r[t] * gh, float(Bm[b, t, g] @ gx)
                out["ddt"][b, t, h] = A[h] * r[t] * gh + float(Bm[b, t, g] @ gx)
                out["dA"][h] += dt[b, t, h] * r[t] * gh
                out["dD"][h] += float(dy[b, t, h] @ x[b, t, h])
                gst = r[t] * gst
            out["dh0"][b, h] = gst
    if terms:
        out["dlogr"], out["beta"] = dlogr, beta
    return out
