"""Independent fp64 NumPy forms of the SSD forward, used to pin the oracle.

TEST INFRASTRUCTURE ONLY (imported by ``tests/`` alone).  None of these
functions shares code with ``ssd_oracle.c`` or with the HIP library; each is a
different way of writing the same mathematics, so that a mistake in any one of
them (a dropped term, a wrong sign, an off-by-one in the decay, a transposed
operand) shows up as a disagreement.

Page cited (by title):
  P1 = "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
        Tensor Cores with cuTile" (disconfirmai.com).

All forms take float32/float64 arrays in the library's layouts
(x [B,L,H,P], dt [B,L,H], A [H], Bm/Cm [B,L,G,N], D [H], h0 [B,H,N,P]) and
compute in float64.  Group of head h: g = h // (H // G).
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def semiseparable_forward(x, dt, A, Bm, Cm, D=None, h0=None):
    """Brute force: materialise the L x L lower-triangular (semiseparable)
    matrix per (batch, head) and multiply.

        M[t, s] = (C_t . B_s) * prod_{k=s+1..t} exp(dt_k A) * dt_s     (s <= t)
        y = M x + D x + C_t^T (prod_{k=0..t} exp(dt_k A)) h0

    The decay is a direct running product of per-token factors, not a
    cumulative sum of logarithms, so it is independent of the log-space route
    (P1, jump-formula paragraph) that the kernels take.
    Returns y [B,L,H,P], final [B,H,N,P].
    """
    x, dt, A, Bm, Cm, D, h0 = map(_f64, (x, dt, A, Bm, Cm, D, h0))
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    y = np.zeros((Bsz, L, H, P))
    fin = np.zeros((Bsz, H, N, P))
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            r = np.exp(dt[b, :, h] * A[h])
            decay = np.zeros((L, L))
            for t in range(L):
                decay[t, t] = 1.0
                for s in range(t - 1, -1, -1):
                    decay[t, s] = decay[t, s + 1] * r[s + 1]
            cb = Cm[b, :, g, :] @ Bm[b, :, g, :].T          # [L, L]  C_t . B_s
            M = cb * decay * dt[b, None, :, h]
            xs = x[b, :, h, :]
            y[b, :, h, :] = M @ xs
            if D is not None:
                y[b, :, h, :] += D[h] * xs
            # final state: sum_s decay[L-1, s] dt_s B_s x_s^T
            w = decay[L - 1, :] * dt[b, :, h]
            fin[b, h] = (Bm[b, :, g, :] * w[:, None]).T @ xs
            if h0 is not None:
                pref = np.cumprod(r)                         # prod_{k<=t} r_k
                y[b, :, h, :] += pref[:, None] * (Cm[b, :, g, :] @ h0[b, h])
                fin[b, h] += pref[-1] * h0[b, h]
    return y, fin


def zero_decay_closed_form(x, dt, Bm, Cm, D=None):
    """A = 0: the state is the running sum of outer products (P1, jump formula
    h(t+T) = h(t) + B X^T with dt folded into B).

        final = (B diag(dt))^T X          -- one matrix product
        y_t   = C_t^T (sum_{s<=t} dt_s B_s x_s^T) + D x_t
    Returns y [B,L,H,P], final [B,H,N,P].
    """
    x, dt, Bm, Cm, D = map(_f64, (x, dt, Bm, Cm, D))
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    y = np.zeros((Bsz, L, H, P))
    fin = np.zeros((Bsz, H, N, P))
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            Bt = Bm[b, :, g, :] * dt[b, :, h][:, None]       # [L, N]
            xs = x[b, :, h, :]                               # [L, P]
            fin[b, h] = np.matmul(Bt.T, xs)
            outer = Bt[:, :, None] * xs[:, None, :]          # [L, N, P]
            states = np.cumsum(outer, axis=0)
            y[b, :, h, :] = np.einsum("tn,tnp->tp", Cm[b, :, g, :], states)
            if D is not None:
                y[b, :, h, :] += D[h] * xs
    return y, fin


def geometric_series(L, dt, A, b, c, xv, D):
    """Scalar case N = P = H = G = 1 with constant inputs:
        h_t = dt b x (1 - r^{t+1}) / (1 - r),  r = exp(dt A)   (A != 0)
        y_t = c h_t + D x
    Returns (y [L], h_final)."""
    r = np.exp(np.float64(dt) * np.float64(A))
    t = np.arange(L, dtype=np.float64)
    h = np.float64(dt) * b * xv * (1.0 - r ** (t + 1)) / (1.0 - r)
    return c * h + D * xv, h[-1]


def chunked_forward(x, dt, A, Bm, Cm, D=None, h0=None, Q=64):
    """The chunked algorithm in fp64, step by step as P1 lays it out (paragraph
    on the three kernels, compute_out paragraph):

    1. chunk cumsum: G_i = sum_{k<=i} dt_k A within the chunk (inclusive);
    2. chunk state (jump formula with rows pre-multiplied by exponentials):
       S_c = sum_j exp(G_last - G_j) dt_j B_j x_j^T;
    3. state passing: H_in[0] = h0, H_in[c+1] = exp(G_last) H_in[c] + S_c;
    4. output: y_i = exp(G_i) C_i^T H_in[c]
                    + sum_{j<=i} (C_i . B_j) exp(G_i - G_j) dt_j x_j + D x_i,
       with the causal condition applied to the exponent before exp.

    A ragged last chunk (L % Q != 0) uses its own last token as G_last.
    Returns dict with y [B,L,H,P], final [B,H,N,P], G [B,H,nc,Q] (zero past a
    ragged end), S and Hin [B,nc,H,N,P].
    """
    x, dt, A, Bm, Cm, D, h0 = map(_f64, (x, dt, A, Bm, Cm, D, h0))
    Bsz, L, H, P = x.shape
    G_, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G_
    nc = (L + Q - 1) // Q
    y = np.zeros((Bsz, L, H, P))
    Gc = np.zeros((Bsz, H, nc, Q))
    S = np.zeros((Bsz, nc, H, N, P))
    Hin = np.zeros((Bsz, nc, H, N, P))
    fin = np.zeros((Bsz, H, N, P))
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            run = h0[b, h].copy() if h0 is not None else np.zeros((N, P))
            for c in range(nc):
                t0, t1 = c * Q, min(L, (c + 1) * Q)
                q = t1 - t0
                a = dt[b, t0:t1, h] * A[h]
                Gi = np.cumsum(a)
                Gc[b, h, c, :q] = Gi
                dtc = dt[b, t0:t1, h]
                Bc, Cc, Xc = Bm[b, t0:t1, g, :], Cm[b, t0:t1, g, :], x[b, t0:t1, h, :]
                # step 2
                w = np.exp(Gi[-1] - Gi) * dtc
                S[b, c, h] = (Bc * w[:, None]).T @ Xc
                # step 4 (uses the carried state before this chunk)
                Hin[b, c, h] = run
                diff = Gi[:, None] - Gi[None, :]
                causal = np.arange(q)[:, None] >= np.arange(q)[None, :]
                decay = np.exp(np.where(causal, diff, -np.inf))
                Mloc = (Cc @ Bc.T) * decay * dtc[None, :]
                yc = np.exp(Gi)[:, None] * (Cc @ run) + Mloc @ Xc
                if D is not None:
                    yc += D[h] * Xc
                y[b, t0:t1, h, :] = yc
                # step 3
                run = np.exp(Gi[-1]) * run + S[b, c, h]
            fin[b, h] = run
    return {"y": y, "final": fin, "G": Gc, "S": S, "Hin": Hin}
