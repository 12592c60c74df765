"""fp64 CPU oracle for the Mamba-2 chunked-SSD forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this module.  It shares no code with
the HIP library (``mamba_ssd_scan_chunk_amd``) and imports nothing from it.

Page cited (by title):
  P1 = "Jane Street ML Engineers Map Mamba-2 Recurrent State Computation to
        Tensor Cores with cuTile" (disconfirmai.com digest of the NVIDIA
        Developer Blog post on Mamba-2 forward kernels in cuTile).

The oracle proper is the plain token recurrence in ``ssd_oracle.c``
(P1 opening paragraph: fixed-size hidden state updated per token; jump-formula
paragraph: the update is an outer product b x^T plus a multiplicative decay):

    h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * B_t x_t^T      (N x P per head)
    y_t = C_t^T h_t + D_h * x_t

This module loads that library through ctypes (``Oracle.decode_step`` is the
same recurrence over one token) and adds two definitional helpers that need no
recurrence:

* ``dA_cumsum_ref``: the in-chunk inclusive sum of dt*A (P1 paragraph on the
  three kernels: per-token, per-head cumulative sums of the decay term inside
  each chunk), in fp64.
* ``chunk_states_ref`` / ``carried_states_ref``: states at chunk boundaries,
  produced by running the recurrence itself (not the chunked algorithm).

Every function here is parity-pinned by ``tests/test_oracle_pins.py`` against
``oracle/forms.py`` (brute-force semiseparable matrix, A=0 closed form,
geometric series, chunked form at every chunk size) and by invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(_HERE, "ssd_oracle.c")
LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")

_I64 = ctypes.c_int64
_PTR = ctypes.c_void_p


def build(src: str = SRC_PATH, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math) into a shared library."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-std=c99", *extra_flags,
           "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 64))


class Oracle:
    """ctypes handle on one build of ``ssd_oracle.c``."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library not built: {path} (run oracle.oracle.build())")
        self.path = path
        self.lib = ctypes.CDLL(path)
        f = self.lib.ssd_oracle_recurrence
        f.restype = ctypes.c_int
        f.argtypes = [_I64] * 6 + [_PTR] * 7 + [_I64, _PTR, _I64, ctypes.c_int, _PTR, _PTR, _PTR, ctypes.c_int]
        self._fn = f

    # ------------------------------------------------------------------ core
    def recurrence(self, x, dt, A, Bm, Cm, D=None, h0=None, pairs=None, chunk=0,
                   reset_each_chunk=False, want_boundary=False, nthreads=None):
        """Run the token recurrence for the (b, h) pairs listed (all if None).

        Arrays are float32 (bf16 inputs are passed already widened to float32,
        which is exact).  ``h0`` is float64 [B,H,N,P] or None.
        Returns ``(y [npairs,L,P], final [npairs,N,P], boundary or None)`` in
        float64, where ``boundary`` is [npairs, nc, N, P] (see ssd_oracle.c).
        """
        x = np.ascontiguousarray(x, dtype=np.float32)
        dt = np.ascontiguousarray(dt, dtype=np.float32)
        A = np.ascontiguousarray(A, dtype=np.float32)
        Bm = np.ascontiguousarray(Bm, dtype=np.float32)
        Cm = np.ascontiguousarray(Cm, dtype=np.float32)
        Bsz, L, H, P = x.shape
        G, N = Bm.shape[2], Bm.shape[3]
        assert dt.shape == (Bsz, L, H) and A.shape == (H,)
        assert Bm.shape == (Bsz, L, G, N) and Cm.shape == (Bsz, L, G, N)
        if D is not None:
            D = np.ascontiguousarray(D, dtype=np.float32)
            assert D.shape == (H,)
        if h0 is not None:
            h0 = np.ascontiguousarray(h0, dtype=np.float64)
            assert h0.shape == (Bsz, H, N, P)
        if pairs is None:
            npairs, pairs_arr = Bsz * H, None
        else:
            pairs_arr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64))
            npairs = int(pairs_arr.size)
        nc = (L + chunk - 1) // chunk if chunk > 0 else 0
        y = np.empty((npairs, L, P), dtype=np.float64)
        fin = np.empty((npairs, N, P), dtype=np.float64)
        bnd = np.empty((npairs, nc, N, P), dtype=np.float64) if want_boundary else None
        nthreads = default_threads() if nthreads is None else int(nthreads)

        def p(a):
            return None if a is None else a.ctypes.data_as(_PTR)

        rc = self._fn(Bsz, L, H, P, N, G, p(x), p(dt), p(A), p(Bm), p(Cm), p(D), p(h0),
                      npairs, p(pairs_arr), int(chunk), int(bool(reset_each_chunk)),
                      p(y), p(fin), p(bnd), nthreads)
        if rc != 0:
            raise RuntimeError(f"ssd_oracle_recurrence failed with code {rc}")
        return y, fin, bnd

    # ------------------------------------------------------------- wrappers
    def forward(self, x, dt, A, Bm, Cm, D=None, h0=None, nthreads=None):
        """Whole-tensor forward: y [B,L,H,P] and final states [B,H,N,P] (fp64)."""
        Bsz, L, H, P = x.shape
        N = Bm.shape[3]
        y, fin, _ = self.recurrence(x, dt, A, Bm, Cm, D, h0, nthreads=nthreads)
        y = y.reshape(Bsz, H, L, P).transpose(0, 2, 1, 3)
        return np.ascontiguousarray(y), fin.reshape(Bsz, H, N, P)

    def decode_step(self, x, dt, A, Bm, Cm, D, state, nthreads=None):
        """One token per sequence (P1 opening paragraph: the fixed-size state
        is updated once per token): the recurrence run over a single token
        from ``state``.  x [B,H,P], dt [B,H], Bm/Cm [B,G,N], state [B,H,N,P].
        Returns (y [B,H,P], new state [B,H,N,P]) in fp64; no arithmetic of its
        own beyond the recurrence."""
        Bsz, H, P = x.shape
        G, N = Bm.shape[1], Bm.shape[2]
        y, fin = self.forward(np.asarray(x)[:, None], np.asarray(dt)[:, None], A, np.asarray(Bm)[:, None],
                              np.asarray(Cm)[:, None], D, h0=state, nthreads=nthreads)
        return y[:, 0], fin

    def forward_pairs(self, x, dt, A, Bm, Cm, D, pairs, h0=None, chunk=0, nthreads=None):
        """y [npairs,L,P], final [npairs,N,P] and (if chunk>0) the states entering
        each chunk [npairs,nc,N,P] for a subset of (b, h) pairs (b*H+h)."""
        return self.recurrence(x, dt, A, Bm, Cm, D, h0, pairs=pairs, chunk=chunk,
                               want_boundary=chunk > 0, nthreads=nthreads)

    def carried_states_ref(self, x, dt, A, Bm, Cm, Q, h0=None, pairs=None, nthreads=None):
        """State entering each chunk, h_{cQ-1} (h0 for c=0), from the full recurrence.

        Returns [B,nc,H,N,P] when pairs is None, else [npairs,nc,N,P]."""
        Bsz, L, H, P = x.shape
        N = Bm.shape[3]
        _, fin, bnd = self.recurrence(x, dt, A, Bm, Cm, None, h0, pairs=pairs, chunk=Q,
                                      want_boundary=True, nthreads=nthreads)
        if pairs is not None:
            return bnd, fin
        nc = bnd.shape[1]
        return np.ascontiguousarray(bnd.reshape(Bsz, H, nc, N, P).transpose(0, 2, 1, 3, 4)), \
            fin.reshape(Bsz, H, N, P)

    def chunk_states_ref(self, x, dt, A, Bm, Cm, Q, pairs=None, nthreads=None):
        """Each chunk's own contribution: the recurrence restarted from zero at
        the chunk's first token, read after its last token.

        Returns [B,nc,H,N,P] when pairs is None, else [npairs,nc,N,P]."""
        Bsz, L, H, P = x.shape
        N = Bm.shape[3]
        _, _, bnd = self.recurrence(x, dt, A, Bm, Cm, None, None, pairs=pairs, chunk=Q,
                                    reset_each_chunk=True, want_boundary=True, nthreads=nthreads)
        if pairs is not None:
            return bnd
        nc = bnd.shape[1]
        return np.ascontiguousarray(bnd.reshape(Bsz, H, nc, N, P).transpose(0, 2, 1, 3, 4))


def dA_cumsum_ref(dt, A, Q):
    """In-chunk inclusive cumulative sum of dt*A, laid out [B,H,nc,Q], fp64.

    P1, paragraph on the three kernels: per-token, per-head cumulative sums of
    the decay term within each chunk; P1, Blackwell-optimisation paragraph: the
    cumulative sums are stored token-contiguous per (batch, head).
    Positions past the end of a ragged last chunk are left at 0.
    """
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    Bsz, L, H = dt.shape
    nc = (L + Q - 1) // Q
    a = np.zeros((Bsz, nc * Q, H), dtype=np.float64)
    a[:, :L, :] = dt * A[None, None, :]
    G = np.cumsum(a.reshape(Bsz, nc, Q, H), axis=2).reshape(Bsz, nc * Q, H)
    G[:, L:, :] = 0.0
    return np.ascontiguousarray(G.reshape(Bsz, nc, Q, H).transpose(0, 3, 1, 2))


def dt_bhl_ref(dt, Q):
    """dt re-laid out as [B,H,nc,Q] (zeros past a ragged end), fp64."""
    dt = np.asarray(dt, dtype=np.float64)
    Bsz, L, H = dt.shape
    nc = (L + Q - 1) // Q
    out = np.zeros((Bsz, nc * Q, H), dtype=np.float64)
    out[:, :L, :] = dt
    return np.ascontiguousarray(out.reshape(Bsz, nc, Q, H).transpose(0, 3, 1, 2))


_DEFAULT = None


def get() -> Oracle:
    """Shared Oracle instance on the default library path (built on demand)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(LIB_PATH):
            build()
        _DEFAULT = Oracle(LIB_PATH)
    return _DEFAULT
