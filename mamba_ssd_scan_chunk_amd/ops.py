"""Python entry points with the C ABI's names, over torch device tensors.

Each function checks that its tensors are CUDA (HIP) tensors of the expected
dtype, shape and contiguity, then calls the matching ``ssd_*`` function of
``libmamba_ssd.so`` on torch's current stream.  Nothing is computed here and
nothing is copied or converted silently: a mismatch raises ``ValueError``, a
failed call raises ``SSDError``.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import torch

from ._lib import MMA, SSD_BF16, SSD_F32, SSDShape, check, load_library

_DT = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}
_DTNAME = {"f32": torch.float32, "bf16": torch.bfloat16}


def _shape(s) -> SSDShape:
    if isinstance(s, SSDShape):
        return s
    return SSDShape.make(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["dstate"], s["ngroups"], s["chunk"])


def _dims(sh: SSDShape):
    nc = -(-sh.seqlen // sh.chunk)
    return sh.batch, sh.seqlen, sh.nheads, sh.headdim, sh.dstate, sh.ngroups, sh.chunk, nc


def _req(t: Optional[torch.Tensor], name: str, shape, dtypes) -> None:
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _mma(mma: str) -> int:
    if mma not in MMA:
        raise ValueError(f"mma must be one of {list(MMA)}")
    return MMA[mma]


def ssd_chunk_cumsum(shape, dt, A, dA_cumsum=None, dt_bhl=None, with_dt=True, stream=None):
    """dA_cumsum, dt_bhl [B,H,nc,Q] from dt [B,L,H], A [H] (fp32)."""
    sh = _shape(shape)
    B, L, H, P, N, G, Q, nc = _dims(sh)
    f32 = (torch.float32,)
    _req(dt, "dt", (B, L, H), f32)
    _req(A, "A", (H,), f32)
    if dA_cumsum is None:
        dA_cumsum = torch.empty((B, H, nc, Q), device=dt.device, dtype=torch.float32)
    if dt_bhl is None and with_dt:
        dt_bhl = torch.empty((B, H, nc, Q), device=dt.device, dtype=torch.float32)
    _req(dA_cumsum, "dA_cumsum", (B, H, nc, Q), f32)
    if dt_bhl is not None:
        _req(dt_bhl, "dt_bhl", (B, H, nc, Q), f32)
    lib = load_library()
    check(lib.ssd_chunk_cumsum(sh, _ptr(dt), _ptr(A), _ptr(dA_cumsum), _ptr(dt_bhl), _stream(stream)))
    return dA_cumsum, dt_bhl


def ssd_chunk_state(shape, x, Bm, dt_bhl, dA_cumsum, states=None, mma="bf16", states_dtype="f32", stream=None):
    """Per-chunk states [B,nc,H,N,P] (jump formula with decay), stored in
    ``states_dtype`` ("f32", or "bf16" rounded to nearest even; a given
    ``states`` tensor's dtype wins)."""
    sh = _shape(shape)
    B, L, H, P, N, G, Q, nc = _dims(sh)
    io = (torch.float32, torch.bfloat16)
    _req(x, "x", (B, L, H, P), io)
    _req(Bm, "Bm", (B, L, G, N), (x.dtype,))
    _req(dt_bhl, "dt_bhl", (B, H, nc, Q), (torch.float32,))
    _req(dA_cumsum, "dA_cumsum", (B, H, nc, Q), (torch.float32,))
    if states is None:
        sdt = _DTNAME[states_dtype] if isinstance(states_dtype, str) else states_dtype
        states = torch.empty((B, nc, H, N, P), device=x.device, dtype=sdt)
    _req(states, "states", (B, nc, H, N, P), io)
    lib = load_library()
    check(lib.ssd_chunk_state(sh, _ptr(x), _ptr(Bm), _DT[x.dtype], _ptr(dt_bhl), _ptr(dA_cumsum),
                              _ptr(states), _DT[states.dtype], _mma(mma), _stream(stream)))
    return states


def ssd_chunk_cumsum_state(shape, x, Bm, dt, A, dA_cumsum=None, dt_bhl=None, states=None, mma="bf16",
                           states_dtype="f32", stream=None):
    """ssd_chunk_cumsum then ssd_chunk_state in one call (one kernel where the
    chunk states have a head-group kernel).  Returns (dA_cumsum, dt_bhl,
    states)."""
    sh = _shape(shape)
    B, L, H, P, N, G, Q, nc = _dims(sh)
    io = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _req(x, "x", (B, L, H, P), io)
    _req(Bm, "Bm", (B, L, G, N), (x.dtype,))
    _req(dt, "dt", (B, L, H), f32)
    _req(A, "A", (H,), f32)
    if dA_cumsum is None:
        dA_cumsum = torch.empty((B, H, nc, Q), device=x.device, dtype=torch.float32)
    if dt_bhl is None:
        dt_bhl = torch.empty((B, H, nc, Q), device=x.device, dtype=torch.float32)
    _req(dA_cumsum, "dA_cumsum", (B, H, nc, Q), f32)
    _req(dt_bhl, "dt_bhl", (B, H, nc, Q), f32)
    if states is None:
        sdt = _DTNAME[states_dtype] if isinstance(states_dtype, str) else states_dtype
        states = torch.empty((B, nc, H, N, P), device=x.device, dtype=sdt)
    _req(states, "states", (B, nc, H, N, P), io)
    lib = load_library()
    check(lib.ssd_chunk_cumsum_state(sh, _ptr(x), _ptr(Bm), _DT[x.dtype], _ptr(dt), _ptr(A), _ptr(dA_cumsum),
                                     _ptr(dt_bhl), _ptr(states), _DT[states.dtype], _mma(mma), _stream(stream)))
    return dA_cumsum, dt_bhl, states


def ssd_state_passing(shape, chunk_states, dA_cumsum, initial_states=None, carried=None, final_states=None,
                      in_place=False, carried_dtype="f32", stream=None):
    """Carried states [B,nc,H,N,P] (state entering each chunk) in
    ``carried_dtype`` ("f32" or "bf16", rounded to nearest even; a given
    ``carried`` tensor's dtype wins) and fp32 final states [B,H,N,P], from
    chunk states in fp32 or bf16 (the recurrence runs in fp32).
    ``in_place=True`` writes the carried states over ``chunk_states``, in
    their dtype."""
    sh = _shape(shape)
    B, L, H, P, N, G, Q, nc = _dims(sh)
    f32 = (torch.float32,)
    _req(chunk_states, "chunk_states", (B, nc, H, N, P), (torch.float32, torch.bfloat16))
    _req(dA_cumsum, "dA_cumsum", (B, H, nc, Q), f32)
    if initial_states is not None:
        _req(initial_states, "initial_states", (B, H, N, P), f32)
    if carried is None:
        cdt = _DTNAME[carried_dtype] if isinstance(carried_dtype, str) else carried_dtype
        if in_place:
            carried = chunk_states
        else:
            carried = torch.empty((B, nc, H, N, P), device=chunk_states.device, dtype=cdt)
    _req(carried, "carried", (B, nc, H, N, P), (torch.float32, torch.bfloat16))
    if final_states is None:
        final_states = torch.empty((B, H, N, P), device=chunk_states.device, dtype=torch.float32)
    _req(final_states, "final_states", (B, H, N, P), f32)
    lib = load_library()
    check(lib.ssd_state_passing(sh, _ptr(chunk_states), _DT[chunk_states.dtype], _ptr(carried), _DT[carried.dtype],
                                _ptr(dA_cumsum), _ptr(initial_states), _ptr(final_states), _stream(stream)))
    return carried, final_states


def ssd_chunk_state_passing(shape, x, Bm, dt_bhl, dA_cumsum, initial_states=None, carried=None,
                            final_states=None, carried_dtype="f32", want_final=True, mma="bf16", stream=None):
    """Fused state path: carried states [B,nc,H,N,P] in ``carried_dtype`` and
    fp32 final states [B,H,N,P] (None when ``want_final`` is false), without
    materialising the chunk states; bit-identical to ssd_chunk_state followed
    by ssd_state_passing."""
    sh = _shape(shape)
    B, L, H, P, N, G, Q, nc = _dims(sh)
    io = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _req(x, "x", (B, L, H, P), io)
    _req(Bm, "Bm", (B, L, G, N), (x.dtype,))
    _req(dt_bhl, "dt_bhl", (B, H, nc, Q), f32)
    _req(dA_cumsum, "dA_cumsum", (B, H, nc, Q), f32)
    if initial_states is not None:
        _req(initial_states, "initial_states", (B, H, N, P), f32)
    if carried is None:
        cdt = _DTNAME[carried_dtype] if isinstance(carried_dtype, str) else carried_dtype
        carried = torch.empty((B, nc, H, N, P), device=x.device, dtype=cdt)
    _req(carried, "carried", (B, nc, H, N, P), (torch.float32, torch.bfloat16))
    if final_states is None and want_final:
        final_states = torch.empty((B, H, N, P), device=x.device, dtype=torch.float32)
    if final_states is not None:
        _req(final_states, "final_states", (B, H, N, P), f32)
    lib = load_library()
    check(lib.ssd_chunk_state_passing(sh, _ptr(x), _ptr(Bm), _DT[x.dtype], _ptr(dt_bhl), _ptr(dA_cumsum),
                                      _ptr(initial_states), _ptr(carried), _DT[carried.dtype],
                                      _ptr(final_states), _mma(mma), _stream(stream)))
    return carried, final_states


def ssd_chunk_scan(shape, x, Bm, Cm, dt_bhl, dA_cumsum, carried, D, y=None, y_dtype=None, mma="bf16",
                   stream=None):
    """y [B,L,H,P] in ``y_dtype`` (default: x's dtype)."""
    sh = _shape(shape)
    B, L, H, P, N, G, Q, nc = _dims(sh)
    io = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _req(x, "x", (B, L, H, P), io)
    _req(Bm, "Bm", (B, L, G, N), (x.dtype,))
    _req(Cm, "Cm", (B, L, G, N), (x.dtype,))
    _req(dt_bhl, "dt_bhl", (B, H, nc, Q), f32)
    _req(dA_cumsum, "dA_cumsum", (B, H, nc, Q), f32)
    _req(carried, "carried", (B, nc, H, N, P), (torch.float32, torch.bfloat16))
    _req(D, "D", (H,), f32)
    ydt = x.dtype if y_dtype is None else (_DTNAME[y_dtype] if isinstance(y_dtype, str) else y_dtype)
    if y is None:
        y = torch.empty((B, L, H, P), device=x.device, dtype=ydt)
    _req(y, "y", (B, L, H, P), io)
    lib = load_library()
    check(lib.ssd_chunk_scan(sh, _ptr(x), _ptr(Bm), _ptr(Cm), _DT[x.dtype], _ptr(dt_bhl), _ptr(dA_cumsum),
                             _ptr(carried), _DT[carried.dtype], _ptr(D), _ptr(y), _DT[y.dtype], _mma(mma),
                             _stream(stream)))
    return y


def ssd_decode_step(x, dt, A, Bm, Cm, D, state, y=None, y_dtype=None, stream=None):
    """One token per sequence: ``state`` [B,H,N,P] fp32 is advanced in place,
    returns y [B,H,P] in ``y_dtype`` (default: x's dtype).  x [B,H,P], dt
    [B,H], A [H], Bm/Cm [B,G,N] (x's dtype), D [H]."""
    if x.dim() != 3 or Bm.dim() != 3 or state.dim() != 4:
        raise ValueError("x must be [B,H,P], Bm/Cm [B,G,N], state [B,H,N,P]")
    B, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    io = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _req(x, "x", (B, H, P), io)
    _req(dt, "dt", (B, H), f32)
    _req(A, "A", (H,), f32)
    _req(Bm, "Bm", (B, G, N), (x.dtype,))
    _req(Cm, "Cm", (B, G, N), (x.dtype,))
    _req(D, "D", (H,), f32)
    _req(state, "state", (B, H, N, P), f32)
    ydt = x.dtype if y_dtype is None else (_DTNAME[y_dtype] if isinstance(y_dtype, str) else y_dtype)
    if y is None:
        y = torch.empty((B, H, P), device=x.device, dtype=ydt)
    _req(y, "y", (B, H, P), io)
    sh = SSDShape.make(B, 1, H, P, N, G, 1)
    lib = load_library()
    check(lib.ssd_decode_step(sh, _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _DT[x.dtype],
                              _ptr(state), _ptr(y), _DT[y.dtype], _stream(stream)))
    return y


def ssd_workspace_bytes(shape) -> int:
    return int(load_library().ssd_workspace_bytes(_shape(shape)))


def ssd_workspace_bytes_varlen(shape) -> int:
    return int(load_library().ssd_workspace_bytes_varlen(_shape(shape)))


def ssd_forward(shape, x, dt, A, Bm, Cm, D, initial_states=None, y=None, y_dtype=None, final_states=None,
                want_final=True, workspace=None, mma="bf16", stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One-call forward.  Returns (y, final_states or None)."""
    sh = _shape(shape)
    B, L, H, P, N, G, Q, nc = _dims(sh)
    io = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _req(x, "x", (B, L, H, P), io)
    _req(dt, "dt", (B, L, H), f32)
    _req(A, "A", (H,), f32)
    _req(Bm, "Bm", (B, L, G, N), (x.dtype,))
    _req(Cm, "Cm", (B, L, G, N), (x.dtype,))
    _req(D, "D", (H,), f32)
    if initial_states is not None:
        _req(initial_states, "initial_states", (B, H, N, P), f32)
    ydt = x.dtype if y_dtype is None else (_DTNAME[y_dtype] if isinstance(y_dtype, str) else y_dtype)
    if y is None:
        y = torch.empty((B, L, H, P), device=x.device, dtype=ydt)
    _req(y, "y", (B, L, H, P), io)
    if final_states is None and want_final:
        final_states = torch.empty((B, H, N, P), device=x.device, dtype=torch.float32)
    if final_states is not None:
        _req(final_states, "final_states", (B, H, N, P), f32)
    lib = load_library()
    need = int(lib.ssd_workspace_bytes(sh))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=x.device, dtype=torch.uint8)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    check(lib.ssd_forward(sh, _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _DT[x.dtype],
                          _ptr(initial_states), _ptr(y), _DT[y.dtype], _ptr(final_states), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _mma(mma), _stream(stream)))
    return y, final_states


def ssd_forward_noalloc(shape, x, dt, A, Bm, Cm, D, initial_states=None, y=None, y_dtype=None,
                        final_states=None, want_final=True, mma="bf16", stream=None):
    """ssd_forward in the library's static device scratch array (no
    workspace; for callers that cannot allocate).  Returns (y,
    final_states or None); y and final_states are allocated here only when
    not given."""
    sh = _shape(shape)
    B, L, H, P, N, G, Q, nc = _dims(sh)
    io = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _req(x, "x", (B, L, H, P), io)
    _req(dt, "dt", (B, L, H), f32)
    _req(A, "A", (H,), f32)
    _req(Bm, "Bm", (B, L, G, N), (x.dtype,))
    _req(Cm, "Cm", (B, L, G, N), (x.dtype,))
    _req(D, "D", (H,), f32)
    if initial_states is not None:
        _req(initial_states, "initial_states", (B, H, N, P), f32)
    ydt = x.dtype if y_dtype is None else (_DTNAME[y_dtype] if isinstance(y_dtype, str) else y_dtype)
    if y is None:
        y = torch.empty((B, L, H, P), device=x.device, dtype=ydt)
    _req(y, "y", (B, L, H, P), io)
    if final_states is None and want_final:
        final_states = torch.empty((B, H, N, P), device=x.device, dtype=torch.float32)
    if final_states is not None:
        _req(final_states, "final_states", (B, H, N, P), f32)
    lib = load_library()
    check(lib.ssd_forward_noalloc(sh, _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _DT[x.dtype],
                                  _ptr(initial_states), _ptr(y), _DT[y.dtype], _ptr(final_states), _mma(mma),
                                  _stream(stream)))
    return y, final_states


def ssd_forward_varlen(shape, x, dt, A, Bm, Cm, D, seq_idx, initial_states=None, y=None, y_dtype=None,
                       final_states=None, want_final=True, seq_last=None, seq_states=None, workspace=None,
                       mma="bf16", stream=None):
    """One-call forward over packed sequences: seq_idx [B,L] int32 names each
    token's sequence; the state restarts from zero wherever it changes along
    a row.  Returns (y, final_states of each row's last sequence or None) and,
    when seq_last (int64 [nseq] flattened token indices b*L+t) is given, also
    seq_states [nseq,H,N,P]: the state after each of those tokens."""
    sh = _shape(shape)
    B, L, H, P, N, G, Q, nc = _dims(sh)
    io = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _req(x, "x", (B, L, H, P), io)
    _req(dt, "dt", (B, L, H), f32)
    _req(A, "A", (H,), f32)
    _req(Bm, "Bm", (B, L, G, N), (x.dtype,))
    _req(Cm, "Cm", (B, L, G, N), (x.dtype,))
    _req(D, "D", (H,), f32)
    _req(seq_idx, "seq_idx", (B, L), (torch.int32,))
    if initial_states is not None:
        _req(initial_states, "initial_states", (B, H, N, P), f32)
    ydt = x.dtype if y_dtype is None else (_DTNAME[y_dtype] if isinstance(y_dtype, str) else y_dtype)
    if y is None:
        y = torch.empty((B, L, H, P), device=x.device, dtype=ydt)
    _req(y, "y", (B, L, H, P), io)
    if final_states is None and want_final:
        final_states = torch.empty((B, H, N, P), device=x.device, dtype=torch.float32)
    if final_states is not None:
        _req(final_states, "final_states", (B, H, N, P), f32)
    nseq = 0
    if seq_last is not None:
        _req(seq_last, "seq_last", (seq_last.numel(),), (torch.int64,))
        nseq = seq_last.numel()
        if seq_states is None:
            seq_states = torch.empty((nseq, H, N, P), device=x.device, dtype=torch.float32)
        _req(seq_states, "seq_states", (nseq, H, N, P), f32)
    lib = load_library()
    need = ssd_workspace_bytes_varlen(sh)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=x.device, dtype=torch.uint8)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    check(lib.ssd_forward_varlen(sh, _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _DT[x.dtype],
                                 _ptr(seq_idx), _ptr(initial_states), _ptr(y), _DT[y.dtype], _ptr(final_states),
                                 nseq, _ptr(seq_last if nseq else None), _ptr(seq_states if nseq else None),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _mma(mma),
                                 _stream(stream)))
    if seq_last is not None:
        return y, final_states, seq_states
    return y, final_states


def ssd_backward(shape, x, dt, A, Bm, Cm, D, dy, initial_states=None, dfinal=None, want_dinitial=True,
                 workspace=None, mma="f32", out=None, stream=None) -> Dict[str, Optional[torch.Tensor]]:
    """Gradients of ``ssd_forward`` for dL/dy = dy and dL/dfinal = dfinal
    (None: zero).  Returns fp32 tensors dx, ddt, dA, dB, dC, dD and dinitial
    (None unless ``want_dinitial``), written into the tensors of ``out`` (a
    dict with those keys) where given.  ``mma``: "f32" (fp32 matrix operands)
    or "bf16" (bf16 operands, fp32 accumulation; faster, ~1e-2 relative)."""
    sh = _shape(shape)
    B, L, H, P, N, G, Q, nc = _dims(sh)
    io = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _req(x, "x", (B, L, H, P), io)
    _req(dt, "dt", (B, L, H), f32)
    _req(A, "A", (H,), f32)
    _req(Bm, "Bm", (B, L, G, N), (x.dtype,))
    _req(Cm, "Cm", (B, L, G, N), (x.dtype,))
    _req(D, "D", (H,), f32)
    _req(dy, "dy", (B, L, H, P), io)
    if initial_states is not None:
        _req(initial_states, "initial_states", (B, H, N, P), f32)
    if dfinal is not None:
        _req(dfinal, "dfinal", (B, H, N, P), f32)
    dev = x.device
    shapes = {"dx": (B, L, H, P), "ddt": (B, L, H), "dA": (H,), "dB": (B, L, G, N), "dC": (B, L, G, N),
              "dD": (H,), "dinitial": (B, H, N, P)}
    given = dict(out or {})
    out = {}
    for k, shp in shapes.items():
        if k == "dinitial" and not want_dinitial:
            out[k] = None
            continue
        out[k] = given[k] if given.get(k) is not None else torch.empty(shp, device=dev)
        _req(out[k], k, shp, f32)
    lib = load_library()
    need = int(lib.ssd_backward_workspace_bytes(sh))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    check(lib.ssd_backward(sh, _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(D), _DT[x.dtype],
                           _ptr(initial_states), _ptr(dy), _DT[dy.dtype], _ptr(dfinal), _ptr(out["dx"]),
                           _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
                           _ptr(out["dinitial"]), _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _mma(mma), _stream(stream)))
    return out


def ssd_backward_workspace_bytes(shape) -> int:
    return int(load_library().ssd_backward_workspace_bytes(_shape(shape)))


def shape_of(inp: Dict[str, torch.Tensor], chunk: int) -> SSDShape:
    """ssd_shape from x [B,L,H,P] and Bm [B,L,G,N]."""
    B, L, H, P = inp["x"].shape
    G, N = inp["Bm"].shape[2], inp["Bm"].shape[3]
    return SSDShape.make(B, L, H, P, N, G, chunk)
