"""The C ABI on the host (no GPU needed): the library loads, exports every
function ``include/ssd.h`` declares, and rejects every invalid argument with
its documented status before making any HIP call."""
import ctypes
import os
import re

import pytest

from mamba_ssd_scan_chunk_amd import _lib
from mamba_ssd_scan_chunk_amd._lib import SSDShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS, ALIGN = 0, 1, 2, 3, 4, 5, 6
FAKE = 0x100000  # a 16-byte-aligned non-null address; never dereferenced (checks fail first)


@pytest.fixture(scope="module")
def lib():
    return _lib.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ["ssd_chunk_cumsum", "ssd_chunk_state", "ssd_chunk_cumsum_state", "ssd_state_passing",
              "ssd_chunk_scan", "ssd_forward",
              "ssd_chunk_state_passing", "ssd_decode_step", "ssd_forward_varlen", "ssd_workspace_bytes",
              "ssd_workspace_bytes_varlen", "ssd_backward", "ssd_backward_workspace_bytes", "ssd_status_string",
              "ssd_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in ssd.h but not exported"
    assert lib.ssd_abi_version() == 4


def test_status_strings(lib):
    for code, name in _lib.STATUS_NAMES.items():
        s = lib.ssd_status_string(code).decode()
        assert s.startswith(name)
    assert lib.ssd_status_string(99).decode() == "unknown ssd_status"


def shape(**kw):
    d = dict(batch=2, seqlen=512, nheads=4, headdim=64, dstate=128, ngroups=1, chunk=256)
    d.update(kw)
    return SSDShape.make(**d)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), SHAPE), (dict(seqlen=0), SHAPE), (dict(nheads=-1), SHAPE), (dict(headdim=0), SHAPE),
    (dict(dstate=0), SHAPE), (dict(ngroups=0), SHAPE), (dict(chunk=0), SHAPE), (dict(nheads=6, ngroups=4), SHAPE),
    (dict(headdim=24), UNSUP), (dict(dstate=40), UNSUP), (dict(headdim=272), UNSUP), (dict(dstate=272), UNSUP),
    (dict(chunk=16), UNSUP), (dict(chunk=96), UNSUP), (dict(chunk=512), UNSUP),
    # in-chunk 32-bit row offsets would overflow: Q*H*P or Q*G*N >= 2^31
    (dict(nheads=32768, headdim=256, chunk=256), UNSUP),
    (dict(nheads=65535, ngroups=65535, dstate=256, headdim=16, chunk=256), UNSUP),
    (dict(nheads=65535, headdim=144, chunk=256), UNSUP),
    # 32-bit block numbering: B * nc * H * (P/16) >= 2^31
    (dict(batch=65535, seqlen=256 * 2048, nheads=16, headdim=64), UNSUP),
])
def test_shape_checks(lib, kw, code):
    s = shape(**kw)
    assert lib.ssd_chunk_cumsum(s, FAKE, FAKE, FAKE, FAKE, None) == code
    assert lib.ssd_chunk_state(s, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 0, 0, None) == code
    assert lib.ssd_state_passing(s, FAKE, 0, FAKE, 0, FAKE, None, FAKE, None) == code
    assert lib.ssd_chunk_scan(s, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1, 0, None) == code
    assert lib.ssd_forward(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, FAKE, 1, FAKE, FAKE, 1 << 40, 0,
                           None) == code
    assert lib.ssd_chunk_cumsum_state(s, FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, None) == code
    assert lib.ssd_workspace_bytes(s) == 0


def test_chunk_cumsum_state_checks(lib):
    s = shape()
    f = lambda *a: lib.ssd_chunk_cumsum_state(s, *a, None)
    assert f(FAKE, FAKE, 1, None, FAKE, FAKE, FAKE, FAKE, 0, 0) == NULL      # dt
    assert f(FAKE, FAKE, 1, FAKE, None, FAKE, FAKE, FAKE, 0, 0) == NULL      # A
    assert f(FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, 0, 0) == NULL      # dt_bhl is required here
    assert f(FAKE, FAKE, 7, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0) == DTYPE
    assert f(FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 9) == DTYPE
    assert f(FAKE, FAKE, 1, FAKE + 4, FAKE, FAKE, FAKE, FAKE, 0, 0) == ALIGN
    assert f(FAKE, FAKE, 1, FAKE, FAKE, FAKE + 8, FAKE, FAKE, 0, 0) == ALIGN


def test_largest_offsets_still_accepted(lib):
    """Just below the 32-bit offset limit the shape is valid (workspace size
    defined), one head more it is refused."""
    ok = shape(nheads=32767, headdim=256, chunk=256, seqlen=256, batch=1)  # 256*32767*256 < 2^31
    assert lib.ssd_workspace_bytes(ok) > 0
    assert lib.ssd_workspace_bytes(shape(nheads=32768, headdim=256, chunk=256, seqlen=256, batch=1)) == 0
    grouped = shape(nheads=32768, ngroups=32768, headdim=16, dstate=256, chunk=256, seqlen=256, batch=1)
    assert lib.ssd_workspace_bytes(grouped) == 0


def test_null_shape(lib):
    assert lib.ssd_chunk_cumsum(None, FAKE, FAKE, FAKE, FAKE, None) == NULL
    assert lib.ssd_workspace_bytes(None) == 0


def test_null_pointers(lib):
    s = shape()
    assert lib.ssd_chunk_cumsum(s, None, FAKE, FAKE, FAKE, None) == NULL
    assert lib.ssd_chunk_cumsum(s, FAKE, None, FAKE, FAKE, None) == NULL
    assert lib.ssd_chunk_cumsum(s, FAKE, FAKE, None, FAKE, None) == NULL
    for i in range(5):
        args = [FAKE] * 5
        args[i] = None
        x, Bm, dtb, dA, st = args
        assert lib.ssd_chunk_state(s, x, Bm, 1, dtb, dA, st, 0, 0, None) == NULL
        assert lib.ssd_chunk_state(s, x, Bm, 1, dtb, dA, st, 1, 0, None) == NULL
    for i in range(3):
        args = [FAKE] * 3
        args[i] = None
        for sdt in (0, 1):
            assert lib.ssd_state_passing(s, args[0], sdt, args[1], 0, args[2], None, FAKE, None) == NULL
            assert lib.ssd_state_passing(s, args[0], sdt, args[1], 1, args[2], None, FAKE, None) == NULL
    for i in range(8):
        args = [FAKE] * 8
        args[i] = None
        x, Bm, Cm, dtb, dA, car, D, y = args
        assert lib.ssd_chunk_scan(s, x, Bm, Cm, 1, dtb, dA, car, 0, D, y, 1, 0, None) == NULL
        assert lib.ssd_chunk_scan(s, x, Bm, Cm, 1, dtb, dA, car, 1, D, y, 1, 0, None) == NULL
    for i in range(7):
        args = [FAKE] * 7
        args[i] = None
        x, dt, A, Bm, Cm, D, y = args
        assert lib.ssd_forward(s, x, dt, A, Bm, Cm, D, 1, None, y, 1, None, FAKE, 1 << 40, 0, None) == NULL


def test_dtype_and_mma_enums(lib):
    s = shape()
    assert lib.ssd_chunk_state(s, FAKE, FAKE, 2, FAKE, FAKE, FAKE, 0, 0, None) == DTYPE
    assert lib.ssd_chunk_state(s, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 0, 2, None) == DTYPE
    assert lib.ssd_chunk_state(s, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 2, 0, None) == DTYPE
    assert lib.ssd_chunk_scan(s, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 7, 0, None) == DTYPE
    assert lib.ssd_chunk_scan(s, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1, -1, None) == DTYPE
    assert lib.ssd_chunk_scan(s, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 3, FAKE, FAKE, 1, 0, None) == DTYPE
    assert lib.ssd_state_passing(s, FAKE, 0, FAKE, 2, FAKE, None, FAKE, None) == DTYPE
    assert lib.ssd_state_passing(s, FAKE, 3, FAKE, 0, FAKE, None, FAKE, None) == DTYPE
    assert lib.ssd_forward(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 5, None, FAKE, 1, FAKE, FAKE, 1 << 40, 0,
                           None) == DTYPE


def test_alignment(lib):
    s = shape()
    odd = FAKE + 4
    assert lib.ssd_chunk_cumsum(s, odd, FAKE, FAKE, FAKE, None) == ALIGN
    assert lib.ssd_chunk_cumsum(s, FAKE, FAKE, FAKE, odd, None) == ALIGN
    assert lib.ssd_chunk_state(s, FAKE, odd, 1, FAKE, FAKE, FAKE, 0, 0, None) == ALIGN
    assert lib.ssd_chunk_state(s, FAKE, FAKE, 1, FAKE, FAKE, odd, 1, 0, None) == ALIGN
    assert lib.ssd_state_passing(s, FAKE, 0, FAKE, 0, FAKE, odd, FAKE, None) == ALIGN
    assert lib.ssd_state_passing(s, FAKE, 0, odd, 1, FAKE, None, FAKE, None) == ALIGN
    assert lib.ssd_state_passing(s, odd, 1, FAKE + 16, 1, FAKE, None, FAKE, None) == ALIGN
    assert lib.ssd_chunk_scan(s, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 0, FAKE, odd, 1, 0, None) == ALIGN
    assert lib.ssd_chunk_scan(s, FAKE, FAKE, FAKE, 1, FAKE, FAKE, odd, 1, FAKE, FAKE, 1, 0, None) == ALIGN
    assert lib.ssd_forward(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, odd, FAKE, 1, FAKE, FAKE, 1 << 40, 0,
                           None) == ALIGN


def test_chunk_state_passing_checks(lib):
    """The fused state path validates like the calls it fuses and refuses what
    its kernel does not cover, all before any HIP call."""
    s = shape()
    for i in range(5):
        args = [FAKE] * 5
        args[i] = None
        x, Bm, dtb, dA, car = args
        assert lib.ssd_chunk_state_passing(s, x, Bm, 1, dtb, dA, None, car, 1, FAKE, 0, None) == NULL
    assert lib.ssd_chunk_state_passing(s, FAKE, FAKE, 2, FAKE, FAKE, None, FAKE, 1, FAKE, 0, None) == DTYPE
    assert lib.ssd_chunk_state_passing(s, FAKE, FAKE, 1, FAKE, FAKE, None, FAKE, 5, FAKE, 0, None) == DTYPE
    assert lib.ssd_chunk_state_passing(s, FAKE, FAKE, 1, FAKE, FAKE, None, FAKE, 1, FAKE, 3, None) == DTYPE
    odd = FAKE + 4
    assert lib.ssd_chunk_state_passing(s, FAKE, FAKE, 1, FAKE, FAKE, odd, FAKE, 1, FAKE, 0, None) == ALIGN
    assert lib.ssd_chunk_state_passing(s, FAKE, FAKE, 1, FAKE, FAKE, None, FAKE, 1, odd, 0, None) == ALIGN
    # fp32 inputs, fp32 matrix operands, N or P not a multiple of 64: not covered
    assert lib.ssd_chunk_state_passing(s, FAKE, FAKE, 0, FAKE, FAKE, None, FAKE, 1, FAKE, 0, None) == UNSUP
    assert lib.ssd_chunk_state_passing(s, FAKE, FAKE, 1, FAKE, FAKE, None, FAKE, 1, FAKE, 1, None) == UNSUP
    assert lib.ssd_chunk_state_passing(shape(dstate=48), FAKE, FAKE, 1, FAKE, FAKE, None, FAKE, 1, FAKE, 0,
                                       None) == UNSUP
    assert lib.ssd_chunk_state_passing(shape(headdim=32), FAKE, FAKE, 1, FAKE, FAKE, None, FAKE, 1, FAKE, 0,
                                       None) == UNSUP
    assert lib.ssd_chunk_state_passing(shape(batch=0), FAKE, FAKE, 1, FAKE, FAKE, None, FAKE, 1, FAKE, 0,
                                       None) == SHAPE


def test_decode_step_checks(lib):
    """The decode step takes one token per sequence (seqlen 1; chunk unused)
    and validates like the other calls, before any HIP call."""
    s = shape(seqlen=1, chunk=0)
    args = [FAKE] * 8
    for i in range(8):
        a = list(args)
        a[i] = None
        x, dt, A, Bm, Cm, D, st, y = a
        assert lib.ssd_decode_step(s, x, dt, A, Bm, Cm, D, 1, st, y, 1, None) == NULL
    assert lib.ssd_decode_step(None, *args[:6], 1, FAKE, FAKE, 1, None) == NULL
    assert lib.ssd_decode_step(shape(seqlen=2), *args[:6], 1, FAKE, FAKE, 1, None) == SHAPE
    assert lib.ssd_decode_step(shape(seqlen=1, nheads=6, ngroups=4), *args[:6], 1, FAKE, FAKE, 1, None) == SHAPE
    assert lib.ssd_decode_step(shape(seqlen=1, batch=0), *args[:6], 1, FAKE, FAKE, 1, None) == SHAPE
    assert lib.ssd_decode_step(s, *args[:6], 2, FAKE, FAKE, 1, None) == DTYPE
    assert lib.ssd_decode_step(s, *args[:6], 1, FAKE, FAKE, 9, None) == DTYPE
    assert lib.ssd_decode_step(shape(seqlen=1, headdim=6), *args[:6], 1, FAKE, FAKE, 1, None) == UNSUP
    assert lib.ssd_decode_step(shape(seqlen=1, headdim=1028), *args[:6], 1, FAKE, FAKE, 1, None) == UNSUP
    # shapes the chunked calls refuse are fine here: P = 20, N = 7, any chunk value
    odd = FAKE + 4
    assert lib.ssd_decode_step(shape(seqlen=1, headdim=20, dstate=7), *args[:6], 1, odd, FAKE, 1, None) == ALIGN
    assert lib.ssd_decode_step(s, odd, *args[1:6], 1, FAKE, FAKE, 1, None) == ALIGN


def test_forward_varlen_checks(lib):
    """The packed-sequence forward validates like ssd_forward, needs seq_idx,
    and its own (larger) workspace."""
    s = shape()
    B, L, H, P, N, Q = 2, 512, 4, 64, 128, 256
    nc = 2
    bhl = 4 * B * H * nc * Q
    ru = lambda v: (v + 255) // 256 * 256
    st = 4 * B * nc * H * N * P
    # dA, dt_bhl, fp32 carried states, bf16 chunk states, sequence starts, dA for the passing, masked dt
    base = ru(ru(ru(ru(bhl) + bhl) + st) + st // 2)
    need = ru(ru(ru(base + 4 * B * nc * Q) + bhl) + bhl)
    assert lib.ssd_workspace_bytes_varlen(s) == need
    assert lib.ssd_workspace_bytes_varlen(None) == 0
    a = [FAKE] * 6  # x, dt, A, Bm, Cm, D
    call = lambda sh, in_, sq, ws, wsb, nseq=0, last=None, st=None, mma=0: lib.ssd_forward_varlen(
        sh, *a, in_, sq, None, FAKE, 1, FAKE, nseq, last, st, ws, wsb, mma, None)
    assert call(s, 1, None, FAKE, need) == NULL
    assert call(s, 1, FAKE, FAKE, need - 1) == WS
    assert call(s, 1, FAKE, None, need) == WS
    assert call(s, 1, FAKE + 4, FAKE, need) == ALIGN
    assert call(s, 7, FAKE, FAKE, need) == DTYPE
    assert call(shape(headdim=24), 1, FAKE, FAKE, need) == UNSUP
    # requested per-sequence states need both arrays, aligned, and nseq >= 0
    assert call(s, 1, FAKE, FAKE, need, nseq=3, last=None, st=FAKE) == NULL
    assert call(s, 1, FAKE, FAKE, need, nseq=3, last=FAKE, st=None) == NULL
    assert call(s, 1, FAKE, FAKE, need, nseq=3, last=FAKE + 8, st=FAKE) == ALIGN
    assert call(s, 1, FAKE, FAKE, need, nseq=-1) == SHAPE


def test_backward_checks(lib):
    """The gradient call validates shape, dtypes, required pointers, its
    workspace and alignment before any HIP call; dfinal, initial_states and
    dinitial are optional."""
    s = shape()
    B, L, H, P, N, Q = 2, 512, 4, 64, 128, 256
    need = lib.ssd_backward_workspace_bytes(s)
    # at least: the chunk states of the four passes, fp32
    assert need >= 4 * 4 * B * (L // Q) * H * N * P
    assert lib.ssd_backward_workspace_bytes(None) == 0
    assert lib.ssd_backward_workspace_bytes(shape(batch=0)) == 0
    a = [FAKE] * 6  # x, dt, A, Bm, Cm, D

    def call(sh, in_=1, dy=FAKE, dy_t=1, outs=None, ws=FAKE, wsb=need, h0=None, dfin=None, dinit=None, mma=0):
        o = [FAKE] * 6 if outs is None else outs  # dx, ddt, dA, dB, dC, dD
        return lib.ssd_backward(sh, *a, in_, h0, dy, dy_t, dfin, *o, dinit, ws, wsb, mma, None)

    assert call(s, dy=None) == NULL
    for k in range(6):
        o = [FAKE] * 6
        o[k] = None
        assert call(s, outs=o) == NULL
    assert call(s, ws=None) == WS
    assert call(s, wsb=need - 1) == WS
    assert call(s, in_=7) == DTYPE
    assert call(s, dy_t=7) == DTYPE
    assert call(s, mma=5) == DTYPE
    assert call(s, dy=FAKE + 4) == ALIGN
    assert call(s, dinit=FAKE + 8) == ALIGN
    assert call(s, dfin=FAKE + 2) == ALIGN
    assert call(s, h0=FAKE + 2) == ALIGN
    assert call(shape(headdim=24), wsb=1 << 40) == UNSUP
    assert call(shape(nheads=6, ngroups=4)) == SHAPE


def test_mixed_dtype_state_passing_has_no_in_place_form(lib):
    """Carried states of another element size than the chunk states cannot be
    written over them (the two layouts would race), so those calls are refused
    before any HIP call; the in-place forms with matching dtypes (fp32 -> fp32,
    bf16 -> bf16) stay valid (exercised on the GPU side)."""
    s = shape()
    assert lib.ssd_state_passing(s, FAKE, 0, FAKE, 1, FAKE, None, FAKE, None) == UNSUP
    assert lib.ssd_state_passing(s, FAKE, 1, FAKE, 0, FAKE, None, FAKE, None) == UNSUP


def test_ragged_last_chunk_is_a_valid_shape(lib):
    """seqlen need not be a multiple of chunk: nc = ceil(L / Q) chunks of Q
    positions (the workspace is sized for them; no call is launched here)."""
    B, L, H, P, N, Q = 2, 500, 4, 64, 128, 256
    nc = 2
    bhl = 4 * B * H * nc * Q
    st = 4 * B * nc * H * N * P
    ru = lambda v: (v + 255) // 256 * 256
    assert lib.ssd_workspace_bytes(shape(seqlen=L)) == ru(ru(ru(bhl) + bhl) + st)
    assert lib.ssd_workspace_bytes(shape(seqlen=1)) > 0


def test_workspace(lib):
    s = shape()
    B, L, H, P, N, Q = 2, 512, 4, 64, 128, 256
    nc = L // Q
    bhl = 4 * B * H * nc * Q
    st = 4 * B * nc * H * N * P
    ru = lambda v: (v + 255) // 256 * 256
    expect = ru(ru(ru(bhl) + bhl) + st)  # dA, dt_bhl, one state area sized for fp32
    assert lib.ssd_workspace_bytes(s) == expect
    assert lib.ssd_forward(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, FAKE, 1, FAKE, None, 1 << 40, 0,
                           None) == WS
    # the fp32 path needs all of it, the bf16-operand path half the state area
    need_bf16 = ru(ru(ru(bhl) + bhl) + st // 2)
    for mma, need in ((1, expect), (0, need_bf16)):
        assert lib.ssd_forward(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None, FAKE, 1, FAKE, FAKE, need - 1, mma,
                               None) == WS


def test_binding_refuses_cpu_tensors():
    import torch
    from mamba_ssd_scan_chunk_amd import ops
    s = dict(batch=1, seqlen=64, nheads=2, headdim=16, dstate=16, ngroups=1, chunk=64)
    with pytest.raises(ValueError):
        ops.ssd_chunk_cumsum(s, torch.zeros(1, 64, 2), torch.zeros(2))
