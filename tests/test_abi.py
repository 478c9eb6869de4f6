"""The C-ABI library: it loads without a GPU, exports every function the
header declares, and rejects bad arguments before touching the device."""

import ctypes

import pytest

from chunked_gated_delta_10_amd import kda

F32, BF16, NONE = kda.KDA_STATE_FP32, kda.KDA_STATE_BF16, kda.KDA_STATE_NONE
P = 0x10000  # a fake, 16-byte aligned "device" address: validation fails before any use


@pytest.fixture(scope="module")
def lib():
    return kda.load()


def test_exports_every_declared_function(lib):
    names = kda.header_functions()
    assert set(names) >= {"kda_fwd", "kda_fwd_varlen", "kda_decode_step", "kda_fwd_workspace_bytes",
                          "kda_status_string", "kda_last_error"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in kda.STATUS.items():
        assert lib.kda_status_string(code).decode() == name


def test_workspace_query(lib):
    ws = lib.kda_fwd_workspace_bytes(2, 16384, 16, 16, 0)
    assert ws >= 2 * 256 * 16 * 66048
    assert lib.kda_fwd_workspace_bytes(1, 16384, 16, 16, 20) > 0
    assert lib.kda_fwd_workspace_bytes(2, 100, 16, 16, 20) == 0   # packed needs B == 1
    assert lib.kda_fwd_workspace_bytes(1, 100, 3, 16, 0) == 0     # H % H_qk != 0
    assert lib.kda_fwd_workspace_bytes(-1, 100, 4, 4, 0) == 0


def fwd(lib, **over):
    a = dict(q=P, k=P, v=P, g=P, beta=P, alog=P, scale=0.088, pc=1, s0=None, s0dt=NONE, out=P, s1=P, s1dt=F32,
             B=1, T=64, Hqk=2, H=2, K=128, V=128, ws=P, wsb=1 << 40)
    a.update(over)
    return lib.kda_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["alog"], a["scale"], a["pc"], a["s0"],
                       a["s0dt"], a["out"], a["s1"], a["s1dt"], a["B"], a["T"], a["Hqk"], a["H"], a["K"], a["V"],
                       a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(K=64), 2), (dict(V=256), 2), (dict(H=3), 2), (dict(T=-1), 2), (dict(B=-2), 2), (dict(pc=2), 2),
    (dict(q=None), 1), (dict(g=None), 1), (dict(out=None), 1),
    (dict(v=P + 8), 6), (dict(s1=P + 4), 6),
    (dict(s0=P, s0dt=BF16), 4), (dict(s1dt=7), 3),
    (dict(ws=None), 5), (dict(wsb=1024), 5),
])
def test_fwd_validation(lib, over, code):
    st = fwd(lib, **over)
    assert st == code, (st, lib.kda_last_error())
    assert lib.kda_last_error().decode() != ""


def test_fwd_empty_batch_is_a_noop(lib):
    assert fwd(lib, B=0) == 0
    assert lib.kda_last_error().decode() == ""


def test_varlen_validation(lib):
    def call(cu, N, **kw):
        a = dict(B=1, T=100)
        return lib.kda_fwd_varlen(P, P, P, P, P, P, 0.088, 1, None, NONE, P, P, F32, cu, N, kw.get("T", 100), 2, 2,
                                  kw.get("K", 128), 128, P, 1 << 40, None)
    assert call(None, 3) == 1
    assert call(P, 3, K=96) == 2
    assert call(P + 2, 3) == 6
    assert call(None, 0) == 0  # no sequences: no-op


def test_decode_validation(lib):
    def call(**over):
        a = dict(q=P, k=P, v=P, g=P, beta=P, alog=P, scale=0.088, pc=1, st=P, dt=F32, out=P, B=4, Hqk=2, H=4,
                 K=128, V=128)
        a.update(over)
        return lib.kda_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["alog"], a["scale"], a["pc"],
                                   a["st"], a["dt"], a["out"], a["B"], a["Hqk"], a["H"], a["K"], a["V"], None)
    assert call(K=64) == 2
    assert call(H=3) == 2
    assert call(dt=NONE) == 3
    assert call(st=None) == 1
    assert call(out=P + 2) == 6
    assert call(B=0) == 0


def test_linear_attention_validation(lib):
    def fwd_la(**over):
        a = dict(q=P, k=P, v=P, g=P, alog=P, scale=0.088, pc=0, s0=None, s0dt=NONE, out=P, s1=P, s1dt=F32,
                 B=1, T=64, Hqk=2, H=2, K=128, V=128, ws=P, wsb=1 << 40)
        a.update(over)
        return lib.kda_la_fwd(a["q"], a["k"], a["v"], a["g"], a["alog"], a["scale"], a["pc"], a["s0"], a["s0dt"],
                              a["out"], a["s1"], a["s1dt"], a["B"], a["T"], a["Hqk"], a["H"], a["K"], a["V"],
                              a["ws"], a["wsb"], None)
    assert fwd_la(K=64) == 2
    assert fwd_la(H=3) == 2
    assert fwd_la(q=None) == 1
    assert fwd_la(alog=None) == 1
    assert fwd_la(out=P + 8) == 6
    assert fwd_la(ws=None) == 5
    assert fwd_la(s0=P, s0dt=BF16) == 4
    assert fwd_la(B=0) == 0
    assert lib.kda_la_fwd_varlen(P, P, P, P, P, 0.088, 0, None, NONE, P, P, F32, None, 3, 100, 2, 2, 128, 128, P,
                                 1 << 40, None) == 1
    assert lib.kda_la_fwd_varlen(P, P, P, P, P, 0.088, 0, None, NONE, P, P, F32, P, 3, 100, 2, 2, 96, 128, P,
                                 1 << 40, None) == 2

    def dec(**over):
        a = dict(q=P, k=P, v=P, g=P, alog=P, scale=0.088, pc=0, st=P, dt=F32, out=P, B=4, Hqk=2, H=4, K=128, V=128)
        a.update(over)
        return lib.kda_la_decode_step(a["q"], a["k"], a["v"], a["g"], a["alog"], a["scale"], a["pc"], a["st"],
                                      a["dt"], a["out"], a["B"], a["Hqk"], a["H"], a["K"], a["V"], None)
    assert dec(K=64) == 2
    assert dec(dt=NONE) == 3
    assert dec(st=None) == 1
    assert dec(B=0) == 0


def fwd_noalloc(lib, **over):
    a = dict(q=P, k=P, v=P, g=P, beta=P, alog=P, scale=0.088, pc=1, s0=None, s0dt=NONE, out=P, s1=P, s1dt=F32,
             B=1, T=64, Hqk=2, H=2, K=128, V=128)
    a.update(over)
    return lib.kda_fwd_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], a["alog"], a["scale"], a["pc"], a["s0"],
                               a["s0dt"], a["out"], a["s1"], a["s1dt"], a["B"], a["T"], a["Hqk"], a["H"], a["K"],
                               a["V"], None)


def test_noalloc_scratch_capacity_matches_header():
    with open(kda.HEADER_PATH) as f:
        text = f.read()
    assert "#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert kda.NOALLOC_SCRATCH_BYTES == 64 << 20


@pytest.mark.parametrize("over,code", [
    (dict(K=64), 2), (dict(H=3), 2), (dict(q=None), 1), (dict(out=P + 8), 6), (dict(s1dt=7), 3),
    # scalar gate (two-kernel path, records of every (chunk, head)): 1100 and
    # 4096 records exceed the scratch; rejected before any device work
    (dict(B=1, T=64 * 1100, Hqk=1, H=1, pc=0), 5),
    (dict(B=4, T=4096, Hqk=16, H=16, pc=0), 5),
])
def test_noalloc_validation(lib, over, code):
    # rejected on the host, before the scratch address is looked up or anything is enqueued
    st = fwd_noalloc(lib, **over)
    assert st == code, (st, lib.kda_last_error())
    if code == 5:
        assert b"static scratch" in lib.kda_last_error()


def test_noalloc_zero_batch_is_a_no_op(lib):
    assert fwd_noalloc(lib, B=0) == 0


# ---- backward --------------------------------------------------------------------------------------------------


def test_bwd_workspace_query(lib):
    # per (chunk, head): two fp16 state blocks (32 KiB each) and a 120 KiB operator record (the per-channel
    # gate's; the scalar gate uses 104 KiB of it)
    ws = lib.kda_bwd_workspace_bytes(1, 32768, 32, 32, 8)
    assert ws >= 512 * 32 * (2 * 32768 + 122880)
    assert lib.kda_bwd_workspace_bytes(2, 1000, 4, 4, 0) > 0
    assert lib.kda_bwd_workspace_bytes(2, 100, 4, 4, 3) == 0    # packed needs B == 1
    assert lib.kda_bwd_workspace_bytes(1, 100, 3, 4, 0) == 0    # H % H_qk != 0
    assert lib.kda_bwd_workspace_bytes(1, -5, 4, 4, 0) == 0


def bwd(lib, **over):
    a = dict(q=P, k=P, v=P, g=P, beta=P, alog=P, scale=0.088, pc=0, s0=None, dout=P, dfin=None, dq=P, dk=P, dv=P,
             dg=P, db=P, dal=P, dinit=None, B=1, T=64, Hqk=2, H=2, K=128, V=128, ws=P, wsb=1 << 40)
    a.update(over)
    return lib.kda_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["alog"], a["scale"], a["pc"], a["s0"], a["dout"],
                       a["dfin"], a["dq"], a["dk"], a["dv"], a["dg"], a["db"], a["dal"], a["dinit"], a["B"], a["T"],
                       a["Hqk"], a["H"], a["K"], a["V"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(pc=1, K=64), 2), (dict(K=64), 2), (dict(pc=1, dq=None), 1), (dict(H=3), 2), (dict(T=-1), 2), (dict(B=-1), 2),
    (dict(dout=None), 1), (dict(dq=None), 1), (dict(dv=None), 1), (dict(dal=None), 1), (dict(beta=None), 1),
    (dict(dk=P + 8), 6), (dict(s0=P + 4), 6), (dict(dinit=P + 2), 6), (dict(ws=P + 16), 6),
    (dict(ws=None), 5), (dict(wsb=4096), 5),
])
def test_bwd_validation(lib, over, code):
    st = bwd(lib, **over)
    assert st == code, (st, lib.kda_last_error())
    assert lib.kda_last_error().decode() != ""


def test_bwd_empty_batch_is_a_noop(lib):
    assert bwd(lib, B=0) == 0


def test_bwd_varlen_validation(lib):
    def call(cu, N):
        return lib.kda_bwd_varlen(P, P, P, P, P, P, 0.088, 0, None, P, None, P, P, P, P, P, P, None, cu, N, 100, 2, 2,
                                  128, 128, P, 1 << 40, None)
    assert call(None, 3) == 1
    assert call(P + 2, 3) == 6
    assert call(None, 0) == 0
