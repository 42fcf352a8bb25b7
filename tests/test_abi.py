"""The C ABI on the CPU: the library loads, exports every function include/moe_route.h declares,
and rejects invalid arguments before touching the GPU (no kernel is launched in these tests)."""
import ctypes
import os
import re

import pytest

from combine_moe_route_03_amd import _lib as moe
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe_route.h")

A16 = ctypes.c_void_p(0x10000)          # stand-in device pointers: never dereferenced here
A16b = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10008)          # 8-byte aligned, not 16
S0 = ctypes.c_void_p(0)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_function():
    lib = moe.load()
    names = _declared_functions()
    assert names == sorted(["moe_combine", "moe_dispatch", "moe_dispatch_layout",
                            "moe_dispatch_pack", "moe_dispatch_workspace_bytes",
                            "moe_route_dispatch", "moe_route_dispatch_noalloc",
                            "moe_route_topk", "moe_status_str",
                            "moe_ep_capacity", "moe_ep_send", "moe_ep_recv", "moe_ep_return",
                            "moe_ep_combine", "moe_ep_partial_rows",
                            "moe_ep_reduce_workspace_bytes", "moe_ep_reduce",
                            "moe_ep_combine_reduced", "moe_check_topk"])
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code, word in [(0, "MOE_OK"), (1, "INVALID"), (2, "UNSUPPORTED"), (3, "WORKSPACE"),
                       (4, "HIP")]:
        assert word in moe.moe_status_str(code)
    assert "unknown" in moe.moe_status_str(99)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert f"#define MOE_MAX_EXPERTS {moe.MOE_MAX_EXPERTS}" in text
    assert f"#define MOE_MAX_TOPK {moe.MOE_MAX_TOPK}" in text
    assert "#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)" in text
    assert moe.MOE_NOALLOC_SCRATCH_BYTES == 16 << 20
    for name, val in [("MOE_F32", 0), ("MOE_BF16", 1), ("MOE_FP8_E4M3", 2), ("MOE_OK", 0),
                      ("MOE_ERR_INVALID", 1), ("MOE_ERR_UNSUPPORTED", 2),
                      ("MOE_ERR_WORKSPACE", 3), ("MOE_ERR_HIP", 4)]:
        assert re.search(rf"\b{name} = {val}\b", text), name


def test_route_validation():
    f = moe.load().moe_route_topk
    assert f(A16, 4, 8, 0, A16, A16, S0) == moe.MOE_ERR_INVALID          # k < 1
    assert f(A16, 4, 8, 9, A16, A16, S0) == moe.MOE_ERR_INVALID          # k > E
    assert f(A16, -1, 8, 2, A16, A16, S0) == moe.MOE_ERR_INVALID         # T < 0
    assert f(A16, 4, 0, 1, A16, A16, S0) == moe.MOE_ERR_INVALID          # E < 1
    assert f(None, 4, 8, 2, A16, A16, S0) == moe.MOE_ERR_INVALID         # null logits
    assert f(A16, 4, 8, 2, None, A16, S0) == moe.MOE_ERR_INVALID
    assert f(A16, 4, 8, 2, A16, None, S0) == moe.MOE_ERR_INVALID
    assert f(A16, 4, 2048, 2, A16, A16, S0) == moe.MOE_ERR_UNSUPPORTED   # E > MOE_MAX_EXPERTS
    assert f(A16, 4, 128, 65, A16, A16, S0) == moe.MOE_ERR_UNSUPPORTED   # k > MOE_MAX_TOPK
    assert f(A16, 2 ** 30, 16, 4, A16, A16, S0) == moe.MOE_ERR_INVALID   # T*k >= 2^31
    assert f(None, 0, 8, 2, None, None, S0) == moe.MOE_OK                # T = 0: no-op


def test_workspace_bytes():
    ws = moe.moe_dispatch_workspace_bytes
    assert ws(-1, 8, 2) == 0 and ws(4, 0, 2) == 0 and ws(4, 8, 0) == 0
    assert ws(2 ** 30, 8, 4) == 0
    assert ws(0, 8, 2) > 0
    # two histogram-sized pieces (E u32 per layout block: one block per 16 routed tokens, or per
    # 256 caller-given ids), the E expert totals, one u32 rank and one (row, token) pair per row,
    # in 256-byte aligned pieces
    R = 4096 * 8
    nblk = max(4096 // 16, R // 256)
    lo = R * 4 + R * 8 + 2 * nblk * 384 * 4 + 384 * 4
    assert lo <= ws(4096, 384, 8) <= lo + 8 + 1280
    assert ws(4096, 384, 8) % 256 == 0
    assert ws(128, 256, 8) >= 128 * 8 * 4


def _out_struct(**override):
    s = moe.moe_dispatch_out_t()
    for name, _ in moe.moe_dispatch_out_t._fields_:
        setattr(s, name, 0x30000)
    for k, v in override.items():
        setattr(s, k, v)
    return s


def test_layout_validation():
    f = moe.load().moe_dispatch_layout
    o = _out_struct()
    big = 1 << 30
    assert f(A16, 4, 2, 8, 3, ctypes.byref(o), A16, big, S0) == moe.MOE_ERR_INVALID  # E % N
    assert f(A16, 4, 2, 8, 0, ctypes.byref(o), A16, big, S0) == moe.MOE_ERR_INVALID  # N < 1
    assert f(A16, 4, 0, 8, 2, ctypes.byref(o), A16, big, S0) == moe.MOE_ERR_INVALID  # k < 1
    assert f(A16, 4, 2, 8, 2, None, A16, big, S0) == moe.MOE_ERR_INVALID             # out NULL
    assert f(None, 4, 2, 8, 2, ctypes.byref(o), A16, big, S0) == moe.MOE_ERR_INVALID
    for field in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets",
                  "token_row", "row_token"):
        o2 = _out_struct(**{field: None})
        assert f(A16, 4, 2, 8, 2, ctypes.byref(o2), A16, big, S0) == moe.MOE_ERR_INVALID, field
    assert f(A16, 4, 2, 2048, 2, ctypes.byref(o), A16, big, S0) == moe.MOE_ERR_UNSUPPORTED
    need = moe.moe_dispatch_workspace_bytes(4, 8, 2)
    assert f(A16, 4, 2, 8, 2, ctypes.byref(o), A16, need - 1, S0) == moe.MOE_ERR_WORKSPACE
    assert f(A16, 4, 2, 8, 2, ctypes.byref(o), None, need, S0) == moe.MOE_ERR_WORKSPACE
    assert f(A16, 4, 2, 8, 2, ctypes.byref(o), MIS, need, S0) == moe.MOE_ERR_UNSUPPORTED


def test_pack_validation():
    f = moe.load().moe_dispatch_pack
    F32, BF16, FP8 = moe.MOE_F32, moe.MOE_BF16, moe.MOE_FP8_E4M3
    assert f(A16, FP8, 4, 256, 2, A16, FP8, A16b, A16, S0) == moe.MOE_ERR_UNSUPPORTED   # x fp8
    assert f(A16, BF16, 4, 256, 2, A16, F32, A16b, None, S0) == moe.MOE_ERR_UNSUPPORTED  # widen
    assert f(A16, BF16, 4, 192, 2, A16, FP8, A16b, A16, S0) == moe.MOE_ERR_UNSUPPORTED   # H%128
    assert f(A16, BF16, 4, 256, 2, A16, FP8, A16b, None, S0) == moe.MOE_ERR_INVALID      # scales
    assert f(A16, BF16, 4, 260, 2, A16, BF16, A16b, None, S0) == moe.MOE_ERR_UNSUPPORTED  # 16 B
    assert f(MIS, BF16, 4, 256, 2, A16, BF16, A16b, None, S0) == moe.MOE_ERR_UNSUPPORTED
    assert f(A16, BF16, 4, 256, 2, A16, BF16, MIS, None, S0) == moe.MOE_ERR_UNSUPPORTED
    assert f(None, BF16, 4, 256, 2, A16, BF16, A16b, None, S0) == moe.MOE_ERR_INVALID
    assert f(A16, BF16, 4, 256, 2, None, BF16, A16b, None, S0) == moe.MOE_ERR_INVALID
    assert f(A16, BF16, -1, 256, 2, A16, BF16, A16b, None, S0) == moe.MOE_ERR_INVALID
    assert f(A16, BF16, 4, 0, 2, A16, BF16, A16b, None, S0) == moe.MOE_ERR_INVALID
    assert f(None, BF16, 0, 256, 2, None, BF16, None, None, S0) == moe.MOE_OK            # T = 0


def test_dispatch_validation_checks_both_halves():
    f = moe.load().moe_dispatch
    o = _out_struct()
    BF16, FP8 = moe.MOE_BF16, moe.MOE_FP8_E4M3
    need = moe.moe_dispatch_workspace_bytes(4, 8, 2)
    assert f(A16, BF16, 4, 256, A16, 2, 8, 3, BF16, ctypes.byref(o), A16, need,
             S0) == moe.MOE_ERR_INVALID                                           # E % N
    o2 = _out_struct(recv_scales=None)
    assert f(A16, BF16, 4, 256, A16, 2, 8, 2, FP8, ctypes.byref(o2), A16, need,
             S0) == moe.MOE_ERR_INVALID                                           # scales
    o3 = _out_struct(recv=0x30008)
    assert f(A16, BF16, 4, 256, A16, 2, 8, 2, BF16, ctypes.byref(o3), A16, need,
             S0) == moe.MOE_ERR_UNSUPPORTED                                       # recv align
    assert f(A16, BF16, 4, 256, A16, 2, 8, 2, BF16, ctypes.byref(o), A16, need - 4,
             S0) == moe.MOE_ERR_WORKSPACE


def test_route_dispatch_validation_checks_every_part():
    f = moe.load().moe_route_dispatch
    o = _out_struct()
    BF16, FP8 = moe.MOE_BF16, moe.MOE_FP8_E4M3
    need = moe.moe_dispatch_workspace_bytes(4, 8, 2)
    args = dict(logits=A16, x=A16, xd=BF16, T=4, H=256, E=8, k=2, N=2, pd=BF16, idx=A16b,
                w=A16b, out=ctypes.byref(o), ws=A16, wsb=need)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["logits"], a["x"], a["xd"], a["T"], a["H"], a["E"], a["k"], a["N"], a["pd"],
                 a["idx"], a["w"], a["out"], a["ws"], a["wsb"], S0)

    assert call(k=9) == moe.MOE_ERR_INVALID                      # k > E
    assert call(logits=None) == moe.MOE_ERR_INVALID
    assert call(idx=None) == moe.MOE_ERR_INVALID
    assert call(w=None) == moe.MOE_ERR_INVALID
    assert call(E=2048) == moe.MOE_ERR_UNSUPPORTED
    assert call(N=3) == moe.MOE_ERR_INVALID                      # E % N
    assert call(out=None) == moe.MOE_ERR_INVALID
    assert call(x=MIS) == moe.MOE_ERR_UNSUPPORTED
    assert call(H=192, pd=FP8) == moe.MOE_ERR_UNSUPPORTED        # H % 128 for fp8
    o2 = _out_struct(recv_scales=None)
    assert call(pd=FP8, out=ctypes.byref(o2)) == moe.MOE_ERR_INVALID
    assert call(wsb=need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(ws=None) == moe.MOE_ERR_WORKSPACE
    assert call(ws=MIS) == moe.MOE_ERR_UNSUPPORTED


def test_layout_calls_reject_k_beyond_max_topk():
    """A token's slots are handled by one wavefront in the one-launch layout, so every call that
    lays out caller-given ids rejects k > MOE_MAX_TOPK before any launch (T = 8, E = 128)."""
    lib = moe.load()
    BF16 = moe.MOE_BF16
    o = _out_struct()
    T, E, N = 8, 128, 2
    for k in (moe.MOE_MAX_TOPK + 1, 80):
        need = moe.moe_dispatch_workspace_bytes(T, E, k)
        assert need > 0
        assert lib.moe_dispatch_layout(A16, T, k, E, N, ctypes.byref(o), A16, need, S0) == \
            moe.MOE_ERR_UNSUPPORTED
        assert lib.moe_dispatch(A16, BF16, T, 256, A16, k, E, N, BF16, ctypes.byref(o), A16,
                                need, S0) == moe.MOE_ERR_UNSUPPORTED
        assert lib.moe_route_dispatch(A16, A16, BF16, T, 256, E, k, N, BF16, A16b, A16b,
                                      ctypes.byref(o), A16, need, S0) == moe.MOE_ERR_UNSUPPORTED
        cap = lib.moe_ep_capacity(T, E, k, N)
        assert lib.moe_ep_send(A16, BF16, T, 256, A16, k, E, N, 0, 1, cap, A16b, A16, A16,
                               A16, need, S0) == moe.MOE_ERR_UNSUPPORTED
    # k = MOE_MAX_TOPK stays accepted up to the workspace check
    k = moe.MOE_MAX_TOPK
    need = moe.moe_dispatch_workspace_bytes(T, E, k)
    assert lib.moe_dispatch_layout(A16, T, k, E, N, ctypes.byref(o), A16, need - 1, S0) == \
        moe.MOE_ERR_WORKSPACE


def test_route_dispatch_noalloc_validation():
    """Argument errors are those of moe_route_dispatch, and a batch whose workspace exceeds the
    fixed scratch is rejected, all before any device call (none is possible here)."""
    f = moe.load().moe_route_dispatch_noalloc
    o = _out_struct()
    BF16, FP8 = moe.MOE_BF16, moe.MOE_FP8_E4M3
    args = dict(logits=A16, x=A16, xd=BF16, T=4, H=256, E=8, k=2, N=2, pd=BF16, idx=A16b,
                w=A16b, out=ctypes.byref(o))

    def call(**kw):
        a = dict(args, **kw)
        return f(a["logits"], a["x"], a["xd"], a["T"], a["H"], a["E"], a["k"], a["N"], a["pd"],
                 a["idx"], a["w"], a["out"], S0)

    assert call(k=9) == moe.MOE_ERR_INVALID                      # k > E
    assert call(logits=None) == moe.MOE_ERR_INVALID
    assert call(E=2048) == moe.MOE_ERR_UNSUPPORTED
    assert call(N=3) == moe.MOE_ERR_INVALID                      # E % N
    assert call(out=None) == moe.MOE_ERR_INVALID
    assert call(x=MIS) == moe.MOE_ERR_UNSUPPORTED
    assert call(H=192, pd=FP8) == moe.MOE_ERR_UNSUPPORTED
    assert call(k=65, E=128) == moe.MOE_ERR_UNSUPPORTED
    # the largest batches: beyond MOE_NOALLOC_SCRATCH_BYTES of workspace
    T, E, k = 65536, 1024, 16
    assert moe.moe_dispatch_workspace_bytes(T, E, k) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert call(T=T, E=E, k=k, N=8, H=128) == moe.MOE_ERR_WORKSPACE
    assert moe.moe_dispatch_workspace_bytes(4096, 384, 8) <= moe.MOE_NOALLOC_SCRATCH_BYTES


def test_ep_capacity_and_validation():
    lib = moe.load()
    assert lib.moe_ep_capacity(512, 384, 8, 8) == 512 * 8
    assert lib.moe_ep_capacity(10, 8, 2, 8) == 10 * 1              # one expert per rank
    assert lib.moe_ep_capacity(10, 8, 2, 3) == 0                   # E % N
    F32, BF16, FP8 = moe.MOE_F32, moe.MOE_BF16, moe.MOE_FP8_E4M3
    need = moe.moe_dispatch_workspace_bytes(10, 8, 2)
    send = lib.moe_ep_send
    ok = dict(x=A16, xd=F32, T=10, H=256, idx=A16, k=2, E=8, N=4, src=1, S=3, cap=20, reg=A16b,
              cnt=A16, row=A16, ws=A16, wsb=need)

    def call(**kw):
        a = dict(ok, **kw)
        return send(a["x"], a["xd"], a["T"], a["H"], a["idx"], a["k"], a["E"], a["N"], a["src"],
                    a["S"], a["cap"], a["reg"], a["cnt"], a["row"], a["ws"], a["wsb"], S0)

    assert call(cap=19) == moe.MOE_ERR_INVALID                       # below the worst case
    assert call(src=3) == moe.MOE_ERR_INVALID                        # source >= S
    assert call(src=-1) == moe.MOE_ERR_INVALID
    assert call(N=3) == moe.MOE_ERR_INVALID                          # E % N
    assert call(cnt=None) == moe.MOE_ERR_INVALID
    assert call(row=None) == moe.MOE_ERR_INVALID
    assert call(xd=FP8) == moe.MOE_ERR_UNSUPPORTED
    assert call(reg=MIS) == moe.MOE_ERR_UNSUPPORTED
    assert call(wsb=need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(S=2 ** 16, cap=2 ** 16) == moe.MOE_ERR_INVALID       # N*S*cap >= 2^31
    recv = lib.moe_ep_recv
    assert recv(A16, BF16, 256, 8, 4, 4, 3, 20, A16, A16b, A16, A16, A16, S0) == \
        moe.MOE_ERR_INVALID                                          # rank >= N
    assert recv(A16, FP8, 256, 8, 4, 0, 3, 20, A16, A16b, A16, A16, A16, S0) == \
        moe.MOE_ERR_UNSUPPORTED
    assert recv(A16, BF16, 256, 1024, 1, 0, 8, 20, A16, A16b, A16, A16, A16, S0) == \
        moe.MOE_ERR_UNSUPPORTED                                      # S*L > 4096
    assert recv(A16, BF16, 256, 8, 4, 0, 3, 20, None, A16b, A16, A16, A16, S0) == \
        moe.MOE_ERR_INVALID
    ret = lib.moe_ep_return
    assert ret(A16, BF16, 256, 8, 4, 3, 20, None, A16, A16b, S0) == moe.MOE_ERR_INVALID
    assert ret(MIS, BF16, 256, 8, 4, 3, 20, A16, A16, A16b, S0) == moe.MOE_ERR_UNSUPPORTED
    comb = lib.moe_ep_combine
    assert comb(A16, BF16, 4, 256, 2, A16, A16, -1, A16b, BF16, S0) == moe.MOE_ERR_INVALID
    assert comb(None, BF16, 0, 256, 2, None, None, 0, None, BF16, S0) == moe.MOE_OK


def test_ep_reduce_validation():
    lib = moe.load()
    BF16, FP8 = moe.MOE_BF16, moe.MOE_FP8_E4M3
    pr = lib.moe_ep_partial_rows
    assert pr(A16, 10, 2, 8, 4, 0, 3, 9, A16, A16, S0) == moe.MOE_ERR_INVALID      # pcap < T
    assert pr(A16, 10, 2, 8, 4, 3, 3, 10, A16, A16, S0) == moe.MOE_ERR_INVALID     # source >= S
    assert pr(A16, 10, 2, 8, 4, 0, 3, 10, A16, None, S0) == moe.MOE_ERR_INVALID
    assert lib.moe_ep_reduce_workspace_bytes(3, 20) >= 3 * 20 * 4
    assert lib.moe_ep_reduce_workspace_bytes(0, 20) == 0
    red = lib.moe_ep_reduce
    need = lib.moe_ep_reduce_workspace_bytes(3, 20)
    ok = dict(y=A16, dt=BF16, H=256, E=8, N=4, rank=1, S=3, cap=20, gs=A16, T=10, k=2, idx=A16,
              w=A16, row=A16, prow=A16, pcap=10, part=A16b, ws=A16, wsb=need)

    def call(**kw):
        a = dict(ok, **kw)
        return red(a["y"], a["dt"], a["H"], a["E"], a["N"], a["rank"], a["S"], a["cap"], a["gs"],
                   a["T"], a["k"], a["idx"], a["w"], a["row"], a["prow"], a["pcap"], a["part"],
                   a["ws"], a["wsb"], S0)

    assert call(rank=4) == moe.MOE_ERR_INVALID
    assert call(pcap=9) == moe.MOE_ERR_INVALID
    assert call(dt=FP8) == moe.MOE_ERR_UNSUPPORTED
    assert call(H=260) == moe.MOE_ERR_UNSUPPORTED                    # rows of 16 bytes, H % 8
    assert call(part=MIS) == moe.MOE_ERR_UNSUPPORTED
    assert call(gs=None) == moe.MOE_ERR_INVALID
    assert call(wsb=need - 4) == moe.MOE_ERR_WORKSPACE
    fin = lib.moe_ep_combine_reduced
    assert fin(A16, BF16, 4, 256, 4, A16, -1, A16b, BF16, S0) == moe.MOE_ERR_INVALID
    assert fin(A16, FP8, 4, 256, 4, A16, 8, A16b, BF16, S0) == moe.MOE_ERR_UNSUPPORTED
    assert fin(A16, BF16, 4, 252, 4, A16, 8, A16b, BF16, S0) == moe.MOE_ERR_UNSUPPORTED
    assert fin(None, BF16, 0, 256, 4, None, 0, None, BF16, S0) == moe.MOE_OK


def test_combine_validation():
    f = moe.load().moe_combine
    F32, BF16, FP8 = moe.MOE_F32, moe.MOE_BF16, moe.MOE_FP8_E4M3
    assert f(A16, FP8, 4, 256, 2, A16, A16, A16b, BF16, S0) == moe.MOE_ERR_UNSUPPORTED
    assert f(A16, BF16, 4, 256, 2, A16, A16, A16b, FP8, S0) == moe.MOE_ERR_UNSUPPORTED
    assert f(A16, BF16, 4, 252, 2, A16, A16, A16b, BF16, S0) == moe.MOE_ERR_UNSUPPORTED  # H%8
    assert f(MIS, BF16, 4, 256, 2, A16, A16, A16b, BF16, S0) == moe.MOE_ERR_UNSUPPORTED
    assert f(A16, F32, 4, 256, 2, A16, A16, MIS, F32, S0) == moe.MOE_ERR_UNSUPPORTED
    assert f(A16, BF16, 4, 256, 2, None, A16, A16b, BF16, S0) == moe.MOE_ERR_INVALID
    assert f(A16, BF16, 4, 256, 2, A16, None, A16b, BF16, S0) == moe.MOE_ERR_INVALID
    assert f(A16, BF16, 4, 256, 0, A16, A16, A16b, BF16, S0) == moe.MOE_ERR_INVALID
    assert f(None, BF16, 0, 256, 2, None, None, None, BF16, S0) == moe.MOE_OK


def test_check_topk_validation():
    f = moe.load().moe_check_topk
    I = moe.MOE_ERR_INVALID
    assert f(A16, 4, 0, 8, A16b, S0) == I           # k < 1
    assert f(A16, 4, 2, 0, A16b, S0) == I           # E < 1
    assert f(A16, -1, 2, 8, A16b, S0) == I          # T < 0
    assert f(A16, 4, 2, 8, None, S0) == I           # no counts
    assert f(None, 4, 2, 8, A16b, S0) == I          # no ids
    assert f(A16, 2**30, 4, 8, A16b, S0) == I       # T * k > INT32_MAX


def test_product_path_does_not_reference_the_oracle():
    """The HIP source and binding never name the oracle; the oracle never names the HIP path."""
    pkg = os.path.join(ROOT, "combine_moe_route_03_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "oracle_" not in text, fn
    for fn in os.listdir(os.path.join(ROOT, "oracle")):
        if fn.endswith((".py", ".c")):
            text = open(os.path.join(ROOT, "oracle", fn)).read()
            assert "combine_moe_route_03_amd" not in text and "moe_route.h" not in text, fn


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", "/nonexistent/libmoe_route.so")
    with pytest.raises(ImportError):
        moe.load()
