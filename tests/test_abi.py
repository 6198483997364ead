"""C-ABI checks that need no GPU: the library loads, exports every function
that include/relation.h declares, and rejects bad arguments on the host
before launching anything (every call below fails validation, so no kernel
is launched)."""
import ctypes
import os
import re

import pytest

import exchange_relation_amd as rel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "relation.h")

REL_OK, REL_ERR_NULL, REL_ERR_SHAPE, REL_ERR_UNSUPPORTED, REL_ERR_PARAM = 0, 1, 2, 3, 4
REL_ERR_CAPACITY, REL_ERR_ALIGN, REL_ERR_WORKSPACE, REL_ERR_HIP, REL_ERR_SCRATCH = 5, 6, 7, 8, 9
F32, BF16 = 0, 1

# Fake device addresses: validation never dereferences them, and every call
# below returns an error before any launch.
P = ctypes.c_void_p(0x7F0000000000)
P_MIS = ctypes.c_void_p(0x7F0000000004)  # 4-byte aligned only
NUL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(relation_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rel.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    return rel.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(rel.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    for s in range(10):
        assert rel.relation_status_string(s)
    assert rel.relation_status_string(99) == "unknown status"
    assert rel.relation_version() == 100


def fwd(lib, dtype=BF16, B=1, H=1, T=8, D=64, q=P, k=P, v=P, y=P, lse=NUL, gate=NUL,
        scale=0.125, tau=2.0, lam=0.5, ws=NUL, wsb=0, lam_dev=NUL):
    return lib.relation_fwd(dtype, B, H, T, D, q, k, v, y, lse, gate, ws, wsb, scale, tau, lam,
                            lam_dev, None)


def test_fwd_split_workspace(lib):
    # a grid that fills the GPU on its own (30M layer) needs none, nor one
    # whose blocks have under 17 historical tiles (the 10M layer: pieces of
    # at least 16 tiles); 4 heads of 8192 tokens split: 64 blocks per head,
    # pieces of 16 tiles, up to 8 per block (126 historical tiles), 128 rows
    # x (64 + 4) fp32 per piece and block
    assert lib.relation_fwd_workspace_bytes(BF16, 16, 8, 2048, 64) == 0
    assert lib.relation_fwd_workspace_bytes(BF16, 8, 8, 1024, 64) == 0
    need = lib.relation_fwd_workspace_bytes(BF16, 1, 4, 8192, 64)
    assert need == 4 * 64 * 8 * 128 * 68 * 4
    assert lib.relation_fwd_workspace_bytes(F32, 1, 4, 8192, 64) == 0
    assert lib.relation_fwd_workspace_bytes(BF16, 1, 4, 8192, 96) == 0
    assert lib.relation_fwd_workspace_bytes(BF16, 0, 4, 8192, 64) == 0
    assert lib.relation_fwd_workspace_bytes(BF16, 1, 2, 300, 64) == 0
    assert fwd(lib, B=1, H=4, T=8192, ws=P, wsb=need - 1) == REL_ERR_WORKSPACE
    assert fwd(lib, B=1, H=4, T=8192, ws=P_MIS, wsb=need) == REL_ERR_ALIGN


def test_fwd_validation(lib):
    assert fwd(lib, q=NUL) == REL_ERR_NULL
    assert fwd(lib, y=NUL) == REL_ERR_NULL
    assert fwd(lib, T=0) == REL_ERR_SHAPE
    assert fwd(lib, B=-1) == REL_ERR_SHAPE
    # one head's rows are indexed with 32-bit offsets: T * D < 2^31
    assert fwd(lib, T=(1 << 25), D=64) == REL_ERR_SHAPE
    assert fwd(lib, T=(1 << 25) - 1, D=64, q=NUL) == REL_ERR_NULL  # the shape itself passes
    assert fwd(lib, dtype=F32, D=48) == REL_ERR_UNSUPPORTED
    assert fwd(lib, dtype=BF16, D=32) == REL_ERR_UNSUPPORTED
    assert fwd(lib, dtype=BF16, D=96) == REL_ERR_UNSUPPORTED
    assert fwd(lib, dtype=7) == REL_ERR_UNSUPPORTED
    assert fwd(lib, tau=0.0) == REL_ERR_PARAM
    assert fwd(lib, tau=-1.0) == REL_ERR_PARAM
    assert fwd(lib, lam=float("nan")) == REL_ERR_PARAM
    assert fwd(lib, scale=float("inf")) == REL_ERR_PARAM
    assert fwd(lib, q=P_MIS) == REL_ERR_ALIGN
    assert fwd(lib, lse=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN
    assert fwd(lib, lam_dev=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN  # device lambda
    assert fwd(lib, lam=float("nan"), lam_dev=P) == REL_ERR_PARAM  # still checked when unused


def test_bwd_validation_and_workspace(lib):
    need = lib.relation_bwd_workspace_bytes(BF16, 2, 3, 100, 64)
    # Dr + dlambda partials + fp32 dq accumulator, each 256-byte padded
    assert need >= 2 * 3 * 100 * 4 + 2 * 3 * 100 * 64 * 4
    assert lib.relation_bwd_workspace_bytes(F32, 2, 3, 100, 64) < need
    assert lib.relation_bwd_workspace_bytes(BF16, 2, 3, 100, 48) > 0
    assert lib.relation_bwd_workspace_bytes(BF16, 2, 3, 100, 80) > 0
    assert lib.relation_bwd_workspace_bytes(BF16, 2, 3, 100, 96) == 0

    def bwd(ws=P, wsb=None, dq=P, lse=P, tau=2.0, T=100, lam_dev=NUL):
        wsb = need if wsb is None else wsb
        return lib.relation_bwd(BF16, 2, 3, T, 64, P, P, P, P, P, lse, dq, P, P, NUL, ws, wsb,
                                0.125, tau, 0.3, lam_dev, None)

    assert bwd(lam_dev=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN  # device lambda

    assert bwd(dq=NUL) == REL_ERR_NULL
    assert bwd(lse=NUL) == REL_ERR_NULL
    assert bwd(ws=NUL) == REL_ERR_WORKSPACE
    assert bwd(wsb=need - 1) == REL_ERR_WORKSPACE
    assert bwd(ws=ctypes.c_void_p(0x7F0000000010)) == REL_ERR_ALIGN
    assert bwd(tau=0.0) == REL_ERR_PARAM
    assert bwd(T=0) == REL_ERR_SHAPE

    # relation_bwd_events validates exactly as relation_bwd (the events are
    # only recorded around a launch, which none of these calls reaches)
    def bwd_ev(ws=P, wsb=None, dq=P, lse=P, tau=2.0, T=100, ev=P):
        wsb = need if wsb is None else wsb
        return lib.relation_bwd_events(BF16, 2, 3, T, 64, P, P, P, P, P, lse, dq, P, P, NUL, ws,
                                       wsb, 0.125, tau, 0.3, NUL, None, ev, ev)

    assert bwd_ev(dq=NUL) == REL_ERR_NULL
    assert bwd_ev(ws=NUL) == REL_ERR_WORKSPACE
    assert bwd_ev(wsb=need - 1) == REL_ERR_WORKSPACE
    assert bwd_ev(ws=ctypes.c_void_p(0x7F0000000010)) == REL_ERR_ALIGN
    assert bwd_ev(tau=0.0) == REL_ERR_PARAM
    assert bwd_ev(T=0, ev=NUL) == REL_ERR_SHAPE


def test_decode_validation(lib):
    need = lib.relation_decode_workspace_bytes(BF16, 2, 3, 64, 4352)
    # one partial (m, l, z[64]) per chunk of about 256 slots (17 for 4352) and head
    assert need == 2 * 3 * 17 * 66 * 4

    def dec(n=10, cap=4352, ws=P, wsb=None, q=P, D=64, dtype=BF16):
        wsb = need if wsb is None else wsb
        return lib.relation_cache_decode(dtype, 2, 3, D, q, P, P, P, P, cap, n, P, NUL, ws, wsb,
                                         0.125, 2.0, 0.3, None)

    assert dec(n=4352) == REL_ERR_CAPACITY      # n_hist + 1 > capacity
    assert dec(n=-1) == REL_ERR_CAPACITY
    assert dec(q=NUL) == REL_ERR_NULL
    assert dec(ws=NUL) == REL_ERR_WORKSPACE
    assert dec(wsb=need - 4) == REL_ERR_WORKSPACE
    assert dec(D=32) == REL_ERR_UNSUPPORTED
    assert dec(cap=0, n=0) == REL_ERR_SHAPE
    assert dec(cap=(1 << 25), n=10) == REL_ERR_SHAPE  # capacity * D >= 2^31
    assert dec(q=P_MIS) == REL_ERR_ALIGN


def test_decode_noalloc_validation(lib):
    """The allocation-free decode validates like relation_cache_decode and
    rejects a call whose workspace would exceed its 8 MiB static scratch (all
    on the host: nothing is launched)."""
    def dec(B=2, H=3, n=10, cap=4352, q=P, D=64, dtype=BF16, y=P):
        return lib.relation_cache_decode_noalloc(dtype, B, H, D, q, P, P, P, P, cap, n, y, NUL,
                                                 0.125, 2.0, 0.3, None)

    assert dec(n=4352) == REL_ERR_CAPACITY
    assert dec(n=-1) == REL_ERR_CAPACITY
    assert dec(q=NUL) == REL_ERR_NULL
    assert dec(y=NUL) == REL_ERR_NULL
    assert dec(D=32) == REL_ERR_UNSUPPORTED
    assert dec(q=P_MIS) == REL_ERR_ALIGN
    # the scratch holds what the step uses: one partial per head and 256-slot
    # chunk below 256 heads. 1 x 100 heads at history 199999: 782 chunks,
    # 100 * 782 * 66 * 4 B = 19.7 MiB > 8 MiB (rejected before any launch)
    assert dec(B=1, H=100, n=199999, cap=200000) == REL_ERR_SCRATCH
    assert dec(B=1, H=100, n=199999, cap=200000, q=NUL) == REL_ERR_NULL
    assert "scratch" in rel.relation_status_string(REL_ERR_SCRATCH)


def test_decode_ragged_validation(lib):
    need = lib.relation_decode_workspace_bytes(BF16, 2, 3, 64, 4352)

    def dec(bound=10, cap=4352, ws=P, wsb=None, q=P, nh=P, D=64):
        wsb = need if wsb is None else wsb
        return lib.relation_cache_decode_ragged(BF16, 2, 3, D, q, P, P, P, P, cap, nh, bound, P,
                                                NUL, ws, wsb, 0.125, 2.0, 0.3, None)

    assert dec(bound=4352) == REL_ERR_CAPACITY  # bound + 1 > capacity
    assert dec(bound=-1) == REL_ERR_CAPACITY
    assert dec(nh=NUL) == REL_ERR_NULL
    assert dec(nh=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN
    assert dec(ws=NUL) == REL_ERR_WORKSPACE
    assert dec(D=32) == REL_ERR_UNSUPPORTED


def test_prefill_validation(lib):
    def pf(m=16, n=10, cap=64, dtype=BF16, D=64, q=P, nh=NUL):
        return lib.relation_cache_prefill(dtype, 2, 3, D, m, q, P, P, P, P, cap, nh, n, P, NUL,
                                          NUL, ws, wsb, 0.125, 2.0, 0.3, None)

    ws, wsb = NUL, 0
    # the ragged-history workload (32 x 12 heads, 256 new tokens, bound 4096)
    # splits; a short history does not
    big = lib.relation_prefill_workspace_bytes(BF16, 32, 12, 64, 256, 4096, 1)
    assert big > 0 and big % (128 * 68 * 4) == 0
    assert lib.relation_prefill_workspace_bytes(BF16, 2, 3, 64, 16, 10, 0) == 0
    assert lib.relation_prefill_workspace_bytes(F32, 32, 12, 64, 256, 4096, 1) == 0
    assert lib.relation_prefill_workspace_bytes(BF16, 32, 12, 64, 256, -1, 1) == 0
    need = lib.relation_prefill_workspace_bytes(BF16, 2, 3, 64, 16, 3000, 0)
    assert need > 0
    ws, wsb = P, need - 1
    assert pf(n=3000, cap=4096) == REL_ERR_WORKSPACE
    ws, wsb = P_MIS, need
    assert pf(n=3000, cap=4096) == REL_ERR_ALIGN
    ws, wsb = NUL, 0

    assert pf(n=49) == REL_ERR_CAPACITY   # 49 + 16 > 64
    assert pf(n=-1) == REL_ERR_CAPACITY
    assert pf(m=0) == REL_ERR_SHAPE
    assert pf(dtype=F32) == REL_ERR_UNSUPPORTED
    assert pf(D=32) == REL_ERR_UNSUPPORTED
    assert pf(q=NUL) == REL_ERR_NULL
    assert pf(q=P_MIS) == REL_ERR_ALIGN
    assert pf(nh=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN


def test_mhr_validation(lib):
    n = 2 * 4 * 128 * 64
    # bf16: rotated keys + mixed values (queries are rotated in registers);
    # fp32: queries too
    assert lib.relation_mhr_fwd_workspace_bytes(BF16, 2, 4, 128, 64) == 2 * n * 2
    assert lib.relation_mhr_fwd_workspace_bytes(F32, 2, 4, 128, 64) == 3 * n * 4
    need = lib.relation_mhr_bwd_workspace_bytes(BF16, 2, 4, 128, 64)
    assert need > lib.relation_bwd_workspace_bytes(BF16, 2, 4, 128, 64)

    def fwd(H=4, cs=P, sn=P, th=P, pairing=0, dtype=BF16, ws=NUL, wsb=0, lam_dev=NUL):
        return lib.relation_mhr_fwd(dtype, 2, H, 128, 64, P, P, P, cs, sn, th, pairing, P, NUL,
                                    NUL, ws, wsb, 0.125, 2.0, 0.3, lam_dev, None)

    assert fwd(lam_dev=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN

    assert fwd(cs=NUL) == REL_ERR_NULL               # tables go together
    assert fwd(H=5) == REL_ERR_SHAPE                 # Givens pairs need even H
    assert fwd(pairing=2) == REL_ERR_PARAM
    assert fwd(th=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN
    assert fwd(cs=P_MIS) == REL_ERR_ALIGN
    assert fwd() == REL_ERR_WORKSPACE                # keys / values go through a workspace

    def bwd(ws=P, wsb=None, fws=NUL):
        wsb = need if wsb is None else wsb
        return lib.relation_mhr_bwd(BF16, 2, 4, 128, 64, P, P, P, P, P, P, 0, P, P, P, P, P, P,
                                    NUL, NUL, fws, ws, wsb, 0.125, 2.0, 0.3, NUL, None)

    assert bwd(wsb=need - 256) == REL_ERR_WORKSPACE
    assert bwd(ws=NUL) == REL_ERR_WORKSPACE
    assert bwd(fws=P_MIS) == REL_ERR_ALIGN  # the forward's workspace, when given


def test_linear_validation(lib):
    def lfwd(dtype=BF16, B=1, H=1, T=8, D=64, p1=P, g=P, y=P, rc=NUL, rs=NUL, cin=NUL,
             cout=NUL, states=NUL, scale=0.125, tau=2.0):
        return lib.relation_linear_fwd(dtype, B, H, T, D, p1, P, P, g, rc, rs, cin, y, cout,
                                       states, scale, tau, None)

    assert lfwd(p1=NUL) == REL_ERR_NULL
    assert lfwd(g=NUL) == REL_ERR_NULL
    assert lfwd(y=NUL) == REL_ERR_NULL
    assert lfwd(rc=P) == REL_ERR_NULL  # one table alone
    assert lfwd(dtype=F32) == REL_ERR_UNSUPPORTED
    assert lfwd(D=48) == REL_ERR_UNSUPPORTED
    assert lfwd(T=0) == REL_ERR_SHAPE
    assert lfwd(tau=0.0) == REL_ERR_PARAM
    assert lfwd(scale=float("nan")) == REL_ERR_PARAM
    assert lfwd(p1=P_MIS) == REL_ERR_ALIGN
    assert lfwd(g=P_MIS) == REL_ERR_ALIGN
    assert lfwd(rc=P_MIS, rs=P) == REL_ERR_ALIGN
    assert lfwd(cout=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN
    assert lfwd(states=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN
    assert lfwd(states=P_MIS) == REL_ERR_ALIGN  # read back with 16-byte loads

    need = lib.relation_linear_bwd_workspace_bytes(BF16, 2, 3, 300, 64)
    # the state before every 128-token chunk and the final one, then the
    # gradient of the state after every chunk
    assert need == 2 * 3 * (2 * 3 + 1) * 64 * 64 * 4
    assert lib.relation_linear_bwd_workspace_bytes(F32, 2, 3, 300, 64) == 0
    assert lib.relation_linear_bwd_workspace_bytes(BF16, 2, 3, 300, 48) == 0
    # with the forward's states: the state gradients only
    need_r = lib.relation_linear_bwd_reuse_workspace_bytes(BF16, 2, 3, 300, 64)
    assert need_r == 2 * 3 * 3 * 64 * 64 * 4
    assert lib.relation_linear_bwd_reuse_workspace_bytes(F32, 2, 3, 300, 64) == 0
    # the states the forward stores: before each of the 3 chunks, then the final one
    assert lib.relation_linear_states_bytes(BF16, 2, 3, 300, 64) == 2 * 3 * 4 * 64 * 64 * 4
    assert lib.relation_linear_states_bytes(BF16, 2, 3, 256, 64) == 2 * 3 * 3 * 64 * 64 * 4
    assert lib.relation_linear_states_bytes(BF16, 2, 3, 0, 64) == 0
    assert lib.relation_linear_states_bytes(BF16, 2, 3, 300, 80) == 0
    assert rel.linear_states_shape(2, 3, 300) == (2, 3, 4, 64, 64)

    def lbwd(dtype=BF16, D=64, dy=P, dg=P, ws=P, wsb=need, dsin=NUL, fst=NUL, tau=2.0):
        return lib.relation_linear_bwd(dtype, 2, 3, 300, D, P, P, P, P, NUL, NUL, NUL, dy, NUL,
                                       P, P, P, dg, dsin, fst, ws, wsb, 0.125, tau, None)

    assert lbwd(dy=NUL) == REL_ERR_NULL
    assert lbwd(dg=NUL) == REL_ERR_NULL
    assert lbwd(dtype=F32) == REL_ERR_UNSUPPORTED
    assert lbwd(D=80) == REL_ERR_UNSUPPORTED
    assert lbwd(tau=0.0) == REL_ERR_PARAM
    assert lbwd(ws=NUL) == REL_ERR_WORKSPACE
    assert lbwd(wsb=need - 1) == REL_ERR_WORKSPACE
    assert lbwd(ws=ctypes.c_void_p(0x7F0000000010)) == REL_ERR_ALIGN
    assert lbwd(dg=P_MIS) == REL_ERR_ALIGN
    assert lbwd(dsin=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN
    assert lbwd(fst=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN  # the forward's states
    assert lbwd(fst=P_MIS) == REL_ERR_ALIGN  # read with 16-byte vector loads
    # with the forward's states the smaller workspace suffices, one byte less does not
    assert lbwd(fst=P, ws=P, wsb=need_r - 1) == REL_ERR_WORKSPACE
    assert lbwd(fst=P, ws=ctypes.c_void_p(0x7F0000000010), wsb=need_r) == REL_ERR_ALIGN

    def lstep(dtype=BF16, B=1, H=1, D=64, st=P, y=P, tau=2.0):
        return lib.relation_linear_step(dtype, B, H, D, P, P, P, P, NUL, NUL, st, y, 0.125, tau,
                                        None)

    assert lstep(st=NUL) == REL_ERR_NULL
    assert lstep(y=NUL) == REL_ERR_NULL
    assert lstep(dtype=F32) == REL_ERR_UNSUPPORTED
    assert lstep(D=80) == REL_ERR_UNSUPPORTED
    assert lstep(B=0) == REL_ERR_SHAPE
    assert lstep(tau=-1.0) == REL_ERR_PARAM
    assert lstep(st=ctypes.c_void_p(0x7F0000000002)) == REL_ERR_ALIGN


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(rel, "_LIB", None)
    monkeypatch.setattr(rel, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        rel.load_library()
