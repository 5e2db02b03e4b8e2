"""The C ABI on the host: the library loads, exports every function that
include/gla.h declares, and rejects every invalid argument with its documented
status before any HIP call. CPU only: every call here fails validation, so
no kernel is ever launched (the pointers passed are never dereferenced)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from chunked_gated_recurrent_amd import gla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")

OK, NULL, SHAPE, DTYPE, DECAY, ALIAS, UNSUP, WS, HIP, ALIGN, TOO_LARGE = range(11)
BF16, F32 = gla.GLA_BF16, gla.GLA_F32


# A host-sanitizer build of the library (tests/test_host_sanitizers.py runs
# this file against one, in a process with the sanitizer runtime preloaded):
# loaded directly, without torch.
HOST_LIB = os.environ.get("GLA_TEST_HOST_LIB")


def lib_path():
    return HOST_LIB or gla.LIB_PATH


@pytest.fixture(scope="module")
def L():
    if HOST_LIB:
        return gla.bind(ctypes.CDLL(HOST_LIB))
    if not os.path.exists(gla.LIB_PATH):
        from chunked_gated_recurrent_amd import build
        build.build(verbose=False)
    return gla.lib()


def status_text(L, code):
    return L.gla_status_str(code).decode()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert set(names) == set(gla.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path()],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gla_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_version_and_status_strings(L):
    assert L.gla_abi_version() == 2
    seen = set()
    for code in range(11):
        s = status_text(L, code)
        assert s and s not in seen
        seen.add(s)
    assert status_text(L, 99) == "unknown status"
    assert status_text(L, -1) == "unknown status"


# fake, 256-byte aligned, far-apart device addresses: never dereferenced
A = [ctypes.c_void_p(0x7f0000000000 + i * (1 << 36)) for i in range(8)]
GOOD = np.array([0.5, 0.9, 0.99, 1.0], np.float32)


def dptr(arr):
    return arr.ctypes.data_as(ctypes.c_void_p)


def fwd(L, dt=BF16, B=2, T=128, H=4, dk=96, dv=192, chunk=0, q=A[0], k=A[1],
        v=A[2], decay=None, scale=1.0, s0=None, o=A[3], sf=None, ws=None,
        wsb=0):
    dec = GOOD if decay is None else decay
    return L.gla_chunk_fwd(dt, B, T, H, dk, dv, chunk, q, k, v,
                           None if decay is False else dptr(dec), scale, s0, o,
                           sf, ws, wsb, None)


def test_fwd_argument_errors(L):
    assert fwd(L, dt=7) == DTYPE
    assert fwd(L, dt=-3) == DTYPE
    assert fwd(L, H=0) == SHAPE
    assert fwd(L, B=0) == SHAPE
    assert fwd(L, T=-1) == SHAPE
    assert fwd(L, B=1 << 16, T=1 << 16) == SHAPE  # 2^32 tokens
    assert fwd(L, H=65, decay=np.full(65, 0.9, np.float32)) == UNSUP
    assert fwd(L, dk=17) == UNSUP
    assert fwd(L, dv=512) == UNSUP
    assert fwd(L, dk=144) == UNSUP
    assert fwd(L, chunk=48) == UNSUP
    # no kernel runs 128-token chunks: refused, not served with 64
    assert fwd(L, chunk=128) == UNSUP
    assert L.gla_chunk_fwd_workspace_bytes(BF16, 1, 65536, 16, 96, 192, 128) == 0
    assert fwd(L, decay=False) == NULL
    assert fwd(L, q=None) == NULL
    assert fwd(L, o=None) == NULL
    assert fwd(L, scale=float("nan")) == SHAPE
    for bad in (0.0, -0.5, 1.0000001, float("nan"), float("inf")):
        d = GOOD.copy()
        d[2] = bad
        assert fwd(L, decay=d) == DECAY, bad
    assert fwd(L, q=ctypes.c_void_p(0x7f0000000008)) == ALIGN
    assert fwd(L, sf=ctypes.c_void_p(0x7f0000000004)) == ALIGN
    # o overlapping q / s_final partially overlapping s0 / s_final on o
    assert fwd(L, o=ctypes.c_void_p(A[0].value + 4096)) == ALIAS
    assert fwd(L, s0=A[4], sf=ctypes.c_void_p(A[4].value + 256)) == ALIAS
    assert fwd(L, sf=A[3]) == ALIAS


class env:
    """Temporarily set environment variables (the library reads its tuning
    knobs at every call)."""

    def __init__(self, **kv):
        self.kv, self.old = kv, {}

    def __enter__(self):
        for k, v in self.kv.items():
            self.old[k] = os.environ.get(k)
            os.environ[k] = v

    def __exit__(self, *a):
        for k, v in self.old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def test_fwd_workspace_contract(L):
    # one long sequence must be split into segments (8 at 16 heads) and needs
    # scratch: the segments' local states for the three launches; with the
    # chained scan (GLA_FWD_CHAIN=1) also the inclusive and incoming states
    # and a flag per (segment, head, d_v tile)
    need = L.gla_chunk_fwd_workspace_bytes(BF16, 1, 65536, 16, 96, 192, 0)
    assert need == 8 * 16 * 96 * 192 * 4
    with env(GLA_FWD_CHAIN="1"):
        assert L.gla_chunk_fwd_workspace_bytes(BF16, 1, 65536, 16, 96, 192, 0) == \
            3 * 8 * 16 * 96 * 192 * 4 + 8 * 16 * 2 * 4
    dec = np.full(16, 0.9, np.float32)
    assert fwd(L, B=1, T=65536, H=16, decay=dec) == WS
    assert fwd(L, B=1, T=65536, H=16, decay=dec, ws=A[5], wsb=need - 1) == WS
    # scratch overlapping an input is rejected
    assert fwd(L, B=1, T=65536, H=16, decay=dec, ws=A[0], wsb=need) == ALIAS
    # the workspace follows the 16-byte alignment of every other pointer
    assert fwd(L, B=1, T=65536, H=16, decay=dec, ws=ctypes.c_void_p(A[5].value + 8),
               wsb=need) == ALIGN
    # Laplace-shaped batch: enough chains, no scratch
    assert L.gla_chunk_fwd_workspace_bytes(BF16, 8, 2048, 16, 96, 192, 0) == 0
    assert L.gla_chunk_fwd_workspace_bytes(BF16, 0, 2048, 16, 96, 192, 0) == 0
    assert L.gla_chunk_fwd_workspace_bytes(9, 1, 2048, 16, 96, 192, 0) == 0


def varlen(L, dt=BF16, N=3, total=300, H=4, dk=96, dv=192, chunk=0, cu=A[6],
           q=A[0], k=A[1], v=A[2], decay=None, s0=None, o=A[3], sf=None,
           ws=None, wsb=0):
    dec = GOOD if decay is None else decay
    return L.gla_chunk_fwd_varlen(dt, N, total, H, dk, dv, chunk, cu, q, k, v,
                                  dptr(dec), 1.0, s0, o, sf, ws, wsb, None)


def test_varlen_argument_errors(L):
    assert varlen(L, N=0) == SHAPE
    assert varlen(L, total=-1) == SHAPE
    assert varlen(L, cu=None) == NULL
    assert varlen(L, k=None) == NULL
    assert varlen(L, cu=ctypes.c_void_p(A[6].value + 2)) == ALIGN
    assert varlen(L, o=A[6]) == ALIAS          # o on top of cu_seqlens
    assert varlen(L, sf=ctypes.c_void_p(A[6].value)) == ALIAS
    assert varlen(L, dk=8) == UNSUP
    d = GOOD.copy()
    d[0] = 0.0
    assert varlen(L, decay=d) == DECAY
    need = L.gla_chunk_fwd_varlen_workspace_bytes(BF16, 1, 65536, 16, 96, 192, 0)
    assert need > 0
    dec = np.full(16, 0.9, np.float32)
    assert varlen(L, N=1, total=65536, H=16, decay=dec) == WS
    # 32 sequences x 16 heads: enough chains, no time segments; the scratch
    # is the dispatch order alone (32 int32, rounded up to 256 bytes)
    assert L.gla_chunk_fwd_varlen_workspace_bytes(BF16, 32, 131072, 16, 96, 192, 0) == 256
    assert varlen(L, N=32, total=131072, H=16, decay=dec) == WS
    assert varlen(L, N=32, total=131072, H=16, decay=dec,
                  ws=ctypes.c_void_p(A[5].value + 4), wsb=4096) == ALIGN
    assert varlen(L, chunk=128) == UNSUP
    # one short sequence needs no scratch at all
    assert L.gla_chunk_fwd_varlen_workspace_bytes(BF16, 1, 100, 16, 96, 192, 0) == 0


def test_noalloc_argument_errors(L, monkeypatch):
    """The allocation-free packed forward validates exactly like
    gla_chunk_fwd_varlen, and refuses a plan larger than its fixed scratch,
    all before any HIP call."""
    def na(dt=BF16, N=3, total=300, H=4, dk=96, dv=192, chunk=0, cu=A[6], q=A[0],
           k=A[1], v=A[2], decay=None, s0=None, o=A[3], sf=None):
        dec = GOOD if decay is None else decay
        return L.gla_chunk_fwd_varlen_noalloc(dt, N, total, H, dk, dv, chunk, cu, q, k, v,
                                              dptr(dec), 1.0, s0, o, sf, None)
    assert na(dt=5) == DTYPE
    assert na(N=0) == SHAPE
    assert na(total=-1) == SHAPE
    assert na(cu=None) == NULL
    assert na(q=None) == NULL
    assert na(chunk=128) == UNSUP
    assert na(dk=8) == UNSUP
    assert na(cu=ctypes.c_void_p(A[6].value + 2)) == ALIGN
    assert na(o=A[6]) == ALIAS
    d = GOOD.copy()
    d[0] = -1.0
    assert na(decay=d) == DECAY
    dec16 = np.full(16, 0.9, np.float32)
    # the largest default plan at the Laplace head shape fits the scratch
    # (7 long sequences, 22 time segments)
    assert L.gla_chunk_fwd_varlen_workspace_bytes(BF16, 7, 7 * 65536, 16, 96, 192, 0) <= 32 << 20
    # a plan beyond the fixed scratch (time segments of 128 tokens forced)
    monkeypatch.setenv("GLA_TARGET_WGS", "100000")
    need = L.gla_chunk_fwd_varlen_workspace_bytes(BF16, 1, 65536, 16, 96, 192, 0)
    assert need > (32 << 20)
    assert na(N=1, total=65536, H=16, decay=dec16) == TOO_LARGE
    assert status_text(L, TOO_LARGE).startswith("the call needs more scratch")


def test_gated_argument_errors(L):
    """The gated forward, packed forward and decode step validate like their
    ungated calls, plus the gate itself and its g array."""
    def fg(gate=1, g=A[7], o=A[3], T=128, **kw):
        return L.gla_chunk_fwd_gated(BF16, 2, T, 4, 96, 192, 0, A[0], A[1], A[2], g, gate,
                                     dptr(GOOD), 1.0, None, o, None, None, 0, None)
    assert fg(gate=0) == UNSUP
    assert fg(gate=3) == UNSUP
    assert fg(g=None) == NULL
    assert fg(g=None, T=0) == OK           # no tokens: nothing read or launched
    assert fg(g=ctypes.c_void_p(A[7].value + 8)) == ALIGN
    assert fg(o=ctypes.c_void_p(A[7].value + 512)) == ALIAS   # o inside g
    assert fg(g=A[3]) == ALIAS                                  # g is o

    def vg(gate=2, g=A[7], o=A[3]):
        return L.gla_chunk_fwd_varlen_gated(BF16, 3, 300, 4, 96, 192, 0, A[6], A[0], A[1], A[2],
                                            g, gate, dptr(GOOD), 1.0, None, o, None, None, 0,
                                            None)
    assert vg(gate=7) == UNSUP
    assert vg(g=None) == NULL
    assert vg(g=A[3]) == ALIAS
    assert vg() == WS          # valid otherwise: the dispatch order needs scratch

    def dg(gate=1, g=A[7], o=A[4], N=4):
        return L.gla_decode_step_gated(BF16, N, 4, 96, 192, A[0], A[1], A[2], g, gate,
                                       dptr(GOOD), 1.0, A[3], o, None)
    assert dg(gate=-1) == UNSUP
    assert dg(g=None) == NULL
    assert dg(g=None, N=0) == OK
    assert dg(g=ctypes.c_void_p(A[3].value + 4096)) == ALIAS    # g inside the state
    assert dg(g=ctypes.c_void_p(A[7].value + 4)) == ALIGN


def test_decode_argument_errors(L):
    def dec(dt=BF16, N=4, H=4, dk=96, dv=192, q=A[0], k=A[1], v=A[2], st=A[3],
            o=A[4], decay=GOOD):
        return L.gla_decode_step(dt, N, H, dk, dv, q, k, v, dptr(decay), 1.0, st, o, None)
    assert dec(dt=3) == DTYPE
    assert dec(N=-1) == SHAPE
    assert dec(N=0) == OK                      # nothing to do, nothing launched
    assert dec(st=None) == NULL
    assert dec(o=None) == NULL
    assert dec(dv=40) == UNSUP
    assert dec(st=ctypes.c_void_p(A[3].value + 8)) == ALIGN
    assert dec(o=ctypes.c_void_p(A[3].value + 1024)) == ALIAS   # o inside state
    assert dec(st=ctypes.c_void_p(A[2].value + 512)) == ALIAS   # state on v
    d = GOOD.copy()
    d[1] = 2.0
    assert dec(decay=d) == DECAY


def test_backward_argument_errors(L):
    # dv = 256: four dv tiles whose partial sums need workspace at any size
    def bwd(dt=BF16, B=2, T=100, H=4, dk=96, dv=256, chunk=0, q=A[0], k=A[1], v=A[2],
            s0=None, do=A[3], dsf=None, dq=A[4], dk_=A[5], dv_=A[6], ds0=None,
            ws=A[7], wsb=1 << 40, decay=GOOD):
        return L.gla_chunk_bwd(dt, B, T, H, dk, dv, chunk, q, k, v, dptr(decay), 1.0, s0,
                               do, dsf, dq, dk_, dv_, ds0, ws, wsb, None)
    assert bwd(dt=7) == DTYPE
    # fp32, other head sizes and 32-token chunks run on the vector ALUs: valid
    # shapes, so here they fail only for want of workspace
    assert bwd(dt=F32, wsb=16) == WS
    assert bwd(dk=64, ws=None) == WS
    assert bwd(chunk=32, ws=None) == WS
    assert bwd(chunk=48) == UNSUP
    assert bwd(dk=100) == UNSUP
    assert bwd(B=0) == SHAPE
    assert bwd(T=-1) == SHAPE
    assert bwd(do=None) == NULL
    assert bwd(dq=None) == NULL
    assert bwd(dq=ctypes.c_void_p(A[4].value + 4)) == ALIGN
    assert bwd(dk_=A[4]) == ALIAS                            # dk on top of dq
    assert bwd(dv_=ctypes.c_void_p(A[3].value + 4096)) == ALIAS  # dv inside dout
    assert bwd(ds0=ctypes.c_void_p(A[1].value)) == ALIAS    # ds0 on k
    assert bwd(ws=None) == WS
    assert bwd(wsb=16) == WS
    assert bwd(ws=A[0]) == ALIAS                             # workspace on q
    d = GOOD.copy()
    d[3] = float("inf")
    assert bwd(decay=d) == DECAY
    need = L.gla_chunk_bwd_workspace_bytes(BF16, 8, 2048, 16, 96, 256, 0)
    # dq and dk partials: 4 dv tiles x 16 heads x 16,384 tokens x 96 fp32, twice
    assert need == 2 * 4 * 16 * 8 * 2048 * 96 * 4
    # dv = 192, 128 and 64: one workgroup per (sequence, head) over all of
    # dv, no partials. The 8 x 16 units of the Laplace batch fill the GPU with
    # both walks in one launch: no time segments, no scratch
    for dv in (192, 128, 64):
        assert L.gla_chunk_bwd_workspace_bytes(BF16, 8, 2048, 16, 96, dv, 0) == 0, dv
    assert L.gla_chunk_bwd_workspace_bytes(BF16, 2, 100, 4, 96, 128, 0) == 0
    assert L.gla_chunk_bwd_workspace_bytes(BF16, 256, 128, 16, 96, 192, 0) == 0
    # 8 x 8 units do not: the walks run one after the other, one workgroup
    # per unit, over 4 time segments per sequence (64 units x 4 fill the 256
    # CUs), whose incoming states and carried gradients (fp32 96 x dv per
    # segment and head) are the workspace
    for dv in (192, 128, 64):
        need = L.gla_chunk_bwd_workspace_bytes(BF16, 8, 2048, 8, 96, dv, 0)
        assert need == 2 * (8 * 4 * 8 * 96 * dv * 4), dv
    # vector-ALU path: dv tiles of 64 columns, dk = 32
    assert L.gla_chunk_bwd_workspace_bytes(F32, 8, 2048, 16, 32, 192, 0) == \
        2 * 3 * 16 * 8 * 2048 * 32 * 4
    assert L.gla_chunk_bwd_workspace_bytes(BF16, 8, 0, 16, 96, 192, 0) == 0


def test_backward_varlen_argument_errors(L):
    def bwd(dt=BF16, N=3, total=300, H=4, dk=96, dv=192, chunk=0, cu=A[7], q=A[0], k=A[1],
            v=A[2], do=A[3], dq=A[4], dk_=A[5], dv_=A[6], ds0=None, ws=None, wsb=0,
            decay=GOOD):
        return L.gla_chunk_bwd_varlen(dt, N, total, H, dk, dv, chunk, cu, q, k, v,
                                      dptr(decay), 1.0, None, do, None, dq, dk_, dv_, ds0,
                                      ws, wsb, None)
    assert bwd(dt=F32) == WS                                # vector-ALU path, no workspace given
    assert bwd(chunk=96) == UNSUP
    assert bwd(N=0) == SHAPE
    assert bwd(total=-2) == SHAPE
    assert bwd(cu=None) == NULL
    assert bwd(cu=ctypes.c_void_p(A[7].value + 2)) == ALIGN
    assert bwd(dq=ctypes.c_void_p(A[7].value)) == ALIAS     # dq on top of cu_seqlens
    assert bwd(dk_=A[4]) == ALIAS
    assert bwd() == WS                                      # N > 1: the order needs scratch
    assert L.gla_chunk_bwd_varlen_workspace_bytes(BF16, 3, 300, 4, 96, 192, 0) > 0
    assert L.gla_chunk_bwd_varlen_workspace_bytes(F32, 3, 300, 4, 96, 192, 0) > 0


def test_short_conv_argument_errors(L):
    def conv(dt=BF16, B=2, T=10, D=3072, x=A[0], w=A[1], b=None, wi=None, y=A[2], wo=A[3]):
        return L.gla_short_conv_fwd(dt, B, T, D, x, w, b, wi, y, wo, None)
    assert conv(dt=4) == DTYPE
    assert conv(B=0) == SHAPE
    assert conv(T=-1) == SHAPE
    assert conv(D=12) == UNSUP
    assert conv(w=None) == NULL
    assert conv(y=None) == NULL
    assert conv(x=ctypes.c_void_p(A[0].value + 8)) == ALIGN
    assert conv(b=ctypes.c_void_p(A[1].value + 2)) == ALIGN
    assert conv(y=ctypes.c_void_p(A[0].value + 4096)) == ALIAS     # y inside x
    assert conv(wo=A[2]) == ALIAS                                   # window_out on y
    assert conv(wi=A[3]) == ALIAS                                   # window_in is window_out

    def dec(dt=BF16, N=4, D=3072, x=A[0], w=A[1], b=None, win=A[3], y=A[2]):
        return L.gla_short_conv_decode_step(dt, N, D, x, w, b, win, y, None)
    assert dec(N=-1) == SHAPE
    assert dec(N=0) == OK
    assert dec(D=4) == UNSUP
    assert dec(win=None) == NULL
    assert dec(y=A[3]) == ALIAS                                     # y on the window


def test_linear_attn_argument_errors(L):
    def la(dt=BF16, B=2, T=128, H=4, dk=96, dv=192, chunk=0, q=A[0], k=A[1], v=A[2],
           s0=None, z0=None, o=A[3], sf=None, zf=None, ws=None, wsb=0):
        return L.gla_linear_attn_fwd(dt, B, T, H, dk, dv, chunk, q, k, v, s0, z0, o,
                                     sf, zf, ws, wsb, None)
    assert la(dt=5) == DTYPE
    assert la(B=0) == SHAPE
    assert la(T=-1) == SHAPE
    assert la(H=65) == UNSUP
    assert la(dk=100) == UNSUP
    assert la(chunk=48) == UNSUP
    assert la(q=None) == NULL
    assert la(o=None) == NULL
    assert la(T=0, q=None, k=None, v=None, o=None) == OK   # nothing to launch
    assert la(z0=ctypes.c_void_p(A[4].value + 4)) == ALIGN
    assert la(o=ctypes.c_void_p(A[2].value + 4096)) == ALIAS    # o inside v
    assert la(s0=A[4], sf=A[4]) == ALIAS                          # no in-place final sums
    assert la(z0=A[5], zf=A[5]) == ALIAS
    assert la(sf=A[4], zf=ctypes.c_void_p(A[4].value + 4096)) == ALIAS
    assert la(zf=A[3]) == ALIAS                                   # z_final on o
    # one batch entry of a long sequence is cut into time segments
    need = L.gla_linear_attn_fwd_workspace_bytes(BF16, 1, 1 << 16, 4, 96, 192, 0)
    plain = L.gla_chunk_fwd_workspace_bytes(BF16, 1, 1 << 16, 4, 96, 192, 0)
    assert need > plain > 0
    assert la(B=1, T=1 << 16) == WS
    assert la(B=1, T=1 << 16, ws=A[6], wsb=need - 1) == WS
    assert la(B=1, T=1 << 16, ws=A[0], wsb=need) == ALIAS         # workspace on q
    assert L.gla_linear_attn_fwd_workspace_bytes(BF16, 64, 2048, 16, 96, 192, 0) == 0


def test_linear_attn_varlen_argument_errors(L):
    def la(dt=BF16, N=3, total=300, H=4, dk=96, dv=192, chunk=0, cu=A[7], q=A[0], k=A[1],
           v=A[2], s0=None, z0=None, o=A[3], sf=None, zf=None, ws=None, wsb=0):
        return L.gla_linear_attn_fwd_varlen(dt, N, total, H, dk, dv, chunk, cu, q, k, v,
                                            s0, z0, o, sf, zf, ws, wsb, None)
    assert la(dt=3) == DTYPE
    assert la(N=0) == SHAPE
    assert la(cu=None) == NULL
    assert la(cu=ctypes.c_void_p(A[7].value + 2)) == ALIGN
    assert la(o=ctypes.c_void_p(A[7].value)) == ALIAS      # o on cu_seqlens
    assert la(s0=A[4], sf=A[4]) == ALIAS
    assert la(zf=A[2]) == ALIAS                            # z_final on v
    assert la() == WS                                      # N > 1: the order needs scratch
    assert L.gla_linear_attn_fwd_varlen_workspace_bytes(BF16, 3, 300, 4, 96, 192, 0) > 0
    # a few long sequences: time segments with their z slots
    a = L.gla_linear_attn_fwd_varlen_workspace_bytes(BF16, 2, 1 << 16, 4, 96, 192, 0)
    b = L.gla_chunk_fwd_varlen_workspace_bytes(BF16, 2, 1 << 16, 4, 96, 192, 0)
    assert a > b > 0


def test_linear_attn_decode_argument_errors(L):
    def la(dt=BF16, N=4, H=4, dk=96, dv=192, q=A[0], k=A[1], v=A[2], st=A[3], z=A[4], o=A[5]):
        return L.gla_linear_attn_decode_step(dt, N, H, dk, dv, q, k, v, st, z, o, None)
    assert la(dt=2) == DTYPE
    assert la(N=-1) == SHAPE
    assert la(N=0) == OK                                          # nothing launched
    assert la(dk=24) == UNSUP
    assert la(z=None) == NULL
    assert la(z=ctypes.c_void_p(A[4].value + 8)) == ALIGN
    assert la(z=ctypes.c_void_p(A[3].value + 4096)) == ALIAS      # z inside the state
    assert la(o=A[0]) == ALIAS                                    # o on q


def test_decode_pool_argument_errors(L):
    def pool(dt=BF16, N=4, H=4, dk=96, dv=192, q=A[0], k=A[1], v=A[2], sl=A[5],
             P=8, st=A[3], o=A[4], decay=GOOD):
        return L.gla_decode_step_pool(dt, N, H, dk, dv, q, k, v, dptr(decay), 1.0,
                                      sl, P, st, o, None)
    assert pool(dt=3) == DTYPE
    assert pool(N=-1) == SHAPE
    assert pool(P=0) == SHAPE
    assert pool(N=0) == OK                     # nothing to do, nothing launched
    assert pool(sl=None) == NULL
    assert pool(st=None) == NULL
    assert pool(dk=8) == UNSUP
    assert pool(sl=ctypes.c_void_p(A[5].value + 2)) == ALIGN
    assert pool(st=ctypes.c_void_p(A[3].value + 8)) == ALIGN
    assert pool(sl=ctypes.c_void_p(A[3].value + 4096)) == ALIAS  # slots inside the pool
    assert pool(o=ctypes.c_void_p(A[5].value)) == ALIAS          # o on the slots
    assert pool(st=ctypes.c_void_p(A[0].value + 512)) == ALIAS   # pool on q
    d = GOOD.copy()
    d[2] = -0.5
    assert pool(decay=d) == DECAY


def test_dk64_forward_plans_on_matrix_cores():
    """bf16 with d_k 64 plans the matrix-core forward (d_v tiles of 64
    columns: 3 per head at d_v 192, 12 units for 4 heads, so 22 time
    segments of 192 tokens for one 4,096-token sequence); fp32 plans the
    vector-ALU forward (16-column tiles: 48 units, 6 segments)."""
    L = gla.lib()
    assert L.gla_chunk_fwd_workspace_bytes(1, 1, 4096, 4, 64, 192, 0) == 22 * 4 * 64 * 192 * 4
    assert L.gla_chunk_fwd_workspace_bytes(0, 1, 4096, 4, 64, 192, 0) == 6 * 4 * 64 * 192 * 4
