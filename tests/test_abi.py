"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects invalid arguments with the documented status before touching
the device (no call here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import w4a16_speculative_verify_amd as w4v

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4v.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, -1, -2, -3, -4
A = 0x10000          # a 256-byte aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+char\s*\*|size_t|int)\s+(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(w4v.LIB_PATH):
        from w4a16_speculative_verify_amd import _build
        _build.build()
    return w4v.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(w4v.SIGNATURES), "binding and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", w4v.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_read_probe_validation(lib):
    assert lib.w4v_read_probe_blocks() > 0
    assert lib.w4v_read_probe(None, 1024, A, None) == INVALID
    assert lib.w4v_read_probe(A, 0, A, None) == INVALID
    assert lib.w4v_read_probe(A, 1000, A, None) == INVALID      # not a multiple of 16
    assert lib.w4v_read_probe(A + 8, 1024, A, None) == ALIGN
    assert lib.w4v_read_probe(A, 1024, None, None) == INVALID


def test_version_and_status_strings(lib):
    assert w4v.abi_version() == 1
    for st in (OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, -5):
        assert w4v.status_string(st)
    assert w4v.status_string(123) == "unknown status"


def gemm(lib, x=A, ldx=2560, qw=A, sc=A, qz=A, y=A * 64, ldy=2560, M=16, N=2560, K=2560, g=128,
         ws=None, wsb=0):
    return lib.w4a16_gemm(x, ldx, qw, sc, qz, y, ldy, M, N, K, g, ctypes.c_float(1.0), ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(g=64), UNSUPPORTED),
    (dict(g=0), INVALID),
    (dict(g=32, K=96, ldx=128), UNSUPPORTED),     # group size 32 needs K % 128 == 0
    (dict(g=32, K=100, ldx=128), INVALID),        # K not a multiple of the group size
    (dict(g=32, x=A + 2), ALIGN),                 # group size 32 reaches the pointer checks
    (dict(K=100, ldx=128), INVALID),
    (dict(K=0), INVALID),
    (dict(N=12, ldy=16), INVALID),
    (dict(M=-1), INVALID),
    (dict(x=None), INVALID),
    (dict(qz=None), INVALID),
    (dict(ldx=2000), INVALID),
    (dict(ldy=2000), INVALID),
    (dict(x=A + 2), ALIGN),
    (dict(ldx=2564), ALIGN),
    (dict(qw=A + 4), ALIGN),
    (dict(y=A * 64 + 8), ALIGN),
    (dict(qz=A + 2), ALIGN),
    (dict(y=A + 256), INVALID),                   # y overlaps x
    (dict(M=0), OK),                              # nothing to do: no launch
    (dict(N=0, ldy=0), OK),
    # 32-bit buffer offsets of the skinny path: weights or x rows of 2 GiB or more
    (dict(N=65536, K=65536, ldx=65536, ldy=65536, y=1 << 40), UNSUPPORTED),
    (dict(ldx=1 << 26, y=1 << 40), UNSUPPORTED),
])
def test_gemm_validation(lib, kw, status):
    assert gemm(lib, **kw) == status


def test_gemm_workspace(lib):
    need = w4v.gemm_workspace_size(16, 2560, 4096)
    assert need > 0                                # O projection splits K
    assert gemm(lib, K=4096, ldx=4096, ws=None, wsb=0) == WORKSPACE
    assert gemm(lib, K=4096, ldx=4096, ws=A * 256, wsb=need - 1) == WORKSPACE
    assert gemm(lib, K=4096, ldx=4096, ws=A * 256 + 16, wsb=need) == ALIGN
    assert w4v.gemm_workspace_size(0, 2560, 4096) == 0
    assert w4v.gemm_workspace_size(16, 2560, 4096, 64) == 0
    # group size 32 runs the same plans
    assert w4v.gemm_workspace_size(16, 2560, 4096, 32) == need
    assert w4v.gemm_workspace_size(16, 2560, 96, 32) == 0
    assert gemm(lib, K=4096, ldx=4096, g=32, ws=None, wsb=0) == WORKSPACE
    # sizes are a function of the shape alone
    assert w4v.gemm_workspace_size(16, 2560, 4096) == need
    # from 33 rows on: the LDS-tiled MFMA kernel; a plan with K-splits keeps the fp32
    # partials of its split tiles, [S][tiles][rows x 256] (128-row tiles up to 128 rows),
    # after the skinny kernel's regions and needs that workspace (none, or a smaller one,
    # is an error); an unsplit plan needs none
    big = w4v.gemm_workspace_size(33, 2560, 4096)
    rest = big - (64 << 10) - (4 << 20)
    tile = 128 * 256 * 4
    assert rest > 0 and rest % (10 * tile) == 0 and rest // (10 * tile) > 1
    # 256 full-size tiles (one round on 256 CUs): whole tiles, no partials
    assert w4v.gemm_workspace_size(8192, 2048, 4096) == 0
    # 320 tiles: 256 whole, the 64 of the partial second round split over the idle CUs
    tail = w4v.gemm_workspace_size(8192, 2560, 4096) - (64 << 10) - (4 << 20)
    assert tail > 0 and tail % (64 * 256 * 256 * 4) == 0
    assert w4v.gemm_workspace_size(33, 2560, 4096, 32) == big   # group size 32: same plan
    assert gemm(lib, M=33, K=4096, ldx=4096, ws=A * 256, wsb=big - 1) == WORKSPACE
    assert gemm(lib, M=33, K=4096, ldx=4096, ws=None, wsb=0) == WORKSPACE
    assert gemm(lib, M=33, K=4096, ldx=4096, ws=A * 256 + 16, wsb=big) == ALIGN
    # buffer resources take 32-bit offsets: weights of 2 GiB or more are refused
    assert gemm(lib, M=64, N=65536, K=65536, ldx=65536, ldy=65536, y=1 << 40,
                ws=None, wsb=0) == UNSUPPORTED


def gemm_na(lib, x=A, ldx=2560, qw=A, sc=A, qz=A, y=A * 64, ldy=2560, M=16, N=2560, K=2560, g=128):
    return lib.w4a16_gemm_noalloc(x, ldx, qw, sc, qz, y, ldy, M, N, K, g, ctypes.c_float(1.0), None)


@pytest.mark.parametrize("kw,status", [
    (dict(g=64), UNSUPPORTED),
    (dict(K=100, ldx=128), INVALID),
    (dict(x=None), INVALID),
    (dict(ldy=2000), INVALID),
    (dict(x=A + 2), ALIGN),
    (dict(y=A + 256), INVALID),                   # y overlaps x
    (dict(M=0), OK),
    # the plan's workspace would not fit the static scratch (43.5 MB > 32 MiB)
    (dict(M=168, N=19456, ldy=19456, y=1 << 40), UNSUPPORTED),
    (dict(M=8192, K=9728, ldx=9728, y=1 << 40), UNSUPPORTED),
])
def test_gemm_noalloc_validation(lib, kw, status):
    assert gemm_na(lib, **kw) == status


def test_static_scratch_limit(lib):
    assert w4v.STATIC_SCRATCH_BYTES == 32 << 20
    # every skinny plan (M <= 32) fits: 64 KiB of tickets + at most 4 MiB of partials
    for m, k, n in ((16, 9728, 2560), (32, 4096, 2560), (1, 2560, 19456)):
        assert w4v.gemm_workspace_size(m, n, k) <= w4v.STATIC_SCRATCH_BYTES
    assert w4v.gemm_workspace_size(168, 6144, 2560) <= w4v.STATIC_SCRATCH_BYTES
    assert w4v.gemm_workspace_size(168, 19456, 2560) > w4v.STATIC_SCRATCH_BYTES


def lm(lib, h=A, ldh=2560, w=A, sc=A, t=A, ml=None, M=16, H=2560, V=4096, ws=A * 256, wsb=1 << 30):
    return lib.w8a16_lmhead_argmax(h, ldh, w, sc, t, ml, M, H, V, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=100, ldh=128), INVALID),
    (dict(H=64, ldh=64), INVALID),
    (dict(V=0), INVALID),
    (dict(M=-3), INVALID),
    (dict(h=None), INVALID),
    (dict(t=None), INVALID),
    (dict(ldh=1000), INVALID),
    (dict(h=A + 8), ALIGN),
    (dict(w=A + 1), ALIGN),
    (dict(ml=A + 2), ALIGN),
    (dict(ws=None, wsb=0), WORKSPACE),
    (dict(wsb=16), WORKSPACE),
    (dict(M=0), OK),
    (dict(H=1 << 16, ldh=1 << 16, V=1 << 15), UNSUPPORTED),   # 2 GiB of weights
])
def test_lmhead_validation(lib, kw, status):
    assert lm(lib, **kw) == status


def test_lmhead_workspace_sizes(lib):
    assert w4v.lmhead_workspace_size(16, 2560, 151936) > 0
    assert w4v.lmhead_workspace_size(168, 2560, 151936) > w4v.lmhead_workspace_size(16, 2560, 151936)
    assert w4v.lmhead_workspace_size(16, 100, 151936) == 0


def gv(lib, t=A, d=A, B=2, K=15, V=4096, acc=A, out=A):
    return lib.greedy_verify(t, d, B, K, V, acc, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID),
    (dict(K=-1), INVALID),
    (dict(V=0), INVALID),
    (dict(t=None), INVALID),
    (dict(d=None), INVALID),
    (dict(acc=None), INVALID),
    (dict(out=None), INVALID),
    (dict(t=A + 2), ALIGN),
    (dict(B=1 << 30, K=100), INVALID),
    (dict(B=0), OK),
])
def test_verify_validation(lib, kw, status):
    assert gv(lib, **kw) == status


def test_fused_validation(lib):
    f = lib.w8a16_lmhead_argmax_verify
    ws = A * 256
    assert f(A, 2560, A, A, A, None, 2560, 4096, A, -1, 15, A, A, ws, 1 << 30, None) == INVALID
    assert f(A, 2560, A, A, A, None, 2560, 4096, None, 1, 15, A, A, ws, 1 << 30, None) == INVALID
    assert f(A, 2560, A, A, A, None, 2560, 4096, A, 1, 15, None, A, ws, 1 << 30, None) == INVALID
    assert f(A, 2560, A, A, A, None, 2560, 4096, A, 1 << 28, 100, A, A, ws, 1 << 30, None) == INVALID
    assert f(A, 2560, A, A, A, None, 100, 4096, A, 1, 15, A, A, ws, 1 << 30, None) == INVALID
    assert f(A, 2560, A, A, A, None, 2560, 4096, A, 1, 15, A, A, None, 0, None) == WORKSPACE
    assert f(A, 2560, A, A, A, None, 2560, 4096, A, 0, 15, A, A, None, 0, None) == OK


def test_binding_refuses_missing_library(tmp_path):
    import importlib
    mod = importlib.import_module("w4a16_speculative_verify_amd")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(RuntimeError, match="no fallback"):
            mod.load(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved


NGRAM_BASE = dict(h=A, ld=64, lens=A + 0x100000, B=4, n_max=4, n_min=1, K=23, d=A + 0x200000)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0, h=None, lens=None, d=None), OK),     # nothing to do
    (dict(B=-1), INVALID),
    (dict(ld=0), INVALID),
    (dict(K=0), INVALID),
    (dict(n_min=0), INVALID),
    (dict(n_min=3, n_max=2), INVALID),
    (dict(n_max=65), UNSUPPORTED),
    (dict(h=None), INVALID),
    (dict(lens=None), INVALID),
    (dict(d=None), INVALID),
    (dict(h=A + 2), ALIGN),
    (dict(d=A + 64), INVALID),                      # drafts overlap the histories
])
def test_ngram_draft_validation(lib, kw, status):
    a = dict(NGRAM_BASE, **kw)
    st = lib.ngram_draft(a["h"], a["ld"], a["lens"], a["B"], a["n_max"], a["n_min"], a["K"],
                         a["d"], None)
    assert st == status


@pytest.mark.parametrize("kw,status", [
    (dict(B=0, h=None), OK),
    (dict(B=-1), INVALID),
    (dict(ld=0), INVALID),
    (dict(K=-1), INVALID),
    (dict(out=None), INVALID),
    (dict(acc=None), INVALID),
    (dict(out=A + 0x300002), ALIGN),
])
def test_append_accepted_validation(lib, kw, status):
    a = dict(h=A, ld=64, lens=A + 0x100000, B=4, K=15, out=A + 0x300000, acc=A + 0x400000)
    a.update(kw)
    st = lib.append_accepted(a["h"], a["ld"], a["lens"], a["B"], a["K"], a["out"], a["acc"], None)
    assert st == status


def f16lm(lib, h=A, ldh=2560, w=A, t=A, ml=None, M=16, H=2560, V=4096, d=None, B=0, K=0,
          acc=None, out=None, ws=A * 256, wsb=1 << 30):
    return lib.f16_lmhead_argmax_verify(h, ldh, w, t, ml, M, H, V, d, B, K, acc, out, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=100, ldh=128), INVALID),
    (dict(h=None), INVALID),
    (dict(w=None), INVALID),
    (dict(t=None), INVALID),
    (dict(w=A + 8), ALIGN),
    (dict(ml=A + 2), ALIGN),
    (dict(ws=None, wsb=0), WORKSPACE),
    (dict(M=0), OK),
    (dict(B=-1), INVALID),
    (dict(B=2, K=15), INVALID),                               # M != B * (K + 1)
    (dict(M=32, B=2, K=15, d=A, acc=None, out=A), INVALID),   # verify outputs missing
    (dict(M=32, B=2, K=15, d=A, acc=A + 2, out=A), ALIGN),
    (dict(H=1 << 15, ldh=1 << 15, V=1 << 15), UNSUPPORTED),  # 2 GiB of fp16 weights
])
def test_f16_lmhead_validation(lib, kw, status):
    assert f16lm(lib, **kw) == status


def f16g(lib, x=A, ldx=2560, w=A * 32, ldw=2560, y=A * 1024, ldy=2560, M=16, N=2560, K=2560,
         ws=A * 256, wsb=1 << 30):
    return lib.f16_gemm(x, ldx, w, ldw, y, ldy, M, N, K, ctypes.c_float(1.0), ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(K=0), INVALID),
    (dict(M=-1), INVALID),
    (dict(x=None), INVALID),
    (dict(w=None), INVALID),
    (dict(ldx=2000), INVALID),
    (dict(ldw=2000), INVALID),
    (dict(ldy=2000), INVALID),
    (dict(x=A + 2), ALIGN),
    (dict(ldw=2564), ALIGN),
    (dict(y=A * 32 + 64), INVALID),              # y overlaps w
    (dict(y=A + 64), INVALID),                   # y overlaps x
    (dict(ws=None, wsb=0), WORKSPACE),
    (dict(wsb=1 << 20), WORKSPACE),
    (dict(M=0), OK),
    (dict(N=0, ldy=0), OK),
])
def test_f16_gemm_validation(lib, kw, status):
    assert f16g(lib, **kw) == status


def test_f16_workspace_sizes(lib):
    assert w4v.f16_gemm_workspace_size(16, 2560, 2560) >= 1 << 20
    assert w4v.f16_gemm_workspace_size(0, 2560, 2560) == 0
    assert lib.f16_lmhead_argmax_workspace_size(16, 2560, 151936) == w4v.lmhead_workspace_size(16, 2560, 151936)


def gdnc(lib, s=A * 256, k=A, v=A * 2, al=A * 3, be=A * 4, acc=A * 5, B=2, T=16, H=4, D=128):
    return lib.gdn_state_commit(s, k, v, al, be, acc, B, T, H, D, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INVALID),
    (dict(T=0), INVALID),
    (dict(H=0), INVALID),
    (dict(T=33), UNSUPPORTED),
    (dict(D=96), UNSUPPORTED),
    (dict(B=0), OK),
    (dict(s=None), INVALID),
    (dict(acc=None), INVALID),
    (dict(s=A * 256 + 4), ALIGN),
    (dict(be=A * 4 + 2), ALIGN),
    (dict(k=A * 256 + 64), INVALID),             # keys overlap the state
    (dict(B=4096, T=32, H=64), UNSUPPORTED),     # keys of 2 GiB or more
])
def test_gdn_commit_validation(lib, kw, status):
    assert gdnc(lib, **kw) == status
