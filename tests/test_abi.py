"""The C-ABI library: it loads, exports every entry point include/pa.h declares,
and rejects malformed host arguments with the documented status before any
HIP call (so these run without a GPU; no kernel is launched)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")


@pytest.fixture(scope="module")
def lib():
    from paged_kv_cache_40_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from paged_kv_cache_40_amd.build import build
        build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("pa_write_kv", "pa_decode", "pa_decode_ext", "pa_copy_blocks", "pa_swap_blocks",
              "pa_decode_workspace_bytes", "pa_strerror"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_signatures_cover_header(lib):
    from paged_kv_cache_40_amd import _lib
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(lib.pa_strerror(code), bytes)
    assert lib.pa_strerror(-4).startswith(b"workspace")


def test_workspace_bytes(lib):
    f = lib.pa_decode_workspace_bytes
    assert f(256, 40, 128, 256) == 0               # one partition: no partials
    # partials, then one int per query row (the longest-first order of the sequences)
    assert f(256, 40, 128, 257) == 256 * 40 * 2 * 130 * 4 + 256 * 4
    assert f(256, 40, 128, 4097) == 256 * 40 * 17 * 130 * 4 + 256 * 4
    assert f(0, 40, 128, 4097) == 0


FAKE = 0x1000  # never dereferenced: every call below fails host validation first


def write_kv(lib, **kw):
    a = dict(k=FAKE, v=FAKE, nb=64, kn=FAKE, vn=FAKE, bt=FAKE, mb=8, cl=FAKE, wsl=None, S=4, T=4,
             H=2, D=64, B=16, dt=0)
    a.update(kw)
    return lib.pa_write_kv(a["k"], a["v"], a["nb"], a["kn"], a["vn"], a["bt"], a["mb"], a["cl"],
                           a["wsl"], a["S"], a["T"], a["H"], a["D"], a["B"], a["dt"], None)


def decode(lib, **kw):
    a = dict(o=FAKE, q=FAKE, k=FAKE, v=FAKE, nb=64, bt=FAKE, mb=8, cl=FAKE, qsl=None, S=4, T=4,
             mcl=100, mql=1, H=2, D=64, B=16, dt=0, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.pa_decode(a["o"], a["q"], a["k"], a["v"], a["nb"], a["bt"], a["mb"], a["cl"],
                         a["qsl"], a["S"], a["T"], a["mcl"], a["mql"], a["H"], a["D"], a["B"],
                         a["dt"], a["ws"], a["wsb"], None)


def decode_ext(lib, window=0, alibi=None, flags=0, **kw):
    a = dict(o=FAKE, q=FAKE, k=FAKE, v=FAKE, nb=64, bt=FAKE, mb=8, cl=FAKE, qsl=None, S=4, T=4,
             mcl=100, mql=1, H=2, D=64, B=16, dt=0, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.pa_decode_ext(a["o"], a["q"], a["k"], a["v"], a["nb"], a["bt"], a["mb"], a["cl"],
                             a["qsl"], a["S"], a["T"], a["mcl"], a["mql"], a["H"], a["D"], a["B"],
                             a["dt"], a["ws"], a["wsb"], window, alibi, flags, None)


@pytest.mark.parametrize("args,code", [
    (dict(window=-1), -2),
    (dict(window=8, mql=2, qsl=FAKE, T=5, dt=0, D=64), -3),       # tile path: fp16 only
    (dict(alibi=FAKE, mql=2, qsl=FAKE, T=5, dt=0, D=128), -3),    # tile path: fp16 only
    (dict(window=8, o=None), -1), (dict(alibi=FAKE, D=32), -3), (dict(window=8, mcl=129), -2),
    (dict(flags=2), -3), (dict(flags=1 << 31), -3),
    (dict(flags=1, H=64, S=65535, T=65535, mcl=2048, mb=128), -2),     # 1-D grid too large
    # grouped decode: group sizes 2..6, fp16 pure decode without window, ALiBi or the hint
    (dict(flags=7 << 8, dt=1), -3), (dict(flags=16 << 8, dt=1), -3), (dict(flags=2 << 8), -3),
    (dict(flags=(2 << 8) | 1, dt=1), -3), (dict(flags=2 << 8, dt=1, window=8), -3),
    (dict(flags=2 << 8, dt=1, qsl=FAKE), -3),
])
def test_decode_ext_rejects(lib, args, code):
    assert decode_ext(lib, **args) == code


def copy_blocks(lib, **kw):
    a = dict(k=FAKE, v=FAKE, nb=64, pairs=FAKE, n=3, H=2, D=64, B=16, dt=1)
    a.update(kw)
    return lib.pa_copy_blocks(a["k"], a["v"], a["nb"], a["pairs"], a["n"], a["H"], a["D"], a["B"],
                              a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=None), -1), (dict(kn=None), -1), (dict(bt=None), -1), (dict(cl=None), -1),
    (dict(D=96), -3), (dict(B=64), -3), (dict(dt=2), -3),
    (dict(H=0), -2), (dict(nb=0), -2), (dict(S=0), -2), (dict(T=-1), -2), (dict(T=5), -2),
    (dict(mb=0), -2),
])
def test_write_kv_rejects(lib, kw, code):
    assert write_kv(lib, **kw) == code


def test_write_kv_zero_tokens_is_a_noop(lib):
    assert write_kv(lib, wsl=FAKE, T=0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(o=None), -1), (dict(q=None), -1), (dict(v=None), -1), (dict(cl=None), -1),
    (dict(D=32), -3), (dict(B=4), -3), (dict(dt=5), -3),
    (dict(mcl=0), -2), (dict(mql=0), -2), (dict(mcl=129), -2), (dict(T=5), -2), (dict(mql=2), -2),
    (dict(S=0), -2), (dict(H=-1), -2), (dict(mql=101), -2),
    (dict(ws=None, mcl=300, mb=32), -4), (dict(wsb=10, mcl=300, mb=32), -4),
])
def test_decode_rejects(lib, kw, code):
    assert decode(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(pairs=None), -1), (dict(v=None), -1), (dict(n=-1), -2), (dict(D=100), -3),
    (dict(nb=-5), -2),
])
def test_copy_blocks_rejects(lib, kw, code):
    assert copy_blocks(lib, **kw) == code


def swap_blocks(lib, **kw):
    a = dict(dk=FAKE, dv=FAKE, nb=64, hk=FAKE, hv=FAKE, nh=32, pairs=FAKE, n=3, dir=0, H=2, D=64,
             B=16, dt=1)
    a.update(kw)
    return lib.pa_swap_blocks(a["dk"], a["dv"], a["nb"], a["hk"], a["hv"], a["nh"], a["pairs"],
                              a["n"], a["dir"], a["H"], a["D"], a["B"], a["dt"], None)


# every case fails before the host-memory query, so no HIP call is made
@pytest.mark.parametrize("kw,code", [
    (dict(dk=None), -1), (dict(hv=None), -1), (dict(pairs=None), -1),
    (dict(nh=0), -2), (dict(n=-1), -2), (dict(dir=2), -2), (dict(dir=-1), -2), (dict(nb=0), -2),
    (dict(D=96), -3), (dict(dt=3), -3),
])
def test_swap_blocks_rejects(lib, kw, code):
    assert swap_blocks(lib, **kw) == code


def test_swap_blocks_zero_pairs_is_a_noop(lib):
    assert swap_blocks(lib, n=0, pairs=None, hk=None) == 0


def test_strerror_host_memory(lib):
    assert b"pinned" in lib.pa_strerror(-6)


def test_copy_blocks_zero_pairs_is_a_noop(lib):
    assert copy_blocks(lib, n=0, pairs=None) == 0


def test_binding_raises_without_library(monkeypatch, tmp_path):
    from paged_kv_cache_40_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError):
        _lib.load(str(tmp_path / "missing.so"))


def test_check_workspace_bytes(lib):
    f = lib.pa_check_workspace_bytes
    assert f(0) == 0 and f(-3) == 0
    assert f(1) == 8                      # two bitmaps of one 32-bit word
    assert f(32) == 8 and f(33) == 16
    assert f(47104 * 16) == 2 * 4 * (47104 * 16 // 32)


def check_attention(lib, **kw):
    a = dict(err=FAKE, nb=64, bt=FAKE, mb=8, cl=FAKE, qsl=None, S=4, T=4, mcl=100, mql=1, B=16,
             W=0)
    a.update(kw)
    return lib.pa_check_attention(a["err"], a["nb"], a["bt"], a["mb"], a["cl"], a["qsl"], a["S"],
                                  a["T"], a["mcl"], a["mql"], a["B"], a["W"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(err=None), -1), (dict(bt=None), -1), (dict(cl=None), -1),
    (dict(nb=0), -2), (dict(S=0), -2), (dict(T=0), -2), (dict(mb=0), -2), (dict(mcl=0), -2),
    (dict(mql=0), -2), (dict(W=-1), -2), (dict(T=5), -2), (dict(B=12), -3),
])
def test_check_attention_rejects(lib, kw, code):
    assert check_attention(lib, **kw) == code


def check_write(lib, **kw):
    a = dict(err=FAKE, ws=FAKE, wsb=1 << 20, nb=64, bt=FAKE, mb=8, cl=FAKE, wsl=None, S=4, T=4,
             B=16)
    a.update(kw)
    return lib.pa_check_write(a["err"], a["ws"], a["wsb"], a["nb"], a["bt"], a["mb"], a["cl"],
                              a["wsl"], a["S"], a["T"], a["B"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(err=None), -1), (dict(bt=None), -1), (dict(cl=None), -1),
    (dict(nb=0), -2), (dict(S=0), -2), (dict(T=-1), -2), (dict(T=5), -2), (dict(mb=0), -2),
    (dict(B=4), -3), (dict(ws=None), -4), (dict(wsb=255), -4),   # 64 x 16 slots need 256 B
])
def test_check_write_rejects(lib, kw, code):
    assert check_write(lib, **kw) == code


def check_pairs(lib, **kw):
    a = dict(err=FAKE, ws=FAKE, wsb=1 << 20, ns=64, nd=64, pairs=FAKE, n=3, same=1)
    a.update(kw)
    return lib.pa_check_pairs(a["err"], a["ws"], a["wsb"], a["ns"], a["nd"], a["pairs"], a["n"],
                              a["same"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(err=None), -1), (dict(pairs=None), -1),
    (dict(ns=0), -2), (dict(nd=-1), -2), (dict(n=-1), -2), (dict(same=2), -2),
    (dict(nd=32), -2),                     # one pool needs equal sizes
    (dict(ws=None), -4), (dict(wsb=15), -4),
])
def test_check_pairs_rejects(lib, kw, code):
    assert check_pairs(lib, **kw) == code


def noalloc(lib, **kw):
    a = dict(o=FAKE, q=FAKE, k=FAKE, v=FAKE, nb=64, bt=FAKE, mb=8, cl=FAKE, qsl=None, S=4, T=4,
             mcl=100, mql=1, H=2, D=64, B=16, dt=0, W=0, al=None, fl=0)
    a.update(kw)
    return lib.pa_decode_noalloc(a["o"], a["q"], a["k"], a["v"], a["nb"], a["bt"], a["mb"],
                                 a["cl"], a["qsl"], a["S"], a["T"], a["mcl"], a["mql"], a["H"],
                                 a["D"], a["B"], a["dt"], a["W"], a["al"], a["fl"], None)


def test_noalloc_rejects_before_any_hip_call(lib):
    from paged_kv_cache_40_amd import _lib
    # the same host checks as pa_decode_ext
    assert noalloc(lib, o=None) == -1
    assert noalloc(lib, D=96) == -3
    assert noalloc(lib, mcl=200, mb=8) == -2          # context past the table width
    assert noalloc(lib, fl=1 << 31) == -3
    # a batch whose partials exceed the library's array: PA_ERR_WORKSPACE, nothing launched
    S, H, D, L = 256, 40, 128, 16384
    need = lib.pa_decode_workspace_bytes(S, H, D, L)
    assert need > _lib.PA_NOALLOC_WORKSPACE_BYTES
    assert noalloc(lib, S=S, T=S, H=H, D=D, mcl=L, mb=L // 16, nb=1 << 20, dt=1) == -4
    # the largest such decode batch that fits: about 12,800 tokens for 256 x 40 heads
    fits = max(L for L in range(256, 20000, 256)
               if lib.pa_decode_workspace_bytes(S, H, D, L) <= _lib.PA_NOALLOC_WORKSPACE_BYTES)
    assert 12000 <= fits <= 13000
