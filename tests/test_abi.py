"""The C ABI library without a GPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import subprocess

import pytest

from block_sparse_attention_16_amd import _lib



@pytest.fixture(scope="module", autouse=True)
def _library():
    """Builds libbsa.so when it is missing and hipcc is present (hipcc
    cross-compiles gfx950 without a GPU), so a fresh checkout runs these tests
    instead of skipping them."""
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_attention_16_amd import build as B
        try:
            B.hipcc()
        except RuntimeError:
            pytest.skip("libbsa.so is not built and hipcc is not available to build it")
        B.build(verbose=False)

FAKE = 0x10000      # a 16-byte aligned address that validation never dereferences


def _shape(**kw):
    s = dict(B=1, H=2, N=1024, D=64, block=64, dtype=_lib.BSA_BF16)
    s.update(kw)
    return _lib.BsaShape(**s)


def _csr(cap=1024):
    return _lib.BsaCsr(FAKE, FAKE + 4096, cap)


def test_library_exports_every_header_function():
    names = _lib.header_functions()
    assert names == sorted(["bsa_backward", "bsa_estimate_mask", "bsa_estimate_mask_hierarchical", "bsa_forward",
                            "bsa_last_error",
                            "bsa_permute_rows", "bsa_select_from_mass", "bsa_select_from_mass_noalloc", "bsa_status_string",
                            "bsa_structured_mask", "bsa_version",
                            "bsa_workspace_size"])
    L = _lib.load()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported


def test_status_strings_and_version():
    L = _lib.load()
    assert L.bsa_status_string(0) == b"ok"
    assert L.bsa_status_string(3) == b"workspace or capacity too small"
    assert L.bsa_version() >= 100


def test_workspace_sizes():
    L = _lib.load()
    s = _shape()
    est = L.bsa_workspace_size(ctypes.byref(s), 0, 0)
    R, D, nb = 2 * 16, 64, 16
    assert est >= 2 * R * D * 4 + R * 4 + R * 4
    fwd = L.bsa_workspace_size(ctypes.byref(s), 1, 100)
    assert fwd >= 100 * 64 * 4          # per-entry, per-query partial sums for the block mass
    sel = L.bsa_workspace_size(ctypes.byref(s), 3, 0)
    assert sel >= R * 4 + R * ((nb + 31) // 32) * 4      # counts + kept-block bitmask
    hier = L.bsa_workspace_size(ctypes.byref(s), 5, 0)
    assert hier >= L.bsa_workspace_size(ctypes.byref(s), 0, 0) + 7 * R * 64 * 4   # 8 key sub-block means per block
    assert L.bsa_workspace_size(ctypes.byref(_shape(D=96)), 0, 0) == 0
    assert L.bsa_workspace_size(ctypes.byref(s), 7, 0) == 0


def _est(L, shape, q=FAKE, k=FAKE, p=0.9, scale=0.0, cand=None, keep=0, out=None, ws=FAKE, ws_bytes=1 << 30):
    out = out if out is not None else _csr()
    return L.bsa_estimate_mask(ctypes.byref(shape), q, k, p, scale, ctypes.byref(cand) if cand else None, keep,
                               ctypes.byref(out), ws, ws_bytes, None)


def test_estimate_validation():
    L = _lib.load()
    s = _shape()
    assert _est(L, s, q=None) == _lib.BSA_ERR_INVALID_ARG
    assert _est(L, s, q=FAKE + 2) == _lib.BSA_ERR_INVALID_ARG          # misaligned
    assert _est(L, s, p=0.0) == _lib.BSA_ERR_INVALID_ARG
    assert _est(L, s, p=1.5) == _lib.BSA_ERR_INVALID_ARG
    assert _est(L, s, p=float("nan")) == _lib.BSA_ERR_INVALID_ARG
    assert _est(L, s, scale=float("inf")) == _lib.BSA_ERR_INVALID_ARG
    assert _est(L, s, keep=-1) == _lib.BSA_ERR_INVALID_ARG
    assert _est(L, s, keep=1025) == _lib.BSA_ERR_INVALID_ARG
    assert _est(L, s, ws_bytes=16) == _lib.BSA_ERR_WORKSPACE
    assert b"workspace" in L.bsa_last_error()
    assert _est(L, _shape(D=96)) == _lib.BSA_ERR_UNSUPPORTED
    assert _est(L, _shape(block=32)) == _lib.BSA_ERR_UNSUPPORTED
    assert _est(L, _shape(dtype=5)) == _lib.BSA_ERR_UNSUPPORTED
    assert _est(L, _shape(N=0)) == _lib.BSA_ERR_INVALID_ARG
    assert _est(L, _shape(N=64 * 4097)) == _lib.BSA_ERR_UNSUPPORTED   # more than 4096 blocks
    assert _est(L, _shape(N=2 ** 31 - 1, block=128)) == _lib.BSA_ERR_UNSUPPORTED   # N + block - 1 past int32
    assert b"blocks per sequence" in L.bsa_last_error()
    out = _csr()
    assert _est(L, s, cand=out, out=out) == _lib.BSA_ERR_INVALID_ARG   # candidate aliases out
    bad = _lib.BsaCsr(FAKE, None, 10)
    assert _est(L, s, out=bad) == _lib.BSA_ERR_INVALID_ARG
    neg = _lib.BsaCsr(FAKE, FAKE, -1)
    assert _est(L, s, out=neg) == _lib.BSA_ERR_INVALID_ARG


def test_hierarchical_estimate_validation():
    L = _lib.load()
    s = _shape()
    need = L.bsa_workspace_size(ctypes.byref(s), 5, 0)

    def call(g, ws_bytes=1 << 30, p=0.9):
        return L.bsa_estimate_mask_hierarchical(ctypes.byref(s), FAKE, FAKE, p, 0.0, None, 0, g,
                                                ctypes.byref(_csr()), FAKE, ws_bytes, None)
    for g in (0, 3, 16, -2):
        assert call(g) == _lib.BSA_ERR_INVALID_ARG
        assert b"sub_blocks" in L.bsa_last_error()
    assert call(4, ws_bytes=need - 256) == _lib.BSA_ERR_WORKSPACE
    assert call(4, p=0.0) == _lib.BSA_ERR_INVALID_ARG


def test_forward_and_backward_validation():
    L = _lib.load()
    s = _shape()
    m = _csr()
    args = [FAKE] * 3
    st = L.bsa_forward(ctypes.byref(s), *args, 0.0, ctypes.byref(m), FAKE, FAKE, FAKE, None, FAKE, 16, None)
    assert st == _lib.BSA_ERR_WORKSPACE
    st = L.bsa_forward(ctypes.byref(s), FAKE, None, FAKE, 0.0, ctypes.byref(m), FAKE, FAKE, None, None, FAKE,
                       1 << 30, None)
    assert st == _lib.BSA_ERR_INVALID_ARG
    st = L.bsa_forward(ctypes.byref(s), *args, 0.0, None, FAKE, FAKE, None, None, FAKE, 1 << 30, None)
    assert st == _lib.BSA_ERR_INVALID_ARG
    st = L.bsa_forward(ctypes.byref(s), *args, 0.0, ctypes.byref(m), FAKE, FAKE, None, FAKE + 4, FAKE, 1 << 30,
                       None)
    assert st == _lib.BSA_ERR_INVALID_ARG                               # misaligned o_f32
    st = L.bsa_forward(ctypes.byref(_shape(dtype=1)), *args, 0.0, ctypes.byref(m), FAKE, FAKE, None, FAKE, FAKE,
                       1 << 30, None)
    assert st == _lib.BSA_ERR_INVALID_ARG                               # o_f32 with fp32 data
    st = L.bsa_backward(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 0.0, ctypes.byref(m), FAKE,
                        FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == _lib.BSA_ERR_INVALID_ARG
    st = L.bsa_backward(ctypes.byref(_shape(dtype=1)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0,
                        ctypes.byref(m), FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == _lib.BSA_ERR_INVALID_ARG                               # o_f32 with fp32 data
    st = L.bsa_backward(ctypes.byref(_shape(D=80)), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 0.0, ctypes.byref(m),
                        FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == _lib.BSA_ERR_UNSUPPORTED


def test_select_from_mass_validation():
    L = _lib.load()
    s = _shape()
    m, o = _csr(), _lib.BsaCsr(FAKE + 8192, FAKE + 16384, 1024)

    def call(shape=s, mask=m, mass=FAKE, p=0.9, keep=0, out=o, ws=FAKE, ws_bytes=1 << 30):
        return L.bsa_select_from_mass(ctypes.byref(shape), ctypes.byref(mask) if mask else None, mass, p, keep,
                                      ctypes.byref(out) if out else None, ws, ws_bytes, None)

    assert call(mass=None) == _lib.BSA_ERR_INVALID_ARG
    assert call(mask=None) == _lib.BSA_ERR_INVALID_ARG
    assert call(out=None) == _lib.BSA_ERR_INVALID_ARG
    assert call(p=0.0) == _lib.BSA_ERR_INVALID_ARG
    assert call(p=1.01) == _lib.BSA_ERR_INVALID_ARG
    assert call(p=float("nan")) == _lib.BSA_ERR_INVALID_ARG
    assert call(keep=-3) == _lib.BSA_ERR_INVALID_ARG
    assert call(out=m) == _lib.BSA_ERR_INVALID_ARG                     # mask aliases out
    assert call(ws_bytes=8) == _lib.BSA_ERR_WORKSPACE
    assert call(shape=_shape(block=96)) == _lib.BSA_ERR_UNSUPPORTED


def test_select_from_mass_noalloc_validation():
    """Host checks of the no-allocation narrowing, before any device call:
    the same argument errors as bsa_select_from_mass, and a shape whose
    counts and bitmask exceed the built-in 16 MiB scratch is refused."""
    L = _lib.load()
    s = _shape()
    m, o = _csr(), _lib.BsaCsr(FAKE + 8192, FAKE + 16384, 1024)

    def call(shape=s, mask=m, mass=FAKE, p=0.9, keep=0, out=o):
        return L.bsa_select_from_mass_noalloc(ctypes.byref(shape), ctypes.byref(mask) if mask else None, mass, p,
                                              keep, ctypes.byref(out) if out else None, None)

    assert call(mass=None) == _lib.BSA_ERR_INVALID_ARG
    assert call(mask=None) == _lib.BSA_ERR_INVALID_ARG
    assert call(out=None) == _lib.BSA_ERR_INVALID_ARG
    assert call(p=0.0) == _lib.BSA_ERR_INVALID_ARG
    assert call(keep=-3) == _lib.BSA_ERR_INVALID_ARG
    assert call(out=m) == _lib.BSA_ERR_INVALID_ARG                     # mask aliases out
    assert call(shape=_shape(block=96)) == _lib.BSA_ERR_UNSUPPORTED
    # 4096 blocks per head, 64 heads: 262,144 rows x (1 + 128) words x 4 bytes > 16 MiB
    big = _shape(B=1, H=64, N=4096 * 64, D=64, block=64)
    assert call(shape=big) == _lib.BSA_ERR_WORKSPACE
    assert b"scratch" in L.bsa_last_error()


def test_structured_mask_validation():
    L = _lib.load()
    s = _shape()
    assert L.bsa_workspace_size(ctypes.byref(s), 4, 0) == L.bsa_workspace_size(ctypes.byref(s), 3, 0)

    def call(kinds=FAKE, prefix=0, frame=16, band=1, period=2, stripes=None, n=0, out=None, ws_bytes=1 << 30,
             shape=s):
        prm = _lib.BsaPatternParams(prefix, frame, band, period, stripes, n)
        o = out if out is not None else _csr()
        return L.bsa_structured_mask(ctypes.byref(shape), kinds, ctypes.byref(prm), ctypes.byref(o), FAKE,
                                     ws_bytes, None)

    assert call(kinds=None) == _lib.BSA_ERR_INVALID_ARG
    assert call(prefix=-1) == _lib.BSA_ERR_INVALID_ARG
    assert call(prefix=1025) == _lib.BSA_ERR_INVALID_ARG
    assert call(frame=0) == _lib.BSA_ERR_INVALID_ARG
    assert call(band=-1) == _lib.BSA_ERR_INVALID_ARG
    assert call(period=0) == _lib.BSA_ERR_INVALID_ARG
    assert call(n=3) == _lib.BSA_ERR_INVALID_ARG                 # stripes count without an array
    assert call(n=-1, stripes=FAKE) == _lib.BSA_ERR_INVALID_ARG
    assert call(ws_bytes=4) == _lib.BSA_ERR_WORKSPACE
    assert call(out=_lib.BsaCsr(FAKE, None, 5)) == _lib.BSA_ERR_INVALID_ARG
    assert call(shape=_shape(D=80)) == _lib.BSA_ERR_UNSUPPORTED


def test_permute_rows_validation():
    L = _lib.load()

    def call(heads=2, n=16, rb=256, src=FAKE, perm=FAKE + (1 << 20), inv=0, dst=FAKE + (1 << 24)):
        return L.bsa_permute_rows(heads, n, rb, src, perm, inv, dst, None)

    assert call(heads=0) == _lib.BSA_ERR_INVALID_ARG
    assert call(n=0) == _lib.BSA_ERR_INVALID_ARG
    assert call(rb=6) == _lib.BSA_ERR_INVALID_ARG
    assert call(rb=0) == _lib.BSA_ERR_INVALID_ARG
    assert call(src=None) == _lib.BSA_ERR_INVALID_ARG
    assert call(perm=None) == _lib.BSA_ERR_INVALID_ARG
    assert call(src=FAKE + 2) == _lib.BSA_ERR_INVALID_ARG           # misaligned
    assert call(inv=2) == _lib.BSA_ERR_INVALID_ARG
    assert call(dst=FAKE + 64) == _lib.BSA_ERR_INVALID_ARG           # overlaps src
    assert call(heads=1 << 20, n=1 << 12, rb=4096) == _lib.BSA_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()
