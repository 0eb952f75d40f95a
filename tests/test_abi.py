"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/nsa.h declares, and every argument check returns its
status code before anything is launched."""
import ctypes
import os
import re

import pytest

import sparse_attention_long_compress_amd as nsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsa.h")

OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EWS, EALIGN = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nsa_[a-z_]+)\s*\(", src)))


def params(**kw):
    base = dict(B=1, T=1024, Hq=4, Hkv=1, D=64, top_k=4, window=128, dtype=nsa.NSA_BF16)
    base.update(kw)
    return nsa.make_params(base["B"], base["T"], base["Hq"], base["Hkv"], base["D"],
                           top_k=base["top_k"], window=base["window"], dtype=base["dtype"],
                           flags=base.get("flags", 0), block=base.get("block", 64))


def test_library_exports_every_declared_function():
    L = nsa.lib()
    names = declared_functions()
    assert set(nsa.EXPORTED) == set(names), names
    for n in names:
        assert hasattr(L, n), n
    assert L.nsa_abi_version() == 1


def test_status_strings_cover_all_codes():
    for code in (OK, ENULL, ESHAPE, EDTYPE, EUNSUP, EWS, EALIGN, -7):
        assert nsa.status_string(code).startswith("NSA_")
    assert "UNKNOWN" in nsa.status_string(-99)


@pytest.mark.parametrize("kw,code", [
    ({}, OK),
    ({"B": 0}, ESHAPE),
    ({"Hq": 6, "Hkv": 4}, ESHAPE),
    ({"top_k": 1}, ESHAPE),
    ({"window": 0}, ESHAPE),
    ({"dtype": 7}, EDTYPE),
    ({"D": 96}, EUNSUP),
    ({"T": 1000}, EUNSUP),
    ({"block": 32}, EUNSUP),
    ({"Hq": 12, "Hkv": 4}, EUNSUP),
    ({"top_k": 33}, EUNSUP),
    ({"flags": 16}, EUNSUP),
    ({"T": 65536 + 64}, EUNSUP),
    ({"Hq": 32, "Hkv": 2, "D": 128}, OK),
    ({"D": 128, "dtype": nsa.NSA_FP32}, EUNSUP),
])
def test_check_params(kw, code):
    p = params(**kw)
    assert nsa.lib().nsa_check_params(ctypes.byref(p)) == code


def test_forward_kernel_names():
    # bf16, head_dim 64, four heads per group, window within 32 blocks: the
    # packed-selection kernel; everything else the general one; NULL if invalid
    assert nsa.forward_kernel(params(T=8192, Hq=16, Hkv=4, top_k=16, window=512)) == "sel_compact_kernel"
    assert nsa.forward_kernel(params(T=8192, Hq=16, Hkv=4, D=128, top_k=16, window=512)) == "sel_win_kernel"
    assert nsa.forward_kernel(params(T=8192, Hq=16, Hkv=4, top_k=16, window=4096)) == "sel_win_kernel"
    assert nsa.forward_kernel(params(dtype=nsa.NSA_FP32)) == "sel_win_kernel"
    assert nsa.lib().nsa_forward_kernel(ctypes.byref(params(D=96))) is None
    with pytest.raises(nsa.NsaError, match="UNSUPPORTED"):
        nsa.forward_kernel(params(D=96))


def test_check_params_null():
    assert nsa.lib().nsa_check_params(None) == ENULL


def test_workspace_size_is_monotone_and_zero_when_invalid():
    L = nsa.lib()
    prev_f = prev_b = 0
    for T in (64, 128, 1024, 4096, 8192, 32768):
        p = params(T=T, Hq=16, Hkv=4, D=128)
        f = L.nsa_workspace_size(ctypes.byref(p), 0)
        b = L.nsa_workspace_size(ctypes.byref(p), 1)
        assert f > prev_f and b > prev_b
        prev_f, prev_b = f, b
    for B in (1, 2, 4):
        p = params(B=B)
        assert L.nsa_workspace_size(ctypes.byref(p), 0) > 0
    assert L.nsa_workspace_size(ctypes.byref(params(D=96)), 0) == 0


FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails its checks first


def test_forward_argument_errors_launch_nothing():
    L = nsa.lib()
    p = params()
    ws = L.nsa_workspace_size(ctypes.byref(p), 0)
    f = lambda *a: L.nsa_forward(*a)
    ok = [FAKE] * 4
    # null inputs / output
    for i in range(4):
        args = list(ok)
        args[i] = None
        assert f(*args, ctypes.byref(p), FAKE, None, None, None, FAKE, ws, None) == ENULL
    assert f(*ok, ctypes.byref(p), None, None, None, None, FAKE, ws, None) == ENULL
    # INDICES_IN needs the table
    pi = params(flags=nsa.INDICES_IN)
    assert f(*ok, ctypes.byref(pi), FAKE, None, None, None, FAKE, ws, None) == ENULL
    # workspace missing / too small
    assert f(*ok, ctypes.byref(p), FAKE, None, None, None, None, ws, None) == EWS
    assert f(*ok, ctypes.byref(p), FAKE, None, None, None, FAKE, ws - 1, None) == EWS
    # misaligned pointers
    assert f(FAKE + 2, *ok[1:], ctypes.byref(p), FAKE, None, None, None, FAKE, ws, None) == EALIGN
    assert f(*ok, ctypes.byref(p), FAKE, None, FAKE + 4, None, FAKE, ws, None) == EALIGN
    assert f(*ok, ctypes.byref(p), FAKE, None, None, None, FAKE + 16, ws, None) == EALIGN
    # bad params come first
    bad = params(D=96)
    assert f(*ok, ctypes.byref(bad), FAKE, None, None, None, FAKE, ws, None) == EUNSUP
    assert f(*ok, None, FAKE, None, None, None, FAKE, ws, None) == ENULL


def test_other_entry_points_argument_errors():
    L = nsa.lib()
    p = params()
    ws = L.nsa_workspace_size(ctypes.byref(p), 0)
    wsb = L.nsa_workspace_size(ctypes.byref(p), 1)
    assert L.nsa_pool(None, FAKE, ctypes.byref(p), FAKE, FAKE, None) == ENULL
    assert L.nsa_pool(FAKE, FAKE, ctypes.byref(p), FAKE + 8, FAKE, None) == EALIGN
    assert L.nsa_compress_select(FAKE, FAKE, FAKE, ctypes.byref(p), FAKE, None, FAKE, ws,
                                 None) == ENULL
    assert L.nsa_compress_select(FAKE, FAKE, FAKE, ctypes.byref(p), FAKE, FAKE, FAKE, ws - 1,
                                 None) == EWS
    args = [FAKE] * 8
    assert L.nsa_select_bwd(*args, ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, wsb - 1, None) == EWS
    args[4] = None
    assert L.nsa_select_bwd(*args, ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, wsb, None) == ENULL


def test_noalloc_argument_errors_launch_nothing():
    # checked before the scratch array's device address is looked up: no GPU needed
    L = nsa.lib()
    f = ctypes.c_void_p(FAKE)
    small = params(T=8192, Hq=16, Hkv=4, top_k=16, window=512)
    assert L.nsa_workspace_size(ctypes.byref(small), 0) <= nsa.NOALLOC_SCRATCH_BYTES
    assert L.nsa_forward_noalloc(None, f, f, f, ctypes.byref(small), f, None, None, None, None) == ENULL
    idx_in = params(T=8192, Hq=16, Hkv=4, top_k=16, window=512, flags=nsa.INDICES_IN)
    assert L.nsa_forward_noalloc(f, f, f, f, ctypes.byref(idx_in), f, None, None, None, None) == ENULL
    big = params(B=4, T=8192, Hq=16, Hkv=4, D=128, top_k=16, window=512)
    assert L.nsa_workspace_size(ctypes.byref(big), 0) > nsa.NOALLOC_SCRATCH_BYTES
    assert L.nsa_forward_noalloc(f, f, f, f, ctypes.byref(big), f, None, None, None, None) == EWS
    assert L.nsa_forward_noalloc(f, f, f, f, ctypes.byref(params(D=96)), f, None, None, None,
                                 None) == EUNSUP
