"""CPU checks of the C-ABI library: it loads, exports every declared entry
point, and its pure host helpers agree with the oracle's readings."""
import ctypes
import os
import re

import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "oasis.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(oasis_[a-z_]+)\s*\(", src)))


def test_header_declares_the_decode_step_calls():
    names = _declared()
    for n in ["oasis_create", "oasis_append_kv", "oasis_predict", "oasis_select_and_fetch",
              "oasis_sparse_attn", "oasis_destroy", "oasis_load_prefix",
              "oasis_topk_from_scores"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    import lookahead_sparse_kv_oasis_amd as L
    lib = L.lib()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(L.EXPORTS) == set(_declared())


def test_kv_bytes_per_token_helper_matches_oracle():
    import lookahead_sparse_kv_oasis_amd as L
    for args in [(126, 8, 128, 2), (80, 8, 128, 2), (36, 8, 128, 2), (1, 2, 64, 4)]:
        assert L.kv_bytes_per_token(*args) == oracle.kv_bytes_per_token(*args)


def test_cap_from_ratio_helper_matches_oracle_reading():
    import lookahead_sparse_kv_oasis_amd as L
    for k in [8, 128, 256]:
        for r in synth.FETCH_RATIO_SWEEP + [0.0, 0.5, 0.999, 1.0, 3.0]:
            exp = oracle.cap_from_ratio(r, k) if r is not None else k
            if r is not None and r >= 1.0:
                exp = k
            got = L.cap_from_ratio(k if r is None else r, k) if r is not None else k
            assert got == exp, (r, k, got, exp)


def test_strerror_covers_every_status():
    import lookahead_sparse_kv_oasis_amd as L
    lib = L.lib()
    for s in range(0, -8, -1):
        assert lib.oasis_strerror(s).decode() != "unknown status"


def test_create_rejects_bad_layouts_without_touching_the_gpu():
    """Shape validation happens before any HIP call."""
    import lookahead_sparse_kv_oasis_amd as L
    lib = L.lib()
    h = ctypes.c_void_p()
    bad = [
        L.oasis_layout(1, 6, 4, 64, 0, 2, 0, 0, 1024),     # Hq % Hkv != 0
        L.oasis_layout(1, 4, 2, 60, 0, 2, 0, 0, 1024),     # d % 8 != 0
        L.oasis_layout(1, 4, 2, 64, 7, 2, 0, 0, 1024),     # dtype
        L.oasis_layout(1, 4, 2, 64, 0, 2, 4, 0, 1024),     # S < K
        L.oasis_layout(0, 4, 2, 64, 0, 2, 0, 0, 1024),     # batch
    ]
    for lay in bad:
        assert lib.oasis_create(ctypes.byref(lay), 16, 128, 0.02, ctypes.byref(h)) == L.OASIS_E_INVAL
    lay = L.oasis_layout(1, 4, 2, 64, 0, 2, 0, 0, 1024)
    assert lib.oasis_create(ctypes.byref(lay), 0, 128, 0.02, ctypes.byref(h)) == L.OASIS_E_INVAL
    assert lib.oasis_create(ctypes.byref(lay), 16, 128, -1.0, ctypes.byref(h)) == L.OASIS_E_INVAL
    assert lib.oasis_create(None, 16, 128, 0.02, ctypes.byref(h)) == L.OASIS_E_INVAL
    assert lib.oasis_destroy(None) == L.OASIS_E_INVAL


def test_stream_read_rejects_bad_arguments_without_touching_the_gpu():
    """Argument checks happen before any launch (the pointers here are never
    dereferenced)."""
    import lookahead_sparse_kv_oasis_amd as L
    f = L.lib().oasis_stream_read
    for buf, nbytes, sink, wgs in [(None, 16, 64, 1), (64, 16, None, 1), (72, 16, 64, 1),
                                   (64, 0, 64, 1), (64, 24, 64, 1), (64, 16, 64, 0),
                                   (64, 16, 64, 65537)]:
        assert f(buf, nbytes, sink, wgs, None) == L.OASIS_E_INVAL, (buf, nbytes, sink, wgs)
