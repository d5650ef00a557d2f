"""Host-side checks of the C ABI: the library loads and exports every entry
point that include/lola.h declares (no compute call; runs without a GPU)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lola.h")
LIB = os.path.join(ROOT, "sparse_kv_caching_amd", "liblola.so")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lola_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared()
    for must in ("lola_state_init", "lola_state_free", "lola_prefill_chunk", "lola_decode_step"):
        assert must in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="liblola.so not built")
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s+(lola_\w+)", out))
    missing = [n for n in declared() if n not in exported]
    assert not missing, missing


@pytest.mark.skipif(not os.path.exists(LIB), reason="liblola.so not built")
def test_library_loads_and_reports_errors_without_a_device():
    lib = ctypes.CDLL(LIB)
    for n in declared():
        assert hasattr(lib, n)
    lib.lola_strerror.restype = ctypes.c_char_p
    assert lib.lola_strerror(0) == b"ok"
    assert lib.lola_strerror(6) == b"workspace too small"
    # argument validation happens before any HIP call
    lib.lola_state_init.argtypes = [ctypes.c_void_p] * 4
    assert lib.lola_state_init(None, None, None, None) == 1
    lib.lola_last_error.restype = ctypes.c_char_p
    assert b"non-NULL" in lib.lola_last_error()
    lib.lola_state_free.argtypes = [ctypes.c_void_p]
    assert lib.lola_state_free(None) == 0
