"""The debug build's precondition checks on the host (no GPU): the range
logic of debug_checks.h compiled with the host compiler and run on edge
values, the error bits the header documents, and which library is which
(the debug library reports itself and takes an error word; the release
library refuses one)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

from hashed_gram_embedding_amd import build as bld
from hashed_gram_embedding_amd import engram as eg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hashed_gram_embedding_amd", "csrc")


def test_range_checks_on_the_host(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "debug_checks_host"
    subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-I", CSRC,
                    os.path.join(ROOT, "tests", "native", "debug_checks_host.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all passed" in r.stdout


def test_error_bits_match_the_header():
    hdr = open(os.path.join(ROOT, "include", "engram.h")).read()
    dev = open(os.path.join(CSRC, "debug_checks.h")).read()
    for name, kname, val in (("TOKEN", "kErrToken", eg.ERR_TOKEN), ("ROW", "kErrRow", eg.ERR_ROW),
                             ("SLOT", "kErrSlot", eg.ERR_SLOT), ("HOT_ROW", "kErrHotRow", eg.ERR_HOT_ROW)):
        m = re.search(rf"#define ENGRAM_ERR_{name} (\d+)u", hdr)
        k = re.search(rf"constexpr uint32_t {kname} = (\d+)u;", dev)
        assert m and k and int(m.group(1)) == int(k.group(1)) == val, name


@pytest.mark.skipif(not (os.path.exists(bld.LIB) and os.path.exists(bld.LIB_DEBUG)), reason="libraries not built")
def test_release_and_debug_libraries():
    rel, dbg = eg.load_library(bld.LIB), eg.load_library(bld.LIB_DEBUG)
    assert rel.engram_debug_checks() == 0 and dbg.engram_debug_checks() == 1
    assert rel.engram_debug_set_error_word(ctypes.c_void_p(0x10000)) == eg.EUNSUPPORTED
    bits = ctypes.c_uint32(7)
    assert rel.engram_debug_read_errors(ctypes.byref(bits)) == eg.EUNSUPPORTED
    assert dbg.engram_debug_set_error_word(ctypes.c_void_p(0x10002)) == eg.EINVAL        # misaligned
    assert dbg.engram_debug_set_error_word(None) == eg.OK
    assert dbg.engram_debug_read_errors(ctypes.byref(bits)) == eg.EINVAL                  # no word set
    assert dbg.engram_debug_read_errors(None) == eg.EINVAL
    # the debug build exports the same entry points
    out = subprocess.run(["nm", "-D", "--defined-only", bld.LIB_DEBUG], capture_output=True, text=True).stdout
    assert sorted(set(re.findall(r" T (engram_\w+)", out))) == sorted(eg.exported_names())
