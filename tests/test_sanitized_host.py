"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the Block Manager against its Python model over random operation
sequences, and every argument-rejection test of the C ABI, run in a child
process against a libmapflow whose host translation units are instrumented.
"""
from __future__ import annotations

import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HOST_TESTS = ["tests/test_block_manager.py", "tests/test_abi_host.py"]

PROBE = r"""
import ctypes, os
import cross_model_sparse_amd as mf
L = mf.load()
maps = open('/proc/self/maps').read()
assert os.environ['MAPFLOW_LIB'] in maps, 'sanitized library not mapped'
ctypes.CDLL(None).__asan_init          # the runtime is live in this process
print('sanitized library loaded, ABI', L.mf_abi_version())
"""


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    import sanitized_host_build as sb
    return sb.build(tmp_path_factory.mktemp("san"))


def _run(args, lib, timeout):
    import sanitized_host_build as sb
    return subprocess.run([sys.executable, *args], cwd=ROOT, env=sb.env_for(lib),
                          capture_output=True, text=True, timeout=timeout)


def test_sanitized_library_is_instrumented(san_lib):
    und = subprocess.run(["nm", "-u", str(san_lib)], capture_output=True, text=True).stdout
    assert "__asan_report_load8" in und and "__ubsan_handle_" in und
    r = _run(["-c", PROBE], san_lib, 120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized library loaded" in r.stdout


def test_host_tests_run_clean_under_sanitizers(san_lib):
    r = _run(["-m", "pytest", *HOST_TESTS, "-m", "not gpu", "-q", "-x", "-p", "no:cacheprovider"],
             san_lib, 900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-6000:]
    assert "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in out and "failed" not in out
