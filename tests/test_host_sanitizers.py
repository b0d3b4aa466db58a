"""The library's host C++ under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU): the
schedule, the draft-tree builder, the commit's path validation and the error text, built with
g++ into a host-only library (gated_deltanet_tree_amd/build_host_san.py).

  * tests/test_schedule_lib.py and tests/test_ddtree_lib.py run against it in a child process
    (the binding's GDN_TREE_HOST_LIB switch, the ASan runtime preloaded): bit-exact schedules of
    every small tree and 10^4 random ones, malformed parents, offsets, capacities and budgets;
  * tests/host_san_commit.cpp drives the commit's path validation with valid and malformed
    paths and offsets, each array in a heap block of exactly its size.
Any sanitizer report ends the child with an error, which fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

from gated_deltanet_tree_amd import build_host_san

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_dir(tmp_path_factory):
    if shutil.which(os.environ.get("CXX", "g++")) is None:
        pytest.skip("no host C++ compiler")
    d = tmp_path_factory.mktemp("gdn_san")
    build_host_san.build(str(d))
    return d


def _clean(out):
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_host_library_tests_under_asan_ubsan(san_dir):
    env = build_host_san.runtime_env(str(san_dir / build_host_san.LIB_NAME))
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join("tests", "test_schedule_lib.py"), os.path.join("tests", "test_ddtree_lib.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    _clean(out)
    assert " passed" in out and " failed" not in out


def test_commit_path_validation_driver(san_dir):
    exe = build_host_san.build_driver(os.path.join(ROOT, "tests", "host_san_commit.cpp"),
                                      str(san_dir))
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    _clean(out)
    assert out.strip().endswith("ok")
