"""Host-only build of the library's plain C++ parts with AddressSanitizer and
UndefinedBehaviorSanitizer (g++; no device code, no HIP runtime): the schedule, the draft-tree
builder, the commit's path validation and the error text.  Host-side tests load it through the
binding's GDN_TREE_HOST_LIB switch:

    python -m gated_deltanet_tree_amd.build_host_san /tmp/gdn_san
    GDN_TREE_HOST_LIB=/tmp/gdn_san/libgdn_host_san.so \\
    LD_PRELOAD=$(g++ -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \\
        python -m pytest tests/test_schedule_lib.py tests/test_ddtree_lib.py

(`tests/test_host_sanitizers.py` does exactly this, plus a sanitized C++ driver of the commit's
path validation.)
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
HOST_SOURCES = ["errors.cpp", "schedule.cpp", "ddtree.cpp", "commit_host.cpp"]
SAN_FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall"]
LIB_NAME = "libgdn_host_san.so"


def _gxx() -> str:
    return os.environ.get("CXX", "g++")


def build(out_dir: str) -> str:
    """Compile the host sources into out_dir/libgdn_host_san.so; returns its path."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, LIB_NAME)
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES]
    subprocess.run([_gxx()] + SAN_FLAGS + ["-shared", "-fPIC", "-o", out] + srcs, check=True)
    return out


def build_driver(driver_src: str, out_dir: str) -> str:
    """A sanitized host executable from driver_src and the host sources (it may call the
    library's internal host functions declared in csrc/gdn_internal.h)."""
    os.makedirs(out_dir, exist_ok=True)
    out = os.path.join(out_dir, os.path.splitext(os.path.basename(driver_src))[0])
    srcs = [driver_src] + [os.path.join(CSRC, s) for s in HOST_SOURCES]
    subprocess.run([_gxx()] + SAN_FLAGS + ["-I", CSRC, "-o", out] + srcs, check=True)
    return out


def runtime_env(lib_path: str | None = None) -> dict:
    """Environment for a Python process that loads the sanitized library: the ASan runtime
    preloaded (the interpreter itself is not instrumented), leak checks off (the interpreter
    keeps its allocations), the first report fatal."""
    env = dict(os.environ)
    asan = subprocess.run([_gxx(), "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    if lib_path:
        env["GDN_TREE_HOST_LIB"] = lib_path
    return env


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(HERE, "_san")))
