"""Host code of the library under AddressSanitizer and UBSan (CPU only).

The host sources (trie build, schedule and plan image, path plan, RL
weights, error reporting) are compiled with g++ -fsanitize=address,undefined
together with tests/asan/host_driver.c, which calls every host entry point
on random and edge-case inputs (empty trees, empty sequences, shared
prefixes, all block sizes, error paths).  Any memory error, leak or
undefined behaviour fails the run."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "prefix_tree_attention_dfs_amd", "csrc")
HOST = ["tree_host.cpp", "path_host.cpp"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc/g++")
def test_host_code_under_asan_ubsan():
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    with tempfile.TemporaryDirectory() as d:
        objs = []
        for src in HOST:
            o = os.path.join(d, src + ".o")
            subprocess.run(["g++", "-std=c++17", "-c", os.path.join(CSRC, src), "-o", o] + flags, check=True)
            objs.append(o)
        drv = os.path.join(d, "drv.o")
        subprocess.run(["gcc", "-std=c11", "-c", os.path.join(ROOT, "tests", "asan", "host_driver.c"), "-o", drv]
                       + flags, check=True)
        exe = os.path.join(d, "drv")
        subprocess.run(["g++", "-o", exe, drv] + objs + ["-fsanitize=address,undefined"], check=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout[-2000:] + r.stderr[-4000:]
