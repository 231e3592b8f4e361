"""The host library's encoder and parser and the oracle's coder built with
AddressSanitizer + UndefinedBehaviorSanitizer (host code only; no GPU code is
involved) and run over random layouts of every container variant and over
corrupted containers (tests/native/sanitize_driver.c). Byte equality of the
two encoders and the oracle's round trip are re-checked under the
sanitizers."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if shutil.which("gcc") is None or shutil.which("g++") is None:
        pytest.skip("needs gcc and g++")
    d = tmp_path_factory.mktemp("san")
    inc = os.path.join(ROOT, "include")
    objs = []
    for src, comp, std in [("oracle/eq_oracle.c", "gcc", "-std=c11"),
                           ("rans_decode_amd/csrc/host_codec.cpp", "g++", "-std=c++17"),
                           ("tests/native/sanitize_driver.c", "gcc", "-std=c11")]:
        o = str(d / (os.path.basename(src) + ".o"))
        subprocess.check_call([comp, std, *SAN, "-ffp-contract=off", "-I", inc, "-c",
                               os.path.join(ROOT, src), "-o", o])
        objs.append(o)
    exe = str(d / "sanitize_driver")
    subprocess.check_call(["g++", *SAN, *objs, "-o", exe, "-lpthread", "-lm"])
    return exe


@pytest.mark.parametrize("seed", [1, 0x5EED])
def test_host_codec_and_oracle_under_sanitizers(driver, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver, "150", str(seed)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("ok")
