import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU check")


def _ensure_built():
    libs = [os.path.join(ROOT, "oracle", "liboracle.so"), os.path.join(ROOT, "synth", "libsynth.so"),
            os.path.join(ROOT, "synth", "libsynth_gpu.so"),
            os.path.join(ROOT, "rans_decode_amd", "libeq.so")]
    if not all(os.path.exists(p) for p in libs):
        import __graft_entry__
        __graft_entry__.build()


_ensure_built()


def read_golden(name):
    """Parse `key = value` lines; repeated keys collect into lists."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            out.setdefault(k, []).append(v)
    return out


def parse_int(tok):
    return int(tok, 0)


@pytest.fixture(scope="session")
def native_checks(tmp_path_factory):
    """Compile tests/native/exhaustive.c (a driver that calls the oracle's
    exported step functions) into a session temp dir."""
    import ctypes
    src = os.path.join(ROOT, "tests", "native", "exhaustive.c")
    out = str(tmp_path_factory.mktemp("native") / "libexhaustive.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", src, "-o", out,
                           "-ldl", "-lpthread"])
    lib = ctypes.CDLL(out)
    return lib


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture
def planted(tmp_path):
    """planted(old, new): a copy of the oracle's C source with one planted
    mistake (old -> new, on the CPU), built and swapped in for the oracle
    package's calls until the test ends."""
    import contextlib

    import oracle

    src_path = os.path.join(ROOT, "oracle", "eq_oracle.c")
    made = []

    def build(old, new):
        src = open(src_path).read()
        assert src.count(old) == 1, f"mutation target not unique: {old!r}"
        p = tmp_path / f"planted{len(made)}.c"
        p.write_text(src.replace(old, new))
        so = str(tmp_path / f"libplanted{len(made)}.so")
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-ffp-contract=off", str(p),
                               "-o", so, "-lpthread"])
        made.append(so)

        @contextlib.contextmanager
        def use():
            saved = oracle.LIB_PATH
            oracle.LIB_PATH = so
            oracle.lib.cache_clear()
            try:
                yield oracle
            finally:
                oracle.LIB_PATH = saved
                oracle.lib.cache_clear()
        return use()

    return build
