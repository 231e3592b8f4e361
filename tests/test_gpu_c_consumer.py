"""The C ABI from plain C: tests/native/c_consumer (built by build(); it
includes only include/eq.h and the HIP runtime's C API) encodes a tensor
with eq_encode_host, allocates its own device buffers, decodes with
eq_decode_dequant_bf16 and eq_decode_block, and writes the outputs; they are
compared here with the oracle, bf16 and byte codes bit for bit. ("Float8@2bits:
Entropy Coding Enables Data-Free Model Compression", technical summary,
section 2: symbols + frequency table + per-channel scales in, a bf16 weight
matrix out.)"""
import os
import subprocess

import numpy as np
import pytest

import synth
from conftest import ROOT, gpu_available
from gpu_util import expected_bf16, log

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

EXE = os.path.join(ROOT, "tests", "native", "c_consumer")


def _ensure_exe():
    """build() compiles the program; if this tree lacks it, compile it the
    same way (one gcc call, host code only)."""
    if os.path.exists(EXE):
        return
    subprocess.check_call(
        ["gcc", "-std=c11", "-O2", "-D__HIP_PLATFORM_AMD__", "-I", "include", "-I", "/opt/rocm/include",
         "tests/native/c_consumer.c", "-o", "tests/native/c_consumer", "-L", "rans_decode_amd", "-l:libeq.so",
         "-Wl,-rpath,$ORIGIN/../../rans_decode_amd", "-L", "/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib"], cwd=ROOT, timeout=120)


@pytest.mark.parametrize("rows,cols,dtype,K,Z,codec,n_esc", [
    (64, 8192, synth.DTYPE_INT8, 8, 16384, 0, 4),      # rANS, super weights
    (37, 3000, synth.DTYPE_INT8, 1, 4096, 0, 0),       # ragged shape, K = 1, tail chunk
    (48, 4096, synth.DTYPE_E4M3, 4, 8192, 1, 3),       # Huffman, E4M3 escapes
])
def test_c_consumer_matches_the_oracle(tmp_path, rows, cols, dtype, K, Z, codec, n_esc):
    _ensure_exe()
    spec = synth.TensorSpec("t", rows, cols, dtype, 2.1 if dtype == synth.DTYPE_INT8 else 2.3, n_esc)
    t = synth.make_tensor(4, 150 + K, 6, spec=spec)
    n = rows * cols
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([dtype, K, Z, codec, t.esc_code if t.esc_idx.size else 0, t.esc_idx.size],
                         dtype=np.uint32).tobytes())
        f.write(np.array([rows, cols], dtype=np.uint64).tobytes())
        f.write(np.ascontiguousarray(t.symbols, dtype=np.uint8).tobytes())
        f.write(np.ascontiguousarray(t.scales, dtype=np.float32).tobytes())
        f.write(np.ascontiguousarray(t.esc_idx, dtype=np.uint64).tobytes())
        f.write(np.ascontiguousarray(t.esc_val, dtype=np.uint16).tobytes())
    log(f"case c_consumer {rows}x{cols} dtype={dtype} K={K} Z={Z} codec={codec} n_esc={n_esc}")
    r = subprocess.run([EXE, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = np.fromfile(outp, dtype=np.uint8)
    status = int(raw[:4].view(np.uint32)[0])
    clen = int(raw[4:12].view(np.uint64)[0])
    bf16 = raw[12:12 + 2 * n].view(np.uint16)
    sym = raw[12 + 2 * n:12 + 3 * n]
    assert status == 0, f"device status {status}"
    assert clen > 0
    assert np.array_equal(sym, t.symbols), "byte codes differ"
    exp = expected_bf16(t)
    bad = np.flatnonzero(bf16 != exp)
    assert bad.size == 0, f"{bad.size} bf16 mismatches, first at {int(bad[0])}"
