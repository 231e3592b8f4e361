"""GPU parity of containers with adaptive (per-segment) frequency tables
through the same C ABI calls: symbols byte-exact, bf16 bit-exact, fused GEMV
one-hot exact and within the fp32 bound. Containers from the library encoder
(byte-equal to the oracle's, CPU tests); expected values from the oracle."""
import numpy as np
import pytest

import oracle
import synth
from conftest import gpu_available
from gpu_util import Packed, assert_same, encode, expected_bf16, log, run_bf16, run_u8
from rans_decode_amd import eq
from test_gpu_gemv import check_close, one_hot_exact, run_gemv

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def seg_encode(t, Z, K, seg):
    sp = t.spec
    esc = t.esc_idx.size > 0
    return eq.encode_host(None, sp.dtype, sp.rows, sp.cols, t.symbols, t.scales,
                          t.esc_idx if esc else None, t.esc_val if esc else None,
                          esc_code=t.esc_code if esc else 0, chunk_symbols=Z, lane_run=K, seg_chunks=seg)


def _check(t, Z, K, seg, what):
    blob = seg_encode(t, Z, K, seg)
    assert eq.parse_header(blob).seg_chunks == seg
    c = eq.DeviceContainer(blob, device="cuda")
    got, st = run_bf16([c], t.spec.n)
    assert st == 0, f"{what}: status {st}"
    assert_same(got, expected_bf16(t), f"{what} bf16")
    sym, st = run_u8([c], t.spec.n)
    assert st == 0
    assert_same(sym, t.symbols, f"{what} symbols")
    return c


def test_drifting_tensor_segments_of_8_and_16():
    t = synth.drift_tensor(512, 8192, bands=16)
    for seg in (8, 16):
        log(f"case segments drift seg={seg}")
        _check(t, 65536, 8, seg, f"drift seg {seg}")
    one = encode(t).size
    many = seg_encode(t, 65536, 8, 8).size
    log(f"drift tensor: one table {one} B, per-segment tables {many} B")
    assert many < one


@pytest.mark.parametrize("K", [1, 4, 8, 16])
def test_lane_runs_escapes_and_tails(K):
    spec = synth.TensorSpec("t", 37, 3000, synth.DTYPE_INT8, 2.4, 3)
    t = synth.make_tensor(4, 120 + K, 6, spec=spec)
    _check(t, 64 * K * 2, K, 8, f"K={K}")
    spec3 = synth.TensorSpec("e", 20, 4096, synth.DTYPE_E4M3, 2.1, 2)
    t3 = synth.make_tensor(3, 130 + K, 6, spec=spec3)
    _check(t3, 64 * K * 4, K, 16, f"E4M3 K={K}")


def test_fused_gemv_and_mixed_block():
    t = synth.drift_tensor(96, 8192, bands=6, seed=3)
    c = eq.DeviceContainer(seg_encode(t, 65536, 8, 8), device="cuda")
    w = expected_bf16(t).reshape(96, 8192)
    x = oracle.bf16_rne(np.random.default_rng(2).standard_normal(8192).astype(np.float32))
    (y,), st = run_gemv([c], [x], [96])
    assert st == 0
    check_close(y, w, x, "segments gemv")
    one_hot_exact(c, w, [0, 4097, 8191], "segments gemv")
    # segments, one table and Huffman tensors in one call
    tensors = [synth.drift_tensor(40, 4096, bands=4, seed=s) for s in range(3)]
    blobs = [seg_encode(tensors[0], 16384, 8, 8), encode(tensors[1]), encode(tensors[2], codec=1)]
    pk = Packed(blobs)
    offs = [0, tensors[0].spec.n, tensors[0].spec.n * 2]
    got, st = run_bf16(pk.items, offs[-1] + tensors[2].spec.n, offsets=offs)
    assert st == 0
    for tt, o in zip(tensors, offs):
        assert_same(got[o:o + tt.spec.n], expected_bf16(tt), "mixed")


def test_single_symbol_segment():
    """A segment whose chunks hold one byte only: its table has f = 4096 in
    every slot-table entry (the other segments are ordinary); decode to
    bytes, bf16 and the fused GEMV against the oracle."""
    rng = np.random.default_rng(17)
    rows, cols, Z, K, seg = 64, 8192, 8192, 8, 8
    spec = synth.TensorSpec("t", rows, cols, synth.DTYPE_INT8, 2.1, 0)
    t = synth.make_tensor(4, 140, 0, spec=spec)
    one = seg * Z                            # segment 1 = flat positions [one, 2 * one)
    t.symbols[one:2 * one] = 0x03
    t.scales = rng.uniform(0.005, 0.015, rows).astype(np.float32)
    blob = seg_encode(t, Z, K, seg)
    h = eq.parse_header(blob)
    tabs = blob[h.off_freq:h.off_freq + 512 * 4].view(np.uint16).reshape(4, 256)
    assert tabs[1, 3] == 4096 and tabs[1].sum() == 4096 and np.count_nonzero(tabs[0]) > 1
    log("case single-symbol segment")
    c = _check(t, Z, K, seg, "single-symbol segment")
    w = expected_bf16(t).reshape(rows, cols)
    x = oracle.bf16_rne(rng.standard_normal(cols).astype(np.float32))
    (y,), st = run_gemv([c], [x], [rows])
    assert st == 0
    check_close(y, w, x, "single-symbol segment gemv")
    one_hot_exact(c, w, [0, 5000, cols - 1], "single-symbol segment gemv")
