"""Pins of the oracle's dequantisation arithmetic against library routines
and hand-derived bit patterns.

The dequantisation (per-channel scales S times the Int8/Float8 code, "Float8@2bits:
Entropy Coding Enables Data-Free Model Compression", section 2, core concept and
technical component 1) is one binary32 multiply followed by bf16
round-to-nearest-even; both are library routines here: numpy's float32 multiply
and torch's float32 -> bfloat16 conversion (CPU)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import parse_int, read_golden


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_exhaustive_all_fp32_patterns():
    """All 2^32 binary32 patterns, in slices, against torch's conversion.
    NaN inputs must give a NaN (payloads are not compared)."""
    step = 1 << 26
    base = np.arange(step, dtype=np.uint32)
    for s in range(0, 1 << 32, step):
        bits = base + np.uint32(s)
        x = bits.view(np.float32)
        ours = oracle.bf16_rne(x)
        ref = _torch_bf16_bits(x)
        nan_in = np.isnan(x)
        ok = (ours == ref) | nan_in
        assert ok.all(), f"slice {s:#x}: first mismatch at {bits[~ok][0]:#010x}"
        o = ours[nan_in]
        assert np.all(((o & 0x7F80) == 0x7F80) & ((o & 0x7F) != 0))


def _cases(name):
    out = []
    for case in read_golden(name)["case"]:
        sym, sbits, exp = case.split()
        out.append((int(sym), parse_int(sbits), parse_int(exp)))
    return out


@pytest.mark.parametrize("name", ["w3_rne_ties.txt", "w4_denormals.txt"])
def test_hand_pins_ties_and_denormals(name):
    for sym, sbits, exp in _cases(name):
        scale = np.array([sbits], np.uint32).view(np.float32)
        code = np.array([sym & 0xFF], np.uint8)
        got = oracle.dequant_direct(oracle.DTYPE_INT8, code, 1, scale)
        assert int(got[0]) == exp, (sym, hex(sbits), hex(int(got[0])), hex(exp))


def test_e4m3_hand_pins():
    vals = oracle.e4m3_values()
    for case in read_golden("e4m3_codes.txt")["code"]:
        code, v = case.split()
        code = parse_int(code)
        got = float(vals[code])
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v)), (hex(code), got)


def test_e4m3_all_codes_vs_torch():
    ours = oracle.e4m3_values()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # incl. -0


def test_int8_values():
    for c in range(256):
        assert oracle.symbol_value(oracle.DTYPE_INT8, c) == (c if c < 128 else c - 256)


def _library_dequant(dtype, sym, cols, scales):
    if dtype == oracle.DTYPE_INT8:
        v = sym.view(np.int8).astype(np.float32)
    else:
        v = torch.from_numpy(sym).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    rows = np.arange(sym.size) // cols
    prod = (v * scales[rows]).astype(np.float32)   # one binary32 multiply (numpy)
    return _torch_bf16_bits(prod)


@pytest.mark.parametrize("cfg,t", [(1, 0), (3, 1), (3, 6)])
def test_dequant_direct_vs_library(cfg, t):
    tensor = synth.make_tensor(cfg, 0, t)
    sp = tensor.spec
    got = oracle.dequant_direct(sp.dtype, tensor.symbols, sp.cols, tensor.scales)
    exp = _library_dequant(sp.dtype, tensor.symbols, sp.cols, tensor.scales)
    assert np.array_equal(got, exp)


def test_dequant_all_codes_times_edge_scales():
    """Every code against scales that reach subnormal, tie and overflow cases."""
    scale_bits = np.array([0x3C23D70A, 0x00080000, 0x00000001, 0x3F808000, 0x3F818000,
                           0x7F7FFFFF, 0xBF800000, 0x80000000, 0x00800000, 0x7E800000,
                           0x3A000000, 0x43E00000], np.uint32)
    scales = scale_bits.view(np.float32)
    for dtype in (oracle.DTYPE_INT8, oracle.DTYPE_E4M3):
        codes = np.arange(256, dtype=np.uint8)
        if dtype == oracle.DTYPE_E4M3:
            codes = codes[(codes & 0x7F) != 0x7F]
        sym = np.tile(codes, scales.size)
        got = oracle.dequant_direct(dtype, sym, codes.size, scales)
        exp = _library_dequant(dtype, sym, codes.size, scales)
        assert np.array_equal(got, exp)


def test_escape_patch_wins():
    sym = np.array([0x80, 0x01, 0x80, 0x02], np.uint8)
    out = oracle.dequant_direct(oracle.DTYPE_INT8, sym, 2, np.array([0.5, 0.25], np.float32),
                                np.array([0, 2], np.uint64), np.array([0x4120, 0xC2C8], np.uint16))
    assert list(out) == [0x4120, _torch_bf16_bits(np.array([0.5], np.float32))[0], 0xC2C8,
                         _torch_bf16_bits(np.array([0.5], np.float32))[0]]
