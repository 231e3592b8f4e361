"""GPU parity past 2^32: a tensor of more than 2^32 elements (64-bit chunk,
row and super-weight positions) and outputs placed beyond element 2^32 of
the output buffer. Checked against the oracle on sampled outputs (whole
chunks around the 2^32 boundary and at the end, 2^20 random positions, every
super weight), which it computes one by one."""
import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import gpu_available
from gpu_util import log, to_u16
from rans_decode_amd import eq

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

TWO32 = 1 << 32


def expected_at(spec, sym, scales, idx, esc_idx, esc_val):
    """The oracle's bf16 outputs at positions idx (one row per element)."""
    idx = np.asarray(idx, np.int64)
    rows = idx // spec.cols
    exp = oracle.dequant_direct(spec.dtype, sym[idx], 1, scales[rows])
    where = {int(p): int(v) for p, v in zip(esc_idx, esc_val)}
    for j, p in enumerate(idx):
        if int(p) in where:
            exp[j] = where[int(p)]
    return exp


def test_tensor_of_more_than_2pow32_elements():
    # 65,600 x 65,536 int8 codes = 2^32 + 4,194,304 elements (65,600 chunks)
    spec = synth.TensorSpec("big", 65600, 65536, synth.DTYPE_INT8, 2.1, 0)
    n = spec.n
    assert n > TWO32
    log(f"case tensor of {n} elements: generating")
    t = synth.make_tensor(4, 7, 0, spec=spec)
    code = synth.ESC_CODE[spec.dtype]
    esc_idx = np.array([5, TWO32 - 1, TWO32, TWO32 + 123457, n - 1], np.uint64)
    esc_val = np.array([0x4049, 0xC2F6, 0x3F80, 0x7F7F, 0x0001], np.uint16)
    t.symbols[esc_idx.astype(np.int64)] = code
    blob = eq.encode_host(eq.build_tables(t.symbols), spec.dtype, spec.rows, spec.cols, t.symbols, t.scales,
                          esc_idx, esc_val, esc_code=code)
    c = eq.DeviceContainer(blob, device="cuda")
    rng = np.random.default_rng(11)
    idx = np.unique(np.concatenate([
        np.arange(TWO32 - 70000, TWO32 + 70000), np.arange(n - 70000, n), np.arange(0, 70000),
        rng.integers(0, n, 1 << 20), esc_idx.astype(np.int64)]))
    exp = expected_at(spec, t.symbols, t.scales, idx, esc_idx, esc_val)
    di = torch.from_numpy(idx).cuda()

    log("case tensor beyond 2^32: bf16 decode")
    out = torch.empty(n, dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    eq.decode_dequant_bf16([c], out, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    got = to_u16(out[di])
    bad = np.flatnonzero(got != exp)
    assert bad.size == 0, f"{bad.size} bf16 mismatches, first at position {int(idx[bad[0]])}"
    del out

    log("case tensor beyond 2^32: u8 decode")
    sym = torch.empty(n, dtype=torch.uint8, device="cuda")
    eq.decode_block([c], sym, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    gs = sym[di].cpu().numpy()
    assert np.array_equal(gs, t.symbols[idx])
    # and every symbol, compared on the device in slices
    for lo in range(0, n, 1 << 30):
        hi = min(n, lo + (1 << 30))
        ref = torch.from_numpy(t.symbols[lo:hi]).cuda()
        assert torch.equal(sym[lo:hi], ref), f"u8 mismatch in [{lo}, {hi})"
        del ref
    del sym

    log("case tensor beyond 2^32: device encoder")
    dsym = torch.from_numpy(t.symbols).cuda()
    dsc = torch.from_numpy(t.scales).cuda()
    dout, dlen, dst = eq.eq_encode_device(spec.dtype, spec.rows, spec.cols, dsym, dsc,
                                          torch.from_numpy(esc_idx.astype(np.int64)).cuda(),
                                          torch.from_numpy(esc_val.view(np.int16)).cuda(), code)
    torch.cuda.synchronize()
    assert int(dst.item()) == 0
    got_blob = dout[:int(dlen.item())].cpu().numpy()
    assert got_blob.size == blob.size and np.array_equal(got_blob, blob)
    log("case tensor beyond 2^32: the oracle's container")
    ref = oracle.encode(spec.dtype, spec.rows, spec.cols, t.symbols, t.scales, oracle.build_freq(t.symbols),
                        esc_enabled=True, esc_code=code, esc_idx=esc_idx, esc_val=esc_val)
    assert ref.size == got_blob.size and np.array_equal(ref, got_blob)


def test_outputs_beyond_element_2pow32():
    # a tensor whose output straddles element 2^32 of the buffer, and one past it
    spec = synth.TensorSpec("down", 16, 32768, synth.DTYPE_INT8, 2.1, 4)
    t = synth.make_tensor(4, 0, 6, spec=spec)
    blob = eq.encode_host(eq.build_tables(t.symbols), spec.dtype, spec.rows, spec.cols, t.symbols, t.scales,
                          t.esc_idx, t.esc_val, esc_code=t.esc_code)
    c0 = eq.DeviceContainer(blob, device="cuda")
    c1 = eq.DeviceContainer(blob, device="cuda")
    offs = [TWO32 - 3 * 65536, TWO32 + (1 << 20) + 512]  # 4096 guard elements around each
    total = offs[1] + spec.n + 4096
    exp = oracle.dequant_direct(spec.dtype, t.symbols, spec.cols, t.scales, t.esc_idx, t.esc_val)
    log("case outputs beyond element 2^32: bf16")
    out = torch.full((total,), 0x1234, dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    eq.decode_dequant_bf16([c0, c1], out, offsets=offs, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for o in offs:
        got = to_u16(out[o:o + spec.n])
        assert np.array_equal(got, exp), f"bf16 output at offset {o}"
        assert np.all(to_u16(out[o - 4096:o]) == 0x1234) and np.all(to_u16(out[o + spec.n:o + spec.n + 4096]) == 0x1234)
    del out
    log("case outputs beyond element 2^32: u8")
    sym = torch.full((total,), 0xA5, dtype=torch.uint8, device="cuda")
    eq.decode_block([c0, c1], sym, offsets=offs, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for o in offs:
        assert np.array_equal(sym[o:o + spec.n].cpu().numpy(), t.symbols), f"u8 output at offset {o}"
        assert np.all(sym[o - 4096:o].cpu().numpy() == 0xA5)
        assert np.all(sym[o + spec.n:o + spec.n + 4096].cpu().numpy() == 0xA5)
