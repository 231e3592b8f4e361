"""Pins of the oracle's container decoder as the CPU baseline runs it:
chunk-parallel decoding (`or_decode_chunks`, any thread count, any chunk
range) with the super-weight patch, against the result's plain definition
(`dequant_direct` on the original symbols: lossless decoding, then one fp32
multiply and a bf16 rounding per weight, then the listed super-weight bits;
"Float8@2bits: Entropy Coding Enables Data-Free Model Compression", section 2,
technical components 1, 3 and 4). Every container here comes from the
oracle's own encoder on oracle-built tables. No GPU code."""
import numpy as np
import pytest

import oracle
import synth


def _escape_tensor(rows, cols, Z, seed):
    """An int8 tensor with super weights at chunk and group boundaries and at
    random places."""
    spec = synth.TensorSpec("down", rows, cols, synth.DTYPE_INT8, 2.1, 0)
    t = synth.make_tensor(4, seed, 6, spec=spec)
    n = rows * cols
    rng = np.random.default_rng(seed)
    pos = {0, n - 1, Z - 1, Z, 2 * Z - 1, 2 * Z + 511, 512, 513}
    pos |= set(int(p) for p in rng.integers(0, n, 12))
    idx = np.array(sorted(p for p in pos if p < n), dtype=np.uint64)
    sym = t.symbols.copy()
    sym[idx.astype(np.int64)] = 0x80
    val = rng.integers(0, 1 << 16, idx.size).astype(np.uint16)
    val[0] = 0x7F80   # +inf: the stored bits win over any arithmetic
    val[1] = 0x0001   # a bf16 subnormal
    return sym, t.scales, idx, val


@pytest.mark.parametrize("codec", [oracle.CODEC_RANS, oracle.CODEC_HUFF])
def test_chunk_parallel_decode_with_escapes_matches_definition(codec):
    rows, cols, Z, K = 24, 4096, 8192, 8
    sym, scales, idx, val = _escape_tensor(rows, cols, Z, 3)
    table = (oracle.build_freq(sym) if codec == oracle.CODEC_RANS
             else oracle.huff_lengths(np.bincount(sym, minlength=256).astype(np.uint64)))
    c = oracle.encode(oracle.DTYPE_INT8, rows, cols, sym, scales, table, Z, K, esc_enabled=True,
                      esc_code=0x80, esc_idx=idx, esc_val=val, codec=codec)
    exp = oracle.dequant_direct(oracle.DTYPE_INT8, sym, cols, scales, idx, val)
    assert np.all(exp[idx.astype(np.int64)] == val)
    n_chunks = oracle.header(c)["n_chunks"]
    for threads in (1, 2, 5, 16):
        out = np.full(sym.size, 0x1234, np.uint16)
        su = np.full(sym.size, 0xA5, np.uint8)
        assert oracle.decode_chunks(c, 0, n_chunks, threads, bf16_out=out, sym_out=su) == 0
        assert np.array_equal(out, exp), threads
        assert np.array_equal(su, sym), threads
    # a sub-range of chunks writes exactly its own positions
    out = np.full(sym.size, 0x1234, np.uint16)
    assert oracle.decode_chunks(c, 1, 3, 4, bf16_out=out) == 0
    lo, hi = Z, 3 * Z
    assert np.array_equal(out[lo:hi], exp[lo:hi])
    assert np.all(out[:lo] == 0x1234) and np.all(out[hi:] == 0x1234)


def test_chunk_parallel_decode_segments_and_e4m3():
    rows, cols, Z, K, seg = 16, 8192, 4096, 4, 8
    spec = synth.TensorSpec("q", rows, cols, synth.DTYPE_E4M3, 2.1, 0)
    t = synth.make_tensor(3, 5, 0, spec=spec)
    sym = t.symbols.copy()
    rng = np.random.default_rng(8)
    idx = np.array(sorted(set(int(p) for p in rng.integers(0, sym.size, 9)) | {Z * seg - 1, Z * seg}),
                   dtype=np.uint64)
    sym[idx.astype(np.int64)] = 0x7F    # the E4M3 escape code (a NaN code otherwise)
    val = rng.integers(0, 1 << 16, idx.size).astype(np.uint16)
    n_chunks = -(-sym.size // Z)
    tabs = np.stack([oracle.build_freq(sym[g * seg * Z:(g + 1) * seg * Z])
                     for g in range(-(-n_chunks // seg))])
    c = oracle.encode(oracle.DTYPE_E4M3, rows, cols, sym, t.scales, tabs, Z, K, esc_enabled=True,
                      esc_code=0x7F, esc_idx=idx, esc_val=val, seg_chunks=seg)
    exp = oracle.dequant_direct(oracle.DTYPE_E4M3, sym, cols, t.scales, idx, val)
    for threads in (1, 3, 16):
        out = np.zeros(sym.size, np.uint16)
        assert oracle.decode_chunks(c, 0, n_chunks, threads, bf16_out=out) == 0
        assert np.array_equal(out, exp), threads
