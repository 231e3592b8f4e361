"""Pins for adaptive (per-segment) frequency tables in the oracle: container
v1 with flags bit 1, one 12-bit table per `seg_chunks` consecutive chunks
(rANS only). No GPU code.

Pinned by: with every segment table equal to the whole-tensor table the lane
states and words are byte-identical to the one-table container (only the
header and the table section differ); round trips over random layouts;
strictly smaller output than one table on a tensor whose statistics drift;
the rejections."""
import numpy as np
import pytest

import oracle


def _seg_tables(sym, Z, seg):
    n_chunks = -(-sym.size // Z)
    n_seg = -(-n_chunks // seg)
    return np.stack([oracle.build_freq(sym[g * seg * Z:(g + 1) * seg * Z]) for g in range(n_seg)])


def test_equal_tables_give_the_one_table_stream():
    rng = np.random.default_rng(1)
    sym = rng.choice([0, 1, 2, 255, 254], 64 * 8192 + 999, p=[0.5, 0.2, 0.1, 0.15, 0.05]).astype(np.uint8)
    rows, cols = 1, sym.size
    sc = np.ones(rows, np.float32)
    f = oracle.build_freq(sym)
    Z = 8192
    n_chunks = -(-sym.size // Z)
    seg = 16
    tabs = np.tile(f, (-(-n_chunks // seg), 1))
    one = oracle.encode(1, rows, cols, sym, sc, f, Z, 8)
    many = oracle.encode(1, rows, cols, sym, sc, tabs, Z, 8, seg_chunks=seg)
    h1, h2 = oracle.header(one), oracle.header(many)
    assert h2["flags"] & 2 and h2["seg_chunks"] == seg and h1["seg_chunks"] == 0
    assert h2["off_scales"] - h2["off_freq"] >= 512 * tabs.shape[0]
    for a, b in [("off_states", "off_words"), ("off_words", "off_esc_idx")]:
        s1 = one[h1[a]:h1[b]]
        s2 = many[h2[a]:h2[b]]
        assert np.array_equal(s1, s2), a
    d, fl = oracle.decode_symbols(many)
    assert fl == 0 and np.array_equal(d, sym)


def test_random_layouts_round_trip():
    rng = np.random.default_rng(7)
    for it in range(40):
        K = int(rng.choice([1, 2, 4, 8, 16]))
        Z = 64 * K * int(rng.integers(1, 4))
        seg = 8 * int(rng.integers(1, 4))
        n = int(rng.integers(1, Z * seg * 3))
        # the alphabet shifts along the tensor
        drift = np.linspace(0, 40, n).astype(np.int64)
        sym = ((rng.geometric(0.4, n) + drift) % 256).astype(np.uint8)
        tabs = _seg_tables(sym, Z, seg)
        sc = rng.uniform(0.5, 2, 1).astype(np.float32)
        blob = oracle.encode(1, 1, n, sym, sc, tabs, Z, K, seg_chunks=seg)
        d, fl = oracle.decode_symbols(blob)
        assert fl == 0 and np.array_equal(d, sym), it
        bf, fl = oracle.decode_dequant(blob)
        assert fl == 0 and np.array_equal(bf, oracle.dequant_direct(1, sym, n, sc))


def test_drifting_statistics_code_smaller():
    """Eight bands with different Laplace widths: per-segment tables beat
    one table for the whole tensor."""
    rng = np.random.default_rng(3)
    bands = []
    for theta in (0.1, 0.6, 0.2, 0.7, 0.15, 0.5, 0.05, 0.65):
        v = rng.geometric(1 - theta, 8 * 65536) - 1
        v *= rng.choice([-1, 1], v.size)
        bands.append(np.clip(v, -127, 127).astype(np.int8).view(np.uint8))
    sym = np.concatenate(bands)
    Z, seg = 65536, 8
    one = oracle.encode(1, 64, sym.size // 64, sym, np.ones(64, np.float32), oracle.build_freq(sym), Z, 8)
    many = oracle.encode(1, 64, sym.size // 64, sym, np.ones(64, np.float32), _seg_tables(sym, Z, seg), Z, 8,
                         seg_chunks=seg)
    assert many.size < 0.95 * one.size, (many.size, one.size)
    d, fl = oracle.decode_symbols(many)
    assert fl == 0 and np.array_equal(d, sym)


def test_rejections():
    sym = np.zeros(4096, np.uint8)
    sym[::7] = 3
    f = oracle.build_freq(sym)
    with pytest.raises(oracle.OracleError):
        oracle.encode(1, 1, 4096, sym, np.ones(1, np.float32), f[None, :], 512, 8, seg_chunks=4)
    with pytest.raises(oracle.OracleError):
        oracle.encode(1, 1, 4096, sym, np.ones(1, np.float32), f[None, :], 512, 8, seg_chunks=8,
                      codec=oracle.CODEC_HUFF)
    # a segment whose table lacks one of its symbols
    bad = f.copy()
    bad[3], bad[0] = 0, 4096
    with pytest.raises(oracle.OracleError):
        oracle.encode(1, 1, 4096, sym, np.ones(1, np.float32), bad[None, :], 512, 8, seg_chunks=8)
