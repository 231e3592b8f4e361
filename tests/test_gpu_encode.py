"""GPU device-side encoder (`eq_encode_device`) against the oracle: every
container must be byte-identical to the oracle's encoder run on the oracle's
own tables (its frequency quantiser, its length-limited Huffman code, its
per-segment quantiser), and a GPU decode of it must reproduce the original
symbols. The host encoder's container is compared too, as an extra check."""
import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import gpu_available
from gpu_util import assert_same, log, run_u8
from rans_decode_amd import eq

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda") if a is not None else None


def device_container(sym, scales, dtype, rows, cols, Z, K, esc_idx=None, esc_val=None, esc_code=0,
                     codec=0, seg=0):
    ds = _dev(sym, None)
    dsc = _dev(scales.astype(np.float32), None)
    di = _dev(esc_idx.astype(np.int64), None) if esc_idx is not None and len(esc_idx) else None
    dv = _dev(esc_val.view(np.int16), None) if esc_val is not None and len(esc_val) else None
    out, d_len, st = eq.eq_encode_device(dtype, rows, cols, ds, dsc, di, dv, esc_code, Z, K,
                                         codec=codec, seg_chunks=seg)
    torch.cuda.synchronize()
    n = int(d_len.item())
    return out[:n].cpu().numpy(), int(st.item())


def host_container(sym, scales, dtype, rows, cols, Z, K, esc_idx=None, esc_val=None, esc_code=0,
                   codec=0, seg=0):
    return eq.encode_host(None if seg else eq.build_tables(sym), dtype, rows, cols, sym, scales,
                          esc_idx if esc_idx is not None and len(esc_idx) else None,
                          esc_val if esc_val is not None and len(esc_val) else None,
                          esc_code=esc_code, chunk_symbols=Z, lane_run=K, codec=codec, seg_chunks=seg)


def oracle_container(sym, scales, dtype, rows, cols, Z, K, esc_idx=None, esc_val=None, esc_code=0,
                     codec=0, seg=0):
    """The oracle's container on the oracle's own tables."""
    esc = esc_idx is not None and len(esc_idx) > 0
    if codec == eq.EQ_CODEC_HUFFMAN:
        table = oracle.huff_lengths(np.bincount(sym, minlength=256).astype(np.uint64))
    elif seg:
        n_chunks = -(-sym.size // Z)
        table = np.stack([oracle.build_freq(sym[g * seg * Z:(g + 1) * seg * Z])
                          for g in range(-(-n_chunks // seg))])
    else:
        table = oracle.build_freq(sym)
    return oracle.encode(dtype, rows, cols, sym, scales, table, Z, K, esc_enabled=esc or esc_code != 0,
                         esc_code=esc_code, esc_idx=esc_idx if esc else None, esc_val=esc_val if esc else None,
                         codec=codec, seg_chunks=seg)


def _same_bytes(got, exp, what):
    assert got.size == exp.size, f"{what}: size {got.size} vs {exp.size}"
    bad = np.flatnonzero(got != exp)
    assert bad.size == 0, f"{what}: {bad.size} bytes differ, first at {bad[0]}"


def check_equal(sym, scales, dtype, rows, cols, Z=65536, K=8, esc_idx=None, esc_val=None, esc_code=0,
                what="", codec=0, seg=0):
    got, st = device_container(sym, scales, dtype, rows, cols, Z, K, esc_idx, esc_val, esc_code, codec, seg)
    assert st == 0, f"{what}: device status {st}"
    _same_bytes(got, oracle_container(sym, scales, dtype, rows, cols, Z, K, esc_idx, esc_val, esc_code, codec,
                                      seg), f"{what} vs the oracle")
    _same_bytes(got, host_container(sym, scales, dtype, rows, cols, Z, K, esc_idx, esc_val, esc_code, codec, seg),
                f"{what} vs the host encoder")
    return got


@pytest.mark.parametrize("cfg", [1, 2])
def test_config_matrices(cfg):
    t = synth.make_tensor(cfg, 0, 0)
    sp = t.spec
    log(f"case device encode config {cfg}")
    c = check_equal(t.symbols, t.scales, sp.dtype, sp.rows, sp.cols, what=f"config {cfg}")
    sym, st = run_u8([eq.DeviceContainer(c, device="cuda")], sp.n)
    assert st == 0
    assert_same(sym, t.symbols, "round trip")


def test_block_tensors_with_escapes_and_e4m3():
    for cfg, i in [(4, 6), (4, 1), (3, 0), (3, 5)]:
        t = synth.make_tensor(cfg, 0, i)
        sp = t.spec
        esc = t.esc_idx.size > 0
        for Z in sorted({synth.config_chunk(cfg), 65536}):
            log(f"case device encode config {cfg} tensor {sp.name}, chunk {Z}")
            check_equal(t.symbols, t.scales, sp.dtype, sp.rows, sp.cols, Z=Z,
                        esc_idx=t.esc_idx if esc else None, esc_val=t.esc_val if esc else None,
                        esc_code=t.esc_code if esc else 0, what=f"cfg {cfg} {sp.name} Z={Z}")
        del t


def test_random_layouts():
    rng = np.random.default_rng(31)
    for it in range(80):
        K = int(rng.choice([1, 2, 4, 8, 16]))
        Z = 64 * K * int(rng.integers(1, 9))
        n = int(rng.integers(1, 5 * Z))
        n = max(16, n - n % 16) if it % 2 else n
        # every tenth layout: all 256 codes near-uniform (~8 bits per symbol,
        # the most words a chunk can hold in flight)
        k = 256 if it % 10 == 9 else int(rng.integers(1, 60))
        present = rng.choice(256, size=k, replace=False)
        w = rng.uniform(0.5, 1.0, k) if k == 256 else rng.exponential(1.0, k) ** 3 + 1e-6
        sym = present[rng.choice(k, size=n, p=w / w.sum())].astype(np.uint8)
        divs = [d for d in range(1, min(n, 64) + 1) if n % d == 0]
        rows = int(rng.choice(divs))
        scales = rng.uniform(-2, 2, rows).astype(np.float32)
        check_equal(sym, scales, 1, rows, n // rows, Z, K, what=f"random {it} K={K} Z={Z} n={n}")


def test_quantiser_excess_and_ties_and_single_symbol():
    rng = np.random.default_rng(2)
    # 200 rare symbols (each rounds up to f = 1) force an excess taken from the largest f
    sym = np.concatenate([np.zeros(10**6, np.uint8), np.arange(1, 201, dtype=np.uint8),
                          np.full(3000, 250, np.uint8)])
    sym = sym[rng.permutation(sym.size)]
    sym = sym[: sym.size - sym.size % 64]
    check_equal(sym, np.ones(64, np.float32), 1, 64, sym.size // 64, 16384, 8, what="excess")
    # equal counts: remainders tie, smaller byte first
    sym = np.tile(np.arange(7, dtype=np.uint8), 3000)
    check_equal(sym, np.ones(3, np.float32), 1, 3, 7000, 4096, 4, what="ties")
    sym = np.full(5000, 0x42, np.uint8)
    c = check_equal(sym, np.ones(50, np.float32), 1, 50, 100, 512, 8, what="single symbol")
    assert eq.parse_header(c).single_symbol == 0x42


def test_bad_inputs_raise_the_device_flag():
    sym = np.zeros(4096, np.uint8)
    sym[10] = 0x80
    idx = np.array([10], np.uint64)
    val = np.array([0x4000], np.uint16)
    _, st = device_container(sym, np.ones(4, np.float32), 1, 4, 1024, 4096, 8, idx, val, 0x80)
    assert st == 0
    _, st = device_container(sym, np.ones(4, np.float32), 1, 4, 1024, 4096, 8,
                             np.array([11], np.uint64), val, 0x80)
    assert st & eq.EQ_DEV_BAD_INPUT  # listed index does not hold the code
    _, st = device_container(sym, np.array([1, np.inf, 1, 1], np.float32), 1, 4, 1024, 4096, 8, idx, val, 0x80)
    assert st & eq.EQ_DEV_BAD_INPUT  # non-finite scale
    sym2 = np.zeros(4096, np.uint8)
    sym2[5] = 0x7F
    _, st = device_container(sym2, np.ones(4, np.float32), 2, 4, 1024, 4096, 8)
    assert st & eq.EQ_DEV_BAD_INPUT  # E4M3 NaN code, not an escape


# --- the Huffman codec and adaptive (per-segment) tables -------------------

@pytest.mark.parametrize("cfg", [1, 2])
def test_huffman_config_matrices(cfg):
    t = synth.make_tensor(cfg, 0, 0)
    sp = t.spec
    log(f"case device Huffman encode config {cfg}")
    c = check_equal(t.symbols, t.scales, sp.dtype, sp.rows, sp.cols, what=f"huffman config {cfg}",
                    codec=eq.EQ_CODEC_HUFFMAN)
    sym, st = run_u8([eq.DeviceContainer(c, device="cuda")], sp.n)
    assert st == 0
    assert_same(sym, t.symbols, "round trip")


def test_huffman_block_tensors_with_escapes_and_e4m3():
    for cfg, i in [(4, 6), (4, 1), (3, 0)]:
        t = synth.make_tensor(cfg, 0, i)
        sp = t.spec
        log(f"case device Huffman encode config {cfg} tensor {sp.name}")
        esc = t.esc_idx.size > 0
        check_equal(t.symbols, t.scales, sp.dtype, sp.rows, sp.cols,
                    esc_idx=t.esc_idx if esc else None, esc_val=t.esc_val if esc else None,
                    esc_code=t.esc_code if esc else 0, what=f"huffman cfg {cfg} {sp.name}",
                    codec=eq.EQ_CODEC_HUFFMAN)
        del t


def test_huffman_random_layouts_and_one_symbol():
    rng = np.random.default_rng(41)
    for it in range(60):
        K = int(rng.choice([1, 2, 4, 8, 16]))
        Z = 64 * K * int(rng.integers(1, 9))
        n = int(rng.integers(1, 5 * Z))
        n = max(16, n - n % 16) if it % 2 else n
        # every tenth layout near-uniform over all 256 codes; every seventh one code
        k = 256 if it % 10 == 9 else (1 if it % 7 == 3 else int(rng.integers(2, 60)))
        present = rng.choice(256, size=k, replace=False)
        w = rng.uniform(0.5, 1.0, k) if k == 256 else rng.exponential(1.0, k) ** 3 + 1e-6
        sym = present[rng.choice(k, size=n, p=w / w.sum())].astype(np.uint8)
        divs = [d for d in range(1, min(n, 64) + 1) if n % d == 0]
        rows = int(rng.choice(divs))
        scales = rng.uniform(-2, 2, rows).astype(np.float32)
        check_equal(sym, scales, 1, rows, n // rows, Z, K, what=f"huffman random {it} K={K} Z={Z} n={n} k={k}",
                    codec=eq.EQ_CODEC_HUFFMAN)


def test_huffman_length_limited_codes_ragged_chunks():
    """Sixteen bytes with Fibonacci counts: an unlimited Huffman code would be
    15 deep, so the 12-bit limit binds and some codewords are 12 bits long;
    ragged chunk and lane ends for every lane run."""
    rng = np.random.default_rng(47)
    fib = [1, 1]
    while len(fib) < 16:
        fib.append(fib[-1] + fib[-2])
    present = rng.choice(256, size=16, replace=False).astype(np.uint8)
    base = np.repeat(present, fib)
    for K in (1, 2, 4, 8, 16):
        Z = 64 * K * 4
        n = 3 * base.size + 64 * K + 37
        sym = np.concatenate([rng.permutation(base) for _ in range(4)])[:n]
        scales = rng.uniform(0.5, 2.0, 1).astype(np.float32)
        log(f"case device Huffman encode 12-bit codes K={K} n={n}")
        c = check_equal(sym, scales, 1, 1, n, Z, K, what=f"huffman 12-bit K={K}", codec=eq.EQ_CODEC_HUFFMAN)
        h = eq.eq_parse_header(c)
        lens = np.frombuffer(c[h.off_freq:h.off_freq + 512].tobytes(), np.uint16)
        assert lens.max() == 12 and np.count_nonzero(lens == 12) >= 2, lens[lens > 0]
        got, st = run_u8([eq.DeviceContainer(c, device="cuda")], n)
        assert st == 0
        assert_same(got, sym, f"round trip K={K}")


def test_adaptive_tables_random_layouts():
    rng = np.random.default_rng(43)
    for it in range(40):
        K = int(rng.choice([1, 4, 8, 16]))
        Z = 64 * K * int(rng.integers(1, 5))
        seg = int(rng.choice([8, 16, 24]))
        n = int(rng.integers(1, 3 * seg * Z))
        # drifting distributions: each quarter of the tensor draws from its own codes
        parts = []
        for q in range(4):
            k = int(rng.integers(1, 40))
            present = rng.choice(256, size=k, replace=False)
            w = rng.exponential(1.0, k) ** 3 + 1e-6
            m = n // 4 + (n % 4 if q == 3 else 0)
            parts.append(present[rng.choice(k, size=m, p=w / w.sum())].astype(np.uint8))
        sym = np.concatenate(parts)
        divs = [d for d in range(1, min(n, 64) + 1) if n % d == 0]
        rows = int(rng.choice(divs))
        scales = rng.uniform(-2, 2, rows).astype(np.float32)
        check_equal(sym, scales, 1, rows, n // rows, Z, K, what=f"segments {it} K={K} Z={Z} seg={seg} n={n}",
                    seg=seg)


def test_adaptive_tables_drifting_tensor_round_trip():
    t = synth.drift_tensor(1024, 8192, seed=3)
    log("case device encode drifting tensor, 8-chunk tables")
    c = check_equal(t.symbols, t.scales, t.spec.dtype, t.spec.rows, t.spec.cols, what="drift seg 8", seg=8)
    sym, st = run_u8([eq.DeviceContainer(c, device="cuda")], t.spec.n)
    assert st == 0
    assert_same(sym, t.symbols, "round trip")


def test_codec_and_segment_argument_errors():
    sym = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    sc = torch.ones(4, dtype=torch.float32, device="cuda")
    with pytest.raises(eq.EqError):
        eq.eq_encode_device(1, 4, 1024, sym, sc, chunk_symbols=512, lane_run=8,
                            codec=eq.EQ_CODEC_HUFFMAN, seg_chunks=8)  # adaptive tables are rANS only
    with pytest.raises(eq.EqError):
        eq.eq_encode_device(1, 4, 1024, sym, sc, chunk_symbols=512, lane_run=8, seg_chunks=4)  # not a multiple of 8
    with pytest.raises(eq.EqError):
        eq.eq_encode_device(1, 4, 1024, sym, sc, chunk_symbols=512, lane_run=8, codec=7)
