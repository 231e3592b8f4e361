"""CPU checks of libeq's host side: the exported C ABI, eq_build_tables and
eq_encode_host against the oracle (byte-equal containers), eq_parse_header
validation and the encoder's argument checks. No GPU call is made here.

Every expected container is built by the oracle alone: its own frequency
quantiser (oracle.build_freq) or code lengths (oracle.huff_lengths on a
plain histogram of the symbols), never the library's tables."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from rans_decode_amd import eq


def test_library_exports_every_declared_function():
    names = eq.declared_functions()
    assert {"eq_build_tables", "eq_encode_host", "eq_decode_block", "eq_decode_dequant_bf16"} <= set(names)
    lib = ctypes.CDLL(eq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_pipeline_mode_argument_checks():
    """eq_pipeline_set_mode rejects a null plan before touching it (no HIP
    call is made on this path)."""
    lib = eq._lib
    assert lib.eq_pipeline_set_mode(None, eq.EQ_PIPELINE_ALTERNATE) == eq.EQ_EINVAL
    assert lib.eq_pipeline_set_mode(None, eq.EQ_PIPELINE_OVERLAP) == eq.EQ_EINVAL


def test_struct_sizes_match_c_layout(tmp_path):
    """The binding's ctypes structs against the C compiler's view of eq.h."""
    import os
    import subprocess
    src = tmp_path / "sizes.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "eq.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu %zu %zu %zu\\n", sizeof(eq_tables),'
                   ' sizeof(eq_tensor_desc), sizeof(eq_header), sizeof(eq_tensor_ref), sizeof(eq_block),'
                   ' offsetof(eq_header, codec), offsetof(eq_header, off_freq)); return 0; }\n')
    exe = tmp_path / "sizes"
    inc = os.path.join(os.path.dirname(eq.HEADER_PATH))
    subprocess.check_call(["gcc", "-std=c11", "-I", inc, str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    assert got == [ctypes.sizeof(eq.eq_tables), ctypes.sizeof(eq.eq_tensor_desc),
                   ctypes.sizeof(eq.eq_header), ctypes.sizeof(eq.eq_tensor_ref),
                   ctypes.sizeof(eq.eq_block), eq.eq_header.codec.offset,
                   eq.eq_header.off_freq.offset]


def test_status_strings():
    assert eq.status_string(0) == "ok"
    assert "corrupt" in eq.status_string(-3)


def _tables_equal_oracle(sym):
    t = eq.build_tables(sym)
    f = np.array(t.freq, dtype=np.uint16)
    assert np.array_equal(f, oracle.build_freq(sym))
    assert list(t.cum) == list(np.concatenate([[0], np.cumsum(f.astype(np.int64))]))
    assert np.array_equal(np.array(t.counts, np.uint64), np.bincount(sym, minlength=256).astype(np.uint64))
    return t


def test_build_tables_matches_oracle_random():
    rng = np.random.default_rng(3)
    for it in range(400):
        n = int(rng.integers(1, 5000))
        k = int(rng.integers(1, 257))
        present = rng.choice(256, size=k, replace=False)
        w = rng.pareto(0.7, k) + 1e-4
        sym = present[rng.choice(k, size=n, p=w / w.sum())].astype(np.uint8)
        _tables_equal_oracle(sym)


def test_build_tables_matches_oracle_quantiser_hand_cases():
    from conftest import read_golden
    for case in read_golden("quantizer_cases.txt")["case"]:
        lhs = case.split("->")[0]
        parts = []
        for tok in lhs.split():
            b, c = tok.split(":")
            parts.append(np.full(int(c), int(b), np.uint8))
        _tables_equal_oracle(np.concatenate(parts))


@pytest.mark.parametrize("cfg", [1, 2])
def test_encode_byte_equal_to_oracle_configs(cfg):
    spec = synth.config_specs(cfg)[0]
    t = synth.make_tensor(cfg, 0, 0)
    tab = _tables_equal_oracle(t.symbols)
    ours = eq.encode_host(tab, spec.dtype, spec.rows, spec.cols, t.symbols, t.scales)
    ref = oracle.encode(spec.dtype, spec.rows, spec.cols, t.symbols, t.scales,
                        oracle.build_freq(t.symbols))
    assert ours.size == ref.size and np.array_equal(ours, ref)


def test_encode_byte_equal_escapes_and_e4m3():
    spec = synth.TensorSpec("down", 48, 4096, synth.DTYPE_INT8, 2.1, 4)
    t = synth.make_tensor(4, 0, 6, spec=spec)
    tab = eq.build_tables(t.symbols)
    ours = eq.encode_host(tab, spec.dtype, spec.rows, spec.cols, t.symbols, t.scales,
                          t.esc_idx, t.esc_val, esc_code=t.esc_code)
    ref = oracle.encode(spec.dtype, spec.rows, spec.cols, t.symbols, t.scales,
                        oracle.build_freq(t.symbols), esc_enabled=True, esc_code=t.esc_code,
                        esc_idx=t.esc_idx, esc_val=t.esc_val)
    assert np.array_equal(ours, ref)
    spec3 = synth.TensorSpec("q", 128, 4096, synth.DTYPE_E4M3, 2.1)
    t3 = synth.make_tensor(3, 0, 0, spec=spec3)
    tab3 = eq.build_tables(t3.symbols)
    ours = eq.encode_host(tab3, spec3.dtype, spec3.rows, spec3.cols, t3.symbols, t3.scales)
    ref = oracle.encode(spec3.dtype, spec3.rows, spec3.cols, t3.symbols, t3.scales,
                        oracle.build_freq(t3.symbols))
    assert np.array_equal(ours, ref)


def test_encode_byte_equal_random_layouts():
    rng = np.random.default_rng(11)
    for it in range(600):
        K = int(rng.choice([1, 2, 4, 8, 16]))
        Z = 64 * K * int(rng.integers(1, 6))
        n = int(rng.integers(1, 4 * Z + 1))
        k = int(rng.integers(1, 30))
        present = rng.choice(256, size=k, replace=False)
        w = rng.exponential(1.0, k) ** 2 + 1e-3
        sym = present[rng.choice(k, size=n, p=w / w.sum())].astype(np.uint8)
        divs = [d for d in range(1, n + 1) if n % d == 0]
        rows = int(rng.choice(divs))
        cols = n // rows
        scales = rng.uniform(-1, 1, rows).astype(np.float32)
        tab = eq.build_tables(sym)
        ours = eq.encode_host(tab, 1, rows, cols, sym, scales, chunk_symbols=Z, lane_run=K)
        ref = oracle.encode(1, rows, cols, sym, scales, oracle.build_freq(sym), Z, K)
        assert np.array_equal(ours, ref), (it, K, Z, n)


def test_encode_custom_table_byte_equal():
    freq = np.zeros(256, np.uint16)
    freq[[0, 1, 0xFF]] = [4000, 80, 16]
    sym = np.array([0xFF, 0xFF, 1, 0], np.uint8)
    ours = eq.encode_host(eq.tables_from_freq(freq), 1, 1, 4, sym, np.array([0.01], np.float32),
                          chunk_symbols=512)
    ref = oracle.encode(1, 1, 4, sym, np.array([0.01], np.float32), freq, 512, 8)
    assert np.array_equal(ours, ref)


def test_parse_header_matches_oracle_fields():
    t = synth.make_tensor(1, 0, 0)
    c = eq.encode_host(eq.build_tables(t.symbols), 1, 1024, 1024, t.symbols, t.scales)
    h = eq.parse_header(c)
    o = oracle.header(c)
    for k in ("rows", "cols", "n", "n_chunks", "n_esc", "n_words", "off_freq", "off_scales",
              "off_dir", "off_states", "off_words", "off_esc_idx", "off_esc_val"):
        assert getattr(h, k) == o[k], k
    assert h.total_bytes == o["total"] and h.chunk_symbols == 65536 and h.lane_run == 8
    assert h.single_symbol == -1


def test_parse_header_single_symbol():
    sym = np.full(5000, 0x07, np.uint8)
    c = eq.encode_host(eq.build_tables(sym), 1, 50, 100, sym, np.ones(50, np.float32))
    assert eq.parse_header(c).single_symbol == 7


def _corrupt_cases(c):
    o = oracle.header(c)
    cases = {}

    def mod(name, fn):
        x = c.copy()
        fn(x)
        cases[name] = x
    mod("magic", lambda x: x.__setitem__(0, 0))
    mod("version", lambda x: x.__setitem__(4, 2))
    mod("dtype", lambda x: x.__setitem__(6, 9))
    mod("lane_run", lambda x: x.__setitem__(36, 3))
    mod("rows", lambda x: x.__setitem__(8, x[8] ^ 1))
    mod("freq_sum", lambda x: x.__setitem__(o["off_freq"], x[o["off_freq"]] ^ 1))
    mod("dir_start", lambda x: x.__setitem__(o["off_dir"] + 16, x[o["off_dir"] + 16] ^ 8))
    mod("dir_count", lambda x: x.__setitem__(o["off_dir"] + 8 + 2, 0x7F))
    mod("state_low", lambda x: x.__setitem__(slice(o["off_states"] + 2, o["off_states"] + 4), 0))
    mod("offset", lambda x: x.__setitem__(96, x[96] ^ 0x80))
    mod("header_pad", lambda x: x.__setitem__(200, 1))
    cases["truncated"] = c[:-256].copy()
    return cases


def test_parse_header_rejects_corruption():
    t = synth.make_tensor(1, 0, 0)
    c = eq.encode_host(eq.build_tables(t.symbols), 1, 1024, 1024, t.symbols, t.scales)
    eq.parse_header(c)
    for name, bad in _corrupt_cases(c).items():
        with pytest.raises(eq.EqError) as ei:
            eq.parse_header(bad)
        assert ei.value.status == eq.EQ_ECORRUPT, name


def test_parse_header_rejects_unsorted_escapes():
    spec = synth.TensorSpec("down", 16, 4096, synth.DTYPE_INT8, 2.1, 4)
    t = synth.make_tensor(4, 0, 6, spec=spec)
    c = eq.encode_host(eq.build_tables(t.symbols), 1, 16, 4096, t.symbols, t.scales, t.esc_idx,
                       t.esc_val, esc_code=0x80)
    h = eq.parse_header(c)
    bad = c.copy()
    a = h.off_esc_idx
    bad[a:a + 8], bad[a + 8:a + 16] = c[a + 8:a + 16], c[a:a + 8]
    with pytest.raises(eq.EqError):
        eq.parse_header(bad)


def test_encode_argument_errors():
    sym = np.zeros(1024, np.uint8)
    sym[5] = 3
    tab = eq.build_tables(sym)
    sc = np.ones(16, np.float32)
    good = dict(dtype=1, rows=16, cols=64)

    def enc(**kw):
        a = dict(good)
        a.update(kw)
        return eq.encode_host(kw.pop("tab", tab), a["dtype"], a["rows"], a["cols"], kw.get("sym", sym),
                              kw.get("sc", sc), kw.get("esc_idx"), kw.get("esc_val"),
                              esc_code=kw.get("esc_code", 0), chunk_symbols=kw.get("Z", 512),
                              lane_run=kw.get("K", 8))
    enc()
    bad_cases = [
        dict(K=3), dict(Z=500), dict(Z=0), dict(dtype=7),
        dict(sc=np.array([np.inf] + [1.0] * 15, np.float32)),
        dict(sym=np.full(1024, 9, np.uint8)),                      # byte with frequency 0
        dict(esc_code=3),                                           # escape code present, not listed
        dict(esc_code=3, esc_idx=np.array([6], np.uint64), esc_val=np.array([1], np.uint16)),
    ]
    for kw in bad_cases:
        with pytest.raises(eq.EqError) as ei:
            enc(**kw)
        assert ei.value.status == eq.EQ_EINVAL, kw
    # E4M3 NaN code outside the escape list
    s8 = np.zeros(1024, np.uint8)
    s8[0] = 0x7F
    with pytest.raises(eq.EqError):
        eq.encode_host(eq.build_tables(s8), 2, 16, 64, s8, sc, chunk_symbols=512)
    # empty input
    with pytest.raises(eq.EqError):
        eq.build_tables(np.zeros(0, np.uint8))


def test_encode_size_query():
    sym = np.zeros(4096, np.uint8)
    sym[::3] = 1
    tab = eq.build_tables(sym)
    d = eq.eq_tensor_desc(dtype=1, lane_run=8, rows=64, cols=64, chunk_symbols=512)
    need = ctypes.c_uint64(0)
    sc = np.ones(64, np.float32)
    st = eq._lib.eq_encode_host(ctypes.byref(tab), ctypes.byref(d), sym.ctypes.data, sc.ctypes.data,
                                None, None, 0, None, 0, ctypes.byref(need))
    assert st == eq.EQ_ERANGE
    c = eq.eq_encode_host(tab, d, sym, sc)
    assert c.size == need.value


# --- Huffman codec (EntroLLM method item 2): the library's encoder against the oracle's

def test_huffman_encode_byte_equal_random_layouts():
    """Code lengths (package-merge), canonical codes, bit packing and the
    interleaved word order: byte-equal containers on random layouts."""
    rng = np.random.default_rng(23)
    for it in range(300):
        K = int(rng.choice([1, 2, 4, 8, 16]))
        Z = 64 * K * int(rng.integers(1, 6))
        n = int(rng.integers(1, 4 * Z + 1))
        k = int(rng.integers(1, 40))
        present = rng.choice(256, size=k, replace=False)
        w = rng.exponential(1.0, k) ** 3 + 1e-4
        sym = present[rng.choice(k, size=n, p=w / w.sum())].astype(np.uint8)
        divs = [d for d in range(1, n + 1) if n % d == 0]
        rows = int(rng.choice(divs))
        cols = n // rows
        scales = rng.uniform(-1, 1, rows).astype(np.float32)
        tab = eq.build_tables(sym)
        ours = eq.encode_host(tab, 1, rows, cols, sym, scales, chunk_symbols=Z, lane_run=K,
                              codec=eq.EQ_CODEC_HUFFMAN)
        lens = oracle.huff_lengths(np.bincount(sym, minlength=256).astype(np.uint64))
        ref = oracle.encode(1, rows, cols, sym, scales, lens, Z, K, codec=oracle.CODEC_HUFF)
        assert np.array_equal(ours, ref), (it, K, Z, n)
        h = eq.parse_header(ours)
        assert h.codec == eq.EQ_CODEC_HUFFMAN
        distinct = sorted(set(sym.tolist()))
        assert h.single_symbol == (distinct[0] if len(distinct) == 1 else -1)


def test_huffman_encode_byte_equal_configs_and_escapes():
    for cfg, spec in [(1, None), (4, synth.TensorSpec("down", 48, 4096, synth.DTYPE_INT8, 2.1, 4)),
                      (3, synth.TensorSpec("q", 64, 4096, synth.DTYPE_E4M3, 2.1, 3))]:
        t = synth.make_tensor(cfg, 0, 6 if spec and spec.n_esc else 0, spec=spec)
        sp = t.spec
        tab = eq.build_tables(t.symbols)
        esc = t.esc_idx.size > 0
        ours = eq.encode_host(tab, sp.dtype, sp.rows, sp.cols, t.symbols, t.scales,
                              t.esc_idx if esc else None, t.esc_val if esc else None,
                              esc_code=t.esc_code if esc else 0, codec=eq.EQ_CODEC_HUFFMAN)
        lens = oracle.huff_lengths(np.bincount(t.symbols, minlength=256).astype(np.uint64))
        ref = oracle.encode(sp.dtype, sp.rows, sp.cols, t.symbols, t.scales, lens,
                            esc_enabled=esc, esc_code=t.esc_code if esc else 0,
                            esc_idx=t.esc_idx if esc else None, esc_val=t.esc_val if esc else None,
                            codec=oracle.CODEC_HUFF)
        assert np.array_equal(ours, ref), cfg
        d, fl = oracle.decode_symbols(ours)
        assert fl == 0 and np.array_equal(d, t.symbols)


def test_huffman_lone_symbol_and_parse_checks():
    sym = np.full(5000, 0x07, np.uint8)
    c = eq.encode_host(eq.build_tables(sym), 1, 50, 100, sym, np.ones(50, np.float32),
                       codec=eq.EQ_CODEC_HUFFMAN)
    h = eq.parse_header(c)
    assert h.single_symbol == 7 and h.n_words == 0 and h.codec == eq.EQ_CODEC_HUFFMAN
    # no lane-state section: words start where the states would
    assert h.off_states == h.off_words
    rng = np.random.default_rng(3)
    sym = rng.choice([1, 2, 3, 200], 9000, p=[0.7, 0.2, 0.07, 0.03]).astype(np.uint8)
    c = eq.encode_host(eq.build_tables(sym), 1, 9, 1000, sym, np.ones(9, np.float32),
                       codec=eq.EQ_CODEC_HUFFMAN)
    h = eq.parse_header(c)
    lens = c[h.off_freq:h.off_freq + 512].view(np.uint16)
    for name, mutate in [("kraft", lambda t: t.__setitem__(1, t[1] + 1)),
                         ("too long", lambda t: t.__setitem__(2, 13)),
                         ("zero-bit with others", lambda t: t.__setitem__(3, 0x100)),
                         ("codec", None)]:
        bad = c.copy()
        if mutate is None:
            bad[144] = 7
        else:
            t = lens.copy()
            mutate(t)
            bad[h.off_freq:h.off_freq + 512] = t.view(np.uint8)
        with pytest.raises(eq.EqError) as ei:
            eq.parse_header(bad)
        assert ei.value.status == eq.EQ_ECORRUPT, name
    # a present symbol without a count cannot get a codeword
    tab = eq.build_tables(sym)
    tab.counts[200] = 0
    with pytest.raises(eq.EqError):
        eq.encode_host(tab, 1, 9, 1000, sym, np.ones(9, np.float32), codec=eq.EQ_CODEC_HUFFMAN)
    with pytest.raises(eq.EqError):
        eq.encode_host(eq.build_tables(sym), 1, 9, 1000, sym, np.ones(9, np.float32), codec=5)


# --- adaptive (per-segment) frequency tables

def _seg_tables_oracle(sym, Z, seg):
    n_chunks = -(-sym.size // Z)
    n_seg = -(-n_chunks // seg)
    return np.stack([oracle.build_freq(sym[g * seg * Z:(g + 1) * seg * Z]) for g in range(n_seg)])


def test_segment_tables_byte_equal_to_oracle():
    rng = np.random.default_rng(29)
    for it in range(120):
        K = int(rng.choice([1, 2, 4, 8, 16]))
        Z = 64 * K * int(rng.integers(1, 4))
        seg = 8 * int(rng.integers(1, 4))
        n = int(rng.integers(1, Z * seg * 3))
        drift = np.linspace(0, int(rng.integers(0, 60)), n).astype(np.int64)
        sym = ((rng.geometric(float(rng.uniform(0.2, 0.8)), n) + drift) % 256).astype(np.uint8)
        divs = [d for d in range(1, min(n, 32) + 1) if n % d == 0]
        rows = int(rng.choice(divs))
        scales = rng.uniform(-1, 1, rows).astype(np.float32)
        ours = eq.encode_host(None, 1, rows, n // rows, sym, scales, chunk_symbols=Z, lane_run=K,
                              seg_chunks=seg)
        ref = oracle.encode(1, rows, n // rows, sym, scales, _seg_tables_oracle(sym, Z, seg), Z, K,
                            seg_chunks=seg)
        assert np.array_equal(ours, ref), (it, K, Z, seg, n)
        h = eq.parse_header(ours)
        assert h.seg_chunks == seg and h.single_symbol == -1


def test_segment_tables_parse_and_argument_checks():
    rng = np.random.default_rng(4)
    sym = rng.choice([0, 1, 2, 250], 64 * 1024, p=[0.6, 0.2, 0.15, 0.05]).astype(np.uint8)
    c = eq.encode_host(None, 1, 64, 1024, sym, np.ones(64, np.float32), chunk_symbols=512, lane_run=8,
                       seg_chunks=16)
    h = eq.parse_header(c)
    assert h.off_scales - h.off_freq == 512 * (-(-128 // 16))
    for name, mutate in [("flag without size", lambda x: x.__setitem__(148, 0)),
                         ("size not a multiple of 8", lambda x: x.__setitem__(148, 12)),
                         ("second table sum", lambda x: x.__setitem__(h.off_freq + 512, x[h.off_freq + 512] ^ 1))]:
        bad = c.copy()
        mutate(bad)
        with pytest.raises(eq.EqError) as ei:
            eq.parse_header(bad)
        assert ei.value.status == eq.EQ_ECORRUPT, name
    for seg, codec in [(4, 0), (8, eq.EQ_CODEC_HUFFMAN)]:
        with pytest.raises(eq.EqError):
            eq.encode_host(eq.build_tables(sym), 1, 64, 1024, sym, np.ones(64, np.float32),
                           chunk_symbols=512, seg_chunks=seg, codec=codec)
