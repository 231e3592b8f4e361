"""Pins of the oracle's coder: hand example, exhaustive step bijection, brute
force over all tiny streams, random round trips, quantiser invariants and
hand cases, and the coded-size bar.

None of these expected values comes from the GPU library: they are hand
derivations (tests/golden), closed forms, invariants, and the losslessness of
the coding ("Float8@2bits: Entropy Coding Enables Data-Free Model
Compression", section 2, core concept: the low-entropy weights are compressed
without loss by an ANS coder)."""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import parse_int, read_golden


# ---------------------------------------------------------------------------
# W1 / W2: hand-worked example
# ---------------------------------------------------------------------------
def test_w1_single_lane_hand_example():
    g = read_golden("w1_single_lane.txt")
    fa, fb, fc = (parse_int(g[k][0]) for k in ("freq_a", "freq_b", "freq_c"))
    tab = {"a": (fa, 0), "b": (fb, fa), "c": (fc, fa + fb)}
    x = 65536
    emitted = []
    trace = []
    for s in "abcc":                       # encoder order = reverse of decode order c c b a
        x, w = oracle.encode_step(x, *tab[s])
        trace.append(x)
        if w is not None:
            emitted.append(w)
    assert trace[:3] == [parse_int(g[k][0]) for k in ("state_after_a", "state_after_b", "state_after_c1")]
    assert x == parse_int(g["final_state"][0]) == parse_int(g["final_state_hex"][0])
    assert emitted == [parse_int(t) for t in g["words"][0].split()]

    # decode back: slot sequence and states
    slots = [int(t) for t in g["decode_slots"][0].split()]
    states = [int(t) for t in g["decode_states"][0].split()]
    words = list(emitted)
    for exp_slot, exp_state, s in zip(slots, states, "ccba"):
        assert x % 4096 == exp_slot
        x, need = oracle.decode_step(x, *tab[s])
        if need:
            x = (x << 16) | words.pop(0)
        assert x == exp_state
    assert x == 65536 and not words


def test_w2_container_hand_example():
    g = read_golden("w2_container.txt")
    sym = np.array([parse_int(t) for t in g["symbols"][0].split()], dtype=np.uint8)
    freq = np.zeros(256, np.uint16)
    for b in (0x00, 0x01, 0xFF):
        freq[b] = parse_int(g[f"freq_0x{b:02X}"][0])
    scale = np.array([parse_int(g["scale_bits"][0])], dtype=np.uint32).view(np.float32)
    c = oracle.encode(oracle.DTYPE_INT8, 1, sym.size, sym, scale, freq,
                      chunk_symbols=parse_int(g["chunk_symbols"][0]),
                      lane_run=parse_int(g["lane_run"][0]))
    h = oracle.header(c)
    assert h["n_chunks"] == 1 and h["n_words"] == 8
    states = c[h["off_states"]:h["off_states"] + 256].view(np.uint32)
    assert states[0] == parse_int(g["state_lane0"][0])
    assert np.all(states[1:] == parse_int(g["state_other_lanes"][0]))
    d = c[h["off_dir"]:h["off_dir"] + 16]
    assert int(d[:8].view(np.uint64)[0]) == 0
    assert int(d[8:12].view(np.uint32)[0]) == parse_int(g["word_count"][0])
    words = c[h["off_words"]:h["off_words"] + 16].view(np.uint16)
    assert list(words) == [parse_int(t) for t in g["words_padded"][0].split()]
    out, flags = oracle.decode_dequant(c)
    assert flags == 0
    assert list(out) == [parse_int(t) for t in g["bf16"][0].split()]
    s, flags = oracle.decode_symbols(c)
    assert flags == 0 and np.array_equal(s, sym)


def _w6_case():
    g = read_golden("w6_two_lanes.txt")
    n = parse_int(g["n"][0])
    sym = np.zeros(n, np.uint8)                       # a = 0x00 everywhere ...
    for p in g["positions_c"][0].split():
        sym[int(p)] = 0xFF                            # ... c at these positions
    for p in g["positions_b"][0].split():
        sym[int(p)] = 0x01                            # ... b here
    freq = _freq({0x00: 4000, 0x01: 80, 0xFF: 16})
    scale = np.array([parse_int(g["scale_bits"][0])], dtype=np.uint32).view(np.float32)
    return g, sym, freq, scale


def _w6_encode(orc, g, sym, freq, scale):
    return orc.encode(orc.DTYPE_INT8, 1, sym.size, sym, scale, freq,
                      chunk_symbols=parse_int(g["chunk_symbols"][0]), lane_run=parse_int(g["lane_run"][0]))


def _w6_mismatches(orc, c, g, sym):
    """What in container c (and its decode) differs from the hand-worked W6."""
    bad = []
    h = orc.header(c)
    st = c[h["off_states"]:h["off_states"] + 256].view(np.uint32)
    if st[0] != parse_int(g["state_lane0"][0]) or st[1] != parse_int(g["state_lane1"][0]) \
            or np.any(st[2:] != parse_int(g["state_other_lanes"][0])):
        bad.append("states")
    wc = int(c[h["off_dir"] + 8:h["off_dir"] + 12].view(np.uint32)[0])
    if wc != parse_int(g["word_count"][0]):
        bad.append("word count")
    words = c[h["off_words"]:h["off_words"] + 16].view(np.uint16)
    if list(words) != [parse_int(t) for t in g["words_padded"][0].split()]:
        bad.append("words")
    s, flags = orc.decode_symbols(c)
    if flags or not np.array_equal(s, sym):
        bad.append("decode")
    return bad


def test_w6_two_lanes_hand_example():
    """Two lanes renormalise in one step (ascending-lane word order); lanes
    >= 1 carry symbols at the positions of the lane-run map."""
    g, sym, freq, scale = _w6_case()
    c = _w6_encode(oracle, g, sym, freq, scale)
    assert _w6_mismatches(oracle, c, g, sym) == []
    out, flags = oracle.decode_dequant(c)
    assert flags == 0
    exp = np.where(sym == 0xFF, parse_int(g["bf16_c"][0]),
                   np.where(sym == 0x01, parse_int(g["bf16_b"][0]), parse_int(g["bf16_a"][0])))
    assert np.array_equal(out, exp.astype(np.uint16))


W6_PLANTS = {
    # encoder walks the lanes of a step upwards: the step's words come out in
    # descending-lane order
    "encoder lanes ascending": ("for (uint32_t jj = OR_LANES; jj-- > 0;) {",
                                "for (uint32_t jj = 0; jj < OR_LANES; jj++) {"),
    # lane j's run placed at j + 64 * (t mod K) instead of j * K + (t mod K)
    "position map transposed": ("return (t / K) * (uint64_t)OR_LANES * K + (uint64_t)j * K + (t % K);",
                                "return (t / K) * (uint64_t)OR_LANES * K + (t % K) * OR_LANES + j;"),
}


@pytest.mark.parametrize("plant", list(W6_PLANTS))
def test_w6_catches_planted_mistakes(planted, plant):
    g, sym, freq, scale = _w6_case()
    with planted(*W6_PLANTS[plant]) as bad:
        c = _w6_encode(bad, g, sym, freq, scale)
        assert _w6_mismatches(bad, c, g, sym) != []


def test_w6_catches_descending_decoder(planted):
    """A decoder that serves the renormalising lanes of a step in descending
    order misreads the hand-worked container."""
    g, sym, freq, scale = _w6_case()
    c = _w6_encode(oracle, g, sym, freq, scale)
    assert _w6_mismatches(oracle, c, g, sym) == []
    old = ("        for (uint32_t j = 0; j < OR_LANES; j++) {\n"
           "            uint64_t p = lane_pos(t, j, K);\n"
           "            if (p >= nk) continue;\n"
           "            uint8_t s = s2s[x[j] % OR_M];")
    new = ("        for (uint32_t j = OR_LANES; j-- > 0;) {\n"
           "            uint64_t p = lane_pos(t, j, K);\n"
           "            if (p >= nk) continue;\n"
           "            uint8_t s = s2s[x[j] % OR_M];")
    with planted(old, new) as bad:
        s, flags = bad.decode_symbols(c)
        assert flags != 0 or not np.array_equal(s, sym)


# ---------------------------------------------------------------------------
# Exhaustive: C(D(x)) = x over every state, with renormalisation words
# ---------------------------------------------------------------------------
def _freq(d):
    f = np.zeros(256, np.uint16)
    for b, v in d.items():
        f[b] = v
    return f


BIJECTION_TABLES = {
    "4000/80/16": _freq({0: 4000, 1: 80, 2: 16}),
    "uniform256x16": np.full(256, 16, np.uint16),
    "single4096": _freq({7: 4096}),
    "4094/1/1": _freq({0: 4094, 0x80: 1, 0xFF: 1}),
}


@pytest.mark.parametrize("name", list(BIJECTION_TABLES))
def test_exhaustive_step_bijection(native_checks, name):
    import ctypes
    import os
    freq = BIJECTION_TABLES[name]
    fn = native_checks.bijection_failures
    fn.restype = ctypes.c_uint64
    fn.argtypes = [ctypes.c_char_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int]
    fails = fn(oracle.LIB_PATH.encode(), freq.ctypes.data, 1 << 16, 1 << 32, os.cpu_count() or 1)
    assert fails == 0


def test_planted_mistake_is_caught(native_checks, tmp_path):
    """The bijection check must fail on a decode step with a wrong bias term
    (a plausible transcription slip). Built from a copy of the oracle source
    with one character changed, on the CPU."""
    import ctypes
    import os
    import subprocess
    src = open(oracle.LIB_PATH.replace("liboracle.so", "eq_oracle.c")).read()
    bad = src.replace("*x = f * (*x / OR_M) + slot - c;", "*x = f * (*x / OR_M) + slot - c + 1;")
    assert bad != src
    p = tmp_path / "bad.c"
    p.write_text(bad)
    so = str(tmp_path / "libbad.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", str(p), "-o", so, "-lpthread"])
    fn = native_checks.bijection_failures
    fn.restype = ctypes.c_uint64
    fn.argtypes = [ctypes.c_char_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int]
    freq = BIJECTION_TABLES["4000/80/16"]
    fails = fn(so.encode(), freq.ctypes.data, 1 << 16, (1 << 16) + 100000, 2)
    assert fails > 0


# ---------------------------------------------------------------------------
# Brute force: every stream of length 1..8 over the table's alphabet
# ---------------------------------------------------------------------------
BRUTE_TABLES = {
    "4096": {0x05: 4096},
    "2048/2048": {0x00: 2048, 0xFF: 2048},
    "4000/80/16": {0x00: 4000, 0x01: 80, 0xFF: 16},
    "4094/1/1": {0x00: 4094, 0x01: 1, 0xFF: 1},
    "1366/1365/1365": {0x00: 1366, 0x01: 1365, 0xFF: 1365},
}


def _roundtrip(sym, rows, cols, freq, K, Z, dtype=oracle.DTYPE_INT8, scales=None):
    if scales is None:
        scales = np.full(rows, 0.01, np.float32)
    c = oracle.encode(dtype, rows, cols, sym, scales, freq, chunk_symbols=Z, lane_run=K)
    dec, flags = oracle.decode_symbols(c)
    assert flags == 0
    assert np.array_equal(dec, sym)
    out, flags = oracle.decode_dequant(c)
    assert flags == 0
    assert np.array_equal(out, oracle.dequant_direct(dtype, sym, cols, scales))
    return c


@pytest.mark.parametrize("name", list(BRUTE_TABLES))
@pytest.mark.parametrize("K", [1, 8])
def test_brute_force_tiny_streams(name, K):
    tab = BRUTE_TABLES[name]
    freq = _freq(tab)
    alphabet = sorted(tab)
    count = 0
    for L in range(1, 9):
        for tup in itertools.product(alphabet, repeat=L):
            sym = np.array(tup, dtype=np.uint8)
            # one chunk of one 64K group (single lane for K = 8, L lanes for K = 1)
            _roundtrip(sym, 1, L, freq, K, 64 * K)
            count += 1
    assert count == sum(len(alphabet) ** L for L in range(1, 9))


def test_brute_force_multichunk_tails():
    """Streams spanning several chunks with ragged tails, all K."""
    rng = np.random.default_rng(1234)
    for K in (1, 2, 4, 8, 16):
        for Z_groups in (1, 2):
            Z = 64 * K * Z_groups
            for n in (1, 63, 64, 65, Z - 1, Z, Z + 1, 2 * Z + 7, 3 * Z):
                for name, tab in BRUTE_TABLES.items():
                    alphabet = np.array(sorted(tab), dtype=np.uint8)
                    sym = alphabet[rng.integers(0, alphabet.size, n)]
                    _roundtrip(sym, 1, n, _freq(tab), K, Z)


def test_random_streams_random_tables():
    rng = np.random.default_rng(99)
    for it in range(2000):
        K = int(rng.choice([1, 2, 4, 8, 16]))
        Z = 64 * K * int(rng.integers(1, 5))
        n = int(rng.integers(1, 3 * 64 * K + 1))
        k = int(rng.integers(1, 40))
        present = rng.choice(256, size=k, replace=False)
        w = rng.exponential(1.0, size=k) ** 3 + 1e-3
        sym = present[rng.choice(k, size=n, p=w / w.sum())].astype(np.uint8)
        freq = oracle.build_freq(sym)
        # random row/col split of n
        divs = [d for d in range(1, n + 1) if n % d == 0]
        rows = int(rng.choice(divs))
        cols = n // rows
        scales = rng.uniform(-2, 2, rows).astype(np.float32)
        dtype = oracle.DTYPE_INT8 if it % 2 else oracle.DTYPE_E4M3
        if dtype == oracle.DTYPE_E4M3:
            sym[(sym & 0x7F) == 0x7F] = 0x00  # no NaN codes in the stream
            freq = oracle.build_freq(sym)
        _roundtrip(sym, rows, cols, freq, K, Z, dtype=dtype, scales=scales)


def test_roundtrip_one_million_symbols_many_chunks():
    spec = synth.TensorSpec("t", 1000, 1000, synth.DTYPE_INT8, 2.1)
    sym = synth.sample(synth.table_for(spec), 12345, 0, spec.n)
    freq = oracle.build_freq(sym)
    c = _roundtrip(sym, spec.rows, spec.cols, freq, 8, 65536,
                   scales=synth.scales_for(9, 0, 0, spec.rows))
    assert oracle.header(c)["n_chunks"] == 16  # 15 full chunks + ragged tail


# ---------------------------------------------------------------------------
# Decoder integrity flags on corrupted containers
# ---------------------------------------------------------------------------
def _small_container():
    spec = synth.TensorSpec("t", 64, 2048, synth.DTYPE_INT8, 2.1)
    sym = synth.sample(synth.table_for(spec), 777, 0, spec.n)
    freq = oracle.build_freq(sym)
    return oracle.encode(1, 64, 2048, sym, np.full(64, 0.01, np.float32), freq), sym


def test_corrupt_state_sets_integrity_flag():
    c, _ = _small_container()
    h = oracle.header(c)
    c[h["off_states"] + 4 * 5] ^= 0x01
    _, flags = oracle.decode_symbols(c)
    assert flags & (oracle.BAD_END_STATE | oracle.WORD_OVERRUN)
    # a lane state that is not a reachable final state (< 2^16) is caught too
    c, _ = _small_container()
    c[h["off_states"] + 4 * 9:h["off_states"] + 4 * 10] = [0xFF, 0xFF, 0, 0]
    _, flags = oracle.decode_symbols(c)
    assert flags != 0


def test_corrupt_word_count_is_detected():
    c, _ = _small_container()
    h = oracle.header(c)
    # claim one word fewer than stored in chunk 0: the decoder runs out of words
    wc = c[h["off_dir"] + 8:h["off_dir"] + 12].view(np.uint32)
    wc[0] -= 1
    _, flags = oracle.decode_symbols(c)
    assert flags & (oracle.BAD_END_STATE | oracle.WORD_OVERRUN)


def test_corrupt_word_sets_a_flag_or_changes_output():
    c, sym = _small_container()
    h = oracle.header(c)
    c[h["off_words"] + 2 * 10] ^= 0x40
    dec, flags = oracle.decode_symbols(c)
    assert flags != 0 or not np.array_equal(dec, sym)


# ---------------------------------------------------------------------------
# Frequency quantiser
# ---------------------------------------------------------------------------
def test_quantizer_hand_cases():
    for case in read_golden("quantizer_cases.txt")["case"]:
        lhs, rhs = case.split("->")
        counts = np.zeros(256, np.uint64)
        for tok in lhs.split():
            b, c = tok.split(":")
            counts[int(b)] = int(c)
        exp = np.zeros(256, np.uint16)
        for tok in rhs.split():
            b, f = tok.split(":")
            exp[int(b)] = int(f)
        assert np.array_equal(oracle.quantize_counts(counts), exp), case


def test_quantizer_invariants_random():
    rng = np.random.default_rng(5)
    for _ in range(3000):
        k = int(rng.integers(1, 257))
        counts = np.zeros(256, np.uint64)
        idx = rng.choice(256, size=k, replace=False)
        scale = 10 ** rng.uniform(0, 9)
        counts[idx] = np.maximum(1, (rng.pareto(1.0, k) * scale).astype(np.uint64))
        f = oracle.quantize_counts(counts)
        assert int(f.astype(np.int64).sum()) == 4096
        assert np.array_equal(f > 0, counts > 0)
        # each frequency stays within the rounding slack of its exact share
        N = float(counts.sum())
        exact = counts.astype(np.float64) * 4096 / N
        assert np.all(f[counts > 0] >= 1)
        assert np.all(np.abs(f - exact)[counts > 0] < k + 1)


def test_quantizer_cross_entropy_small_on_config_tables():
    for cfg in (1, 2):
        spec = synth.config_specs(cfg)[0]
        sym = synth.sample(synth.table_for(spec), synth.stream_key(cfg, 0, 0, 0), 0, 1 << 20)
        counts = np.bincount(sym, minlength=256).astype(np.float64)
        f = oracle.build_freq(sym).astype(np.float64)
        p = counts / counts.sum()
        m = counts > 0
        H = -(p[m] * np.log2(p[m])).sum()
        CE = -(p[m] * np.log2(f[m] / 4096)).sum()
        assert 0 <= CE - H <= 0.005 * H


# ---------------------------------------------------------------------------
# Coded size: within 1 % of N x empirical entropy
# ---------------------------------------------------------------------------
def _size_check(sym):
    counts = np.bincount(sym, minlength=256).astype(np.float64)
    p = counts[counts > 0] / sym.size
    H = float(-(p * np.log2(p)).sum())
    ideal_bytes = sym.size * H / 8
    freq = oracle.build_freq(sym)
    single = oracle.single_lane_bytes(sym, freq)
    # Shannon: a lossless code cannot beat N*H by more than the final state's 4 bytes
    assert single >= ideal_bytes - 4
    assert abs(single / ideal_bytes - 1) <= 0.01, (single, ideal_bytes)
    return H, ideal_bytes, freq


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_size_within_one_percent_of_entropy(cfg):
    for t, spec in enumerate(synth.config_specs(cfg)):
        sym = synth.make_tensor(cfg, 0, t).symbols
        H, ideal, freq = _size_check(sym)
        c = oracle.encode(spec.dtype, spec.rows, spec.cols, sym,
                          np.full(spec.rows, 0.01, np.float32), freq)
        h = oracle.header(c)
        dirs = c[h["off_dir"]:h["off_dir"] + 16 * h["n_chunks"]].reshape(-1, 16)
        words = int(dirs[:, 8:12].copy().view(np.uint32).astype(np.int64).sum())
        # container word stream at the shipping chunk size (64 Ki symbols, 64 lanes)
        assert abs(2 * words / ideal - 1) <= 0.01, (cfg, spec.name, 2 * words / ideal)
        # effective bits/weight including lane states, tables, scales: reported, not gated
        assert h["total"] * 8 / spec.n < H + 0.1


def test_size_config4_tensors_single_lane():
    """70B-block tensors (k and v in full, the others on a 16 Mi-symbol prefix)."""
    for t, spec in enumerate(synth.config_specs(4)):
        n = spec.n if spec.name in ("k", "v") else 1 << 24
        sym = synth.sample(synth.table_for(spec), synth.stream_key(4, 0, t, 0), 0, n)
        _size_check(sym)
