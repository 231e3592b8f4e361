"""Pins for the oracle's Huffman codec (EntroLLM technical overview, method
item 2: frequent weight values get short variable-length codes; item 3: the
coded stream is cut into independently decoded chunks). No GPU code.

Pinned by: a hand-derived 6-symbol code and a hand-worked one-lane container
(`tests/golden/w5_huffman_lane.txt`); brute-force optimality of the code
lengths over every complete length vector on small alphabets, with and
without a length limit; Kraft equality, the 12-bit limit and monotonicity on
random tables; the average code length within [H, H + 1) when the limit
does not bind; round trips over every short stream and random layouts;
corruption flags."""
import itertools
import math

import numpy as np
import pytest

import oracle
from conftest import read_golden

CLRS_LIKE = [45, 13, 12, 16, 9, 5]


def _counts(weights, syms=None):
    c = np.zeros(256, np.uint64)
    for i, w in enumerate(weights):
        c[syms[i] if syms else i] = w
    return c


def _len_of(table):
    t = np.asarray(table).astype(np.int64)
    return np.where(t == oracle.HUFF_ZERO, 0, t)


def test_hand_derived_six_symbol_code():
    # merges: 5+9=14, 12+13=25, 14+16=30, 25+30=55, 45+55=100, so the depths are
    # 45 -> 1; 12, 13, 16 -> 3; 5, 9 -> 4 (cost 224)
    t = oracle.huff_lengths(_counts(CLRS_LIKE))
    assert t[:6].tolist() == [1, 3, 3, 3, 4, 4]
    assert int((_len_of(t)[:6] * np.array(CLRS_LIKE)).sum()) == 224
    # canonical: (length, byte) order -> 0, 100, 101, 110, 1110, 1111
    assert oracle.huff_codes(t)[:6].tolist() == [0b0, 0b100, 0b101, 0b110, 0b1110, 0b1111]


def _brute_best(weights, L):
    """Least sum w_i * l_i over complete prefix codes with lengths in 1..L."""
    n = len(weights)
    best = None
    for ls in itertools.product(range(1, L + 1), repeat=n):
        if sum(2.0 ** -l for l in ls) != 1.0:
            continue
        cost = sum(w * l for w, l in zip(weights, ls))
        best = cost if best is None else min(best, cost)
    return best


@pytest.mark.parametrize("L", [3, 4, 12])
def test_lengths_are_optimal_by_brute_force(L):
    rng = np.random.default_rng(L)
    for trial in range(40):
        n = int(rng.integers(2, 7 if L > 3 else 9))
        if n > 2 ** L:
            continue
        w = [int(x) for x in rng.integers(1, 60, n)]
        if trial % 3 == 0:
            w = [int(x) for x in rng.geometric(0.35, n) ** 3]  # very skewed: the limit binds
        t = oracle.huff_lengths(_counts(w), L)
        ls = _len_of(t)[:n]
        assert ls.max() <= L
        assert sum(2.0 ** -int(l) for l in ls) == 1.0
        Lb = min(L, n - 1)  # lengths above n - 1 never help
        assert int((ls * np.array(w)).sum()) == _brute_best(w, max(Lb, 1) if n > 1 else 1), (w, ls.tolist())


def test_invariants_on_random_256_symbol_tables():
    rng = np.random.default_rng(5)
    for trial in range(30):
        k = int(rng.integers(2, 257))
        syms = rng.choice(256, k, replace=False)
        c = np.zeros(256, np.uint64)
        c[syms] = (rng.pareto(0.7, k) * 1e3 + 1).astype(np.uint64)
        t = oracle.huff_lengths(c)
        ls = _len_of(t)
        assert ls.max() <= 12
        assert np.all((ls > 0) == (c > 0))
        assert sum(2.0 ** -int(l) for l in ls[ls > 0]) == 1.0
        # a heavier symbol never gets a longer codeword
        order = np.argsort(-c[syms].astype(np.float64), kind="stable")
        s_sorted = syms[order]
        assert np.all(np.diff(ls[s_sorted]) >= 0) or all(
            ls[a] <= ls[b] or c[a] == c[b] for a, b in zip(s_sorted[:-1], s_sorted[1:]))


def test_average_length_within_entropy_plus_one():
    rng = np.random.default_rng(9)
    for theta in (0.2, 0.31, 0.5):
        v = np.arange(-20, 21)
        p = theta ** np.abs(v)
        p /= p.sum()
        sym = rng.choice(v, 200000, p=p).astype(np.int8).view(np.uint8)
        c = np.bincount(sym, minlength=256).astype(np.uint64)
        ls = _len_of(oracle.huff_lengths(c))
        q = c[c > 0] / c.sum()
        H = float(-(q * np.log2(q)).sum())
        avg = float((ls * c).sum() / c.sum())
        assert H <= avg < H + 1, (theta, H, avg)


def test_canonical_codes_are_prefix_free_and_ordered():
    rng = np.random.default_rng(2)
    c = np.zeros(256, np.uint64)
    c[rng.choice(256, 40, replace=False)] = rng.integers(1, 10**6, 40).astype(np.uint64)
    t = oracle.huff_lengths(c)
    code = oracle.huff_codes(t)
    ls = _len_of(t)
    present = [s for s in range(256) if ls[s]]
    words = {s: format(int(code[s]), f"0{int(ls[s])}b") for s in present}
    for a in present:
        for b in present:
            if a != b:
                assert not words[b].startswith(words[a])
    # (length, byte) order gives increasing left-aligned values
    order = sorted(present, key=lambda s: (ls[s], s))
    vals = [int(code[s]) << (12 - int(ls[s])) for s in order]
    assert vals == sorted(vals) and len(set(vals)) == len(vals)


def test_lone_symbol_is_a_zero_bit_code():
    t = oracle.huff_lengths(_counts([7], [200]))
    assert t[200] == oracle.HUFF_ZERO and np.count_nonzero(t) == 1
    sym = np.full(1000, 200, np.uint8)
    blob = oracle.encode(1, 10, 100, sym, np.ones(10, np.float32), t, 512, 8, codec=oracle.CODEC_HUFF)
    h = oracle.header(blob)
    assert h["n_words"] == 0 and h["codec"] == 1
    d, fl = oracle.decode_symbols(blob)
    assert fl == 0 and np.array_equal(d, sym)


def test_golden_one_lane_container():
    g = {k: v[0] for k, v in read_golden("w5_huffman_lane.txt").items()}
    lens = dict(tuple(int(x) for x in kv.split(":")) for kv in g["lengths"].split())
    t = np.zeros(256, np.uint16)
    for s, l in lens.items():
        t[s] = l
    codes = oracle.huff_codes(t)
    for kv in g["codes"].split():
        s, v = kv.split(":")
        assert int(codes[int(s)]) == int(v, 2)
    msg = np.array([int(x) for x in g["message"].split()], np.uint8)
    blob = oracle.encode(1, 1, msg.size, msg, np.ones(1, np.float32), t, 512, 8, codec=oracle.CODEC_HUFF)
    h = oracle.header(blob)
    exp_words = [int(w, 16) for w in g["words"].split()]
    dirw = blob[h["off_dir"]:h["off_dir"] + 16]
    assert int(dirw[8:12].view(np.uint32)[0]) == len(exp_words)
    words = blob[h["off_words"]:h["off_words"] + 2 * len(exp_words)].view(np.uint16).tolist()
    assert words == exp_words
    d, fl = oracle.decode_symbols(blob)
    assert fl == 0 and np.array_equal(d, msg)


def _w7_case():
    g = {k: v[0] for k, v in read_golden("w7_huffman_two_lanes.txt").items()}
    t = np.zeros(256, np.uint16)
    for kv in g["lengths"].split():
        sy, ln = kv.split(":")
        t[int(sy)] = int(ln)
    msg = np.array([int(x) for x in g["message"].split()], np.uint8)
    return g, t, msg


def _w7_mismatches(orc, g, t, msg):
    blob = orc.encode(1, 1, msg.size, msg, np.ones(1, np.float32), t, int(g["chunk_symbols"]),
                      int(g["lane_run"]), codec=orc.CODEC_HUFF)
    h = orc.header(blob)
    bad = []
    if int(blob[h["off_dir"] + 8:h["off_dir"] + 12].view(np.uint32)[0]) != int(g["word_count"]):
        bad.append("word count")
    exp = [int(w, 16) for w in g["words_padded"].split()]
    if blob[h["off_words"]:h["off_words"] + 2 * len(exp)].view(np.uint16).tolist() != exp:
        bad.append("words")
    d, fl = orc.decode_symbols(blob)
    if fl or not np.array_equal(d, msg):
        bad.append("decode")
    return bad, blob


def test_golden_two_lane_container():
    """Two Huffman lanes take words in the same steps (ascending lanes), lane
    1's bitstream packed like lane 0's."""
    g, t, msg = _w7_case()
    bad, _ = _w7_mismatches(oracle, g, t, msg)
    assert bad == []


def test_two_lane_golden_catches_planted_mistakes(planted):
    g, t, msg = _w7_case()
    # the encoder's replay of the refills serves the lanes in descending order
    old = ("        for (uint32_t j = 0; j < OR_LANES; j++) {\n"
           "            if (lane_pos(t, j, K) >= nk || have[j] >= 12) continue;")
    new = ("        for (uint32_t j = OR_LANES; j-- > 0;) {\n"
           "            if (lane_pos(t, j, K) >= nk || have[j] >= 12) continue;")
    with planted(old, new) as orc:
        assert _w7_mismatches(orc, g, t, msg)[0] != []
    # the decoder refills in descending lane order: it misreads the good container
    _, blob = _w7_mismatches(oracle, g, t, msg)
    old = ("        for (uint32_t j = 0; j < OR_LANES; j++) {\n"
           "            if (lane_pos(t, j, K) >= nk || n[j] >= 12) continue;")
    new = ("        for (uint32_t j = OR_LANES; j-- > 0;) {\n"
           "            if (lane_pos(t, j, K) >= nk || n[j] >= 12) continue;")
    with planted(old, new) as orc:
        d, fl = orc.decode_symbols(blob)
        assert fl != 0 or not np.array_equal(d, msg)
    # a lane refills while it holds fewer than 13 bits instead of 12
    with planted("if (lane_pos(t, j, K) >= nk || have[j] >= 12) continue;",
                 "if (lane_pos(t, j, K) >= nk || have[j] >= 13) continue;") as orc:
        assert _w7_mismatches(orc, g, t, msg)[0] != []


def test_every_short_stream_round_trips():
    tables = [
        {0: 1, 1: 1},
        {3: 1, 4: 2, 5: 2},
        {0: 2, 1: 2, 2: 2, 3: 2},
        {9: 1, 10: 3, 11: 3, 12: 3, 13: 3},
    ]
    for tab in tables:
        t = np.zeros(256, np.uint16)
        for s, l in tab.items():
            t[s] = l
        alphabet = list(tab)
        for n in range(1, 6):
            for seq in itertools.product(alphabet, repeat=n):
                sym = np.array(seq, np.uint8)
                for K in (1, 8):
                    blob = oracle.encode(1, 1, n, sym, np.ones(1, np.float32), t, 64 * K, K,
                                         codec=oracle.CODEC_HUFF)
                    d, fl = oracle.decode_symbols(blob)
                    assert fl == 0 and np.array_equal(d, sym), (tab, seq, K)


def test_random_layouts_round_trip_and_dequant():
    rng = np.random.default_rng(17)
    for trial in range(60):
        K = int(rng.choice([1, 2, 4, 8, 16]))
        Z = 64 * K * int(rng.integers(1, 9))
        rows, cols = int(rng.integers(1, 9)), int(rng.integers(1, 700))
        n = rows * cols
        k = int(rng.integers(1, 40))
        alpha = rng.choice(256, k, replace=False)
        p = rng.dirichlet(np.full(k, 0.3))
        sym = rng.choice(alpha, n, p=p).astype(np.uint8)
        dtype = int(rng.choice([1, 2]))
        if dtype == 2:
            sym[(sym & 0x7F) == 0x7F] = 0x10  # no E4M3 NaN codes
        t = oracle.huff_lengths(np.bincount(sym, minlength=256))
        scales = rng.uniform(0.5, 2.0, rows).astype(np.float32)
        blob = oracle.encode(dtype, rows, cols, sym, scales, t, Z, K, codec=oracle.CODEC_HUFF)
        d, fl = oracle.decode_symbols(blob)
        assert fl == 0 and np.array_equal(d, sym), trial
        bf, fl = oracle.decode_dequant(blob)
        assert fl == 0
        assert np.array_equal(bf, oracle.dequant_direct(dtype, sym, cols, scales))


def test_corruption_is_flagged():
    rng = np.random.default_rng(4)
    sym = rng.choice([0, 1, 2, 255], 4096, p=[0.6, 0.2, 0.15, 0.05]).astype(np.uint8)
    t = oracle.huff_lengths(np.bincount(sym, minlength=256))
    blob = oracle.encode(1, 4, 1024, sym, np.ones(4, np.float32), t, 4096, 8, codec=oracle.CODEC_HUFF)
    h = oracle.header(blob)
    # fewer words in the directory than the lanes take: overrun
    bad = blob.copy()
    wc = int(bad[h["off_dir"] + 8:h["off_dir"] + 12].view(np.uint32)[0])
    bad[h["off_dir"] + 8:h["off_dir"] + 12] = np.array([wc - 1], np.uint32).view(np.uint8)
    _, fl = oracle.decode_symbols(bad)
    assert fl & oracle.WORD_OVERRUN
    # an extra word the lanes never take
    bad = blob.copy()
    bad[h["off_dir"] + 8:h["off_dir"] + 12] = np.array([wc + 1], np.uint32).view(np.uint8)
    _, fl = oracle.decode_symbols(bad)
    assert fl & oracle.BAD_END_STATE
    # an incomplete length table is rejected by the parser
    bad = blob.copy()
    lt = bad[h["off_freq"]:h["off_freq"] + 512].view(np.uint16).copy()
    lt[np.flatnonzero(lt)[0]] += 1
    bad[h["off_freq"]:h["off_freq"] + 512] = lt.view(np.uint8)
    with pytest.raises(oracle.OracleError):
        oracle.decode_symbols(bad)


def test_tie_rule_hand_derived():
    """Five equal counts (bytes 0..4). Coins sorted by (count, byte); a coin
    goes before a package of equal weight. Deep lists settle into
    [c0..c4, (c0,c1), (c2,c3), (c4, (c0,c1)'), ...]; the first 2n - 2 = 8 items
    of the top list are c0..c4, (c0,c1), (c2,c3), (c4, (c0,c1)'), so bytes 0
    and 1 occur 3 times and bytes 2, 3, 4 twice. Canonical codes: length 2 ->
    00, 01, 10 for bytes 2, 3, 4; length 3 starts at (0 + 3) << 1 = 110."""
    t = oracle.huff_lengths(_counts([1, 1, 1, 1, 1]))
    assert t[:5].tolist() == [3, 3, 2, 2, 2]
    assert oracle.huff_codes(t)[:5].tolist() == [0b110, 0b111, 0b00, 0b01, 0b10]
