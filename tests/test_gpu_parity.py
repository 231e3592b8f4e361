"""GPU parity: libeq's HIP decode (through the C ABI) against the oracle,
bit-exact (0 ULP for bf16, byte-exact for the decoded symbols).

The expected outputs come only from the oracle (`oracle.dequant_direct` on
the original symbols, i.e. the exact result of lossless decoding followed by
the per-row dequantisation) and from the original symbols themselves."""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import gpu_available
from gpu_util import Packed, assert_same, encode, expected_bf16, log, run_bf16, run_u8
from rans_decode_amd import eq

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _dev(blob):
    return eq.DeviceContainer(blob, device="cuda")


def _check_tensor(t, chunk_symbols=65536, lane_run=8, what=""):
    blob = encode(t, chunk_symbols, lane_run)
    c = _dev(blob)
    got, st = run_bf16([c], t.spec.n)
    assert st == 0, f"{what}: device status {st}"
    assert_same(got, expected_bf16(t), f"{what} bf16")
    sym, st = run_u8([c], t.spec.n)
    assert st == 0
    assert_same(sym, t.symbols, f"{what} symbols")


def test_smoke_int8_escapes():
    spec = synth.TensorSpec("down", 16, 8192, synth.DTYPE_INT8, 2.1, 4)
    t = synth.make_tensor(4, 0, 6, spec=spec)
    log(f"case smoke {spec}")
    _check_tensor(t, what="smoke")


@pytest.mark.parametrize("cfg", [1, 2])
def test_config_single_matrix(cfg):
    t = synth.make_tensor(cfg, 0, 0)
    Z = synth.config_chunk(cfg)
    log(f"case config {cfg}: {t.spec}, {Z}-symbol chunks")
    _check_tensor(t, Z, what=f"config {cfg}")
    if Z != 65536:
        _check_tensor(t, 65536, what=f"config {cfg}, 64 Ki chunks")


def _block_case(cfg, layer=0, chunk=None):
    specs = synth.config_specs(cfg)
    offs = synth.block_offsets(specs)
    tensors = [synth.make_tensor(cfg, layer, i) for i in range(len(specs))]
    blobs = [encode(t, chunk or synth.config_chunk(cfg)) for t in tensors]
    return specs, offs, tensors, blobs


@pytest.mark.parametrize("cfg,chunk", [(3, None), (4, None), (3, 65536), (4, 65536)])
def test_config_block_full(cfg, chunk):
    """The whole block into one buffer, one call (config 3: 7B E4M3 block,
    202 M weights; config 4: 70B int8 block with escapes, 856 M weights),
    every output element compared; at the configuration's chunk size and at
    64 Ki."""
    log(f"case config {cfg} block, chunk {chunk or synth.config_chunk(cfg)}: generating")
    specs, offs, tensors, blobs = _block_case(cfg, chunk=chunk)
    conts = [_dev(b) for b in blobs]
    log(f"case config {cfg} block: decode")
    got, st = run_bf16(conts, offs[-1], offsets=offs[:-1])
    assert st == 0
    for t, o in zip(tensors, offs):
        assert_same(got[o:o + t.spec.n], expected_bf16(t), f"config {cfg} {t.spec.name}")
    del got
    sym, st = run_u8(conts, offs[-1], offsets=offs[:-1])
    assert st == 0
    for t, o in zip(tensors, offs):
        assert_same(sym[o:o + t.spec.n], t.symbols, f"config {cfg} {t.spec.name} symbols")


@pytest.mark.parametrize("K", [1, 2, 4, 8, 16])
def test_lane_runs_and_ragged_tails(K):
    """Every lane run K, chunk sizes down to one 64K group, tensors ending in a
    partial group and a partial lane run, fast and general store paths."""
    rng = np.random.default_rng(K)
    cases = []
    for (rows, cols), zmul in itertools.product([(1, 1), (3, 7), (7, 1000), (64, 8 * K + 3),
                                                 (33, 64 * K), (5, 8192), (130, 520)], [1, 3, 16]):
        Z = 64 * K * zmul
        dtype = synth.DTYPE_INT8 if (rows + cols) % 2 else synth.DTYPE_E4M3
        spec = synth.TensorSpec("t", rows, cols, dtype, 2.1 if zmul != 3 else 4.5)
        t = synth.make_tensor(90 + K, rows, cols, spec=spec)
        t.scales = rng.uniform(-0.02, 0.02, rows).astype(np.float32)
        cases.append((t, Z))
    blobs = [encode(t, Z, K) for t, Z in cases]
    pk = Packed(blobs)
    offs, o = [], 0
    for t, _ in cases:
        offs.append(o)
        o += t.spec.n
    log(f"case K={K}: {len(cases)} tensors")
    got, st = run_bf16(pk.items, o, offsets=offs)
    assert st == 0
    sym, st2 = run_u8(pk.items, o, offsets=offs)
    assert st2 == 0
    for (t, Z), off in zip(cases, offs):
        assert_same(got[off:off + t.spec.n], expected_bf16(t), f"K={K} Z={Z} {t.spec.rows}x{t.spec.cols}")
        assert_same(sym[off:off + t.spec.n], t.symbols, f"K={K} symbols")


def test_unaligned_offsets_touch_nothing_else():
    spec = synth.TensorSpec("t", 40, 4096, synth.DTYPE_INT8, 2.1)
    t = synth.make_tensor(77, 0, 0, spec=spec)
    c = _dev(encode(t))
    for off in (1, 3, 5, 8, 13):
        got, st = run_bf16([c], off + spec.n + 11, offsets=[off], fill=0x1234)
        assert st == 0
        assert np.all(got[:off] == 0x1234) and np.all(got[off + spec.n:] == 0x1234)
        assert_same(got[off:off + spec.n], expected_bf16(t), f"offset {off}")
        sym, st = run_u8([c], off + spec.n + 7, offsets=[off], fill=0xA5)
        assert np.all(sym[:off] == 0xA5) and np.all(sym[off + spec.n:] == 0xA5)
        assert_same(sym[off:off + spec.n], t.symbols, f"offset {off} symbols")


def test_escapes_at_boundaries():
    """Super weights at chunk starts/ends, in partial groups and lane runs,
    and many of them in one group."""
    rows, cols = 37, 4100
    spec = synth.TensorSpec("t", rows, cols, synth.DTYPE_INT8, 2.1)
    t = synth.make_tensor(78, 0, 0, spec=spec)
    n = spec.n
    Z = 4096
    pos = sorted({0, 1, 7, 8, 511, 512, Z - 1, Z, Z + 1, 2 * Z + 300, n - 1, n - 2, n - 513,
                  *range(5000, 5100, 3)})
    sym = t.symbols.copy()
    sym[sym == 0x80] = 0
    sym[np.array(pos)] = 0x80
    t.symbols = sym
    t.esc_idx = np.array(pos, np.uint64)
    t.esc_val = (np.arange(len(pos), dtype=np.uint16) * 977 + 0x3F00).astype(np.uint16)
    for K in (1, 8, 16):
        c = _dev(encode(t, Z, K))
        got, st = run_bf16([c], n)
        assert st == 0
        assert_same(got, expected_bf16(t), f"escapes K={K}")


def test_e4m3_all_codes_and_escape_code():
    """Every non-NaN E4M3 code, through the kernel's FP8 conversion, with
    the NaN code 0x7F used as the super-weight escape."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    rng = np.random.default_rng(5)
    rows, cols = 64, 2048
    sym = codes[rng.integers(0, codes.size, rows * cols)]
    esc = np.sort(rng.choice(rows * cols, 9, replace=False)).astype(np.uint64)
    sym[esc.astype(np.int64)] = 0x7F
    spec = synth.TensorSpec("e", rows, cols, synth.DTYPE_E4M3, 8.0)
    t = synth.Tensor(spec, sym, rng.uniform(-3, 3, rows).astype(np.float32), esc,
                     rng.integers(0, 0x7F00, esc.size).astype(np.uint16))
    _check_tensor(t, 8192, 8, "e4m3 all codes")


def test_edge_scales_denormals_ties_and_overflow():
    """Scales that make products subnormal, exact bf16 ties and overflow to
    inf, through the fused multiply + bf16 rounding."""
    scale_bits = np.array([0x3C23D70A, 0x00080000, 0x00000001, 0x3F808000, 0x3F818000,
                           0x7F7FFFFF, 0xBF800000, 0x80000000, 0x00800000, 0x7E800000,
                           0x3A000000, 0x43E00000, 0x00010000, 0x3F80FFFF], np.uint32)
    rows = scale_bits.size
    cols = 1024
    rng = np.random.default_rng(8)
    for dtype in (synth.DTYPE_INT8, synth.DTYPE_E4M3):
        codes = np.arange(256, dtype=np.uint8)
        if dtype == synth.DTYPE_E4M3:
            codes = codes[(codes & 0x7F) != 0x7F]
        sym = np.concatenate([codes, codes[rng.integers(0, codes.size, rows * cols - codes.size)]])
        sym = sym.astype(np.uint8)
        spec = synth.TensorSpec("s", rows, cols, dtype, 8.0)
        t = synth.Tensor(spec, sym, scale_bits.view(np.float32).copy())
        _check_tensor(t, 65536, 8, f"edge scales dtype {dtype}")


def test_single_symbol_tensor_and_empty_block():
    spec = synth.TensorSpec("c", 20, 3000, synth.DTYPE_INT8, 0.0)
    sym = np.full(spec.n, 0xFE, np.uint8)
    t = synth.Tensor(spec, sym, np.linspace(0.001, 1.0, 20).astype(np.float32))
    _check_tensor(t, 65536, 8, "single symbol")
    # with escapes too
    sym2 = sym.copy()
    idx = np.array([3, 59999], np.uint64)
    sym2[idx.astype(np.int64)] = 0x80
    t2 = synth.Tensor(spec, sym2, t.scales, idx, np.array([0x4000, 0xC000], np.uint16))
    _check_tensor(t2, 4096, 4, "two symbols + escapes")
    # empty block: nothing enqueued, nothing written
    out = torch.full((16,), 7, dtype=torch.int16, device="cuda")
    eq.decode_dequant_bf16([], out)
    torch.cuda.synchronize()
    assert torch.all(out == 7)


def test_many_tensors_mixed_lane_runs_in_one_call():
    """More tensors than one launch holds, with different K: the library
    splits the call into several launches on the same stream."""
    tensors, blobs = [], []
    for i in range(41):
        K = [8, 8, 4, 16, 1, 2][i % 6]
        spec = synth.TensorSpec(f"t{i}", 3 + i, 700 + 37 * i,
                                synth.DTYPE_INT8 if i % 3 else synth.DTYPE_E4M3, 2.1 + (i % 4))
        t = synth.make_tensor(79, i, 0, spec=spec)
        tensors.append(t)
        blobs.append(encode(t, 64 * K * (1 + i % 3), K))
    pk = Packed(blobs)
    offs = synth.block_offsets([t.spec for t in tensors])
    got, st = run_bf16(pk.items, offs[-1], offsets=offs[:-1])
    assert st == 0
    for t, o in zip(tensors, offs):
        assert_same(got[o:o + t.spec.n], expected_bf16(t), t.spec.name)


def test_brute_force_tiny_streams_batched():
    """All streams of length 1..7 over 3 symbols, tables from the oracle's
    hand set, K in {1, 8}: ~6.5k tiny tensors decoded in batched launches."""
    tables = {"4000/80/16": {0x00: 4000, 0x01: 80, 0xFF: 16},
              "1366/1365/1365": {0x00: 1366, 0x01: 1365, 0xFF: 1365},
              "4094/1/1": {0x00: 4094, 0x01: 1, 0xFF: 1}}
    for name, tab in tables.items():
        freq = np.zeros(256, np.uint16)
        for b, f in tab.items():
            freq[b] = f
        et = eq.tables_from_freq(freq)
        for K in (1, 8):
            streams = [np.array(s, np.uint8) for L in range(1, 8)
                       for s in itertools.product(sorted(tab), repeat=L)]
            blobs, tens = [], []
            for s in streams:
                spec = synth.TensorSpec("b", 1, s.size, synth.DTYPE_INT8, 1.0)
                t = synth.Tensor(spec, s, np.array([0.37], np.float32))
                tens.append(t)
                blobs.append(encode(t, 64 * K, K, tables=et))
            pk = Packed(blobs)
            offs = synth.block_offsets([t.spec for t in tens])
            got, st = run_bf16(pk.items, offs[-1], offsets=offs[:-1])
            assert st == 0
            exp = np.concatenate([expected_bf16(t) for t in tens])
            assert_same(got, exp, f"brute force {name} K={K}")
            sym, st = run_u8(pk.items, offs[-1], offsets=offs[:-1])
            assert st == 0
            assert_same(sym, np.concatenate(streams), f"brute force symbols {name} K={K}")


def test_max_chunk_size_single_chunk():
    spec = synth.TensorSpec("big", 1024, 4096, synth.DTYPE_INT8, 2.1)
    t = synth.make_tensor(80, 0, 0, spec=spec)
    _check_tensor(t, 1 << 22, 16, "4 Mi-symbol chunk")


def test_corruption_sets_device_flags():
    """Bit flips in the device copy of words / states: the kernel stays in
    bounds and reports through the status word (or the output differs)."""
    spec = synth.TensorSpec("t", 64, 8192, synth.DTYPE_INT8, 2.1)
    t = synth.make_tensor(81, 0, 0, spec=spec)
    blob = encode(t)
    h = eq.parse_header(blob)
    exp = expected_bf16(t)
    for where in ("state", "word"):
        bad = blob.copy()
        if where == "state":
            bad[h.off_states + 4 * 70 + 1] ^= 0x10
        else:
            bad[h.off_words + 2 * 100] ^= 0x21
        c = eq.DeviceContainer.__new__(eq.DeviceContainer)
        c.host, c.hdr = bad, h
        c.dev = torch.from_numpy(bad).cuda()
        got, st = run_bf16([c], spec.n)
        assert st != 0 or not np.array_equal(got, exp), where
        assert st in (0, 1, 2, 3)


def test_bf16_rounding_exhaustive_all_fp32_patterns():
    """The decode kernel's fp32 -> bf16 rounding (v_cvt_pk_bf16_f32) over all
    2^32 inputs against the oracle's definition (NaN: any NaN)."""
    step = 1 << 28
    for s in range(0, 1 << 32, step):
        bits = torch.arange(s, s + step, dtype=torch.int64, device="cuda").to(torch.int32)
        x = bits.view(torch.float32)
        out = torch.empty(step, dtype=torch.int16, device="cuda")
        eq.eq_bf16_from_f32(x, out)
        got = out.cpu().numpy().view(np.uint16)
        xh = (np.arange(step, dtype=np.uint64) + s).astype(np.uint32).view(np.float32)
        exp = oracle.bf16_rne(xh)
        nan = np.isnan(xh)
        ok = (got == exp) | nan
        assert ok.all(), f"slice {s:#x}: first bad {int(np.flatnonzero(~ok)[0]) + s:#x}"
        g = got[nan]
        assert np.all(((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0))
        log(f"bf16 slice {s >> 28}/16 ok")


def test_gemv_matches_fp64_within_bound():
    rng = np.random.default_rng(4)
    for rows, cols in ((1024, 8192), (300, 2056), (64, 28672)):
        w = torch.from_numpy(rng.standard_normal((rows, cols)).astype(np.float32)).to(torch.bfloat16)
        x = torch.from_numpy(rng.standard_normal(cols).astype(np.float32)).to(torch.bfloat16)
        wd, xd = w.cuda(), x.cuda()
        y = torch.empty(rows, dtype=torch.float32, device="cuda")
        eq.eq_gemv_bf16(wd.view(torch.int16), rows, cols, xd.view(torch.int16), y)
        torch.cuda.synchronize()
        w64 = w.double().numpy()
        x64 = x.double().numpy()
        ref = w64 @ x64
        bound = cols * 2.0 ** -23 * (np.abs(w64) @ np.abs(x64))
        assert np.all(np.abs(y.cpu().numpy() - ref) <= bound), (rows, cols)


@pytest.mark.parametrize("mode", [eq.EQ_PIPELINE_ALTERNATE, eq.EQ_PIPELINE_OVERLAP])
def test_pipeline_double_buffered_small_model(mode):
    """Block-by-block schedule on two streams (decode into alternating
    buffers, GEMVs on the other stream): every GEMV output equals the same
    GEMV over that block decoded into its own buffer, bit for bit, and every
    decoded block equals the oracle."""
    L = 5
    shapes = [("q", 256, 1024), ("k", 64, 1024), ("v", 64, 1024), ("o", 256, 1024),
              ("gate", 512, 1024), ("up", 512, 1024), ("down", 256, 2048)]
    specs = [synth.TensorSpec(nm, r, c, synth.DTYPE_INT8, 2.1, 2 if nm == "down" else 0)
             for nm, r, c in shapes]
    offs = synth.block_offsets(specs)
    blocks, tens, xs, ys = [], [], [], []
    for layer in range(L):
        ts = [synth.make_tensor(95, layer, i, spec=sp) for i, sp in enumerate(specs)]
        tens.append(ts)
        conts = [eq.DeviceContainer(encode(t, 16384, 8)) for t in ts]
        blocks.append(eq.Block(conts, offs[:-1]))
        xs.append([torch.from_numpy(synth.gemv_activation(95, layer, i, sp.cols)).to(torch.bfloat16).cuda()
                   for i, sp in enumerate(specs)])
        ys.append([torch.full((sp.rows,), float("nan"), dtype=torch.float32, device="cuda") for sp in specs])
    n = offs[-1]
    bufs = [torch.empty(n, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ds, gs = torch.cuda.Stream(), torch.cuda.Stream()
    pipe = eq.Pipeline(L, mode)
    with pytest.raises(eq.EqError):
        pipe.set_mode(2)  # unknown mode: EQ_EINVAL, the plan keeps its mode
    for _ in range(2):
        pipe.run(blocks, bufs[0], bufs[1], xs, ys, ds, gs)
    torch.cuda.synchronize()
    # reference: each block decoded into its own buffer, same GEMV kernel
    for layer in range(L):
        own = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        eq.eq_decode_dequant_bf16(blocks[layer], own)
        torch.cuda.synchronize()
        got = own.view(torch.int16).cpu().numpy().view(np.uint16)
        for t, o in zip(tens[layer], offs):
            assert_same(got[o:o + t.spec.n], expected_bf16(t), f"layer {layer} {t.spec.name}")
        for i, (sp, o) in enumerate(zip(specs, offs)):
            yr = torch.empty(sp.rows, dtype=torch.float32, device="cuda")
            eq.eq_gemv_bf16(own.view(torch.int16), sp.rows, sp.cols, xs[layer][i].view(torch.int16), yr,
                            w_offset_elems=o)
            torch.cuda.synchronize()
            assert torch.equal(yr.view(torch.int32), ys[layer][i].view(torch.int32)), (layer, sp.name)
    pipe.close()
