"""GPU parity of the Huffman codec (EntroLLM technical overview, method item
2: Huffman weight coding; item 3: independently decoded chunks) through the
same C ABI calls as the rANS codec: decoded symbols byte-exact, bf16 outputs
bit-exact (0 ULP), the fused GEMV one-hot exact and within the fp32 bound.

Containers come from the library's encoder, which is byte-equal to the
oracle's Huffman encoder (CPU tests); expected outputs come only from the
oracle (`oracle.dequant_direct` on the original symbols, `oracle.gemv_f64`)
and from the original symbols."""
import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import gpu_available
from gpu_util import Packed, assert_same, encode, expected_bf16, log, run_bf16, run_u8
from rans_decode_amd import eq
from test_gpu_gemv import check_close, one_hot_exact, run_gemv

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

HUFF = eq.EQ_CODEC_HUFFMAN


def _check(t, Z=65536, K=8, what=""):
    blob = encode(t, Z, K, codec=HUFF)
    assert eq.parse_header(blob).codec == HUFF
    d, fl = oracle.decode_symbols(blob)
    assert fl == 0 and np.array_equal(d, t.symbols)
    c = eq.DeviceContainer(blob, device="cuda")
    got, st = run_bf16([c], t.spec.n)
    assert st == 0, f"{what}: device status {st}"
    assert_same(got, expected_bf16(t), f"{what} bf16")
    sym, st = run_u8([c], t.spec.n)
    assert st == 0
    assert_same(sym, t.symbols, f"{what} symbols")
    return c


@pytest.mark.parametrize("K", [1, 2, 4, 8, 16])
def test_lane_runs_and_ragged_tails(K):
    for rows, cols, Z in [(3, 1000, 64 * K * 3), (7, 4096, 65536 // K * K), (1, 777, 64 * K)]:
        spec = synth.TensorSpec("t", rows, cols, synth.DTYPE_INT8, 2.1, 2)
        t = synth.make_tensor(4, 90 + K, 6, spec=spec)
        log(f"case huffman K={K} {rows}x{cols} Z={Z}")
        _check(t, Z, K, f"K={K} {rows}x{cols}")


@pytest.mark.parametrize("dtype,bits", [(synth.DTYPE_INT8, 2.1), (synth.DTYPE_INT8, 3.0),
                                        (synth.DTYPE_E4M3, 2.1), (synth.DTYPE_E4M3, 4.5)])
def test_entropies_and_dtypes(dtype, bits):
    spec = synth.TensorSpec("t", 256, 4096, dtype, bits, 5)
    t = synth.make_tensor(3 if dtype == synth.DTYPE_E4M3 else 4, 7, 6, spec=spec)
    log(f"case huffman dtype={dtype} H={bits}")
    c = _check(t, what=f"dtype {dtype} H {bits}")
    h = eq.parse_header(c.host)
    lens = c.host[h.off_freq:h.off_freq + 512].view(np.uint16)
    assert lens.max() <= 12


def test_wide_alphabet_hits_the_length_limit():
    """Near-uniform bytes plus a few very rare ones: long codewords, the
    12-bit limit, every one of the 256 symbols present."""
    rng = np.random.default_rng(5)
    n = 64 * 4096
    p = np.full(256, 1.0)
    p[:8] = 4000.0
    p[200:] = 1e-3
    sym = rng.choice(256, n, p=p / p.sum()).astype(np.uint8)
    sym[:256] = np.arange(256, dtype=np.uint8)
    spec = synth.TensorSpec("w", 64, 4096, synth.DTYPE_INT8, 0.0)
    t = synth.Tensor(spec, sym, np.linspace(0.5, 2.0, 64).astype(np.float32))
    c = _check(t, 16384, 8, "wide alphabet")
    h = eq.parse_header(c.host)
    lens = c.host[h.off_freq:h.off_freq + 512].view(np.uint16)
    assert lens.max() == 12 and np.count_nonzero(lens) == 256


def test_single_symbol_and_all_escapes():
    spec = synth.TensorSpec("c", 20, 3000, synth.DTYPE_E4M3, 0.0)
    t = synth.Tensor(spec, np.full(spec.n, 0x38, np.uint8), np.linspace(0.001, 1.0, 20).astype(np.float32))
    c = _check(t, 192000, 8, "single symbol")
    assert eq.parse_header(c.host).single_symbol == 0x38
    # two symbols: 1-bit codes
    sym = np.where(np.arange(spec.n) % 3 == 0, 0x38, 0x40).astype(np.uint8)
    t2 = synth.Tensor(spec, sym, t.scales)
    _check(t2, 4096, 4, "two symbols")


def test_config_3_and_4_blocks_every_element():
    for cfg in (3, 4):
        specs = synth.config_specs(cfg)
        offs = synth.block_offsets(specs)
        log(f"case huffman config {cfg} block")
        tensors = [synth.make_tensor(cfg, 0, i) for i in range(len(specs))]
        conts = [eq.DeviceContainer(encode(t, codec=HUFF), device="cuda") for t in tensors]
        got, st = run_bf16(conts, offs[-1], offsets=offs[:-1])
        assert st == 0
        for t, o in zip(tensors, offs):
            assert_same(got[o:o + t.spec.n], expected_bf16(t), f"config {cfg} {t.spec.name}")
        del got, tensors, conts


def test_mixed_codecs_in_one_call():
    """rANS and Huffman tensors, different K, in one block call."""
    tensors, blobs = [], []
    for i in range(10):
        K = [8, 4, 8, 16, 2][i % 5]
        spec = synth.TensorSpec(f"t{i}", 16 + i, 1024, synth.DTYPE_INT8 if i % 3 else synth.DTYPE_E4M3,
                                2.1 + 0.2 * i, i % 3)
        t = synth.make_tensor(3 if spec.dtype == synth.DTYPE_E4M3 else 4, 40 + i, 6, spec=spec)
        tensors.append(t)
        blobs.append(encode(t, 64 * K * 4, K, codec=HUFF if i % 2 else 0))
    pk = Packed(blobs)
    offs, o = [], 0
    for t in tensors:
        offs.append(o)
        o += t.spec.n + 24
    got, st = run_bf16(pk.items, o, offsets=offs)
    assert st == 0
    for t, off in zip(tensors, offs):
        assert_same(got[off:off + t.spec.n], expected_bf16(t), t.spec.name)


def test_fused_gemv_on_huffman_containers():
    spec = synth.TensorSpec("down", 24, 28672, synth.DTYPE_INT8, 2.1, 4)
    t = synth.make_tensor(4, 60, 6, spec=spec)
    c = eq.DeviceContainer(encode(t, 57344, 8, codec=HUFF), device="cuda")
    w = expected_bf16(t).reshape(spec.rows, spec.cols)
    x = oracle.bf16_rne(np.random.default_rng(1).standard_normal(spec.cols).astype(np.float32))
    (y,), st = run_gemv([c], [x], [spec.rows])
    assert st == 0
    check_close(y, w, x, "huffman gemv")
    one_hot_exact(c, w, [0, 12345, spec.cols - 1], "huffman gemv")


def test_corrupted_words_set_device_flags():
    rng = np.random.default_rng(8)
    spec = synth.TensorSpec("t", 64, 4096, synth.DTYPE_INT8, 2.1)
    t = synth.make_tensor(4, 33, 0, spec=spec)
    blob = encode(t, 65536, 8, codec=HUFF)
    h = eq.parse_header(blob)
    flags_seen = 0
    for trial in range(6):
        bad = blob.copy()
        w = bad[h.off_words:h.off_words + 2 * h.n_words].view(np.uint16)
        i = int(rng.integers(0, int(h.n_words) // 2))
        w[i] ^= np.uint16(1 << int(rng.integers(0, 16)))
        c = eq.DeviceContainer(bad, device="cuda")
        got, st = run_u8([c], spec.n)
        assert st in (0, 1, 2, 3)
        flags_seen |= st
        if st == 0:
            # an undetected flip must still have changed some symbol
            assert not np.array_equal(got, t.symbols)
    assert flags_seen != 0
