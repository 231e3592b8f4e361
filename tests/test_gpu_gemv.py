"""GPU parity of the fused decode + batch-1 GEMV (`eq_decode_gemv_bf16`),
through the C ABI, against the oracle.

The fused kernel never writes the weights, so the decode is pinned through
the product: with x a one-hot vector every y[r] is one weight times 1.0 plus
exact zeros, which must equal the oracle's bf16 weight bit for bit; with a
random x, y must lie within cols * 2^-23 * sum_c |W[r, c] x[c]| of the
oracle's binary64 product (fp32 accumulation in a different order from the
oracle's; every bf16 x bf16 product is exact in fp32, so only the additions
round). Expected weights come only from the oracle (`oracle.dequant_direct`
on the original symbols, i.e. lossless decoding followed by the per-row
dequantisation) and expected products from `oracle.gemv_f64`."""
import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import gpu_available
from gpu_util import encode, expected_bf16, log
from rans_decode_amd import eq

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _x_bits(cols, seed):
    rng = np.random.default_rng(seed)
    return oracle.bf16_rne(rng.standard_normal(cols).astype(np.float32))


def _dev_x(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def run_gemv(containers, x_bits_list, rows_list, stream=None):
    xs = [_dev_x(b) for b in x_bits_list]
    ys = [torch.full((r,), float("nan"), dtype=torch.float32, device="cuda") for r in rows_list]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    blk = eq.Block(containers, status=status)
    eq.eq_decode_gemv_bf16(blk, xs, ys, stream)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys], int(status.item())


def check_close(y, w_bits, x_bits, what):
    y64, absdot = oracle.gemv_f64(w_bits, x_bits)
    cols = w_bits.shape[1]
    assert np.isfinite(y).all(), f"{what}: non-finite output"
    err = np.abs(y.astype(np.float64) - y64)
    tol = cols * 2.0**-23 * absdot
    bad = np.flatnonzero(err > tol)
    assert bad.size == 0, (f"{what}: {bad.size} rows out of bound, first {bad[0]}: "
                           f"got {y[bad[0]]!r} exact {y64[bad[0]]!r} tol {tol[bad[0]]!r}")


def one_hot_exact(c, w_bits, cols_list, what):
    """y for x = e_col must be exactly column col of W (as fp32)."""
    rows, cols = w_bits.shape
    for col in cols_list:
        x = np.zeros(cols, np.uint16)
        x[col] = 0x3F80
        (y,), st = run_gemv([c], [x], [rows])
        assert st == 0
        exp = (w_bits[:, col].astype(np.uint32) << 16).view(np.float32)
        got = y.view(np.uint32)
        # +0 and -0 both stand for a zero weight times 1.0 plus zeros
        same = (got == exp.view(np.uint32)) | ((exp == 0) & (y == 0))
        assert same.all(), f"{what}: column {col}, first bad row {np.flatnonzero(~same)[0]}"


def _case(spec, Z, K, seed=0, what=""):
    t = synth.make_tensor(4, 50 + seed, 6 if spec.n_esc else 0, spec=spec)
    blob = encode(t, Z, K)
    c = eq.DeviceContainer(blob, device="cuda")
    w = expected_bf16(t).reshape(spec.rows, spec.cols)
    x = _x_bits(spec.cols, seed)
    log(f"case {what}: {spec} Z={Z} K={K}")
    (y,), st = run_gemv([c], [x], [spec.rows])
    assert st == 0, f"{what}: device status {st}"
    check_close(y, w, x, what)
    return t, c, w, x, y


@pytest.mark.parametrize("rows,cols,Z,K,dtype,n_esc", [
    (64, 1024, 65536, 8, synth.DTYPE_INT8, 0),     # row-uniform groups, one chunk
    (300, 2048, 16384, 8, synth.DTYPE_INT8, 5),    # 38 chunks, tail chunk of 4 rows
    (150, 1000, 64000, 8, synth.DTYPE_INT8, 3),    # groups straddle rows
    (100, 64, 4096, 8, synth.DTYPE_E4M3, 4),       # 8 rows per group
    (40, 4096, 16384, 1, synth.DTYPE_INT8, 2),
    (40, 4096, 16384, 2, synth.DTYPE_E4M3, 2),
    (24, 11008, 44032, 4, synth.DTYPE_E4M3, 3),    # 7B down_proj row length
    (130, 1040, 66560, 16, synth.DTYPE_INT8, 3),   # K = 16, straddling groups
    (16, 28672, 57344, 8, synth.DTYPE_INT8, 4),    # 70B down_proj row length, 2 rows/chunk
])
def test_fused_gemv_shapes(rows, cols, Z, K, dtype, n_esc):
    spec = synth.TensorSpec("t", rows, cols, dtype, 2.1 if dtype == synth.DTYPE_INT8 else 2.3, n_esc)
    t, c, w, x, y = _case(spec, Z, K, seed=rows, what=f"{rows}x{cols}")
    one_hot_exact(c, w, [0, cols // 2 + 1, cols - 1], f"{rows}x{cols}")
    # deterministic: a second call gives the same bits
    (y2,), _ = run_gemv([c], [x], [rows])
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_super_weights_reach_the_product():
    """One-hot columns through each super weight: y[row] is the listed bf16
    value itself."""
    spec = synth.TensorSpec("down", 32, 8192, synth.DTYPE_INT8, 2.1, 6)
    t = synth.make_tensor(4, 61, 6, spec=spec)
    c = eq.DeviceContainer(encode(t, 65536, 8), device="cuda")
    w = expected_bf16(t).reshape(spec.rows, spec.cols)
    for idx, val in zip(t.esc_idx.tolist(), t.esc_val.tolist()):
        r, col = divmod(int(idx), spec.cols)
        x = np.zeros(spec.cols, np.uint16)
        x[col] = 0x3F80
        (y,), st = run_gemv([c], [x], [spec.rows])
        assert st == 0
        assert int(y[r:r + 1].view(np.uint32)[0]) == int(val) << 16
        assert w[r, col] == val


def test_single_symbol_tensors():
    # every weight the same code: the constant path
    spec = synth.TensorSpec("c", 20, 3000, synth.DTYPE_INT8, 0.0)
    t = synth.Tensor(spec, np.full(spec.n, 0xFE, np.uint8), np.linspace(0.001, 1.0, 20).astype(np.float32))
    c = eq.DeviceContainer(encode(t, 192000, 8), device="cuda")  # lcm(512, 3000)
    w = expected_bf16(t).reshape(20, 3000)
    x = _x_bits(3000, 5)
    (y,), st = run_gemv([c], [x], [20])
    assert st == 0
    check_close(y, w, x, "single symbol")
    one_hot_exact(c, w, [0, 1234, 2999], "single symbol")
    # every position an escape (the escape code is then the only symbol)
    spec2 = synth.TensorSpec("e", 4, 64, synth.DTYPE_INT8, 0.0)
    idx = np.arange(spec2.n, dtype=np.uint64)
    vals = oracle.bf16_rne(np.linspace(-3, 3, spec2.n).astype(np.float32))
    t2 = synth.Tensor(spec2, np.full(spec2.n, 0x80, np.uint8), np.ones(4, np.float32), idx, vals)
    c2 = eq.DeviceContainer(encode(t2, 512, 8), device="cuda")
    w2 = expected_bf16(t2).reshape(4, 64)
    x2 = _x_bits(64, 6)
    (y2,), st = run_gemv([c2], [x2], [4])
    assert st == 0
    check_close(y2, w2, x2, "all escapes")


def test_block_of_mixed_tensors_and_lane_runs():
    """Several tensors with different K and shapes in one call: the library
    groups them into launches; each y goes to its own tensor."""
    cases = [(64, 1024, 65536, 8, synth.DTYPE_INT8), (48, 2048, 16384, 4, synth.DTYPE_E4M3),
             (33, 1000, 64000, 8, synth.DTYPE_INT8), (20, 4096, 65536, 16, synth.DTYPE_INT8),
             (70, 512, 8192, 8, synth.DTYPE_E4M3)]
    conts, ws, xs, rows = [], [], [], []
    for i, (r, cl, Z, K, dt) in enumerate(cases):
        spec = synth.TensorSpec(f"t{i}", r, cl, dt, 2.2, 2)
        t = synth.make_tensor(4, 70 + i, 6, spec=spec)
        conts.append(eq.DeviceContainer(encode(t, Z, K), device="cuda"))
        ws.append(expected_bf16(t).reshape(r, cl))
        xs.append(_x_bits(cl, 100 + i))
        rows.append(r)
    ys, st = run_gemv(conts, xs, rows)
    assert st == 0
    for i, (y, w, x) in enumerate(zip(ys, ws, xs)):
        check_close(y, w, x, f"tensor {i}")


def test_unsupported_layouts_and_bad_arguments():
    spec = synth.TensorSpec("t", 8, 1000, synth.DTYPE_INT8, 2.1)
    t = synth.make_tensor(4, 80, 0, spec=spec)
    # chunks of 8192 symbols do not hold whole 1000-column rows
    c = eq.DeviceContainer(encode(t, 8192, 8), device="cuda")
    with pytest.raises(eq.EqError) as ei:
        run_gemv([c], [_x_bits(1000, 1)], [8])
    assert ei.value.status == -5
    # a lane run of 16 does not divide 1000 columns (Z = 128000 = lcm(1024, 1000))
    c16 = eq.DeviceContainer(encode(t, 128000, 16), device="cuda")
    with pytest.raises(eq.EqError) as ei:
        run_gemv([c16], [_x_bits(1000, 1)], [8])
    assert ei.value.status == -5
    # x not 16-byte aligned
    c_ok = eq.DeviceContainer(encode(t, 64000, 8), device="cuda")
    xbuf = _dev_x(np.zeros(1008, np.uint16))
    y = torch.zeros(8, dtype=torch.float32, device="cuda")
    blk = eq.Block([c_ok])
    with pytest.raises(eq.EqError) as ei:
        eq.eq_decode_gemv_bf16(blk, [xbuf[1:1001]], [y])
    assert ei.value.status == -1
    # empty block: nothing enqueued
    eq.eq_decode_gemv_bf16(eq.Block([]), [], [])
    torch.cuda.synchronize()


def test_70b_block_fused_sampled_rows():
    """The 70B-shaped block with whole-row chunks (down_proj: two 28,672-column
    rows per chunk), one call over all seven tensors, in the launch
    configuration the benchmark times; rows sampled in every tensor."""
    specs = synth.config_specs(4)
    conts, xs = [], []
    log("case 70B fused block: encoding")
    for i, sp in enumerate(specs):
        t = synth.make_tensor(4, 0, i)
        Z = 65536 if 65536 % sp.cols == 0 else 2 * sp.cols
        conts.append(eq.DeviceContainer(encode(t, Z, 8), device="cuda"))
        xs.append(oracle.bf16_rne(synth.gemv_activation(4, 0, i, sp.cols)))
        del t
    log("case 70B fused block: decode + GEMV")
    ys, st = run_gemv(conts, xs, [sp.rows for sp in specs])
    assert st == 0
    rng = np.random.default_rng(7)
    for i, sp in enumerate(specs):
        rows = np.unique(np.concatenate([[0, sp.rows - 1], rng.integers(0, sp.rows, 6)]))
        t_rows = []
        for r in rows.tolist():
            sym = synth.symbols_slice(4, 0, i, r * sp.cols, sp.cols)
            sc = synth.scales_for(4, 0, i, sp.rows)[r:r + 1]
            ei, ev = (synth.escapes_for(4, 0, i, sp) if sp.n_esc else
                      (np.zeros(0, np.uint64), np.zeros(0, np.uint16)))
            keep = (ei >= r * sp.cols) & (ei < (r + 1) * sp.cols)
            w = oracle.dequant_direct(sp.dtype, sym, sp.cols, sc, ei[keep] - r * sp.cols, ev[keep])
            t_rows.append(w)
        check_close(ys[i][rows], np.stack(t_rows), xs[i], f"70B {sp.name}")
