"""The whole 70B-shaped model stream under the GPU tests: 80 blocks (layers
0..79, each with its own seeded int8 codes, scales and four super weights in
down), resident as containers, decoded block by block into two alternating
bf16 buffers on one stream while the other stream runs each block's seven
batch-1 GEMVs (eq_pipeline_run; "Float8@2bits: Entropy Coding Enables
Data-Free Model Compression", section 2, technical component 3).

Checked against the oracle:
  - every block's decode into a bf16 buffer: whole chunks of every tensor
    (first, last, one at random and each one holding a super weight) equal
    oracle.dequant_direct on the symbols regenerated on the host, bit for bit;
  - every block's GEMV outputs from the schedule: sampled rows of every
    tensor (first, last, random, each super weight's row) lie within
    cols * 2^-23 * sum_c |W[r, c] x[c]| of oracle.gemv_f64 over the oracle's
    bf16 row (fp32 accumulation in another order than the oracle's);
  - a second token enqueued right behind the first, without a synchronise,
    gives the same outputs bit for bit.
The codes are drawn on the GPU by the seeded sampler (the host sampler's
values, checked on sampled ranges) and encoded by eq_encode_device, whose
containers for one layer are compared byte for byte with the oracle's."""
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

CFG = 5


class _Resident:
    """A device container built on the device (header parsed on the host)."""

    def __init__(self, dev, hdr):
        self.dev, self.hdr = dev, hdr


def _build(layers):
    specs = synth.config_specs(CFG)
    Z = synth.config_chunk(CFG)
    nmax = max(sp.n for sp in specs)
    d_sym = torch.empty(nmax, dtype=torch.uint8, device="cuda")
    wsb = max(int(eq._lib.eq_encode_device_workspace(sp.rows, sp.cols, Z)) for sp in specs)
    cap = max(int(eq._lib.eq_encode_device_bound(sp.rows, sp.cols, Z, sp.n_esc)) for sp in specs)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    d_len = torch.zeros(1, dtype=torch.int64, device="cuda")
    d_st = torch.zeros(1, dtype=torch.int32, device="cuda")
    blocks, meta = [], []
    for layer in range(layers):
        conts, tens = [], []
        for i, sp in enumerate(specs):
            sym = d_sym[:sp.n]
            t = synth.make_tensor_gpu(CFG, layer, i, sym, spec=sp)
            esc = t.esc_idx.size > 0
            eq.eq_encode_device(sp.dtype, sp.rows, sp.cols, sym, torch.from_numpy(t.scales).cuda(),
                                torch.from_numpy(t.esc_idx.astype(np.int64)).cuda() if esc else None,
                                torch.from_numpy(t.esc_val.view(np.int16)).cuda() if esc else None,
                                t.esc_code if esc else 0, Z, synth.LANE_RUN, workspace=ws, out=out,
                                d_len=d_len, d_status=d_st)
            n = int(d_len.item())
            assert int(d_st.item()) == 0, f"layer {layer} {sp.name}: encoder flagged its input"
            dev = out[:n].clone()
            host = dev.cpu().numpy()
            if layer == 0 and i in (1, 6):
                # the GPU draw is the host draw, and the container is the oracle's
                hs = synth.make_tensor(CFG, 0, i, spec=sp)
                assert torch.equal(sym.cpu(), torch.from_numpy(hs.symbols)), f"GPU sampler {sp.name}"
                ref = oracle.encode(sp.dtype, sp.rows, sp.cols, hs.symbols, hs.scales,
                                    oracle.build_freq(hs.symbols), Z, synth.LANE_RUN, esc_enabled=esc,
                                    esc_code=hs.esc_code if esc else 0, esc_idx=hs.esc_idx if esc else None,
                                    esc_val=hs.esc_val if esc else None)
                assert ref.size == host.size and np.array_equal(ref, host), f"container {sp.name}"
                del hs, ref
            conts.append(_Resident(dev, eq.parse_header(host)))
            tens.append(t)
            del host
        blocks.append(eq.Block(conts, synth.block_offsets(specs)[:-1]))
        meta.append(tens)
        if layer % 10 == 9:
            log(f"model80: {layer + 1} blocks built")
    return specs, blocks, meta


def _row_symbols(layer, i, sp, r):
    return synth.symbols_slice(CFG, layer, i, r * sp.cols, sp.cols, spec=sp)


def _esc_in(t, lo, hi):
    m = (t.esc_idx >= lo) & (t.esc_idx < hi)
    return (t.esc_idx[m] - lo).astype(np.uint64), t.esc_val[m]


def test_model80_pipeline_against_the_oracle():
    L = synth.N_LAYERS_MODEL
    log("model80: building 80 blocks on the device")
    specs, blocks, meta = _build(L)
    offs = synth.block_offsets(specs)
    nblk = offs[-1]
    Z = synth.config_chunk(CFG)
    rng = np.random.default_rng(80)

    # decode of every block, sampled whole chunks against the oracle
    buf = torch.empty(nblk, dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for layer in range(L):
        blocks[layer].c.d_status = status.data_ptr()
        eq.eq_decode_dequant_bf16(blocks[layer], buf)
        blocks[layer].c.d_status = None
        for i, (sp, o) in enumerate(zip(specs, offs)):
            t = meta[layer][i]
            nch = -(-sp.n // Z)
            ks = {0, nch - 1, int(rng.integers(0, nch))} | {int(e) // Z for e in t.esc_idx}
            for k in sorted(ks):
                lo, hi = k * Z, min(sp.n, (k + 1) * Z)
                sym = synth.symbols_slice(CFG, layer, i, lo, hi - lo, spec=sp)
                r0 = lo // sp.cols
                rows = np.arange(lo, hi) // sp.cols
                ei, ev = _esc_in(t, lo, hi)
                exp = oracle.dequant_direct(sp.dtype, sym, 1, t.scales[rows], ei, ev)
                got = to_u16(buf[o + lo:o + hi])
                bad = np.flatnonzero(got != exp)
                assert bad.size == 0, (f"layer {layer} {sp.name} chunk {k} (row {r0}): {bad.size} "
                                       f"mismatches, first at {lo + int(bad[0])}")
        torch.cuda.synchronize()
        assert int(status.item()) == 0, f"layer {layer}: device status {int(status.item())}"
    del buf
    log("model80: every block's sampled chunks bit-exact")

    # one token through the double-buffered schedule, and a second right behind it
    xs_f = [[synth.gemv_activation(CFG, layer, i, sp.cols) for i, sp in enumerate(specs)] for layer in range(L)]
    xs = [[torch.from_numpy(x).to(torch.bfloat16).cuda() for x in row] for row in xs_f]
    ys = [[torch.full((sp.rows,), float("nan"), dtype=torch.float32, device="cuda") for sp in specs]
          for _ in range(L)]
    ys2 = [[torch.full_like(y, float("nan")) for y in row] for row in ys]
    bufs = [torch.empty(nblk, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ds, gs = torch.cuda.Stream(), torch.cuda.Stream()
    pipe = eq.Pipeline(L)
    pipe.run(blocks, bufs[0], bufs[1], xs, ys, ds, gs)
    pipe.run(blocks, bufs[0], bufs[1], xs, ys2, ds, gs)   # same plan, no synchronise in between
    torch.cuda.synchronize()
    log("model80: two tokens done")
    for layer in range(L):
        for i, sp in enumerate(specs):
            assert torch.equal(ys[layer][i].view(torch.int32), ys2[layer][i].view(torch.int32)), \
                f"second token differs: layer {layer} {sp.name}"
            t = meta[layer][i]
            rows = {0, sp.rows - 1, int(rng.integers(0, sp.rows))} | {int(e) // sp.cols for e in t.esc_idx}
            y = ys[layer][i].cpu().numpy()
            x_bits = oracle.bf16_rne(xs_f[layer][i])
            for r in sorted(rows):
                ei, ev = _esc_in(t, r * sp.cols, (r + 1) * sp.cols)
                w = oracle.dequant_direct(sp.dtype, _row_symbols(layer, i, sp, r), sp.cols,
                                          t.scales[r:r + 1], ei, ev)
                y64, absdot = oracle.gemv_f64(w.reshape(1, -1), x_bits)
                tol = sp.cols * 2.0 ** -23 * absdot[0]
                assert np.isfinite(y[r]) and abs(float(y[r]) - y64[0]) <= tol, \
                    f"layer {layer} {sp.name} row {r}: {y[r]!r} vs {y64[0]!r} (tol {tol!r})"
    pipe.close()
    log("model80: sampled GEMV rows of every block within the fp32 bound")
