"""The encoder entry point that allocates nothing (eq_encode_device_static,
a static per-GPU scratch array instead of a workspace argument) against the
workspace entry point (eq_encode_device), byte for byte, on two calls in a
row, the second with a smaller input; and the clear error for a tensor whose
scratch need exceeds the array."""
import numpy as np
import pytest
import torch

import synth
from conftest import gpu_available
from gpu_util import log
from rans_decode_amd import eq

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _inputs(cfg, layer, t, spec):
    tt = synth.make_tensor(cfg, layer, t, spec=spec)
    esc = tt.esc_idx.size > 0
    return dict(sym=torch.from_numpy(tt.symbols).cuda(), sc=torch.from_numpy(tt.scales).cuda(),
                ei=torch.from_numpy(tt.esc_idx.astype(np.int64)).cuda() if esc else None,
                ev=torch.from_numpy(tt.esc_val.view(np.int16)).cuda() if esc else None,
                code=tt.esc_code if esc else 0, spec=spec)


def _reference(x, Z, codec):
    sp = x["spec"]
    out, d_len, st = eq.eq_encode_device(sp.dtype, sp.rows, sp.cols, x["sym"], x["sc"], x["ei"], x["ev"],
                                         x["code"], Z, 8, codec=codec)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return out[:int(d_len.item())].cpu().numpy()


def test_static_scratch_encoder_matches_the_workspace_entry_point():
    cases = [  # the larger first, then a smaller one: the array keeps the first call's contents
        (synth.TensorSpec("q", 8192, 8192, synth.DTYPE_INT8, 2.1, 0), 4, 0, 65536, eq.EQ_CODEC_RANS),
        (synth.TensorSpec("down", 512, 4096, synth.DTYPE_INT8, 2.1, 4), 4, 6, 16384, eq.EQ_CODEC_HUFFMAN),
    ]
    for sp, cfg, t, Z, codec in cases:
        assert eq._lib.eq_encode_device_workspace(sp.rows, sp.cols, Z) <= eq.EQ_ENCODE_STATIC_SCRATCH_BYTES
    cap = max(int(eq._lib.eq_encode_device_bound(sp.rows, sp.cols, Z, sp.n_esc)) for sp, _, _, Z, _ in cases)
    out = torch.empty(cap, dtype=torch.uint8, device="cuda")
    d_len = torch.zeros(1, dtype=torch.int64, device="cuda")
    d_st = torch.zeros(1, dtype=torch.int32, device="cuda")
    for sp, cfg, t, Z, codec in cases:
        log(f"case static-scratch encoder {sp.rows}x{sp.cols} codec {codec}")
        x = _inputs(cfg, 3, t, sp)
        out.fill_(0xCD)
        eq.eq_encode_device_static(sp.dtype, sp.rows, sp.cols, x["sym"], x["sc"], out, d_len, d_st,
                                   x["ei"], x["ev"], x["code"], Z, 8, codec=codec)
        torch.cuda.synchronize()
        assert int(d_st.item()) == 0
        got = out[:int(d_len.item())].cpu().numpy()
        exp = _reference(x, Z, codec)
        assert got.size == exp.size and np.array_equal(got, exp), f"{sp.rows}x{sp.cols}"
        del x


def test_static_scratch_encoder_rejects_oversized_tensors():
    sp = synth.TensorSpec("gate", 28672, 8192, synth.DTYPE_INT8, 2.1, 0)
    assert eq._lib.eq_encode_device_workspace(sp.rows, sp.cols, 32768) > eq.EQ_ENCODE_STATIC_SCRATCH_BYTES
    sym = torch.zeros(16, dtype=torch.uint8, device="cuda")   # never read: the size check comes first
    sc = torch.ones(16, dtype=torch.float32, device="cuda")
    out = torch.empty(256, dtype=torch.uint8, device="cuda")
    d_len = torch.zeros(1, dtype=torch.int64, device="cuda")
    d_st = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(eq.EqError) as ei:
        eq.eq_encode_device_static(sp.dtype, sp.rows, sp.cols, sym, sc, out, d_len, d_st, chunk_symbols=32768)
    assert ei.value.status == eq.EQ_ERANGE
