"""Helpers for the GPU tests: encode with the library's host encoder, place
containers in device memory, decode through the C ABI, compare with the
oracle."""
import numpy as np
import torch

import oracle
import synth
from rans_decode_amd import eq


def log(msg):
    print(msg, flush=True)


def encode(t: synth.Tensor, chunk_symbols=65536, lane_run=8, tables=None, codec=0):
    sp = t.spec
    tab = tables if tables is not None else eq.build_tables(t.symbols)
    esc = t.esc_idx.size > 0
    return eq.encode_host(tab, sp.dtype, sp.rows, sp.cols, t.symbols, t.scales,
                          t.esc_idx if esc else None, t.esc_val if esc else None,
                          esc_code=t.esc_code if esc else 0, chunk_symbols=chunk_symbols,
                          lane_run=lane_run, codec=codec)


class Packed:
    """Many containers in one device allocation (each at a 256-byte offset)."""

    def __init__(self, blobs, device="cuda"):
        offs, o = [], 0
        for b in blobs:
            offs.append(o)
            o += (b.size + 255) // 256 * 256
        host = np.zeros(max(o, 256), np.uint8)
        for b, off in zip(blobs, offs):
            host[off:off + b.size] = b
        self.dev = torch.from_numpy(host).to(device)
        self.items = []
        for b, off in zip(blobs, offs):
            c = eq.DeviceContainer.__new__(eq.DeviceContainer)
            c.host = b
            c.hdr = eq.parse_header(b)
            c.dev = self.dev[off:off + b.size]
            self.items.append(c)


def expected_bf16(t: synth.Tensor) -> np.ndarray:
    sp = t.spec
    return oracle.dequant_direct(sp.dtype, t.symbols, sp.cols, t.scales, t.esc_idx, t.esc_val)


def to_u16(x: torch.Tensor) -> np.ndarray:
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


def run_bf16(containers, n_out, offsets=None, fill=0x7FBF, device="cuda"):
    out = torch.full((n_out,), fill, dtype=torch.int16, device=device)
    status = torch.zeros(1, dtype=torch.int32, device=device)
    eq.decode_dequant_bf16(containers, out, offsets=offsets, status=status)
    torch.cuda.synchronize()
    return to_u16(out), int(status.item())


def run_u8(containers, n_out, offsets=None, fill=0xA5, device="cuda"):
    out = torch.full((n_out,), fill, dtype=torch.uint8, device=device)
    status = torch.zeros(1, dtype=torch.int32, device=device)
    eq.decode_block(containers, out, offsets=offsets, status=status)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(status.item())


def assert_same(got: np.ndarray, exp: np.ndarray, what: str):
    if got.shape != exp.shape:
        raise AssertionError(f"{what}: shape {got.shape} vs {exp.shape}")
    bad = np.flatnonzero(got != exp)
    if bad.size:
        i = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} mismatches, first at {i}: "
                             f"got {int(got[i]):#x} expected {int(exp[i]):#x}")
