"""Python face of the plain CPU oracle (``eq_oracle.c``).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The product library
(``rans_decode_amd``) never imports it, and it never imports the product.

Every function is a thin ctypes call into ``liboracle.so``; the arithmetic
lives in the C file, each function there citing the passage it follows.
"""
from __future__ import annotations

import ctypes
import os
from functools import lru_cache

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_INT8 = 1
DTYPE_E4M3 = 2
BAD_END_STATE = 1
WORD_OVERRUN = 2

_P = ctypes.c_void_p
_U64 = ctypes.c_uint64
_U32 = ctypes.c_uint32


@lru_cache(maxsize=1)
def lib():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "or_bf16_rne": (ctypes.c_uint16, [ctypes.c_float]),
        "or_bf16_rne_array": (None, [_P, _U64, _P]),
        "or_e4m3_value": (ctypes.c_float, [ctypes.c_uint8]),
        "or_symbol_value": (ctypes.c_float, [_U32, ctypes.c_uint8]),
        "or_dequant_direct": (None, [_U32, _P, _U64, _U64, _P, _P, _P, _U64, _P]),
        "or_quantize_counts": (ctypes.c_int, [_P, _P]),
        "or_build_freq": (ctypes.c_int, [_P, _U64, _P]),
        "or_encode_step": (ctypes.c_int, [ctypes.POINTER(_U32), _U32, _U32,
                                          ctypes.POINTER(ctypes.c_uint16)]),
        "or_decode_step": (ctypes.c_int, [ctypes.POINTER(_U32), _U32, _U32]),
        "or_single_lane_bytes": (_U64, [_P, _U64, _P]),
        "or_encode": (ctypes.c_int, [_U32, _U64, _U64, _P, _P, _P, _U32, _U32, _U32,
                                     ctypes.c_uint8, _P, _P, _U64,
                                     ctypes.POINTER(_P), ctypes.POINTER(_U64)]),
        "or_encode_codec": (ctypes.c_int, [_U32, _U32, _U64, _U64, _P, _P, _P, _U32, _U32, _U32,
                                           ctypes.c_uint8, _P, _P, _U64,
                                           ctypes.POINTER(_P), ctypes.POINTER(_U64)]),
        "or_encode_seg": (ctypes.c_int, [_U32, _U32, _U64, _U64, _P, _P, _P, _U32, _U32, _U32, _U32,
                                         ctypes.c_uint8, _P, _P, _U64,
                                         ctypes.POINTER(_P), ctypes.POINTER(_U64)]),
        "or_huff_lengths": (ctypes.c_int, [_P, _U32, _P]),
        "or_huff_codes": (ctypes.c_int, [_P, _P]),
        "or_free": (None, [_P]),
        "or_decode_chunks": (ctypes.c_int64, [_P, _U64, _U64, _U64, _U32, _P, _P]),
        "or_decode_symbols": (ctypes.c_int64, [_P, _U64, _P]),
        "or_decode_dequant": (ctypes.c_int64, [_P, _U64, _P]),
        "or_header_fields": (ctypes.c_int, [_P, _U64, _P]),
        "or_gemv_f64": (None, [_P, _U64, _U64, _P, _P, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


class OracleError(RuntimeError):
    pass


def bf16_rne(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().or_bf16_rne_array(x.ctypes.data, x.size, out.ctypes.data)
    return out


def e4m3_values() -> np.ndarray:
    return np.array([lib().or_e4m3_value(c) for c in range(256)], dtype=np.float32)


def symbol_value(dtype: int, code: int) -> float:
    return lib().or_symbol_value(dtype, code)


def dequant_direct(dtype: int, symbols: np.ndarray, cols: int, scales: np.ndarray,
                   esc_idx: np.ndarray | None = None, esc_val: np.ndarray | None = None) -> np.ndarray:
    """Exact bf16 result computed straight from the original symbols."""
    symbols = np.ascontiguousarray(symbols, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    esc_idx = np.ascontiguousarray(esc_idx if esc_idx is not None else [], dtype=np.uint64)
    esc_val = np.ascontiguousarray(esc_val if esc_val is not None else [], dtype=np.uint16)
    out = np.empty(symbols.size, dtype=np.uint16)
    lib().or_dequant_direct(dtype, symbols.ctypes.data, symbols.size, cols, scales.ctypes.data,
                            esc_idx.ctypes.data, esc_val.ctypes.data, esc_idx.size, out.ctypes.data)
    return out


def quantize_counts(counts) -> np.ndarray:
    c = np.ascontiguousarray(counts, dtype=np.uint64)
    assert c.size == 256
    f = np.zeros(256, dtype=np.uint16)
    rc = lib().or_quantize_counts(c.ctypes.data, f.ctypes.data)
    if rc:
        raise OracleError(f"or_quantize_counts: {rc}")
    return f


def build_freq(symbols: np.ndarray) -> np.ndarray:
    symbols = np.ascontiguousarray(symbols, dtype=np.uint8)
    f = np.zeros(256, dtype=np.uint16)
    rc = lib().or_build_freq(symbols.ctypes.data, symbols.size, f.ctypes.data)
    if rc:
        raise OracleError(f"or_build_freq: {rc}")
    return f


def encode_step(x: int, f: int, c: int) -> tuple[int, int | None]:
    xs = _U32(x)
    w = ctypes.c_uint16(0)
    emitted = lib().or_encode_step(ctypes.byref(xs), f, c, ctypes.byref(w))
    return xs.value, (w.value if emitted else None)


def decode_step(x: int, f: int, c: int) -> tuple[int, bool]:
    xs = _U32(x)
    need = lib().or_decode_step(ctypes.byref(xs), f, c)
    return xs.value, bool(need)


def single_lane_bytes(symbols: np.ndarray, freq: np.ndarray) -> int:
    symbols = np.ascontiguousarray(symbols, dtype=np.uint8)
    freq = np.ascontiguousarray(freq, dtype=np.uint16)
    return int(lib().or_single_lane_bytes(symbols.ctypes.data, symbols.size, freq.ctypes.data))


CODEC_RANS = 0
CODEC_HUFF = 1
HUFF_ZERO = 0x100   # table value of a lone symbol coded in zero bits


def huff_lengths(counts, max_len: int = 12) -> np.ndarray:
    """Optimal code lengths of at most max_len bits (package-merge); u16 table
    in the container's form (0 absent, HUFF_ZERO for a lone symbol)."""
    c = np.ascontiguousarray(counts, dtype=np.uint64)
    ln = np.zeros(256, np.uint8)
    rc = lib().or_huff_lengths(_ptr(c), max_len, _ptr(ln))
    if rc:
        raise OracleError(f"or_huff_lengths: {rc}")
    t = ln.astype(np.uint16)
    if np.count_nonzero(c) == 1:
        t[np.flatnonzero(c)[0]] = HUFF_ZERO
    return t


def huff_codes(table) -> np.ndarray:
    """Canonical codeword of every symbol of a length table (0 if absent)."""
    t = np.ascontiguousarray(table, dtype=np.uint16)
    code = np.zeros(256, np.uint32)
    if not lib().or_huff_codes(_ptr(t), _ptr(code)):
        raise OracleError("or_huff_codes: not a complete prefix code")
    return code


def encode(dtype: int, rows: int, cols: int, symbols: np.ndarray, scales: np.ndarray,
           freq: np.ndarray, chunk_symbols: int = 65536, lane_run: int = 8,
           esc_enabled: bool = False, esc_code: int = 0, esc_idx=None, esc_val=None,
           codec: int = CODEC_RANS, seg_chunks: int = 0) -> np.ndarray:
    """Container v1 bytes (np.uint8). freq is the rANS frequency table, or for
    codec=CODEC_HUFF the code-length table; with seg_chunks > 0 (adaptive
    tables) freq is [n_segments, 256], one table per seg_chunks chunks."""
    symbols = np.ascontiguousarray(symbols, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    freq = np.ascontiguousarray(freq, dtype=np.uint16).reshape(-1)
    esc_idx = np.ascontiguousarray(esc_idx if esc_idx is not None else [], dtype=np.uint64)
    esc_val = np.ascontiguousarray(esc_val if esc_val is not None else [], dtype=np.uint16)
    assert symbols.size == rows * cols and scales.size == rows and esc_idx.size == esc_val.size
    out = _P()
    n = _U64()
    rc = lib().or_encode_seg(codec, dtype, rows, cols, symbols.ctypes.data, scales.ctypes.data,
                             freq.ctypes.data, seg_chunks, chunk_symbols, lane_run, int(esc_enabled),
                             esc_code, esc_idx.ctypes.data, esc_val.ctypes.data, esc_idx.size,
                             ctypes.byref(out), ctypes.byref(n))
    if rc:
        raise OracleError(f"or_encode: {rc}")
    try:
        buf = np.ctypeslib.as_array(ctypes.cast(out, ctypes.POINTER(ctypes.c_uint8)), (n.value,)).copy()
    finally:
        lib().or_free(out)
    return buf


def header(container: np.ndarray) -> dict:
    v = np.zeros(21, dtype=np.uint64)
    rc = lib().or_header_fields(container.ctypes.data, container.size, v.ctypes.data)
    if rc:
        raise OracleError(f"or_header_fields: {rc}")
    keys = ("dtype", "flags", "rows", "cols", "n", "chunk_symbols", "lane_run", "n_chunks",
            "n_esc", "esc_code", "n_words", "off_freq", "off_scales", "off_dir", "off_states",
            "off_words", "off_esc_idx", "off_esc_val", "total", "codec", "seg_chunks")
    return {k: int(x) for k, x in zip(keys, v)}


def decode_symbols(container: np.ndarray) -> tuple[np.ndarray, int]:
    h = header(container)
    out = np.zeros(h["n"], dtype=np.uint8)
    flags = lib().or_decode_symbols(container.ctypes.data, container.size, out.ctypes.data)
    if flags < 0:
        raise OracleError(f"or_decode_symbols: {flags}")
    return out, int(flags)


def decode_dequant(container: np.ndarray) -> tuple[np.ndarray, int]:
    h = header(container)
    out = np.zeros(h["n"], dtype=np.uint16)
    flags = lib().or_decode_dequant(container.ctypes.data, container.size, out.ctypes.data)
    if flags < 0:
        raise OracleError(f"or_decode_dequant: {flags}")
    return out, int(flags)


def decode_chunks(container: np.ndarray, k_lo: int, k_hi: int, threads: int,
                  bf16_out: np.ndarray | None = None, sym_out: np.ndarray | None = None) -> int:
    """Decode chunks [k_lo, k_hi) into full-size flat outputs with `threads`
    threads (chunk-parallel); returns the ORed decode flags."""
    flags = lib().or_decode_chunks(container.ctypes.data, container.size, k_lo, k_hi, threads,
                                   _ptr(sym_out), _ptr(bf16_out))
    if flags < 0:
        raise OracleError(f"or_decode_chunks: {flags}")
    return int(flags)


def gemv_f64(w_bits: np.ndarray, x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """y = W @ x in binary64 for bf16 bit patterns W [rows, cols] and x [cols];
    also sum_c |W[r, c] x[c]| per row."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, cols = w.shape
    if x.shape != (cols,):
        raise ValueError("x must have one entry per column")
    y = np.empty(rows, np.float64)
    a = np.empty(rows, np.float64)
    lib().or_gemv_f64(_ptr(w), rows, cols, _ptr(x), _ptr(y), _ptr(a))
    return y, a
