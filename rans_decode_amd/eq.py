"""Python binding of libeq.so (include/eq.h): argument marshalling only.

Every step of the decode runs in the library's HIP kernels; PyTorch provides
device memory and streams. There is no CPU fallback: if libeq.so is missing
or cannot be loaded, importing this module raises.

The functions keep the C names (``eq_build_tables``, ``eq_tables_from_freq``, ``eq_encode_host``,
``eq_parse_header``, ``eq_decode_block``, ``eq_decode_dequant_bf16``,
``eq_decode_gemv_bf16``, ``eq_gemv_bf16``, ``eq_pipeline_*``, ``eq_bf16_from_f32``) as thin wrappers
over numpy / torch arrays, plus a few conveniences (``build_tables``,
``encode_host``, ``DeviceContainer``, ``decode_dequant_bf16``, ...).
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# EQ_LIBRARY may name another build of the same library (e.g. a tuning build
# with different compile-time parameters); the default is the in-tree build.
LIB_PATH = os.environ.get("EQ_LIBRARY") or os.path.join(_HERE, "libeq.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "eq.h")

EQ_OK, EQ_EINVAL, EQ_ERANGE, EQ_ECORRUPT, EQ_EHIP, EQ_EUNSUPPORTED, EQ_ENOMEM = 0, -1, -2, -3, -4, -5, -6
EQ_DEV_BAD_END_STATE, EQ_DEV_WORD_OVERRUN = 1, 2
EQ_DTYPE_INT8, EQ_DTYPE_E4M3 = 1, 2
EQ_MAX_BLOCK_TENSORS = 16
EQ_CODEC_RANS = 0
EQ_CODEC_HUFFMAN = 1
EQ_PIPELINE_ALTERNATE, EQ_PIPELINE_OVERLAP = 0, 1

_u32, _u64, _i32, _vp = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p


class eq_tables(ctypes.Structure):
    _fields_ = [("counts", _u64 * 256), ("n", _u64), ("freq", ctypes.c_uint16 * 256),
                ("cum", _u32 * 257)]


class eq_tensor_desc(ctypes.Structure):
    _fields_ = [("dtype", _u32), ("lane_run", _u32), ("rows", _u64), ("cols", _u64),
                ("chunk_symbols", _u32), ("esc_enabled", _u32), ("esc_code", _u32),
                ("codec", _u32), ("seg_chunks", _u32), ("reserved", _u32)]


class eq_header(ctypes.Structure):
    _fields_ = [("dtype", _u32), ("flags", _u32), ("chunk_symbols", _u32), ("lane_run", _u32),
                ("rows", _u64), ("cols", _u64), ("n", _u64), ("n_chunks", _u64), ("n_esc", _u64),
                ("n_words", _u64), ("esc_code", _u32), ("single_symbol", _i32),
                ("codec", _u32), ("seg_chunks", _u32), ("off_freq", _u64), ("off_scales", _u64), ("off_dir", _u64), ("off_states", _u64),
                ("off_words", _u64), ("off_esc_idx", _u64), ("off_esc_val", _u64),
                ("total_bytes", _u64)]


class eq_tensor_ref(ctypes.Structure):
    _fields_ = [("d_container", _vp), ("hdr", eq_header), ("out_offset", _u64)]


class eq_block(ctypes.Structure):
    _fields_ = [("n_tensors", _u32), ("reserved", _u32), ("tensors", ctypes.POINTER(eq_tensor_ref)),
                ("d_status", _vp)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sig = {
        "eq_build_tables": [_vp, _u64, P(eq_tables)],
        "eq_tables_from_freq": [_vp, P(eq_tables)],
        "eq_encode_host": [P(eq_tables), P(eq_tensor_desc), _vp, _vp, _vp, _vp, _u64, _vp, _u64, P(_u64)],
        "eq_parse_header": [_vp, _u64, P(eq_header)],
        "eq_decode_block": [P(eq_block), _vp, _vp],
        "eq_decode_dequant_bf16": [P(eq_block), _vp, _vp],
        "eq_decode_gemv_bf16": [P(eq_block), _vp, _vp, _vp],
        "eq_gemv_bf16": [_vp, _u64, _u64, _vp, _vp, _vp],
        "eq_pipeline_create": [_u32, P(_vp)],
        "eq_pipeline_set_mode": [_vp, _u32],
        "eq_pipeline_run": [_vp, P(eq_block), _u32, _vp, _vp, _vp, _vp, _vp, _vp],
        "eq_pipeline_destroy": [_vp],
        "eq_bf16_from_f32": [_vp, _u64, _vp, _vp],
        "eq_encode_device": [P(eq_tensor_desc), _vp, _vp, _vp, _vp, _u64, _vp, _u64, _vp, _u64, _vp, _vp, _vp],
        "eq_encode_device_static": [P(eq_tensor_desc), _vp, _vp, _vp, _vp, _u64, _vp, _u64, _vp, _vp, _vp],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.restype = ctypes.c_int32
        fn.argtypes = args
    for name in ("eq_encode_device_bound", "eq_encode_device_workspace"):
        fn = getattr(L, name)
        fn.restype = _u64
    L.eq_encode_device_bound.argtypes = [_u64, _u64, _u32, _u64]
    L.eq_encode_device_workspace.argtypes = [_u64, _u64, _u32]
    L.eq_status_string.restype = ctypes.c_char_p
    L.eq_status_string.argtypes = [ctypes.c_int32]
    return L


_lib = _load()


def declared_functions() -> list[str]:
    """Names of the functions include/eq.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(eq_[a-z0-9_]+)\s*\(", text)))


class EqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {_lib.eq_status_string(status).decode()} ({status})")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != EQ_OK:
        raise EqError(fn, status)


def status_string(status: int) -> str:
    return _lib.eq_status_string(status).decode()


# ---------------------------------------------------------------------------
# Host side
# ---------------------------------------------------------------------------
def eq_build_tables(symbols: np.ndarray) -> eq_tables:
    symbols = np.ascontiguousarray(symbols, dtype=np.uint8)
    t = eq_tables()
    _check("eq_build_tables", _lib.eq_build_tables(symbols.ctypes.data, symbols.size, ctypes.byref(t)))
    return t


build_tables = eq_build_tables


def eq_tables_from_freq(freq) -> eq_tables:
    """A custom table (any valid 12-bit frequencies) in eq_tables form; the
    library derives the cumulative frequencies."""
    f = np.ascontiguousarray(freq, dtype=np.uint16)
    if f.size != 256:
        raise ValueError("a frequency table has 256 entries")
    t = eq_tables()
    _check("eq_tables_from_freq", _lib.eq_tables_from_freq(f.ctypes.data, ctypes.byref(t)))
    return t


tables_from_freq = eq_tables_from_freq


def eq_encode_host(tables: eq_tables, desc: eq_tensor_desc, symbols: np.ndarray, scales: np.ndarray,
                   esc_idx: np.ndarray | None = None, esc_val: np.ndarray | None = None) -> np.ndarray:
    symbols = np.ascontiguousarray(symbols, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    esc_idx = np.ascontiguousarray(esc_idx if esc_idx is not None else [], dtype=np.uint64)
    esc_val = np.ascontiguousarray(esc_val if esc_val is not None else [], dtype=np.uint16)
    if symbols.size != desc.rows * desc.cols or scales.size != desc.rows or esc_idx.size != esc_val.size:
        raise ValueError("symbols / scales / escape arrays do not match the descriptor")
    need = _u64(0)
    args = (ctypes.byref(tables) if tables is not None else None, ctypes.byref(desc), symbols.ctypes.data, scales.ctypes.data,
            esc_idx.ctypes.data if esc_idx.size else None,
            esc_val.ctypes.data if esc_val.size else None, esc_idx.size)
    # upper bound of the container size (at most one word per symbol), then
    # one encoding pass; EQ_ERANGE reports the exact size if the bound is short
    n_chunks = -(-symbols.size // desc.chunk_symbols) if desc.chunk_symbols else 1
    n_tab = -(-n_chunks // desc.seg_chunks) if desc.seg_chunks else 1
    bound = (256 + 512 * n_tab + 4 * desc.rows + 16 * n_chunks + 256 * n_chunks
             + 2 * (symbols.size + 8 * n_chunks) + 10 * esc_idx.size + 8 * 256)
    buf = np.empty(bound, dtype=np.uint8)
    st = _lib.eq_encode_host(*args, buf.ctypes.data, buf.size, ctypes.byref(need))
    if st == EQ_ERANGE:
        buf = np.empty(need.value, dtype=np.uint8)
        st = _lib.eq_encode_host(*args, buf.ctypes.data, buf.size, ctypes.byref(need))
    _check("eq_encode_host", st)
    return buf[:need.value].copy()


def encode_host(tables: eq_tables, dtype: int, rows: int, cols: int, symbols: np.ndarray,
                scales: np.ndarray, esc_idx=None, esc_val=None, esc_code: int = 0,
                chunk_symbols: int = 65536, lane_run: int = 8, codec: int = 0,
                seg_chunks: int = 0) -> np.ndarray:
    n_esc = 0 if esc_idx is None else len(esc_idx)
    d = eq_tensor_desc(dtype=dtype, lane_run=lane_run, rows=rows, cols=cols,
                       chunk_symbols=chunk_symbols, esc_enabled=1 if n_esc or esc_code else 0,
                       esc_code=esc_code, codec=codec, seg_chunks=seg_chunks)
    return eq_encode_host(tables, d, symbols, scales, esc_idx, esc_val)


def eq_parse_header(container: np.ndarray) -> eq_header:
    container = np.ascontiguousarray(container, dtype=np.uint8)
    h = eq_header()
    _check("eq_parse_header", _lib.eq_parse_header(container.ctypes.data, container.size, ctypes.byref(h)))
    return h


parse_header = eq_parse_header


# ---------------------------------------------------------------------------
# Device side (torch for memory and streams)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_handle(stream) -> int | None:
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class DeviceContainer:
    """A validated container resident in device memory."""

    def __init__(self, container: np.ndarray, device="cuda"):
        torch = _torch()
        self.host = np.ascontiguousarray(container, dtype=np.uint8)
        self.hdr = eq_parse_header(self.host)
        self.dev = torch.from_numpy(self.host).to(device)
        if self.dev.data_ptr() % 16:
            raise RuntimeError("device allocation is not 16-byte aligned")

    @property
    def n(self) -> int:
        return int(self.hdr.n)

    @property
    def nbytes(self) -> int:
        return int(self.hdr.total_bytes)


class Block:
    """eq_block for a list of device containers with their output offsets
    (default: concatenated in order). Keeps the ctypes arrays alive."""

    def __init__(self, containers, offsets=None, status=None):
        self.containers = list(containers)
        if offsets is None:
            offsets, o = [], 0
            for c in self.containers:
                offsets.append(o)
                o += c.n
        self.offsets = [int(o) for o in offsets]
        n = len(self.containers)
        self.refs = (eq_tensor_ref * max(1, n))()
        for i, (c, o) in enumerate(zip(self.containers, self.offsets)):
            self.refs[i].d_container = c.dev.data_ptr()
            self.refs[i].hdr = c.hdr
            self.refs[i].out_offset = o
        self.status = status
        self.c = eq_block(n_tensors=n, reserved=0, tensors=self.refs,
                          d_status=status.data_ptr() if status is not None else None)

    @property
    def n_out(self) -> int:
        return max([o + c.n for c, o in zip(self.containers, self.offsets)], default=0)


def eq_decode_dequant_bf16(block: Block, out, stream=None) -> None:
    _check("eq_decode_dequant_bf16",
           _lib.eq_decode_dequant_bf16(ctypes.byref(block.c), out.data_ptr(), _stream_handle(stream)))


def eq_decode_gemv_bf16(block: Block, xs, ys, stream=None) -> None:
    """Fused decode + batch-1 GEMV: ys[i] (fp32 [rows_i]) = W_i @ xs[i] (bf16 [cols_i])."""
    n = block.c.n_tensors
    if len(xs) != n or len(ys) != n:
        raise ValueError("one x and one y per tensor")
    xa = (ctypes.c_void_p * max(n, 1))(*[x.data_ptr() for x in xs])
    ya = (ctypes.c_void_p * max(n, 1))(*[y.data_ptr() for y in ys])
    _check("eq_decode_gemv_bf16",
           _lib.eq_decode_gemv_bf16(ctypes.byref(block.c), xa, ya, _stream_handle(stream)))


def eq_decode_block(block: Block, out, stream=None) -> None:
    _check("eq_decode_block",
           _lib.eq_decode_block(ctypes.byref(block.c), out.data_ptr(), _stream_handle(stream)))


def decode_dequant_bf16(containers, out, offsets=None, status=None, stream=None) -> Block:
    b = Block(containers, offsets, status)
    if b.n_out > out.numel():
        raise ValueError("output buffer too small")
    eq_decode_dequant_bf16(b, out, stream)
    return b


def decode_block(containers, out, offsets=None, status=None, stream=None) -> Block:
    b = Block(containers, offsets, status)
    if b.n_out > out.numel():
        raise ValueError("output buffer too small")
    eq_decode_block(b, out, stream)
    return b


def eq_gemv_bf16(w, rows: int, cols: int, x, y, stream=None, w_offset_elems: int = 0) -> None:
    _check("eq_gemv_bf16", _lib.eq_gemv_bf16(w.data_ptr() + 2 * w_offset_elems, rows, cols,
                                             x.data_ptr(), y.data_ptr(), _stream_handle(stream)))


def eq_bf16_from_f32(x, out, stream=None) -> None:
    _check("eq_bf16_from_f32", _lib.eq_bf16_from_f32(x.data_ptr(), x.numel(), out.data_ptr(),
                                                     _stream_handle(stream)))


class Pipeline:
    """eq_pipeline_*: blocks decoded into two alternating bf16 buffers on
    decode_stream, each decoded block's GEMVs on gemv_stream; mode
    EQ_PIPELINE_ALTERNATE (the default: the streams take turns) or
    EQ_PIPELINE_OVERLAP (a decode runs beside the previous block's GEMVs)."""

    def __init__(self, n_blocks: int, mode: int = None):
        self.h = _vp()
        _check("eq_pipeline_create", _lib.eq_pipeline_create(n_blocks, ctypes.byref(self.h)))
        self.n_blocks = n_blocks
        if mode is not None:
            self.set_mode(mode)

    def set_mode(self, mode: int) -> None:
        _check("eq_pipeline_set_mode", _lib.eq_pipeline_set_mode(self.h, mode))

    def run(self, blocks: list[Block], buf0, buf1, xs, ys, decode_stream, gemv_stream) -> None:
        n = len(blocks)
        arr = (eq_block * n)(*[b.c for b in blocks])
        xrows = [(_vp * max(1, len(x)))(*[t.data_ptr() for t in x]) for x in xs]
        yrows = [(_vp * max(1, len(y)))(*[t.data_ptr() for t in y]) for y in ys]
        xptrs = (_vp * n)(*[ctypes.cast(r, _vp) for r in xrows])
        yptrs = (_vp * n)(*[ctypes.cast(r, _vp) for r in yrows])
        self._keep = (arr, xrows, yrows, xptrs, yptrs)
        _check("eq_pipeline_run", _lib.eq_pipeline_run(
            self.h, arr, n, buf0.data_ptr(), buf1.data_ptr(), ctypes.cast(xptrs, _vp),
            ctypes.cast(yptrs, _vp), _stream_handle(decode_stream), _stream_handle(gemv_stream)))

    def close(self) -> None:
        if self.h:
            _lib.eq_pipeline_destroy(self.h)
            self.h = _vp()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


EQ_DEV_BAD_INPUT = 4


def eq_encode_device(dtype: int, rows: int, cols: int, d_symbols, d_scales, d_esc_idx=None,
                     d_esc_val=None, esc_code: int = 0, chunk_symbols: int = 65536, lane_run: int = 8,
                     workspace=None, out=None, stream=None, d_len=None, d_status=None,
                     codec: int = 0, seg_chunks: int = 0):
    """Device-side encode (torch tensors on the GPU). Returns (out, d_len,
    d_status) without synchronising: out[:int(d_len)] is the container once
    the stream has run. A d_status passed in is not cleared (flags of
    several calls accumulate).

    Lifetimes: the kernels run on `stream` (default: the current stream).
    Buffers this function allocates (workspace, out, d_len, d_status when not
    given) are marked as used on `stream`, so torch's caching allocator does
    not hand their memory out again before the kernels finish. Buffers the
    caller passes stay the caller's to keep alive until then."""
    torch = _torch()
    n_esc = 0 if d_esc_idx is None else int(d_esc_idx.numel())
    d = eq_tensor_desc(dtype=dtype, lane_run=lane_run, rows=rows, cols=cols,
                       chunk_symbols=chunk_symbols, esc_enabled=1 if n_esc or esc_code else 0,
                       esc_code=esc_code, codec=codec, seg_chunks=seg_chunks)
    dev = d_symbols.device
    wsb = int(_lib.eq_encode_device_workspace(rows, cols, chunk_symbols))
    cap = int(_lib.eq_encode_device_bound(rows, cols, chunk_symbols, n_esc))
    made = []
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
        made.append(workspace)
    if out is None:
        out = torch.empty(max(cap, 16), dtype=torch.uint8, device=dev)
        made.append(out)
    if d_len is None:
        d_len = torch.zeros(1, dtype=torch.int64, device=dev)
        made.append(d_len)
    if d_status is None:
        d_status = torch.zeros(1, dtype=torch.int32, device=dev)
        made.append(d_status)
    if made and stream is not None and not isinstance(stream, int) and stream != torch.cuda.current_stream(dev):
        for t in made:
            t.record_stream(stream)
        # the zero fills above ran on the current stream: the encode must see them
        stream.wait_stream(torch.cuda.current_stream(dev))
    _check("eq_encode_device", _lib.eq_encode_device(
        ctypes.byref(d), d_symbols.data_ptr(), d_scales.data_ptr(),
        d_esc_idx.data_ptr() if n_esc else None, d_esc_val.data_ptr() if n_esc else None, n_esc,
        workspace.data_ptr(), workspace.numel(), out.data_ptr(), out.numel(), d_len.data_ptr(),
        d_status.data_ptr(), _stream_handle(stream)))
    return out, d_len, d_status


EQ_ENCODE_STATIC_SCRATCH_BYTES = 136 << 20


def eq_encode_device_static(dtype: int, rows: int, cols: int, d_symbols, d_scales, out, d_len, d_status,
                            d_esc_idx=None, d_esc_val=None, esc_code: int = 0, chunk_symbols: int = 65536,
                            lane_run: int = 8, stream=None, codec: int = 0, seg_chunks: int = 0) -> None:
    """eq_encode_device with the library's static per-GPU scratch instead of
    a workspace: the caller passes every buffer (out of at least
    eq_encode_device_bound bytes, d_len u64, d_status u32, all on the GPU),
    and the call allocates nothing. Calls that overlap on one GPU race."""
    n_esc = 0 if d_esc_idx is None else int(d_esc_idx.numel())
    d = eq_tensor_desc(dtype=dtype, lane_run=lane_run, rows=rows, cols=cols,
                       chunk_symbols=chunk_symbols, esc_enabled=1 if n_esc or esc_code else 0,
                       esc_code=esc_code, codec=codec, seg_chunks=seg_chunks)
    _check("eq_encode_device_static", _lib.eq_encode_device_static(
        ctypes.byref(d), d_symbols.data_ptr(), d_scales.data_ptr(),
        d_esc_idx.data_ptr() if n_esc else None, d_esc_val.data_ptr() if n_esc else None, n_esc,
        out.data_ptr(), out.numel(), d_len.data_ptr(), d_status.data_ptr(), _stream_handle(stream)))
