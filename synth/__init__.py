"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws inputs: byte codes with a prescribed distribution,
per-row scales and super-weight side lists. It contains none of the decode
method's arithmetic, and neither the oracle nor the product library imports it;
callers pass its arrays to both.

The pages measure on trained open-weight LLMs ("Float8@2bits: Entropy Coding
Enables Data-Free Model Compression", technical summary section 4) that are not
available here; these recipes stand in for them with the layer shapes of a 7B
and a 70B decoder block and code distributions at the entropies the pages
quote (about 2.1 and 3.0 bits per parameter, same section and section 3 item 2):

* Int8 codes: discrete Laplace P(k) ~ theta^|k| on [-127, 127], theta chosen by
  bisection so that the distribution's entropy is the target.
* E4M3 codes: the code of round-to-nearest-even(z * s) for z ~ N(0, 1), drawn
  directly from its exact distribution (the N(0,1) mass of each code's rounding
  interval); s chosen by bisection so the code entropy is the target.
* Scales: fp32 of a uniform draw in [0.005, 0.015] per output row.
* Super weights (70B block, down projection): 4 distinct seeded flat positions
  hold the escape code; their stored values are +-100 x the population std of
  that row's weights (fp64) rounded to bf16.

Every stream is SplitMix64 of a key derived from
(0xE0A5, config, layer, tensor, purpose); see ``sampler.c``.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from functools import lru_cache

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15

DTYPE_INT8 = 1
DTYPE_E4M3 = 2
ESC_CODE = {DTYPE_INT8: 0x80, DTYPE_E4M3: 0x7F}

PURPOSE_SYMBOLS, PURPOSE_SCALES, PURPOSE_ESCAPES, PURPOSE_ACT = 0, 1, 2, 3
TENSOR_NAMES = ("q", "k", "v", "o", "gate", "up", "down")


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


@lru_cache(maxsize=1)
def _lib():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    lib.synth_u64.restype = ctypes.c_uint64
    lib.synth_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.synth_fill_u64.restype = None
    lib.synth_fill_u64.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
    lib.synth_categorical.restype = ctypes.c_int
    lib.synth_categorical.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p, ctypes.c_int]
    return lib


def sm64(key: int, i: int) -> int:
    """Output i of SplitMix64 seeded with key (pure Python, for keys)."""
    z = (key + (i + 1) * GOLDEN) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def stream_key(*parts: int) -> int:
    k = 0xE0A5
    for p in parts:
        k = sm64(k ^ (p & MASK64), 0)
    return k


def u64s(key: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    if n:
        _lib().synth_fill_u64(key, start, n, out.ctypes.data)
    return out


def uniform01(key: int, start: int, n: int) -> np.ndarray:
    """53-bit uniform doubles in [0, 1)."""
    return (u64s(key, start, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


# --------------------------------------------------------------------------
# Categorical distributions over byte codes
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Categorical:
    syms: np.ndarray   # uint8, most probable first
    thr: np.ndarray    # uint64 cumulative thresholds on the 2^64 grid
    probs: np.ndarray  # float64, same order

    @property
    def entropy(self) -> float:
        p = self.probs[self.probs > 0]
        return float(-(p * np.log2(p)).sum())


def _categorical(byte_probs: dict[int, float]) -> Categorical:
    items = [(b, p) for b, p in byte_probs.items() if p > 0.0]
    total = math.fsum(p for _, p in items)
    items = sorted(((b, p / total) for b, p in items), key=lambda bp: (-bp[1], bp[0]))
    syms = np.array([b for b, _ in items], dtype=np.uint8)
    probs = np.array([p for _, p in items], dtype=np.float64)
    thr = []
    acc = []
    for _, p in items:
        acc.append(p)
        c = math.fsum(acc)
        thr.append(min(MASK64, int(c * 2.0 ** 64)))
    thr[-1] = MASK64
    return Categorical(syms, np.array(thr, dtype=np.uint64), probs)


def laplace_table(theta: float) -> Categorical:
    """Discrete Laplace on [-127, 127]: P(k) ~ theta^|k|; byte = k mod 256."""
    probs = {}
    w = 1.0
    for a in range(0, 128):
        if a == 0:
            probs[0] = 1.0
        else:
            probs[a & 0xFF] = w
            probs[(-a) & 0xFF] = w
        w *= theta
    return _categorical(probs)


def _bisect(fn, lo: float, hi: float, target: float, iters: int = 200) -> float:
    flo = fn(lo) - target
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        fm = fn(mid) - target
        if (fm < 0) == (flo < 0):
            lo, flo = mid, fm
        else:
            hi = mid
    return 0.5 * (lo + hi)


@lru_cache(maxsize=None)
def theta_for_entropy(bits: float) -> float:
    return _bisect(lambda th: laplace_table(th).entropy, 1e-6, 0.999, bits)


@lru_cache(maxsize=1)
def _e4m3_values() -> np.ndarray:
    import torch  # library routine for the E4M3 code values (input synthesis only)
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return codes.to(torch.float64).numpy()


def e4m3_table(s: float) -> Categorical:
    """Codes of RNE(z * s), z ~ N(0, 1): each code gets the N(0,1) mass of its
    rounding interval (ties have measure zero)."""
    vals = _e4m3_values()
    pos = sorted((float(vals[c]), c) for c in range(128) if not math.isnan(vals[c]))
    probs = {}
    r2 = math.sqrt(2.0)
    for i, (v, c) in enumerate(pos):
        lo = 0.0 if i == 0 else 0.5 * (pos[i - 1][0] + v)
        hi = 0.5 * (v + pos[i + 1][0]) if i + 1 < len(pos) else v + 0.5 * (v - pos[i - 1][0])
        p = 0.5 * (math.erfc(lo / (s * r2)) - math.erfc(hi / (s * r2)))
        probs[c] = p          # +v
        probs[c | 0x80] = p   # -v (and -0 for c = 0)
    return _categorical(probs)


@lru_cache(maxsize=None)
def e4m3_scale_for_entropy(bits: float) -> float:
    log2s = _bisect(lambda l2: e4m3_table(2.0 ** l2).entropy, -20.0, 4.0, bits)
    return 2.0 ** log2s


def sample(cat: Categorical, key: int, start: int, n: int, threads: int | None = None) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    if n:
        rc = _lib().synth_categorical(key, start, n, cat.syms.ctypes.data, cat.thr.ctypes.data,
                                      len(cat.syms), out.ctypes.data, threads or default_threads())
        if rc:
            raise RuntimeError("synth_categorical failed")
    return out


GPU_LIB_PATH = os.path.join(_HERE, "libsynth_gpu.so")


@lru_cache(maxsize=1)
def _gpu_lib():
    if not os.path.exists(GPU_LIB_PATH):
        raise RuntimeError(f"{GPU_LIB_PATH} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(GPU_LIB_PATH)
    lib.synth_categorical_gpu.restype = ctypes.c_int
    lib.synth_categorical_gpu.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def sample_gpu(cat: Categorical, key: int, start: int, out, stream=None) -> None:
    """The bytes `sample` draws for stream indices start .. start+out.numel()-1,
    drawn on the GPU into the uint8 device tensor `out` (same values)."""
    import torch
    dev = out.device
    syms = torch.from_numpy(cat.syms).to(dev)
    thr = torch.from_numpy(cat.thr.view(np.int64)).to(dev)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    rc = _gpu_lib().synth_categorical_gpu(key, start, out.numel(), syms.data_ptr(), thr.data_ptr(),
                                          len(cat.syms), out.data_ptr(), s.cuda_stream)
    if rc:
        raise RuntimeError("synth_categorical_gpu failed")
    s.synchronize()  # the category tables are freed on return


def make_tensor_gpu(cfg: int, layer: int, t: int, out, spec: TensorSpec | None = None) -> Tensor:
    """make_tensor with the symbols drawn on the GPU into the uint8 device
    tensor `out` (spec.n elements): the returned Tensor carries the scales
    and the super-weight list, and symbols = None."""
    import torch
    spec = spec or config_specs(cfg)[t]
    if out.numel() != spec.n or out.dtype != torch.uint8:
        raise ValueError("out must be a uint8 device tensor of spec.n elements")
    sample_gpu(table_for(spec), stream_key(cfg, layer, t, PURPOSE_SYMBOLS), 0, out)
    tensor = Tensor(spec, None, scales_for(cfg, layer, t, spec.rows))
    if spec.n_esc:
        tensor.esc_idx, tensor.esc_val = escapes_for(cfg, layer, t, spec)
        out[torch.from_numpy(tensor.esc_idx.astype(np.int64)).to(out.device)] = ESC_CODE[spec.dtype]
    return tensor


def empirical_entropy(sym: np.ndarray) -> float:
    c = np.bincount(sym, minlength=256).astype(np.float64)
    p = c[c > 0] / c.sum()
    return float(-(p * np.log2(p)).sum())


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class TensorSpec:
    name: str
    rows: int
    cols: int
    dtype: int
    bits: float
    n_esc: int = 0

    @property
    def n(self) -> int:
        return self.rows * self.cols


@dataclass
class Tensor:
    spec: TensorSpec
    symbols: np.ndarray          # uint8 [rows * cols], escape code at escape positions
    scales: np.ndarray           # float32 [rows]
    esc_idx: np.ndarray = field(default_factory=lambda: np.zeros(0, np.uint64))
    esc_val: np.ndarray = field(default_factory=lambda: np.zeros(0, np.uint16))

    @property
    def esc_code(self) -> int:
        return ESC_CODE[self.spec.dtype]


def _block(h: int, kv: int, f: int, dtype: int, bits: float, down_esc: int) -> list[TensorSpec]:
    shapes = [(h, h), (kv, h), (kv, h), (h, h), (f, h), (f, h), (h, f)]
    return [TensorSpec(nm, r, c, dtype, bits, down_esc if nm == "down" else 0)
            for nm, (r, c) in zip(TENSOR_NAMES, shapes)]


CONFIG_NAMES = {
    1: "1024x1024 int8, 2.1-bit Laplace",
    2: "4096x4096 int8, 3.0-bit Laplace (7B q_proj)",
    3: "7B block, E4M3, 2.1 bit, 7 tensors",
    4: "70B block, int8, 2.1 bit, 4 super-weight escapes",
    5: "80 x 70B block, double-buffered decode + bf16 GEMV",
}
CHUNK_SYMBOLS = 65536
LANE_RUN = 8
N_LAYERS_MODEL = 80

# Chunk size of each configuration's containers (symbols per chunk). The
# 4096x4096 matrix mandates 64 Ki; elsewhere the size is a container field,
# chosen by measured decode time (compressed data read from HBM, not from the
# last-level cache) against the 256 B of lane states each chunk adds: smaller
# chunks shorten the serial work of the last waves of a launch. The fused
# decode + GEMV wants longer chunks that hold whole rows (GEMV_CHUNK_TARGET).
GEMV_CHUNK_TARGET = 32768
CONFIG_CHUNK = {1: 8192, 2: 65536, 3: 16896, 4: 32768, 5: 32768}


def config_chunk(cfg: int) -> int:
    return CONFIG_CHUNK[cfg]


def config_specs(cfg: int) -> list[TensorSpec]:
    if cfg == 1:
        return [TensorSpec("w", 1024, 1024, DTYPE_INT8, 2.1)]
    if cfg == 2:
        return [TensorSpec("q", 4096, 4096, DTYPE_INT8, 3.0)]
    if cfg == 3:
        return _block(4096, 4096, 11008, DTYPE_E4M3, 2.1, 0)
    if cfg in (4, 5):
        return _block(8192, 1024, 28672, DTYPE_INT8, 2.1, 4)
    raise ValueError(f"unknown config {cfg}")


def block_offsets(specs: list[TensorSpec]) -> list[int]:
    """Element offsets of each tensor inside the concatenated block buffer."""
    offs, o = [], 0
    for s in specs:
        offs.append(o)
        o += s.n
    offs.append(o)
    return offs


def table_for(spec: TensorSpec) -> Categorical:
    if spec.dtype == DTYPE_INT8:
        return laplace_table(theta_for_entropy(spec.bits))
    return e4m3_table(e4m3_scale_for_entropy(spec.bits))


def scales_for(cfg: int, layer: int, t: int, rows: int) -> np.ndarray:
    u = uniform01(stream_key(cfg, layer, t, PURPOSE_SCALES), 0, rows)
    return (0.005 + 0.01 * u).astype(np.float32)


def _escape_positions(key: int, n: int, count: int) -> tuple[list[int], list[int]]:
    pos, signs, i = [], [], 0
    while len(pos) < count:
        u = sm64(key, i)
        i += 1
        p = u % n
        if p in pos:
            continue
        pos.append(p)
        signs.append(1 if (sm64(key, 1 << 40 | i) >> 63) else -1)
    order = sorted(range(count), key=lambda a: pos[a])
    return [pos[a] for a in order], [signs[a] for a in order]


def _row_values_f64(spec: TensorSpec, sym_row: np.ndarray, scale: float) -> np.ndarray:
    if spec.dtype == DTYPE_INT8:
        v = sym_row.view(np.int8).astype(np.float64)
    else:
        v = _e4m3_values()[sym_row]
    return v * float(scale)


def escapes_for(cfg: int, layer: int, t: int, spec: TensorSpec) -> tuple[np.ndarray, np.ndarray]:
    """Super-weight side list (ascending flat indices, bf16 bits) of a tensor;
    each value is +-100 x the std of its row's weights before substitution."""
    if not spec.n_esc:
        return np.zeros(0, np.uint64), np.zeros(0, np.uint16)
    import torch  # bf16 rounding of the stored super-weight values (library routine)
    pos, signs = _escape_positions(stream_key(cfg, layer, t, PURPOSE_ESCAPES), spec.n, spec.n_esc)
    scales = scales_for(cfg, layer, t, spec.rows)
    tab = table_for(spec)
    key = stream_key(cfg, layer, t, PURPOSE_SYMBOLS)
    vals = []
    for p, sg in zip(pos, signs):
        r = p // spec.cols
        row = sample(tab, key, r * spec.cols, spec.cols)
        std = float(np.std(_row_values_f64(spec, row, scales[r])))
        v32 = torch.tensor([sg * 100.0 * std], dtype=torch.float32)
        vals.append(int(v32.to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF)
    return np.array(pos, dtype=np.uint64), np.array(vals, dtype=np.uint16)


def make_tensor(cfg: int, layer: int, t: int, spec: TensorSpec | None = None,
                threads: int | None = None) -> Tensor:
    spec = spec or config_specs(cfg)[t]
    sym = sample(table_for(spec), stream_key(cfg, layer, t, PURPOSE_SYMBOLS), 0, spec.n, threads)
    tensor = Tensor(spec, sym, scales_for(cfg, layer, t, spec.rows))
    if spec.n_esc:
        tensor.esc_idx, tensor.esc_val = escapes_for(cfg, layer, t, spec)
        sym[tensor.esc_idx.astype(np.int64)] = ESC_CODE[spec.dtype]
    return tensor


def symbols_slice(cfg: int, layer: int, t: int, start: int, n: int,
                  spec: TensorSpec | None = None) -> np.ndarray:
    """Symbols [start, start+n) of a tensor without generating the rest
    (escape positions hold the escape code)."""
    spec = spec or config_specs(cfg)[t]
    sym = sample(table_for(spec), stream_key(cfg, layer, t, PURPOSE_SYMBOLS), start, n)
    if spec.n_esc:
        pos, _ = _escape_positions(stream_key(cfg, layer, t, PURPOSE_ESCAPES), spec.n, spec.n_esc)
        for p in pos:
            if start <= p < start + n:
                sym[p - start] = ESC_CODE[spec.dtype]
    return sym


def gemv_activation(cfg: int, layer: int, t: int, cols: int) -> np.ndarray:
    """N(0,1) activation vector (float32; the caller rounds to bf16), Box-Muller
    on the seeded uniform stream."""
    key = stream_key(cfg, layer, t, PURPOSE_ACT)
    m = (cols + 1) // 2
    u1 = uniform01(key, 0, m)
    u2 = uniform01(key, m, m)
    r = np.sqrt(-2.0 * np.log1p(-u1))
    z = np.concatenate([r * np.cos(2 * np.pi * u2), r * np.sin(2 * np.pi * u2)])[:cols]
    return z.astype(np.float32)


DRIFT_BITS = (0.8, 2.1, 3.2, 1.4)


def drift_tensor(rows: int, cols: int, bands: int = 16, bits=DRIFT_BITS, seed: int = 0) -> Tensor:
    """Int8 tensor whose statistics drift along the rows: the rows are cut into
    `bands` equal bands, band b drawn i.i.d. from the discrete Laplace whose
    entropy is bits[b % len(bits)]. Per-row scales as for the configs. Input
    for the adaptive-table comparison (one table vs one table per segment)."""
    spec = TensorSpec("drift", rows, cols, DTYPE_INT8, 0.0)
    sym = np.empty(rows * cols, np.uint8)
    edges = [rows * b // bands for b in range(bands + 1)]
    for b in range(bands):
        lo, hi = edges[b] * cols, edges[b + 1] * cols
        cat = laplace_table(theta_for_entropy(bits[b % len(bits)]))
        sym[lo:hi] = sample(cat, stream_key(99, seed, b, PURPOSE_SYMBOLS), 0, hi - lo)
    return Tensor(spec, sym, scales_for(4, seed, 4, rows))
