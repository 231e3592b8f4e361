#!/usr/bin/env python3
"""Benchmark: decode + dequant of one 70B-shaped transformer block on one GPU.

Workload (the block the metric is quoted on): q, o 8192x8192; k, v 1024x8192;
gate, up 28672x8192; down 8192x28672 -- 855,638,016 int8 weights whose codes
are a 2.1-bit discrete Laplace, one 12-bit frequency table per tensor, fp32
per-row scales, 4 super-weight escapes in down, container v1 with 32 Ki-symbol
chunks and lane run 8. A step is one eq_decode_dequant_bf16 call over the
whole block (one kernel launch) into a 1.71 GB bf16 buffer; containers are
resident in HBM before timing starts, in several copies: each launch decodes
the next copy, so its compressed reads come from HBM as in a forward pass
(one copy decoded again and again would stay in the 256 MB last-level cache;
that figure is reported as warm_llc).

Prints one JSON line. `--workload model80` instead runs the 80-block
double-buffered decode + GEMV schedule and prints its own line.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cpus() -> dict:
    """What the host offers: logical CPUs (os.cpu_count), those this process
    may run on (affinity) and the CPU model (/proc/cpuinfo, as lscpu shows it)."""
    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:
        aff = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity": aff, "model": model}


def host_cores() -> int:
    """Threads for the CPU baseline: every CPU this process may use, capped at
    16, the host share a one-GPU machine gives a job (whatever nproc reports)."""
    return max(1, min(16, host_cpus()["affinity"]))


def algorithmic_bytes(conts) -> tuple[int, int]:
    """(compressed bytes a decode must read, bf16 bytes it must write): words
    actually stored, lane states, chunk directory, frequency table, scales and
    side list; 2 bytes per output weight."""
    import numpy as np
    comp = 0
    n = 0
    for c in conts:
        h = c.hdr
        dirs = c.host[h.off_dir:h.off_dir + 16 * h.n_chunks].reshape(-1, 16)
        words = int(dirs[:, 8:12].copy().view(np.uint32).astype(np.int64).sum())
        comp += 2 * words + 256 * h.n_chunks + 16 * h.n_chunks + 512 + 4 * h.rows + 10 * h.n_esc
        n += h.n
    return comp, 2 * n


def traffic_record(kernel_src: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "decode_block70b_traffic.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = (s.strip() for s in line.split("=", 1))
            rec[k] = v
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None
    try:
        return int(float(rec["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def whole_row_chunk(cols: int, lane_run: int, target: int = 65536) -> int:
    """Chunk size for the fused decode + GEMV: a multiple of both the row
    length and 64 * K (so chunks hold whole rows), as close to target as
    that allows."""
    g = 64 * lane_run
    lcm = cols * g // math.gcd(cols, g)
    return lcm * max(1, round(target / lcm))


VALU_PEAK_GINST = 256 * 4 * 2.4 / 4  # wave64 VALU instructions per ns: 256 CUs x 4 SIMDs, 4 cycles each, 2.4 GHz


def counter_record(name: str, key: str, kernel_src: str):
    """A per-launch figure measured with rocprofv3 counters (profiles/<name>),
    if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if "=" in line:
            k, v = (t.strip() for t in line.split("=", 1))
            rec[k] = v
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha:
        return None
    try:
        return int(float(rec[key]))
    except (KeyError, ValueError):
        return None


def build_block(cfg: int, layer: int = 0, lane_run: int = 8, use_cache: bool = True,
                tensors=None, whole_rows: bool = False, codec: int = 0, bits: float | None = None,
                chunk: int | None = None):
    """Encode one block with the library's host encoder and place its
    containers in device memory (all tensors, or the listed indices). Chunks
    are the configuration's size (synth.config_chunk) or `chunk` symbols, or
    with whole_rows the multiple of the row length nearest to that size (what
    the fused decode + GEMV needs). codec 0 = rANS, 1 = Huffman.
    With EQ_BENCH_CACHE=<dir> the encoded containers are kept there as .npy
    files and reused. bits: another entropy for the synthetic codes (bits
    per weight) than the configuration's."""
    import dataclasses
    import numpy as np
    import synth
    from rans_decode_amd import eq
    specs = synth.config_specs(cfg)
    if bits is not None:
        specs = [dataclasses.replace(sp, bits=bits) for sp in specs]
    cache = os.environ.get("EQ_BENCH_CACHE") if use_cache else None
    conts = []
    for i, sp in enumerate(specs):
        if tensors is not None and i not in tensors:
            continue
        target = chunk or synth.config_chunk(cfg)
        Z = whole_row_chunk(sp.cols, lane_run, target) if whole_rows else target
        btag = "" if bits is None else f"_b{bits:g}"
        path = (os.path.join(cache, f"cfg{cfg}_layer{layer}_t{i}_k{lane_run}_z{Z}_c{codec}{btag}.npy")
                if cache else None)
        if path and os.path.exists(path):
            blob = np.load(path)
        else:
            t = synth.make_tensor(cfg, layer, i, spec=sp)
            tab = eq.build_tables(t.symbols)
            esc = t.esc_idx.size > 0
            blob = eq.encode_host(tab, sp.dtype, sp.rows, sp.cols, t.symbols, t.scales,
                                  t.esc_idx if esc else None, t.esc_val if esc else None,
                                  esc_code=t.esc_code if esc else 0,
                                  chunk_symbols=Z, lane_run=lane_run, codec=codec)
            del t
            if path:
                os.makedirs(cache, exist_ok=True)
                np.save(path, blob)
        conts.append(eq.DeviceContainer(blob, device="cuda"))
    return specs, conts


class DeviceEncoder:
    """Builds a block's containers on the device: codes drawn by the seeded
    GPU sampler (the host sampler's values) and encoded by eq_encode_device;
    each container is parsed on the host (its header) and kept on the device.
    Buffers are sized for the largest tensor and reused."""

    def __init__(self, specs, chunk: int, lane_run: int):
        import torch
        from rans_decode_amd import eq
        self.Z, self.K = chunk, lane_run
        self.sym = torch.empty(max(sp.n for sp in specs), dtype=torch.uint8, device="cuda")
        self.ws = torch.empty(max(int(eq._lib.eq_encode_device_workspace(sp.rows, sp.cols, chunk)) for sp in specs),
                              dtype=torch.uint8, device="cuda")
        self.out = torch.empty(max(int(eq._lib.eq_encode_device_bound(sp.rows, sp.cols, chunk, sp.n_esc))
                                   for sp in specs), dtype=torch.uint8, device="cuda")
        self.d_len = torch.zeros(1, dtype=torch.int64, device="cuda")
        self.d_st = torch.zeros(1, dtype=torch.int32, device="cuda")

    def container(self, cfg: int, layer: int, i: int, sp, Z: int | None = None):
        import numpy as np
        import torch
        import synth
        from rans_decode_amd import eq
        Zc = Z or self.Z
        need_ws = int(eq._lib.eq_encode_device_workspace(sp.rows, sp.cols, Zc))
        need_out = int(eq._lib.eq_encode_device_bound(sp.rows, sp.cols, Zc, sp.n_esc))
        if need_ws > self.ws.numel():
            self.ws = torch.empty(need_ws, dtype=torch.uint8, device="cuda")
        if need_out > self.out.numel():
            self.out = torch.empty(need_out, dtype=torch.uint8, device="cuda")
        sym = self.sym[:sp.n]
        t = synth.make_tensor_gpu(cfg, layer, i, sym, spec=sp)
        esc = t.esc_idx.size > 0
        eq.eq_encode_device(sp.dtype, sp.rows, sp.cols, sym, torch.from_numpy(t.scales).cuda(),
                            torch.from_numpy(t.esc_idx.astype(np.int64)).cuda() if esc else None,
                            torch.from_numpy(t.esc_val.view(np.int16)).cuda() if esc else None,
                            t.esc_code if esc else 0, Zc, self.K, workspace=self.ws, out=self.out,
                            d_len=self.d_len, d_status=self.d_st)
        n = int(self.d_len.item())
        if int(self.d_st.item()):
            raise RuntimeError(f"device encoder flagged config {cfg} layer {layer} tensor {i}")
        c = eq.DeviceContainer.__new__(eq.DeviceContainer)
        c.dev = self.out[:n].clone()
        c.host = c.dev.cpu().numpy()
        c.hdr = eq.parse_header(c.host)
        return c


def sampled_symbols_check(cfg, layer, specs, conts, rng_seed=1) -> int:
    """Decode-only pass (eq_decode_block, u8 codes) over the same containers;
    whole chunks (first, last and 3 random per tensor) are compared with the
    seeded generator's symbols. Returns the number of mismatching codes."""
    import numpy as np
    import torch
    import synth
    from rans_decode_amd import eq
    offs = [0]
    for sp in specs:
        offs.append(offs[-1] + sp.n)
    out = torch.empty(offs[-1], dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    eq.eq_decode_block(eq.Block(conts, offs[:-1], status), out)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())}")
    rng = np.random.default_rng(rng_seed)
    bad = 0
    for i, (sp, c, o) in enumerate(zip(specs, conts, offs)):
        nch = int(c.hdr.n_chunks)
        Z = int(c.hdr.chunk_symbols)
        for k in sorted(set(rng.integers(0, nch, 3).tolist() + [0, nch - 1])):
            lo, hi = k * Z, min(sp.n, (k + 1) * Z)
            exp = synth.symbols_slice(cfg, layer, i, lo, hi - lo, spec=sp)
            got = out[o + lo:o + hi].cpu().numpy()
            bad += int((got != exp).sum())
    del out
    return bad


def cpu_baseline(conts, target_s: float = 10.0):
    """The oracle, as it stands, decoding + dequantising the same containers
    on the host cores (chunk-parallel, static partition). The sample grows
    from one chunk per thread per tensor up to the whole block, and the whole
    block is decoded repeatedly when one pass takes less than target_s."""
    import numpy as np
    import oracle
    threads = host_cores()
    outs = [np.zeros(int(c.hdr.n), np.uint16) for c in conts]

    def run(per_tensor, nthreads=threads):
        t0 = time.perf_counter()
        n = 0
        for c, k, o in zip(conts, per_tensor, outs):
            flags = oracle.decode_chunks(c.host, 0, k, nthreads, bf16_out=o)
            if flags:
                raise RuntimeError(f"oracle decode flags {flags}")
            n += min(int(c.hdr.n), k * int(c.hdr.chunk_symbols))
        return time.perf_counter() - t0, n

    ks = [min(int(c.hdr.n_chunks), threads) for c in conts]
    dt, n = run(ks)
    scale = max(1.0, target_s / max(dt, 1e-3))
    ks = [min(int(c.hdr.n_chunks), max(1, int(k * scale))) for c, k in zip(conts, ks)]
    dt, n = run(ks)
    reps = 1
    if dt < target_s:
        reps = max(1, int(target_s / max(dt, 1e-3)))
        total_t, total_n = 0.0, 0
        for _ in range(reps):
            d, m = run(ks)
            total_t += d
            total_n += m
        dt, n = total_t, total_n
    whole = all(k == int(c.hdr.n_chunks) for c, k in zip(conts, ks))
    what = (f"the whole {len(conts)}-tensor block" if len(conts) > 1 else "the whole tensor") if whole \
        else f"chunks [0, k) of each tensor, k = {ks}"
    desc = (f"{what} ({n // reps / 1e6:.1f} M weights per pass, {reps} pass(es)), decoded + "
            f"dequantised to bf16 by the oracle with {threads} threads")
    # the same oracle on one thread: one chunk of each tensor, repeated to ~2 s
    one = [1 for _ in conts]
    d1, n1 = run(one, 1)
    r1 = max(1, int(2.0 / max(d1, 1e-3)))
    t1, m1 = 0.0, 0
    for _ in range(r1):
        d, m = run(one, 1)
        t1 += d
        m1 += m
    return {"value": round(2.0 * n / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": desc, "seconds": round(dt, 2), "host": host_cpus(),
            "single_thread": {"value": round(2.0 * m1 / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "sample": f"chunk 0 of each of the {len(conts)} tensor(s), {r1} pass(es)",
                              "seconds": round(t1, 2)}}


def copy_ceiling(nbytes: int) -> tuple[float, float, float]:
    """GB/s (read + write) of a plain device-to-device copy of nbytes (torch's
    copy), GB/s of a read-only pass over the same bytes (the library's batch-1
    GEMV, eq_gemv_bf16, over them as a bf16 [rows, 8192] matrix, which reads
    each weight once; x and y are 16 KiB and rows x 4 B), and GB/s of a
    write-only pass (torch's fill of the same bytes). The copy and the GEMV
    are also the known-size references that scale the HBM byte counters."""
    import torch
    from rans_decode_amd import eq
    cols = 8192
    rows = nbytes // 2 // cols
    a = torch.ones(rows * cols, dtype=torch.int16, device="cuda")
    b = torch.empty_like(a)
    x = torch.ones(cols, dtype=torch.int16, device="cuda")
    y = torch.empty(rows, dtype=torch.float32, device="cuda")
    for _ in range(2):
        b.copy_(a)
        eq.eq_gemv_bf16(a, rows, cols, x, y)
        b.fill_(3)
    torch.cuda.synchronize()
    reps = 10

    def per_call(fn):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    copy_ms = per_call(lambda: b.copy_(a))
    read_ms = per_call(lambda: eq.eq_gemv_bf16(a, rows, cols, x, y))
    write_ms = per_call(lambda: b.fill_(3))
    del a, b
    nb = rows * cols * 2
    return 2.0 * nb / (copy_ms * 1e-3) / 1e9, nb / (read_ms * 1e-3) / 1e9, nb / (write_ms * 1e-3) / 1e9


CODECS = {"rans": 0, "huffman": 1}

WORKLOADS = {
    "block70b": (4, "70B-shaped block decode+dequant: q,o 8192x8192; k,v 1024x8192; gate,up 28672x8192; "
                    "down 8192x28672; int8 2.1-bit Laplace codes, 4 super-weight escapes"),
    "cfg1": (1, "single 1024x1024 int8 matrix, 2.1-bit Laplace codes"),
    "cfg2": (2, "single 4096x4096 int8 matrix (7B q_proj), 3.0-bit Laplace codes"),
    "cfg3": (3, "7B-shaped block decode+dequant: q,k,v,o 4096x4096; gate,up 11008x4096; down 4096x11008; "
                "E4M3 codes at 2.1 bits"),
}


def bench_block(args):
    import numpy as np
    import torch
    import synth
    from rans_decode_amd import eq

    cfg, what = WORKLOADS[args.workload]
    codec = CODECS[args.codec]
    t0 = time.perf_counter()
    specs, conts = build_block(cfg, 0, args.lane_run, codec=codec, bits=args.bits, chunk=args.chunk)
    Z = int(conts[0].hdr.chunk_symbols)
    offs = synth.block_offsets(specs)
    n = offs[-1]
    log(f"block built in {time.perf_counter() - t0:.1f} s: {n} weights, "
        f"{sum(c.nbytes for c in conts) / 1e6:.1f} MB of containers")
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    reps = replicas(conts)
    blocks = [eq.Block(cc, offs[:-1], status) for cc in reps]
    block = blocks[0]
    rot = Rotation(blocks)
    stream = torch.cuda.current_stream()

    # one decode of every copy and the status, the clock settle and the
    # warm-up right before the timed launches, and the host-side decode check
    # after them (an idle GPU between warm-up and timing would start the
    # timing at low clocks). Each launch decodes the next copy of the block.
    for b in blocks:
        eq.eq_decode_dequant_bf16(b, out, stream)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())}")
    settle = clock_settle(lambda: eq.eq_decode_dequant_bf16(rot.next(), out, stream), stream, args.settle_ms)
    for _ in range(args.warmup):
        eq.eq_decode_dequant_bf16(rot.next(), out, stream)

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for s, e in evs:
        s.record(stream)
        eq.eq_decode_dequant_bf16(rot.next(), out, stream)
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = [s.elapsed_time(e) for s, e in evs]
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())}")
    # the same block decoded again and again: its containers stay in the
    # last-level cache (a repeated single block, not a forward pass)
    for _ in range(3):
        eq.eq_decode_dequant_bf16(block, out, stream)
    wevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)]
    for s, e in wevs:
        s.record(stream)
        eq.eq_decode_dequant_bf16(block, out, stream)
        e.record(stream)
    torch.cuda.synchronize()
    warm_ms = float(np.mean([s.elapsed_time(e) for s, e in wevs]))
    u8_ms = decode_only_ms(rot, n, stream, args.steps)
    bad = sampled_symbols_check(cfg, 0, specs, conts)
    log(f"sampled decode check vs the generated symbols: {bad} mismatching codes")
    if bad:
        raise RuntimeError("decoded symbols differ from the encoded ones")
    avg_ms = float(np.mean(ms))
    comp, outb = algorithmic_bytes(conts)
    algo = comp + outb
    achieved = algo / (avg_ms * 1e-3) / 1e9
    traffic = (traffic_record(os.path.join(ROOT, "rans_decode_amd", "csrc", "decode.hip"))
               if cfg == 4 and codec == 0 and args.bits is None else None)
    total_container = sum(c.nbytes for c in conts)
    rec = {
        "metric": "decoded weight GB/s (bf16 out) and % HBM roofline, 70B-shaped block decode"
                  if cfg == 4 else f"decoded weight GB/s (bf16 out) and % HBM roofline, {args.workload}",
        "value": round(outb / (avg_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32/f32",
        "data": "synthetic",
        "config": {
            "workload": f"{what}; {args.codec} codec, {Z // 1024} Ki-symbol chunks, 64 lanes, K={args.lane_run}, bf16 out"
                        + ("" if args.bits is None else f"; codes drawn at {args.bits:g} bits per weight")
                        + f"; {len(blocks)} HBM-resident copies of the containers, one per launch in turn",
            "copies": len(blocks),
            "codec": args.codec,
            "chunk_symbols": Z,
            "weights": n,
            "container_bytes": total_container,
            "effective_bits_per_weight": round(8.0 * total_container / n, 4),
            "algorithmic_bytes_per_launch": algo,
            "parallelism": "1 GPU",
        },
        "kernel_ms": {"mean": round(avg_ms, 4), "median": round(float(np.median(ms)), 4),
                      "min": round(float(np.min(ms)), 4), "all": [round(x, 4) for x in ms]},
        "compressed_read_GBps": round(comp / (avg_ms * 1e-3) / 1e9, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        "clock_settle": settle,
        "decode_only_u8": {"kernel_ms": round(u8_ms, 4),
                           "frac": round((comp + n) / (u8_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                           "note": "eq_decode_block over the same copies (u8 codes out, n bytes written), "
                                   "timed right after the bf16 launches"},
        "warm_llc": {"kernel_ms": round(warm_ms, 4),
                     "frac": round(algo / (warm_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "note": "one copy decoded again and again: its containers stay in the 256 MB last-level "
                             "cache, so the compressed reads do not reach HBM"},
    }
    if not args.no_copy_ceiling:
        cc, rc, wc = copy_ceiling(algo)
        rec["copy_ceiling_GBps"] = round(cc, 1)
        rec["read_ceiling_GBps"] = round(rc, 1)
        rec["write_ceiling_GBps"] = round(wc, 1)
        rec["frac_of_copy_ceiling"] = round(achieved / cc, 4)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(conts, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def decode_only_ms(rot, n: int, stream, steps: int) -> float:
    """Mean kernel time of eq_decode_block (u8 codes out), `steps` launches
    back to back over the rotation's blocks, right after the bf16 timing."""
    import numpy as np
    import torch
    from rans_decode_amd import eq
    sym = torch.empty(n, dtype=torch.uint8, device="cuda")
    eq.eq_decode_block(rot.next(), sym, stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s, e in evs:
        s.record(stream)
        eq.eq_decode_block(rot.next(), sym, stream)
        e.record(stream)
    torch.cuda.synchronize()
    del sym
    return float(np.mean([s.elapsed_time(e) for s, e in evs]))


def replicas(conts, min_bytes: float = 600e6, min_copies: int = 8, max_copies: int = 4096):
    """Distinct device copies of a block's containers (the first is the
    original). A step decodes the next copy in turn, so no launch finds its
    containers in the 256 MB last-level cache: the copies between two visits
    of one copy hold at least min_bytes. A model's forward pass decodes each
    block once, from HBM, the same way."""
    import math
    from rans_decode_amd import eq
    size = sum(c.nbytes for c in conts)
    n = max(min_copies, min(max_copies, math.ceil(min_bytes / max(1, size)) + 1))
    out = [list(conts)]
    for _ in range(n - 1):
        cc = []
        for c in conts:
            d = eq.DeviceContainer.__new__(eq.DeviceContainer)
            d.__dict__.update(c.__dict__)
            d.dev = c.dev.clone()
            cc.append(d)
        out.append(cc)
    return out


class Rotation:
    """Hands out the replicas' blocks in turn."""

    def __init__(self, blocks):
        self.blocks, self.i = blocks, 0

    def next(self):
        b = self.blocks[self.i % len(self.blocks)]
        self.i += 1
        return b


def clock_settle(launch, stream, ms: float) -> dict:
    """Back-to-back launches of the measured call for at least `ms` of GPU
    time before the warm-up steps, untimed: an idle MI355X sits at ~160 MHz
    and its clocks take tens of milliseconds of load to settle, longer than a
    few warm-up launches of this kernel. Returns what ran (for the record)."""
    import torch
    if ms <= 0:
        return {"launches": 0, "ms": 0.0}
    n, total = 0, 0.0
    while total < ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(10):
            launch()
        b.record(stream)
        b.synchronize()
        total += a.elapsed_time(b)
        n += 10
    return {"launches": n, "ms": round(total, 1)}


def gemv_bound(w_bf16, x_bf16):
    """2 * cols * 2^-23 * sum_c |W[r, c] x[c]| per row: twice the fp32
    summation bound, since both compared results carry one."""
    import torch
    a = w_bf16.float().abs() @ x_bf16.float().abs()
    return 2.0 * w_bf16.shape[1] * 2.0**-23 * a


def bench_gemv(args):
    """Fused decode + batch-1 GEMV of the 70B-shaped block (whole-row
    chunks), one eq_decode_gemv_bf16 call per step over the 7 tensors, each
    step on the next HBM-resident copy of the containers; next to it the
    unfused path (decode to bf16, then 7 GEMVs), the GEMVs alone over the
    bf16 weights, and the fused call repeated on one copy (warm_llc_ms)."""
    import numpy as np
    import torch
    import synth
    from rans_decode_amd import eq

    t0 = time.perf_counter()
    specs, conts = build_block(4, 0, args.lane_run, whole_rows=True,
                               chunk=args.chunk or synth.GEMV_CHUNK_TARGET)
    offs = synth.block_offsets(specs)
    n = offs[-1]
    log(f"block built in {time.perf_counter() - t0:.1f} s (whole-row chunks)")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    blocks = [eq.Block(cc, offs[:-1], status) for cc in replicas(conts)]
    block = blocks[0]
    rot = Rotation(blocks)
    xs = [torch.from_numpy(synth.gemv_activation(4, 0, i, sp.cols)).to(torch.bfloat16).cuda()
          for i, sp in enumerate(specs)]
    ys = [torch.empty(sp.rows, dtype=torch.float32, device="cuda") for sp in specs]
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        eq.eq_decode_gemv_bf16(block, xs, ys, stream)
    torch.cuda.synchronize()
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())}")
    bad = sampled_symbols_check(4, 0, specs, conts)
    if bad:
        raise RuntimeError("decoded symbols differ from the encoded ones")

    # the unfused path on the same containers, and the product check
    buf = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    y_ref = [torch.empty_like(y) for y in ys]

    def unfused(gemv_only=False, b=None):
        if not gemv_only:
            eq.eq_decode_dequant_bf16(b or rot.next(), buf, stream)
        for i, (sp, o) in enumerate(zip(specs, offs)):
            eq.eq_gemv_bf16(buf.view(torch.int16), sp.rows, sp.cols, xs[i].view(torch.int16), y_ref[i],
                            stream, w_offset_elems=o)

    unfused(b=block)
    torch.cuda.synchronize()
    worst = 0.0
    for i, (sp, o) in enumerate(zip(specs, offs)):
        w = buf[o:o + sp.n].view(sp.rows, sp.cols)
        tol = gemv_bound(w, xs[i])
        ratio = float(((ys[i] - y_ref[i]).abs() / tol.clamp_min(1e-30)).max())
        worst = max(worst, ratio)
        del w, tol
    if worst > 1.0:
        raise RuntimeError(f"fused GEMV differs from decode + GEMV beyond the fp32 bound ({worst:.3f})")
    log(f"fused vs unfused outputs: worst |diff| / bound = {worst:.4f}")

    def timed(fn):
        ms = []
        for _ in range(args.steps):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            fn()
            e.record(stream)
            torch.cuda.synchronize()
            ms.append(s.elapsed_time(e))
        return ms

    settle = clock_settle(lambda: eq.eq_decode_gemv_bf16(rot.next(), xs, ys, stream), stream, args.settle_ms)
    for _ in range(args.warmup):  # warm-up right before the timed launches
        eq.eq_decode_gemv_bf16(rot.next(), xs, ys, stream)
    wall0 = time.perf_counter()
    fused_ms = timed(lambda: eq.eq_decode_gemv_bf16(rot.next(), xs, ys, stream))
    wall = time.perf_counter() - wall0
    warm_ms = timed(lambda: eq.eq_decode_gemv_bf16(block, xs, ys, stream))
    unfused_ms = timed(unfused)
    gemv_ms = timed(lambda: unfused(gemv_only=True))
    if int(status.item()) != 0:
        raise RuntimeError(f"device status {int(status.item())}")
    f = float(np.mean(fused_ms))
    comp, _ = algorithmic_bytes(conts)
    xy = sum(2 * sp.cols + 4 * sp.rows for sp in specs)
    valu = counter_record("decode_gemv70b_counters.txt", "valu_wave_instructions_per_launch",
                          os.path.join(ROOT, "rans_decode_amd", "csrc", "decode.hip"))
    roof = {"bound": "alu", "achieved": None, "peak": VALU_PEAK_GINST, "unit": "Ginst/s",
            "frac": None, "traffic": None,
            "hbm_GBps": round((comp + xy) / (f * 1e-3) / 1e9, 1),
            "hbm_frac": round((comp + xy) / (f * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    if valu:
        ach = valu / (f * 1e-3) / 1e9
        roof.update(achieved=round(ach, 2), frac=round(ach / VALU_PEAK_GINST, 4))
    rec = {
        "metric": "fused decode + batch-1 GEMV of the 70B-shaped block (weights never written)",
        "value": round(f, 4), "unit": "ms/block", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "u32/f32",
        "data": "synthetic",
        "config": {"workload": "70B-shaped block (q,o 8192x8192; k,v 1024x8192; gate,up 28672x8192; "
                               "down 8192x28672; int8 2.1-bit codes, 4 super weights) with whole-row "
                               f"chunks, K={args.lane_run}; x ~ N(0,1) in bf16, y fp32",
                   "weights": n, "chunk_symbols": [int(c.hdr.chunk_symbols) for c in conts],
                   "copies": len(blocks), "parallelism": "1 GPU"},
        "kernel_ms": {"mean": round(f, 4), "median": round(float(np.median(fused_ms)), 4),
                      "min": round(float(np.min(fused_ms)), 4)},
        "weights_per_s_G": round(n / (f * 1e-3) / 1e9, 1),
        "unfused_decode_then_gemv_ms": round(float(np.mean(unfused_ms)), 4),
        "bf16_resident_gemv_ms": round(float(np.mean(gemv_ms)), 4),
        "speedup_vs_unfused": round(float(np.mean(unfused_ms)) / f, 3),
        "ratio_vs_bf16_resident": round(f / float(np.mean(gemv_ms)), 3),
        "roofline": roof,
        "fused_vs_unfused_worst_over_bound": round(worst, 5),
        "clock_settle": settle,
        "warm_llc_ms": round(float(np.mean(warm_ms)), 4),
    }
    print(json.dumps(rec), flush=True)


def bench_encode(args):
    """Device-side encode (eq_encode_device) of the 70B-shaped block's seven
    tensors, symbols and scales already in HBM; each container is checked
    byte-for-byte against the host encoder's. Next to it: the host encoder
    (eq_encode_host, all host cores) on the same tensors."""
    import numpy as np
    import torch
    import synth
    from rans_decode_amd import eq

    codec = CODECS[args.codec]
    specs = synth.config_specs(4)
    Z4 = args.chunk or synth.config_chunk(4)
    tensors = []
    t0 = time.perf_counter()
    for i, sp in enumerate(specs):
        t = synth.make_tensor(4, 0, i)
        esc = t.esc_idx.size > 0
        tensors.append(dict(
            spec=sp, sym=torch.from_numpy(t.symbols).cuda(), sc=torch.from_numpy(t.scales).cuda(),
            ei=torch.from_numpy(t.esc_idx.astype(np.int64)).cuda() if esc else None,
            ev=torch.from_numpy(t.esc_val.view(np.int16)).cuda() if esc else None,
            code=t.esc_code if esc else 0))
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    # one workspace per tensor: the seven calls can run on seven streams
    wss = [torch.empty(int(eq._lib.eq_encode_device_workspace(sp.rows, sp.cols, Z4)),
                       dtype=torch.uint8, device="cuda") for sp in specs]
    streams = [torch.cuda.Stream() for _ in specs]  # default priority
    outs = [torch.empty(int(eq._lib.eq_encode_device_bound(sp.rows, sp.cols, Z4, sp.n_esc)),
                        dtype=torch.uint8, device="cuda") for sp in specs]
    stream = torch.cuda.current_stream()
    # per-tensor length words and status flags, allocated once (flags of all
    # passes accumulate; any flag fails the run)
    lens = [torch.zeros(1, dtype=torch.int64, device="cuda") for _ in specs]
    stats = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in specs]

    def block(concurrent=False):
        # one stream, or each call on its own stream (joined back to `stream`)
        if concurrent:
            for st_ in streams:
                st_.wait_stream(stream)
        for d, o, ln, st, w, st_ in zip(tensors, outs, lens, stats, wss, streams):
            sp = d["spec"]
            eq.eq_encode_device(sp.dtype, sp.rows, sp.cols, d["sym"], d["sc"], d["ei"], d["ev"],
                                d["code"], Z4, args.lane_run, workspace=w,
                                out=o, stream=st_ if concurrent else stream, d_len=ln, d_status=st,
                                codec=codec)
        if concurrent:
            for st_ in streams:
                stream.wait_stream(st_)

    for _ in range(args.warmup):
        block()
    torch.cuda.synchronize()
    if any(int(st.item()) for st in stats):
        raise RuntimeError("device encode flagged its input")
    # byte-for-byte against the host encoder (its containers, built or cached)
    _, host = build_block(4, 0, args.lane_run, codec=codec, chunk=Z4)
    for i, (c, o, ln) in enumerate(zip(host, outs, lens)):
        got = o[:int(ln.item())].cpu().numpy()
        if got.size != c.host.size or not np.array_equal(got, c.host):
            raise RuntimeError(f"tensor {i}: device container differs from the host encoder's")
    log("device containers byte-identical to the host encoder's")
    def timed(concurrent):
        for _ in range(args.warmup):  # warm-up right before the timed passes
            block(concurrent)
        out_ms = []
        for _ in range(args.steps):
            s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            block(concurrent)
            e0.record(stream)
            torch.cuda.synchronize()
            out_ms.append(s0.elapsed_time(e0))
        return out_ms

    seq_ms = timed(False)
    ms = timed(True)
    # the concurrent passes' containers are the same bytes
    for i, (c, o, ln) in enumerate(zip(host, outs, lens)):
        if not np.array_equal(o[:int(ln.item())].cpu().numpy(), c.host):
            raise RuntimeError(f"tensor {i}: container differs after the concurrent passes")
    if any(int(st.item()) for st in stats):
        raise RuntimeError("device encode flagged its input")
    # the host encoder (eq_build_tables + eq_encode_host, all host cores) on
    # the same tensors, one pass
    host_enc_s = 0.0
    for i, sp in enumerate(specs):
        t = synth.make_tensor(4, 0, i)
        esc = t.esc_idx.size > 0
        t_enc0 = time.perf_counter()
        tab = eq.build_tables(t.symbols)
        eq.encode_host(tab, sp.dtype, sp.rows, sp.cols, t.symbols, t.scales, t.esc_idx if esc else None,
                       t.esc_val if esc else None, esc_code=t.esc_code if esc else 0,
                       chunk_symbols=Z4, lane_run=args.lane_run, codec=codec)
        host_enc_s += time.perf_counter() - t_enc0
        del t
    n = sum(sp.n for sp in specs)
    f = float(np.mean(ms))
    # algorithmic bytes of a static-table encoder: the symbols are read twice
    # (histogram, then encode) and the containers written once
    cont_bytes = sum(int(ln.item()) for ln in lens)
    algo = 2 * n + cont_bytes
    rec = {
        "metric": "device-side encode of the 70B-shaped block (histogram, quantiser, rANS encode, container)"
                  if codec == 0 else
                  "device-side encode of the 70B-shaped block (histogram, Huffman code, encode, container)",
        "value": round(n / (f * 1e-3) / 1e9, 2), "unit": "G symbols/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(f, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": "70B-shaped block, 855,638,016 int8 codes (2.1-bit Laplace), 4 super weights, "
                               f"{Z4 // 1024} Ki chunks, K={args.lane_run}; {args.codec} codec; one eq_encode_device call per "
                               "tensor, the seven on seven HIP streams",
                   "weights": n},
        "kernel_ms": {"mean": round(f, 4), "median": round(float(np.median(ms)), 4),
                      "min": round(float(np.min(ms)), 4)},
        "one_stream_ms": round(float(np.mean(seq_ms)), 4),
        "host_encoder_s": round(host_enc_s, 3),
        "host_encoder_G_symbols_per_s": round(n / host_enc_s / 1e9, 3),
        "host_cores": host_cores(),
        "speedup_vs_host_encoder": round(host_enc_s * 1e3 / f, 1),
        "roofline": {"bound": "hbm", "scope": "all launches of the seven calls",
                     "achieved": round(algo / (f * 1e-3) / 1e9, 2), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(algo / (f * 1e-3) / 1e9 / 8000.0, 4), "traffic": None,
                     "algorithmic_bytes": algo},
    }
    print(json.dumps(rec), flush=True)


def bench_drift(args):
    """Adaptive tables: one 28672 x 8192 int8 tensor whose rows come in 16
    bands of different entropy (0.8 / 2.1 / 3.2 / 1.4 bits, repeating),
    encoded with one table and with one table per 8 chunks; container size
    and decode + dequant time of each."""
    import numpy as np
    import torch
    import synth
    from rans_decode_amd import eq

    t = synth.drift_tensor(28672, 8192, bands=16)
    n = t.spec.n
    res = {}
    for name, seg in (("one_table", 0), ("per_8_chunks", 8)):
        blob = eq.encode_host(eq.build_tables(t.symbols) if not seg else None, t.spec.dtype, t.spec.rows,
                              t.spec.cols, t.symbols, t.scales, chunk_symbols=synth.CHUNK_SYMBOLS,
                              lane_run=args.lane_run, seg_chunks=seg)
        c = eq.DeviceContainer(blob, device="cuda")
        out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        blk = eq.Block([c], None, status)
        rot = Rotation([eq.Block(cc, None, status) for cc in replicas([c])])
        for _ in range(args.warmup):
            eq.eq_decode_dequant_bf16(rot.next(), out)
        torch.cuda.synchronize()
        ms = []
        for _ in range(args.steps):
            s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record()
            eq.eq_decode_dequant_bf16(rot.next(), out)
            e0.record()
            torch.cuda.synchronize()
            ms.append(s0.elapsed_time(e0))
        if int(status.item()):
            raise RuntimeError(f"device status {int(status.item())}")
        sym = torch.empty(n, dtype=torch.uint8, device="cuda")
        eq.eq_decode_block(blk, sym)
        torch.cuda.synchronize()
        if not np.array_equal(sym.cpu().numpy(), t.symbols):
            raise RuntimeError("decoded symbols differ from the encoded ones")
        f = float(np.mean(ms))
        # the same container from the device encoder: byte-identical, and its time
        dsym = torch.from_numpy(t.symbols).cuda()
        dsc = torch.from_numpy(t.scales).cuda()
        ws = torch.empty(int(eq._lib.eq_encode_device_workspace(t.spec.rows, t.spec.cols, synth.CHUNK_SYMBOLS)),
                         dtype=torch.uint8, device="cuda")
        dout = torch.empty(int(eq._lib.eq_encode_device_bound(t.spec.rows, t.spec.cols, synth.CHUNK_SYMBOLS, 0)),
                           dtype=torch.uint8, device="cuda")
        enc = lambda: eq.eq_encode_device(t.spec.dtype, t.spec.rows, t.spec.cols, dsym, dsc,  # noqa: E731
                                          chunk_symbols=synth.CHUNK_SYMBOLS, lane_run=args.lane_run,
                                          workspace=ws, out=dout, seg_chunks=seg)
        _, dlen, dst = enc()
        torch.cuda.synchronize()
        if int(dst.item()) or not np.array_equal(dout[:int(dlen.item())].cpu().numpy(), blob):
            raise RuntimeError("device encoder's container differs from the host encoder's")
        for _ in range(args.warmup):
            enc()
        ems = []
        for _ in range(args.steps):
            s0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record()
            enc()
            e0.record()
            torch.cuda.synchronize()
            ems.append(s0.elapsed_time(e0))
        res[name] = {"container_bytes": int(blob.size), "bits_per_weight": round(8.0 * blob.size / n, 4),
                     "kernel_ms": round(f, 4), "bf16_GBps": round(2 * n / (f * 1e-3) / 1e9, 1),
                     "device_encode_ms": round(float(np.mean(ems)), 4)}
        del c, out, sym, dsym, dsc, ws, dout, rot
    rec = {
        "metric": "adaptive (per-segment) frequency tables vs one table on a tensor with drifting statistics",
        "value": round(res["one_table"]["container_bytes"] / res["per_8_chunks"]["container_bytes"], 4),
        "unit": "size ratio (one table / per-segment)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["per_8_chunks"]["kernel_ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u32/f32", "data": "synthetic",
        "config": {"workload": "28672 x 8192 int8, 16 row bands of 0.8/2.1/3.2/1.4-bit discrete Laplace, "
                               f"64 Ki chunks, K={args.lane_run}",
                   "empirical_entropy_bits": round(synth.empirical_entropy(t.symbols), 4)},
        "one_table": res["one_table"], "per_8_chunks": res["per_8_chunks"],
    }
    print(json.dumps(rec), flush=True)


def bench_model(args):
    """80 blocks of the 70B-shaped layer, resident as containers (about 18 GB);
    each token pass decodes block b into bf16 buffer b % 2 on one stream and
    runs its seven batch-1 GEMVs on the other (eq_pipeline; timed in the
    alternating mode, where the decode of block b + 1 follows the GEMVs of
    block b, and in the overlapped mode, where it runs beside them).
    Also timed: the 80 decodes alone (sustained decode rate) and the 80 x 7
    GEMVs over all blocks resident in bf16 (137 GB), the uncompressed
    baseline the pages compare with."""
    import numpy as np
    import torch
    import synth
    from rans_decode_amd import eq

    L = args.layers
    specs = synth.config_specs(5)
    offs = synth.block_offsets(specs)
    nblk = offs[-1]
    t0 = time.perf_counter()
    blocks, xs, ys = [], [], []
    comp_bytes = 0
    Z = args.chunk or synth.config_chunk(5)
    enc = DeviceEncoder(specs, Z, args.lane_run)
    for layer in range(L):
        conts = [enc.container(5, layer, i, sp) for i, sp in enumerate(specs)]
        comp_bytes += algorithmic_bytes(conts)[0]
        for c in conts:
            c.host = None  # the header is parsed; the bytes stay on the device
        blocks.append(eq.Block(conts, offs[:-1], None))
        xs.append([torch.from_numpy(synth.gemv_activation(5, layer, i, sp.cols)).to(torch.bfloat16).cuda()
                   for i, sp in enumerate(specs)])
        ys.append([torch.empty(sp.rows, dtype=torch.float32, device="cuda") for sp in specs])
        if layer % 8 == 7 or layer == L - 1:
            log(f"built {layer + 1}/{L} blocks in {time.perf_counter() - t0:.0f} s")
    resident_bytes = sum(c.nbytes for b in blocks for c in b.containers)
    bufs = [torch.empty(nblk, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ds, gs = torch.cuda.Stream(), torch.cuda.Stream()
    pipe = eq.Pipeline(L)

    def token():
        pipe.run(blocks, bufs[0], bufs[1], xs, ys, ds, gs)

    for _ in range(args.warmup):
        token()
    torch.cuda.synchronize()
    tok_ms = []
    for _ in range(args.steps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(ds)
        token()
        gs.wait_stream(ds)
        e.record(gs)
        torch.cuda.synchronize()
        tok_ms.append(s.elapsed_time(e))
    y_pipe = [[y.clone() for y in yl] for yl in ys]

    # the same schedule with each decode beside the previous block's GEMVs
    pipe.set_mode(eq.EQ_PIPELINE_OVERLAP)
    token()
    torch.cuda.synchronize()
    ovl_ms = []
    for _ in range(args.steps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(ds)
        token()
        gs.wait_stream(ds)
        e.record(gs)
        torch.cuda.synchronize()
        ovl_ms.append(s.elapsed_time(e))
    same_ovl = all(torch.equal(a.view(torch.int32), b.view(torch.int32))
                   for al, bl in zip(y_pipe, ys) for a, b in zip(al, bl))
    if not same_ovl:
        raise RuntimeError("the overlapped schedule's GEMV outputs differ from the alternating one's")
    pipe.set_mode(eq.EQ_PIPELINE_ALTERNATE)

    # decodes alone, back to back on one stream
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(ds)
    for b in range(L):
        eq.eq_decode_dequant_bf16(blocks[b], bufs[b & 1], ds)
    e.record(ds)
    torch.cuda.synchronize()
    dec_ms = s.elapsed_time(e)

    # every block resident in bf16, then the GEMVs alone
    resident = torch.empty(L * nblk, dtype=torch.bfloat16, device="cuda")
    for b in range(L):
        eq.eq_decode_dequant_bf16(blocks[b], resident[b * nblk:(b + 1) * nblk], ds)
    torch.cuda.synchronize()
    y_res = [[torch.empty_like(y) for y in yl] for yl in ys]

    def gemvs():
        for b in range(L):
            for i, (sp, o) in enumerate(zip(specs, offs)):
                eq.eq_gemv_bf16(resident.view(torch.int16), sp.rows, sp.cols, xs[b][i].view(torch.int16),
                                y_res[b][i], gs, w_offset_elems=b * nblk + o)

    gemvs()
    torch.cuda.synchronize()
    res_ms = []
    for _ in range(args.steps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(gs)
        gemvs()
        e.record(gs)
        torch.cuda.synchronize()
        res_ms.append(s.elapsed_time(e))
    same = all(torch.equal(a.view(torch.int32), b.view(torch.int32))
               for al, bl in zip(y_pipe, y_res) for a, b in zip(al, bl))
    if not same:
        raise RuntimeError("pipeline GEMV outputs differ from the bf16-resident GEMVs")
    bad = 0
    for b in range(0, L, max(1, L // 8)):
        bad += sampled_symbols_check(5, b, specs, blocks[b].containers, rng_seed=b)
    if bad:
        raise RuntimeError(f"sampled decode check: {bad} mismatching codes")
    log(f"pipeline GEMV outputs identical to resident GEMVs; sampled decode check 0 mismatches")

    # fused decode + GEMV per token (one stream): the block re-encoded with
    # chunks of whole rows near synth.GEMV_CHUNK_TARGET symbols (shared where
    # the decode's containers already are such chunks)
    t1 = time.perf_counter()
    fblocks = []
    zf = [whole_row_chunk(sp.cols, args.lane_run, synth.GEMV_CHUNK_TARGET) for sp in specs]
    for layer in range(L):
        fc = []
        for i, sp in enumerate(specs):
            if zf[i] == int(blocks[layer].containers[i].hdr.chunk_symbols):
                fc.append(blocks[layer].containers[i])
            else:
                c = enc.container(5, layer, i, sp, Z=zf[i])
                c.host = None
                fc.append(c)
        fblocks.append(eq.Block(fc, offs[:-1], None))
    log(f"whole-row containers for the fused path built in {time.perf_counter() - t1:.0f} s")
    yf = [[torch.empty_like(y) for y in yl] for yl in ys]

    def fused_token():
        for b in range(L):
            eq.eq_decode_gemv_bf16(fblocks[b], xs[b], yf[b], ds)

    fused_token()
    torch.cuda.synchronize()
    worst = 0.0
    for b in sorted({0, L // 2, L - 1}):
        for i, (sp, o) in enumerate(zip(specs, offs)):
            w = resident[b * nblk + o:b * nblk + o + sp.n].view(sp.rows, sp.cols)
            tol = gemv_bound(w, xs[b][i])
            worst = max(worst, float(((yf[b][i] - y_res[b][i]).abs() / tol.clamp_min(1e-30)).max()))
            del w, tol
    if worst > 1.0:
        raise RuntimeError(f"fused GEMV differs from the resident GEMV beyond the fp32 bound ({worst:.3f})")
    fused_ms = []
    for _ in range(args.steps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(ds)
        fused_token()
        e.record(ds)
        torch.cuda.synchronize()
        fused_ms.append(s.elapsed_time(e))
    fus = float(np.median(fused_ms))
    tok = float(np.median(tok_ms))
    res = float(np.median(res_ms))
    dec_bytes = 2 * nblk * L
    rec = {
        "metric": "per-token time of the 80-block decode + batch-1 GEMV schedule (bf16 weights decoded per token)",
        "value": round(tok, 3), "unit": "ms/token", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(tok, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "u32/f32", "data": "synthetic",
        "config": {"workload": f"{L} x 70B-shaped block (int8 2.1-bit, K={args.lane_run}) resident as "
                               "containers; double-buffered decode on one HIP stream, 7 bf16 GEMVs per "
                               "block (batch 1, N(0,1) activations) on another, the streams taking turns "
                               "(eq_pipeline's alternating mode)",
                   "layers": L, "resident_container_bytes": resident_bytes,
                   "resident_GiB": round(resident_bytes / 2 ** 30, 3),
                   "effective_bits_per_weight": round(8.0 * resident_bytes / (nblk * L), 4)},
        "sustained_decode_GBps": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
        "decode_only_ms_per_token": round(dec_ms, 3),
        "bf16_resident_gemv_ms_per_token": round(res, 3),
        "slowdown_vs_bf16_resident": round(tok / res, 3),
        "token_ms_all": [round(x, 3) for x in tok_ms],
        "overlapped_mode_ms_per_token": round(float(np.median(ovl_ms)), 3),
        "fused_decode_gemv_ms_per_token": round(fus, 3),
        "fused_ratio_vs_bf16_resident": round(fus / res, 3),
        "fused_speedup_vs_pipeline": round(tok / fus, 3),
        "fused_vs_resident_worst_over_bound": round(worst, 5),
    }
    print(json.dumps(rec), flush=True)
    pipe.close()


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=["block70b", "model80", "gemv70b", "encode70b", "drift", "cfg1",
                                           "cfg2", "cfg3"],
                    default="block70b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ceiling", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="block workloads: untimed back-to-back launches for this much GPU time before "
                         "the warm-up steps, so the timing starts at settled clocks (0: none)")
    ap.add_argument("--bits", type=float, default=None,
                    help="block workloads: entropy of the synthetic codes in bits per weight "
                         "(default: the configuration's)")
    ap.add_argument("--layers", type=int, default=80, help="blocks in the model80 workload")
    ap.add_argument("--chunk", type=int, default=None,
                    help="symbols per chunk of the encoded containers (default: the configuration's; "
                         "whole-row containers take the nearest multiple of the row length)")
    ap.add_argument("--codec", choices=sorted(CODECS), default="rans",
                    help="entropy coder of the block workloads' containers (rANS: EntQuant's ANS; "
                         "huffman: EntroLLM's coder, for comparison)")
    ap.add_argument("--lane-run", type=int, default=8, choices=[1, 2, 4, 8, 16],
                    help="container lane run K of the encoded block (workload parameter)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this decoder has no multi-GPU path "
              "(chunks are independent; a sharded model decodes each GPU's shard alone). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload == "model80":
        bench_model(args)
    elif args.workload == "gemv70b":
        bench_gemv(args)
    elif args.workload == "encode70b":
        bench_encode(args)
    elif args.workload == "drift":
        bench_drift(args)
    else:
        bench_block(args)


if __name__ == "__main__":
    main()
