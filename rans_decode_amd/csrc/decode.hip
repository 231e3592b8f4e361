// decode.hip -- gfx950 (CDNA4, wave64) kernels of libeq and their launchers.
//
// What runs here is the inference-time half of EntQuant ("Float8@2bits:
// Entropy Coding Enables Data-Free Model Compression", technical summary,
// section 2): the ANS-compressed weights stay in GPU memory and, just before a
// transformer block runs, a parallel ANS decoder expands them into a buffer
// (technical component 3), multiplying by the per-channel scales S
// (technical component 1) and restoring the super weights kept out of the
// coded stream (technical component 4). Chunks are independent, as in
// EntroLLM's parallel decoding ("EntroLLM: Entropy Encoded Weight Compression
// for Efficient Large Language Model Inference on Edge Devices", technical
// overview, method item 3).
//
// Mapping to the hardware:
//  * one wave64 decodes one chunk; its 64 lanes are the container's 64
//    interleaved rANS states, so a decode step is one instruction stream with
//    no divergence;
//  * a workgroup of 8 waves decodes 8 chunks of one tensor and shares one
//    4096-entry slot table in LDS (8 bytes per entry: frequency | symbol
//    byte << 24, slot - cumulative frequency), built by a running maximum of
//    the symbols' start marks;
//  * renormalisation words are read in the container's order with a wave
//    ballot of the lanes that need a word plus a masked popcount (mbcnt) of
//    the lanes below, from a per-wave LDS ring that is refilled 1 KiB at a
//    time with 16-byte coalesced loads;
//  * after K steps each lane holds K consecutive outputs: the fp32 scale
//    multiply, the RNE bf16 conversion (v_cvt_pk_bf16_f32) and one 16-byte
//    non-temporal store per lane (K = 8), i.e. a 1 KiB contiguous store per
//    wave; the fused GEMV variant dots them with x instead (v_dot2c).
//  * Huffman-coded tensors (EntroLLM's codec) share everything but the table
//    build and the step.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/eq.h"
#include "format.hpp"

namespace {

// Tunables (compile-time): chunks (waves) per workgroup and the per-wave
// ring of renormalisation words in LDS.
#ifndef EQ_WAVES
#define EQ_WAVES 8
#endif
#ifndef EQ_RING_WORDS
#define EQ_RING_WORDS 1024
#endif
#ifndef EQ_RENORM_BRANCHLESS
#define EQ_RENORM_BRANCHLESS 1
#endif
#ifndef EQ_SADDR_STORE
#define EQ_SADDR_STORE 1  // K = 8 bf16 stores with a scalar base address
#endif
#ifndef EQ_RENORM_EXEC
#define EQ_RENORM_EXEC 1
#endif
#ifndef EQ_NT_STORES
#define EQ_NT_STORES 1
#endif
#if EQ_NT_STORES
// non-temporal, system scope: with the compressed reads coming from HBM this
// is 2.5% faster than non-temporal alone (0.389 vs 0.399 ms on the 70B block)
#define EQ_NT_SUFFIX " nt sc1"
#else
#define EQ_NT_SUFFIX ""
#endif
constexpr int kWaves = EQ_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr uint32_t kRing = EQ_RING_WORDS;       // power of two
constexpr uint32_t kBlk = kRing / 2;            // words per refill
constexpr uint32_t kLaneWords = kBlk / 64;      // words each lane loads per refill
constexpr uint32_t kCheck = kBlk / 64;          // steps between refill checks
constexpr uint32_t kRingAlloc = kRing + 64;     // + copy of the ring's first 64 words
static_assert(kRing == 2048 || kRing == 1024 || kRing == 512 || kRing == 256,
              "ring of 256 to 2048 words");

// Output modes of a tensor (host-chosen).
enum : uint32_t {
    M_GENERAL = 0,  // any shape / alignment: per-element scale and stores
    M_ROW1 = 1,     // every 64K group lies in one row (bf16), or aligned u8 stores
    M_ROW2 = 2,     // a 64K group spans at most two rows (bf16)
};

struct TArgs {
    const uint8_t *base;  // container (device)
    uint64_t out_offset, n, cols, rows, n_chunks, n_words, n_esc;
    uint64_t off_scales, off_dir, off_states, off_words, off_esc_idx, off_esc_val, off_freq;
    uint32_t Z, dtype, mode, const_sym;
    uint32_t is_const, wg_begin;
    uint32_t codec;       // entropy coder: eqfmt::kCodecRans or kCodecHuffman
    uint32_t seg;         // adaptive tables: chunks per table (a multiple of kWaves), 0 = one table
    const uint16_t *x;  // fused GEMV: the tensor's bf16 input vector [cols]
    float *y;           // fused GEMV: its fp32 output [rows]
};

struct LArgs {
    TArgs t[EQ_MAX_BLOCK_TENSORS];
    void *out;
    uint32_t *status;
    uint32_t n_tensors;
    uint32_t pad;
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even, gradual underflow), packed.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    floatx2 f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// acc + w.lo * x.lo + w.hi * x.hi for two packed bf16 pairs (fp32 result).
__device__ __forceinline__ float dot2_bf16(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, x),
                                           acc, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes (all active), fixed order: quad butterflies, half-row
// and row mirrors (DPP), then the four row sums in lane order. Every lane
// gets the same value.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);  // row_half_mirror
    v += dpp_f<0x140>(v);  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return ((r0 + r1) + r2) + r3;
}

// A lane's K consecutive bf16 inputs of the fused GEMV, as packed pairs.
template <int K> struct XRun { uint32_t p[(K + 1) / 2]; };
template <int K>
__device__ __forceinline__ XRun<K> load_x(const uint16_t *x) {
    XRun<K> r;
    if constexpr (K == 1) {
        r.p[0] = *x;
    } else if constexpr (K == 2) {
        r.p[0] = *reinterpret_cast<const uint32_t *>(x);
    } else if constexpr (K == 4) {
        const uint2 v = *reinterpret_cast<const uint2 *>(x);
        r.p[0] = v.x; r.p[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < K / 8; ++i) {
            const uint4 v = reinterpret_cast<const uint4 *>(x)[i];
            r.p[4 * i] = v.x; r.p[4 * i + 1] = v.y; r.p[4 * i + 2] = v.z; r.p[4 * i + 3] = v.w;
        }
    }
    return r;
}

// The same K inputs through a buffer resource over the input vector: the
// lane's constant byte offset in a VGPR and the group's wave-uniform byte
// offset in an SGPR (no per-group VALU address work); bytes past the
// resource's end read as zero.
constexpr int kRawBufferWord3 = 0x00020000;  // raw (untyped) buffer, 32-bit data format
template <int K>
__device__ __forceinline__ XRun<K> load_x_buffer(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    XRun<K> r;
    if constexpr (K == 1) {
        r.p[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)voff, (int)soff, 0);
    } else if constexpr (K == 2) {
        r.p[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)voff, (int)soff, 0);
    } else if constexpr (K == 4) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)voff, (int)soff, 0);
        r.p[0] = v.x; r.p[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < K / 8; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(voff + 16u * i), (int)soff, 0);
            r.p[4 * i] = v.x; r.p[4 * i + 1] = v.y; r.p[4 * i + 2] = v.z; r.p[4 * i + 3] = v.w;
        }
    }
    return r;
}

// 8-byte slot-table entry: lo = f | symbol << 24, hi = slot - cum. f is at
// most 4096 (a segment of an adaptive-table container can hold one symbol),
// so it fits bits 0..12 and bits 13..23 are zero: a 24-bit multiply by lo
// sees f alone.
typedef uint2 LutEnt;
constexpr int kSymShift = 24;
__device__ __forceinline__ uint32_t ent_bits(LutEnt e) { return e.x; }
__device__ __forceinline__ LutEnt make_ent(uint32_t s, uint32_t f, uint32_t bias) {
    return make_uint2(f | (s << 24), bias);
}
__device__ __forceinline__ uint32_t ent_next(LutEnt e, uint32_t x) {
    return __umul24(e.x, x >> 12) + e.y;
}

// Value of the symbol byte held in a slot-table entry's bits kSymShift..+8.
template <uint32_t DT>
__device__ __forceinline__ float sym_value(uint32_t bits) {
    if constexpr (DT == EQ_DTYPE_INT8) {
        return (float)(int32_t)(int8_t)((bits >> kSymShift) & 0xFFu);
    } else {
        return __builtin_amdgcn_cvt_f32_fp8((int)bits, kSymShift / 8);  // OCP E4M3FN on gfx950
    }
}
__device__ __forceinline__ uint32_t sym_byte(uint32_t bits) { return (bits >> kSymShift) & 0xFFu; }

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

__device__ __forceinline__ void raise_flag(uint32_t *status, uint32_t bits, uint32_t lane) {
    if (status && bits && lane == 0) atomicOr(status, bits);
}

// Inclusive prefix sum / prefix maximum over the 64 lanes with DPP moves
// (row shifts, then the row broadcasts of lanes 15 and 31), no LDS traffic.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x) {
    auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : a + b; };
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false));  // row_shr:1
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false));  // row_shr:2
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false));  // row_shr:4
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false));  // row_shr:8
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false));  // row_bcast:15
    x = op(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false));  // row_bcast:31
    return x;
}

// Slot table of the tensor (or of one segment's table): for every slot in
// [0, 4096) the byte s with cum[s] <= slot < cum[s] + f[s], as the entry
// (f[s], s, slot - cum[s]). A one-symbol tensor never builds a table; a
// one-symbol segment does, with f = 4096 in every entry.
// Each wave fills its own 4096 / kWaves slots with no workgroup barrier: it
// computes the cumulative frequencies itself (a wave scan), every present
// byte s whose first slot cum[s] lies in the wave's range marks it with
// s + 1, and the byte of a slot is the running maximum of the marks up to it
// (present bytes have increasing cum), started from the byte that owns the
// range's first slot. wscr: the wave's own scratch (its ring, not yet in
// use). The caller's barrier publishes the table to the other waves.
constexpr uint32_t kSlotsPerWave = 4096u / kWaves;
constexpr uint32_t kSlotsPerLane = kSlotsPerWave / 64u;
static_assert(kSlotsPerLane * 64u * kWaves == 4096u && kSlotsPerLane % 8u == 0, "slots per lane");

__device__ __forceinline__ void build_lut(const uint16_t *freq, LutEnt *lut, uint32_t *wscr) {
    constexpr uint32_t P = kSlotsPerLane;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t lo = (threadIdx.x >> 6) * kSlotsPerWave;  // the wave's first slot
    uint32_t *cum = wscr;                                     // [257]
    uint16_t *mark = reinterpret_cast<uint16_t *>(wscr + 260);  // [kSlotsPerWave]
    // bytes 4 lane .. 4 lane + 3
    const uint2 fv = reinterpret_cast<const uint2 *>(freq)[lane];
    const uint32_t f[4] = {fv.x & 0xFFFFu, fv.x >> 16, fv.y & 0xFFFFu, fv.y >> 16};
    const uint32_t sum = f[0] + f[1] + f[2] + f[3];
    const uint32_t incl = wave_scan<false>(sum);
#pragma unroll
    for (uint32_t j = 0; j < P; j += 8)
        *reinterpret_cast<uint4 *>(mark + P * lane + j) = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();
    uint32_t c = incl - sum, cs[4], carry = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        cs[i] = c;
        const uint32_t sym1 = 4u * lane + (uint32_t)i + 1u;
        if (f[i]) {
            if (c >= lo && c < lo + kSlotsPerWave) mark[c - lo] = (uint16_t)sym1;
            if (c <= lo) carry = sym1;  // the latest present byte starting at or before lo
        }
        c += f[i];
    }
    *reinterpret_cast<uint4 *>(cum + 4u * lane) = make_uint4(cs[0], cs[1], cs[2], cs[3]);
    if (lane == 63u) cum[256] = incl;
    carry = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan<true>(carry), 63);
    __builtin_amdgcn_wave_barrier();
    uint32_t run[P];
    uint32_t m = 0;
#pragma unroll
    for (uint32_t j = 0; j < P; j += 8) {
        const uint4 v = *reinterpret_cast<const uint4 *>(mark + P * lane + j);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k) {
            const uint32_t mk = (w[k / 2] >> (16u * (k % 2))) & 0xFFFFu;
            m = mk > m ? mk : m;
            run[j + k] = m;
        }
    }
    // the running maximum of the lanes before this one (wave_shr:1), and the
    // byte owning the range's first slot
    uint32_t before = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)wave_scan<true>(m), 0x138, 0xF, 0xF, false);
    before = before > carry ? before : carry;
#pragma unroll
    for (uint32_t j = 0; j < P; ++j) {
        const uint32_t slot = lo + P * lane + j;
        const uint32_t sym = (run[j] > before ? run[j] : before) - 1u;
        const uint32_t c0 = cum[sym];
        lut[slot] = make_ent(sym, cum[sym + 1] - c0, slot - c0);
    }
}

// Huffman decoding table of the tensor (codec 1), 4096 four-byte entries in
// the slot-table memory: entry[v] = length | symbol << 24 of the codeword
// whose bits, first bit in bit 0, are the low `length` bits of v (the
// canonical code of the length table, codewords of at most 12 bits).
// Wave 0 ranks the symbols of each length with ballots (bytes ascending) and
// lays out the canonical tables in `scr`; then every thread resolves its
// slots by trying the lengths in order (the code is prefix-free, so the
// first match is the codeword). Slots no codeword covers (impossible for a
// complete code, which the host checks) take 12 bits and symbol 0.
__device__ __forceinline__ void build_lut_huff(const uint16_t *tab, uint32_t *lut, uint32_t *scr) {
    const uint32_t tid = threadIdx.x;
    constexpr uint32_t L = eqfmt::kHuffMaxLen;
    uint32_t *sorted = scr;            // [256] symbols in (length, byte) order
    uint32_t *first = scr + 256;       // [L + 1] first code value of each length
    uint32_t *cnt = scr + 256 + 16;    // [L + 1] codewords of each length
    uint32_t *off = scr + 256 + 32;    // [L + 1] index in sorted[] of each length's first
    if (tid < 64) {
        uint32_t len[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) len[r] = tab[64 * r + tid];
        uint32_t c[L + 1] = {}, o[L + 1] = {}, f[L + 1] = {}, run[L + 1] = {};
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (uint32_t l = 1; l <= L; ++l)
                c[l] += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(len[r] == l));
        uint32_t code = 0, at = 0;
#pragma unroll
        for (uint32_t l = 1; l <= L; ++l) {
            f[l] = code;
            o[l] = at;
            code = (code + c[l]) << 1;
            at += c[l];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (uint32_t l = 1; l <= L; ++l) {
                const uint64_t m = __builtin_amdgcn_ballot_w64(len[r] == l);
                const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                if (len[r] == l) sorted[o[l] + run[l] + below] = 64u * r + tid;
                run[l] += (uint32_t)__builtin_popcountll(m);
            }
        }
        if (tid <= L) {
            uint32_t fv = 0, cv = 0, ov = 0;
#pragma unroll
            for (uint32_t l = 0; l <= L; ++l)
                if (tid == l) { fv = f[l]; cv = c[l]; ov = o[l]; }
            first[tid] = fv;
            cnt[tid] = cv;
            off[tid] = ov;
        }
    }
    __syncthreads();
    // the per-length tables in registers (every slot tests the same ones;
    // LDS reads in a dependent loop would serialise)
    uint32_t fr[L + 1], cr[L + 1], orr[L + 1];
#pragma unroll
    for (uint32_t l = 1; l <= L; ++l) {
        fr[l] = first[l];
        cr[l] = cnt[l];
        orr[l] = off[l];
    }
    for (uint32_t v = tid; v < 4096u; v += kThreads) {
        const uint32_t rv = __builtin_bitreverse32(v);
        // the shortest length whose code range holds the low bits of v
        uint32_t len = L, idx = 0xFFFFFFFFu;  // fallback: 12 bits, symbol 0
#pragma unroll
        for (uint32_t l = L; l >= 1; --l) {
            const uint32_t i = (rv >> (32u - l)) - fr[l];  // the low l bits of v, first bit highest
            if (i < cr[l]) {
                len = l;
                idx = orr[l] + i;
            }
        }
        lut[v] = len | ((idx != 0xFFFFFFFFu ? sorted[idx] : 0u) << 24);
    }
    __syncthreads();
}

template <uint32_t LW> struct LaneBlock;
struct uint8x { uint4 a, b; };
template <> struct LaneBlock<16> { using type = uint8x; };
template <> struct LaneBlock<8> { using type = uint4; };
template <> struct LaneBlock<4> { using type = uint2; };
template <> struct LaneBlock<2> { using type = uint32_t; };
using Blk = LaneBlock<kLaneWords>::type;

__device__ __forceinline__ Blk load_block(const uint16_t *words, uint32_t b, uint32_t wpad,
                                          uint32_t lane) {
    const uint32_t w0 = b * kBlk + lane * kLaneWords;
    Blk v{};
    if (w0 < wpad) v = *reinterpret_cast<const Blk *>(words + w0);
    return v;
}

// Block b lands at ring position (b * kBlk) mod R; the block written at 0 is
// also copied to [R, R + 64) so that a read at (ptr mod R) + rank, rank < 64,
// never has to wrap.
__device__ __forceinline__ void put_block(uint16_t *ring, uint32_t b, Blk v, uint32_t lane) {
    const uint32_t pos = (b * kBlk) & (kRing - 1u);
    *reinterpret_cast<Blk *>(ring + pos + lane * kLaneWords) = v;
    if (pos == 0 && lane < 64u / kLaneWords)
        *reinterpret_cast<Blk *>(ring + kRing + lane * kLaneWords) = v;
}

// Per-chunk decoder state of one wave. Positions inside the chunk are u32
// (a chunk holds at most 2^24 symbols); wave-uniform values stay in SGPRs.
template <int K, bool BF16, uint32_t DT, int MODE, bool GEMV = false, uint32_t CODEC = 0>
struct Chunk {
    const TArgs &T;
    const LutEnt *lut;
    uint16_t *ring;
    uint32_t lane;
    uint64_t p0;   // flat position of the chunk's first symbol
    uint32_t nk;   // symbols in the chunk
    uint32_t wc, wpad, nblocks, nb;
    const uint16_t *words;
    Blk pend;
    uint32_t x;    // this lane's rANS state, or its Huffman bit buffer (next bit in bit 0)
    uint32_t nbits;  // Huffman: valid bits in x
    uint32_t ptr;  // words consumed (wave-uniform)
    uint64_t row;  // row of the current group's first symbol (modes 1, 2)
    uint32_t col;  // its column
    float s_cur, s_next;  // scales of rows row and row + 1
    uint64_t esc_i;       // index of the next super weight in the side list
    uint32_t esc_loc;     // its chunk-local position, ~0u if none left in the chunk
    // tensor fields used inside the loop, read once per chunk
    uint64_t cols, rows, n_esc;
    uint32_t cols32;
    const float *scales;
    const uint64_t *eidx;
    const uint16_t *eval;
    char *ob;             // output of the chunk's first symbol
    // fused GEMV (the chunk starts at a row boundary and holds whole rows)
    const uint16_t *xv;   // the tensor's input vector
    __amdgpu_buffer_rsrc_t xrsrc;  // the same as a buffer resource (cols < 2^31 bf16)
    float *yv;            // the tensor's output vector
    uint64_t row0;        // first row of the chunk
    float acc;            // row-uniform groups: this lane's partial of the current row
    float racc;           // other groups: running sum of the current row (wave-uniform)

    static constexpr uint32_t G = 64u * K;  // symbols per group of K steps

    __device__ __forceinline__ const uint64_t *esc_idx() const { return eidx; }
    __device__ __forceinline__ const uint16_t *esc_val() const { return eval; }
    __device__ __forceinline__ void load_esc() {
        esc_loc = ~0u;
        if (esc_i < n_esc) {
            const uint64_t e = esc_idx()[esc_i];
            if (e < p0 + nk) esc_loc = (uint32_t)(e - p0);
        }
    }

    // Keep at least kBlk staged words ahead of ptr: kCheck steps read at most
    // 64 * kCheck = kBlk words.
    __device__ __forceinline__ void refill() {
        if (nb < nblocks && (int32_t)(nb * kBlk - ptr) < (int32_t)kBlk) {
            put_block(ring, nb, pend, lane);
            ++nb;
            if (nb < nblocks) pend = load_block(words, nb, wpad, lane);
        }
    }

    // One decode step of this lane (inactive lanes keep their state, which is
    // >= 2^16, so they never ask for a word).
    // Huffman step: a lane holding fewer than 12 bits first takes one word
    // (ballot + rank as for rANS), then decodes one codeword with one table
    // read: the entry's low 5 bits are the length, its top byte the symbol.
    template <bool MASKED>
    __device__ __forceinline__ uint32_t step_huff(bool active) {
        const uint32_t *tab = reinterpret_cast<const uint32_t *>(lut);
        const bool need = (MASKED ? active : true) && nbits < 12u;
        const uint64_t m = __builtin_amdgcn_ballot_w64(need);
        const uint32_t rank = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        const uint32_t w = ring[(ptr & (kRing - 1u)) + rank];
        uint32_t b = x, nb = nbits;
#if EQ_RENORM_EXEC
        // under an exec mask of the refilling lanes (see the rANS step)
        uint64_t saved;
        asm volatile("s_and_saveexec_b64 %2, %3\n\t"
                     "v_lshl_or_b32 %0, %4, %1, %0\n\t"
                     "v_add_u32 %1, 16, %1\n\t"
                     "s_mov_b64 exec, %2"
                     : "+v"(b), "+v"(nb), "=&s"(saved)
                     : "s"(m), "v"(w)
                     : "scc");
#else
        const uint32_t merged = (w << nbits) | x;
        asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(b) : "v"(x), "v"(merged), "s"(m));
        asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(nb) : "v"(nbits), "v"(nbits + 16u), "s"(m));
#endif
        ptr += (uint32_t)__builtin_popcountll(m);
        const uint32_t e = tab[b & 4095u];
        const uint32_t bn = b >> (e & 31u);
        const uint32_t nn = nb - (e & 0xFFu);
        if (MASKED) {
            // a lane past the chunk keeps its final bits for the end check
            x = active ? bn : b;
            nbits = active ? nn : nb;
        } else {
            x = bn;
            nbits = nn;
        }
        return e;
    }

    template <bool MASKED>
    __device__ __forceinline__ uint32_t step(bool active) {
        if constexpr (CODEC == eqfmt::kCodecHuffman) return step_huff<MASKED>(active);
        const LutEnt ent = lut[x & 4095u];
        uint32_t xn = ent_next(ent, x);
        if (MASKED) xn = active ? xn : x;
        const bool need = xn < 65536u;
        const uint64_t m = __builtin_amdgcn_ballot_w64(need);
        const uint32_t rank = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
#if EQ_RENORM_BRANCHLESS
        // every lane reads ring[ptr + rank] (always inside the staged window
        // plus its 64-word copy); only lanes that need a word keep it
        const uint32_t w = ring[(ptr & (kRing - 1u)) + rank];
#if EQ_RENORM_EXEC
        // merge under an exec mask of the renormalising lanes: one VALU
        // instruction, the mask set and restored by the scalar unit (the
        // VALU, not the SALU, is the saturated resource)
        uint64_t saved;
        asm volatile("s_and_saveexec_b64 %1, %2\n\t"
                     "v_lshl_or_b32 %0, %0, 16, %3\n\t"
                     "s_mov_b64 exec, %1"
                     : "+v"(xn), "=&s"(saved)
                     : "s"(m), "v"(w)
                     : "scc");
#else
        const uint32_t merged = (xn << 16) | w;
        uint32_t sel;
        // a VALU select on the ballot mask (keeps the ring read unconditional)
        asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(sel) : "v"(xn), "v"(merged), "s"(m));
        xn = sel;
#endif
#else
        if (need) xn = (xn << 16) | ring[(ptr & (kRing - 1u)) + rank];
#endif
        ptr += (uint32_t)__builtin_popcountll(m);
        x = xn;
        return ent_bits(ent);
    }

    __device__ __forceinline__ float row_scale(uint64_t r) const {
        typedef const float __attribute__((address_space(4))) cfloat;
        cfloat *sc = (cfloat *)scales;
        return sc[r < rows ? r : rows - 1];
    }

    // The K outputs of this lane for group g, super-weight patches, store.
    template <bool MASKED>
    __device__ __forceinline__ void group(uint32_t g, void *out) {
        const uint32_t g0 = g * G;                        // chunk-local group start
        const uint32_t q0 = g0 + lane * (uint32_t)K;      // this lane's first position
        XRun<K> xr{};
        uint32_t rl = 0;  // GEMV: chunk-local row of this lane's run
        if constexpr (GEMV) {
            // the run's inputs, fetched before the K steps hide their latency
            // (a lane's run lies in one row; lanes past the chunk load nothing)
            if constexpr (MODE == M_ROW1) {
                if (!MASKED) {
                    // a full group: every lane's run is inside the row; the
                    // group's inputs start at a wave-uniform address (scalar
                    // base + the lane's constant offset, no VALU address or
                    // validity work)
                    xr = load_x_buffer<K>(xrsrc, lane * (uint32_t)(2 * K), col * 2u);
                } else if (q0 < nk) {
                    xr = load_x<K>(xv + col + lane * (uint32_t)K);
                }
            } else {
                rl = q0 / cols32;
                if (q0 < nk) xr = load_x<K>(xv + (q0 - rl * cols32));
            }
        }
        uint32_t ent[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if ((k & (kCheck - 1)) == 0) refill();
            ent[k] = step<MASKED>(q0 + (uint32_t)k < nk);
        }
        if constexpr (GEMV) {
            gemv_group<MASKED>(g0, q0, rl, ent, xr);
            return;
        }
        if constexpr (BF16) {
            uint16_t *ob = reinterpret_cast<uint16_t *>(this->ob);
            if constexpr (MODE != M_GENERAL) {
                if (!MASKED) {
                    float s = s_cur;
                    if constexpr (MODE == M_ROW2) {
                        // lanes below b are in `row`, the others in row + 1
                        const uint32_t left = (cols32 - col) / (uint32_t)K;
                        const uint32_t b = left < 64u ? left : 64u;
                        s = lane < b ? s_cur : s_next;
                    }
                    uint32_t pk[(K + 1) / 2];
#pragma unroll
                    for (int k = 0; k < K; k += 2) {
                        const float v0 = sym_value<DT>(ent[k]) * s;
                        const float v1 = (k + 1 < K) ? sym_value<DT>(ent[k + 1]) * s : 0.0f;
                        pk[k / 2] = pack_bf16(v0, v1);
                    }
                    if (esc_loc < g0 + G) patch_packed(g0, pk);
                    uint16_t *gb = ob + g0;  // wave-uniform base of the group
#if EQ_SADDR_STORE
                    if constexpr (K == 8) {
                        // scalar base + the lane's constant 32-bit offset: no
                        // per-group 64-bit address arithmetic on the VALU.
                        // Wait states the compiler cannot see inside the asm:
                        // 5 before (a VALU write of the base SGPRs, e.g. by
                        // v_readfirstlane, before a memory instruction reads
                        // them) and 1 after (a wide store's data registers are
                        // not rewritten by the next VALU instruction)
                        const uint64_t b = reinterpret_cast<uint64_t>(gb);
                        // (readfirstlane returns int: widen through uint32_t,
                        // never by sign extension)
                        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
                        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
                        const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
                        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
                        const u32x4 v = {pk[0], pk[1], pk[2], pk[3]};
                        asm volatile("s_nop 4\n\tglobal_store_dwordx4 %0, %1, %2" EQ_NT_SUFFIX "\n\ts_nop 0"
                                     :
                                     : "v"(lane * 16u), "v"(v), "s"(sb)
                                     : "memory");
                    } else
#endif
                    store_packed(reinterpret_cast<uint64_t>(gb) + lane * (2u * K), pk);
                    advance_row();
                    return;
                }
            }
            // general path: any shape, partial groups, unaligned output
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if (q0 + (uint32_t)k < nk) {
                    const uint64_t pos = p0 + q0 + (uint32_t)k;
                    const float v = sym_value<DT>(ent[k]) * scales[pos / cols];
                    ob[q0 + k] = (uint16_t)(pack_bf16(v, 0.0f) & 0xFFFFu);
                }
            }
            // super weights of this group: the owning lane rewrites them after
            // its own store of that element (same thread, same address)
            while (esc_loc < g0 + G) {
                if (lane == (esc_loc - g0) / (uint32_t)K) ob[esc_loc] = esc_val()[esc_i];
                ++esc_i;
                load_esc();
            }
            if constexpr (MODE != M_GENERAL) advance_row();
        } else {
            uint8_t *ob = reinterpret_cast<uint8_t *>(this->ob);
            if (MODE != M_GENERAL && !MASKED) {
                store_bytes(reinterpret_cast<char *>(ob + g0) + lane * (uint32_t)K, ent);
            } else {
#pragma unroll
                for (int k = 0; k < K; ++k)
                    if (q0 + (uint32_t)k < nk) ob[q0 + k] = (uint8_t)sym_byte(ent[k]);
            }
        }
    }

    // Fused GEMV epilogue of group g0: the lane's K weights exactly as the
    // bf16 decode would store them (scale, RNE, super weights), dotted with
    // its K inputs; row-uniform groups keep a per-lane partial until the row
    // ends, other groups reduce every row they touch at once.
    template <bool MASKED>
    __device__ __forceinline__ void gemv_group(uint32_t g0, uint32_t q0, uint32_t rl, const uint32_t *ent,
                                               const XRun<K> &xr) {
        const bool valid = !MASKED || q0 < nk;
        float s;
        if constexpr (MODE == M_ROW1) {
            s = s_cur;
        } else {
            const uint64_t r = row0 + rl;
            s = scales[r < rows ? r : rows - 1];
        }
        uint32_t pk[(K + 1) / 2];
#pragma unroll
        for (int k = 0; k < K; k += 2) {
            const float v0 = sym_value<DT>(ent[k]) * s;
            const float v1 = (k + 1 < K) ? sym_value<DT>(ent[k + 1]) * s : 0.0f;
            pk[k / 2] = pack_bf16(v0, v1);
        }
        if (esc_loc < g0 + G) patch_packed(g0, pk);
        if constexpr (MODE == M_ROW1) {
            float a = acc;
#pragma unroll
            for (int i = 0; i < (K + 1) / 2; ++i) a = dot2_bf16(pk[i], xr.p[i], a);
            if constexpr (MASKED) acc = valid ? a : acc;
            else acc = a;
            advance_row();
        } else {
            float d = 0.0f;
#pragma unroll
            for (int i = 0; i < (K + 1) / 2; ++i) d = dot2_bf16(pk[i], xr.p[i], d);
            d = valid ? d : 0.0f;
            const uint32_t end = g0 + G < nk ? g0 + G : nk;
            const uint32_t r_first = g0 / cols32, r_last = (end - 1u) / cols32;
            for (uint32_t r = r_first; r <= r_last; ++r) {
                racc += wave_sum(rl == r ? d : 0.0f);
                if ((r + 1u) * cols32 <= end) {
                    if (lane == 0) yv[row0 + r] = racc;
                    racc = 0.0f;
                }
            }
        }
    }

    __device__ __forceinline__ void advance_row() {
        if constexpr (BF16 && MODE == M_ROW1) {
            col += G;
            if (col == cols32) {
                if constexpr (GEMV) {
                    const float t = wave_sum(acc);
                    if (lane == 0) yv[row] = t;
                    acc = 0.0f;
                }
                col = 0;
                ++row;
                s_cur = row_scale(row);
            }
        } else if constexpr (BF16 && MODE == M_ROW2) {
            col += G;
            if (col >= cols32) {
                col -= cols32;
                ++row;
                s_cur = s_next;
                s_next = row_scale(row + 1);
            }
        }
    }

    // Super weights inside group g0 (fast paths): fix the owning lane's
    // packed registers before the store.
    __device__ __forceinline__ void patch_packed(uint32_t g0, uint32_t *pk) {
        do {
            const uint32_t off = esc_loc - g0;
            const uint32_t owner = off / (uint32_t)K, e = off % (uint32_t)K;
            const uint32_t v = esc_val()[esc_i];
            if (lane == owner) {
#pragma unroll
                for (int i = 0; i < (K + 1) / 2; ++i) {
                    if (e == 2u * i) pk[i] = (pk[i] & 0xFFFF0000u) | v;
                    if (e == 2u * i + 1u) pk[i] = (pk[i] & 0x0000FFFFu) | (v << 16);
                }
            }
            ++esc_i;
            load_esc();
        } while (esc_loc < g0 + G);
    }

    // dst is a global-memory address (the output buffer)
    __device__ __forceinline__ void store_packed(uint64_t dst, const uint32_t *pk) {
        typedef __attribute__((address_space(1))) uint16_t g16;
        typedef __attribute__((address_space(1))) uint32_t g32;
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(1))) u32x2 g64;
        if constexpr (K == 1) {
            *reinterpret_cast<g16 *>(dst) = (uint16_t)pk[0];
        } else if constexpr (K == 2) {
            *reinterpret_cast<g32 *>(dst) = pk[0];
        } else if constexpr (K == 4) {
            const u32x2 v = {pk[0], pk[1]};
            *reinterpret_cast<g64 *>(dst) = v;
        } else {
            typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(1))) u32x4 g128;
#pragma unroll
            for (int i = 0; i < K / 8; ++i) {
                u32x4 v = {pk[4 * i], pk[4 * i + 1], pk[4 * i + 2], pk[4 * i + 3]};
#if EQ_NT_STORES
                __builtin_nontemporal_store(v, reinterpret_cast<g128 *>(dst) + i);
#else
                reinterpret_cast<g128 *>(dst)[i] = v;
#endif
            }
        }
    }

    __device__ __forceinline__ void store_bytes(char *dst, const uint32_t *ent) {
        if constexpr (K == 1) {
            *reinterpret_cast<uint8_t *>(dst) = (uint8_t)sym_byte(ent[0]);
        } else if constexpr (K == 2) {
            *reinterpret_cast<uint16_t *>(dst) = (uint16_t)(sym_byte(ent[0]) | (sym_byte(ent[1]) << 8));
        } else {
            uint32_t w[K / 4];
#pragma unroll
            for (int i = 0; i < K / 4; ++i)
                w[i] = sym_byte(ent[4 * i]) | (sym_byte(ent[4 * i + 1]) << 8) |
                       (sym_byte(ent[4 * i + 2]) << 16) | (sym_byte(ent[4 * i + 3]) << 24);
            if constexpr (K == 4) {
                *reinterpret_cast<uint32_t *>(dst) = w[0];
            } else if constexpr (K == 8) {
                *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
            } else {
                *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }

    // (always inlined: an outlined copy would take the kernel argument's
    // address, which makes the compiler copy the whole argument block into
    // scratch memory)
    // ws, wc_: the chunk's directory entry (first word, word count), loaded
    // by the caller before the slot-table build
    __device__ __forceinline__ void run(uint64_t chunk, void *out, uint32_t *status, uint64_t ws, uint32_t wc_) {
        wc = wc_;
        wpad = (wc + 7u) & ~7u;
        if (wc > nk || ws + wpad > T.n_words) {
            raise_flag(status, EQ_DEV_WORD_OVERRUN, lane);
            return;
        }
        words = reinterpret_cast<const uint16_t *>(T.base + T.off_words) + ws;
        if constexpr (CODEC == eqfmt::kCodecHuffman) {
            x = 0;
            nbits = 0;
        } else {
            x = reinterpret_cast<const uint32_t *>(T.base + T.off_states)[chunk * 64u + lane];
        }
        nblocks = (wpad + kBlk - 1u) / kBlk;
        nb = 0;
        ptr = 0;
        pend = Blk{};
        if (nblocks) {
            put_block(ring, 0, load_block(words, 0, wpad, lane), lane);
            nb = 1;
            if (nb < nblocks) pend = load_block(words, nb, wpad, lane);
        }
        cols = T.cols;
        cols32 = (uint32_t)T.cols;
        rows = T.rows;
        n_esc = T.n_esc;
        scales = reinterpret_cast<const float *>(T.base + T.off_scales);
        eidx = reinterpret_cast<const uint64_t *>(T.base + T.off_esc_idx);
        eval = reinterpret_cast<const uint16_t *>(T.base + T.off_esc_val);
        if constexpr (GEMV) {
            xv = T.x;
            if constexpr (MODE == M_ROW1)
                xrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(T.x), (short)0,
                                                          (int)(uint32_t)(T.cols * 2u), kRawBufferWord3);
            yv = T.y;
            row0 = p0 / cols;
            acc = 0.0f;
            racc = 0.0f;
            ob = nullptr;
        } else {
            ob = static_cast<char *>(out) + (T.out_offset + p0) * (BF16 ? 2u : 1u);
        }
        if constexpr (BF16 && MODE != M_GENERAL) {
            row = p0 / cols;
            col = (uint32_t)(p0 - row * cols);
            s_cur = row_scale(row);
            s_next = row_scale(row + 1);
        }
        esc_i = 0;
        esc_loc = ~0u;
        if (BF16 && n_esc) {
            // first super weight at or after p0
            uint64_t lo = 0, hi = n_esc;
            while (lo < hi) {
                const uint64_t mid = (lo + hi) >> 1;
                if (esc_idx()[mid] < p0) lo = mid + 1; else hi = mid;
            }
            esc_i = lo;
            load_esc();
        }
        // settle the set-up loads here rather than at the loop header, where
        // the wait would be repeated every group
        __builtin_amdgcn_s_waitcnt(0);
        const uint32_t nfull = nk / G;
        for (uint32_t g = 0; g < nfull; ++g) group<false>(g, out);
        if (nfull * G < nk) group<true>(nfull, out);

        // integrity: every lane back at 2^16 and every word consumed
        // (Huffman: every lane's leftover bits must be the zero padding)
        const uint64_t bad = __builtin_amdgcn_ballot_w64(CODEC == eqfmt::kCodecHuffman ? x != 0u : x != 65536u);
        uint32_t bits = 0;
        if (ptr > wc) bits |= EQ_DEV_WORD_OVERRUN;
        else if (ptr != wc || bad) bits |= EQ_DEV_BAD_END_STATE;
        raise_flag(status, bits, lane);
    }
};

// One-symbol tensor: every state must be 2^16 and no word stored; the output
// is the symbol's dequantised value everywhere (escapes patched).
template <bool BF16>
__device__ __forceinline__ void const_chunk(const TArgs &T, uint64_t chunk, uint32_t lane, void *out,
                            uint32_t *status) {
    const uint64_t p0 = chunk * T.Z;
    const uint32_t nk = (uint32_t)umin64(T.Z, T.n - p0);
    const uint8_t *dir = T.base + T.off_dir + chunk * 16u;
    const uint32_t wc = *reinterpret_cast<const uint32_t *>(dir + 8);
    // (the Huffman codec stores no lane states)
    const uint32_t xs = T.codec == eqfmt::kCodecRans
                            ? reinterpret_cast<const uint32_t *>(T.base + T.off_states)[chunk * 64u + lane]
                            : 65536u;
    const uint64_t bad = __builtin_amdgcn_ballot_w64(xs != 65536u);
    raise_flag(status, (bad || wc) ? EQ_DEV_BAD_END_STATE : 0u, lane);
    const float *sc = reinterpret_cast<const float *>(T.base + T.off_scales);
    for (uint32_t q = lane; q < nk; q += 64u) {
        const uint64_t pos = p0 + q;
        if constexpr (BF16) {
            const uint32_t bits = T.const_sym << kSymShift;
            const float v = (T.dtype == EQ_DTYPE_INT8 ? sym_value<EQ_DTYPE_INT8>(bits)
                                                       : sym_value<EQ_DTYPE_E4M3>(bits)) *
                            sc[pos / T.cols];
            static_cast<uint16_t *>(out)[T.out_offset + pos] = (uint16_t)(pack_bf16(v, 0.0f) & 0xFFFFu);
        } else {
            static_cast<uint8_t *>(out)[T.out_offset + pos] = (uint8_t)T.const_sym;
        }
    }
    if constexpr (BF16) {
        if (T.n_esc) {
            // the lane that stored an element also patches it (program order)
            const uint64_t *eidx = reinterpret_cast<const uint64_t *>(T.base + T.off_esc_idx);
            const uint16_t *eval = reinterpret_cast<const uint16_t *>(T.base + T.off_esc_val);
            for (uint64_t e = 0; e < T.n_esc; ++e) {
                const uint64_t p = eidx[e];
                if (p >= p0 && p < p0 + nk && (uint32_t)((p - p0) % 64u) == lane)
                    static_cast<uint16_t *>(out)[T.out_offset + p] = eval[e];
            }
        }
    }
}

// One-symbol tensor, fused GEMV: per row, lanes stride over the columns with
// the row's weight (super weights substituted where listed), then reduce.
__device__ __forceinline__ void const_chunk_gemv(const TArgs &T, uint64_t chunk, uint32_t lane,
                                                 uint32_t *status) {
    const uint64_t p0 = chunk * T.Z;
    const uint32_t nk = (uint32_t)umin64(T.Z, T.n - p0);
    const uint8_t *dir = T.base + T.off_dir + chunk * 16u;
    const uint32_t wc = *reinterpret_cast<const uint32_t *>(dir + 8);
    // (the Huffman codec stores no lane states)
    const uint32_t xs = T.codec == eqfmt::kCodecRans
                            ? reinterpret_cast<const uint32_t *>(T.base + T.off_states)[chunk * 64u + lane]
                            : 65536u;
    const uint64_t bad = __builtin_amdgcn_ballot_w64(xs != 65536u);
    raise_flag(status, (bad || wc) ? EQ_DEV_BAD_END_STATE : 0u, lane);
    const float *sc = reinterpret_cast<const float *>(T.base + T.off_scales);
    const uint64_t *eidx = reinterpret_cast<const uint64_t *>(T.base + T.off_esc_idx);
    const uint16_t *eval = reinterpret_cast<const uint16_t *>(T.base + T.off_esc_val);
    const uint32_t bits = T.const_sym << kSymShift;
    const float v = T.dtype == EQ_DTYPE_INT8 ? sym_value<EQ_DTYPE_INT8>(bits) : sym_value<EQ_DTYPE_E4M3>(bits);
    const uint64_t cols = T.cols, row0 = p0 / cols, nrows = nk / cols;
    // this lane's next super weight (lanes walk their own positions in order)
    uint64_t e = 0, hi = T.n_esc;
    while (e < hi) {
        const uint64_t mid = (e + hi) >> 1;
        if (eidx[mid] < p0) e = mid + 1; else hi = mid;
    }
    for (uint64_t r = 0; r < nrows; ++r) {
        const uint32_t w = pack_bf16(v * sc[row0 + r], 0.0f) & 0xFFFFu;
        float acc = 0.0f;
        for (uint64_t c = lane; c < cols; c += 64u) {
            const uint64_t pos = p0 + r * cols + c;
            while (e < T.n_esc && eidx[e] < pos) ++e;
            const uint32_t wb = (e < T.n_esc && eidx[e] == pos) ? eval[e] : w;
            acc = dot2_bf16(wb, T.x[c], acc);
        }
        const float t = wave_sum(acc);
        if (lane == 0) T.y[row0 + r] = t;
    }
}

// Output kinds of the decode kernel.
enum : int { OUT_U8 = 0, OUT_BF16 = 1, OUT_GEMV = 2 };

// (the slot table and rings of three workgroups fill a CU's LDS: six waves
// per SIMD, which the register allocation must not undercut)
template <int K, int OUT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6)))
k_decode(LArgs a) {
    constexpr bool BF16 = OUT != OUT_U8;
    constexpr bool GEMV = OUT == OUT_GEMV;
    __shared__ LutEnt lut[4096];
    __shared__ __attribute__((aligned(16))) uint16_t rings[kWaves][kRingAlloc];
    // the slot-table build's scratch (cum, wave maxima) lives in the rings
    static_assert(sizeof(rings[0]) >= 260 * 4 + 2 * kSlotsPerWave, "a ring holds its wave's table-build scratch");
    static_assert(sizeof(rings) >= (256 + 16 * 3) * 4, "the rings hold the Huffman table build's scratch");

    // Work item of this workgroup. The hardware hands workgroups to the 8
    // XCDs in turn (block b to XCD b mod 8); the mapping below gives each XCD
    // a contiguous run of work items instead, so the workgroups an XCD runs
    // together read neighbouring chunks through its own L2 and write
    // neighbouring stretches of the output (measured: -6% on the 70B block
    // with 32 Ki chunks, -3% with 64 Ki).
    const uint32_t G = gridDim.x, xcd = blockIdx.x & 7u, per = G >> 3, extra = G & 7u;
    const uint32_t wg = xcd * per + (xcd < extra ? xcd : extra) + (blockIdx.x >> 3);
    uint32_t ti = 0;
    while (ti + 1 < a.n_tensors && wg >= a.t[ti + 1].wg_begin) ++ti;
    const TArgs &T = a.t[ti];
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t chunk = (uint64_t)(wg - T.wg_begin) * kWaves + wave;
    const bool is_const = T.is_const != 0;
    // the chunk's directory entry (scalar loads): in flight during the table build
    uint64_t dir_ws = 0;
    uint32_t dir_wc = 0;
    if (!is_const && chunk < T.n_chunks) {
        const uint8_t *dir = T.base + T.off_dir + chunk * 16u;
        dir_ws = *reinterpret_cast<const uint64_t *>(dir);
        dir_wc = *reinterpret_cast<const uint32_t *>(dir + 8);
    }
    // the table builds' scratch reuses the (not yet filled) rings
    if (!is_const) {
        if (T.codec == eqfmt::kCodecHuffman) {
            build_lut_huff(reinterpret_cast<const uint16_t *>(T.base + T.off_freq),
                           reinterpret_cast<uint32_t *>(lut), reinterpret_cast<uint32_t *>(&rings[0][0]));
        } else {
            // the workgroup's chunks share one table (with adaptive tables the
            // segment size is a multiple of the waves per workgroup); each
            // wave builds its slice in its own ring's memory, then one
            // barrier publishes the table
            build_lut(reinterpret_cast<const uint16_t *>(
                          T.base + T.off_freq +
                          (T.seg ? 512ull * (((uint64_t)(wg - T.wg_begin) * kWaves) / T.seg) : 0ull)),
                      lut, reinterpret_cast<uint32_t *>(&rings[wave][0]));
            __syncthreads();
        }
    }
    if (chunk >= T.n_chunks) return;
    if (is_const) {
        if constexpr (GEMV) const_chunk_gemv(T, chunk, lane, a.status);
        else const_chunk<BF16>(T, chunk, lane, a.out, a.status);
        return;
    }
    const uint64_t p0 = chunk * T.Z;
    const uint32_t nk = (uint32_t)umin64(T.Z, T.n - p0);
#define EQ_RUN_C(BF, DT, MO, CO)                                                       \
    do {                                                                               \
        Chunk<K, BF, DT, MO, GEMV, CO> c{T, lut, rings[wave], lane, p0, nk};           \
        c.run(chunk, a.out, a.status, dir_ws, dir_wc);                                                 \
    } while (0)
#define EQ_RUN(BF, DT, MO)                                                             \
    do {                                                                               \
        if (T.codec == eqfmt::kCodecHuffman) EQ_RUN_C(BF, DT, MO, eqfmt::kCodecHuffman); \
        else EQ_RUN_C(BF, DT, MO, eqfmt::kCodecRans);                                  \
    } while (0)
    if constexpr (GEMV) {
        if (T.dtype == EQ_DTYPE_INT8) {
            if (T.mode == M_ROW1) EQ_RUN(true, EQ_DTYPE_INT8, M_ROW1);
            else EQ_RUN(true, EQ_DTYPE_INT8, M_GENERAL);
        } else {
            if (T.mode == M_ROW1) EQ_RUN(true, EQ_DTYPE_E4M3, M_ROW1);
            else EQ_RUN(true, EQ_DTYPE_E4M3, M_GENERAL);
        }
    } else if constexpr (BF16) {
        if (T.dtype == EQ_DTYPE_INT8) {
            if (T.mode == M_ROW1) EQ_RUN(true, EQ_DTYPE_INT8, M_ROW1);
            else if (T.mode == M_ROW2) EQ_RUN(true, EQ_DTYPE_INT8, M_ROW2);
            else EQ_RUN(true, EQ_DTYPE_INT8, M_GENERAL);
        } else {
            if (T.mode == M_ROW1) EQ_RUN(true, EQ_DTYPE_E4M3, M_ROW1);
            else if (T.mode == M_ROW2) EQ_RUN(true, EQ_DTYPE_E4M3, M_ROW2);
            else EQ_RUN(true, EQ_DTYPE_E4M3, M_GENERAL);
        }
    } else {
        if (T.mode == M_ROW1) EQ_RUN(false, 0u, M_ROW1); else EQ_RUN(false, 0u, M_GENERAL);
    }
#undef EQ_RUN
#undef EQ_RUN_C
}

// ---------------------------------------------------------------------------
// Batch-1 bf16 GEMV (the consumer of a decoded block): one wave per row,
// 16-byte loads, fp32 accumulation, wave reduction.
// ---------------------------------------------------------------------------
constexpr int kGemvWaves = 4;

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ float dot8(uint4 w, uint4 v, float acc) {
    acc = fmaf(bf_lo(w.x), bf_lo(v.x), acc);
    acc = fmaf(bf_hi(w.x), bf_hi(v.x), acc);
    acc = fmaf(bf_lo(w.y), bf_lo(v.y), acc);
    acc = fmaf(bf_hi(w.y), bf_hi(v.y), acc);
    acc = fmaf(bf_lo(w.z), bf_lo(v.z), acc);
    acc = fmaf(bf_hi(w.z), bf_hi(v.z), acc);
    acc = fmaf(bf_lo(w.w), bf_lo(v.w), acc);
    acc = fmaf(bf_hi(w.w), bf_hi(v.w), acc);
    return acc;
}

__global__ void __launch_bounds__(64 * kGemvWaves)
k_gemv(const uint16_t *__restrict__ W, uint64_t rows, uint64_t cols, const uint16_t *__restrict__ xv,
       float *__restrict__ y) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t row = (uint64_t)blockIdx.x * kGemvWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    const uint16_t *w = W + row * cols;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    uint64_t c = lane * 8u;
    for (; c + 3 * 512 < cols; c += 4 * 512) {
        const uint4 w0 = *reinterpret_cast<const uint4 *>(w + c);
        const uint4 w1 = *reinterpret_cast<const uint4 *>(w + c + 512);
        const uint4 w2 = *reinterpret_cast<const uint4 *>(w + c + 1024);
        const uint4 w3 = *reinterpret_cast<const uint4 *>(w + c + 1536);
        a0 = dot8(w0, *reinterpret_cast<const uint4 *>(xv + c), a0);
        a1 = dot8(w1, *reinterpret_cast<const uint4 *>(xv + c + 512), a1);
        a2 = dot8(w2, *reinterpret_cast<const uint4 *>(xv + c + 1024), a2);
        a3 = dot8(w3, *reinterpret_cast<const uint4 *>(xv + c + 1536), a3);
    }
    for (; c < cols; c += 512)
        a0 = dot8(*reinterpret_cast<const uint4 *>(w + c), *reinterpret_cast<const uint4 *>(xv + c), a0);
    float acc = (a0 + a1) + (a2 + a3);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if (lane == 0) y[row] = acc;
}

// Diagnostic: the decode kernel's fp32 -> bf16 rounding on an array.
__global__ void k_bf16(const float *__restrict__ in, uint64_t n, uint16_t *__restrict__ out) {
    const uint64_t i = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * 2u;
    if (i + 1 < n) {
        const uint32_t p = pack_bf16(in[i], in[i + 1]);
        out[i] = (uint16_t)p;
        out[i + 1] = (uint16_t)(p >> 16);
    } else if (i < n) {
        out[i] = (uint16_t)pack_bf16(in[i], 0.0f);
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
using KernelFn = void (*)(LArgs);

template <int OUT>
KernelFn pick_kernel(uint32_t K) {
    switch (K) {
        case 1: return k_decode<1, OUT>;
        case 2: return k_decode<2, OUT>;
        case 4: return k_decode<4, OUT>;
        case 8: return k_decode<8, OUT>;
        case 16: return k_decode<16, OUT>;
        default: return nullptr;
    }
}

// Header fields the kernel relies on, re-checked against each other.
bool header_ok(const eq_header &h) {
    if (h.dtype != EQ_DTYPE_INT8 && h.dtype != EQ_DTYPE_E4M3) return false;
    if (!eqfmt::valid_lane_run(h.lane_run)) return false;
    if (h.chunk_symbols == 0 || h.chunk_symbols > eqfmt::kMaxChunk ||
        h.chunk_symbols % (64u * h.lane_run))
        return false;
    if (h.rows == 0 || h.cols == 0 || h.rows * h.cols != h.n) return false;
    if (h.n_chunks != (h.n + h.chunk_symbols - 1) / h.chunk_symbols) return false;
    if (h.codec != eqfmt::kCodecRans && h.codec != eqfmt::kCodecHuffman) return false;
    if (h.seg_chunks && (h.seg_chunks % 8 || h.codec != eqfmt::kCodecRans)) return false;
    const eqfmt::Sections s = eqfmt::layout(h.rows, h.n_chunks, h.n_words, h.n_esc, h.codec,
                                            eqfmt::n_tables(h.n_chunks, h.seg_chunks));
    return s.freq == h.off_freq && s.scales == h.off_scales && s.dir == h.off_dir &&
           s.states == h.off_states && s.words == h.off_words && s.esc_idx == h.off_esc_idx &&
           s.esc_val == h.off_esc_val && s.total == h.total_bytes;
}

// One launch per run of up to EQ_MAX_BLOCK_TENSORS consecutive tensors with
// the same lane run. OUT_GEMV takes x[i] / y[i] per tensor instead of `out`.
template <int OUT>
eq_status launch_block(const eq_block *b, void *out, const uint16_t *const *x, float *const *y,
                       void *stream) {
    constexpr bool BF16 = OUT != OUT_U8;
    constexpr bool GEMV = OUT == OUT_GEMV;
    if (!b || (b->n_tensors && !b->tensors)) return EQ_EINVAL;
    if (b->n_tensors && (GEMV ? (!x || !y) : !out)) return EQ_EINVAL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uintptr_t obase = reinterpret_cast<uintptr_t>(out);
    uint32_t i = 0;
    while (i < b->n_tensors) {
        LArgs a{};
        a.out = out;
        a.status = b->d_status;
        const uint32_t K = b->tensors[i].hdr.lane_run;
        uint64_t wgs = 0;
        uint32_t nt = 0;
        for (; i < b->n_tensors && nt < EQ_MAX_BLOCK_TENSORS; ++i, ++nt) {
            const eq_tensor_ref &r = b->tensors[i];
            const eq_header &h = r.hdr;
            if (h.lane_run != K) break;
            if (!r.d_container || (reinterpret_cast<uintptr_t>(r.d_container) & 15u)) return EQ_EINVAL;
            if (!header_ok(h)) return EQ_EINVAL;
            TArgs &t = a.t[nt];
            t.base = static_cast<const uint8_t *>(r.d_container);
            t.out_offset = r.out_offset;
            t.n = h.n;
            t.cols = h.cols;
            t.rows = h.rows;
            t.n_chunks = h.n_chunks;
            t.n_words = h.n_words;
            t.n_esc = h.n_esc;
            t.off_freq = h.off_freq;
            t.off_scales = h.off_scales;
            t.off_dir = h.off_dir;
            t.off_states = h.off_states;
            t.off_words = h.off_words;
            t.off_esc_idx = h.off_esc_idx;
            t.off_esc_val = h.off_esc_val;
            t.Z = h.chunk_symbols;
            t.dtype = h.dtype;
            t.codec = h.codec;
            t.seg = h.seg_chunks;
            if (t.seg % kWaves) return EQ_EUNSUPPORTED;
            t.is_const = 0;
            t.const_sym = 0;
            if (h.single_symbol >= 0) {
                t.is_const = 1;
                t.const_sym = (uint32_t)h.single_symbol;
            }
            const uint64_t G = 64u * K;
            t.x = nullptr;
            t.y = nullptr;
            if constexpr (GEMV) {
                // chunks must hold whole rows and a lane's run one row
                if (h.chunk_symbols % h.cols != 0 || h.cols % K != 0) return EQ_EUNSUPPORTED;
                if (!x[i] || !y[i] || (reinterpret_cast<uintptr_t>(x[i]) & 15u) ||
                    (reinterpret_cast<uintptr_t>(y[i]) & 3u))
                    return EQ_EINVAL;
                t.x = x[i];
                t.y = y[i];
                t.mode = (h.cols % G == 0 && h.cols < (1ull << 31)) ? M_ROW1 : M_GENERAL;
            } else {
                const uint32_t vec = BF16 ? 2u * (K < 8 ? K : 8u) : K;  // bytes per store
                const uint64_t elem = BF16 ? 2u : 1u;
                const bool aligned = ((obase + r.out_offset * elem) % vec) == 0;
                t.mode = M_GENERAL;
                if (aligned && !BF16) t.mode = M_ROW1;
                if (aligned && BF16 && h.cols < (1ull << 31)) {
                    if (h.cols % G == 0) t.mode = M_ROW1;
                    else if (h.cols >= G && h.cols % K == 0) t.mode = M_ROW2;
                }
            }
            t.wg_begin = (uint32_t)wgs;
            wgs += (h.n_chunks + kWaves - 1) / kWaves;
        }
        a.n_tensors = nt;
        if (wgs > 0x7FFFFFFFull) return EQ_EINVAL;
        if (wgs) {
            KernelFn fn = pick_kernel<OUT>(K);
            if (!fn) return EQ_EINVAL;
            hipLaunchKernelGGL(fn, dim3((uint32_t)wgs), dim3(kThreads), 0, s, a);
            if (hipGetLastError() != hipSuccess) return EQ_EHIP;
        }
    }
    return EQ_OK;
}

}  // namespace

extern "C" {

eq_status eq_decode_block(const eq_block *b, uint8_t *d_symbols, void *stream) {
    return launch_block<OUT_U8>(b, d_symbols, nullptr, nullptr, stream);
}

eq_status eq_decode_dequant_bf16(const eq_block *b, uint16_t *d_bf16, void *stream) {
    return launch_block<OUT_BF16>(b, d_bf16, nullptr, nullptr, stream);
}

eq_status eq_decode_gemv_bf16(const eq_block *b, const uint16_t *const *d_x, float *const *d_y,
                              void *stream) {
    return launch_block<OUT_GEMV>(b, nullptr, d_x, d_y, stream);
}

eq_status eq_gemv_bf16(const uint16_t *d_w, uint64_t rows, uint64_t cols, const uint16_t *d_x,
                       float *d_y, void *stream) {
    if (!d_w || !d_x || !d_y || rows == 0 || cols == 0 || cols % 8) return EQ_EINVAL;
    if ((reinterpret_cast<uintptr_t>(d_w) | reinterpret_cast<uintptr_t>(d_x)) & 15u) return EQ_EINVAL;
    const uint64_t grid = (rows + kGemvWaves - 1) / kGemvWaves;
    if (grid > 0x7FFFFFFFull) return EQ_EINVAL;
    hipLaunchKernelGGL(k_gemv, dim3((uint32_t)grid), dim3(64 * kGemvWaves), 0,
                       static_cast<hipStream_t>(stream), d_w, rows, cols, d_x, d_y);
    return hipGetLastError() == hipSuccess ? EQ_OK : EQ_EHIP;
}

eq_status eq_bf16_from_f32(const float *d_in, uint64_t n, uint16_t *d_out, void *stream) {
    if (!d_in || !d_out) return EQ_EINVAL;
    if (n == 0) return EQ_OK;
    const uint64_t threads = (n + 1) / 2;
    const uint64_t grid = (threads + 255) / 256;
    if (grid > 0x7FFFFFFFull) return EQ_EINVAL;
    hipLaunchKernelGGL(k_bf16, dim3((uint32_t)grid), dim3(256), 0,
                       static_cast<hipStream_t>(stream), d_in, n, d_out);
    return hipGetLastError() == hipSuccess ? EQ_OK : EQ_EHIP;
}

}  // extern "C"
