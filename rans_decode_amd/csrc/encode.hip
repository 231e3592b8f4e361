// encode.hip -- device-side compression of one tensor into a container v1
// (rANS codec) on gfx950: histogram, the 12-bit frequency quantiser,
// chunk-parallel interleaved encoding, container assembly. The result is
// byte-for-byte what eq_encode_host writes for the same inputs.
//
// EntQuant summary ("Float8@2bits: Entropy Coding Enables Data-Free Model
// Compression", section 2, technical component 2): the weights are flattened
// into one symbol stream and ANS-compressed; bitstream + scales + metadata
// are stored. The summary also reports compressing a 70B model in minutes;
// this is the encode half of that, on the GPU (the scale optimisation before
// it is not part of this library).
//
// Pipeline (one stream, six launches, no host synchronisation):
//   check   super-weight list and scales (and copy the scales); clear the
//           workspace counters
//   hist    per-workgroup LDS histograms (32 copies, one per LDS bank, so
//           the few frequent codes of a low-entropy tensor do not serialise
//           the atomics) -> 256 u64 counts (global atomics, nonzero
//           counts only)
//   quant   the quantiser (rule stated in include/eq.h) -> freq/cum, header,
//           frequency section
//   chunks  one wave per chunk: lanes walk the chunk's steps backwards; a lane
//           whose state reached f * 2^20 emits its low 16 bits first; the
//           words of one step take consecutive slots in ascending lane order
//           (ballot + mbcnt), filled from the end of the chunk's scratch
//           region, so they come out in the decoder's reading order. Words
//           collect in a per-wave LDS ring and leave in 1 KiB aligned blocks;
//           the division by f is one binary64 fused multiply-add with the
//           symbol's reciprocal (exact, see enc_div)
//   scan    one workgroup: padded word counts -> directory, n_words, the
//           offsets that depend on it, the total size
//   copy    words to their final place (16-byte stores; the word offset
//           inside the scratch is wave-uniform, so each lane realigns two
//           aligned loads), escape list, zero gaps
#include <hip/hip_runtime.h>
#include <type_traits>

#include <atomic>
#include <cstdint>
#include <mutex>

#include "../../include/eq.h"
#include "format.hpp"

namespace {

using namespace eqfmt;

constexpr int kEncWaves = 4;                   // chunks per workgroup
constexpr int kEncThreads = 64 * kEncWaves;

// Per-symbol encoder constants: the reciprocal of f for the division, f and
// 4096 - f, the cumulative frequency.
struct EncSym {
    double rcp;    // 1 / f rounded to binary64 (0 for absent symbols)
    uint32_t fg;   // 16 f (0xFFFF for f = 4096) | (4096 - f) << 16
    uint32_t cum;
};
static_assert(sizeof(EncSym) == 16, "one 16-byte LDS read per step");

constexpr uint32_t kEncRing = 2048;   // words of a wave's output ring
constexpr uint32_t kHistMaxGrid = 1024;  // histogram workgroups at most (4 per CU)
constexpr uint32_t kEncFlush = 512;   // words per ring flush (8 per lane)

// Tables a container can have: one, or one per segment of seg_chunks chunks
// (a multiple of 8), so at most ceil(n_chunks / 8).
__host__ __device__ inline uint64_t max_tables(uint64_t n_chunks) { return n_chunks > 8 ? (n_chunks + 7) / 8 : 1; }

// Workspace layout (bytes from the start; all 256-byte aligned).
struct WsLayout {
    uint64_t counts;   // tables x 256 x u64
    uint64_t table;    // tables x 256 x EncSym (rANS), or 256 x u32 Huffman codewords
    uint64_t misc;     // u64 n_words, u64 total, u64 escape codes seen
    uint64_t wstart;   // n_chunks x u32: first word of the chunk inside its scratch region
    uint64_t wcount;   // n_chunks x u32: the chunk's word count
    uint64_t first;    // n_chunks x u64: first word in the container
    uint64_t scratch;  // n + 16 x u16 (chunk k uses [k*Z, k*Z + nk); the tail chunk's
                       // last aligned block and the copy's read-ahead go past n)
    uint64_t total;
};

__host__ __device__ inline WsLayout ws_layout(uint64_t n, uint64_t n_chunks) {
    WsLayout w{};
    uint64_t at = 0;
    auto place = [&](uint64_t bytes) {
        const uint64_t start = round_up(at, 256);
        at = start + bytes;
        return start;
    };
    const uint64_t tabs = max_tables(n_chunks);
    w.counts = place(tabs * 256 * 8);
    w.table = place(tabs * 256 * sizeof(EncSym));
    w.misc = place(24);
    w.wstart = place(n_chunks * 4);
    w.wcount = place(n_chunks * 4);
    w.first = place(n_chunks * 8);
    w.scratch = place((n + 16) * 2);
    w.total = round_up(at, 256);
    return w;
}

struct EncArgs {
    const uint8_t *sym;
    const float *scales;
    const uint64_t *esc_idx;
    const uint16_t *esc_val;
    uint8_t *ws;
    uint8_t *out;
    uint64_t *out_len;
    uint32_t *status;
    uint64_t rows, cols, n, n_chunks, n_esc;
    uint32_t Z, K, dtype, esc_enabled, esc_code;
    uint32_t codec, seg;  // codec; chunks per table segment (0: one table)
    uint64_t n_tab;       // tables in the container
    uint64_t seg_syms;    // symbols per table segment (n with one table)
    WsLayout w;
    Sections sec;  // n_words-independent offsets (freq, scales, dir, states, words)
};

__device__ inline void flag(uint32_t *status, uint32_t bits) {
    if (status) atomicOr(status, bits);
}

template <typename T>
__device__ inline T *at(uint8_t *base, uint64_t off) {
    return reinterpret_cast<T *>(base + off);
}


// Histogram: 32 copies of the 256 counters per workgroup, bin-major, copy =
// lane mod 32, so the 32 lanes an LDS atomic serves at once hit 32 different
// banks whatever their codes; 16 symbols per thread per iteration.
constexpr uint32_t kHistCopies = 32;

__global__ void __launch_bounds__(256) k_enc_hist(EncArgs a) {
    __shared__ uint32_t h[256 * kHistCopies];
    for (uint32_t i = threadIdx.x; i < 256 * kHistCopies; i += blockDim.x) h[i] = 0;
    __syncthreads();
    const uint32_t c = threadIdx.x & (kHistCopies - 1u);
    // this grid row's table segment (a multiple of 512 symbols from the start)
    const uint64_t base = (uint64_t)blockIdx.y * a.seg_syms;
    const uint64_t len = a.n - base < a.seg_syms ? a.n - base : a.seg_syms;
    const uint8_t *sym = a.sym + base;
    const uint64_t n16 = len / 16;
    const uint4 *v = reinterpret_cast<const uint4 *>(sym);
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    auto count4 = [&](uint32_t wd) {
#pragma unroll
        for (int b = 0; b < 4; ++b) atomicAdd(&h[((wd >> (8 * b)) & 0xFFu) * kHistCopies + c], 1u);
    };
    uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + stride < n16; i += 2 * stride) {  // two 16-byte loads in flight per thread
        const uint4 q0 = v[i], q1 = v[i + stride];
        count4(q0.x); count4(q0.y); count4(q0.z); count4(q0.w);
        count4(q1.x); count4(q1.y); count4(q1.z); count4(q1.w);
    }
    if (i < n16) {
        const uint4 q0 = v[i];
        count4(q0.x); count4(q0.y); count4(q0.z); count4(q0.w);
    }
    for (uint64_t j = n16 * 16 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < len; j += stride)
        atomicAdd(&h[sym[j] * kHistCopies + c], 1u);
    __syncthreads();
    if (threadIdx.x < 256) {
        const uint32_t s = threadIdx.x;
        uint64_t sum = 0;
        // rotated start: the lanes of a wave read different banks
        for (uint32_t j = 0; j < kHistCopies; ++j) sum += h[s * kHistCopies + ((j + s) & (kHistCopies - 1u))];
        if (sum)
            atomicAdd(reinterpret_cast<unsigned long long *>(at<uint64_t>(a.ws, a.w.counts) + 256 * blockIdx.y + s),
                      (unsigned long long)sum);
    }
}

// Super-weight list (ascending, in range, escape code at each index) and
// finite scales; the scales are copied into the container on the way.
// Runs first: workgroup 0 also clears the workspace counters.
__global__ void k_enc_check(EncArgs a) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (uint64_t i = tid; i < a.n_tab * 256; i += stride) at<uint64_t>(a.ws, a.w.counts)[i] = 0;
    if (tid < 3) at<uint64_t>(a.ws, a.w.misc)[tid] = 0;
    float *osc = at<float>(a.out, a.sec.scales);
    for (uint64_t r = tid; r < a.rows; r += stride) {
        const float v = a.scales[r];
        if (!__builtin_isfinite(v)) flag(a.status, EQ_DEV_BAD_INPUT);
        osc[r] = v;
    }
    for (uint64_t e = tid; e < a.n_esc; e += stride) {
        const uint64_t i = a.esc_idx[e];
        bool bad = i >= a.n || (e && i <= a.esc_idx[e - 1]);
        if (!bad) bad = a.sym[i] != a.esc_code;
        if (bad) flag(a.status, EQ_DEV_BAD_INPUT);
    }
}

// Container header (one thread; the caller has zeroed its 256 bytes): the
// fields that do not depend on the word counts (k_enc_scan adds those).
__device__ __forceinline__ void write_header(const EncArgs &a) {
    uint8_t *b = a.out;
    *reinterpret_cast<uint32_t *>(b + H_MAGIC) = kMagic;
    *reinterpret_cast<uint16_t *>(b + H_VERSION) = kVersion;
    b[H_DTYPE] = (uint8_t)a.dtype;
    b[H_FLAGS] = (a.esc_enabled ? kFlagEsc : 0) | (a.seg ? kFlagSeg : 0);
    *reinterpret_cast<uint64_t *>(b + H_ROWS) = a.rows;
    *reinterpret_cast<uint64_t *>(b + H_COLS) = a.cols;
    *reinterpret_cast<uint64_t *>(b + H_N) = a.n;
    *reinterpret_cast<uint32_t *>(b + H_CHUNK) = a.Z;
    *reinterpret_cast<uint32_t *>(b + H_LANE_RUN) = a.K;
    *reinterpret_cast<uint32_t *>(b + H_LANES) = kLanes;
    *reinterpret_cast<uint32_t *>(b + H_PROB_BITS) = a.codec == kCodecHuffman ? kHuffMaxLen : kProbBits;
    *reinterpret_cast<uint64_t *>(b + H_NCHUNKS) = a.n_chunks;
    *reinterpret_cast<uint64_t *>(b + H_NESC) = a.n_esc;
    b[H_ESC_CODE] = a.esc_enabled ? (uint8_t)a.esc_code : 0;
    *reinterpret_cast<uint64_t *>(b + H_OFF_FREQ) = a.sec.freq;
    *reinterpret_cast<uint64_t *>(b + H_OFF_SCALES) = a.sec.scales;
    *reinterpret_cast<uint64_t *>(b + H_OFF_DIR) = a.sec.dir;
    *reinterpret_cast<uint64_t *>(b + H_OFF_STATES) = a.sec.states;
    *reinterpret_cast<uint64_t *>(b + H_OFF_WORDS) = a.sec.words;
    *reinterpret_cast<uint32_t *>(b + H_CODEC) = a.codec;
    *reinterpret_cast<uint32_t *>(b + H_SEG) = a.seg;
}

// Sum, maximum and minimum over a 256-thread workgroup (every thread calls
// them; red holds 4 ints): a shuffle butterfly per wave, then the four wave
// results.
template <typename Op>
__device__ __forceinline__ int32_t block_reduce256(int32_t v, int32_t *red, Op op) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o, 64));
    __syncthreads();  // the previous call's readers are done with red
    if ((threadIdx.x & 63u) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    return op(op(red[0], red[1]), op(red[2], red[3]));
}
__device__ __forceinline__ int32_t block_sum256(int32_t v, int32_t *red) {
    return block_reduce256(v, red, [](int32_t x, int32_t y) { return x + y; });
}
__device__ __forceinline__ int32_t block_max256(int32_t v, int32_t *red) {
    return block_reduce256(v, red, [](int32_t x, int32_t y) { return x > y ? x : y; });
}
__device__ __forceinline__ int32_t block_min256(int32_t v, int32_t *red) {
    return block_reduce256(v, red, [](int32_t x, int32_t y) { return x < y ? x : y; });
}

// Per-table checks (thread 0): E4M3 NaN codes only as the escape code; the
// escape codes seen are summed for k_enc_scan, which compares the total with
// the list.
__device__ __forceinline__ void check_counts(const EncArgs &a, const uint64_t *counts) {
    if (a.dtype == EQ_DTYPE_E4M3) {
        if (counts[0x7F] && !(a.esc_enabled && a.esc_code == 0x7Fu)) flag(a.status, EQ_DEV_BAD_INPUT);
        if (counts[0xFF] && !(a.esc_enabled && a.esc_code == 0xFFu)) flag(a.status, EQ_DEV_BAD_INPUT);
    }
    if (a.esc_enabled && counts[a.esc_code])
        atomicAdd(reinterpret_cast<unsigned long long *>(at<uint64_t>(a.ws, a.w.misc) + 2),
                  (unsigned long long)counts[a.esc_code]);
}

// Quantiser + frequency section (one workgroup of 256 threads per table, one
// symbol per thread; workgroup 0 also writes the header):
//   f_s = max(1, floor(c_s * 4096 / N)) for present bytes; a shortfall goes
//   +1 to the present bytes ranked first by (remainder c_s * 4096 mod N
//   descending, byte ascending); an excess is taken -1 at a time from the
//   largest f_s > 1 (smallest byte among equals), computed here in closed
//   form.
__global__ void __launch_bounds__(256) k_enc_quant(EncArgs a) {
    __shared__ __align__(16) uint64_t key[256];
    __shared__ __align__(16) int32_t f[256];
    __shared__ int32_t red[4];
    const uint32_t s = threadIdx.x;
    const uint64_t g = blockIdx.x;  // table (segment)
    const uint64_t N = a.n - g * a.seg_syms < a.seg_syms ? a.n - g * a.seg_syms : a.seg_syms;
    __shared__ uint64_t counts[256];  // read by every thread below: staged in LDS
    const uint64_t c = at<uint64_t>(a.ws, a.w.counts)[256 * g + s];
    counts[s] = c;
    const uint64_t scaled = c * (uint64_t)kProbScale;
    const bool present = c != 0;
    int32_t fs = 0;
    if (present) {
        const uint64_t q = scaled / N;
        fs = q > 1 ? (int32_t)q : 1;
    }
    f[s] = fs;
    // key = remainder above the byte's complement, so a larger key ranks
    // first; an absent byte's key is 0 and never counts (a strictly larger
    // key is needed)
    key[s] = present ? ((scaled % N) << 8 | (255u - s)) : 0;
    const int32_t deficit = (int32_t)kProbScale - block_sum256(fs, red);
    if (deficit > 0) {
        if (present) {
            // rank among present bytes by (remainder descending, byte
            // ascending): one branch-free u64 key compare per byte
            uint32_t rank = 0;
            const uint64_t ks = key[s];
            const ulonglong2 *k2 = reinterpret_cast<const ulonglong2 *>(key);
#pragma unroll 8
            for (uint32_t q = 0; q < 128; ++q) {  // 16-byte reads, many in flight
                const ulonglong2 w = k2[q];
                rank += (w.x > ks ? 1u : 0u) + (w.y > ks ? 1u : 0u);
            }
            if ((int32_t)rank < deficit) f[s] = fs + 1;
        }
        __syncthreads();
    } else if (deficit < 0) {
        // Taking 1 from the largest f > 1 (smallest byte first) E times
        // lowers the top level evenly: with cost(v) = sum of max(0, f - v)
        // and v the smallest level with cost(v) < E, every f above v comes
        // down to v and the remaining E - cost(v) decrements go to the
        // bytes then at v in ascending order (each leaves the top level
        // after its one decrement). v = 1 would mean too few f > 1.
        // E <= 256 (each present byte's f is rounded up by less than 2), and
        // v lies in (max f - E, max f] (the largest f alone costs E at
        // max f - E): thread u tests the level max f - u.
        const int32_t E = -deficit;
        const int32_t top = block_max256(fs, red);
        int32_t cand = 0x7FFFFFFF;
        const int32_t level = top - (int32_t)s;
        if ((int32_t)s < E && level >= 1) {
            int32_t c = 0;
            const int4 *f4 = reinterpret_cast<const int4 *>(f);
#pragma unroll 8
            for (uint32_t q = 0; q < 64; ++q) {  // 16-byte reads, many in flight
                const int4 w = f4[q];
                c += (w.x > level ? w.x - level : 0) + (w.y > level ? w.y - level : 0) +
                     (w.z > level ? w.z - level : 0) + (w.w > level ? w.w - level : 0);
            }
            if (c < E) cand = level;
        }
        const int32_t v = block_min256(cand, red);
        if (v == 1) {
            if (s == 0) flag(a.status, EQ_DEV_BAD_INPUT);
        } else {
            const int32_t r = E - block_sum256(fs > v ? fs - v : 0, red);
            // bytes below s at the top level after the cut: the ballot's
            // lanes below s plus the earlier waves' counts
            const bool at_top = fs >= v;
            const uint64_t m = __builtin_amdgcn_ballot_w64(at_top);
            __shared__ uint32_t wcnt[4];
            if ((s & 63u) == 0) wcnt[s >> 6] = (uint32_t)__builtin_popcountll(m);
            __syncthreads();
            uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            for (uint32_t w = 0; w < (s >> 6); ++w) rank += wcnt[w];
            if (at_top) f[s] = v - ((int32_t)rank < r ? 1 : 0);
        }
        __syncthreads();
    }
    // cumulative frequencies: exclusive prefix sum over bytes (log-step scan)
    __shared__ uint32_t cum[256];
    {
        uint32_t v = (uint32_t)f[s];
        cum[s] = v;
        for (uint32_t o = 1; o < 256; o <<= 1) {
            __syncthreads();
            const uint32_t add = s >= o ? cum[s - o] : 0u;
            __syncthreads();
            v += add;
            cum[s] = v;
        }
        __syncthreads();
        cum[s] = v - (uint32_t)f[s];
        __syncthreads();
    }
    if (s == 0) check_counts(a, counts);
    __syncthreads();
    EncSym es;
    es.rcp = f[s] ? 1.0 / (double)f[s] : 0.0;
    // 16 f (the emit threshold on x >> 16; f = 4096, a one-symbol table that
    // never emits, gets 0xFFFF, above any x >> 16 its state reaches)
    es.fg = (f[s] < (int32_t)kProbScale ? (uint32_t)f[s] << 4 : 0xFFFFu) |
            ((kProbScale - (uint32_t)f[s]) << 16);
    es.cum = cum[s];
    at<EncSym>(a.ws, a.w.table)[256 * g + s] = es;
    reinterpret_cast<uint16_t *>(a.out + a.sec.freq)[256 * g + s] = (uint16_t)f[s];
    if (g != 0) return;
    // header: every byte written; n_words-dependent fields are filled by k_enc_scan
    if (s < kHeaderBytes / 4) reinterpret_cast<uint32_t *>(a.out)[s] = 0;
    __syncthreads();
    if (s == 0) write_header(a);
}

// floor(x / f) for 1 <= f <= 4096 and x < f * 2^20 (the state after the
// encoder's renormalisation), from r = 1/f rounded to binary64 (relative
// error <= 2^-53): x/f < 2^20, so x*r is within 2^-33 of x/f and the fused
// multiply-add's one rounding adds at most 2^-33 more; fma(x, r, 2^-14) lies
// in (x/f, x/f + 2^-13). The fractional part of x/f is 0 or in
// [1/f, 1 - 1/f] with 1/f >= 2^-12, so truncation gives the exact quotient.
__device__ __forceinline__ uint32_t enc_div(uint32_t x, double rcp) {
    return (uint32_t)__builtin_fma((double)x, rcp, 0x1p-14);
}

// A lane's K symbols of one group, packed four to a word (byte i of the run
// in bits 8*(i%4) of word i/4); positions past the chunk read as 0.
template <int K>
__device__ __forceinline__ void load_run(const uint8_t *sym, uint32_t q0, uint32_t nk,
                                         uint32_t (&w)[(K + 3) / 4]) {
    if (K >= 4 && q0 + (uint32_t)K <= nk) {
        // a full run: one aligned load (q0 and the chunk start are multiples of K)
        if constexpr (K == 16) {
            const uint4 v = *reinterpret_cast<const uint4 *>(sym + q0);
            w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
        } else if constexpr (K == 8) {
            const uint2 v = *reinterpret_cast<const uint2 *>(sym + q0);
            w[0] = v.x; w[1] = v.y;
        } else if constexpr (K == 4) {
            w[0] = *reinterpret_cast<const uint32_t *>(sym + q0);
        }
    } else {
#pragma unroll
        for (int j = 0; j < (K + 3) / 4; ++j) w[j] = 0;
#pragma unroll
        for (int i = 0; i < K; ++i)
            if (q0 + (uint32_t)i < nk) w[i / 4] |= (uint32_t)sym[q0 + i] << (8 * (i % 4));
    }
}

// One wave per chunk: the rANS encoder of the container's coder, steps
// walked backwards. Chunk-local word positions p land in ring[p mod 2048];
// [wpos, nk) holds the chunk's words so far, [flushed, ...) is already in the
// scratch. Whole 8-word blocks above wpos leave 512 words at a time; at the
// end every block that holds a word leaves (the part of a block below wpos,
// or above nk in the tail chunk, is scratch nobody reads).
template <int K>
__global__ void __launch_bounds__(kEncThreads) k_enc_chunks(EncArgs a) {
    __shared__ __align__(16) EncSym tab[256];
    __shared__ __align__(16) uint16_t rings[kEncWaves][kEncRing];
    // the workgroup's table: its chunks lie in one segment (kEncWaves divides seg)
    const uint64_t tsel = a.seg ? (uint64_t)blockIdx.x * kEncWaves / a.seg : 0;
    for (uint32_t i = threadIdx.x; i < 256; i += blockDim.x) tab[i] = at<EncSym>(a.ws, a.w.table)[256 * tsel + i];
    __syncthreads();
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint64_t k = (uint64_t)blockIdx.x * kEncWaves + wave;
    if (k >= a.n_chunks) return;
    uint16_t *ring = rings[wave];
    const uint64_t p0 = k * a.Z;
    const uint32_t nk = (uint32_t)(a.n - p0 < a.Z ? a.n - p0 : a.Z);
    const uint8_t *sym = a.sym + p0;
    uint16_t *scr = at<uint16_t>(a.ws, a.w.scratch) + p0;
    constexpr uint32_t G = 64u * K;
    constexpr int W = (K + 3) / 4;             // packed words per run
    constexpr int D = K >= 4 ? 64 / K : 16;    // groups per batch (64 bytes per lane for K >= 4)
    const uint32_t groups = (nk + G - 1) / G;
    uint32_t x = kStateLow;
    uint32_t wpos = nk;                   // words fill [wpos, nk)
    uint32_t flushed = (uint32_t)round_up(nk, 8);

    // groups ghi-1, ghi-2, ... (D of them, those >= 0) into nxt[0], nxt[1], ...
    uint32_t nxt[D][W];
    auto load_batch = [&](uint32_t ghi) {
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (ghi > (uint32_t)d) load_run<K>(sym, (ghi - 1u - (uint32_t)d) * G + lane * K, nk, nxt[d]);
    };
    typedef __attribute__((address_space(3))) uint16_t lds_u16;
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_u16 *)ring;  // LDS byte address
    auto group = [&](uint32_t g, const uint32_t (&w)[W], bool full) {
        const uint32_t q0 = g * G + lane * K;
        wpos = __builtin_amdgcn_readfirstlane(wpos);  // wave-uniform: keep it scalar
        // the run's table entries do not depend on the state: all K reads
        // are issued before the serial steps. In a group that reaches past
        // the chunk, such a position gets an entry that never emits (16 f
        // field 0xFFFF) and leaves the state as it is (4096 - f and cum
        // fields 0), so the steps need no lane mask.
        EncSym es[K];
#pragma unroll
        for (int i = 0; i < K; ++i) {
            es[i] = tab[(w[i / 4] >> (8 * (i % 4))) & 0xFFu];
            if (!full && q0 + (uint32_t)i >= nk) {
                es[i].fg = 0xFFFFu;  // 16 f field above any reachable x >> 16
                es[i].cum = 0;
            }
        }
#pragma unroll
        for (int i = K - 1; i >= 0; --i) {
            const EncSym e = es[i];
            // x >= f * 2^20  <=>  x >> 16 >= 16 f  (one compare on the high half)
            const bool emit = (x >> 16) >= (e.fg & 0xFFFFu);
            const uint64_t m = __builtin_amdgcn_ballot_w64(emit);
            const uint32_t cnt = (uint32_t)__builtin_popcountll(m);
            wpos -= cnt;
            // slot of this lane's word: wpos + rank (ascending lanes)
            const uint32_t slot = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, wpos));
            // ring address (slot mod 2048 words), then under an exec mask of
            // the emitting lanes (set and restored by the scalar unit) the
            // store of the low 16 bits and x >>= 16
            uint64_t saved;
            uint32_t addr;
            asm volatile("v_and_b32 %1, 0x7ff, %3\n\t"
                         "v_lshl_add_u32 %1, %1, 1, %4\n\t"
                         "s_and_saveexec_b64 %0, %5\n\t"
                         "ds_write_b16 %1, %2\n\t"
                         "v_lshrrev_b32 %2, 16, %2\n\t"
                         "s_mov_b64 exec, %0"
                         : "=&s"(saved), "=&v"(addr), "+v"(x)
                         : "v"(slot), "s"(ring_lds), "s"(m)
                         : "memory", "scc");
            // (x / f) * 4096 + x mod f + cum = x + (x / f) * (4096 - f) + cum
            const uint32_t qq = enc_div(x, e.rcp);
            x = x + __umul24(qq, e.fg >> 16) + e.cum;
        }
        while (flushed >= wpos + kEncFlush) {
            const uint32_t b = flushed - kEncFlush + lane * 8u;
            *reinterpret_cast<uint4 *>(scr + b) =
                *reinterpret_cast<const uint4 *>(ring + (b & (kEncRing - 1u)));
            flushed -= kEncFlush;
        }
    };

    // double-buffered batches: the next D groups' symbols are in flight while
    // the current D groups are encoded
    load_batch(groups);
    for (uint32_t ghi = groups; ghi > 0;) {
        uint32_t cur[D][W];
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
            for (int j = 0; j < W; ++j) cur[d][j] = nxt[d][j];
        const uint32_t glo = ghi > (uint32_t)D ? ghi - (uint32_t)D : 0u;
        if (glo) load_batch(glo);
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (ghi > (uint32_t)d) {
                const uint32_t g = ghi - 1u - (uint32_t)d;
                if ((g + 1u) * G <= nk) group(g, cur[d], true);
                else group(g, cur[d], false);
            }
        }
        ghi = glo;
    }
    {
        const uint32_t lo = wpos & ~7u;
        const uint32_t b = lo + lane * 8u;
        if (b < flushed)
            *reinterpret_cast<uint4 *>(scr + b) = *reinterpret_cast<const uint4 *>(ring + (b & (kEncRing - 1u)));
    }
    at<uint32_t>(a.out, a.sec.states)[k * kLanes + lane] = x;
    if (lane == 0) {
        at<uint32_t>(a.ws, a.w.wstart)[k] = wpos;
        at<uint32_t>(a.ws, a.w.wcount)[k] = nk - wpos;
    }
}

// ---------------------------------------------------------------------------
// Huffman codec (codec 1): code lengths, canonical codewords, chunk encoder.
// ---------------------------------------------------------------------------

// Code lengths of at most 12 bits by package-merge, as the host encoder
// computes them: the present bytes sorted by (count, byte) are the leaves;
// the list of level d (11 = deepest, 0 = top) is the merge of the leaves
// with the packages (consecutive pairs) of the list of level d + 1, a leaf
// first on equal weights; a byte's length is the number of its occurrences
// among the 2n - 2 first items of the top list and, recursively, the
// children of the packages among them. The chosen items of every level form
// a prefix (packages appear in pair order), so level by level only the count
// of leaves in that prefix is needed. Then the canonical codewords
// ((length, byte) order), each stored bit-reversed for the LSB-first packing,
// the length table, the header (one workgroup of 512 threads).
__global__ void __launch_bounds__(512) k_enc_huff(EncArgs a) {
    constexpr uint32_t L = kHuffMaxLen;
    __shared__ uint64_t cnt[256];
    __shared__ __align__(16) uint64_t key[256];  // count << 8 | byte for present bytes, else all ones
    __shared__ uint64_t leafw[256];   // present counts, ascending (bytes ascending on ties)
    __shared__ uint32_t leafsym[256];
    __shared__ uint64_t wbuf[2][512];  // item weights of a level and of the level below
    __shared__ uint8_t kind[L][512];   // 1: the item is a leaf
    __shared__ uint32_t mlev[L];       // leaves in each level's chosen prefix
    __shared__ uint32_t nlen[L + 1];   // codewords of each length
    __shared__ __align__(16) uint32_t len[256];
    __shared__ uint32_t npresent;
    const uint32_t t = threadIdx.x;
    if (t < 256) {
        const uint64_t c = at<uint64_t>(a.ws, a.w.counts)[t];
        cnt[t] = c;
        key[t] = c ? (c << 8 | t) : ~0ull;
        len[t] = 0;
    }
    if (t <= L) nlen[t] = 0;
    if (t == 0) npresent = 0;
    __syncthreads();
    if (t == 0) check_counts(a, cnt);
    if (t < 256 && cnt[t]) {
        // rank by (count, byte): the keys below this byte's (16-byte reads,
        // many in flight)
        const uint64_t kt = key[t];
        const ulonglong2 *k2 = reinterpret_cast<const ulonglong2 *>(key);
        uint32_t r = 0;
#pragma unroll 8
        for (uint32_t q = 0; q < 128; ++q) {
            const ulonglong2 w = k2[q];
            r += (w.x < kt ? 1u : 0u) + (w.y < kt ? 1u : 0u);
        }
        leafw[r] = cnt[t];
        leafsym[r] = t;
        atomicAdd(&npresent, 1u);
    }
    __syncthreads();
    const uint32_t n = npresent;
    uint32_t *hs = at<uint32_t>(a.ws, a.w.table);  // [256] reversed code | length << 16, [256] lone flag
    if (n == 1) {
        // one byte: a zero-bit code, no words at all
        if (t < 256) {
            hs[t] = 0;
            reinterpret_cast<uint16_t *>(a.out + a.sec.freq)[t] = cnt[t] ? kHuffZero : 0;
        }
        if (t == 0) hs[256] = 1;
    } else {
        uint32_t below = 0;  // size of the level below
        for (int d = (int)L - 1; d >= 0; --d) {
            const uint64_t *deep = wbuf[(d + 1) & 1];
            uint64_t *cur = wbuf[d & 1];
            const uint32_t packs = below / 2;
            if (t < n) {  // leaf t: after the packages lighter than it
                const uint64_t w = leafw[t];
                uint32_t lo = 0, hi = packs;
                while (lo < hi) {
                    const uint32_t mid = (lo + hi) / 2;
                    if (deep[2 * mid] + deep[2 * mid + 1] < w) lo = mid + 1;
                    else hi = mid;
                }
                cur[t + lo] = w;
                kind[d][t + lo] = 1;
            }
            if (t < packs) {  // package t: after the leaves not heavier than it
                const uint64_t pw = deep[2 * t] + deep[2 * t + 1];
                uint32_t lo = 0, hi = n;
                while (lo < hi) {
                    const uint32_t mid = (lo + hi) / 2;
                    if (leafw[mid] <= pw) lo = mid + 1;
                    else hi = mid;
                }
                cur[t + lo] = pw;
                kind[d][t + lo] = 0;
            }
            below = n + packs;
            __syncthreads();
        }
        // chosen prefixes, top down
        uint32_t P = 2 * n - 2;
        for (uint32_t d = 0; d < L; ++d) {
            const uint32_t leaves = (uint32_t)__syncthreads_count(t < P && kind[d][t]);
            if (t == 0) mlev[d] = leaves;
            P = 2 * (P - leaves);
        }
        __syncthreads();
        if (t < n) {
            uint32_t l = 0;
            for (uint32_t d = 0; d < L; ++d) l += t < mlev[d] ? 1u : 0u;
            len[leafsym[t]] = l;
            atomicAdd(&nlen[l], 1u);
        }
        __syncthreads();
        if (t < 256) {
            const uint32_t l = len[t];
            uint32_t code = 0;
            if (l) {
                // first codeword of length l, then the rank among its bytes
                uint32_t c = 0;
                for (uint32_t j = 1; j < l; ++j) c = (c + nlen[j]) << 1;
                uint32_t r = 0;
                const uint4 *l4 = reinterpret_cast<const uint4 *>(len);
#pragma unroll 8
                for (uint32_t q = 0; q < 64; ++q) {
                    const uint4 w = l4[q];
                    const uint32_t u = 4 * q;
                    r += (u < t && w.x == l ? 1u : 0u) + (u + 1 < t && w.y == l ? 1u : 0u) +
                         (u + 2 < t && w.z == l ? 1u : 0u) + (u + 3 < t && w.w == l ? 1u : 0u);
                }
                code = c + r;
            }
            hs[t] = l ? (__builtin_bitreverse32(code) >> (32u - l)) | (l << 16) : 0u;
            reinterpret_cast<uint16_t *>(a.out + a.sec.freq)[t] = (uint16_t)l;
        }
        if (t == 0) hs[256] = 0;
    }
    if (t < kHeaderBytes / 4) reinterpret_cast<uint32_t *>(a.out)[t] = 0;
    __syncthreads();
    if (t == 0) write_header(a);
}

constexpr uint32_t kHuffAhead = 28;   // steps a lane's stream is packed ahead of the decoder replay
constexpr uint32_t kWordRow = 33;     // u16 per lane row of the 32-word stream ring
constexpr uint32_t kHuffRing = 1024;  // words of a wave's output ring (flushed every 8 steps)
constexpr uint32_t kHuffBlk = 32;     // steps per unrolled block: the lane's bytes of a block in 8 dwords

// This lane's 32 bytes of the steps [32 b, 32 b + 32), in step order (its
// K-runs of the block's 32 / K groups); positions past the chunk read as 0.
template <int K>
__device__ __forceinline__ void load_block(const uint8_t *sym, uint32_t b, uint32_t lane, uint32_t nk,
                                           uint32_t (&v)[8]) {
    constexpr uint32_t G = 64u * K;
    constexpr int W = (K + 3) / 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0;
#pragma unroll
    for (uint32_t r = 0; r < kHuffBlk / K; ++r) {
        uint32_t w[W];
        load_run<K>(sym, (b * (kHuffBlk / K) + r) * G + lane * K, nk, w);
        if constexpr (K >= 4) {
#pragma unroll
            for (int j = 0; j < W; ++j) v[r * K / 4 + j] = w[j];
        } else {
            v[r * K / 4] |= w[0] << (8 * ((r * K) % 4));
        }
    }
}

__device__ __forceinline__ uint32_t byte_of(const uint32_t (&v)[8], uint32_t j) {
    return (v[j / 4] >> (8 * (j % 4))) & 0xFFu;
}

// One wave per chunk, steps walked forwards, replaying the decoder: at each
// step a lane holding (decoder side) fewer than 12 bits takes its next
// 16-bit word, ascending lanes in one step taking consecutive slots (ballot
// + mbcnt). Every lane packs its own codeword stream (codewords from bit 0
// up, each first bit first) 28 steps ahead of the replay, one codeword per
// step, into a 32-word LDS ring; the word a lane takes is always complete
// by then: when it needs one it holds < 12 bits, so the 16 bits it takes
// end within its next 28 codewords (each at least one bit), and a lane's
// unused packed bits stay below 28 * 12 + 16. The lane's symbol bytes stay
// in registers, 32 steps to a block (the block being replayed, the next
// one, which the packing reaches into, and one in flight), and both walks
// look their (reversed codeword, length) up in the LDS code table; a step
// past the lane's last symbol looks up the empty entry (table index 256,
// which holds 0), so no step needs a lane mask. At its end step the lane's
// pack writes the zero-padded partial word and one zero word after it: a
// lane asks for at most one word past its stream (after it, it holds >= 16
// bits more than it will consume). Words leave through a 1,024-word LDS
// output ring, 512 at a time, checked every 8 steps (a step adds at most 64).
template <int K>
__global__ void __launch_bounds__(kEncThreads) k_enc_hchunks(EncArgs a) {
    __shared__ uint32_t hs[257];
    __shared__ __align__(16) uint16_t wordring[kEncWaves][64 * kWordRow];
    __shared__ __align__(16) uint16_t rings[kEncWaves][kHuffRing];
    for (uint32_t i = threadIdx.x; i < 257; i += blockDim.x) hs[i] = at<uint32_t>(a.ws, a.w.table)[i];
    __syncthreads();
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint64_t k = (uint64_t)blockIdx.x * kEncWaves + wave;
    if (k >= a.n_chunks) return;
    const uint64_t p0 = k * a.Z;
    const uint32_t nk = (uint32_t)(a.n - p0 < a.Z ? a.n - p0 : a.Z);
    uint32_t words = 0;
    if (hs[256] == 0) {
        const uint8_t *sym = a.sym + p0;
        uint16_t *scr = at<uint16_t>(a.ws, a.w.scratch) + p0;
        uint16_t *ring = rings[wave];
        uint16_t *wr = &wordring[wave][lane * kWordRow];
        constexpr uint32_t G = 64u * K;
        const uint32_t groups = (nk + G - 1) / G;
        const uint32_t full = nk / G;          // groups with every lane's run inside the chunk
        const uint32_t tail = nk - full * G;   // symbols of the partial group
        // this lane's symbols in the partial group; the step its stream ends
        const uint32_t mine = tail > lane * K ? (tail - lane * K < (uint32_t)K ? tail - lane * K : (uint32_t)K) : 0u;
        const uint32_t endst = full * K + mine;
        const uint32_t nblk = (groups * K + kHuffBlk - 1) / kHuffBlk;  // steps past the chunk do nothing
        const uint32_t all_in = full * K;      // steps below it lie in every lane's stream
        // (reversed codeword | length << 16) of step st's byte; CHECK: the
        // empty entry from the lane's end step on
        auto entry = [&](uint32_t byte, uint32_t st, auto check) -> uint32_t {
            if constexpr (decltype(check)::value) return hs[st < endst ? byte : 256u];
            else return hs[byte];
        };
        uint32_t acc = 0, ab = 0;  // packed bits not yet in a word, their count
        uint32_t wprod = 0;        // words packed
        auto pack = [&](uint32_t e, uint32_t st) {
            acc |= (e & 0xFFFu) << ab;
            ab += e >> 16;
            if (ab >= 16u) {
                wr[wprod & 31u] = (uint16_t)acc;
                ++wprod;
                acc >>= 16;
                ab -= 16u;
            }
            if (st == endst) {
                // the stream ended before this step (whose entry is empty)
                if (ab != 0u) {
                    wr[wprod & 31u] = (uint16_t)acc;
                    ++wprod;
                }
                wr[wprod & 31u] = 0;
                acc = 0;
                ab = 0;
            }
        };
        uint32_t cur[8], nxt[8], pre[8];
        load_block<K>(sym, 0, lane, nk, cur);
        load_block<K>(sym, 1, lane, nk, nxt);
        load_block<K>(sym, 2, lane, nk, pre);
#pragma unroll
        for (uint32_t st = 0; st < kHuffAhead; ++st) pack(entry(byte_of(cur, st), st, std::true_type{}), st);
        uint32_t held = 0;                    // the decoder's bits at this step
        uint32_t wnext = 0;                   // this lane's next word to hand out
        uint32_t ptr = 0, flushed = 0;        // words written; words already in the scratch
        for (uint32_t bk = 0; bk < nblk; ++bk) {
            auto body = [&](auto check) {
                constexpr bool C = decltype(check)::value;
#pragma unroll
                for (uint32_t j = 0; j < kHuffBlk; ++j) {
                    const uint32_t t = bk * kHuffBlk + j;
                    // read before this step's packing: a word the lane takes
                    // now was complete 28 steps ahead, as was the zero word
                    // after its stream (the stream ends within 12 steps then)
                    const uint16_t w = wr[wnext & 31u];
                    const uint32_t len = entry(byte_of(cur, j), t, check) >> 16;
                    const uint32_t jp = j + kHuffAhead;
                    uint32_t bp;
                    if (jp < kHuffBlk) bp = byte_of(cur, jp);
                    else bp = byte_of(nxt, jp - kHuffBlk);
                    pack(entry(bp, t + kHuffAhead, check), t + kHuffAhead);
                    const bool need = C ? held < 12u && t < endst : held < 12u;
                    const uint64_t m = __builtin_amdgcn_ballot_w64(need);
                    if (need) {
                        const uint32_t slot = __builtin_amdgcn_mbcnt_hi(
                            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, ptr));
                        ring[slot & (kHuffRing - 1u)] = w;
                        ++wnext;
                        held += 16u;
                    }
                    held -= len;
                    ptr += (uint32_t)__builtin_popcountll(m);
                    if (j % 8u == 7u) {
                        while (ptr >= flushed + kEncFlush) {
                            const uint32_t b = flushed + lane * 8u;
                            *reinterpret_cast<uint4 *>(scr + b) =
                                *reinterpret_cast<const uint4 *>(ring + (b & (kHuffRing - 1u)));
                            flushed += kEncFlush;
                        }
                    }
                }
            };
            // every step of this block and of the next (which the packing reaches) inside every lane's stream
            if ((bk + 2u) * kHuffBlk <= all_in) body(std::false_type{});
            else body(std::true_type{});
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                cur[i] = nxt[i];
                nxt[i] = pre[i];
            }
            if (bk + 3u < nblk) load_block<K>(sym, bk + 3u, lane, nk, pre);
        }
        // the last words (the rest of their 8-word block is scratch nobody reads)
        const uint32_t b = flushed + lane * 8u;
        if (b < ptr) *reinterpret_cast<uint4 *>(scr + b) = *reinterpret_cast<const uint4 *>(ring + (b & (kHuffRing - 1u)));
        words = ptr;
    }
    if (lane == 0) {
        at<uint32_t>(a.ws, a.w.wstart)[k] = 0;
        at<uint32_t>(a.ws, a.w.wcount)[k] = words;
    }
}

// Directory, n_words and the offsets that follow the words (one workgroup).
__global__ void __launch_bounds__(1024) k_enc_scan(EncArgs a) {
    __shared__ uint64_t part[1024];
    __shared__ uint64_t carry;
    const uint32_t t = threadIdx.x;
    if (t == 0) carry = 0;
    __syncthreads();
    const uint32_t *wcount = at<uint32_t>(a.ws, a.w.wcount);
    uint64_t *first = at<uint64_t>(a.ws, a.w.first);
    for (uint64_t base = 0; base < a.n_chunks; base += 1024) {
        const uint64_t k = base + t;
        uint64_t cnt = 0, padded = 0;
        if (k < a.n_chunks) {
            cnt = wcount[k];
            padded = round_up(cnt, kWordPad);
        }
        part[t] = padded;
        __syncthreads();
        for (uint32_t o = 1; o < 1024; o <<= 1) {  // inclusive scan
            const uint64_t v = t >= o ? part[t - o] : 0;
            __syncthreads();
            part[t] += v;
            __syncthreads();
        }
        if (k < a.n_chunks) {
            const uint64_t fst = carry + part[t] - padded;
            first[k] = fst;
            uint8_t *d = a.out + a.sec.dir + kDirEntryBytes * k;
            *reinterpret_cast<uint64_t *>(d) = fst;
            *reinterpret_cast<uint32_t *>(d + 8) = (uint32_t)cnt;
            *reinterpret_cast<uint32_t *>(d + 12) = 0;
        }
        __syncthreads();
        if (t == 1023) carry += part[1023];
        __syncthreads();
    }
    if (t == 0) {
        const uint64_t n_words = carry;
        const uint64_t esc_idx = round_up(a.sec.words + 2 * n_words, kSectionAlign);
        const uint64_t esc_val = round_up(esc_idx + 8 * a.n_esc, kSectionAlign);
        const uint64_t total = round_up(esc_val + 2 * a.n_esc, kSectionAlign);
        uint8_t *b = a.out;
        *reinterpret_cast<uint64_t *>(b + H_NWORDS) = n_words;
        *reinterpret_cast<uint64_t *>(b + H_OFF_ESC_IDX) = esc_idx;
        *reinterpret_cast<uint64_t *>(b + H_OFF_ESC_VAL) = esc_val;
        *reinterpret_cast<uint64_t *>(b + H_TOTAL) = total;
        uint64_t *misc = at<uint64_t>(a.ws, a.w.misc);
        misc[0] = n_words;
        misc[1] = total;
        if (a.out_len) *a.out_len = total;
        // the escape codes counted by the table kernels against the list
        if (misc[2] != (a.esc_enabled ? a.n_esc : 0)) flag(a.status, EQ_DEV_BAD_INPUT);
    }
}

// Eight words starting S words into the 16 words held by lo and hi.
template <uint32_t S>
__device__ __forceinline__ uint4 words_at(uint4 lo, uint4 hi) {
    const uint32_t d[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    constexpr uint32_t h = S / 2;
    uint32_t o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
        o[t] = (S & 1u) ? __builtin_amdgcn_alignbyte(d[h + t + 1], d[h + t], 2) : d[h + t];
    return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ uint4 words_at(uint32_t s, uint4 lo, uint4 hi) {
    switch (s) {  // wave-uniform
        case 0: return words_at<0>(lo, hi);
        case 1: return words_at<1>(lo, hi);
        case 2: return words_at<2>(lo, hi);
        case 3: return words_at<3>(lo, hi);
        case 4: return words_at<4>(lo, hi);
        case 5: return words_at<5>(lo, hi);
        case 6: return words_at<6>(lo, hi);
        default: return words_at<7>(lo, hi);
    }
}

// Words to their final place (one wave per chunk, 8 words per lane and
// block; padding words are zero), then the escape list and the zero gaps
// between sections (workgroup 0). The chunk's words start at scratch
// position wpos, s = wpos mod 8 words past an aligned block; the read of the
// block after the last one stays inside the scratch's 16 spare words.
__global__ void __launch_bounds__(kEncThreads) k_enc_copy(EncArgs a) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t k = (uint64_t)blockIdx.x * kEncWaves + (threadIdx.x >> 6);
    if (k < a.n_chunks) {
        const uint64_t p0 = k * a.Z;
        const uint32_t ws = at<uint32_t>(a.ws, a.w.wstart)[k];
        const uint32_t cnt = at<uint32_t>(a.ws, a.w.wcount)[k];
        const uint32_t nblk = (uint32_t)round_up(cnt, kWordPad) / 8u;
        const uint32_t s = ws & 7u;
        const uint4 *src = reinterpret_cast<const uint4 *>(at<uint16_t>(a.ws, a.w.scratch) + p0 + (ws - s));
        uint4 *dst = reinterpret_cast<uint4 *>(at<uint16_t>(a.out, a.sec.words) + at<uint64_t>(a.ws, a.w.first)[k]);
        constexpr uint32_t U = 4;  // blocks per lane in flight
        for (uint32_t j0 = 0; j0 < nblk; j0 += 64u * U) {
            uint4 lo[U], hi[U];
#pragma unroll
            for (uint32_t u = 0; u < U; ++u) {
                const uint32_t j = j0 + u * 64u + lane;
                if (j < nblk) {
                    lo[u] = src[j];
                    hi[u] = src[j + 1];
                }
            }
#pragma unroll
            for (uint32_t u = 0; u < U; ++u) {
                const uint32_t j = j0 + u * 64u + lane;
                if (j < nblk) {
                    uint4 v = words_at(s, lo[u], hi[u]);
                    const uint32_t left = cnt - 8u * j;  // words of the chunk in this block
                    if (left < 8u) {
                        uint32_t o[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (uint32_t t = 0; t < 4; ++t) {
                            if (2u * t >= left) o[t] = 0;
                            else if (2u * t + 1u == left) o[t] &= 0xFFFFu;
                        }
                        v = make_uint4(o[0], o[1], o[2], o[3]);
                    }
                    dst[j] = v;
                }
            }
        }
    }
    if (blockIdx.x != 0) return;
    const uint64_t *misc = at<uint64_t>(a.ws, a.w.misc);
    const uint64_t n_words = misc[0], total = misc[1];
    const uint64_t esc_idx = round_up(a.sec.words + 2 * n_words, kSectionAlign);
    const uint64_t esc_val = round_up(esc_idx + 8 * a.n_esc, kSectionAlign);
    for (uint64_t e = threadIdx.x; e < a.n_esc; e += blockDim.x) {
        at<uint64_t>(a.out, esc_idx)[e] = a.esc_idx[e];
        at<uint16_t>(a.out, esc_val)[e] = a.esc_val[e];
    }
    // zero gaps: after scales, after the directory, after the padded words,
    // after each escape section, up to the total size
    const uint64_t gaps[4][2] = {{a.sec.scales + 4 * a.rows, a.sec.dir},
                                 {a.sec.dir + kDirEntryBytes * a.n_chunks, a.sec.states},
                                 {a.sec.words + 2 * n_words, esc_idx},
                                 {esc_idx + 8 * a.n_esc, esc_val}};
    for (int g = 0; g < 4; ++g)
        for (uint64_t i = gaps[g][0] + threadIdx.x; i < gaps[g][1]; i += blockDim.x) a.out[i] = 0;
    for (uint64_t i = esc_val + 2 * a.n_esc + threadIdx.x; i < total; i += blockDim.x) a.out[i] = 0;
}

// The encoder's scratch for callers that cannot allocate: one array per GPU,
// held for the life of the process, shared by every call on that GPU.
static __device__ __align__(256) uint8_t scratch[EQ_ENCODE_STATIC_SCRATCH_BYTES];

// Device address of `scratch` on each GPU, looked up once per GPU with that
// GPU current. The array's name in host code is only a stand-in for the
// symbol: kernels get this address, never the name.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

void *scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

template <int K>
void launch_chunks(uint32_t grid, hipStream_t s, const EncArgs &a) {
    if (a.codec == kCodecHuffman) hipLaunchKernelGGL(k_enc_hchunks<K>, dim3(grid), dim3(kEncThreads), 0, s, a);
    else hipLaunchKernelGGL(k_enc_chunks<K>, dim3(grid), dim3(kEncThreads), 0, s, a);
}

}  // namespace

extern "C" {

uint64_t eq_encode_device_bound(uint64_t rows, uint64_t cols, uint32_t chunk_symbols, uint64_t n_esc) {
    if (rows == 0 || cols == 0 || chunk_symbols == 0 || cols > (1ull << 40) / rows) return 0;
    const uint64_t n = rows * cols;
    const uint64_t n_chunks = (n + chunk_symbols - 1) / chunk_symbols;
    // the largest variant: rANS lane states and the most tables
    return layout(rows, n_chunks, n + kWordPad * n_chunks, n_esc, kCodecRans, max_tables(n_chunks)).total;
}

uint64_t eq_encode_device_workspace(uint64_t rows, uint64_t cols, uint32_t chunk_symbols) {
    if (rows == 0 || cols == 0 || chunk_symbols == 0 || cols > (1ull << 40) / rows) return 0;
    const uint64_t n = rows * cols;
    return ws_layout(n, (n + chunk_symbols - 1) / chunk_symbols).total;
}

eq_status eq_encode_device(const eq_tensor_desc *d, const uint8_t *d_symbols, const float *d_scales,
                           const uint64_t *d_esc_idx, const uint16_t *d_esc_bf16, uint64_t n_esc,
                           void *d_workspace, uint64_t workspace_bytes, void *d_out, uint64_t cap,
                           uint64_t *d_out_len, uint32_t *d_status, void *stream) {
    if (!d || !d_symbols || !d_scales || !d_workspace || !d_out) return EQ_EINVAL;
    if (n_esc && (!d_esc_idx || !d_esc_bf16)) return EQ_EINVAL;
    if (d->codec != kCodecRans && d->codec != kCodecHuffman) return EQ_EINVAL;
    // adaptive tables: a multiple of 8 chunks per table, rANS only
    if (d->seg_chunks && (d->seg_chunks % 8 || d->codec != kCodecRans)) return EQ_EINVAL;
    if (d->reserved) return EQ_EINVAL;
    if (d->dtype != EQ_DTYPE_INT8 && d->dtype != EQ_DTYPE_E4M3) return EQ_EINVAL;
    if (d->rows == 0 || d->cols == 0 || d->cols > (1ull << 40) / d->rows) return EQ_EINVAL;
    if (!valid_lane_run(d->lane_run)) return EQ_EINVAL;
    const uint32_t K = d->lane_run, Z = d->chunk_symbols;
    if (Z == 0 || Z > kMaxChunk || Z % (kLanes * K) != 0) return EQ_EINVAL;
    if ((!d->esc_enabled && n_esc) || (d->esc_enabled && d->esc_code > 255)) return EQ_EINVAL;
    if ((reinterpret_cast<uintptr_t>(d_symbols) | reinterpret_cast<uintptr_t>(d_workspace) |
         reinterpret_cast<uintptr_t>(d_out)) & 15u)
        return EQ_EINVAL;
    const uint64_t n = d->rows * d->cols;
    const uint64_t n_chunks = (n + Z - 1) / Z;
    if (cap < eq_encode_device_bound(d->rows, d->cols, Z, n_esc)) return EQ_ERANGE;
    const WsLayout w = ws_layout(n, n_chunks);
    if (workspace_bytes < w.total) return EQ_ERANGE;

    EncArgs a{};
    a.sym = d_symbols;
    a.scales = d_scales;
    a.esc_idx = d_esc_idx;
    a.esc_val = d_esc_bf16;
    a.ws = static_cast<uint8_t *>(d_workspace);
    a.out = static_cast<uint8_t *>(d_out);
    a.out_len = d_out_len;
    a.status = d_status;
    a.rows = d->rows;
    a.cols = d->cols;
    a.n = n;
    a.n_chunks = n_chunks;
    a.n_esc = n_esc;
    a.Z = Z;
    a.K = K;
    a.dtype = d->dtype;
    a.esc_enabled = d->esc_enabled;
    a.esc_code = d->esc_code;
    a.codec = d->codec;
    a.seg = d->seg_chunks;
    a.n_tab = n_tables(n_chunks, a.seg);
    a.seg_syms = a.seg ? (uint64_t)a.seg * Z : n;
    a.w = w;
    // fields before the words do not depend on the counts
    a.sec = layout(d->rows, n_chunks, 0, 0, a.codec, a.n_tab);

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t cgrid = (uint32_t)((n_chunks + kEncWaves - 1) / kEncWaves);
    if (n_chunks > 0xFFFFFFFFull / 4) return EQ_EINVAL;
    if (a.n_tab > 65535) return EQ_EINVAL;
    hipLaunchKernelGGL(k_enc_check, dim3(64), dim3(256), 0, s, a);
    // one grid row per table; about 32 KiB of symbols per workgroup and pass,
    // at most kHistMaxGrid workgroups in all (and at least one per table)
    const uint64_t hg = (a.seg_syms + 32767) / 32768;
    const uint64_t hcap = kHistMaxGrid / a.n_tab ? kHistMaxGrid / a.n_tab : 1;
    const uint32_t hgrid = (uint32_t)(hg < hcap ? (hg ? hg : 1) : hcap);
    hipLaunchKernelGGL(k_enc_hist, dim3(hgrid, (uint32_t)a.n_tab), dim3(256), 0, s, a);
    if (a.codec == kCodecHuffman) hipLaunchKernelGGL(k_enc_huff, dim3(1), dim3(512), 0, s, a);
    else hipLaunchKernelGGL(k_enc_quant, dim3((uint32_t)a.n_tab), dim3(256), 0, s, a);
    switch (K) {
        case 1: launch_chunks<1>(cgrid, s, a); break;
        case 2: launch_chunks<2>(cgrid, s, a); break;
        case 4: launch_chunks<4>(cgrid, s, a); break;
        case 8: launch_chunks<8>(cgrid, s, a); break;
        default: launch_chunks<16>(cgrid, s, a); break;
    }
    hipLaunchKernelGGL(k_enc_scan, dim3(1), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(k_enc_copy, dim3(cgrid), dim3(kEncThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? EQ_OK : EQ_EHIP;
}

eq_status eq_encode_device_static(const eq_tensor_desc *d, const uint8_t *d_symbols, const float *d_scales,
                                  const uint64_t *d_esc_idx, const uint16_t *d_esc_bf16, uint64_t n_esc,
                                  void *d_out, uint64_t cap, uint64_t *d_out_len, uint32_t *d_status,
                                  void *stream) {
    if (!d || d->rows == 0 || d->cols == 0 || d->chunk_symbols == 0) return EQ_EINVAL;
    const uint64_t need = eq_encode_device_workspace(d->rows, d->cols, d->chunk_symbols);
    if (need == 0) return EQ_EINVAL;
    if (need > EQ_ENCODE_STATIC_SCRATCH_BYTES) return EQ_ERANGE;
    void *ws = scratch_on_current_device();
    if (!ws) return EQ_EHIP;
    return eq_encode_device(d, d_symbols, d_scales, d_esc_idx, d_esc_bf16, n_esc, ws,
                            EQ_ENCODE_STATIC_SCRATCH_BYTES, d_out, cap, d_out_len, d_status, stream);
}

}  // extern "C"
