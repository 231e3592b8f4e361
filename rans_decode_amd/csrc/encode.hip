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
// Pipeline (one stream, seven launches, no host synchronisation):
//   zero    workspace counters
//   hist    per-workgroup LDS histograms -> 256 u64 counts
//   check   super-weight list and scales (and copy the scales)
//   quant   the quantiser (rule stated in include/eq.h) -> freq/cum, header,
//           frequency section
//   chunks  one wave per chunk: lanes walk the chunk's steps backwards; a lane
//           whose state reached f * 2^20 emits its low 16 bits first; the
//           words of one step take consecutive slots in ascending lane order
//           (ballot + mbcnt), filled from the end of the chunk's scratch
//           region, so they come out in the decoder's reading order
//   scan    one workgroup: padded word counts -> directory, n_words, the
//           offsets that depend on it, the total size
//   copy    words to their final place, escape list, zero gaps
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/eq.h"
#include "format.hpp"

namespace {

using namespace eqfmt;

constexpr int kEncWaves = 4;                   // chunks per workgroup
constexpr int kEncThreads = 64 * kEncWaves;

// Workspace layout (bytes from the start; all 256-byte aligned).
struct WsLayout {
    uint64_t counts;   // 256 x u64
    uint64_t table;    // 256 x u32: freq | cum << 16
    uint64_t misc;     // u64 n_words, u64 total
    uint64_t wstart;   // n_chunks x u32: first word of the chunk inside its scratch region
    uint64_t first;    // n_chunks x u64: first word in the container
    uint64_t scratch;  // n x u16 (chunk k uses [k*Z, k*Z + nk))
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
    w.counts = place(256 * 8);
    w.table = place(256 * 4);
    w.misc = place(16);
    w.wstart = place(n_chunks * 4);
    w.first = place(n_chunks * 8);
    w.scratch = place(n * 2);
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

__global__ void k_enc_zero(EncArgs a) {
    const uint32_t i = threadIdx.x;
    if (i < 256) at<uint64_t>(a.ws, a.w.counts)[i] = 0;
    if (i < 2) at<uint64_t>(a.ws, a.w.misc)[i] = 0;
}

// Histogram: each wave keeps its own 256 LDS counters (fewer collisions on
// the few frequent codes), 16 symbols per thread per iteration.
__global__ void __launch_bounds__(256) k_enc_hist(EncArgs a) {
    __shared__ uint32_t h[4][256];
    const uint32_t wave = threadIdx.x >> 6;
    for (uint32_t i = threadIdx.x; i < 4 * 256; i += blockDim.x) (&h[0][0])[i] = 0;
    __syncthreads();
    const uint64_t n16 = a.n / 16;
    const uint4 *v = reinterpret_cast<const uint4 *>(a.sym);
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const uint4 q = v[i];
        const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int b = 0; b < 4; ++b) atomicAdd(&h[wave][(wd[j] >> (8 * b)) & 0xFFu], 1u);
    }
    for (uint64_t i = n16 * 16 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n; i += stride)
        atomicAdd(&h[wave][a.sym[i]], 1u);
    __syncthreads();
    if (threadIdx.x < 256) {
        const uint32_t s = threadIdx.x;
        const uint64_t c = (uint64_t)h[0][s] + h[1][s] + h[2][s] + h[3][s];
        if (c) atomicAdd(reinterpret_cast<unsigned long long *>(at<uint64_t>(a.ws, a.w.counts) + s),
                         (unsigned long long)c);
    }
}

// Super-weight list (ascending, in range, escape code at each index) and
// finite scales; the scales are copied into the container on the way.
__global__ void k_enc_check(EncArgs a) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
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

// Quantiser + header + frequency section (one workgroup of 256 threads, one
// symbol per thread):
//   f_s = max(1, floor(c_s * 4096 / N)) for present bytes; a shortfall goes
//   +1 to the present bytes ranked first by (remainder c_s * 4096 mod N
//   descending, byte ascending); an excess is taken -1 at a time from the
//   largest f_s > 1 (smallest byte among equals).
__global__ void __launch_bounds__(256) k_enc_quant(EncArgs a) {
    __shared__ uint64_t rem[256];
    __shared__ int32_t f[256];
    __shared__ int32_t red_v[256];
    __shared__ int32_t red_s[256];
    __shared__ int32_t total;
    const uint32_t s = threadIdx.x;
    const uint64_t *counts = at<uint64_t>(a.ws, a.w.counts);
    const uint64_t c = counts[s];
    const uint64_t scaled = c * (uint64_t)kProbScale;
    const bool present = c != 0;
    int32_t fs = 0;
    if (present) {
        const uint64_t q = scaled / a.n;
        fs = q > 1 ? (int32_t)q : 1;
    }
    f[s] = fs;
    rem[s] = present ? scaled % a.n : 0;
    if (s == 0) total = 0;
    __syncthreads();
    atomicAdd(&total, fs);
    __syncthreads();
    const int32_t deficit = (int32_t)kProbScale - total;
    if (deficit > 0) {
        if (present) {
            uint32_t rank = 0;
            for (uint32_t t = 0; t < 256; ++t)
                if (counts[t] && (rem[t] > rem[s] || (rem[t] == rem[s] && t < s))) ++rank;
            if ((int32_t)rank < deficit) f[s] = fs + 1;
        }
        __syncthreads();
    } else {
        for (int32_t d = deficit; d < 0; ++d) {
            // argmax of f over f > 1, smallest byte among equals
            red_v[s] = f[s] > 1 ? f[s] : -1;
            red_s[s] = (int32_t)s;
            __syncthreads();
            for (uint32_t o = 128; o > 0; o >>= 1) {
                if (s < o) {
                    const int32_t v2 = red_v[s + o], s2 = red_s[s + o];
                    if (v2 > red_v[s] || (v2 == red_v[s] && s2 < red_s[s])) {
                        red_v[s] = v2;
                        red_s[s] = s2;
                    }
                }
                __syncthreads();
            }
            if (s == 0 && red_v[0] > 0) f[red_s[0]] -= 1;
            if (s == 0 && red_v[0] <= 0) flag(a.status, EQ_DEV_BAD_INPUT);
            __syncthreads();
        }
    }
    // cumulative frequencies (serial over 256 entries, thread 0)
    __shared__ uint32_t cum[257];
    if (s == 0) {
        uint32_t acc = 0;
        for (int t = 0; t < 256; ++t) {
            cum[t] = acc;
            acc += (uint32_t)f[t];
        }
        cum[256] = acc;
        // E4M3 NaN codes are only allowed as the escape code; the escape count
        // must match the list
        if (a.dtype == EQ_DTYPE_E4M3) {
            if (counts[0x7F] && !(a.esc_enabled && a.esc_code == 0x7Fu)) flag(a.status, EQ_DEV_BAD_INPUT);
            if (counts[0xFF] && !(a.esc_enabled && a.esc_code == 0xFFu)) flag(a.status, EQ_DEV_BAD_INPUT);
        }
        if (a.esc_enabled ? counts[a.esc_code] != a.n_esc : a.n_esc != 0) flag(a.status, EQ_DEV_BAD_INPUT);
    }
    __syncthreads();
    at<uint32_t>(a.ws, a.w.table)[s] = (uint32_t)f[s] | (cum[s] << 16);
    reinterpret_cast<uint16_t *>(a.out + a.sec.freq)[s] = (uint16_t)f[s];
    // header: every byte written; n_words-dependent fields are filled by k_enc_scan
    if (s < kHeaderBytes / 4) reinterpret_cast<uint32_t *>(a.out)[s] = 0;
    __syncthreads();
    if (s == 0) {
        uint8_t *b = a.out;
        *reinterpret_cast<uint32_t *>(b + H_MAGIC) = kMagic;
        *reinterpret_cast<uint16_t *>(b + H_VERSION) = kVersion;
        b[H_DTYPE] = (uint8_t)a.dtype;
        b[H_FLAGS] = a.esc_enabled ? 1 : 0;
        *reinterpret_cast<uint64_t *>(b + H_ROWS) = a.rows;
        *reinterpret_cast<uint64_t *>(b + H_COLS) = a.cols;
        *reinterpret_cast<uint64_t *>(b + H_N) = a.n;
        *reinterpret_cast<uint32_t *>(b + H_CHUNK) = a.Z;
        *reinterpret_cast<uint32_t *>(b + H_LANE_RUN) = a.K;
        *reinterpret_cast<uint32_t *>(b + H_LANES) = kLanes;
        *reinterpret_cast<uint32_t *>(b + H_PROB_BITS) = kProbBits;
        *reinterpret_cast<uint64_t *>(b + H_NCHUNKS) = a.n_chunks;
        *reinterpret_cast<uint64_t *>(b + H_NESC) = a.n_esc;
        b[H_ESC_CODE] = a.esc_enabled ? (uint8_t)a.esc_code : 0;
        *reinterpret_cast<uint64_t *>(b + H_OFF_FREQ) = a.sec.freq;
        *reinterpret_cast<uint64_t *>(b + H_OFF_SCALES) = a.sec.scales;
        *reinterpret_cast<uint64_t *>(b + H_OFF_DIR) = a.sec.dir;
        *reinterpret_cast<uint64_t *>(b + H_OFF_STATES) = a.sec.states;
        *reinterpret_cast<uint64_t *>(b + H_OFF_WORDS) = a.sec.words;
        *reinterpret_cast<uint32_t *>(b + H_CODEC) = kCodecRans;
    }
}

// One wave per chunk: the rANS encoder of the container's coder, steps
// walked backwards.
template <int K>
__global__ void __launch_bounds__(kEncThreads) k_enc_chunks(EncArgs a) {
    __shared__ uint32_t tab[256];
    for (uint32_t i = threadIdx.x; i < 256; i += blockDim.x) tab[i] = at<uint32_t>(a.ws, a.w.table)[i];
    __syncthreads();
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t k = (uint64_t)blockIdx.x * kEncWaves + (threadIdx.x >> 6);
    if (k >= a.n_chunks) return;
    const uint64_t p0 = k * a.Z;
    const uint32_t nk = (uint32_t)(a.n - p0 < a.Z ? a.n - p0 : a.Z);
    const uint8_t *sym = a.sym + p0;
    uint16_t *scr = at<uint16_t>(a.ws, a.w.scratch) + p0;
    constexpr uint32_t G = 64u * K;
    const uint32_t groups = (nk + G - 1) / G;
    uint32_t x = kStateLow;
    uint32_t wpos = nk;  // words fill scr[wpos, nk)
    for (uint32_t g = groups; g-- > 0;) {
        const uint32_t q0 = g * G + lane * K;
        uint8_t run[K];
#pragma unroll
        for (int i = 0; i < K; ++i) run[i] = q0 + (uint32_t)i < nk ? sym[q0 + i] : 0;
#pragma unroll
        for (int i = K - 1; i >= 0; --i) {
            const bool active = q0 + (uint32_t)i < nk;
            const uint32_t e = tab[run[i]];
            const uint32_t fr = e & 0xFFFFu, cu = e >> 16;
            const bool emit = active && (uint64_t)x >= ((uint64_t)fr << 20);
            const uint64_t m = __builtin_amdgcn_ballot_w64(emit);
            const uint32_t cnt = (uint32_t)__builtin_popcountll(m);
            const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (emit) {
                scr[wpos - cnt + rank] = (uint16_t)(x & 0xFFFFu);
                x >>= 16;
            }
            wpos -= cnt;
            if (active) {
                const uint32_t qq = x / fr;
                x = (qq << kProbBits) + (x - qq * fr) + cu;
            }
        }
    }
    at<uint32_t>(a.out, a.sec.states)[k * kLanes + lane] = x;
    if (lane == 0) at<uint32_t>(a.ws, a.w.wstart)[k] = wpos;
}

// Directory, n_words and the offsets that follow the words (one workgroup).
__global__ void __launch_bounds__(1024) k_enc_scan(EncArgs a) {
    __shared__ uint64_t part[1024];
    __shared__ uint64_t carry;
    const uint32_t t = threadIdx.x;
    if (t == 0) carry = 0;
    __syncthreads();
    const uint32_t *wstart = at<uint32_t>(a.ws, a.w.wstart);
    uint64_t *first = at<uint64_t>(a.ws, a.w.first);
    for (uint64_t base = 0; base < a.n_chunks; base += 1024) {
        const uint64_t k = base + t;
        uint64_t cnt = 0, padded = 0;
        if (k < a.n_chunks) {
            const uint32_t nk = (uint32_t)(a.n - k * a.Z < a.Z ? a.n - k * a.Z : a.Z);
            cnt = nk - wstart[k];
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
    }
}

// Words to their final place (one wave per chunk; zero padding words), then
// the escape list and the zero gaps between sections (workgroup 0).
__global__ void __launch_bounds__(kEncThreads) k_enc_copy(EncArgs a) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint64_t k = (uint64_t)blockIdx.x * kEncWaves + (threadIdx.x >> 6);
    if (k < a.n_chunks) {
        const uint64_t p0 = k * a.Z;
        const uint32_t nk = (uint32_t)(a.n - p0 < a.Z ? a.n - p0 : a.Z);
        const uint32_t ws = at<uint32_t>(a.ws, a.w.wstart)[k];
        const uint32_t cnt = nk - ws;
        const uint32_t padded = (uint32_t)round_up(cnt, kWordPad);
        const uint16_t *src = at<uint16_t>(a.ws, a.w.scratch) + p0 + ws;
        uint16_t *dst = at<uint16_t>(a.out, a.sec.words) + at<uint64_t>(a.ws, a.w.first)[k];
        for (uint32_t i = lane; i < padded; i += 64u) dst[i] = i < cnt ? src[i] : 0;
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

template <int K>
void launch_chunks(uint32_t grid, hipStream_t s, const EncArgs &a) {
    hipLaunchKernelGGL(k_enc_chunks<K>, dim3(grid), dim3(kEncThreads), 0, s, a);
}

}  // namespace

extern "C" {

uint64_t eq_encode_device_bound(uint64_t rows, uint64_t cols, uint32_t chunk_symbols, uint64_t n_esc) {
    if (rows == 0 || cols == 0 || chunk_symbols == 0 || cols > (1ull << 40) / rows) return 0;
    const uint64_t n = rows * cols;
    const uint64_t n_chunks = (n + chunk_symbols - 1) / chunk_symbols;
    return layout(rows, n_chunks, n + kWordPad * n_chunks, n_esc).total;
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
    if (d->codec != kCodecRans || d->seg_chunks) return EQ_EUNSUPPORTED;
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
    a.w = w;
    a.sec = layout(d->rows, n_chunks, 0, 0);  // fields before the words do not depend on the counts

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t cgrid = (uint32_t)((n_chunks + kEncWaves - 1) / kEncWaves);
    if (n_chunks > 0xFFFFFFFFull / 4) return EQ_EINVAL;
    hipLaunchKernelGGL(k_enc_zero, dim3(1), dim3(256), 0, s, a);
    const uint64_t hgrid = (n / 16 + 255) / 256;
    hipLaunchKernelGGL(k_enc_hist, dim3((uint32_t)(hgrid < 2048 ? (hgrid ? hgrid : 1) : 2048)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_enc_check, dim3(64), dim3(256), 0, s, a);
    hipLaunchKernelGGL(k_enc_quant, dim3(1), dim3(256), 0, s, a);
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

}  // extern "C"
