// host_codec.cpp -- host side of libeq: frequency tables, the offline
// container encoder and container validation.
//
// The pages' encoding step ("Float8@2bits: Entropy Coding Enables Data-Free
// Model Compression", EntQuant technical summary, section 2, technical
// component 2): the optimised weights are flattened into a symbol stream and
// compressed with an ANS coder; the stored artefact is the compressed
// bitstream, the scaling parameters and metadata. The chunking follows
// "EntroLLM: Entropy Encoded Weight Compression for Efficient Large Language
// Model Inference on Edge Devices", technical overview, method item 3: the
// coded parameter space is split into independent chunks that keep the
// tensor's structure.
#include <algorithm>
#include <array>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <new>
#include <thread>
#include <vector>

#include "../../include/eq.h"
#include "format.hpp"

using namespace eqfmt;

namespace {

unsigned worker_count(uint64_t units) {
    unsigned hw = std::thread::hardware_concurrency();
    if (const char *env = std::getenv("EQ_HOST_THREADS")) hw = (unsigned)std::atoi(env);
    if (hw == 0) hw = 1;
    hw = std::min(hw, 64u);
    return (unsigned)std::max<uint64_t>(1, std::min<uint64_t>(hw, units));
}

// Run fn(i) for i in [0, count) on worker threads, handing out indices from
// a shared counter.
template <class F>
void parallel_for(uint64_t count, F &&fn) {
    unsigned nw = worker_count(count);
    if (nw <= 1) {
        for (uint64_t i = 0; i < count; ++i) fn(i);
        return;
    }
    std::atomic<uint64_t> next{0};
    auto body = [&] {
        for (uint64_t i; (i = next.fetch_add(1)) < count;) fn(i);
    };
    std::vector<std::thread> pool;
    pool.reserve(nw - 1);
    for (unsigned w = 1; w < nw; ++w) pool.emplace_back(body);
    body();
    for (auto &t : pool) t.join();
}

inline void wr16(uint8_t *p, uint16_t v) { std::memcpy(p, &v, 2); }
inline void wr32(uint8_t *p, uint32_t v) { std::memcpy(p, &v, 4); }
inline void wr64(uint8_t *p, uint64_t v) { std::memcpy(p, &v, 8); }
inline uint16_t rd16(const uint8_t *p) { uint16_t v; std::memcpy(&v, p, 2); return v; }
inline uint32_t rd32(const uint8_t *p) { uint32_t v; std::memcpy(&v, p, 4); return v; }
inline uint64_t rd64(const uint8_t *p) { uint64_t v; std::memcpy(&v, p, 8); return v; }

// ---------------------------------------------------------------------------
// 12-bit frequency quantiser (rule stated in include/eq.h).
// ---------------------------------------------------------------------------
eq_status quantise(const uint64_t counts[256], uint64_t N, uint16_t freq[256]) {
    struct Entry {
        int sym;
        uint64_t rem;
    };
    std::vector<Entry> present;
    int64_t f[256];
    int64_t total = 0;
    for (int s = 0; s < 256; ++s) {
        f[s] = 0;
        if (!counts[s]) continue;
        const uint64_t scaled = counts[s] * (uint64_t)kProbScale;
        f[s] = std::max<int64_t>(1, (int64_t)(scaled / N));
        present.push_back({s, scaled % N});
        total += f[s];
    }
    int64_t deficit = (int64_t)kProbScale - total;
    if (deficit > 0) {
        // hand the shortfall to the largest remainders, smaller byte first on ties
        std::stable_sort(present.begin(), present.end(),
                         [](const Entry &a, const Entry &b) { return a.rem > b.rem; });
        if ((uint64_t)deficit > present.size()) return EQ_EINVAL;
        for (int64_t i = 0; i < deficit; ++i) f[present[(size_t)i].sym] += 1;
    } else {
        // take the excess one at a time from the currently largest f > 1
        for (; deficit < 0; ++deficit) {
            int pick = -1;
            for (int s = 255; s >= 0; --s)
                if (f[s] > 1 && (pick < 0 || f[s] >= f[pick])) pick = s;
            if (pick < 0) return EQ_EINVAL;
            f[pick] -= 1;
        }
    }
    for (int s = 0; s < 256; ++s) freq[s] = (uint16_t)f[s];
    return EQ_OK;
}

// ---------------------------------------------------------------------------
// Chunk encoder.
// ---------------------------------------------------------------------------
struct SymInfo {
    uint32_t freq;
    uint32_t start;
    uint64_t renorm_at;  // state at and above which one word is flushed first: freq << 20
};

// Encodes one chunk of nk symbols with 64 interleaved lanes. The symbols are
// visited from the last (step, lane) back to the first, and each flushed
// word is written just before the previous one, so the words come out in the
// decoder's reading order. `wend` points one past the chunk's word region,
// which has room for nk words (at most one word per symbol). Returns the
// number of words; they occupy [wend - count, wend).
uint64_t encode_chunk(const uint8_t *sym, uint32_t nk, uint32_t K, const SymInfo *tab,
                      uint32_t *final_states, uint16_t *wend) {
    uint32_t lane_state[kLanes];
    for (uint32_t j = 0; j < kLanes; ++j) lane_state[j] = kStateLow;
    uint16_t *w = wend;
    const uint32_t group = kLanes * K;
    const uint32_t groups = (nk + group - 1) / group;
    for (uint32_t g = groups; g-- > 0;) {
        const uint32_t gbase = g * group;
        for (uint32_t r = K; r-- > 0;) {
            for (uint32_t j = kLanes; j-- > 0;) {
                const uint32_t pos = gbase + j * K + r;
                if (pos >= nk) continue;
                const SymInfo &si = tab[sym[pos]];
                uint32_t x = lane_state[j];
                if ((uint64_t)x >= si.renorm_at) {
                    *--w = (uint16_t)(x & 0xFFFFu);
                    x >>= 16;
                }
                const uint32_t q = x / si.freq;
                lane_state[j] = (q << kProbBits) + (x - q * si.freq) + si.start;
            }
        }
    }
    std::memcpy(final_states, lane_state, sizeof lane_state);
    return (uint64_t)(wend - w);
}

bool is_e4m3_nan(uint8_t c) { return (c & 0x7Fu) == 0x7Fu; }

// ---------------------------------------------------------------------------
// Huffman codec (EntroLLM technical overview, method item 2).
// ---------------------------------------------------------------------------

// Code lengths of at most kHuffMaxLen bits minimising sum count * length
// (package-merge). Items of one list are kept sorted by weight; a package of
// the deeper list is placed after coins of the same weight. Coins are the
// present symbols in (count, byte) order. Returns false if none is present.
// A lone present symbol gets kHuffZero.
bool huffman_lengths(const uint64_t counts[256], uint16_t table[256]) {
    struct Node { uint64_t weight; int32_t sym; uint32_t left; };  // package: children left, left + 1
    std::vector<uint32_t> present;
    for (uint32_t c = 0; c < 256; ++c)
        if (counts[c]) present.push_back(c);
    std::fill(table, table + 256, 0);
    if (present.empty()) return false;
    if (present.size() == 1) {
        table[present[0]] = kHuffZero;
        return true;
    }
    std::stable_sort(present.begin(), present.end(),
                     [&](uint32_t a, uint32_t b) { return counts[a] < counts[b]; });
    const size_t n = present.size();
    // level[L - 1] is the deepest list; level[0] the top one
    std::vector<std::vector<Node>> level(kHuffMaxLen);
    for (uint32_t d = kHuffMaxLen; d-- > 0;) {
        std::vector<Node> &cur = level[d];
        const std::vector<Node> *deeper = d + 1 < kHuffMaxLen ? &level[d + 1] : nullptr;
        const size_t packs = deeper ? deeper->size() / 2 : 0;
        cur.reserve(n + packs);
        size_t c = 0, q = 0;
        while (c < n || q < packs) {
            const uint64_t pw = q < packs ? (*deeper)[2 * q].weight + (*deeper)[2 * q + 1].weight : 0;
            if (q == packs || (c < n && counts[present[c]] <= pw)) {
                cur.push_back({counts[present[c]], (int32_t)present[c], 0});
                ++c;
            } else {
                cur.push_back({pw, -1, (uint32_t)(2 * q)});
                ++q;
            }
        }
    }
    // each symbol's length = its occurrences in the 2n - 2 cheapest top items
    std::vector<std::pair<uint32_t, uint32_t>> stack;  // (depth, index)
    for (uint32_t i = 0; i < 2 * n - 2; ++i) stack.push_back({0, i});
    while (!stack.empty()) {
        const auto [d, i] = stack.back();
        stack.pop_back();
        const Node &nd = level[d][i];
        if (nd.sym >= 0) {
            ++table[nd.sym];
        } else {
            stack.push_back({d + 1, nd.left});
            stack.push_back({d + 1, nd.left + 1});
        }
    }
    return true;
}

// Canonical codewords of a complete length table: (length, byte) order,
// consecutive values, shifted left when the length grows.
void huffman_codes(const uint16_t table[256], uint32_t code[256]) {
    uint32_t count[kHuffMaxLen + 2] = {};
    for (int s = 0; s < 256; ++s)
        if (table[s] && table[s] <= kHuffMaxLen) ++count[table[s]];
    uint32_t next[kHuffMaxLen + 2] = {};
    uint32_t c = 0;
    for (uint32_t l = 1; l <= kHuffMaxLen; ++l) {
        next[l] = c;
        c = (c + count[l]) << 1;
    }
    for (int s = 0; s < 256; ++s) code[s] = (table[s] && table[s] <= kHuffMaxLen) ? next[table[s]]++ : 0;
}

// True iff the table is a complete prefix code of lengths 1..12, or exactly
// one kHuffZero entry and nothing else; sets *lone to that symbol or -1.
bool huffman_table_ok(const uint16_t table[256], int32_t *lone) {
    uint64_t kraft = 0;
    int zeros = 0, coded = 0;
    *lone = -1;
    for (int s = 0; s < 256; ++s) {
        const uint16_t l = table[s];
        if (l == kHuffZero) { ++zeros; *lone = s; continue; }
        if (l > kHuffMaxLen) return false;
        if (l) { ++coded; kraft += 1ull << (kHuffMaxLen - l); }
    }
    if (zeros) return zeros == 1 && coded == 0;
    return kraft == (1ull << kHuffMaxLen);
}

// Huffman-codes one chunk: each lane's codewords go into its own 16-bit word
// list (most significant codeword bit first, from bit 0 of a word up); then
// the decoder's step loop is replayed to interleave those lists: at each
// step an active lane holding fewer than 12 bits takes its next word (zero
// once its list is used up). `out` has room for nk words. Returns the count.
uint64_t huffman_encode_chunk(const uint8_t *sym, uint32_t nk, uint32_t K, const uint16_t table[256],
                              const uint32_t code[256], uint16_t *out) {
    for (int s = 0; s < 256; ++s)
        if (table[s] == kHuffZero) return 0;  // a lone zero-bit symbol: no words
    const uint32_t group = kLanes * K;
    const uint32_t steps = (nk + group - 1) / group * K;
    auto pos_of = [&](uint32_t t, uint32_t j) { return (t / K) * group + j * K + (t % K); };
    std::vector<std::vector<uint16_t>> lane_words(kLanes);
    for (uint32_t j = 0; j < kLanes; ++j) {
        uint64_t acc = 0;
        uint32_t bits = 0;
        std::vector<uint16_t> &w = lane_words[j];
        for (uint32_t t = 0; t < steps; ++t) {
            const uint32_t p = pos_of(t, j);
            if (p >= nk) break;  // a lane's positions only grow with t
            const uint32_t l = table[sym[p]];
            const uint32_t c = code[sym[p]];
            for (uint32_t i = 0; i < l; ++i)  // codeword MSB first into rising bit positions
                acc |= (uint64_t)((c >> (l - 1 - i)) & 1u) << (bits + i);
            bits += l;
            while (bits >= 16) {
                w.push_back((uint16_t)acc);
                acc >>= 16;
                bits -= 16;
            }
        }
        if (bits) w.push_back((uint16_t)acc);
    }
    uint32_t held[kLanes] = {};
    size_t next[kLanes] = {};
    uint64_t nw = 0;
    for (uint32_t t = 0; t < steps; ++t) {
        for (uint32_t j = 0; j < kLanes; ++j) {
            const uint32_t p = pos_of(t, j);
            if (p >= nk) continue;
            if (held[j] < 12) {
                out[nw++] = next[j] < lane_words[j].size() ? lane_words[j][next[j]] : 0;
                ++next[j];
                held[j] += 16;
            }
            held[j] -= table[sym[p]];
        }
    }
    return nw;
}

}  // namespace

extern "C" {

const char *eq_status_string(eq_status s) {
    switch (s) {
        case EQ_OK: return "ok";
        case EQ_EINVAL: return "invalid argument";
        case EQ_ERANGE: return "output buffer too small";
        case EQ_ECORRUPT: return "corrupt container";
        case EQ_EHIP: return "HIP runtime error";
        case EQ_EUNSUPPORTED: return "unsupported";
        case EQ_ENOMEM: return "out of host memory";
        default: return "unknown status";
    }
}

eq_status eq_build_tables(const uint8_t *symbols, uint64_t n, eq_tables *out) {
    if (!symbols || !out || n == 0 || n >= (1ull << 51)) return EQ_EINVAL;
    const uint64_t slice = 1ull << 22;
    const uint64_t nslices = (n + slice - 1) / slice;
    std::vector<std::array<uint64_t, 256>> part(nslices);
    parallel_for(nslices, [&](uint64_t i) {
        auto &h = part[i];
        h.fill(0);
        const uint64_t lo = i * slice, hi = std::min(n, lo + slice);
        for (uint64_t k = lo; k < hi; ++k) h[symbols[k]]++;
    });
    std::memset(out, 0, sizeof *out);
    for (const auto &h : part)
        for (int s = 0; s < 256; ++s) out->counts[s] += h[s];
    out->n = n;
    eq_status st = quantise(out->counts, n, out->freq);
    if (st != EQ_OK) return st;
    out->cum[0] = 0;
    for (int s = 0; s < 256; ++s) out->cum[s + 1] = out->cum[s] + out->freq[s];
    return EQ_OK;
}

eq_status eq_tables_from_freq(const uint16_t *freq, eq_tables *out) {
    if (!freq || !out) return EQ_EINVAL;
    uint32_t sum = 0;
    for (int s = 0; s < 256; ++s) sum += freq[s];
    if (sum != eqfmt::kProbScale) return EQ_EINVAL;
    std::memset(out, 0, sizeof *out);
    for (int s = 0; s < 256; ++s) {
        out->freq[s] = freq[s];
        out->cum[s + 1] = out->cum[s] + freq[s];
    }
    return EQ_OK;
}

eq_status eq_encode_host(const eq_tables *t, const eq_tensor_desc *d, const uint8_t *symbols,
                         const float *scales, const uint64_t *esc_idx, const uint16_t *esc_bf16,
                         uint64_t n_esc, void *out, uint64_t cap, uint64_t *out_len) {
    if (!d || !symbols || !scales || !out_len) return EQ_EINVAL;
    const uint32_t seg = d->seg_chunks;
    if ((!t && !seg) || d->reserved) return EQ_EINVAL;
    if (seg && (seg % 8 || d->codec != kCodecRans)) return EQ_EINVAL;
    if (n_esc && (!esc_idx || !esc_bf16)) return EQ_EINVAL;
    if (d->dtype != EQ_DTYPE_INT8 && d->dtype != EQ_DTYPE_E4M3) return EQ_EINVAL;
    if (d->rows == 0 || d->cols == 0 || d->cols > (1ull << 40) / d->rows) return EQ_EINVAL;
    if (!valid_lane_run(d->lane_run)) return EQ_EINVAL;
    const uint32_t K = d->lane_run, Z = d->chunk_symbols;
    if (Z == 0 || Z > kMaxChunk || Z % (kLanes * K) != 0) return EQ_EINVAL;
    if (!d->esc_enabled && n_esc) return EQ_EINVAL;
    if (d->esc_enabled && d->esc_code > 255) return EQ_EINVAL;
    if (d->codec != kCodecRans && d->codec != kCodecHuffman) return EQ_EINVAL;
    const bool huff = d->codec == kCodecHuffman;
    // the per-symbol table the container stores: rANS frequencies, or
    // Huffman code lengths derived from the counts
    uint16_t table[256];
    if (huff) {
        if (!huffman_lengths(t->counts, table)) return EQ_EINVAL;
    } else if (!seg) {
        uint32_t fsum = 0;
        for (int s = 0; s < 256; ++s) {
            fsum += t->freq[s];
            table[s] = t->freq[s];
        }
        if (fsum != kProbScale) return EQ_EINVAL;
    }

    const uint64_t n = d->rows * d->cols;
    for (uint64_t r = 0; r < d->rows; ++r)
        if (!std::isfinite(scales[r])) return EQ_EINVAL;
    for (uint64_t e = 0; e < n_esc; ++e) {
        if (esc_idx[e] >= n || (e && esc_idx[e] <= esc_idx[e - 1])) return EQ_EINVAL;
        if (symbols[esc_idx[e]] != d->esc_code) return EQ_EINVAL;
    }

    // per-slice symbol validation (frequency present, NaN codes, escape count)
    const uint64_t slice = 1ull << 22;
    const uint64_t nslices = (n + slice - 1) / slice;
    std::vector<uint64_t> esc_seen(nslices, 0);
    std::vector<uint8_t> bad(nslices, 0);
    parallel_for(nslices, [&](uint64_t i) {
        const uint64_t lo = i * slice, hi = std::min(n, lo + slice);
        uint64_t seen = 0;
        bool b = false;
        for (uint64_t k = lo; k < hi; ++k) {
            const uint8_t c = symbols[k];
            b |= !seg && table[c] == 0;
            const bool is_esc = d->esc_enabled && c == d->esc_code;
            seen += is_esc;
            b |= d->dtype == EQ_DTYPE_E4M3 && is_e4m3_nan(c) && !is_esc;
        }
        esc_seen[i] = seen;
        bad[i] = b;
    });
    uint64_t esc_total = 0;
    for (uint64_t i = 0; i < nslices; ++i) {
        if (bad[i]) return EQ_EINVAL;
        esc_total += esc_seen[i];
    }
    if (esc_total != n_esc) return EQ_EINVAL;

    const uint64_t n_chunks = (n + Z - 1) / Z;
    const uint64_t n_tab = n_tables(n_chunks, seg);
    // the stored tables: one (the caller's, or the Huffman lengths), or with
    // adaptive tables each segment's own quantised counts
    std::vector<uint16_t> tables(256 * n_tab);
    if (seg) {
        std::vector<uint8_t> bad_seg(n_tab, 0);
        parallel_for(n_tab, [&](uint64_t g) {
            uint64_t counts[256] = {};
            const uint64_t lo = g * seg * Z, hi = std::min(n, (g + 1) * seg * Z);
            for (uint64_t i = lo; i < hi; ++i) ++counts[symbols[i]];
            bad_seg[g] = quantise(counts, hi - lo, &tables[256 * g]) != EQ_OK;
        });
        for (uint64_t g = 0; g < n_tab; ++g)
            if (bad_seg[g]) return EQ_EINVAL;
    } else {
        std::copy(table, table + 256, tables.begin());
    }
    std::vector<SymInfo> tab(huff ? 0 : 256 * n_tab);
    uint32_t hcode[256];
    if (huff) {
        huffman_codes(table, hcode);
    } else {
        for (uint64_t g = 0; g < n_tab; ++g) {
            uint32_t c = 0;
            for (int s = 0; s < 256; ++s) {
                const uint16_t f = tables[256 * g + s];
                SymInfo &si = tab[256 * g + s];
                si.freq = f ? f : 1;
                si.start = c;
                si.renorm_at = (uint64_t)f << 20;
                c += f;
            }
        }
        if (!seg) {
            uint32_t c = 0;  // the caller's cum must match its freq
            for (int s = 0; s < 256; ++s) {
                if (t->cum[s] != c) return EQ_EINVAL;
                c += t->freq[s];
            }
        }
    }

    std::unique_ptr<uint16_t[]> scratch(new (std::nothrow) uint16_t[n]);
    std::unique_ptr<uint32_t[]> states(new (std::nothrow) uint32_t[huff ? 1 : n_chunks * kLanes]);
    std::unique_ptr<uint64_t[]> wcount(new (std::nothrow) uint64_t[n_chunks]);
    if (!scratch || !states || !wcount) return EQ_ENOMEM;

    // chunk k encodes into scratch[k*Z, k*Z + nk): rANS fills it from its
    // end, Huffman from its start
    parallel_for(n_chunks, [&](uint64_t k) {
        const uint64_t p0 = k * Z;
        const uint32_t nk = (uint32_t)std::min<uint64_t>(Z, n - p0);
        if (huff)
            wcount[k] = huffman_encode_chunk(symbols + p0, nk, K, table, hcode, scratch.get() + p0);
        else
            wcount[k] = encode_chunk(symbols + p0, nk, K, &tab[256 * (seg ? k / seg : 0)],
                                     &states[k * kLanes], scratch.get() + p0 + nk);
    });

    uint64_t n_words = 0;
    for (uint64_t k = 0; k < n_chunks; ++k) n_words += round_up(wcount[k], kWordPad);
    const Sections sec = layout(d->rows, n_chunks, n_words, n_esc, d->codec, n_tab);
    *out_len = sec.total;
    if (!out || cap < sec.total) return EQ_ERANGE;

    uint8_t *b = static_cast<uint8_t *>(out);
    std::memset(b, 0, sec.freq);
    wr32(b + H_MAGIC, kMagic);
    wr16(b + H_VERSION, kVersion);
    b[H_DTYPE] = (uint8_t)d->dtype;
    b[H_FLAGS] = (d->esc_enabled ? kFlagEsc : 0) | (seg ? kFlagSeg : 0);
    wr64(b + H_ROWS, d->rows);
    wr64(b + H_COLS, d->cols);
    wr64(b + H_N, n);
    wr32(b + H_CHUNK, Z);
    wr32(b + H_LANE_RUN, K);
    wr32(b + H_LANES, kLanes);
    wr32(b + H_PROB_BITS, huff ? kHuffMaxLen : kProbBits);
    wr64(b + H_NCHUNKS, n_chunks);
    wr64(b + H_NESC, n_esc);
    b[H_ESC_CODE] = d->esc_enabled ? (uint8_t)d->esc_code : 0;
    wr64(b + H_NWORDS, n_words);
    const uint64_t offs[8] = {sec.freq, sec.scales, sec.dir, sec.states,
                              sec.words, sec.esc_idx, sec.esc_val, sec.total};
    for (int i = 0; i < 8; ++i) wr64(b + H_OFF_FREQ + 8 * i, offs[i]);

    auto zero_to = [&](uint64_t from, uint64_t to) {
        if (to > from) std::memset(b + from, 0, to - from);
    };
    zero_to(H_CODEC, sec.freq);
    wr32(b + H_CODEC, d->codec);
    wr32(b + H_SEG, seg);
    zero_to(sec.freq, sec.total);  // gaps and padding words are zero
    for (uint64_t i = 0; i < 256 * n_tab; ++i) wr16(b + sec.freq + 2 * i, tables[i]);
    std::memcpy(b + sec.scales, scales, d->rows * 4);

    std::vector<uint64_t> first(n_chunks);
    for (uint64_t k = 0, at = 0; k < n_chunks; ++k) {
        first[k] = at;
        at += round_up(wcount[k], kWordPad);
        wr64(b + sec.dir + kDirEntryBytes * k, first[k]);
        wr32(b + sec.dir + kDirEntryBytes * k + 8, (uint32_t)wcount[k]);
    }
    if (!huff) std::memcpy(b + sec.states, states.get(), n_chunks * kLanes * 4);
    parallel_for(n_chunks, [&](uint64_t k) {
        const uint64_t p0 = k * Z;
        const uint64_t nk = std::min<uint64_t>(Z, n - p0);
        const uint16_t *src = huff ? scratch.get() + p0 : scratch.get() + p0 + nk - wcount[k];
        std::memcpy(b + sec.words + 2 * first[k], src, 2 * wcount[k]);
    });
    for (uint64_t e = 0; e < n_esc; ++e) {
        wr64(b + sec.esc_idx + 8 * e, esc_idx[e]);
        wr16(b + sec.esc_val + 2 * e, esc_bf16[e]);
    }
    return EQ_OK;
}

eq_status eq_parse_header(const void *bytes, uint64_t len, eq_header *out) {
    if (!bytes || !out) return EQ_EINVAL;
    const uint8_t *b = static_cast<const uint8_t *>(bytes);
    if (len < kHeaderBytes) return EQ_ECORRUPT;
    if (rd32(b + H_MAGIC) != kMagic || rd16(b + H_VERSION) != kVersion) return EQ_ECORRUPT;
    eq_header h{};
    h.dtype = b[H_DTYPE];
    h.flags = b[H_FLAGS];
    h.rows = rd64(b + H_ROWS);
    h.cols = rd64(b + H_COLS);
    h.n = rd64(b + H_N);
    h.chunk_symbols = rd32(b + H_CHUNK);
    h.lane_run = rd32(b + H_LANE_RUN);
    h.n_chunks = rd64(b + H_NCHUNKS);
    h.n_esc = rd64(b + H_NESC);
    h.esc_code = b[H_ESC_CODE];
    h.n_words = rd64(b + H_NWORDS);
    h.off_freq = rd64(b + H_OFF_FREQ);
    h.off_scales = rd64(b + H_OFF_SCALES);
    h.off_dir = rd64(b + H_OFF_DIR);
    h.off_states = rd64(b + H_OFF_STATES);
    h.off_words = rd64(b + H_OFF_WORDS);
    h.off_esc_idx = rd64(b + H_OFF_ESC_IDX);
    h.off_esc_val = rd64(b + H_OFF_ESC_VAL);
    h.total_bytes = rd64(b + H_TOTAL);
    h.single_symbol = -1;
    h.codec = rd32(b + H_CODEC);
    h.seg_chunks = rd32(b + H_SEG);
    if (h.codec != kCodecRans && h.codec != kCodecHuffman) return EQ_ECORRUPT;
    const bool huff = h.codec == kCodecHuffman;
    const uint32_t seg = h.seg_chunks;
    if (((h.flags & kFlagSeg) != 0) != (seg != 0)) return EQ_ECORRUPT;
    if (seg && (seg % 8 || huff)) return EQ_ECORRUPT;

    if (h.dtype != EQ_DTYPE_INT8 && h.dtype != EQ_DTYPE_E4M3) return EQ_ECORRUPT;
    if (h.flags > (kFlagEsc | kFlagSeg) || (!(h.flags & kFlagEsc) && (h.n_esc || h.esc_code)))
        return EQ_ECORRUPT;
    if (rd32(b + H_LANES) != kLanes || rd32(b + H_PROB_BITS) != (huff ? kHuffMaxLen : kProbBits))
        return EQ_ECORRUPT;
    if (!valid_lane_run(h.lane_run)) return EQ_ECORRUPT;
    if (h.chunk_symbols == 0 || h.chunk_symbols > kMaxChunk ||
        h.chunk_symbols % (kLanes * h.lane_run))
        return EQ_ECORRUPT;
    if (h.rows == 0 || h.cols == 0 || h.cols > (1ull << 40) / h.rows || h.rows * h.cols != h.n)
        return EQ_ECORRUPT;
    if (h.n_chunks != (h.n + h.chunk_symbols - 1) / h.chunk_symbols) return EQ_ECORRUPT;
    if (h.n_esc > h.n || h.n_words > h.n + 8 * h.n_chunks) return EQ_ECORRUPT;
    for (size_t i = 65; i < 72; ++i)
        if (b[i]) return EQ_ECORRUPT;
    for (size_t i = H_SEG + 4; i < kHeaderBytes; ++i)
        if (b[i]) return EQ_ECORRUPT;
    const uint64_t n_tab = n_tables(h.n_chunks, seg);
    const Sections sec = layout(h.rows, h.n_chunks, h.n_words, h.n_esc, h.codec, n_tab);
    if (h.off_freq != sec.freq || h.off_scales != sec.scales || h.off_dir != sec.dir ||
        h.off_states != sec.states || h.off_words != sec.words || h.off_esc_idx != sec.esc_idx ||
        h.off_esc_val != sec.esc_val || h.total_bytes != sec.total)
        return EQ_ECORRUPT;
    if (len < h.total_bytes) return EQ_ECORRUPT;

    if (huff) {
        uint16_t table[256];
        for (int s = 0; s < 256; ++s) table[s] = rd16(b + h.off_freq + 2 * s);
        int32_t lone;
        if (!huffman_table_ok(table, &lone)) return EQ_ECORRUPT;
        h.single_symbol = lone;
    } else {
        for (uint64_t g = 0; g < n_tab; ++g) {
            uint32_t fsum = 0;
            for (int s = 0; s < 256; ++s) {
                const uint16_t f = rd16(b + h.off_freq + 512 * g + 2 * s);
                fsum += f;
                if (f == kProbScale && !seg) h.single_symbol = s;
            }
            if (fsum != kProbScale) return EQ_ECORRUPT;
        }
    }

    // directory: consecutive padded word ranges covering exactly n_words
    uint64_t at = 0;
    for (uint64_t k = 0; k < h.n_chunks; ++k) {
        const uint8_t *e = b + h.off_dir + kDirEntryBytes * k;
        const uint64_t first = rd64(e);
        const uint32_t count = rd32(e + 8);
        const uint64_t nk = std::min<uint64_t>(h.chunk_symbols, h.n - k * h.chunk_symbols);
        if (first != at || count > nk || rd32(e + 12) != 0) return EQ_ECORRUPT;
        at += round_up(count, kWordPad);
    }
    if (at != h.n_words) return EQ_ECORRUPT;
    // lane states: a valid encoder end state lies in [2^16, 2^32)
    if (!huff)
        for (uint64_t i = 0; i < h.n_chunks * kLanes; ++i)
            if (rd32(b + h.off_states + 4 * i) < kStateLow) return EQ_ECORRUPT;
    for (uint64_t e = 0; e < h.n_esc; ++e) {
        const uint64_t idx = rd64(b + h.off_esc_idx + 8 * e);
        if (idx >= h.n || (e && idx <= rd64(b + h.off_esc_idx + 8 * (e - 1)))) return EQ_ECORRUPT;
    }
    *out = h;
    return EQ_OK;
}

}  // extern "C"
