/*
 * eq_oracle.c -- plain, slow, scalar CPU oracle for entropy-coded weight decode.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this library. The product library never
 * links, loads or calls it, and the two share no source, header, table or
 * helper: this file defines its own container parser, coder and dequantiser.
 *
 * What is computed, and where the pages say so:
 *
 *  [EQ] "Float8@2bits: Entropy Coding Enables Data-Free Model Compression"
 *       (EntQuant technical summary), section 2 (method):
 *        - "core concept": weights stay in a Float8 or Int8 base format, are
 *          made low-entropy, and are then compressed losslessly by an ANS coder;
 *        - technical component 1: per-channel scaling parameters S;
 *        - technical component 2 (weight encoding): the weights are flattened
 *          into one symbol stream and ANS-compressed; the stored artefact is
 *          the compressed bitstream + the scales + metadata;
 *        - technical component 3 (inference-time decoding): a parallel ANS
 *          decoder expands the weights into a buffer just before each
 *          transformer block's forward pass;
 *        - technical component 4 (super weights): extreme outliers are kept
 *          out of the entropy-optimised stream (Int8 base format).
 *  [EL] "EntroLLM: Entropy Encoded Weight Compression for Efficient Large
 *       Language Model Inference on Edge Devices", technical overview,
 *       method item 2 (Huffman weight encoding: frequent weight values get
 *       short variable-length codes, rare ones long codes) and item 3
 *       (parallel decoding): the coded parameter space is cut into chunks
 *       that keep the tensor structure and are decoded independently and
 *       concurrently.
 *
 * The pages fix none of the coder's bit-level choices (they only say "ANS").
 * This oracle implements "container v1", whose every choice is stated where
 * it is used below: static rANS over the 256 byte codes, 12-bit quantised
 * frequencies (M = 4096), a u32 state in [2^16, 2^32), 16-bit renormalisation
 * words, 64 interleaved lane states per chunk, a lane run of K consecutive
 * symbols, fixed-size chunks that never span tensors.
 *
 * Parity pins (all tested without any GPU code): the decoded symbols must be
 * the encoded ones (losslessness, [EQ] core concept); a hand-worked
 * three-symbol example; exhaustive C(D(x)) = x over every state; brute force
 * over all tiny streams; bf16 rounding against a library routine over all
 * 2^32 fp32 patterns; E4M3 decoding against a library routine over all 256
 * codes; coded size against N x empirical entropy.
 *
 * Plain C11 + pthreads. No intrinsics. Floating point: one IEEE binary32
 * multiply per weight (x86-64 SSE, FLT_EVAL_METHOD == 0, no contraction).
 */
#include <float.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if FLT_EVAL_METHOD != 0
#error "the oracle needs binary32 evaluation of float expressions"
#endif

/* ------------------------------------------------------------------------ */
/* Container v1 constants (this file's own copy; the product has its own).  */
/* ------------------------------------------------------------------------ */
#define OR_MAGIC 0x31525145u  /* bytes 'E','Q','R','1' */
#define OR_VERSION 1u
#define OR_DTYPE_INT8 1u
#define OR_DTYPE_E4M3 2u
#define OR_FLAG_ESC 1u
#define OR_FLAG_SEG 2u        /* one frequency table per segment of chunks */
#define OR_LANES 64u
#define OR_PROB_BITS 12u
#define OR_M 4096u            /* 2^12: sum of the quantised frequencies */
#define OR_L 65536u           /* 2^16: lower bound of the coder state  */
#define OR_HDR_BYTES 256u
#define OR_ALIGN 256u
#define OR_CODEC_RANS 0u      /* header offset 144: entropy coder of the stream */
#define OR_CODEC_HUFF 1u
#define OR_HUFF_MAXLEN 12u    /* longest Huffman codeword (bits) */
#define OR_HUFF_ZERO 0x100u   /* table value: the only symbol, coded in zero bits */

/* Status / flag values returned by the oracle. */
#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ECORRUPT (-3)
#define OR_ENOMEM (-6)
/* decode flags (ORed) */
#define OR_BAD_END_STATE 1u
#define OR_WORD_OVERRUN 2u

/* ------------------------------------------------------------------------ */
/* Little-endian field access on a byte buffer.                              */
/* ------------------------------------------------------------------------ */
static void put_u16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)v; p[1] = (uint8_t)(v >> 8); }
static void put_u32(uint8_t *p, uint32_t v) {
    for (int i = 0; i < 4; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static void put_u64(uint8_t *p, uint64_t v) {
    for (int i = 0; i < 8; i++) p[i] = (uint8_t)(v >> (8 * i));
}
static uint16_t get_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static uint32_t get_u32(const uint8_t *p) {
    uint32_t v = 0;
    for (int i = 3; i >= 0; i--) v = (v << 8) | p[i];
    return v;
}
static uint64_t get_u64(const uint8_t *p) {
    uint64_t v = 0;
    for (int i = 7; i >= 0; i--) v = (v << 8) | p[i];
    return v;
}
static float get_f32(const uint8_t *p) {
    uint32_t b = get_u32(p);
    float f;
    memcpy(&f, &b, 4);
    return f;
}
static uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

/* ------------------------------------------------------------------------ */
/* Numeric definitions of the dequantisation.                                */
/* ------------------------------------------------------------------------ */

/* fp32 -> bf16, round to nearest, ties to even, on the bit pattern.
 * Keeps the top 16 bits of the binary32 pattern after adding half of the
 * dropped part (0x7FFF) plus the lowest kept bit (which breaks ties toward an
 * even result). Overflow of the largest finite values carries into the
 * exponent and yields +-inf, as RNE requires. NaN inputs give a quiet NaN with
 * the same sign. */
uint16_t or_bf16_rne(float v) {
    uint32_t b;
    memcpy(&b, &v, 4);
    if ((b & 0x7F800000u) == 0x7F800000u && (b & 0x007FFFFFu) != 0)
        return (uint16_t)((b >> 16) | 0x0040u);
    uint32_t lsb = (b >> 16) & 1u;
    return (uint16_t)((b + 0x7FFFu + lsb) >> 16);
}

/* OCP FP8 E4M3FN byte -> value. [EQ] "core concept" names Float8 as a base
 * format; the E4M3FN reading (bias 7, no infinities, only S.1111.111 is NaN,
 * largest finite 448, subnormals m * 2^-9) is the OCP 8-bit floating point
 * definition, written out here from that definition. */
float or_e4m3_value(uint8_t c) {
    int sign = (c >> 7) & 1;
    int e = (c >> 3) & 0xF;
    int m = c & 7;
    float mag;
    if (e == 0xF && m == 7) {
        uint32_t nan = sign ? 0xFFC00000u : 0x7FC00000u;
        memcpy(&mag, &nan, 4);
        return mag;
    }
    if (e == 0) {
        mag = (float)m / 512.0f; /* m * 2^-9, exact */
    } else {
        /* (1 + m/8) * 2^(e-7), built from exact powers of two */
        float p = 1.0f;
        for (int i = 0; i < e; i++) p *= 2.0f;
        mag = (8.0f + (float)m) / 8.0f * p / 128.0f;
    }
    return sign ? -mag : mag;
}

/* Value of a byte code in the tensor's base format ([EQ] "core concept":
 * Int8 or Float8). Int8 codes are two's-complement bytes. */
float or_symbol_value(uint32_t dtype, uint8_t c) {
    if (dtype == OR_DTYPE_INT8) return (float)(int8_t)c;
    return or_e4m3_value(c);
}

/* The exact result of the whole decode + dequant path, written from its
 * definition and computed straight from the ORIGINAL symbols (no decoder):
 * because the coding is lossless ([EQ] "core concept"), the decoded tensor is
 *   out[i] = bf16_RNE( fp32( value(s[i]) * S[row(i)] ) ),  row(i) = i / cols
 * with the scales applied per output channel (= row of the [out, in] matrix,
 * [EQ] technical component 1) and each super weight ([EQ] technical component
 * 4) replaced by its stored bf16 bits. */
void or_dequant_direct(uint32_t dtype, const uint8_t *sym, uint64_t n, uint64_t cols,
                       const float *scales, const uint64_t *esc_idx, const uint16_t *esc_val,
                       uint64_t n_esc, uint16_t *out) {
    for (uint64_t i = 0; i < n; i++) {
        float v = or_symbol_value(dtype, sym[i]);
        float prod = v * scales[i / cols];
        out[i] = or_bf16_rne(prod);
    }
    for (uint64_t e = 0; e < n_esc; e++)
        if (esc_idx[e] < n) out[esc_idx[e]] = esc_val[e];
}

/* ------------------------------------------------------------------------ */
/* Frequency table: counts -> 12-bit quantised frequencies.                  */
/* ------------------------------------------------------------------------ */

/* The pages give no quantiser ("ANS" only). Container v1 uses this integer
 * rule, so that any two implementations agree without floating point:
 *   (i)   f_s = max(1, floor(c_s * 4096 / N)) for every present symbol, else 0;
 *   (ii)  D = 4096 - sum f;
 *   (iii) if D > 0, the D present symbols with the largest remainder
 *         (c_s * 4096) mod N get +1 each (ties: smaller byte first);
 *   (iv)  while D < 0, the symbol with the largest f_s among those with
 *         f_s > 1 gets -1 (ties: smaller byte first), and D grows by one.
 * Afterwards sum f = 4096 and f_s > 0 exactly for present symbols.
 * Requires N < 2^51 so that c_s * 4096 fits in 64 bits. */
int or_quantize_counts(const uint64_t counts[256], uint16_t freq[256]) {
    uint64_t N = 0;
    for (int s = 0; s < 256; s++) N += counts[s];
    if (N == 0 || N >= ((uint64_t)1 << 51)) return OR_EINVAL;

    int64_t f[256];
    int64_t sum = 0;
    for (int s = 0; s < 256; s++) {
        if (counts[s] == 0) {
            f[s] = 0;
        } else {
            int64_t q = (int64_t)(counts[s] * OR_M / N);
            f[s] = q < 1 ? 1 : q;
        }
        sum += f[s];
    }
    int64_t D = (int64_t)OR_M - sum;

    if (D > 0) {
        int taken[256] = {0};
        for (int64_t k = 0; k < D; k++) {
            int best = -1;
            uint64_t best_r = 0;
            for (int s = 0; s < 256; s++) {
                if (counts[s] == 0 || taken[s]) continue;
                uint64_t r = (counts[s] * OR_M) % N;
                if (best < 0 || r > best_r) { best = s; best_r = r; }
            }
            if (best < 0) return OR_EINVAL; /* cannot happen: D < |present| */
            taken[best] = 1;
            f[best] += 1;
        }
    }
    while (D < 0) {
        int best = -1;
        for (int s = 0; s < 256; s++) {
            if (f[s] <= 1) continue;
            if (best < 0 || f[s] > f[best]) best = s;
        }
        if (best < 0) return OR_EINVAL; /* cannot happen: some f > 1 */
        f[best] -= 1;
        D += 1;
    }
    for (int s = 0; s < 256; s++) freq[s] = (uint16_t)f[s];
    return OR_OK;
}

/* Histogram of the byte stream, then the quantiser above. */
int or_build_freq(const uint8_t *sym, uint64_t n, uint16_t freq[256]) {
    uint64_t counts[256] = {0};
    for (uint64_t i = 0; i < n; i++) counts[sym[i]]++;
    return or_quantize_counts(counts, freq);
}

/* cum_s = sum of f_t over bytes t < s; slot2sym maps each of the 4096 slots to
 * the byte s with cum_s <= slot < cum_s + f_s. Returns 0 if sum f != 4096. */
static int make_tables(const uint16_t freq[256], uint32_t cum[257], uint8_t slot2sym[4096]) {
    cum[0] = 0;
    for (int s = 0; s < 256; s++) cum[s + 1] = cum[s] + freq[s];
    if (cum[256] != OR_M) return 0;
    for (int s = 0; s < 256; s++)
        for (uint32_t k = 0; k < freq[s]; k++) slot2sym[cum[s] + k] = (uint8_t)s;
    return 1;
}

/* ------------------------------------------------------------------------ */
/* The rANS step (one symbol, one state).                                    */
/* ------------------------------------------------------------------------ */

/* Encoder step for symbol (f, c): first the renormalisation, then the state
 * map x -> 4096 * floor(x / f) + (x mod f) + c. The renorm condition
 * x >= f * 2^20 is the point past which the new state would leave [2^16, 2^32);
 * it is compared in 64 bits because f = 4096 gives 2^32. At most one word is
 * emitted, because x < 2^32 implies floor(x / 2^16) < 2^16 <= f * 2^20.
 * Returns 1 and sets *word when a word is emitted. */
int or_encode_step(uint32_t *x, uint32_t f, uint32_t c, uint16_t *word) {
    int emitted = 0;
    uint64_t xv = *x;
    if (xv >= ((uint64_t)f << 20)) {
        *word = (uint16_t)(xv & 0xFFFFu);
        xv >>= 16;
        emitted = 1;
    }
    xv = (xv / f) * OR_M + (xv % f) + c;
    *x = (uint32_t)xv;
    return emitted;
}

/* Decoder step given the slot's symbol (f, c): x -> f * floor(x / 4096) +
 * (x mod 4096) - c. Returns 1 when the result is below 2^16 and therefore
 * needs one renormalisation word. */
int or_decode_step(uint32_t *x, uint32_t f, uint32_t c) {
    uint32_t slot = *x % OR_M;
    *x = f * (*x / OR_M) + slot - c;
    return *x < OR_L;
}

/* ------------------------------------------------------------------------ */
/* Interleaving: chunk-local position of lane j at step t.                   */
/* ------------------------------------------------------------------------ */

/* Container v1 lays a chunk out as groups of 64*K positions: in step t, lane
 * j handles position (t / K) * 64K + j * K + (t mod K), so over K consecutive
 * steps each lane produces a run of K consecutive symbols and the 64 lanes
 * together produce 64*K consecutive symbols. */
static uint64_t lane_pos(uint64_t t, uint32_t j, uint32_t K) {
    return (t / K) * (uint64_t)OR_LANES * K + (uint64_t)j * K + (t % K);
}
static uint64_t chunk_steps(uint64_t nk, uint32_t K) {
    uint64_t g = (uint64_t)OR_LANES * K;
    return (nk + g - 1) / g * K;
}

/* ------------------------------------------------------------------------ */
/* Single-lane whole-tensor coder: coded size only (the size bar).            */
/* ------------------------------------------------------------------------ */

/* Bytes of a single-lane rANS encoding of the whole stream with the given
 * table: 2 bytes per emitted word + 4 bytes of final state. */
uint64_t or_single_lane_bytes(const uint8_t *sym, uint64_t n, const uint16_t freq[256]) {
    uint32_t cum[257];
    uint8_t s2s[4096];
    if (!make_tables(freq, cum, s2s)) return 0;
    uint32_t x = OR_L;
    uint64_t words = 0;
    uint16_t w;
    for (uint64_t i = n; i-- > 0;) {
        uint8_t s = sym[i];
        if (freq[s] == 0) return 0;
        words += (uint64_t)or_encode_step(&x, freq[s], cum[s], &w);
    }
    return 2 * words + 4;
}

/* ------------------------------------------------------------------------ */
/* Huffman codec ([EL] method item 2).                                        */
/* ------------------------------------------------------------------------ */
/*
 * The pages say only "Huffman coding": frequent weight values get short
 * variable-length codes. Container v1 with codec 1 uses, as its readings:
 *  - code lengths from the exact symbol counts, optimal among prefix codes
 *    whose codewords have at most 12 bits (Larmore and Hirschberg's
 *    package-merge; when no codeword of an optimal unlimited Huffman code is
 *    longer than 12 bits the total length is the same). Coins are sorted by
 *    (count, byte); when a coin and a package weigh the same the coin comes
 *    first. One present symbol: length 0 ("zero-bit" code).
 *  - canonical codewords: symbols ordered by (length, byte) get consecutive
 *    code values, the value shifted left whenever the length grows.
 *  - each lane's bitstream is the concatenation of its codewords, each sent
 *    most significant bit first, packed into 16-bit words from bit 0 up
 *    (stream bit i is bit i mod 16 of the lane's word i / 16).
 *  - interleaving: a lane holds a bit buffer of n bits; at every step of the
 *    chunk (same positions and lane order as the rANS codec), each active
 *    lane with n < 12 first takes the next word of the chunk's word list
 *    (lanes in ascending order), then every active lane decodes one codeword
 *    from its buffer. The encoder walks the same steps to lay the words out;
 *    a lane that runs past its bitstream takes zero words. A chunk is valid
 *    iff every word is taken and every lane's leftover bits are zero.
 */

/* Optimal code lengths (at most L bits) for the counts: package-merge.
 * Returns OR_OK, or OR_EINVAL if no symbol is present or 256 symbols cannot
 * fit in L bits. len[s] = 0 for absent symbols; a lone symbol gets 0. */
typedef struct {
    uint64_t w;
    int32_t leaf;      /* symbol, or -1 for a package */
    int32_t a, b;      /* package: its two items in the previous (deeper) list */
} or_pm_item;

static void pm_count(or_pm_item *const *lists, uint32_t level, int32_t i, uint8_t len[256]) {
    const or_pm_item *it = &lists[level][i];
    if (it->leaf >= 0) {
        len[it->leaf]++;
        return;
    }
    pm_count(lists, level + 1, it->a, len);
    pm_count(lists, level + 1, it->b, len);
}

int or_huff_lengths(const uint64_t counts[256], uint32_t L, uint8_t len[256]) {
    memset(len, 0, 256);
    uint32_t n = 0;
    or_pm_item coins[256];
    for (int s = 0; s < 256; s++)
        if (counts[s]) coins[n++] = (or_pm_item){counts[s], s, -1, -1};
    if (n == 0 || L == 0 || L > 30 || (L < 8 && n > (1u << L))) return OR_EINVAL;
    if (n == 1) return OR_OK;
    /* sort coins by (count, byte): insertion sort, stable on the byte order */
    for (uint32_t i = 1; i < n; i++) {
        or_pm_item c = coins[i];
        uint32_t j = i;
        while (j > 0 && coins[j - 1].w > c.w) { coins[j] = coins[j - 1]; j--; }
        coins[j] = c;
    }
    /* lists[d] for depth d = 1..L; lists[L] = the coins; lists[d] = coins
     * merged with the pairs of lists[d + 1] */
    or_pm_item *lists[32] = {0};
    uint32_t sizes[32] = {0};
    for (uint32_t d = 1; d <= L; d++) {
        lists[d] = malloc(2 * n * sizeof(or_pm_item));
        if (!lists[d]) {
            for (uint32_t e = 1; e <= L; e++) free(lists[e]);
            return OR_ENOMEM;
        }
    }
    memcpy(lists[L], coins, n * sizeof(or_pm_item));
    sizes[L] = n;
    for (uint32_t d = L - 1; d >= 1; d--) {
        uint32_t np = sizes[d + 1] / 2, ic = 0, ip = 0, m = 0;
        while (ic < n || ip < np) {
            uint64_t pw = ip < np ? lists[d + 1][2 * ip].w + lists[d + 1][2 * ip + 1].w : 0;
            if (ip >= np || (ic < n && coins[ic].w <= pw)) {
                lists[d][m++] = coins[ic++];
            } else {
                lists[d][m++] = (or_pm_item){pw, -1, (int32_t)(2 * ip), (int32_t)(2 * ip + 1)};
                ip++;
            }
        }
        sizes[d] = m;
        if (d == 1) break;
    }
    /* the 2n - 2 cheapest items of the top list; a symbol's length is the
     * number of times it occurs in them */
    for (uint32_t i = 0; i < 2 * n - 2; i++) pm_count(lists, 1, (int32_t)i, len);
    for (uint32_t d = 1; d <= L; d++) free(lists[d]);
    return OR_OK;
}

/* Canonical decoding tables of a length table: count[l] codewords of length
 * l, first[l] = the code value of the first of them, sorted[] = symbols by
 * (length, byte), offset[l] = index in sorted[] of the first of length l.
 * Returns 1 iff the lengths form a complete prefix code (Kraft sum exactly
 * 1), or a single zero-length symbol. */
typedef struct {
    uint32_t count[OR_HUFF_MAXLEN + 1], first[OR_HUFF_MAXLEN + 1], offset[OR_HUFF_MAXLEN + 1];
    uint8_t sorted[256];
    uint32_t nsym;
    int zero_sym; /* the lone zero-bit symbol, or -1 */
} or_canon;

static int huff_canon(const uint16_t tab[256], or_canon *c) {
    memset(c, 0, sizeof *c);
    c->zero_sym = -1;
    uint32_t nz = 0;
    for (int s = 0; s < 256; s++) {
        if (tab[s] == OR_HUFF_ZERO) { c->zero_sym = s; nz++; continue; }
        if (tab[s] > OR_HUFF_MAXLEN) return 0;
        if (tab[s]) c->count[tab[s]]++;
    }
    for (uint32_t l = 1; l <= OR_HUFF_MAXLEN; l++) c->nsym += c->count[l];
    if (nz) return nz == 1 && c->nsym == 0;
    uint64_t kraft = 0; /* in units of 2^-12 */
    for (uint32_t l = 1; l <= OR_HUFF_MAXLEN; l++) kraft += (uint64_t)c->count[l] << (OR_HUFF_MAXLEN - l);
    if (kraft != (1u << OR_HUFF_MAXLEN)) return 0;
    uint32_t code = 0, off = 0;
    for (uint32_t l = 1; l <= OR_HUFF_MAXLEN; l++) {
        c->first[l] = code;
        c->offset[l] = off;
        code = (code + c->count[l]) << 1;
        off += c->count[l];
    }
    uint32_t fill[OR_HUFF_MAXLEN + 1];
    memcpy(fill, c->offset, sizeof fill);
    for (int s = 0; s < 256; s++)
        if (tab[s] && tab[s] != OR_HUFF_ZERO) c->sorted[fill[tab[s]]++] = (uint8_t)s;
    return 1;
}

/* Canonical codeword of every symbol (0 for absent ones). Returns 1 on a
 * valid table (see huff_canon). */
int or_huff_codes(const uint16_t tab[256], uint32_t code[256]) {
    or_canon c;
    if (!huff_canon(tab, &c)) return 0;
    memset(code, 0, 256 * sizeof(uint32_t));
    for (uint32_t l = 1; l <= OR_HUFF_MAXLEN; l++)
        for (uint32_t i = 0; i < c.count[l]; i++) code[c.sorted[c.offset[l] + i]] = c.first[l] + i;
    return 1;
}

/* Encode one chunk with the Huffman codec: the lanes' bitstreams, then the
 * decoder's refill schedule walked forward to order the words. words must
 * hold nk entries (at most one word per lane-step). Returns the word count. */
static uint64_t huff_encode_chunk(const uint8_t *sym, uint64_t nk, uint32_t K, const uint16_t tab[256],
                                  const uint32_t code[256], uint16_t *words) {
    uint64_t T = chunk_steps(nk, K);
    for (int s = 0; s < 256; s++)
        if (tab[s] == OR_HUFF_ZERO) return 0; /* a lone symbol: no bits, no words */
    /* each lane's bitstream, one bit per byte (plain and slow) */
    uint64_t bits_max = T * OR_HUFF_MAXLEN + 64;
    uint8_t *bits = calloc(OR_LANES * bits_max, 1);
    uint64_t nbits[64] = {0};
    if (!bits) return UINT64_MAX;
    for (uint64_t t = 0; t < T; t++) {
        for (uint32_t j = 0; j < OR_LANES; j++) {
            uint64_t p = lane_pos(t, j, K);
            if (p >= nk) continue;
            uint32_t l = tab[sym[p]] == OR_HUFF_ZERO ? 0 : tab[sym[p]];
            for (uint32_t i = l; i-- > 0;) bits[j * bits_max + nbits[j]++] = (code[sym[p]] >> i) & 1u;
        }
    }
    uint64_t nw = 0, taken[64] = {0};
    uint32_t have[64] = {0};
    for (uint64_t t = 0; t < T; t++) {
        for (uint32_t j = 0; j < OR_LANES; j++) {
            if (lane_pos(t, j, K) >= nk || have[j] >= 12) continue;
            uint16_t w = 0;
            for (uint32_t i = 0; i < 16; i++) {
                uint64_t b = 16 * taken[j] + i;
                if (b < nbits[j] && bits[j * bits_max + b]) w |= (uint16_t)(1u << i);
            }
            words[nw++] = w;
            taken[j]++;
            have[j] += 16;
        }
        for (uint32_t j = 0; j < OR_LANES; j++) {
            uint64_t p = lane_pos(t, j, K);
            if (p >= nk) continue;
            have[j] -= tab[sym[p]] == OR_HUFF_ZERO ? 0 : tab[sym[p]];
        }
    }
    free(bits);
    return nw;
}

/* Decode one Huffman chunk: refills as above, then each active lane reads
 * bits one at a time (least significant first), growing a code value until
 * it names a canonical codeword of that length. Returns the flags. */
static uint32_t huff_decode_chunk(const uint8_t *words_le, uint64_t nwords, uint64_t nk, uint32_t K,
                                  const or_canon *c, uint8_t *sym_out) {
    if (c->zero_sym >= 0) {
        for (uint64_t p = 0; p < nk; p++) sym_out[p] = (uint8_t)c->zero_sym;
        return nwords ? OR_BAD_END_STATE : 0;
    }
    uint32_t b[64] = {0}, n[64] = {0};
    uint64_t ptr = 0;
    uint64_t T = chunk_steps(nk, K);
    for (uint64_t t = 0; t < T; t++) {
        for (uint32_t j = 0; j < OR_LANES; j++) {
            if (lane_pos(t, j, K) >= nk || n[j] >= 12) continue;
            if (ptr >= nwords) return OR_WORD_OVERRUN;
            b[j] |= (uint32_t)get_u16(words_le + 2 * ptr) << n[j];
            n[j] += 16;
            ptr++;
        }
        for (uint32_t j = 0; j < OR_LANES; j++) {
            uint64_t p = lane_pos(t, j, K);
            if (p >= nk) continue;
            uint32_t v = 0, l = 0;
            int s = -1;
            while (s < 0) {
                if (l == OR_HUFF_MAXLEN) return OR_BAD_END_STATE; /* not a codeword */
                v = (v << 1) | (b[j] & 1u);
                b[j] >>= 1;
                n[j]--;
                l++;
                if (v - c->first[l] < c->count[l]) s = c->sorted[c->offset[l] + v - c->first[l]];
            }
            sym_out[p] = (uint8_t)s;
        }
    }
    uint32_t flags = 0;
    for (uint32_t j = 0; j < OR_LANES; j++)
        if (b[j]) flags |= OR_BAD_END_STATE;
    if (ptr != nwords) flags |= OR_BAD_END_STATE;
    return flags;
}

/* ------------------------------------------------------------------------ */
/* Container v1 encoder.                                                     */
/* ------------------------------------------------------------------------ */
/*
 * Layout, little-endian. Header of 256 bytes:
 *   0 u32 magic 'EQR1'     4 u16 version = 1     6 u8 dtype (1 int8, 2 e4m3)
 *   7 u8 flags (bit 0: escapes)                  8 u64 rows    16 u64 cols
 *  24 u64 n = rows*cols   32 u32 chunk_symbols Z 36 u32 lane run K
 *  40 u32 lanes = 64      44 u32 prob bits = 12  48 u64 n_chunks
 *  56 u64 n_esc           64 u8 escape code (rest of that 8-byte slot zero)
 *  72 u64 n_words (all chunks, with padding)
 *  80 off_freq  88 off_scales  96 off_dir  104 off_states  112 off_words
 * 120 off_esc_idx  128 off_esc_val  136 total_bytes   (all u64 byte offsets)
 * 144 u32 codec: 0 rANS (this section's coder), 1 Huffman (further below)
 * 148 u32 segment size in chunks (flags bit 1; 0 otherwise)
 * 152..255 zero.
 * Adaptive tables (flags bit 1, rANS only): the chunks are grouped into
 * segments of `seg` consecutive chunks (seg a multiple of 8) and each
 * segment is coded with its own 12-bit table; the freq section then holds
 * the tables of all segments in order (512 bytes each). Nothing else
 * changes: the chunk coder is the same, with the segment's table.
 * Sections, each starting on a 256-byte boundary, gaps zero:
 *   freq[256] u16 | scales[rows] f32 | dir[n_chunks] {u64 word_start,
 *   u32 word_count, u32 0} | states[n_chunks][64] u32 | words u16 (each
 *   chunk's words padded with zeros to a multiple of 8) | esc_idx[n_esc] u64
 *   strictly ascending | esc_val[n_esc] u16 (bf16 bits).
 * total_bytes = end of the last section rounded up to 256.
 */

typedef struct {
    uint32_t dtype, flags, Z, K, codec, seg;
    uint64_t rows, cols, n, n_chunks, n_esc, n_words;
    uint8_t esc_code;
    uint64_t off_freq, off_scales, off_dir, off_states, off_words, off_esc_idx, off_esc_val,
        total;
} or_hdr;

/* Encode one chunk: lanes start at state 2^16; steps are walked backwards
 * (t from T-1 down to 0, lane 63 down to 0) because rANS decodes in the
 * reverse order of encoding; the emitted words are then reversed so that the
 * decoder reads them front to back. words must hold nk entries (at most one
 * word per symbol). Returns the word count. */
static uint64_t encode_chunk(const uint8_t *sym, uint64_t nk, uint32_t K, const uint16_t freq[256],
                             const uint32_t cum[257], uint32_t states[64], uint16_t *words) {
    uint32_t x[64];
    for (uint32_t j = 0; j < OR_LANES; j++) x[j] = OR_L;
    uint64_t nw = 0;
    uint64_t T = chunk_steps(nk, K);
    for (uint64_t t = T; t-- > 0;) {
        for (uint32_t jj = OR_LANES; jj-- > 0;) {
            uint64_t p = lane_pos(t, jj, K);
            if (p >= nk) continue;
            uint8_t s = sym[p];
            uint16_t w;
            if (or_encode_step(&x[jj], freq[s], cum[s], &w)) words[nw++] = w;
        }
    }
    for (uint64_t a = 0, b = nw; a + 1 < b; a++, b--) {
        uint16_t tmp = words[a];
        words[a] = words[b - 1];
        words[b - 1] = tmp;
    }
    for (uint32_t j = 0; j < OR_LANES; j++) states[j] = x[j];
    return nw;
}

void or_free(void *p) { free(p); }

/* Build a container v1 for one [rows, cols] tensor of byte codes.
 * codec 0 (rANS): table = freq (sum 4096, nonzero for every present byte).
 * codec 1 (Huffman): table = code lengths (1..12, 0 absent, 0x100 for a lone
 *   zero-bit symbol), a complete prefix code covering every present byte.
 * esc_*: super-weight side list ([EQ] technical component 4), only with
 * esc_enabled; the stream holds esc_code exactly at the listed indices.
 * On success *out is a malloc'd buffer of *out_len bytes (free with or_free). */
int or_encode_seg(uint32_t codec, uint32_t dtype, uint64_t rows, uint64_t cols, const uint8_t *sym,
                  const float *scales, const uint16_t *tables, uint32_t seg, uint32_t Z, uint32_t K,
                  uint32_t esc_enabled, uint8_t esc_code, const uint64_t *esc_idx,
                  const uint16_t *esc_val, uint64_t n_esc, uint8_t **out, uint64_t *out_len);

int or_encode_codec(uint32_t codec, uint32_t dtype, uint64_t rows, uint64_t cols, const uint8_t *sym,
                    const float *scales, const uint16_t table[256], uint32_t Z, uint32_t K,
                    uint32_t esc_enabled, uint8_t esc_code, const uint64_t *esc_idx,
                    const uint16_t *esc_val, uint64_t n_esc, uint8_t **out, uint64_t *out_len) {
    return or_encode_seg(codec, dtype, rows, cols, sym, scales, table, 0, Z, K, esc_enabled, esc_code,
                         esc_idx, esc_val, n_esc, out, out_len);
}

/* As or_encode_codec; with seg > 0 (rANS only, a multiple of 8) `tables`
 * holds one frequency table per segment of seg chunks (ceil(n_chunks / seg)
 * tables of 256 entries) and chunk k is coded with table k / seg. */
int or_encode_seg(uint32_t codec, uint32_t dtype, uint64_t rows, uint64_t cols, const uint8_t *sym,
                  const float *scales, const uint16_t *tables, uint32_t seg, uint32_t Z, uint32_t K,
                  uint32_t esc_enabled, uint8_t esc_code, const uint64_t *esc_idx,
                  const uint16_t *esc_val, uint64_t n_esc, uint8_t **out, uint64_t *out_len) {
    *out = NULL;
    *out_len = 0;
    if (codec != OR_CODEC_RANS && codec != OR_CODEC_HUFF) return OR_EINVAL;
    if (seg && (codec != OR_CODEC_RANS || seg % 8)) return OR_EINVAL;
    if (dtype != OR_DTYPE_INT8 && dtype != OR_DTYPE_E4M3) return OR_EINVAL;
    if (rows == 0 || cols == 0) return OR_EINVAL;
    if (!(K == 1 || K == 2 || K == 4 || K == 8 || K == 16)) return OR_EINVAL;
    if (Z == 0 || Z % (OR_LANES * K) != 0) return OR_EINVAL;
    if (!esc_enabled && n_esc) return OR_EINVAL;
    uint64_t n = rows * cols;
    uint64_t n_chunks = (n + Z - 1) / Z;
    uint64_t n_tab = seg ? (n_chunks + seg - 1) / seg : 1;
    uint32_t cum[257];
    uint8_t s2s[4096];
    uint32_t code[256];
    for (uint64_t g = 0; g < n_tab; g++) {
        const uint16_t *table = tables + 256 * g;
        if (codec == OR_CODEC_RANS ? !make_tables(table, cum, s2s) : !or_huff_codes(table, code))
            return OR_EINVAL;
    }
    for (uint64_t i = 0; i < n; i++)
        if (tables[256 * (seg ? (i / Z) / seg : 0) + sym[i]] == 0) return OR_EINVAL;
    for (uint64_t e = 0; e < n_esc; e++) {
        if (esc_idx[e] >= n || (e > 0 && esc_idx[e] <= esc_idx[e - 1])) return OR_EINVAL;
        if (sym[esc_idx[e]] != esc_code) return OR_EINVAL;
    }
    if (esc_enabled) {
        uint64_t cnt = 0;
        for (uint64_t i = 0; i < n; i++) cnt += sym[i] == esc_code;
        if (cnt != n_esc) return OR_EINVAL;
    }

    uint64_t n_states = codec == OR_CODEC_RANS ? n_chunks * OR_LANES : 0;
    uint32_t *states = malloc((n_states ? n_states : 1) * sizeof(uint32_t));
    uint64_t *wcount = malloc(n_chunks * sizeof(uint64_t));
    uint16_t *cw = malloc((n ? n : 1) * sizeof(uint16_t)); /* words of all chunks, unpadded */
    uint64_t *wstart_unpadded = malloc(n_chunks * sizeof(uint64_t));
    if (!states || !wcount || !cw || !wstart_unpadded) {
        free(states); free(wcount); free(cw); free(wstart_unpadded);
        return OR_ENOMEM;
    }
    uint64_t used = 0, n_words = 0;
    for (uint64_t k = 0; k < n_chunks; k++) {
        uint64_t p0 = k * Z;
        uint64_t nk = (n - p0 < Z) ? n - p0 : Z;
        wstart_unpadded[k] = used;
        const uint16_t *table = tables + 256 * (seg ? k / seg : 0);
        if (codec == OR_CODEC_RANS) {
            make_tables(table, cum, s2s);
            wcount[k] = encode_chunk(sym + p0, nk, K, table, cum, states + k * OR_LANES, cw + used);
        } else {
            wcount[k] = huff_encode_chunk(sym + p0, nk, K, table, code, cw + used);
        }
        if (wcount[k] == UINT64_MAX) {
            free(states); free(wcount); free(cw); free(wstart_unpadded);
            return OR_ENOMEM;
        }
        used += wcount[k];
        n_words += align_up(wcount[k], 8);
    }

    or_hdr h;
    memset(&h, 0, sizeof h);
    h.off_freq = OR_HDR_BYTES;
    h.off_scales = align_up(h.off_freq + 512 * n_tab, OR_ALIGN);
    h.off_dir = align_up(h.off_scales + rows * 4, OR_ALIGN);
    h.off_states = align_up(h.off_dir + n_chunks * 16, OR_ALIGN);
    h.off_words = align_up(h.off_states + n_states * 4, OR_ALIGN);
    h.off_esc_idx = align_up(h.off_words + n_words * 2, OR_ALIGN);
    h.off_esc_val = align_up(h.off_esc_idx + n_esc * 8, OR_ALIGN);
    h.total = align_up(h.off_esc_val + n_esc * 2, OR_ALIGN);

    uint8_t *buf = calloc(h.total, 1);
    if (!buf) {
        free(states); free(wcount); free(cw); free(wstart_unpadded);
        return OR_ENOMEM;
    }
    put_u32(buf + 0, OR_MAGIC);
    put_u16(buf + 4, OR_VERSION);
    buf[6] = (uint8_t)dtype;
    buf[7] = (esc_enabled ? OR_FLAG_ESC : 0) | (seg ? OR_FLAG_SEG : 0);
    put_u64(buf + 8, rows);
    put_u64(buf + 16, cols);
    put_u64(buf + 24, n);
    put_u32(buf + 32, Z);
    put_u32(buf + 36, K);
    put_u32(buf + 40, OR_LANES);
    put_u32(buf + 44, codec == OR_CODEC_RANS ? OR_PROB_BITS : OR_HUFF_MAXLEN);
    put_u64(buf + 48, n_chunks);
    put_u64(buf + 56, n_esc);
    buf[64] = esc_enabled ? esc_code : 0;
    put_u64(buf + 72, n_words);
    put_u64(buf + 80, h.off_freq);
    put_u64(buf + 88, h.off_scales);
    put_u64(buf + 96, h.off_dir);
    put_u64(buf + 104, h.off_states);
    put_u64(buf + 112, h.off_words);
    put_u64(buf + 120, h.off_esc_idx);
    put_u64(buf + 128, h.off_esc_val);
    put_u64(buf + 136, h.total);
    put_u32(buf + 144, codec);
    put_u32(buf + 148, seg);

    for (uint64_t i = 0; i < 256 * n_tab; i++) put_u16(buf + h.off_freq + 2 * i, tables[i]);
    for (uint64_t r = 0; r < rows; r++) {
        uint32_t b;
        memcpy(&b, &scales[r], 4);
        put_u32(buf + h.off_scales + 4 * r, b);
    }
    uint64_t wpos = 0;
    for (uint64_t k = 0; k < n_chunks; k++) {
        put_u64(buf + h.off_dir + 16 * k, wpos);
        put_u32(buf + h.off_dir + 16 * k + 8, (uint32_t)wcount[k]);
        for (uint64_t i = 0; i < wcount[k]; i++)
            put_u16(buf + h.off_words + 2 * (wpos + i), cw[wstart_unpadded[k] + i]);
        wpos += align_up(wcount[k], 8);
        if (codec == OR_CODEC_RANS)
            for (uint32_t j = 0; j < OR_LANES; j++)
                put_u32(buf + h.off_states + 4 * (k * OR_LANES + j), states[k * OR_LANES + j]);
    }
    for (uint64_t e = 0; e < n_esc; e++) {
        put_u64(buf + h.off_esc_idx + 8 * e, esc_idx[e]);
        put_u16(buf + h.off_esc_val + 2 * e, esc_val[e]);
    }
    free(states); free(wcount); free(cw); free(wstart_unpadded);
    *out = buf;
    *out_len = h.total;
    return OR_OK;
}

/* The rANS container (codec 0) with its frequency table. */
int or_encode(uint32_t dtype, uint64_t rows, uint64_t cols, const uint8_t *sym,
              const float *scales, const uint16_t freq[256], uint32_t Z, uint32_t K,
              uint32_t esc_enabled, uint8_t esc_code, const uint64_t *esc_idx,
              const uint16_t *esc_val, uint64_t n_esc, uint8_t **out, uint64_t *out_len) {
    return or_encode_codec(OR_CODEC_RANS, dtype, rows, cols, sym, scales, freq, Z, K, esc_enabled,
                           esc_code, esc_idx, esc_val, n_esc, out, out_len);
}

/* ------------------------------------------------------------------------ */
/* Container v1 parser and decoder.                                          */
/* ------------------------------------------------------------------------ */

static int parse(const uint8_t *b, uint64_t len, or_hdr *h) {
    if (len < OR_HDR_BYTES) return OR_ECORRUPT;
    if (get_u32(b) != OR_MAGIC || get_u16(b + 4) != OR_VERSION) return OR_ECORRUPT;
    h->dtype = b[6];
    h->flags = b[7];
    h->rows = get_u64(b + 8);
    h->cols = get_u64(b + 16);
    h->n = get_u64(b + 24);
    h->Z = get_u32(b + 32);
    h->K = get_u32(b + 36);
    h->n_chunks = get_u64(b + 48);
    h->n_esc = get_u64(b + 56);
    h->esc_code = b[64];
    h->n_words = get_u64(b + 72);
    h->off_freq = get_u64(b + 80);
    h->off_scales = get_u64(b + 88);
    h->off_dir = get_u64(b + 96);
    h->off_states = get_u64(b + 104);
    h->off_words = get_u64(b + 112);
    h->off_esc_idx = get_u64(b + 120);
    h->off_esc_val = get_u64(b + 128);
    h->total = get_u64(b + 136);
    h->codec = get_u32(b + 144);
    h->seg = get_u32(b + 148);
    if (((h->flags & OR_FLAG_SEG) != 0) != (h->seg != 0)) return OR_ECORRUPT;
    if (h->seg && (h->seg % 8 || h->codec != OR_CODEC_RANS)) return OR_ECORRUPT;
    if (h->codec != OR_CODEC_RANS && h->codec != OR_CODEC_HUFF) return OR_ECORRUPT;
    if (h->dtype != OR_DTYPE_INT8 && h->dtype != OR_DTYPE_E4M3) return OR_ECORRUPT;
    if (!(h->K == 1 || h->K == 2 || h->K == 4 || h->K == 8 || h->K == 16)) return OR_ECORRUPT;
    if (h->Z == 0 || h->Z % (OR_LANES * h->K)) return OR_ECORRUPT;
    if (h->rows == 0 || h->cols == 0 || h->n / h->rows != h->cols || h->n % h->rows) return OR_ECORRUPT;
    if (h->n_chunks != (h->n + h->Z - 1) / h->Z) return OR_ECORRUPT;
    if (h->total > len) return OR_ECORRUPT;
    if (h->off_freq + 512 * (h->seg ? (h->n_chunks + h->seg - 1) / h->seg : 1) > h->total ||
        h->off_scales + 4 * h->rows > h->total ||
        h->off_dir + 16 * h->n_chunks > h->total ||
        h->off_states + (h->codec == OR_CODEC_RANS ? 4 * OR_LANES * h->n_chunks : 0) > h->total ||
        h->off_words + 2 * h->n_words > h->total || h->off_esc_idx + 8 * h->n_esc > h->total ||
        h->off_esc_val + 2 * h->n_esc > h->total)
        return OR_ECORRUPT;
    return OR_OK;
}

/* Decode one chunk into sym_out[0..nk): lanes start from the stored states;
 * step t ascending, lane j ascending; each active lane looks its slot up,
 * emits the symbol, steps its state back, and if the state fell below 2^16
 * reads the next word of the chunk. Accept iff every lane ends at 2^16 and
 * every stored word was read. Returns the flags. */
static uint32_t decode_chunk(const uint8_t *words_le, uint64_t nwords, const uint8_t *states_le,
                             uint64_t nk, uint32_t K, const uint16_t freq[256],
                             const uint32_t cum[257], const uint8_t s2s[4096], uint8_t *sym_out) {
    uint32_t x[64];
    for (uint32_t j = 0; j < OR_LANES; j++) x[j] = get_u32(states_le + 4 * j);
    uint64_t ptr = 0;
    uint32_t flags = 0;
    uint64_t T = chunk_steps(nk, K);
    for (uint64_t t = 0; t < T; t++) {
        for (uint32_t j = 0; j < OR_LANES; j++) {
            uint64_t p = lane_pos(t, j, K);
            if (p >= nk) continue;
            uint8_t s = s2s[x[j] % OR_M];
            sym_out[p] = s;
            if (or_decode_step(&x[j], freq[s], cum[s])) {
                if (ptr >= nwords) return flags | OR_WORD_OVERRUN;
                x[j] = (x[j] << 16) | get_u16(words_le + 2 * ptr);
                ptr++;
            }
        }
    }
    for (uint32_t j = 0; j < OR_LANES; j++)
        if (x[j] != OR_L) flags |= OR_BAD_END_STATE;
    if (ptr != nwords) flags |= OR_BAD_END_STATE;
    return flags;
}

typedef struct {
    const uint8_t *buf;
    const or_hdr *h;
    const uint16_t *freq;
    const uint32_t *cum;
    const uint8_t *s2s;
    const or_canon *canon; /* Huffman codec */
    uint64_t k_lo, k_hi;
    uint8_t *sym_out;   /* flat, indexed by position; may be NULL */
    uint16_t *bf16_out; /* flat, indexed by position; may be NULL */
    uint32_t flags;
} or_job;

static uint32_t decode_range(or_job *jb) {
    const or_hdr *h = jb->h;
    const uint8_t *b = jb->buf;
    uint32_t flags = 0;
    uint8_t *tmp = NULL;
    if (!jb->sym_out) {
        tmp = malloc(h->Z);
        if (!tmp) return OR_WORD_OVERRUN;
    }
    /* adaptive tables: the segment's own table (rebuilt when the segment changes) */
    uint16_t sfreq[256];
    uint32_t scum[257];
    uint8_t ss2s[4096];
    uint64_t cur_seg = UINT64_MAX;
    for (uint64_t k = jb->k_lo; k < jb->k_hi; k++) {
        const uint16_t *freq = jb->freq;
        const uint32_t *cum = jb->cum;
        const uint8_t *s2s = jb->s2s;
        if (h->seg) {
            if (k / h->seg != cur_seg) {
                cur_seg = k / h->seg;
                for (int t = 0; t < 256; t++) sfreq[t] = get_u16(b + h->off_freq + 512 * cur_seg + 2 * t);
                make_tables(sfreq, scum, ss2s); /* validated by or_decode_chunks */
            }
            freq = sfreq;
            cum = scum;
            s2s = ss2s;
        }
        uint64_t p0 = k * h->Z;
        uint64_t nk = (h->n - p0 < h->Z) ? h->n - p0 : h->Z;
        uint64_t ws = get_u64(b + h->off_dir + 16 * k);
        uint64_t wc = get_u32(b + h->off_dir + 16 * k + 8);
        if (ws + wc > h->n_words) { flags |= OR_WORD_OVERRUN; continue; }
        uint8_t *dst = jb->sym_out ? jb->sym_out + p0 : tmp;
        if (h->codec == OR_CODEC_RANS)
            flags |= decode_chunk(b + h->off_words + 2 * ws, wc, b + h->off_states + 4 * OR_LANES * k,
                                  nk, h->K, freq, cum, s2s, dst);
        else
            flags |= huff_decode_chunk(b + h->off_words + 2 * ws, wc, nk, h->K, jb->canon, dst);
        if (jb->bf16_out) {
            for (uint64_t i = 0; i < nk; i++) {
                uint64_t pos = p0 + i;
                float sc = get_f32(b + h->off_scales + 4 * (pos / h->cols));
                float prod = or_symbol_value(h->dtype, dst[i]) * sc;
                jb->bf16_out[pos] = or_bf16_rne(prod);
            }
            /* super weights inside this chunk: stored bf16 bits win */
            for (uint64_t e = 0; e < h->n_esc; e++) {
                uint64_t idx = get_u64(b + h->off_esc_idx + 8 * e);
                if (idx >= p0 && idx < p0 + nk)
                    jb->bf16_out[idx] = get_u16(b + h->off_esc_val + 2 * e);
            }
        }
    }
    free(tmp);
    return flags;
}

static void *decode_thread(void *arg) {
    or_job *jb = arg;
    jb->flags = decode_range(jb);
    return NULL;
}

/* Decode chunks [k_lo, k_hi) of a container with nthreads threads, each
 * taking a contiguous share of the chunks (the chunks are independent:
 * [EL] method item 3). sym_out / bf16_out are full-size flat outputs (either
 * may be NULL). Returns the ORed decode flags, or a negative status. */
int64_t or_decode_chunks(const uint8_t *buf, uint64_t len, uint64_t k_lo, uint64_t k_hi,
                         uint32_t nthreads, uint8_t *sym_out, uint16_t *bf16_out) {
    or_hdr h;
    int st = parse(buf, len, &h);
    if (st) return st;
    if (k_hi > h.n_chunks) k_hi = h.n_chunks;
    if (k_lo > k_hi) return OR_EINVAL;
    uint16_t freq[256];
    for (int s = 0; s < 256; s++) freq[s] = get_u16(buf + h.off_freq + 2 * s);
    uint32_t cum[257];
    uint8_t s2s[4096];
    or_canon canon;
    if (h.codec == OR_CODEC_RANS ? !make_tables(freq, cum, s2s) : !huff_canon(freq, &canon))
        return OR_ECORRUPT;
    if (h.seg) {
        uint16_t f2[256];
        uint32_t c2[257];
        uint8_t s2[4096];
        for (uint64_t g = 0; g < (h.n_chunks + h.seg - 1) / h.seg; g++) {
            for (int t = 0; t < 256; t++) f2[t] = get_u16(buf + h.off_freq + 512 * g + 2 * t);
            if (!make_tables(f2, c2, s2)) return OR_ECORRUPT;
        }
    }
    if (nthreads < 1) nthreads = 1;
    uint64_t nk = k_hi - k_lo;
    if (nthreads > nk) nthreads = nk ? (uint32_t)nk : 1;
    or_job *jobs = calloc(nthreads, sizeof(or_job));
    pthread_t *tid = calloc(nthreads, sizeof(pthread_t));
    if (!jobs || !tid) { free(jobs); free(tid); return OR_ENOMEM; }
    for (uint32_t i = 0; i < nthreads; i++) {
        jobs[i] = (or_job){buf, &h, freq, cum, s2s, &canon, k_lo + nk * i / nthreads,
                           k_lo + nk * (i + 1) / nthreads, sym_out, bf16_out, 0};
    }
    for (uint32_t i = 1; i < nthreads; i++) pthread_create(&tid[i], NULL, decode_thread, &jobs[i]);
    decode_thread(&jobs[0]);
    uint32_t flags = jobs[0].flags;
    for (uint32_t i = 1; i < nthreads; i++) {
        pthread_join(tid[i], NULL);
        flags |= jobs[i].flags;
    }
    free(jobs);
    free(tid);
    return flags;
}

/* Whole-container conveniences (single thread). */
int64_t or_decode_symbols(const uint8_t *buf, uint64_t len, uint8_t *sym_out) {
    return or_decode_chunks(buf, len, 0, UINT64_MAX, 1, sym_out, NULL);
}
int64_t or_decode_dequant(const uint8_t *buf, uint64_t len, uint16_t *bf16_out) {
    return or_decode_chunks(buf, len, 0, UINT64_MAX, 1, NULL, bf16_out);
}

/* Header fields for the Python side: fills v[0..16) with dtype, flags, rows,
 * cols, n, Z, K, n_chunks, n_esc, esc_code, n_words, off_freq, off_scales,
 * off_dir, off_states, off_words; v[16..21) = off_esc_idx, off_esc_val, total, codec, seg. */
int or_header_fields(const uint8_t *buf, uint64_t len, uint64_t v[21]) {
    or_hdr h;
    int st = parse(buf, len, &h);
    if (st) return st;
    uint64_t f[21] = {h.dtype, h.flags, h.rows, h.cols, h.n, h.Z, h.K, h.n_chunks, h.n_esc,
                      h.esc_code, h.n_words, h.off_freq, h.off_scales, h.off_dir, h.off_states,
                      h.off_words, h.off_esc_idx, h.off_esc_val, h.total, h.codec, h.seg};
    memcpy(v, f, sizeof f);
    return OR_OK;
}

/* Array form of or_bf16_rne (one call per element would be slow through
 * ctypes for the exhaustive checks). */
void or_bf16_rne_array(const float *v, uint64_t n, uint16_t *out) {
    for (uint64_t i = 0; i < n; i++) out[i] = or_bf16_rne(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Batch-1 GEMV over decoded weights.                                        */
/* ------------------------------------------------------------------------ */
/* [EQ] section 2, technical component 3: the decoded bf16 weights feed the
 * block's forward kernels; its limitations / future-work part proposes
 * fusing the decompression into the matrix-multiply kernel. For one token
 * that product is y[r] = sum_c W[r][c] * x[c] over a row-major [rows][cols]
 * bf16 W and a bf16 x. Here in binary64: a bf16 x bf16 product has at most
 * 16 significant bits, so every product is exact in double, and the sum in
 * ascending c is within (cols - 1) * 2^-53 * sum |W x| of the exact value.
 * absdot[r] = sum_c |W[r][c] * x[c]| (the scale of a summation-order error
 * bound). bf16 bits widen to binary32 by a 16-bit shift (the format is the
 * upper half of binary32). */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

void or_gemv_f64(const uint16_t *w, uint64_t rows, uint64_t cols, const uint16_t *x, double *y,
                 double *absdot) {
    for (uint64_t r = 0; r < rows; r++) {
        double s = 0.0, a = 0.0;
        for (uint64_t c = 0; c < cols; c++) {
            const double p = bf16_to_double(w[r * cols + c]) * bf16_to_double(x[c]);
            s += p;
            a += p < 0 ? -p : p;
        }
        y[r] = s;
        if (absdot) absdot[r] = a;
    }
}
