/*
 * Sanitizer driver: the host library's encoder / parser and the oracle's
 * encoder / decoder, built together with AddressSanitizer and
 * UndefinedBehaviorSanitizer (host code only), on random layouts of every
 * container variant (rANS, Huffman, per-segment tables, super-weight
 * escapes, int8 and E4M3), plus corrupted containers fed to both parsers.
 * Checks byte equality of the two encoders' containers and the oracle's
 * round trip; any sanitizer report aborts the process.
 * Usage: sanitize_driver <iterations> <seed>. Exit 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "eq.h"

int or_build_freq(const uint8_t *sym, uint64_t n, uint16_t freq[256]);
int or_huff_lengths(const uint64_t counts[256], uint32_t L, uint8_t len[256]);
int or_encode_seg(uint32_t codec, uint32_t dtype, uint64_t rows, uint64_t cols, const uint8_t *sym,
                  const float *scales, const uint16_t *tables, uint32_t seg, uint32_t Z, uint32_t K,
                  uint32_t esc_enabled, uint8_t esc_code, const uint64_t *esc_idx,
                  const uint16_t *esc_val, uint64_t n_esc, uint8_t **out, uint64_t *out_len);
int64_t or_decode_symbols(const uint8_t *buf, uint64_t len, uint8_t *sym_out);
int64_t or_decode_dequant(const uint8_t *buf, uint64_t len, uint16_t *bf16_out);
void or_dequant_direct(uint32_t dtype, const uint8_t *sym, uint64_t n, uint64_t cols, const float *scales,
                       const uint64_t *esc_idx, const uint16_t *esc_val, uint64_t n_esc, uint16_t *out);
void or_free(void *p);

static uint64_t st;
static uint64_t rnd(void) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return st;
}

#define FAIL(...)                          \
    do {                                   \
        fprintf(stderr, __VA_ARGS__);      \
        fprintf(stderr, " (iter %d)\n", it); \
        return 1;                          \
    } while (0)

int main(int argc, char **argv) {
    int iters = argc > 1 ? atoi(argv[1]) : 200;
    st = argc > 2 ? strtoull(argv[2], NULL, 0) : 88172645463325252ull;
    if (!st) st = 1;
    static const uint32_t Ks[5] = {1, 2, 4, 8, 16};
    for (int it = 0; it < iters; it++) {
        const uint32_t K = Ks[rnd() % 5];
        const uint32_t codec = it % 3 == 1 ? EQ_CODEC_HUFFMAN : EQ_CODEC_RANS;
        const uint32_t seg = (it % 3 == 2) ? 8u * (uint32_t)(1 + rnd() % 2) : 0u;
        const uint32_t Z = 64u * K * (uint32_t)(1 + rnd() % 4);
        const uint64_t n = 1 + rnd() % (seg ? 3ull * seg * Z : 3ull * Z);
        uint64_t rows = 1;
        for (uint64_t d = 1 + rnd() % 16; d >= 1; d--)
            if (n % d == 0) { rows = d; break; }
        const uint64_t cols = n / rows;
        const uint32_t dtype = (it % 5 == 4) ? EQ_DTYPE_E4M3 : EQ_DTYPE_INT8;
        const int esc = (it % 4 == 3);
        const uint8_t esc_code = dtype == EQ_DTYPE_INT8 ? 0x80 : 0x7F;
        /* symbols: a skewed draw over k distinct bytes (never the escape code
         * or an E4M3 NaN code) */
        uint8_t alpha[40];
        uint32_t k = 1 + (uint32_t)(rnd() % 30), na = 0;
        while (na < k) {
            uint8_t b = (uint8_t)rnd();
            if (b == 0x80 || b == 0x7F || b == 0xFF) continue;
            int dup = 0;
            for (uint32_t i = 0; i < na; i++) dup |= alpha[i] == b;
            if (!dup) alpha[na++] = b;
        }
        uint8_t *sym = malloc(n);
        float *sc = malloc(rows * sizeof(float));
        for (uint64_t i = 0; i < n; i++) {
            uint32_t r = (uint32_t)(rnd() % 1000), j = 0;
            while (j + 1 < k && r < 500) { r = r * 2 + 1; j++; } /* geometric-ish */
            sym[i] = alpha[(j + (uint32_t)(rnd() % 2)) % k];
        }
        for (uint64_t r = 0; r < rows; r++) sc[r] = ((float)(rnd() % 20001) - 10000.0f) * 1e-6f;
        uint64_t eidx[6];
        uint16_t evals[6];
        uint64_t n_esc = 0;
        if (esc) {
            uint64_t p = rnd() % n;
            while (n_esc < 6 && p < n) {
                eidx[n_esc] = p;
                evals[n_esc] = (uint16_t)rnd();
                sym[p] = esc_code;
                n_esc++;
                p += 1 + rnd() % (n / 3 + 1);
            }
        }
        /* the library */
        eq_tables t;
        if (eq_build_tables(sym, n, &t) != EQ_OK) FAIL("eq_build_tables");
        eq_tensor_desc d = {dtype, K, rows, cols, Z, (uint32_t)esc, esc ? esc_code : 0u, codec, seg, 0};
        uint64_t need = 0;
        eq_status s = eq_encode_host(seg ? NULL : &t, &d, sym, sc, n_esc ? eidx : NULL,
                                     n_esc ? evals : NULL, n_esc, NULL, 0, &need);
        if (s != EQ_ERANGE) FAIL("size query %d", s);
        uint8_t *lib = malloc(need);
        uint64_t got = 0;
        s = eq_encode_host(seg ? NULL : &t, &d, sym, sc, n_esc ? eidx : NULL, n_esc ? evals : NULL, n_esc,
                           lib, need, &got);
        if (s != EQ_OK || got != need) FAIL("eq_encode_host %d", s);
        eq_header h;
        if (eq_parse_header(lib, got, &h) != EQ_OK) FAIL("eq_parse_header");
        /* the oracle, on its own tables */
        uint64_t n_chunks = (n + Z - 1) / Z, n_tab = seg ? (n_chunks + seg - 1) / seg : 1;
        uint16_t *tabs = calloc(256 * n_tab, sizeof(uint16_t));
        if (codec == EQ_CODEC_HUFFMAN) {
            uint64_t counts[256] = {0};
            uint8_t len[256];
            for (uint64_t i = 0; i < n; i++) counts[sym[i]]++;
            if (or_huff_lengths(counts, 12, len)) FAIL("or_huff_lengths");
            uint32_t present = 0;
            for (int b = 0; b < 256; b++) present += counts[b] != 0;
            for (int b = 0; b < 256; b++) tabs[b] = (present == 1 && counts[b]) ? 0x100 : len[b];
        } else {
            for (uint64_t g = 0; g < n_tab; g++) {
                uint64_t lo = g * (seg ? seg : 1) * (uint64_t)Z, hi = seg ? lo + (uint64_t)seg * Z : n;
                if (hi > n) hi = n;
                if (or_build_freq(sym + lo, hi - lo, tabs + 256 * g)) FAIL("or_build_freq");
            }
        }
        uint8_t *orc = NULL;
        uint64_t olen = 0;
        if (or_encode_seg(codec, dtype, rows, cols, sym, sc, tabs, seg, Z, K, (uint32_t)esc, esc ? esc_code : 0,
                          eidx, evals, n_esc, &orc, &olen))
            FAIL("or_encode_seg");
        if (olen != got || memcmp(orc, lib, got) != 0) FAIL("containers differ");
        uint8_t *dec = malloc(n);
        uint16_t *bf = malloc(n * 2), *ref = malloc(n * 2);
        if (or_decode_symbols(lib, got, dec) != 0 || memcmp(dec, sym, n) != 0) FAIL("round trip");
        if (or_decode_dequant(lib, got, bf) != 0) FAIL("dequant flags");
        or_dequant_direct(dtype, sym, n, cols, sc, eidx, evals, n_esc, ref);
        if (memcmp(bf, ref, n * 2) != 0) FAIL("dequant differs");
        /* corrupted copies: any status is fine, no crash and no report */
        uint8_t *bad = malloc(got);
        for (int c = 0; c < 12; c++) {
            memcpy(bad, lib, got);
            uint64_t at = c < 6 ? rnd() % 256 : rnd() % got;
            bad[at] ^= (uint8_t)(1u << (rnd() % 8));
            uint64_t len = c == 11 ? got - 1 - rnd() % (got < 256 ? got - 1 : 256) : got;
            eq_header hb;
            (void)eq_parse_header(bad, len, &hb);
            (void)or_decode_symbols(bad, len, dec);
        }
        free(bad);
        free(dec);
        free(bf);
        free(ref);
        or_free(orc);
        free(tabs);
        free(lib);
        free(sc);
        free(sym);
    }
    printf("ok %d\n", iters);
    return 0;
}
