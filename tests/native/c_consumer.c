/*
 * A plain C consumer of libeq: it includes only include/eq.h and the HIP
 * runtime's C API, encodes one tensor with eq_encode_host, uploads the
 * container, decodes it with eq_decode_dequant_bf16 and eq_decode_block into
 * device buffers it allocated itself, and writes the outputs to a file. The
 * GPU test that runs it compares them with the oracle (this program computes
 * no expected values of its own).
 *
 * usage: c_consumer <input> <output>
 * input  (little-endian): u32 dtype, u32 lane_run, u32 chunk_symbols,
 *        u32 codec, u32 esc_code, u32 n_esc, u64 rows, u64 cols,
 *        u8 symbols[rows*cols], f32 scales[rows], u64 esc_idx[n_esc],
 *        u16 esc_bf16[n_esc]
 * output: u32 status word, u64 container bytes, u16 bf16[rows*cols],
 *         u8 symbols[rows*cols]
 * Exit status 0 on success; any library or runtime error prints its name and
 * exits with 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "eq.h"

#define CHECK_EQ(call)                                                                      \
    do {                                                                                    \
        eq_status st_ = (call);                                                             \
        if (st_ != EQ_OK) {                                                                 \
            fprintf(stderr, "%s: %s (%d)\n", #call, eq_status_string(st_), (int)st_);      \
            exit(1);                                                                        \
        }                                                                                   \
    } while (0)
#define CHECK_HIP(call)                                                                     \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess) {                                                             \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                     \
            exit(1);                                                                        \
        }                                                                                   \
    } while (0)

static void read_exact(FILE *f, void *p, size_t n) {
    if (n && fread(p, 1, n, f) != n) {
        fprintf(stderr, "short input\n");
        exit(1);
    }
}

static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of host memory\n");
        exit(1);
    }
    return p;
}

int main(int argc, char **argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s <input> <output>\n", argv[0]);
        return 2;
    }
    FILE *in = fopen(argv[1], "rb");
    if (!in) {
        perror(argv[1]);
        return 1;
    }
    uint32_t hdr6[6];
    uint64_t rc[2];
    read_exact(in, hdr6, sizeof hdr6);
    read_exact(in, rc, sizeof rc);
    const uint64_t rows = rc[0], cols = rc[1], n = rows * cols;
    const uint32_t n_esc = hdr6[5];
    uint8_t *sym = xmalloc(n);
    float *scales = xmalloc(rows * sizeof(float));
    uint64_t *esc_idx = xmalloc(n_esc * sizeof(uint64_t));
    uint16_t *esc_val = xmalloc(n_esc * sizeof(uint16_t));
    read_exact(in, sym, n);
    read_exact(in, scales, rows * sizeof(float));
    read_exact(in, esc_idx, n_esc * sizeof(uint64_t));
    read_exact(in, esc_val, n_esc * sizeof(uint16_t));
    fclose(in);

    /* encode on the host */
    eq_tables tab;
    CHECK_EQ(eq_build_tables(sym, n, &tab));
    eq_tensor_desc d;
    memset(&d, 0, sizeof d);
    d.dtype = hdr6[0];
    d.lane_run = hdr6[1];
    d.rows = rows;
    d.cols = cols;
    d.chunk_symbols = hdr6[2];
    d.codec = hdr6[3];
    d.esc_enabled = n_esc ? 1u : 0u;
    d.esc_code = hdr6[4];
    uint64_t len = 0;
    eq_status st = eq_encode_host(&tab, &d, sym, scales, n_esc ? esc_idx : NULL, n_esc ? esc_val : NULL, n_esc,
                                  NULL, 0, &len);
    if (st != EQ_ERANGE || len == 0) {
        fprintf(stderr, "size query: %s (%d)\n", eq_status_string(st), (int)st);
        return 1;
    }
    uint8_t *blob = xmalloc(len);
    CHECK_EQ(eq_encode_host(&tab, &d, sym, scales, n_esc ? esc_idx : NULL, n_esc ? esc_val : NULL, n_esc, blob,
                            len, &len));
    eq_tensor_ref ref;
    memset(&ref, 0, sizeof ref);
    CHECK_EQ(eq_parse_header(blob, len, &ref.hdr));

    /* device buffers of our own */
    void *d_cont = NULL, *d_bf16 = NULL, *d_u8 = NULL, *d_status = NULL;
    CHECK_HIP(hipMalloc(&d_cont, len));
    CHECK_HIP(hipMalloc(&d_bf16, n * 2));
    CHECK_HIP(hipMalloc(&d_u8, n));
    CHECK_HIP(hipMalloc(&d_status, sizeof(uint32_t)));
    CHECK_HIP(hipMemcpy(d_cont, blob, len, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(d_status, 0, sizeof(uint32_t)));
    hipStream_t s;
    CHECK_HIP(hipStreamCreate(&s));
    ref.d_container = d_cont;
    ref.out_offset = 0;
    eq_block b;
    memset(&b, 0, sizeof b);
    b.n_tensors = 1;
    b.tensors = &ref;
    b.d_status = (uint32_t *)d_status;
    CHECK_EQ(eq_decode_dequant_bf16(&b, (uint16_t *)d_bf16, s));
    CHECK_EQ(eq_decode_block(&b, (uint8_t *)d_u8, s));
    CHECK_HIP(hipStreamSynchronize(s));

    uint32_t status = 0;
    uint16_t *bf16 = xmalloc(n * 2);
    CHECK_HIP(hipMemcpy(&status, d_status, sizeof status, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(bf16, d_bf16, n * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(sym, d_u8, n, hipMemcpyDeviceToHost));

    FILE *out = fopen(argv[2], "wb");
    if (!out) {
        perror(argv[2]);
        return 1;
    }
    if (fwrite(&status, sizeof status, 1, out) != 1 || fwrite(&len, sizeof len, 1, out) != 1 ||
        fwrite(bf16, 2, n, out) != n || fwrite(sym, 1, n, out) != n) {
        fprintf(stderr, "short write\n");
        return 1;
    }
    fclose(out);
    CHECK_HIP(hipStreamDestroy(s));
    CHECK_HIP(hipFree(d_cont));
    CHECK_HIP(hipFree(d_bf16));
    CHECK_HIP(hipFree(d_u8));
    CHECK_HIP(hipFree(d_status));
    free(sym);
    free(scales);
    free(esc_idx);
    free(esc_val);
    free(blob);
    free(bf16);
    return 0;
}
