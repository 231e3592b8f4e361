/*
 * eq.h -- C ABI of libeq.so: entropy-coded Int8 / Float8 weight streams,
 * decoded on an MI355X (gfx950) into bf16 weight buffers.
 *
 * The operation, as the pages state it ("Float8@2bits: Entropy Coding Enables
 * Data-Free Model Compression", EntQuant technical summary, section 2):
 *  - core concept: weights keep an Int8 or Float8 base format, are made
 *    low-entropy, and are compressed losslessly with an ANS coder;
 *  - technical component 1: per-channel scaling parameters S;
 *  - technical component 2 (weight encoding): the weights are flattened into
 *    one symbol stream and ANS-compressed; what is stored is the compressed
 *    bitstream, the scales and metadata;
 *  - technical component 3 (inference-time decoding): the bitstream stays in
 *    GPU memory and, just before each transformer block runs, a parallel ANS
 *    decoder expands that block's weights into a buffer;
 *  - technical component 4 (super weights): extreme outliers are excluded
 *    from the entropy-optimised stream (Int8 base format).
 * "EntroLLM: Entropy Encoded Weight Compression for Efficient Large Language
 * Model Inference on Edge Devices", technical overview, method item 2: the
 * quantised weights are Huffman-coded (frequent values get short codes);
 * method item 3: the coded parameter space is split into chunks that keep
 * the tensor structure and are decoded independently and concurrently.
 *
 * So: byte symbols + a frequency table + per-row fp32 scales in, a bf16
 * [rows, cols] weight matrix out, with
 *     out[i] = bf16_RNE( fp32( value(sym[i]) * S[i / cols] ) )
 * (value: two's-complement int8, or OCP E4M3FN), and each super weight's
 * stored bf16 bits written over its position.
 *
 * CONTAINER v1 (one per tensor; little-endian; the pages fix no bit-level
 * choice, so this layout is this library's own):
 *  - static rANS over the 256 byte codes; 12-bit frequencies (sum 4096);
 *    u32 state in [2^16, 2^32); 16-bit renormalisation words;
 *  - the tensor's row-major symbol stream is cut into chunks of Z symbols
 *    (Z a multiple of 64*K; the last chunk may be shorter); each chunk is
 *    coded by 64 interleaved lanes: at step t lane j codes chunk position
 *    (t / K) * 64K + j * K + (t mod K), so K consecutive steps of one lane
 *    produce K consecutive symbols (the lane run K is 1, 2, 4, 8 or 16);
 *  - within a chunk, words are read in order of increasing step and, within
 *    a step, increasing lane among the lanes whose state fell below 2^16;
 *    each chunk stores its 64 final encoder states, which are the decoder's
 *    start states; a lane with no symbols stores 2^16;
 *  - header (256 bytes): 0 u32 magic "EQR1", 4 u16 version 1, 6 u8 dtype,
 *    7 u8 flags (bit 0: super-weight escapes), 8 u64 rows, 16 u64 cols,
 *    24 u64 n, 32 u32 Z, 36 u32 K, 40 u32 lanes (64), 44 u32 probability bits
 *    (12), 48 u64 n_chunks, 56 u64 n_esc, 64 u8 escape code, 72 u64 n_words,
 *    80..136 u64 byte offsets of: freq, scales, dir, states, words, esc_idx,
 *    esc_val, then total size; the rest zero;
 *  - sections, each at a 256-byte boundary: freq[256] u16 | scales[rows] f32 |
 *    dir[n_chunks] {u64 first word, u32 word count, u32 0} | states
 *    [n_chunks][64] u32 | words u16 (each chunk padded with zeros to a
 *    multiple of 8 words) | esc_idx[n_esc] u64 ascending | esc_val[n_esc] u16.
 *  - frequency quantiser (eq_build_tables): f_s = max(1, floor(c_s*4096/N))
 *    for present bytes; the shortfall goes +1 each to the present bytes with
 *    the largest (c_s*4096) mod N (ties: smaller byte); an excess is taken -1
 *    at a time from the largest f_s > 1 (ties: smaller byte).
 *  - super weights: the stream holds the escape code exactly at the listed
 *    flat indices (the code is coded like any symbol); decode writes the
 *    listed bf16 bits there.
 *  - header offset 144, u32 codec: 0 = the rANS coder above; 1 = Huffman
 *    (EntroLLM's coder, same chunks, lanes, sections and outputs):
 *      - the freq section holds code lengths (u16: 0 absent, 1..12 bits, or
 *        0x100 for a lone symbol coded in zero bits); probability bits
 *        (offset 44) = 12, the longest codeword; no states section (size 0);
 *      - lengths: optimal prefix code over the exact symbol counts with
 *        codewords of at most 12 bits (package-merge; coins sorted by
 *        (count, byte), a coin before a package of equal weight);
 *        canonical codewords in (length, byte) order;
 *      - each lane's bitstream is its codewords, most significant bit
 *        first, packed into 16-bit words from bit 0 up; at every step each
 *        active lane holding fewer than 12 bits first takes the next word
 *        of the chunk (lanes in ascending order; zero words once its
 *        bitstream has ended), then every active lane decodes one codeword;
 *      - a chunk is valid iff all its words are taken and every lane's
 *        leftover bits are zero.
 *  - adaptive tables (flags bit 1, rANS only): header offset 148 u32
 *    seg_chunks (a multiple of 8); chunks are grouped into segments of
 *    seg_chunks consecutive chunks, each coded with its own 12-bit table
 *    (the quantiser above on the segment's counts); the freq section holds
 *    the ceil(n_chunks / seg_chunks) tables in order, 512 bytes each.
 *
 * CONVENTIONS
 *  - Every function returns an eq_status; no exception crosses the ABI.
 *  - Ownership: the caller owns every host and device buffer. Decode calls
 *    never allocate, free or synchronise: they only enqueue kernels on the
 *    given stream (a hipStream_t passed as void*; NULL = the null stream).
 *  - Device errors found while decoding are ORed into *d_status as
 *    EQ_DEV_* bits; read them after synchronising. After such an error the
 *    output contents are unspecified.
 *  - Thread-safe and reentrant; no global mutable state, except the per-GPU
 *    scratch array of eq_encode_device_static (see there).
 */
#ifndef EQ_H
#define EQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t eq_status;
#define EQ_OK 0
#define EQ_EINVAL (-1)       /* bad argument (NULL, size, unsupported value) */
#define EQ_ERANGE (-2)       /* output buffer too small; *out_len holds the size */
#define EQ_ECORRUPT (-3)     /* container header or tables inconsistent */
#define EQ_EHIP (-4)         /* HIP launch / runtime error */
#define EQ_EUNSUPPORTED (-5) /* valid container this library version cannot decode */
#define EQ_ENOMEM (-6)       /* host allocation failed (encoder scratch) */

/* Device status bits (ORed into eq_block.d_status). */
#define EQ_DEV_BAD_END_STATE 1u /* a lane did not end at 2^16, or words left over */
#define EQ_DEV_WORD_OVERRUN 2u  /* a chunk read past its word count / bad dir entry */
#define EQ_DEV_BAD_INPUT 4u     /* eq_encode_device: invalid symbols, escapes or scales */

#define EQ_DTYPE_INT8 1u /* two's-complement int8 codes */
#define EQ_DTYPE_E4M3 2u /* OCP FP8 E4M3FN codes */

#define EQ_CODEC_RANS 0u    /* container codec: interleaved rANS (EntQuant's ANS) */
#define EQ_CODEC_HUFFMAN 1u /* container codec: interleaved canonical Huffman (EntroLLM) */
#define EQ_HUFF_MAX_LEN 12u /* longest Huffman codeword, bits */

#define EQ_LANES 64u
#define EQ_MAX_BLOCK_TENSORS 16u /* tensors per kernel launch (more: several launches) */

/* Frequency table of one tensor. */
typedef struct eq_tables {
    uint64_t counts[256]; /* histogram of the symbols */
    uint64_t n;           /* number of symbols */
    uint16_t freq[256];   /* quantised frequencies, sum 4096 */
    uint32_t cum[257];    /* cum[s] = sum of freq[t] for t < s; cum[256] = 4096 */
} eq_tables;

/* What eq_encode_host is asked to produce. */
typedef struct eq_tensor_desc {
    uint32_t dtype;         /* EQ_DTYPE_INT8 or EQ_DTYPE_E4M3 */
    uint32_t lane_run;      /* K: 1, 2, 4, 8 or 16 */
    uint64_t rows, cols;    /* [rows, cols] row-major, rows = output channels */
    uint32_t chunk_symbols; /* Z: multiple of 64*K, at most 2^24 */
    uint32_t esc_enabled;   /* 1: stream carries super-weight escapes */
    uint32_t esc_code;      /* the escape byte (used when esc_enabled) */
    uint32_t codec;         /* EQ_CODEC_RANS (0) or EQ_CODEC_HUFFMAN */
    uint32_t seg_chunks;    /* 0: one table per tensor; else chunks per table (a multiple of 8, rANS) */
    uint32_t reserved;      /* 0 */
} eq_tensor_desc;

/* Parsed, validated container header (host copy). */
typedef struct eq_header {
    uint32_t dtype, flags, chunk_symbols, lane_run;
    uint64_t rows, cols, n, n_chunks, n_esc, n_words;
    uint32_t esc_code;
    int32_t single_symbol; /* byte of a one-symbol tensor (f = 4096 / zero-bit code), else -1 */
    uint32_t codec;        /* EQ_CODEC_RANS or EQ_CODEC_HUFFMAN */
    uint32_t seg_chunks;   /* chunks per frequency table (adaptive tables), 0 = one table */
    uint64_t off_freq, off_scales, off_dir, off_states, off_words, off_esc_idx, off_esc_val;
    uint64_t total_bytes;
} eq_header;

/* One tensor of a block: its container in device memory and where its
 * output goes. */
typedef struct eq_tensor_ref {
    const void *d_container; /* device pointer, 16-byte aligned, immutable while decoding */
    eq_header hdr;           /* from eq_parse_header on the same bytes */
    uint64_t out_offset;     /* element offset of this tensor in the output buffer */
} eq_tensor_ref;

/* A set of tensors decoded by one call (e.g. a transformer block's q, k, v,
 * o, gate, up, down into one buffer). */
typedef struct eq_block {
    uint32_t n_tensors;             /* 0 is allowed (nothing is enqueued) */
    uint32_t reserved;              /* 0 */
    const eq_tensor_ref *tensors;   /* host array of n_tensors */
    uint32_t *d_status;             /* device u32, caller-zeroed; may be NULL */
} eq_block;

/*
 * eq_build_tables -- histogram + 12-bit frequency quantiser (the container's
 * "metadata", technical component 2 of the EntQuant summary).
 * symbols: host array of n byte codes (escape codes included). out: caller's.
 * Errors: EQ_EINVAL if symbols/out is NULL, n == 0 or n >= 2^51.
 */
eq_status eq_build_tables(const uint8_t *symbols, uint64_t n, eq_tables *out);

/*
 * eq_tables_from_freq -- an eq_tables for a given 12-bit frequency table (any
 * valid table, not necessarily the quantiser's): copies freq and derives the
 * cumulative frequencies cum (counts and n are zero). The metadata half of
 * technical component 2 of the EntQuant summary, for callers that bring
 * their own table. freq: host array of 256 entries summing to 4096.
 * Errors: EQ_EINVAL (NULL, or the entries do not sum to 4096).
 */
eq_status eq_tables_from_freq(const uint16_t *freq, eq_tables *out);

/*
 * eq_encode_host -- offline ANS encoding of one tensor into container v1
 * (technical component 2 of the EntQuant summary: flatten, ANS-compress,
 * store bitstream + scales + metadata). Host only, multi-threaded over chunks.
 * t: tables whose freq covers every symbol present (eq_build_tables output or
 *    any valid table); with d->codec = EQ_CODEC_HUFFMAN the code lengths are
 *    derived from t->counts instead (EntroLLM method item 2), so every
 *    present symbol needs a nonzero count; with d->seg_chunks > 0 (adaptive
 *    tables) each segment's table is quantised from its own counts and t is
 *    not read (may be NULL); d: shape and layout; symbols: rows*cols bytes; scales:
 *    rows finite fp32; esc_idx / esc_bf16: n_esc strictly ascending flat
 *    indices and their bf16 bits (NULL when n_esc == 0).
 * out / cap: caller's buffer. If out is NULL or cap is too small the call
 *    returns EQ_ERANGE with *out_len = the exact container size; on success
 *    *out_len = bytes written.
 * Errors (EQ_EINVAL): a symbol with frequency 0; freq not summing to 4096;
 *    an escape list that does not match the escape-code positions (or
 *    escapes without esc_enabled); an E4M3 NaN code outside the escapes; a
 *    non-finite scale; K not in {1,2,4,8,16}; Z not a multiple of 64*K or
 *    above 2^24; rows or cols 0; an unknown codec. EQ_ENOMEM if scratch
 *    allocation fails.
 */
eq_status eq_encode_host(const eq_tables *t, const eq_tensor_desc *d, const uint8_t *symbols,
                         const float *scales, const uint64_t *esc_idx, const uint16_t *esc_bf16,
                         uint64_t n_esc, void *out, uint64_t cap, uint64_t *out_len);

/*
 * eq_parse_header -- full host-side validation of a container (header,
 * section bounds and alignment, frequency sum, chunk directory, escape list)
 * and extraction of its header. bytes: host copy of the whole container.
 * Errors: EQ_EINVAL (NULL), EQ_ECORRUPT (any inconsistency).
 */
eq_status eq_parse_header(const void *bytes, uint64_t len, eq_header *out);

/*
 * eq_decode_block -- enqueue the parallel ANS decode of every tensor in b
 * (technical component 3 of the EntQuant summary; chunks decoded
 * concurrently as in EntroLLM's method item 3), writing the raw byte codes
 * (escape codes included) to d_symbols + tensor.out_offset.
 * d_symbols: device buffer of u8. stream: hipStream_t or NULL.
 * Errors: EQ_EINVAL (NULL pointers, header/offset inconsistencies),
 * EQ_EHIP (launch failure). Device-side integrity flags go to b->d_status.
 */
eq_status eq_decode_block(const eq_block *b, uint8_t *d_symbols, void *stream);

/*
 * eq_decode_dequant_bf16 -- enqueue decode + per-row dequantisation + bf16
 * rounding (RNE) + super-weight patch for every tensor in b, into the bf16
 * buffer d_bf16 (u16 bit patterns) at each tensor's out_offset: the
 * decompression into a buffer just before a block's forward pass
 * (technical component 3 of the EntQuant summary), with the per-channel
 * scales of technical component 1 and the super weights of component 4.
 * Errors: as eq_decode_block.
 */
eq_status eq_decode_dequant_bf16(const eq_block *b, uint16_t *d_bf16, void *stream);

/*
 * eq_decode_gemv_bf16 -- fused decode + dequantisation + batch-1 GEMV for
 * every tensor i of b: y_i[r] = sum_c W_i[r, c] * x_i[c], where W_i is
 * exactly the bf16 matrix eq_decode_dequant_bf16 would write (scales, RNE,
 * super weights), but is never written: each wave multiplies the weights it
 * decodes by x in registers. This is the decompression fused into the
 * matrix-multiply kernel that the EntQuant summary names as future work (its
 * limitations / future-directions part); HBM traffic per weight falls from
 * the compressed bytes + 2 B written + 2 B read back to the compressed bytes.
 * d_x: host array of n_tensors device pointers, tensor i's bf16 input
 *    [cols_i] (16-byte aligned). d_y: host array of n_tensors device
 *    pointers, its fp32 output [rows_i]. tensors[i].out_offset is ignored.
 * Requirements: chunk_symbols a multiple of cols (chunks hold whole rows) and
 *    cols a multiple of lane_run; otherwise EQ_EUNSUPPORTED (encode with such
 *    a chunk size, e.g. two 28672-column rows per chunk).
 * Arithmetic: fp32 accumulation of exact bf16 x bf16 products (v_dot2 on
 *    pairs, per-lane partials, fixed-order wave reduction): deterministic, but
 *    not bit-reproducible against other summation orders.
 * Errors: as eq_decode_block, plus EQ_EUNSUPPORTED.
 */
eq_status eq_decode_gemv_bf16(const eq_block *b, const uint16_t *const *d_x, float *const *d_y,
                              void *stream);

/*
 * eq_encode_device -- the encoder of eq_encode_host on the GPU, for every
 * container variant: rANS with one table, rANS with one table per segment of
 * seg_chunks chunks, Huffman. Histogram(s), the same 12-bit quantiser (as
 * eq_build_tables) or the same length-limited Huffman code, chunk-parallel
 * interleaved encoding, container assembly; the container is byte-for-byte
 * what eq_encode_host writes for the same descriptor with the tables built
 * from the symbols (eq_build_tables; with seg_chunks, tables NULL). This is
 * the offline ANS compression of technical component 2 of the EntQuant
 * summary (flatten, ANS-compress, store bitstream + scales + metadata), done
 * where the weights already are.
 * d: as for eq_encode_host (codec EQ_CODEC_RANS or EQ_CODEC_HUFFMAN;
 *    seg_chunks 0 or a multiple of 8 with the rANS codec, else EQ_EINVAL).
 *    Device pointers: d_symbols (rows*cols bytes, 16-byte aligned), d_scales
 *    (rows fp32), d_esc_idx / d_esc_bf16 (n_esc entries, may be NULL when
 *    n_esc == 0), d_workspace (workspace_bytes >= eq_encode_device_workspace(),
 *    16-byte aligned, contents ignored), d_out (cap >= eq_encode_device_bound(),
 *    16-byte aligned), d_out_len (device u64 receiving the container size; may
 *    be NULL), d_status (device u32, caller zeroed, may be NULL:
 *    EQ_DEV_BAD_INPUT when a symbol, escape list or scale is invalid; the
 *    container is then unspecified).
 * eq_encode_device_bound is an upper bound for every codec and segment size
 * (lane states and the most tables included).
 * Enqueues six kernels on stream; never allocates or synchronises.
 * Errors: EQ_EINVAL (arguments, codec, segment size), EQ_ERANGE (workspace or
 * cap too small), EQ_EHIP (launch).
 */
uint64_t eq_encode_device_bound(uint64_t rows, uint64_t cols, uint32_t chunk_symbols, uint64_t n_esc);
uint64_t eq_encode_device_workspace(uint64_t rows, uint64_t cols, uint32_t chunk_symbols);
eq_status eq_encode_device(const eq_tensor_desc *d, const uint8_t *d_symbols, const float *d_scales,
                           const uint64_t *d_esc_idx, const uint16_t *d_esc_bf16, uint64_t n_esc,
                           void *d_workspace, uint64_t workspace_bytes, void *d_out, uint64_t cap,
                           uint64_t *d_out_len, uint32_t *d_status, void *stream);

/*
 * eq_encode_device_static -- eq_encode_device without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). The
 * encoder's scratch is a static device array of
 * EQ_ENCODE_STATIC_SCRATCH_BYTES that every GPU the library runs on holds
 * until the process ends; the call allocates and frees nothing. Tensors whose
 * eq_encode_device_workspace() exceeds that size (e.g. 28672 x 8192) get
 * EQ_ERANGE; 8192 x 8192 and smaller fit.
 * Arguments, output and errors as eq_encode_device; the stream must belong
 * to the current device. Every call on one GPU shares that GPU's array and
 * finds the previous call's contents in it (the kernels clear what they
 * need): calls that overlap in time on one GPU (several streams or host
 * threads) race and must be serialised by the caller.
 */
#define EQ_ENCODE_STATIC_SCRATCH_BYTES (136ull << 20)
eq_status eq_encode_device_static(const eq_tensor_desc *d, const uint8_t *d_symbols, const float *d_scales,
                                  const uint64_t *d_esc_idx, const uint16_t *d_esc_bf16, uint64_t n_esc,
                                  void *d_out, uint64_t cap, uint64_t *d_out_len, uint32_t *d_status,
                                  void *stream);

/*
 * eq_gemv_bf16 -- y[r] = sum_c W[r, c] * x[c] for a row-major bf16 [rows,
 * cols] matrix W and bf16 vector x, fp32 accumulation, fp32 y. The batch-1
 * forward consumer of a decoded buffer (the "forward kernels" that follow
 * the decompression, technical component 3 of the EntQuant summary). Not
 * bit-reproducible against other summation orders.
 * All pointers are device pointers; cols must be a multiple of 8 and W, x
 * 16-byte aligned. Errors: EQ_EINVAL, EQ_EHIP.
 */
eq_status eq_gemv_bf16(const uint16_t *d_w, uint64_t rows, uint64_t cols, const uint16_t *d_x,
                       float *d_y, void *stream);

/*
 * Block-by-block schedule (technical component 3 of the EntQuant summary:
 * decompression interleaved with the forward kernels, block by block, into a
 * buffer): n_blocks blocks are decoded in order into two alternating bf16
 * buffers on decode_stream while gemv_stream runs each decoded block's
 * GEMVs on the other buffer; events gate buffer reuse.
 *
 * eq_pipeline_create makes a plan holding 2 * n_blocks + 1 HIP events (no
 * device memory), in mode EQ_PIPELINE_ALTERNATE. eq_pipeline_run enqueues
 * one pass: decode_stream first waits for everything already enqueued on
 * gemv_stream (a previous run's GEMVs may still read either buffer); then
 * for block b, decode into buf[b % 2] after the GEMVs of block b - 1
 * (EQ_PIPELINE_ALTERNATE: the streams take turns, each kernel has the GPU to
 * itself) or of block b - 2 (EQ_PIPELINE_OVERLAP: the decode of block b runs
 * beside the GEMVs of block b - 1; b - 2 was the last reader of its buffer),
 * then the GEMVs of block b (tensor i: W = buf[b % 2] +
 * tensors[i].out_offset, rows/cols from its header, x = d_x[b][i],
 * y = d_y[b][i]) after that decode. Both modes give the same results. On
 * MI355X the two HBM-bound kernels slow each other down when they share the
 * GPU, so the alternating mode is the faster one there. The last
 * GEMVs are on gemv_stream: the y of a run are complete once gemv_stream
 * reaches the end of that run (an event recorded there, or a synchronise);
 * runs may be enqueued back to back without a synchronise.
 * d_x / d_y: host arrays of n_blocks pointers to host arrays of device
 * pointers (one per tensor). Errors: EQ_EINVAL, EQ_EHIP.
 */
typedef struct eq_pipeline eq_pipeline;
#define EQ_PIPELINE_ALTERNATE 0u
#define EQ_PIPELINE_OVERLAP 1u
eq_status eq_pipeline_create(uint32_t n_blocks, eq_pipeline **out);
/* Selects the gating of later runs (EQ_PIPELINE_ALTERNATE or
 * EQ_PIPELINE_OVERLAP). Errors: EQ_EINVAL (null plan, unknown mode). */
eq_status eq_pipeline_set_mode(eq_pipeline *p, uint32_t mode);
eq_status eq_pipeline_run(eq_pipeline *p, const eq_block *blocks, uint32_t n_blocks,
                          uint16_t *d_buf0, uint16_t *d_buf1, const uint16_t *const *const *d_x,
                          float *const *const *d_y, void *decode_stream, void *gemv_stream);
eq_status eq_pipeline_destroy(eq_pipeline *p);

/*
 * eq_bf16_from_f32 -- diagnostic: the decode kernel's own fp32 -> bf16
 * rounding applied to n values (device pointers), so that the rounding can be
 * checked over all 2^32 inputs. Errors: EQ_EINVAL, EQ_EHIP.
 */
eq_status eq_bf16_from_f32(const float *d_in, uint64_t n, uint16_t *d_out, void *stream);

/* Static text for a status code. */
const char *eq_status_string(eq_status s);

#ifdef __cplusplus
}
#endif

#endif /* EQ_H */
