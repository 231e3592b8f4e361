// format.hpp -- container v1 layout shared by the library's host codec and
// its device launcher (the layout itself is specified in include/eq.h).
#pragma once
#include <cstdint>

namespace eqfmt {

constexpr uint32_t kMagic = 0x31525145u;  // "EQR1" read as little-endian u32
constexpr uint16_t kVersion = 1;
constexpr uint32_t kLanes = 64;
constexpr uint32_t kProbBits = 12;
constexpr uint32_t kProbScale = 1u << kProbBits;  // 4096
constexpr uint32_t kStateLow = 1u << 16;          // L
constexpr uint64_t kHeaderBytes = 256;
constexpr uint64_t kSectionAlign = 256;
constexpr uint32_t kWordPad = 8;                  // words per chunk padded to a multiple of 8
constexpr uint32_t kMaxChunk = 1u << 24;
constexpr uint64_t kDirEntryBytes = 16;
constexpr uint32_t kCodecRans = 0;
constexpr uint32_t kCodecHuffman = 1;
constexpr uint32_t kHuffMaxLen = 12;        // longest codeword
constexpr uint16_t kHuffZero = 0x100;       // length-table value of a lone zero-bit symbol

// Header byte offsets.
enum HeaderField : uint32_t {
    H_MAGIC = 0, H_VERSION = 4, H_DTYPE = 6, H_FLAGS = 7, H_ROWS = 8, H_COLS = 16, H_N = 24,
    H_CHUNK = 32, H_LANE_RUN = 36, H_LANES = 40, H_PROB_BITS = 44, H_NCHUNKS = 48, H_NESC = 56,
    H_ESC_CODE = 64, H_NWORDS = 72, H_OFF_FREQ = 80, H_OFF_SCALES = 88, H_OFF_DIR = 96,
    H_OFF_STATES = 104, H_OFF_WORDS = 112, H_OFF_ESC_IDX = 120, H_OFF_ESC_VAL = 128, H_TOTAL = 136,
    H_CODEC = 144, H_SEG = 148,
};
constexpr uint8_t kFlagEsc = 1, kFlagSeg = 2;

constexpr uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

struct Sections {
    uint64_t freq, scales, dir, states, words, esc_idx, esc_val, total;
};

// Section offsets of a container with the given counts: each section starts
// on a 256-byte boundary right after the previous one (the Huffman codec
// stores no lane states).
inline Sections layout(uint64_t rows, uint64_t n_chunks, uint64_t n_words, uint64_t n_esc,
                       uint32_t codec = kCodecRans, uint64_t n_tables = 1) {
    Sections s{};
    uint64_t at = kHeaderBytes;
    auto place = [&](uint64_t bytes) {
        uint64_t start = round_up(at, kSectionAlign);
        at = start + bytes;
        return start;
    };
    s.freq = place(256 * 2 * n_tables);
    s.scales = place(rows * 4);
    s.dir = place(n_chunks * kDirEntryBytes);
    s.states = place(codec == kCodecRans ? n_chunks * kLanes * 4 : 0);
    s.words = place(n_words * 2);
    s.esc_idx = place(n_esc * 8);
    s.esc_val = place(n_esc * 2);
    s.total = round_up(at, kSectionAlign);
    return s;
}

// Frequency tables of a container: one, or one per segment of seg chunks.
inline uint64_t n_tables(uint64_t n_chunks, uint32_t seg) { return seg ? (n_chunks + seg - 1) / seg : 1; }

inline bool valid_lane_run(uint32_t k) { return k == 1 || k == 2 || k == 4 || k == 8 || k == 16; }

}  // namespace eqfmt
