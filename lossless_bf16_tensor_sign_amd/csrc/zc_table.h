// zc_table.h -- the library's code table (table_id 1) and its generator.
#pragma once

#include <cstdint>

namespace zc {

constexpr int kEscapeFrom = 16;          // d >= 16 is escaped
constexpr int kEscape = kEscapeFrom;     // symbol index of ESC
constexpr int kSymbols = kEscapeFrom + 1;
constexpr int kMaxCodeLen = 24;          // longest code word the kernels take
#ifndef ZC_LUT_BITS
#define ZC_LUT_BITS 11
#endif
#ifndef ZC_TAIL_BITS
#define ZC_TAIL_BITS (14 - ZC_LUT_BITS)
#endif
constexpr int kLutBits = ZC_LUT_BITS;    // decoder first-level lookup width
constexpr int kTailBits = ZC_TAIL_BITS;  // second level (codes up to 14 bits)

struct Table {
    double prob[kSymbols];
    int len[kSymbols];
    uint32_t code[kSymbols];
    uint8_t lut[1 << kLutBits];          // (symbol << 4) | length, 0 = long
    uint32_t limit[kMaxCodeLen + 1];     // canonical decode, per length
    int32_t base[kMaxCodeLen + 1];
    uint8_t sorted_sym[kSymbols];        // symbols by (length, symbol)
    // Second decoder level: every code word longer than kLutBits bits must
    // start with kLutBits ones and be at most kLutBits + kTailBits long; the
    // kTailBits bits after that prefix then select its entry.
    bool tail_ok;
    uint16_t tail[1 << kTailBits];       // (symbol << 8) | length
};

// Phase-averaged law of d = E_max - e: w[0..15] = P(d), w[16] = P(d >= 16).
void exponent_law(double* w);
// Huffman code lengths; equal weights take the earlier-created node first.
void huffman(const double* w, int nsym, int* len);
// Canonical code values for the given lengths.
void canonical(const int* len, int nsym, uint32_t* code);
// Whole table of table_id 1, with the decoder's lookup structures.
bool build_table(Table* t);

}  // namespace zc
