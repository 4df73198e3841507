/*
 * Drives every entry point of the oracle (oracle/zc_oracle.c) for a build
 * under AddressSanitizer and UndefinedBehaviorSanitizer on the CPU: the code
 * table functions, compress and strict decompress of ragged chunks (empty,
 * one value, partial tiles), all 65 536 bf16 patterns, incompressible data,
 * truncated and mutated streams (each decoded with exactly its own length
 * readable, in a heap block of that size, so any read past it is caught), the
 * slot-layout calls, and the reduce-step sums.
 *
 * Test infrastructure: built and run by tests/test_oracle_sanitized.py.
 * Exits 0 and prints "sanitized oracle run ok" when every check passed.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zc_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void)   /* splitmix64 */
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

#define CHECK(cond)                                                         \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            exit(1);                                                        \
        }                                                                   \
    } while (0)

/* bf16 values near a Gaussian (exponents spread around 120) with a few
 * arbitrary patterns, so escapes and raw groups occur */
static void fill(uint16_t *w, int64_t n, int wild_per_mille)
{
    for (int64_t i = 0; i < n; ++i) {
        uint64_t r = next_u64();
        if ((int)(r % 1000) < wild_per_mille) {
            w[i] = (uint16_t)(r >> 16);
        } else {
            unsigned e = 116 + (unsigned)((r >> 10) % 7);
            w[i] = (uint16_t)(((r >> 20) & 1) << 15 | e << 7 | ((r >> 24) & 0x7F));
        }
    }
}

/* Compresses w[0..n) and decodes it with exactly comp_bytes readable. */
static void roundtrip(const uint16_t *w, int64_t n)
{
    int64_t cap = zco_chunk_bound(n);
    uint8_t *buf = (uint8_t *)malloc((size_t)cap);
    CHECK(buf);
    int64_t comp = zco_compress_chunk(w, n, buf, cap, NULL);
    CHECK(comp >= 32 && comp <= cap);
    uint8_t *exact = (uint8_t *)malloc((size_t)comp);
    CHECK(exact);
    memcpy(exact, buf, (size_t)comp);
    uint16_t *back = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * 2);
    CHECK(back);
    CHECK(zco_decompress_chunk(exact, comp, n, back) == 0);
    CHECK(n == 0 || memcmp(back, w, (size_t)n * 2) == 0);
    /* truncated: every strict prefix is rejected, reading only that prefix */
    for (int64_t cut = 0; cut < comp; cut += 1 + comp / 7) {
        uint8_t *pre = (uint8_t *)malloc((size_t)(cut > 0 ? cut : 1));
        CHECK(pre);
        memcpy(pre, exact, (size_t)cut);
        CHECK(zco_decompress_chunk(pre, cut, n, back) != 0);
        free(pre);
    }
    /* mutated: any verdict is allowed, but no access may leave the stream */
    for (int i = 0; i < 40; ++i) {
        uint8_t *m = (uint8_t *)malloc((size_t)comp);
        CHECK(m);
        memcpy(m, exact, (size_t)comp);
        uint64_t r = next_u64();
        m[r % (uint64_t)comp] ^= (uint8_t)(1u << ((r >> 32) % 8));
        if (i % 3 == 0)
            m[(r >> 40) % (uint64_t)comp] = (uint8_t)(r >> 8);
        (void)zco_decompress_chunk(m, comp, n, back);
        free(m);
    }
    free(back);
    free(exact);
    free(buf);
}

int main(void)
{
    /* code table, law, Huffman, canonical codes */
    double p[17], q[17], w8[8] = {0.5, 0.2, 0.1, 0.1, 0.05, 0.03, 0.01, 0.01};
    int len[17], l8[8];
    uint32_t code[17], c8[8];
    zco_law_fixed_sigma(128, 16, 0.02, p);
    zco_law_phase_avg(128, 16, 64, q);
    zco_law_phase_avg(2, 16, 8, q);
    CHECK(zco_huffman_lengths(w8, 8, l8) == 0);
    zco_canonical_codes(l8, 8, c8);
    CHECK(zco_build_table(1, p, len, code) == 0);
    CHECK(zco_build_table(2, p, len, code) != 0);

    /* ragged sizes, with and without wild patterns */
    static const int64_t sizes[] = {0, 1, 2, 7, 8, 9, 127, 128, 129, 511, 512, 513,
                                    8191, 8192, 8193, 16384 + 17, 3 * 8192 + 4000};
    for (size_t s = 0; s < sizeof sizes / sizeof sizes[0]; ++s) {
        int64_t n = sizes[s];
        uint16_t *w = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * 2);
        CHECK(w);
        fill(w, n, 0);
        roundtrip(w, n);
        fill(w, n, 20);
        roundtrip(w, n);
        fill(w, n, 1000);              /* uniform patterns: raw groups */
        roundtrip(w, n);
        free(w);
    }

    /* all 65 536 patterns in order */
    uint16_t *all = (uint16_t *)malloc(65536 * 2);
    CHECK(all);
    for (int i = 0; i < 65536; ++i)
        all[i] = (uint16_t)i;
    roundtrip(all, 65536);
    free(all);

    /* slot layout of several chunks, decoded in place and at packed offsets */
    int64_t counts[5] = {5, 0, 8192, 9000, 1};
    int64_t total = 0;
    for (int c = 0; c < 5; ++c)
        total += counts[c];
    uint16_t *x = (uint16_t *)malloc((size_t)total * 2);
    CHECK(x);
    fill(x, total, 30);
    int64_t off[5];
    int64_t slots = zco_slot_offsets(counts, 5, off);
    uint8_t *buf = (uint8_t *)malloc((size_t)slots);
    CHECK(buf);
    int64_t comp[5];
    CHECK(zco_compress(x, counts, 5, buf, slots, comp, NULL) == 0);
    uint16_t *y = (uint16_t *)malloc((size_t)total * 2);
    CHECK(y);
    int bad = -1;
    CHECK(zco_decompress(buf, slots, NULL, counts, 5, y, &bad) == 0);
    CHECK(memcmp(x, y, (size_t)total * 2) == 0);
    int64_t poff[5], pos = 0;
    for (int c = 0; c < 5; ++c) {
        poff[c] = pos;
        pos += (comp[c] + 15) / 16 * 16;
    }
    uint8_t *packed = (uint8_t *)calloc((size_t)pos, 1);
    CHECK(packed);
    for (int c = 0; c < 5; ++c)
        memcpy(packed + poff[c], buf + off[c], (size_t)comp[c]);
    CHECK(zco_decompress(packed, pos, poff, counts, 5, y, &bad) == 0);
    CHECK(memcmp(x, y, (size_t)total * 2) == 0);
    free(packed);
    free(y);
    free(buf);
    free(x);

    /* reduce step: 5 contributions of 1000 values, fp32 and bf16 delivery */
    uint16_t *contrib = (uint16_t *)malloc(5000 * 2);
    float *f = (float *)malloc(1000 * sizeof(float));
    uint16_t *h = (uint16_t *)malloc(1000 * 2);
    CHECK(contrib && f && h);
    fill(contrib, 5000, 50);
    zco_reduce_bf16_f32(contrib, 1000, 5, f);
    zco_reduce_bf16_bf16(contrib, 1000, 5, h);
    for (int i = 0; i < 65536; ++i) {
        uint32_t u = (uint32_t)i << 16 | (uint32_t)(next_u64() & 0xFFFF);
        float v;
        memcpy(&v, &u, 4);
        (void)zco_f32_to_bf16(v);
    }
    free(h);
    free(f);
    free(contrib);

    puts("sanitized oracle run ok");
    return 0;
}
