/*
 * zc_oracle.h -- interface of the ORACLE (test infrastructure only).
 *
 * Only tests/, the smoke check and the CPU-baseline leg of bench.py may use
 * this.  The GPU library never includes it, and this header includes nothing
 * from the library.
 */
#ifndef ZC_ORACLE_H
#define ZC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes (negative).  The decoder's codes say which check failed. */
enum {
    ZCO_EINVAL = -1,
    ZCO_ENOSPC = -2,
    ZCO_E_HEADER = -10,   /* magic / version / table / flags / n           */
    ZCO_E_SIZE = -11,     /* comp_bytes or a stream runs past the data     */
    ZCO_E_GAP = -12,      /* a gap byte between sections is not zero       */
    ZCO_E_TILE = -13,     /* tile_off is not the running sum               */
    ZCO_E_GROUP = -14,    /* glen > 8 n_g, or an empty group with emax != 0 */
    ZCO_E_SYMBOL = -15,   /* no code word fits, or d > E_max               */
    ZCO_E_ESCAPE = -16,   /* escaped exponent with E_max - e < 16          */
    ZCO_E_LENGTH = -17,   /* a coded group does not use exactly glen bits  */
    ZCO_E_EMAX = -18,     /* decoded max exponent differs from E_max       */
    ZCO_E_RAWMODE = -19,  /* raw group whose coded form would be shorter   */
    ZCO_E_PADDING = -20   /* a pad bit at a tile end is not zero           */
};

typedef struct {
    int64_t raw_groups;   /* groups stored in raw mode            */
    int64_t escapes;      /* escaped exponents in coded groups    */
} zco_stats;

/* Closed-form law of d = E_max - e, out[0..K-1] = P(d=j), out[K] = P(d>=K). */
void zco_law_fixed_sigma(int G, int K, double sigma, double *out);
void zco_law_phase_avg(int G, int K, int Q, double *out);

/* Huffman lengths (deterministic tie-break) and canonical code values. */
int zco_huffman_lengths(const double *w, int nsym, int *len);
void zco_canonical_codes(const int *len, int nsym, uint32_t *code);

/* Table of table_id 1 (17 symbols: d = 0..15 then ESC). prob may be NULL. */
int zco_build_table(int table_id, double *prob, int *len, uint32_t *code);

/* Geometry of one chunk stream of n values. */
void zco_geometry(int64_t n, int64_t *T, int64_t *NG, int64_t *R, int64_t *X);
int64_t zco_chunk_bound(int64_t n);
/* Slot offsets (off may be NULL); returns the total slot bytes. */
int64_t zco_slot_offsets(const int64_t *counts, int num_chunks, int64_t *off);

/* One chunk.  Returns comp_bytes, or a negative error.  cap >= bound. */
int64_t zco_compress_chunk(const uint16_t *in, int64_t n, uint8_t *out,
                           int64_t cap, zco_stats *st);
/* One chunk; avail = readable bytes from `in`.  Returns 0 or an error. */
int zco_decompress_chunk(const uint8_t *in, int64_t avail, int64_t n,
                         uint16_t *out);

/* Whole buffers in the slot layout (offsets == NULL) or at given offsets. */
int zco_compress(const uint16_t *in, const int64_t *counts, int num_chunks,
                 uint8_t *out, int64_t cap, int64_t *comp_sizes,
                 zco_stats *st);
int zco_decompress(const uint8_t *in, int64_t in_bytes, const int64_t *offsets,
                   const int64_t *counts, int num_chunks, uint16_t *out,
                   int *bad_chunk);

/* Receive side of a reduce-scatter (pith.science, Figure 5: zipccl
 * ReduceScatter; Figure 3: ReduceScatter): num_chunks decoded contributions
 * of n bf16 values each, contribution c at x[c * n .. c * n + n), summed
 * element by element in fp32, in chunk order, from +0:
 *   out[i] = (((+0 + x_0[i]) + x_1[i]) + ...) + x_{C-1}[i]. */
void zco_reduce_bf16_f32(const uint16_t *x, int64_t n, int num_chunks,
                         float *out);

/* fp32 to bf16, round to nearest with ties to even (NaN -> 0x7FC0). */
uint16_t zco_f32_to_bf16(float x);

/* The same sum delivered in bf16: accumulated in fp32 exactly as
 * zco_reduce_bf16_f32, then rounded once, to nearest with ties to even. */
void zco_reduce_bf16_bf16(const uint16_t *x, int64_t n, int num_chunks,
                          uint16_t *out);

#ifdef __cplusplus
}
#endif
#endif
