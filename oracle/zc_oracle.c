/*
 * zc_oracle.c -- the ORACLE for the lossless bf16 exponent codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load,
 * call or execute this file: only tests/, the smoke check and the CPU
 * baseline leg of bench.py use it.  It is plain, slow, single-threaded C99
 * written for readability, and it shares no code, header, table or constant
 * generator with the GPU library.  It builds its own code table from the
 * closed-form Gaussian exponent law with libm's erf.
 *
 * What it computes (the method's steps, in order):
 *   ZipCCL (arXiv 2604.27844), abstract, technique (1): the exponent of each
 *   value is coded with a code derived in closed form from the Gaussian law
 *   of training tensors, so no histogram is taken at run time.  The Chinese
 *   summary page ("key design" paragraph) says frequent exponents get short
 *   codes and rare ones long codes.  The Figure 6 caption gives the target of
 *   the split: a 16-bit value shrinks to about 11 bits, i.e. only the 8
 *   exponent bits are coded and the sign+mantissa byte is kept as is.
 *   Every byte-level choice the pages leave open (group shape, escape,
 *   raw fallback, container) is the frozen "ZCB1" format, written out in the
 *   functions below; each reading is listed in the design notes.
 *
 * Parity status: every function here is pinned by tests that do not reuse
 * this code (Monte-Carlo law, package-merge optimality, hand-derived golden
 * streams, brute-force enumeration of all 65 536 bf16 patterns, invariants).
 */
#include "zc_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Constants of the ZCB1 format (table_id 1)                                */
/* ------------------------------------------------------------------------ */
enum {
    O_LANES = 64,               /* groups per tile                           */
    O_VALS_PER_STEP = 8,        /* consecutive values a group takes per step */
    O_STEPS = 16,               /* steps per tile                            */
    O_G = O_VALS_PER_STEP * O_STEPS,   /* 128 members per group             */
    O_TILE = O_LANES * O_G,            /* 8192 values per tile              */
    O_K = 16,                   /* d >= 16 is escaped                        */
    O_NSYM = O_K + 1,           /* symbols d = 0..15 and ESC (= 16)          */
    O_ESC = O_K,
    O_Q = 64,                   /* scale phases averaged in the law          */
    O_HDR = 32
};
#define O_MAGIC 0x3142435Au     /* bytes 'Z' 'C' 'B' '1' */

/* ------------------------------------------------------------------------ */
/* a0: the closed-form exponent law                                         */
/* ------------------------------------------------------------------------ */

/* Probability that |X| < x for X ~ N(0, sigma^2). */
static double gauss_abs_cdf(double x, double sigma)
{
    return erf(x / (sigma * sqrt(2.0)));
}

/*
 * Law of d = E_max - e for one member of a group of G i.i.d. N(0, sigma^2)
 * values, where e is the binary exponent (binade index) of a value and E_max
 * the largest exponent in the group.  With F(x) = P(|X| < x) and
 * p_k = F(2^(k+1)) - F(2^k) (probability of binade k):
 *   P(d = 0)  = sum_m p_m * F(2^(m+1))^(G-1)
 *   P(d = j)  = sum_m p_(m-j) * [F(2^(m+1))^(G-1) - F(2^m)^(G-1)],  j >= 1
 *   P(d >= K) = sum_m F(2^(m-K+1)) * [F(2^(m+1))^(G-1) - F(2^m)^(G-1)]
 * (the member sits j binades below the binade m that holds the maximum of
 * the other G-1 values; for j = 0 the others only have to stay below 2^(m+1)).
 * out[0..K-1] = P(d = j), out[K] = P(d >= K).
 */
void zco_law_fixed_sigma(int G, int K, double sigma, double *out)
{
    const int MLO = -80, MHI = 40;       /* binades that carry the maxima */
    int j, m;
    for (j = 0; j <= K; ++j)
        out[j] = 0.0;
    for (m = MLO; m <= MHI; ++m) {
        double Fm = gauss_abs_cdf(ldexp(1.0, m), sigma);
        double Fm1 = gauss_abs_cdf(ldexp(1.0, m + 1), sigma);
        double below = pow(Fm, (double)(G - 1));
        double upto = pow(Fm1, (double)(G - 1));
        double in_binade = upto - below;   /* others' max lies in binade m */
        /* j = 0: the member is in binade m, the others are all below 2^(m+1) */
        out[0] += (Fm1 - Fm) * upto;
        for (j = 1; j < K; ++j) {
            double pk = gauss_abs_cdf(ldexp(1.0, m - j + 1), sigma)
                      - gauss_abs_cdf(ldexp(1.0, m - j), sigma);
            out[j] += pk * in_binade;
        }
        out[K] += gauss_abs_cdf(ldexp(1.0, m - K + 1), sigma) * in_binade;
    }
}

/*
 * Scale-free law: the fixed-sigma law depends only on where sigma sits inside
 * its octave, so it is averaged over Q phases sigma = 2^((q + 1/2)/Q).
 */
void zco_law_phase_avg(int G, int K, int Q, double *out)
{
    double tmp[64];
    int q, j;
    for (j = 0; j <= K; ++j)
        out[j] = 0.0;
    for (q = 0; q < Q; ++q) {
        zco_law_fixed_sigma(G, K, pow(2.0, (q + 0.5) / Q), tmp);
        for (j = 0; j <= K; ++j)
            out[j] += tmp[j] / Q;
    }
}

/*
 * Huffman code lengths for nsym weights.  Each round merges the two lightest
 * live nodes; equal weights go to the node created first (leaves are created
 * first, in symbol order; merged nodes after, in merge order).
 */
int zco_huffman_lengths(const double *w, int nsym, int *len)
{
    double weight[2 * 64];
    int parent[2 * 64];
    int alive[2 * 64];
    int nodes = nsym, live = nsym, i;
    if (nsym < 2 || nsym > 64)
        return -1;
    for (i = 0; i < nsym; ++i) {
        weight[i] = w[i];
        alive[i] = 1;
        parent[i] = -1;
    }
    while (live > 1) {
        int a = -1, b = -1;
        for (i = 0; i < nodes; ++i) {
            if (!alive[i])
                continue;
            if (a < 0 || weight[i] < weight[a]) {
                b = a;
                a = i;
            } else if (b < 0 || weight[i] < weight[b]) {
                b = i;
            }
        }
        weight[nodes] = weight[a] + weight[b];
        alive[nodes] = 1;
        parent[nodes] = -1;
        alive[a] = alive[b] = 0;
        parent[a] = parent[b] = nodes;
        ++nodes;
        --live;
    }
    for (i = 0; i < nsym; ++i) {
        int d = 0, x = i;
        while (parent[x] >= 0) {
            x = parent[x];
            ++d;
        }
        len[i] = d;
    }
    return 0;
}

/*
 * Canonical code: symbols sorted by (length, symbol) get consecutive code
 * values, the value being shifted left whenever the length grows.
 */
void zco_canonical_codes(const int *len, int nsym, uint32_t *code)
{
    uint32_t next = 0;
    int prev_len = 0, L, s, first = 1;
    for (L = 1; L <= 32; ++L) {
        for (s = 0; s < nsym; ++s) {
            if (len[s] != L)
                continue;
            if (first) {
                next = 0;
                first = 0;
            } else {
                next = (next + 1) << (L - prev_len);
            }
            code[s] = next;
            prev_len = L;
        }
    }
}

/* The table of table_id 1: G = 128, K = 16, Q = 64. */
int zco_build_table(int table_id, double *prob, int *len, uint32_t *code)
{
    double p[O_NSYM];
    if (table_id != 1)
        return -1;
    zco_law_phase_avg(O_G, O_K, O_Q, p);
    if (prob)
        memcpy(prob, p, sizeof p);
    if (zco_huffman_lengths(p, O_NSYM, len) != 0)
        return -1;
    zco_canonical_codes(len, O_NSYM, code);
    return 0;
}

typedef struct {
    int len[O_NSYM];
    uint32_t code[O_NSYM];
} otable;

static int get_table(otable *tb)
{
    return zco_build_table(1, NULL, tb->len, tb->code);
}

/* ------------------------------------------------------------------------ */
/* Chunk geometry                                                           */
/* ------------------------------------------------------------------------ */

static int64_t align_up(int64_t x, int64_t a)
{
    return (x + a - 1) / a * a;
}

/* T tiles, NG groups, raw section at R, exponent section at X. */
void zco_geometry(int64_t n, int64_t *T, int64_t *NG, int64_t *R, int64_t *X)
{
    int64_t t = (n + O_TILE - 1) / O_TILE;
    int64_t r = align_up(O_HDR + 196 * t, 16);
    *T = t;
    *NG = (int64_t)O_LANES * t;
    *R = r;
    *X = align_up(r + n, 16);
}

/* Worst case: every tile raw, i.e. n exponent bytes plus word padding. */
int64_t zco_chunk_bound(int64_t n)
{
    int64_t T, NG, R, X;
    zco_geometry(n, &T, &NG, &R, &X);
    return X + n + 4 * T;
}

int64_t zco_slot_offsets(const int64_t *counts, int num_chunks, int64_t *off)
{
    int64_t acc = 0;
    int c;
    for (c = 0; c < num_chunks; ++c) {
        if (off)
            off[c] = acc;
        acc += align_up(zco_chunk_bound(counts[c]), 256);
    }
    return acc;
}

/* Index inside the chunk of member m (0..127, stream order) of group g. */
static int64_t member_index(int64_t g, int m)
{
    int64_t t = g / O_LANES;
    int lane = (int)(g % O_LANES);
    int k = m / O_VALS_PER_STEP, j = m % O_VALS_PER_STEP;
    return t * O_TILE + (int64_t)k * (O_LANES * O_VALS_PER_STEP)
         + (int64_t)lane * O_VALS_PER_STEP + j;
}

/* ------------------------------------------------------------------------ */
/* Little-endian field access and MSB-first bit I/O                         */
/* ------------------------------------------------------------------------ */

static void put_le(uint8_t *p, uint64_t v, int bytes)
{
    int i;
    for (i = 0; i < bytes; ++i)
        p[i] = (uint8_t)(v >> (8 * i));
}

static uint64_t get_le(const uint8_t *p, int bytes)
{
    uint64_t v = 0;
    int i;
    for (i = 0; i < bytes; ++i)
        v |= (uint64_t)p[i] << (8 * i);
    return v;
}

/*
 * The exponent section is a sequence of 32-bit little-endian words; stream
 * bit p lives in word p/32 at bit position 31 - p%32 (most significant first).
 */
static void put_bit(uint8_t *sec, int64_t p, int bit)
{
    if (bit) {
        int64_t word = p / 32;
        int pos = 31 - (int)(p % 32);
        sec[4 * word + pos / 8] |= (uint8_t)(1u << (pos % 8));
    }
}

static int get_bit(const uint8_t *sec, int64_t p)
{
    int64_t word = p / 32;
    int pos = 31 - (int)(p % 32);
    return (sec[4 * word + pos / 8] >> (pos % 8)) & 1;
}

static void put_bits(uint8_t *sec, int64_t *p, uint32_t v, int nbits)
{
    int i;
    for (i = nbits - 1; i >= 0; --i)
        put_bit(sec, (*p)++, (int)((v >> i) & 1u));
}

/* ------------------------------------------------------------------------ */
/* Split and join of a bf16 bit pattern                                     */
/* ------------------------------------------------------------------------ */

static uint8_t raw_byte(uint16_t w)    /* sign bit, then 7 mantissa bits */
{
    return (uint8_t)(((w >> 8) & 0x80) | (w & 0x7F));
}

static int exponent_of(uint16_t w)     /* the 8-bit biased exponent field */
{
    return (w >> 7) & 0xFF;
}

static uint16_t join(uint8_t raw, int e)
{
    return (uint16_t)(((raw & 0x80) << 8) | (e << 7) | (raw & 0x7F));
}

/* ------------------------------------------------------------------------ */
/* Encoder                                                                  */
/* ------------------------------------------------------------------------ */

static int coded_bits(const otable *tb, int d)
{
    return d < O_K ? tb->len[d] : tb->len[O_ESC] + 8;
}

int64_t zco_compress_chunk(const uint16_t *in, int64_t n, uint8_t *out,
                           int64_t cap, zco_stats *st)
{
    otable tb;
    int64_t T, NG, R, X, bound, t, g, sec_bits;
    uint8_t *sec;

    if (n < 0 || (n > 0 && !in) || !out)
        return ZCO_EINVAL;
    bound = zco_chunk_bound(n);
    if (cap < bound)
        return ZCO_ENOSPC;
    if (get_table(&tb) != 0)
        return ZCO_EINVAL;
    zco_geometry(n, &T, &NG, &R, &X);
    memset(out, 0, (size_t)bound);          /* every gap and pad is zero */

    /* 1. raw section: one sign+mantissa byte per value, in value order */
    for (t = 0; t < n; ++t)
        out[R + t] = raw_byte(in[t]);

    /* 2. groups: max exponent, bit count, coded or raw stream */
    sec = out + X;
    sec_bits = 0;
    for (t = 0; t < T; ++t) {
        int64_t tile_start_bits = sec_bits;
        put_le(out + O_HDR + 4 * t, (uint64_t)(tile_start_bits / 8), 4);
        for (g = t * O_LANES; g < (t + 1) * O_LANES; ++g) {
            int e[O_G];
            int ng = 0, m, emax = 0;
            int64_t bits = 0;
            for (m = 0; m < O_G; ++m) {
                int64_t i = member_index(g, m);
                if (i < n)
                    e[ng++] = exponent_of(in[i]);
            }
            for (m = 0; m < ng; ++m)
                if (e[m] > emax)
                    emax = e[m];
            for (m = 0; m < ng; ++m)
                bits += coded_bits(&tb, emax - e[m]);
            if (ng > 0 && bits >= 8 * (int64_t)ng) {
                /* raw mode: every exponent as 8 plain bits */
                for (m = 0; m < ng; ++m)
                    put_bits(sec, &sec_bits, (uint32_t)e[m], 8);
                bits = 8 * (int64_t)ng;
                if (st)
                    st->raw_groups++;
            } else {
                for (m = 0; m < ng; ++m) {
                    int d = emax - e[m];
                    if (d < O_K) {
                        put_bits(sec, &sec_bits, tb.code[d], tb.len[d]);
                    } else {
                        put_bits(sec, &sec_bits, tb.code[O_ESC], tb.len[O_ESC]);
                        put_bits(sec, &sec_bits, (uint32_t)e[m], 8);
                        if (st)
                            st->escapes++;
                    }
                }
            }
            out[O_HDR + 4 * T + g] = (uint8_t)emax;
            put_le(out + O_HDR + 68 * T + 2 * g, (uint64_t)bits, 2);
        }
        /* zero bits up to the next 32-bit word */
        sec_bits = align_up(sec_bits, 32);
        (void)tile_start_bits;
    }

    /* 3. header */
    put_le(out + 0, O_MAGIC, 4);
    put_le(out + 4, 1, 2);                 /* version  */
    put_le(out + 6, 1, 2);                 /* table_id */
    put_le(out + 8, 0, 4);                 /* flags    */
    put_le(out + 12, 0, 4);                /* reserved */
    put_le(out + 16, (uint64_t)n, 8);
    put_le(out + 24, (uint64_t)(X + sec_bits / 8), 8);
    return X + sec_bits / 8;
}

/* ------------------------------------------------------------------------ */
/* Strict decoder: accepts exactly the streams the encoder can produce      */
/* ------------------------------------------------------------------------ */

/* Reads one code word bit by bit; returns the symbol or -1. */
static int read_symbol(const otable *tb, const uint8_t *sec, int64_t *p,
                       int64_t end)
{
    uint32_t acc = 0;
    int L, s;
    for (L = 1; L <= 32; ++L) {
        if (*p >= end)
            return -1;
        acc = (acc << 1) | (uint32_t)get_bit(sec, (*p)++);
        for (s = 0; s < O_NSYM; ++s)
            if (tb->len[s] == L && tb->code[s] == acc)
                return s;
    }
    return -1;
}

static uint32_t read_bits(const uint8_t *sec, int64_t *p, int nbits)
{
    uint32_t v = 0;
    int i;
    for (i = 0; i < nbits; ++i)
        v = (v << 1) | (uint32_t)get_bit(sec, (*p)++);
    return v;
}

int zco_decompress_chunk(const uint8_t *in, int64_t avail, int64_t n,
                         uint16_t *out)
{
    otable tb;
    int64_t T, NG, R, X, comp, t, g, i, sec_bits, sec_len;
    const uint8_t *sec;

    if (!in || n < 0 || (n > 0 && !out))
        return ZCO_EINVAL;
    if (get_table(&tb) != 0)
        return ZCO_EINVAL;
    if (avail < O_HDR)
        return ZCO_E_SIZE;
    if (get_le(in + 0, 4) != O_MAGIC || get_le(in + 4, 2) != 1
        || get_le(in + 6, 2) != 1 || get_le(in + 8, 4) != 0
        || get_le(in + 12, 4) != 0)
        return ZCO_E_HEADER;
    if ((int64_t)get_le(in + 16, 8) != n)
        return ZCO_E_HEADER;
    zco_geometry(n, &T, &NG, &R, &X);
    comp = (int64_t)get_le(in + 24, 8);
    if (comp < X || comp > avail || comp > zco_chunk_bound(n))
        return ZCO_E_SIZE;
    for (i = O_HDR + 196 * T; i < R; ++i)
        if (in[i])
            return ZCO_E_GAP;
    for (i = R + n; i < X; ++i)
        if (in[i])
            return ZCO_E_GAP;

    sec = in + X;
    sec_len = comp - X;
    sec_bits = 0;
    for (t = 0; t < T; ++t) {
        if ((int64_t)get_le(in + O_HDR + 4 * t, 4) * 8 != sec_bits)
            return ZCO_E_TILE;
        for (g = t * O_LANES; g < (t + 1) * O_LANES; ++g) {
            int e[O_G];
            int ng = 0, m, emax, dmax_seen = -1;
            int64_t glen, p0, coded = 0;
            for (m = 0; m < O_G; ++m)
                if (member_index(g, m) < n)
                    ++ng;
            emax = in[O_HDR + 4 * T + g];
            glen = (int64_t)get_le(in + O_HDR + 68 * T + 2 * g, 2);
            if (glen > 8 * (int64_t)ng || (ng == 0 && emax != 0))
                return ZCO_E_GROUP;
            if (sec_bits + glen > 8 * sec_len)
                return ZCO_E_SIZE;
            p0 = sec_bits;
            if (ng > 0 && glen == 8 * (int64_t)ng) {
                int mx = 0;
                for (m = 0; m < ng; ++m) {
                    e[m] = (int)read_bits(sec, &sec_bits, 8);
                    if (e[m] > mx)
                        mx = e[m];
                }
                if (mx != emax)
                    return ZCO_E_EMAX;
                for (m = 0; m < ng; ++m)
                    coded += coded_bits(&tb, emax - e[m]);
                if (coded < 8 * (int64_t)ng)
                    return ZCO_E_RAWMODE;   /* should have been coded */
            } else {
                for (m = 0; m < ng; ++m) {
                    int s = read_symbol(&tb, sec, &sec_bits, p0 + glen);
                    if (s < 0)
                        return ZCO_E_SYMBOL;
                    if (s == O_ESC) {
                        if (sec_bits + 8 > p0 + glen)
                            return ZCO_E_SYMBOL;
                        e[m] = (int)read_bits(sec, &sec_bits, 8);
                        if (emax - e[m] < O_K)
                            return ZCO_E_ESCAPE;   /* e above emax or short d */
                    } else {
                        if (s > emax)
                            return ZCO_E_SYMBOL;   /* exponent would be < 0 */
                        e[m] = emax - s;
                    }
                    if (e[m] == emax)
                        dmax_seen = 0;
                }
                if (sec_bits != p0 + glen)
                    return ZCO_E_LENGTH;
                if (ng > 0 && dmax_seen != 0)
                    return ZCO_E_EMAX;
            }
            for (m = 0; m < ng; ++m) {
                i = member_index(g, m);
                out[i] = join(in[R + i], e[m]);
            }
        }
        while (sec_bits % 32) {
            if (sec_bits >= 8 * sec_len)
                return ZCO_E_SIZE;
            if (get_bit(sec, sec_bits++))
                return ZCO_E_PADDING;
        }
    }
    if (X + sec_bits / 8 != comp)
        return ZCO_E_SIZE;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Whole buffers: chunks back to back in, one 256-byte aligned slot each    */
/* ------------------------------------------------------------------------ */

int zco_compress(const uint16_t *in, const int64_t *counts, int num_chunks,
                 uint8_t *out, int64_t cap, int64_t *comp_sizes,
                 zco_stats *st)
{
    int64_t voff = 0;
    int c;
    if (num_chunks < 0 || !counts)
        return ZCO_EINVAL;
    for (c = 0; c < num_chunks; ++c)
        if (counts[c] < 0)
            return ZCO_EINVAL;
    if (cap < zco_slot_offsets(counts, num_chunks, NULL))
        return ZCO_ENOSPC;
    for (c = 0; c < num_chunks; ++c) {
        int64_t slot = zco_slot_offsets(counts, c, NULL);
        int64_t r = zco_compress_chunk(in + voff, counts[c], out + slot,
                                       zco_chunk_bound(counts[c]), st);
        if (r < 0)
            return (int)r;
        if (comp_sizes)
            comp_sizes[c] = r;
        voff += counts[c];
    }
    return 0;
}

int zco_decompress(const uint8_t *in, int64_t in_bytes, const int64_t *offsets,
                   const int64_t *counts, int num_chunks, uint16_t *out,
                   int *bad_chunk)
{
    int64_t voff = 0;
    int c;
    if (num_chunks < 0 || !counts)
        return ZCO_EINVAL;
    for (c = 0; c < num_chunks; ++c) {
        int64_t off = offsets ? offsets[c] : zco_slot_offsets(counts, c, NULL);
        int r;
        if (counts[c] < 0 || off < 0 || off > in_bytes)
            return ZCO_EINVAL;
        r = zco_decompress_chunk(in + off, in_bytes - off, counts[c],
                                 out + voff);
        if (r != 0) {
            if (bad_chunk)
                *bad_chunk = c;
            return r;
        }
        voff += counts[c];
    }
    return 0;
}

/* ---------------------------------------------------------------- reduce */

/* A bf16 bit pattern is the top half of the fp32 with the same value. */
static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

void zco_reduce_bf16_f32(const uint16_t *x, int64_t n, int num_chunks,
                         float *out)
{
    int64_t i;
    int c;
    for (i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (c = 0; c < num_chunks; ++c)
            acc = acc + bf16_to_f32(x[(int64_t)c * n + i]);
        out[i] = acc;
    }
}

/* fp32 to bf16 with round to nearest, ties to even, at bf16's precision and
 * range.  The two bf16 values that bracket x (the one toward zero and the next
 * one out, 2^128 standing for the step past the largest finite value) are
 * compared by distance in double precision, where the differences are exact;
 * a tie takes the one with an even last significand bit.  A NaN becomes the
 * quiet NaN 0x7FC0; infinities and zeros keep their sign. */
uint16_t zco_f32_to_bf16(float x)
{
    uint32_t u;
    uint16_t lo, hi;
    double ax, dlo, dhi;
    memcpy(&u, &x, sizeof u);
    if (isnan(x))
        return 0x7FC0;
    lo = (uint16_t)(u >> 16);
    if ((u & 0xFFFFu) == 0 || isinf(x))
        return lo;
    hi = (uint16_t)(lo + 1);
    ax = fabs((double)x);
    dlo = fabs((double)bf16_to_f32(lo));
    dhi = ((hi & 0x7FFF) == 0x7F80) ? ldexp(1.0, 128) : fabs((double)bf16_to_f32(hi));
    if (ax - dlo < dhi - ax)
        return lo;
    if (dhi - ax < ax - dlo)
        return hi;
    return (lo & 1) ? hi : lo;
}

void zco_reduce_bf16_bf16(const uint16_t *x, int64_t n, int num_chunks,
                          uint16_t *out)
{
    int64_t i;
    int c;
    for (i = 0; i < n; ++i) {
        float acc = 0.0f;
        for (c = 0; c < num_chunks; ++c)
            acc = acc + bf16_to_f32(x[(int64_t)c * n + i]);
        out[i] = zco_f32_to_bf16(acc);
    }
}
