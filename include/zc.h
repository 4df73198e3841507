/*
 * zc.h -- C ABI of libzc: lossless bf16 exponent-coding codec for MI355X.
 *
 * The operation: ZipCCL (arXiv 2604.27844), abstract, techniques (1) and (2).
 * Each bf16 value is split into a sign+mantissa byte, stored as is, and an
 * 8-bit exponent.  The exponent is coded, relative to the largest exponent of
 * its 128-value group, with a fixed canonical prefix code whose lengths come
 * from the closed-form exponent law of a zero-mean Gaussian (no run-time
 * statistics).  An escape symbol and a per-group raw mode keep any input
 * lossless.  A 16-bit Gaussian value shrinks to about 11 bits (pith.science,
 * Figure 6 caption).
 *
 * Buffers are pre-partitioned into per-destination chunks (the pages'
 * communication-aware layout, abstract technique (2)): chunk c holds counts[c]
 * values, chunks lie back to back in the uncompressed buffer, and each chunk
 * is compressed into its own self-describing ZCB1 stream, so it can be sent
 * and decoded on its own (compress before the collective, decompress after
 * it: shd-paper.top summary, technical framework).
 *
 * ZCB1 stream of one chunk of n values (offsets from the stream start, all
 * fields little-endian; T = ceil(n / 8192) tiles, 64 groups per tile):
 *   0          header: u32 magic 0x3142435A, u16 version 1, u16 table_id 1,
 *              u32 flags 0, u32 reserved 0, u64 n, u64 comp_bytes
 *   32         u32 tile_off[T]  byte offset of each tile's exponent stream
 *   32 + 4T    u8  emax[64T]    largest exponent of each group
 *   32 + 68T   u16 glen[64T]    bits of each group's exponent stream
 *   R          u8  raw[n]       sign<<7 | mantissa,  R = align16(32 + 196T)
 *   X          exponent streams, most significant bit first inside
 *              little-endian u32 words, one zero-padded word run per tile,
 *              X = align16(R + n)
 * Group l of tile t owns the values 8192t + 512k + 8l + j (k = 0..15,
 * j = 0..7) that are < n, in that order.  Gap and pad bytes are zero.
 *
 * Slot layout: chunk c's stream starts at
 *   slot_off[c] = sum over c' < c of align256(zc_chunk_bound(counts[c'])).
 *
 * All calls are thread-safe and keep no state between calls.  The library
 * allocates no memory: the caller owns every buffer.  GPU calls are
 * asynchronous on the given stream (a hipStream_t; NULL is the null stream).
 */
#ifndef ZC_H
#define ZC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ZC_OK = 0,
    ZC_EINVAL = -1,    /* bad argument: null pointer, negative count,
                          misaligned buffer, too many values per chunk     */
    ZC_ENOSPC = -2,    /* output capacity or workspace too small          */
    ZC_ECORRUPT = -3,  /* a stream failed validation (decoder status)     */
    ZC_EHIP = -4       /* a HIP runtime call failed                       */
} zc_status_t;

/* Largest count per chunk (values). */
#define ZC_MAX_CHUNK_VALUES 2147483647LL

/* Largest num_chunks of any call: a decoder failure names its chunk in the
 * low 24 bits of the status word, so every chunk index must fit there. */
#define ZC_MAX_CHUNKS (1 << 24)

/*
 * Worst-case bytes of the ZCB1 stream of one chunk of n values (every group
 * in raw mode): X + n + 4T, with X and T as in the layout above.  A function
 * of the ZCB1 container of this file, not of the pages.  Host only; returns 0
 * for n < 0.
 */
size_t zc_chunk_bound(int64_t n);

/*
 * Bytes of a slot-layout buffer for num_chunks chunks: the sum of
 * align256(zc_chunk_bound(counts[c])) (the slot layout above).  counts is a
 * host array.  Returns 0 if an argument is invalid (a count outside
 * 0 .. ZC_MAX_CHUNK_VALUES, or num_chunks outside 0 .. ZC_MAX_CHUNKS).
 */
size_t zc_bound(const int64_t* counts, int32_t num_chunks);

/*
 * Device workspace bytes that zc_compress needs for these counts: a fixed
 * header (the last launch's tag and 64 counters of finished workgroups) and
 * one look-back status word per tile of the largest launch (a launch takes
 * up to 64 chunks).  Sizing only, no passage of the pages behind it.  Host
 * only; 0 if an argument is invalid.
 *
 * A workspace must hold zeros before the first call that uses it (a
 * one-time initialisation, e.g. at allocation); every call leaves it ready
 * for the next.  Each launch tags the status words it writes with a number
 * one above the tag stored in the header, and its last workgroup stores that
 * tag once every other workgroup has finished, so no call has to clear the
 * words of an earlier one (graph replays included).  When the tag wraps
 * (after 2^32 - 1 launches on one workspace) that launch clears every status
 * word first.
 */
size_t zc_workspace_bytes(const int64_t* counts, int32_t num_chunks);

/*
 * Compress num_chunks chunks (ZipCCL abstract, techniques (1)-(2)).
 *   d_in          device, bf16 bit patterns, chunks back to back in counts
 *                 order; 2-byte aligned (16-byte aligned chunk starts take
 *                 the vector path)
 *   counts        host, values per chunk, 0 <= counts[c] <= ZC_MAX_CHUNK_VALUES
 *   d_out         device, 16-byte aligned, out_capacity >= zc_bound(...);
 *                 chunk c's stream is written at slot_off[c]; bytes after a
 *                 stream's end inside its slot are left unwritten
 *   d_comp_sizes  device int64[num_chunks]: comp_bytes of each stream
 *   d_ws          device workspace of ws_bytes >= zc_workspace_bytes(...),
 *                 8-byte aligned (its status words are 64-bit atomics),
 *                 zero-filled before its first use (see zc_workspace_bytes)
 *   stream        hipStream_t the work is queued on
 * Returns ZC_OK once the work is queued, or an error before anything is
 * queued (ZC_EINVAL, ZC_ENOSPC) or when a launch fails (ZC_EHIP).  Calls that
 * share a workspace must be ordered on one stream.
 * Every wait inside the kernel is bounded: a tile whose look-back finds a
 * predecessor unpublished after a fixed number of polls recomputes that
 * predecessor's size from the input, which gives the same stream.  The
 * environment variable ZC_LOOKBACK_SPIN_LIMIT (a decimal poll count, read
 * once per process, at the first compress call) overrides that bound.
 */
int zc_compress(const uint16_t* d_in, const int64_t* counts,
                int32_t num_chunks, void* d_out, size_t out_capacity,
                int64_t* d_comp_sizes, void* d_ws, size_t ws_bytes,
                void* stream);

/* Size of the library-owned workspace of zc_compress_noalloc (per GPU). */
#define ZC_NOALLOC_WORKSPACE_BYTES ((size_t)4 << 20)

/*
 * zc_compress for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace: the look-back status words live in a library-owned
 * device array of ZC_NOALLOC_WORKSPACE_BYTES, one per GPU, held from the first
 * call on that GPU until the process ends.  The call itself allocates
 * nothing (no hipMalloc, no allocating library routine); the caller still
 * owns d_in, d_out and d_comp_sizes.
 *   arguments     as zc_compress, without d_ws / ws_bytes; the current device
 *                 must be the one the buffers and the stream belong to
 * Limit: zc_workspace_bytes(counts, num_chunks) <= ZC_NOALLOC_WORKSPACE_BYTES
 * (about 65 000 tiles of 8192 values per launch of up to 64 chunks, i.e.
 * about 535 M values), else ZC_ENOSPC before anything is queued.
 * Every call on one GPU shares that GPU's array and starts by clearing the
 * part it uses, so calls on one GPU must not overlap in time: calls on
 * different streams of one GPU race unless the caller orders them.
 * Returns as zc_compress; ZC_EHIP also if the array's device address cannot
 * be found.  The output is byte-identical to zc_compress's.
 */
int zc_compress_noalloc(const uint16_t* d_in, const int64_t* counts,
                        int32_t num_chunks, void* d_out, size_t out_capacity,
                        int64_t* d_comp_sizes, void* stream);

/*
 * Decompress num_chunks ZCB1 streams back to bf16: the inverse of
 * zc_compress, run after the collective has delivered the streams (ZipCCL
 * abstract, technique (2): the GPU decompression kernels; shd-paper.top
 * summary, technical framework: decompress after communication).  The codec
 * is lossless (abstract), so the output is bit-identical to the compressed
 * input.  Strict: a stream is accepted only if it is the exact output of
 * zc_compress for its values.
 *   d_in        device, in_bytes readable bytes holding the streams
 *   in_offsets  host int64[num_chunks]: byte offset of stream c in d_in, each
 *               a multiple of 16; NULL means the slot layout
 *   counts      host, expected values per chunk (must match each header)
 *   d_out       device, sum(counts) bf16 values written back to back
 *   d_status    device int32, must be 0 on entry.  After the stream has run
 *               it is 0 if every stream was valid; otherwise it holds
 *               (reason << 24) | chunk for one failed check, reason >= 1,
 *               chunk = the failing chunk's index in this call (0-based)
 *               (see zc_strerror of ZC_ECORRUPT; the reasons are listed with
 *               ZC_REASON_*).  Output values of a corrupt chunk are undefined,
 *               but nothing is written outside that chunk's part of d_out,
 *               and nothing is read outside [offset, offset + max(comp_bytes,
 *               X)) of a stream (X = the stream's fixed part, see the layout
 *               above; the header and index are read before comp_bytes is
 *               checked) nor past in_bytes.
 *   stream      hipStream_t
 * No workspace: every tile's offset is read from the stream's tile index.
 * Returns ZC_OK once queued; ZC_EINVAL / ZC_EHIP as for zc_compress.
 */
int zc_decompress(const void* d_in, size_t in_bytes,
                  const int64_t* in_offsets, const int64_t* counts,
                  int32_t num_chunks, uint16_t* d_out, int32_t* d_status,
                  void* stream);

/* Reasons reported through d_status (bits 24..30). */
#define ZC_REASON_HEADER 1    /* magic, version, table, flags or n         */
#define ZC_REASON_SIZE 2      /* comp_bytes or a stream beyond the data    */
#define ZC_REASON_GAP 3       /* nonzero gap byte                          */
#define ZC_REASON_TILE 4      /* tile_off is not the running sum           */
#define ZC_REASON_GROUP 5     /* glen > 8 n_g, or empty group with emax != 0 */
#define ZC_REASON_SYMBOL 6    /* no code word fits, or d > E_max           */
#define ZC_REASON_ESCAPE 7    /* escaped exponent within 16 of E_max       */
#define ZC_REASON_LENGTH 8    /* coded group does not use exactly glen bits */
#define ZC_REASON_EMAX 9      /* decoded maximum differs from E_max        */
#define ZC_REASON_RAWMODE 10  /* raw group whose coded form is shorter     */
#define ZC_REASON_PADDING 11  /* nonzero pad bit                           */

/*
 * Device-resident split.  In an MoE all-to-all the per-destination counts
 * come out of the router on the GPU (pith.science, Figure 2: the All-to-All;
 * Figure 8: unevenly loaded experts).  These calls take the counts (and, for
 * decoding, the stream offsets) in device memory, so no host synchronisation
 * sits between the router and the codec.  The host gives only the number of
 * chunks and the total number of values, which fix the launch sizes and the
 * capacity bounds.  A one-wave planning kernel builds, on the device, the
 * chunk table the host calls build from host counts; the codec kernels are
 * the same, so the streams are byte-identical to zc_compress's.
 */

/*
 * The largest zc_bound over every split of total_values values into
 * num_chunks chunks: 2 t + 200 (floor(t / 8192) + C) + 317 C for t values
 * and C chunks.  Host only; 0 if an argument is invalid (negative, or
 * values without chunks).
 */
size_t zc_bound_max(int64_t total_values, int32_t num_chunks);

/*
 * Device workspace bytes that zc_compress_dev and zc_decompress_dev need for
 * any split of total_values values into num_chunks chunks.  Host only; 0 if
 * an argument is invalid.
 */
size_t zc_workspace_bytes_max(int64_t total_values, int32_t num_chunks);

/*
 * zc_compress with the counts in device memory.
 *   d_counts      device int64[num_chunks], 8-byte aligned: values per chunk,
 *                 each in 0 .. ZC_MAX_CHUNK_VALUES, summing to total_values
 *   d_slot_off    device int64[num_chunks], written: the byte offset of chunk
 *                 c's stream in d_out (the slot layout of those counts)
 *   d_out         out_capacity >= zc_bound_max(total_values, num_chunks)
 *   d_ws          256-byte aligned, ws_bytes >= zc_workspace_bytes_max(...),
 *                 zero-filled before its first use, as for zc_compress
 *   other arguments as zc_compress.
 * The counts are checked on the device.  If they are out of range or do not
 * sum to total_values, nothing is compressed and every d_comp_sizes and
 * d_slot_off entry of the affected launch (up to 64 chunks) is -1.
 * Returns as zc_compress.
 */
int zc_compress_dev(const uint16_t* d_in, const int64_t* d_counts,
                    int32_t num_chunks, int64_t total_values, void* d_out,
                    size_t out_capacity, int64_t* d_comp_sizes,
                    int64_t* d_slot_off, void* d_ws, size_t ws_bytes,
                    void* stream);

/*
 * zc_decompress with the counts and offsets in device memory.
 *   d_in_offsets  device int64[num_chunks], 8-byte aligned: byte offset of
 *                 stream c in d_in (16-byte aligned), for example the
 *                 d_slot_off of zc_compress_dev; or NULL for the slot layout
 *   d_counts      device int64[num_chunks], summing to total_values
 *   d_ws          256-byte aligned, ws_bytes >= zc_workspace_bytes_max(...)
 *   other arguments as zc_decompress.
 * Counts or offsets that are out of range record ZC_REASON_SIZE in
 * *d_status and decode nothing of the affected launch.
 */
int zc_decompress_dev(const void* d_in, size_t in_bytes,
                      const int64_t* d_in_offsets, const int64_t* d_counts,
                      int32_t num_chunks, int64_t total_values,
                      uint16_t* d_out, int32_t* d_status, void* d_ws,
                      size_t ws_bytes, void* stream);

/*
 * Receive side of a compressed reduce-scatter (pith.science, Figure 5: the
 * zipccl ReduceScatter workflow; Figure 3: ReduceScatter).  A rank receives
 * one compressed copy of its shard from each of num_chunks peers, decodes
 * them, and sums them element by element:
 *   d_out[i] = (((+0 + x_0[i]) + x_1[i]) + ...) + x_{C-1}[i]
 * in fp32 with round-to-nearest-even, added in chunk order c = 0 .. C-1, where
 * x_c[i] is value i of stream c widened exactly from bf16.  The result is
 * bit-identical to that order of additions; only NaN sign and payload are
 * unspecified.
 *   d_in, in_bytes, in_offsets  as for zc_decompress; every stream must hold
 *               exactly n values
 *   n           values per stream (the shard length), 0 .. ZC_MAX_CHUNK_VALUES
 *   num_chunks  streams to sum, >= 0 (0 writes n zeros)
 *   d_out       device fp32[n], 16-byte aligned
 *   d_status    device int32, 0 on entry; as for zc_decompress.  If it is
 *               nonzero after the stream has run, d_out is undefined.
 *   d_scratch   device, 16-byte aligned, scratch_bytes >=
 *               zc_reduce_scratch_bytes(n, num_chunks) (may be NULL when
 *               that is 0): the decoded bf16 contributions are staged
 *               there, one or two slabs at a time; caller-owned, contents
 *               undefined after
 *   stream      hipStream_t; every launch is queued on it
 * With 8 to 64 streams of T = ceil(n / 8192) >= 512 tiles, where T is at
 * least 27/32 of ceil(T / 512) * 512 (a launch runs 512 tile positions at
 * once), one launch decodes and sums with nothing staged: a workgroup per
 * tile position decodes that tile of eight streams at a time and adds them
 * in LDS, in chunk order.  Otherwise the shard is processed in slabs of whole
 * 8192-value tiles, about 128 MiB of staged values per slab over all
 * streams, so that a slab is summed while it is still in the device's
 * 256 MB last-level cache.  With at most 64 streams and more than one slab,
 * launch i decodes slab i into one of two slab buffers and sums slab i - 1
 * from the other; with more streams, each slab is decoded and then summed.
 * Returns ZC_OK once queued; ZC_EINVAL for a bad argument, ZC_ENOSPC for a
 * short scratch buffer (nothing queued), ZC_EHIP if a launch fails.
 */
int zc_decompress_reduce(const void* d_in, size_t in_bytes,
                         const int64_t* in_offsets, int64_t n,
                         int32_t num_chunks, float* d_out, int32_t* d_status,
                         void* d_scratch, size_t scratch_bytes, void* stream);

/*
 * Scratch bytes that zc_decompress_reduce and zc_decompress_reduce_bf16 need
 * for num_chunks streams of n values: 0 when one launch decodes and sums
 * (see zc_decompress_reduce); otherwise 2 num_chunks s per slab
 * buffer, where s (values per stream per slab) is n rounded up to 8 when
 * one slab holds the whole shard (one buffer), else the slab's whole tiles
 * (two buffers for at most 64 streams, one for more).  At most about
 * 256 MiB whatever n (more only when one tile per stream exceeds a slab); 0
 * for n == 0 or an argument out of range.  A property of this library's
 * kernels and slab size, not of the stream format.
 */
size_t zc_reduce_scratch_bytes(int64_t n, int32_t num_chunks);

/*
 * zc_decompress_reduce delivering bf16: the same chunk-order fp32 sums,
 * each rounded once to bf16, to nearest with ties to even (a sum beyond the
 * largest bf16 becomes infinity; a NaN sum becomes 0x7FC0).  d_out is device
 * uint16[n] of bf16 bit patterns, 16-byte aligned; everything else as for
 * zc_decompress_reduce.  This is the dtype a bf16 gradient shard is kept in
 * (pith.science, Figure 5: the zipped ReduceScatter hands the sum back to
 * training).
 */
int zc_decompress_reduce_bf16(const void* d_in, size_t in_bytes,
                              const int64_t* in_offsets, int64_t n,
                              int32_t num_chunks, uint16_t* d_out,
                              int32_t* d_status, void* d_scratch,
                              size_t scratch_bytes, void* stream);

/*
 * Chunk-pipelined exchange (abstract, technique (2): pipelining in the GPU
 * kernels; pith.science, Figure 5: compress before the collective, decompress
 * after it; Figure 14 caption: the pipelined Design-2 of the zipped
 * All-to-All).  The chunks are split into `groups` consecutive groups (group
 * g holds chunks floor(g C / groups) .. floor((g + 1) C / groups) - 1 of
 * C = num_chunks).  Each group is compressed on s_comp into d_send, its
 * streams are carried to d_recv on s_link, and it is decoded from d_recv on
 * s_dec; an event per stage boundary orders the three stages of one group,
 * so stage k of group g + 1 can run while stage k + 1 of group g does.  On
 * one GPU the carrier is a device copy of comp_sizes[c] bytes per slot, the
 * stand-in for a peer-to-peer send.
 *   d_in, counts, num_chunks   as zc_compress
 *   groups         1 .. num_chunks
 *   d_send, d_recv device, 16-byte aligned, capacity >= zc_bound(...) bytes
 *                  each, slot layout; d_recv receives only the stream bytes
 *   d_comp_sizes   device int64[num_chunks], as zc_compress
 *   d_out          device, sum(counts) bf16 values
 *   d_status       device int32, 0 on entry; as zc_decompress
 *   d_ws, ws_bytes as zc_compress; the compress stages run in order on
 *                  s_comp and share it
 *   s_comp, s_link, s_dec  hipStream_t (equal streams serialise the stages)
 * All buffers are caller-owned.  The call creates two events per group and
 * releases them once their waits are queued.  Returns ZC_OK once everything
 * is queued (d_out is complete when s_dec reaches this point);
 * ZC_EINVAL / ZC_ENOSPC before anything is queued for a bad argument;
 * ZC_EHIP if a launch or event call fails (earlier groups may be queued).
 */
int zc_pipeline(const uint16_t* d_in, const int64_t* counts, int32_t num_chunks,
                int32_t groups, void* d_send, void* d_recv, size_t capacity,
                int64_t* d_comp_sizes, uint16_t* d_out, int32_t* d_status,
                void* d_ws, size_t ws_bytes, void* s_comp, void* s_link,
                void* s_dec);

/*
 * Adaptive switch (abstract, technique (3): compressed or plain collective,
 * chosen from the workload and the system; pith.science, Figure 15 caption:
 * the adaptive switcher).  zc_estimate predicts the compressed size from a
 * sample of tiles; zc_switch_decide compares the two collectives' times.
 */

/*
 * Estimated ZCB1 stream bytes of each chunk, from samples_per_chunk tiles
 * spread evenly over it (tile floor(i T / k), i < k = min(samples, T) of its
 * T tiles): the stream's fixed part (header, index, raw bytes: X) plus the
 * sampled tiles' exponent-stream bytes scaled by T / k, rounded half up.
 * With samples_per_chunk >= T the estimate is the exact comp_bytes that
 * zc_compress writes.
 *   d_in         device bf16[total_values], chunks back to back
 *   d_counts     device int64[num_chunks], summing to total_values
 *   d_est        device int64[num_chunks]: the estimates, or -1 in every
 *                entry if a count is outside 0 .. ZC_MAX_CHUNK_VALUES or the
 *                counts do not sum to total_values
 * Reads every count once per chunk (one workgroup per chunk).  Returns ZC_OK
 * once queued, ZC_EINVAL (samples_per_chunk < 1, negative sizes, null
 * pointers) or ZC_EHIP.
 */
int zc_estimate(const uint16_t* d_in, const int64_t* d_counts,
                int32_t num_chunks, int64_t total_values,
                int32_t samples_per_chunk, int64_t* d_est, void* stream);

/* Collectives modelled by zc_switch_decide. */
#define ZC_COLL_ALLGATHER 0
#define ZC_COLL_REDUCE_SCATTER 1
#define ZC_COLL_ALLTOALL 2

typedef struct {
    double link_GBps;        /* per-rank bandwidth of the plain collective   */
    double step_latency_us;  /* latency of each of its ranks - 1 steps       */
    double compress_GBps;    /* codec rates, in GB/s of uncompressed bytes:  */
    double decompress_GBps;  /*   zc_compress, zc_decompress,                */
    double reduce_GBps;      /*   zc_decompress_reduce (reduce-scatter only) */
} zc_switch_params;

typedef struct {
    int32_t use_compressed;  /* 1 if the compressed collective is faster     */
    double plain_us;         /* modelled time of the plain collective        */
    double compressed_us;    /* ... of compress, exchange, decompress        */
    double breakeven_GBps;   /* compression wins on links slower than this;
                                0 if it never does                          */
} zc_switch_result;

/*
 * Host-only cost model of one collective on `ranks` ranks.  Per rank, with
 * S = bytes (the uncompressed collective buffer), C = comp_bytes (its
 * compressed size, e.g. the sum of zc_estimate), W = S (P-1)/P and
 * W_c = C (P-1)/P:
 *   plain       (P-1) a + W / B
 *   compressed  (P-1) a + W_c / B + codec, with codec =
 *     ZC_COLL_ALLGATHER       (S/P) / R_comp + W / R_dec
 *     ZC_COLL_ALLTOALL        S / R_comp + W / R_dec
 *     ZC_COLL_REDUCE_SCATTER  S / R_comp + S / R_red  (all-to-all, then
 *                             decode and sum: pith.science, Figure 5)
 * so compression wins exactly below B* = (W - W_c) / codec.  Returns ZC_OK,
 * or ZC_EINVAL for an unknown collective, ranks < 1, negative or non-finite
 * sizes, C = 0 with S > 0, or a rate the collective needs that is not
 * positive and finite.
 */
int zc_switch_decide(int32_t collective, int32_t ranks, double bytes,
                     double comp_bytes, const zc_switch_params* params,
                     zc_switch_result* result);

/* Static text for a zc_status_t value. */
const char* zc_strerror(int code);

/*
 * The library's code table for table_id 1, regenerated on the host from the
 * closed-form law and checked against the table compiled into the kernels.
 * lengths[17] and codes[17] (d = 0..15, then ESC); prob[17] may be NULL.
 * Returns ZC_OK, or ZC_EINVAL for another table_id or a self-check mismatch.
 */
int zc_code_table(int32_t table_id, int32_t* lengths, uint32_t* codes,
                  double* prob);

#ifdef __cplusplus
}
#endif
#endif /* ZC_H */
