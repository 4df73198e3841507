// zc_kernels.hip -- gfx950 compress / decompress kernels and the C ABI.
//
// Method: ZipCCL (arXiv 2604.27844), abstract, techniques (1) and (2).  The
// bf16 exponent is coded relative to the largest exponent of its group with
// a fixed canonical prefix code derived from the Gaussian law (no run-time
// statistics); the sign+mantissa byte is stored raw, which is how a 16-bit
// value reaches about 11 bits (pith.science, Figure 6 caption).
//
// GPU mapping (MI355X, wave64; the code tables live in LDS):
//  * a tile holds 8192 values in 64 groups; group 64t + l takes 8 consecutive
//    bf16 (one 16-byte load) at each of 16 steps, so every global load and
//    store of the raw data is fully coalesced;
//  * compress gives a tile to one workgroup of four waves: lane l of each
//    wave works on group l, wave w on steps 4w..4w+3, and the four partial
//    maxima and code lengths meet in LDS; decompress gives a tile to one
//    wave, lane l decoding group l;
//  * a wave prefix sum over the 64 group lengths places the lane streams in
//    an LDS copy of the tile stream (the pages stage data in shared memory,
//    Figure 7 caption), which is stored coalesced;
//  * the byte offset of a tile inside its chunk's exponent section is an
//    exclusive scan over the tiles of the chunk, done in the same pass with a
//    decoupled look-back over per-tile status words.  A workgroup's tile
//    comes from its grid position, chunk by chunk, so neighbouring
//    workgroups stream neighbouring bytes.  Every wait is bounded: past the
//    bound a missing predecessor's size is recomputed from its input, so no
//    order of dispatch can stall it;
//  * all chunks of a call form one flat list of tiles, so uneven chunk sizes
//    (the imbalance of Figure 8) still fill the GPU;
//  * the inner loops are branch-free: the encoder appends code words (two
//    members per table entry where no escape occurs) to a 64-bit
//    accumulator and ORs each finished word into LDS; the decoder refills a
//    64-bit window from LDS every four or eight symbols and takes one table
//    lookup per symbol (code words longer than the lookup width, and
//    escapes, take a rare second lookup);
//  * no value is carried in a register that a memory load must refill inside
//    a loop or across the encoder's emission: on this hardware the wait for
//    such a load also waits for every older store of the wave.
// The codec itself is integer arithmetic; only the decode + sum of a
// reduce-scatter's received copies adds in fp32.  For a long shard of 8 to
// 64 received copies that sum runs in one kernel: a workgroup per tile
// position decodes that tile of eight copies at a time and adds them
// through LDS in chunk order, with nothing staged in memory; other shapes
// decode into slab buffers and sum them.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>
#include <algorithm>

#include "zc.h"
#include "zc_table.h"
#include "zc_table_v1.inc"

namespace {

constexpr int kLanes = 64;
constexpr int kWaves = 4;                          // waves per workgroup
constexpr int kBlock = kLanes * kWaves;
constexpr int kSteps = 16;
constexpr int kTile = 8192;
constexpr int kStageWords = 1024;                 // LDS tile-stream buffer per wave (4 KiB)
constexpr int kStageAlloc = kStageWords + 8;      // + guard and carry words
constexpr int kMinWavesEnc = 8;                   // occupancy targets, waves per SIMD
constexpr int kMinWavesDec = 8;
constexpr int kMaxChunks = 64;                     // chunks per launch
constexpr uint32_t kMagic = 0x3142435Au;
constexpr uint32_t kVerTable = 0x00010001u;        // version 1, table_id 1
constexpr int kEsc = ZC_T1_NSYM - 1;
constexpr int kEscLen = ZC_T1_ESC_LEN;
constexpr int kLutBits = ZC_T1_LUT_BITS;          // first decode level (byte entries)
constexpr int kTailBits = ZC_T1_TAIL_BITS;        // second level
constexpr int kLutRaw = 1 << kLutBits;            // raw-mode byte entries follow
constexpr uint32_t kSpinLimit = 1u << 14;          // look-back polls before recomputing
constexpr uint32_t kPollLanes = 12;                // predecessors read per look-back poll

// Compress workspace: a header, then one 8-byte look-back status word per
// tile, one per 64-byte line (a tile's status is written through to
// device-coherent memory, and tiles sharing a line would serialize those
// writes).  Header: the last launch's tag (epoch, u32) at byte 0, then 64
// counters of finished workgroups, one u32 per 128-byte line from byte 128.
constexpr uint32_t kCounters = 64;
constexpr uint32_t kCounterStride = 32;            // u32 index step between counters
constexpr uint32_t kHdrEpoch = 0;                  // u32 index
constexpr uint32_t kHdrCounters = 32;              // u32 index (byte 128)
constexpr size_t kWsHeader = 128 + kCounters * 128 + 128;   // 8448 bytes
constexpr uint32_t kDoneSpinLimit = 1u << 22;      // polls of the last workgroup
constexpr uint32_t kStatusStride = 8;              // u64 index step between status words
// A status word: the launch's tag (epoch) in bits 32-63, the flag in bits
// 30-31 (1 = the tile's own size is known, 2 = its inclusive prefix is),
// the value in 32-bit words in bits 0-29.  Words with another launch's tag
// read as "not yet published", so no launch has to clear them first.
constexpr uint32_t kFlagAgg = 1;
constexpr uint32_t kFlagInc = 2;

static_assert(ZC_T1_NSYM == 17, "table_id 1 has 17 symbols");
static_assert(ZC_T1_TAIL_OK == 1, "long code words must share the all-ones prefix");
static_assert(ZC_T1_MAXLEN <= kLutBits + kTailBits, "code words must fit two lookup levels");
static_assert(kEscLen + 8 <= 32, "escape payload must fit the window");
static_assert(kLutBits >= 8 && kLutBits <= 12, "first level of 256 to 4096 byte entries");
constexpr int kLutWords = (1 << kLutBits) / 4;     // first level, 32-bit words
constexpr int kLutPer = (kLutWords + kBlock - 1) / kBlock;   // words loaded per thread

__constant__ __align__(16) uint8_t c_lut[1 << kLutBits] = ZC_T1_LUT_INIT;

// The lengths and second-level entries of table_id 1 as compile-time
// constants: the decoder's threads pick theirs with selects, so its small
// LDS tables are set up without a memory round trip.
constexpr uint32_t kLenT1[ZC_T1_NSYM] = ZC_T1_LEN_INIT;
constexpr uint32_t kCodeT1[ZC_T1_NSYM] = ZC_T1_CODE_INIT;
constexpr uint32_t kTailT1[1 << kTailBits] = ZC_T1_TAIL_INIT;

__device__ inline uint32_t len_of(uint32_t s)
{
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < ZC_T1_NSYM; ++i)
        v = s == static_cast<uint32_t>(i) ? kLenT1[i] : v;
    return v;
}

__device__ inline uint32_t tail_of(uint32_t i)
{
    uint32_t v = 0;
#pragma unroll
    for (int j = 0; j < (1 << kTailBits); ++j)
        v = i == static_cast<uint32_t>(j) ? kTailT1[j] : v;
    return v;
}

// Chunks of one launch.  Work item = one tile; an empty chunk gets one item
// that only writes its header.
struct ChunkTable {
    int32_t nchunks;
    int32_t chunk_base;            // index of the launch's first chunk in the call (status reports)
    uint32_t nitems;
    uint32_t spin_limit;           // compress: look-back polls before recomputing
    uint32_t tile0;                // decompress: index of each chunk's first tile in the launch
    uint32_t item_begin[kMaxChunks + 1];
    uint32_t n[kMaxChunks];
    uint64_t voff[kMaxChunks];     // value offset of the chunk (bf16 side)
    uint64_t boff[kMaxChunks];     // byte offset of the chunk stream
    uint64_t bavail[kMaxChunks];   // decompress: readable bytes from boff
};

struct Geom {
    uint32_t T;
    uint64_t R, X;
};

__host__ __device__ inline uint64_t align16(uint64_t x) { return (x + 15) & ~uint64_t(15); }
__host__ __device__ inline uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

__host__ __device__ inline Geom geometry(uint64_t n)
{
    Geom g;
    g.T = static_cast<uint32_t>((n + kTile - 1) / kTile);
    g.R = align16(32 + 196ull * g.T);
    g.X = align16(g.R + n);
    return g;
}

__host__ __device__ inline uint64_t chunk_bound(uint64_t n)
{
    Geom g = geometry(n);
    return g.X + n + 4ull * g.T;
}

// ------------------------------------------------------------ wave utils

// Keeps this wave's LDS accesses in program order (the LDS unit performs one
// wave's operations in order, so no wait is needed).
__device__ inline void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ inline uint32_t wave_excl_scan(uint32_t x, uint32_t lane, uint32_t* total)
{
    uint32_t incl = x;
#pragma unroll
    for (int o = 1; o < kLanes; o <<= 1) {
        uint32_t y = __shfl_up(incl, o);
        if (lane >= static_cast<uint32_t>(o))
            incl += y;
    }
    *total = __shfl(incl, kLanes - 1);
    return incl - x;
}

__device__ inline uint32_t wave_sum(uint32_t x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}

// Values of this lane's group inside a tile holding `rem` values.
__device__ inline uint32_t group_members(uint32_t rem, uint32_t lane)
{
    uint32_t ng = 0;
#pragma unroll
    for (int k = 0; k < kSteps; ++k) {
        int left = static_cast<int>(rem) - k * 512 - static_cast<int>(lane) * 8;
        ng += left <= 0 ? 0u : (left >= 8 ? 8u : static_cast<uint32_t>(left));
    }
    return ng;
}

// Word `lane` (0..7) of a chunk header.
__device__ inline uint32_t header_word(uint32_t lane, uint64_t n, uint64_t comp)
{
    uint32_t v = 0;
    v = lane == 0 ? kMagic : v;
    v = lane == 1 ? kVerTable : v;
    v = lane == 4 ? static_cast<uint32_t>(n) : v;
    v = lane == 5 ? static_cast<uint32_t>(n >> 32) : v;
    v = lane == 6 ? static_cast<uint32_t>(comp) : v;
    v = lane == 7 ? static_cast<uint32_t>(comp >> 32) : v;
    return v;
}

__device__ inline int find_chunk(const ChunkTable& tab, uint32_t item)
{
    int lo = 0, hi = tab.nchunks;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (tab.item_begin[mid] <= item)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

__device__ inline uint32_t hi32(uint64_t x) { return static_cast<uint32_t>(x >> 32); }
__device__ inline uint32_t max3(uint32_t a, uint32_t b, uint32_t c) { return max(a, max(b, c)); }
__device__ inline uint32_t lo32(uint64_t x) { return static_cast<uint32_t>(x); }

// Streaming accesses: every input byte is read once and every output byte
// written once, so they are marked nontemporal (no reuse expected in the
// caches).  On gfx950 this nearly doubles the rate of plain 16-byte loads
// over a large buffer.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__device__ inline uint4 ld_nt4(const void* p)
{
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint2 ld_nt2(const void* p)
{
    const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
    return make_uint2(v.x, v.y);
}
__device__ inline uint32_t ld_nt1(const uint32_t* p) { return __builtin_nontemporal_load(p); }
// A plain (cached) 8-byte load.  The sign+mantissa section starts 16-byte
// aligned, so its 512-byte rows straddle 128-byte lines; where a row is read
// in two halves at different times, the line they share can still be in L2
// for the second half.
__device__ inline uint2 ld2(const void* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ inline void st_nt4(void* p, uint4 v)
{
    __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(p));
}
__device__ inline void st_nt2(void* p, uint2 v)
{
    __builtin_nontemporal_store(v2u{v.x, v.y}, reinterpret_cast<v2u*>(p));
}

// ------------------------------------------------------------ compress

// Indexed by d = E_max - e (0..255).  esc[d] = code word | length << 24,
// with bit 31 set and the code word shifted left by 8 for an escape (d >= 16),
// whose 8 exponent bits follow it.
struct __align__(16) EncTables {
    uint32_t esc[256];
    uint32_t pcode[256];  // member pair (d0, d1 < 16) at index d0 | d1 << 4: code words back to back
    uint8_t len[256];     // coded length of d, escape payload included
    uint8_t plen[256];    // the pair's total length (at most 28)
};
static_assert(sizeof(EncTables) % 16 == 0, "copied to LDS in 16-byte words");

// The encoder's tables of table_id 1, evaluated at compile time; each
// workgroup copies them into LDS with one 16-byte load per thread.
__host__ __device__ constexpr EncTables make_enc_tables()
{
    EncTables t{};
    for (int i = 0; i < 256; ++i) {
        const int sym = i < kEsc ? i : kEsc;
        uint32_t code = kCodeT1[sym], len = kLenT1[sym];
        if (sym == kEsc) {      // escape: code word, then 8 exponent bits
            code <<= 8;
            len += 8;
        }
        t.esc[i] = code | (len << 24) | (sym == kEsc ? 0x80000000u : 0u);
        t.len[i] = static_cast<uint8_t>(len);
        const int d0 = i & 15, d1 = i >> 4;
        t.pcode[i] = (kCodeT1[d0] << kLenT1[d1]) | kCodeT1[d1];
        t.plen[i] = static_cast<uint8_t>(kLenT1[d0] + kLenT1[d1]);
    }
    return t;
}
__constant__ EncTables c_enc = make_enc_tables();

// A tile is compressed by the four waves of a workgroup.  Lane l of every
// wave works on group l; wave w takes steps 4w..4w+3 of it, which are members
// 32w..32w+31 in the group's order.  The four partial maxima and partial code
// lengths of a group meet in LDS, so each thread knows where its quarter of
// the group's stream starts; the four waves then write their code words into
// one LDS copy of the tile stream, and wave 0 places it in the chunk.
constexpr int kEncWaves = 4;                       // waves per compress workgroup
constexpr int kEncBlock = kLanes * kEncWaves;
constexpr int kQSteps = kSteps / kEncWaves;        // steps per wave
constexpr int kQMembers = kQSteps * 8;             // members per wave and group
constexpr int kTileWordsMax = kTile / 4;           // an all-raw tile stream
constexpr int kEncStage = kTileWordsMax + 8;       // + guard words

struct EncShared {
    EncTables tb;
    uint32_t stage[kEncStage];              // the tile stream being built (zero between tiles)
    uint16_t part_max[kEncWaves][kLanes];   // at most 255
    uint16_t part_bits[kEncWaves][kLanes];  // at most 64 * 22
};

// One tile of a launch: its chunk, place and geometry (all uniform).
struct TileCtx {
    const uint16_t* src;
    uint8_t* dst;
    Geom G;
    uint32_t n, t, base, rem, item, first, lane, wave;
    int c;
};

__device__ inline TileCtx tile_ctx(const ChunkTable& tab, uint32_t item,
                                   const uint16_t* __restrict__ in, uint8_t* __restrict__ out,
                                   uint32_t lane, uint32_t wave)
{
    TileCtx x;
    x.c = find_chunk(tab, item);
    x.n = tab.n[x.c];
    x.first = tab.item_begin[x.c];
    x.item = item;
    x.t = item - x.first;
    x.base = x.t * kTile;
    x.rem = x.n ? min(x.n - x.base, static_cast<uint32_t>(kTile)) : 0u;
    x.src = in + tab.voff[x.c];
    x.dst = out + tab.boff[x.c];
    x.G = geometry(x.n);
    x.lane = lane;
    x.wave = wave;
    return x;
}

// A whole tile of 8192 values at a 16-byte aligned address takes the vector
// path (tile starts are 16 KiB apart inside a chunk).
__device__ inline bool tile_full(const TileCtx& x)
{
    return x.rem == kTile && (reinterpret_cast<uintptr_t>(x.src) & 15) == 0;
}

// Loads this wave's four steps of the tile (16 bytes per lane each; FULL =
// 8192 values at a 16-byte aligned address; otherwise missing members read
// as 0).
template <bool FULL>
__device__ inline void load_tile(const TileCtx& x, uint4 (&v)[kQSteps])
{
    const uint32_t k0 = x.wave * kQSteps;
    const char* sbase = reinterpret_cast<const char*>(x.src + x.base) + k0 * 1024 + x.lane * 16;
    if (FULL) {
#pragma unroll
        for (int k = 0; k < kQSteps; ++k)
            v[k] = ld_nt4(sbase + k * 1024);
        return;
    }
    // every segment of 8 values wholly inside the chunk is one load when
    // the chunk is 16-byte aligned; these are all issued before the ragged
    // end (or an unaligned chunk) is read value by value
    const bool aligned = (reinterpret_cast<uintptr_t>(x.src) & 15) == 0;
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) {
        const uint32_t i0 = x.base + (k0 + k) * 512 + x.lane * 8;
        v[k] = make_uint4(0, 0, 0, 0);
        if (aligned && i0 + 8 <= x.n)
            v[k] = ld_nt4(sbase + k * 1024);
    }
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) {
        const uint32_t i0 = x.base + (k0 + k) * 512 + x.lane * 8;
        if (!(aligned && i0 + 8 <= x.n) && i0 < x.n) {
            uint32_t w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                w[j] = (i0 + j < x.n) ? x.src[i0 + j] : 0u;
            v[k].x = w[0] | (w[1] << 16);
            v[k].y = w[2] | (w[3] << 16);
            v[k].z = w[4] | (w[5] << 16);
            v[k].w = w[6] | (w[7] << 16);
        }
    }
}

// Splits the loaded steps: raw bytes are stored at once, exponents stay
// packed 4 per word, the maximum exponent is returned.
template <bool FULL>
__device__ inline uint32_t split_tile(const TileCtx& x, const uint4 (&v)[kQSteps],
                                      uint32_t (&ex)[kQSteps][2])
{
    const uint32_t k0 = x.wave * kQSteps;
    char* rbase = reinterpret_cast<char*>(x.dst + x.G.R + x.base) + k0 * 512 + x.lane * 8;
    uint32_t mx = 0;
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) {
        const uint4 q = v[k];
        const uint32_t lo_a = __builtin_amdgcn_perm(q.y, q.x, 0x06040200u);
        const uint32_t hi_a = __builtin_amdgcn_perm(q.y, q.x, 0x07050301u);
        const uint32_t lo_b = __builtin_amdgcn_perm(q.w, q.z, 0x06040200u);
        const uint32_t hi_b = __builtin_amdgcn_perm(q.w, q.z, 0x07050301u);
        const uint32_t raw_a = (hi_a & 0x80808080u) | (lo_a & 0x7F7F7F7Fu);
        const uint32_t raw_b = (hi_b & 0x80808080u) | (lo_b & 0x7F7F7F7Fu);
        ex[k][0] = ((hi_a << 1) & 0xFEFEFEFEu) | ((lo_a >> 7) & 0x01010101u);
        ex[k][1] = ((hi_b << 1) & 0xFEFEFEFEu) | ((lo_b >> 7) & 0x01010101u);
        mx = max(mx, max(max(q.x & 0x7F80u, (q.x >> 16) & 0x7F80u),
                         max(q.y & 0x7F80u, (q.y >> 16) & 0x7F80u)));
        mx = max(mx, max(max(q.z & 0x7F80u, (q.z >> 16) & 0x7F80u),
                         max(q.w & 0x7F80u, (q.w >> 16) & 0x7F80u)));
        if (FULL) {
            *reinterpret_cast<uint2*>(rbase + k * 512) = make_uint2(raw_a, raw_b);
        } else {
            const uint32_t i0 = x.base + (k0 + k) * 512 + x.lane * 8;
            uint8_t* rdst = x.dst + x.G.R + i0;      // 8-byte aligned (R and i0 are)
            if (i0 + 8 <= x.n) {
                st_nt2(rdst, make_uint2(raw_a, raw_b));
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (i0 + j < x.n)
                        rdst[j] = static_cast<uint8_t>(((j < 4 ? raw_a : raw_b) >> (8 * (j & 3))) & 0xFF);
            }
        }
    }
    return mx >> 7;   // missing members were loaded as 0
}

// Decoupled look-back over per-tile status words (see kFlagAgg / kFlagInc).
// Publishing comes first; the exclusive offset is resolved later, so the
// caller can do other work while predecessors finish.  Sizes and prefixes
// are in 32-bit words (tile streams are whole words).

__device__ inline uint64_t status_word(uint32_t epoch, uint32_t flag, uint32_t words)
{
    return (static_cast<uint64_t>(epoch) << 32) | (flag << 30) | words;
}

// A polled status word as (flag << 62) | words, or 0 if it does not carry
// this launch's tag (written by an earlier launch, or never).
__device__ inline uint64_t status_norm(uint64_t s, uint32_t epoch)
{
    return hi32(s) == epoch
               ? (static_cast<uint64_t>(lo32(s) >> 30) << 62) | (lo32(s) & 0x3FFFFFFFu)
               : 0ull;
}

__device__ inline void look_back_publish(uint64_t* __restrict__ status, uint32_t item, uint32_t t,
                                         uint32_t tile_words, uint32_t lane, uint32_t epoch)
{
    if (lane == 0)
        __hip_atomic_store(&status[item * kStatusStride],
                           status_word(epoch, t == 0 ? kFlagInc : kFlagAgg, tile_words),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One poll of the look-back window: the status words of the kPollLanes
// tiles below `top` (lane l reads tile top - l), zero where they belong to no
// predecessor.
__device__ inline uint64_t look_back_poll(const uint64_t* __restrict__ status, int64_t top,
                                          uint32_t first, uint32_t lane, uint32_t epoch)
{
    const int64_t idx = top - static_cast<int64_t>(lane);
    uint64_t s = 0;
    if (lane < kPollLanes && idx >= static_cast<int64_t>(first))
        s = status_norm(__hip_atomic_load(&status[idx * kStatusStride], __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT), epoch);
    return s;
}

// The size in words of tile `t`'s stream for a chunk (`src`, `n` values),
// recomputed from its input: the encoder's group maxima, code lengths and
// mode, one group per lane.  The look-back falls back on it for a
// predecessor that has not published within the spin limit, so that no wait
// is unbounded.
__device__ inline uint32_t tile_words_from_input(
    const uint16_t* __restrict__ src, uint32_t n, uint32_t t, uint32_t lane,
    const uint8_t* __restrict__ len)
{
    const uint32_t base = t * kTile;
    const uint32_t ng = group_members(min(n - base, static_cast<uint32_t>(kTile)), lane);
    uint32_t emax = 0;
#pragma unroll 1
    for (int k = 0; k < kSteps; ++k)
        for (int j = 0; j < 8; ++j) {
            const uint32_t i = base + k * 512 + lane * 8 + j;
            if (i < n)
                emax = max(emax, (static_cast<uint32_t>(src[i]) >> 7) & 0xFF);
        }
    uint32_t bits = 0;
#pragma unroll 1
    for (int k = 0; k < kSteps; ++k)
        for (int j = 0; j < 8; ++j) {
            const uint32_t i = base + k * 512 + lane * 8 + j;
            if (i < n)
                bits += len[emax - ((static_cast<uint32_t>(src[i]) >> 7) & 0xFF)];
        }
    const uint32_t glen = (ng > 0 && bits >= 8 * ng) ? 8 * ng : bits;
    return (wave_sum(glen) + 31) >> 5;
}

// The exclusive word offset of tile `t`: sums predecessors' sizes down to
// the nearest one whose inclusive prefix is known.  After `spin_limit` polls
// that still miss a predecessor, the missing sizes are recomputed from the
// input instead (the chunk is `src`, `n` values).
__device__ inline uint32_t look_back_resolve(const uint64_t* __restrict__ status, uint32_t item,
                                             uint32_t t, uint32_t first, uint32_t lane,
                                             uint32_t epoch, const uint16_t* __restrict__ src,
                                             uint32_t n, const uint8_t* __restrict__ len,
                                             uint32_t spin_limit)
{
    if (t == 0)
        return 0;
    int64_t top = static_cast<int64_t>(item) - 1;
    uint64_t s = look_back_poll(status, top, first, lane, epoch);
    uint32_t acc = 0;
    uint32_t spins = 0;
    while (true) {
        const bool in_range = lane < kPollLanes &&
                              top - static_cast<int64_t>(lane) >= static_cast<int64_t>(first);
        const uint32_t flag = static_cast<uint32_t>(s >> 62);
        const uint64_t inc_mask = __ballot(in_range && flag == kFlagInc);
        const uint64_t zero_mask = __ballot(in_range && flag == 0);
        if (inc_mask) {
            const int p = __ffsll(static_cast<unsigned long long>(inc_mask)) - 1;
            const uint64_t below = (p == 0) ? 0ull : ((1ull << p) - 1);
            if ((zero_mask & below) == 0) {
                acc += wave_sum(lane <= static_cast<uint32_t>(p) ? static_cast<uint32_t>(s) : 0u);
                break;
            }
        } else if (zero_mask == 0) {
            acc += wave_sum(static_cast<uint32_t>(s));
            top -= kPollLanes;
            s = look_back_poll(status, top, first, lane, epoch);
            continue;
        }
        if (spins < spin_limit) {
            // a predecessor has not published yet: poll the same window again
            ++spins;
            __builtin_amdgcn_s_sleep(1);
            s = look_back_poll(status, top, first, lane, epoch);
            continue;
        }
        // waited too long: recompute the missing sizes (the chunk's first
        // tile counts as an inclusive prefix)
        for (uint64_t miss = zero_mask; miss; miss &= miss - 1) {
            const int i = __ffsll(static_cast<unsigned long long>(miss)) - 1;
            const uint32_t p = static_cast<uint32_t>(top - i);
            const uint32_t words = tile_words_from_input(src, n, p - first, lane, len);
            if (lane == static_cast<uint32_t>(i))
                s = (static_cast<uint64_t>(p == first ? kFlagInc : kFlagAgg) << 62) | words;
        }
    }
    return acc;
}

// Appends code words to a thread's stream accumulator: `acc` holds the
// stream's pending bits (nacc of them, fewer than 32, at the bottom), and
// each whole 32-bit word is ORed into the LDS tile stream at word wi.  One
// call appends `len` <= 32 bits of `code`.
__device__ __forceinline__ void emit_bits(uint32_t* __restrict__ s, uint64_t& acc, uint32_t& nacc,
                                          uint32_t& wi, uint32_t code, uint32_t len)
{
    acc = (acc << len) | code;
    nacc += len;
    const uint32_t wv = __builtin_amdgcn_alignbit(hi32(acc), lo32(acc), nacc);
    const uint32_t f = nacc >> 5;
    atomicOr(&s[wi], f ? wv : 0u);
    wi += f;
    nacc &= 31;
}

// Appends this thread's members of its group to the LDS tile stream from bit
// `off`: one code word per value, or for a raw group (MIXED waves only) the
// exponents as 8-bit words.  Only the thread's first `nv` members are
// written (all 32 in a full tile; in a partial one the members present are a
// prefix of the group's member order).
//  * A step in which no coded lane of the wave has an escape takes two
//    members per lookup of the member-pair table (full tiles) and four
//    members per LDS OR when their words fit in 32 bits on every lane.
//  * A step with an escape looks each member up in the escape table (code
//    word, or escape code and the exponent's 8 bits: at most 22 bits) and
//    appends four members per OR when their words fit in 32 bits on every
//    lane (an escape beside three short codes; a raw lane's four exponents
//    are exactly 32 bits), else two per OR when every pair fits, else one.
template <bool FULL, bool MIXED>
__device__ __forceinline__ void emit_quarter(uint32_t* __restrict__ s, const EncTables& tb,
                                    const uint32_t (&dd)[kQSteps][2], uint32_t emax,
                                    uint32_t nv, bool raw_mode, uint32_t off)
{
    uint64_t acc = 0;
    uint32_t nacc = off & 31;
    uint32_t wi = off >> 5;
    const bool coded = !raw_mode;
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) {
        const uint32_t d4[2] = {dd[k][0], dd[k][1]};
        const bool esc_here = coded && (((d4[0] | d4[1]) & 0xF0F0F0F0u) != 0);
        // in a partial tile a thread's step is whole, absent (no member in
        // the tile: it emits nothing) or, at the ragged end, in between
        const bool absent = !FULL && static_cast<uint32_t>(k * 8) >= nv;
        const bool ragged = !FULL && !absent && static_cast<uint32_t>(k * 8 + 8) > nv;
        if (__ballot((esc_here && !absent) || ragged) == 0) {
            // every d of the step's coded lanes is below 16, so two members
            // index one pair entry: d0 | d1 << 4 is read off the packed
            // bytes as (w | w >> 4)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t w = d4[h];
                const uint32_t nib = w | (w >> 4);
                uint32_t c01 = tb.pcode[nib & 0xFF], l01 = tb.plen[nib & 0xFF];
                uint32_t c23 = tb.pcode[(nib >> 16) & 0xFF], l23 = tb.plen[(nib >> 16) & 0xFF];
                if (MIXED && raw_mode) {
                    // raw group: the exponents e = E_max - d as 8-bit words
                    const uint32_t e4 = emax * 0x01010101u - w;
                    c01 = __builtin_amdgcn_perm(0u, e4, 0x0c0c0001u);
                    c23 = __builtin_amdgcn_perm(0u, e4, 0x0c0c0203u);
                    l01 = 16;
                    l23 = 16;
                }
                if (!FULL && absent) {
                    c01 = c23 = 0;
                    l01 = l23 = 0;
                }
                if (__ballot(l01 + l23 > 32u) == 0) {
                    emit_bits(s, acc, nacc, wi, (c01 << l23) | c23, l01 + l23);
                } else {
                    emit_bits(s, acc, nacc, wi, c01, l01);
                    emit_bits(s, acc, nacc, wi, c23, l23);
                }
            }
        } else {
            // escape step: each member's word from the escape table; the
            // quad's words are combined in 64 bits and go out in one append
            // when they fit in 32 bits on every lane, else in two; a quad of
            // more than 64 bits (three escapes) is looked up again, pair by
            // pair
            auto member = [&](int u, uint32_t w, int jj, uint32_t& c, uint32_t& L) {
                const uint32_t d = (w >> (8 * u)) & 0xFF;
                uint32_t ent = tb.esc[d];
                if (MIXED && raw_mode)
                    ent = ((emax - d) & 0xFF) | (8u << 24);
                const bool valid = FULL || static_cast<uint32_t>(k * 8 + jj) < nv;
                ent = valid ? ent : 0u;
                L = (ent >> 24) & 31;
                const uint32_t esc = static_cast<uint32_t>(static_cast<int32_t>(ent) >> 31);
                c = (ent & 0x3FFFFFu) | ((emax - d) & esc & 0xFFu);
            };
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t w = d4[h];
                uint64_t cq = 0;
                uint32_t lq = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    uint32_t c, L;
                    member(u, w, 4 * h + u, c, L);
                    cq = (cq << L) | c;
                    lq += L;
                }
                if (__ballot(lq > 32u) == 0) {
                    emit_bits(s, acc, nacc, wi, lo32(cq), lq);
                } else if (__ballot(lq > 64u) == 0) {
                    // at most 64 bits on every lane: the bits above the low
                    // 32 first, then the low 32
                    const bool two = lq > 32u;
                    emit_bits(s, acc, nacc, wi, hi32(cq), two ? lq - 32u : 0u);
                    emit_bits(s, acc, nacc, wi, lo32(cq), two ? 32u : lq);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; u += 2) {
                        uint32_t c0, l0, c1, l1;
                        member(u, w, 4 * h + u, c0, l0);
                        member(u + 1, w, 4 * h + u + 1, c1, l1);
                        if (__ballot(l0 + l1 > 32u) == 0) {
                            emit_bits(s, acc, nacc, wi, (c0 << l1) | c1, l0 + l1);
                        } else {
                            emit_bits(s, acc, nacc, wi, c0, l0);
                            emit_bits(s, acc, nacc, wi, c1, l1);
                        }
                    }
                }
            }
        }
    }
    if (nacc)
        atomicOr(&s[wi], lo32(acc) << (32 - nacc));
}

// Wave 0 of a tile: the tile's index entries; the last tile of a chunk also
// writes the header, the zero gaps and the chunk's size.
__device__ inline void write_tile_index(const TileCtx& x, uint32_t toff, uint32_t tile_bytes,
                                        uint32_t emax, uint32_t glen,
                                        int64_t* __restrict__ comp_sizes)
{
    const uint32_t lane = x.lane;
    if (lane == 0)
        *reinterpret_cast<uint32_t*>(x.dst + 32 + 4ull * x.t) = toff;
    x.dst[32 + 4ull * x.G.T + 64ull * x.t + lane] = static_cast<uint8_t>(emax);
    *reinterpret_cast<uint16_t*>(x.dst + 32 + 68ull * x.G.T + 2ull * (64ull * x.t + lane)) =
        static_cast<uint16_t>(glen);
    if (x.t == x.G.T - 1) {
        const uint64_t comp = x.G.X + toff + tile_bytes;
        if (lane < 8)
            reinterpret_cast<uint32_t*>(x.dst)[lane] = header_word(lane, x.n, comp);
        const uint64_t g1 = 32 + 196ull * x.G.T;
        if (g1 + lane < x.G.R)
            x.dst[g1 + lane] = 0;
        if (x.G.R + x.n + lane < x.G.X)
            x.dst[x.G.R + x.n + lane] = 0;
        if (lane == 0)
            comp_sizes[x.c] = static_cast<int64_t>(comp);
    }
}

// Everything after the loads: the partial maxima of the four waves are in
// sh.part_max (written before the barrier that precedes this call).  Waves
// 1-3 return after the emission; wave 0 resolves the tile's offset, stores
// the stream and the index entries, then publishes.
template <bool FULL>
__device__ __forceinline__ void compress_tile_back(const TileCtx& x, uint32_t (&dd)[kQSteps][2],
                                   int64_t* __restrict__ comp_sizes,
                                   uint64_t* __restrict__ status, EncShared& sh,
                                   uint32_t epoch, uint32_t spin_limit)
{
    const uint32_t lane = x.lane, wave = x.wave;
    const uint32_t ng = FULL ? 128u : group_members(x.rem, lane);
    const uint32_t first = wave * kQMembers;     // group index of this thread's first member
    // members of this thread present in the tile (a prefix of its 32)
    const uint32_t nv = FULL ? static_cast<uint32_t>(kQMembers)
                             : min(ng > first ? ng - first : 0u, static_cast<uint32_t>(kQMembers));

    // 1. the group maximum from the waves' partial ones
    uint32_t emax = sh.part_max[0][lane];
#pragma unroll
    for (int w = 1; w < kEncWaves; ++w)
        emax = max(emax, static_cast<uint32_t>(sh.part_max[w][lane]));

    // 2. distances d = E_max - e (bytes never borrow: e <= E_max) and the
    //    coded length of this thread's members
    const uint32_t em4 = emax * 0x01010101u;
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) {
        dd[k][0] = em4 - dd[k][0];
        dd[k][1] = em4 - dd[k][1];
        // opaque from here on: the emission recomputes a raw group's
        // exponents as E_max - d instead of keeping the exponent words alive
        // beside the distances (which spilled registers)
        asm volatile("" : "+v"(dd[k][0]), "+v"(dd[k][1]));
    }
    uint32_t bits = 0;
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t d = (dd[k][j >> 2] >> (8 * (j & 3))) & 0xFF;
            const uint32_t L = sh.tb.len[d];
            bits += (FULL || static_cast<uint32_t>(k * 8 + j) < nv) ? L : 0u;
        }
    }
    sh.part_bits[wave][lane] = static_cast<uint16_t>(bits);
    __syncthreads();

    // 3. the group's length and mode, where this thread's part starts, and
    //    the lane offsets of the tile stream
    uint32_t gbits = 0, pre = 0;
#pragma unroll
    for (int w = 0; w < kEncWaves; ++w) {
        const uint32_t b = sh.part_bits[w][lane];
        pre += wave > static_cast<uint32_t>(w) ? b : 0u;
        gbits += b;
    }
    const bool raw_mode = ng > 0 && gbits >= 8 * ng;
    const uint32_t glen = raw_mode ? 8 * ng : gbits;
    if (raw_mode)
        pre = 8 * min(ng, first);
    uint32_t tile_bits;
    const uint32_t off = wave_excl_scan(glen, lane, &tile_bits);
    tile_bits = __builtin_amdgcn_readfirstlane(tile_bits);
    // at most 64 groups of 1024 bits: the bound keeps the stores of step 5
    // inside the tile's share of the chunk bound whatever the scan gives
    const uint32_t tile_words = min((tile_bits + 31) >> 5, static_cast<uint32_t>(kTileWordsMax));
    if (wave == 0)
        look_back_publish(status, x.item, x.t, tile_words, lane, epoch);

    // 4. code words into the LDS tile stream (zeroed at the kernel's start)
    if (__ballot(raw_mode) == 0)
        emit_quarter<FULL, false>(sh.stage, sh.tb, dd, emax, nv, raw_mode, off + pre);
    else
        emit_quarter<FULL, true>(sh.stage, sh.tb, dd, emax, nv, raw_mode, off + pre);
    __syncthreads();
    if (wave != 0)
        return;

    // 5. wave 0: the tile's offset, the stream, the index arrays
    const uint32_t toff_w = look_back_resolve(status, x.item, x.t, x.first, lane, epoch, x.src,
                                              x.n, sh.tb.len, spin_limit);
    // the inclusive prefix goes out at once: later tiles stop their walks
    // at it instead of summing further back
    if (x.t != 0 && lane == 0)
        __hip_atomic_store(&status[x.item * kStatusStride],
                           status_word(epoch, kFlagInc, toff_w + tile_words), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t toff = toff_w * 4, tile_bytes = tile_words * 4;
    // stores never leave the chunk's bound, whatever the offsets say (a
    // correct stream always fits; this only keeps a fault impossible)
    const bool fits = static_cast<uint64_t>(x.G.X) + toff + tile_bytes <= chunk_bound(x.n);
    // eight rows of LDS read ahead of their stores
    uint32_t* gstream = reinterpret_cast<uint32_t*>(x.dst + x.G.X + toff);
    for (uint32_t r0 = 0; r0 < tile_words; r0 += 8 * kLanes) {
        uint32_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            v[i] = sh.stage[min(r0 + i * kLanes + lane, static_cast<uint32_t>(kEncStage - 1))];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (fits && r0 + i * kLanes + lane < tile_words)
                gstream[r0 + i * kLanes + lane] = v[i];
    }
    write_tile_index(x, toff, tile_bytes, emax, glen, comp_sizes);
}

// Tiles that are partial (a chunk's last tile) or unaligned: the same
// steps with the members past the chunk's end masked off.
__device__ __forceinline__ void compress_tile_partial(
    TileCtx x, int64_t* __restrict__ comp_sizes, uint64_t* __restrict__ status,
    EncShared* sh, uint32_t epoch, uint32_t spin_limit)
{
    uint32_t dd[kQSteps][2];
    uint4 u[kQSteps];
    load_tile<false>(x, u);
    sh->part_max[x.wave][x.lane] = static_cast<uint16_t>(split_tile<false>(x, u, dd));
    __syncthreads();
    compress_tile_back<false>(x, dd, comp_sizes, status, *sh, epoch, spin_limit);
}

// The end of a launch for wave 0 of each workgroup.  Every workgroup but the
// last in grid order adds itself to one of 64 counters (spread over separate
// lines) and leaves; the last one waits, bounded, until the others have all
// counted (each counts after its last status access), then stores this
// launch's tag for the next launch and resets the counters.  No workgroup
// waits on the last one, so its wait ends.  When the tag wraps, or if the
// wait ran out, every status slot is cleared first (a slot cleared under a
// still-running look-back only sends it to the recomputation path).
__device__ inline void finish_launch(uint32_t* __restrict__ hdr, uint64_t* __restrict__ status,
                                     uint32_t status_slots, uint32_t epoch, uint32_t lane)
{
    uint32_t* counters = hdr + kHdrCounters;
    if (blockIdx.x != gridDim.x - 1) {
        if (lane == 0)
            __hip_atomic_fetch_add(&counters[(blockIdx.x % kCounters) * kCounterStride], 1u,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    bool done = false;
    for (uint32_t spin = 0; spin < kDoneSpinLimit && !done; ++spin) {
        const uint32_t c = __hip_atomic_load(&counters[lane * kCounterStride], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        done = wave_sum(c) >= gridDim.x - 1;
        if (!done)
            __builtin_amdgcn_s_sleep(2);
    }
    if (epoch == 0xFFFFFFFFu || !done) {
        for (uint32_t i = lane; i < status_slots; i += kLanes)
            __hip_atomic_store(&status[static_cast<size_t>(i) * kStatusStride], 0ull,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __hip_atomic_store(&counters[lane * kCounterStride], 0u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0)
        __hip_atomic_store(&hdr[kHdrEpoch], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// This launch's tag: one more than the last launch's, stored in the
// workspace (0 is never a tag, so a zeroed workspace holds no valid word).
// It is read with a scalar load through the constant address space: the
// scalar cache is invalidated at every kernel dispatch, and the word changes
// only at the very end of a launch, after every workgroup has read it.  (A
// device-coherent vector load of this one word by every workgroup cost
// about 15 % of the kernel's time.)
typedef const __attribute__((address_space(4))) uint32_t* ConstU32;

__device__ inline uint32_t launch_epoch(const uint32_t* __restrict__ hdr)
{
    const uint32_t e = ((ConstU32)hdr)[kHdrEpoch] + 1u;
    return e == 0 ? 1u : e;
}

// One tile per workgroup, in grid order (chunk by chunk, so neighbouring
// workgroups stream neighbouring bytes).  The look-back never waits without
// bound, so the order needs no assumption about dispatch order.  The
// launch's tag (epoch) is one more than the one stored in the workspace.
template <class Tab>
__device__ __forceinline__ void compress_body(const Tab& tab, const uint16_t* __restrict__ in,
                                              uint8_t* __restrict__ out,
                                              int64_t* __restrict__ comp_sizes,
                                              uint8_t* __restrict__ ws, uint32_t status_slots)
{
    __shared__ __align__(16) EncShared sh;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kLanes - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kLanes);   // uniform: scalar
    uint32_t* hdr = reinterpret_cast<uint32_t*>(ws);
    uint64_t* status = reinterpret_cast<uint64_t*>(ws + kWsHeader);
    const uint32_t item = blockIdx.x;
    if (item >= tab.nitems) {      // device-split grids are sized for the bound
        if (wave == 0)
            finish_launch(hdr, status, status_slots, launch_epoch(hdr), lane);
        return;
    }
    const TileCtx x = tile_ctx(tab, item, in, out, lane, wave);

    // a full tile issues its loads first, so that their latency covers the
    // table set-up below; the launch's tag is read after them and first
    // needed when the tile publishes its size
    const bool full = tile_full(x);
    uint4 v[kQSteps];
    if (full)
        load_tile<true>(x, v);
    const uint32_t epoch = launch_epoch(hdr);
    constexpr uint32_t kTbWords = sizeof(EncTables) / 16;
#pragma unroll
    for (uint32_t i = tid; i < kTbWords; i += kEncBlock)
        reinterpret_cast<uint4*>(&sh.tb)[i] = reinterpret_cast<const uint4*>(&c_enc)[i];
    for (uint32_t i = tid * 4; i < static_cast<uint32_t>(kEncStage); i += kEncBlock * 4)
        *reinterpret_cast<uint4*>(&sh.stage[i]) = make_uint4(0, 0, 0, 0);

    if (x.n == 0) {
        if (tid < 8)
            reinterpret_cast<uint32_t*>(x.dst)[tid] = header_word(tid, 0, 32);
        if (tid == 0)
            comp_sizes[x.c] = 32;
    } else if (full) {
        uint32_t dd[kQSteps][2];
        sh.part_max[wave][lane] = static_cast<uint16_t>(split_tile<true>(x, v, dd));
        __syncthreads();
        compress_tile_back<true>(x, dd, comp_sizes, status, sh, epoch, tab.spin_limit);
    } else {
        compress_tile_partial(x, comp_sizes, status, &sh, epoch, tab.spin_limit);
    }
    if (wave == 0)
        finish_launch(hdr, status, status_slots, epoch, lane);
}

__global__ __launch_bounds__(kEncBlock, kMinWavesEnc)
void zc_compress_kernel(const uint16_t* __restrict__ in, uint8_t* __restrict__ out,
                        int64_t* __restrict__ comp_sizes, uint8_t* __restrict__ ws,
                        uint32_t status_slots, ChunkTable tab)
{
    compress_body(tab, in, out, comp_sizes, ws, status_slots);
}

// The same with the chunk table in device memory (built on the device from
// device-resident counts); the grid is an upper bound on the tile count and
// workgroups past the table's tiles only take part in the launch's end.
__global__ __launch_bounds__(kEncBlock, kMinWavesEnc)
void zc_compress_dev_kernel(const uint16_t* __restrict__ in, uint8_t* __restrict__ out,
                            int64_t* __restrict__ comp_sizes, uint8_t* __restrict__ ws,
                            uint32_t status_slots, const ChunkTable* __restrict__ tab)
{
    compress_body(*tab, in, out, comp_sizes, ws, status_slots);
}

// ------------------------------------------------------------ decompress

// Records one failed check (the first to arrive wins).  Callers pass a
// wave-uniform reason; only one lane touches the status word, and not at all
// once a failure is recorded, so a wholly corrupt buffer cannot flood it.
__device__ inline void report(int32_t* status, int reason, int c)
{
    if (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
        atomicCAS(status, 0, (reason << 24) | (c & 0xFFFFFF));
}

// 64 stream bits from bit `pos` of a tile stream staged in LDS (word index
// clamped to `cap`, where the buffer holds zero guard words).
struct LdsWindow {
    const uint32_t* s;
    uint32_t cap;
    __device__ inline uint64_t operator()(uint32_t pos) const
    {
        const uint32_t wi = min(pos >> 5, cap);
        const uint32_t w0 = s[wi], w1 = s[wi + 1], w2 = s[wi + 2];
        const uint32_t sh = pos & 31;
        const uint32_t hi = hi32(((static_cast<uint64_t>(w0) << 32) | w1) << sh);
        const uint32_t lo = hi32(((static_cast<uint64_t>(w1) << 32) | w2) << sh);
        return (static_cast<uint64_t>(hi) << 32) | lo;
    }
};

// The same from the tile stream in global memory (words past `nwords` read
// as zero); used for tile streams longer than the LDS buffer.
struct GlobalWindow {
    const uint32_t* g;
    uint32_t nwords;
    __device__ inline uint64_t operator()(uint32_t pos) const
    {
        const uint32_t wi = pos >> 5;
        const uint32_t w0 = wi < nwords ? g[wi] : 0u;
        const uint32_t w1 = wi + 1 < nwords ? g[wi + 1] : 0u;
        const uint32_t w2 = wi + 2 < nwords ? g[wi + 2] : 0u;
        const uint32_t sh = pos & 31;
        const uint32_t hi = hi32(((static_cast<uint64_t>(w0) << 32) | w1) << sh);
        const uint32_t lo = hi32(((static_cast<uint64_t>(w1) << 32) | w2) << sh);
        return (static_cast<uint64_t>(hi) << 32) | lo;
    }
};

// Per-lane decoding parameters.  Coded groups look the first 11 stream bits
// up in (symbol << 4 | length) byte entries (every code word but the four
// longest fits); raw groups look their 8 bits up in entries that hold 255 - e
// and always advance by 8.
struct LaneCode {
    uint32_t ish;        // the table index is the window's top 32 - ish bits
    uint32_t base;       // LDS byte index of the lane's table
    uint32_t sym_sh;     // entry >> sym_sh = symbol
    uint32_t smask;      // (entry & smask) | sor = bits consumed
    uint32_t sor;
    uint32_t lmark;      // entry value that means "longer code word"
    uint32_t emax_eff;   // e = emax_eff - symbol
};

// Symbol and length of the code word at the top of a window.  Code words
// longer than the first level take the second: an escape then yields
// d = E_max - e as its symbol (so that E_max - symbol is e) and lowers
// esc_min, since a valid escape has d >= 16.
__device__ inline void decode_sym(const uint8_t* __restrict__ s_lut8,
                                  const uint16_t* __restrict__ s_tail, uint32_t top,
                                  const LaneCode& q, uint32_t emax, bool valid,
                                  int32_t& esc_min, uint32_t& sym, uint32_t& sh)
{
    const uint32_t ent = s_lut8[(top >> q.ish) + q.base];
    sym = ent >> q.sym_sh;
    sh = (ent & q.smask) | q.sor;
    if (ent == q.lmark) {
        const uint32_t t2 = s_tail[(top >> (32 - kLutBits - kTailBits)) & ((1u << kTailBits) - 1)];
        sym = t2 >> 8;
        sh = t2 & 0xFF;
        if (sym == static_cast<uint32_t>(kEsc)) {
            const uint32_t e = (top >> (32 - kEscLen - 8)) & 0xFF;
            const int32_t d = static_cast<int32_t>(emax) - static_cast<int32_t>(e);
            if (valid)
                esc_min = min(esc_min, d);
            sym = static_cast<uint32_t>(d);
            sh = kEscLen + 8;
        }
    }
}

// Joins 8 exponents with their sign+mantissa bytes and stores them.
template <bool FULL>
__device__ inline void put_values(uint16_t* __restrict__ dst, const uint8_t* __restrict__ rsrc,
                                  uint32_t n, uint32_t i0, uint2 r, const uint32_t (&e8)[8],
                                  bool vec_out)
{
    // in a partial tile, r holds the segment's sign+mantissa bytes when its
    // 8 values lie wholly inside the chunk; they take the vector form when
    // the output is 16-byte aligned, and the ragged end goes value by value
    const bool whole = FULL || i0 + 8 <= n;
    const bool vec = FULL ? vec_out
                          : (whole && (reinterpret_cast<uintptr_t>(dst + i0) & 15) == 0);
    if (vec) {
        uint4 o;
        o.x = (__builtin_amdgcn_perm(r.x, r.x, 0x01010000u) & 0x807F807Fu) | (e8[0] << 7) | (e8[1] << 23);
        o.y = (__builtin_amdgcn_perm(r.x, r.x, 0x03030202u) & 0x807F807Fu) | (e8[2] << 7) | (e8[3] << 23);
        o.z = (__builtin_amdgcn_perm(r.y, r.y, 0x01010000u) & 0x807F807Fu) | (e8[4] << 7) | (e8[5] << 23);
        o.w = (__builtin_amdgcn_perm(r.y, r.y, 0x03030202u) & 0x807F807Fu) | (e8[6] << 7) | (e8[7] << 23);
        st_nt4(dst + i0, o);
    } else if (whole) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t b = ((j < 4 ? r.x : r.y) >> (8 * (j & 3))) & 0xFFu;
            dst[i0 + j] = static_cast<uint16_t>(((b & 0x80u) << 8) | ((e8[j] & 0xFF) << 7) | (b & 0x7Fu));
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (i0 + j < n) {
                const uint32_t b = rsrc[i0 + j];
                dst[i0 + j] = static_cast<uint16_t>(((b & 0x80u) << 8) | ((e8[j] & 0xFF) << 7) | (b & 0x7Fu));
            }
        }
    }
}

struct DecState {
    uint32_t pos;        // bit position in the tile stream
    uint32_t seen_max;   // largest decoded exponent
    uint32_t raw_coded;  // raw groups: coded length their values would take
    int32_t esc_min;     // smallest E_max - e over escapes
};

// Decodes the 128 members of this lane's group from a window source and
// writes the values.  MIXED: the wave has raw groups (otherwise the lookup
// parameters are constants).
template <bool FULL, int kSym, bool MIXED, class Win>
__device__ __forceinline__ void decode_group(const Win& win, const uint8_t* __restrict__ s_lut8,
                                    const uint16_t* __restrict__ s_tail,
                                    const uint8_t* __restrict__ s_len, const uint8_t* __restrict__ rsrc,
                                    uint16_t* __restrict__ dst, uint32_t n, uint32_t base,
                                    uint32_t lane, uint32_t ng, uint32_t emax, bool raw_mode,
                                    bool vec_out, DecState& st)
{
    const bool raw = MIXED && raw_mode;
    LaneCode q;
    q.ish = raw ? 24u : static_cast<uint32_t>(32 - kLutBits);
    q.base = raw ? static_cast<uint32_t>(kLutRaw) : 0u;
    q.sym_sh = raw ? 0u : 4u;
    q.smask = raw ? 0u : 15u;
    q.sor = raw ? 8u : 0u;
    q.lmark = raw ? 256u : 0u;
    q.emax_eff = raw ? 255u : emax;

    // Sign+mantissa bytes, prefetched kRing steps ahead into a ring that the
    // unrolled inner loop indexes statically: each slot is reloaded right
    // after its last use, so no register is copied while its load is in
    // flight and each wait leaves the younger loads and stores outstanding.
    constexpr int kRing = 1;
    static_assert(kSteps % kRing == 0, "whole rounds of the prefetch ring");
    // (in a partial tile, only segments wholly inside the chunk are read)
    const uint2* rsrc2 = reinterpret_cast<const uint2*>(rsrc + base) + lane;
    auto raw_at = [&](int k) {
        return (FULL || base + k * 512 + lane * 8 + 8 <= n) ? ld_nt2(rsrc2 + k * 64)
                                                            : make_uint2(0, 0);
    };
    uint2 ring[kRing];
#pragma unroll
    for (int j = 0; j < kRing; ++j)
        ring[j] = raw_at(j);
#pragma unroll 1
    for (int k0 = 0; k0 < kSteps; k0 += kRing)
#pragma unroll
    for (int kj = 0; kj < kRing; ++kj) {
        const int k = k0 + kj;
        // kSym symbols per 64-bit window; a lane whose code words overrun
        // the window (several escapes) decodes them again one at a time
        uint32_t e8[8];
#pragma unroll
        for (int h = 0; h < 8 / kSym; ++h) {
            const uint32_t pos0 = st.pos;
            uint64_t W = win(pos0);
            uint32_t used = 0;
            int32_t esc_w = 255;
#pragma unroll
            for (int jj = 0; jj < kSym; ++jj) {
                const int j = h * kSym + jj;
                const bool valid = FULL || static_cast<uint32_t>(k * 8 + j) < ng;
                uint32_t sym, sh;
                decode_sym(s_lut8, s_tail, hi32(W), q, emax, valid, esc_w, sym, sh);
                if (!FULL && !valid)
                    sh = 0;
                e8[j] = q.emax_eff - sym;
                W <<= sh;
                used += sh;
            }
            const bool slow = used > 64;
            if (!slow)
                st.esc_min = min(st.esc_min, esc_w);
            if (__ballot(slow)) {
                if (slow) {
                    uint32_t p = pos0;
                    int32_t esc_h = 255;
#pragma unroll
                    for (int jj = 0; jj < kSym; ++jj) {
                        const int j = h * kSym + jj;
                        const bool valid = FULL || static_cast<uint32_t>(k * 8 + j) < ng;
                        uint32_t sym, sh;
                        decode_sym(s_lut8, s_tail, hi32(win(p)), q, emax, valid, esc_h, sym, sh);
                        if (!FULL && !valid)
                            sh = 0;
                        e8[j] = q.emax_eff - sym;
                        p += sh;
                    }
                    used = p - pos0;
                    st.esc_min = min(st.esc_min, esc_h);
                }
            }
            st.pos = pos0 + used;
        }
        if (FULL) {
            st.seen_max = max(st.seen_max, max3(e8[0], e8[1], e8[2]));
            st.seen_max = max(st.seen_max, max3(e8[3], e8[4], e8[5]));
            st.seen_max = max(st.seen_max, max(e8[6], e8[7]));
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (static_cast<uint32_t>(k * 8 + j) < ng)
                    st.seen_max = max(st.seen_max, e8[j]);
        }
        if (MIXED) {
            // a raw group must not have been codable in fewer bits
            if (raw_mode) {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (FULL || static_cast<uint32_t>(k * 8 + j) < ng)
                        st.raw_coded += s_len[(emax - e8[j]) & 0xFF];
            }
        }
        put_values<FULL>(dst, rsrc, n, base + k * 512 + lane * 8, ring[kj], e8, vec_out);
        // the last round reloads the last row (in bounds, unused)
        ring[kj] = raw_at(min(k + kRing, kSteps - 1));
    }
}

// The symbols of step k of this lane's group, as in decode_group's loop: the
// 8 exponents in e8, and the bit position, the largest exponent and (raw
// groups) the coded length advanced in st.  The fused decode + sum below
// takes its steps from here; decode_group keeps its own copy of the loop,
// whose code generation the plain decompress is tuned on.
template <bool FULL, int kSym, bool MIXED, class Win>
__device__ __forceinline__ void decode_step(const Win& win, const uint8_t* __restrict__ s_lut8,
                                            const uint16_t* __restrict__ s_tail,
                                            const uint8_t* __restrict__ s_len, const LaneCode& q,
                                            int k, uint32_t ng, uint32_t emax, bool raw_mode,
                                            DecState& st, uint32_t (&e8)[8])
{
    // kSym symbols per 64-bit window; a lane whose code words overrun
    // the window (several escapes) decodes them again one at a time
#pragma unroll
    for (int h = 0; h < 8 / kSym; ++h) {
        const uint32_t pos0 = st.pos;
        uint64_t W = win(pos0);
        uint32_t used = 0;
        int32_t esc_w = 255;
#pragma unroll
        for (int jj = 0; jj < kSym; ++jj) {
            const int j = h * kSym + jj;
            const bool valid = FULL || static_cast<uint32_t>(k * 8 + j) < ng;
            uint32_t sym, sh;
            decode_sym(s_lut8, s_tail, hi32(W), q, emax, valid, esc_w, sym, sh);
            if (!FULL && !valid)
                sh = 0;
            e8[j] = q.emax_eff - sym;
            W <<= sh;
            used += sh;
        }
        const bool slow = used > 64;
        if (!slow)
            st.esc_min = min(st.esc_min, esc_w);
        if (__ballot(slow)) {
            if (slow) {
                uint32_t p = pos0;
                int32_t esc_h = 255;
#pragma unroll
                for (int jj = 0; jj < kSym; ++jj) {
                    const int j = h * kSym + jj;
                    const bool valid = FULL || static_cast<uint32_t>(k * 8 + j) < ng;
                    uint32_t sym, sh;
                    decode_sym(s_lut8, s_tail, hi32(win(p)), q, emax, valid, esc_h, sym, sh);
                    if (!FULL && !valid)
                        sh = 0;
                    e8[j] = q.emax_eff - sym;
                    p += sh;
                }
                used = p - pos0;
                st.esc_min = min(st.esc_min, esc_h);
            }
        }
        st.pos = pos0 + used;
    }
    if (FULL) {
        st.seen_max = max(st.seen_max, max3(e8[0], e8[1], e8[2]));
        st.seen_max = max(st.seen_max, max3(e8[3], e8[4], e8[5]));
        st.seen_max = max(st.seen_max, max(e8[6], e8[7]));
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (static_cast<uint32_t>(k * 8 + j) < ng)
                st.seen_max = max(st.seen_max, e8[j]);
    }
    if (MIXED) {
        // a raw group must not have been codable in fewer bits
        if (raw_mode) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (FULL || static_cast<uint32_t>(k * 8 + j) < ng)
                    st.raw_coded += s_len[(emax - e8[j]) & 0xFF];
        }
    }
}

// Copies `words` (1..1024) tile-stream words from global memory into LDS.
// Every load of a lane is issued before the first is written, so the copy
// costs one memory round trip; rows past the end are skipped as a whole and
// the last row's addresses are clamped to the last word.
__device__ inline void stage_words(uint32_t* __restrict__ s, const uint32_t* __restrict__ g,
                                   uint32_t words, uint32_t lane)
{
    constexpr int kRows = kStageWords / kLanes;
    uint32_t v[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i)
        if (static_cast<uint32_t>(i * kLanes) < words)
            v[i] = ld_nt1(g + min(lane + i * kLanes, words - 1));
#pragma unroll
    for (int i = 0; i < kRows; ++i)
        if (lane + i * kLanes < words)
            s[lane + i * kLanes] = v[i];
}

// A full tile whose 64 groups are all raw: every group stream is 1024 bits
// of plain exponents at bit 1024 * lane.  The 8 KiB tile stream is staged in
// two halves of 32 groups, each decoded by all 64 lanes, two per group.
__device__ inline void decode_all_raw(const uint32_t* __restrict__ gstream,
                                      uint32_t* __restrict__ s, const uint8_t* __restrict__ s_len,
                                      const uint8_t* __restrict__ rsrc, uint16_t* __restrict__ dst,
                                      uint32_t n, uint32_t base, uint32_t lane, uint32_t emax,
                                      bool vec_out, DecState& st)
{
    uint32_t seen = 0, coded = 0;
#pragma unroll 1
    for (int h = 0; h < 2; ++h) {
        wave_lds_sync();
        stage_words(s, gstream + h * kStageWords, kStageWords, lane);
        wave_lds_sync();
        // lane l takes group 32 h + l % 32, steps 8 (l / 32) .. 8 (l / 32) + 7:
        // a raw group's members sit at fixed bit positions, so its two lanes
        // need nothing from each other until the checks
        const uint32_t g = 32u * static_cast<uint32_t>(h) + (lane & 31);
        const uint32_t k0 = (lane >> 5) * 8;
        const uint32_t eg = __shfl(emax, g);
        const uint32_t* mine = s + (lane & 31) * 32 + 2 * k0;
        const uint2* rsrc2 = reinterpret_cast<const uint2*>(rsrc + base) + g;
        uint32_t sm = 0, rc = 0;
#pragma unroll 2
        for (int k = 0; k < kSteps / 2; ++k) {
            const uint2 ew = *reinterpret_cast<const uint2*>(mine + 2 * k);
            const uint32_t e4a = __builtin_amdgcn_perm(ew.x, ew.x, 0x00010203u);
            const uint32_t e4b = __builtin_amdgcn_perm(ew.y, ew.y, 0x00010203u);
            uint32_t e8[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                e8[j] = (e4a >> (8 * j)) & 0xFF;
                e8[4 + j] = (e4b >> (8 * j)) & 0xFF;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sm = max(sm, e8[j]);
                rc += s_len[(eg - e8[j]) & 0xFF];
            }
            const uint32_t ks = k0 + static_cast<uint32_t>(k);
            put_values<true>(dst, rsrc, n, base + ks * 512 + g * 8, ld2(rsrc2 + ks * 64), e8, vec_out);
        }
        // the group's two halves meet; lane l keeps the totals of group l
        const uint32_t sm2 = max(sm, static_cast<uint32_t>(__shfl_xor(sm, 32)));
        const uint32_t rc2 = rc + static_cast<uint32_t>(__shfl_xor(rc, 32));
        if ((lane >> 5) == static_cast<uint32_t>(h)) {
            seen = sm2;
            coded = rc2;
        }
    }
    st.seen_max = max(st.seen_max, seen);
    st.raw_coded += coded;
    st.pos += 1024;
}

// A tile's header word, offsets and group metadata, loaded together (only
// once the chunk's readable bytes are known to hold its index arrays).
struct TileMeta {
    uint32_t hw, toff, tnext, emax, glen;
};

__device__ inline TileMeta load_meta(const uint8_t* __restrict__ src, const Geom& G, uint32_t t,
                                     uint32_t lane)
{
    TileMeta m;
    m.hw = lane < 8 ? reinterpret_cast<const uint32_t*>(src)[lane] : 0u;
    const uint32_t* toffs = reinterpret_cast<const uint32_t*>(src + 32);
    m.toff = toffs[t];
    m.tnext = (t + 1 < G.T) ? toffs[t + 1] : 0u;
    m.emax = src[32 + 4ull * G.T + 64ull * t + lane];
    m.glen = *reinterpret_cast<const uint16_t*>(src + 32 + 68ull * G.T + 2ull * (64ull * t + lane));
    return m;
}

template <bool FULL>
__device__ __forceinline__ void decompress_tile(const uint8_t* __restrict__ src, uint16_t* __restrict__ dst,
                                int32_t* __restrict__ status, int c, uint32_t n, uint32_t t,
                                uint64_t bavail, uint32_t lane, uint32_t* __restrict__ s,
                                const uint8_t* __restrict__ s_lut8,
                                const uint16_t* __restrict__ s_tail,
                                const uint8_t* __restrict__ s_len, const TileMeta& meta)
{
    const Geom G = geometry(n);
    const uint32_t base = t * kTile;
    const uint32_t rem = min(n - base, static_cast<uint32_t>(kTile));
    const uint32_t ng = FULL ? 128u : group_members(rem, lane);
    if (G.X > bavail) {          // the index arrays and raw bytes cannot fit
        if (lane == 0)
            report(status, ZC_REASON_SIZE, c);
        return;
    }
    const uint32_t hw = meta.hw, toff = meta.toff, tnext = meta.tnext, emax = meta.emax,
                   glen = meta.glen;

    const uint32_t h0 = __shfl(hw, 0), h1 = __shfl(hw, 1), h2 = __shfl(hw, 2),
                   h3 = __shfl(hw, 3), h4 = __shfl(hw, 4), h5 = __shfl(hw, 5),
                   h6 = __shfl(hw, 6), h7 = __shfl(hw, 7);
    if (h0 != kMagic || h1 != kVerTable || h2 != 0 || h3 != 0 || h4 != n || h5 != 0) {
        if (lane == 0)
            report(status, ZC_REASON_HEADER, c);
        return;
    }
    const uint64_t comp = h6 | (static_cast<uint64_t>(h7) << 32);
    if (comp < G.X || comp > bavail || comp > chunk_bound(n)) {
        if (lane == 0)
            report(status, ZC_REASON_SIZE, c);
        return;
    }
    const uint64_t next = (t + 1 < G.T) ? tnext : comp - G.X;
    if ((t == 0 && toff != 0) || toff > next || next > comp - G.X) {
        if (lane == 0)
            report(status, ZC_REASON_TILE, c);
        return;
    }
    const uint32_t tile_bytes = static_cast<uint32_t>(next - toff);
    if (__ballot(glen > 8 * ng || (ng == 0 && emax != 0))) {
        if (lane == 0)
            report(status, ZC_REASON_GROUP, c);
        return;
    }
    uint32_t tile_bits;
    const uint32_t off = wave_excl_scan(glen, lane, &tile_bits);
    const uint32_t tile_words = (tile_bits + 31) >> 5;
    if (tile_bytes != 4 * tile_words) {
        if (lane == 0)
            report(status, ZC_REASON_TILE, c);
        return;
    }

    const uint32_t* gstream = reinterpret_cast<const uint32_t*>(src + G.X + toff);
    int err = 0;
    if (t == 0) {
        const uint64_t g1 = 32 + 196ull * G.T;
        if (g1 + lane < G.R && src[g1 + lane] != 0)
            err = ZC_REASON_GAP;
    }
    if (t == G.T - 1) {
        if (G.R + n + lane < G.X && src[G.R + n + lane] != 0)
            err = ZC_REASON_GAP;
    }
    if ((tile_bits & 31) && lane == 0) {
        const uint32_t last = gstream[tile_words - 1];
        if (last & ((1u << (32 - (tile_bits & 31))) - 1))
            err = ZC_REASON_PADDING;
    }

    const bool raw_mode = ng > 0 && glen == 8 * ng;
    const uint64_t raw_lanes = __ballot(raw_mode);
    // full tiles are only taken with 16-byte aligned output (decompress_body)
    const bool vec_out = FULL;
    const uint8_t* rsrc = src + G.R;
    DecState st;
    st.pos = off;
    st.seen_max = 0;
    st.raw_coded = 0;
    st.esc_min = 255;
    if (FULL && raw_lanes == ~0ull) {
        decode_all_raw(gstream, s, s_len, rsrc, dst, n, base, lane, emax, vec_out, st);
    } else if (tile_words <= static_cast<uint32_t>(kStageWords)) {
        stage_words(s, gstream, tile_words, lane);
        if (lane < 4)
            s[tile_words + lane] = 0;
        wave_lds_sync();
        // 8 symbols per window unless a coded group of the tile averages
        // more than 5 bits per value (its windows would often overrun)
        const LdsWindow lw{s, tile_words};
        if (__ballot(!raw_mode && glen > 5 * ng) == 0) {
            if (raw_lanes == 0)
                decode_group<FULL, 8, false>(lw, s_lut8, s_tail, s_len, rsrc, dst, n, base, lane,
                                             ng, emax, raw_mode, vec_out, st);
            else
                decode_group<FULL, 8, true>(lw, s_lut8, s_tail, s_len, rsrc, dst, n, base, lane,
                                            ng, emax, raw_mode, vec_out, st);
        } else {
            if (raw_lanes == 0)
                decode_group<FULL, 4, false>(lw, s_lut8, s_tail, s_len, rsrc, dst, n, base, lane,
                                             ng, emax, raw_mode, vec_out, st);
            else
                decode_group<FULL, 4, true>(lw, s_lut8, s_tail, s_len, rsrc, dst, n, base, lane,
                                            ng, emax, raw_mode, vec_out, st);
        }
    } else {
        decode_group<FULL, 4, true>(GlobalWindow{gstream, tile_words}, s_lut8, s_tail, s_len, rsrc,
                                    dst, n, base, lane, ng, emax, raw_mode, vec_out, st);
    }
    if (err == 0 && ng > 0) {
        if (st.pos != off + glen)
            err = ZC_REASON_LENGTH;
        else if (st.seen_max != emax)
            err = ZC_REASON_EMAX;
        else if (!raw_mode && st.esc_min < kEsc)
            err = ZC_REASON_ESCAPE;
        else if (raw_mode && st.raw_coded < 8 * ng)
            err = ZC_REASON_RAWMODE;
    }
    // one report per wave: the lowest failing lane's reason
    const uint64_t bad = __ballot(err != 0);
    if (bad) {
        const int first = __ffsll(static_cast<unsigned long long>(bad)) - 1;
        const int reason = __shfl(err, first);
        if (lane == 0)
            report(status, reason, c);
    }
}

// A chunk's last, partial tile, or any tile of an output that is not 16-byte
// aligned: the same steps with the values past the chunk's end masked off.
__device__ __forceinline__ void decompress_tile_partial(
    const uint8_t* __restrict__ src, uint16_t* __restrict__ dst, int32_t* __restrict__ status,
    int c, uint32_t n, uint32_t t, uint64_t bavail, uint32_t lane, uint32_t* __restrict__ s,
    const uint8_t* __restrict__ s_lut8, const uint16_t* __restrict__ s_tail,
    const uint8_t* __restrict__ s_len, TileMeta meta)
{
    decompress_tile<false>(src, dst, status, c, n, t, bavail, lane, s, s_lut8, s_tail, s_len, meta);
}

__device__ __forceinline__ void decompress_body(const uint8_t* __restrict__ in,
                                                uint16_t* __restrict__ out,
                                                int32_t* __restrict__ status,
                                                const ChunkTable& tab)
{
    __shared__ __align__(16) uint32_t s_stage[kWaves][kStageAlloc];
    __shared__ __align__(16) uint8_t s_lut8[kLutRaw + 256];
    __shared__ uint16_t s_tail[1 << kTailBits];
    __shared__ uint8_t s_len[256];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kLanes - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kLanes);
    // The first-level table is the only one read from memory: its load is
    // issued first and written to LDS just before the barrier, after this
    // wave's chunk lookup (scalar loads) and tile metadata loads.
    uint32_t lut_part[kLutPer];
#pragma unroll
    for (int i = 0; i < kLutPer; ++i)
        if (kLutWords % kBlock == 0 || tid + i * kBlock < static_cast<uint32_t>(kLutWords))
            lut_part[i] = reinterpret_cast<const uint32_t*>(c_lut)[tid + i * kBlock];
    // raw groups: 8 bits b decode to 255 - b
    s_lut8[kLutRaw + tid] = static_cast<uint8_t>(255u - tid);
    if (tid < (1u << kTailBits))
        s_tail[tid] = static_cast<uint16_t>(tail_of(tid));
    {
        const uint32_t s = tid < static_cast<uint32_t>(kEsc) ? tid : static_cast<uint32_t>(kEsc);
        s_len[tid] = static_cast<uint8_t>(len_of(s) + (s == static_cast<uint32_t>(kEsc) ? 8 : 0));
    }
    const uint32_t item = blockIdx.x * kWaves + wave;
    const bool live = item < tab.nitems;
    int c = 0;
    uint32_t n = 0, t = 0;
    TileMeta meta = {0, 0, 0, 0, 0};
    if (live) {
        c = find_chunk(tab, item);
        n = tab.n[c];
        t = tab.tile0 + item - tab.item_begin[c];
        const Geom G = geometry(n);
        if (n != 0 && G.X <= tab.bavail[c])
            meta = load_meta(in + tab.boff[c], G, t, lane);
    }
#pragma unroll
    for (int i = 0; i < kLutPer; ++i)
        if (kLutWords % kBlock == 0 || tid + i * kBlock < static_cast<uint32_t>(kLutWords))
            reinterpret_cast<uint32_t*>(s_lut8)[tid + i * kBlock] = lut_part[i];
    __syncthreads();

    if (!live)
        return;
    const int cid = tab.chunk_base + c;     // the chunk's index in the call, for reports
    if (n == 0) {
        // a header-only stream
        const uint8_t* src = in + tab.boff[c];
        const uint32_t hw = lane < 8 ? reinterpret_cast<const uint32_t*>(src)[lane] : 0u;
        if (__ballot(lane < 8 && hw != header_word(lane, 0, 32)) && lane == 0)
            report(status, ZC_REASON_HEADER, cid);
        return;
    }
    const uint8_t* src = in + tab.boff[c];
    uint16_t* dst = out + tab.voff[c];
    const uint32_t rem = min(n - t * kTile, static_cast<uint32_t>(kTile));
    if (rem == kTile && (reinterpret_cast<uintptr_t>(dst) & 15) == 0)
        decompress_tile<true>(src, dst, status, cid, n, t, tab.bavail[c], lane, s_stage[wave],
                              s_lut8, s_tail, s_len, meta);
    else
        decompress_tile_partial(src, dst, status, cid, n, t, tab.bavail[c], lane, s_stage[wave],
                                s_lut8, s_tail, s_len, meta);
}

__global__ __launch_bounds__(kBlock, kMinWavesDec)
void zc_decompress_kernel(const uint8_t* __restrict__ in, uint16_t* __restrict__ out,
                          int32_t* __restrict__ status, ChunkTable tab)
{
    decompress_body(in, out, status, tab);
}

// The same with the chunk table in device memory; waves past the table's
// tiles pass the table barrier and return.
__global__ __launch_bounds__(kBlock, kMinWavesDec)
void zc_decompress_dev_kernel(const uint8_t* __restrict__ in, uint16_t* __restrict__ out,
                              int32_t* __restrict__ status, const ChunkTable* __restrict__ tab)
{
    decompress_body(in, out, status, *tab);
}

// ------------------------------------------------------------ pipeline link

// Slots of the chunks of one pipeline group, relative to the group's first.
struct LinkTable {
    uint64_t slot[kMaxChunks];     // byte offset of the chunk's slot
    uint64_t bound[kMaxChunks];    // slot size: nothing past it is read or written
};

// The stand-in for the link of a pipelined exchange on one GPU: copies each
// chunk's compressed stream (comp_sizes[c] bytes, read on the device, capped
// at the slot size) from the sender's slot to the same slot of the receiver.
// Grid: x = blocks per chunk, y = chunk.
__global__ __launch_bounds__(kBlock)
void zc_link_copy_kernel(const uint8_t* __restrict__ send, uint8_t* __restrict__ recv,
                         const int64_t* __restrict__ comp_sizes, LinkTable tab)
{
    const uint32_t c = blockIdx.y;
    const int64_t sz = comp_sizes[c];
    const uint64_t bytes = sz < 0 ? 0 : min(static_cast<uint64_t>(sz), tab.bound[c]);
    const uint8_t* s = send + tab.slot[c];
    uint8_t* d = recv + tab.slot[c];
    const uint64_t quads = bytes / 16;
    const uint64_t step = static_cast<uint64_t>(gridDim.x) * kBlock;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kBlock + threadIdx.x; i < quads; i += step)
        st_nt4(reinterpret_cast<uint4*>(d) + i, ld_nt4(reinterpret_cast<const uint4*>(s) + i));
    if (blockIdx.x == 0)
        for (uint64_t b = quads * 16 + threadIdx.x; b < bytes; b += kBlock)
            d[b] = s[b];
}

// ------------------------------------------------------------ reduce

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline void add8(float (&acc)[8], const uint4 v)
{
    acc[0] = acc[0] + bf16_lo(v.x);
    acc[1] = acc[1] + bf16_hi(v.x);
    acc[2] = acc[2] + bf16_lo(v.y);
    acc[3] = acc[3] + bf16_hi(v.y);
    acc[4] = acc[4] + bf16_lo(v.z);
    acc[5] = acc[5] + bf16_hi(v.z);
    acc[6] = acc[6] + bf16_lo(v.w);
    acc[7] = acc[7] + bf16_hi(v.w);
}

// fp32 to bf16, round to nearest with ties to even: adding 0x7FFF plus the
// kept part's last bit carries into the kept half exactly when the dropped
// half is above one half, or equal to it with an odd kept part (overflow
// carries into the exponent and gives infinity).  NaN gives 0x7FC0.
__device__ inline uint32_t f32_to_bf16_rne(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Receive side of a reduce-scatter (pith.science, Figure 5: zipccl
// ReduceScatter): num_chunks decoded contributions of n bf16 values each
// (contribution c at x + c stride) summed element by element in fp32, in
// chunk order, from +0; BF16OUT rounds each sum once to bf16 (to nearest
// even).  Each thread owns 8 consecutive elements; rows are read with
// 16-byte nontemporal loads, 8 contributions in flight at a time, and the
// sums are added strictly in chunk order.
template <bool BF16OUT>
__device__ __forceinline__ void reduce_body(const uint16_t* __restrict__ x, uint64_t n,
                                            uint64_t stride, int32_t num_chunks,
                                            void* __restrict__ out, uint32_t block)
{
    const uint64_t i0 = (static_cast<uint64_t>(block) * kBlock + threadIdx.x) * 8;
    if (i0 >= n)
        return;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc[j] = 0.0f;
    if (i0 + 8 <= n && (stride & 7) == 0) {
        const uint16_t* p = x + i0;
        int32_t c = 0;
        for (; c + 8 <= num_chunks; c += 8) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = ld_nt4(p + static_cast<uint64_t>(c + u) * stride);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                add8(acc, v[u]);
        }
        for (; c < num_chunks; ++c)
            add8(acc, ld_nt4(p + static_cast<uint64_t>(c) * stride));
        if (BF16OUT) {
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                h[j] = f32_to_bf16_rne(acc[j]);
            st_nt4(static_cast<uint16_t*>(out) + i0,
                   make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                              h[6] | (h[7] << 16)));
        } else {
            float* o = static_cast<float*>(out) + i0;
            st_nt4(o, make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                                 __float_as_uint(acc[2]), __float_as_uint(acc[3])));
            st_nt4(o + 4, make_uint4(__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                                     __float_as_uint(acc[6]), __float_as_uint(acc[7])));
        }
    } else {
        for (int j = 0; j < 8 && i0 + j < n; ++j) {
            float a = 0.0f;
            for (int32_t c = 0; c < num_chunks; ++c)
                a = a + bf16_lo(x[static_cast<uint64_t>(c) * stride + i0 + j]);
            if (BF16OUT)
                static_cast<uint16_t*>(out)[i0 + j] = static_cast<uint16_t>(f32_to_bf16_rne(a));
            else
                static_cast<float*>(out)[i0 + j] = a;
        }
    }
}

template <bool BF16OUT>
__global__ __launch_bounds__(kBlock)
void zc_reduce_kernel(const uint16_t* __restrict__ x, uint64_t n, uint64_t stride,
                      int32_t num_chunks, void* __restrict__ out)
{
    reduce_body<BF16OUT>(x, n, stride, num_chunks, out, blockIdx.x);
}

// One slab's decode and the previous slab's sum in one launch: the first
// dec_blocks workgroups decode (as zc_decompress_kernel) into one slab
// buffer, the rest sum the other (as zc_reduce_kernel).  The sum
// workgroups come last in the grid, so they run while the decode drains.
template <bool BF16OUT>
__global__ __launch_bounds__(kBlock, kMinWavesDec)
void zc_decode_sum_kernel(const uint8_t* __restrict__ in, uint16_t* __restrict__ dec,
                          int32_t* __restrict__ status, ChunkTable tab, uint32_t dec_blocks,
                          const uint16_t* __restrict__ x, uint64_t n, uint64_t stride,
                          int32_t num_chunks, void* __restrict__ out)
{
    if (blockIdx.x < dec_blocks)
        decompress_body(in, dec, status, tab);
    else
        reduce_body<BF16OUT>(x, n, stride, num_chunks, out, blockIdx.x - dec_blocks);
}

// ------------------------------------------------------------ decode and sum in one kernel

// One workgroup per tile position t: its eight waves decode tile t of eight
// streams at a time, one stream each.  After every two steps the waves'
// 1024 values each meet in LDS, and each thread adds two values of one of
// the two steps, over the streams in stream order, to its accumulators.
// Rounds of eight streams follow each other, so every sum takes the streams
// in chunk order; nothing decoded leaves the workgroup.
constexpr int kSumWaves = 8;                     // streams decoded together
constexpr int kSumBlock = kSumWaves * kLanes;    // threads: two values of one of two steps each
constexpr int kSumMinWaves = 4;                  // occupancy target, waves per SIMD
// Tile positions that run at once: two workgroups for each of the 256
// compute units.  The fused form's parallelism is 8 waves per tile
// position, and each wave decodes ceil(C / 8) tiles one after another, so a
// launch takes about the same time for every generation of 512 positions,
// however full; the staged form's time grows with the tile count.  The
// fused form is taken for 8 to 64 streams when its generations are at
// least 27/32 full (measured break-even: 864 positions, 2 generations).
constexpr uint64_t kSumMinTiles = 512;

// The streams of one fused call.
struct SumTable {
    int32_t nstreams;
    uint32_t n;                       // values per stream
    uint64_t boff[kMaxChunks];        // byte offset of stream c
    uint64_t bavail[kMaxChunks];      // readable bytes from boff[c]
};

// Per-thread place in the step exchange.
struct SumCtx {
    uint16_t* buf;        // LDS: two exchange buffers of kSumWaves x 2 x 512 values
    uint32_t wave, tid;
    uint32_t nround;      // streams of this round (waves 0 .. nround - 1)
};

// One exchange, steps k and k + 1 (k even): this wave's values of the two
// steps go into buffer (k / 2) % 2, and after the barrier thread tid adds
// values 2p and 2p + 1 (p = tid % 256) of step k + tid / 256 of the round's
// streams, in stream order, to acc[k] and acc[k + 1] (so acc[k + j] of
// thread tid sums value 2p + j of step k + tid / 256).  Two buffers need one
// barrier per exchange: a buffer is written again one exchange later, after
// every thread has passed the barrier in between, and so has finished
// reading it.
__device__ __forceinline__ void sum_step(const SumCtx& sc, float (&acc)[kSteps], int k, uint4 v0,
                                         uint4 v1)
{
    constexpr int kV = kLanes * 8;       // values per step
    uint16_t* b = sc.buf + ((k >> 1) & 1) * (kSumWaves * 2 * kV);
    uint16_t* mine = b + sc.wave * (2 * kV) + (sc.tid & (kLanes - 1)) * 8;
    *reinterpret_cast<uint4*>(mine) = v0;
    *reinterpret_cast<uint4*>(mine + kV) = v1;
    __syncthreads();
    const uint32_t* b32 = reinterpret_cast<const uint32_t*>(b) + (sc.tid >> 8) * (kV / 2) + (sc.tid & 255);
    const int e = k >> 1;
    float a0 = acc[2 * e], a1 = acc[2 * e + 1];
#pragma unroll
    for (int s = 0; s < kSumWaves; ++s)
        if (static_cast<uint32_t>(s) < sc.nround) {
            const uint32_t w = b32[s * kV];
            a0 = a0 + bf16_lo(w);
            a1 = a1 + bf16_hi(w);
        }
    acc[2 * e] = a0;
    acc[2 * e + 1] = a1;
}

// The 8 values of a segment as 16-bit words (the join of put_values); in a
// partial tile the ragged segment's sign+mantissa bytes are read one by one,
// and values past the end are left 0.
template <bool FULL>
__device__ __forceinline__ uint4 join_values(const uint8_t* __restrict__ rsrc, uint32_t n,
                                             uint32_t i0, uint2 r, const uint32_t (&e8)[8])
{
    if (!FULL && i0 < n && i0 + 8 > n) {
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (i0 + j < n)
                w[j >> 2] |= static_cast<uint32_t>(rsrc[i0 + j]) << (8 * (j & 3));
        r = make_uint2(w[0], w[1]);
    }
    uint4 o;
    o.x = (__builtin_amdgcn_perm(r.x, r.x, 0x01010000u) & 0x807F807Fu) | ((e8[0] & 0xFF) << 7) | ((e8[1] & 0xFF) << 23);
    o.y = (__builtin_amdgcn_perm(r.x, r.x, 0x03030202u) & 0x807F807Fu) | ((e8[2] & 0xFF) << 7) | ((e8[3] & 0xFF) << 23);
    o.z = (__builtin_amdgcn_perm(r.y, r.y, 0x01010000u) & 0x807F807Fu) | ((e8[4] & 0xFF) << 7) | ((e8[5] & 0xFF) << 23);
    o.w = (__builtin_amdgcn_perm(r.y, r.y, 0x03030202u) & 0x807F807Fu) | ((e8[6] & 0xFF) << 7) | ((e8[7] & 0xFF) << 23);
    return o;
}

// decode_group with every two steps handed to the exchange instead of
// stored; the sign+mantissa bytes are prefetched two steps ahead.
template <bool FULL, int kSym, bool MIXED, class Win>
__device__ __forceinline__ void decode_group_sum(const Win& win, const uint8_t* __restrict__ s_lut8,
                                                 const uint16_t* __restrict__ s_tail,
                                                 const uint8_t* __restrict__ s_len,
                                                 const uint8_t* __restrict__ rsrc, uint32_t n,
                                                 uint32_t base, uint32_t lane, uint32_t ng,
                                                 uint32_t emax, bool raw_mode, DecState& st,
                                                 const SumCtx& sc, float (&acc)[kSteps])
{
    const bool raw = MIXED && raw_mode;
    LaneCode q;
    q.ish = raw ? 24u : static_cast<uint32_t>(32 - kLutBits);
    q.base = raw ? static_cast<uint32_t>(kLutRaw) : 0u;
    q.sym_sh = raw ? 0u : 4u;
    q.smask = raw ? 0u : 15u;
    q.sor = raw ? 8u : 0u;
    q.lmark = raw ? 256u : 0u;
    q.emax_eff = raw ? 255u : emax;
    const uint2* rsrc2 = reinterpret_cast<const uint2*>(rsrc + base) + lane;
    auto raw_at = [&](int k) {
        return (FULL || base + k * 512 + lane * 8 + 8 <= n) ? ld_nt2(rsrc2 + k * 64)
                                                            : make_uint2(0, 0);
    };
    uint2 ring[2] = {raw_at(0), raw_at(1)};
#pragma unroll 1
    for (int k = 0; k < kSteps; k += 2) {
        uint32_t e8[8];
        decode_step<FULL, kSym, MIXED>(win, s_lut8, s_tail, s_len, q, k, ng, emax, raw_mode, st, e8);
        const uint4 v0 = join_values<FULL>(rsrc, n, base + k * 512 + lane * 8, ring[0], e8);
        ring[0] = raw_at(min(k + 2, kSteps - 1));
        decode_step<FULL, kSym, MIXED>(win, s_lut8, s_tail, s_len, q, k + 1, ng, emax, raw_mode, st, e8);
        const uint4 v1 = join_values<FULL>(rsrc, n, base + (k + 1) * 512 + lane * 8, ring[1], e8);
        ring[1] = raw_at(min(k + 3, kSteps - 1));
        sum_step(sc, acc, k, v0, v1);
    }
}

// A wave with no stream this round (or one whose tile failed a check) still
// takes part in every step of the exchange.
__device__ __forceinline__ void idle_sum(const SumCtx& sc, float (&acc)[kSteps])
{
#pragma unroll 1
    for (int k = 0; k < kSteps; k += 2)
        sum_step(sc, acc, k, make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0));
}

// decompress_tile's checks and decode for one stream's tile t, feeding the
// exchange; every path runs the 16 steps of the exchange exactly once.
template <bool FULL>
__device__ __forceinline__ void decode_tile_sum(const uint8_t* __restrict__ src,
                                                int32_t* __restrict__ status, int c, uint32_t n,
                                                uint32_t t, uint64_t bavail, uint32_t lane,
                                                uint32_t* __restrict__ s,
                                                const uint8_t* __restrict__ s_lut8,
                                                const uint16_t* __restrict__ s_tail,
                                                const uint8_t* __restrict__ s_len,
                                                const SumCtx& sc, float (&acc)[kSteps])
{
    const Geom G = geometry(n);
    const uint32_t base = t * kTile;
    const uint32_t rem = min(n - base, static_cast<uint32_t>(kTile));
    const uint32_t ng = FULL ? 128u : group_members(rem, lane);
    int fail = 0;
    TileMeta meta = {0, 0, 0, 0, 0};
    if (G.X > bavail)
        fail = ZC_REASON_SIZE;
    else
        meta = load_meta(src, G, t, lane);
    const uint32_t hw = meta.hw, toff = meta.toff, tnext = meta.tnext, emax = meta.emax,
                   glen = meta.glen;
    const uint32_t h0 = __shfl(hw, 0), h1 = __shfl(hw, 1), h2 = __shfl(hw, 2),
                   h3 = __shfl(hw, 3), h4 = __shfl(hw, 4), h5 = __shfl(hw, 5),
                   h6 = __shfl(hw, 6), h7 = __shfl(hw, 7);
    if (!fail && (h0 != kMagic || h1 != kVerTable || h2 != 0 || h3 != 0 || h4 != n || h5 != 0))
        fail = ZC_REASON_HEADER;
    const uint64_t comp = h6 | (static_cast<uint64_t>(h7) << 32);
    if (!fail && (comp < G.X || comp > bavail || comp > chunk_bound(n)))
        fail = ZC_REASON_SIZE;
    const uint64_t next = (t + 1 < G.T) ? tnext : comp - G.X;
    if (!fail && ((t == 0 && toff != 0) || toff > next || next > comp - G.X))
        fail = ZC_REASON_TILE;
    if (!fail && __ballot(glen > 8 * ng || (ng == 0 && emax != 0)))
        fail = ZC_REASON_GROUP;
    uint32_t tile_bits;
    const uint32_t off = wave_excl_scan(glen, lane, &tile_bits);
    // uniform: it chooses between paths that hold barriers
    tile_bits = __builtin_amdgcn_readfirstlane(tile_bits);
    const uint32_t tile_words = (tile_bits + 31) >> 5;
    if (!fail && static_cast<uint32_t>(next - toff) != 4 * tile_words)
        fail = ZC_REASON_TILE;
    fail = __builtin_amdgcn_readfirstlane(fail);
    if (fail) {
        if (lane == 0)
            report(status, fail, c);
        idle_sum(sc, acc);
        return;
    }

    const uint32_t* gstream = reinterpret_cast<const uint32_t*>(src + G.X + toff);
    int err = 0;
    if (t == 0) {
        const uint64_t g1 = 32 + 196ull * G.T;
        if (g1 + lane < G.R && src[g1 + lane] != 0)
            err = ZC_REASON_GAP;
    }
    if (t == G.T - 1) {
        if (G.R + n + lane < G.X && src[G.R + n + lane] != 0)
            err = ZC_REASON_GAP;
    }
    if ((tile_bits & 31) && lane == 0) {
        const uint32_t last = gstream[tile_words - 1];
        if (last & ((1u << (32 - (tile_bits & 31))) - 1))
            err = ZC_REASON_PADDING;
    }
    const bool raw_mode = ng > 0 && glen == 8 * ng;
    const uint64_t raw_lanes = __ballot(raw_mode);
    const uint8_t* rsrc = src + G.R;
    DecState st;
    st.pos = off;
    st.seen_max = 0;
    st.raw_coded = 0;
    st.esc_min = 255;
    if (tile_words <= static_cast<uint32_t>(kStageWords)) {
        wave_lds_sync();
        stage_words(s, gstream, tile_words, lane);
        if (lane < 4)
            s[tile_words + lane] = 0;
        wave_lds_sync();
        const LdsWindow lw{s, tile_words};
        if (__ballot(!raw_mode && glen > 5 * ng) == 0) {
            if (raw_lanes == 0)
                decode_group_sum<FULL, 8, false>(lw, s_lut8, s_tail, s_len, rsrc, n, base, lane,
                                                 ng, emax, raw_mode, st, sc, acc);
            else
                decode_group_sum<FULL, 8, true>(lw, s_lut8, s_tail, s_len, rsrc, n, base, lane,
                                                ng, emax, raw_mode, st, sc, acc);
        } else {
            if (raw_lanes == 0)
                decode_group_sum<FULL, 4, false>(lw, s_lut8, s_tail, s_len, rsrc, n, base, lane,
                                                 ng, emax, raw_mode, st, sc, acc);
            else
                decode_group_sum<FULL, 4, true>(lw, s_lut8, s_tail, s_len, rsrc, n, base, lane,
                                                ng, emax, raw_mode, st, sc, acc);
        }
    } else {
        decode_group_sum<FULL, 4, true>(GlobalWindow{gstream, tile_words}, s_lut8, s_tail, s_len,
                                        rsrc, n, base, lane, ng, emax, raw_mode, st, sc, acc);
    }
    if (err == 0 && ng > 0) {
        if (st.pos != off + glen)
            err = ZC_REASON_LENGTH;
        else if (st.seen_max != emax)
            err = ZC_REASON_EMAX;
        else if (!raw_mode && st.esc_min < kEsc)
            err = ZC_REASON_ESCAPE;
        else if (raw_mode && st.raw_coded < 8 * ng)
            err = ZC_REASON_RAWMODE;
    }
    const uint64_t bad = __ballot(err != 0);
    if (bad) {
        const int first = __ffsll(static_cast<unsigned long long>(bad)) - 1;
        const int reason = __shfl(err, first);
        if (lane == 0)
            report(status, reason, c);
    }
}

// Tile position blockIdx.x of every stream in tab, decoded and summed in
// chunk order (fp32 sums, or each rounded once to bf16).  128 VGPRs (four
// waves per SIMD) and 68 KiB of LDS: two workgroups per compute unit.
template <bool BF16OUT>
__global__ __launch_bounds__(kSumBlock, kSumMinWaves)
void zc_decode_sum_fused_kernel(const uint8_t* __restrict__ in, int32_t* __restrict__ status,
                                SumTable tab, void* __restrict__ out)
{
    __shared__ __align__(16) uint32_t s_stage[kSumWaves][kStageAlloc];
    __shared__ __align__(16) uint16_t s_step[2 * kSumWaves * 2 * kLanes * 8];
    __shared__ __align__(16) uint8_t s_lut8[kLutRaw + 256];
    __shared__ uint16_t s_tail[1 << kTailBits];
    __shared__ uint8_t s_len[256];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kLanes - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kLanes);
    for (uint32_t i = tid; i < static_cast<uint32_t>(kLutWords); i += kSumBlock)
        reinterpret_cast<uint32_t*>(s_lut8)[i] = reinterpret_cast<const uint32_t*>(c_lut)[i];
    if (tid < 256) {
        s_lut8[kLutRaw + tid] = static_cast<uint8_t>(255u - tid);
        const uint32_t sy = tid < static_cast<uint32_t>(kEsc) ? tid : static_cast<uint32_t>(kEsc);
        s_len[tid] = static_cast<uint8_t>(len_of(sy) + (sy == static_cast<uint32_t>(kEsc) ? 8 : 0));
    }
    if (tid < (1u << kTailBits))
        s_tail[tid] = static_cast<uint16_t>(tail_of(tid));
    __syncthreads();

    const uint32_t n = tab.n;
    const uint32_t t = blockIdx.x;
    const bool full = n - t * kTile >= static_cast<uint32_t>(kTile);
    float acc[kSteps];
#pragma unroll
    for (int k = 0; k < kSteps; ++k)
        acc[k] = 0.0f;
    for (int32_t r0 = 0; r0 < tab.nstreams; r0 += kSumWaves) {
        const int32_t c = r0 + static_cast<int32_t>(wave);
        const SumCtx sc{s_step, wave, tid, static_cast<uint32_t>(min(kSumWaves, tab.nstreams - r0))};
        if (c < tab.nstreams) {
            const uint8_t* src = in + tab.boff[c];
            if (full)
                decode_tile_sum<true>(src, status, c, n, t, tab.bavail[c], lane, s_stage[wave],
                                      s_lut8, s_tail, s_len, sc, acc);
            else
                decode_tile_sum<false>(src, status, c, n, t, tab.bavail[c], lane, s_stage[wave],
                                       s_lut8, s_tail, s_len, sc, acc);
        } else {
            idle_sum(sc, acc);
        }
    }
    // acc[2e], acc[2e + 1]: values 2p, 2p + 1 of step 2e + tid / 256
#pragma unroll
    for (int e = 0; e < kSteps / 2; ++e) {
        const uint32_t i = t * kTile + (2 * e + (tid >> 8)) * 512 + 2 * (tid & 255);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (i + j < n) {
                if (BF16OUT)
                    static_cast<uint16_t*>(out)[i + j] = static_cast<uint16_t>(f32_to_bf16_rne(acc[2 * e + j]));
                else
                    __builtin_nontemporal_store(acc[2 * e + j], static_cast<float*>(out) + i + j);
            }
        }
    }
}

// ------------------------------------------------------------ device-resident split

__device__ inline uint64_t wave_excl_scan64(uint64_t x, uint32_t lane, uint64_t* total)
{
    uint64_t incl = x;
#pragma unroll
    for (int o = 1; o < kLanes; o <<= 1) {
        const uint64_t y = __shfl_up(incl, o);
        if (lane >= static_cast<uint32_t>(o))
            incl += y;
    }
    *total = __shfl(incl, kLanes - 1);
    return incl - x;
}

__device__ inline uint64_t wave_sum64(uint64_t x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}

// Builds the chunk table of one launch (chunks c0 .. c0 + m - 1 of
// num_chunks) in device memory from counts that live on the device: the
// same table the host builds from host counts.  One wave; lane c handles
// chunk c0 + c.  The whole split is checked first: every count within
// 0 .. ZC_MAX_CHUNK_VALUES and their sum equal to `total` (and, when
// decoding from explicit offsets, each offset 16-byte aligned with a header's
// room in the input).  An invalid split leaves a table without tiles, so the
// codec kernels that follow do nothing, and is reported: compress writes -1
// to the launch's comp_sizes and slot_off entries, decompress records
// ZC_REASON_SIZE in *status.
__global__ __launch_bounds__(kLanes)
void zc_plan_kernel(const int64_t* __restrict__ counts, int32_t num_chunks, int32_t c0, int32_t m,
                    int64_t total, const int64_t* __restrict__ in_offsets, uint64_t in_bytes,
                    uint32_t max_items, uint32_t spin_limit, int32_t decode,
                    ChunkTable* __restrict__ tab, int64_t* __restrict__ slot_off,
                    int64_t* __restrict__ comp_sizes, int32_t* __restrict__ status)
{
    const uint32_t lane = threadIdx.x;
    uint64_t sum = 0, slot_before = 0, voff_before = 0;
    bool bad = false;
    for (int32_t c = static_cast<int32_t>(lane); c < num_chunks; c += kLanes) {
        const int64_t n = counts[c];
        if (n < 0 || n > ZC_MAX_CHUNK_VALUES) {
            bad = true;
            continue;
        }
        sum += static_cast<uint64_t>(n);
        if (c < c0) {
            slot_before += align256(chunk_bound(static_cast<uint64_t>(n)));
            voff_before += static_cast<uint64_t>(n);
        }
    }
    sum = wave_sum64(sum);
    slot_before = wave_sum64(slot_before);
    voff_before = wave_sum64(voff_before);
    bad = __ballot(bad) != 0 || total < 0 || sum != static_cast<uint64_t>(total);

    const bool mine = lane < static_cast<uint32_t>(m);
    const uint64_t n = (mine && !bad) ? static_cast<uint64_t>(counts[c0 + lane]) : 0u;
    const uint32_t T = static_cast<uint32_t>((n + kTile - 1) / kTile);
    const uint32_t items_c = mine ? (T ? T : 1u) : 0u;
    uint32_t items;
    const uint32_t ibegin = wave_excl_scan(items_c, lane, &items);
    uint64_t vtotal, stotal;
    const uint64_t voff = voff_before + wave_excl_scan64(n, lane, &vtotal);
    const uint64_t slot = slot_before +
                          wave_excl_scan64(mine ? align256(chunk_bound(n)) : 0u, lane, &stotal);
    uint64_t boff = slot;
    if (decode && in_offsets && mine) {
        const int64_t o = in_offsets[c0 + lane];
        boff = static_cast<uint64_t>(o);
        if (o < 0 || (o & 15) || static_cast<uint64_t>(o) + 32 > in_bytes)
            bad = true;
    } else if (decode && mine && boff + 32 > in_bytes) {
        bad = true;
    }
    bad = __ballot(bad) != 0 || items > max_items;

    if (mine) {
        tab->item_begin[lane] = ibegin;
        tab->n[lane] = static_cast<uint32_t>(n);
        tab->voff[lane] = voff;
        tab->boff[lane] = boff;
        tab->bavail[lane] = in_bytes > boff ? in_bytes - boff : 0u;
        if (!decode) {
            slot_off[c0 + lane] = bad ? -1 : static_cast<int64_t>(boff);
            if (bad)
                comp_sizes[c0 + lane] = -1;
        }
    }
    if (lane == 0) {
        tab->item_begin[m] = items;
        tab->nchunks = m;
        tab->chunk_base = c0;
        tab->nitems = bad ? 0u : items;
        tab->spin_limit = spin_limit;
        tab->tile0 = 0;
        if (decode && bad && status)
            atomicCAS(status, 0, (ZC_REASON_SIZE << 24) | (c0 & 0xFFFFFF));
    }
}

// ------------------------------------------------------------ size estimate

__device__ inline uint32_t exp_of(const uint4& v, int j)
{
    const uint32_t w = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
    return (w >> ((j & 1) ? 23 : 7)) & 0xFFu;
}

// Bytes of tile t's exponent stream, from the input values: per group (one
// per lane) the maximum exponent, the code length of every member (escape:
// code word plus 8 bits), and raw mode when that reaches 8 bits per member;
// the tile's bits rounded up to whole 32-bit words.  This is the size the
// encoder writes for the tile.  A whole, 16-byte aligned tile is read with
// all of a lane's 16 loads in flight; other tiles value by value.  bits_of[d]
// is the stream length of a member d below its group's maximum.
__device__ inline uint32_t tile_stream_bytes(const uint16_t* __restrict__ chunk, uint32_t n,
                                             uint32_t t, uint32_t lane,
                                             const uint8_t* __restrict__ bits_of)
{
    const uint16_t* src = chunk + static_cast<uint64_t>(t) * kTile;
    const uint32_t rem = min(n - t * kTile, static_cast<uint32_t>(kTile));
    uint32_t bits = 0;
    if (rem == kTile && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
        uint4 v[kSteps];
#pragma unroll
        for (int k = 0; k < kSteps; ++k)
            v[k] = *reinterpret_cast<const uint4*>(src + k * 512 + lane * 8);
        uint32_t emax = 0;
#pragma unroll
        for (int k = 0; k < kSteps; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                emax = max(emax, exp_of(v[k], j));
#pragma unroll
        for (int k = 0; k < kSteps; ++k)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                bits += bits_of[emax - exp_of(v[k], j)];
    } else {
        uint32_t emax = 0;
#pragma unroll 1
        for (uint32_t i = lane * 8; i < rem; i += (i & 7) == 7 ? 512 - 7 : 1)
            emax = max(emax, (static_cast<uint32_t>(src[i]) >> 7) & 0xFFu);
#pragma unroll 1
        for (uint32_t i = lane * 8; i < rem; i += (i & 7) == 7 ? 512 - 7 : 1)
            bits += bits_of[emax - ((static_cast<uint32_t>(src[i]) >> 7) & 0xFFu)];
    }
    const uint32_t ng = group_members(rem, lane);
    const uint32_t glen = (ng > 0 && bits >= 8 * ng) ? 8 * ng : bits;
    return ((wave_sum(glen) + 31) >> 5) * 4;
}

// Estimated stream size of each chunk, for the switch between compressed and
// plain collectives (abstract, technique (3); pith.science, Figure 15
// caption), which needs the compressed size before it decides.  Workgroup c
// handles chunk c: it checks the split, finds the chunk's value offset, and
// sizes `samples` tiles spread evenly over the chunk (tile floor(i T / k)
// for i < k = min(samples, T)).  The estimate is the exact fixed part of the
// stream plus the sampled tile bytes scaled by T / k, rounded half up; with
// k = T it is the exact size zc_compress writes.  -1 for an invalid split.
__global__ __launch_bounds__(kBlock)
void zc_estimate_kernel(const uint16_t* __restrict__ in, const int64_t* __restrict__ counts,
                        int32_t num_chunks, int64_t total, int32_t samples,
                        int64_t* __restrict__ est)
{
    __shared__ uint64_t s_part[kWaves][3];
    __shared__ uint8_t s_bits[256];
    const uint32_t tid = threadIdx.x;
    s_bits[tid] = static_cast<uint8_t>(tid < static_cast<uint32_t>(kEsc) ? len_of(tid)
                                                                          : len_of(kEsc) + 8u);
    const uint32_t lane = tid & (kLanes - 1);
    const uint32_t wave = tid / kLanes;
    const int32_t c = static_cast<int32_t>(blockIdx.x);
    uint64_t before = 0, sum = 0, bad = 0;
    for (int32_t j = static_cast<int32_t>(tid); j < num_chunks; j += kBlock) {
        const int64_t v = counts[j];
        if (v < 0 || v > ZC_MAX_CHUNK_VALUES)
            bad = 1;
        else {
            sum += static_cast<uint64_t>(v);
            before += j < c ? static_cast<uint64_t>(v) : 0u;
        }
    }
    before = wave_sum64(before);
    sum = wave_sum64(sum);
    bad = wave_sum64(bad);
    if (lane == 0) {
        s_part[wave][0] = before;
        s_part[wave][1] = sum;
        s_part[wave][2] = bad;
    }
    __syncthreads();
    before = sum = bad = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        before += s_part[w][0];
        sum += s_part[w][1];
        bad += s_part[w][2];
    }
    __syncthreads();
    if (bad || sum != static_cast<uint64_t>(total)) {
        if (tid == 0)
            est[c] = -1;
        return;
    }
    const uint32_t n = static_cast<uint32_t>(counts[c]);
    const Geom G = geometry(n);
    const uint32_t k = min(static_cast<uint32_t>(samples), G.T);
    uint64_t bytes = 0;
    for (uint32_t i = wave; i < k; i += kWaves) {
        const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(i) * G.T) / k);
        bytes += tile_stream_bytes(in + before, n, t, lane, s_bits);
    }
    if (lane == 0)
        s_part[wave][0] = bytes;
    __syncthreads();
    if (tid == 0) {
        uint64_t s = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
            s += s_part[w][0];
        const uint64_t scaled = k ? (s * G.T + k / 2) / k : 0;
        est[c] = static_cast<int64_t>(G.X + scaled);
    }
}

// ------------------------------------------------------------ host side

struct Counts {
    bool ok;
    uint64_t total_values;
    uint64_t total_items;
};

Counts check_counts(const int64_t* counts, int32_t num_chunks)
{
    Counts r{false, 0, 0};
    if (num_chunks < 0 || num_chunks > ZC_MAX_CHUNKS || (num_chunks > 0 && !counts))
        return r;
    for (int32_t c = 0; c < num_chunks; ++c) {
        if (counts[c] < 0 || counts[c] > ZC_MAX_CHUNK_VALUES)
            return r;
        r.total_values += static_cast<uint64_t>(counts[c]);
        const uint64_t T = (static_cast<uint64_t>(counts[c]) + kTile - 1) / kTile;
        r.total_items += T ? T : 1;
    }
    r.ok = true;
    return r;
}


// Look-back polls a tile makes before it recomputes a missing predecessor's
// size from the input.  The environment variable ZC_LOOKBACK_SPIN_LIMIT, read
// once per process at the first compress call, overrides the default (tests
// set 0 in a child process to run the recomputation path).
uint32_t lookback_spin_limit()
{
    static const uint32_t limit = [] {
        const char* e = std::getenv("ZC_LOOKBACK_SPIN_LIMIT");
        if (!e || !*e)
            return kSpinLimit;
        char* end = nullptr;
        const unsigned long v = std::strtoul(e, &end, 10);
        return (end && *end == 0 && v <= 0xFFFFFFFFul) ? static_cast<uint32_t>(v) : kSpinLimit;
    }();
    return limit;
}

// Zeroes `words` 32-bit words (a workspace that must start at zero).
__global__ void zc_zero_kernel(uint32_t* __restrict__ p, uint64_t words)
{
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < words;
         i += static_cast<uint64_t>(gridDim.x) * blockDim.x)
        p[i] = 0;
}


}  // namespace

namespace {

// ---- compress without a caller workspace

// The workspace of zc_compress_noalloc: one copy per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not device
// memory: kernels and copies get the per-device address that
// hipGetSymbolAddress returns (noalloc_scratch below), never the name.
constexpr size_t kNoallocBytes = ZC_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoallocBytes];

constexpr int kMaxDevices = 64;

// The device address of this GPU's scratch array, looked up once per device
// with that device current; nullptr if the lookup or its clearing failed.
// The array must start at zero (a compress workspace does), so the first call
// on a device clears it with a fill kernel on that call's stream, ahead of
// the call's own launches.
void* noalloc_scratch(int device, hipStream_t stream)
{
    static std::once_flag once[kMaxDevices];
    static void* ptr[kMaxDevices];
    std::call_once(once[device], [device, stream] {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return;
        hipLaunchKernelGGL(zc_zero_kernel, dim3(256), dim3(256), 0, stream,
                           static_cast<uint32_t*>(p), static_cast<uint64_t>(kNoallocBytes / 4));
        if (hipGetLastError() == hipSuccess)
            ptr[device] = p;
    });
    return ptr[device];
}

// ---- device-resident split: bounds and workspace layout

// Tiles of one launch of m chunks holding at most `total` values:
// sum of max(1, ceil(n_c / 8192)) <= floor(total / 8192) + m.
uint64_t dev_max_items(int64_t total, int32_t m)
{
    return static_cast<uint64_t>(total) / kTile + static_cast<uint64_t>(m);
}

bool dev_args_ok(int64_t total, int32_t num_chunks)
{
    return num_chunks >= 0 && num_chunks <= ZC_MAX_CHUNKS && total >= 0 &&
           (num_chunks > 0 || total == 0) &&
           dev_max_items(total, num_chunks < kMaxChunks ? num_chunks : kMaxChunks) < (1ull << 31);
}

// Workspace layout of the device-split calls: header, look-back
// status words for the largest launch, then one chunk table per launch.
uint64_t dev_tables_offset(int64_t total, int32_t num_chunks)
{
    const int32_t m = num_chunks < kMaxChunks ? num_chunks : kMaxChunks;
    return align256(kWsHeader + 8ull * kStatusStride * dev_max_items(total, m));
}

}  // namespace

namespace {

// Staged bytes of one slab of zc_decompress_reduce, over all contributions:
// large enough that a slab's decode fills the device, and small enough that
// two of them (one being decoded, one being summed) fit the 256 MB
// last-level cache.
constexpr uint64_t kReduceSlabBytes = 128ull << 20;

// Values per contribution in one slab (also the contributions' spacing in
// the scratch buffer): whole tiles, or all n values rounded up to 8 when
// they fit in one slab.
uint64_t reduce_stride(uint64_t n, int32_t num_chunks)
{
    const uint64_t c = num_chunks > 0 ? static_cast<uint64_t>(num_chunks) : 1u;
    const uint64_t tiles = std::max<uint64_t>(1, kReduceSlabBytes / (2 * c) / kTile);
    return std::min<uint64_t>(tiles * kTile, (n + 7) & ~7ull);
}

// Decode and sum in one kernel, nothing staged (zc_decode_sum_fused_kernel).
bool reduce_fused(uint64_t n, int32_t num_chunks)
{
    const uint64_t T = (n + kTile - 1) / kTile;
    const uint64_t gens = (T + kSumMinTiles - 1) / kSumMinTiles;
    return num_chunks >= kSumWaves && num_chunks <= kMaxChunks && T >= kSumMinTiles &&
           T * 32 >= gens * kSumMinTiles * 27;
}

// More than one slab of at most 64 streams: each launch decodes one slab
// and sums the one before, so two slab buffers alternate.
bool reduce_pipelined(uint64_t n, int32_t num_chunks)
{
    return num_chunks > 0 && num_chunks <= kMaxChunks && n > reduce_stride(n, num_chunks);
}

// Scratch bytes of zc_decompress_reduce (none for the fused form).
uint64_t reduce_scratch(uint64_t n, int32_t num_chunks)
{
    if (reduce_fused(n, num_chunks))
        return 0;
    return 2ull * reduce_stride(n, num_chunks) * static_cast<uint64_t>(num_chunks) *
           (reduce_pipelined(n, num_chunks) ? 2u : 1u);
}

// A slab of a decode: tiles tile0 .. tile0 + tiles - 1 of every chunk, value
// i of chunk c written at c stride + i - tile0 kTile of the output.
struct Slab {
    uint32_t tile0, tiles;
    uint64_t stride;
};

// zc_decompress; reported chunk indices start at chunk_base (zc_pipeline
// decodes group by group and reports indices of the whole call).
int decompress_chunks(const void* d_in, size_t in_bytes, const int64_t* in_offsets,
                      const int64_t* counts, int32_t num_chunks, uint16_t* d_out,
                      int32_t* d_status, void* stream, int32_t chunk_base,
                      const Slab* slab = nullptr)
{
    const Counts k = check_counts(counts, num_chunks);
    if (!k.ok)
        return ZC_EINVAL;
    if (num_chunks == 0)
        return ZC_OK;
    if (!d_in || !d_status || (k.total_values && !d_out))
        return ZC_EINVAL;
    if ((reinterpret_cast<uintptr_t>(d_in) & 15) || (reinterpret_cast<uintptr_t>(d_out) & 1)
        || (reinterpret_cast<uintptr_t>(d_status) & 3))
        return ZC_EINVAL;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t* in = static_cast<const uint8_t*>(d_in);
    uint64_t voff = 0, slot = 0;
    for (int32_t c0 = 0; c0 < num_chunks; c0 += kMaxChunks) {
        ChunkTable tab;
        std::memset(&tab, 0, sizeof tab);
        uint32_t items = 0;
        int32_t m = 0;
        for (int32_t c = c0; c < num_chunks && c < c0 + kMaxChunks; ++c, ++m) {
            const uint64_t n = static_cast<uint64_t>(counts[c]);
            const uint64_t T = (n + kTile - 1) / kTile;
            const int64_t off = in_offsets ? in_offsets[c] : static_cast<int64_t>(slot);
            if (off < 0 || (off & 15) || static_cast<uint64_t>(off) + 32 > in_bytes)
                return ZC_EINVAL;
            tab.item_begin[m] = items;
            tab.n[m] = static_cast<uint32_t>(n);
            tab.voff[m] = voff;
            tab.boff[m] = static_cast<uint64_t>(off);
            tab.bavail[m] = in_bytes - static_cast<uint64_t>(off);
            if (slab) {
                // tiles tile0 .. tile0 + tiles - 1 of every chunk (all of n
                // values); value i of chunk c lands at c stride + i - s0,
                // an offset that wraps below zero only before the slab's
                // first value, which is never written
                tab.voff[m] = static_cast<uint64_t>(c) * slab->stride -
                              static_cast<uint64_t>(slab->tile0) * kTile;
                items += slab->tiles;
            } else {
                items += static_cast<uint32_t>(T ? T : 1);
            }
            voff += n;
            slot += align256(chunk_bound(n));
        }
        tab.nchunks = m;
        tab.chunk_base = chunk_base + c0;
        tab.tile0 = slab ? slab->tile0 : 0u;
        tab.nitems = items;
        tab.item_begin[m] = items;
        hipLaunchKernelGGL(zc_decompress_kernel, dim3((items + kWaves - 1) / kWaves), dim3(kBlock), 0, s, in,
                           d_out, d_status, tab);
        if (hipGetLastError() != hipSuccess)
            return ZC_EHIP;
    }
    return ZC_OK;
}

// Decode num_chunks streams of n values and sum them (fp32 output, or bf16
// when `bf16`).  With 8 to 64 streams of at least kSumMinTiles tiles that
// fill the fused kernel's generations (reduce_fused), one launch decodes and
// sums with nothing staged.  Otherwise slab by slab: each
// slab is a run of whole tiles of every stream, decoded into a slab buffer
// (contribution c at c stride) and summed while it is still in the device's
// last-level cache.  With up to 64 streams, launch i decodes slab i into
// buffer i % 2 and sums slab i - 1 from the other buffer (the sum's
// workgroups run as the decode drains); with more, each slab is decoded (64
// streams per launch) and then summed.
int decompress_reduce(const void* d_in, size_t in_bytes, const int64_t* in_offsets, int64_t n,
                      int32_t num_chunks, void* d_out, bool bf16, int32_t* d_status,
                      void* d_scratch, size_t scratch_bytes, void* stream)
{
    if (n < 0 || n > ZC_MAX_CHUNK_VALUES || num_chunks < 0 || num_chunks > ZC_MAX_CHUNKS)
        return ZC_EINVAL;
    if (n == 0)
        return ZC_OK;
    const uint64_t need = reduce_scratch(static_cast<uint64_t>(n), num_chunks);
    if (!d_out || !d_status || (num_chunks > 0 && (!d_in || (need > 0 && !d_scratch))))
        return ZC_EINVAL;
    if ((reinterpret_cast<uintptr_t>(d_out) & 15) || (reinterpret_cast<uintptr_t>(d_scratch) & 15))
        return ZC_EINVAL;
    if (scratch_bytes < need)
        return ZC_ENOSPC;
    if (reduce_fused(static_cast<uint64_t>(n), num_chunks)) {
        const uint8_t* in = static_cast<const uint8_t*>(d_in);
        const uint64_t slot_bytes = align256(chunk_bound(static_cast<uint64_t>(n)));
        SumTable tab;
        std::memset(&tab, 0, sizeof tab);
        tab.nstreams = num_chunks;
        tab.n = static_cast<uint32_t>(n);
        for (int32_t c = 0; c < num_chunks; ++c) {
            const int64_t off = in_offsets ? in_offsets[c] : static_cast<int64_t>(c * slot_bytes);
            if (off < 0 || (off & 15) || static_cast<uint64_t>(off) + 32 > in_bytes)
                return ZC_EINVAL;
            tab.boff[c] = static_cast<uint64_t>(off);
            tab.bavail[c] = in_bytes - static_cast<uint64_t>(off);
        }
        if ((reinterpret_cast<uintptr_t>(d_in) & 15) || (reinterpret_cast<uintptr_t>(d_status) & 3))
            return ZC_EINVAL;
        hipStream_t s = static_cast<hipStream_t>(stream);
        const dim3 grid(static_cast<uint32_t>((static_cast<uint64_t>(n) + kTile - 1) / kTile));
        if (bf16)
            hipLaunchKernelGGL(zc_decode_sum_fused_kernel<true>, grid, dim3(kSumBlock), 0, s, in,
                               d_status, tab, d_out);
        else
            hipLaunchKernelGGL(zc_decode_sum_fused_kernel<false>, grid, dim3(kSumBlock), 0, s, in,
                               d_status, tab, d_out);
        return hipGetLastError() == hipSuccess ? ZC_OK : ZC_EHIP;
    }
    const uint64_t stride = reduce_stride(static_cast<uint64_t>(n), num_chunks);
    const uint64_t T = (static_cast<uint64_t>(n) + kTile - 1) / kTile;
    const uint64_t slab_tiles = (stride + kTile - 1) / kTile;
    const uint64_t slabs = (T + slab_tiles - 1) / slab_tiles;
    const uint64_t buf_values = stride * static_cast<uint64_t>(num_chunks);
    if (reduce_pipelined(static_cast<uint64_t>(n), num_chunks)) {
        const uint8_t* in = static_cast<const uint8_t*>(d_in);
        const uint64_t slot_bytes = align256(chunk_bound(static_cast<uint64_t>(n)));
        for (int32_t c = 0; c < num_chunks; ++c) {
            const int64_t off = in_offsets ? in_offsets[c] : static_cast<int64_t>(c * slot_bytes);
            if (off < 0 || (off & 15) || static_cast<uint64_t>(off) + 32 > in_bytes)
                return ZC_EINVAL;
        }
        if ((reinterpret_cast<uintptr_t>(d_in) & 15) || (reinterpret_cast<uintptr_t>(d_status) & 3))
            return ZC_EINVAL;
        hipStream_t s = static_cast<hipStream_t>(stream);
        for (uint64_t i = 0; i <= slabs; ++i) {
            ChunkTable tab;
            std::memset(&tab, 0, sizeof tab);
            uint32_t dec_blocks = 0;
            uint16_t* dec = static_cast<uint16_t*>(d_scratch) + (i & 1) * buf_values;
            if (i < slabs) {
                const uint64_t t0 = i * slab_tiles;
                const uint32_t tiles = static_cast<uint32_t>(std::min<uint64_t>(slab_tiles, T - t0));
                uint32_t items = 0;
                for (int32_t c = 0; c < num_chunks; ++c) {
                    const uint64_t off = in_offsets ? static_cast<uint64_t>(in_offsets[c]) : c * slot_bytes;
                    tab.item_begin[c] = items;
                    tab.n[c] = static_cast<uint32_t>(n);
                    tab.voff[c] = static_cast<uint64_t>(c) * stride - t0 * kTile;
                    tab.boff[c] = off;
                    tab.bavail[c] = in_bytes - off;
                    items += tiles;
                }
                tab.nchunks = num_chunks;
                tab.chunk_base = 0;
                tab.tile0 = static_cast<uint32_t>(t0);
                tab.nitems = items;
                tab.item_begin[num_chunks] = items;
                dec_blocks = (items + kWaves - 1) / kWaves;
            }
            const uint16_t* x = static_cast<const uint16_t*>(d_scratch) + ((i + 1) & 1) * buf_values;
            uint64_t len = 0, s0 = 0;
            if (i >= 1) {
                s0 = (i - 1) * slab_tiles * kTile;
                len = std::min<uint64_t>(static_cast<uint64_t>(n) - s0, stride);
            }
            const uint32_t sum_blocks = static_cast<uint32_t>(((len + 7) / 8 + kBlock - 1) / kBlock);
            const dim3 grid(dec_blocks + sum_blocks);
            if (bf16)
                hipLaunchKernelGGL(zc_decode_sum_kernel<true>, grid, dim3(kBlock), 0, s,
                                   in, dec, d_status, tab, dec_blocks, x, len, stride, num_chunks,
                                   static_cast<void*>(static_cast<uint16_t*>(d_out) + s0));
            else
                hipLaunchKernelGGL(zc_decode_sum_kernel<false>, grid, dim3(kBlock), 0, s,
                                   in, dec, d_status, tab, dec_blocks, x, len, stride, num_chunks,
                                   static_cast<void*>(static_cast<float*>(d_out) + s0));
            if (hipGetLastError() != hipSuccess)
                return ZC_EHIP;
        }
        return ZC_OK;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const std::vector<int64_t> counts(static_cast<size_t>(num_chunks), n);
    const uint16_t* x = static_cast<const uint16_t*>(d_scratch);
    for (uint64_t t0 = 0; t0 < T; t0 += slab_tiles) {
        const uint64_t s0 = t0 * kTile;
        const uint64_t len = std::min<uint64_t>(static_cast<uint64_t>(n) - s0, stride);
        if (num_chunks > 0) {
            const Slab slab{static_cast<uint32_t>(t0),
                            static_cast<uint32_t>(std::min<uint64_t>(slab_tiles, T - t0)), stride};
            const int r = decompress_chunks(d_in, in_bytes, in_offsets, counts.data(), num_chunks,
                                            static_cast<uint16_t*>(d_scratch), d_status, stream, 0,
                                            &slab);
            if (r != ZC_OK)
                return r;
        }
        const uint64_t threads = (len + 7) / 8;
        const dim3 grid(static_cast<uint32_t>((threads + kBlock - 1) / kBlock));
        if (bf16)
            hipLaunchKernelGGL(zc_reduce_kernel<true>, grid, dim3(kBlock), 0, s, x, len, stride,
                               num_chunks, static_cast<void*>(static_cast<uint16_t*>(d_out) + s0));
        else
            hipLaunchKernelGGL(zc_reduce_kernel<false>, grid, dim3(kBlock), 0, s, x, len, stride,
                               num_chunks, static_cast<void*>(static_cast<float*>(d_out) + s0));
        if (hipGetLastError() != hipSuccess)
            return ZC_EHIP;
    }
    return ZC_OK;
}

}  // namespace

extern "C" {

size_t zc_chunk_bound(int64_t n)
{
    if (n < 0)
        return 0;
    return static_cast<size_t>(chunk_bound(static_cast<uint64_t>(n)));
}

size_t zc_bound(const int64_t* counts, int32_t num_chunks)
{
    if (!check_counts(counts, num_chunks).ok)
        return 0;
    uint64_t acc = 0;
    for (int32_t c = 0; c < num_chunks; ++c)
        acc += align256(chunk_bound(static_cast<uint64_t>(counts[c])));
    return static_cast<size_t>(acc);
}

size_t zc_workspace_bytes(const int64_t* counts, int32_t num_chunks)
{
    const Counts k = check_counts(counts, num_chunks);
    if (!k.ok)
        return 0;
    // status words are reused by successive launches of one call
    uint64_t most = 0;
    for (int32_t c0 = 0; c0 < num_chunks; c0 += kMaxChunks) {
        uint64_t items = 0;
        for (int32_t c = c0; c < num_chunks && c < c0 + kMaxChunks; ++c) {
            const uint64_t T = (static_cast<uint64_t>(counts[c]) + kTile - 1) / kTile;
            items += T ? T : 1;
        }
        most = items > most ? items : most;
    }
    return static_cast<size_t>(kWsHeader + 8ull * kStatusStride * most);
}

int zc_compress(const uint16_t* d_in, const int64_t* counts, int32_t num_chunks,
                void* d_out, size_t out_capacity, int64_t* d_comp_sizes, void* d_ws,
                size_t ws_bytes, void* stream)
{
    const Counts k = check_counts(counts, num_chunks);
    if (!k.ok)
        return ZC_EINVAL;
    if (num_chunks == 0)
        return ZC_OK;
    if (!d_out || !d_comp_sizes || !d_ws || (k.total_values && !d_in))
        return ZC_EINVAL;
    if ((reinterpret_cast<uintptr_t>(d_out) & 15) || (reinterpret_cast<uintptr_t>(d_in) & 1)
        || (reinterpret_cast<uintptr_t>(d_ws) & 7) || (reinterpret_cast<uintptr_t>(d_comp_sizes) & 7))
        return ZC_EINVAL;
    if (out_capacity < zc_bound(counts, num_chunks))
        return ZC_ENOSPC;
    if (ws_bytes < zc_workspace_bytes(counts, num_chunks))
        return ZC_ENOSPC;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t spin_limit = lookback_spin_limit();
    uint8_t* ws = static_cast<uint8_t*>(d_ws);
    const uint64_t slots64 = (ws_bytes - kWsHeader) / (8ull * kStatusStride);
    const uint32_t slots = static_cast<uint32_t>(slots64 < 0xFFFFFFFFull ? slots64 : 0xFFFFFFFFull);
    uint8_t* out = static_cast<uint8_t*>(d_out);

    uint64_t voff = 0, boff = 0;
    for (int32_t c0 = 0; c0 < num_chunks; c0 += kMaxChunks) {
        ChunkTable tab;
        std::memset(&tab, 0, sizeof tab);
        uint32_t items = 0;
        int32_t m = 0;
        for (int32_t c = c0; c < num_chunks && c < c0 + kMaxChunks; ++c, ++m) {
            const uint64_t n = static_cast<uint64_t>(counts[c]);
            const uint64_t T = (n + kTile - 1) / kTile;
            tab.item_begin[m] = items;
            tab.n[m] = static_cast<uint32_t>(n);
            tab.voff[m] = voff;
            tab.boff[m] = boff;
            items += static_cast<uint32_t>(T ? T : 1);
            voff += n;
            boff += align256(chunk_bound(n));
        }
        tab.nchunks = m;
        tab.chunk_base = c0;
        tab.nitems = items;
        tab.item_begin[m] = items;
        tab.spin_limit = spin_limit;
        // one workgroup per tile; the status words need no clearing (each
        // launch tags its own)
        hipLaunchKernelGGL(zc_compress_kernel, dim3(items), dim3(kEncBlock), 0, s, d_in, out,
                           d_comp_sizes + c0, ws, slots, tab);
        if (hipGetLastError() != hipSuccess)
            return ZC_EHIP;
    }
    return ZC_OK;
}

int zc_compress_noalloc(const uint16_t* d_in, const int64_t* counts, int32_t num_chunks,
                        void* d_out, size_t out_capacity, int64_t* d_comp_sizes, void* stream)
{
    const Counts k = check_counts(counts, num_chunks);
    if (!k.ok)
        return ZC_EINVAL;
    if (num_chunks == 0)
        return ZC_OK;
    const size_t need = zc_workspace_bytes(counts, num_chunks);
    if (need > kNoallocBytes)
        return ZC_ENOSPC;
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess || device < 0 || device >= kMaxDevices)
        return ZC_EHIP;
    void* ws = noalloc_scratch(device, static_cast<hipStream_t>(stream));   // current device's
    if (!ws)
        return ZC_EHIP;
    // the same launch as zc_compress: the array is this device's workspace,
    // which every call leaves ready for the next
    return zc_compress(d_in, counts, num_chunks, d_out, out_capacity, d_comp_sizes, ws,
                       kNoallocBytes, stream);
}

size_t zc_bound_max(int64_t total_values, int32_t num_chunks)
{
    if (!dev_args_ok(total_values, num_chunks))
        return 0;
    // per chunk: align256(bound(n)) <= 317 + 200 T + 2n, and the T sum to at
    // most floor(total / 8192) + num_chunks
    const uint64_t t = static_cast<uint64_t>(total_values), c = static_cast<uint64_t>(num_chunks);
    return static_cast<size_t>(2 * t + 200 * (t / kTile + c) + 317 * c);
}

size_t zc_workspace_bytes_max(int64_t total_values, int32_t num_chunks)
{
    if (!dev_args_ok(total_values, num_chunks))
        return 0;
    const uint64_t launches = (static_cast<uint64_t>(num_chunks) + kMaxChunks - 1) / kMaxChunks;
    return static_cast<size_t>(dev_tables_offset(total_values, num_chunks) +
                               launches * align256(sizeof(ChunkTable)));
}

int zc_compress_dev(const uint16_t* d_in, const int64_t* d_counts, int32_t num_chunks,
                    int64_t total_values, void* d_out, size_t out_capacity,
                    int64_t* d_comp_sizes, int64_t* d_slot_off, void* d_ws, size_t ws_bytes,
                    void* stream)
{
    if (!dev_args_ok(total_values, num_chunks))
        return ZC_EINVAL;
    if (num_chunks == 0)
        return ZC_OK;
    if (!d_counts || !d_out || !d_comp_sizes || !d_slot_off || !d_ws || (total_values && !d_in))
        return ZC_EINVAL;
    if ((reinterpret_cast<uintptr_t>(d_out) & 15) || (reinterpret_cast<uintptr_t>(d_in) & 1)
        || (reinterpret_cast<uintptr_t>(d_ws) & 255) || (reinterpret_cast<uintptr_t>(d_counts) & 7)
        || (reinterpret_cast<uintptr_t>(d_comp_sizes) & 7) || (reinterpret_cast<uintptr_t>(d_slot_off) & 7))
        return ZC_EINVAL;
    if (out_capacity < zc_bound_max(total_values, num_chunks))
        return ZC_ENOSPC;
    if (ws_bytes < zc_workspace_bytes_max(total_values, num_chunks))
        return ZC_ENOSPC;

    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(d_ws);
    const uint64_t tables_at = dev_tables_offset(total_values, num_chunks);
    uint8_t* tables = ws + tables_at;
    const uint32_t slots = static_cast<uint32_t>((tables_at - kWsHeader) / (8ull * kStatusStride));
    const uint32_t spin_limit = lookback_spin_limit();
    for (int32_t c0 = 0, g = 0; c0 < num_chunks; c0 += kMaxChunks, ++g) {
        const int32_t m = num_chunks - c0 < kMaxChunks ? num_chunks - c0 : kMaxChunks;
        const uint32_t items = static_cast<uint32_t>(dev_max_items(total_values, m));
        ChunkTable* tab = reinterpret_cast<ChunkTable*>(tables + g * align256(sizeof(ChunkTable)));
        hipLaunchKernelGGL(zc_plan_kernel, dim3(1), dim3(kLanes), 0, s, d_counts, num_chunks, c0, m,
                           total_values, static_cast<const int64_t*>(nullptr), uint64_t(0), items,
                           spin_limit, 0, tab, d_slot_off, d_comp_sizes, static_cast<int32_t*>(nullptr));
        hipLaunchKernelGGL(zc_compress_dev_kernel, dim3(items), dim3(kEncBlock), 0, s, d_in,
                           static_cast<uint8_t*>(d_out), d_comp_sizes + c0, ws, slots,
                           static_cast<const ChunkTable*>(tab));
        if (hipGetLastError() != hipSuccess)
            return ZC_EHIP;
    }
    return ZC_OK;
}

int zc_decompress_dev(const void* d_in, size_t in_bytes, const int64_t* d_in_offsets,
                      const int64_t* d_counts, int32_t num_chunks, int64_t total_values,
                      uint16_t* d_out, int32_t* d_status, void* d_ws, size_t ws_bytes, void* stream)
{
    if (!dev_args_ok(total_values, num_chunks))
        return ZC_EINVAL;
    if (num_chunks == 0)
        return ZC_OK;
    if (!d_in || !d_counts || !d_status || !d_ws || (total_values && !d_out))
        return ZC_EINVAL;
    if ((reinterpret_cast<uintptr_t>(d_in) & 15) || (reinterpret_cast<uintptr_t>(d_out) & 1)
        || (reinterpret_cast<uintptr_t>(d_status) & 3) || (reinterpret_cast<uintptr_t>(d_ws) & 255)
        || (reinterpret_cast<uintptr_t>(d_counts) & 7) || (reinterpret_cast<uintptr_t>(d_in_offsets) & 7))
        return ZC_EINVAL;
    if (ws_bytes < zc_workspace_bytes_max(total_values, num_chunks))
        return ZC_ENOSPC;

    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* tables = static_cast<uint8_t*>(d_ws) + dev_tables_offset(total_values, num_chunks);
    const uint8_t* in = static_cast<const uint8_t*>(d_in);
    for (int32_t c0 = 0, g = 0; c0 < num_chunks; c0 += kMaxChunks, ++g) {
        const int32_t m = num_chunks - c0 < kMaxChunks ? num_chunks - c0 : kMaxChunks;
        const uint32_t items = static_cast<uint32_t>(dev_max_items(total_values, m));
        ChunkTable* tab = reinterpret_cast<ChunkTable*>(tables + g * align256(sizeof(ChunkTable)));
        hipLaunchKernelGGL(zc_plan_kernel, dim3(1), dim3(kLanes), 0, s, d_counts, num_chunks, c0, m,
                           total_values, d_in_offsets, static_cast<uint64_t>(in_bytes), items, 0u, 1,
                           tab, static_cast<int64_t*>(nullptr), static_cast<int64_t*>(nullptr), d_status);
        hipLaunchKernelGGL(zc_decompress_dev_kernel, dim3((items + kWaves - 1) / kWaves), dim3(kBlock),
                           0, s, in, d_out, d_status, static_cast<const ChunkTable*>(tab));
        if (hipGetLastError() != hipSuccess)
            return ZC_EHIP;
    }
    return ZC_OK;
}

int zc_estimate(const uint16_t* d_in, const int64_t* d_counts, int32_t num_chunks,
                int64_t total_values, int32_t samples_per_chunk, int64_t* d_est, void* stream)
{
    if (num_chunks < 0 || num_chunks > ZC_MAX_CHUNKS || total_values < 0 ||
        samples_per_chunk < 1 || (num_chunks == 0 && total_values != 0))
        return ZC_EINVAL;
    if (num_chunks == 0)
        return ZC_OK;
    if (!d_counts || !d_est || (total_values > 0 && !d_in))
        return ZC_EINVAL;
    hipLaunchKernelGGL(zc_estimate_kernel, dim3(static_cast<uint32_t>(num_chunks)), dim3(kBlock), 0,
                       static_cast<hipStream_t>(stream), d_in, d_counts, num_chunks, total_values,
                       samples_per_chunk, d_est);
    return hipGetLastError() == hipSuccess ? ZC_OK : ZC_EHIP;
}

size_t zc_reduce_scratch_bytes(int64_t n, int32_t num_chunks)
{
    if (n < 0 || n > ZC_MAX_CHUNK_VALUES || num_chunks < 0 || num_chunks > ZC_MAX_CHUNKS)
        return 0;
    return static_cast<size_t>(reduce_scratch(static_cast<uint64_t>(n), num_chunks));
}

int zc_decompress_reduce(const void* d_in, size_t in_bytes, const int64_t* in_offsets,
                         int64_t n, int32_t num_chunks, float* d_out, int32_t* d_status,
                         void* d_scratch, size_t scratch_bytes, void* stream)
{
    return decompress_reduce(d_in, in_bytes, in_offsets, n, num_chunks, d_out, false, d_status,
                             d_scratch, scratch_bytes, stream);
}

int zc_decompress_reduce_bf16(const void* d_in, size_t in_bytes, const int64_t* in_offsets,
                              int64_t n, int32_t num_chunks, uint16_t* d_out, int32_t* d_status,
                              void* d_scratch, size_t scratch_bytes, void* stream)
{
    return decompress_reduce(d_in, in_bytes, in_offsets, n, num_chunks, d_out, true, d_status,
                             d_scratch, scratch_bytes, stream);
}

int zc_decompress(const void* d_in, size_t in_bytes, const int64_t* in_offsets,
                  const int64_t* counts, int32_t num_chunks, uint16_t* d_out,
                  int32_t* d_status, void* stream)
{
    return decompress_chunks(d_in, in_bytes, in_offsets, counts, num_chunks, d_out, d_status,
                             stream, 0);
}

int zc_pipeline(const uint16_t* d_in, const int64_t* counts, int32_t num_chunks,
                int32_t groups, void* d_send, void* d_recv, size_t capacity,
                int64_t* d_comp_sizes, uint16_t* d_out, int32_t* d_status, void* d_ws,
                size_t ws_bytes, void* s_comp, void* s_link, void* s_dec)
{
    const Counts k = check_counts(counts, num_chunks);
    if (!k.ok || groups < 1 || (num_chunks > 0 && groups > num_chunks))
        return ZC_EINVAL;
    if (num_chunks == 0)
        return ZC_OK;
    if (!d_send || !d_recv || !d_comp_sizes || !d_status || !d_ws
        || (k.total_values && (!d_in || !d_out)))
        return ZC_EINVAL;
    if ((reinterpret_cast<uintptr_t>(d_send) & 15) || (reinterpret_cast<uintptr_t>(d_recv) & 15)
        || (reinterpret_cast<uintptr_t>(d_in) & 1) || (reinterpret_cast<uintptr_t>(d_out) & 1)
        || (reinterpret_cast<uintptr_t>(d_comp_sizes) & 7))
        return ZC_EINVAL;
    if (capacity < zc_bound(counts, num_chunks))
        return ZC_ENOSPC;
    if (ws_bytes < zc_workspace_bytes(counts, num_chunks))
        return ZC_ENOSPC;

    // value offsets and slot offsets of every chunk
    std::vector<uint64_t> voff(static_cast<size_t>(num_chunks) + 1, 0);
    std::vector<uint64_t> soff(static_cast<size_t>(num_chunks) + 1, 0);
    for (int32_t c = 0; c < num_chunks; ++c) {
        voff[c + 1] = voff[c] + static_cast<uint64_t>(counts[c]);
        soff[c + 1] = soff[c] + align256(chunk_bound(static_cast<uint64_t>(counts[c])));
    }
    hipStream_t sc = static_cast<hipStream_t>(s_comp);
    hipStream_t sl = static_cast<hipStream_t>(s_link);
    hipStream_t sd = static_cast<hipStream_t>(s_dec);
    uint8_t* send = static_cast<uint8_t*>(d_send);
    uint8_t* recv = static_cast<uint8_t*>(d_recv);

    for (int32_t g = 0; g < groups; ++g) {
        const int32_t c0 = static_cast<int32_t>(static_cast<int64_t>(g) * num_chunks / groups);
        const int32_t c1 = static_cast<int32_t>(static_cast<int64_t>(g + 1) * num_chunks / groups);
        const int32_t m = c1 - c0;
        const uint64_t gbytes = soff[c1] - soff[c0];
        // 1. compress the group into the sender's slots (in order on s_comp,
        //    so every group may use the one workspace)
        int r = zc_compress(d_in + voff[c0], counts + c0, m, send + soff[c0], gbytes,
                            d_comp_sizes + c0, d_ws, ws_bytes, sc);
        if (r != ZC_OK)
            return r;
        hipEvent_t compressed, sent;
        if (hipEventCreateWithFlags(&compressed, hipEventDisableTiming) != hipSuccess)
            return ZC_EHIP;
        if (hipEventCreateWithFlags(&sent, hipEventDisableTiming) != hipSuccess) {
            (void)hipEventDestroy(compressed);
            return ZC_EHIP;
        }
        bool ok = hipEventRecord(compressed, sc) == hipSuccess
                  && hipStreamWaitEvent(sl, compressed, 0) == hipSuccess;
        // 2. the link: the group's streams, comp_sizes bytes each
        for (int32_t b0 = c0; ok && b0 < c1; b0 += kMaxChunks) {
            const int32_t bm = std::min(c1 - b0, kMaxChunks);
            LinkTable lt;
            std::memset(&lt, 0, sizeof lt);
            for (int32_t i = 0; i < bm; ++i) {
                lt.slot[i] = soff[b0 + i] - soff[b0];
                lt.bound[i] = soff[b0 + i + 1] - soff[b0 + i];
            }
            const uint32_t bx = std::max(1u, 2048u / static_cast<uint32_t>(bm));
            hipLaunchKernelGGL(zc_link_copy_kernel, dim3(bx, static_cast<uint32_t>(bm)), dim3(kBlock),
                               0, sl, send + soff[b0], recv + soff[b0], d_comp_sizes + b0, lt);
            ok = hipGetLastError() == hipSuccess;
        }
        ok = ok && hipEventRecord(sent, sl) == hipSuccess
             && hipStreamWaitEvent(sd, sent, 0) == hipSuccess;
        // the waits have been queued: the events are released once they complete
        (void)hipEventDestroy(compressed);
        (void)hipEventDestroy(sent);
        if (!ok)
            return ZC_EHIP;
        // 3. decompress the group from the receiver's slots
        r = decompress_chunks(recv + soff[c0], gbytes, nullptr, counts + c0, m, d_out + voff[c0],
                              d_status, sd, c0);
        if (r != ZC_OK)
            return r;
    }
    return ZC_OK;
}

const char* zc_strerror(int code)
{
    switch (code) {
    case ZC_OK: return "ok";
    case ZC_EINVAL: return "invalid argument";
    case ZC_ENOSPC: return "output or workspace capacity too small";
    case ZC_ECORRUPT: return "corrupt stream";
    case ZC_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

int zc_code_table(int32_t table_id, int32_t* lengths, uint32_t* codes, double* prob)
{
    if (table_id != 1 || !lengths || !codes)
        return ZC_EINVAL;
    static std::once_flag once;
    static zc::Table tab;
    static bool ok = false;
    std::call_once(once, [] {
        ok = zc::build_table(&tab);
        static const uint32_t built_len[] = ZC_T1_LEN_INIT;
        static const uint32_t built_code[] = ZC_T1_CODE_INIT;
        static const uint32_t built_lut[] = ZC_T1_LUT_INIT;
        static const uint32_t built_tail[] = ZC_T1_TAIL_INIT;
        static_assert(sizeof(built_lut) / sizeof(built_lut[0]) == (1 << kLutBits), "lookup size");
        for (int s = 0; ok && s < ZC_T1_NSYM; ++s)
            ok = static_cast<uint32_t>(tab.len[s]) == built_len[s] && tab.code[s] == built_code[s];
        for (int i = 0; ok && i < (1 << kLutBits); ++i)
            ok = tab.lut[i] == built_lut[i];
        for (int i = 0; ok && i < (1 << kTailBits); ++i)
            ok = tab.tail[i] == built_tail[i] && tab.tail_ok;
    });
    if (!ok)
        return ZC_EINVAL;
    for (int s = 0; s < ZC_T1_NSYM; ++s) {
        lengths[s] = tab.len[s];
        codes[s] = tab.code[s];
        if (prob)
            prob[s] = tab.prob[s];
    }
    return ZC_OK;
}

}  // extern "C"
