// zc_kernels.hip -- gfx950 compress / decompress kernels and the C ABI.
//
// Method: ZipCCL (arXiv 2604.27844), abstract, techniques (1) and (2).  The
// bf16 exponent is coded relative to the largest exponent of its group with
// a fixed canonical prefix code derived from the Gaussian law (no run-time
// statistics); the sign+mantissa byte is stored raw, which is how a 16-bit
// value reaches about 11 bits (pith.science, Figure 6 caption).
//
// GPU mapping (MI355X, wave64):
//  * one wave owns one tile of 8192 values; lane l owns group 64t + l, whose
//    values are 8 consecutive bf16 (one 16-byte load) at each of 16 steps,
//    so every global load and store of the raw data is fully coalesced;
//  * the group maximum is lane-local (no cross-lane reduction);
//  * a wave prefix sum over the 64 group lengths places the lane streams,
//    which are packed into an LDS copy of the tile stream (the pages stage
//    data in shared memory, Figure 7 caption) and stored coalesced;
//  * the byte offset of a tile inside its chunk's exponent section is an
//    exclusive scan over the tiles of the chunk, done in the same pass with a
//    decoupled look-back over per-tile status words; tiles are taken from a
//    ticket counter, so every tile a wave waits on is already running;
//  * all chunks of a call form one flat list of tiles, so uneven chunk sizes
//    (the imbalance of Figure 8) still fill the GPU.
// No floating point runs on the device.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "zc.h"
#include "zc_table.h"
#include "zc_table_v1.inc"

namespace {

constexpr int kLanes = 64;
constexpr int kSteps = 16;
constexpr int kTile = 8192;
constexpr int kGroupVals = 128;
constexpr int kTileWords = kTile * 8 / 32;        // raw tile stream: 2048 words
constexpr int kMaxChunks = 64;                     // chunks per launch
constexpr uint32_t kMagic = 0x3142435Au;
constexpr uint32_t kVerTable = 0x00010001u;        // version 1, table_id 1
constexpr int kEsc = ZC_T1_NSYM - 1;
constexpr int kLutBits = 10;
constexpr uint64_t kFlagAgg = 1ull << 62;
constexpr uint64_t kFlagInc = 2ull << 62;

static_assert(ZC_T1_NSYM == 17, "table_id 1 has 17 symbols");
static_assert(ZC_T1_MAXLEN + 8 <= 32, "escape payload must fit the window");

__constant__ uint16_t c_lut[1 << kLutBits] = ZC_T1_LUT_INIT;
__constant__ uint32_t c_limit[25] = ZC_T1_LIMIT_INIT;
__constant__ uint32_t c_base[25] = ZC_T1_BASE_INIT;
__constant__ uint8_t c_sorted[ZC_T1_NSYM] = ZC_T1_SORTED_INIT;
__constant__ uint8_t c_len[ZC_T1_NSYM] = ZC_T1_LEN_INIT;
__constant__ uint32_t c_code[ZC_T1_NSYM] = ZC_T1_CODE_INIT;

// Chunks of one launch.  Work item = one tile; an empty chunk gets one item
// that only writes its header.
struct ChunkTable {
    int32_t nchunks;
    uint32_t nitems;
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

// ------------------------------------------------------------ compress

__global__ void zc_clear_kernel(uint64_t* __restrict__ p, uint32_t words)
{
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += gridDim.x * blockDim.x)
        p[i] = 0;
}

__global__ __launch_bounds__(kLanes)
void zc_compress_kernel(const uint16_t* __restrict__ in, uint8_t* __restrict__ out,
                        int64_t* __restrict__ comp_sizes,
                        uint64_t* __restrict__ status, uint32_t* __restrict__ ticket,
                        ChunkTable tab)
{
    __shared__ uint32_t s_bits[kTileWords + 1];
    __shared__ uint32_t s_enc[256];   // d -> code | len << 24 (d >= 16: ESC)

    const uint32_t lane = threadIdx.x;
    for (uint32_t d = lane; d < 256; d += kLanes) {
        const int s = d < kEsc ? static_cast<int>(d) : kEsc;
        uint32_t code = c_code[s], len = c_len[s];
        if (s == kEsc) {
            code <<= 8;               // payload: the exponent, 8 bits
            len += 8;
        }
        s_enc[d] = code | (len << 24);
    }

    uint32_t item = 0;
    if (lane == 0)
        item = atomicAdd(ticket, 1u);
    item = __builtin_amdgcn_readfirstlane(item);

    const int c = find_chunk(tab, item);
    const uint32_t n = tab.n[c];
    const uint32_t t = item - tab.item_begin[c];
    const uint16_t* src = in + tab.voff[c];
    uint8_t* dst = out + tab.boff[c];
    const Geom G = geometry(n);

    if (n == 0) {
        if (lane < 8)
            reinterpret_cast<uint32_t*>(dst)[lane] = header_word(lane, 0, 32);
        if (lane == 0)
            comp_sizes[c] = 32;
        return;
    }

    const uint32_t base = t * kTile;
    const uint32_t rem = min(n - base, static_cast<uint32_t>(kTile));
    const bool vec = rem == kTile && ((reinterpret_cast<uintptr_t>(src) & 15) == 0);
    const uint32_t ng = group_members(rem, lane);

    // 1. load, split, raw bytes out, exponents kept packed 4 per word
    uint32_t ex[kSteps][2];
    uint32_t mx = 0;
#pragma unroll
    for (int k = 0; k < kSteps; ++k) {
        const uint32_t i0 = base + k * 512 + lane * 8;
        uint4 v;
        if (vec) {
            v = *reinterpret_cast<const uint4*>(src + i0);
        } else {
            uint32_t w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                w[j] = (i0 + j < n) ? src[i0 + j] : 0u;
            v.x = w[0] | (w[1] << 16);
            v.y = w[2] | (w[3] << 16);
            v.z = w[4] | (w[5] << 16);
            v.w = w[6] | (w[7] << 16);
        }
        const uint32_t lo_a = __builtin_amdgcn_perm(v.y, v.x, 0x06040200u);
        const uint32_t hi_a = __builtin_amdgcn_perm(v.y, v.x, 0x07050301u);
        const uint32_t lo_b = __builtin_amdgcn_perm(v.w, v.z, 0x06040200u);
        const uint32_t hi_b = __builtin_amdgcn_perm(v.w, v.z, 0x07050301u);
        const uint32_t raw_a = (hi_a & 0x80808080u) | (lo_a & 0x7F7F7F7Fu);
        const uint32_t raw_b = (hi_b & 0x80808080u) | (lo_b & 0x7F7F7F7Fu);
        ex[k][0] = ((hi_a << 1) & 0xFEFEFEFEu) | ((lo_a >> 7) & 0x01010101u);
        ex[k][1] = ((hi_b << 1) & 0xFEFEFEFEu) | ((lo_b >> 7) & 0x01010101u);
        mx = max(mx, max(max(v.x & 0x7F80u, (v.x >> 16) & 0x7F80u),
                         max(v.y & 0x7F80u, (v.y >> 16) & 0x7F80u)));
        mx = max(mx, max(max(v.z & 0x7F80u, (v.z >> 16) & 0x7F80u),
                         max(v.w & 0x7F80u, (v.w >> 16) & 0x7F80u)));
        uint8_t* rdst = dst + G.R + i0;
        if (vec) {
            *reinterpret_cast<uint2*>(rdst) = make_uint2(raw_a, raw_b);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (i0 + j < n)
                    rdst[j] = static_cast<uint8_t>(((j < 4 ? raw_a : raw_b) >> (8 * (j & 3))) & 0xFF);
        }
    }
    const uint32_t emax = mx >> 7;   // missing members were loaded as 0

    __syncthreads();                 // s_enc ready

    // 2. coded length of the group, raw decision
    uint32_t bits = 0;
#pragma unroll 1
    for (int k = 0; k < kSteps; ++k) {
        const uint32_t e4[2] = {ex[k][0], ex[k][1]};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t e = (e4[j >> 2] >> (8 * (j & 3))) & 0xFF;
            const uint32_t L = s_enc[emax - e] >> 24;
            bits += (static_cast<uint32_t>(k * 8 + j) < ng) ? L : 0u;
        }
    }
    const bool raw_mode = ng > 0 && bits >= 8 * ng;
    const uint32_t glen = raw_mode ? 8 * ng : bits;

    // 3. lane offsets inside the tile stream, tile size
    uint32_t tile_bits;
    const uint32_t off = wave_excl_scan(glen, lane, &tile_bits);
    const uint32_t tile_words = (tile_bits + 31) >> 5;
    const uint32_t tile_bytes = tile_words * 4;

    // 4. decoupled look-back over the tiles of this chunk
    uint32_t toff = 0;
    const uint32_t first = tab.item_begin[c];
    if (t == 0) {
        if (lane == 0)
            __hip_atomic_store(&status[item], kFlagInc | tile_bytes, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else {
        if (lane == 0)
            __hip_atomic_store(&status[item], kFlagAgg | tile_bytes, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        int64_t top = static_cast<int64_t>(item) - 1;
        uint32_t acc = 0;
        while (true) {
            const int64_t idx = top - static_cast<int64_t>(lane);
            const bool in_range = idx >= static_cast<int64_t>(first);
            uint64_t s = 0;
            if (in_range)
                s = __hip_atomic_load(&status[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t flag = static_cast<uint32_t>(s >> 62);
            const uint64_t inc_mask = __ballot(in_range && flag == 2);
            const uint64_t zero_mask = __ballot(in_range && flag == 0);
            if (inc_mask) {
                const int p = __ffsll(static_cast<unsigned long long>(inc_mask)) - 1;
                const uint64_t below = (p == 0) ? 0ull : ((1ull << p) - 1);
                if (zero_mask & below) {
                    __builtin_amdgcn_s_sleep(1);
                    continue;
                }
                acc += wave_sum(lane <= static_cast<uint32_t>(p) ? static_cast<uint32_t>(s) : 0u);
                break;
            }
            if (zero_mask) {
                __builtin_amdgcn_s_sleep(1);
                continue;
            }
            acc += wave_sum(static_cast<uint32_t>(s));
            top -= kLanes;
        }
        toff = acc;
        if (lane == 0)
            __hip_atomic_store(&status[item], kFlagInc | (toff + tile_bytes), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }

    // 5. index arrays
    if (lane == 0)
        *reinterpret_cast<uint32_t*>(dst + 32 + 4ull * t) = toff;
    dst[32 + 4ull * G.T + 64ull * t + lane] = static_cast<uint8_t>(emax);
    *reinterpret_cast<uint16_t*>(dst + 32 + 68ull * G.T + 2ull * (64ull * t + lane)) =
        static_cast<uint16_t>(glen);

    // 6. pack the lane streams into the LDS tile stream, MSB first
    for (uint32_t w = lane; w < tile_words; w += kLanes)
        s_bits[w] = 0;
    __syncthreads();
    {
        uint64_t acc = 0;
        uint32_t nacc = off & 31;
        uint32_t wi = off >> 5;
#pragma unroll 1
        for (int k = 0; k < kSteps; ++k) {
            const uint32_t e4[2] = {ex[k][0], ex[k][1]};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (static_cast<uint32_t>(k * 8 + j) < ng) {
                    const uint32_t e = (e4[j >> 2] >> (8 * (j & 3))) & 0xFF;
                    uint32_t code, L;
                    if (raw_mode) {
                        code = e;
                        L = 8;
                    } else {
                        const uint32_t d = emax - e;
                        const uint32_t ent = s_enc[d];
                        L = ent >> 24;
                        code = (ent & 0xFFFFFFu) | (d >= static_cast<uint32_t>(kEsc) ? e : 0u);
                    }
                    acc = (acc << L) | code;
                    nacc += L;
                    if (nacc >= 32) {
                        nacc -= 32;
                        atomicOr(&s_bits[wi], static_cast<uint32_t>(acc >> nacc));
                        ++wi;
                    }
                }
            }
        }
        if (nacc)
            atomicOr(&s_bits[wi], static_cast<uint32_t>(acc << (32 - nacc)));
    }
    __syncthreads();

    // 7. coalesced store of the tile stream
    uint32_t* sdst = reinterpret_cast<uint32_t*>(dst + G.X + toff);
    for (uint32_t w = lane; w < tile_words; w += kLanes)
        sdst[w] = s_bits[w];

    // 8. the last tile finishes the chunk: header, gaps, size
    if (t == G.T - 1) {
        const uint64_t comp = G.X + toff + tile_bytes;
        if (lane < 8)
            reinterpret_cast<uint32_t*>(dst)[lane] = header_word(lane, n, comp);
        const uint64_t g1 = 32 + 196ull * G.T;
        if (g1 + lane < G.R)
            dst[g1 + lane] = 0;
        if (G.R + n + lane < G.X)
            dst[G.R + n + lane] = 0;
        if (lane == 0)
            comp_sizes[c] = static_cast<int64_t>(comp);
    }
}

// ------------------------------------------------------------ decompress

__device__ inline void report(int32_t* status, int reason, int c)
{
    atomicCAS(status, 0, (reason << 24) | (c & 0xFFFFFF));
}

__global__ __launch_bounds__(kLanes)
void zc_decompress_kernel(const uint8_t* __restrict__ in, uint16_t* __restrict__ out,
                          int32_t* __restrict__ status, ChunkTable tab)
{
    __shared__ uint32_t s_bits[kTileWords + 2];
    __shared__ uint16_t s_lut[1 << kLutBits];
    __shared__ uint8_t s_len[ZC_T1_NSYM];

    const uint32_t lane = threadIdx.x;
    for (uint32_t i = lane; i < (1u << kLutBits); i += kLanes)
        s_lut[i] = c_lut[i];
    if (lane < ZC_T1_NSYM)
        s_len[lane] = c_len[lane];

    const uint32_t item = blockIdx.x;
    const int c = find_chunk(tab, item);
    const uint32_t n = tab.n[c];
    const uint32_t t = item - tab.item_begin[c];
    const uint8_t* src = in + tab.boff[c];
    uint16_t* dst = out + tab.voff[c];
    const Geom G = geometry(n);

    // header (the host has checked that 32 bytes are readable)
    const uint32_t hw = lane < 8 ? reinterpret_cast<const uint32_t*>(src)[lane] : 0u;
    const uint32_t h0 = __shfl(hw, 0), h1 = __shfl(hw, 1), h2 = __shfl(hw, 2),
                   h3 = __shfl(hw, 3), h4 = __shfl(hw, 4), h5 = __shfl(hw, 5),
                   h6 = __shfl(hw, 6), h7 = __shfl(hw, 7);
    if (h0 != kMagic || h1 != kVerTable || h2 != 0 || h3 != 0 || h4 != n || h5 != 0) {
        if (lane == 0)
            report(status, ZC_REASON_HEADER, c);
        return;
    }
    const uint64_t comp = h6 | (static_cast<uint64_t>(h7) << 32);
    if (comp < G.X || comp > tab.bavail[c] || comp > chunk_bound(n)) {
        if (lane == 0)
            report(status, ZC_REASON_SIZE, c);
        return;
    }
    if (n == 0)
        return;

    // tile extent
    const uint32_t* toffs = reinterpret_cast<const uint32_t*>(src + 32);
    const uint32_t toff = toffs[t];
    const uint64_t next = (t + 1 < G.T) ? toffs[t + 1] : comp - G.X;
    const uint32_t base = t * kTile;
    const uint32_t rem = min(n - base, static_cast<uint32_t>(kTile));
    if ((t == 0 && toff != 0) || toff > next || next > comp - G.X) {
        if (lane == 0)
            report(status, ZC_REASON_TILE, c);
        return;
    }
    const uint32_t tile_bytes = static_cast<uint32_t>(next - toff);

    // group metadata
    const uint32_t ng = group_members(rem, lane);
    const uint32_t emax = src[32 + 4ull * G.T + 64ull * t + lane];
    const uint32_t glen =
        *reinterpret_cast<const uint16_t*>(src + 32 + 68ull * G.T + 2ull * (64ull * t + lane));
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

    // stage the tile stream in LDS (plus two zero guard words)
    const uint32_t* ssrc = reinterpret_cast<const uint32_t*>(src + G.X + toff);
    for (uint32_t w = lane; w < tile_words; w += kLanes)
        s_bits[w] = ssrc[w];
    if (lane < 2)
        s_bits[tile_words + lane] = 0;
    __syncthreads();

    int err = 0;
    if ((tile_bits & 31) && lane == 0) {
        const uint32_t last = s_bits[tile_words - 1];
        if (last & ((1u << (32 - (tile_bits & 31))) - 1))
            err = ZC_REASON_PADDING;
    }
    if (t == 0) {
        const uint64_t g1 = 32 + 196ull * G.T;
        if (g1 + lane < G.R && src[g1 + lane] != 0)
            err = ZC_REASON_GAP;
    }
    if (t == G.T - 1) {
        if (G.R + n + lane < G.X && src[G.R + n + lane] != 0)
            err = ZC_REASON_GAP;
    }

    const bool raw_mode = ng > 0 && glen == 8 * ng;
    const bool vec_out = rem == kTile && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0);
    const uint8_t* rsrc = src + G.R;
    uint32_t pos = off;
    const uint32_t end = off + glen;
    uint32_t seen_max = 0, coded_len = 0;

#pragma unroll 1
    for (int k = 0; k < kSteps; ++k) {
        uint32_t e8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t e = 0;
            if (static_cast<uint32_t>(k * 8 + j) < ng && err == 0) {
                if (pos >= end) {
                    err = ZC_REASON_LENGTH;
                } else {
                    const uint32_t w0 = s_bits[pos >> 5], w1 = s_bits[(pos >> 5) + 1];
                    const uint32_t sh = pos & 31;
                    const uint32_t win = sh ? (w0 << sh) | (w1 >> (32 - sh)) : w0;
                    if (raw_mode) {
                        e = win >> 24;
                        pos += 8;
                        const uint32_t d = emax - e;   // may wrap: then >= 16
                        coded_len += d < static_cast<uint32_t>(kEsc) ? s_len[d] : s_len[kEsc] + 8u;
                    } else {
                        uint32_t ent = s_lut[win >> (32 - kLutBits)];
                        uint32_t sym, L;
                        if (ent != 0) {
                            sym = ent >> 8;
                            L = ent & 0xFF;
                        } else {
                            sym = 0xFFFFFFFFu;
                            L = 0;
                            for (uint32_t l = kLutBits + 1; l <= ZC_T1_MAXLEN; ++l) {
                                const uint32_t v = win >> (32 - l);
                                if (v < c_limit[l]) {
                                    const uint32_t rank = v - c_base[l];
                                    sym = c_sorted[rank < ZC_T1_NSYM ? rank : ZC_T1_NSYM - 1];
                                    L = l;
                                    break;
                                }
                            }
                        }
                        if (sym == 0xFFFFFFFFu) {
                            err = ZC_REASON_SYMBOL;
                        } else if (sym == static_cast<uint32_t>(kEsc)) {
                            e = (win >> (32 - L - 8)) & 0xFF;
                            L += 8;
                            if (e + kEsc > emax)
                                err = ZC_REASON_ESCAPE;
                        } else if (sym > emax) {
                            err = ZC_REASON_SYMBOL;
                        } else {
                            e = emax - sym;
                        }
                        pos += L;
                        if (pos > end && err == 0)
                            err = ZC_REASON_SYMBOL;
                    }
                    seen_max = max(seen_max, e);
                }
            }
            e8[j] = e;
        }
        const uint32_t i0 = base + k * 512 + lane * 8;
        if (vec_out) {
            const uint2 rw = *reinterpret_cast<const uint2*>(rsrc + i0);
            uint4 o;
            o.x = (__builtin_amdgcn_perm(rw.x, rw.x, 0x01010000u) & 0x807F807Fu) | (e8[0] << 7) | (e8[1] << 23);
            o.y = (__builtin_amdgcn_perm(rw.x, rw.x, 0x03030202u) & 0x807F807Fu) | (e8[2] << 7) | (e8[3] << 23);
            o.z = (__builtin_amdgcn_perm(rw.y, rw.y, 0x01010000u) & 0x807F807Fu) | (e8[4] << 7) | (e8[5] << 23);
            o.w = (__builtin_amdgcn_perm(rw.y, rw.y, 0x03030202u) & 0x807F807Fu) | (e8[6] << 7) | (e8[7] << 23);
            *reinterpret_cast<uint4*>(dst + i0) = o;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (i0 + j < n) {
                    const uint32_t r = rsrc[i0 + j];
                    dst[i0 + j] = static_cast<uint16_t>(((r & 0x80u) << 8) | (e8[j] << 7) | (r & 0x7Fu));
                }
            }
        }
    }
    if (err == 0 && ng > 0) {
        if (raw_mode) {
            if (seen_max != emax)
                err = ZC_REASON_EMAX;
            else if (coded_len < 8 * ng)
                err = ZC_REASON_RAWMODE;
        } else {
            if (pos != end)
                err = ZC_REASON_LENGTH;
            else if (seen_max != emax)
                err = ZC_REASON_EMAX;
        }
    }
    if (err)
        report(status, err, c);
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
    if (num_chunks < 0 || (num_chunks > 0 && !counts))
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

uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

constexpr size_t kWsHeader = 256;   // ticket counter(s)

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
    return static_cast<size_t>(kWsHeader + 8 * most);
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
    uint32_t* ticket = static_cast<uint32_t*>(d_ws);
    uint64_t* status = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(d_ws) + kWsHeader);
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
        tab.nitems = items;
        tab.item_begin[m] = items;

        // the ticket word and the look-back status words start at zero
        const uint32_t words = items + static_cast<uint32_t>(kWsHeader / 8);
        const uint32_t cblocks = (words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024;
        hipLaunchKernelGGL(zc_clear_kernel, dim3(cblocks), dim3(256), 0, s,
                           static_cast<uint64_t*>(d_ws), words);
        hipLaunchKernelGGL(zc_compress_kernel, dim3(items), dim3(kLanes), 0, s, d_in, out,
                           d_comp_sizes + c0, status, ticket, tab);
        if (hipGetLastError() != hipSuccess)
            return ZC_EHIP;
    }
    return ZC_OK;
}

int zc_decompress(const void* d_in, size_t in_bytes, const int64_t* in_offsets,
                  const int64_t* counts, int32_t num_chunks, uint16_t* d_out,
                  int32_t* d_status, void* stream)
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
            items += static_cast<uint32_t>(T ? T : 1);
            voff += n;
            slot += align256(chunk_bound(n));
        }
        tab.nchunks = m;
        tab.nitems = items;
        tab.item_begin[m] = items;
        hipLaunchKernelGGL(zc_decompress_kernel, dim3(items), dim3(kLanes), 0, s, in, d_out,
                           d_status, tab);
        if (hipGetLastError() != hipSuccess)
            return ZC_EHIP;
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
        for (int s = 0; ok && s < ZC_T1_NSYM; ++s)
            ok = static_cast<uint32_t>(tab.len[s]) == built_len[s] && tab.code[s] == built_code[s];
        for (int i = 0; ok && i < (1 << kLutBits); ++i)
            ok = tab.lut[i] == built_lut[i];
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
