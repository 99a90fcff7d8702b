// splitzip_device.h -- device helpers shared by the gfx950 kernels of the SplitZip codec
// (BF16 words and FP8 E5M2 bytes): streaming memory access, wave64 prefix sums and lane
// exchange, byte permutes, XCD-aware tile order, segment lookup of ragged batches, and the
// in-tile escape ranking and escape destination of the pack kernels, and the look-back of
// the one-pass encode.
#pragma once

#include "splitzip_internal.h"

namespace sz {
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// 12-byte vectors (the E5M2 field stream) sit at 4-byte-aligned addresses
typedef unsigned int u32x3 __attribute__((ext_vector_type(3), aligned(4)));

// Pointers read from a segment table are generic to the compiler, which then emits flat
// memory instructions; flat accesses also count against the LDS wait counter, so a wait for
// an LDS read would wait for them too.  Every caller buffer is device (global) memory: the
// streaming accesses below say so, and become global loads and stores.
#define SZ_GLOBAL __attribute__((address_space(1)))

template <typename T>
__device__ __forceinline__ SZ_GLOBAL T *as_global(T *p)
{
    return (SZ_GLOBAL T *)p;
}

template <typename T>
__device__ __forceinline__ const SZ_GLOBAL T *as_global(const T *p)
{
    return (const SZ_GLOBAL T *)p;
}

// Streaming accesses of the pack and decode kernels: every byte is touched once, so the loads
// and stores carry the nontemporal hint and do not displace other data in the caches.
__device__ __forceinline__ uint4 load_stream16(const void *p)
{
    const u32x4 t = __builtin_nontemporal_load(as_global(reinterpret_cast<const u32x4 *>(p)));
    return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void store_stream16(void *p, uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    const u32x4 t = {a, b, c, d};
    __builtin_nontemporal_store(t, as_global(reinterpret_cast<u32x4 *>(p)));
}

__device__ __forceinline__ void store_stream12(void *p, uint32_t a, uint32_t b, uint32_t c)
{
    const u32x3 t = {a, b, c};
    __builtin_nontemporal_store(t, (SZ_GLOBAL u32x3 *)p);     // keeps the 4-byte alignment
}

__device__ __forceinline__ void store_stream8(void *p, uint32_t lo, uint32_t hi)
{
    const u32x2 t = {lo, hi};
    __builtin_nontemporal_store(t, as_global(reinterpret_cast<u32x2 *>(p)));
}

__device__ __forceinline__ void store_stream4(void *p, uint32_t x)
{
    __builtin_nontemporal_store(x, as_global(reinterpret_cast<uint32_t *>(p)));
}

// ---- small wave64 helpers -------------------------------------------------------------

__device__ __forceinline__ uint32_t lane_id()
{
    return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// A 64-bit value that is the same in every lane, as scalar registers.  (The builtin returns
// int: each half goes through uint32_t, or the low half would be sign-extended into the high
// one when the two are combined.)
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t shfl_u32(uint32_t v, uint32_t src_lane)
{
    return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(src_lane << 2), (int)v);
}

// Inclusive prefix sum over the 64 lanes (all lanes must be active).  Used on words that
// pack two 16-bit counters whose sums stay below 65536.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v, uint32_t lane)
{
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1) {
        uint32_t t = shfl_u32(v, lane >= d ? lane - d : lane);
        if (lane >= d)
            v += t;
    }
    return v;
}

__device__ __forceinline__ uint64_t wave_total_u64(uint64_t v, uint32_t lane)
{
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1) {
        uint32_t lo = shfl_u32((uint32_t)v, lane ^ d);
        uint32_t hi = shfl_u32((uint32_t)(v >> 32), lane ^ d);
        v += ((uint64_t)hi << 32) | lo;
    }
    return v;
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    // v_perm_b32: selector byte s picks byte s of the 8-byte value {hi, lo} (s < 8).
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// A compile-time flag passed to generic lambdas.
template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// Set-bit table of the one-pass packs: entry m (an 8-bit mask) holds the indices of m's set
// bits, lowest first, one per byte (0 past the last).
__device__ __forceinline__ uint2 set_bit_indices(uint32_t m)
{
    uint64_t e = 0;
    uint32_t c = 0;
#pragma unroll
    for (uint32_t b = 0; b < 8; ++b)
        if ((m >> b) & 1u) {
            e |= (uint64_t)b << (8 * c);
            ++c;
        }
    return make_uint2((uint32_t)e, (uint32_t)(e >> 32));
}

// Entry k (0..15) of a codebook held as 4 little-endian dwords.
__device__ __forceinline__ uint32_t codebook_byte(const uint32_t cb[4], uint32_t k)
{
    const bool upper = (k & 8u) != 0;
    return __builtin_amdgcn_perm(upper ? cb[3] : cb[1], upper ? cb[2] : cb[0], k & 7u) & 0xFFu;
}

// Workgroups are started round robin over the 8 XCDs (workgroup b on XCD b mod 8).  Giving
// each XCD a contiguous range of tiles instead of every 8th one streams measurably better
// (about 3 % in a copy probe).  The mapping is a bijection on [0, n_tiles) whatever the
// hardware does; extra workgroups of the rounded-up grid find t >= n_tiles and exit.
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint32_t xcd_tile(uint32_t b, uint32_t n_tiles)
{
    const uint32_t per_xcd = (n_tiles + kXcds - 1) / kXcds;
    return (b % kXcds) * per_xcd + b / kXcds;
}

static inline uint32_t xcd_grid(uint32_t n_tiles) { return (n_tiles + kXcds - 1) / kXcds * kXcds; }

// Segment that owns global tile t: the largest s with tile_start[s] <= t.
// By one thread: a binary search over tile_start limited to the bracket
// that seg_at gives (usually a single segment, so no load at all).
__device__ __forceinline__ uint32_t find_segment(const uint32_t *tile_start, const uint32_t *seg_at,
                                                 uint32_t t)
{
    uint32_t lo = seg_at[t >> kSegAtShift];
    uint32_t hi = seg_at[(t >> kSegAtShift) + 1] + 1;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (tile_start[mid] <= t)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// Segment of tile t, found by the whole workgroup: seg_at brackets it, and the segments
// inside the bracket (usually none) are counted with one round of independent loads, the
// number of s in the bracket with tile_start[s] <= t.  Call from uniform control flow with t
// uniform; contains barriers when the bracket holds more than one segment.
__device__ uint32_t find_segment_block(const uint32_t *tile_start, const uint32_t *seg_at, uint32_t t,
                                       uint32_t tid, uint32_t lane, uint32_t *s_cnt)
{
    const uint32_t s0 = seg_at[t >> kSegAtShift];
    const uint32_t s1 = seg_at[(t >> kSegAtShift) + 1];
    if (s0 == s1)
        return s0;
    uint32_t c = 0;
    for (uint32_t k = s0 + 1 + tid; k <= s1; k += kThreads)
        c += tile_start[k] <= t ? 1u : 0u;
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1)
        c += shfl_u32(c, lane ^ d);
    if (lane == 0)
        s_cnt[tid >> 6] = c;
    __syncthreads();
    uint32_t seg = s0;
    for (int w = 0; w < kWaves; ++w)
        seg += s_cnt[w];
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(seg);
}

// Index s of a sorted start array with starts[s] <= b < starts[s + 1], by the whole workgroup
// with one round of loads over all n entries (the calibration histograms, where n is the
// number of tensors).  Call from uniform control flow; contains barriers.
__device__ uint32_t find_range_block(const uint32_t *starts, uint32_t n, uint32_t b, uint32_t tid,
                                     uint32_t lane, uint32_t *s_cnt)
{
    uint32_t c = 0;
    for (uint32_t k = 1 + tid; k < n; k += kThreads)
        c += starts[k] <= b ? 1u : 0u;
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1)
        c += shfl_u32(c, lane ^ d);
    if (lane == 0)
        s_cnt[tid >> 6] = c;
    __syncthreads();
    uint32_t r = 0;
    for (int w = 0; w < kWaves; ++w)
        r += s_cnt[w];
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(r);
}

// Segment of global tile t (uniform when t is).
__device__ __forceinline__ uint32_t tile_segment(const EncodeArgs &a, uint32_t t)
{
    return a.n_seg > 1 ? find_segment(a.tile_start, a.seg_at, t) : 0u;
}

// A word of a table no kernel writes while it runs, read through the scalar data cache (a
// load from the constant address space): the wait for it is not a wait for this wave's
// vector memory operations.
__device__ __forceinline__ uint32_t load_const_u32(const uint32_t *p, uint32_t i)
{
    return ((const __attribute__((address_space(4))) uint32_t *)p)[i];
}

__device__ __forceinline__ uint32_t segment_first_tile(const EncodeArgs &a, uint32_t s)
{
    return a.n_seg > 1 ? load_const_u32(a.tile_start, s) : 0u;
}

__device__ __forceinline__ uint32_t segment_end_tile(const EncodeArgs &a, uint32_t s)
{
    return a.n_seg > 1 ? load_const_u32(a.tile_start, s + 1) : a.n_tiles;
}

// Descriptor s of a segment table the host wrote before the launch (s uniform): a read
// through the constant address space, so scalar loads, not vector loads that the wave's
// later loads would queue behind.
__device__ __forceinline__ SegDesc load_const_segdesc(const SegDesc *segs, uint32_t s)
{
    static_assert(sizeof(SegDesc) % 4 == 0, "whole dwords");
    constexpr uint32_t kWords = sizeof(SegDesc) / 4;
    const uint32_t *p = reinterpret_cast<const uint32_t *>(segs + s);
    uint32_t w[kWords];
#pragma unroll
    for (uint32_t k = 0; k < kWords; ++k)
        w[k] = load_const_u32(p, k);
    SegDesc d;
    __builtin_memcpy(&d, w, sizeof(d));
    return d;
}

__device__ __forceinline__ SegDesc segment_desc(const EncodeArgs &a, uint32_t s)
{
    if (a.n_seg > 1)
        return load_const_segdesc(a.segs, s);
    return a.seg0;
}

// ---- pack kernels: escape ranks inside a tile and where the tile's escapes go -----------

// Escape ranks inside a tile whose lanes hold G groups each, in word order (wave, group j,
// lane, position inside the group).  counts[j]: escapes of the lane's group j (at most
// 65535 per group and wave).  Per-group counts are packed two per dword (16-bit fields) and
// prefix-summed over the lanes; each group is then offset by the wave totals of the groups
// before it, and the waves by the totals of the earlier waves (through LDS).  rank[j]: the
// escapes before the lane's group j within the tile.  Contains a barrier.
template <int G>
__device__ __forceinline__ void tile_escape_ranks(const uint32_t (&counts)[G], uint32_t lane,
                                                  uint32_t wave, uint32_t *s_wave_total,
                                                  uint32_t (&rank)[G], uint32_t &tile_total,
                                                  uint32_t &wave_end)
{
    static_assert(G % 2 == 0, "groups are ranked in pairs");
    uint32_t wave_sum = 0;
#pragma unroll
    for (int j = 0; j < G; j += 2) {
        const uint32_t packed = counts[j] | (counts[j + 1] << 16);
        const uint32_t incl = wave_inclusive_sum(packed, lane);
        const uint32_t excl = incl - packed;
        const uint32_t tot = __builtin_amdgcn_readlane(incl, 63);
        rank[j] = wave_sum + (excl & 0xFFFFu);
        wave_sum += tot & 0xFFFFu;
        rank[j + 1] = wave_sum + (excl >> 16);
        wave_sum += tot >> 16;
    }
    if (lane == 0)
        s_wave_total[wave] = wave_sum;
    __syncthreads();
    uint32_t wave_base = 0;
    tile_total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t x = s_wave_total[w];
        wave_base += (w < (int)wave) ? x : 0u;
        tile_total += x;
    }
#pragma unroll
    for (int j = 0; j < G; ++j)
        rank[j] += wave_base;
    wave_end = wave_base + wave_sum;
}

// Where tile t's escapes go: its slot of a.slot_escapes entries, or, past that, the tile's
// own region of the overflow area (calls with private_ovf) or a range of it reserved with one
// 64-bit atomic that also appends the tile to the overflow list.  room: entries that may be
// written there.  Also stores the tile's escape count.  Call from uniform control flow
// (contains a barrier when the tile overflows).
__device__ __forceinline__ uint32_t *tile_escape_dest(const EncodeArgs &a, uint32_t t,
                                                      uint32_t tile_total, uint32_t tid,
                                                      uint64_t *s_ovf, uint64_t &room)
{
    uint32_t *dst = a.slots + (uint64_t)t * a.slot_escapes;
    room = a.slot_escapes;
    if (tile_total > a.slot_escapes && a.private_ovf) {
        // the tile's own region, as long as the tile: nothing to reserve
        const uint64_t off = (uint64_t)t << a.tile_shift;
        if (tid == 0)
            a.tile_ovf[t] = off;
        dst = a.ovf + off;
        room = 1ull << a.tile_shift;
    } else if (tile_total > a.slot_escapes) {
        if (tid == 0) {
            const uint64_t old = atomicAdd(a.ovf_ctr, (unsigned long long)tile_total + (1ull << kOvfTileShift));
            const uint64_t off = old & kOvfOffsetMask;
            *s_ovf = off;
            a.tile_ovf[t] = off;
            a.ovf_tiles[old >> kOvfTileShift] = t;
            if (off + tile_total > a.ovf_cap)
                atomicOr(a.err, kErrOverflowArea);
        }
        __syncthreads();
        // the same in every lane: keep it in scalar registers
        const uint64_t v = *s_ovf;
        const uint64_t off = uniform_u64(v);
        dst = a.ovf + off;
        room = off < a.ovf_cap ? a.ovf_cap - off : 0;
    }
    if (tid == 0)
        a.tile_count[t] = tile_total;
    return dst;
}

// ---- one-pass encode: copies from the LDS stash to the final arrays -----------------------

// Four dwords of LDS starting at byte offset o (any alignment): five aligned dword loads,
// realigned by byte funnel shifts.
__device__ __forceinline__ u32x4 lds_load16_unaligned(const uint8_t *lds, uint32_t o)
{
    const uint32_t *w = reinterpret_cast<const uint32_t *>(lds + (o & ~3u));
    const uint32_t m = o & 3u;
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3], w4 = w[4];
    const u32x4 r = {__builtin_amdgcn_alignbyte(w1, w0, m), __builtin_amdgcn_alignbyte(w2, w1, m),
                     __builtin_amdgcn_alignbyte(w3, w2, m), __builtin_amdgcn_alignbyte(w4, w3, m)};
    return r;
}

// dst[0, ne) = src[0, ne) for elements of kBytes (1 or 2) bytes, src in LDS, by one wave: the
// destination is cut at its 16-byte boundaries; each lane stores whole 16-byte pieces, and
// the elements before the first boundary and after the last are stored one per lane.  dst
// must be kBytes-aligned; the LDS from 16 bytes before src to 19 bytes past its end is read
// (and those bytes not stored).
template <int kBytes, typename T>
__device__ __forceinline__ void stash_copy(SZ_GLOBAL T *dst, const T *src, uint32_t ne, uint32_t lane)
{
    constexpr uint32_t kPer = 16 / kBytes;
    const uint32_t lead = (uint32_t)(reinterpret_cast<uintptr_t>(dst) & 15u) / kBytes;
    const uint32_t head = lead ? (kPer - lead < ne ? kPer - lead : ne) : 0u;   // before the first boundary
    const uint32_t full = (ne - head) / kPer;
    const uint32_t tail_at = head + full * kPer;
    const uint8_t *sb = reinterpret_cast<const uint8_t *>(src) - 16;
#pragma unroll 2
    for (uint32_t j = lane; j < full; j += 64) {
        const uint32_t i0 = head + j * kPer;
        *reinterpret_cast<SZ_GLOBAL u32x4 *>(dst + i0) = lds_load16_unaligned(sb, 16 + i0 * kBytes);
    }
    if (lane < head)
        dst[lane] = src[lane];
    if (lane < ne - tail_at)
        dst[tail_at + lane] = src[tail_at + lane];
}

// One-pass encode, early release: a tile's escapes past its stash (rank kStash and up, in a tile
// of kTileElems elements), written by the waves that hold them once wave 0 has copied the stash
// out (*s_out set, the tile's escape offset in *s_before).  When a tile holds at most twice the
// stash, each such wave puts them in the stash at rank - kStash (the waves' ranges do not
// overlap) and copies its range out; in longer tiles each owns a quarter of the stash and sends
// them through it a quarter at a time.  A wave's escapes have ranks wave_first .. wave_end - 1;
// stash(tag, lo, hi, at) puts the calling wave's escapes of rank lo .. hi - 1 in the stash at
// rank - lo + at.  The wait is bounded (kChainSpinMax polls, then an error bit), so every wave
// ends.
template <uint32_t kStash, uint32_t kTileElems, typename Stash>
__device__ __forceinline__ void stash_rest(const EncodeArgs &a, const SegDesc &sd, const uint32_t *s_out,
                                           const uint64_t *s_before, uint32_t wave, uint32_t wave_first,
                                           uint32_t wave_end, uint32_t lane, uint16_t *s_pos, uint8_t *s_exp,
                                           Stash &&stash)
{
    static_assert(kStash % kWaves == 0 && kTileElems % kStash == 0, "stash parts");
    uint32_t polls = 0;
    while (__hip_atomic_load(s_out, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u) {
        if (++polls > kChainSpinMax) {
            if (lane == 0)
                atomicOr(a.err, kErrChainStall);
            return;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    const uint64_t sb = *s_before;
    const uint64_t before = uniform_u64(sb);
    const uint64_t left = sd.esc > before && sd.esc_exp ? sd.esc - before : 0;
    const uint32_t end = (uint64_t)wave_end < left ? wave_end : (uint32_t)left;
    const uint32_t lo0 = wave_first > kStash ? wave_first : kStash;
    if (kTileElems <= 2 * kStash) {
        if (lo0 >= end)
            return;
        stash(BoolTag<true>{}, kStash, 2 * kStash, 0u);
        stash_copy<2>(as_global(sd.esc_pos + before + lo0), s_pos + (lo0 - kStash), end - lo0, lane);
        stash_copy<1>(as_global(sd.esc_exp + before + lo0), s_exp + (lo0 - kStash), end - lo0, lane);
        return;
    }
    // (a loop with a trip count known at compile time: in a loop of unknown count the stash's
    // unrolled steps took more than twice the registers)
    constexpr uint32_t kPart = kStash / kWaves;
    constexpr uint32_t kParts = kTileElems / kStash;      // a wave holds at most kTileElems / kWaves
    const uint32_t at = wave * kPart;
#pragma unroll
    for (uint32_t q = 0; q < kParts; ++q) {
        const uint32_t lo = lo0 + q * kPart;
        if (lo >= end)
            break;
        stash(BoolTag<true>{}, lo, lo + kPart, at);
        const uint32_t ne = end - lo < kPart ? end - lo : kPart;
        stash_copy<2>(as_global(sd.esc_pos + before + lo), s_pos + at, ne, lane);
        stash_copy<1>(as_global(sd.esc_exp + before + lo), s_exp + at, ne, lane);
    }
}

// ---- one-pass encode: the look-back over the status words of earlier tiles -------------

__device__ __forceinline__ uint64_t chain_word(uint64_t tag, uint64_t kind, uint64_t count)
{
    return (tag << kChainTagShift) | (kind << kChainKindShift) | count;
}

__device__ __forceinline__ void chain_publish(const EncodeArgs &a, uint32_t t, uint64_t word)
{
    __hip_atomic_store(a.chain_status + (uint64_t)t * kChainStride, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The status words of the 64 * kRows tiles below `top` (row h, lane l: the tile 64 h + l below
// it), as loaded; a tile before `first` loads the word of `first` instead (chain_lookback reads
// it as a running total of 0).  Loads are issued for every lane and row, so that the wave
// waits for them once.
template <int kRows>
__device__ __forceinline__ void chain_load(const EncodeArgs &a, uint32_t top, uint32_t first, uint32_t lane,
                                           uint64_t (&w)[kRows])
{
#pragma unroll
    for (int h = 0; h < kRows; ++h) {
        const uint32_t d = 64u * h + lane;
        w[h] = __hip_atomic_load(a.chain_status + (uint64_t)(d <= top - first ? top - d : first) * kChainStride,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Escapes of the segment's tiles before tile t (t > first, the segment's first tile), by a
// decoupled look-back run by one whole wave; tile t's own count must already be published,
// and w must hold chain_load(a, t - 1, first, lane, w) (issued early, so that its latency
// overlaps other work).  Tiles up to and including the nearest one below t that holds a
// running total must all be written (else the wave sleeps and loads the window again), and
// their counts give the result; when none of the window's tiles holds a running total their
// counts are added and the next window is loaded.  Tiles before `first` read as a running
// total of 0, so the walk ends at the segment's start.  Every lane gets the result.
// (Reading 128 or 256 tiles per round was slower, on 4096 tiles by 8 and 13 %.)
template <int kRows>
__device__ __forceinline__ uint64_t chain_lookback(const EncodeArgs &a, uint64_t tag, uint32_t t, uint32_t first,
                                                   uint32_t lane, uint64_t (&w)[kRows])
{
    uint64_t before = 0;
    uint32_t top = t - 1;            // highest tile not yet counted
    uint32_t polls = 0;
    for (;;) {
        // the first row holding a running total (kRows if none)
        int hs = kRows;
        bool ok = true;
        uint64_t part = 0;
#pragma unroll
        for (int h = 0; h < kRows; ++h) {
            const bool inside = 64u * h + lane <= top - first;             // tile top - d >= first
            const uint64_t x = inside ? w[h] : chain_word(tag, kChainPrefix, 0);
            const uint64_t kind = (x >> kChainKindShift) & 3u;
            const bool written = (x >> kChainTagShift) == tag && kind != 0;
            const uint64_t totals = __ballot(written && kind == kChainPrefix);
            const uint64_t ready = __ballot(written);
            if (hs == kRows) {
                // rows before hs must be written whole, row hs up to its first running total
                const uint32_t st = totals ? (uint32_t)__builtin_ctzll(totals) : 63u;
                const uint64_t need = st == 63u ? ~0ull : (2ull << st) - 1u;
                ok = ok && (ready & need) == need;
                part += lane <= st ? (x & kChainCountMask) : 0ull;
                if (totals)
                    hs = h;
            }
        }
        if (ok) {
            before += wave_total_u64(part, lane);
            if (hs < kRows)
                break;
            // 64 kRows written tiles without a running total are all inside the segment, and
            // the segment's first tile holds one: at least one tile is left below them.
            // Checked anyway, so that no status word read can move the walk below `first`.
            if (top - first < 64u * kRows) {
                if (lane == 0)
                    atomicOr(a.err, kErrChainStall);
                break;
            }
            top -= 64u * kRows;
        } else {
            if (++polls > kChainSpinMax) {
                if (lane == 0)
                    atomicOr(a.err, kErrChainStall);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        chain_load<kRows>(a, top, first, lane, w);
    }
    return uniform_u64(before);
}

}  // namespace sz
