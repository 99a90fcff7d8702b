// splitzip_e5m2.hip -- gfx950 (CDNA4) pack and decode kernels of the SplitZip codec for FP8
// E5M2 elements.
//
// Method ("SplitZip: Ultra-Fast Lossless KV Compression for Disaggregated LLM Serving",
// README "FAQ" and arXiv abstract: the exponent-split codec also applies on top of an FP8
// E5M2 KV cache): an E5M2 byte is a sign (bit 7), a 5-bit exponent (bits 6..2) and 2
// mantissa bits.  Sign and mantissa stay exact as the 3-bit field (sign << 2) | mantissa,
// packed into a little-endian bit stream (element i at bits 3i..3i+2); the exponent becomes
// a 4-bit code into a top-16 codebook over the 32 exponent values, and exponents outside it
// go to the same chunk-local escape stream as for BF16.  Codes, chunk offsets and escapes
// have the BF16 layout, so the escape placement launches (sums, place and spill, or finish)
// are shared.
//
// Per lane, groups of 32 consecutive elements: their 32 fields fill 12 bytes (one 12-byte
// store) and their codes 16 bytes (one 16-byte store), so each store instruction of a wave
// covers one contiguous range.  The 32 input bytes of a lane (pack) and its 32 output bytes
// (decode) would take two 16-byte accesses 32 bytes apart, which leave every cache line half
// covered per instruction; they go through LDS instead, so that each global access
// instruction of a wave covers 1 KiB contiguously.  For the same reason a group with many
// escapes is gathered in LDS before its escape entries are stored.  All work is integer byte
// manipulation: no floating point touches a value and no MFMA is used.
#include "splitzip_device.h"

namespace sz {

constexpr uint32_t kErrBadExponent = 32u;    // decode: escape exponent above 31

// ---- pack -----------------------------------------------------------------------------------

// Escape flag bits of the 8 elements of dword-group d (elements 8d..8d+7) inside a group's
// flag word; within one mask, ascending bits are ascending elements.
__device__ __forceinline__ uint32_t e8_flag_mask(int d)
{
    return d == 0 ? 0x30303030u : d == 1 ? 0xC0C0C0C0u : d == 2 ? 0x03030303u : 0x0C0C0C0Cu;
}

// Element (0..31) of flag bit b: bit 8i + 2c + r is element 8d + 2i + r of dword-group
// d = (c + 2) mod 4.
__device__ __forceinline__ uint32_t e8_flag_element(uint32_t b)
{
    const uint32_t d = (((b >> 1) & 3u) + 2u) & 3u;
    return 8u * d + 2u * (b >> 3) + (b & 1u);
}

// Split one group of 32 bytes (byte k of dword m is element 4m + k) with the byte LUT
// (lut[b]: code in bits 0..3, escape flag in bit 4, field (sign << 2) | mantissa in 5..7).
//   sm:    the 32 fields as 96 bits, element k at bits 3k..3k+2
//   codes: nibble 2i + r of codes[d] = code of element 8d + 2i + r (0 for escapes)
//   flags: escape flags, bit b for element e8_flag_element(b)
__device__ __forceinline__ void split_group32(const uint32_t (&x)[8], const uint8_t *lut,
                                              uint32_t (&sm)[3], uint32_t (&codes)[4], uint32_t &flags)
{
    uint32_t fl = 0, y[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lo = x[2 * d], hi = x[2 * d + 1];
        const uint32_t c0 = lut[lo & 0xFFu], c1 = lut[(lo >> 8) & 0xFFu];
        const uint32_t c2 = lut[(lo >> 16) & 0xFFu], c3 = lut[lo >> 24];
        const uint32_t c4 = lut[hi & 0xFFu], c5 = lut[(hi >> 8) & 0xFFu];
        const uint32_t c6 = lut[(hi >> 16) & 0xFFu], c7 = lut[hi >> 24];
        const uint32_t even = c0 | (c2 << 8) | (c4 << 16) | (c6 << 24);   // elements 8d + 2i
        const uint32_t odd = c1 | (c3 << 8) | (c5 << 16) | (c7 << 24);    // elements 8d + 2i + 1
        codes[d] = (even & 0x0F0F0F0Fu) | ((odd & 0x0F0F0F0Fu) << 4);
        const uint32_t f = (even & 0x10101010u) | ((odd & 0x10101010u) << 1);   // bits 8i+4+r
        fl |= d == 0 ? f : d == 1 ? (f << 2) : d == 2 ? (f >> 4) : (f >> 2);
        // byte i of g: the 6 field bits of elements 8d + 2i and 8d + 2i + 1; then 4 x 6 bits
        // become 24 contiguous bits
        const uint32_t g = ((even >> 5) & 0x07070707u) | ((odd >> 2) & 0x38383838u);
        const uint32_t g2 = (g & 0x003F003Fu) | ((g >> 2) & 0x0FC00FC0u);
        y[d] = (g2 & 0xFFFu) | ((g2 >> 4) & 0xFFF000u);
    }
    sm[0] = y[0] | (y[1] << 24);
    sm[1] = (y[1] >> 8) | (y[2] << 16);
    sm[2] = (y[2] >> 16) | (y[3] << 8);
    flags = fl;
}

// kChain: the one-pass build (chained tiles), which writes the escapes to their final places.
// G: groups per lane (4: tiles of 2^kE8EncTileShift elements; the one-pass build also runs
// 2: tiles of 2^kE8ChainTileShift).
template <bool kStage, bool kChain, int G>
__global__ __launch_bounds__(kThreads) void encode_pack_e5m2_kernel(const EncodeArgs a)
{
    static_assert(G == kE8EncGroups || (kChain && G == kE8ChainGroups), "E5M2 pack tile");
    constexpr int kShift = G == kE8EncGroups ? kE8EncTileShift : kE8ChainTileShift;
    constexpr uint32_t kStashChunks = (1u << kShift) / 16;
    static_assert(kE8StashEscapes >= (1u << kShift) / kWaves && kE8StashEscapes % kWaves == 0,
                  "wave 0's escapes fit the stash");
    __shared__ uint8_t s_lut[256];
    __shared__ uint32_t s_wave_total[kWaves];
    __shared__ uint64_t s_ovf;
    // per wave: one 2048-byte group, regrouped (s_in), and one group's escapes (s_stage: 11-bit
    // place, exponent); in the one-pass build the same LDS also holds the early-release stash
    // (its use begins after the last regroup and excludes the staged stores)
    constexpr uint32_t kInWords = kWaves * 128 * 4, kStageWords = kWaves * 2048 / 2;
    constexpr uint32_t kStashExpAt = kStashPosAt + 2 * kE8StashEscapes + 16;
    constexpr uint32_t kStashWords = (kStashExpAt + kE8StashEscapes + 2 * kStashChunks + 3) / 4;
    constexpr uint32_t kRawWords = kChain ? (kStashWords > kInWords ? kStashWords : kInWords) : kInWords + kStageWords;
    __shared__ uint32_t s_raw[kRawWords];
    __shared__ uint2 s_bitpos[kChain ? 256 : 1];      // one-pass build: set_bit_indices of each byte
    // one-pass build: set when wave 0 has copied the stash out and put the tile's escape offset
    // in s_before (stash_rest)
    __shared__ uint32_t s_out;
    __shared__ uint64_t s_before;
    uint4(*s_in)[128] = reinterpret_cast<uint4(*)[128]>(s_raw);
    uint16_t(*s_stage)[2048] = reinterpret_cast<uint16_t(*)[2048]>(s_raw + kInWords);

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t t = blockIdx.x;

    const uint32_t s = a.n_seg > 1 ? find_segment_block(a.tile_start, a.seg_at, t, tid, lane, s_wave_total) : 0u;
    const SegDesc sd = segment_desc(a, s);
    // the inverse LUT: loaded now, put in LDS once the tile's loads are issued
    const uint8_t *lut = a.multi_book ? a.lut + 256u * sd.book : a.lut;
    const uint32_t lut_word = tid < 64 ? reinterpret_cast<const uint32_t *>(lut)[tid & 63u] : 0u;
    if (!kChain && a.packed && tid == 0 && t == segment_first_tile(a, s))
        a.seg_total[s] = 0;      // the sums launch adds the segment's escapes into it
    if (kChain) {
        s_bitpos[tid & 255u] = set_bit_indices(tid & 255u);
        if (tid == 0)
            s_out = 0;
    }
    const uint64_t n = sd.n;
    const uint64_t base = (uint64_t)(t - segment_first_tile(a, s)) << kShift;
    const uint64_t cmask = (1ull << a.log2_chunk) - 1;
    const SZ_GLOBAL uint8_t *xb = as_global(reinterpret_cast<const uint8_t *>(sd.data));
    SZ_GLOBAL uint8_t *smb = as_global(sd.sm);
    SZ_GLOBAL uint8_t *cdb = as_global(sd.codes);
    SZ_GLOBAL uint64_t *chunk_off = as_global(sd.chunk_off);
    const uint64_t sm_bytes = (3 * n + 7) >> 3;
    const uint64_t code_bytes = (n + 1) >> 1;

    // element order inside the tile: wave w covers 64 * 32 * G consecutive elements, its group
    // j covers 2048 of them, lane l the 32 at offset 32 l.  A whole group is loaded 16 bytes
    // per lane at offsets 16 l and 1024 + 16 l and regrouped through LDS; the segment's last,
    // partial group is read byte by byte.
    uint64_t g0[G];
    uint32_t v[G][8];
    uint4 ld[G][2];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint64_t gbase = base + ((uint64_t)(wave * G + j) << 11);
        g0[j] = gbase + (uint64_t)lane * kE8GroupElems;
        const uint8_t *src = reinterpret_cast<const uint8_t *>(sd.data) + gbase;
        if (gbase + 2048 <= n) {                       // uniform in the wave
            ld[j][0] = load_stream16(src + 16 * lane);
            ld[j][1] = load_stream16(src + 1024 + 16 * lane);
        } else {
            // the segment's last group: the same 16-byte pieces byte by byte, 0 past the end
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t w[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    w[m] = 0;
                    for (uint32_t k = 0; k < 4; ++k) {
                        const uint64_t at = gbase + 1024u * h + 16u * lane + 4u * m + k;
                        if (at < n)
                            w[m] |= (uint32_t)xb[at] << (8 * k);
                    }
                }
                ld[j][h] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }
    if (tid < 64)
        reinterpret_cast<uint32_t *>(s_lut)[tid] = lut_word;
    __syncthreads();   // LUT in LDS
    // Regroup, one group at a time through the wave's own buffer: lane l loaded bytes 16 l and
    // 1024 + 16 l of the group and takes bytes 32 l .. 32 l + 31.  A wave's LDS accesses are
    // performed in the order it issues them, so the wavefront-scope fences (which keep the
    // compiler from reordering them) are all the ordering these exchanges need.
#pragma unroll
    for (int j = 0; j < G; ++j) {
        s_in[wave][lane] = ld[j][0];
        s_in[wave][64 + lane] = ld[j][1];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const uint4 lo = s_in[wave][2 * lane], hi = s_in[wave][2 * lane + 1];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        v[j][0] = lo.x; v[j][1] = lo.y; v[j][2] = lo.z; v[j][3] = lo.w;
        v[j][4] = hi.x; v[j][5] = hi.y; v[j][6] = hi.z; v[j][7] = hi.w;
    }

    // ---- a2: dense split and pack ---------------------------------------------------------
    uint32_t flags[G], counts[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        uint32_t sm[3], codes[4], fl;
        split_group32(v[j], s_lut, sm, codes, fl);
        const uint64_t q = g0[j] / kE8GroupElems;
        if (g0[j] + kE8GroupElems <= n) {
            store_stream12(sd.sm + 12 * q, sm[0], sm[1], sm[2]);
            store_stream16(sd.codes + 16 * q, codes[0], codes[1], codes[2], codes[3]);
        } else if (g0[j] < n) {
            // last group of the segment: keep the codes and flags of its nv elements, write the
            // bytes that lie inside the sections (fields past n are 0: those bytes were 0)
            const uint32_t nv = (uint32_t)(n - g0[j]);
            uint32_t keep = 0;
            for (uint32_t b = 0; b < 32; ++b)
                keep |= (e8_flag_element(b) < nv ? 1u : 0u) << b;
            fl &= keep;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const int vd = (int)nv - 8 * d;
                codes[d] &= vd >= 8 ? ~0u : vd <= 0 ? 0u : (1u << (4 * vd)) - 1u;
            }
            for (uint32_t k = 0; k < 12 && 12 * q + k < sm_bytes; ++k)
                smb[12 * q + k] = (uint8_t)(sm[k >> 2] >> (8 * (k & 3)));
            for (uint32_t k = 0; k < 16 && 16 * q + k < code_bytes; ++k)
                cdb[16 * q + k] = (uint8_t)(codes[k >> 2] >> (8 * (k & 3)));
        } else {
            fl = 0;
        }
        flags[j] = fl;
        counts[j] = __popc(fl);
    }

    // ---- a3: escape ranks inside the tile ---------------------------------------------------
    uint32_t rank[G];
    uint32_t tile_total;
    uint32_t wave_end;
    tile_escape_ranks<G>(counts, lane, wave, s_wave_total, rank, tile_total, wave_end);
    if (a.first_tile_escapes && t == 0 && tid == 0) {
        // the count scaled to a tile of the launch sequences, and whether it falls unevenly
        uint32_t lo = s_wave_total[0], hi = s_wave_total[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            lo = s_wave_total[w] < lo ? s_wave_total[w] : lo;
            hi = s_wave_total[w] > hi ? s_wave_total[w] : hi;
        }
        const uint32_t uneven = hi > 2 * lo + 64 ? kHintUneven : 0u;
        __hip_atomic_store(a.first_tile_escapes, (tile_total << (kE8EncTileShift - kShift)) | uneven,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }

    if (kChain) {
        // one pass, early release, as in the BF16 pack: the escapes of rank below
        // kE8StashEscapes and the chunk starts' ranks wait in LDS; waves whose escapes all fit
        // end, wave 0 waits for the tile's escape offset, a wave with escapes past the stash
        // gets it from wave 0 and writes those itself
        uint8_t *lds = reinterpret_cast<uint8_t *>(s_raw);
        uint16_t *s_pos = reinterpret_cast<uint16_t *>(lds + kStashPosAt);
        uint8_t *s_exp = lds + kStashExpAt;
        uint16_t *s_start = reinterpret_cast<uint16_t *>(s_exp + kE8StashEscapes);
        const uint64_t tag = a.chain_tag;
        const uint32_t first = segment_first_tile(a, s);
        const bool last = t + 1 == segment_end_tile(a, s);
        if (tid == 0)
            chain_publish(a, t, chain_word(tag, t > first ? kChainAggregate : kChainPrefix, tile_total));
        uint64_t w[kChainRows];
        if (wave == 0 && t > first)
            chain_load<kChainRows>(a, t - 1, first, lane, w);
        const uint32_t cm = (uint32_t)cmask;
        // the lane's escapes of rank lo .. hi - 1 to LDS at rank - lo, as in the BF16 pack, per
        // 8 elements of a lane's 32 (positions two per byte permute, exponents four); without
        // a range check (kRanged false) every escape of the lane must lie in lo .. hi - 1
        auto stash = [&](auto ranged, uint32_t lo, uint32_t hi, uint32_t at) {
            constexpr bool kRanged = decltype(ranged)::value;
#pragma unroll
            for (int j = 0; j < G; ++j) {
                uint32_t r = rank[j];
                const uint32_t fl = flags[j];
                if (fl && (!kRanged || (r < hi && r + 32u > lo))) {
                    // the group's first element (recomputed: g0 is not kept)
                    const uint32_t q0 = (uint32_t)base + ((wave * G + j) << 11) + lane * kE8GroupElems;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        // escape flags of elements 8d .. 8d + 7, bit k for element 8d + k
                        const uint32_t sh = 2u * (((uint32_t)d + 2u) & 3u);
                        const uint32_t f = (((fl >> sh) & 0x03030303u) * 0x01041040u) >> 24;
                        const uint32_t cnt = __popc(f);
                        const uint2 ks = s_bitpos[f];
                        // elements 8d .. 8d + 7 start 8-aligned inside their chunk
                        const uint32_t pq = ((q0 + 8u * d) & cm) * 0x10001u;
                        uint32_t pp = 0, ee = 0;
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            if (!__ballot((uint32_t)i < cnt))
                                break;
                            const uint32_t kx = i < 4 ? ks.x : ks.y;
                            if ((i & 1) == 0)
                                pp = pq + perm(0u, kx, (i & 2) ? 0x0C030C02u : 0x0C010C00u);
                            if ((i & 3) == 0)
                                ee = (perm(v[j][2 * d + 1], v[j][2 * d], kx) >> 2) & 0x1F1F1F1Fu;
                            const uint32_t ri = r + i;
                            if ((uint32_t)i < cnt && (!kRanged || (ri >= lo && ri < hi))) {
                                s_pos[ri - lo + at] = (uint16_t)(pp >> (16 * (i & 1)));
                                s_exp[ri - lo + at] = (uint8_t)(ee >> (8 * (i & 3)));
                            }
                        }
                        r += cnt;
                    }
                }
            }
        };
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint32_t p0 = (uint32_t)(g0[j] - base);
            if (g0[j] < n && (g0[j] & cmask) == 0)
                s_start[p0 >> a.log2_chunk] = (uint16_t)rank[j];
            if (a.log2_chunk == 4 && g0[j] + 16 < n)
                s_start[(p0 + 16) >> 4] = (uint16_t)(rank[j] + __popc(flags[j] & 0xF0F0F0F0u));
        }
        const bool past = wave_end > kE8StashEscapes;                 // uniform in the wave
        if (past)
            stash(BoolTag<true>{}, 0, kE8StashEscapes, 0);
        else
            stash(BoolTag<false>{}, 0, kE8StashEscapes, 0);
        __syncthreads();
        if (wave != 0 && !past)
            return;
        if (wave == 0) {
            const uint64_t before = t > first ? chain_lookback<kChainRows>(a, tag, t, first, lane, w) : 0ull;
            if (lane == 0) {
                if (t > first)
                    chain_publish(a, t, chain_word(tag, kChainPrefix, before + tile_total));
                if (last) {
                    chunk_off[(n + cmask) >> a.log2_chunk] = before + tile_total;
                    a.seg_escapes[s] = before + tile_total;
                }
                if (tile_total > kE8StashEscapes)
                    s_before = before;
            }
            const uint64_t tile_end = base + (1u << kShift) < n ? base + (1u << kShift) : n;
            const uint32_t starts = a.log2_chunk <= (uint32_t)kShift
                                  ? (uint32_t)((tile_end - base + cmask) >> a.log2_chunk)
                                  : ((base & cmask) == 0 ? 1u : 0u);
            SZ_GLOBAL uint64_t *co = chunk_off + (base >> a.log2_chunk);
            for (uint32_t i = lane; i < starts; i += 64)
                co[i] = before + s_start[i];
            const uint64_t left = sd.esc > before && sd.esc_exp ? sd.esc - before : 0;
            uint32_t ne = left < tile_total ? (uint32_t)left : tile_total;
            ne = ne < kE8StashEscapes ? ne : kE8StashEscapes;
            if (ne) {
                stash_copy<2>(as_global(sd.esc_pos + before), s_pos, ne, lane);
                stash_copy<1>(as_global(sd.esc_exp + before), s_exp, ne, lane);
            }
            if (tile_total > kE8StashEscapes && lane == 0)    // the stash is out
                __hip_atomic_store(&s_out, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            return;
        }
        // a wave with escapes past the stash: once wave 0 has copied it out, they go through it
        // again (stash_rest)
        const uint32_t wave_first = (uint32_t)__builtin_amdgcn_readfirstlane(rank[0]);   // lane 0's group 0
        stash_rest<kE8StashEscapes, (1u << kShift)>(a, sd, &s_out, &s_before, wave, wave_first, wave_end, lane,
                                                    s_pos, s_exp, stash);
        return;
    }

    // where the tile's escapes go: its slot or the overflow area
    uint64_t room = 0;
    uint32_t *dst = tile_escape_dest(a, t, tile_total, tid, &s_ovf, room);
    SZ_GLOBAL uint32_t *gdst = as_global(dst);

    // escapes: (position inside the tile, exponent); tile-local chunk offsets (a chunk of 16
    // elements also starts in the middle of a group)
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint32_t r0 = rank[j];
        if (g0[j] < n && (g0[j] & cmask) == 0)
            chunk_off[g0[j] >> a.log2_chunk] = r0;
        if (a.log2_chunk == 4 && g0[j] + 16 < n)
            chunk_off[(g0[j] + 16) >> 4] = r0 + __popc(flags[j] & 0xF0F0F0F0u);
        // a wave's escapes of one group have consecutive ranks; more than kStageMin of them
        // are gathered in the wave's LDS buffer (place inside the group in 11 bits, exponent
        // in 5) and stored 64 consecutive entries per instruction: stored by the lanes that
        // hold them, a lane's 32 elements put its escapes up to 32 entries apart, and one
        // store instruction touched as many cache lines as the wave has lanes
        const uint32_t w0 = __builtin_amdgcn_readfirstlane(r0);
        const uint32_t wcnt = (j + 1 < G ? __builtin_amdgcn_readfirstlane(rank[j + 1]) : wave_end) - w0;
        const bool staged = kStage && __builtin_expect(wcnt > kStageMin, 0);   // uniform in the wave
        if (flags[j]) {
            const uint32_t p0 = (uint32_t)(g0[j] - base);
            uint32_t r = r0;
            if (staged) {
                // place inside the group: the lane's first element is 32 lane
                const uint32_t q0 = lane * kE8GroupElems;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint32_t z = flags[j] & e8_flag_mask(d);
                    const uint64_t bytes8 = ((uint64_t)v[j][2 * d + 1] << 32) | v[j][2 * d];
                    while (z) {
                        const uint32_t b = (uint32_t)__builtin_ctz(z);
                        const uint32_t k = 2u * (b >> 3) + (b & 1u);          // element 8d + k
                        const uint32_t e = (uint32_t)(bytes8 >> (8 * k + 2)) & 0x1Fu;
                        s_stage[wave][r - w0] = (uint16_t)((q0 + 8u * d + k) | (e << 11));
                        ++r;
                        z &= z - 1;
                    }
                }
            } else {
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    uint32_t z = flags[j] & e8_flag_mask(d);
                    const uint64_t bytes8 = ((uint64_t)v[j][2 * d + 1] << 32) | v[j][2 * d];
                    while (z) {
                        const uint32_t b = (uint32_t)__builtin_ctz(z);
                        const uint32_t k = 2u * (b >> 3) + (b & 1u);          // element 8d + k
                        const uint32_t e = (uint32_t)(bytes8 >> (8 * k + 2)) & 0x1Fu;
                        if (r < room)
                            gdst[r] = (p0 + 8u * d + k) | (e << 16);
                        ++r;
                        z &= z - 1;
                    }
                }
            }
        }
        if (staged) {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            const uint32_t gp = (uint32_t)(wave * G + j) << 11;   // the group's place in the tile
            for (uint32_t i = lane; i < wcnt; i += 64)
                if (w0 + i < room) {
                    const uint32_t h = s_stage[wave][i];
                    gdst[w0 + i] = (gp + (h & 0x7FFu)) | ((h >> 11) << 16);
                }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
    }
}

hipError_t launch_encode_pack_e5m2(const EncodeArgs &a, hipStream_t stream)
{
    const unsigned lds = a.n_tiles >= kPackCapTiles ? kE8PackLdsReserve : 0u;
    constexpr int G = kE8EncGroups, G1 = kE8ChainGroups;
    if (a.chain_status && a.tile_shift == (uint32_t)kE8ChainTileShift) {
        if (a.stage)
            encode_pack_e5m2_kernel<true, true, G1><<<a.n_tiles, kThreads, 0, stream>>>(a);
        else
            encode_pack_e5m2_kernel<false, true, G1><<<a.n_tiles, kThreads, 0, stream>>>(a);
    } else if (a.chain_status) {
        if (a.stage)
            encode_pack_e5m2_kernel<true, true, G><<<a.n_tiles, kThreads, 0, stream>>>(a);
        else
            encode_pack_e5m2_kernel<false, true, G><<<a.n_tiles, kThreads, 0, stream>>>(a);
    } else {
        if (a.stage)
            encode_pack_e5m2_kernel<true, false, G><<<a.n_tiles, kThreads, lds, stream>>>(a);
        else
            encode_pack_e5m2_kernel<false, false, G><<<a.n_tiles, kThreads, 0, stream>>>(a);
    }
    return hipGetLastError();
}

// ---- decode ---------------------------------------------------------------------------------

// 12 bits of 4 fields (field k at bits 3k..3k+2) spread to one field per byte.
__device__ __forceinline__ uint32_t unpack_fields4(uint32_t z)
{
    const uint32_t y = (z | (z << 10)) & 0x003F003Fu;   // fields 0,1 in byte 0, 2,3 in byte 2
    return (y | (y << 5)) & 0x07070707u;
}

// Four E5M2 bytes from exponent bytes (already shifted to bits 6..2) and fields.
__device__ __forceinline__ uint32_t e8_assemble(uint32_t ex4, uint32_t f)
{
    return ex4 | (f & 0x03030303u) | ((f << 5) & 0x80808080u);
}

// G: groups per lane (kE8DecGroups, or kE8DecShortGroups in the short tiles).
template <bool kLarge, int G>
__global__ __launch_bounds__(kThreads) void decode_e5m2_kernel(const DecodeArgs a)
{
    static_assert(G == kE8DecGroups || G == kE8DecShortGroups, "E5M2 decode tile");
    constexpr int kShift = G == kE8DecGroups ? kE8DecTileShift : kE8DecShortTileShift;
    constexpr uint32_t kTile = 1u << kShift;
    __shared__ uint32_t s_exp[kTile / 4];              // exponent bytes of the tile
    __shared__ uint64_t s_off[kTile / 16 + 1];         // chunk offsets of the tile
    __shared__ uint16_t s_pair[256];                   // codes byte -> its two exponent bytes
    __shared__ uint32_t s_cnt[kWaves];

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const uint32_t wave = tid >> 6;
    const uint32_t t = xcd_tile(blockIdx.x, a.n_tiles);
    if (t >= a.n_tiles)
        return;

    uint32_t first = 0;
    SegDesc sd = a.seg0;
    if (a.n_seg > 1) {
        const uint32_t s = find_segment_block(a.tile_start, a.seg_at, t, tid, lane, s_cnt);
        first = load_const_u32(a.tile_start, s);
        sd = load_const_segdesc(a.segs, s);
    }
    const uint64_t n = sd.n;
    const uint64_t base = (uint64_t)(t - first) << kShift;
    if (base >= n)
        return;                                              // empty segment
    const uint64_t valid = n - base < (uint64_t)kTile ? n - base : (uint64_t)kTile;
    const uint32_t log2c = a.log2_chunk;
    const uint64_t C = 1ull << log2c;
    const uint64_t E = sd.esc;
    const uint64_t sm_bytes = (3 * n + 7) >> 3;
    const uint64_t code_bytes = (n + 1) >> 1;
    uint8_t *yb = reinterpret_cast<uint8_t *>(sd.data);
    uint32_t cb[4] = {a.cb[0], a.cb[1], a.cb[2], a.cb[3]};
    if (a.multi_book) {
        const uint32_t *c = a.cbs + 4u * sd.book;
        cb[0] = load_const_u32(c, 0);
        cb[1] = load_const_u32(c, 1);
        cb[2] = load_const_u32(c, 2);
        cb[3] = load_const_u32(c, 3);
    }

    // ---- loads ---------------------------------------------------------------------------
    // a packed stream's header, through scalar loads as in the BF16 decode
    uint4 h0{}, h1{}, h2{}, h3{};
    if (sd.header) {
        const uint32_t *h = reinterpret_cast<const uint32_t *>(sd.header);
        uint32_t w[16];
#pragma unroll
        for (uint32_t k = 0; k < 16; ++k)
            w[k] = load_const_u32(h, k);
        h0 = make_uint4(w[0], w[1], w[2], w[3]);
        h1 = make_uint4(w[4], w[5], w[6], w[7]);
        h2 = make_uint4(w[8], w[9], w[10], w[11]);
        h3 = make_uint4(w[12], w[13], w[14], w[15]);
    }
    uint32_t smv[G][3], cw[G][4];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint64_t g0 = base + (uint64_t)(((wave * G + j) << 6) + lane) * kE8GroupElems;
        const uint64_t q = g0 / kE8GroupElems;
        if (g0 + kE8GroupElems <= n) {
            const u32x3 s3 = __builtin_nontemporal_load((const SZ_GLOBAL u32x3 *)(sd.sm + 12 * q));
            const u32x4 c4 = __builtin_nontemporal_load(as_global(reinterpret_cast<const u32x4 *>(sd.codes + 16 * q)));
            smv[j][0] = s3.x; smv[j][1] = s3.y; smv[j][2] = s3.z;
            cw[j][0] = c4.x; cw[j][1] = c4.y; cw[j][2] = c4.z; cw[j][3] = c4.w;
        } else {
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                uint32_t w = 0;
                for (uint32_t k = 0; k < 4; ++k)
                    if (12 * q + 4 * m + k < sm_bytes)
                        w |= (uint32_t)sd.sm[12 * q + 4 * m + k] << (8 * k);
                smv[j][m] = w;
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                uint32_t w = 0;
                for (uint32_t k = 0; k < 4; ++k)
                    if (16 * q + 4 * m + k < code_bytes)
                        w |= (uint32_t)sd.codes[16 * q + 4 * m + k] << (8 * k);
                cw[j][m] = w;
            }
        }
    }

    // The codebook as a table over codes bytes: entry c holds the exponents (moved to bits 6..2
    // of an output byte) of the codes c & 15 (low byte) and c >> 4 (high byte).  A packed
    // stream brings its own codebook (its header is checked below, before any store).
    if (sd.header) {
        cb[0] = h2.z;
        cb[1] = h2.w;
        cb[2] = h3.x;
        cb[3] = h3.y;
    }
    for (uint32_t c = tid; c < 256; c += kThreads) {
        const uint32_t e_lo = codebook_byte(cb, c & 15u) & 0x1Fu, e_hi = codebook_byte(cb, c >> 4) & 0x1Fu;
        s_pair[c] = (uint16_t)((e_lo | (e_hi << 8)) << 2);
    }

    // ---- escape range of the tile --------------------------------------------------------
    const bool sub_chunk = log2c > (uint32_t)kShift;   // the tile lies inside one chunk
    const uint64_t c0 = base >> log2c;
    const uint64_t nc = sub_chunk ? 1 : (valid + C - 1) >> log2c;
    for (uint32_t i = tid; i <= nc; i += kThreads)
        s_off[i] = sd.chunk_off[c0 + i];
    __syncthreads();
    const uint64_t j0 = s_off[0], j1 = s_off[nc];
    bool patch = j1 > j0;
    // at most one escape per element: a tile's range may not exceed its elements (a tile
    // inside one chunk: that chunk's), which also keeps tile-relative ranks below 2^32
    const uint64_t c0_len = n - (c0 << log2c) < C ? n - (c0 << log2c) : C;
    if (j0 > j1 || j1 > E || j1 - j0 > (sub_chunk ? c0_len : valid)) {
        patch = false;
        if (tid == 0 && a.err)
            atomicOr(a.err, kErrBadOffsets);
    }

    if (sd.header) {
        // packed stream: it must describe exactly the segment the caller gave (E5M2 flags,
        // n, chunk size, E) and carries its own codebook, whose entries must be 5-bit
        // exponents.  Loaded with the data, checked before any store.
        const uint64_t hn = h1.x | ((uint64_t)h1.y << 32), hc = h1.z | ((uint64_t)h1.w << 32);
        const uint64_t he = h2.x | ((uint64_t)h2.y << 32);
        const bool ok = h0.x == 0x31425A53u && h0.y == (1u | (64u << 16)) && h0.z == (uint32_t)C &&
                        h0.w == kElemE5M2 && hn == n && hc == ((n + C - 1) >> log2c) && he == E &&
                        h3.z == 0u && h3.w == 0u && ((h2.z | h2.w | h3.x | h3.y) & 0xE0E0E0E0u) == 0u;
        if (!ok) {
            if (tid == 0 && a.err)
                atomicOr(a.err, kErrBadHeader);
            return;
        }
    }

    // ---- a5: dense path: exponent bytes of 4 elements per dword, in element order ----------
    uint32_t ex[G][8];
#pragma unroll
    for (int j = 0; j < G; ++j)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t c = cw[j][d];
            ex[j][2 * d] = s_pair[c & 0xFFu] | ((uint32_t)s_pair[(c >> 8) & 0xFFu] << 16);
            ex[j][2 * d + 1] = s_pair[(c >> 16) & 0xFFu] | ((uint32_t)s_pair[c >> 24] << 16);
        }

    // ---- a6: sparse escape correction (exponent bytes in LDS, element p at byte p) -------
    if (patch) {
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint32_t q = ((wave * G + j) << 6) + lane;
#pragma unroll
            for (int m = 0; m < 8; ++m)
                s_exp[8 * q + m] = ex[j][m];
        }
        __syncthreads();
        uint8_t *bytes = reinterpret_cast<uint8_t *>(s_exp);
        uint32_t bad = 0;               // error bits this thread found
        // the tile's escapes are the contiguous range [j0, j1), kPatch per thread and round;
        // every load of a round goes out before its LDS writes, at an index clamped into the
        // range (global pointers: the loads cannot alias LDS, so nothing holds them back)
        constexpr int kPatch = kLarge ? 8 : 4;
        const SZ_GLOBAL uint16_t *gpos = as_global(static_cast<const uint16_t *>(sd.esc_pos));
        const SZ_GLOBAL uint8_t *gexp = as_global(static_cast<const uint8_t *>(sd.esc_exp));
        if (!sub_chunk) {
            for (uint64_t ci = tid; ci < nc; ci += kThreads) {
                const uint64_t cs = (c0 + ci) << log2c;
                if (s_off[ci] > s_off[ci + 1] || s_off[ci + 1] - s_off[ci] > (n - cs < C ? n - cs : C))
                    bad |= kErrBadOffsets;
            }
            if (j1 - j0 > (uint64_t)kThreads) {
                // more escapes than threads: each chunk's escapes [s_off[c], s_off[c + 1]) are
                // patched by `per` threads (as in the BF16 decode), so an escape's chunk is known
                // without a search; a chunk whose offsets are out of order, too long or outside
                // the tile's range (flagged above) is skipped
                const uint32_t lgc = nc > 1 ? 32u - (uint32_t)__builtin_clz((uint32_t)nc - 1u) : 0u;   // ceil log2(nc)
                const uint32_t pshift = lgc >= 8u ? 0u : 8u - lgc;
                const uint32_t per = 1u << pshift;
                const uint32_t sub = tid & (per - 1u);
                const uint32_t tvalid = (uint32_t)valid;
                for (uint32_t c = tid >> pshift; c < (uint32_t)nc; c += kThreads >> pshift) {
                    const uint64_t e0 = s_off[c], e1 = s_off[c + 1];
                    const uint32_t cs = c << log2c;
                    const uint32_t clen = tvalid - cs < (uint32_t)C ? tvalid - cs : (uint32_t)C;
                    if (e0 > e1 || e1 - e0 > clen || e0 < j0 || e1 > j1)
                        continue;
                    const uint32_t m = (uint32_t)(e1 - e0);
                    const SZ_GLOBAL uint16_t *cpos = gpos + e0;
                    const SZ_GLOBAL uint8_t *cexp = gexp + e0;
                    for (uint32_t rb = sub; rb < m; rb += kPatch * per) {
                        uint32_t pos[kPatch], ev[kPatch];
#pragma unroll
                        for (int k = 0; k < kPatch; ++k) {
                            const uint32_t r = rb + (uint32_t)k * per;
                            const uint32_t rc = r < m ? r : m - 1u;
                            pos[k] = cpos[rc];
                            ev[k] = cexp[rc];
                        }
#pragma unroll
                        for (int k = 0; k < kPatch; ++k) {
                            if (rb + (uint32_t)k * per >= m)
                                continue;
                            if (pos[k] < clen && ev[k] <= 31u)
                                bytes[cs + pos[k]] = (uint8_t)(ev[k] << 2);
                            else
                                bad |= pos[k] >= clen ? kErrBadPosition : kErrBadExponent;
                        }
                    }
                }
            } else {
                // chunk of escape jj: the last c with s_off[c] <= jj.  In the large-call build a
                // tile of at most kFew chunks (chunk size 1024 or more) counts the tile-relative
                // chunk starts at or below each escape's rank: the starts of chunks 1..kFew, two
                // per dword (absent ones 0x7FFF), are subtracted from the rank with packed 16-bit
                // subtractions (ranks and starts are below 2^14, so a half's sign bit says rank <
                // start), and the sign bits are counted.  Otherwise a binary search in LDS
                // (three or more dependent LDS reads per escape).
                constexpr int kFew = 16;
                const bool few = kLarge && nc <= (uint64_t)kFew;       // uniform
                static_assert(kTile < (1 << 15), "tile ranks fit a signed 16-bit half");
                uint32_t starts[kFew / 2];
#pragma unroll
                for (int m = 0; m < kFew / 2; ++m) {
                    uint32_t h[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int c = 2 * m + 1 + i;
                        h[i] = (few && (uint64_t)c < nc) ? (uint32_t)(s_off[c] - j0) : 0x7FFFu;
                        h[i] = h[i] < 0x7FFFu ? h[i] : 0x7FFFu;
                    }
                    starts[m] = __builtin_amdgcn_readfirstlane(h[0] | (h[1] << 16));
                }
                // 32-bit arithmetic relative to the tile: escape rank r in [0, cnt), chunk starts
                // lo << log2c inside the tile (a chunk is at most a tile here), cnt <= valid
                const uint32_t cnt = (uint32_t)(j1 - j0);
                const SZ_GLOBAL uint16_t *tpos = gpos + j0;
                const SZ_GLOBAL uint8_t *texp = gexp + j0;
                const uint32_t tvalid = (uint32_t)valid;
                for (uint32_t rb = tid; rb < cnt; rb += kPatch * kThreads) {
                    uint32_t pos[kPatch], ev[kPatch];
#pragma unroll
                    for (int k = 0; k < kPatch; ++k) {
                        const uint32_t r = rb + (uint32_t)k * kThreads;
                        const uint32_t rc = r < cnt ? r : cnt - 1;
                        pos[k] = tpos[rc];
                        ev[k] = texp[rc];
                    }
#pragma unroll
                    for (int k = 0; k < kPatch; ++k) {
                        const uint32_t r = rb + (uint32_t)k * kThreads;
                        if (r >= cnt)
                            continue;
                        uint32_t lo = 0;
                        if (few) {
                            typedef short s16x2 __attribute__((ext_vector_type(2)));
                            const s16x2 rr = {(short)r, (short)r};
                            uint32_t below = 0;             // chunk starts above r
#pragma unroll
                            for (int m = 0; m < kFew / 2; ++m) {
                                const s16x2 st = __builtin_bit_cast(s16x2, starts[m]);
                                const uint32_t d = __builtin_bit_cast(uint32_t, (s16x2)(rr - st));
                                below += (uint32_t)__popc(d & 0x80008000u);
                            }
                            lo = kFew - below;              // halves hold chunks 1 .. kFew
                            lo = lo < (uint32_t)nc ? lo : (uint32_t)nc - 1u;
                        } else {
                            const uint64_t jj = j0 + r;
                            uint32_t hi = (uint32_t)nc;          // s_off[lo] <= jj < s_off[hi]
                            while (hi - lo > 1) {
                                const uint32_t mid = (lo + hi) >> 1;
                                if (s_off[mid] <= jj)
                                    lo = mid;
                                else
                                    hi = mid;
                            }
                        }
                        const uint32_t cs = lo << log2c;
                        const uint32_t clen = tvalid - cs < (uint32_t)C ? tvalid - cs : (uint32_t)C;
                        if (pos[k] < clen && ev[k] <= 31u)
                            bytes[cs + pos[k]] = (uint8_t)(ev[k] << 2);
                        else
                            bad |= pos[k] >= clen ? kErrBadPosition : kErrBadExponent;
                    }
                }
            }
        } else {
            const uint64_t lo = base - (c0 << log2c);
            const uint64_t clen = n - (c0 << log2c) < C ? n - (c0 << log2c) : C;
            for (uint64_t jb = j0 + tid; jb < j1; jb += kPatch * kThreads) {
                uint32_t pos[kPatch], ev[kPatch];
#pragma unroll
                for (int k = 0; k < kPatch; ++k) {
                    const uint64_t jj = jb + (uint64_t)k * kThreads;
                    const uint64_t jc = jj < j1 ? jj : j1 - 1;
                    pos[k] = gpos[jc];
                    ev[k] = gexp[jc];
                }
#pragma unroll
                for (int k = 0; k < kPatch; ++k) {
                    if (jb + (uint64_t)k * kThreads >= j1)
                        continue;
                    if (pos[k] >= clen || ev[k] > 31u)
                        bad |= pos[k] >= clen ? kErrBadPosition : kErrBadExponent;
                    else if (pos[k] >= lo && pos[k] < lo + valid)
                        bytes[pos[k] - lo] = (uint8_t)(ev[k] << 2);
                }
            }
        }
        if (bad && a.err)
            atomicOr(a.err, bad);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const uint32_t q = ((wave * G + j) << 6) + lane;
#pragma unroll
            for (int m = 0; m < 8; ++m)
                ex[j][m] = s_exp[8 * q + m];
        }
    }

    // ---- assemble and store ------------------------------------------------------------------
    // A whole 2048-element group of a wave is regrouped through the wave's own 2 KiB of s_exp
    // (since the patch, only this wave reads it) and stored 16 bytes per lane at offsets 16 l
    // and 1024 + 16 l; the segment's last, partial group is written byte by byte.  A wave's LDS
    // accesses are performed in the order it issues them, so wavefront-scope fences suffice.
#pragma unroll
    for (int j = 0; j < G; ++j) {
        const uint64_t g0 = base + (uint64_t)(((wave * G + j) << 6) + lane) * kE8GroupElems;
        const uint32_t s0 = smv[j][0], s1 = smv[j][1], s2 = smv[j][2];
        // 12-bit field quads of elements 4m..4m+3 at bits 12m of the 96-bit field stream
        const uint32_t z[8] = {
            s0 & 0xFFFu,
            (s0 >> 12) & 0xFFFu,
            (uint32_t)((((uint64_t)s1 << 32) | s0) >> 24) & 0xFFFu,
            (s1 >> 4) & 0xFFFu,
            (s1 >> 16) & 0xFFFu,
            (uint32_t)((((uint64_t)s2 << 32) | s1) >> 28) & 0xFFFu,
            (s2 >> 8) & 0xFFFu,
            s2 >> 20,
        };
        uint32_t out[8];
#pragma unroll
        for (int m = 0; m < 8; ++m)
            out[m] = e8_assemble(ex[j][m], unpack_fields4(z[m]));
        const uint64_t gbase = base + ((uint64_t)(wave * G + j) << 11);
        if (gbase + 2048 <= n) {                        // uniform in the wave
            uint4 *grp = reinterpret_cast<uint4 *>(s_exp) + ((wave * G + j) << 7);
            grp[2 * lane] = make_uint4(out[0], out[1], out[2], out[3]);
            grp[2 * lane + 1] = make_uint4(out[4], out[5], out[6], out[7]);
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            const uint4 lo = grp[lane], hi = grp[64 + lane];
            store_stream16(yb + gbase + 16 * lane, lo.x, lo.y, lo.z, lo.w);
            store_stream16(yb + gbase + 1024 + 16 * lane, hi.x, hi.y, hi.z, hi.w);
        } else {
            // the lane's own 32 elements, those below n
            for (uint32_t k = 0; k < kE8GroupElems && g0 + k < n; ++k)
                yb[g0 + k] = (uint8_t)(out[k >> 2] >> (8 * (k & 3)));
        }
    }
}

hipError_t launch_decode_e5m2(const DecodeArgs &a, hipStream_t stream)
{
    const unsigned grid = (a.n_tiles + kXcds - 1) / kXcds * kXcds;
    constexpr int G = kE8DecGroups, G1 = kE8DecShortGroups;
    if (a.tile_shift == (uint32_t)kE8DecShortTileShift) {
        if (a.large)
            decode_e5m2_kernel<true, G1><<<grid, kThreads, 0, stream>>>(a);
        else
            decode_e5m2_kernel<false, G1><<<grid, kThreads, 0, stream>>>(a);
    } else {
        if (a.large)
            decode_e5m2_kernel<true, G><<<grid, kThreads, 0, stream>>>(a);
        else
            decode_e5m2_kernel<false, G><<<grid, kThreads, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace sz
