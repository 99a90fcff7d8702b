// splitzip_kernels.hip -- gfx950 (CDNA4) kernels of the SplitZip BF16 exponent-split codec.
//
// Method ("SplitZip: Ultra-Fast Lossless KV Compression for Disaggregated LLM Serving",
// README "Abstract" and "Highlights"; arXiv abstract): each BF16 word keeps its sign and
// 7 mantissa bits exactly in one byte; its 8-bit exponent becomes a 4-bit code into a
// top-16 exponent codebook calibrated offline; exponents outside the codebook go to a
// chunk-local sparse escape stream of (position, exponent).  Decoding is the dense path
// (code -> codebook exponent) plus a sparse correction at the escape positions.
//
// The work is pure integer/byte manipulation and bound by HBM bandwidth: no floating
// point touches a value and no MFMA is used.  Design points:
//   - 16-byte, lane-contiguous loads and stores (a wave touches 1 KiB per instruction);
//   - encode: 256-byte inverse LUT in LDS (exponent -> code or escape bit), sign+mantissa
//     bytes gathered with v_perm_b32, codes packed two per byte;
//   - encode: escape ranks inside a tile by a wave prefix of packed per-group counts plus
//     an LDS prefix over the 4 waves; the tile's escapes go compacted to a scratch slot
//     (escape-heavy groups gathered in LDS first, so a wave stores them contiguously), and
//     three small launches turn the per-tile counts into global offsets (segmented sums),
//     move the escapes into place and move those of escape-heavy tiles (one launch for
//     calls of at most kSmallTiles tiles), so no workgroup ever waits on another;
//   - decode: codebook lookup with two v_perm_b32 byte selects per 4 codes (codebook in
//     SGPRs), exponent bytes staged in LDS only for tiles that hold escapes, where the
//     escapes overwrite them before the words are assembled.
#include "splitzip_device.h"

namespace sz {

// ======================================================================================
// a1  exponent histograms (calibration, and the per-tensor exponent statistics)
// ======================================================================================

// Workgroup b histograms its share of one tensor (grid-stride over that tensor's 16-byte
// groups: 8 BF16 words or 16 E5M2 bytes) into per-wave LDS sub-histograms and writes the 256
// sums to partial[b] (an E5M2 exponent is 5 bits: bins 32..255 stay 0).
template <uint32_t kElem>
__global__ __launch_bounds__(kThreads) void hist_kernel(const HistArgs a)
{
    // one sub-histogram per wave keeps LDS atomic contention on the few hot exponents down
    __shared__ uint32_t h[kWaves][256];
    __shared__ uint32_t s_cnt[kWaves];
    constexpr uint32_t kPerGroup = kElem == kElemE5M2 ? 16u : 8u;   // elements per 16 bytes
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const uint32_t b = blockIdx.x;
    for (uint32_t i = tid; i < kWaves * 256; i += kThreads)
        (&h[0][0])[i] = 0;
    HistSeg sg = a.seg0;
    uint32_t first = 0, nb = a.n_blocks;
    if (a.n_seg > 1) {
        const uint32_t s = find_range_block(a.block_start, a.n_seg, b, tid, lane, s_cnt);
        first = a.block_start[s];
        nb = a.block_start[s + 1] - first;
        sg = a.segs[s];
    }
    __syncthreads();
    uint32_t *mine = h[tid >> 6];
    const uint8_t *bytes = reinterpret_cast<const uint8_t *>(sg.x);

    const uint64_t groups = sg.n / kPerGroup;
    const uint64_t stride = (uint64_t)nb * kThreads;
    for (uint64_t g = (uint64_t)(b - first) * kThreads + tid; g < groups; g += stride) {
        const uint4 v = *reinterpret_cast<const uint4 *>(bytes + g * 16);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (kElem == kElemE5M2) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    atomicAdd(&mine[(w[k] >> (8 * i + 2)) & 0x1Fu], 1u);
            } else {
                atomicAdd(&mine[(w[k] >> 7) & 0xFFu], 1u);
                atomicAdd(&mine[(w[k] >> 23) & 0xFFu], 1u);
            }
        }
    }
    // ragged tail (fewer than one group), handled by the tensor's first workgroup
    if (b == first && tid < sg.n - groups * kPerGroup) {
        const uint64_t i = groups * kPerGroup + tid;
        const uint32_t e = kElem == kElemE5M2 ? (bytes[i] >> 2) & 0x1Fu : (sg.x[i] >> 7) & 0xFFu;
        atomicAdd(&mine[e], 1u);
    }
    __syncthreads();
    for (uint32_t e = tid; e < 256; e += kThreads) {
        uint32_t sum = 0;
        for (int w = 0; w < kWaves; ++w)
            sum += h[w][e];
        a.partial[(uint64_t)b * 256 + e] = sum;
    }
}

// One workgroup per (tensor, exponent value): its threads add up that bin over the tensor's
// partial histograms.
__global__ __launch_bounds__(kThreads) void hist_reduce_kernel(const HistArgs a)
{
    __shared__ uint64_t s_wave[kWaves];
    const uint32_t s = blockIdx.x >> 8;
    const uint32_t e = blockIdx.x & 255u;
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const uint32_t first = a.n_seg > 1 ? a.block_start[s] : 0u;
    const uint32_t end = a.n_seg > 1 ? a.block_start[s + 1] : a.n_blocks;
    uint64_t sum = 0;
    for (uint32_t b = first + tid; b < end; b += kThreads)
        sum += a.partial[(uint64_t)b * 256 + e];
    sum = wave_total_u64(sum, lane);
    if (lane == 0)
        s_wave[tid >> 6] = sum;
    __syncthreads();
    if (tid == 0) {
        uint64_t t = 0;
        for (int w = 0; w < kWaves; ++w)
            t += s_wave[w];
        a.hist[(uint64_t)s * 256 + e] = t;
    }
}

// Workgroups for one tensor of n words: one per 16 K words, at least 1, at most
// kHistBlocksMax (then each grid-strides).
uint32_t hist_blocks(uint64_t n)
{
    const uint64_t per_block = (uint64_t)kThreads * kGroupWords * 8;
    uint64_t b = (n + per_block - 1) / per_block;
    if (b < 1)
        b = 1;
    if (b > kHistBlocksMax)
        b = kHistBlocksMax;
    return (uint32_t)b;
}

hipError_t launch_histogram(const HistArgs &a, hipStream_t stream)
{
    if (a.elem == kElemE5M2)
        hist_kernel<kElemE5M2><<<a.n_blocks, kThreads, 0, stream>>>(a);
    else
        hist_kernel<kElemBF16><<<a.n_blocks, kThreads, 0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hist_reduce_kernel<<<a.n_seg * 256u, kThreads, 0, stream>>>(a);
    return hipGetLastError();
}

// ======================================================================================
// a2-a4, a7  encode
//
// Four launches (two for small calls), none of which waits on another workgroup:
//   pack   (one workgroup per tile: kEncTileWords BF16 words, or 2^kE8EncTileShift E5M2
//          bytes in splitzip_e5m2.hip): sign+mantissa bits and codes,
//          escape ranks inside the tile, escapes written compacted to the tile's scratch slot
//          (or, past its size, to an overflow area reserved with one atomic), tile-local
//          chunk offsets into chunk_off, the tile's escape count;
//   sums   (one workgroup per kSumTiles tiles): segmented sums of the tile counts;
//   place  (one workgroup per kPlaceTiles tiles): each tile's escape offset from those sums,
//          slot escapes moved to their final positions, chunk offsets made global,
//          per-segment totals;
//   spill  (a fixed grid over the list of overflow tiles): their escapes moved into place,
//          one tile per workgroup at a time, so escape-heavy inputs keep the whole GPU busy.
// Calls of at most kSmallTiles tiles (up to 64 MiB of input) replace sums, place and spill
// with one launch, finish (one workgroup per tile), which adds up the earlier tiles' escape
// counts itself: on inputs of a few MiB every launch costs a few microseconds of the GPU's
// time, more than the data takes to move.
// The one-pass build of pack (kChain) does it all in one launch: each tile publishes its
// escape count in a status word, finds the escapes of the earlier tiles by a decoupled
// look-back over theirs, and writes its escapes, chunk offsets and (as a segment's last tile)
// E to their final places, staging the escapes in LDS so that most of its waves can end
// before the look-back does.  Its E5M2 tiles are half as long (2^kE8ChainTileShift bytes).
// ======================================================================================

// Split one group of 8 words (4 dwords, word 2m in the low half of dword m).
//   sm_lo/sm_hi: sign+mantissa bytes of words 0..3 / 4..7
//   codes:       nibble k = code of word k (0 for escapes)
//   flags:       escape bit of word k at bit 8*(k>>1) + 4 + (k&1)
__device__ __forceinline__ void split_group(const uint4 v, const uint8_t *lut, uint32_t &sm_lo,
                                            uint32_t &sm_hi, uint32_t &codes, uint32_t &flags)
{
    // sign+mantissa: low byte of each word gives mantissa (bits 0..6), high byte gives the
    // sign (bit 7); gather the 4 low and the 4 high bytes, then merge with one bit-select.
    sm_lo = (perm(v.y, v.x, 0x07050301u) & 0x80808080u) | (perm(v.y, v.x, 0x06040200u) & 0x7F7F7F7Fu);
    sm_hi = (perm(v.w, v.z, 0x07050301u) & 0x80808080u) | (perm(v.w, v.z, 0x06040200u) & 0x7F7F7F7Fu);

    const uint32_t c0 = lut[(v.x >> 7) & 0xFFu], c1 = lut[(v.x >> 23) & 0xFFu];
    const uint32_t c2 = lut[(v.y >> 7) & 0xFFu], c3 = lut[(v.y >> 23) & 0xFFu];
    const uint32_t c4 = lut[(v.z >> 7) & 0xFFu], c5 = lut[(v.z >> 23) & 0xFFu];
    const uint32_t c6 = lut[(v.w >> 7) & 0xFFu], c7 = lut[(v.w >> 23) & 0xFFu];
    const uint32_t even = c0 | (c2 << 8) | (c4 << 16) | (c6 << 24);
    const uint32_t odd = c1 | (c3 << 8) | (c5 << 16) | (c7 << 24);
    codes = (even & 0x0F0F0F0Fu) | ((odd & 0x0F0F0F0Fu) << 4);
    flags = (even & 0x10101010u) | ((odd & 0x10101010u) << 1);
}

__device__ __forceinline__ uint32_t flag_bit_to_word(uint32_t b) { return ((b >> 3) << 1) | (b & 1u); }

// Mask keeping the codes / escape flags of the first nv (< 8) words of a group.
__device__ __forceinline__ uint32_t codes_keep(uint32_t nv) { return nv >= 8 ? ~0u : (1u << (4 * nv)) - 1u; }
__device__ __forceinline__ uint32_t flags_keep(uint32_t nv)
{
    return nv >= 8 ? ~0u : (1u << (8 * (nv >> 1) + 4 + (nv & 1))) - 1u;
}

// ---- pack ---------------------------------------------------------------------------------

// kChain: the one-pass build (chained tiles), which writes the escapes to their final places.
template <bool kStage, bool kChain>
__global__ __launch_bounds__(kThreads) void encode_pack_kernel(const EncodeArgs a)
{
    __shared__ uint8_t s_lut[256];
    __shared__ uint32_t s_wave_total[kWaves];
    __shared__ uint64_t s_ovf;
    // one group's escapes per wave; in the one-pass build also the early-release stash
    constexpr uint32_t kStageWords = kWaves * 64 * kGroupWords;
    constexpr uint32_t kStashExpAt = kStashPosAt + 2 * kStashEscapes + 16;
    constexpr uint32_t kStashWords = (kStashExpAt + kStashEscapes + 2 * kStashChunks + 3) / 4;
    __shared__ uint32_t s_stage[kChain && kStashWords > kStageWords ? kStashWords : kStageWords];
    // one-pass build: for each 8-bit escape mask, the indices of its set bits (set_bit_indices)
    __shared__ uint2 s_bitpos[kChain ? 256 : 1];
    // one-pass build: set when wave 0 has copied the stash out and put the tile's escape offset
    // in s_before (stash_rest)
    __shared__ uint32_t s_out;
    __shared__ uint64_t s_before;

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t t = blockIdx.x;

    const uint32_t s = a.n_seg > 1 ? find_segment_block(a.tile_start, a.seg_at, t, tid, lane, s_wave_total) : 0u;
    const SegDesc sd = segment_desc(a, s);
    // the segment's inverse LUT (several codebooks in one call: one LUT per codebook), loaded
    // now and put in LDS after the tile's loads are issued, so that none of them waits for it
    const uint8_t *lut = a.multi_book ? a.lut + 256u * sd.book : a.lut;
    const uint32_t lut_word = tid < 64 ? reinterpret_cast<const uint32_t *>(lut)[tid & 63u] : 0u;
    if (!kChain && a.packed && tid == 0 && t == segment_first_tile(a, s))
        a.seg_total[s] = 0;      // the sums launch adds the segment's escapes into it
    if (kChain) {
        s_bitpos[tid & 255u] = set_bit_indices(tid & 255u);
        if (tid == 0)
            s_out = 0;
    }
    const uint64_t tag = a.chain_tag;
    const uint64_t n = sd.n;
    const SZ_GLOBAL uint16_t *xw = as_global(sd.data);
    SZ_GLOBAL uint8_t *smb = as_global(sd.sm);
    SZ_GLOBAL uint8_t *cdb = as_global(sd.codes);
    SZ_GLOBAL uint64_t *chunk_off = as_global(sd.chunk_off);
    const uint64_t base = (uint64_t)(t - segment_first_tile(a, s)) << kEncTileShift;
    const uint64_t cmask = (1ull << a.log2_chunk) - 1;

    // word order inside the tile: wave w covers 64 * 8 * kEncGroups consecutive words, its group
    // j covers 512 of them, lane l the 8 at offset 8 l.
    uint64_t g0[kEncGroups];
    uint4 v[kEncGroups];
#pragma unroll
    for (int j = 0; j < kEncGroups; ++j) {
        g0[j] = base + (uint64_t)(((wave * kEncGroups + j) << 6) + lane) * kGroupWords;
        if (g0[j] + kGroupWords <= n) {
            v[j] = load_stream16(sd.data + g0[j]);
        } else {
            uint16_t wds[8];
#pragma unroll
            for (int k = 0; k < 8; ++k)
                wds[k] = (g0[j] + k < n) ? xw[g0[j] + k] : (uint16_t)0;
            v[j] = make_uint4(wds[0] | ((uint32_t)wds[1] << 16), wds[2] | ((uint32_t)wds[3] << 16),
                              wds[4] | ((uint32_t)wds[5] << 16), wds[6] | ((uint32_t)wds[7] << 16));
        }
    }
    if (tid < 64)
        reinterpret_cast<uint32_t *>(s_lut)[tid] = lut_word;
    __syncthreads();   // LUT in LDS

    // ---- a2: dense split and pack ---------------------------------------------------------
    uint32_t flags[kEncGroups];
    uint32_t counts[kEncGroups];
#pragma unroll
    for (int j = 0; j < kEncGroups; ++j) {
        uint32_t sm_lo, sm_hi, codes, fl;
        split_group(v[j], s_lut, sm_lo, sm_hi, codes, fl);
        if (g0[j] + kGroupWords <= n) {
            store_stream8(sd.sm + g0[j], sm_lo, sm_hi);
            store_stream4(sd.codes + (g0[j] >> 1), codes);
        } else {
            const uint32_t nv = g0[j] < n ? (uint32_t)(n - g0[j]) : 0u;
            codes &= codes_keep(nv);
            fl &= flags_keep(nv);
            for (uint32_t k = 0; k < nv; ++k)
                smb[g0[j] + k] = (uint8_t)((k < 4 ? sm_lo : sm_hi) >> (8 * (k & 3)));
            for (uint32_t k = 0; k < (nv + 1) / 2; ++k)
                cdb[(g0[j] >> 1) + k] = (uint8_t)(codes >> (8 * k));
        }
        flags[j] = fl;
        counts[j] = __popc(fl);
    }

    // ---- a3: escape ranks inside the tile ---------------------------------------------------
    // Word order inside a wave is (group j, lane, word k).
    uint32_t rank[kEncGroups];
    uint32_t tile_total;
    uint32_t wave_end;
    tile_escape_ranks<kEncGroups>(counts, lane, wave, s_wave_total, rank, tile_total, wave_end);
    if (a.first_tile_escapes && t == 0 && tid == 0)
        __hip_atomic_store(a.first_tile_escapes, tile_total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);

    if (kChain) {
        // one pass, early release: the escapes of rank below kStashEscapes (every escape of a
        // tile with at most that many) wait in LDS with their final u16 position and exponent
        // byte, and the chunk starts' ranks with them.  Waves whose escapes all fit end;
        // wave 0 (whose escapes always fit) waits for the tile's escape offset and writes
        // them to their final places; a wave with escapes past the stash gets the offset
        // from wave 0 through LDS and writes those itself.
        uint8_t *lds = reinterpret_cast<uint8_t *>(s_stage);
        uint16_t *s_pos = reinterpret_cast<uint16_t *>(lds + kStashPosAt);
        uint8_t *s_exp = lds + kStashExpAt;
        uint16_t *s_start = reinterpret_cast<uint16_t *>(s_exp + kStashEscapes);
        const uint32_t first = segment_first_tile(a, s);
        const bool last = t + 1 == segment_end_tile(a, s);        // loaded before the waits below
        if (tid == 0)
            chain_publish(a, t, chain_word(tag, t > first ? kChainAggregate : kChainPrefix, tile_total));
        // wave 0 issues the look-back's first loads now; they return while the escapes go to LDS
        uint64_t w[kChainRows];
        if (wave == 0 && t > first)
            chain_load<kChainRows>(a, t - 1, first, lane, w);
        const uint32_t cm = (uint32_t)cmask;
        // the lane's escapes of rank lo .. hi - 1 to LDS at rank - lo: a lane's escapes of
        // group j have ranks rank[j], rank[j] + 1, ...; the i-th goes in step i.  The word
        // indices of a group's escapes come from the table of set bits, one per byte: one byte
        // permute turns two of them into two u16 positions (a group starts 8-aligned inside its
        // chunk, so position = the group's place in the chunk + index), and one more four of
        // them into their exponent bytes.  Without a range check (kRanged false) every escape
        // of the lane must lie in lo .. hi - 1.
        auto stash = [&](auto ranged, uint32_t lo, uint32_t hi, uint32_t at) {
            constexpr bool kRanged = decltype(ranged)::value;
#pragma unroll
            for (int j = 0; j < kEncGroups; ++j) {
                const uint32_t r0 = rank[j];
                const uint32_t z = flags[j];
                if (z && (!kRanged || (r0 < hi && r0 + 8u > lo))) {
                    const uint32_t elo = perm(v[j].y >> 7, v[j].x >> 7, 0x06040200u);   // exponents, words 0..3
                    const uint32_t ehi = perm(v[j].w >> 7, v[j].z >> 7, 0x06040200u);   // words 4..7
                    const uint32_t f = (((z >> 4) & 0x03030303u) * 0x01041040u) >> 24;   // bit k: word k escapes
                    const uint32_t cnt = __popc(f);
                    const uint2 ks = s_bitpos[f];
                    // the group's place in its chunk, in both halves (recomputed: g0 is not kept)
                    const uint32_t pq = (((uint32_t)base + ((wave * kEncGroups + j) << 9) + lane * kGroupWords) & cm) *
                                        0x10001u;
                    uint32_t pp = 0, ee = 0;
#pragma unroll
                    for (int i = 0; i < kGroupWords; ++i) {
                        if (!__ballot((uint32_t)i < cnt))
                            break;
                        const uint32_t kx = i < 4 ? ks.x : ks.y;
                        if ((i & 1) == 0)    // positions of escapes i, i + 1
                            pp = pq + perm(0u, kx, (i & 2) ? 0x0C030C02u : 0x0C010C00u);
                        if ((i & 3) == 0)    // exponents of escapes i .. i + 3
                            ee = perm(ehi, elo, kx);
                        const uint32_t r = r0 + i;
                        if ((uint32_t)i < cnt && (!kRanged || (r >= lo && r < hi))) {
                            s_pos[r - lo + at] = (uint16_t)(pp >> (16 * (i & 1)));
                            s_exp[r - lo + at] = (uint8_t)(ee >> (8 * (i & 3)));
                        }
                    }
                }
            }
        };
#pragma unroll
        for (int j = 0; j < kEncGroups; ++j) {
            const uint32_t p0 = (uint32_t)(g0[j] - base);
            if (g0[j] < n && (g0[j] & cmask) == 0)
                s_start[p0 >> a.log2_chunk] = (uint16_t)rank[j];
        }
        const bool past = wave_end > kStashEscapes;                 // uniform in the wave
        if (past)
            stash(BoolTag<true>{}, 0, kStashEscapes, 0);
        else
            stash(BoolTag<false>{}, 0, kStashEscapes, 0);
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
                if (tile_total > kStashEscapes)
                    s_before = before;
            }
            const uint64_t tile_end = base + kEncTileWords < n ? base + kEncTileWords : n;
            const uint32_t starts = a.log2_chunk <= (uint32_t)kEncTileShift
                                  ? (uint32_t)((tile_end - base + cmask) >> a.log2_chunk)
                                  : ((base & cmask) == 0 ? 1u : 0u);
            SZ_GLOBAL uint64_t *co = chunk_off + (base >> a.log2_chunk);
            for (uint32_t i = lane; i < starts; i += 64)
                co[i] = before + s_start[i];
            const uint64_t left = sd.esc > before && sd.esc_exp ? sd.esc - before : 0;
            uint32_t ne = left < tile_total ? (uint32_t)left : tile_total;
            ne = ne < kStashEscapes ? ne : kStashEscapes;
            if (ne) {
                stash_copy<2>(as_global(sd.esc_pos + before), s_pos, ne, lane);
                stash_copy<1>(as_global(sd.esc_exp + before), s_exp, ne, lane);
            }
            if (tile_total > kStashEscapes && lane == 0)      // the stash is out
                __hip_atomic_store(&s_out, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            return;
        }
        // a wave with escapes past the stash: once wave 0 has copied it out, they go through it
        // again (stash_rest)
        const uint32_t wave_first = (uint32_t)__builtin_amdgcn_readfirstlane(rank[0]);   // lane 0's group 0
        stash_rest<kStashEscapes, kEncTileWords>(a, sd, &s_out, &s_before, wave, wave_first, wave_end, lane,
                                                 s_pos, s_exp, stash);
        return;
    }

    // where the tile's escapes go: its slot, or a range of the overflow area
    uint64_t room = 0;
    uint32_t *dst = tile_escape_dest(a, t, tile_total, tid, &s_ovf, room);

    // escapes: (position inside the tile, exponent); tile-local chunk offsets.  A wave's
    // escapes of one group have consecutive ranks.  When there are more than kStageMin of
    // them they are gathered in the wave's LDS buffer first (each word in turn, at its rank)
    // and stored 64 consecutive entries per instruction; a few are stored directly by the
    // lanes that hold them.
    SZ_GLOBAL uint32_t *gdst = as_global(dst);
    uint32_t *stage = s_stage + wave * 64 * kGroupWords;
#pragma unroll
    for (int j = 0; j < kEncGroups; ++j) {
        const uint32_t r0 = rank[j];
        if (g0[j] < n && (g0[j] & cmask) == 0)
            chunk_off[g0[j] >> a.log2_chunk] = r0;
        const uint32_t z = flags[j];
        const uint32_t w0 = __builtin_amdgcn_readfirstlane(r0);
        const uint32_t wcnt = (j + 1 < kEncGroups ? __builtin_amdgcn_readfirstlane(rank[j + 1]) : wave_end) - w0;
        const bool staged = kStage && __builtin_expect(wcnt > kStageMin, 0);   // uniform in the wave
        if (z) {
            // the group's 8 exponents, word k in byte k (a dword >> 7 holds the exponent of its
            // low word in byte 0 and of its high word in byte 2)
            const uint64_t ex8 = perm(v[j].y >> 7, v[j].x >> 7, 0x06040200u)
                               | ((uint64_t)perm(v[j].w >> 7, v[j].z >> 7, 0x06040200u) << 32);
            const uint32_t p0 = (uint32_t)(g0[j] - base);
            if (staged) {
                // each of the 8 words in turn: an escape goes to its rank in the wave's buffer
                const uint32_t at = r0 - w0;
#pragma unroll
                for (int k = 0; k < kGroupWords; ++k) {
                    const uint32_t bit = ((k >> 1) << 3) + 4 + (k & 1);    // flag bit of word k
                    if ((z >> bit) & 1u)
                        stage[at + __popc(z & ((1u << bit) - 1u))] =
                            (p0 + k) | ((uint32_t)(uint8_t)(ex8 >> (8 * k)) << 16);
                }
            } else {
                uint32_t zz = z, r = r0;
                do {
                    const uint32_t k = flag_bit_to_word((uint32_t)__builtin_ctz(zz));
                    if (r < room)
                        gdst[r] = (p0 + k) | ((uint32_t)(uint8_t)(ex8 >> (8 * k)) << 16);
                    ++r;
                    zz &= zz - 1;
                } while (zz);
            }
        }
        if (staged) {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            for (uint32_t i = lane; i < wcnt; i += 64) {
                if (w0 + i < room)
                    gdst[w0 + i] = stage[i];
            }
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        }
    }
}

// ---- sums ---------------------------------------------------------------------------------

// Segmented sum: (head, value) pairs combined in order; a head (first tile of a segment)
// discards what came before it.
struct SegSum {
    uint32_t head;
    uint64_t v;
};

__device__ __forceinline__ SegSum seg_combine(SegSum a, SegSum b)
{
    return SegSum{a.head | b.head, b.head ? b.v : a.v + b.v};
}

__device__ __forceinline__ SegSum seg_shfl_up(SegSum x, uint32_t d, uint32_t lane)
{
    const uint32_t src = lane >= d ? lane - d : lane;
    SegSum y;
    y.head = shfl_u32(x.head, src);
    y.v = ((uint64_t)shfl_u32((uint32_t)(x.v >> 32), src) << 32) | shfl_u32((uint32_t)x.v, src);
    return y;
}

// Inclusive segmented scan over the 256 threads of the workgroup (thread order).
__device__ SegSum block_seg_scan(SegSum x, uint32_t tid, uint32_t lane, SegSum *s_wave)
{
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const SegSum y = seg_shfl_up(x, d, lane);
        if (lane >= d)
            x = seg_combine(y, x);
    }
    if (lane == 63)
        s_wave[tid >> 6] = x;
    __syncthreads();
    SegSum carry{0, 0};
    for (uint32_t w = 0; w < (tid >> 6); ++w)
        carry = seg_combine(carry, s_wave[w]);
    __syncthreads();
    return seg_combine(carry, x);
}

__device__ __forceinline__ bool is_segment_head(const EncodeArgs &a, uint32_t u)
{
    return segment_first_tile(a, tile_segment(a, u)) == u;
}

// Segmented fold of the tile counts [u, u + len) ∩ [0, limit) in order.
__device__ __forceinline__ SegSum fold_tiles(const EncodeArgs &a, uint32_t u, uint32_t len,
                                             uint32_t limit)
{
    SegSum acc{0, 0};
    for (uint32_t i = 0; i < len && u + i < limit; ++i)
        acc = seg_combine(acc, SegSum{is_segment_head(a, u + i) ? 1u : 0u, a.tile_count[u + i]});
    return acc;
}

__global__ __launch_bounds__(kThreads) void encode_sums_kernel(const EncodeArgs a)
{
    __shared__ SegSum s_wave[kWaves];
    __shared__ SegSum s_incl[kThreads];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const uint32_t per = kSumTiles / kThreads;
    const uint32_t u0 = blockIdx.x * kSumTiles + tid * per;
    const SegSum mine = fold_tiles(a, u0, per, a.n_tiles);

    // one sum per group of kPlaceTiles tiles (kPlaceTiles / per consecutive lanes)
    constexpr uint32_t kLanesPerGroup = kPlaceTiles / (kSumTiles / kThreads);
    SegSum g = mine;
#pragma unroll
    for (uint32_t d = 1; d < kLanesPerGroup; d <<= 1) {
        const SegSum y = seg_shfl_up(g, d, lane);
        if ((lane & (kLanesPerGroup - 1)) >= d)
            g = seg_combine(y, g);
    }
    const uint32_t group = blockIdx.x * (kSumTiles / kPlaceTiles) + tid / kLanesPerGroup;
    if ((lane & (kLanesPerGroup - 1)) == kLanesPerGroup - 1 && group * kPlaceTiles < a.n_tiles)
        a.group_sum[group] = g.v | ((uint64_t)g.head << 63);

    const SegSum all = block_seg_scan(mine, tid, lane, s_wave);
    if (tid == kThreads - 1)
        a.block_sum[blockIdx.x] = all.v | ((uint64_t)all.head << 63);
    if (blockIdx.x == 0 && tid == 0) {
        // the pack launch of this encode has finished with the counter: keep its final value
        // for the spill launch and leave it at 0 for the next encode
        a.ovf_ctr[1] = a.ovf_ctr[0];
        a.ovf_ctr[0] = 0;
    }
    if (a.packed) {
        // E of every segment, needed before placement (the exponents follow the E positions).
        // Each thread adds up its tiles per segment, starting from the earlier threads' running
        // sum of its first segment, and adds a segment's part of this block to its total where
        // that part ends: at a segment end inside the thread's tiles, at the end of the
        // thread's tiles if the segment ends there, or at the end of the block.
        s_incl[tid] = all;
        __syncthreads();
        const uint32_t end = u0 + per < a.n_tiles ? u0 + per : a.n_tiles;
        if (u0 < end) {
            uint32_t sg = tile_segment(a, u0);
            uint64_t acc = (tid > 0 && segment_first_tile(a, sg) != u0) ? s_incl[tid - 1].v : 0;
            for (uint32_t u = u0; u < end; ++u) {
                if (u == segment_end_tile(a, sg)) {
                    if (acc)
                        atomicAdd((unsigned long long *)&a.seg_total[sg], (unsigned long long)acc);
                    acc = 0;
                    ++sg;
                }
                acc += a.tile_count[u];
            }
            if (acc && (tid == kThreads - 1 || end == a.n_tiles || segment_end_tile(a, sg) == end))
                atomicAdd((unsigned long long *)&a.seg_total[sg], (unsigned long long)acc);
        }
    }
}

// ---- packed layout --------------------------------------------------------------------------

// Exponent array of a packed stream holding E escapes: right after the E positions.  NULL
// when E exceeds the escape capacity (the exponents would run past the buffer): then no
// escape is stored and the caller sees E > capacity.
__device__ __forceinline__ uint8_t *packed_exps(const SegDesc &sd, uint64_t E)
{
    return E <= sd.esc ? reinterpret_cast<uint8_t *>(sd.esc_pos + E) : nullptr;
}

// The 64-byte canonical header: "SZB1", version 1, header bytes 64, chunk size, flags (the
// element type: 0 BF16, 1 E5M2), n, n_chunks, E, the segment's codebook, 8 zero bytes (all
// little-endian).
__device__ void write_header(const SegDesc &sd, const EncodeArgs &a, uint64_t E)
{
    const uint64_t C = 1ull << a.log2_chunk;
    const uint64_t n_chunks = (sd.n + C - 1) >> a.log2_chunk;
    const uint32_t *cb = a.cbs + 4u * sd.book;
    uint4 *h = reinterpret_cast<uint4 *>(sd.header);
    h[0] = make_uint4(0x31425A53u, 1u | (64u << 16), (uint32_t)C, a.elem);
    h[1] = make_uint4((uint32_t)sd.n, (uint32_t)(sd.n >> 32), (uint32_t)n_chunks, (uint32_t)(n_chunks >> 32));
    h[2] = make_uint4((uint32_t)E, (uint32_t)(E >> 32), cb[0], cb[1]);
    h[3] = make_uint4(cb[2], cb[3], 0u, 0u);
}

// ---- place --------------------------------------------------------------------------------

// Index i in [0, n) of a sorted start array with first[i] <= j < first[i + 1].
__device__ __forceinline__ uint32_t range_of(const uint32_t *first, uint32_t n, uint32_t j)
{
    uint32_t lo = 0, hi = n;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (first[mid] <= j)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// Inclusive segmented scan over the 64 lanes of a wave (all lanes active).
__device__ __forceinline__ SegSum wave_seg_scan(SegSum x, uint32_t lane)
{
#pragma unroll
    for (uint32_t d = 1; d < 64; d <<= 1) {
        const SegSum y = seg_shfl_up(x, d, lane);
        if (lane >= d)
            x = seg_combine(y, x);
    }
    return x;
}

__device__ __forceinline__ SegSum lane63(SegSum x)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)x.v, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(x.v >> 32), 63);
    return SegSum{(uint32_t)__builtin_amdgcn_readlane(x.head, 63), ((uint64_t)hi << 32) | lo};
}

__device__ __forceinline__ SegSum unpack_sum(uint64_t x)
{
    return SegSum{(uint32_t)(x >> 63), x & ~(1ull << 63)};
}

__global__ __launch_bounds__(kThreads) void encode_place_kernel(const EncodeArgs a)
{
    static_assert(kPlaceTiles == 64, "a placement group is one wave: one lane per tile");
    // per tile, so that the loops below load no segment descriptor
    __shared__ uint64_t s_prefix[kPlaceTiles];   // escape offset of the tile in its segment
    __shared__ uint64_t s_base[kPlaceTiles];     // first word of the tile in its segment
    __shared__ uint64_t s_room[kPlaceTiles];     // escape capacity left from s_prefix on
    __shared__ uint64_t *s_cptr[kPlaceTiles];    // first chunk offset that starts in the tile
    __shared__ uint16_t *s_pos[kPlaceTiles];     // the segment's escape positions
    __shared__ uint8_t *s_exps[kPlaceTiles];     // its escape exponents (NULL: none written)
    __shared__ uint32_t s_first[kPlaceTiles + 1];   // escapes: start of each tile's range
    __shared__ uint32_t s_cfirst[kPlaceTiles + 1];  // chunk offsets: start of each tile's range

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const uint32_t group = blockIdx.x;
    const uint32_t u_first = group * kPlaceTiles;
    const uint64_t cmask = (1ull << a.log2_chunk) - 1;

    // Wave 0 (one lane per tile) works out each tile's escape offset and the flattened ranges
    // of the group's escapes and chunk offsets, with wave-level scans only: every load it needs
    // is known up front, and no workgroup barrier stands between them.
    if (tid < 64) {
        const uint32_t u = u_first + lane;
        const bool valid = u < a.n_tiles;
        const uint32_t count = valid ? a.tile_count[u] : 0u;
        const uint32_t seg = valid ? tile_segment(a, u) : 0u;
        const uint32_t head = valid && segment_first_tile(a, seg) == u ? 1u : 0u;

        // carry-in: segmented sum of every tile before u_first, folded in order from the sums of
        // the earlier sum blocks (64 at a time) and of this block's earlier groups
        const uint32_t sum_block = u_first / kSumTiles;
        const uint32_t g0 = sum_block * (kSumTiles / kPlaceTiles);
        const SegSum grp = g0 + lane < group ? unpack_sum(a.group_sum[g0 + lane]) : SegSum{0, 0};
        SegSum before{0, 0};
        for (uint32_t r = 0; r < sum_block; r += 64) {
            const uint32_t b = r + lane;
            const SegSum blk = b < sum_block ? unpack_sum(a.block_sum[b]) : SegSum{0, 0};
            before = seg_combine(before, lane63(wave_seg_scan(blk, lane)));
        }
        before = seg_combine(before, lane63(wave_seg_scan(grp, lane)));

        // exclusive segmented prefix of each tile = carry-in combined with the earlier tiles
        const SegSum incl = wave_seg_scan(SegSum{head, count}, lane);
        const SegSum with_carry = seg_combine(before, incl);
        const uint64_t prefix = head ? 0 : with_carry.v - count;
        uint64_t base = 0, room = 0;
        uint64_t *cptr = nullptr;
        uint16_t *pos = nullptr;
        uint8_t *exps = nullptr;
        uint32_t n_chunks_here = 0;
        if (valid) {
            const SegDesc sd = segment_desc(a, seg);
            base = (uint64_t)(u - segment_first_tile(a, seg)) << a.tile_shift;
            if (u + 1 == segment_end_tile(a, seg)) {
                // the segment's last tile knows the segment's escape count
                const uint64_t E = prefix + count;
                sd.chunk_off[(sd.n + cmask) >> a.log2_chunk] = E;
                a.seg_escapes[seg] = E;
                if (a.packed)
                    write_header(sd, a, E);
            }
            if (base < sd.n) {
                // chunks that start inside this tile
                const uint64_t tile_words = 1ull << a.tile_shift;
                const uint64_t words = sd.n - base < tile_words ? sd.n - base : tile_words;
                const uint64_t c_first = (base + cmask) >> a.log2_chunk;
                n_chunks_here = (uint32_t)(((base + words + cmask) >> a.log2_chunk) - c_first);
                cptr = sd.chunk_off + c_first;
            }
            pos = sd.esc_pos;
            exps = a.packed ? packed_exps(sd, a.seg_total[seg]) : sd.esc_exp;
            room = prefix < sd.esc ? sd.esc - prefix : 0;
        }
        // overflow tiles are moved by the spill launch; the others here, from their slots
        const bool spilled = count > a.slot_escapes;
        if (valid && (spilled || a.private_ovf)) {
            // the spill launch's record (with private regions every tile has one, so that spill
            // reads it alone): escapes past the escape capacity, or with no exponent section,
            // or outside the overflow area, are not moved
            uint64_t lim = 0, off = 0;
            if (spilled && exps) {
                off = a.tile_ovf[u];
                const uint64_t ovf_room = off < a.ovf_cap ? a.ovf_cap - off : 0;
                lim = count < ovf_room ? count : ovf_room;
                lim = lim < room ? lim : room;
            }
            SpillRec r;
            r.pos = pos + prefix;
            r.exp = exps ? exps + prefix : nullptr;
            r.base = base;
            r.src = off | (lim << kOvfTileShift);
            a.spill_rec[u] = r;
        }
        s_prefix[lane] = prefix;
        s_base[lane] = base;
        s_room[lane] = room;
        s_cptr[lane] = cptr;
        s_pos[lane] = pos;
        s_exps[lane] = exps;
        // where each tile's escapes and chunk offsets fall in the group's flattened ranges (at
        // most 64 slots of escapes and 64 x 2048 chunk starts: both fit 32 bits)
        s_first[lane + 1] = wave_inclusive_sum(spilled ? 0u : count, lane);
        s_cfirst[lane + 1] = wave_inclusive_sum(n_chunks_here, lane);
        if (lane == 0) {
            s_first[0] = 0;
            s_cfirst[0] = 0;
        }
    }
    __syncthreads();

    // tile-local chunk offsets become segment offsets: consecutive threads take consecutive
    // entries, four loads in flight before the stores
    constexpr int kBatch = 4;
    const uint32_t total_c = s_cfirst[kPlaceTiles];
    for (uint32_t e0 = tid; e0 < total_c; e0 += kBatch * kThreads) {
        uint64_t *where[kBatch];
        uint64_t val[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const uint32_t e = e0 + k * kThreads;
            where[k] = nullptr;
            if (e < total_c) {
                const uint32_t i = range_of(s_cfirst, kPlaceTiles, e);
                where[k] = s_cptr[i] + (e - s_cfirst[i]);
                val[k] = *as_global(where[k]) + s_prefix[i];
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (where[k])
                *as_global(where[k]) = val[k];
    }

    // move the slot escapes: consecutive threads take consecutive escapes (coalesced reads of
    // the scratch entries, coalesced writes of the final arrays), four loads in flight
    const uint32_t total = s_first[kPlaceTiles];
    for (uint32_t j0 = tid; j0 < total; j0 += kBatch * kThreads) {
        uint32_t ent[kBatch], tile_of[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const uint32_t j = j0 + k * kThreads;
            tile_of[k] = kPlaceTiles;
            if (j < total) {
                const uint32_t i = range_of(s_first, kPlaceTiles, j);
                tile_of[k] = i;
                ent[k] = a.slots[(uint64_t)(u_first + i) * a.slot_escapes + (j - s_first[i])];
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const uint32_t i = tile_of[k];
            if (i == kPlaceTiles)
                continue;
            const uint32_t r = j0 + k * kThreads - s_first[i];
            uint8_t *exps = s_exps[i];
            if (r < s_room[i] && exps) {
                const uint64_t d = s_prefix[i] + r;
                as_global(s_pos[i])[d] = (uint16_t)((s_base[i] + (ent[k] & 0xFFFFu)) & cmask);
                as_global(exps)[d] = (uint8_t)(ent[k] >> 16);
            }
        }
    }
}

// ---- spill --------------------------------------------------------------------------------

// Moves lim scratch escapes src[0 .. lim) of the tile whose words start at `base` to their
// final places pos[0 .. lim) and ex[0 .. lim), kMovePass at a time: loaded 16 per thread
// (consecutive threads, consecutive entries), split into position and exponent in LDS at
// indices shifted so that LDS quads line up with 8-byte (positions) and 4-byte (exponents)
// boundaries of the destination, then stored a whole quad per store, the partial quads at the
// two ends element by element.  Stored one element per lane, the 2- and 1-byte stores cost
// four times as many store instructions.  Contains barriers: lim must be the same in every
// thread of the workgroup.
constexpr int kMoveBatch = 16;
constexpr uint32_t kMovePass = kMoveBatch * kThreads;
struct MoveLds {
    __align__(16) uint16_t pos[kMovePass + 8];
    __align__(16) uint8_t exp[kMovePass + 8];
};

__device__ void move_escapes(const uint32_t *src, uint64_t lim, uint16_t *pos, uint8_t *ex,
                             uint64_t base, uint64_t cmask, uint32_t tid, MoveLds &L)
{
    const SZ_GLOBAL uint32_t *gsrc = as_global(src);
    for (uint64_t p0 = 0; p0 < lim; p0 += kMovePass) {
        const uint32_t m = lim - p0 < kMovePass ? (uint32_t)(lim - p0) : kMovePass;
        SZ_GLOBAL uint16_t *gpos = as_global(pos + p0);
        SZ_GLOBAL uint8_t *gexp = as_global(ex + p0);
        const uint32_t shp = (uint32_t)(((uintptr_t)(pos + p0) >> 1) & 3u);
        const uint32_t shx = (uint32_t)((uintptr_t)(ex + p0) & 3u);
        uint32_t e[kMoveBatch];
#pragma unroll
        for (int k = 0; k < kMoveBatch; ++k)
            if (tid + k * kThreads < m)
                e[k] = gsrc[p0 + tid + k * kThreads];
#pragma unroll
        for (int k = 0; k < kMoveBatch; ++k) {
            const uint32_t r = tid + k * kThreads;
            if (r < m) {
                L.pos[shp + r] = (uint16_t)((base + (e[k] & 0xFFFFu)) & cmask);
                L.exp[shx + r] = (uint8_t)(e[k] >> 16);
            }
        }
        __syncthreads();
        // LDS quad q holds destination elements 4 q - sh .. 4 q - sh + 3 of this pass
        const uint32_t nqp = (shp + m + 3) >> 2;
        for (uint32_t q = tid; q < nqp; q += kThreads) {
            const uint32_t lo = 4 * q, hi = 4 * q + 4;
            if (lo >= shp && hi <= shp + m) {
                *reinterpret_cast<SZ_GLOBAL uint64_t *>(gpos + lo - shp) =
                    *reinterpret_cast<const uint64_t *>(L.pos + lo);
            } else {
                for (uint32_t x = lo; x < hi; ++x)
                    if (x >= shp && x < shp + m)
                        gpos[x - shp] = L.pos[x];
            }
        }
        const uint32_t nqx = (shx + m + 3) >> 2;
        for (uint32_t q = tid; q < nqx; q += kThreads) {
            const uint32_t lo = 4 * q, hi = 4 * q + 4;
            if (lo >= shx && hi <= shx + m) {
                *reinterpret_cast<SZ_GLOBAL uint32_t *>(gexp + lo - shx) =
                    *reinterpret_cast<const uint32_t *>(L.exp + lo);
            } else {
                for (uint32_t x = lo; x < hi; ++x)
                    if (x >= shx && x < shx + m)
                        gexp[x - shx] = L.exp[x];
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(kThreads) void encode_spill_kernel(const EncodeArgs a)
{
    __shared__ MoveLds s_move;
    const uint32_t tid = threadIdx.x;
    const uint64_t cmask = (1ull << a.log2_chunk) - 1;
    // the overflow tiles: listed by the pack launch, or, with private regions, every tile (its
    // record says how many entries it has to move: 0 when it fit its slot).  One workgroup per
    // tile: splitting tiles, in this grid or in one sized to them, was slower.
    const uint32_t n_items = a.private_ovf ? a.n_tiles : (uint32_t)(a.ovf_ctr[1] >> kOvfTileShift);
    for (uint32_t i = blockIdx.x; i < n_items; i += gridDim.x) {
        const uint32_t t = a.private_ovf ? i : a.ovf_tiles[i];
        const SpillRec r = a.spill_rec[t];
        const uint64_t lim = r.src >> kOvfTileShift;
        if (lim == 0)
            continue;                                  // uniform
        move_escapes(a.ovf + (r.src & kOvfOffsetMask), lim, r.pos, r.exp, r.base, cmask, tid, s_move);
    }
}

// ---- finish (calls of at most kSmallTiles tiles) ------------------------------------------

// log2 of the finish workgroups per tile: several in the large-call build (they share an
// escape-heavy tile's moves), one in calls of more than kFinishPartTiles tiles, whose every
// workgroup also adds up the counts of the earlier tiles.
__host__ __device__ inline uint32_t finish_part_shift(const EncodeArgs &a)
{
    return a.stage && a.n_tiles <= kFinishPartTiles ? kFinishPartShift : 0u;
}

// Sum of v over the workgroup, in every thread.  Contains barriers.
__device__ __forceinline__ uint64_t block_total_u64(uint64_t v, uint32_t tid, uint32_t lane,
                                                    uint64_t *s_part)
{
    v = wave_total_u64(v, lane);
    if (lane == 0)
        s_part[tid >> 6] = v;
    __syncthreads();
    uint64_t total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
        total += s_part[w];
    __syncthreads();
    return total;
}

// One workgroup per tile does the work of the sums, place and spill launches for its own
// tile: its escape offset is the sum of the escape counts of its segment's earlier tiles
// (fewer than kSmallTiles, all loaded at once), then its chunk offsets become segment offsets
// and its escapes move from the slot, or from the overflow area, to their final positions.
// The segment's last tile also writes E (and the header of a packed stream).
__global__ __launch_bounds__(kThreads) void encode_finish_kernel(const EncodeArgs a)
{
    __shared__ uint32_t s_cnt[kWaves];
    __shared__ uint64_t s_part[kWaves];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    // In the large-call build each tile has kFinishParts workgroups, which share its escape
    // moves: a tile whose elements all escape needs several rounds of loads and stores, most
    // tiles one, and the slowest tiles set the launch's time.  Part 0 also makes the chunk
    // offsets global and writes the segment's totals.
    const uint32_t pshift = finish_part_shift(a);
    const uint32_t t = blockIdx.x >> pshift;
    const uint32_t part = blockIdx.x & ((1u << pshift) - 1u);
    const uint64_t cmask = (1ull << a.log2_chunk) - 1;

    const uint32_t s = a.n_seg > 1 ? find_segment_block(a.tile_start, a.seg_at, t, tid, lane, s_cnt) : 0u;
    const SegDesc sd = segment_desc(a, s);
    const uint32_t first = segment_first_tile(a, s);
    const uint32_t end = segment_end_tile(a, s);
    const uint32_t count = a.tile_count[t];

    // The tile's escapes: from its slot, or, past the slot, from its range of the overflow
    // area; this part's share of them.  An overflow tile holds thousands: sixteen loads in
    // flight per thread, the first sixteen issued together with the loads of the earlier
    // tiles' counts below (their stores need the sum of those).  (The spill launch's
    // LDS-staged stores gained nothing here, and the larger code cost a cold call 0.8 us.)
    constexpr int kOvfBatch = 16;
    const uint32_t *src = a.slots + (uint64_t)t * a.slot_escapes;
    uint64_t have = count;
    if (count > a.slot_escapes) {
        const uint64_t off = a.tile_ovf[t];
        const uint64_t room = off < a.ovf_cap ? a.ovf_cap - off : 0;
        src = a.ovf + off;
        have = count < room ? count : room;
    }
    // (every load below is issued unconditionally, at an index clamped into its array, so
    // that the compiler does not wait for each one before the next)
    const SZ_GLOBAL uint32_t *gsrc = as_global(have ? src : a.slots);
    const uint32_t share = (uint32_t)((have + (1u << pshift) - 1u) >> pshift);
    const uint32_t r_begin = part * share;
    const uint32_t r_end = (uint64_t)r_begin + share < have ? r_begin + share : (uint32_t)have;
    const uint32_t r_last = r_end ? r_end - 1 : 0;

    // the escapes before this tile in its segment; a packed stream needs the segment's E
    // as well (its exponents follow the E positions).  One round of 16-byte loads covers the
    // counts of every tile of a finish call (at most kSmallTiles); a block of 4 counts past
    // the array's end stays inside the scratch (each array is padded to 256 bytes).  They go
    // out just before the escape loads, so that the sum waits only for them.
    static_assert(kSmallTiles == 16 * kThreads, "one round of four 16-byte count loads per thread");
    const uint32_t stop = a.packed ? end : t;
    const uint32_t blk0 = first >> 2, blk1 = (stop + 3) >> 2;
    const SZ_GLOBAL u32x4 *cnt4 = as_global(reinterpret_cast<const u32x4 *>(a.tile_count));
    u32x4 q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t b = blk0 + tid + k * kThreads;
        q[k] = cnt4[b < blk1 ? b : blk0];
    }
    uint32_t e[kOvfBatch];
#pragma unroll
    for (int k = 0; k < kOvfBatch; ++k) {
        const uint32_t r = r_begin + tid + k * kThreads;
        e[k] = gsrc[r < r_end ? r : r_last];
    }
    uint64_t before = 0, all = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t b = blk0 + tid + k * kThreads;
        const uint32_t c[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t u = 4 * b + i;
            const bool in = b < blk1 && u >= first;
            before += in && u < t ? c[i] : 0u;
            all += in && u < stop ? c[i] : 0u;
        }
    }
    const uint64_t prefix = block_total_u64(before, tid, lane, s_part);
    const uint64_t E = a.packed ? block_total_u64(all, tid, lane, s_part) : prefix + count;
    if (part == 0 && t + 1 == end && tid == 0) {
        sd.chunk_off[(sd.n + cmask) >> a.log2_chunk] = E;
        a.seg_escapes[s] = E;
        if (a.packed)
            write_header(sd, a, E);
    }
    if (blockIdx.x == 0 && tid == 0)
        a.ovf_ctr[0] = 0;    // the pack launch has finished with the overflow counter

    // tile-local chunk offsets become segment offsets, four loads in flight before the stores
    constexpr int kBatch = 4;
    const uint64_t base = (uint64_t)(t - first) << a.tile_shift;
    if (part == 0 && base < sd.n) {
        const uint64_t tile_words = 1ull << a.tile_shift;
        const uint64_t words = sd.n - base < tile_words ? sd.n - base : tile_words;
        const uint64_t c0 = (base + cmask) >> a.log2_chunk;
        const uint32_t nc = (uint32_t)(((base + words + cmask) >> a.log2_chunk) - c0);
        SZ_GLOBAL uint64_t *co = as_global(sd.chunk_off + c0);
        for (uint32_t i0 = tid; i0 < nc; i0 += kBatch * kThreads) {
            uint64_t v[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                if (i0 + k * kThreads < nc)
                    v[k] = co[i0 + k * kThreads];
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                if (i0 + k * kThreads < nc)
                    co[i0 + k * kThreads] = v[k] + prefix;
        }
    }

    // the escapes' final places: at most the escape capacity left is written
    uint8_t *exps = a.packed ? packed_exps(sd, E) : sd.esc_exp;
    const uint64_t dlim = prefix < sd.esc ? sd.esc - prefix : 0;
    const uint64_t lim = exps ? (have < dlim ? have : dlim) : 0;
    const uint32_t w_end = r_end < lim ? r_end : (uint32_t)lim;   // stores: ranks below this
    SZ_GLOBAL uint16_t *pos = as_global(lim ? sd.esc_pos + prefix : sd.esc_pos);
    SZ_GLOBAL uint8_t *ex = as_global(lim ? exps + prefix : exps);
    for (uint32_t r0 = r_begin + tid; r0 < w_end; r0 += kOvfBatch * kThreads) {
        if (r0 != r_begin + tid) {
#pragma unroll
            for (int k = 0; k < kOvfBatch; ++k) {
                const uint32_t r = r0 + k * kThreads;
                e[k] = gsrc[r < r_end ? r : r_last];
            }
        }
#pragma unroll
        for (int k = 0; k < kOvfBatch; ++k) {
            const uint32_t r = r0 + k * kThreads;
            if (r < w_end) {
                pos[r] = (uint16_t)((base + (e[k] & 0xFFFFu)) & cmask);
                ex[r] = (uint8_t)(e[k] >> 16);
            }
        }
    }
}

// ---- set-up of an encode with a fixed scratch array ------------------------------------------

__global__ __launch_bounds__(64) void setup_kernel(const SetupArgs a)
{
    const uint32_t i = threadIdx.x;
    if (i < a.count) {
        a.d_segs[a.first + i] = a.segs[i];
        a.d_tiles[a.first + i] = a.tiles[i];
    }
    if (a.last && i == a.count)
        a.d_tiles[a.first + a.count] = a.tiles[a.count];
    if (a.ovf_ctr && i < 2)
        a.ovf_ctr[i] = 0;
}

// Entry g < n_groups: the segment holding tile g << kSegAtShift (the largest s with
// tile_start[s] <= that tile); entry n_groups: the last segment.
__global__ __launch_bounds__(kThreads) void seg_at_kernel(const uint32_t *tile_start, uint32_t n_seg,
                                                          uint32_t n_groups, uint32_t *seg_at)
{
    const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
    if (g > n_groups)
        return;
    if (g == n_groups) {
        seg_at[g] = n_seg - 1;
        return;
    }
    const uint32_t t = g << kSegAtShift;
    uint32_t lo = 0, hi = n_seg;
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (tile_start[mid] <= t)
            lo = mid;
        else
            hi = mid;
    }
    seg_at[g] = lo;
}

// Every status word of a one-pass state unwritten.
__global__ __launch_bounds__(kThreads) void chain_clear_kernel(uint64_t *status, uint64_t words)
{
    const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < words)
        status[i] = 0;
}

hipError_t launch_chain_clear(uint64_t *status, uint32_t cap, hipStream_t stream)
{
    const uint64_t words = (uint64_t)cap * kChainStride;
    chain_clear_kernel<<<(unsigned)(words / kThreads + 1), kThreads, 0, stream>>>(status, words);
    return hipGetLastError();
}

hipError_t launch_setup(const SetupArgs &a, hipStream_t stream)
{
    if (a.count > kSetupSegs)
        return hipErrorInvalidValue;
    setup_kernel<<<1, 64, 0, stream>>>(a);
    return hipGetLastError();
}

hipError_t launch_seg_at(const uint32_t *tile_start, uint32_t n_seg, uint32_t n_tiles, uint32_t *seg_at,
                         hipStream_t stream)
{
    const uint32_t n_groups = (n_tiles + (1u << kSegAtShift) - 1) >> kSegAtShift;
    seg_at_kernel<<<n_groups / kThreads + 1, kThreads, 0, stream>>>(tile_start, n_seg, n_groups, seg_at);
    return hipGetLastError();
}

hipError_t launch_encode_stage(int stage, const EncodeArgs &a, hipStream_t stream)
{
    switch (stage) {
    case kStagePack:
        if (a.chain_status)
            return hipErrorInvalidValue;
        if (a.elem == kElemE5M2)
            return launch_encode_pack_e5m2(a, stream);
        if (a.stage)
            encode_pack_kernel<true, false><<<a.n_tiles, kThreads,
                                              a.n_tiles >= kPackCapTiles ? kPackLdsReserve : 0u, stream>>>(a);
        else
            encode_pack_kernel<false, false><<<a.n_tiles, kThreads, 0, stream>>>(a);
        break;
    case kStageOnePass:
        // tiles in launch order: workgroup t codes tile t, so every tile it waits for was
        // started before it
        if (a.packed || !a.chain_status || a.chain_cap < a.n_tiles || a.chain_tag > kChainTagMask)
            return hipErrorInvalidValue;
        if (a.elem == kElemE5M2)
            return launch_encode_pack_e5m2(a, stream);
        // (the early-release stash already holds occupancy at 4 workgroups per CU)
        if (a.stage)
            encode_pack_kernel<true, true><<<a.n_tiles, kThreads, 0, stream>>>(a);
        else
            encode_pack_kernel<false, true><<<a.n_tiles, kThreads, 0, stream>>>(a);
        break;
    case kStageSums:
        encode_sums_kernel<<<(a.n_tiles + kSumTiles - 1) / kSumTiles, kThreads, 0, stream>>>(a);
        break;
    case kStagePlace:
        encode_place_kernel<<<(a.n_tiles + kPlaceTiles - 1) / kPlaceTiles, kThreads, 0, stream>>>(a);
        break;
    case kStageSpill:
        encode_spill_kernel<<<a.n_tiles < kSpillBlocks ? a.n_tiles : kSpillBlocks, kThreads, 0, stream>>>(a);
        break;
    case kStageFinish:
        if (a.n_tiles > kSmallTiles)
            return hipErrorInvalidValue;
        encode_finish_kernel<<<a.n_tiles << finish_part_shift(a), kThreads, 0, stream>>>(a);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ======================================================================================
// a5-a7  decode
// ======================================================================================

// Codebook lookup of 4 codes (one per byte, each 0..15): two byte-permutes over the
// low and high halves of the 16-byte codebook, merged on bit 3 of each code.
__device__ __forceinline__ uint32_t codebook_lookup(uint32_t x, const uint32_t cb[4])
{
    const uint32_t sel = x & 0x07070707u;
    const uint32_t lo = perm(cb[1], cb[0], sel);
    const uint32_t hi = perm(cb[3], cb[2], sel);
    const uint32_t b3 = (x >> 3) & 0x01010101u;
    const uint32_t m = (b3 << 8) - b3;   // 0xFF in every byte whose code has bit 3 set
    return (hi & m) | (lo & ~m);
}

// Two BF16 words from sign+mantissa bytes s (words 2m, 2m+1 at bytes 2m', 2m'+1 of s, per
// selector) and exponent bytes taken from even/odd.
__device__ __forceinline__ uint32_t assemble(uint32_t s, uint32_t sm_sel, uint32_t even,
                                             uint32_t odd, uint32_t ex_sel)
{
    const uint32_t p = perm(s, s, sm_sel);          // [s1 s1 s0 s0]
    const uint32_t q = perm(odd, even, ex_sel);     // [0 e1 0 e0]
    return (p & 0x807F807Fu) | (q << 7);
}

template <bool kLarge>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeArgs a)
{
    __shared__ uint32_t s_exp[kDecTileWords / 4];              // exponent bytes of the tile
    __shared__ uint64_t s_off[kDecTileWords / 16 + 1];         // chunk offsets of the tile

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
    const uint64_t base = (uint64_t)(t - first) << kDecTileShift;
    if (base >= n)
        return;                                              // empty segment
    const uint64_t valid = n - base < (uint64_t)kDecTileWords ? n - base : (uint64_t)kDecTileWords;
    const uint32_t log2c = a.log2_chunk;
    const uint64_t C = 1ull << log2c;
    const uint64_t E = sd.esc;
    uint32_t cb[4] = {a.cb[0], a.cb[1], a.cb[2], a.cb[3]};
    if (a.multi_book) {
        // the segment's own codebook (uniform and read-only: scalar loads)
        const uint32_t *c = a.cbs + 4u * sd.book;
        cb[0] = load_const_u32(c, 0);
        cb[1] = load_const_u32(c, 1);
        cb[2] = load_const_u32(c, 2);
        cb[3] = load_const_u32(c, 3);
    }

    // ---- loads ---------------------------------------------------------------------------
    // a packed stream's header, through scalar loads (read-only here), so that the data loads
    // below do not queue behind it
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
    uint2 smv[kDecGroups];
    uint32_t cw[kDecGroups];
#pragma unroll
    for (int j = 0; j < kDecGroups; ++j) {
        const uint64_t g0 = base + (uint64_t)(((wave * kDecGroups + j) << 6) + lane) * kGroupWords;
        if (g0 + kGroupWords <= n) {
            const u32x2 s2 = __builtin_nontemporal_load(as_global(reinterpret_cast<const u32x2 *>(sd.sm + g0)));
            smv[j] = make_uint2(s2.x, s2.y);
            cw[j] = __builtin_nontemporal_load(as_global(reinterpret_cast<const uint32_t *>(sd.codes + (g0 >> 1))));
        } else {
            uint32_t b[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            uint32_t c = 0;
            for (uint32_t k = 0; k < 8; ++k)
                if (g0 + k < n)
                    b[k] = sd.sm[g0 + k];
            for (uint32_t k = 0; k < 4; ++k)
                if (g0 + 2 * k < n)
                    c |= (uint32_t)sd.codes[(g0 >> 1) + k] << (8 * k);
            smv[j] = make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                                b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
            cw[j] = c;
        }
    }

    // ---- escape range of the tile --------------------------------------------------------
    const bool sub_chunk = log2c > (uint32_t)kDecTileShift;     // the tile lies inside one chunk
    const uint64_t c0 = base >> log2c;
    const uint64_t nc = sub_chunk ? 1 : (valid + C - 1) >> log2c;   // chunks of this tile
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
        // packed stream: it must describe exactly the segment the caller gave, and it carries
        // its own codebook.  Loaded with the data, checked here (the loads above all stay
        // inside the buffer, whose length the host checked); nothing is written before it.
        const uint64_t hn = h1.x | ((uint64_t)h1.y << 32), hc = h1.z | ((uint64_t)h1.w << 32);
        const uint64_t he = h2.x | ((uint64_t)h2.y << 32);
        const bool ok = h0.x == 0x31425A53u && h0.y == (1u | (64u << 16)) && h0.z == (uint32_t)C &&
                        h0.w == 0u && hn == n && hc == ((n + C - 1) >> log2c) && he == E &&
                        h3.z == 0u && h3.w == 0u;
        if (!ok) {
            if (tid == 0 && a.err)
                atomicOr(a.err, kErrBadHeader);
            return;
        }
        cb[0] = h2.z;
        cb[1] = h2.w;
        cb[2] = h3.x;
        cb[3] = h3.y;
    }

    // ---- a5: dense path ------------------------------------------------------------------
    uint32_t ex_even[kDecGroups], ex_odd[kDecGroups];
#pragma unroll
    for (int j = 0; j < kDecGroups; ++j) {
        ex_even[j] = codebook_lookup(cw[j] & 0x0F0F0F0Fu, cb);
        ex_odd[j] = codebook_lookup((cw[j] >> 4) & 0x0F0F0F0Fu, cb);
    }

    // ---- a6: sparse escape correction (exponent bytes in LDS) ----------------------------
    // A tile with escapes keeps its exponent bytes in LDS in word order (byte p: word p): each
    // group's two dwords in code order (even words, odd words) become two dwords in word
    // order by two byte permutes, so that an escape's byte is at its word's index.
    uint32_t asel[4] = {0x0C040C00u, 0x0C050C01u, 0x0C060C02u, 0x0C070C03u};   // code order
    if (patch) {
#pragma unroll
        for (int j = 0; j < kDecGroups; ++j) {
            const uint32_t q = ((wave * kDecGroups + j) << 6) + lane;
            s_exp[2 * q] = perm(ex_odd[j], ex_even[j], 0x05010400u);
            s_exp[2 * q + 1] = perm(ex_odd[j], ex_even[j], 0x07030602u);
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
            // escape jj belongs to the last chunk ci whose offset s_off[ci] <= jj
            for (uint64_t ci = tid; ci < nc; ci += kThreads) {
                const uint64_t cs = (c0 + ci) << log2c;
                if (s_off[ci] > s_off[ci + 1] || s_off[ci + 1] - s_off[ci] > (n - cs < C ? n - cs : C))
                    bad |= kErrBadOffsets;
            }
            if (j1 - j0 > (uint64_t)kThreads) {
                // more escapes than threads: each chunk's escapes [s_off[c], s_off[c + 1]) are
                // patched by `per` threads (the 256 threads split evenly over the tile's chunks,
                // a power of two each; at least one chunk per thread), so an escape's chunk is
                // known without a search; a chunk whose offsets are out of order, too long or
                // outside the tile's range (flagged above) is skipped
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
                            if (pos[k] < clen)
                                bytes[cs + pos[k]] = (uint8_t)ev[k];
                            else
                                bad |= kErrBadPosition;
                        }
                    }
                }
            } else {
                // chunk of escape jj: the last c with s_off[c] <= jj.  In the large-call build a
                // tile of at most kFew chunks (chunk size 1024 or more) counts the tile-relative
                // chunk starts at or below each escape's rank: the starts of chunks 1..kFew, two
                // per dword (absent ones 0x7FFF), are subtracted from the rank with packed 16-bit
                // subtractions (ranks and starts are below 2^13, so a half's sign bit says rank <
                // start), and the sign bits are counted.  Otherwise a binary search in LDS
                // (three or more dependent LDS reads per escape).
                constexpr int kFew = 8;
                const bool few = kLarge && nc <= (uint64_t)kFew;       // uniform
                static_assert(kDecTileWords < (1 << 15), "tile ranks fit a signed 16-bit half");
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
                        if (pos[k] < clen)
                            bytes[cs + pos[k]] = (uint8_t)ev[k];
                        else
                            bad |= kErrBadPosition;
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
                    if (pos[k] >= clen)
                        bad |= kErrBadPosition;
                    else if (pos[k] >= lo && pos[k] < lo + valid)
                        bytes[pos[k] - lo] = (uint8_t)ev[k];
                }
            }
        }
        if (bad && a.err)
            atomicOr(a.err, bad);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kDecGroups; ++j) {
            const uint32_t q = ((wave * kDecGroups + j) << 6) + lane;
            ex_even[j] = s_exp[2 * q];              // words 8 q .. 8 q + 3
            ex_odd[j] = s_exp[2 * q + 1];           // words 8 q + 4 .. 8 q + 7
        }
        asel[0] = 0x0C010C00u;
        asel[1] = 0x0C030C02u;
        asel[2] = 0x0C050C04u;
        asel[3] = 0x0C070C06u;
    }

    // ---- assemble and store ------------------------------------------------------------------
#pragma unroll
    for (int j = 0; j < kDecGroups; ++j) {
        const uint64_t g0 = base + (uint64_t)(((wave * kDecGroups + j) << 6) + lane) * kGroupWords;
        uint4 o;
        o.x = assemble(smv[j].x, 0x01010000u, ex_even[j], ex_odd[j], asel[0]);
        o.y = assemble(smv[j].x, 0x03030202u, ex_even[j], ex_odd[j], asel[1]);
        o.z = assemble(smv[j].y, 0x01010000u, ex_even[j], ex_odd[j], asel[2]);
        o.w = assemble(smv[j].y, 0x03030202u, ex_even[j], ex_odd[j], asel[3]);
        if (g0 + kGroupWords <= n) {
            store_stream16(sd.data + g0, o.x, o.y, o.z, o.w);
        } else {
            const uint32_t w[4] = {o.x, o.y, o.z, o.w};
            for (uint32_t k = 0; g0 + k < n; ++k)
                sd.data[g0 + k] = (uint16_t)(w[k >> 1] >> (16 * (k & 1)));
        }
    }
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream)
{
    if (a.elem == kElemE5M2)
        return launch_decode_e5m2(a, stream);
    // The dynamic LDS reservation is unused: on large calls it caps decode at 5 workgroups per
    // CU (see kDecodeLdsReserve).
    const unsigned lds = a.n_tiles >= kDecodeCapTiles ? kDecodeLdsReserve : 0u;
    if (a.large)
        decode_kernel<true><<<xcd_grid(a.n_tiles), kThreads, lds, stream>>>(a);
    else
        decode_kernel<false><<<xcd_grid(a.n_tiles), kThreads, lds, stream>>>(a);
    return hipGetLastError();
}

}  // namespace sz
