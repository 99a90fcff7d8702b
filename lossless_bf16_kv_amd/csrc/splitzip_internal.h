// splitzip_internal.h -- types shared by the gfx950 kernels and the host runtime of the
// SplitZip BF16 exponent-split codec.  Not part of the public ABI (include/splitzip.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sz {

// ---- tiling -------------------------------------------------------------------------
// A workgroup is 4 wave64s.  Each lane owns k*Groups groups of 8 consecutive words (one
// 16-byte load each); wave w's groups cover 64 * 8 * k*Groups consecutive words.  An encode
// tile is 16384 words (32 KiB of BF16), a decode tile 8192 words.
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kGroupWords = 8;
constexpr int kEncGroups = 8;
constexpr int kEncTileShift = 14;
constexpr int kEncTileWords = 1 << kEncTileShift;
constexpr int kDecGroups = 4;
constexpr int kDecTileShift = 13;
constexpr int kDecTileWords = 1 << kDecTileShift;
static_assert(kThreads * kEncGroups * kGroupWords == kEncTileWords, "encode tile geometry");
static_assert(kThreads * kDecGroups * kGroupWords == kDecTileWords, "decode tile geometry");
// Extra LDS reserved per decode workgroup of calls of at least kDecodeCapTiles tiles, to hold
// occupancy at 5 workgroups per CU: on inputs of GBs that streams faster than the 6 that
// registers allow (less contention for HBM); smaller calls run uncapped (an escape-heavy
// 64 M-word input decodes 3 % faster at 6 than at 5).
constexpr unsigned kDecodeLdsReserve = 16384;
constexpr uint32_t kDecodeCapTiles = 65536;
// The same for the pack kernels of calls of at least kPackCapTiles tiles: 4 BF16 workgroups
// per CU (registers allow 5) and 5 E5M2 workgroups (registers and LDS allow 6) stream 2 % and
// 2.5 % faster on inputs of GBs (fewer concurrent tiles, each a long run of reads and writes);
// on a grid of a few thousand tiles the cap costs more in its last, partly filled round.
constexpr unsigned kPackLdsReserve = 31744;
constexpr unsigned kE8PackLdsReserve = 8192;
constexpr uint32_t kPackCapTiles = 16384;

// ---- element types ----------------------------------------------------------------------
// BF16 words (sign bit 15, exponent bits 14..7, mantissa bits 6..0) or FP8 E5M2 bytes (sign
// bit 7, exponent bits 6..2, mantissa bits 1..0).  The value is the stream header's flags.
constexpr uint32_t kElemBF16 = 0;
constexpr uint32_t kElemE5M2 = 1;

// E5M2 tiling: each lane owns groups of 32 consecutive bytes (two 16-byte loads), whose
// 3-bit sign+mantissa fields fill 12 bytes and whose codes fill 16.  A pack tile is 32768
// elements (4 groups per lane), a decode tile 16384 (2 groups per lane).  A one-pass encode
// of at most kE8ShortChainTiles such pack tiles runs tiles of 16384 instead: on a grid far
// from filling the GPU, twice as many tiles of half the work each end sooner; on larger ones
// the longer chain of look-backs costs more.
constexpr int kE8GroupElems = 32;
constexpr int kE8EncGroups = 4;
constexpr int kE8EncTileShift = 15;
constexpr int kE8ChainGroups = 2;
constexpr int kE8ChainTileShift = 14;
constexpr uint32_t kE8ShortChainTiles = 512;
// Bit of the first-tile escape count (EncodeArgs::first_tile_escapes) set when that tile's
// escapes fall unevenly over its waves (the most over twice the fewest, plus 64): an input
// whose escapes cluster, for which the short one-pass tiles also pay at larger sizes.
constexpr uint32_t kHintUneven = 0x80000000u;
constexpr int kE8DecGroups = 2;
constexpr int kE8DecTileShift = 14;
// A decode call with more than one escape per kE8ShortDecodeDensity elements, or of at most
// kE8ShortDecodeTiles tiles, runs tiles of 8192 (1 group per lane): the escape patch, not the
// stream, sets the time of escape-heavy tiles, and half-length tiles halve the escapes each
// workgroup patches; on inputs with few escapes the longer tiles stream better.
constexpr int kE8DecShortGroups = 1;
constexpr int kE8DecShortTileShift = 13;
constexpr uint32_t kE8ShortDecodeDensity = 32;
constexpr uint32_t kE8ShortDecodeTiles = 512;
static_assert(kThreads * kE8EncGroups * kE8GroupElems == (1 << kE8EncTileShift), "E5M2 encode tile");
static_assert(kThreads * kE8ChainGroups * kE8GroupElems == (1 << kE8ChainTileShift), "E5M2 one-pass tile");
static_assert(kThreads * kE8DecGroups * kE8GroupElems == (1 << kE8DecTileShift), "E5M2 decode tile");
static_assert(kThreads * kE8DecShortGroups * kE8GroupElems == (1 << kE8DecShortTileShift), "E5M2 short decode tile");

// Inverse-LUT entry of an exponent outside the codebook: nibble 0 plus an escape bit.
constexpr uint8_t kEscapeEntry = 0x10;

// ---- encode scratch --------------------------------------------------------------------
// Each tile's escapes are first written compacted to a slot (or, if more, to an overflow
// area) as (position inside the tile | exponent << 16), then moved to their final place once
// the tile's escape offset is known.  A slot holds 1/128 of the tile's elements: enough for
// nearly every tile of KV-like inputs (about 0.3 % escapes, unevenly spread), so that few
// tiles go to the overflow area and its spill launch.
constexpr uint32_t kSlotEscapes = 128;                        // BF16 tiles
constexpr uint32_t kE8SlotEscapes = 256;                      // E5M2 tiles (twice as long)
constexpr uint32_t kSumTiles = 2048;          // tiles per segmented-sum block
constexpr uint32_t kPlaceTiles = 64;          // tiles per placement workgroup
constexpr uint32_t kSpillBlocks = 4096;       // workgroups moving the overflow tiles' escapes
constexpr uint32_t kFinishPartShift = 2;     // large-call finish: 4 workgroups per tile ...
constexpr uint32_t kFinishPartTiles = 2048;  // ... in calls of at most this many tiles
// a wave gathers one group's escapes in LDS before storing them when it has more than this
constexpr uint32_t kStageMin = 64;
// calls of more than this many pack tiles (decode: twice as many decode tiles, the same
// elements) run the kernel builds tuned for escape-heavy inputs: pack gathers escape-heavy
// groups in LDS, decode finds an escape's chunk among offsets held in scalar registers and
// loads 8 escapes per thread and round.  Smaller calls, whose time is mostly the launch and
// its first instruction fetches, run the smaller builds without them.
constexpr uint32_t kStageTiles = 1024;
// calls whose tiles' worst-case overflow regions (one entry per element, 4 bytes each) fit
// this many bytes give every tile its own region of the overflow area: no tile reserves space
// with the overflow counter, which thousands of escape-heavy tiles contend for
constexpr uint64_t kPrivateOvfBytes = 256ull << 20;
// Calls of at most this many tiles finish in one launch after pack (kStageFinish, one
// workgroup per tile) instead of sums, place and spill: each workgroup adds up the escape
// counts of its segment's earlier tiles itself (at most kSmallTiles - 1 loads, which the
// workgroups of a call make T^2 / 2 of, from L2: a few microseconds at 4096 tiles).
constexpr uint32_t kSmallTiles = 4096;
// ---- one-pass encode (chained tiles) ----------------------------------------------------
// In a one-pass encode the pack launch places every escape itself: tile t learns the escapes
// of its segment's earlier tiles from their status words (a decoupled look-back over tiles in
// launch order) and writes its escapes, chunk offsets and, as a segment's last tile, E to
// their final places, with no scratch and no later launch.  Tile t's status word:
//   bits 0..38  escape count: the tile's own (kChainAggregate) or the segment's escapes up to
//               and including the tile (kChainPrefix)
//   bits 39..40 kind: 0 = not written in this launch, kChainAggregate, kChainPrefix
//   bits 41..63 tag: the launch's number modulo 2^23 (a kernel argument, counted by the host
//               per state); a word with another tag is left from an earlier launch and reads
//               as not written.  When the count wraps the host clears the state first, so no
//               word can outlive 2^23 launches.
// (A device-side launch counter, advanced by each launch's last workgroup, was measured:
// the one atomic per workgroup on one address costs about 76 ns each, serialized, 20 ms
// for 262144 tiles.)
constexpr uint64_t kChainCountMask = (1ull << 39) - 1;
constexpr uint32_t kChainKindShift = 39;
constexpr uint32_t kChainTagShift = 41;
constexpr uint64_t kChainTagMask = (1ull << 23) - 1;
constexpr uint64_t kChainAggregate = 1;
constexpr uint64_t kChainPrefix = 2;
// a look-back poll that finds a predecessor not yet written sleeps and polls again, at most
// this many times per tile (far longer than any tile takes) before it gives up, flags
// kErrChainStall and goes on as if the rest had no escapes: a launch always ends
constexpr uint32_t kChainSpinMax = 1u << 22;
// rows of 64 status words the look-back reads per round
constexpr int kChainRows = 1;
// u64 words per tile in the one-pass state: each tile's status word sits alone in its 32 bytes.
// Packed 16 to a 128-byte line, the words that hundreds of waiting waves poll and that their
// tiles write queued on a few lines (4096 tiles at 30 % escapes: 86 against 80 us).
constexpr uint32_t kChainStride = 4;
// One-pass encode, early release: a tile keeps its escapes of rank below kStashEscapes (u16
// position, u8 exponent) and its chunk starts' escape ranks (u16, at most one per 16 words)
// in LDS; waves whose escapes all fit end and free their registers while wave 0 waits for
// the tile's escape offset and writes them; a wave with escapes past the stash waits too and
// then sends those through the stash again (stash_rest: a second round in tiles of at most
// twice the stash, a quarter of it per wave in longer ones).
constexpr uint32_t kStashEscapes = 8192;
constexpr uint32_t kStashChunks = kEncTileWords / 16;
// byte offset of the positions in the stash: the copy out reads 16 bytes before each array
constexpr uint32_t kStashPosAt = 16;
constexpr uint32_t kE8StashEscapes = 8192;            // a quarter of an E5M2 pack tile
static_assert(kChainCountMask >= (1ull << 38), "a segment's escape count fits the status word");

// overflow counter: escapes reserved so far (low 40 bits) and overflow tiles listed (high 24)
constexpr int kOvfTileShift = 40;
constexpr uint64_t kOvfOffsetMask = (1ull << kOvfTileShift) - 1;
constexpr uint64_t kMaxSegmentWords = 1ull << 38;
static_assert(kEncTileWords <= 65536 && (1 << kE8EncTileShift) <= 65536, "in-tile positions must fit 16 bits");
static_assert(kSlotEscapes * 128 == kEncTileWords && kE8SlotEscapes * 128 == (1 << kE8EncTileShift), "slots");
static_assert(kSumTiles % kThreads == 0 && kSumTiles % kPlaceTiles == 0, "sum blocks");
static_assert(kSumTiles / kPlaceTiles <= kThreads, "group sums of a block fit one pass");
static_assert(kPlaceTiles % (kSumTiles / kThreads) == 0 && kPlaceTiles <= kThreads, "groups");

// error bits written by the kernels
constexpr uint32_t kErrBadOffsets = 2u;      // decode: chunk offsets out of range
constexpr uint32_t kErrBadPosition = 4u;     // decode: escape position outside its chunk
constexpr uint32_t kErrOverflowArea = 8u;    // encode: overflow area too small
constexpr uint32_t kErrBadHeader = 16u;      // decode: packed stream header does not match
constexpr uint32_t kErrChainStall = 32u;     // one-pass encode: a look-back gave up waiting

struct SegDesc {
    uint16_t *data;         // encode: input words; decode: output words (E5M2: bytes)
    uint8_t *sm;            // [n] (E5M2: the 3-bit field stream, [ceil(3n/8)])
    uint8_t *codes;         // [ceil(n/2)]
    uint64_t *chunk_off;    // [n_chunks + 1]
    uint16_t *esc_pos;      // encode: [esc] slots; decode: [esc] entries
    uint8_t *esc_exp;
    uint64_t n;
    uint64_t esc;           // encode: escape capacity; decode: E
    uint32_t book;          // the segment's codebook (read only when multi_book is set)
    uint32_t pad;
    // packed layout: the canonical stream's 64-byte header, followed by sm, codes and
    // chunk_off (which the pointers above address) and then esc_pos[E], esc_exp[E]: the
    // exponents start right after the E positions, so esc_exp above is unused and a kernel
    // that writes or reads them needs E first.  NULL for separate section buffers.
    uint8_t *header;
};

// Several segments: seg_at[g] is the segment holding tile g << kSegAtShift, and the table
// ends with the last segment (ceil(n_tiles / 2^kSegAtShift) + 1 entries), so tile t's
// segment lies between seg_at[t >> kSegAtShift] and the entry after it.
constexpr int kSegAtShift = 6;

// What the spill launch needs of one tile, written by place (which has it at hand) so that a
// spill workgroup waits on one load before its data loads: the final places of the tile's
// first escape, the tile's first word in its segment, and its range of the overflow area
// (offset in the low 40 bits, entries to move in the high 24; 0 entries: nothing to move).
struct __align__(16) SpillRec {
    uint16_t *pos;
    uint8_t *exp;
    uint64_t base;
    uint64_t src;
};

struct EncodeArgs {
    SegDesc seg0;                 // the only segment when n_seg == 1
    const SegDesc *segs;          // device table when n_seg > 1
    const uint32_t *tile_start;   // device [n_seg + 1] first tile of each segment
    const uint32_t *seg_at;       // device, n_seg > 1: segment of every (1 << kSegAtShift)-th tile
    const uint8_t *lut;           // device inverse LUT (code, or kEscapeEntry): [256], or
                                  // [256 * books] indexed by SegDesc::book when multi_book.
                                  // BF16: by exponent.  E5M2: by element byte, with the
                                  // byte's 3-bit field in bits 5..7
    uint32_t *tile_count;         // [n_tiles] escapes per tile
    uint64_t *tile_ovf;           // [n_tiles] overflow offset of tiles past slot_escapes
    SpillRec *spill_rec;          // [n_tiles] written by place for the spill launch
    uint32_t *ovf_tiles;          // [n_tiles] list of the overflow tiles
    uint32_t *slots;              // [n_tiles * slot_escapes]
    uint32_t *ovf;                // [ovf_cap]
    unsigned long long *ovf_ctr;  // [2]: running overflow counter (0 between encodes), and
                                  // its final value saved by the sums launch
    uint64_t ovf_cap;
    uint64_t *block_sum;          // [ceil(n_tiles / kSumTiles)] segmented sums, bit 63 = head
    uint64_t *group_sum;          // [ceil(n_tiles / kPlaceTiles)] the same per placement group
    uint64_t *seg_escapes;        // [n_seg] OUT: E per segment
    uint64_t *seg_total;          // [n_seg] packed layout: E per segment, from the sums launch
    const uint32_t *cbs;          // device [4 * books] codebooks (packed layout: the header's)
    uint32_t *err;                // OUT: error bits
    uint32_t n_seg;
    uint32_t n_tiles;
    uint32_t log2_chunk;
    uint32_t multi_book;          // segments use different codebooks
    uint32_t packed;              // segments are packed streams (SegDesc::header)
    uint32_t elem;                // kElemBF16 or kElemE5M2
    uint32_t tile_shift;          // log2 of the elements per pack tile
    uint32_t slot_escapes;        // entries per tile slot
    uint32_t stage;               // pack: gather escape-heavy groups in LDS (the larger build)
    uint32_t private_ovf;         // each tile owns entries [t << tile_shift, +1 << tile_shift) of ovf
    // one-pass encode: status words of chain_cap tiles (chain_cap >= n_tiles), and the
    // launch's tag (see kChainTagShift)
    uint64_t *chain_status;
    uint32_t chain_cap;
    uint32_t chain_tag;
    // optional, host memory mapped for the device: the call's first tile stores its escape
    // count there (E5M2: scaled to a tile of the launch sequences, with kHintUneven); the host
    // picks the next call's launch sequence and one-pass tile length with it
    uint32_t *first_tile_escapes;
};

struct DecodeArgs {
    SegDesc seg0;
    const SegDesc *segs;
    const uint32_t *tile_start;
    const uint32_t *seg_at;       // as in EncodeArgs, for the decode tiles
    uint32_t *err;                // optional
    const uint32_t *cbs;          // device [4 * books] codebooks, read when multi_book
    uint32_t cb[4];               // codebook bytes 0..15 as 4 little-endian words
    uint32_t n_seg;
    uint32_t n_tiles;
    uint32_t log2_chunk;
    uint32_t multi_book;
    uint32_t elem;                // kElemBF16 or kElemE5M2
    uint32_t large;               // the build for large calls (chunk lookup in scalar registers)
    uint32_t tile_shift;          // log2 of the elements per decode tile
};

// Exponent histograms of one or more tensors: per-workgroup partial counts (each tensor
// gets up to kHistBlocksMax workgroups), then one reduction per (tensor, exponent).
constexpr int kHistBlocksMax = 1024;

struct HistSeg {
    const uint16_t *x;
    uint64_t n;
};

struct HistArgs {
    HistSeg seg0;                   // the only tensor when n_seg == 1
    const HistSeg *segs;            // device [n_seg] when n_seg > 1
    const uint32_t *block_start;    // device [n_seg + 1] first workgroup of each tensor
    uint32_t *partial;              // [n_blocks * 256]
    uint64_t *hist;                 // OUT [n_seg * 256]
    uint32_t n_seg;
    uint32_t n_blocks;
    uint32_t elem;                  // kElemBF16 (words) or kElemE5M2 (bytes)
    uint32_t pad;
};

// Set-up of an encode whose scratch is a fixed device array (no allocation anywhere): the
// segment descriptors and tile starts travel as kernel arguments, kSetupSegs per launch, and
// are written to the scratch; the first launch also clears the overflow counter.
constexpr uint32_t kSetupSegs = 24;

struct SetupArgs {
    SegDesc segs[kSetupSegs];
    uint32_t tiles[kSetupSegs + 1];   // tile starts of segs[], then the next segment's start
    SegDesc *d_segs;                  // device [n_seg] (NULL for a one-segment call)
    uint32_t *d_tiles;                // device [n_seg + 1] tile starts
    unsigned long long *ovf_ctr;      // [2] set to 0 when not NULL
    uint32_t first;                   // index of segs[0] in the call
    uint32_t count;                   // descriptors in this launch
    uint32_t last;                    // this launch also writes the final tile start
    uint32_t pad;
};

hipError_t launch_setup(const SetupArgs &a, hipStream_t stream);
// Clears cap one-pass status words, with a kernel.
hipError_t launch_chain_clear(uint64_t *status, uint32_t cap, hipStream_t stream);
// The coarse segment table (see kSegAtShift) of n_seg segments with these device tile starts.
hipError_t launch_seg_at(const uint32_t *tile_start, uint32_t n_seg, uint32_t n_tiles, uint32_t *seg_at,
                         hipStream_t stream);

uint32_t hist_blocks(uint64_t n);
hipError_t launch_histogram(const HistArgs &a, hipStream_t stream);
// Encode stages, launched in order on one stream: pack, sums, place, spill; or, for calls of
// at most kSmallTiles tiles, pack and finish.
// kStageOnePass: the one-pass pack, alone (not for packed streams).
enum EncodeStage { kStagePack = 0, kStageSums, kStagePlace, kStageSpill, kStageFinish, kStageOnePass };
hipError_t launch_encode_stage(int stage, const EncodeArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// E5M2 pack and decode (the other encode stages are shared with BF16).
hipError_t launch_encode_pack_e5m2(const EncodeArgs &a, hipStream_t stream);
hipError_t launch_decode_e5m2(const DecodeArgs &a, hipStream_t stream);

}  // namespace sz
