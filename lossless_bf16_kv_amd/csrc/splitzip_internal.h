// splitzip_internal.h -- types shared by the gfx950 kernels and the host runtime of the
// SplitZip BF16 exponent-split codec.  Not part of the public ABI (include/splitzip.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sz {

// ---- tiling -------------------------------------------------------------------------
// A workgroup is 4 wave64s.  Each lane owns kGroupsPerLane groups of 8 consecutive
// words (one 16-byte load each); wave w's groups cover 64 * 8 * kGroupsPerLane
// consecutive words, so a tile is 8192 words (16 KiB of BF16) handled by one workgroup.
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kGroupsPerLane = 4;
constexpr int kGroupWords = 8;
constexpr int kTileShift = 13;
constexpr int kTileWords = 1 << kTileShift;
static_assert(kThreads * kGroupsPerLane * kGroupWords == kTileWords, "tile geometry");

// Inverse-LUT entry of an exponent outside the codebook: nibble 0 plus an escape bit.
constexpr uint8_t kEscapeEntry = 0x10;

// ---- decoupled look-back tile status (one u64 per tile) ------------------------------
//   bits 63..40  epoch of the launch that wrote it (never 0)
//   bits 39..38  1 = tile aggregate only, 2 = inclusive prefix
//   bits 37..0   escape count
constexpr int kValueBits = 38;
constexpr uint64_t kValueMask = (1ull << kValueBits) - 1;
constexpr uint64_t kFlagAggregate = 1ull << kValueBits;
constexpr uint64_t kFlagPrefix = 2ull << kValueBits;
constexpr uint64_t kFlagMask = 3ull << kValueBits;
constexpr int kEpochShift = 40;
constexpr uint32_t kEpochMax = (1u << 24) - 1;
constexpr uint64_t kMaxSegmentWords = 1ull << kValueBits;
// Bounded waits: a look-back that sees no progress for this many polls gives up, flags
// an error and lets the grid drain instead of spinning forever.
constexpr uint32_t kSpinLimit = 1u << 20;

// error bits written by the kernels
constexpr uint32_t kErrLookbackTimeout = 1u;
constexpr uint32_t kErrBadOffsets = 2u;
constexpr uint32_t kErrBadPosition = 4u;
constexpr uint32_t kErrBadTicket = 8u;

struct SegDesc {
    uint16_t *data;         // encode: input words; decode: output words
    uint8_t *sm;            // [n]
    uint8_t *codes;         // [ceil(n/2)]
    uint64_t *chunk_off;    // [n_chunks + 1]
    uint16_t *esc_pos;      // encode: [esc] slots; decode: [esc] entries
    uint8_t *esc_exp;
    uint64_t n;
    uint64_t esc;           // encode: escape capacity; decode: E
};

struct EncodeArgs {
    SegDesc seg0;                 // the only segment when n_seg == 1
    const SegDesc *segs;          // device table when n_seg > 1
    const uint32_t *tile_start;   // device [n_seg + 1] first tile of each segment
    const uint8_t *lut;           // device [256] inverse LUT (code, or kEscapeEntry)
    uint64_t *status;             // [n_tiles] look-back words
    unsigned long long *ticket;   // dynamic tile counter (monotone across launches)
    uint64_t *seg_escapes;        // [n_seg] OUT: E per segment
    uint32_t *err;                // OUT: error bits
    uint64_t ticket_base;         // counter value when this launch starts
    uint64_t epoch_tag;           // epoch << kEpochShift
    uint32_t n_seg;
    uint32_t n_tiles;
    uint32_t log2_chunk;
    uint32_t pad;
};

struct DecodeArgs {
    SegDesc seg0;
    const SegDesc *segs;
    const uint32_t *tile_start;
    uint32_t *err;                // optional
    uint32_t cb[4];               // codebook bytes 0..15 as 4 little-endian words
    uint32_t n_seg;
    uint32_t n_tiles;
    uint32_t log2_chunk;
    uint32_t pad;
};

// Calibration histogram: per-workgroup partial counts, then one reduction.
constexpr int kCalibBlocksMax = 1024;

hipError_t launch_calibrate(const uint16_t *d_x, uint64_t n, uint32_t *d_partial,
                            uint32_t n_blocks, uint64_t *d_hist, hipStream_t stream);
uint32_t calibrate_blocks(uint64_t n);
hipError_t launch_encode(const EncodeArgs &a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

}  // namespace sz
