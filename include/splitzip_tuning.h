/*
 * splitzip_tuning.h -- launch tuning and per-kernel timing of the SplitZip codec library
 * (libsplitzip.so).  No page fixes any of these: they choose between kernel builds and
 * launch sequences that write identical bytes, or time the kernels.  Tests and benchmarks
 * use them; a codec works with their defaults without ever calling them.  Conventions
 * (handles, streams, status codes) as in splitzip.h.
 */
#ifndef SPLITZIP_TUNING_H
#define SPLITZIP_TUNING_H

#include "splitzip.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ---- launch sequence of an encode ---- */

/* Default and largest value of splitzip_set_small_tiles. */
#define SPLITZIP_SMALL_TILES 4096

/*
 * How the encode of README "Codec API" is launched; no page fixes it, and the bytes
 * written are the same either way.
 * An encode call (any of the encode entry points) splits its segments into tiles of
 * 16384 BF16 words or 32768 E5M2 bytes, at least one per segment.  A call of at most
 * max_tiles tiles runs two kernel launches (pack, then finish: each tile's escape offset,
 * escape placement, chunk offsets), a larger call four (pack, sums, place, spill); on
 * inputs of a few MiB the launches, not the bytes, set the time.  Both sequences write
 * identical bytes.  max_tiles <= SPLITZIP_SMALL_TILES (default), 0 = always four launches;
 * larger values give SPLITZIP_E_INVALID.  Applies to calls that start after it returns.
 */
int splitzip_set_small_tiles(splitzip_codec *codec, uint32_t max_tiles);

/* Default of splitzip_set_onepass_tiles. */
#define SPLITZIP_ONEPASS_TILES 2048u

/*
 * Whether an encode runs as one launch; no page fixes it, and the bytes written are the same
 * either way.  An encode call into separate section buffers (not a packed stream) of at most
 * max_tiles tiles (tiles as for splitzip_set_small_tiles) runs one pack launch that also
 * places every escape: each tile reads how many escapes its segment's earlier tiles hold from
 * their status words (a decoupled look-back over tiles in launch order) and writes its
 * escapes, chunk offsets and, as a segment's last tile, E straight to their final places
 * (an E5M2 call of at most 512 tiles runs it on tiles of half the length, 16384 bytes: on a
 * grid that far from fills the GPU, more tiles of less work each end sooner; so does any
 * escape-heavy E5M2 call after one whose first tile had its escapes unevenly spread).
 * Other calls (larger ones, packed streams, and calls on a stream that is being captured
 * into a graph, since each launch's tag is a kernel argument that a replay would repeat) run
 * the launch sequences of splitzip_set_small_tiles, with one exception: when the previous
 * encode on the same stream had more escapes in its first tile than a tile's slot in the
 * launch sequences holds (128 BF16, 256 E5M2), a larger call runs in one launch too, since
 * the launch sequences would move each escape through scratch.  On inputs with few escapes
 * one launch is faster up to about 2048 tiles (no second launch); on larger calls, with many
 * tiles in flight, each tile's wait for the earlier ones costs more than the other launches
 * do.  The codec's workspace for the stream keeps 32 bytes per one-pass tile of state for it,
 * and a word of host memory mapped for the GPU that each encode's first tile writes its
 * escape count to.  0 = never (also for escape-heavy inputs), UINT32_MAX = always; any value
 * is accepted.  Applies to calls that start after it returns.
 */
int splitzip_set_onepass_tiles(splitzip_codec *codec, uint32_t max_tiles);

/*
 * Tests of the one-pass state: set the count of one-pass launches made with the codec's
 * workspace for `stream`, whose low 23 bits tag the next launch's status words (at a tag of
 * 0 the state is cleared before the launch).  SPLITZIP_E_INVALID when the codec has no
 * workspace with one-pass state for the stream.
 */
int splitzip_set_onepass_launches(splitzip_codec *codec, void *stream, uint64_t launches);

/* Default of splitzip_set_stage_tiles. */
#define SPLITZIP_STAGE_TILES 1024

/*
 * Which builds of the pack and decode kernels a call runs; no page fixes it, and the bytes
 * written are the same either way.  An encode call of more than min_tiles tiles (tiles as
 * for splitzip_set_small_tiles), and a decode call of more than 2 * min_tiles decode tiles
 * (8192 BF16 words or 16384 E5M2 bytes, at least one per segment: the same elements; an
 * E5M2 call with more than one escape per 32 bytes, or of at most 512 such tiles, decodes on
 * tiles of 8192 bytes, which count here), run
 * the builds tuned for escape-heavy inputs: in pack a wave gathers a group's escapes in LDS
 * and stores them as one contiguous run when there are more than 64 of them; in decode an
 * escape finds its chunk among offsets held in scalar registers when a tile spans at most 8
 * chunks (16 for E5M2) instead of by a binary search in LDS.  Smaller calls run the builds
 * without them, whose smaller code costs less when the call is short and its instructions
 * are not yet in the caches.  Any value is accepted: 0 = always the tuned builds,
 * UINT32_MAX = never.  Applies to calls that start after it returns.
 */
int splitzip_set_stage_tiles(splitzip_codec *codec, uint32_t min_tiles);

/* Default of splitzip_set_private_overflow: 256 MiB. */
#define SPLITZIP_PRIVATE_OVERFLOW_BYTES (256ull << 20)

/*
 * Where an encode call's escape-heavy tiles put the escapes that do not fit their slot; no
 * page fixes it, and the bytes written are the same either way.  When 4 bytes per element
 * of all the call's tiles (tiles as for splitzip_set_small_tiles) come to at most max_bytes,
 * every tile gets its own region of the library's scratch memory, so no tile waits on a
 * shared counter; otherwise tiles reserve ranges of one area, as large as the call's escape
 * capacity, with an atomic counter (thousands of escape-heavy tiles contend for it).  The
 * scratch memory stays allocated with the codec's workspace.  0 = always the shared area.
 * Applies to calls that start after it returns.
 */
int splitzip_set_private_overflow(splitzip_codec *codec, uint64_t max_bytes);

/* ---- per-kernel timing (for benchmarks and profilers: the codec throughput measurement
 *      of README "Quick Start") ---- */

/* Kernels whose durations splitzip_profile_read reports, in this order. */
#define SPLITZIP_KERNEL_PACK 0    /* encode: split, pack, in-tile escape compaction      */
#define SPLITZIP_KERNEL_SUMS 1    /* encode: segmented sums of per-tile escape counts    */
#define SPLITZIP_KERNEL_PLACE 2   /* encode: escape placement, global chunk offsets      */
#define SPLITZIP_KERNEL_SPILL 3   /* encode: placement of escape-heavy tiles' escapes    */
#define SPLITZIP_KERNEL_DECODE 4  /* decode                                               */
#define SPLITZIP_KERNEL_FINISH 5  /* encode, small calls: offsets and placement per tile  */
#define SPLITZIP_KERNEL_ONEPASS 6 /* encode in one launch: pack and placement together    */
#define SPLITZIP_KERNELS 7

/*
 * Timing of the codec's kernels, which README "Quick Start" measures as codec throughput.
 * enable != 0: every later encode/decode call on this codec records HIP events around
 * each of its kernel launches, on the call's stream.  enable == 0 stops recording and
 * discards accumulated timings.
 */
int splitzip_profile(splitzip_codec *codec, int enable);

/*
 * (README "Quick Start": codec throughput.)
 * Wait for `stream`, then report for each kernel kind the mean duration in ms and the
 * number of launches timed on that stream since profiling was enabled or last reset
 * (reset != 0 clears the totals after reading).  avg_ms and counts: host arrays of
 * SPLITZIP_KERNELS entries.
 */
int splitzip_profile_read(splitzip_codec *codec, void *stream, double *avg_ms, uint64_t *counts,
                          int reset);

/*
 * Device bytes of the workspace a codec keeps for `stream` (0 when it has none; see
 * splitzip_release_stream in splitzip.h), for tests and memory accounting.
 */
int splitzip_workspace_bytes(const splitzip_codec *codec, void *stream, uint64_t *bytes);

#ifdef __cplusplus
}
#endif

#endif /* SPLITZIP_TUNING_H */
