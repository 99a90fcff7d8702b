/*
 * splitzip.h -- C ABI of the SplitZip BF16 exponent-split codec for AMD MI355X (gfx950).
 *
 * The calls follow the stateful codec the SplitZip README describes ("SplitZip:
 * Ultra-Fast Lossless KV Compression for Disaggregated LLM Serving", sections
 * "Codec API" and "Highlights"): a codec is built for one chunk size, calibrated once
 * on a separate calibration tensor (which fixes its top-16 exponent codebook and
 * returns the coverage), then encodes BF16 tensors into a compressed form whose size
 * is reported, and decodes them back bit for bit.  Per the README "Abstract" and the
 * arXiv abstract, the compressed form of n BF16 words is
 *
 *   sm[n]         one byte per word: (sign << 7) | 7-bit mantissa, kept exactly
 *   codes[n/2]    one 4-bit code per word (word 2j in the low nibble of byte j) that
 *                 indexes the 16-entry exponent codebook; 0 for escaped words
 *   chunk_off[]   u64, n_chunks + 1 entries: escapes before each chunk start, then E
 *   esc_pos[E]    u16 position of each escaped word inside its chunk
 *   esc_exp[E]    u8 exponent of each escaped word (any exponent outside the codebook)
 *
 * with chunks of chunk_size words and escapes listed in ascending word order.  Its
 * canonical serialization is a 64-byte header followed by the five sections;
 * compressed_bytes = 64 + n + ceil(n/2) + 8 (n_chunks + 1) + 3 E.
 *
 * FP8 E5M2 elements (README "FAQ" and arXiv abstract: the codec also runs on top of an
 * FP8 E5M2 KV cache).  An E5M2 codec (splitzip_calibrate_e5m2 and the other *_e5m2
 * constructors) codes bytes with sign bit 7, exponent bits 6..2 and mantissa bits 1..0.
 * The same calls encode and decode them; a segment's `data` then points to n bytes and
 * `sm` to the 3-bit field stream
 *
 *   sm[ceil(3n/8)] field (sign << 2) | mantissa of element i at bits 3i..3i+2 of a
 *                  little-endian bit stream (byte j holds bits 8j..8j+7)
 *
 * while codes, chunk_off, esc_pos and esc_exp keep the layout above (exponents 0..31,
 * codebook entries 0..31).  The header's flags field is 1 and
 * compressed_bytes = 64 + ceil(3n/8) + ceil(n/2) + 8 (n_chunks + 1) + 3 E.
 *
 * Conventions for every call
 *   - Pointers named d_* and every pointer inside splitzip_segment are DEVICE
 *     pointers on the codec's GPU; everything else is host memory.
 *   - Device buffers are owned by the caller (they may be PyTorch tensors); the
 *     library never frees them.  The codec owns only its small tables and a
 *     per-stream workspace, released by splitzip_free.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream) of the device
 *     that was current when the codec was created; work is enqueued on it.
 *   - Every call returns a splitzip_status and never throws.  On error, a message
 *     is available from splitzip_last_error() (per host thread).
 *   - Alignment: data (BF16 or E5M2), sm and codes 16-byte aligned; chunk_off 8-byte;
 *     esc_pos 2-byte.  n per segment < 2^38.
 *   - A codec may be used from several host threads and streams; calls on one
 *     stream are ordered, calls on different streams use different workspaces.
 *
 * The calls that choose between kernel builds and launch sequences, and per-kernel timing,
 * are in splitzip_tuning.h: no page fixes them and the bytes written do not depend on them.
 */
#ifndef SPLITZIP_H
#define SPLITZIP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPLITZIP_ABI_VERSION 5
#define SPLITZIP_HEADER_BYTES 64
#define SPLITZIP_MIN_CHUNK 16
#define SPLITZIP_MAX_CHUNK 65536
#define SPLITZIP_MAX_BOOKS 4096   /* codebooks per codec */
#define SPLITZIP_ELEM_BF16 0      /* element types; the stream header's flags field */
#define SPLITZIP_ELEM_E5M2 1

typedef enum splitzip_status {
    SPLITZIP_OK = 0,
    SPLITZIP_E_INVALID = 1,  /* null or misaligned pointer, bad chunk size, bad size   */
    SPLITZIP_E_NOMEM = 2,    /* device or pinned host allocation failed                */
    SPLITZIP_E_DEVICE = 3,   /* HIP runtime or kernel error                            */
    SPLITZIP_E_CODEBOOK = 4, /* stream codebook differs from the codec's               */
    SPLITZIP_E_FORMAT = 5,   /* bad magic, version, sizes or escape metadata           */
    SPLITZIP_E_CAPACITY = 6  /* encode: more escapes than esc_capacity (see below)     */
} splitzip_status;

typedef struct splitzip_codec splitzip_codec;

/*
 * One tensor ("segment") of an encode or decode call.  A call may carry many
 * segments (a ragged batch, one kernel launch); each has its own chunking, which
 * restarts at the segment's first word, and its own output sections.
 *
 *   data             BF16 words (E5M2 codec: bytes), n of them.  encode reads, decode
 *                    writes.
 *   sm, codes,       compressed sections (sizes above; sm is the 3-bit field stream for
 *                    E5M2).  encode writes, decode reads.
 *   chunk_off
 *   esc_pos, esc_exp escape arrays with esc_capacity slots.
 *   esc_capacity     encode: slots available.  decode: ignored.
 *   n_escapes        encode: OUT, the segment's E (also when E > esc_capacity).
 *                    decode: IN, the E the sections were written with.
 *   compressed_bytes encode: OUT, canonical stream size.  decode: ignored.
 *   book             which of the codec's codebooks the segment is coded with (0 for a
 *                    codec with one codebook); decode must use the book it was encoded
 *                    with, which the stream header identifies by its codebook copy.
 *   reserved         set to 0.
 */
typedef struct splitzip_segment {
    uint16_t *data;
    uint64_t n;
    uint8_t *sm;
    uint8_t *codes;
    uint64_t *chunk_off;
    uint16_t *esc_pos;
    uint8_t *esc_exp;
    uint64_t esc_capacity;
    uint64_t n_escapes;
    uint64_t compressed_bytes;
    uint32_t book;
    uint32_t reserved;
} splitzip_segment;

/*
 * Calibrate a new codec on d_cal[0..n_cal) (README "Codec API": calibrate on a
 * separate calibration set; README "Highlights" and arXiv abstract: top-16 exponent
 * codebook fixed offline).  The codebook is the 16 exponents ranked first by
 * (count descending, exponent ascending); *out_coverage = fraction of the n_cal
 * exponents it holds (0 when n_cal = 0).  out_hist (optional, host uint64[256])
 * receives the exponent histogram.  Blocks until the histogram is on the host.
 * chunk_size: power of two in [16, 65536].  *out_codec is released by splitzip_free.
 */
int splitzip_calibrate(const uint16_t *d_cal, uint64_t n_cal, uint32_t chunk_size, void *stream,
                       splitzip_codec **out_codec, double *out_coverage, uint64_t *out_hist);

/*
 * Build a codec from a known codebook (16 distinct exponents), e.g. the one carried by
 * a received stream header (README "Roadmap": codebook metadata that travels with the
 * payload).  The codec is bound to the current HIP device.
 */
int splitzip_codec_from_codebook(const uint8_t codebook[16], uint32_t chunk_size,
                                 splitzip_codec **out_codec);

/*
 * A codec with several codebooks (README "Highlights": offline-calibrated top-16 exponent
 * codebooks), for example one per layer, or one for K and one for V: book b is calibrated
 * on d_cal[b][0..n_cal[b]) exactly as splitzip_calibrate does for one tensor, and every
 * segment of an encode or decode call names its book.  d_cal and n_cal are host arrays of
 * n_books (1..SPLITZIP_MAX_BOOKS) device pointers and sizes.  coverage (optional, host
 * double[n_books]) and hist (optional, host uint64[n_books * 256]) receive each book's
 * coverage and calibration histogram.  All histograms are taken in one pass (two
 * launches).  Blocks until they are on the host.
 */
int splitzip_calibrate_books(uint32_t n_books, const uint16_t *const *d_cal, const uint64_t *n_cal,
                             uint32_t chunk_size, void *stream, splitzip_codec **out_codec,
                             double *coverage, uint64_t *hist);

/* A codec from n_books known codebooks (host uint8[n_books * 16], book b at 16 b), each
 * 16 distinct exponents, bound to the current HIP device (README "Highlights": codebooks
 * calibrated offline; "Roadmap": codebook metadata that travels with the payload). */
int splitzip_codec_from_codebooks(uint32_t n_books, const uint8_t *codebooks, uint32_t chunk_size,
                                  splitzip_codec **out_codec);

/*
 * FP8 E5M2 codecs (README "FAQ" and arXiv abstract: the method applied on top of an FP8
 * E5M2 KV cache): as splitzip_calibrate, splitzip_calibrate_books and
 * splitzip_codec_from_codebooks, for tensors of E5M2 bytes.  The codebook is the 16 of the
 * 32 exponent values ranked first by (count descending, exponent ascending); hist
 * (optional) receives 32 bins per book.  Known codebooks must hold 16 distinct values
 * below 32.
 */
int splitzip_calibrate_e5m2(const uint8_t *d_cal, uint64_t n_cal, uint32_t chunk_size, void *stream,
                            splitzip_codec **out_codec, double *out_coverage, uint64_t *out_hist);
int splitzip_calibrate_books_e5m2(uint32_t n_books, const uint8_t *const *d_cal, const uint64_t *n_cal,
                                  uint32_t chunk_size, void *stream, splitzip_codec **out_codec,
                                  double *coverage, uint64_t *hist);
int splitzip_codec_from_codebooks_e5m2(uint32_t n_books, const uint8_t *codebooks, uint32_t chunk_size,
                                       splitzip_codec **out_codec);

/* The element type a codec codes: SPLITZIP_ELEM_BF16 or SPLITZIP_ELEM_E5M2 (README "FAQ":
 * BF16 and FP8 E5M2 KV caches). */
int splitzip_codec_element(const splitzip_codec *codec, uint32_t *elem);

/* Number of codebooks of a codec and (if codebooks != NULL) all of them, host
 * uint8[n_books * 16] (README "Codec API": the codec's calibrated state). */
int splitzip_codec_books(const splitzip_codec *codec, uint32_t *n_books, uint8_t *codebooks);

/* Read back a codec's codebook (book 0), chunk size and device (any output may be NULL;
 * README "Codec API": the codec's calibrated state). */
int splitzip_codec_info(const splitzip_codec *codec, uint8_t codebook[16], uint32_t *chunk_size,
                        int *device);

/*
 * Encode (README "Abstract" and "Highlights", arXiv abstract: each word's sign and mantissa
 * kept exactly, its exponent as a 4-bit code into the codebook, exponents outside it in a
 * chunk-local escape stream; README "Codec API": encode, then compressed_bytes).
 * Encode n_seg segments (host array `segs`) in one launch.  Blocks until each
 * segment's escape count is known, then fills n_escapes and compressed_bytes.
 * Returns SPLITZIP_E_CAPACITY if some segment has more escapes than esc_capacity:
 * its n_escapes then holds the count needed and the caller re-encodes with larger escape
 * arrays.  Such a segment's sm, codes and chunk_off are complete; of its escape arrays,
 * entries below esc_capacity are either the final escape or left unwritten (which ones
 * depends on the order in which tiles reserve scratch space).
 * Segments with n = 0 are allowed (chunk_off[0] = 0 is written).
 */
int splitzip_encode(splitzip_codec *codec, uint32_t n_seg, splitzip_segment *segs, void *stream);

/*
 * Non-blocking encode (the encode of README "Codec API", left on the stream so that a
 * transfer can follow it without a host round trip): the same launches as
 * splitzip_encode without the wait.  The
 * kernels write into d_result (device, caller-owned, 1 + n_seg uint64 words):
 * d_result[1 + s] = E of segment s, and error bits are OR-ed into d_result[0] (the
 * caller zeroes it; bit 3 alone means some segment exceeded its escape capacity).
 * segs[].n_escapes / compressed_bytes are not filled.  Once the stream has passed
 * this work, a segment with E > esc_capacity holds only part of its escapes and must be
 * re-encoded with larger escape arrays.  The input and output buffers must stay valid
 * until then.
 */
int splitzip_encode_async(splitzip_codec *codec, uint32_t n_seg, const splitzip_segment *segs,
                          void *stream, uint64_t *d_result);

/*
 * Allocation-free encode, for callers that cannot allocate device memory during the call:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same encode as splitzip_encode_async (same arguments, same d_result contract, the same
 * kernels and the same bytes written), except that its scratch is one fixed device array of
 * SPLITZIP_NOALLOC_SCRATCH_BYTES per GPU, held from the library's load until the process
 * ends, instead of the codec's per-stream workspace.  The call allocates nothing (no
 * hipMalloc, pinned staging or host heap) and only enqueues kernels on `stream`; segment
 * descriptors travel to the GPU as kernel arguments.  Per-kernel timing does not cover it.
 *
 * Limits.  At most SPLITZIP_NOALLOC_MAX_SEGMENTS segments.  The last 4 MiB of the array
 * hold the state of the one-pass encode (splitzip_tuning.h): a call that runs in one pass
 * (at most 131072 one-pass tiles, and the codec's one-pass limit) needs no other scratch.
 * Any other call's scratch must fit the rest of the array, 60 MiB:
 *   256 + [n_seg > 1] (80 n_seg + 4 (n_seg + 2 + ceil(tiles / 64)))
 *       + about 560 B per tile (BF16 tile = 16384 words; E5M2: 1072 B per 32768-byte tile)
 *       + 4 (1 + sum of esc_capacity)
 * (each part rounded up to 256 bytes); e.g. about 2.3 GB of BF16 input with an escape
 * capacity of 0.5 % of its words.  A call over a limit returns SPLITZIP_E_INVALID before
 * anything is enqueued, with the bytes it would need in the message.
 *
 * Every call on one GPU shares that GPU's array and leaves its contents behind; each call
 * clears what must start at zero.  Calls whose GPU work overlaps on one GPU (different
 * streams, or other host threads) race on the array and corrupt each other's output: order
 * them on one stream or with events.
 */
#define SPLITZIP_NOALLOC_SCRATCH_BYTES (64ull << 20)
#define SPLITZIP_NOALLOC_MAX_SEGMENTS 4096u
int splitzip_encode_noalloc(splitzip_codec *codec, uint32_t n_seg, const splitzip_segment *segs,
                            void *stream, uint64_t *d_result);

/*
 * Decode (README "Abstract": the dense path looks each code up in the codebook, the sparse
 * escape correction restores the other exponents; "Codec API": decode returns the tensor
 * bit for bit).  Decode n_seg segments (host array `segs`, n_escapes as written by encode) into
 * their `data` buffers, in one launch.  Asynchronous: only enqueues work on `stream`.
 * The kernel never reads or writes outside the given sections even when the escape
 * metadata is corrupt; it then ORs a nonzero flag into *d_error (optional device
 * uint32, caller-owned, caller zeroes it) and leaves the affected words unpatched.
 */
int splitzip_decode(splitzip_codec *codec, uint32_t n_seg, const splitzip_segment *segs,
                    void *stream, uint32_t *d_error);

/* ---- packed streams: one contiguous device buffer per tensor (README "Roadmap":
 *      codebook and payload metadata that travel with the payload across a transfer
 *      boundary) ---- */

/*
 * One tensor whose compressed form is the canonical stream itself, laid out in one device
 * buffer exactly as the serialization above: the 64-byte header, sm, codes, chunk_off,
 * esc_pos[E], esc_exp[E].  Encode writes all of it on the GPU (no host copy, no second
 * pass); decode reads it there.  The header carries the codebook, so a packed stream is
 * decoded with its own codebook by any codec of the same chunk size.
 *
 *   data          BF16 words (E5M2 codec: bytes), n of them (16-byte aligned).  encode
 *                 reads, decode writes.
 *   n             elements; a multiple of 16 for BF16, of 128 for E5M2 (then every
 *                 section of the stream is aligned for vector access; KV tensors with a
 *                 head dimension that is a multiple of 128 qualify).
 *   buf           device, 16-byte aligned: the stream.  Placed 64 bytes before a 256-byte
 *                 boundary, every section after the header starts on whole cache lines
 *                 (n a multiple of 256), which the kernels stream fastest.
 *   buf_bytes     encode: capacity of buf; splitzip_compressed_bytes(n, chunk_size, e)
 *                 (E5M2: splitzip_e5m2_compressed_bytes) bytes hold up to e escapes (the
 *                 capacity hint).  decode: the stream's length, which fixes E.
 *   stream_bytes  blocking encode: OUT, the stream's length (also when it exceeds
 *                 buf_bytes).  Otherwise ignored.
 *   n_escapes     blocking encode: OUT, E.  Otherwise ignored.
 *   book          encode: which codebook of the codec.  decode: ignored.
 *   reserved      set to 0.
 */
typedef struct splitzip_packed {
    uint16_t *data;
    uint64_t n;
    uint8_t *buf;
    uint64_t buf_bytes;
    uint64_t stream_bytes;
    uint64_t n_escapes;
    uint32_t book;
    uint32_t reserved;
} splitzip_packed;

/*
 * The encode of README "Codec API" into the portable form of README "Roadmap".
 * Encode n_seg tensors into packed streams in one launch sequence.  d_result == NULL:
 * blocking, fills stream_bytes and n_escapes, and returns SPLITZIP_E_CAPACITY if a stream
 * does not fit its buffer (its escapes are then not written; stream_bytes says how many
 * bytes it needs).  d_result != NULL: non-blocking, as splitzip_encode_async (E of segment
 * s in d_result[1 + s]; a stream with splitzip_compressed_bytes(n, chunk_size, E) >
 * buf_bytes holds no escapes and must be re-encoded into a larger buffer).
 */
int splitzip_encode_packed(splitzip_codec *codec, uint32_t n_seg, splitzip_packed *segs,
                           void *stream, uint64_t *d_result);

/*
 * The decode of README "Codec API" from the portable form of README "Roadmap", with the
 * codebook the stream carries.
 * Decode n_seg packed streams (buf, buf_bytes) into their data buffers, in one launch.
 * Asynchronous.  The host checks that buf_bytes fits a stream of n words (else
 * SPLITZIP_E_FORMAT); the kernel checks each header against n, the chunk size and the E
 * the length implies, and for a stream whose header does not match writes nothing and ORs
 * 16 into *d_error (optional).  Other metadata errors are flagged as by splitzip_decode.
 */
int splitzip_decode_packed(splitzip_codec *codec, uint32_t n_seg, const splitzip_packed *segs,
                           void *stream, uint32_t *d_error);

/* Release a codec, its tables and workspaces (NULL is a no-op; the end of the stateful
 * codec object of README "Codec API").  Work that uses the codec must have completed;
 * freeing its device memory synchronizes the device. */
void splitzip_free(splitzip_codec *codec);

/*
 * Release the workspace a codec keeps for one stream (no page defines it; the stateful
 * codec of README "Codec API" keeps scratch between calls).  A codec creates one workspace
 * per stream it is used on and keeps it, with its encode scratch (about 1/30 of the largest
 * input encoded on that stream, plus 4 bytes per entry of escape capacity or per element of
 * the tiles' own overflow regions), until this call or splitzip_free: a long-lived codec
 * used from short-lived streams calls this before destroying such a stream.  Waits for the
 * stream, then frees; a stream with no workspace is a no-op (SPLITZIP_OK).  The codec stays
 * usable on any stream; a later call on the same stream makes a new workspace.
 */
int splitzip_release_stream(splitzip_codec *codec, void *stream);

/* ---- exponent statistics (README "Repository Contents" and "Reproducing Paper Artifact
 *      Scripts": BF16 KV exponent entropy and top-16 coverage analysis) ---- */

/*
 * Exponent histograms (README "Reproducing Paper Artifact Scripts": the exponent analysis;
 * "Highlights": the histogram calibration takes offline) of n_seg BF16 tensors in one pass
 * (two launches):
 * hist[256 s + e] = number of words of tensor s whose exponent field (bits 14..7) is e.
 * d_x and n are host arrays of n_seg device pointers (16-byte aligned) and word counts
 * (n[s] = 0 allowed).  hist is host memory; the call blocks until it is filled.  Scratch
 * device memory is allocated for the call and released before it returns.
 */
int splitzip_histogram(uint32_t n_seg, const uint16_t *const *d_x, const uint64_t *n, void *stream,
                       uint64_t *hist);

/* The same for n_seg tensors of E5M2 bytes (README "FAQ": FP8 E5M2 KV caches):
 * hist[32 s + e] = number of bytes of tensor s whose exponent field (bits 6..2) is e. */
int splitzip_histogram_e5m2(uint32_t n_seg, const uint8_t *const *d_x, const uint64_t *n, void *stream,
                            uint64_t *hist);

/*
 * Statistics of one exponent histogram (host only, no device work): the Shannon entropy
 * in bits, -sum p log2 p over the exponent values that occur with p = count / total
 * (ZipServ guide, "Information-Theoretic Limits and Exponent Entropy Bounds"); the top-16
 * codebook a calibration on this histogram picks (count descending, exponent ascending);
 * its coverage; and the number of distinct exponent values.  Any output may be NULL.  An
 * empty histogram gives entropy 0 and coverage 0.  For an E5M2 histogram pass its 32 bins
 * followed by 224 zero bins: the ranking then stays inside the 32 exponent values.
 */
int splitzip_exponent_stats(const uint64_t hist[256], double *entropy_bits, double *coverage,
                            uint8_t codebook[16], uint32_t *distinct);

/* ---- host helpers (no device work) ---- */

/* ceil(n / chunk_size), the chunk count of README "Highlights" (chunk-local escape
 * metadata); 0 for an invalid chunk size. */
uint64_t splitzip_chunk_count(uint64_t n, uint32_t chunk_size);

/* The compressed_bytes of README "Codec API": 64 + n + ceil(n/2) + 8 (n_chunks + 1) +
 * 3 n_escapes; 0 for an invalid chunk size or for n or n_escapes not below 2^38 (the
 * largest segment). */
uint64_t splitzip_compressed_bytes(uint64_t n, uint32_t chunk_size, uint64_t n_escapes);

/* E5M2 streams (README "FAQ"): 64 + ceil(3n/8) + ceil(n/2) + 8 (n_chunks + 1) +
 * 3 n_escapes; 0 as above. */
uint64_t splitzip_e5m2_compressed_bytes(uint64_t n, uint32_t chunk_size, uint64_t n_escapes);

/*
 * The header that carries the codebook and payload metadata with a stream (README
 * "Roadmap": portable transfer boundaries); its layout is this library's reading.
 * The canonical 64-byte stream header (little-endian): "SZB1", version u16 = 1,
 * header bytes u16 = 64, chunk_size u32, flags u32 = the codec's element type (0 BF16,
 * 1 E5M2), n u64, n_chunks u64, n_escapes u64, codebook[16] (that of `book`), 8 zero
 * bytes.  SPLITZIP_E_INVALID for n not below 2^38 or n_escapes above n.
 */
int splitzip_write_header(const splitzip_codec *codec, uint32_t book, uint64_t n,
                          uint64_t n_escapes, uint8_t out[SPLITZIP_HEADER_BYTES]);

/*
 * (README "Roadmap": the receiving side of a portable transfer boundary.)
 * Parse a header; total_len is the full stream length (checked against the sizes of the
 * element type the flags name).  *elem receives that type.  Returns SPLITZIP_E_FORMAT for a
 * malformed header (including n not below 2^38, E above n and E5M2 codebook entries above
 * 31).
 */
int splitzip_read_header(const uint8_t *buf, uint64_t total_len, uint64_t *n,
                         uint32_t *chunk_size, uint64_t *n_escapes, uint8_t codebook[16],
                         uint32_t *elem);

/*
 * Check that a received stream (header + total length) can be decoded by this codec:
 * SPLITZIP_E_FORMAT if the header is malformed, SPLITZIP_E_CODEBOOK if its chunk size or
 * element type differs from the codec's or its codebook is none of the codec's (README "Codec API":
 * encoded objects are decoded with the same calibrated state).  On success *book
 * (optional) receives the first book whose codebook the header carries.
 */
int splitzip_check_header(const splitzip_codec *codec, const uint8_t *buf, uint64_t total_len,
                          uint32_t *book);

/* Error reporting of this ABI (no page defines it): a fixed description of a status. */
const char *splitzip_status_string(int status);

/* Error reporting of this ABI (no page defines it): the message of the last failing call
 * on this host thread ("" if none), valid until that thread's next call. */
const char *splitzip_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPLITZIP_H */
