/*
 * splitzip_oracle.h -- plain CPU oracle of the SplitZip BF16 exponent-split codec.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, single-threaded, obviously
 * correct definition that the GPU library is checked against.  Only the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark may build,
 * load or call it.  It shares no code, header, table or constant with the GPU
 * library, and the GPU library never calls it.
 *
 * What is computed (SplitZip README, "Abstract" and "Highlights"; SplitZip
 * arXiv abstract): every BF16 word is split into its exact sign+mantissa bits
 * and its 8-bit exponent.  The exponent is replaced by a fixed 4-bit code that
 * indexes a top-16 exponent codebook calibrated offline; exponents outside the
 * codebook go to a sparse, chunk-local escape stream of (position, exponent).
 * Decoding rebuilds every word bit for bit.
 *
 * The byte format below is this project's reading of those pages (they print
 * no stream layout):
 *   - sm[i]     = (sign << 7) | mantissa                       (u8, one per element)
 *   - codes[j]  = code(2j) | code(2j+1) << 4                   (u8, two per byte)
 *   - chunk_off = exclusive escape count at each chunk start,
 *                 n_chunks + 1 entries, last one = E            (u64)
 *   - esc_pos   = position of each escape inside its chunk     (u16)
 *   - esc_exp   = raw 8-bit exponent of each escape            (u8)
 * Escaped elements carry code 0 in the nibble stream.  Escapes are listed in
 * ascending element order.
 *
 * Canonical serialized stream (little-endian, no padding):
 *   0  "SZB1"            4 B     32 n_escapes     u64
 *   4  version = 1       u16     40 codebook      16 B
 *   6  header_bytes = 64 u16     56 reserved = 0  8 B
 *   8  chunk_size        u32     64 sm[n], codes[ceil(n/2)], chunk_off[n_chunks+1] (u64),
 *  12  flags = 0         u32        esc_pos[E] (u16), esc_exp[E] (u8)
 *  16  n                 u64
 *  24  n_chunks          u64
 * total = 64 + n + ceil(n/2) + 8 (n_chunks + 1) + 3 E bytes.
 */
#ifndef SPLITZIP_ORACLE_H
#define SPLITZIP_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes of the oracle (its own numbering). */
#define SZO_OK 0
#define SZO_BAD_ARGUMENT 1
#define SZO_BAD_STREAM 2
#define SZO_NO_ROOM 3
#define SZO_WRONG_CODEBOOK 4

/* hist[e] = number of i < m whose exponent field equals e. */
void szo_histogram(const uint16_t *x, uint64_t m, uint64_t hist[256]);

/* The 16 exponents ranked first by (count descending, exponent ascending). */
void szo_codebook(const uint64_t hist[256], uint8_t cb[16]);

/* Fraction of the m counted exponents that the codebook holds (0 if m == 0). */
double szo_coverage(const uint64_t hist[256], const uint8_t cb[16], uint64_t m);

/* Shannon entropy, in bits, of the exponent distribution hist (0 for an empty one). */
double szo_entropy(const uint64_t hist[256]);

/* Number of bytes of the canonical stream. */
uint64_t szo_compressed_bytes(uint64_t n, uint32_t chunk_size, uint64_t n_escapes);

/*
 * Encode x[0..n).  Output arrays are caller-owned: sm[n], codes[ceil(n/2)],
 * chunk_off[ceil(n/C)+1], esc_pos[esc_capacity], esc_exp[esc_capacity].
 * *n_escapes receives E even when E > esc_capacity (then SZO_NO_ROOM is
 * returned and only the first esc_capacity escapes are stored).
 */
int szo_encode(const uint16_t *x, uint64_t n, const uint8_t cb[16], uint32_t chunk_size,
               uint8_t *sm, uint8_t *codes, uint64_t *chunk_off, uint16_t *esc_pos,
               uint8_t *esc_exp, uint64_t esc_capacity, uint64_t *n_escapes);

/* Decode the sections back into y[0..n).  Checks the escape metadata first. */
int szo_decode(const uint8_t *sm, const uint8_t *codes, const uint64_t *chunk_off,
               const uint16_t *esc_pos, const uint8_t *esc_exp, uint64_t n, uint64_t n_escapes,
               const uint8_t cb[16], uint32_t chunk_size, uint16_t *y);

/* Write the canonical stream into out[out_len]; out_len must equal szo_compressed_bytes. */
/* The 64-byte header of a canonical stream (flags 0: BF16 words, 1: E5M2 bytes). */
void szo_header(uint64_t n, uint32_t chunk_size, uint64_t n_escapes, const uint8_t cb[16],
                uint32_t flags, uint8_t out[64]);
int szo_serialize(const uint8_t *sm, const uint8_t *codes, const uint64_t *chunk_off,
                  const uint16_t *esc_pos, const uint8_t *esc_exp, uint64_t n, uint64_t n_escapes,
                  const uint8_t cb[16], uint32_t chunk_size, uint8_t *out, uint64_t out_len);

/* Read n, chunk_size, E and the codebook from a canonical stream header. */
int szo_stream_info(const uint8_t *buf, uint64_t len, uint64_t *n, uint32_t *chunk_size,
                    uint64_t *n_escapes, uint8_t cb[16]);

/*
 * Decode a canonical stream into y[n].  The stream must have been written with
 * the codec's codebook cb (a stateful codec decodes only its own streams).
 */
int szo_decode_stream(const uint8_t *buf, uint64_t len, const uint8_t cb[16], uint16_t *y,
                      uint64_t y_len);

/* ---- FP8 E5M2 elements (sign bit 7, exponent bits 6..2, mantissa bits 1..0) ----------
 * Same method and stream as above with: a 3-bit field (sign << 2) | mantissa per element
 * packed into a little-endian bit stream sm3[ceil(3n/8)] (element i at bits 3i..3i+2); a
 * codebook of 16 of the 32 exponent values; escape exponents 0..31; header flags = 1.
 * total = 64 + ceil(3n/8) + ceil(n/2) + 8 (n_chunks + 1) + 3 E bytes. */
void szo8_histogram(const uint8_t *x, uint64_t m, uint64_t hist[32]);
void szo8_codebook(const uint64_t hist[32], uint8_t cb[16]);
double szo8_coverage(const uint64_t hist[32], const uint8_t cb[16], uint64_t m);
uint64_t szo8_compressed_bytes(uint64_t n, uint32_t chunk_size, uint64_t n_escapes);
int szo8_encode(const uint8_t *x, uint64_t n, const uint8_t cb[16], uint32_t chunk_size,
                uint8_t *sm3, uint8_t *codes, uint64_t *chunk_off, uint16_t *esc_pos,
                uint8_t *esc_exp, uint64_t esc_capacity, uint64_t *n_escapes);
int szo8_decode(const uint8_t *sm3, const uint8_t *codes, const uint64_t *chunk_off,
                const uint16_t *esc_pos, const uint8_t *esc_exp, uint64_t n, uint64_t n_escapes,
                const uint8_t cb[16], uint32_t chunk_size, uint8_t *y);
int szo8_serialize(const uint8_t *sm3, const uint8_t *codes, const uint64_t *chunk_off,
                   const uint16_t *esc_pos, const uint8_t *esc_exp, uint64_t n, uint64_t n_escapes,
                   const uint8_t cb[16], uint32_t chunk_size, uint8_t *out, uint64_t out_len);
int szo8_decode_stream(const uint8_t *buf, uint64_t len, const uint8_t cb[16], uint8_t *y,
                       uint64_t y_len);

#ifdef __cplusplus
}
#endif

#endif /* SPLITZIP_ORACLE_H */
