/*
 * splitzip_oracle.c -- plain CPU oracle of the SplitZip BF16 exponent-split codec.
 *
 * TEST INFRASTRUCTURE ONLY (see splitzip_oracle.h).  Single-threaded, scalar,
 * no blocking, fusion or reordering: each function follows the steps of the
 * method in the order the pages give them, so that it can be checked by eye.
 *
 * Sources (cited by page title and section):
 *   [README]   "SplitZip: Ultra-Fast Lossless KV Compression for Disaggregated
 *              LLM Serving" (GitHub README): Abstract, Highlights, Codec API, FAQ,
 *              Roadmap.
 *   [ABSTRACT] "SplitZip: Ultra Fast Lossless KV Compression for Disaggregated
 *              LLM Serving" (arXiv abstract page): Abstract (arXiv).
 *   [ZIPSERV]  "ZipServ Guide: Lossless BF16 Compression for Fast LLMs":
 *              "Problem" (BF16 = 1 sign, 8 exponent, 7 mantissa bits) and
 *              "Implementation", Step 1 (field extraction by shift and mask;
 *              one byte holding the sign above the 7 mantissa bits).
 */
#include "splitzip_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- BF16 fields: sign bit 15, exponent bits 14..7, mantissa bits 6..0 [ZIPSERV, Problem] ---- */

static unsigned bf16_sign(uint16_t u) { return (u >> 15) & 0x1u; }
static unsigned bf16_exponent(uint16_t u) { return (u >> 7) & 0xFFu; }
static unsigned bf16_mantissa(uint16_t u) { return u & 0x7Fu; }

static uint16_t bf16_join(unsigned sign, unsigned exponent, unsigned mantissa)
{
    return (uint16_t)((sign << 15) | (exponent << 7) | mantissa);
}

static int chunk_size_ok(uint32_t c)
{
    /* Chunk-local escape positions are stored as u16, so a chunk holds at most 65536
     * elements; 16 is the smallest chunk this format accepts. */
    return c >= 16u && c <= 65536u && (c & (c - 1u)) == 0u;
}

static uint64_t ceil_div(uint64_t a, uint64_t b) { return a / b + (a % b != 0); }

/* Index of exponent e in the codebook, or -1 when e is not one of its 16 entries. */
static int codebook_index(const uint8_t cb[16], unsigned e)
{
    int k;
    for (k = 0; k < 16; ++k)
        if (cb[k] == e)
            return k;
    return -1;
}

static int codebook_distinct(const uint8_t cb[16])
{
    int a, b;
    for (a = 0; a < 16; ++a)
        for (b = a + 1; b < 16; ++b)
            if (cb[a] == cb[b])
                return 0;
    return 1;
}

/* ---- calibration [README, Highlights and Codec API: offline top-16 codebook; calibrate
 *      returns the coverage] ---- */

void szo_histogram(const uint16_t *x, uint64_t m, uint64_t hist[256])
{
    uint64_t i;
    int e;
    for (e = 0; e < 256; ++e)
        hist[e] = 0;
    for (i = 0; i < m; ++i)
        hist[bf16_exponent(x[i])] += 1;
}

/* The top-16 codebook [README Highlights]; ties by the smaller exponent (this project's reading). */
void szo_codebook(const uint64_t hist[256], uint8_t cb[16])
{
    /* Rank the 256 exponent values by count, most frequent first; equal counts are
     * ranked by the smaller exponent first.  Slot k holds the k-th ranked value. */
    int taken[256];
    int e, k;
    for (e = 0; e < 256; ++e)
        taken[e] = 0;
    for (k = 0; k < 16; ++k) {
        int best = -1;
        for (e = 0; e < 256; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || hist[e] > hist[best])
                best = e;
        }
        taken[best] = 1;
        cb[k] = (uint8_t)best;
    }
}

/* The coverage that calibrate returns [README Codec API]. */
double szo_coverage(const uint64_t hist[256], const uint8_t cb[16], uint64_t m)
{
    uint64_t covered = 0;
    int k;
    if (m == 0)
        return 0.0;
    for (k = 0; k < 16; ++k)
        covered += hist[cb[k]];
    return (double)covered / (double)m;
}

/* ---- exponent statistics [README, Repository Contents and Reproducing Paper Artifact
 *      Scripts: exponent entropy and top-16 coverage analysis of KV tensors; ZIPSERV,
 *      Information-Theoretic Limits and Exponent Entropy Bounds: Shannon entropy of the
 *      exponent field] ---- */

double szo_entropy(const uint64_t hist[256])
{
    /* H = -sum over exponent values of p log2 p, with p = count / total; values that
     * never occur contribute nothing. */
    uint64_t m = 0;
    double h = 0.0;
    int e;
    for (e = 0; e < 256; ++e)
        m += hist[e];
    if (m == 0)
        return 0.0;
    for (e = 0; e < 256; ++e) {
        if (hist[e] != 0) {
            const double p = (double)hist[e] / (double)m;
            h -= p * log2(p);
        }
    }
    return h;
}

/* ---- sizes: n sign+mantissa bytes + n/2 code bytes + escape bytes + chunk metadata ---- */

uint64_t szo_compressed_bytes(uint64_t n, uint32_t chunk_size, uint64_t n_escapes)
{
    uint64_t n_chunks = ceil_div(n, chunk_size);
    return 64u + n + ceil_div(n, 2) + 8u * (n_chunks + 1u) + 3u * n_escapes;
}

/* ---- encode [README Abstract; arXiv abstract: fixed 4-bit codes, exact sign and
 *      mantissa, rare exponents to a sparse (position, value) escape stream; README
 *      Highlights: escape metadata is chunk-local] ---- */

int szo_encode(const uint16_t *x, uint64_t n, const uint8_t cb[16], uint32_t chunk_size,
               uint8_t *sm, uint8_t *codes, uint64_t *chunk_off, uint16_t *esc_pos,
               uint8_t *esc_exp, uint64_t esc_capacity, uint64_t *n_escapes)
{
    uint64_t n_chunks, c, i, E;

    if (!chunk_size_ok(chunk_size) || !codebook_distinct(cb))
        return SZO_BAD_ARGUMENT;
    n_chunks = ceil_div(n, chunk_size);

    for (i = 0; i < ceil_div(n, 2); ++i)
        codes[i] = 0;

    E = 0;
    for (c = 0; c < n_chunks; ++c) {
        uint64_t start = c * chunk_size;
        uint64_t end = start + chunk_size < n ? start + chunk_size : n;
        chunk_off[c] = E;
        for (i = start; i < end; ++i) {
            uint16_t u = x[i];
            unsigned e = bf16_exponent(u);
            int k = codebook_index(cb, e);
            unsigned code;

            /* the sign and mantissa are kept exactly: sign above the 7 mantissa bits */
            sm[i] = (uint8_t)((bf16_sign(u) << 7) | bf16_mantissa(u));

            if (k >= 0) {
                code = (unsigned)k;
            } else {
                /* escape: record (position inside the chunk, exponent); the nibble is 0 */
                code = 0;
                if (E < esc_capacity) {
                    esc_pos[E] = (uint16_t)(i - start);
                    esc_exp[E] = (uint8_t)e;
                }
                E += 1;
            }
            /* element 2j in the low nibble of byte j, element 2j+1 in the high nibble */
            codes[i / 2] = (uint8_t)(codes[i / 2] | (code << (4 * (i % 2))));
        }
    }
    chunk_off[n_chunks] = E;
    *n_escapes = E;
    return E <= esc_capacity ? SZO_OK : SZO_NO_ROOM;
}

/* ---- decode [arXiv abstract: dense path plus sparse escape correction; README Codec
 *      API: the decoded tensor equals the input bit for bit] ---- */

static int escape_metadata_ok(const uint64_t *chunk_off, const uint16_t *esc_pos, uint64_t n,
                              uint64_t n_escapes, uint32_t chunk_size)
{
    uint64_t n_chunks = ceil_div(n, chunk_size);
    uint64_t c, j;
    if (chunk_off[0] != 0 || chunk_off[n_chunks] != n_escapes)
        return 0;
    for (c = 0; c < n_chunks; ++c) {
        uint64_t start = c * chunk_size;
        uint64_t len = start + chunk_size < n ? chunk_size : n - start;
        if (chunk_off[c + 1] < chunk_off[c] || chunk_off[c + 1] > n_escapes)
            return 0;
        for (j = chunk_off[c]; j < chunk_off[c + 1]; ++j) {
            if (esc_pos[j] >= len)
                return 0;
            if (j > chunk_off[c] && esc_pos[j] <= esc_pos[j - 1])
                return 0;
        }
    }
    return 1;
}

/* Decode [README Abstract]: codebook lookup of every code, then the sparse escape correction. */
int szo_decode(const uint8_t *sm, const uint8_t *codes, const uint64_t *chunk_off,
               const uint16_t *esc_pos, const uint8_t *esc_exp, uint64_t n, uint64_t n_escapes,
               const uint8_t cb[16], uint32_t chunk_size, uint16_t *y)
{
    uint64_t n_chunks, c, i, j;

    if (!chunk_size_ok(chunk_size) || !codebook_distinct(cb))
        return SZO_BAD_ARGUMENT;
    if (!escape_metadata_ok(chunk_off, esc_pos, n, n_escapes, chunk_size))
        return SZO_BAD_STREAM;
    n_chunks = ceil_div(n, chunk_size);

    /* dense path: code -> codebook exponent, sign and mantissa from the exact byte */
    for (i = 0; i < n; ++i) {
        unsigned code = (codes[i / 2] >> (4 * (i % 2))) & 0xFu;
        y[i] = bf16_join(sm[i] >> 7, cb[code], sm[i] & 0x7Fu);
    }
    /* sparse correction: put the stored exponent back at every escape position */
    for (c = 0; c < n_chunks; ++c) {
        for (j = chunk_off[c]; j < chunk_off[c + 1]; ++j) {
            i = c * chunk_size + esc_pos[j];
            y[i] = bf16_join(bf16_sign(y[i]), esc_exp[j], bf16_mantissa(y[i]));
        }
    }
    return SZO_OK;
}

/* ---- canonical serialized stream (this project's layout; the README Roadmap asks for
 *      codebook metadata that travels with the payload) ---- */

static void put_le(uint8_t *p, uint64_t v, int bytes)
{
    int b;
    for (b = 0; b < bytes; ++b)
        p[b] = (uint8_t)(v >> (8 * b));
}

static uint64_t get_le(const uint8_t *p, int bytes)
{
    uint64_t v = 0;
    int b;
    for (b = 0; b < bytes; ++b)
        v |= (uint64_t)p[b] << (8 * b);
    return v;
}

/* The 64-byte header of a canonical stream [README Roadmap: the codebook and payload
 * metadata travel with the payload]: "SZB1", version 1, header bytes 64, chunk size, flags
 * (0 BF16, 1 E5M2), n, n_chunks, E, the codebook, 8 reserved zero bytes; little-endian. */
void szo_header(uint64_t n, uint32_t chunk_size, uint64_t n_escapes, const uint8_t cb[16],
                uint32_t flags, uint8_t out[64])
{
    int i;

    memset(out, 0, 64);
    out[0] = 'S';
    out[1] = 'Z';
    out[2] = 'B';
    out[3] = '1';
    put_le(out + 4, 1, 2);          /* version */
    put_le(out + 6, 64, 2);         /* header bytes */
    put_le(out + 8, chunk_size, 4);
    put_le(out + 12, flags, 4);
    put_le(out + 16, n, 8);
    put_le(out + 24, ceil_div(n, chunk_size), 8);
    put_le(out + 32, n_escapes, 8);
    for (i = 0; i < 16; ++i)
        out[40 + i] = cb[i];
    /* bytes 56..63 stay zero (reserved) */
}

/* The canonical stream: header with the codebook, then the sections [README Roadmap]. */
int szo_serialize(const uint8_t *sm, const uint8_t *codes, const uint64_t *chunk_off,
                  const uint16_t *esc_pos, const uint8_t *esc_exp, uint64_t n, uint64_t n_escapes,
                  const uint8_t cb[16], uint32_t chunk_size, uint8_t *out, uint64_t out_len)
{
    uint64_t n_chunks, p, i;

    if (!chunk_size_ok(chunk_size))
        return SZO_BAD_ARGUMENT;
    if (out_len != szo_compressed_bytes(n, chunk_size, n_escapes))
        return SZO_BAD_ARGUMENT;
    n_chunks = ceil_div(n, chunk_size);

    szo_header(n, chunk_size, n_escapes, cb, 0, out);
    p = 64;
    for (i = 0; i < n; ++i)
        out[p++] = sm[i];
    for (i = 0; i < ceil_div(n, 2); ++i)
        out[p++] = codes[i];
    for (i = 0; i < n_chunks + 1; ++i) {
        put_le(out + p, chunk_off[i], 8);
        p += 8;
    }
    for (i = 0; i < n_escapes; ++i) {
        put_le(out + p, esc_pos[i], 2);
        p += 2;
    }
    for (i = 0; i < n_escapes; ++i)
        out[p++] = esc_exp[i];
    return p == out_len ? SZO_OK : SZO_BAD_ARGUMENT;
}

/* Header of a canonical stream [README Roadmap: payload metadata that travels with it]. */
int szo_stream_info(const uint8_t *buf, uint64_t len, uint64_t *n, uint32_t *chunk_size,
                    uint64_t *n_escapes, uint8_t cb[16])
{
    uint64_t nn, n_chunks, E, i;
    uint32_t C;

    if (len < 64)
        return SZO_BAD_STREAM;
    if (buf[0] != 'S' || buf[1] != 'Z' || buf[2] != 'B' || buf[3] != '1')
        return SZO_BAD_STREAM;
    if (get_le(buf + 4, 2) != 1 || get_le(buf + 6, 2) != 64 || get_le(buf + 12, 4) != 0)
        return SZO_BAD_STREAM;
    for (i = 56; i < 64; ++i)
        if (buf[i] != 0)
            return SZO_BAD_STREAM;
    C = (uint32_t)get_le(buf + 8, 4);
    nn = get_le(buf + 16, 8);
    n_chunks = get_le(buf + 24, 8);
    E = get_le(buf + 32, 8);
    if (!chunk_size_ok(C) || n_chunks != ceil_div(nn, C))
        return SZO_BAD_STREAM;
    /* an escape list longer than the element count, or a size that does not match the
     * layout, cannot come from the encoder */
    if (E > nn || len != szo_compressed_bytes(nn, C, E))
        return SZO_BAD_STREAM;
    *n = nn;
    *chunk_size = C;
    *n_escapes = E;
    for (i = 0; i < 16; ++i)
        cb[i] = buf[40 + i];
    return SZO_OK;
}

/* Decode a stream with the codec's own codebook [README Codec API: same calibrated state]. */
int szo_decode_stream(const uint8_t *buf, uint64_t len, const uint8_t cb[16], uint16_t *y,
                      uint64_t y_len)
{
    uint64_t n, E, n_chunks, i, p;
    uint32_t C;
    uint8_t stream_cb[16];
    uint64_t *chunk_off;
    uint16_t *esc_pos;
    int rc;

    rc = szo_stream_info(buf, len, &n, &C, &E, stream_cb);
    if (rc != SZO_OK)
        return rc;
    if (memcmp(stream_cb, cb, 16) != 0)
        return SZO_WRONG_CODEBOOK;
    if (y_len != n)
        return SZO_BAD_ARGUMENT;
    n_chunks = ceil_div(n, C);

    /* the multi-byte sections are unaligned inside the stream: copy them out */
    chunk_off = (uint64_t *)malloc((n_chunks + 1) * sizeof(uint64_t));
    esc_pos = (uint16_t *)malloc((E ? E : 1) * sizeof(uint16_t));
    if (!chunk_off || !esc_pos) {
        free(chunk_off);
        free(esc_pos);
        return SZO_BAD_ARGUMENT;
    }
    p = 64 + n + ceil_div(n, 2);
    for (i = 0; i < n_chunks + 1; ++i)
        chunk_off[i] = get_le(buf + p + 8 * i, 8);
    p += 8 * (n_chunks + 1);
    for (i = 0; i < E; ++i)
        esc_pos[i] = (uint16_t)get_le(buf + p + 2 * i, 2);
    p += 2 * E;

    rc = szo_decode(buf + 64, buf + 64 + n, chunk_off, esc_pos, buf + p, n, E, cb, C, y);
    free(chunk_off);
    free(esc_pos);
    return rc;
}

/* ======================================================================================
 * FP8 E5M2 elements [README FAQ and arXiv abstract: the same method applied on top of an
 * FP8 E5M2 KV cache, up to 1.14x over native E5M2].  E5M2 = 1 sign bit (7), 5 exponent
 * bits (6..2), 2 mantissa bits (1..0).  The 3 sign+mantissa bits are kept exactly, the
 * 5-bit exponent becomes a 4-bit code into a top-16 codebook over the 32 exponent values,
 * and exponents outside it go to the same chunk-local escape stream.  The layout is this
 * project's reading (the pages print none):
 *   - sm3: field (sign << 2) | mantissa of element i at bits 3i..3i+2 of a little-endian
 *     bit stream (byte j holds bits 8j..8j+7), ceil(3n/8) bytes;
 *   - codes, chunk_off, esc_pos, esc_exp: as for BF16 (exponents 0..31);
 *   - serialized header as for BF16 with flags = 1.
 * ====================================================================================== */

static unsigned e5m2_sign(uint8_t b) { return (b >> 7) & 0x1u; }
static unsigned e5m2_exponent(uint8_t b) { return (b >> 2) & 0x1Fu; }
static unsigned e5m2_mantissa(uint8_t b) { return b & 0x3u; }

static uint8_t e5m2_join(unsigned sign, unsigned exponent, unsigned mantissa)
{
    return (uint8_t)((sign << 7) | (exponent << 2) | mantissa);
}

/* A codebook of 16 distinct 5-bit exponents. */
static int codebook8_ok(const uint8_t cb[16])
{
    int k;
    for (k = 0; k < 16; ++k)
        if (cb[k] > 31)
            return 0;
    return codebook_distinct(cb);
}

/* The 3-bit field of element i in the bit stream, and setting it (stream starts zeroed). */
static unsigned field3_get(const uint8_t *s, uint64_t i)
{
    unsigned v = 0, b;
    for (b = 0; b < 3; ++b) {
        uint64_t bit = 3 * i + b;
        v |= ((s[bit / 8] >> (bit % 8)) & 1u) << b;
    }
    return v;
}

static void field3_set(uint8_t *s, uint64_t i, unsigned v)
{
    unsigned b;
    for (b = 0; b < 3; ++b) {
        uint64_t bit = 3 * i + b;
        if ((v >> b) & 1u)
            s[bit / 8] = (uint8_t)(s[bit / 8] | (1u << (bit % 8)));
    }
}

/* E5M2 exponent histogram [README FAQ], as szo_histogram. */
void szo8_histogram(const uint8_t *x, uint64_t m, uint64_t hist[32])
{
    uint64_t i;
    int e;
    for (e = 0; e < 32; ++e)
        hist[e] = 0;
    for (i = 0; i < m; ++i)
        hist[e5m2_exponent(x[i])] += 1;
}

/* E5M2 top-16 codebook over the 32 exponent values [README FAQ], as szo_codebook. */
void szo8_codebook(const uint64_t hist[32], uint8_t cb[16])
{
    /* as for BF16, over the 32 exponent values: most frequent first, equal counts by the
     * smaller exponent first */
    int taken[32];
    int e, k;
    for (e = 0; e < 32; ++e)
        taken[e] = 0;
    for (k = 0; k < 16; ++k) {
        int best = -1;
        for (e = 0; e < 32; ++e) {
            if (taken[e])
                continue;
            if (best == -1 || hist[best] < hist[e])
                best = e;
        }
        taken[best] = 1;
        cb[k] = (uint8_t)best;
    }
}

/* E5M2 coverage [README FAQ, Codec API], as szo_coverage. */
double szo8_coverage(const uint64_t hist[32], const uint8_t cb[16], uint64_t m)
{
    uint64_t covered = 0;
    int k;
    if (m == 0)
        return 0.0;
    for (k = 0; k < 16; ++k)
        covered += hist[cb[k]];
    return (double)covered / (double)m;
}

/* E5M2 stream size [README FAQ]: the 3-bit field stream replaces the sign+mantissa bytes. */
uint64_t szo8_compressed_bytes(uint64_t n, uint32_t chunk_size, uint64_t n_escapes)
{
    if (!chunk_size_ok(chunk_size))
        return 0;
    return 64u + ceil_div(3u * n, 8u) + ceil_div(n, 2u) + 8u * (ceil_div(n, chunk_size) + 1u) +
           3u * n_escapes;
}

/* E5M2 encode [README FAQ; arXiv abstract], in the order of szo_encode. */
int szo8_encode(const uint8_t *x, uint64_t n, const uint8_t cb[16], uint32_t chunk_size,
                uint8_t *sm3, uint8_t *codes, uint64_t *chunk_off, uint16_t *esc_pos,
                uint8_t *esc_exp, uint64_t esc_capacity, uint64_t *n_escapes)
{
    uint64_t n_chunks, c, i, E;

    if (!chunk_size_ok(chunk_size) || !codebook8_ok(cb))
        return SZO_BAD_ARGUMENT;
    n_chunks = ceil_div(n, chunk_size);
    for (i = 0; i < ceil_div(3u * n, 8u); ++i)
        sm3[i] = 0;
    for (i = 0; i < ceil_div(n, 2); ++i)
        codes[i] = 0;

    E = 0;
    for (c = 0; c < n_chunks; ++c) {
        uint64_t start = c * chunk_size;
        uint64_t end = start + chunk_size < n ? start + chunk_size : n;
        chunk_off[c] = E;
        for (i = start; i < end; ++i) {
            uint8_t b = x[i];
            unsigned e = e5m2_exponent(b);
            int k = codebook_index(cb, e);
            unsigned code;

            /* sign and mantissa kept exactly: the sign above the 2 mantissa bits */
            field3_set(sm3, i, (e5m2_sign(b) << 2) | e5m2_mantissa(b));

            if (k >= 0) {
                code = (unsigned)k;
            } else {
                code = 0;
                if (E < esc_capacity) {
                    esc_pos[E] = (uint16_t)(i - start);
                    esc_exp[E] = (uint8_t)e;
                }
                E += 1;
            }
            codes[i / 2] = (uint8_t)(codes[i / 2] | (code << (4 * (i % 2))));
        }
    }
    chunk_off[n_chunks] = E;
    *n_escapes = E;
    return E <= esc_capacity ? SZO_OK : SZO_NO_ROOM;
}

/* E5M2 decode [README FAQ], in the order of szo_decode. */
int szo8_decode(const uint8_t *sm3, const uint8_t *codes, const uint64_t *chunk_off,
                const uint16_t *esc_pos, const uint8_t *esc_exp, uint64_t n, uint64_t n_escapes,
                const uint8_t cb[16], uint32_t chunk_size, uint8_t *y)
{
    uint64_t n_chunks, c, i, j;

    if (!chunk_size_ok(chunk_size) || !codebook8_ok(cb))
        return SZO_BAD_ARGUMENT;
    if (!escape_metadata_ok(chunk_off, esc_pos, n, n_escapes, chunk_size))
        return SZO_BAD_STREAM;
    for (j = 0; j < n_escapes; ++j)
        if (esc_exp[j] > 31)
            return SZO_BAD_STREAM;
    n_chunks = ceil_div(n, chunk_size);

    for (i = 0; i < n; ++i) {
        unsigned code = (codes[i / 2] >> (4 * (i % 2))) & 0xFu;
        unsigned f = field3_get(sm3, i);
        y[i] = e5m2_join(f >> 2, cb[code], f & 0x3u);
    }
    for (c = 0; c < n_chunks; ++c) {
        for (j = chunk_off[c]; j < chunk_off[c + 1]; ++j) {
            i = c * chunk_size + esc_pos[j];
            y[i] = e5m2_join(e5m2_sign(y[i]), esc_exp[j], e5m2_mantissa(y[i]));
        }
    }
    return SZO_OK;
}

/* E5M2 canonical stream [README FAQ, Roadmap], flags = 1. */
int szo8_serialize(const uint8_t *sm3, const uint8_t *codes, const uint64_t *chunk_off,
                   const uint16_t *esc_pos, const uint8_t *esc_exp, uint64_t n, uint64_t n_escapes,
                   const uint8_t cb[16], uint32_t chunk_size, uint8_t *out, uint64_t out_len)
{
    uint64_t n_chunks, p, i;

    if (!chunk_size_ok(chunk_size))
        return SZO_BAD_ARGUMENT;
    if (out_len != szo8_compressed_bytes(n, chunk_size, n_escapes))
        return SZO_BAD_ARGUMENT;
    n_chunks = ceil_div(n, chunk_size);

    szo_header(n, chunk_size, n_escapes, cb, 1, out);     /* flags 1: E5M2 elements */
    p = 64;
    for (i = 0; i < ceil_div(3u * n, 8u); ++i)
        out[p++] = sm3[i];
    for (i = 0; i < ceil_div(n, 2); ++i)
        out[p++] = codes[i];
    for (i = 0; i < n_chunks + 1; ++i) {
        put_le(out + p, chunk_off[i], 8);
        p += 8;
    }
    for (i = 0; i < n_escapes; ++i) {
        put_le(out + p, esc_pos[i], 2);
        p += 2;
    }
    for (i = 0; i < n_escapes; ++i)
        out[p++] = esc_exp[i];
    return p == out_len ? SZO_OK : SZO_BAD_ARGUMENT;
}

/* Decode an E5M2 stream with the codec's own codebook [README FAQ, Codec API]. */
int szo8_decode_stream(const uint8_t *buf, uint64_t len, const uint8_t cb[16], uint8_t *y,
                       uint64_t y_len)
{
    uint64_t n, E, n_chunks, i, p, s3;
    uint32_t C;
    uint64_t *chunk_off;
    uint16_t *esc_pos;
    int rc;

    if (len < 64 || buf[0] != 'S' || buf[1] != 'Z' || buf[2] != 'B' || buf[3] != '1')
        return SZO_BAD_STREAM;
    if (get_le(buf + 4, 2) != 1 || get_le(buf + 6, 2) != 64 || get_le(buf + 12, 4) != 1)
        return SZO_BAD_STREAM;
    for (i = 56; i < 64; ++i)
        if (buf[i] != 0)
            return SZO_BAD_STREAM;
    C = (uint32_t)get_le(buf + 8, 4);
    n = get_le(buf + 16, 8);
    n_chunks = get_le(buf + 24, 8);
    E = get_le(buf + 32, 8);
    if (!chunk_size_ok(C) || n_chunks != ceil_div(n, C))
        return SZO_BAD_STREAM;
    if (E > n || len != szo8_compressed_bytes(n, C, E))
        return SZO_BAD_STREAM;
    if (memcmp(buf + 40, cb, 16) != 0)
        return SZO_WRONG_CODEBOOK;
    if (y_len != n)
        return SZO_BAD_ARGUMENT;

    chunk_off = (uint64_t *)malloc((n_chunks + 1) * sizeof(uint64_t));
    esc_pos = (uint16_t *)malloc((E ? E : 1) * sizeof(uint16_t));
    if (!chunk_off || !esc_pos) {
        free(chunk_off);
        free(esc_pos);
        return SZO_BAD_ARGUMENT;
    }
    s3 = ceil_div(3u * n, 8u);
    p = 64 + s3 + ceil_div(n, 2);
    for (i = 0; i < n_chunks + 1; ++i)
        chunk_off[i] = get_le(buf + p + 8 * i, 8);
    p += 8 * (n_chunks + 1);
    for (i = 0; i < E; ++i)
        esc_pos[i] = (uint16_t)get_le(buf + p + 2 * i, 2);
    p += 2 * E;

    rc = szo8_decode(buf + 64, buf + 64 + s3, chunk_off, esc_pos, buf + p, n, E, cb, C, y);
    free(chunk_off);
    free(esc_pos);
    return rc;
}
