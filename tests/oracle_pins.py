"""Pins that tie the CPU oracle to something other than itself.

Each check takes an ``oracle.Oracle`` instance so that the mutation test can run
the same battery against deliberately broken copies of the oracle.  The
expected values come from: the hand-derived worked example under tests/golden
(with its citations), closed forms of the exhaustive 65 536-word tensor, a
brute-force re-derivation that reads BF16 fields through floating-point
semantics (frexp, copysign) instead of bit masks, and invariants the pages fix
(bitwise round trip; size = n + n/2 + escape bytes + chunk metadata).  The FP8 E5M2
variant has the same kinds of pin: a hand-derived example, the closed form of all 256
bytes, fields read through torch's float8_e5m2 values, round trips and the 8/7 best case.
"""
from __future__ import annotations

import collections
import math

import numpy as np

from conftest import hex_bytes, ints, load_golden


# ---- worked example -------------------------------------------------------------------

def worked_example():
    g = load_golden("worked_example_c16.txt")
    cal = np.array([e << 7 for e in range(112, 128) for _ in range(e - 111)], np.uint16)
    x = np.array([int(t, 16) for t in g["input_u16"].split()], np.uint16)
    return g, cal, x


def check_worked_example(o) -> None:
    g, cal, x = worked_example()
    C = int(g["chunk_size"])
    cb, cov, _ = o.calibrate(cal)
    assert bytes(cb) == hex_bytes(g["codebook"]), "codebook"
    assert cov == float(g["calibration_coverage"]), "calibration coverage"
    enc = o.encode(x, cb, C)
    assert bytes(enc["sm"]) == hex_bytes(g["sm"]), "sm"
    assert bytes(enc["codes"]) == hex_bytes(g["codes"]), "codes"
    assert enc["chunk_off"].tolist() == ints(g["chunk_off"]), "chunk_off"
    assert enc["esc_pos"].tolist() == ints(g["esc_pos"]), "esc_pos"
    assert enc["esc_exp"].tolist() == ints(g["esc_exp"]), "esc_exp"
    assert enc["n_escapes"] == int(g["n_escapes"])
    assert enc["compressed_bytes"] == int(g["compressed_bytes"])
    s = o.serialize(enc)
    assert len(s) == int(g["compressed_bytes"])
    assert s[:64] == hex_bytes(g["header"]), "header"
    assert o.header(x.size, C, enc["n_escapes"], cb, 0) == hex_bytes(g["header"]), "header writer"
    # body = sections in order, little-endian
    body = (hex_bytes(g["sm"]) + hex_bytes(g["codes"])
            + b"".join(v.to_bytes(8, "little") for v in ints(g["chunk_off"]))
            + b"".join(v.to_bytes(2, "little") for v in ints(g["esc_pos"]))
            + bytes(ints(g["esc_exp"])))
    assert s[64:] == body, "stream body"
    num, den = (int(t) for t in g["input_coverage"].split("/"))
    assert (x.size - enc["n_escapes"], x.size) == (num, den)
    assert np.array_equal(o.decode(enc), x)
    assert np.array_equal(o.decode_stream(s, cb), x)
    # odd-length prefix and empty input
    e7 = o.encode(x[:7], cb, C)
    assert bytes(e7["codes"]) == hex_bytes(g["prefix7_codes"])
    assert e7["chunk_off"].tolist() == ints(g["prefix7_chunk_off"])
    assert len(o.serialize(e7)) == int(g["prefix7_compressed_bytes"])
    assert np.array_equal(o.decode(e7), x[:7])
    e0 = o.encode(x[:0], cb, C)
    s0 = o.serialize(e0)
    assert len(s0) == int(g["empty_compressed_bytes"])
    hdr = bytearray(hex_bytes(g["header"]))
    hdr[16:40] = bytes(24)
    assert s0[:64] == bytes(hdr) and s0[64:] == bytes(8)
    assert o.decode_stream(s0, cb).size == 0


# ---- exhaustive tensor: every 16-bit word once ------------------------------------------

def check_exhaustive(o, C: int = 1024) -> None:
    x = np.arange(1 << 16, dtype=np.uint16)
    cb, cov, h = o.calibrate(x)
    # Each exponent value is shared by 2 signs x 128 mantissas = 256 words: all tie, so the
    # exponent-ascending tie-break gives the first 16 exponents.
    assert h.tolist() == [256] * 256
    assert cb.tolist() == list(range(16))
    assert cov == 16 * 256 / 65536
    enc = o.encode(x, cb, C)
    E = 65536 - 16 * 256
    assert enc["n_escapes"] == E
    n_chunks = 65536 // C
    assert enc["compressed_bytes"] == 64 + 65536 + 32768 + 8 * (n_chunks + 1) + 3 * E
    if C == 1024:
        assert enc["compressed_bytes"] == 283208
    # Words w with (w mod 2^15) < 16*128 = 2048 have exponent < 16 (in the codebook); the
    # rest escape.  Chunk c holds words [cC, cC+C).
    escaped = [[w - c * C for w in range(c * C, (c + 1) * C) if w % 32768 >= 2048]
               for c in range(n_chunks)]
    assert enc["chunk_off"].tolist() == [sum(len(e) for e in escaped[:c])
                                         for c in range(n_chunks + 1)]
    assert enc["esc_pos"].tolist() == [p for e in escaped for p in e]
    # the escaped exponent of word w is floor((w mod 32768) / 128)
    assert enc["esc_exp"].tolist() == [(w % 32768) // 128 for w in range(65536)
                                       if (w % 32768) >= 2048]
    # sign+mantissa byte: words w and w + 128 (next exponent) share it; w + 32768 flips bit 7
    sm = enc["sm"].astype(np.int64)
    assert np.array_equal(sm[:128], np.arange(128))
    assert np.array_equal(sm, np.tile(np.concatenate([np.arange(128)] * 256), 2)
                          + np.repeat([0, 128], 32768))
    # codes: for a codebook word, the code is its exponent floor(w / 128); escapes give 0
    nib = np.zeros(65536, np.int64)
    nib[0::2] = enc["codes"] & 0xF
    nib[1::2] = enc["codes"] >> 4
    expect = np.array([(w % 32768) // 128 if (w % 32768) < 2048 else 0 for w in range(65536)])
    assert np.array_equal(nib, expect)
    assert np.array_equal(o.decode(enc), x)


# ---- brute force through float semantics --------------------------------------------------

def fields_by_value(word: int):
    """(sign, exponent field, mantissa field) of a BF16 word, read from the value it encodes
    (BF16 is the upper half of an IEEE binary32) instead of masking bits."""
    f = float(np.array([word << 16], np.uint32).view(np.float32)[0])
    sign = 1 if math.copysign(1.0, f) < 0 else 0
    a = abs(f)
    if math.isnan(f):
        return sign, 255, word & 0x7F          # the payload has no value semantics
    if math.isinf(f):
        return sign, 255, 0
    if a == 0.0:
        return sign, 0, 0
    if a < 2.0 ** -126:                        # subnormal: a = mantissa * 2^-133
        return sign, 0, int(a / 2.0 ** -133)
    m, q = math.frexp(a)                       # a = m 2^q, 1/2 <= m < 1
    return sign, q + 126, int((2 * m - 1) * 128)


def brute_force(words, C: int):
    """Expected codebook and stream sections for a small input, by plain enumeration."""
    fields = [fields_by_value(int(w)) for w in words]
    counts = collections.Counter(e for _, e, _ in fields)
    cb = sorted(range(256), key=lambda e: (-counts[e], e))[:16]
    sm = [s * 128 + m for s, _, m in fields]
    codes_per_elem, esc, chunk_off = [], [], []
    for c in range(-(-len(words) // C)):
        chunk_off.append(len(esc))
        for p, (s, e, m) in enumerate(fields[c * C:(c + 1) * C]):
            if e in cb:
                codes_per_elem.append(cb.index(e))
            else:
                codes_per_elem.append(0)
                esc.append((p, e))
    chunk_off.append(len(esc))
    if len(codes_per_elem) % 2:
        codes_per_elem.append(0)
    codes = [codes_per_elem[2 * j] + 16 * codes_per_elem[2 * j + 1]
             for j in range(len(codes_per_elem) // 2)]
    return cb, sm, codes, chunk_off, esc


def check_brute_force(o, seeds=range(12)) -> None:
    specials = [0x0000, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC1, 0xFFFF, 0x0080, 0x7F7F]
    for seed in seeds:
        rng = np.random.default_rng(1000 + seed)
        n = int(rng.integers(16, 65))
        # mostly a narrow exponent band (so the codebook matters), some wide, some special
        z = rng.standard_normal(n).astype(np.float32) * np.float32(2.0 ** int(rng.integers(-3, 4)))
        words = (z.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        wide = rng.random(n) < 0.3
        words[wide] = rng.integers(0, 1 << 16, size=int(wide.sum())).astype(np.uint16)
        for k in rng.choice(n, size=min(n, 6), replace=False):
            words[k] = specials[int(rng.integers(0, len(specials)))]
        for C in (16, 32):
            cb, sm, codes, chunk_off, esc = brute_force(words, C)
            got_cb, _, _ = o.calibrate(words)
            assert got_cb.tolist() == cb, f"codebook seed {seed}"
            enc = o.encode(words, got_cb, C)
            assert enc["sm"].tolist() == sm, f"sm seed {seed}"
            assert enc["codes"].tolist() == codes, f"codes seed {seed}"
            assert enc["chunk_off"].tolist() == chunk_off, f"chunk_off seed {seed}"
            assert list(zip(enc["esc_pos"].tolist(), enc["esc_exp"].tolist())) == esc
            assert enc["compressed_bytes"] == (64 + n + -(-n // 2) + 8 * (len(chunk_off))
                                               + 3 * len(esc))
            assert np.array_equal(o.decode(enc), words), f"round trip seed {seed}"


# ---- round trip on varied inputs -----------------------------------------------------------

def check_round_trips(o) -> None:
    from workloads import mixed_words, normal_words, random_words
    cal = normal_words(4096, 5)
    cb, _, _ = o.calibrate(cal)
    for n, C, gen in [(1, 16, random_words), (17, 16, random_words), (1000, 64, mixed_words),
                      (4097, 1024, mixed_words), (12345, 4096, random_words),
                      (70001, 65536, mixed_words)]:
        x = gen(n, n)
        enc = o.encode(x, cb, C)
        s = o.serialize(enc)
        assert len(s) == enc["compressed_bytes"] == o.compressed_bytes(n, C, enc["n_escapes"])
        assert np.array_equal(o.decode(enc), x)
        assert np.array_equal(o.decode_stream(s, cb), x)


def check_codebook_rules(o) -> None:
    # ties broken toward the smaller exponent; zero counts fill the tail in ascending order
    h = np.zeros(256, np.uint64)
    h[200], h[100], h[150], h[7] = 5, 5, 9, 5
    cb = o.codebook(h)
    assert cb[:4].tolist() == [150, 7, 100, 200]
    assert cb[4:].tolist() == [e for e in range(256) if e not in (7, 100, 150, 200)][:12]
    # a single repeated word: one exponent observed, coverage 1
    cb1, cov1, _ = o.calibrate(np.full(10, 0x3F80, np.uint16))
    assert cb1[0] == 127 and cov1 == 1.0
    assert o.calibrate(np.zeros(0, np.uint16))[1] == 0.0


def check_entropy(o) -> None:
    """Exponent entropy against values the definition fixes exactly: the exhaustive word
    set has 256 equally likely exponents (8 bits); a dyadic distribution (1/2, 1/4, 1/8,
    1/8) has 1.75 bits; one value or none has 0; random histograms agree with scipy's
    entropy routine in base 2."""
    from scipy.stats import entropy as scipy_entropy
    x = np.arange(65536, dtype=np.uint16)
    assert o.entropy(o.histogram(x)) == 8.0
    h = np.zeros(256, np.uint64)
    assert o.entropy(h) == 0.0
    h[77] = 1000
    assert o.entropy(h) == 0.0
    h[:] = 0
    h[[127, 3, 200, 0]] = [4000, 2000, 1000, 1000]
    assert o.entropy(h) == 1.75
    h[:] = 0
    h[[5, 250]] = [3, 3]
    assert o.entropy(h) == 1.0
    rng = np.random.default_rng(123)
    for k in range(20):
        h = rng.integers(0, 1000, 256).astype(np.uint64)
        h[rng.random(256) < 0.7] = 0
        h[rng.integers(256)] += 1
        want = float(scipy_entropy(h.astype(np.float64), base=2))
        assert abs(o.entropy(h) - want) <= 1e-12 * max(1.0, want)


# ---- FP8 E5M2 ---------------------------------------------------------------------------------

def check_worked_example8(o) -> None:
    """The hand-derived E5M2 example (tests/golden/worked_example_e5m2_c16.txt)."""
    g = load_golden("worked_example_e5m2_c16.txt")
    C = int(g["chunk_size"])
    cal = np.frombuffer(hex_bytes(g["calibration_u8"]), np.uint8)
    cb, cov, _ = o.calibrate8(cal)
    assert bytes(cb) == hex_bytes(g["codebook"])
    num, den = (int(t) for t in g["calibration_coverage"].split("/"))
    assert cov == num / den
    x = np.frombuffer(hex_bytes(g["input_u8"]), np.uint8)
    e = o.encode8(x, cb, C)
    assert bytes(e["sm3"]) == hex_bytes(g["sm3"])
    assert bytes(e["codes"]) == hex_bytes(g["codes"])
    assert e["chunk_off"].tolist() == ints(g["chunk_off"])
    assert e["esc_pos"].tolist() == ints(g["esc_pos"])
    assert e["esc_exp"].tolist() == ints(g["esc_exp"])
    assert e["n_escapes"] == int(g["n_escapes"])
    assert e["compressed_bytes"] == int(g["compressed_bytes"])
    s = o.serialize8(e)
    assert len(s) == int(g["compressed_bytes"]) and s[:64] == hex_bytes(g["header"])
    assert o.header(x.size, C, e["n_escapes"], cb, 1) == hex_bytes(g["header"]), "header writer"
    assert np.array_equal(o.decode8(e), x)
    assert np.array_equal(o.decode_stream8(s, cb), x)
    e7 = o.encode8(x[:7], cb, C)
    assert bytes(e7["sm3"]) == hex_bytes(g["prefix7_sm3"])
    assert bytes(e7["codes"]) == hex_bytes(g["prefix7_codes"])
    assert e7["chunk_off"].tolist() == ints(g["prefix7_chunk_off"])
    assert e7["compressed_bytes"] == int(g["prefix7_compressed_bytes"])
    assert o.encode8(x[:0], cb, C)["compressed_bytes"] == int(g["empty_compressed_bytes"])


def check_exhaustive8(o, C: int = 16) -> None:
    """All 256 bytes once each: every exponent value occurs 8 times (2 signs x 4
    mantissas), so the codebook is 0..15 and the escapes are the bytes whose exponent,
    (b mod 128) // 4, is 16 or more.  Fields and codes from that arithmetic (division, not
    bit masks)."""
    x = np.arange(256, dtype=np.uint8)
    cb, cov, h = o.calibrate8(x)
    assert h.tolist() == [8] * 32
    assert bytes(cb) == bytes(range(16)) and cov == 0.5
    e = o.encode8(x, cb, C)
    expo = [(b % 128) // 4 for b in range(256)]
    field = [(b // 128) * 4 + b % 4 for b in range(256)]
    bits = sum(f * 8 ** i for i, f in enumerate(field))            # 3 bits per element
    assert bytes(e["sm3"]) == bits.to_bytes(96, "little")
    want_codes = bytes((expo[2 * j] if expo[2 * j] < 16 else 0) + 16 * (expo[2 * j + 1] if expo[2 * j + 1] < 16 else 0)
                       for j in range(128))
    assert bytes(e["codes"]) == want_codes
    assert e["n_escapes"] == 128
    want_pos, want_exp, want_off = [], [], [0]
    for c in range(-(-256 // C)):
        for b in range(c * C, min(256, (c + 1) * C)):
            if expo[b] >= 16:
                want_pos.append(b - c * C)
                want_exp.append(expo[b])
        want_off.append(len(want_pos))
    assert e["esc_pos"].tolist() == want_pos and e["esc_exp"].tolist() == want_exp
    assert e["chunk_off"].tolist() == want_off
    assert e["compressed_bytes"] == 64 + 96 + 128 + 8 * (len(want_off)) + 3 * 128
    assert np.array_equal(o.decode8(e), x)


def e5m2_fields_by_value(b: int):
    """(sign, exponent, mantissa) of an E5M2 byte from the value torch's float8_e5m2 type
    gives it: frexp for normals, multiples of 2^-16 for subnormals, 31 for Inf/NaN."""
    import torch
    v = float(torch.tensor([b], dtype=torch.uint8).view(torch.float8_e5m2).float()[0])
    if math.isnan(v) or math.isinf(v):
        return b >> 7, 31, b & 3                     # the non-finite codes, read as stored
    sign = 1 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a < 2.0 ** -14:
        return sign, 0, int(round(a / 2.0 ** -16))
    f, q = math.frexp(a)                             # a = f 2^q, f in [0.5, 1)
    return sign, q + 14, int(round((2 * f - 1) * 4))


def brute_force8(x: np.ndarray, C: int):
    from collections import Counter
    fields = [e5m2_fields_by_value(int(b)) for b in x]
    cnt = Counter(e for _, e, _ in fields)
    cb = sorted(range(32), key=lambda e: (-cnt.get(e, 0), e))[:16]
    pos = {e: k for k, e in enumerate(cb)}
    bits = 0
    codes = [0] * ((len(x) + 1) // 2)
    esc = []
    off = []
    for i, (s, e, m) in enumerate(fields):
        if i % C == 0:
            off.append(len(esc))
        bits += (s * 4 + m) << (3 * i)
        if e in pos:
            codes[i // 2] += pos[e] << (4 * (i % 2))
        else:
            esc.append((i % C, e))
    off.append(len(esc))
    sm3 = bits.to_bytes(-(-3 * len(x) // 8), "little")
    return bytes(cb), sm3, bytes(codes), off, esc


def check_brute_force8(o, seeds=range(12)) -> None:
    for seed in seeds:
        rng = np.random.default_rng(1000 + seed)
        n = int(rng.integers(16, 80))
        C = [16, 32][seed % 2]
        # mostly a narrow exponent band, some anywhere (specials included)
        x = ((rng.integers(0, 2, n) << 7) | (rng.integers(12, 19, n) << 2) | rng.integers(0, 4, n)).astype(np.uint8)
        wide = rng.random(n) < 0.25
        x[wide] = rng.integers(0, 256, int(wide.sum())).astype(np.uint8)
        cb, sm3, codes, off, esc = brute_force8(x, C)
        ocb, _, _ = o.calibrate8(x)
        assert bytes(ocb) == cb
        e = o.encode8(x, ocb, C)
        assert bytes(e["sm3"]) == sm3 and bytes(e["codes"]) == codes
        assert e["chunk_off"].tolist() == off
        assert list(zip(e["esc_pos"].tolist(), e["esc_exp"].tolist())) == esc
        assert np.array_equal(o.decode8(e), x)


def check_round_trips8(o) -> None:
    rng = np.random.default_rng(77)
    for n in (0, 1, 7, 8, 9, 31, 100, 1000):
        for C in (16, 64, 65536):
            x = rng.integers(0, 256, n).astype(np.uint8)
            cb = o.calibrate8(rng.integers(0, 256, 500).astype(np.uint8))[0]
            e = o.encode8(x, cb, C)
            assert np.array_equal(o.decode8(e), x)
            s = o.serialize8(e)
            assert len(s) == 64 + -(-3 * n // 8) + (n + 1) // 2 + 8 * (-(-n // C) + 1) + 3 * e["n_escapes"]
            assert np.array_equal(o.decode_stream8(s, cb), x)
    # no escapes: 7 bits per element past the metadata, the pages' 8/7 best case
    x = ((rng.integers(12, 28, 8000) << 2) | rng.integers(0, 4, 8000)).astype(np.uint8)
    cb = o.calibrate8(x)[0]
    e = o.encode8(x, cb, 1024)
    assert e["n_escapes"] == 0
    assert e["compressed_bytes"] - 64 - 8 * (8 + 1) == 8000 * 7 // 8


def run_all(o) -> None:
    check_worked_example(o)
    check_exhaustive(o, 1024)
    check_exhaustive(o, 16)
    check_exhaustive(o, 65536)
    check_brute_force(o)
    check_round_trips(o)
    check_codebook_rules(o)
    check_entropy(o)
    check_worked_example8(o)
    check_exhaustive8(o, 16)
    check_exhaustive8(o, 64)
    check_brute_force8(o)
    check_round_trips8(o)
