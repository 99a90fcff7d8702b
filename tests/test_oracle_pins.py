"""CPU tests: the oracle against its pins (worked example, closed forms, brute force,
statistics of the normal distribution), its error handling, and a mutation check
that planted mistakes in the oracle are caught by the pins."""
from __future__ import annotations

import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import oracle_pins as pins
import workloads

O = oracle.get()


def test_worked_example_bytes():
    pins.check_worked_example(O)


@pytest.mark.parametrize("C", [16, 1024, 4096, 65536])
def test_exhaustive_words_closed_form(C):
    pins.check_exhaustive(O, C)


def test_brute_force_float_semantics():
    pins.check_brute_force(O, seeds=range(40))


def test_round_trips():
    pins.check_round_trips(O)


def test_codebook_rules():
    pins.check_codebook_rules(O)


def test_no_escape_and_all_escape():
    cb = np.arange(100, 116, dtype=np.uint8)
    # every exponent in the codebook: no escapes, chunk_off all zero
    x = np.array([(e << 7) | (e % 128) for e in range(100, 116)] * 7, np.uint16)
    enc = O.encode(x, cb, 16)
    assert enc["n_escapes"] == 0 and not enc["chunk_off"].any()
    # no exponent in the codebook: every element escapes, positions 0..len-1 per chunk
    y = np.array([((e % 90) << 7) | 0x8000 for e in range(50)], np.uint16)
    enc = O.encode(y, cb, 16)
    assert enc["n_escapes"] == 50
    assert enc["esc_pos"].tolist() == list(range(16)) * 3 + [0, 1]
    assert enc["chunk_off"].tolist() == [0, 16, 32, 48, 50]
    assert not enc["codes"].any()
    assert np.array_equal(O.decode(enc), y)


def test_normal_calibration_statistics():
    """N(0,1) rounded to BF16: exponent field e holds |x| in [2^(e-127), 2^(e-126)) up to
    rounding.  The 16 most likely fields are 114..129 and the mass outside them is
    P(|x| < 2^-13) + P(|x| >= 8); the observed coverage must sit within 5 binomial sigma."""
    wl = workloads.config1()
    cb, cov, _ = O.calibrate(wl.calibration)
    assert sorted(cb.tolist()) == list(range(114, 130))
    p_out = math.erf(2.0 ** -13 / math.sqrt(2)) + math.erfc(8 / math.sqrt(2))
    m = wl.calibration.size
    assert abs((1 - cov) - p_out) < 5 * math.sqrt(p_out / m)
    enc = O.encode(wl.segments[0], cb, 1024)
    assert abs(enc["n_escapes"] / m - p_out) < 5 * math.sqrt(p_out / m)
    assert np.array_equal(O.decode(enc), wl.segments[0])


def test_e5m2_worked_example():
    pins.check_worked_example8(O)


@pytest.mark.parametrize("C", [16, 64, 1024])
def test_e5m2_all_bytes_closed_form(C):
    pins.check_exhaustive8(O, C)


def test_e5m2_brute_force_float_semantics():
    pins.check_brute_force8(O, seeds=range(40))


def test_e5m2_round_trips_and_best_case():
    pins.check_round_trips8(O)


def test_e5m2_rejects_bad_streams():
    g, cal, x = None, None, None
    x = np.arange(256, dtype=np.uint8)
    cb = O.calibrate8(x)[0]
    with pytest.raises(oracle.OracleError):
        O.encode8(x, np.arange(20, 36, dtype=np.uint8), 16)      # exponents above 31
    s = O.serialize8(O.encode8(x, cb, 16))
    b = bytearray(s); b[12] = 0                                  # BF16 flags
    with pytest.raises(oracle.OracleError):
        O.decode_stream8(bytes(b), cb)
    with pytest.raises(oracle.OracleError):
        O.decode_stream(s, cb)                                   # not a BF16 stream
    with pytest.raises(oracle.OracleError):
        O.decode_stream8(s[:-1], cb)


def test_entropy_closed_forms():
    pins.check_entropy(O)


def test_normal_exponent_entropy():
    """Exponent entropy of N(0,1) rounded to BF16, from the normal CDF: field e holds
    |x| in [2^(e-127) (1 - 2^-9), 2^(e-126) (1 - 2^-9)) (round to nearest even of the
    8-bit significand moves the upper 2^-9 of each binade up).  The entropy of the
    config-1 calibration draw must sit within 5 sigma of the analytic value, with sigma
    the standard error of the plug-in estimate, sqrt(Var[log2 p] / m)."""
    def cdf_abs(t):                       # P(|x| < t)
        return math.erf(t / math.sqrt(2))
    lo_edge = 1 - 2.0 ** -9
    p = {}
    for e in range(1, 255):
        a = 2.0 ** (e - 127) * lo_edge
        b = 2.0 ** (e - 126) * lo_edge
        if a > 40:
            break
        q = cdf_abs(b) - cdf_abs(a)
        if q > 0:
            p[e] = q
    p[0] = cdf_abs(2.0 ** -126 * lo_edge)
    total = sum(p.values())
    assert abs(total - 1) < 1e-12
    h_true = -sum(q * math.log2(q) for q in p.values() if q > 0)
    second = sum(q * math.log2(q) ** 2 for q in p.values() if q > 0)
    wl = workloads.config1()
    m = wl.calibration.size
    sigma = math.sqrt((second - h_true ** 2) / m)
    h = O.entropy(O.histogram(wl.calibration))
    assert abs(h - h_true) < 5 * sigma, (h, h_true, sigma)


def test_rejects_bad_arguments_and_streams():
    _, cal, x = pins.worked_example()
    cb, _, _ = O.calibrate(cal)
    for C in (0, 8, 15, 24, 1000, 131072):
        with pytest.raises(oracle.OracleError):
            O.encode(x, cb, C)
    with pytest.raises(oracle.OracleError):
        O.encode(x, np.zeros(16, np.uint8), 16)          # codebook entries must differ
    enc = O.encode(x, cb, 16)
    s = O.serialize(enc)
    bad = []
    b = bytearray(s); b[0] ^= 1; bad.append(bytes(b))             # magic
    b = bytearray(s); b[4] = 2; bad.append(bytes(b))              # version
    b = bytearray(s); b[8] = 24; bad.append(bytes(b))             # chunk size not 2^k
    b = bytearray(s); b[24] = 3; bad.append(bytes(b))             # n_chunks
    b = bytearray(s); b[60] = 1; bad.append(bytes(b))             # reserved
    bad.append(s[:-1])                                            # truncated
    for t in bad:
        with pytest.raises(oracle.OracleError) as ei:
            O.decode_stream(t, cb)
        assert ei.value.code == oracle.BAD_STREAM
    with pytest.raises(oracle.OracleError) as ei:
        O.decode_stream(s, cb[::-1].copy())
    assert ei.value.code == oracle.WRONG_CODEBOOK
    # escape metadata: unsorted positions, position past the chunk, broken offsets
    for mutate in (lambda e: e["esc_pos"].__setitem__(1, 4),
                   lambda e: e["esc_pos"].__setitem__(10, 4),
                   lambda e: e["chunk_off"].__setitem__(1, 12),
                   lambda e: e["chunk_off"].__setitem__(2, 10)):
        e = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in enc.items()}
        mutate(e)
        with pytest.raises(oracle.OracleError):
            O.decode(e)


# ---- mutation check: planted mistakes must fail a pin --------------------------------------

MUTANTS = [
    ("sign bit read from bit 14", "(u >> 15) & 0x1u", "(u >> 14) & 0x1u"),
    ("exponent shifted by 8", "(u >> 7) & 0xFFu", "(u >> 8) & 0xFFu"),
    ("exponent mask 7 bits", "(u >> 7) & 0xFFu", "(u >> 7) & 0x7Fu"),
    ("mantissa mask 6 bits", "return u & 0x7Fu;", "return u & 0x3Fu;"),
    ("ties ranked toward the larger exponent", "hist[e] > hist[best]", "hist[e] >= hist[best]"),
    ("least frequent first", "hist[e] > hist[best]", "hist[e] < hist[best]"),
    ("nibbles swapped in encode", "(code << (4 * (i % 2)))", "(code << (4 * (1 - i % 2)))"),
    ("escape position not chunk-local", "esc_pos[E] = (uint16_t)(i - start);",
     "esc_pos[E] = (uint16_t)(i);"),
    ("escape keeps the exponent's low 7 bits", "esc_exp[E] = (uint8_t)e;",
     "esc_exp[E] = (uint8_t)(e & 0x7Fu);"),
    ("escape nibble set to 15", "code = 0;\n                if", "code = 15;\n                if"),
    ("inclusive chunk offsets", "chunk_off[c] = E;\n        for", "for"),
    ("total missing", "chunk_off[n_chunks] = E;\n    *n_escapes", "chunk_off[n_chunks] = 0;\n    *n_escapes"),
    ("size without the final offset", "8u * (n_chunks + 1u)", "8u * n_chunks"),
    ("big-endian fields", "p[b] = (uint8_t)(v >> (8 * b));", "p[b] = (uint8_t)(v >> (8 * (bytes - 1 - b)));"),
    ("header version 2", "put_le(out + 4, 1, 2);", "put_le(out + 4, 2, 2);"),
    ("sign dropped in sm", "sm[i] = (uint8_t)((bf16_sign(u) << 7) | bf16_mantissa(u));",
     "sm[i] = (uint8_t)(bf16_mantissa(u));"),
    ("decode patch ignores the stored exponent", "bf16_join(bf16_sign(y[i]), esc_exp[j], bf16_mantissa(y[i]))",
     "bf16_join(bf16_sign(y[i]), cb[0], bf16_mantissa(y[i]))"),
    ("decode reads the wrong nibble", "unsigned code = (codes[i / 2] >> (4 * (i % 2))) & 0xFu;",
     "unsigned code = (codes[i / 2] >> (4 * (1 - i % 2))) & 0xFu;"),
    ("entropy in nats", "h -= p * log2(p);", "h -= p * log(p);"),
    ("entropy sign", "h -= p * log2(p);", "h += p * log2(p);"),
    ("entropy of unnormalized counts", "const double p = (double)hist[e] / (double)m;",
     "const double p = (double)hist[e];"),
    ("E5M2 sign from bit 6", "static unsigned e5m2_sign(uint8_t b) { return (b >> 7) & 0x1u; }",
     "static unsigned e5m2_sign(uint8_t b) { return (b >> 6) & 0x1u; }"),
    ("E5M2 exponent shifted by 3", "return (b >> 2) & 0x1Fu;", "return (b >> 3) & 0x1Fu;"),
    ("E5M2 mantissa 1 bit", "static unsigned e5m2_mantissa(uint8_t b) { return b & 0x3u; }",
     "static unsigned e5m2_mantissa(uint8_t b) { return b & 0x1u; }"),
    ("E5M2 field with the sign below", "field3_set(sm3, i, (e5m2_sign(b) << 2) | e5m2_mantissa(b));",
     "field3_set(sm3, i, (e5m2_mantissa(b) << 1) | e5m2_sign(b));"),
    ("E5M2 bit stream big-endian in a byte", "s[bit / 8] = (uint8_t)(s[bit / 8] | (1u << (bit % 8)));",
     "s[bit / 8] = (uint8_t)(s[bit / 8] | (1u << (7 - bit % 8)));"),
    ("E5M2 ranking misses exponent 31", "for (e = 0; e < 32; ++e) {\n            if (taken[e])",
     "for (e = 0; e < 31; ++e) {\n            if (taken[e])"),
    ("E5M2 ties ranked toward the larger exponent", "hist[best] < hist[e]", "hist[best] <= hist[e]"),
    ("E5M2 header flags 0", "szo_header(n, chunk_size, n_escapes, cb, 1, out);",
     "szo_header(n, chunk_size, n_escapes, cb, 0, out);"),
    ("header without n_chunks", "put_le(out + 24, ceil_div(n, chunk_size), 8);", "put_le(out + 24, n, 8);"),
    ("codebook of 15", "for (k = 0; k < 16; ++k)\n        if (cb[k] == e)",
     "for (k = 0; k < 15; ++k)\n        if (cb[k] == e)"),
]


# the same statement in the E5M2 functions (second occurrence in the source)
MUTANTS += [
    ("E5M2 nibbles swapped in encode", "(code << (4 * (i % 2)))", "(code << (4 * (1 - i % 2)))", 1),
    ("E5M2 escape position not chunk-local", "esc_pos[E] = (uint16_t)(i - start);",
     "esc_pos[E] = (uint16_t)(i);", 1),
    ("E5M2 escape nibble set to 15", "code = 0;\n                if", "code = 15;\n                if", 1),
    ("E5M2 inclusive chunk offsets", "chunk_off[c] = E;\n        for", "for", 1),
    ("E5M2 decode reads the wrong nibble", "unsigned code = (codes[i / 2] >> (4 * (i % 2))) & 0xFu;",
     "unsigned code = (codes[i / 2] >> (4 * (1 - i % 2))) & 0xFu;", 1),
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, mutant):
    """Each mutant replaces the nth occurrence (default the first, which is in the BF16
    functions; 1 = the E5M2 copy of the statement) of a statement of the oracle."""
    name, old, new = mutant[:3]
    nth = mutant[3] if len(mutant) > 3 else 0
    src = open(os.path.join(os.path.dirname(oracle.__file__), "splitzip_oracle.c")).read()
    assert src.count(old) > nth, f"mutation site for '{name}' missing"
    at = -1
    for _ in range(nth + 1):
        at = src.index(old, at + 1)
    d = tmp_path / "mutant"
    d.mkdir()
    shutil.copy(os.path.join(os.path.dirname(oracle.__file__), "splitzip_oracle.h"), d)
    (d / "splitzip_oracle.c").write_text(src[:at] + new + src[at + len(old):])
    lib = str(d / "libmutant.so")
    oracle.build(out=lib, src=str(d / "splitzip_oracle.c"))
    mutant = oracle.Oracle(lib)
    with pytest.raises((AssertionError, oracle.OracleError)):
        pins.run_all(mutant)
