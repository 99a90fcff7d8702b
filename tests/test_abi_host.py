"""CPU tests of the C ABI library: it loads, exports every symbol include/splitzip.h
declares, and its host-side logic (sizes, header parsing, argument validation) agrees
with the oracle.  No compute call is made (there is no GPU here)."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

import lossless_bf16_kv_amd as sz
import oracle
import oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


HEADERS = ("splitzip.h", "splitzip_tuning.h")


def declared_functions() -> list:
    text = "".join(open(os.path.join(ROOT, "include", h)).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(splitzip_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"splitzip_calibrate", "splitzip_encode", "splitzip_decode", "splitzip_free",
            "splitzip_release_stream", "splitzip_encode_noalloc", "splitzip_set_small_tiles",
            "splitzip_profile", "splitzip_workspace_bytes"} <= set(names)
    # the tuning and timing calls live in their own header
    main = open(os.path.join(ROOT, "include", "splitzip.h")).read()
    for f in ("splitzip_set_small_tiles", "splitzip_set_stage_tiles", "splitzip_set_private_overflow",
              "splitzip_profile", "splitzip_profile_read", "splitzip_workspace_bytes"):
        assert f + "(" not in main, f
    L = sz.lib()
    for name in names:
        assert hasattr(L, name), name


def test_segment_struct_matches_header():
    # ten 8-byte fields and two 4-byte ones, no padding
    assert ctypes.sizeof(sz.splitzip_segment) == 88
    assert sz.splitzip_segment.book.offset == 80


@pytest.mark.parametrize("n,C,E", [(0, 16, 0), (7, 16, 3), (20, 16, 11), (1 << 32, 1024, 12345),
                                   (65536, 1024, 61440), (1000003, 4096, 77)])
def test_sizes_match_oracle(n, C, E):
    o = oracle.get()
    assert sz.splitzip_compressed_bytes(n, C, E) == o.compressed_bytes(n, C, E)
    assert sz.splitzip_chunk_count(n, C) == -(-n // C)


@pytest.mark.parametrize("n,C,E", [(0, 16, 0), (7, 16, 3), (20, 16, 9), (1 << 32, 1024, 12345),
                                   (256, 16, 128), (1000003, 4096, 77)])
def test_e5m2_sizes_match_oracle(n, C, E):
    assert sz.splitzip_e5m2_compressed_bytes(n, C, E) == oracle.get().compressed_bytes8(n, C, E)


def test_bad_chunk_sizes_have_no_size():
    for C in (0, 8, 24, 131072):
        assert sz.splitzip_compressed_bytes(100, C, 0) == 0
        assert sz.splitzip_e5m2_compressed_bytes(100, C, 0) == 0
        assert sz.splitzip_chunk_count(100, C) == 0


def test_read_header_of_oracle_streams():
    o = oracle.get()
    g, cal, x = pins.worked_example()
    cb, _, _ = o.calibrate(cal)
    for n in (0, 7, 20):
        s = o.serialize(o.encode(x[:n], cb, 16))
        h = sz.splitzip_read_header(s)
        assert h == {"n": n, "chunk_size": 16, "n_escapes": o.stream_info(s)["n_escapes"],
                     "codebook": bytes(cb), "elem": sz.ELEM_BF16}


def test_read_header_of_oracle_e5m2_streams():
    o = oracle.get()
    x = np.random.default_rng(3).integers(0, 256, 300).astype(np.uint8)
    cb = o.calibrate8(x[:100])[0]
    for n, C in ((0, 16), (7, 16), (300, 64)):
        e = o.encode8(x[:n], cb, C)
        s = o.serialize8(e)
        assert sz.splitzip_read_header(s) == {"n": n, "chunk_size": C, "n_escapes": e["n_escapes"],
                                              "codebook": bytes(cb), "elem": sz.ELEM_E5M2}
    # an E5M2 header whose codebook holds a value above 31 is malformed
    b = bytearray(o.serialize8(o.encode8(x, cb, 64)))
    b[40] = 32
    with pytest.raises(sz.SplitZipError) as ei:
        sz.splitzip_read_header(bytes(b))
    assert ei.value.status == sz.E_FORMAT


def test_read_header_rejects_malformed():
    o = oracle.get()
    _, cal, x = pins.worked_example()
    cb, _, _ = o.calibrate(cal)
    s = o.serialize(o.encode(x, cb, 16))
    for i, val in ((0, 0x54), (4, 2), (6, 65), (8, 24), (12, 1), (12, 2), (24, 9), (60, 1)):
        b = bytearray(s)
        b[i] = val
        with pytest.raises(sz.SplitZipError) as ei:
            sz.splitzip_read_header(bytes(b))
        assert ei.value.status == sz.E_FORMAT
    with pytest.raises(sz.SplitZipError):
        sz.splitzip_read_header(s[:-1])
    with pytest.raises(sz.SplitZipError):
        sz.splitzip_read_header(s[:10])


def test_argument_validation_before_any_device_call():
    L = sz.lib()
    h = ctypes.c_void_p()
    cov = ctypes.c_double()
    for C in (0, 8, 1000, 1 << 17):
        assert L.splitzip_calibrate(None, 0, C, None, ctypes.byref(h), ctypes.byref(cov), None) == sz.E_INVALID
    # misaligned calibration pointer
    assert L.splitzip_calibrate(ctypes.c_void_p(0x1002), 8, 1024, None, ctypes.byref(h),
                                ctypes.byref(cov), None) == sz.E_INVALID
    assert b"aligned" in L.splitzip_last_error()
    # no codec
    segs = (sz.splitzip_segment * 1)()
    assert L.splitzip_encode(None, 1, segs, None) == sz.E_INVALID
    assert L.splitzip_decode(None, 1, segs, None, None) == sz.E_INVALID
    res = ctypes.c_uint64(0)
    assert L.splitzip_encode_noalloc(None, 1, segs, None, ctypes.byref(res)) == sz.E_INVALID
    assert L.splitzip_encode_noalloc(None, 1, segs, None, None) == sz.E_INVALID
    assert b"d_result" in L.splitzip_last_error()
    # duplicate codebook entries
    cb = (ctypes.c_uint8 * 16)(*([5] * 16))
    assert L.splitzip_codec_from_codebook(cb, 1024, ctypes.byref(h)) == sz.E_INVALID
    L.splitzip_free(None)   # no-op
    assert sz.lib().splitzip_status_string(6) == b"escape capacity exceeded"


def test_codebook_and_statistics_validation_before_any_device_call():
    L = sz.lib()
    h = ctypes.c_void_p()
    P = ctypes.c_void_p * 2
    N = ctypes.c_uint64 * 2
    ok, bad = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008)
    for k in (0, sz.MAX_BOOKS + 1):
        assert L.splitzip_calibrate_books(k, P(ok, ok), N(8, 8), 1024, None, ctypes.byref(h),
                                          None, None) == sz.E_INVALID
    assert L.splitzip_calibrate_books(2, P(ok, bad), N(8, 8), 1024, None, ctypes.byref(h),
                                      None, None) == sz.E_INVALID
    assert b"tensor 1" in L.splitzip_last_error()
    assert L.splitzip_calibrate_books(2, P(ok, ok), N(8, 8), 48, None, ctypes.byref(h),
                                      None, None) == sz.E_INVALID
    hist = (ctypes.c_uint64 * 512)()
    assert L.splitzip_histogram(0, P(ok, ok), N(8, 8), None, hist) == sz.E_INVALID
    assert L.splitzip_histogram(2, P(bad, ok), N(8, 8), None, hist) == sz.E_INVALID
    books = list(range(16)) + list(range(16, 32)) + [7] * 16
    cbs = (ctypes.c_uint8 * 48)(*books)
    assert L.splitzip_codec_from_codebooks(3, cbs, 1024, ctypes.byref(h)) == sz.E_INVALID
    assert b"codebook 2" in L.splitzip_last_error()
    assert L.splitzip_codec_from_codebooks(0, cbs, 1024, ctypes.byref(h)) == sz.E_INVALID
    out = (ctypes.c_uint8 * 64)()
    assert L.splitzip_write_header(None, 0, 10, 0, out) == sz.E_INVALID
    assert L.splitzip_check_header(None, out, 64, None) == sz.E_INVALID
    assert L.splitzip_exponent_stats(None, None, None, None, None) == sz.E_INVALID


def test_e5m2_validation_before_any_device_call():
    L = sz.lib()
    h = ctypes.c_void_p()
    cov = ctypes.c_double()
    for C in (0, 8, 1000):
        assert L.splitzip_calibrate_e5m2(None, 0, C, None, ctypes.byref(h), ctypes.byref(cov), None) == sz.E_INVALID
    assert L.splitzip_calibrate_e5m2(ctypes.c_void_p(0x1004), 8, 1024, None, ctypes.byref(h),
                                     ctypes.byref(cov), None) == sz.E_INVALID
    P = ctypes.c_void_p * 1
    N = ctypes.c_uint64 * 1
    assert L.splitzip_calibrate_books_e5m2(0, P(0x1000), N(8), 1024, None, ctypes.byref(h),
                                           None, None) == sz.E_INVALID
    hist = (ctypes.c_uint64 * 32)()
    assert L.splitzip_histogram_e5m2(1, P(0x1001), N(8), None, hist) == sz.E_INVALID
    # codebook values must be 16 distinct 5-bit exponents
    cb = (ctypes.c_uint8 * 16)(*range(16, 32))
    cb[0] = 32
    assert L.splitzip_codec_from_codebooks_e5m2(1, cb, 1024, ctypes.byref(h)) == sz.E_INVALID
    assert b"5-bit" in L.splitzip_last_error()
    assert L.splitzip_codec_element(None, None) == sz.E_INVALID

def _stats_agree(o, hist):
    st = sz.exponent_stats(hist)
    h = np.asarray(hist, np.uint64)
    want_h = o.entropy(h)
    assert abs(st["entropy_bits"] - want_h) <= 1e-12 * max(1.0, want_h)
    assert st["codebook"] == bytes(o.codebook(h))
    m = int(h.sum())
    assert st["coverage"] == o.coverage(h, o.codebook(h), m)
    assert st["distinct"] == int(np.count_nonzero(h))


def test_exponent_stats_match_oracle():
    """The library's host statistics of a histogram (entropy, codebook, coverage, distinct
    values) against the oracle's on the same histograms."""
    o = oracle.get()
    _stats_agree(o, [0] * 256)
    _stats_agree(o, o.histogram(np.arange(65536, dtype=np.uint16)).tolist())
    g, cal, x = pins.worked_example()
    _stats_agree(o, o.histogram(cal).tolist())
    rng = np.random.default_rng(5)
    for _ in range(30):
        h = rng.integers(0, 1 << 40, 256, dtype=np.uint64)
        h[rng.random(256) < rng.random()] = 0
        _stats_agree(o, h.tolist())
    st = sz.exponent_stats(o.histogram(np.arange(65536, dtype=np.uint16)).tolist())
    assert st["entropy_bits"] == 8.0 and st["coverage"] == 1 / 16 and st["distinct"] == 256


def test_e5m2_exponent_stats_match_oracle():
    """A 32-bin E5M2 histogram (padded by the binding): the codebook the library ranks
    equals the oracle's E5M2 codebook, coverage and distinct count too."""
    o = oracle.get()
    rng = np.random.default_rng(9)
    for _ in range(30):
        h = rng.integers(0, 1 << 30, 32, dtype=np.uint64)
        h[rng.random(32) < rng.random()] = 0
        st = sz.exponent_stats(h.tolist())
        cb = o.codebook8(h)
        assert st["codebook"] == bytes(cb)
        assert st["coverage"] == o.coverage8(h, cb, int(h.sum()))
        assert st["distinct"] == int(np.count_nonzero(h))
        assert max(st["codebook"]) < 32


def test_no_cpu_fallback():
    # the product path refuses to run without a GPU instead of computing on the CPU
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    with pytest.raises(sz.SplitZipError):
        sz.Codec("cuda", 1024)


C_CONSUMER = r"""
#include <splitzip.h>
#include <splitzip_tuning.h>
#include <stdio.h>
#include <string.h>

int main(void)
{
    /* host helpers only: sizes, a header round trip through the parser, status strings */
    if (splitzip_compressed_bytes(20, 16, 11) != 151) return 1;
    if (splitzip_e5m2_compressed_bytes(20, 16, 9) != 64 + 8 + 10 + 24 + 27) return 2;
    if (splitzip_chunk_count(1u << 20, 1024) != 1024) return 3;
    uint8_t h[SPLITZIP_HEADER_BYTES + 8 + 4 + 8 * 2] = {0};
    memcpy(h, "SZB1", 4);
    h[4] = 1; h[6] = SPLITZIP_HEADER_BYTES; h[8] = 16; h[12] = SPLITZIP_ELEM_BF16;
    h[16] = 8; h[24] = 1;
    for (int k = 0; k < 16; ++k) h[40 + k] = (uint8_t)(100 + k);
    uint64_t n = 0, e = 1;
    uint32_t c = 0, elem = 7;
    uint8_t cb[16];
    if (splitzip_read_header(h, sizeof h, &n, &c, &e, cb, &elem) != SPLITZIP_OK) return 4;
    if (n != 8 || c != 16 || e != 0 || elem != SPLITZIP_ELEM_BF16 || cb[15] != 115) return 5;
    if (splitzip_read_header(h, sizeof h - 1, 0, 0, 0, 0, 0) != SPLITZIP_E_FORMAT) return 6;
    if (strcmp(splitzip_status_string(SPLITZIP_E_CAPACITY), "escape capacity exceeded") != 0) return 7;
    splitzip_free(NULL);
    /* calls without a codec fail cleanly, before any device work */
    uint64_t ws = 1;
    if (splitzip_release_stream(NULL, NULL) != SPLITZIP_E_INVALID) return 8;
    if (splitzip_workspace_bytes(NULL, NULL, &ws) != SPLITZIP_E_INVALID) return 9;
    if (splitzip_set_small_tiles(NULL, 0) != SPLITZIP_E_INVALID) return 10;
    if (splitzip_set_onepass_tiles(NULL, SPLITZIP_ONEPASS_TILES) != SPLITZIP_E_INVALID) return 11;
    if (splitzip_set_onepass_launches(NULL, NULL, 0) != SPLITZIP_E_INVALID) return 12;
    printf("ok\n");
    return 0;
}
"""


def test_header_compiles_as_c_and_links(tmp_path):
    """A plain C99 program includes include/splitzip.h and splitzip_tuning.h, links against
    the library and uses its host helpers (no device call)."""
    import subprocess
    src = tmp_path / "consumer.c"
    src.write_text(C_CONSUMER)
    exe = tmp_path / "consumer"
    lib_dir = os.path.dirname(sz.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
           "-o", str(exe), "-L", lib_dir, "-lsplitzip", f"-Wl,-rpath,{lib_dir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)


# ---- header parsing of untrusted bytes ------------------------------------------------

def exact_stream_bytes(elem: int, n: int, C: int, E: int) -> int:
    """The canonical size in unbounded integers (no wrap-around)."""
    sm = -(-3 * n // 8) if elem == 1 else n
    return 64 + sm + -(-n // 2) + 8 * (-(-n // C) + 1) + 3 * E


def header(n: int, C: int, E: int, flags: int = 0, cb: bytes = bytes(range(16))) -> bytes:
    import struct
    return (b"SZB1" + struct.pack("<HHII", 1, 64, C, flags) +
            struct.pack("<QQQ", n % (1 << 64), (-(-n // C)) % (1 << 64), E % (1 << 64)) + cb + bytes(8))


def test_read_header_rejects_sizes_that_wrap_around():
    """n near 2^64 whose size sum wraps to a small buffer length must not parse."""
    C = 65536
    lo, hi = 0, 1 << 64
    while hi - lo > 1:                        # smallest n whose true size reaches 2^64
        mid = (lo + hi) // 2
        lo, hi = (lo, mid) if exact_stream_bytes(0, mid, C, 0) >= 1 << 64 else (mid, hi)
    n = hi + 700
    wrapped = exact_stream_bytes(0, n, C, 0) % (1 << 64)
    assert 64 < wrapped < 4096
    buf = header(n, C, 0) + bytes(wrapped - 64)
    with pytest.raises(sz.SplitZipError) as ei:
        sz.splitzip_read_header(buf)
    assert ei.value.status == sz.E_FORMAT
    assert sz.splitzip_compressed_bytes(1 << 38, 1024, 0) == 0
    assert sz.splitzip_compressed_bytes((1 << 38) - 16, 1024, 1 << 38) == 0
    assert sz.splitzip_compressed_bytes((1 << 38) - 16, 1024, 5) == exact_stream_bytes(0, (1 << 38) - 16, 1024, 5)


def test_read_header_fuzz():
    """Random headers (valid ones with fields and lengths perturbed, huge n and E included):
    every header the parser accepts is self-consistent in exact arithmetic."""
    from hypothesis import given, settings, strategies as st

    big = st.one_of(st.integers(0, 1 << 20), st.integers(0, (1 << 64) - 1),
                    st.integers((1 << 38) - 4, (1 << 38) + 4))

    @settings(max_examples=400, deadline=None, derandomize=True)
    @given(n=big, e=big, c_log=st.integers(3, 17), flags=st.integers(0, 2),
           extra=st.integers(-3, 3), flip=st.one_of(st.none(), st.integers(0, 63)))
    def check(n, e, c_log, flags, extra, flip):
        C = 1 << c_log
        hdr = bytearray(header(n, C, e, flags, bytes(range(16))))
        if flip is not None:
            hdr[flip] ^= 0x01
        length = max(0, min(exact_stream_bytes(flags, n % (1 << 64), C, e % (1 << 64)) + extra, 1 << 22))
        buf = bytes(hdr) + bytes(max(0, length - 64))
        try:
            r = sz.splitzip_read_header(buf[:length] if length >= 64 else buf[:length])
        except sz.SplitZipError as err:
            assert err.status in (sz.E_FORMAT, sz.E_INVALID)
            return
        assert r["n"] < 1 << 38 and r["n_escapes"] <= r["n"]
        assert r["elem"] in (0, 1) and 16 <= r["chunk_size"] <= 65536
        assert exact_stream_bytes(r["elem"], r["n"], r["chunk_size"], r["n_escapes"]) == length

    check()


def test_python_constants_match_the_headers():
    import re
    text = open(os.path.join(ROOT, "include", "splitzip.h")).read() + \
        open(os.path.join(ROOT, "include", "splitzip_tuning.h")).read()

    def define(name):
        m = re.search(r"#define\s+" + name + r"\s+\(?([0-9a-fx]+)(?:ull|u)?(?:\s*<<\s*(\d+))?\)?", text)
        assert m, name
        v = int(m.group(1), 0)
        return v << int(m.group(2)) if m.group(2) else v
    assert sz.SMALL_TILES == define("SPLITZIP_SMALL_TILES")
    assert sz.STAGE_TILES == define("SPLITZIP_STAGE_TILES")
    assert sz.ONEPASS_TILES == define("SPLITZIP_ONEPASS_TILES")
    assert sz.PRIVATE_OVERFLOW_BYTES == define("SPLITZIP_PRIVATE_OVERFLOW_BYTES")
    assert sz.NOALLOC_SCRATCH_BYTES == define("SPLITZIP_NOALLOC_SCRATCH_BYTES")
    assert sz.NOALLOC_MAX_SEGMENTS == define("SPLITZIP_NOALLOC_MAX_SEGMENTS")
    assert len(sz.KERNELS) == define("SPLITZIP_KERNELS")
