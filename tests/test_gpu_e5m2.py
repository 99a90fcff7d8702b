"""GPU parity of the FP8 E5M2 codec (the same calls through the C ABI, E5M2 codec)
against the CPU oracle's E5M2 functions.

Streams must equal the oracle's byte for byte (3-bit field stream, codes, chunk offsets,
escapes, canonical serialization), decode must return the input bit for bit, and
calibration must give the oracle's 32-bin histogram, codebook and coverage.  Sizes span
several pack tiles (32768 elements) and decode tiles (16384) with ragged tails, every
chunk-size regime (chunks that start inside a 32-element lane group at C = 16, chunks
larger than a decode tile), empty and tiny segments, several codebooks, packed streams,
corrupt metadata, and the 4.3 GB E5M2 long-prefill KV at full size."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import lossless_bf16_kv_amd as sz
import oracle
import oracle_pins as pins
import stream_check
import workloads
from conftest import hex_bytes, ints, load_golden

pytestmark = pytest.mark.gpu

O = oracle.get()
DEV = torch.device("cuda:0")


def dev8(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.array(b, np.uint8, copy=True)).to(DEV)


def host(t: torch.Tensor, dtype) -> np.ndarray:
    if t.dtype == torch.float8_e5m2:
        t = t.view(torch.uint8)
    return t.cpu().numpy().view(dtype)


def codec_for(cal: np.ndarray, C: int) -> sz.Codec:
    c = sz.Codec(DEV, C, elem="e5m2")
    c.calibrate(dev8(cal))
    return c


def assert_same_stream(codec: sz.Codec, enc: sz.Encoded, x: np.ndarray):
    cb = np.frombuffer(enc.codebook, np.uint8)
    ref = O.encode8(x, cb, codec.chunk_size)
    assert enc.n_escapes == ref["n_escapes"]
    assert enc.compressed_bytes == ref["compressed_bytes"]
    assert np.array_equal(host(enc.sm, np.uint8), ref["sm3"])
    assert np.array_equal(host(enc.codes, np.uint8), ref["codes"])
    assert np.array_equal(host(enc.chunk_off, np.uint64), ref["chunk_off"])
    assert np.array_equal(host(enc.esc_pos, np.uint16), ref["esc_pos"])
    assert np.array_equal(host(enc.esc_exp, np.uint8), ref["esc_exp"])
    assert enc.to_bytes(codec) == O.serialize8(ref)
    return ref


def test_worked_example():
    g = load_golden("worked_example_e5m2_c16.txt")
    C = int(g["chunk_size"])
    cal = np.frombuffer(hex_bytes(g["calibration_u8"]), np.uint8)
    codec = sz.Codec(DEV, C, elem="e5m2")
    cov = codec.calibrate(dev8(cal))
    assert codec.codebook == hex_bytes(g["codebook"])
    num, den = (int(t) for t in g["calibration_coverage"].split("/"))
    assert cov == num / den
    x = np.frombuffer(hex_bytes(g["input_u8"]), np.uint8)
    enc = codec.encode(dev8(x))
    assert bytes(host(enc.sm, np.uint8)) == hex_bytes(g["sm3"])
    assert bytes(host(enc.codes, np.uint8)) == hex_bytes(g["codes"])
    assert host(enc.chunk_off, np.uint64).tolist() == ints(g["chunk_off"])
    assert host(enc.esc_pos, np.uint16).tolist() == ints(g["esc_pos"])
    assert host(enc.esc_exp, np.uint8).tolist() == ints(g["esc_exp"])
    assert enc.compressed_bytes == int(g["compressed_bytes"])
    assert enc.to_bytes(codec)[:64] == hex_bytes(g["header"])
    y = codec.decode(enc)
    assert y.dtype == torch.uint8 and np.array_equal(host(y, np.uint8), x)   # the input's dtype
    y8 = codec.decode(codec.encode(dev8(x).view(torch.float8_e5m2)))
    assert y8.dtype == torch.float8_e5m2 and np.array_equal(host(y8, np.uint8), x)
    e7 = codec.encode(dev8(x[:7]))
    assert bytes(host(e7.sm, np.uint8)) == hex_bytes(g["prefix7_sm3"])
    assert bytes(host(e7.codes, np.uint8)) == hex_bytes(g["prefix7_codes"])
    assert e7.compressed_bytes == int(g["prefix7_compressed_bytes"])
    assert np.array_equal(host(codec.decode(e7), np.uint8), x[:7])
    e0 = codec.encode(dev8(x[:0]))
    assert e0.compressed_bytes == int(g["empty_compressed_bytes"])


@pytest.mark.parametrize("C", [16, 64, 1024, 65536])
def test_every_byte_value(C):
    """All 256 bytes, repeated 300 times: every exponent occurs equally often, so the
    codebook is 0..15 and half the elements escape."""
    x = np.tile(np.arange(256, dtype=np.uint8), 300)
    codec = codec_for(x, C)
    assert codec.codebook == bytes(range(16)) and codec.coverage == 0.5
    enc = codec.encode(dev8(x))
    ref = assert_same_stream(codec, enc, x)
    assert ref["n_escapes"] == x.size // 2
    assert np.array_equal(host(codec.decode(enc), np.uint8), x)


@pytest.mark.parametrize("n", [1, 5, 16, 17, 4099, 1000003])
def test_calibration_matches_oracle(n):
    x = workloads.e5m2_mixed(n, seed=n, wide_fraction=0.3)
    codec = codec_for(x, 1024)
    cb, cov, h = O.calibrate8(x)
    assert codec.histogram == h.tolist()
    assert codec.codebook == bytes(cb)
    assert codec.coverage == cov
    assert sz.histograms([dev8(x)], elem="e5m2")[0] == h.tolist()


FUZZ = [(n, C, gen) for n, C, gen in [
    (1, 16, "random"), (9, 16, "mixed"), (31, 16, "random"), (33, 32, "mixed"),
    (16383, 1024, "mixed"), (16384, 1024, "normal"), (16385, 16, "random"),
    (32767, 64, "mixed"), (32768 + 5, 16, "mixed"), (3 * 32768 + 13, 32, "random"),
    (100003, 1024, "random"), (100003, 4096, "mixed"), (196613, 16384, "mixed"),
    (196613, 32768, "random"), (196613, 65536, "mixed"), ((1 << 20) + 77, 1024, "mixed"),
    ((1 << 20) + 77, 16, "random"),
]]


@pytest.mark.parametrize("n,C,gen", FUZZ)
def test_fuzz_stream_parity(n, C, gen):
    make = {"random": workloads.e5m2_random, "mixed": workloads.e5m2_mixed,
            "normal": workloads.e5m2_normal}[gen]
    x = make(n, 19 * n + C)
    codec = codec_for(workloads.e5m2_normal(50000, 3), C)
    enc = codec.encode(dev8(x))
    ref = assert_same_stream(codec, enc, x)
    assert np.array_equal(host(codec.decode(enc), np.uint8), x)
    y = codec.decode_bytes(O.serialize8(ref))
    assert np.array_equal(host(y, np.uint8), x)


def test_batch_with_empty_and_tiny_segments():
    sizes = [0, 1, 7, 16384, 32769, 0, 100, 3 * 32768 + 5]
    xs = [workloads.e5m2_mixed(n, 100 + i, wide_fraction=0.3) for i, n in enumerate(sizes)]
    codec = codec_for(workloads.e5m2_normal(20000, 4), 16)
    encs = codec.encode_batch([dev8(x) for x in xs])
    for x, e in zip(xs, encs):
        assert_same_stream(codec, e, x)
    for x, y in zip(xs, codec.decode_batch(encs)):
        assert np.array_equal(host(y, np.uint8), x)


@pytest.mark.parametrize("C", [64, 1024, 65536])
def test_several_codebooks(C):
    """Three books calibrated on differently scaled draws; segments coded with their own
    book and with another scale's book, one encode and one decode launch."""
    cals = [workloads.e5m2_normal(40000, 60 + k, sigma=s) for k, s in enumerate((1.0, 300.0, 0.01))]
    codec = sz.Codec(DEV, C, elem="e5m2")
    covs = codec.calibrate_books([dev8(c) for c in cals])
    for cal, book, cov in zip(cals, codec.books, covs):
        cb, ocov, _ = O.calibrate8(cal)
        assert book == bytes(cb) and cov == ocov
    xs = [workloads.e5m2_normal(n, 70 + i, sigma=s) for i, (n, s) in
          enumerate([(50000, 1.0), (70001, 300.0), (3, 0.01), (40000, 300.0), (0, 1.0)])]
    books = [0, 1, 2, 0, 1]
    encs = codec.encode_batch([dev8(x) for x in xs], books=books)
    for x, e in zip(xs, encs):
        assert_same_stream(codec, e, x)
    for x, y in zip(xs, codec.decode_batch(encs)):
        assert np.array_equal(host(y, np.uint8), x)


def test_capacity_retry_gives_identical_stream():
    x = workloads.e5m2_random(50000, 9)
    codec = codec_for(workloads.e5m2_normal(20000, 5), 1024)
    enc = codec.empty_encoded(x.size, escape_capacity=10)
    assert codec.encode_into([dev8(x)], [enc]) == sz.E_CAPACITY
    ref = O.encode8(x, np.frombuffer(codec.codebook, np.uint8), 1024)
    assert enc.n_escapes == ref["n_escapes"]
    assert_same_stream(codec, codec.encode(dev8(x)), x)


@pytest.mark.parametrize("stage_tiles", [sz.STAGE_TILES, 0])
def test_decode_flags_corrupt_metadata_without_faulting(stage_tiles):
    """Both decode builds flag corrupt metadata without a fault (0: the large-call build)."""
    x = workloads.e5m2_mixed(4 * 16384, 12, wide_fraction=0.2)
    codec = codec_for(workloads.e5m2_normal(20000, 7), 1024)
    codec.set_stage_tiles(stage_tiles)
    enc = codec.encode(dev8(x))
    assert enc.n_escapes > 100
    y = torch.empty_like(codec.decode(enc))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    assert int(enc.chunk_off[9]) > int(enc.chunk_off[3])
    for field, idx, val in (("chunk_off", 3, enc.n_escapes + 1000), ("esc_pos_buf", 5, 4000),
                            ("esc_exp_buf", 7, 40), ("chunk_off", 2, int(enc.chunk_off[9]))):
        bad = dataclasses.replace(enc, chunk_off=enc.chunk_off.clone(), esc_pos_buf=enc.esc_pos_buf.clone(),
                                  esc_exp_buf=enc.esc_exp_buf.clone())
        getattr(bad, field)[idx] = val
        err.zero_()
        codec.decode_into([bad], [y], d_error=err.data_ptr())
        torch.cuda.synchronize()
        assert int(err.item()) != 0, field
    # every escape in the last chunk: more than that chunk's elements
    bad = dataclasses.replace(enc, chunk_off=enc.chunk_off.clone())
    bad.chunk_off[:-1] = 0
    assert enc.n_escapes > 1024
    err.zero_()
    codec.decode_into([bad], [y], d_error=err.data_ptr())
    torch.cuda.synchronize()
    assert int(err.item()) & 2
    err.zero_()
    codec.decode_into([enc], [y], d_error=err.data_ptr())
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and np.array_equal(host(y, np.uint8), x)
    # more escapes than the last tile has elements
    x2 = workloads.e5m2_mixed(4 * 16384, 13, wide_fraction=0.7)
    enc2 = codec.encode(dev8(x2))
    assert enc2.n_escapes > 16384
    bad = dataclasses.replace(enc2, chunk_off=enc2.chunk_off.clone())
    bad.chunk_off[:-1] = 0
    err.zero_()
    codec.decode_into([bad], [torch.empty_like(y)], d_error=err.data_ptr())
    torch.cuda.synchronize()
    assert int(err.item()) & 2


def test_element_type_and_codebook_checks():
    x = workloads.e5m2_normal(5000, 1)
    a = codec_for(workloads.e5m2_normal(5000, 2), 1024)
    enc = a.encode(dev8(x))
    s = enc.to_bytes(a)
    assert sz.splitzip_read_header(s)["elem"] == sz.ELEM_E5M2
    # a BF16 codec with the same codebook bytes refuses the E5M2 stream
    b = sz.Codec.from_codebook(a.codebook, 1024, DEV)
    with pytest.raises(sz.SplitZipError) as ei:
        b.decode_bytes(s)
    assert ei.value.status == sz.E_CODEBOOK
    # an E5M2 codec rebuilt from the header decodes it
    c = sz.Codec.from_codebook(sz.splitzip_read_header(s)["codebook"], 1024, DEV, elem="e5m2")
    assert np.array_equal(host(c.decode_bytes(s), np.uint8), x)
    assert sz.splitzip_codec_element(c.handle) == sz.ELEM_E5M2


# ---- packed streams ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,C", [(0, 1024), (128, 16), (32768 * 3 + 128 * 7, 1024), ((1 << 20) + 256, 65536)])
def test_packed_stream_equals_oracle_serialization(n, C):
    x = workloads.e5m2_mixed(n, 500 + n, wide_fraction=0.05)
    codec = codec_for(workloads.e5m2_normal(30000, 13), C)
    p = codec.encode_packed(dev8(x))
    ref = O.encode8(x, np.frombuffer(codec.codebook, np.uint8), C)
    assert p.n_escapes == ref["n_escapes"]
    assert p.to_bytes() == O.serialize8(ref)
    assert np.array_equal(host(codec.decode_packed(p), np.uint8), x)
    # an oracle-written stream decodes through the packed path
    buf = sz.packed_buffer(len(O.serialize8(ref)), DEV)
    buf.copy_(torch.from_numpy(np.frombuffer(O.serialize8(ref), np.uint8).copy()))
    y = codec.decode_packed(buf, n=n)
    assert np.array_equal(host(y, np.uint8), x)


def test_packed_header_checks():
    n = 4096
    x = workloads.e5m2_mixed(n, 3)
    codec = codec_for(workloads.e5m2_normal(30000, 14), 1024)
    p = codec.encode_packed(dev8(x))
    good = p.to_bytes()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    for off, val in ((12, 0), (40, 33), (16, 0x80), (0, 0x41)):
        b = bytearray(good)
        b[off] = val
        buf = sz.packed_buffer(len(b), DEV)
        buf.copy_(torch.from_numpy(np.frombuffer(bytes(b), np.uint8).copy()))
        err.zero_()
        out = codec.decode_packed_batch([buf], [n], d_error=err.data_ptr())[0]
        torch.cuda.synchronize()
        assert int(err.item()) & 16, off
    with pytest.raises(sz.SplitZipError):
        codec.encode_packed(dev8(x[:100]))         # not a multiple of 128


# ---- full size: the long-prefill KV cast to E5M2 (2^32 bytes) ---------------------------------

@pytest.fixture(scope="module")
def kv8():
    return workloads.config3_e5m2()


def test_long_prefill_e5m2_full_size(kv8):
    x = kv8.segments[0]
    assert x.size == 1 << 32
    C = kv8.chunk_size
    xd = dev8(x)
    codec = codec_for(kv8.calibration, C)
    cb, cov, _ = O.calibrate8(kv8.calibration)
    assert codec.codebook == bytes(cb) and codec.coverage == cov
    enc = codec.encode(xd)
    # E from the oracle's exact histogram of the whole input; offsets and size
    h = O.histogram8(x)
    E = int(x.size - sum(int(h[e]) for e in cb))
    assert enc.n_escapes == E and enc.compressed_bytes == O.compressed_bytes8(x.size, C, E)
    off = enc.chunk_off
    assert int(off[0]) == 0 and int(off[-1]) == E and bool((off[1:] >= off[:-1]).all())
    # every byte of every section against the oracle, window by window
    stream_check.check_cases([stream_check.case_from_encoded("config3 e5m2", enc, x,
                                                             stream_check.ELEM_E5M2)])
    y = codec.decode(enc)
    assert torch.equal(y.view(torch.uint8), xd)


# ---- the escape-stress input and the ragged batch, cast to E5M2 --------------------------------

def test_escape_stress_e5m2():
    """Config 4 (N(0,1) x 2^k per 4096-element block, 1 % specials) cast to E5M2: a large share
    of escapes, every tile over its slot; the whole stream against the oracle."""
    wl = workloads.cast_e5m2(workloads.config4())
    x = wl.segments[0]
    codec = codec_for(wl.calibration, 1024)
    enc = codec.encode(dev8(x))
    ref = assert_same_stream(codec, enc, x)
    assert ref["n_escapes"] > 0.05 * x.size
    assert np.array_equal(host(codec.decode(enc), np.uint8), x)


def test_ragged_batch_e5m2():
    """Config 5 (512 K/V segments of 256 requests, one launch) cast to E5M2: every stream whole
    against the oracle, E and offsets of every segment from the oracle's histograms, and
    round trips."""
    wl = workloads.cast_e5m2(workloads.config5())
    assert len(wl.segments) == 512
    codec = codec_for(wl.calibration, 1024)
    cb = np.frombuffer(codec.codebook, np.uint8)
    xds = [dev8(s) for s in wl.segments]
    encs = codec.encode_batch(xds)
    stream_check.check_cases([stream_check.case_from_encoded(f"segment {i}", e, x, stream_check.ELEM_E5M2)
                              for i, (x, e) in enumerate(zip(wl.segments, encs))])
    for x, e in zip(wl.segments, encs):
        h = O.histogram8(x)
        E = int(x.size - sum(int(h[v]) for v in cb))
        assert e.n_escapes == E and e.compressed_bytes == O.compressed_bytes8(x.size, 1024, E)
        off = e.chunk_off
        assert int(off[0]) == 0 and int(off[-1]) == E and bool((off[1:] >= off[:-1]).all())
    for xd, y in zip(xds, codec.decode_batch(encs)):
        assert torch.equal(y, xd)


def test_async_and_prepared_e5m2():
    """Non-blocking encode and prepared batches (sections and packed streams) on E5M2."""
    xs_np = [workloads.e5m2_mixed(n, 400 + n, wide_fraction=0.05) for n in (3 * 32768 + 11, 70000, 0, 5)]
    codec = codec_for(workloads.e5m2_normal(30000, 15), 1024)
    xs = [dev8(x) for x in xs_np]
    ref = codec.encode_batch(xs)
    encs = [codec.empty_encoded(e.n, escape_capacity=max(e.n_escapes, 1)) for e in ref]
    result = torch.zeros(1 + len(xs), dtype=torch.int64, device=DEV)
    codec.encode_into_async(xs, encs, result)
    torch.cuda.synchronize()
    assert codec.finish_async(encs, result) == sz.OK
    for x, e in zip(xs_np, encs):
        assert_same_stream(codec, e, x)
    ys = [torch.empty_like(x) for x in xs]
    batch = codec.prepare(xs, encs, ys)
    for _ in range(3):
        batch.encode_async(result)
        batch.decode()
    torch.cuda.synchronize()
    assert batch.finish(result) == sz.OK
    for x, y in zip(xs_np, ys):
        assert np.array_equal(host(y, np.uint8), x)
    # packed streams (sizes a multiple of 128)
    xs8 = [dev8(workloads.e5m2_mixed(n, 500 + n)) for n in (128 * 513, 32768 * 2)]
    packed = codec.encode_packed_batch(xs8)
    outs = [torch.empty_like(x) for x in xs8]
    pb = codec.prepare_packed(xs8, packed, outs)
    res = torch.zeros(1 + len(xs8), dtype=torch.int64, device=DEV)
    for _ in range(2):
        pb.encode_async(res)
        pb.decode()
    torch.cuda.synchronize()
    assert pb.finish(res) == sz.OK
    for x, y, p in zip(xs8, outs, packed):
        assert torch.equal(x, y)
        ref = O.encode8(x.cpu().numpy(), np.frombuffer(codec.codebook, np.uint8), 1024)
        assert p.to_bytes() == O.serialize8(ref)


def test_packed_several_codebooks_e5m2():
    """E5M2 packed streams coded with three codebooks in one launch: each equals the oracle's
    serialization with its own book, and all decode in one launch through a codec that holds
    none of those books (each stream brings its codebook in its header)."""
    cals = [workloads.e5m2_normal(40000, 80 + k, sigma=s) for k, s in enumerate((1.0, 300.0, 0.01))]
    codec = sz.Codec(DEV, 1024, elem="e5m2")
    codec.calibrate_books([dev8(c) for c in cals])
    xs = [workloads.e5m2_normal(n, 90 + i, sigma=s) for i, (n, s) in
          enumerate([(128 * 400, 1.0), (128 * 777, 300.0), (128, 0.01), (0, 1.0)])]
    books = [0, 1, 2, 1]
    packed = codec.encode_packed_batch([dev8(x) for x in xs], books=books)
    for x, p, b in zip(xs, packed, books):
        ref = O.encode8(x, np.frombuffer(codec.books[b], np.uint8), 1024)
        assert p.to_bytes() == O.serialize8(ref)
    other = sz.Codec.from_codebook(bytes(range(16, 32)), 1024, DEV, elem="e5m2")
    ys = other.decode_packed_batch(packed)
    for x, y in zip(xs, ys):
        assert np.array_equal(host(y, np.uint8), x)
