"""GPU parity of packed streams: the canonical stream (header + sections) written into one
contiguous device buffer by the encode kernels must equal the oracle's serialization byte
for byte, and the decode kernel must rebuild the input from such a buffer (including
streams the oracle wrote), with its own codebook, and refuse a header that does not
describe the buffer."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import lossless_bf16_kv_amd as sz
import oracle
import stream_check
import workloads
from test_gpu_parity import DEV, codec_for, dev, host

pytestmark = pytest.mark.gpu

O = oracle.get()


def oracle_stream(x: np.ndarray, cb: bytes, C: int) -> bytes:
    return O.serialize(O.encode(x, np.frombuffer(cb, np.uint8), C))


def to_dev_bytes(b: bytes) -> torch.Tensor:
    return torch.from_numpy(np.frombuffer(b, np.uint8).copy()).to(DEV)


SIZES = [0, 16, 32, 8192, 3 * 16384 + 16, 1_000_000, (1 << 20) + 80]


@pytest.mark.parametrize("C", [16, 1024, 65536])
def test_packed_stream_equals_oracle_serialization(C):
    cal = workloads.mixed_words(300_000, 41, wide_fraction=0.05)
    codec = codec_for(cal, C)
    xs = [workloads.mixed_words(n, 700 + n % 97, wide_fraction=0.05) for n in SIZES]
    packed = codec.encode_packed_batch([dev(x) for x in xs])
    for x, p in zip(xs, packed):
        want = oracle_stream(x, codec.codebook, C)
        assert p.stream_bytes == len(want)
        assert p.to_bytes() == want
    ys = codec.decode_packed_batch(packed)
    for x, y in zip(xs, ys):
        assert np.array_equal(host(y, np.uint16), x)


def test_packed_books_async_and_capacity():
    cals = [workloads.normal_words(100_000, 60 + k, sigma=2.0 ** (6 * k - 6)) for k in range(3)]
    codec = sz.Codec(DEV, 1024)
    codec.calibrate_books([dev(c) for c in cals])
    xs = [workloads.normal_words(n, 80 + i, sigma=2.0 ** (6 * (i % 3) - 6))
          for i, n in enumerate([16384 * 7 + 48, 4096, 250_000])]
    books = [0, 1, 2]
    packed = codec.encode_packed_batch([dev(x) for x in xs], books=books)
    for x, p, b in zip(xs, packed, books):
        assert p.to_bytes() == oracle_stream(x, codec.books[b], 1024)
    # non-blocking: E per stream in the result words, same bytes in fresh buffers
    segs = (sz.splitzip_packed * len(xs))()
    bufs = [torch.full((p.buf.numel(),), 0xA5, dtype=torch.uint8, device=DEV) for p in packed]
    xds = [dev(x) for x in xs]
    for i, (xd, p, b) in enumerate(zip(xds, packed, bufs)):
        segs[i] = sz.splitzip_packed(xd.data_ptr(), p.n, b.data_ptr(), b.numel(), 0, 0, p.book, 0)
    res = torch.zeros(1 + len(xs), dtype=torch.int64, device=DEV)
    sz.splitzip_encode_packed(codec.handle, segs, torch.cuda.current_stream(DEV).cuda_stream, res.data_ptr())
    r = res.cpu().tolist()
    assert r[0] == 0 and r[1:] == [p.n_escapes for p in packed]
    for p, b in zip(packed, bufs):
        assert b[:p.stream_bytes].cpu().numpy().tobytes() == p.to_bytes()
    # a buffer too small for the escapes: E_CAPACITY, the size needed, no escape written
    x = xs[2]
    need, E = packed[2].stream_bytes, packed[2].n_escapes
    assert E >= 2
    fixed = need - 3 * E
    small = torch.zeros(fixed + 3 * (E // 2), dtype=torch.uint8, device=DEV)
    seg = (sz.splitzip_packed * 1)()
    seg[0] = sz.splitzip_packed(xds[2].data_ptr(), x.size, small.data_ptr(), small.numel(), 0, 0, 2, 0)
    assert sz.splitzip_encode_packed(codec.handle, seg, torch.cuda.current_stream(DEV).cuda_stream) == sz.E_CAPACITY
    assert seg[0].stream_bytes == need and seg[0].n_escapes == E
    assert not bool(small[fixed:].any())
    # the Python API retries into a larger buffer
    p2 = codec.encode_packed(xds[2], book=2, capacity=small.numel())
    assert p2.to_bytes() == packed[2].to_bytes()


def test_decode_oracle_streams_with_their_own_codebooks():
    """Streams written by the oracle with three different codebooks, decoded in one launch
    by a codec that holds none of them (same chunk size): the header's codebook is used."""
    C = 4096
    xs = [workloads.mixed_words(n, 900 + n % 13, wide_fraction=0.1) for n in (16 * 1001, 65536 + 16, 32)]
    cbs = [bytes(O.calibrate(workloads.normal_words(50_000, 5 + k, sigma=4.0 ** k))[0]) for k in range(3)]
    streams = [oracle_stream(x, cb, C) for x, cb in zip(xs, cbs)]
    other = sz.Codec.from_codebook(bytes(range(200, 216)), C, DEV)
    ys = other.decode_packed_batch([to_dev_bytes(s) for s in streams], ns=[x.size for x in xs])
    for x, y in zip(xs, ys):
        assert np.array_equal(host(y, np.uint16), x)


def test_packed_header_and_length_checks():
    C = 1024
    x = workloads.mixed_words(16 * 5000, 77, wide_fraction=0.05)
    codec = codec_for(x, C)
    good = oracle_stream(x, codec.codebook, C)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    # header fields that disagree with the buffer: nothing is written, bit 16 is flagged
    for off, val in ((0, 0x00), (4, 2), (8, 0x00), (16, 0x01), (32, 0x07), (60, 1)):
        b = bytearray(good)
        b[off] = val if b[off] != val else val ^ 1
        sentinel = torch.full((x.size,), 0x1234, dtype=torch.int16, device=DEV)
        segs = (sz.splitzip_packed * 1)()
        buf = to_dev_bytes(bytes(b))
        segs[0] = sz.splitzip_packed(sentinel.data_ptr(), x.size, buf.data_ptr(), buf.numel(), 0, 0, 0, 0)
        err.zero_()
        sz.splitzip_decode_packed(codec.handle, segs, torch.cuda.current_stream(DEV).cuda_stream, err.data_ptr())
        assert int(err.item()) & 16, off
        assert bool((sentinel == 0x1234).all()), off
    # a length that fits no stream of n words, and n not a multiple of 16: refused on the host
    buf = to_dev_bytes(good + b"\0")
    with pytest.raises(sz.SplitZipError) as ei:
        codec.decode_packed(buf, x.size)
    assert ei.value.status == sz.E_FORMAT
    with pytest.raises(sz.SplitZipError) as ei:
        codec.encode_packed(dev(x[:100]))
    assert ei.value.status == sz.E_INVALID
    # a misaligned buffer is refused
    big = torch.zeros(len(good) + 16, dtype=torch.uint8, device=DEV)
    segs = (sz.splitzip_packed * 1)()
    xd = dev(x)
    segs[0] = sz.splitzip_packed(xd.data_ptr(), x.size, big.data_ptr() + 8, len(good), 0, 0, 0, 0)
    with pytest.raises(sz.SplitZipError) as ei:
        sz.splitzip_encode_packed(codec.handle, segs, 0)
    assert ei.value.status == sz.E_INVALID


def test_config5_ragged_batch_packed():
    """512 packed streams in one launch: every stream whole against the oracle."""
    wl = workloads.config5()
    codec = codec_for(wl.calibration, wl.chunk_size)
    cb = np.frombuffer(codec.codebook, np.uint8)
    xds = [dev(s) for s in wl.segments]
    packed = codec.encode_packed_batch(xds)
    cases = []
    for i, (x, p) in enumerate(zip(wl.segments, packed)):
        case, head = stream_check.case_from_packed(f"segment {i}", p.stream, x, cb, wl.chunk_size)
        assert head == O.header(x.size, wl.chunk_size, p.n_escapes, cb, 0)
        cases.append(case)
    stream_check.check_cases(cases)
    encs = codec.encode_batch(xds)
    assert [p.n_escapes for p in packed] == [e.n_escapes for e in encs]
    for xd, y in zip(xds, codec.decode_packed_batch(packed)):
        assert torch.equal(y, xd)


def test_config3_packed_full_size():
    """2^32 words into one 6.5 GB packed stream: the header and every byte of every section
    at its packed offset against the oracle, and the bitwise round trip."""
    wl = workloads.config3()
    x = wl.segments[0]
    C = 1024
    codec = codec_for(wl.calibration, C)
    xd = dev(x)
    p = codec.encode_packed(xd)
    n, E = x.size, p.n_escapes
    hist = O.histogram(x)
    assert E == n - sum(int(hist[e]) for e in codec.codebook)
    assert p.stream_bytes == O.compressed_bytes(n, C, E)
    cb = np.frombuffer(codec.codebook, np.uint8)
    case, head = stream_check.case_from_packed("config3 packed", p.stream, x, cb, C)
    assert head == O.header(n, C, E, cb, 0)
    stream_check.check_cases([case])
    del case
    y = codec.decode_packed(p)
    assert torch.equal(y.view(torch.int16), xd)
