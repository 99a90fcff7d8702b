"""GPU parity of the exponent statistics and of codecs with several codebooks.

The GPU histograms (one pass over many tensors) must equal the oracle's, the statistics
derived from them must equal the oracle's entropy, codebook and coverage, and a ragged
batch whose segments use different codebooks must give, segment by segment, the oracle's
stream for that segment's codebook."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import lossless_bf16_kv_amd as sz
import oracle
import workloads
import stream_check
from test_gpu_parity import DEV, assert_same_stream, check_properties, dev, host

pytestmark = pytest.mark.gpu

O = oracle.get()


def test_histograms_of_many_tensors_match_oracle():
    sizes = [0, 1, 7, 8, 17, 4099, 3 * 16384 + 5, 1_000_003, 5_000_000]
    xs = [workloads.mixed_words(n, seed=300 + i, wide_fraction=0.1 * (i % 3)) for i, n in enumerate(sizes)]
    hs = sz.histograms([dev(x) for x in xs])
    for x, h in zip(xs, hs):
        assert h == O.histogram(x).tolist()
    # one tensor alone takes the single-tensor path of the same kernels
    assert sz.histograms([dev(xs[-1])])[0] == O.histogram(xs[-1]).tolist()


def test_exponent_statistics_of_kv_tensors():
    """Entropy, top-16 codebook and coverage of K and V of a GQA layer, from the GPU
    histogram, against the oracle's on the same tensors."""
    wl = workloads.config2()
    hs = sz.histograms([dev(s) for s in wl.segments])
    for x, h in zip(wl.segments, hs):
        st = sz.exponent_stats(h)
        ho = O.histogram(x)
        cb = O.codebook(ho)
        assert abs(st["entropy_bits"] - O.entropy(ho)) <= 1e-12 * O.entropy(ho)
        assert st["codebook"] == bytes(cb)
        assert st["coverage"] == O.coverage(ho, cb, x.size)
        assert st["distinct"] == int(np.count_nonzero(ho))
        assert 1.5 < st["entropy_bits"] < 4.5


def three_distributions():
    # three normal scales 2^5 apart: their top-16 exponent windows differ
    return [workloads.normal_words(200_000, 10 + k, sigma=2.0 ** (5 * k - 5)) for k in range(3)]


def test_calibrate_books_match_oracle_per_book():
    cals = three_distributions()
    codec = sz.Codec(DEV, 1024)
    cov = codec.calibrate_books([dev(c) for c in cals])
    books = codec.books
    assert len(books) == 3 and len(set(books)) == 3
    for b, c in enumerate(cals):
        cb, cv, h = O.calibrate(c)
        assert books[b] == bytes(cb)
        assert cov[b] == cv
        assert codec.histogram[b] == h.tolist()
    assert codec.codebook == books[0]


@pytest.mark.parametrize("C", [64, 1024, 65536])
def test_segments_with_different_books_in_one_launch(C):
    cals = three_distributions()
    codec = sz.Codec(DEV, C)
    codec.calibrate_books([dev(c) for c in cals])
    # segments drawn from the three scales; some coded with another scale's book (valid,
    # just more escapes); ragged sizes spanning several tiles
    plan = [(0, 0, 70_001), (1, 1, 16384 * 5 + 3), (2, 2, 9), (1, 0, 40_000), (0, 2, 0),
            (2, 1, 123_457), (1, 1, 1)]
    xs = [workloads.normal_words(n, 500 + i, sigma=2.0 ** (5 * k - 5)) for i, (k, _, n) in enumerate(plan)]
    books = [b for _, b, _ in plan]
    encs = codec.encode_batch([dev(x) for x in xs], books=books)
    for x, e, b in zip(xs, encs, books):
        assert e.book == b and e.codebook == codec.books[b]
        assert_same_stream(codec, e, x)
        assert e.to_bytes(codec)[40:56] == codec.books[b]
    ys = codec.decode_batch(encs)                       # one launch, mixed books
    for x, y in zip(xs, ys):
        assert np.array_equal(host(y, np.uint16), x)
    for x, e, b in zip(xs, encs, books):                # streams name their book by codebook
        assert sz.splitzip_check_header(codec.handle, e.to_bytes(codec)) == b
        assert np.array_equal(host(codec.decode_bytes(e.to_bytes(codec)), np.uint16), x)
    # one segment, and a batch whose segments share one book: the single-book paths
    e = codec.encode(dev(xs[5]), book=1)
    assert_same_stream(codec, e, xs[5])
    assert np.array_equal(host(codec.decode(e), np.uint16), xs[5])
    same = codec.encode_batch([dev(xs[0]), dev(xs[1])], books=[2, 2])
    for x, e in zip(xs[:2], same):
        assert_same_stream(codec, e, x)
    for x, y in zip(xs[:2], codec.decode_batch(same)):
        assert np.array_equal(host(y, np.uint16), x)


def test_book_out_of_range_rejected():
    codec = sz.Codec(DEV, 1024)
    codec.calibrate_books([dev(c) for c in three_distributions()[:2]])
    x = workloads.normal_words(1000, 1)
    enc = codec.empty_encoded(x.size, book=1)
    enc.book = 2
    with pytest.raises(sz.SplitZipError) as ei:
        codec.encode_into([dev(x)], [enc])
    assert ei.value.status == sz.E_INVALID


LAYERS, TOKENS, CAL_TOKENS = 8, 32768, 2048


@pytest.fixture(scope="module")
def kv8():
    return workloads.config3(layers=LAYERS, tokens=TOKENS, cal_tokens=CAL_TOKENS)


def test_per_layer_kv_books_long_prefill(kv8):
    """8 layers of the long-prefill KV generator (2^29 words), one codebook per layer and
    K/V (16 books), all 16 tensors in one encode and one decode launch: codebooks from the
    oracle's calibration of each part, E per tensor from the oracle's histogram, every
    stream whole against the oracle with its own book, bitwise round trip, and fewer
    escapes than one codebook."""
    wl = kv8
    parts = workloads.kv_parts(wl.segments[0], LAYERS, TOKENS)
    cals = workloads.kv_parts(wl.calibration, LAYERS, CAL_TOKENS)
    codec = sz.Codec(DEV, 1024)
    cov = codec.calibrate_books([dev(c) for c in cals])
    for b, c in enumerate(cals):
        cb, cv, _ = O.calibrate(c)
        assert codec.books[b] == bytes(cb) and cov[b] == cv
    xds = [dev(p) for p in parts]
    encs = codec.encode_batch(xds, books=list(range(len(parts))))
    for x, e in zip(parts, encs):
        check_properties(codec, e, x, O.histogram(x))
    stream_check.check_cases([stream_check.case_from_encoded(f"layer {i // 2} {'KV'[i % 2]}", e, x)
                              for i, (x, e) in enumerate(zip(parts, encs))])
    for xd, y in zip(xds, codec.decode_batch(encs)):
        assert torch.equal(y, xd)
    one = sz.Codec(DEV, 1024)
    one.calibrate(dev(wl.calibration))
    e1 = one.encode(dev(wl.segments[0]))
    assert sum(e.n_escapes for e in encs) < e1.n_escapes
