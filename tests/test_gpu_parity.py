"""GPU parity: the HIP codec (through the C ABI) against the CPU oracle.

Encoded streams must equal the oracle's byte for byte, decode must return the input
bit for bit, and calibration must give the oracle's histogram, codebook and coverage.
Small and mid-size inputs are compared element by element in one piece; the full-size
workloads (8.6 GB long-prefill KV, 512-segment ragged batch) are compared whole too, every
byte of every section, against the oracle encoding the input window by window
(tests/stream_check.py)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import lossless_bf16_kv_amd as sz
import oracle
import oracle_pins as pins
import stream_check
import workloads
from conftest import hex_bytes, ints

pytestmark = pytest.mark.gpu

O = oracle.get()
DEV = torch.device("cuda:0")


def dev(words: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words, np.uint16).view(np.int16)).to(DEV)


def host(t: torch.Tensor, dtype) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(dtype)


def codec_for(cal: np.ndarray, C: int) -> sz.Codec:
    c = sz.Codec(DEV, C)
    c.calibrate(dev(cal))
    return c


def assert_same_stream(codec: sz.Codec, enc: sz.Encoded, x: np.ndarray):
    cb = np.frombuffer(enc.codebook, np.uint8)
    ref = O.encode(x, cb, codec.chunk_size)
    assert enc.n_escapes == ref["n_escapes"]
    assert enc.compressed_bytes == ref["compressed_bytes"]
    assert np.array_equal(host(enc.sm, np.uint8), ref["sm"])
    assert np.array_equal(host(enc.codes, np.uint8), ref["codes"])
    assert np.array_equal(host(enc.chunk_off, np.uint64), ref["chunk_off"])
    assert np.array_equal(host(enc.esc_pos, np.uint16), ref["esc_pos"])
    assert np.array_equal(host(enc.esc_exp, np.uint8), ref["esc_exp"])
    assert enc.to_bytes(codec) == O.serialize(ref)
    return ref


# ---- worked example and exhaustive words ----------------------------------------------

def test_worked_example():
    g, cal, x = pins.worked_example()
    codec = sz.Codec(DEV, int(g["chunk_size"]))
    cov = codec.calibrate(dev(cal))
    assert codec.codebook == hex_bytes(g["codebook"])
    assert cov == float(g["calibration_coverage"])
    enc = codec.encode(dev(x))
    assert bytes(host(enc.sm, np.uint8)) == hex_bytes(g["sm"])
    assert bytes(host(enc.codes, np.uint8)) == hex_bytes(g["codes"])
    assert host(enc.chunk_off, np.uint64).tolist() == ints(g["chunk_off"])
    assert host(enc.esc_pos, np.uint16).tolist() == ints(g["esc_pos"])
    assert host(enc.esc_exp, np.uint8).tolist() == ints(g["esc_exp"])
    assert enc.compressed_bytes == int(g["compressed_bytes"])
    assert enc.to_bytes(codec)[:64] == hex_bytes(g["header"])
    assert np.array_equal(host(codec.decode(enc), np.uint16), x)
    for n in (0, 7):
        e = codec.encode(dev(x[:n]))
        assert_same_stream(codec, e, x[:n])
        assert np.array_equal(host(codec.decode(e), np.uint16), x[:n])


@pytest.mark.parametrize("C", [16, 1024, 4096, 65536])
def test_exhaustive_words(C):
    x = np.arange(1 << 16, dtype=np.uint16)
    codec = codec_for(x, C)
    assert codec.codebook == bytes(range(16))
    assert codec.coverage == 1 / 16
    enc = codec.encode(dev(x))
    assert_same_stream(codec, enc, x)
    assert np.array_equal(host(codec.decode(enc), np.uint16), x)


# ---- calibration --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 5, 8, 17, 4099, 1000003])
def test_calibration_matches_oracle(n):
    x = workloads.mixed_words(n, seed=n, wide_fraction=0.2)
    codec = codec_for(x, 1024)
    cb, cov, h = O.calibrate(x)
    assert codec.histogram == h.tolist()
    assert codec.codebook == bytes(cb)
    assert codec.coverage == cov


def test_calibration_empty_and_few_exponents():
    codec = sz.Codec(DEV, 64)
    assert codec.calibrate(torch.empty(0, dtype=torch.int16, device=DEV)) == 0.0
    assert codec.codebook == bytes(range(16))
    x = np.full(100, 0x3F80, np.uint16)
    codec.calibrate(dev(x))
    assert codec.codebook == bytes(O.calibrate(x)[0])


# ---- fuzz: sizes spanning several tiles with ragged tails, every chunk-size regime ---------

FUZZ = [(n, C, gen) for n, C, gen in [
    (1, 16, "random"), (9, 16, "mixed"), (8191, 1024, "mixed"), (8192, 1024, "normal"),
    (8193, 16, "random"), (3 * 8192 + 13, 64, "mixed"), (100003, 1024, "random"),
    (100003, 4096, "mixed"), (65536 * 3 + 5, 16384, "mixed"), (65536 * 3 + 5, 65536, "random"),
    ((1 << 20) + 77, 1024, "mixed"), ((1 << 20) + 77, 32, "random"),
]]


@pytest.mark.parametrize("n,C,gen", FUZZ)
def test_fuzz_stream_parity(n, C, gen):
    make = {"random": workloads.random_words, "mixed": workloads.mixed_words,
            "normal": workloads.normal_words}[gen]
    x = make(n, 17 * n + C)
    codec = codec_for(workloads.normal_words(50000, 3), C)
    enc = codec.encode(dev(x))
    ref = assert_same_stream(codec, enc, x)
    assert np.array_equal(host(codec.decode(enc), np.uint16), x)
    # the GPU decodes the oracle's serialized stream too
    y = codec.decode_bytes(O.serialize(ref))
    assert np.array_equal(host(y, np.uint16), x)


def test_batch_with_empty_and_tiny_segments():
    sizes = [0, 1, 7, 8192, 8193, 0, 100, 3 * 8192 + 5]
    xs = [workloads.mixed_words(n, 100 + i, wide_fraction=0.3) for i, n in enumerate(sizes)]
    codec = codec_for(workloads.normal_words(20000, 4), 16)
    encs = codec.encode_batch([dev(x) for x in xs])
    for x, e in zip(xs, encs):
        assert_same_stream(codec, e, x)
    ys = codec.decode_batch(encs)
    for x, y in zip(xs, ys):
        assert np.array_equal(host(y, np.uint16), x)


def test_capacity_retry_gives_identical_stream():
    x = workloads.random_words(50000, 9)           # ~94 % escapes
    codec = codec_for(workloads.normal_words(20000, 5), 1024)
    enc = codec.empty_encoded(x.size, escape_capacity=10)
    st = codec.encode_into([dev(x)], [enc])
    assert st == sz.E_CAPACITY
    ref = O.encode(x, np.frombuffer(codec.codebook, np.uint8), 1024)
    assert enc.n_escapes == ref["n_escapes"]
    enc2 = codec.encode(dev(x))
    assert_same_stream(codec, enc2, x)


def test_deterministic_and_stream_independent():
    x = workloads.mixed_words(5 * 8192 + 3, 11, wide_fraction=0.1)
    codec = codec_for(workloads.normal_words(20000, 6), 1024)
    xd = dev(x)
    a = codec.encode(xd).to_bytes(codec)
    b = codec.encode(xd).to_bytes(codec)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        c = codec.encode(xd)
    with torch.cuda.stream(s2):
        d = codec.encode(xd)
    torch.cuda.synchronize()
    assert a == b == c.to_bytes(codec) == d.to_bytes(codec)


@pytest.mark.parametrize("stage_tiles", [sz.STAGE_TILES, 0])
def test_decode_flags_corrupt_metadata_without_faulting(stage_tiles):
    """Both decode builds (0: the large-call build, whose escapes find their chunk by
    counting offsets held in scalar registers) flag corrupt metadata without a fault."""
    x = workloads.mixed_words(4 * 8192, 12, wide_fraction=0.2)
    codec = codec_for(workloads.normal_words(20000, 7), 1024)
    codec.set_stage_tiles(stage_tiles)
    enc = codec.encode(dev(x))
    assert enc.n_escapes > 100
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    bad = dataclass_copy(enc)
    bad.chunk_off[3] = enc.n_escapes + 1000            # offset beyond E
    bad.esc_pos_buf[5] = 4000                          # position beyond its chunk
    y = torch.empty_like(codec.decode(enc))
    codec.decode_into([bad], [y], d_error=err.data_ptr())
    torch.cuda.synchronize()
    assert int(err.item()) != 0
    # offsets that decrease inside a tile but stay below E
    bad = dataclass_copy(enc)
    bad.chunk_off[2] = enc.chunk_off[6]
    assert int(enc.chunk_off[6]) > int(enc.chunk_off[3])
    err.zero_()
    codec.decode_into([bad], [y], d_error=err.data_ptr())
    torch.cuda.synchronize()
    assert int(err.item()) != 0
    # every escape in the last chunk (offsets 0 up to the final E): more escapes than that
    # chunk has words
    bad = dataclass_copy(enc)
    bad.chunk_off[:-1] = 0
    assert enc.n_escapes > 1024
    err.zero_()
    codec.decode_into([bad], [y], d_error=err.data_ptr())
    torch.cuda.synchronize()
    assert int(err.item()) & 2
    # an intact stream leaves the flag at zero
    err.zero_()
    codec.decode_into([enc], [y], d_error=err.data_ptr())
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and np.array_equal(host(y, np.uint16), x)
    # more escapes than the last tile has words: flagged, that tile left unpatched
    x2 = workloads.mixed_words(4 * 8192, 13, wide_fraction=0.6)
    enc2 = codec.encode(dev(x2))
    assert enc2.n_escapes > 8192
    bad = dataclass_copy(enc2)
    bad.chunk_off[:-1] = 0
    y2 = torch.empty_like(y)
    err.zero_()
    codec.decode_into([bad], [y2], d_error=err.data_ptr())
    torch.cuda.synchronize()
    assert int(err.item()) & 2


def dataclass_copy(e: sz.Encoded) -> sz.Encoded:
    import dataclasses
    return dataclasses.replace(e, sm=e.sm.clone(), codes=e.codes.clone(),
                               chunk_off=e.chunk_off.clone(), esc_pos_buf=e.esc_pos_buf.clone(),
                               esc_exp_buf=e.esc_exp_buf.clone())


def test_codebook_mismatch_rejected():
    x = workloads.normal_words(1000, 1)
    a = codec_for(workloads.normal_words(5000, 2), 1024)
    b = sz.Codec.from_codebook(bytes(range(100, 116)), 1024, DEV)
    enc = a.encode(dev(x))
    with pytest.raises(sz.SplitZipError) as ei:
        b.decode(enc)
    assert ei.value.status == sz.E_CODEBOOK
    with pytest.raises(sz.SplitZipError) as ei:
        b.decode_bytes(enc.to_bytes(a))
    assert ei.value.status == sz.E_CODEBOOK
    # a codec rebuilt from the stream header decodes it
    c = sz.Codec.from_codebook(sz.splitzip_read_header(enc.to_bytes(a))["codebook"], 1024, DEV)
    assert np.array_equal(host(c.decode_bytes(enc.to_bytes(a)), np.uint16), x)


# ---- the five workloads -------------------------------------------------------------------

def test_config1_single_tensor():
    wl = workloads.config1()
    codec = codec_for(wl.calibration, wl.chunk_size)
    cb, cov, _ = O.calibrate(wl.calibration)
    assert codec.codebook == bytes(cb) and codec.coverage == cov
    x = wl.segments[0]
    enc = codec.encode(dev(x).view(1024, 4096))
    assert_same_stream(codec, enc, x)
    y = codec.decode(enc)
    assert y.shape == (1024, 4096)
    assert np.array_equal(host(y, np.uint16).reshape(-1), x)


def test_config2_kv_layer_two_segments():
    wl = workloads.config2()
    codec = codec_for(wl.calibration, wl.chunk_size)
    assert codec.codebook == bytes(O.calibrate(wl.calibration)[0])
    encs = codec.encode_batch([dev(s) for s in wl.segments])
    for x, e in zip(wl.segments, encs):
        assert_same_stream(codec, e, x)
    for x, y in zip(wl.segments, codec.decode_batch(encs)):
        assert np.array_equal(host(y, np.uint16), x)


@pytest.mark.parametrize("private", [True, False])
@pytest.mark.parametrize("C", [1024, 4096])
def test_config4_escape_stress(C, private):
    """The escape-stress input (4096 pack tiles, about 29 % escapes, every tile past its
    slot): whole stream against the oracle, with the tiles' own overflow regions (the
    default at this size) and with the shared area that they reserve from one counter."""
    wl = workloads.config4(chunk_size=C)
    codec = codec_for(wl.calibration, C)
    if not private:
        codec.set_private_overflow(0)
    x = wl.segments[0]
    enc = codec.encode(dev(x))
    ref = assert_same_stream(codec, enc, x)
    assert 0.2 < ref["n_escapes"] / x.size < 0.4
    assert np.array_equal(host(codec.decode(enc), np.uint16), x)


def check_properties(codec, enc, x, hist_x):
    """Size-independent checks: E from the oracle's exact histogram, offsets, sizes."""
    C = codec.chunk_size
    cb = np.frombuffer(enc.codebook, np.uint8)
    E = int(x.size - sum(int(hist_x[e]) for e in cb))
    assert enc.n_escapes == E
    off = enc.chunk_off
    assert int(off[0]) == 0 and int(off[-1]) == E
    assert bool((off[1:] >= off[:-1]).all())
    assert bool((off[1:] - off[:-1] <= C).all())
    assert enc.compressed_bytes == O.compressed_bytes(x.size, C, E)


@pytest.fixture(scope="module")
def config3_data():
    wl = workloads.config3()
    return wl


@pytest.mark.parametrize("C", [1024, 4096])
def test_config3_long_prefill_full_size(config3_data, C):
    """2^32 words in one segment, the launch sequence the bench times: every byte of every
    section against the oracle, E from the oracle's histogram, the size, the round trip."""
    wl = config3_data
    x = wl.segments[0]
    assert x.size == 1 << 32
    xd = dev(x)
    codec = codec_for(wl.calibration, C)
    cb, cov, _ = O.calibrate(wl.calibration)
    assert codec.codebook == bytes(cb) and codec.coverage == cov
    enc = codec.encode(xd)
    check_properties(codec, enc, x, O.histogram(x))
    stream_check.check_cases([stream_check.case_from_encoded(f"config3 C={C}", enc, x)])
    y = codec.decode(enc)
    assert torch.equal(y, xd)
    del y


def test_config3_full_size_histogram(config3_data):
    x = config3_data.segments[0]
    c = codec_for(x, 1024)             # calibrating on the data itself gives its histogram
    assert c.histogram == O.histogram(x).tolist()


def test_config5_ragged_batch():
    """512 segments in one encode launch and one decode launch: every stream whole."""
    wl = workloads.config5()
    codec = codec_for(wl.calibration, wl.chunk_size)
    assert len(wl.segments) == 512
    xds = [dev(s) for s in wl.segments]
    encs = codec.encode_batch(xds)                 # one launch, 512 segments
    for x, e in zip(wl.segments, encs):
        check_properties(codec, e, x, O.histogram(x))
    stream_check.check_cases([stream_check.case_from_encoded(f"config5 segment {i}", e, x)
                              for i, (x, e) in enumerate(zip(wl.segments, encs))])
    ys = codec.decode_batch(encs)                  # one launch
    for xd, y in zip(xds, ys):
        assert torch.equal(y, xd)


# ---- non-blocking encode, per-kernel timing ----------------------------------------------------

def test_async_encode_matches_blocking_and_reports_capacity():
    xs_np = [workloads.mixed_words(n, 200 + n, wide_fraction=0.05) for n in (3 * 16384 + 11, 70000, 0, 5)]
    codec = codec_for(workloads.normal_words(30000, 8), 1024)
    xs = [dev(x) for x in xs_np]
    ref = codec.encode_batch(xs)
    encs = [codec.empty_encoded(e.n, escape_capacity=max(e.n_escapes, 1)) for e in ref]
    result = torch.zeros(1 + len(xs), dtype=torch.int64, device=DEV)
    codec.encode_into_async(xs, encs, result)
    torch.cuda.synchronize()
    assert codec.finish_async(encs, result) == sz.OK
    for x, e, r in zip(xs_np, encs, ref):
        assert e.n_escapes == r.n_escapes and e.to_bytes(codec) == r.to_bytes(codec)
        assert_same_stream(codec, e, x)
    # too little room: reported after the fact, counts still exact
    small = [codec.empty_encoded(e.n, escape_capacity=1) for e in ref]
    result.zero_()
    codec.encode_into_async(xs, small, result)
    torch.cuda.synchronize()
    assert codec.finish_async(small, result) == sz.E_CAPACITY
    assert [e.n_escapes for e in small] == [e.n_escapes for e in ref]


def test_kernel_timing():
    x = dev(workloads.normal_words(5 * 16384, 9))
    codec = codec_for(workloads.normal_words(30000, 10), 1024)
    codec.profile(True)
    for _ in range(3):
        codec.decode(codec.encode(x))
    times = codec.kernel_times(reset=True)
    assert set(times) == {"encode_pack", "encode_sums", "encode_place", "encode_spill", "decode",
                          "encode_finish", "encode_onepass"}
    # a BF16 call of 5 tiles runs the one-pass launch; the other encode kernels are not launched
    for k, (ms, count) in times.items():
        if k in ("encode_onepass", "decode"):
            assert count == 3 and ms > 0, k
        else:
            assert count == 0, k
    # without it, pack + finish
    codec.set_onepass_tiles(0)
    codec.encode(x)
    times = codec.kernel_times(reset=True)
    assert times["encode_pack"][1] == times["encode_finish"][1] == 1 and times["encode_onepass"][1] == 0
    codec.set_onepass_tiles()
    assert all(c == 0 for _, c in codec.kernel_times().values())
    codec.profile(False)
    codec.decode(codec.encode(x))
    assert all(c == 0 for _, c in codec.kernel_times().values())


def test_prepared_batch_round_trip():
    xs_np = [workloads.mixed_words(n, 300 + n, wide_fraction=0.02) for n in (16384 * 2 + 7, 100, 0, 40000)]
    codec = codec_for(workloads.normal_words(30000, 11), 64)
    xs = [dev(x) for x in xs_np]
    encs = codec.encode_batch(xs)
    ys = [torch.empty_like(x) for x in xs]
    batch = codec.prepare(xs, encs, ys)
    result = torch.zeros(1 + len(xs), dtype=torch.int64, device=DEV)
    for _ in range(3):
        batch.encode_async(result)
        batch.decode()
    torch.cuda.synchronize()
    assert batch.finish(result) == sz.OK
    for x, e, y in zip(xs_np, encs, ys):
        assert_same_stream(codec, e, x)
        assert np.array_equal(host(y, np.uint16), x)


def test_descriptor_tables_reused_and_replaced():
    """Calls on the same segment buffers reuse the device copy of their descriptor table.
    New contents in those buffers, escape counts that change between decodes, and more
    distinct tables in between than the library keeps staged must still give the oracle's
    streams and bitwise round trips."""
    codec = codec_for(workloads.normal_words(30000, 12), 256)
    sizes = [5000, 17000, 0, 40000]
    xs = [torch.empty(n, dtype=torch.int16, device=DEV) for n in sizes]
    encs = [codec.empty_encoded(n, escape_capacity=max(n, 1)) for n in sizes]
    ys = [torch.empty_like(x) for x in xs]
    for rnd in range(3):
        xs_np = [workloads.mixed_words(n, 100 * rnd + i, wide_fraction=0.05 * rnd)
                 for i, n in enumerate(sizes)]
        for x, x_np in zip(xs, xs_np):
            x.copy_(dev(x_np))
        assert codec.encode_into(xs, encs) == sz.OK
        for x_np, e in zip(xs_np, encs):
            assert_same_stream(codec, e, x_np)
        codec.decode_into(encs, ys)
        for x_np, y in zip(xs_np, ys):
            assert np.array_equal(host(y, np.uint16), x_np)
        # twenty other two-segment batches: their tables replace every staged one
        for k in range(20):
            other_np = [workloads.mixed_words(1000 + 37 * k, 7 * k + rnd), workloads.normal_words(7 + k, k)]
            other = codec.encode_batch([dev(o) for o in other_np])
            for o_np, e in zip(other_np, other):
                assert e.n_escapes == O.encode(o_np, np.frombuffer(codec.codebook, np.uint8), 256)["n_escapes"]
            if k % 5 == 0:
                for o_np, y in zip(other_np, codec.decode_batch(other)):
                    assert np.array_equal(host(y, np.uint16), o_np)


def test_readme_codec_api_usage():
    """The usage the SplitZip README's Codec API shows, under its class name: constructor
    (device, chunk_size), calibrate -> coverage, encode -> object with compressed_bytes,
    decode -> a tensor equal bit for bit, of the input's shape and dtype."""
    torch.manual_seed(0)
    x = torch.randn(1024, 4096, dtype=torch.bfloat16, device="cuda")
    codec = sz.ChunkLocalSplitZipGPU(device="cuda", chunk_size=1024)
    coverage = codec.calibrate(x)
    encoded = codec.encode(x)
    decoded = codec.decode(encoded)
    assert torch.equal(x.view(torch.int16), decoded.view(torch.int16))
    assert decoded.shape == x.shape and decoded.dtype == x.dtype
    words = x.view(torch.int16).cpu().numpy().view(np.uint16).ravel()
    cb, cov, _ = O.calibrate(words)
    assert codec.codebook == bytes(cb) and coverage == cov
    assert encoded.compressed_bytes == O.encode(words, np.frombuffer(bytes(cb), np.uint8), 1024)["compressed_bytes"]


def test_concurrent_host_threads_share_one_codec():
    """Four host threads, each with its own stream, encode and decode different batches
    (one and several segments, blocking and non-blocking) through one codec at the same
    time (ctypes releases the GIL during the library calls), while a fifth thread switches
    per-kernel timing on and off: every stream equals the oracle's and every round trip is
    bitwise."""
    import threading
    codec = codec_for(workloads.normal_words(30000, 21), 256)
    cb = np.frombuffer(codec.codebook, np.uint8)
    errors = []

    def work(tid):
        try:
            stream = torch.cuda.Stream(device=DEV)
            with torch.cuda.stream(stream):
                for it in range(12):
                    sizes = [int(n) for n in np.random.default_rng(100 * tid + it).integers(0, 70_000, 1 + (it % 3))]
                    xs_np = [workloads.mixed_words(n, 1000 * tid + 10 * it + k, wide_fraction=0.05)
                             for k, n in enumerate(sizes)]
                    xs = [dev(x) for x in xs_np]
                    if it % 2:
                        encs = codec.encode_batch(xs)
                    else:
                        encs = [codec.empty_encoded(x.numel(), escape_capacity=max(x.numel(), 1)) for x in xs]
                        result = torch.zeros(1 + len(xs), dtype=torch.int64, device=DEV)
                        codec.encode_into_async(xs, encs, result)
                        stream.synchronize()
                        assert codec.finish_async(encs, result) == sz.OK
                    ys = codec.decode_batch(encs)
                    stream.synchronize()
                    for x_np, e, y in zip(xs_np, encs, ys):
                        ref = O.encode(x_np, cb, 256)
                        assert e.n_escapes == ref["n_escapes"]
                        assert np.array_equal(host(e.chunk_off, np.uint64), ref["chunk_off"])
                        assert np.array_equal(host(e.esc_pos, np.uint16), ref["esc_pos"])
                        assert np.array_equal(host(y, np.uint16), x_np)
        except Exception as ex:          # reported by the main thread
            errors.append((tid, repr(ex)))

    done = threading.Event()

    def toggle_profiling():
        # a fifth thread switches per-kernel timing on and off and reads its totals meanwhile
        try:
            while not done.is_set():
                codec.profile(True)
                codec.kernel_times()
                codec.profile(False)
        except Exception as ex:
            errors.append(("profiling", repr(ex)))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
    prof = threading.Thread(target=toggle_profiling)
    prof.start()
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    done.set()
    prof.join()
    assert not errors, errors


def test_release_stream_frees_its_workspace():
    """A codec keeps one workspace per stream it encodes on; splitzip_release_stream frees
    it (the C ABI reports 0 bytes afterwards) and a later call on that stream makes a new
    one, with the same stream."""
    codec = codec_for(workloads.normal_words(20000, 2), 1024)
    s = torch.cuda.Stream(DEV)
    assert sz.splitzip_workspace_bytes(codec.handle, s.cuda_stream) == 0
    x_np = workloads.mixed_words(3_000_000, 5)
    x = dev(x_np)
    with torch.cuda.stream(s):
        enc = codec.encode(x)
    used = sz.splitzip_workspace_bytes(codec.handle, s.cuda_stream)
    assert used >= (x_np.size // 16384) * 8              # at least the tiles' one-pass status words
    codec.set_onepass_tiles(0)
    with torch.cuda.stream(s):
        assert codec.encode(x).to_bytes(codec) == enc.to_bytes(codec)
    used = sz.splitzip_workspace_bytes(codec.handle, s.cuda_stream)
    assert used >= (x_np.size // 16384) * 512            # and the launch sequences' escape slots
    codec.set_onepass_tiles()
    sz.splitzip_release_stream(codec.handle, s.cuda_stream)
    assert sz.splitzip_workspace_bytes(codec.handle, s.cuda_stream) == 0
    sz.splitzip_release_stream(codec.handle, s.cuda_stream)          # nothing left: a no-op
    with torch.cuda.stream(s):
        again = codec.encode(x)
        y = codec.decode(again)
    s.synchronize()
    assert sz.splitzip_workspace_bytes(codec.handle, s.cuda_stream) > 0
    assert again.to_bytes(codec) == enc.to_bytes(codec)
    assert np.array_equal(host(y, np.uint16), x_np)
    codec.release_stream(s)
    assert codec.workspace_bytes(s) == 0
