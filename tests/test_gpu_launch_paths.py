"""GPU parity of every encode launch sequence and both pack builds: calls into separate
sections run one launch (each tile places its own escapes after a look-back over the
earlier tiles' status words) up to ONEPASS_TILES tiles; other calls of at most SMALL_TILES
tiles run pack and finish (one workgroup per tile adds up the earlier tiles' escape counts
itself), larger calls run pack, sums, place and spill; calls of more than STAGE_TILES tiles
run the pack build in which a wave gathers a group's escapes in LDS when it has more than
64; escapes past a tile's slot go to the tile's own region or to a shared area reserved with
a counter.  Each case is encoded six ways, which cover every pair of the launch settings
(``Codec.set_small_tiles``, ``Codec.set_stage_tiles``, ``Codec.set_private_overflow``) with
the one-pass launch off, and the one-pass launch with both pack builds; each must equal the
oracle byte for byte: BF16 and E5M2 streams spanning several tiles with ragged tails, tiles
whose escapes overflow their slot, batches with empty and tiny segments and several
codebooks, packed streams, too little escape room, and the 4096 / 4097-tile boundary of the
default."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import lossless_bf16_kv_amd as sz
import oracle
import workloads
from test_gpu_parity import DEV, assert_same_stream, codec_for, dev, host
import test_gpu_e5m2 as t8

pytestmark = pytest.mark.gpu

O = oracle.get()
NEVER = (1 << 32) - 1
PRIV = sz.PRIVATE_OVERFLOW_BYTES
# (set_small_tiles, set_stage_tiles, set_private_overflow, set_onepass_tiles): with the
# one-pass launch off, every pair of the first three settings appears with both of its
# values; the one-pass launch runs with both pack builds (packed streams, which it does not
# take, then run pack + finish or the four launches)
MODES = {"four_launches_shared": (0, NEVER, 0, 0), "pack_finish_private": (sz.SMALL_TILES, NEVER, PRIV, 0),
         "four_launches_gather_private": (0, 0, PRIV, 0), "pack_finish_gather_shared": (sz.SMALL_TILES, 0, 0, 0),
         "onepass": (0, NEVER, PRIV, NEVER), "onepass_gather": (sz.SMALL_TILES, 0, 0, NEVER)}


def use_mode(codec, mode):
    small, stage, private, onepass = MODES[mode]
    codec.set_small_tiles(small)
    codec.set_stage_tiles(stage)
    codec.set_private_overflow(private)
    codec.set_onepass_tiles(onepass)
TILE = 16384          # BF16 words per pack tile
TILE8 = 32768         # E5M2 bytes per pack tile of the launch sequences (one pass: 16384)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("n,C,wide", [
    (1, 16, 0.02), (TILE - 1, 1024, 0.02), (TILE + 1, 16, 0.3), (5 * TILE + 3, 64, 0.02),
    (5 * TILE + 3, 1024, 0.3), (300_007, 4096, 0.05), (300_007, 65536, 0.3),
])
def test_bf16_streams(mode, n, C, wide):
    # wide = 0.3 puts about 30 % of the words outside the codebook: every tile overflows its
    # 128-entry slot and its escapes go through the overflow area
    x = workloads.mixed_words(n, 31 * n + C, wide_fraction=wide)
    codec = codec_for(workloads.normal_words(50_000, 3), C)
    use_mode(codec, mode)
    enc = codec.encode(dev(x))
    assert_same_stream(codec, enc, x)
    assert np.array_equal(host(codec.decode(enc), np.uint16), x)


@pytest.mark.parametrize("mode", MODES)
def test_bf16_batch_empty_tiny_and_books(mode):
    cals = [workloads.normal_words(60_000, 70 + k, sigma=2.0 ** (6 * k - 6)) for k in range(3)]
    codec = sz.Codec(DEV, 64)
    codec.calibrate_books([dev(c) for c in cals])
    use_mode(codec, mode)
    sizes = [0, 1, 7, TILE, TILE + 1, 0, 100, 3 * TILE + 5, 40_000]
    xs = [workloads.mixed_words(n, 500 + i, wide_fraction=0.1 * (i % 4)) for i, n in enumerate(sizes)]
    books = [i % 3 for i in range(len(xs))]
    encs = codec.encode_batch([dev(x) for x in xs], books=books)
    for x, e, b in zip(xs, encs, books):
        assert e.book == b
        assert_same_stream(codec, e, x)
    for x, y in zip(xs, codec.decode_batch(encs)):
        assert np.array_equal(host(y, np.uint16), x)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("escapes", ["in_slots", "overflowing"])
def test_bf16_too_little_escape_room(mode, escapes):
    """E_CAPACITY with the exact count; sm, codes and chunk offsets complete.  Escapes of
    tiles that fit their slot are all written below the capacity; an overflowing tile's
    escapes only when its range of the overflow area (sized from the capacity, reserved in
    whatever order the tiles finish) lies inside it, so there every entry is either final
    or untouched."""
    n = 4 * TILE + 9
    if escapes == "in_slots":       # N(0,1) against its own calibration: ~0.01 % escapes
        x = workloads.normal_words(n, 77)
    else:                           # ~30 % escapes: every tile overflows its slot
        x = workloads.mixed_words(n, 77, wide_fraction=0.3)
    codec = codec_for(workloads.normal_words(20_000, 5), 1024)
    use_mode(codec, mode)
    ref = O.encode(x, np.frombuffer(codec.codebook, np.uint8), 1024)
    assert ref["n_escapes"] >= 3
    cap = ref["n_escapes"] // 3
    enc = codec.empty_encoded(x.size, escape_capacity=cap)
    enc.esc_pos_buf.fill_(-1)            # 0xFFFF: no position inside a 1024-word chunk
    enc.esc_exp_buf.fill_(0)
    assert codec.encode_into([dev(x)], [enc]) == sz.E_CAPACITY
    assert enc.n_escapes == ref["n_escapes"]
    assert np.array_equal(host(enc.sm, np.uint8), ref["sm"])
    assert np.array_equal(host(enc.codes, np.uint8), ref["codes"])
    assert np.array_equal(host(enc.chunk_off, np.uint64), ref["chunk_off"])
    pos = host(enc.esc_pos_buf, np.uint16)[:cap]
    exp = host(enc.esc_exp_buf, np.uint8)[:cap]
    written = pos != 0xFFFF
    if escapes == "in_slots":
        assert written.all()
    assert np.array_equal(pos[written], ref["esc_pos"][:cap][written])
    assert np.array_equal(exp[written], ref["esc_exp"][:cap][written])
    assert not exp[~written].any()


@pytest.mark.parametrize("mode", MODES)
def test_packed_streams(mode):
    C = 1024
    codec = codec_for(workloads.mixed_words(100_000, 41, wide_fraction=0.05), C)
    use_mode(codec, mode)
    xs = [workloads.mixed_words(n, 900 + n % 97, wide_fraction=w)
          for n, w in [(0, 0.0), (16, 0.1), (3 * TILE + 16, 0.3), (250_000, 0.05)]]
    packed = codec.encode_packed_batch([dev(x) for x in xs])
    for x, p in zip(xs, packed):
        assert p.to_bytes() == O.serialize(O.encode(x, np.frombuffer(codec.codebook, np.uint8), C))
    for x, y in zip(xs, codec.decode_packed_batch(packed)):
        assert np.array_equal(host(y, np.uint16), x)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("n,C,wide", [
    (1, 16, 0.02), (TILE8 + 5, 16, 0.3), (3 * TILE8 + 77, 1024, 0.02), (200_003, 4096, 0.3),
])
def test_e5m2_streams(mode, n, C, wide):
    x = workloads.e5m2_mixed(n, 13 * n + C, wide_fraction=wide)
    codec = t8.codec_for(workloads.e5m2_normal(50_000, 4), C)
    use_mode(codec, mode)
    enc = codec.encode(t8.dev8(x))
    t8.assert_same_stream(codec, enc, x)
    assert np.array_equal(t8.host(codec.decode(enc), np.uint8), x)


@pytest.mark.parametrize("mode", MODES)
def test_e5m2_packed_batch(mode):
    C = 64
    codec = t8.codec_for(workloads.e5m2_normal(50_000, 8), C)
    use_mode(codec, mode)
    xs = [workloads.e5m2_mixed(n, 40 + n % 89, wide_fraction=0.2) for n in (0, 128, TILE8 * 2 + 256)]
    packed = codec.encode_packed_batch([t8.dev8(x) for x in xs])
    for x, p in zip(xs, packed):
        assert p.to_bytes() == O.serialize8(O.encode8(x, np.frombuffer(codec.codebook, np.uint8), C))


@pytest.mark.parametrize("tiles", [sz.SMALL_TILES, sz.SMALL_TILES + 1])
def test_default_boundary(tiles):
    """The last call size that runs pack + finish and the first that runs four launches."""
    n = (tiles - 1) * TILE + 1
    x = workloads.mixed_words(n, tiles, wide_fraction=0.01)
    codec = codec_for(workloads.normal_words(50_000, 9), 1024)
    codec.set_onepass_tiles(0)
    codec.profile(True)
    enc = codec.encode(dev(x))
    times = codec.kernel_times()
    codec.profile(False)
    small = tiles <= sz.SMALL_TILES
    packs = times["encode_pack"][1]        # one per encode attempt (a retry adds one)
    assert packs >= 1
    assert times["encode_finish"][1] == (packs if small else 0)
    assert times["encode_sums"][1] == (0 if small else packs)
    assert_same_stream(codec, enc, x)


def test_launch_counts_and_limit():
    x = dev(workloads.normal_words(5 * TILE, 9))
    codec = codec_for(workloads.normal_words(30_000, 10), 1024)
    codec.set_onepass_tiles(0)
    codec.profile(True)
    codec.encode(x)
    codec.set_small_tiles(0)
    codec.encode(x)
    codec.set_small_tiles(5)
    codec.encode(x)
    codec.set_small_tiles(4)
    codec.encode(x)
    times = codec.kernel_times(reset=True)
    codec.profile(False)
    assert times["encode_pack"][1] == 4
    assert times["encode_finish"][1] == 2
    assert all(times[k][1] == 2 for k in ("encode_sums", "encode_place", "encode_spill"))
    with pytest.raises(sz.SplitZipError) as e:
        codec.set_small_tiles(sz.SMALL_TILES + 1)
    assert e.value.status == sz.E_INVALID


def test_setting_kept_across_calibrations():
    """set_small_tiles and set_onepass_tiles before the first calibration, and every
    calibration makes a new C codec: the settings apply to each."""
    x = dev(workloads.normal_words(3 * TILE, 9))
    codec = sz.Codec(DEV, 1024)
    codec.set_small_tiles(0)
    codec.set_onepass_tiles(0)
    codec.calibrate(dev(workloads.normal_words(30_000, 10)))
    codec.calibrate(dev(workloads.normal_words(30_000, 11)))
    codec.profile(True)
    codec.encode(x)
    times = codec.kernel_times()
    codec.profile(False)
    assert times["encode_sums"][1] == times["encode_pack"][1] >= 1
    assert times["encode_finish"][1] == 0


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("elem", ["bf16", "e5m2"])
def test_many_tiny_segments(mode, elem):
    """300 segments of 0 to 3 pack tiles (many empty or of a few elements) in one call: a
    group of 64 tiles then holds many segments, so the lookup counts inside its bracket;
    every stream equals the oracle's and decodes in one launch."""
    rng = np.random.default_rng(4)
    tile = TILE8 if elem == "e5m2" else TILE
    sizes = []
    for i in range(300):
        kind = rng.integers(0, 4)
        sizes.append(0 if kind == 0 else int(rng.integers(1, 40)) if kind == 1 else
                     int(rng.integers(1, 3 * tile)))
    C = 256
    if elem == "e5m2":
        xs_np = [workloads.e5m2_mixed(n, 900 + i, wide_fraction=0.05) for i, n in enumerate(sizes)]
        codec = t8.codec_for(workloads.e5m2_normal(50_000, 6), C)
        to_dev, check, back = t8.dev8, t8.assert_same_stream, (lambda y: t8.host(y, np.uint8))
    else:
        xs_np = [workloads.mixed_words(n, 900 + i, wide_fraction=0.05) for i, n in enumerate(sizes)]
        codec = codec_for(workloads.normal_words(50_000, 6), C)
        to_dev, check, back = dev, assert_same_stream, (lambda y: host(y, np.uint16))
    use_mode(codec, mode)
    encs = codec.encode_batch([to_dev(x) for x in xs_np])
    for x, e in zip(xs_np, encs):
        check(codec, e, x)
    for x, y in zip(xs_np, codec.decode_batch(encs)):
        assert np.array_equal(back(y), x)


def test_onepass_launch_counts_and_limit():
    """A call into sections of at most ONEPASS_TILES tiles is one launch (BF16 and E5M2); a
    packed stream and a call over the limit run the launch sequences."""
    x = dev(workloads.normal_words(5 * TILE, 9))
    codec = codec_for(workloads.normal_words(30_000, 10), 1024)
    codec.profile(True)
    enc = codec.encode(x)
    codec.set_onepass_tiles(5)
    codec.encode(x)
    codec.set_onepass_tiles(4)
    codec.encode(x)
    codec.set_onepass_tiles()
    codec.encode_packed(x)
    times = codec.kernel_times(reset=True)
    codec.profile(False)
    assert times["encode_onepass"][1] == 2
    assert times["encode_pack"][1] == times["encode_finish"][1] == 2
    assert times["encode_sums"][1] == 0
    assert_same_stream(codec, enc, host(x, np.uint16))
    c8 = t8.codec_for(workloads.e5m2_normal(50_000, 6), 1024)
    c8.profile(True)
    x8 = workloads.e5m2_normal(3 * TILE8, 7)
    e8 = c8.encode(t8.dev8(x8))
    c8.encode_packed(t8.dev8(x8))
    t = c8.kernel_times()
    assert t["encode_onepass"][1] == 1 and t["encode_pack"][1] == 1
    t8.assert_same_stream(c8, e8, x8)


def test_onepass_for_escape_heavy_input_past_the_limit():
    """A call over the one-pass limit runs the launch sequences; after an encode on the same
    stream whose first tile had more escapes than a slot holds, it runs in one launch (same
    bytes); with the one-pass launch off it never does; a call with few escapes in its first
    tile turns the rule off again.  E5M2 likewise."""
    n = 6 * TILE - 7
    x_np = workloads.mixed_words(n, 31, wide_fraction=0.3)
    x = dev(x_np)
    codec = codec_for(workloads.normal_words(30_000, 10), 1024)
    codec.set_onepass_tiles(4)                      # the call has 6 tiles
    codec.profile(True)
    first = codec.encode(x, escape_capacity=n)      # a new workspace: no hint yet
    second = codec.encode(x, escape_capacity=n)
    t = codec.kernel_times(reset=True)
    assert t["encode_onepass"][1] == 1 and t["encode_pack"][1] == 1
    for name in ("sm", "codes", "chunk_off", "esc_pos", "esc_exp"):
        assert torch.equal(getattr(first, name), getattr(second, name)), name
    assert_same_stream(codec, second, x_np)
    codec.set_onepass_tiles(0)
    codec.encode(x, escape_capacity=n)
    t = codec.kernel_times(reset=True)
    assert t["encode_onepass"][1] == 0 and t["encode_pack"][1] == 1
    codec.set_onepass_tiles(4)
    y_np = workloads.normal_words(n, 32)
    y = dev(y_np)
    codec.encode(y, escape_capacity=n)              # after the heavy call: one launch
    last = codec.encode(y, escape_capacity=n)       # after a light one: the launch sequences
    t = codec.kernel_times(reset=True)
    codec.profile(False)
    assert t["encode_onepass"][1] == 1 and t["encode_pack"][1] == 1
    assert_same_stream(codec, last, y_np)

    n8 = 6 * TILE8 - 5
    x8 = workloads.e5m2_mixed(n8, 57, wide_fraction=0.3)
    c8 = t8.codec_for(workloads.e5m2_normal(50_000, 6), 1024)
    c8.set_onepass_tiles(4)
    c8.profile(True)
    e1 = c8.encode(t8.dev8(x8), escape_capacity=n8)
    e2 = c8.encode(t8.dev8(x8), escape_capacity=n8)
    t = c8.kernel_times(reset=True)
    c8.profile(False)
    assert t["encode_onepass"][1] == 1 and t["encode_pack"][1] == 1
    for name in ("sm", "codes", "chunk_off", "esc_pos", "esc_exp"):
        assert torch.equal(getattr(e1, name), getattr(e2, name)), name
    t8.assert_same_stream(c8, e2, x8)



def test_e5m2_clustered_escapes_switch_the_onepass_tile():
    """An E5M2 call of 600 pack tiles whose escapes cluster (blocks of 4096 bytes scaled by
    2^k, k from -8 to 8, as in the escape-stress input): the first call runs one pass on tiles
    of 32768 bytes, and its first tile marks the input escape-heavy and uneven, so the later
    ones run on tiles of 16384; every call's stream equals the oracle's.  A uniform draw of
    the same size stays on the long tiles (the same bytes either way)."""
    n = 600 * TILE8 - 1000
    rng = np.random.default_rng(61)
    z = rng.standard_normal(n).astype(np.float32)
    z *= np.repeat(np.exp2(rng.integers(-8, 9, -(-n // 4096))).astype(np.float32), 4096)[:n]
    x = workloads.e5m2_bits(z)
    c8 = t8.codec_for(workloads.e5m2_normal(50_000, 6), 1024)
    c8.profile(True)
    encs = [c8.encode(t8.dev8(x), escape_capacity=n) for _ in range(3)]
    t = c8.kernel_times(reset=True)
    c8.profile(False)
    assert t["encode_onepass"][1] == 3
    for e in encs[1:]:
        for name in ("sm", "codes", "chunk_off", "esc_pos", "esc_exp"):
            assert torch.equal(getattr(e, name), getattr(encs[0], name)), name
    t8.assert_same_stream(c8, encs[2], x)
    u = workloads.e5m2_mixed(n, 62, wide_fraction=0.3)
    eu = [c8.encode(t8.dev8(u), escape_capacity=n) for _ in range(2)]
    for name in ("sm", "codes", "chunk_off", "esc_pos", "esc_exp"):
        assert torch.equal(getattr(eu[1], name), getattr(eu[0], name)), name
    t8.assert_same_stream(c8, eu[1], u)

@pytest.mark.parametrize("wide", [0.0, 0.02, 1.0])
def test_onepass_many_tiles_and_repeats(wide):
    """1100 tiles (more than one round of the GPU's workgroups, so look-backs find earlier
    tiles still running) with few escapes, 2 % and (uniformly random words) about 94 %; the
    same call three times in a row on one workspace, so every call reads status words that
    the previous call left with the previous launch number."""
    n = 1100 * TILE - 5
    x = workloads.mixed_words(n, 77, wide_fraction=wide) if wide < 1.0 else workloads.random_words(n, 77)
    codec = codec_for(workloads.normal_words(50_000, 9), 4096)
    codec.set_stage_tiles(0)
    xd = dev(x)
    encs = [codec.encode(xd) for _ in range(3)]
    for e in encs[1:]:
        assert e.n_escapes == encs[0].n_escapes
        for name in ("sm", "codes", "chunk_off", "esc_pos", "esc_exp"):
            assert torch.equal(getattr(e, name), getattr(encs[0], name)), name
    assert_same_stream(codec, encs[2], x)


def test_onepass_e5m2_many_tiles():
    """E5M2 in one pass over 700 tiles, with both pack builds, at 20 % escapes and C = 16
    (chunks start inside a lane's group)."""
    n = 700 * TILE8 - 3
    x = workloads.e5m2_mixed(n, 55, wide_fraction=0.2)
    for stage in (0, NEVER):
        c8 = t8.codec_for(workloads.e5m2_normal(50_000, 6), 16)
        c8.set_stage_tiles(stage)
        c8.profile(True)
        e8 = c8.encode(t8.dev8(x))
        assert c8.kernel_times()["encode_onepass"][1] >= 1
        t8.assert_same_stream(c8, e8, x)


def test_onepass_tag_wrap():
    """The launch tag is the low 23 bits of a count kept per workspace: at the wrap to 0 the
    state is cleared before the launch, and the launches before, at and after the wrap (their
    status words all written with other tags) each give the oracle's stream."""
    x = workloads.mixed_words(300 * TILE + 7, 5, wide_fraction=0.05)
    codec = codec_for(workloads.normal_words(50_000, 9), 1024)
    xd = dev(x)
    first = codec.encode(xd)
    stream = torch.cuda.current_stream(DEV).cuda_stream
    sz.splitzip_set_onepass_launches(codec.handle, stream, (1 << 23) - 2)
    for _ in range(3):
        e = codec.encode(xd)
        assert e.to_bytes(codec) == first.to_bytes(codec)
    assert_same_stream(codec, e, x)
    with pytest.raises(sz.SplitZipError):
        sz.splitzip_set_onepass_launches(codec.handle, torch.cuda.Stream(DEV).cuda_stream, 0)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("C", [16, 1024])
def test_exact_escape_counts_per_tile(mode, C):
    """Tiles with exactly 0, 127, 128, 129 (around the 128-entry slot), 1023, 1024, 1025, all
    16384, 5000 and 1 escapes, then a partial tile with 2000, at random places: the stream
    equals the oracle's in every launch sequence and build."""
    rng = np.random.default_rng(8)
    counts = [0, 127, 128, 129, 1023, 1024, 1025, TILE, 5000, 1]
    n = len(counts) * TILE + 5000
    # exponent 127 everywhere (inside any codebook of N(0,1) data), random sign and mantissa
    x = (0x3F80 | rng.integers(0, 128, n) | (rng.integers(0, 2, n) << 15)).astype(np.uint16)
    for t, k in enumerate(counts + [2000]):
        size = min(TILE, n - t * TILE)
        at = t * TILE + rng.choice(size, size=k, replace=False)
        x[at] = (x[at] & 0x807F) | 0x7F00          # exponent 254: an escape
    codec = codec_for(workloads.normal_words(50_000, 9), C)
    assert 254 not in np.frombuffer(codec.codebook, np.uint8) and 127 in np.frombuffer(codec.codebook, np.uint8)
    use_mode(codec, mode)
    enc = codec.encode(dev(x))
    assert enc.n_escapes == sum(counts) + 2000
    assert_same_stream(codec, enc, x)
    assert np.array_equal(host(codec.decode(enc), np.uint16), x)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("C", [16, 1024])
def test_exact_escape_counts_per_tile_e5m2(mode, C):
    """E5M2 blocks of 16384 bytes (a one-pass tile; two make a tile of the launch sequences)
    with exactly 0, 127, 128, 128, 128, 129 escapes (pairs of 127, 256 and 257 around the
    256-entry slot), 8191, 8192, 8193 (around the one-pass stash), all 16384 twice, 16383,
    5000 and 1, then a partial block with 2000, at random places: the stream equals the
    oracle's in every launch sequence and build."""
    rng = np.random.default_rng(18)
    B = 16384
    counts = [0, 127, 128, 128, 128, 129, 8191, 8192, 8193, B, B, B - 1, 5000, 1]
    n = len(counts) * B + 5000
    # exponent 15 everywhere (inside any codebook of N(0,1) data), random sign and mantissa
    x = ((15 << 2) | rng.integers(0, 4, n) | (rng.integers(0, 2, n) << 7)).astype(np.uint8)
    for t, k in enumerate(counts + [2000]):
        size = min(B, n - t * B)
        at = t * B + rng.choice(size, size=k, replace=False)
        x[at] = (x[at] & 0x83) | (30 << 2)          # exponent 30: an escape
    codec = t8.codec_for(workloads.e5m2_normal(50_000, 6), C)
    book = np.frombuffer(codec.codebook, np.uint8)
    assert 30 not in book and 15 in book
    use_mode(codec, mode)
    enc = codec.encode(t8.dev8(x))
    assert enc.n_escapes == sum(counts) + 2000
    t8.assert_same_stream(codec, enc, x)
    assert np.array_equal(t8.host(codec.decode(enc), np.uint8), x)


@pytest.mark.parametrize("onepass", [True, False])
def test_exact_escape_counts_long_e5m2_call(onepass):
    """An E5M2 call of 520 pack tiles of 32768 bytes (past the short-tile limit of the one-pass
    encode, so its one-pass tiles are that long too), whose first 16 tiles hold exactly 0, 8191,
    8192, 8193, 16383, 16384, 16385, 24575, 24576, 24577, 32767, all 32768, 1, 5000, 20000 and
    12345 escapes (around each round of the 8192-entry stash) and the rest 0 to 300: the stream
    equals the oracle's, in one pass and in the launch sequences."""
    rng = np.random.default_rng(28)
    counts = [0, 8191, 8192, 8193, 16383, 16384, 16385, 24575, 24576, 24577, TILE8 - 1, TILE8, 1, 5000, 20000, 12345]
    n_tiles = 520
    counts += [int(c) for c in rng.integers(0, 301, n_tiles - len(counts))]
    n = n_tiles * TILE8 - 77
    x = ((15 << 2) | rng.integers(0, 4, n) | (rng.integers(0, 2, n) << 7)).astype(np.uint8)
    for t, k in enumerate(counts):
        size = min(TILE8, n - t * TILE8)
        k = min(k, size)
        at = t * TILE8 + rng.choice(size, size=k, replace=False)
        x[at] = (x[at] & 0x83) | (30 << 2)          # exponent 30: an escape
    codec = t8.codec_for(workloads.e5m2_normal(50_000, 6), 1024)
    codec.set_onepass_tiles(NEVER if onepass else 0)
    codec.profile(True)
    enc = codec.encode(t8.dev8(x), escape_capacity=n)
    times = codec.kernel_times(reset=True)
    codec.profile(False)
    assert (times["encode_onepass"][1] == 1) == onepass
    assert enc.n_escapes == sum(min(k, min(TILE8, n - t * TILE8)) for t, k in enumerate(counts))
    t8.assert_same_stream(codec, enc, x)
    assert np.array_equal(t8.host(codec.decode(enc), np.uint8), x)
