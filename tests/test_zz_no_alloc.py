"""GPU test of the allocation-free encode (splitzip_encode_noalloc, for callers that cannot
allocate): through the C ABI, its output equals that of splitzip_encode_async, the entry
point it is a variant of, byte for byte, and the oracle's, on two calls in a row whose
second input is smaller; and a call over its scratch limit is refused before any work."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import lossless_bf16_kv_amd as sz
import oracle
import stream_check
import workloads

pytestmark = pytest.mark.gpu

O = oracle.get()
DEV = torch.device("cuda:0")


def dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint8:
        return torch.from_numpy(a.copy()).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).to(DEV)


def launch(codec, fn, xs, caps):
    """Encode device tensors xs through entry point fn into fresh sections; returns the
    Encoded list (n_escapes from the result words) and the result words."""
    encs = [codec.empty_encoded(x.numel(), escape_capacity=c) for x, c in zip(xs, caps)]
    for e in encs:                       # stale bytes that an unwritten entry would show
        for t in (e.sm, e.codes, e.esc_pos_buf, e.esc_exp_buf):
            t.fill_(0x5A)
        e.chunk_off.fill_(-1)
    segs = (sz.splitzip_segment * len(xs))()
    for i, (x, e) in enumerate(zip(xs, encs)):
        segs[i] = e.segment(x.data_ptr() if x.numel() else 0)
    res = torch.zeros(1 + len(xs), dtype=torch.int64, device=DEV)
    fn(codec.handle, segs, torch.cuda.current_stream(DEV).cuda_stream, res.data_ptr())
    return encs, res


def finish(encs, res):
    torch.cuda.synchronize()
    r = res.cpu().tolist()
    for e, E in zip(encs, r[1:]):
        e.n_escapes = int(E)
    return r


def same_sections(a, b):
    assert a.n_escapes == b.n_escapes
    for name in ("sm", "codes", "chunk_off", "esc_pos", "esc_exp"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


def run_pair(codec, inputs, caps, elem=stream_check.ELEM_BF16):
    """Two no-alloc calls in a row (the second input smaller), then the same two through
    splitzip_encode_async; outputs compared with each other and with the oracle."""
    (xa, ca), (xb, cb_) = zip(inputs, caps)
    da, db = [dev(x) for x in xa], [dev(x) for x in xb]
    assert sum(x.size for x in xb) < sum(x.size for x in xa)
    na, ra = launch(codec, sz.splitzip_encode_noalloc, da, ca)
    nb, rb = launch(codec, sz.splitzip_encode_noalloc, db, cb_)
    wa = finish(na, ra)
    wb = finish(nb, rb)
    aa, ra2 = launch(codec, sz.splitzip_encode_async, da, ca)
    ab, rb2 = launch(codec, sz.splitzip_encode_async, db, cb_)
    assert finish(aa, ra2) == wa and finish(ab, rb2) == wb
    assert wa[0] == 0 and wb[0] == 0
    for x_list, n_list, a_list in ((xa, na, aa), (xb, nb, ab)):
        for e1, e2 in zip(n_list, a_list):
            same_sections(e1, e2)
        stream_check.check_cases([stream_check.case_from_encoded(f"segment {i}", e, x, elem)
                                  for i, (x, e) in enumerate(zip(x_list, n_list))])
    return na, nb


def bf16_codec(C=1024):
    codec = sz.Codec(DEV, C)
    codec.calibrate(dev(workloads.normal_words(1 << 18, seed=3)))
    return codec


@pytest.mark.parametrize("small_tiles", [None, 0, -1])
def test_noalloc_matches_async_bf16(small_tiles):
    """A ragged three-segment call, then a smaller one-segment call; one pass (default),
    pack + finish (None), and (small_tiles 0) the four launches with their overflow
    counter."""
    codec = bf16_codec()
    if small_tiles != -1:
        codec.set_onepass_tiles(0)
    if small_tiles not in (None, -1):
        codec.set_small_tiles(small_tiles)
    xa = [workloads.mixed_words(5_000_003, 11), workloads.mixed_words(0, 12),
          workloads.mixed_words(1_234_567, 13)]
    xb = [workloads.mixed_words(300_007, 14)]
    run_pair(codec, (xa, xb), ([x.size // 8 + 64 for x in xa], [x.size // 8 + 64 for x in xb]))


@pytest.mark.parametrize("onepass", [False, True])
def test_noalloc_escape_heavy_and_many_segments(onepass):
    """About 30 % escapes (every tile past its slot, escapes reserved from the overflow
    counter; or, in one pass, placed by each tile) over 61 segments (three set-up launches
    of descriptors), then 2 segments."""
    codec = bf16_codec(256)
    codec.set_small_tiles(0)
    if not onepass:
        codec.set_onepass_tiles(0)
    rng = np.random.default_rng(21)
    xa = [workloads.mixed_words(int(n), 100 + i, wide_fraction=0.3)
          for i, n in enumerate(rng.integers(0, 90_000, 61))]
    xb = [workloads.mixed_words(70_001, 200, wide_fraction=0.3), workloads.mixed_words(16, 201)]
    na, _ = run_pair(codec, (xa, xb), ([x.size for x in xa], [x.size for x in xb]))
    assert sum(e.n_escapes for e in na) > 0.2 * sum(x.size for x in xa)


@pytest.mark.parametrize("first", [3_000_017, 18_000_011])
def test_noalloc_e5m2(first):
    """E5M2 in one pass; the larger first call (550 pack tiles) runs the one-pass encode on
    tiles of 32768 bytes, the second on tiles of 16384, over the same one-pass state."""
    codec = sz.Codec(DEV, 1024, elem="e5m2")
    codec.calibrate(dev(workloads.e5m2_normal(1 << 18, seed=4)))
    xa = [workloads.e5m2_mixed(first, 31, wide_fraction=0.2), workloads.e5m2_mixed(40_000, 32)]
    xb = [workloads.e5m2_mixed(2_099_999, 33, wide_fraction=0.2)]
    run_pair(codec, (xa, xb), ([x.size // 2 + 64 for x in xa], [x.size // 2 + 64 for x in xb]),
             stream_check.ELEM_E5M2)


def test_noalloc_refuses_calls_over_its_scratch():
    """The launch sequences' overflow area is as long as the escape capacity: a capacity
    past the array is refused before any work.  The one-pass launch needs no overflow area
    and takes the same call."""
    codec = bf16_codec()
    codec.set_onepass_tiles(0)
    x = dev(workloads.normal_words(1 << 16, seed=5))
    # an escape capacity whose overflow area (4 bytes an entry) exceeds the fixed array;
    # the escape arrays are really that long, so nothing could be written out of bounds
    cap = sz.NOALLOC_SCRATCH_BYTES // 4 + 1
    enc = codec.empty_encoded(x.numel(), escape_capacity=cap)
    segs = (sz.splitzip_segment * 1)()
    segs[0] = enc.segment(x.data_ptr())
    res = torch.zeros(2, dtype=torch.int64, device=DEV)
    L = sz.lib()
    st = L.splitzip_encode_noalloc(codec.handle, 1, segs, torch.cuda.current_stream(DEV).cuda_stream,
                                   ctypes.c_void_p(res.data_ptr()))
    assert st == sz.E_INVALID
    assert b"scratch" in L.splitzip_last_error()
    torch.cuda.synchronize()
    assert res.cpu().tolist() == [0, 0]
    # the same input within the limit
    ok = codec.empty_encoded(x.numel(), escape_capacity=4096)
    segs[0] = ok.segment(x.data_ptr())
    sz.splitzip_encode_noalloc(codec.handle, segs, torch.cuda.current_stream(DEV).cuda_stream, res.data_ptr())
    torch.cuda.synchronize()
    ok.n_escapes = int(res[1].item())
    stream_check.check_cases([stream_check.case_from_encoded("x", ok, x.cpu().numpy().view(np.uint16))])
    # one pass: the same oversized capacity is fine
    codec.set_onepass_tiles()
    big = codec.empty_encoded(x.numel(), escape_capacity=cap)
    segs[0] = big.segment(x.data_ptr())
    res.zero_()
    sz.splitzip_encode_noalloc(codec.handle, segs, torch.cuda.current_stream(DEV).cuda_stream, res.data_ptr())
    torch.cuda.synchronize()
    assert res[0].item() == 0
    big.n_escapes = int(res[1].item())
    assert big.n_escapes == ok.n_escapes
    stream_check.check_cases([stream_check.case_from_encoded("x", big, x.cpu().numpy().view(np.uint16))])
