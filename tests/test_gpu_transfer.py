"""GPU parity of the compressed, pipelined transfer across the host link: what crosses the
link for each tensor is exactly the oracle's serialized stream (header with the tensor's
codebook, then the five sections), and the receiving side's decode returns every tensor bit
for bit, for BF16 with several codebooks and for E5M2; the raw transfer returns the tensors
unchanged; a sending buffer too small for a tensor's escapes is enlarged."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import lossless_bf16_kv_amd as sz
import oracle
import workloads
from lossless_bf16_kv_amd.transfer import TransferPlan
from test_gpu_parity import DEV, dev, host
import test_gpu_e5m2 as t8

pytestmark = pytest.mark.gpu

O = oracle.get()


def test_bf16_transfer_streams_and_round_trip():
    C = 1024
    cals = [workloads.normal_words(60_000, 90 + k, sigma=2.0 ** (6 * k - 6)) for k in range(3)]
    codec = sz.Codec(DEV, C)
    codec.calibrate_books([dev(c) for c in cals])
    sizes = [16 * 1000, 0, 16, 16384 * 3 + 48, 250_000 - 250_000 % 16, 16 * 5]
    xs_np = [workloads.mixed_words(n, 300 + i, wide_fraction=0.05 * (i % 3)) for i, n in enumerate(sizes)]
    books = [i % 3 for i in range(len(sizes))]
    xs = [dev(x) for x in xs_np]
    ys = [torch.full_like(x, 0x5A5A) for x in xs]
    plan = TransferPlan(codec, xs, ys, books)
    for rnd in range(2):                        # the plan's buffers are reused
        for y in ys:
            y.fill_(0x5A5A)
        moved = plan.run(compress=True)
        want = [O.serialize(O.encode(x, np.frombuffer(codec.books[b], np.uint8), C))
                for x, b in zip(xs_np, books)]
        # the spans also carry the gaps between streams (capacity left over, alignment)
        assert sum(len(w) for w in want) <= moved <= plan.send.numel()
        for k, w in enumerate(want):
            assert plan.stream_bytes[k] == len(w)
            o = plan.offs[k]
            assert plan.host[o:o + len(w)].numpy().tobytes() == w       # what crossed the link
            assert np.array_equal(host(ys[k], np.uint16), xs_np[k])
    for y in ys:
        y.zero_()
    assert plan.run(compress=False) == 2 * sum(sizes)
    for x_np, y in zip(xs_np, ys):
        assert np.array_equal(host(y, np.uint16), x_np)


def test_e5m2_transfer():
    C = 256
    codec = t8.codec_for(workloads.e5m2_normal(50_000, 12), C)
    sizes = [128 * 300, 128, 32768 * 2 + 256]
    xs_np = [workloads.e5m2_mixed(n, 50 + i, wide_fraction=0.1) for i, n in enumerate(sizes)]
    xs = [t8.dev8(x) for x in xs_np]
    ys = [torch.zeros_like(x) for x in xs]
    plan = TransferPlan(codec, xs, ys)
    plan.run(compress=True)
    cb = np.frombuffer(codec.codebook, np.uint8)
    for k, x_np in enumerate(xs_np):
        w = O.serialize8(O.encode8(x_np, cb, C))
        o = plan.offs[k]
        assert plan.host[o:o + len(w)].numpy().tobytes() == w
        assert np.array_equal(t8.host(ys[k], np.uint8), x_np)


def test_sending_buffer_grows():
    """A sending buffer sized for 100 escapes, for a tensor with ~94 % escapes: the plan
    takes the size the library reports, encodes again, and what crosses the link is still
    the oracle's stream."""
    x_np = workloads.random_words(16 * 4096, 3)
    codec = sz.Codec(DEV, 1024)
    codec.calibrate(dev(workloads.normal_words(20_000, 4)))
    xs = [dev(x_np)]
    ys = [torch.zeros_like(xs[0])]
    plan = TransferPlan(codec, xs, ys, escapes=[100])
    plan.run(compress=True)
    w = O.serialize(O.encode(x_np, np.frombuffer(codec.codebook, np.uint8), 1024))
    assert plan.stream_bytes[0] == len(w)
    assert plan.host[plan.offs[0]:plan.offs[0] + len(w)].numpy().tobytes() == w
    assert np.array_equal(host(ys[0], np.uint16), x_np)


def test_spans_over_a_pool():
    """Tensors that are consecutive views of one buffer (a KV pool) cross the link in spans
    of up to SPAN_BYTES, compressed and raw; tensors of other allocations never share one."""
    from lossless_bf16_kv_amd.transfer import SPAN_BYTES, _spans
    sizes = [16 * 250_000, 16 * 1000, 0, 16 * 3_000_000, 16 * 700_000, 16 * 64]
    total = sum(sizes)
    pool_in = torch.empty(total, dtype=torch.int16, device=DEV)
    pool_out = torch.zeros(total, dtype=torch.int16, device=DEV)
    xs_np = [workloads.mixed_words(n, 700 + i, wide_fraction=0.03) for i, n in enumerate(sizes)]
    xs, ys, o = [], [], 0
    for x_np, n in zip(xs_np, sizes):
        xs.append(pool_in[o:o + n])
        ys.append(pool_out[o:o + n])
        xs[-1].copy_(dev(x_np))
        o += n
    codec = sz.Codec(DEV, 4096)
    codec.calibrate(dev(workloads.normal_words(50_000, 13)))
    plan = TransferPlan(codec, xs, ys)
    for compress in (True, False, True):
        pool_out.zero_()
        plan.run(compress=compress)
        for x_np, y in zip(xs_np, ys):
            assert np.array_equal(host(y, np.uint16), x_np)
    # grouping rule: consecutive items up to SPAN_BYTES, one larger item alone
    assert _spans([0, 10, 20, 30], [10, 10, 10, 10], lambda k: True) == [(0, 4)]
    big = SPAN_BYTES
    assert _spans([0, 10, 10 + big], [10, big, 5], lambda k: True) == [(0, 1), (1, 2), (2, 3)]
    assert _spans([0, 10, 20], [10, 10, 10], lambda k: k != 2) == [(0, 2), (2, 3)]
