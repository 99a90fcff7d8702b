"""Host logic of the transfer plan (no GPU): where streams lie in the arenas and how
consecutive tensors are grouped into copies."""
from __future__ import annotations

import random

from lossless_bf16_kv_amd import PACKED_OFFSET
from lossless_bf16_kv_amd.transfer import SPAN_BYTES, _arena_offsets, _spans


def test_arena_offsets_place_streams_back_to_back_and_aligned():
    rng = random.Random(3)
    for _ in range(200):
        caps = [rng.randint(72, 5000) for _ in range(rng.randint(1, 40))]
        offs, size = _arena_offsets(caps)
        assert all(o % 256 == PACKED_OFFSET for o in offs)
        for a, b, c in zip(offs, offs[1:], caps):
            assert a + c <= b < a + c + 256          # no overlap, less than 256 bytes of gap
        assert size == offs[-1] + caps[-1]


def test_spans_group_consecutive_items_up_to_the_limit():
    rng = random.Random(4)
    for _ in range(300):
        n = rng.randint(1, 60)
        lengths = [rng.choice([1, 1000, SPAN_BYTES // 3, SPAN_BYTES, SPAN_BYTES + 7]) for _ in range(n)]
        starts, pos = [], 0
        for ln in lengths:
            pos += rng.choice([0, 0, 192])              # gaps between items
            starts.append(pos)
            pos += ln
        breaks = {k for k in range(1, n) if rng.random() < 0.1}
        spans = _spans(starts, lengths, lambda k: k not in breaks)
        # a partition of 0..n-1 into consecutive runs
        assert spans[0][0] == 0 and spans[-1][1] == n
        assert all(a < b for a, b in spans) and all(x[1] == y[0] for x, y in zip(spans, spans[1:]))
        for a, b in spans:
            assert all(k not in breaks for k in range(a + 1, b))
            extent = starts[b - 1] + lengths[b - 1] - starts[a]
            assert b - a == 1 or extent <= SPAN_BYTES   # one larger item alone
        # maximal: the next item could not have joined
        for (a, b), (c, _) in zip(spans, spans[1:]):
            assert c in breaks or starts[c] + lengths[c] - starts[a] > SPAN_BYTES
