"""GPU parity at the API's limits: a codec with the maximum number of codebooks
(SPLITZIP_MAX_BOOKS = 4096) encoding and decoding 4096 segments in one call, each coded
with its own book."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import lossless_bf16_kv_amd as sz
import oracle
import stream_check
import workloads
from test_gpu_parity import DEV, dev

pytestmark = pytest.mark.gpu

O = oracle.get()
MAX_BOOKS = sz.MAX_BOOKS


def test_max_books_and_4096_segments_in_one_call():
    rng = np.random.default_rng(9)
    # 16 distinct exponents per book, each book a different window and order
    books = [bytes(rng.permutation(np.arange(100 + k % 40, 116 + k % 40)).astype(np.uint8))
             for k in range(MAX_BOOKS)]
    C = 64
    codec = sz.Codec.from_codebooks(books, chunk_size=C, device=DEV)
    assert codec.books == books
    sizes = [int(n) for n in rng.integers(0, 300, MAX_BOOKS)]
    xs_np = [workloads.mixed_words(n, 10 + i, wide_fraction=0.1) for i, n in enumerate(sizes)]
    encs = codec.encode_batch([dev(x) for x in xs_np], books=range(MAX_BOOKS))
    for i, (x, e) in enumerate(zip(xs_np, encs)):
        ref = O.encode(x, np.frombuffer(books[i], np.uint8), C)
        assert e.book == i
        assert e.n_escapes == ref["n_escapes"] and e.compressed_bytes == ref["compressed_bytes"]
    stream_check.check_cases([stream_check.case_from_encoded(f"segment {i}", e, x)
                              for i, (x, e) in enumerate(zip(xs_np, encs))])
    ys = codec.decode_batch(encs)
    got = torch.cat([y.view(torch.int16).reshape(-1) for y in ys]).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, np.concatenate(xs_np))
    with pytest.raises(sz.SplitZipError) as e:
        sz.Codec.from_codebooks(books + [books[0]], chunk_size=C, device=DEV)
    assert e.value.status == sz.E_INVALID
