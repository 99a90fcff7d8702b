"""CPU tests of the whole-stream checker the full-size GPU parity tests use: a stream the
oracle encodes in one piece passes the window-by-window comparison at any window size, and
a change to any single byte of any section, or to the escape count, fails it."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import stream_check as sc
import workloads

O = oracle.get()


def _whole(x, cb, C, elem):
    if elem == sc.ELEM_BF16:
        r = O.encode(x, cb, C)
        sm = r["sm"]
    else:
        r = O.encode8(x, cb, C)
        sm = r["sm3"]
    return r, sc.Case("t", x, cb, C, sm.copy(), r["codes"].copy(), r["chunk_off"].copy(),
                      r["esc_pos"].copy(), r["esc_exp"].copy(), r["n_escapes"], elem)


def _inputs(elem, n, seed):
    if elem == sc.ELEM_BF16:
        x = workloads.mixed_words(n, seed=seed, wide_fraction=0.2)
        cb, _, _ = O.calibrate(workloads.normal_words(4096, seed=seed + 1))
    else:
        x = workloads.e5m2_mixed(n, seed=seed, wide_fraction=0.2)
        cb, _, _ = O.calibrate8(workloads.e5m2_normal(4096, seed=seed + 1))
    return x, cb


@pytest.mark.parametrize("elem", [sc.ELEM_BF16, sc.ELEM_E5M2])
@pytest.mark.parametrize("n,C,window", [(0, 16, 64), (1, 16, 16), (5000, 16, 64), (5000, 64, 16),
                                        (70001, 1024, 4096), (70001, 4096, 1024),
                                        (65536, 65536, 16384)])
def test_whole_stream_passes_at_any_window(elem, n, C, window):
    x, cb = _inputs(elem, n, seed=n + C)
    _, case = _whole(x, cb, C, elem)
    sc.check_cases([case], window=window)


@pytest.mark.parametrize("elem", [sc.ELEM_BF16, sc.ELEM_E5M2])
def test_any_changed_byte_fails(elem):
    x, cb = _inputs(elem, 9001, seed=3)
    r, base = _whole(x, cb, 64, elem)
    assert base.E > 50
    rng = np.random.default_rng(5)
    for field in ("sm", "codes", "chunk_off", "esc_pos", "esc_exp"):
        for _ in range(6):
            _, case = _whole(x, cb, 64, elem)
            arr = getattr(case, field)
            size = case.E if field.startswith("esc") else arr.size
            i = int(rng.integers(0, size))
            if field == "chunk_off":
                i = int(rng.integers(1, arr.size - 1))    # the ends are checked on their own
            arr[i] ^= 1
            with pytest.raises(AssertionError):
                sc.check_cases([case], window=512)
    # a stream that claims one escape more or less
    for d in (-1, 1):
        _, case = _whole(x, cb, 64, elem)
        case.E += d
        case.chunk_off[-1] = case.E
        with pytest.raises(AssertionError):
            sc.check_cases([case], window=512)


def test_packed_layout_and_header():
    x, cb = _inputs(sc.ELEM_BF16, 4096 + 48, seed=11)
    r = O.encode(x, cb, 256)
    buf = np.frombuffer(O.serialize(r), np.uint8)
    case, head = sc.case_from_packed("p", buf, x, cb, 256)
    assert head == O.header(x.size, 256, r["n_escapes"], cb, 0)
    sc.check_cases([case], window=1024)
    x8, cb8 = _inputs(sc.ELEM_E5M2, 4096 + 128, seed=12)
    r8 = O.encode8(x8, cb8, 256)
    buf8 = np.frombuffer(O.serialize8(r8), np.uint8)
    case8, head8 = sc.case_from_packed("p8", buf8, x8, cb8, 256, sc.ELEM_E5M2)
    assert head8 == O.header(x8.size, 256, r8["n_escapes"], cb8, 1)
    sc.check_cases([case8], window=1024)
    bad = buf.copy()
    bad[64 + 100] ^= 0x80
    case, _ = sc.case_from_packed("p", bad, x, cb, 256)
    with pytest.raises(AssertionError):
        sc.check_cases([case], window=1024)
