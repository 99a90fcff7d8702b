"""Whole-stream parity at any size: every byte of a GPU-encoded stream against the oracle.

The oracle encodes the input in windows of whole chunks, several windows at a time on the
host's cores (the oracle call releases the interpreter lock).  Chunks are independent
except for the running escape offset, so a window's stream is the whole stream's slice
over those chunks with its chunk offsets rebased to the window's first escape:

  - sign+mantissa bytes and codes: the same bytes at the window's position (windows start
    at a multiple of 16 elements, so the E5M2 3-bit field stream and the nibbles start on
    a byte);
  - chunk offsets: the whole stream's offsets of the window's chunks minus the first;
  - escapes: the whole stream's escapes from that first offset on.

Every window is compared, the windows' escape counts must add up to E, and the offsets
must start at 0 and end at E, so the comparison covers the whole canonical stream: the
header is checked against the oracle's header writer.  No window needs escape arrays
longer than the window, so the oracle never holds an input-sized escape buffer.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle

WINDOW = 1 << 26
ELEM_BF16, ELEM_E5M2 = 0, 1


def workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def host(a, dtype) -> np.ndarray:
    """A host numpy copy (or view) of a torch tensor or numpy array, reinterpreted as dtype."""
    if isinstance(a, np.ndarray):
        return a.reshape(-1).view(dtype)
    import torch
    if a.dtype == torch.bfloat16:
        a = a.view(torch.int16)
    return a.detach().reshape(-1).cpu().numpy().view(dtype)


def _ceil(a: int, b: int) -> int:
    return -(-a // b)


def _first_diff(a: np.ndarray, b: np.ndarray) -> str:
    if a.size != b.size:
        return f"length {a.size} != {b.size}"
    i = int(np.flatnonzero(a != b)[0])
    return f"first difference at {i}: {int(a[i])} != {int(b[i])}"


class Case:
    """One stream to compare: the input and the host copies of the GPU's sections."""

    def __init__(self, name, x, cb, chunk_size, sm, codes, chunk_off, esc_pos, esc_exp,
                 n_escapes, elem=ELEM_BF16):
        self.name = name
        self.x = x
        self.cb = np.ascontiguousarray(cb, np.uint8)
        self.C = int(chunk_size)
        self.sm, self.codes = sm, codes
        self.chunk_off, self.esc_pos, self.esc_exp = chunk_off, esc_pos, esc_exp
        self.E = int(n_escapes)
        self.elem = elem

    @property
    def n(self) -> int:
        return int(self.x.size)


def case_from_encoded(name, enc, x, elem=ELEM_BF16) -> Case:
    """A Case from the binding's sectioned Encoded (device sections copied to the host)."""
    return Case(name, x, np.frombuffer(enc.codebook, np.uint8), enc.chunk_size,
                host(enc.sm, np.uint8), host(enc.codes, np.uint8),
                host(enc.chunk_off, np.uint64), host(enc.esc_pos, np.uint16),
                host(enc.esc_exp, np.uint8), enc.n_escapes, elem)


def case_from_packed(name, buf: np.ndarray, x, cb, chunk_size, elem=ELEM_BF16):
    """A Case over the sections of a packed stream (the canonical serialization in one
    buffer), plus its header bytes, which the caller compares with the oracle's header."""
    buf = host(buf, np.uint8)
    n = int(x.size)
    C = int(chunk_size)
    E = int(buf[32:40].view(np.uint64)[0])
    sm_len = n if elem == ELEM_BF16 else _ceil(3 * n, 8)
    p = 64
    sm = buf[p:p + sm_len]
    p += sm_len
    codes = buf[p:p + _ceil(n, 2)]
    p += _ceil(n, 2)
    n_chunks = _ceil(n, C)
    chunk_off = buf[p:p + 8 * (n_chunks + 1)].copy().view(np.uint64)
    p += 8 * (n_chunks + 1)
    esc_pos = buf[p:p + 2 * E].copy().view(np.uint16)
    p += 2 * E
    esc_exp = buf[p:p + E]
    p += E
    assert p == buf.size, f"{name}: stream length {buf.size}, sections end at {p}"
    return Case(name, x, cb, C, sm, codes, chunk_off, esc_pos, esc_exp, E, elem), bytes(buf[:64])


def _check_window(case: Case, lo: int, window: int):
    O = oracle.get()
    hi = min(case.n, lo + window)
    xs = case.x[lo:hi]
    if case.elem == ELEM_BF16:
        ref = O.encode(xs, case.cb, case.C)
        sm_ref, sm_at = ref["sm"], lo
    else:
        ref = O.encode8(xs, case.cb, case.C)
        sm_ref, sm_at = ref["sm3"], 3 * lo // 8
    errs = []
    c0 = lo // case.C
    c1 = c0 + ref["chunk_off"].size - 1
    base = int(case.chunk_off[c0])
    offs = case.chunk_off[c0:c1 + 1].astype(np.int64) - base
    if not np.array_equal(offs, ref["chunk_off"].astype(np.int64)):
        errs.append("chunk_off " + _first_diff(offs, ref["chunk_off"].astype(np.int64)))
    got = case.sm[sm_at:sm_at + sm_ref.size]
    if not np.array_equal(got, sm_ref):
        errs.append("sm " + _first_diff(got, sm_ref))
    got = case.codes[lo // 2:lo // 2 + ref["codes"].size]
    if not np.array_equal(got, ref["codes"]):
        errs.append("codes " + _first_diff(got, ref["codes"]))
    e = int(ref["n_escapes"])
    got = case.esc_pos[base:base + e]
    if not np.array_equal(got, ref["esc_pos"]):
        errs.append("esc_pos " + _first_diff(got, ref["esc_pos"]))
    got = case.esc_exp[base:base + e]
    if not np.array_equal(got, ref["esc_exp"]):
        errs.append("esc_exp " + _first_diff(got, ref["esc_exp"]))
    return case.name, lo, errs, e


def check_cases(cases, window: int = WINDOW) -> None:
    """Compare every byte of every case's stream with the oracle (see the module text)."""
    jobs = []
    for c in cases:
        n_chunks = _ceil(c.n, c.C)
        sm_len = c.n if c.elem == ELEM_BF16 else _ceil(3 * c.n, 8)
        assert c.sm.size == sm_len, f"{c.name}: sm length {c.sm.size} != {sm_len}"
        assert c.codes.size == _ceil(c.n, 2), f"{c.name}: codes length"
        assert c.chunk_off.size == n_chunks + 1, f"{c.name}: chunk_off length"
        assert int(c.chunk_off[0]) == 0 and int(c.chunk_off[-1]) == c.E, f"{c.name}: offsets end"
        assert c.esc_pos.size >= c.E and c.esc_exp.size >= c.E, f"{c.name}: escape arrays"
        w = max(window, c.C)       # powers of two: whole chunks, a multiple of 16 elements
        jobs += [(c, lo, w) for lo in range(0, c.n, w)]
    totals = {id(c): 0 for c in cases}
    failures = []
    with cf.ThreadPoolExecutor(workers()) as ex:
        futs = {ex.submit(_check_window, c, lo, w): c for c, lo, w in jobs}
        for f in cf.as_completed(futs):
            name, lo, errs, e = f.result()
            totals[id(futs[f])] += e
            if errs:
                failures.append(f"{name} window at {lo}: " + "; ".join(errs))
    assert not failures, f"{len(failures)} windows differ from the oracle: " + " | ".join(sorted(failures)[:4])
    for c in cases:
        assert totals[id(c)] == c.E, f"{c.name}: windows hold {totals[id(c)]} escapes, stream {c.E}"
