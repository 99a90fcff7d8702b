"""Compressed transfer of a batch of tensors across a link, pipelined.

The method exists to cut KV-cache transfer time between prefill and decode workers: the
sending GPU compresses, the receiving GPU decompresses, and both run far faster than the
link, so the bytes saved become time saved ([README] *FAQ*; [ABSTRACT], end-to-end transfer
speedup).

One GPU plays both ends here.  The link is the PCIe path through pinned host memory:
device to host (the sender's side), then host to device (the receiver's side), about
56 GB/s each way on MI355X, two orders of magnitude below HBM.  Each tensor (for KV, one
layer's K or V) becomes one packed stream, and the streams lie back to back in one device
arena on each side, mirrored by one pinned host arena:

    encode every tensor into the sending arena (one launch sequence)
    for each span of consecutive streams (up to 32 MiB, or one larger stream):
        device-to-host copy of the span -> host-to-device copy of the span
    decode every stream from the receiving arena (one launch)

on three streams, so span j's host-to-device copy overlaps span j+1's device-to-host copy.
Copies are grouped into spans because the link pays a fixed cost per copy: pipelined copies
of about 5 MB moved 26 GB/s, of 64 MB 47 GB/s.  The sender encodes everything before the
first copy because the runtime performs device-to-host copies into pinned memory with a
copy kernel that holds compute units while it waits on PCIe: an encode running beside it
took 30 times as long.  On a real sender the network card's DMA engine reads the buffers,
and the encode (about 0.3 ms per GB) is a small part of the transfer either way.

The raw transfer moves the uncompressed tensors through the same copies on the same
streams, with the same grouping where consecutive tensors are adjacent in memory (as in a
KV pool).  A plan allocates every buffer once, so repeated runs time only the transfer.
"""
from __future__ import annotations

from . import (E_CAPACITY, PACKED_OFFSET, Codec, SplitZipError, splitzip_decode_packed,
               splitzip_encode_packed, splitzip_packed)

SPAN_BYTES = 32 << 20      # copies group consecutive tensors up to this many bytes


def _arena_offsets(caps):
    """Offsets of streams of the given capacities placed back to back, each 64 bytes before
    a 256-byte boundary (so that the sections after the 64-byte header start on whole
    cache lines, as the kernels prefer), and the arena size."""
    offs, end = [], 0
    for c in caps:
        o = end + (PACKED_OFFSET - end) % 256
        offs.append(o)
        end = o + c
    return offs, end


def _spans(starts, lengths, adjacent):
    """Group consecutive items into (first, last + 1) runs of at most SPAN_BYTES (an item
    larger than that alone); adjacent(k) tells whether item k may join item k - 1's run."""
    spans, k0 = [], 0
    for k in range(1, len(starts) + 1):
        if k == len(starts) or not adjacent(k) or \
                starts[k] + lengths[k] - starts[k0] > SPAN_BYTES:
            spans.append((k0, k))
            k0 = k
    return spans


class TransferPlan:
    """Buffers and streams to move tensors xs (device) into ys (device, same sizes) across
    the host link, compressed (`run(compress=True)`) or raw (`run(compress=False)`).

    Packed streams need numel a multiple of 16 (BF16) or 128 (E5M2).  books[i] is the
    codebook of tensor i (default 0).  `escapes`: escape capacity per tensor for the
    sending arena (default: the codec's guess from its calibration); a tensor with more
    escapes gets a larger arena during run(), which is then slower."""

    def __init__(self, codec: Codec, xs, ys, books=None, escapes=None):
        codec._need_handle()
        if len(xs) != len(ys):
            raise ValueError("xs and ys must have the same length")
        self.codec = codec
        self.xs = [codec._elements(x) for x in xs]
        self.ys = [codec._elements(y) for y in ys]
        for x, y in zip(self.xs, self.ys):
            if x.numel() != y.numel():
                raise ValueError("each output must have its input's size")
        self.books = list(books) if books is not None else [0] * len(xs)
        self._allocate([codec.packed_capacity(x.numel(), None if escapes is None else escapes[i])
                        for i, x in enumerate(self.xs)])
        import torch
        self.streams = [torch.cuda.Stream(device=codec.device) for _ in range(3)]   # default priority
        k = len(self.xs)
        self.stream_bytes = [0] * k
        self.n_escapes = [0] * k

    def close(self) -> None:
        """Free the workspaces the codec keeps for this plan's streams (the plan is unusable
        afterwards; the codec is not)."""
        for st in getattr(self, "streams", []):
            self.codec.release_stream(st)
        self.streams = []

    def _allocate(self, caps) -> None:
        """Sending and receiving arenas for streams of capacities caps, and the pinned host
        arena (large enough for the raw bytes too)."""
        import torch
        self.caps = list(caps)
        self.offs, size = _arena_offsets(self.caps)
        dev = self.codec.device
        self.send = torch.empty(size, dtype=torch.uint8, device=dev)
        self.recv = torch.empty(size, dtype=torch.uint8, device=dev)
        self.raw_bytes = [x.numel() * x.element_size() for x in self.xs]
        self.raw_offs = [sum(self.raw_bytes[:k]) for k in range(len(self.xs))]
        self.host = torch.empty(max(size, sum(self.raw_bytes)), dtype=torch.uint8, pin_memory=True)

    def _encode_all(self, stream) -> None:
        """Encode every tensor into the sending arena in one launch sequence on `stream` and
        wait for it (the copies need the stream sizes).  If some stream does not fit, the
        arenas are allocated again with the sizes the library reports and the batch encoded
        again; no buffer is in use then, since every run ends with a synchronization."""
        import torch
        for attempt in range(2):
            segs = (splitzip_packed * len(self.xs))()
            base = self.send.data_ptr()
            for k, x in enumerate(self.xs):
                segs[k] = splitzip_packed(x.data_ptr() if x.numel() else None, x.numel(),
                                          base + self.offs[k], self.caps[k], 0, 0, self.books[k], 0)
            st = splitzip_encode_packed(self.codec.handle, segs, stream.cuda_stream)
            if st != E_CAPACITY:
                break
            if attempt:
                raise SplitZipError(E_CAPACITY, "stream buffers still too small after a resize")
            torch.cuda.synchronize(self.codec.device)
            self._allocate([max(c, int(segs[k].stream_bytes)) for k, c in enumerate(self.caps)])
        for k in range(len(self.xs)):
            self.stream_bytes[k], self.n_escapes[k] = int(segs[k].stream_bytes), int(segs[k].n_escapes)

    def run(self, compress: bool = True) -> int:
        """Move every tensor across the link and wait for the last decode (or copy); returns
        the bytes that crossed the link (each counted once, device to host)."""
        import torch
        s_d2h, s_h2d, s_dec = self.streams
        codec = self.codec
        # everything this run reads was written on the caller's stream
        start = torch.cuda.current_stream(codec.device)
        for s in self.streams:
            s.wait_stream(start)
        if compress:
            self._encode_all(s_d2h)          # the copies below follow it on the same stream
            starts, lengths = self.offs, self.stream_bytes
            spans = _spans(starts, lengths, lambda k: True)
            # a span runs from its first stream's start to its last stream's end
            pieces = [(self.send, self.recv, self.offs[a], self.offs[a],
                       self.offs[b - 1] + self.stream_bytes[b - 1] - self.offs[a]) for a, b in spans]
        else:
            xs, ys, nb = self.xs, self.ys, self.raw_bytes

            def adjacent(k):
                # back to back in the same allocation, inputs and outputs alike
                return all(t[k].untyped_storage().data_ptr() == t[k - 1].untyped_storage().data_ptr()
                           and t[k].data_ptr() == t[k - 1].data_ptr() + nb[k - 1] for t in (xs, ys))
            spans = _spans([xs[k].data_ptr() for k in range(len(xs))], nb, adjacent)
            pieces = []
            for a, b in spans:
                n = sum(nb[a:b])
                if n:
                    pieces.append((xs[a], ys[a], None, self.raw_offs[a], n))
        moved = 0
        for src, dst, dev_off, host_off, n in pieces:
            if dev_off is None:                      # raw: the tensors themselves
                s = src.view(-1).view(torch.uint8)
                s = torch.as_strided(s, (n,), (1,))
                d = torch.as_strided(dst.view(-1).view(torch.uint8), (n,), (1,))
            else:
                s, d = src[dev_off:dev_off + n], dst[dev_off:dev_off + n]
            h = self.host[host_off:host_off + n]
            ev = torch.cuda.Event()
            with torch.cuda.stream(s_d2h):
                h.copy_(s, non_blocking=True)
                ev.record(s_d2h)
            with torch.cuda.stream(s_h2d):
                s_h2d.wait_event(ev)
                d.copy_(h, non_blocking=True)
            moved += n
        if compress:
            # the receiver: one decode launch over every stream once the last span has landed
            s_dec.wait_stream(s_h2d)
            segs = (splitzip_packed * len(self.xs))()
            base = self.recv.data_ptr()
            for k, y in enumerate(self.ys):
                segs[k] = splitzip_packed(y.data_ptr() if y.numel() else None, y.numel(),
                                          base + self.offs[k], self.stream_bytes[k], 0, 0, 0, 0)
            splitzip_decode_packed(codec.handle, segs, s_dec.cuda_stream)
        for s in self.streams:
            start.wait_stream(s)
        torch.cuda.synchronize(codec.device)
        return moved


__all__ = ["TransferPlan", "SPAN_BYTES"]
