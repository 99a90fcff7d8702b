"""SplitZip BF16 exponent-split codec on AMD MI355X (gfx950): Python binding.

Every step of calibrate / encode / decode runs in the HIP kernels of
``libsplitzip.so`` (sources in ``csrc/``); this module only marshals arguments
through ctypes.  PyTorch provides device memory and streams.  There is no CPU
fallback: if the library is missing or no GPU is present the calls raise.

Two layers, mirroring the codec API of "SplitZip: Ultra-Fast Lossless KV
Compression for Disaggregated LLM Serving" (README, "Codec API"):

* the C ABI under the same names (``splitzip_calibrate``, ``splitzip_encode``,
  ``splitzip_decode``, ``splitzip_free`` and host helpers), taking raw device
  pointers as Python ints;
* ``Codec(device, chunk_size)`` with ``calibrate(x) -> coverage``,
  ``encode(x) -> Encoded`` (``.compressed_bytes``) and ``decode(encoded)``,
  plus ``encode_batch`` / ``decode_batch`` for ragged batches in one launch,
  and ``calibrate_books`` for several codebooks (per layer, per K and V);
* ``histograms`` / ``exponent_stats``: the exponent entropy and top-16 coverage
  analysis of BF16 tensors.

``Codec(..., elem="e5m2")`` codes FP8 E5M2 tensors with the same calls (README "FAQ" and
arXiv abstract: the codec also runs on top of an FP8 E5M2 KV cache): the 3-bit
sign+mantissa fields form a bit stream, the 5-bit exponents take 4-bit codes and escapes.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsplitzip.so")

OK, E_INVALID, E_NOMEM, E_DEVICE, E_CODEBOOK, E_FORMAT, E_CAPACITY = range(7)
HEADER_BYTES = 64
ONEPASS_TILES = 2048    # section encodes of at most this many tiles run one launch
SMALL_TILES = 4096      # other encodes of at most this many tiles run pack + finish (two launches)
STAGE_TILES = 1024      # larger calls run the kernel builds tuned for escape-heavy inputs
PRIVATE_OVERFLOW_BYTES = 256 << 20   # calls up to this much per-tile overflow scratch use it
MIN_CHUNK, MAX_CHUNK = 16, 65536
MAX_BOOKS = 4096
ELEM_BF16, ELEM_E5M2 = 0, 1
ELEMS = {"bf16": ELEM_BF16, "e5m2": ELEM_E5M2}


class SplitZipError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"splitzip status {status}: {message}")
        self.status = status


class splitzip_segment(ctypes.Structure):
    """Mirror of ``splitzip_segment`` in include/splitzip.h."""
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("n", ctypes.c_uint64),
        ("sm", ctypes.c_void_p),
        ("codes", ctypes.c_void_p),
        ("chunk_off", ctypes.c_void_p),
        ("esc_pos", ctypes.c_void_p),
        ("esc_exp", ctypes.c_void_p),
        ("esc_capacity", ctypes.c_uint64),
        ("n_escapes", ctypes.c_uint64),
        ("compressed_bytes", ctypes.c_uint64),
        ("book", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


class splitzip_packed(ctypes.Structure):
    """Mirror of ``splitzip_packed`` in include/splitzip.h."""
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("n", ctypes.c_uint64),
        ("buf", ctypes.c_void_p),
        ("buf_bytes", ctypes.c_uint64),
        ("stream_bytes", ctypes.c_uint64),
        ("n_escapes", ctypes.c_uint64),
        ("book", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsplitzip.so (built by ``__graft_entry__.build()``); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise SplitZipError(E_DEVICE, f"{LIB_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, u64, u32, i32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int
    P = ctypes.POINTER
    L.splitzip_calibrate.argtypes = [vp, u64, u32, vp, P(vp), P(ctypes.c_double), P(u64)]
    L.splitzip_codec_from_codebook.argtypes = [P(ctypes.c_uint8), u32, P(vp)]
    L.splitzip_calibrate_books.argtypes = [u32, P(vp), P(u64), u32, vp, P(vp), P(ctypes.c_double),
                                           P(u64)]
    L.splitzip_codec_from_codebooks.argtypes = [u32, P(ctypes.c_uint8), u32, P(vp)]
    L.splitzip_codec_books.argtypes = [vp, P(u32), P(ctypes.c_uint8)]
    L.splitzip_histogram.argtypes = [u32, P(vp), P(u64), vp, P(u64)]
    L.splitzip_exponent_stats.argtypes = [P(u64), P(ctypes.c_double), P(ctypes.c_double),
                                          P(ctypes.c_uint8), P(u32)]
    L.splitzip_codec_info.argtypes = [vp, P(ctypes.c_uint8), P(u32), P(i32)]
    L.splitzip_calibrate_e5m2.argtypes = [vp, u64, u32, vp, P(vp), P(ctypes.c_double), P(u64)]
    L.splitzip_calibrate_books_e5m2.argtypes = [u32, P(vp), P(u64), u32, vp, P(vp),
                                                P(ctypes.c_double), P(u64)]
    L.splitzip_codec_from_codebooks_e5m2.argtypes = [u32, P(ctypes.c_uint8), u32, P(vp)]
    L.splitzip_codec_element.argtypes = [vp, P(u32)]
    L.splitzip_histogram_e5m2.argtypes = [u32, P(vp), P(u64), vp, P(u64)]
    L.splitzip_e5m2_compressed_bytes.argtypes = [u64, u32, u64]
    L.splitzip_e5m2_compressed_bytes.restype = u64
    L.splitzip_encode.argtypes = [vp, u32, P(splitzip_segment), vp]
    L.splitzip_encode_async.argtypes = [vp, u32, P(splitzip_segment), vp, vp]
    L.splitzip_encode_noalloc.argtypes = [vp, u32, P(splitzip_segment), vp, vp]
    L.splitzip_decode.argtypes = [vp, u32, P(splitzip_segment), vp, vp]
    L.splitzip_encode_packed.argtypes = [vp, u32, P(splitzip_packed), vp, vp]
    L.splitzip_decode_packed.argtypes = [vp, u32, P(splitzip_packed), vp, vp]
    L.splitzip_profile.argtypes = [vp, i32]
    L.splitzip_set_small_tiles.argtypes = [vp, u32]
    L.splitzip_set_onepass_tiles.argtypes = [vp, u32]
    L.splitzip_set_onepass_launches.argtypes = [vp, vp, u64]
    L.splitzip_set_stage_tiles.argtypes = [vp, u32]
    L.splitzip_set_private_overflow.argtypes = [vp, ctypes.c_uint64]
    L.splitzip_profile_read.argtypes = [vp, vp, P(ctypes.c_double), P(u64), i32]
    L.splitzip_free.argtypes = [vp]
    L.splitzip_free.restype = None
    L.splitzip_release_stream.argtypes = [vp, vp]
    L.splitzip_workspace_bytes.argtypes = [vp, vp, P(u64)]
    L.splitzip_chunk_count.argtypes = [u64, u32]
    L.splitzip_chunk_count.restype = u64
    L.splitzip_compressed_bytes.argtypes = [u64, u32, u64]
    L.splitzip_compressed_bytes.restype = u64
    L.splitzip_write_header.argtypes = [vp, u32, u64, u64, P(ctypes.c_uint8)]
    L.splitzip_read_header.argtypes = [P(ctypes.c_uint8), u64, P(u64), P(u32), P(u64),
                                       P(ctypes.c_uint8), P(u32)]
    L.splitzip_check_header.argtypes = [vp, P(ctypes.c_uint8), u64, P(u32)]
    L.splitzip_status_string.argtypes = [i32]
    L.splitzip_status_string.restype = ctypes.c_char_p
    L.splitzip_last_error.argtypes = []
    L.splitzip_last_error.restype = ctypes.c_char_p
    for f in ("splitzip_calibrate", "splitzip_codec_from_codebook", "splitzip_codec_info",
              "splitzip_calibrate_books", "splitzip_codec_from_codebooks", "splitzip_codec_books",
              "splitzip_histogram", "splitzip_exponent_stats", "splitzip_encode_packed",
              "splitzip_decode_packed",
              "splitzip_encode", "splitzip_encode_async", "splitzip_encode_noalloc", "splitzip_decode",
              "splitzip_write_header", "splitzip_profile", "splitzip_profile_read",
              "splitzip_set_small_tiles", "splitzip_set_stage_tiles", "splitzip_set_private_overflow",
              "splitzip_set_onepass_tiles", "splitzip_set_onepass_launches",
              "splitzip_read_header", "splitzip_check_header", "splitzip_calibrate_e5m2",
              "splitzip_calibrate_books_e5m2", "splitzip_codec_from_codebooks_e5m2",
              "splitzip_codec_element", "splitzip_histogram_e5m2", "splitzip_release_stream",
              "splitzip_workspace_bytes"):
        getattr(L, f).restype = i32
    _lib = L
    return L


def _check(status: int, allow=()) -> int:
    if status != OK and status not in allow:
        msg = lib().splitzip_last_error().decode() or lib().splitzip_status_string(status).decode()
        raise SplitZipError(status, msg)
    return status


def _u8buf(b: bytes):
    return (ctypes.c_uint8 * len(b)).from_buffer_copy(b) if b else (ctypes.c_uint8 * 1)()


# ---- C ABI, same names (pointers are Python ints) -------------------------------------

def splitzip_calibrate(d_cal: int, n_cal: int, chunk_size: int, stream: int = 0):
    """-> (codec handle, coverage, histogram list[256])."""
    h = ctypes.c_void_p()
    cov = ctypes.c_double()
    hist = (ctypes.c_uint64 * 256)()
    _check(lib().splitzip_calibrate(d_cal or None, n_cal, chunk_size, stream or None,
                                    ctypes.byref(h), ctypes.byref(cov), hist))
    return h.value, cov.value, list(hist)


def splitzip_codec_from_codebook(codebook: bytes, chunk_size: int) -> int:
    if len(codebook) != 16:
        raise ValueError("codebook must be 16 bytes")
    h = ctypes.c_void_p()
    _check(lib().splitzip_codec_from_codebook(_u8buf(bytes(codebook)), chunk_size, ctypes.byref(h)))
    return h.value


def _ptr_array(ptrs):
    return (ctypes.c_void_p * len(ptrs))(*[p or None for p in ptrs])


def splitzip_calibrate_books(d_cal, n_cal, chunk_size: int, stream: int = 0):
    """d_cal, n_cal: one device pointer and size per book.
    -> (codec handle, coverage list, histogram list of 256-lists)."""
    k = len(d_cal)
    h = ctypes.c_void_p()
    cov = (ctypes.c_double * max(k, 1))()
    hist = (ctypes.c_uint64 * (256 * max(k, 1)))()
    _check(lib().splitzip_calibrate_books(k, _ptr_array(d_cal), (ctypes.c_uint64 * max(k, 1))(*n_cal),
                                          chunk_size, stream or None, ctypes.byref(h), cov, hist))
    return h.value, list(cov)[:k], [list(hist[256 * b:256 * b + 256]) for b in range(k)]


def splitzip_codec_from_codebooks(codebooks: bytes, chunk_size: int) -> int:
    """codebooks: 16 bytes per book, concatenated."""
    if not codebooks or len(codebooks) % 16:
        raise ValueError("codebooks must be a non-empty multiple of 16 bytes")
    h = ctypes.c_void_p()
    _check(lib().splitzip_codec_from_codebooks(len(codebooks) // 16, _u8buf(bytes(codebooks)),
                                               chunk_size, ctypes.byref(h)))
    return h.value


def splitzip_codec_books(codec: int) -> list:
    """The codec's codebooks, 16 bytes each."""
    k = ctypes.c_uint32()
    _check(lib().splitzip_codec_books(codec, ctypes.byref(k), None))
    buf = (ctypes.c_uint8 * (16 * k.value))()
    _check(lib().splitzip_codec_books(codec, ctypes.byref(k), buf))
    raw = bytes(buf)
    return [raw[16 * b:16 * b + 16] for b in range(k.value)]


def splitzip_calibrate_e5m2(d_cal: int, n_cal: int, chunk_size: int, stream: int = 0):
    """E5M2 codec -> (codec handle, coverage, histogram list[32])."""
    h = ctypes.c_void_p()
    cov = ctypes.c_double()
    hist = (ctypes.c_uint64 * 32)()
    _check(lib().splitzip_calibrate_e5m2(d_cal or None, n_cal, chunk_size, stream or None,
                                         ctypes.byref(h), ctypes.byref(cov), hist))
    return h.value, cov.value, list(hist)


def splitzip_calibrate_books_e5m2(d_cal, n_cal, chunk_size: int, stream: int = 0):
    """E5M2 codec with one book per calibration tensor -> (handle, coverages, 32-bin hists)."""
    k = len(d_cal)
    h = ctypes.c_void_p()
    cov = (ctypes.c_double * max(k, 1))()
    hist = (ctypes.c_uint64 * (32 * max(k, 1)))()
    _check(lib().splitzip_calibrate_books_e5m2(k, _ptr_array(d_cal), (ctypes.c_uint64 * max(k, 1))(*n_cal),
                                               chunk_size, stream or None, ctypes.byref(h), cov, hist))
    return h.value, list(cov)[:k], [list(hist[32 * b:32 * b + 32]) for b in range(k)]


def splitzip_codec_from_codebooks_e5m2(codebooks: bytes, chunk_size: int) -> int:
    if not codebooks or len(codebooks) % 16:
        raise ValueError("codebooks must be a non-empty multiple of 16 bytes")
    h = ctypes.c_void_p()
    _check(lib().splitzip_codec_from_codebooks_e5m2(len(codebooks) // 16, _u8buf(bytes(codebooks)),
                                                    chunk_size, ctypes.byref(h)))
    return h.value


def splitzip_codec_element(codec: int) -> int:
    e = ctypes.c_uint32()
    _check(lib().splitzip_codec_element(codec, ctypes.byref(e)))
    return e.value


def splitzip_histogram_e5m2(d_x, n, stream: int = 0) -> list:
    """Exponent histograms of several E5M2 device tensors in one pass -> list of 32-lists."""
    k = len(d_x)
    hist = (ctypes.c_uint64 * (32 * max(k, 1)))()
    _check(lib().splitzip_histogram_e5m2(k, _ptr_array(d_x), (ctypes.c_uint64 * max(k, 1))(*n),
                                         stream or None, hist))
    return [list(hist[32 * b:32 * b + 32]) for b in range(k)]


def splitzip_histogram(d_x, n, stream: int = 0) -> list:
    """Exponent histograms of several device tensors in one pass -> list of 256-lists."""
    k = len(d_x)
    hist = (ctypes.c_uint64 * (256 * max(k, 1)))()
    _check(lib().splitzip_histogram(k, _ptr_array(d_x), (ctypes.c_uint64 * max(k, 1))(*n),
                                    stream or None, hist))
    return [list(hist[256 * b:256 * b + 256]) for b in range(k)]


def splitzip_exponent_stats(hist) -> dict:
    """Entropy (bits), top-16 codebook, its coverage and the distinct exponent count of
    one exponent histogram (host computation): 256 bins (BF16) or 32 (E5M2, padded with
    zero bins)."""
    if len(hist) == 32:
        hist = list(hist) + [0] * 224
    if len(hist) != 256:
        raise ValueError("hist must have 256 (BF16) or 32 (E5M2) bins")
    h = (ctypes.c_uint64 * 256)(*[int(v) for v in hist])
    ent, cov = ctypes.c_double(), ctypes.c_double()
    cb = (ctypes.c_uint8 * 16)()
    d = ctypes.c_uint32()
    _check(lib().splitzip_exponent_stats(h, ctypes.byref(ent), ctypes.byref(cov), cb, ctypes.byref(d)))
    return {"entropy_bits": ent.value, "coverage": cov.value, "codebook": bytes(cb),
            "distinct": d.value}


def splitzip_codec_info(codec: int):
    cb = (ctypes.c_uint8 * 16)()
    c, d = ctypes.c_uint32(), ctypes.c_int()
    _check(lib().splitzip_codec_info(codec, cb, ctypes.byref(c), ctypes.byref(d)))
    return bytes(cb), c.value, d.value


def splitzip_encode(codec: int, segs, stream: int = 0) -> int:
    """Encode a ctypes array of splitzip_segment in place; returns OK or E_CAPACITY."""
    return _check(lib().splitzip_encode(codec, len(segs), segs, stream or None), allow=(E_CAPACITY,))


def splitzip_encode_async(codec: int, segs, stream: int, d_result: int) -> None:
    """Enqueue an encode; error bits and per-segment E land in d_result (device u64[1+n])."""
    _check(lib().splitzip_encode_async(codec, len(segs), segs, stream or None, d_result))


def splitzip_encode_noalloc(codec: int, segs, stream: int, d_result: int) -> None:
    """splitzip_encode_async with its scratch in the library's fixed device array: the call
    allocates nothing (for callers that cannot allocate); the same d_result contract."""
    _check(lib().splitzip_encode_noalloc(codec, len(segs), segs, stream or None, d_result))


NOALLOC_SCRATCH_BYTES = 64 << 20      # SPLITZIP_NOALLOC_SCRATCH_BYTES
NOALLOC_MAX_SEGMENTS = 4096           # SPLITZIP_NOALLOC_MAX_SEGMENTS


def splitzip_decode(codec: int, segs, stream: int = 0, d_error: int = 0) -> None:
    _check(lib().splitzip_decode(codec, len(segs), segs, stream or None, d_error or None))


def splitzip_encode_packed(codec: int, segs, stream: int = 0, d_result: int = 0) -> int:
    """Encode a ctypes array of splitzip_packed; blocking (OK or E_CAPACITY) unless d_result."""
    return _check(lib().splitzip_encode_packed(codec, len(segs), segs, stream or None, d_result or None),
                  allow=(E_CAPACITY,))


def splitzip_decode_packed(codec: int, segs, stream: int = 0, d_error: int = 0) -> None:
    _check(lib().splitzip_decode_packed(codec, len(segs), segs, stream or None, d_error or None))


KERNELS = ("encode_pack", "encode_sums", "encode_place", "encode_spill", "decode", "encode_finish",
           "encode_onepass")


def splitzip_set_onepass_tiles(codec: int, max_tiles: int) -> None:
    _check(lib().splitzip_set_onepass_tiles(codec, max_tiles))


def splitzip_set_onepass_launches(codec: int, stream: int, launches: int) -> None:
    _check(lib().splitzip_set_onepass_launches(codec, stream or None, launches))


def splitzip_set_small_tiles(codec: int, max_tiles: int) -> None:
    _check(lib().splitzip_set_small_tiles(codec, max_tiles))


def splitzip_set_stage_tiles(codec: int, min_tiles: int) -> None:
    _check(lib().splitzip_set_stage_tiles(codec, min_tiles))


def splitzip_set_private_overflow(codec: int, max_bytes: int) -> None:
    _check(lib().splitzip_set_private_overflow(codec, max_bytes))


def splitzip_profile(codec: int, enable: bool) -> None:
    _check(lib().splitzip_profile(codec, 1 if enable else 0))


def splitzip_profile_read(codec: int, stream: int = 0, reset: bool = False) -> dict:
    """{kernel: (mean ms, launches timed)} for the calls made on `stream`."""
    avg = (ctypes.c_double * len(KERNELS))()
    cnt = (ctypes.c_uint64 * len(KERNELS))()
    _check(lib().splitzip_profile_read(codec, stream or None, avg, cnt, 1 if reset else 0))
    return {k: (avg[i], int(cnt[i])) for i, k in enumerate(KERNELS)}


def splitzip_release_stream(codec: int, stream: int = 0) -> None:
    """Free the workspace the codec keeps for `stream` (waits for the stream first)."""
    _check(lib().splitzip_release_stream(codec, stream or None))


def splitzip_workspace_bytes(codec: int, stream: int = 0) -> int:
    """Device bytes of the workspace the codec keeps for `stream` (0: none)."""
    b = ctypes.c_uint64()
    _check(lib().splitzip_workspace_bytes(codec, stream or None, ctypes.byref(b)))
    return b.value


def splitzip_free(codec: int) -> None:
    if codec:
        lib().splitzip_free(codec)


def splitzip_chunk_count(n: int, chunk_size: int) -> int:
    return int(lib().splitzip_chunk_count(n, chunk_size))


def splitzip_compressed_bytes(n: int, chunk_size: int, n_escapes: int) -> int:
    return int(lib().splitzip_compressed_bytes(n, chunk_size, n_escapes))


def splitzip_e5m2_compressed_bytes(n: int, chunk_size: int, n_escapes: int) -> int:
    return int(lib().splitzip_e5m2_compressed_bytes(n, chunk_size, n_escapes))


def stream_bytes(elem: int, n: int, chunk_size: int, n_escapes: int) -> int:
    """Canonical stream size of n elements of type elem (ELEM_BF16 or ELEM_E5M2)."""
    if elem == ELEM_E5M2:
        return splitzip_e5m2_compressed_bytes(n, chunk_size, n_escapes)
    return splitzip_compressed_bytes(n, chunk_size, n_escapes)


def splitzip_write_header(codec: int, book: int, n: int, n_escapes: int) -> bytes:
    out = (ctypes.c_uint8 * HEADER_BYTES)()
    _check(lib().splitzip_write_header(codec, book, n, n_escapes, out))
    return bytes(out)


def splitzip_read_header(buf: bytes) -> dict:
    n, e = ctypes.c_uint64(), ctypes.c_uint64()
    c, el = ctypes.c_uint32(), ctypes.c_uint32()
    cb = (ctypes.c_uint8 * 16)()
    _check(lib().splitzip_read_header(_u8buf(buf[:HEADER_BYTES]), len(buf), ctypes.byref(n),
                                      ctypes.byref(c), ctypes.byref(e), cb, ctypes.byref(el)))
    return {"n": n.value, "chunk_size": c.value, "n_escapes": e.value, "codebook": bytes(cb),
            "elem": el.value}


def splitzip_check_header(codec: int, buf: bytes) -> int:
    """Raises unless the codec can decode the stream; returns the book it was coded with."""
    book = ctypes.c_uint32()
    _check(lib().splitzip_check_header(codec, _u8buf(buf[:HEADER_BYTES]), len(buf), ctypes.byref(book)))
    return book.value


# ---- README-style stateful codec --------------------------------------------------------

@dataclasses.dataclass
class Encoded:
    """Compressed form of one tensor: device sections plus the sizes the codec reported."""
    n: int
    shape: tuple
    dtype: object
    chunk_size: int
    codebook: bytes
    sm: object            # torch.uint8 [n]
    codes: object         # torch.uint8 [ceil(n/2)]
    chunk_off: object     # torch.int64 [n_chunks + 1] (u64 values)
    esc_pos_buf: object   # torch.int16 [capacity] (u16 values)
    esc_exp_buf: object   # torch.uint8 [capacity]
    n_escapes: int = 0
    compressed_bytes: int = 0
    book: int = 0         # which of the codec's codebooks
    elem: int = ELEM_BF16  # element type (E5M2: sm is the 3-bit field stream)

    @property
    def esc_pos(self):
        return self.esc_pos_buf[:self.n_escapes]

    @property
    def esc_exp(self):
        return self.esc_exp_buf[:self.n_escapes]

    @property
    def ratio(self) -> float:
        return _elem_bytes(self.elem) * self.n / self.compressed_bytes

    def segment(self, data_ptr: int = 0) -> splitzip_segment:
        return splitzip_segment(data_ptr or None, self.n, _ptr(self.sm), _ptr(self.codes),
                                _ptr(self.chunk_off), _ptr(self.esc_pos_buf),
                                _ptr(self.esc_exp_buf), self.esc_pos_buf.numel(),
                                self.n_escapes, self.compressed_bytes, self.book, 0)

    def to_bytes(self, codec: "Codec") -> bytes:
        """Canonical serialized stream: 64-byte header, then the five sections."""
        import torch
        head = splitzip_write_header(codec.handle, self.book, self.n, self.n_escapes)
        parts = [self.sm, self.codes, self.chunk_off.view(torch.uint8),
                 self.esc_pos.contiguous().view(torch.uint8), self.esc_exp]
        body = b"".join(p.cpu().numpy().tobytes() for p in parts)
        return head + body


@dataclasses.dataclass
class Packed:
    """A tensor compressed into one contiguous device buffer holding the canonical stream
    (64-byte header with the codebook, then the five sections)."""
    n: int
    shape: tuple
    dtype: object
    buf: object              # torch.uint8 device buffer (capacity)
    stream_bytes: int = 0
    n_escapes: int = 0
    book: int = 0
    elem: int = ELEM_BF16

    @property
    def stream(self):
        """Device view of the stream (its exact length)."""
        return self.buf[:self.stream_bytes]

    def to_bytes(self) -> bytes:
        return self.stream.cpu().numpy().tobytes()

    @property
    def ratio(self) -> float:
        return _elem_bytes(self.elem) * self.n / self.stream_bytes

    @property
    def compressed_bytes(self) -> int:
        return self.stream_bytes


PACKED_OFFSET = 192


def packed_buffer(nbytes: int, device):
    """A device buffer for a packed stream, placed 64 bytes before a 256-byte boundary so
    that the sections after the 64-byte header start on whole cache lines (the kernels
    stream them in full lines; a stream at any other 16-byte-aligned place is correct but
    slower)."""
    import torch
    raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (PACKED_OFFSET - raw.data_ptr()) % 256
    return raw[off:off + nbytes]


def _ptr(t) -> int | None:
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _elem_bytes(elem: int) -> int:
    return 1 if elem == ELEM_E5M2 else 2


def _elements(x, device, elem: int):
    """Flat contiguous view of a device tensor as the codec's element words: int16 for BF16,
    uint8 for E5M2 (float8_e5m2 or any 1-byte tensor)."""
    import torch
    if elem != ELEM_E5M2:
        return _words(x, device)
    if x.element_size() != 1:
        raise TypeError(f"expected a 1-byte tensor (E5M2 bytes), got {x.dtype}")
    if x.device != device:
        raise ValueError(f"tensor is on {x.device}, codec is on {device}")
    if not x.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return x.reshape(-1).view(torch.uint8)


def _words(x, device):
    """Flat contiguous 16-bit view of a BF16 (or int16/uint16) device tensor."""
    import torch
    if x.element_size() != 2:
        raise TypeError(f"expected a 16-bit tensor (BF16 words), got {x.dtype}")
    if x.device != device:
        raise ValueError(f"tensor is on {x.device}, codec is on {device}")
    if not x.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return x.reshape(-1).view(torch.int16)


class Codec:
    """Stateful SplitZip codec bound to one GPU, one chunk size and one element type
    (``elem="bf16"`` or ``"e5m2"``)."""

    def __init__(self, device="cuda", chunk_size: int = 1024, elem: str = "bf16"):
        import torch
        if elem not in ELEMS:
            raise ValueError(f"elem must be one of {sorted(ELEMS)}")
        if not torch.cuda.is_available():
            raise SplitZipError(E_DEVICE, "no GPU: the SplitZip codec runs only on the GPU")
        d = torch.device(device)
        if d.index is None:
            d = torch.device(d.type, torch.cuda.current_device())
        if not (MIN_CHUNK <= chunk_size <= MAX_CHUNK and chunk_size & (chunk_size - 1) == 0):
            raise ValueError("chunk_size must be a power of two in [16, 65536]")
        lib()
        self.device = d
        self.chunk_size = chunk_size
        self.elem = ELEMS[elem]
        self.elem_name = elem
        self.handle = 0
        self.coverage = None
        self.histogram = None
        self._escape_rate = 0.0
        self._small_tiles = SMALL_TILES
        self._onepass_tiles = ONEPASS_TILES
        self._stage_tiles = STAGE_TILES
        self._private_overflow = PRIVATE_OVERFLOW_BYTES

    # -- state -----------------------------------------------------------------------
    @classmethod
    def from_codebook(cls, codebook: bytes, chunk_size: int = 1024, device="cuda",
                      elem: str = "bf16") -> "Codec":
        return cls.from_codebooks([codebook], chunk_size, device, elem)

    @property
    def codebook(self) -> bytes:
        """Codebook of book 0 (the only one after ``calibrate``)."""
        self._need_handle()
        return splitzip_codec_info(self.handle)[0]

    @property
    def books(self) -> list:
        """All codebooks, 16 bytes each."""
        self._need_handle()
        return splitzip_codec_books(self.handle)

    @classmethod
    def from_codebooks(cls, codebooks, chunk_size: int = 1024, device="cuda",
                       elem: str = "bf16") -> "Codec":
        import torch
        c = cls(device, chunk_size, elem)
        books = b"".join(bytes(b) for b in codebooks)
        with torch.cuda.device(c.device):
            if c.elem == ELEM_E5M2:
                c._set_handle(splitzip_codec_from_codebooks_e5m2(books, chunk_size))
            else:
                c._set_handle(splitzip_codec_from_codebooks(books, chunk_size))
        return c

    def _elements(self, x):
        return _elements(x, self.device, self.elem)

    def stream_bytes(self, n: int, n_escapes: int) -> int:
        """Canonical stream size of n elements with n_escapes escapes."""
        return stream_bytes(self.elem, n, self.chunk_size, n_escapes)

    def _need_handle(self):
        if not self.handle:
            raise SplitZipError(E_INVALID, "codec is not calibrated")

    def _set_handle(self, h: int) -> None:
        """Replace the C codec (a new calibration) and carry the launch setting over."""
        splitzip_free(self.handle)
        self.handle = h
        if self._small_tiles != SMALL_TILES:
            splitzip_set_small_tiles(h, self._small_tiles)
        if self._onepass_tiles != ONEPASS_TILES:
            splitzip_set_onepass_tiles(h, self._onepass_tiles)
        if self._stage_tiles != STAGE_TILES:
            splitzip_set_stage_tiles(h, self._stage_tiles)
        if self._private_overflow != PRIVATE_OVERFLOW_BYTES:
            splitzip_set_private_overflow(h, self._private_overflow)

    def _stream(self) -> int:
        import torch
        return torch.cuda.current_stream(self.device).cuda_stream

    def set_small_tiles(self, max_tiles: int = SMALL_TILES) -> None:
        """Encodes of at most max_tiles tiles run two launches instead of four (same bytes);
        0: always four.  Kept across later calibrations of this codec."""
        if not 0 <= max_tiles <= SMALL_TILES:
            raise SplitZipError(E_INVALID, f"max_tiles must be in [0, {SMALL_TILES}]")
        if self.handle:
            splitzip_set_small_tiles(self.handle, max_tiles)
        self._small_tiles = max_tiles

    def set_onepass_tiles(self, max_tiles: int = ONEPASS_TILES) -> None:
        """Encodes into separate sections of at most max_tiles tiles run as one launch whose
        tiles place their own escapes after a look-back over the earlier tiles (same bytes);
        0: never.  Kept across later calibrations of this codec."""
        if not 0 <= max_tiles < 1 << 32:
            raise SplitZipError(E_INVALID, "max_tiles must fit 32 bits")
        if self.handle:
            splitzip_set_onepass_tiles(self.handle, max_tiles)
        self._onepass_tiles = max_tiles

    def set_stage_tiles(self, min_tiles: int = STAGE_TILES) -> None:
        """Encodes of more than min_tiles tiles, and decodes of more than 2 * min_tiles decode
        tiles (the same elements), run the kernel builds tuned for escape-heavy inputs (same
        bytes; larger code, which costs short calls more); 0: always, 2**32 - 1: never.
        Kept across later calibrations of this codec."""
        if not 0 <= min_tiles < 1 << 32:
            raise SplitZipError(E_INVALID, "min_tiles must fit 32 bits")
        if self.handle:
            splitzip_set_stage_tiles(self.handle, min_tiles)
        self._stage_tiles = min_tiles

    def set_private_overflow(self, max_bytes: int = PRIVATE_OVERFLOW_BYTES) -> None:
        """Encodes whose tiles' own overflow regions (4 bytes per element) fit max_bytes of
        scratch use them instead of reserving from one shared counter (same bytes; faster
        on escape-heavy inputs); 0: never.  Kept across later calibrations of this codec."""
        if not 0 <= max_bytes < 1 << 64:
            raise SplitZipError(E_INVALID, "max_bytes must fit 64 bits")
        if self.handle:
            splitzip_set_private_overflow(self.handle, max_bytes)
        self._private_overflow = max_bytes

    def profile(self, enable: bool = True) -> None:
        """Time every kernel launch of later calls with HIP events (see kernel_times)."""
        self._need_handle()
        splitzip_profile(self.handle, enable)

    def kernel_times(self, reset: bool = False) -> dict:
        """{kernel: (mean ms, launches)} over the profiled calls on the current stream."""
        import torch
        self._need_handle()
        with torch.cuda.device(self.device):
            return splitzip_profile_read(self.handle, self._stream(), reset)

    def release_stream(self, stream=None) -> None:
        """Free the workspace this codec keeps for a stream (a torch.cuda.Stream, a raw
        hipStream_t, or None for the current stream); call before dropping a stream the codec
        was used on."""
        import torch
        self._need_handle()
        if stream is None:
            raw = self._stream()
        elif isinstance(stream, torch.cuda.Stream):
            raw = stream.cuda_stream
        else:
            raw = int(stream)
        splitzip_release_stream(self.handle, raw)

    def workspace_bytes(self, stream=None) -> int:
        """Device bytes of the workspace this codec keeps for a stream (0: none)."""
        import torch
        self._need_handle()
        raw = self._stream() if stream is None else (stream.cuda_stream if isinstance(stream, torch.cuda.Stream)
                                                     else int(stream))
        return splitzip_workspace_bytes(self.handle, raw)

    def __del__(self):
        try:
            splitzip_free(self.handle)
        except Exception:
            pass
        self.handle = 0

    # -- a1 -------------------------------------------------------------------------
    def calibrate(self, x) -> float:
        """Fix the top-16 exponent codebook from a calibration tensor; returns its coverage."""
        import torch
        w = self._elements(x)
        cal = splitzip_calibrate_e5m2 if self.elem == ELEM_E5M2 else splitzip_calibrate
        with torch.cuda.device(self.device):
            h, cov, hist = cal(w.data_ptr() if w.numel() else 0, w.numel(), self.chunk_size,
                               self._stream())
        self._set_handle(h)
        self.coverage, self.histogram = cov, hist
        self._escape_rate = 1.0 - cov if w.numel() else 0.0
        return cov

    def calibrate_books(self, cals) -> list:
        """One codebook per calibration tensor (e.g. per layer, per K and V), all histograms
        in one pass; returns the coverage of each.  Segments then pick a book on encode."""
        import torch
        ws = [self._elements(x) for x in cals]
        cal = splitzip_calibrate_books_e5m2 if self.elem == ELEM_E5M2 else splitzip_calibrate_books
        with torch.cuda.device(self.device):
            h, cov, hist = cal([w.data_ptr() if w.numel() else 0 for w in ws], [w.numel() for w in ws],
                               self.chunk_size, self._stream())
        self._set_handle(h)
        self.coverage, self.histogram = cov, hist
        rates = [1.0 - c for c, w in zip(cov, ws) if w.numel()]
        self._escape_rate = max(rates) if rates else 0.0
        return cov

    # -- a2-a4, a7 -----------------------------------------------------------------
    def empty_encoded(self, n: int, shape=None, dtype=None, escape_capacity: int | None = None,
                      book: int = 0):
        """Allocate the device sections for an n-element tensor coded with codebook `book`."""
        import torch
        n_chunks = -(-n // self.chunk_size)
        if escape_capacity is None:
            guess = math.ceil(n * max(self._escape_rate, 1e-4) * 1.25) + 64 * (n_chunks + 1)
            escape_capacity = min(n, max(1024, guess))
        kw = dict(device=self.device)
        e5m2 = self.elem == ELEM_E5M2
        return Encoded(
            n=n, shape=tuple(shape) if shape is not None else (n,),
            dtype=dtype if dtype is not None else (torch.float8_e5m2 if e5m2 else torch.bfloat16),
            chunk_size=self.chunk_size, codebook=self.books[book], book=book, elem=self.elem,
            sm=torch.empty((3 * n + 7) // 8 if e5m2 else n, dtype=torch.uint8, **kw),
            codes=torch.empty((n + 1) // 2, dtype=torch.uint8, **kw),
            chunk_off=torch.empty(n_chunks + 1, dtype=torch.int64, **kw),
            esc_pos_buf=torch.empty(max(escape_capacity, 1), dtype=torch.int16, **kw),
            esc_exp_buf=torch.empty(max(escape_capacity, 1), dtype=torch.uint8, **kw))

    def encode_into(self, xs, encs) -> int:
        """One encode launch over tensors xs into preallocated encs; returns OK or E_CAPACITY
        (then the Encoded whose n_escapes exceeds its capacity must be re-allocated)."""
        import torch
        self._need_handle()
        words = [self._elements(x) for x in xs]
        segs = (splitzip_segment * len(words))()
        for i, (w, e) in enumerate(zip(words, encs)):
            if w.numel() != e.n:
                raise ValueError("tensor size differs from the preallocated sections")
            segs[i] = e.segment(w.data_ptr() if w.numel() else 0)
        with torch.cuda.device(self.device):
            st = splitzip_encode(self.handle, segs, self._stream())
        for i, e in enumerate(encs):
            e.n_escapes = int(segs[i].n_escapes)
            e.compressed_bytes = int(segs[i].compressed_bytes)
        return st

    def encode_into_async(self, xs, encs, result) -> None:
        """Enqueue one encode launch without waiting.  `result` is a device int64 tensor
        of 1 + len(xs) words: [error bits, E per segment].  The Encoded objects' n_escapes
        / compressed_bytes are left as they are; call `finish_async` after the stream has
        passed this work to fill them and check capacities."""
        import torch
        self._need_handle()
        if result.dtype != torch.int64 or result.numel() < 1 + len(xs):
            raise ValueError("result must be an int64 device tensor of 1 + len(xs) words")
        words = [self._elements(x) for x in xs]
        segs = (splitzip_segment * len(words))()
        for i, (w, e) in enumerate(zip(words, encs)):
            if w.numel() != e.n:
                raise ValueError("tensor size differs from the preallocated sections")
            segs[i] = e.segment(w.data_ptr() if w.numel() else 0)
        with torch.cuda.device(self.device):
            splitzip_encode_async(self.handle, segs, self._stream(), result.data_ptr())

    def finish_async(self, encs, result) -> int:
        """Read the result words of an encode_into_async (synchronizes with the host)."""
        r = result.cpu().tolist()
        st = OK
        for i, e in enumerate(encs):
            e.n_escapes = int(r[1 + i])
            e.compressed_bytes = self.stream_bytes(e.n, e.n_escapes)
            if e.n_escapes > e.esc_pos_buf.numel():
                st = E_CAPACITY
        overflow_area = 8
        if r[0] & ~overflow_area or (r[0] and st != E_CAPACITY):
            raise SplitZipError(E_DEVICE, f"encode kernel reported error bits {r[0]:#x}")
        return st

    def prepare(self, xs, encs, outs=None) -> "PreparedBatch":
        """Fix the tensors of a batch once (inputs, their Encoded sections, optional decode
        outputs) so that repeated encode/decode calls skip the per-call argument marshalling."""
        return PreparedBatch(self, xs, encs, outs)

    def encode(self, x, escape_capacity: int | None = None, book: int = 0) -> Encoded:
        return self.encode_batch([x], escape_capacity, [book])[0]

    def encode_batch(self, xs, escape_capacity: int | None = None, books=None) -> list:
        """Encode several tensors (a ragged batch) in one launch; books[i] (default 0) is
        the codebook of tensor i."""
        self._need_handle()
        books = list(books) if books is not None else [0] * len(xs)
        if len(books) != len(xs):
            raise ValueError("one book per tensor")
        encs = [self.empty_encoded(x.numel(), x.shape, x.dtype, escape_capacity, b)
                for x, b in zip(xs, books)]
        st = self.encode_into(xs, encs)
        if st == E_CAPACITY:
            for i, e in enumerate(encs):
                if e.n_escapes > e.esc_pos_buf.numel():
                    encs[i] = self.empty_encoded(e.n, e.shape, e.dtype, e.n_escapes, e.book)
            st = self.encode_into(xs, encs)
            assert st == OK
        total = sum(e.n for e in encs)
        if total:
            self._escape_rate = max(self._escape_rate, sum(e.n_escapes for e in encs) / total)
        return encs

    # -- packed streams -------------------------------------------------------------
    def packed_capacity(self, n: int, escapes: int | None = None) -> int:
        """Buffer bytes for an n-element packed stream with up to `escapes` escapes (default:
        a guess from the calibration coverage)."""
        if escapes is None:
            n_chunks = -(-n // self.chunk_size)
            escapes = min(n, max(1024, math.ceil(n * max(self._escape_rate, 1e-4) * 1.25) + 64 * (n_chunks + 1)))
        return self.stream_bytes(n, escapes)

    def encode_packed(self, x, book: int = 0, capacity: int | None = None) -> Packed:
        return self.encode_packed_batch([x], [book], None if capacity is None else [capacity])[0]

    def encode_packed_batch(self, xs, books=None, capacities=None) -> list:
        """Encode tensors (numel a multiple of 16 for BF16, of 128 for E5M2) into packed
        streams, one launch sequence; a buffer that turns out too small is reallocated and the
        batch re-encoded."""
        import torch
        self._need_handle()
        books = list(books) if books is not None else [0] * len(xs)
        words = [self._elements(x) for x in xs]
        caps = list(capacities) if capacities is not None else [self.packed_capacity(w.numel()) for w in words]
        out = [Packed(w.numel(), tuple(x.shape), x.dtype, packed_buffer(c, self.device), 0, 0, b, self.elem)
               for x, w, c, b in zip(xs, words, caps, books)]
        for attempt in range(2):
            segs = (splitzip_packed * len(out))()
            for i, (w, p) in enumerate(zip(words, out)):
                segs[i] = splitzip_packed(w.data_ptr() if w.numel() else None, p.n, p.buf.data_ptr(),
                                          p.buf.numel(), 0, 0, p.book, 0)
            with torch.cuda.device(self.device):
                st = splitzip_encode_packed(self.handle, segs, self._stream())
            for i, p in enumerate(out):
                p.stream_bytes, p.n_escapes = int(segs[i].stream_bytes), int(segs[i].n_escapes)
            if st == OK:
                break
            for p in out:
                if p.stream_bytes > p.buf.numel():
                    p.buf = packed_buffer(p.stream_bytes, self.device)
        assert st == OK
        total = sum(p.n for p in out)
        if total:
            self._escape_rate = max(self._escape_rate, sum(p.n_escapes for p in out) / total)
        return out

    def prepare_packed(self, xs, packed, outs=None) -> "PreparedPackedBatch":
        """Fix the tensors and packed buffers of a batch for repeated encode/decode calls."""
        return PreparedPackedBatch(self, xs, packed, outs)

    def decode_packed(self, stream, n: int | None = None, shape=None, dtype=None):
        return self.decode_packed_batch([stream], [n], [shape], [dtype])[0]

    def decode_packed_batch(self, streams, ns=None, shapes=None, dtypes=None, d_error: int = 0) -> list:
        """Decode packed streams (Packed objects, or device uint8 tensors holding a stream
        with n given) in one launch; each stream is decoded with the codebook in its header."""
        import torch
        self._need_handle()
        k = len(streams)
        ns, shapes, dtypes = ns or [None] * k, shapes or [None] * k, dtypes or [None] * k
        outs, segs = [], (splitzip_packed * k)()
        for i, st in enumerate(streams):
            buf = st.stream if isinstance(st, Packed) else st
            n = st.n if isinstance(st, Packed) else ns[i]
            shape = shapes[i] or (st.shape if isinstance(st, Packed) else (n,))
            default = torch.float8_e5m2 if self.elem == ELEM_E5M2 else torch.bfloat16
            dtype = dtypes[i] or (st.dtype if isinstance(st, Packed) else default)
            if buf.dtype != torch.uint8 or buf.device != self.device or not buf.is_contiguous():
                raise ValueError("a packed stream is a contiguous uint8 tensor on the codec's device")
            y = torch.empty(shape, dtype=dtype, device=self.device)
            w = self._elements(y)
            if w.numel() != n:
                raise ValueError("output shape does not hold n elements")
            outs.append(y)
            segs[i] = splitzip_packed(w.data_ptr() if n else None, n, buf.data_ptr(), buf.numel(), 0, 0, 0, 0)
        with torch.cuda.device(self.device):
            splitzip_decode_packed(self.handle, segs, self._stream(), d_error)
        return outs

    # -- a5-a7 ------------------------------------------------------------------------
    def decode_into(self, encs, outs, d_error: int = 0) -> None:
        import torch
        self._need_handle()
        segs = (splitzip_segment * len(encs))()
        books = self.books
        for i, (e, y) in enumerate(zip(encs, outs)):
            w = self._elements(y)
            if w.numel() != e.n:
                raise ValueError("output size differs from the encoded tensor")
            if (e.chunk_size != self.chunk_size or e.elem != self.elem or e.book >= len(books)
                    or e.codebook != books[e.book]):
                raise SplitZipError(E_CODEBOOK, "encoded with a different codec state")
            segs[i] = e.segment(w.data_ptr() if w.numel() else 0)
        with torch.cuda.device(self.device):
            splitzip_decode(self.handle, segs, self._stream(), d_error)

    def decode(self, enc: Encoded):
        return self.decode_batch([enc])[0]

    def decode_batch(self, encs) -> list:
        import torch
        outs = [torch.empty(e.shape, dtype=e.dtype, device=self.device) for e in encs]
        self.decode_into(encs, outs)
        return outs

    def decode_bytes(self, buf: bytes, shape=None, dtype=None):
        """Decode a canonical serialized stream written by a codec with the same state."""
        import numpy as np
        import torch
        self._need_handle()
        book = splitzip_check_header(self.handle, buf)
        h = splitzip_read_header(buf)
        n, E = h["n"], h["n_escapes"]
        n_chunks = splitzip_chunk_count(n, self.chunk_size)
        enc = self.empty_encoded(n, shape, dtype, max(E, 1), book)
        b = np.frombuffer(buf, np.uint8)
        p = HEADER_BYTES
        sm_bytes = (3 * n + 7) // 8 if self.elem == ELEM_E5M2 else n
        sizes = [sm_bytes, (n + 1) // 2, 8 * (n_chunks + 1), 2 * E, E]
        dests = [enc.sm, enc.codes, enc.chunk_off.view(torch.uint8),
                 enc.esc_pos_buf[:E].view(torch.uint8), enc.esc_exp_buf[:E]]
        for size, dst in zip(sizes, dests):
            if size:
                dst.copy_(torch.from_numpy(b[p:p + size].copy()))
            p += size
        enc.n_escapes = E
        enc.compressed_bytes = len(buf)
        return self.decode(enc)


# The class name of the codec the SplitZip README's *Codec API* shows, with the same
# constructor (device, chunk_size), calibrate -> coverage, encode -> object with
# compressed_bytes, and decode.
ChunkLocalSplitZipGPU = Codec


class PreparedBatch:
    """A batch whose device buffers stay fixed across calls (e.g. one serving step after
    another): the segment descriptors are built once."""

    def __init__(self, codec: Codec, xs, encs, outs=None):
        if len(xs) != len(encs) or (outs is not None and len(outs) != len(xs)):
            raise ValueError("xs, encs and outs must have the same length")
        self.codec = codec
        self.xs, self.encs, self.outs = list(xs), list(encs), (list(outs) if outs is not None else None)
        self._enc = (splitzip_segment * len(xs))()
        for i, (x, e) in enumerate(zip(self.xs, self.encs)):
            w = codec._elements(x)
            if w.numel() != e.n:
                raise ValueError("tensor size differs from the preallocated sections")
            self._enc[i] = e.segment(w.data_ptr() if w.numel() else 0)
        self._dec = None
        if self.outs is not None:
            self._dec = (splitzip_segment * len(xs))()
            for i, (y, e) in enumerate(zip(self.outs, self.encs)):
                w = codec._elements(y)
                if w.numel() != e.n:
                    raise ValueError("output size differs from the encoded tensor")
                self._dec[i] = e.segment(w.data_ptr() if w.numel() else 0)

    def encode_async(self, result) -> None:
        """Enqueue the encode; see Codec.encode_into_async and Codec.finish_async.  (The
        library makes the codec's device current itself; the stream is the device's current
        one.)"""
        splitzip_encode_async(self.codec.handle, self._enc, self.codec._stream(), result.data_ptr())

    def finish(self, result) -> int:
        st = self.codec.finish_async(self.encs, result)
        if self._dec is not None:
            for i, e in enumerate(self.encs):
                self._dec[i].n_escapes = e.n_escapes
        return st

    def decode(self, d_error: int = 0) -> None:
        """Enqueue the decode of the batch into its outputs (n_escapes as of the last finish)."""
        if self._dec is None:
            raise ValueError("no decode outputs were given")
        splitzip_decode(self.codec.handle, self._dec, self.codec._stream(), d_error)


# ---- exponent statistics ----------------------------------------------------------------

def histograms(xs, device=None, elem: str = "bf16") -> list:
    """Exponent histograms of device tensors, one pass on the GPU: 256 bins each for BF16,
    32 for E5M2."""
    import torch
    if not torch.cuda.is_available():
        raise SplitZipError(E_DEVICE, "no GPU: histograms run only on the GPU")
    dev = torch.device(device) if device is not None else xs[0].device
    el = ELEMS[elem]
    ws = [_elements(x, dev, el) for x in xs]
    fn = splitzip_histogram_e5m2 if el == ELEM_E5M2 else splitzip_histogram
    with torch.cuda.device(dev):
        return fn([w.data_ptr() if w.numel() else 0 for w in ws], [w.numel() for w in ws],
                  torch.cuda.current_stream(dev).cuda_stream)


def exponent_stats(hist) -> dict:
    """Entropy in bits, top-16 codebook, coverage and distinct exponents of a histogram."""
    return splitzip_exponent_stats(hist)


class PreparedPackedBatch:
    """PreparedBatch for packed streams: descriptors built once, then repeated
    non-blocking encodes into the same buffers and decodes from them."""

    def __init__(self, codec: Codec, xs, packed, outs=None):
        if len(xs) != len(packed) or (outs is not None and len(outs) != len(xs)):
            raise ValueError("xs, packed and outs must have the same length")
        self.codec, self.packed = codec, list(packed)
        self._enc = (splitzip_packed * len(xs))()
        for i, (x, p) in enumerate(zip(xs, self.packed)):
            w = codec._elements(x)
            if w.numel() != p.n:
                raise ValueError("tensor size differs from the packed stream")
            self._enc[i] = splitzip_packed(w.data_ptr() if p.n else None, p.n, p.buf.data_ptr(),
                                           p.buf.numel(), 0, 0, p.book, 0)
        self._dec = None
        if outs is not None:
            self._dec = (splitzip_packed * len(xs))()
            for i, (y, p) in enumerate(zip(outs, self.packed)):
                w = codec._elements(y)
                if w.numel() != p.n:
                    raise ValueError("output size differs from the packed stream")
                self._dec[i] = splitzip_packed(w.data_ptr() if p.n else None, p.n, p.buf.data_ptr(),
                                               p.stream_bytes, 0, 0, 0, 0)

    def encode_async(self, result) -> None:
        splitzip_encode_packed(self.codec.handle, self._enc, self.codec._stream(), result.data_ptr())

    def finish(self, result) -> int:
        """Read E per stream (synchronizes); E_CAPACITY if a stream outgrew its buffer."""
        r = result.cpu().tolist()
        st = OK
        for i, p in enumerate(self.packed):
            p.n_escapes = int(r[1 + i])
            p.stream_bytes = self.codec.stream_bytes(p.n, p.n_escapes)
            if p.stream_bytes > p.buf.numel():
                st = E_CAPACITY
            if self._dec is not None:
                self._dec[i].buf_bytes = p.stream_bytes
        if r[0] & ~8 or (r[0] and st != E_CAPACITY):
            raise SplitZipError(E_DEVICE, f"encode kernel reported error bits {r[0]:#x}")
        return st

    def decode(self, d_error: int = 0) -> None:
        if self._dec is None:
            raise ValueError("no decode outputs were given")
        splitzip_decode_packed(self.codec.handle, self._dec, self.codec._stream(), d_error)
