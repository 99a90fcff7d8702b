"""Seeded synthetic BF16 KV workloads shared by the tests and the benchmark.

This module only *generates inputs*: it holds none of the codec's arithmetic
(no exponent statistics, no codebook, no packing).  Both the oracle-side tests
and the GPU-side tests and benchmark draw their inputs from here, so that the
two sides see the same words.

The pages measure on real Qwen3-32B KV activations from WikiText-2 ("SplitZip:
Ultra-Fast Lossless KV Compression for Disaggregated LLM Serving" README,
"Reproducing Paper Artifact Scripts"); neither the model nor the dataset is
available, so these KV-shaped Gaussian draws stand in for them.  KV tensors are
laid out [tokens, 8 KV heads, 128 head_dim] row-major (GQA), i.e. 1024 channels
per token.

Random numbers: numpy PCG64 via ``numpy.random.default_rng``; normals are
``standard_normal(dtype=float32)`` and scaling happens in float32.  Conversion
to BF16 is round-to-nearest-even of the float32 bits.  Special values are
written as raw bit patterns.

FP8 E5M2 inputs (an FP8 E5M2 KV cache, which the pages' README "FAQ" names) are the
same draws cast to E5M2: float32 to FP16 (numpy, round to nearest even), then FP16 to
E5M2 by rounding the FP16 bits to their top byte (nearest even; both formats have a
5-bit exponent with bias 15, so this is exact E5M2 rounding of the FP16 value).
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

KV_HEADS = 8
HEAD_DIM = 128
CHANNELS = KV_HEADS * HEAD_DIM
ZERO_FRACTION = 0.0005       # exact +0.0 entries per KV tensor
OUTLIER_FRACTION = 0.02      # outlier channels per K tensor
OUTLIER_SCALE = 32.0
CHANNEL_SIGMA = 0.75         # s_c = exp(0.75 * N(0,1))
LAYER_SIGMA = 0.3            # g_l = exp(0.3 * N(0,1))


def bf16_bits(f32: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest BF16 (ties to even); returns the uint16 words.

    Inputs must be finite (every generator below draws finite values)."""
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    u = f32.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(words: np.ndarray) -> np.ndarray:
    return (np.asarray(words, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def e5m2_bits(f32: np.ndarray) -> np.ndarray:
    """Cast float32 values to FP8 E5M2 bytes: to FP16 (round to nearest even, overflow to
    Inf), then the FP16 bits rounded to their top byte (nearest even).  Inputs must not be
    NaN."""
    with np.errstate(over="ignore"):
        h = np.ascontiguousarray(f32, dtype=np.float32).astype(np.float16)
    h = h.view(np.uint16).astype(np.uint32)
    return ((h + np.uint32(0x7F) + ((h >> np.uint32(8)) & np.uint32(1))) >> np.uint32(8)).astype(np.uint8)


@dataclasses.dataclass
class Workload:
    """Segments to encode (each a flat uint16 array) plus the separate calibration draw."""
    name: str
    segments: list
    calibration: np.ndarray
    chunk_size: int
    description: str

    @property
    def n_elements(self) -> int:
        return int(sum(s.size for s in self.segments))


# ---- config 1: one N(0,1) tensor -------------------------------------------------------

def config1(rows: int = 1024, hidden: int = 4096) -> Workload:
    x = bf16_bits(np.random.default_rng(0).standard_normal((rows, hidden), dtype=np.float32))
    cal = bf16_bits(np.random.default_rng(1).standard_normal((rows, hidden), dtype=np.float32))
    return Workload(f"single_tensor_{rows}x{hidden}_normal", [x.reshape(-1)], cal.reshape(-1), 1024,
                    f"one [{rows},{hidden}] BF16 N(0,1) tensor (seed 0), calibrated on a "
                    f"separate N(0,1) draw (seed 1), chunk 1024")


# ---- config 2 generator: one layer of GQA KV --------------------------------------------

@dataclasses.dataclass
class KVParams:
    """Per-layer "model parameters": channel scales with outlier channels, layer scale."""
    channel_scale: np.ndarray   # float32 [1024], applied to K
    layer_scale: np.float32     # applied to K and V


def kv_params(rng: np.random.Generator, with_layer_scale: bool) -> KVParams:
    g = np.float32(1.0)
    if with_layer_scale:
        g = np.float32(np.exp(np.float32(LAYER_SIGMA) * rng.standard_normal(dtype=np.float32)))
    s = np.exp(np.float32(CHANNEL_SIGMA) * rng.standard_normal(CHANNELS, dtype=np.float32))
    outliers = rng.choice(CHANNELS, size=int(round(OUTLIER_FRACTION * CHANNELS)), replace=False)
    s[outliers] *= np.float32(OUTLIER_SCALE)
    return KVParams(s.astype(np.float32), g)


def _kv_tensor(rng: np.random.Generator, tokens: int, scale: np.ndarray | None,
               g: np.float32, out: np.ndarray) -> None:
    """One [tokens, 8, 128] tensor: N(0,1) (times per-channel scale for K) times the layer
    scale, then an exact ZERO_FRACTION of its entries set to +0.0; written into `out`."""
    z = rng.standard_normal((tokens, CHANNELS), dtype=np.float32)
    if scale is not None:
        z *= scale
    if g != np.float32(1.0):
        z *= g
    n = tokens * CHANNELS
    k = int(round(ZERO_FRACTION * n))
    if k:
        z.reshape(-1)[rng.choice(n, size=k, replace=False)] = np.float32(0.0)
    out[:] = bf16_bits(z).reshape(-1)


def kv_layer(rng: np.random.Generator, params: KVParams, tokens: int,
             out: np.ndarray | None = None) -> np.ndarray:
    """K then V of one layer, flat [2, tokens, 8, 128] uint16."""
    n = tokens * CHANNELS
    if out is None:
        out = np.empty(2 * n, np.uint16)
    _kv_tensor(rng, tokens, params.channel_scale, params.layer_scale, out[:n])
    _kv_tensor(rng, tokens, None, params.layer_scale, out[n:])
    return out


def config2(tokens: int = 4096) -> Workload:
    params = kv_params(np.random.default_rng(20), with_layer_scale=False)
    kv = kv_layer(np.random.default_rng(21), params, tokens)
    cal = kv_layer(np.random.default_rng(22), params, tokens)
    n = tokens * CHANNELS
    return Workload("gqa_kv_layer_4096x8x128", [kv[:n], kv[n:]], cal, 1024,
                    f"one layer of GQA KV, K and V [{tokens},8,128]: V~N(0,1), K~N(0,1)*s_c, "
                    f"s_c=exp(0.75 N(0,1)), 2% outlier channels x32, 0.05% exact zeros; "
                    f"params seed 20, tokens seed 21, calibration seed 22; chunk 1024")


# ---- config 3: long-prefill KV of a 64-layer model ---------------------------------------

def config3_params(layers: int = 64) -> list:
    rng = np.random.default_rng(30)
    return [kv_params(rng, with_layer_scale=True) for _ in range(layers)]


def _threads(threads: int | None) -> int:
    if threads:
        return threads
    return max(1, min(16, os.cpu_count() or 1))


def config3(layers: int = 64, tokens: int = 32768, cal_tokens: int = 2048,
            chunk_size: int = 1024, threads: int | None = None,
            with_calibration: bool = True) -> Workload:
    """Long-prefill KV: [layer][K|V][token][8][128], n = layers * 2 * tokens * 1024.

    With the defaults n = 2**32 (8.6 GB).  One segment.  Layers are generated in
    parallel; each layer's token draw has its own seed [31, layer], so the result does
    not depend on the thread count."""
    params = config3_params(layers)
    per_layer = 2 * tokens * CHANNELS
    data = np.empty(layers * per_layer, np.uint16)
    cal = np.empty(layers * 2 * cal_tokens * CHANNELS, np.uint16) if with_calibration else None

    def make(layer: int) -> None:
        kv_layer(np.random.default_rng([31, layer]), params[layer], tokens,
                 data[layer * per_layer:(layer + 1) * per_layer])
        if with_calibration:
            m = 2 * cal_tokens * CHANNELS
            kv_layer(np.random.default_rng([32, layer]), params[layer], cal_tokens,
                     cal[layer * m:(layer + 1) * m])

    with _cf.ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(make, range(layers)))
    return Workload(f"long_prefill_kv_{layers}L_{tokens}tok_8x128", [data],
                    cal if cal is not None else np.zeros(0, np.uint16), chunk_size,
                    f"{layers}-layer K+V, 8 KV heads x 128, {tokens} tokens per layer "
                    f"({data.size} BF16 = {2 * data.size / 1e9:.2f} GB) generated per layer as "
                    f"the GQA layer generator with layer scale exp(0.3 N(0,1)) (params seed 30, "
                    f"token seeds [31,l]); calibration = separate {cal_tokens}-token draw per "
                    f"layer (seeds [32,l]); chunk {chunk_size}")


def kv_parts(flat: np.ndarray, layers: int, tokens: int) -> list:
    """Views of a [layer][K|V][token][channel] array as its 2 * layers tensors of
    tokens * 1024 words (layer 0 K, layer 0 V, layer 1 K, ...)."""
    per = tokens * CHANNELS
    assert flat.size == 2 * layers * per
    return [flat[i * per:(i + 1) * per] for i in range(2 * layers)]


# ---- config 4: escape stress --------------------------------------------------------------

def special_words(rng: np.random.Generator, count: int) -> np.ndarray:
    """Uniformly one of {0, subnormal, Inf, NaN}, random sign; subnormal and NaN mantissas
    uniform in 1..127 (raw bit patterns)."""
    cls = rng.integers(0, 4, size=count)
    sign = rng.integers(0, 2, size=count).astype(np.uint16) << np.uint16(15)
    mant = rng.integers(1, 128, size=count).astype(np.uint16)
    w = np.where(cls == 0, np.uint16(0),
        np.where(cls == 1, mant,
        np.where(cls == 2, np.uint16(0x7F80), np.uint16(0x7F80) | mant))).astype(np.uint16)
    return (w | sign).astype(np.uint16)


def config4(n: int = 1 << 26, block: int = 4096, chunk_size: int = 1024) -> Workload:
    rng = np.random.default_rng(40)
    z = rng.standard_normal(n, dtype=np.float32)
    k = rng.integers(-8, 8, size=-(-n // block), endpoint=True)
    z *= np.repeat(np.exp2(k).astype(np.float32), block)[:n]
    x = bf16_bits(z)
    count = int(round(0.01 * n))
    idx = rng.choice(n, size=count, replace=False)
    x[idx] = special_words(rng, count)
    cal = config1().calibration
    return Workload("escape_stress_64M", [x], cal, chunk_size,
                    f"{n} BF16 = N(0,1)*2^k, k~U{{-8..8}} per {block}-element block (seed 40), "
                    f"plus exactly 1% specials (+-0, +-subnormal, +-Inf, +-NaN with random "
                    f"payload); calibrated on N(0,1) (seed 1); chunk {chunk_size}")


# ---- config 5: ragged batch ---------------------------------------------------------------

def config5_lengths(requests: int = 256) -> np.ndarray:
    return np.random.default_rng(7).integers(128, 8192, size=requests, endpoint=True)


def config5(requests: int = 256, threads: int | None = None) -> Workload:
    params = kv_params(np.random.default_rng(20), with_layer_scale=False)
    lens = config5_lengths(requests)
    offs = np.concatenate([[0], np.cumsum(2 * lens * CHANNELS)])
    data = np.empty(int(offs[-1]), np.uint16)

    def make(r: int) -> None:
        kv_layer(np.random.default_rng([50, r]), params, int(lens[r]),
                 data[offs[r]:offs[r + 1]])

    with _cf.ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(make, range(requests)))
    segs = []
    for r in range(requests):
        n = int(lens[r]) * CHANNELS
        segs.append(data[offs[r]:offs[r] + n])
        segs.append(data[offs[r] + n:offs[r + 1]])
    cal = config2().calibration
    return Workload("ragged_batch_256req", segs, cal, 1024,
                    f"{requests} requests, lengths U[128,8192] tokens (seed 7), K and V "
                    f"[len,8,128] per request from the GQA layer generator (token seeds "
                    f"[50,r]) = {2 * requests} segments, one launch; calibrated on the GQA "
                    f"layer calibration draw; chunk 1024")


# ---- FP8 E5M2: the long-prefill KV cast to E5M2 -------------------------------------------

def config3_e5m2(layers: int = 64, tokens: int = 32768, cal_tokens: int = 2048,
                 chunk_size: int = 1024, threads: int | None = None) -> Workload:
    """The long-prefill KV of config3 (same parameters and token draws, hence the same BF16
    values) cast to E5M2: an FP8 E5M2 KV cache, n = layers * 2 * tokens * 1024 bytes (2**32
    = 4.3 GB with the defaults), one segment; calibration = the cast calibration draw."""
    params = config3_params(layers)
    per_layer = 2 * tokens * CHANNELS
    m = 2 * cal_tokens * CHANNELS
    data = np.empty(layers * per_layer, np.uint8)
    cal = np.empty(layers * m, np.uint8)

    def make(layer: int) -> None:
        w = kv_layer(np.random.default_rng([31, layer]), params[layer], tokens)
        data[layer * per_layer:(layer + 1) * per_layer] = e5m2_bits(bf16_to_f32(w))
        c = kv_layer(np.random.default_rng([32, layer]), params[layer], cal_tokens)
        cal[layer * m:(layer + 1) * m] = e5m2_bits(bf16_to_f32(c))

    with _cf.ThreadPoolExecutor(min(_threads(threads), 8)) as ex:
        list(ex.map(make, range(layers)))
    return Workload(f"long_prefill_kv_e5m2_{layers}L_{tokens}tok_8x128", [data], cal, chunk_size,
                    f"the {layers}-layer long-prefill K+V ({tokens} tokens per layer, 8 KV heads "
                    f"x 128; params seed 30, token seeds [31,l]) cast to FP8 E5M2 ({data.size} "
                    f"bytes = {data.size / 1e9:.2f} GB); calibration = the separate "
                    f"{cal_tokens}-token draw per layer (seeds [32,l]) cast the same way; chunk "
                    f"{chunk_size}")


def cast_e5m2(wl: Workload, chunk_size: int | None = None) -> Workload:
    """A workload's BF16 segments and calibration draw cast to E5M2 (segment by segment), e.g.
    the escape-stress input or the ragged batch as an FP8 E5M2 KV cache."""
    def cast(words: np.ndarray) -> np.ndarray:
        out = np.empty(words.size, np.uint8)
        step = 1 << 24
        for i in range(0, words.size, step):
            out[i:i + step] = e5m2_bits(bf16_to_f32(words[i:i + step]))
        return out
    return Workload(wl.name + "_e5m2", [cast(x) for x in wl.segments], cast(wl.calibration),
                    chunk_size or wl.chunk_size, wl.description + "; cast to FP8 E5M2")


def e5m2_special_bytes(rng: np.random.Generator, count: int) -> np.ndarray:
    """Uniformly one of {0, subnormal, Inf, NaN}, random sign; subnormal mantissas 1..3,
    NaN mantissas 1..3 (raw bit patterns)."""
    cls = rng.integers(0, 4, size=count)
    sign = rng.integers(0, 2, size=count).astype(np.uint8) << np.uint8(7)
    mant = rng.integers(1, 4, size=count).astype(np.uint8)
    b = np.where(cls == 0, np.uint8(0),
        np.where(cls == 1, mant,
        np.where(cls == 2, np.uint8(0x7C), np.uint8(0x7C) | mant))).astype(np.uint8)
    return (b | sign).astype(np.uint8)


def e5m2_mixed(n: int, seed: int, wide_fraction: float = 0.02,
               special_fraction: float = 0.01) -> np.ndarray:
    """N(0,1) cast to E5M2, where a fraction gets a random power-of-two scale in 2^-20..2^20
    and a fraction is replaced by special values (zeros, subnormals, Inf, NaN)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(n, dtype=np.float32)
    wide = rng.random(n) < wide_fraction
    z[wide] *= np.exp2(rng.integers(-20, 20, size=int(wide.sum()), endpoint=True)).astype(np.float32)
    x = e5m2_bits(z)
    k = int(round(special_fraction * n))
    if k:
        x[rng.choice(n, size=k, replace=False)] = e5m2_special_bytes(rng, k)
    return x


def e5m2_random(n: int, seed: int) -> np.ndarray:
    """Uniformly random bytes (every E5M2 exponent equally likely)."""
    return np.random.default_rng(seed).integers(0, 256, size=n, dtype=np.uint8)


def e5m2_normal(n: int, seed: int, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return e5m2_bits(rng.standard_normal(n, dtype=np.float32) * np.float32(sigma))


# ---- small fuzz inputs for parity tests -------------------------------------------------

def mixed_words(n: int, seed: int, wide_fraction: float = 0.02,
                special_fraction: float = 0.01) -> np.ndarray:
    """N(0,1) BF16 words where a fraction gets a random power-of-two scale in 2^-60..2^60
    and a fraction is replaced by special values (zeros, subnormals, Inf, NaN)."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(n, dtype=np.float32)
    wide = rng.random(n) < wide_fraction
    z[wide] *= np.exp2(rng.integers(-60, 60, size=int(wide.sum()), endpoint=True)).astype(np.float32)
    x = bf16_bits(z)
    k = int(round(special_fraction * n))
    if k:
        x[rng.choice(n, size=k, replace=False)] = special_words(rng, k)
    return x


def random_words(n: int, seed: int) -> np.ndarray:
    """Uniformly random 16-bit words (every exponent equally likely)."""
    return np.random.default_rng(seed).integers(0, 1 << 16, size=n, dtype=np.uint16)


def normal_words(n: int, seed: int, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return bf16_bits(rng.standard_normal(n, dtype=np.float32) * np.float32(sigma))


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}
