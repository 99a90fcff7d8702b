"""Benchmark of the SplitZip BF16 codec on one MI355X.

A step is one pass of the hot path over one batch: encode the whole input (split,
pack, escape compaction, chunk offsets) and decode it back.  The codebook is
calibrated once on the workload's separate calibration draw before timing, as the
pages prescribe (offline calibration).  Inputs are resident in HBM before timing.

Prints one JSON line.  Throughput is GB/s of BF16 input (2 bytes per word, 10^9).
``--elem e5m2`` measures the FP8 E5M2 codec on the same inputs cast to E5M2 (GB/s of E5M2
input, 1 byte per element).  The timing protocol follows the SplitZip README's throughput
benchmark (Reproducing Paper Artifact Scripts): 10 warmup steps, 50 timed steps, reported
also as the median of 5 repeats (the timed steps in 5 equal blocks).  The line also holds
the achievable streaming ceiling of the same GPU (read, write and copy kernels shaped like
the codec's), SHA-256 digests of the input and calibration words, and the host's CPU model
and core count.  ``--input`` / ``--calibration-input`` run on saved tensors instead of the
synthetic workloads; ``--stats`` prints per-tensor exponent statistics instead of timing.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.txt")


def kernel_source_hash() -> str:
    """Identifies the kernel code the counters were taken on: the device sources with
    comments, trailing spaces and blank lines removed (a comment edit changes no kernel)."""
    h = hashlib.sha256()
    for name in ("splitzip_kernels.hip", "splitzip_e5m2.hip", "splitzip_device.h", "splitzip_internal.h"):
        with open(os.path.join(ROOT, "lossless_bf16_kv_amd", "csrc", name)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None when they
    were taken on another kernel source or workload."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    src = kernel_source_hash()
    with open(TRAFFIC_FILE) as f:
        for line in f:
            p = line.split()
            if len(p) == 5 and not line.startswith("#") and p[0] == kernel and p[1] == workload \
                    and p[2] == src:
                return {"fetch_bytes": int(p[3]), "write_bytes": int(p[4]),
                        "total_bytes": int(p[3]) + int(p[4])}
    return None


def workloads_kv_parts(flat, layers, tokens):
    import workloads
    return workloads.kv_parts(flat, layers, tokens)


def load_workload(args):
    import workloads
    if args.elem == "e5m2":
        if args.config == 3:
            return workloads.config3_e5m2(layers=args.layers, chunk_size=args.chunk_size)
        args_bf16 = argparse.Namespace(**{**vars(args), "elem": "bf16"})
        return workloads.cast_e5m2(load_workload(args_bf16), args.chunk_size)
    if args.config == 3:
        return workloads.config3(layers=args.layers, chunk_size=args.chunk_size)
    if args.config == 1 and (args.rows or args.hidden_dim):
        wl = workloads.config1(args.rows or 1024, args.hidden_dim or 4096)
        wl.chunk_size = args.chunk_size
        return wl
    if args.config == 4:
        return workloads.config4(chunk_size=args.chunk_size)
    wl = workloads.CONFIGS[args.config]()
    wl.chunk_size = args.chunk_size
    return wl


ENC_TILE_WORDS = 16384     # encode tile (words per workgroup)
ENC_TILE_E5M2 = 32768      # encode tile (E5M2 bytes per workgroup)


def algorithmic_bytes(ns, Es, C, e5m2: bool = False):
    """Bytes each kernel must move per launch (reads + writes), from the stream format.

    encode (all its launches together) reads 2n and writes the sections
    n + ceil(n/2) + 8 (n_chunks + 1) + 3E; decode is the reverse.  The pack kernel reads
    2n and writes sm, codes, tile-local chunk offsets, 4-byte scratch escapes and one
    count per tile; sums reads one count per tile; place reads the scratch escapes,
    counts and chunk offsets and writes escapes (3E) and chunk offsets.  The spill launch
    moves only the escapes of tiles with more than a slot's worth (a data-dependent
    amount), so it has no fixed figure.  Calls of at most 4096 tiles run finish instead of
    sums, place and spill: it moves what place and spill move.  The one-pass encode (one
    launch) moves exactly the encode's bytes."""
    out = {"encode": 0, "decode": 0, "encode_pack": 0, "encode_sums": 0, "encode_place": 0,
           "encode_finish": 0, "encode_onepass": 0}
    for n, E in zip(ns, Es):
        n_ch = -(-n // C)
        tiles = max(1, -(-n // (ENC_TILE_E5M2 if e5m2 else ENC_TILE_WORDS)))
        x_bytes = n if e5m2 else 2 * n                    # input elements
        sm_bytes = -(-3 * n // 8) if e5m2 else n          # sign+mantissa section
        sections = sm_bytes + (n + 1) // 2 + 8 * (n_ch + 1) + 3 * E
        out["encode"] += x_bytes + sections
        out["encode_onepass"] += x_bytes + sections
        out["decode"] += sections + x_bytes
        out["encode_pack"] += x_bytes + sm_bytes + (n + 1) // 2 + 8 * n_ch + 4 * E + 4 * tiles
        out["encode_sums"] += 4 * tiles + 8 * (-(-tiles // 2048))
        out["encode_place"] += 4 * tiles + 4 * E + 3 * E + 16 * n_ch + 8
        out["encode_finish"] += 4 * tiles + 4 * E + 3 * E + 16 * n_ch + 8
    return out


def roofline(name, bytes_, ms, workload):
    achieved = bytes_ / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
    return {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(name, workload), "algorithmic_bytes": bytes_,
            "avg_launch_ms": round(ms, 4)}


def cpu_baseline(segments, codebooks, chunk_size: int, sample_words: int, e5m2: bool = False):
    """The plain single-threaded oracle timed on a bounded prefix of the same workload
    (the first segments, each with its own codebook, up to sample_words elements)."""
    import numpy as np
    import oracle
    o = oracle.get()
    encode, decode = (o.encode8, o.decode8) if e5m2 else (o.encode, o.decode)
    t_enc = t_dec = 0.0
    words = 0
    for x, cb in zip(segments, codebooks):
        x = x[:sample_words - words]
        if x.size == 0:
            break
        t0 = time.perf_counter()
        enc = encode(x, np.frombuffer(cb, np.uint8), chunk_size)
        t1 = time.perf_counter()
        y = decode(enc)
        t2 = time.perf_counter()
        assert np.array_equal(y, x)
        t_enc += t1 - t0
        t_dec += t2 - t1
        words += x.size
    gb = (1 if e5m2 else 2) * words / 1e9
    kind = "E5M2 bytes" if e5m2 else "BF16 words"
    return {"value": round(gb / (t_enc + t_dec), 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {words} {kind} of the timed workload, encode + decode, "
                      f"single-threaded plain C",
            "encode_GBps": round(gb / t_enc, 4), "decode_GBps": round(gb / t_dec, 4)}


def sha256_words(arrays) -> str:
    """SHA-256 of the arrays' bytes, in order (little-endian words as stored)."""
    import numpy as np
    h = hashlib.sha256()
    step = 1 << 28
    for a in arrays:
        b = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
        for i in range(0, b.size, step):
            h.update(memoryview(b[i:i + step]))
    return h.hexdigest()


def host_info() -> dict:
    """CPU model and core counts of the host this runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cores": usable}


def ceiling_leg(dev, reps: int = 10, mib: int = 4096) -> dict:
    """Median GB/s (bytes read + written) of streaming kernels shaped like the codec's:
    16-byte lane-contiguous nontemporal accesses, 32 KiB per 256-thread workgroup, tiles in
    contiguous ranges per XCD; read and write over mib MiB, copy of mib/2 MiB."""
    import ctypes
    import torch
    from lossless_bf16_kv_amd import build as szbuild
    if not os.path.exists(szbuild.CEILING_PATH):
        raise RuntimeError(f"{szbuild.CEILING_PATH} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(szbuild.CEILING_PATH)
    L.szc_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                             ctypes.c_void_p, ctypes.c_void_p]
    L.szc_stream.restype = ctypes.c_int
    nb = mib << 20
    a = torch.ones(nb // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for kind, name in enumerate(("read", "write", "copy")):
        nbytes = nb if kind != 2 else nb // 2
        times = []
        for r in range(reps + 2):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            rc = L.szc_stream(kind, a.data_ptr(), b.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream)
            ev[1].record(stream)
            if rc != 0:
                raise RuntimeError(f"ceiling kernel {name}: HIP error {rc}")
            torch.cuda.synchronize()
            if r >= 2:
                times.append(ev[0].elapsed_time(ev[1]))
        moved = nb                       # copy: nb / 2 read + nb / 2 written
        out[name + "_GBps"] = round(moved / (sorted(times)[len(times) // 2] * 1e-3) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    out["kernels"] = "stream_ceiling.hip: 16 B per lane, 32 KiB per workgroup, XCD-contiguous tiles, " \
                     f"nontemporal; read/write {mib} MiB, copy {mib // 2} MiB; median of {reps}"
    return out


def floor_leg(dev, nbytes: int, flush, reps: int = 10) -> dict:
    """What a call on this small input costs before any codec work: median microseconds,
    with the caches flushed before each launch as in the timed steps, of a launch whose one
    tile reads 16 bytes, and of the copy kernel of ceiling_leg over the call's own
    input (reads and writes nbytes, about as many bytes as an encode or a decode moves)."""
    import ctypes
    import torch
    from lossless_bf16_kv_amd import build as szbuild
    L = ctypes.CDLL(szbuild.CEILING_PATH)
    L.szc_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                             ctypes.c_void_p, ctypes.c_void_p]
    L.szc_stream.restype = ctypes.c_int
    nbytes = (nbytes + 15) // 16 * 16
    a = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    b = torch.empty_like(a)
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, kind, size in (("one_tile_launch_us", 0, 16), ("copy_input_us", 2, nbytes)):
        times = []
        for r in range(reps + 2):
            flush()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            rc = L.szc_stream(kind, a.data_ptr(), b.data_ptr(), size, sink.data_ptr(), stream.cuda_stream)
            ev[1].record(stream)
            if rc != 0:
                raise RuntimeError(f"floor kernel {name}: HIP error {rc}")
            torch.cuda.synchronize()
            if r >= 2:
                times.append(ev[0].elapsed_time(ev[1]) * 1e3)
        out[name] = round(sorted(times)[len(times) // 2], 2)
    out["copy_bytes"] = 2 * nbytes
    out["copy_GBps"] = round(2 * nbytes / (out["copy_input_us"] * 1e-6) / 1e9, 1)
    out["basis"] = f"median of {reps} launches, caches flushed before each, events on the launch stream"
    return out


def ceiling_fraction(read_bytes: int, write_bytes: int, ms: float, ceil: dict) -> float:
    """Time a kernel would take reading and then writing its bytes at the measured read and
    write ceilings, over its measured time."""
    model_s = read_bytes / (ceil["read_GBps"] * 1e9) + write_bytes / (ceil["write_GBps"] * 1e9)
    return round(model_s / (ms * 1e-3), 4)


def load_saved(path: str, elem: str) -> list:
    """(name, flat numpy array) of every tensor in a saved file, loaded without executing
    anything from it: .safetensors, .pt/.pth (torch.load with weights_only), .npy (no
    pickles).  BF16 tensors give their uint16 words (raw int16/uint16 arrays are taken as
    words); for --elem e5m2, float8_e5m2 tensors or raw uint8 bytes."""
    import numpy as np
    import torch
    ext = os.path.splitext(path)[1].lower()
    if ext == ".safetensors":
        from safetensors.torch import load_file
        items = list(load_file(path).items())
    elif ext in (".pt", ".pth"):
        obj = torch.load(path, map_location="cpu", weights_only=True)
        if isinstance(obj, torch.Tensor):
            items = [(os.path.basename(path), obj)]
        elif isinstance(obj, dict):
            items = list(obj.items())
        elif isinstance(obj, (list, tuple)):
            items = [(f"{i}", t) for i, t in enumerate(obj)]
        else:
            raise SystemExit(f"{path}: expected a tensor, a dict or a list of tensors")
    elif ext == ".npy":
        items = [(os.path.basename(path), torch.from_numpy(np.load(path, allow_pickle=False)))]
    else:
        raise SystemExit(f"{path}: unsupported file type (use .safetensors, .pt/.pth or .npy)")
    out = []
    for name, t in items:
        if not isinstance(t, torch.Tensor):
            raise SystemExit(f"{path}: entry {name} is not a tensor")
        t = t.contiguous().reshape(-1)
        if elem == "e5m2":
            if t.dtype not in (torch.float8_e5m2, torch.uint8):
                raise SystemExit(f"{path}: {name} is {t.dtype}; --elem e5m2 needs float8_e5m2 or uint8")
            out.append((str(name), t.view(torch.uint8).numpy().copy()))
        else:
            if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
                raise SystemExit(f"{path}: {name} is {t.dtype}; the BF16 codec needs bfloat16 "
                                 f"(or raw 16-bit words)")
            out.append((str(name), t.view(torch.int16).numpy().view(np.uint16).copy()))
    if not out:
        raise SystemExit(f"{path}: no tensors")
    return out


def saved_workload(args):
    """A workload from --input (every tensor a segment) and --calibration-input (all its
    tensors pooled; default: the input itself)."""
    import numpy as np
    import workloads
    parts = load_saved(args.input, args.elem)
    if args.calibration_input:
        cal = np.concatenate([a for _, a in load_saved(args.calibration_input, args.elem)])
        cal_note = f"calibrated on {os.path.basename(args.calibration_input)}"
    else:
        cal = np.concatenate([a for _, a in parts])
        cal_note = "calibrated on the input itself"
    names = [nm for nm, _ in parts]
    wl = workloads.Workload(name="saved_" + os.path.splitext(os.path.basename(args.input))[0],
                            segments=[a for _, a in parts], calibration=cal, chunk_size=args.chunk_size,
                            description=f"saved tensors from {os.path.basename(args.input)} "
                                        f"({len(parts)} tensors); {cal_note}")
    return wl, names


def exponent_report(xs, names, elem: str) -> list:
    """Per tensor: exponent entropy (bits), top-16 codebook and its coverage, distinct
    exponents (histograms on the GPU, one pass over all tensors)."""
    import lossless_bf16_kv_amd as sz
    hists = sz.histograms(xs, elem=elem)
    out = []
    for name, x, h in zip(names, xs, hists):
        st = sz.exponent_stats(list(h) + [0] * (256 - len(h)))
        out.append({"tensor": name, "elements": int(x.numel()), "entropy_bits": round(st["entropy_bits"], 6),
                    "coverage_top16": st["coverage"], "distinct_exponents": st["distinct"],
                    "codebook": st["codebook"].hex()})
    return out


def transfer_bench(args, codec, xs, books, wl, esize, coverage):
    """Compressed against raw transfer of the tensors xs across the host link (one JSON line)."""
    import torch
    from lossless_bf16_kv_amd.transfer import TransferPlan
    # the tensors as consecutive views of one pool on each side, as a KV pool holds them
    sizes = [x.numel() for x in xs]
    pool_in = torch.cat([x.view(-1) for x in xs])
    pool_out = torch.empty_like(pool_in)
    xs[:] = list(pool_in.split(sizes))
    ys = list(pool_out.split(sizes))
    # the sending buffers sized from the escape counts of a first encode
    first = codec.encode_packed_batch(xs, books=books)
    escapes = [p.n_escapes for p in first]
    del first
    plan = TransferPlan(codec, xs, ys, books, escapes=escapes)
    n = sum(x.numel() for x in xs)
    times = {True: [], False: []}
    link = {}
    for k in range(args.warmup + args.steps):
        for compress in (True, False):        # interleaved
            pool_out.zero_()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            link[compress] = plan.run(compress)
            dt = time.perf_counter() - t0
            assert all(torch.equal(x, y) for x, y in zip(xs, ys)), "transfer is not bitwise"
            if k >= args.warmup:
                times[compress].append(dt)
    comp_s = sorted(times[True])[len(times[True]) // 2]
    raw_s = sorted(times[False])[len(times[False]) // 2]
    out = {
        "metric": "KV transfer across the PCIe link (device to pinned host to device, spans of "
                  "streams pipelined): GB/s of " + ("E5M2" if esize == 1 else "BF16") + " moved, compressed",
        "value": round(esize * n / comp_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(comp_s * 1e3, 3),
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": "u8" if esize == 1 else "u16",
        "data": "synthetic",
        "config": {"workload": wl.name, "element": args.elem, "n_elements": n, "tensors": len(xs),
                   "chunk_size": wl.chunk_size, "input_bytes": esize * n},
        "raw_GBps": round(esize * n / raw_s / 1e9, 2),
        "speedup": round(raw_s / comp_s, 4),
        "ms": {"compressed_median": round(comp_s * 1e3, 3), "raw_median": round(raw_s * 1e3, 3),
               "compressed_min": round(min(times[True]) * 1e3, 3), "raw_min": round(min(times[False]) * 1e3, 3)},
        "link_bytes": {"compressed": link[True], "raw": link[False]},
        "compression_ratio": round(link[False] / link[True], 5),
        "n_escapes": sum(plan.n_escapes),
        "coverage_calibration": coverage,
        "timing": "wall clock of each whole transfer (all tensors), from the first encode to the "
                  "last decode; median over the timed runs",
        "round_trip_bitwise": True,
    }
    plan.close()
    emit(out, args.output)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", "--iters", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--repeats", type=int, default=5,
                    help="the timed steps in this many equal blocks; their median is reported too")
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--chunk-size", type=int, default=1024)
    ap.add_argument("--rows", type=int, default=0,
                    help="single N(0,1) tensor of [rows, hidden-dim] (selects --config 1)")
    ap.add_argument("--hidden-dim", type=int, default=0, help="see --rows (default 4096)")
    ap.add_argument("--calibrate-on-input", action="store_true",
                    help="calibrate on the benchmark input itself instead of the workload's "
                         "separate calibration draw")
    ap.add_argument("--layers", type=int, default=64, help="long-prefill KV layers (64 = 8.6 GB)")
    ap.add_argument("--books", choices=["one", "layer-kv"], default="one",
                    help="one codebook for the whole input, or (long-prefill KV) one per layer "
                         "and K/V, each tensor its own segment")
    ap.add_argument("--packed", action="store_true",
                    help="encode into / decode from one contiguous packed stream per segment")
    ap.add_argument("--elem", choices=["bf16", "e5m2"], default="bf16",
                    help="element type: BF16 words, or the configuration's inputs cast to FP8 E5M2")
    ap.add_argument("--scrub-mb", type=int, default=-1,
                    help="MiB read between timed steps to flush the 256 MB Infinity Cache "
                         "(default: 2048 when the input is under 1 GiB, else 0)")
    ap.add_argument("--transfer", action="store_true",
                    help="time the compressed, pipelined transfer of the input's tensors (the "
                         "long-prefill KV: one per layer and K/V) across the PCIe link through "
                         "pinned host memory against the raw transfer, instead of the codec")
    ap.add_argument("--input", default="",
                    help="saved tensors to encode (.safetensors, .pt/.pth loaded weights-only, "
                         ".npy): every tensor one segment")
    ap.add_argument("--calibration-input", default="",
                    help="saved tensors to calibrate on (default: the input itself)")
    ap.add_argument("--output", default="", help="also write the JSON line to this file")
    ap.add_argument("--stats", action="store_true",
                    help="print per-tensor exponent statistics (entropy, top-16 coverage, distinct "
                         "exponents; the long-prefill KV per layer and K/V) instead of timing")
    ap.add_argument("--cpu-sample-words", type=int, default=1 << 30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-digests", action="store_true", help="skip the SHA-256 of the inputs")
    args = ap.parse_args(argv)
    if args.rows or args.hidden_dim:
        args.config = 1
    args.repeats = max(1, min(args.repeats, args.steps))

    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1 (segments "
                                   "shard across GPUs with no exchange between them)"}))
        sys.exit(2)

    import numpy as np
    import torch
    import lossless_bf16_kv_amd as sz

    t_gen = time.perf_counter()
    seg_names = None
    if args.input:
        wl, seg_names = saved_workload(args)
    else:
        wl = load_workload(args)
    if args.calibrate_on_input:
        wl.calibration = np.concatenate(wl.segments) if len(wl.segments) > 1 else wl.segments[0]
        wl.description += "; calibrated on the input itself"
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    C = wl.chunk_size

    segments, cal_parts, books = wl.segments, [wl.calibration], None
    if args.input and (args.books != "one" or args.transfer):
        raise SystemExit("--books layer-kv and --transfer apply to the synthetic long-prefill KV only")
    if args.transfer and args.config == 3:
        # one tensor per layer and K/V, as a serving stack would send them
        tokens = wl.segments[0].size // (2 * args.layers * 1024)
        segments = workloads_kv_parts(wl.segments[0], args.layers, tokens)
    if args.books == "layer-kv":
        if args.config != 3:
            raise SystemExit("--books layer-kv applies to the long-prefill KV workload (--config 3)")
        tokens = wl.segments[0].size // (2 * args.layers * 1024)
        segments = workloads_kv_parts(wl.segments[0], args.layers, tokens)
        cal_parts = workloads_kv_parts(wl.calibration, args.layers, wl.calibration.size // (2 * args.layers * 1024))
        books = list(range(len(segments)))
    e5m2 = args.elem == "e5m2"
    esize = 1 if e5m2 else 2                      # bytes per input element
    view = (lambda a: a) if e5m2 else (lambda a: a.view(np.int16))
    if args.stats:
        xs = [torch.from_numpy(view(s)).to(dev) for s in segments]
        names = seg_names or [f"segment {i}" for i in range(len(xs))]
        if args.config == 3 and not args.input and len(xs) == 1:
            # the long-prefill KV: one tensor per layer and K/V
            tokens = wl.segments[0].size // (2 * args.layers * 1024)
            xs = list(xs[0].split(tokens * 1024))
            names = [f"layer {i // 2} {'KV'[i % 2]}" for i in range(len(xs))]
        out = {"metric": "exponent statistics per tensor (entropy bits, top-16 coverage, distinct "
                         "exponents)", "element": args.elem, "data": "synthetic" if not args.input else "saved",
               "config": {"workload": wl.name, "tensors": len(xs), "description": wl.description},
               "tensors": exponent_report(xs, names, args.elem)}
        emit(out, args.output)
        return
    xs = [torch.from_numpy(view(s)).to(dev) for s in segments]
    cals = [torch.from_numpy(view(c)).to(dev) for c in cal_parts]
    codec = sz.Codec(dev, C, elem=args.elem)
    if books is None:
        coverage = codec.calibrate(cals[0])
    else:
        coverage = min(codec.calibrate_books(cals))
    del cals
    if args.transfer:
        transfer_bench(args, codec, xs, books, wl, esize, coverage)
        return
    # exponent statistics of the input itself (one pass on the GPU)
    hist_in = np.sum(np.array(sz.histograms(xs, elem=args.elem), dtype=np.uint64), axis=0).tolist()
    stats_in = sz.exponent_stats(hist_in)
    # no coder that keeps the sign+mantissa bits exact beats (element bits) / (kept bits + H)
    kept_bits = 3 if e5m2 else 8
    entropy_bound = 8 * esize / (kept_bits + stats_in["entropy_bits"])

    # sizes the escape arrays or stream buffers (retry if needed)
    if args.packed:
        encs = codec.encode_packed_batch(xs, books=books)
    else:
        encs = codec.encode_batch(xs, books=books)
    ys = [torch.empty_like(x) for x in xs]
    result = torch.zeros(1 + len(xs), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    # buffers fixed across steps
    batch = codec.prepare_packed(xs, encs, ys) if args.packed else codec.prepare(xs, encs, ys)
    batch.encode_async(result)
    torch.cuda.synchronize()
    assert batch.finish(result) == sz.OK

    # One step = encode (non-blocking: escape counts stay in device memory, as a transfer
    # engine would consume them) + decode, both enqueued on the same stream.  The encoded
    # sizes do not change from step to step, so decode uses the counts read after warmup.
    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        batch.encode_async(result)
        if ev is not None:
            ev[1].record(stream)
        batch.decode()
        if ev is not None:
            ev[2].record(stream)

    # Inputs that fit the 256 MB Infinity Cache would otherwise be timed hot: a read of a larger
    # buffer between steps (outside the timed events) evicts them.  Then the step time comes
    # from the events, since the wall clock also holds the scrubs.
    input_bytes = sum(x.numel() * x.element_size() for x in xs)
    scrub_mb = args.scrub_mb if args.scrub_mb >= 0 else (2048 if input_bytes < (1 << 30) else 0)
    scrub = torch.ones(scrub_mb << 18, dtype=torch.int32, device=dev) if scrub_mb else None
    sink = torch.zeros((), dtype=torch.int64, device=dev)

    def flush():
        if scrub is not None:
            sink.add_(torch.sum(scrub, dtype=torch.int64))

    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize()
    assert batch.finish(result) == sz.OK

    def timed(per_kernel):
        """K steps; per_kernel: HIP events around every kernel launch as well."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        codec.profile(per_kernel)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            flush()
            step(evs[k])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        kt = codec.kernel_times() if per_kernel else None
        codec.profile(False)
        return evs, t1 - t0, kt

    # The step time comes from K steps with events only between encode and decode.  The events
    # around each kernel launch add a few microseconds per launch on the GPU timeline (twice
    # the time of an 8 MB encode), so the per-kernel times come from a second pass of K steps.
    events, wall_s, _ = timed(False)
    prof_events, _, ktimes = timed(True)

    # verify the escape counts and the bitwise round trip before reporting
    assert batch.finish(result) == sz.OK
    for x, y in zip(xs, ys):
        assert torch.equal(x, y), "round trip is not bitwise"

    # the timed steps in args.repeats equal blocks (step times from the events)
    blocks = []
    per = args.steps // args.repeats
    for r in range(args.repeats):
        evb = events[r * per:(r + 1) * per if r + 1 < args.repeats else args.steps]
        if scrub is None:
            ms = evb[0][0].elapsed_time(evb[-1][2])
        else:
            ms = sum(e[0].elapsed_time(e[2]) for e in evb)
        blocks.append(round(esize * sum(x.numel() for x in xs) * len(evb) / (ms * 1e-3) / 1e9, 2))
    enc_ms = sorted(e[0].elapsed_time(e[1]) for e in events)
    dec_ms = sorted(e[1].elapsed_time(e[2]) for e in events)
    enc_avg = sum(enc_ms) / len(enc_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    ns = [e.n for e in encs]
    Es = [e.n_escapes for e in encs]
    n = sum(ns)
    E = sum(Es)
    comp = sum(e.compressed_bytes for e in encs)
    alg = algorithmic_bytes(ns, Es, C, e5m2)
    prof_ms = sum(e[0].elapsed_time(e[2]) for e in prof_events) / len(prof_events)
    if scrub is None:
        value = esize * n * args.steps / wall_s / 1e9
        step_ms = wall_s / args.steps * 1e3
    else:
        step_ms = enc_avg + dec_avg
        value = esize * n / (step_ms * 1e-3) / 1e9
    wname = wl.name + f"_c{C}" + ("_books_layer_kv" if books is not None else "") + \
        ("_packed" if args.packed else "")

    # Place and spill split the escapes between them by a data-dependent rule (a tile's
    # escapes beyond its slot go through spill), so only the pair has a fixed figure:
    # place's algorithmic bytes over the two launches' times together.
    pair = "encode_place" in alg and all(ktimes.get(k, (0, 0))[1]
                                         for k in ("encode_place", "encode_spill"))
    kernels = {k: roofline(k, alg[k], ms, wname) for k, (ms, cnt) in ktimes.items()
               if cnt and k in alg and not (pair and k == "encode_place")}
    kernels.update({k: {"kernel": k, "avg_launch_ms": round(ms, 4)}
                    for k, (ms, cnt) in ktimes.items()
                    if cnt and (k not in alg or (pair and k == "encode_place"))})
    for k, (ms, cnt) in ktimes.items():
        if k in kernels:
            kernels[k]["launches_timed"] = cnt
    if pair:
        kernels["encode_place+spill"] = roofline(
            "encode_place+spill", alg["encode_place"],
            ktimes["encode_place"][0] + ktimes["encode_spill"][0], wname)
        kernels["encode_place+spill"]["launches_timed"] = ktimes["encode_place"][1]
    # the kernel that moves the data: on small inputs a short launch can outlast it
    dominant = max((k for k in ("encode_pack", "encode_onepass", "decode") if k in kernels),
                   key=lambda k: kernels[k]["avg_launch_ms"])
    ops = {"encode": roofline("encode (all launches)", alg["encode"], enc_avg, wname),
           "decode": roofline("decode", alg["decode"], dec_avg, wname)}

    ceiling = None
    if not args.no_ceiling:
        ceiling = ceiling_leg(dev)
        # the same bytes read and then written at the read and write ceilings, over the
        # measured time: how close each op and kernel comes to what the GPU streams
        comp_bytes = sum(e.compressed_bytes for e in encs)
        x_bytes = esize * n
        ceiling["frac_of_read_then_write"] = {
            "encode": ceiling_fraction(x_bytes, comp_bytes, enc_avg, ceiling),
            "decode": ceiling_fraction(comp_bytes, x_bytes, dec_avg, ceiling)}
        for k in ("encode_pack", "encode_onepass"):
            if k in kernels:
                pk = kernels[k]
                ceiling["frac_of_read_then_write"][k] = ceiling_fraction(
                    x_bytes, pk["algorithmic_bytes"] - x_bytes, pk["avg_launch_ms"], ceiling)
        if "decode" in kernels:
            ceiling["frac_of_read_then_write"]["decode_kernel"] = ceiling_fraction(
                comp_bytes, x_bytes, kernels["decode"]["avg_launch_ms"], ceiling)

    floor = None
    if scrub is not None and not args.no_ceiling:
        floor = floor_leg(dev, esize * n, flush)

    digests = None
    if not args.no_digests:
        digests = {"input_sha256": sha256_words(segments), "calibration_sha256": sha256_words(cal_parts),
                   "basis": "SHA-256 of the input words (all segments in order) and of the "
                            "calibration words, as stored (little-endian)"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(segments, [codec.books[e.book] for e in encs], C, args.cpu_sample_words, e5m2)

    metric = "encode & decode GB/s (BF16 in) + % HBM roofline + compression ratio" + \
        (", 8.6 GB KV" if args.config == 3 and args.layers == 64 and not args.input else "")
    if e5m2:
        metric = "encode & decode GB/s (E5M2 in) + % HBM roofline + compression ratio" + \
            (", 4.3 GB E5M2 KV" if args.config == 3 and args.layers == 64 and not args.input else "")
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8" if e5m2 else "u16",
        "data": "synthetic",
        "config": {"workload": wl.name, "element": args.elem, "n_elements": n, "segments": len(ns),
                   "chunk_size": C, "codebooks": len(codec.books), "packed_streams": bool(args.packed),
                   "input_bytes": esize * n, "description": wl.description},
        "encode_GBps": round(esize * n / (enc_avg * 1e-3) / 1e9, 2),
        "decode_GBps": round(esize * n / (dec_avg * 1e-3) / 1e9, 2),
        "encode_hbm_frac": ops["encode"]["frac"],
        "decode_hbm_frac": ops["decode"]["frac"],
        "encode_ms": {"avg": round(enc_avg, 4), "min": round(enc_ms[0], 4),
                      "median": round(enc_ms[len(enc_ms) // 2], 4)},
        "decode_ms": {"avg": round(dec_avg, 4), "min": round(dec_ms[0], 4),
                      "median": round(dec_ms[len(dec_ms) // 2], 4)},
        "compression_ratio": round(esize * n / comp, 5),
        "compressed_bytes": comp,
        "n_escapes": E,
        "coverage_calibration": coverage,
        "coverage_input": 1 - E / n if n else None,
        "exponent_entropy_bits": round(stats_in["entropy_bits"], 5),
        "entropy_bound_ratio": round(entropy_bound, 5),
        "roofline": kernels[dominant],
        "roofline_ops": ops,
        "roofline_kernels": kernels,
        "kernel_times_basis": "a second pass of the same steps with HIP events around every "
                              "kernel launch on the launch stream",
        "profiled_pass_ms_per_step": round(prof_ms, 4),
        "repeats": {"n": args.repeats, "GBps": blocks, "median_GBps": sorted(blocks)[len(blocks) // 2],
                    "basis": f"the {args.steps} timed steps in {args.repeats} blocks, each timed with "
                             "events"},
        "ceiling": ceiling,
        "small_call_floor": floor,
        "cpu_baseline": cpu,
        "host": host_info(),
        "inputs": digests,
        "generate_s": round(t_gen, 1),
        "kernel_source": kernel_source_hash(),
        "round_trip_bitwise": True,
        "cache_scrub_mb": scrub_mb,
        "value_basis": "wall clock over the timed steps" if scrub is None else
                       "encode + decode events (cache flushed between steps)",
    }
    emit(out, args.output)


def emit(out: dict, path: str = "") -> None:
    line = json.dumps(out)
    print(line, flush=True)
    if path:
        with open(path, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
