"""GPU tests of the benchmark's own paths: saved input tensors (calibrated on a saved
calibration file), the per-tensor exponent statistics against the oracle's, the JSON line's
sizes, escape counts and digests against the oracle and hashlib, and the streaming ceiling
kernels."""
from __future__ import annotations

import hashlib
import json

import numpy as np
import pytest
import torch
from safetensors.torch import save_file

import bench
import oracle
import workloads

pytestmark = pytest.mark.gpu

O = oracle.get()
DEV = torch.device("cuda:0")


def bf16(words: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words, np.uint16).view(np.int16)).view(torch.bfloat16)


@pytest.fixture(scope="module")
def saved(tmp_path_factory):
    d = tmp_path_factory.mktemp("saved")
    wl = workloads.config2(tokens=700)                # K and V of one GQA layer, 700 tokens
    k, v = wl.segments
    path = str(d / "kv.safetensors")
    save_file({"k": bf16(k).reshape(700, 8, 128), "v": bf16(v).reshape(700, 8, 128)}, path)
    cal = str(d / "cal.safetensors")
    save_file({"cal": bf16(wl.calibration)}, cal)
    return path, cal, {"k": k, "v": v}, wl.calibration, d


def test_stats_mode_equals_oracle_per_tensor(saved):
    path, _, parts, _, d = saved
    out = str(d / "stats.json")
    bench.main(["--input", path, "--stats", "--output", out])
    rec = json.loads(open(out).read())
    assert [t["tensor"] for t in rec["tensors"]] == ["k", "v"]
    for t in rec["tensors"]:
        x = parts[t["tensor"]]
        h = O.histogram(x)
        cb = O.codebook(h)
        assert t["elements"] == x.size
        assert t["codebook"] == bytes(cb).hex()
        assert t["coverage_top16"] == O.coverage(h, cb, x.size)
        assert t["distinct_exponents"] == int(np.count_nonzero(h))
        assert abs(t["entropy_bits"] - O.entropy(h)) <= 1e-6


def test_saved_input_bench_line(saved):
    path, cal, parts, cal_words, d = saved
    out = str(d / "bench.json")
    bench.main(["--input", path, "--calibration-input", cal, "--steps", "6", "--warmup", "2",
                "--repeats", "3", "--no-cpu-baseline", "--no-ceiling", "--output", out])
    rec = json.loads(open(out).read())
    cb, _, _ = O.calibrate(cal_words)
    refs = [O.encode(parts[k], cb, 1024) for k in ("k", "v")]
    assert rec["n_escapes"] == sum(r["n_escapes"] for r in refs)
    assert rec["compressed_bytes"] == sum(r["compressed_bytes"] for r in refs)
    assert rec["round_trip_bitwise"] and rec["config"]["segments"] == 2
    assert rec["inputs"]["input_sha256"] == hashlib.sha256(parts["k"].tobytes() + parts["v"].tobytes()).hexdigest()
    assert rec["inputs"]["calibration_sha256"] == hashlib.sha256(cal_words.tobytes()).hexdigest()
    assert rec["repeats"]["n"] == 3 and len(rec["repeats"]["GBps"]) == 3
    assert rec["steps"] == 6 and rec["warmup"] == 2


def test_ceiling_kernels():
    c = bench.ceiling_leg(DEV, reps=2, mib=256)
    for k in ("read_GBps", "write_GBps", "copy_GBps"):
        assert 100.0 < c[k] < 20000.0, (k, c[k])
    # the copy kernel copies: a pattern survives it
    import ctypes
    from lossless_bf16_kv_amd import build as szbuild
    L = ctypes.CDLL(szbuild.CEILING_PATH)
    L.szc_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                             ctypes.c_void_p, ctypes.c_void_p]
    a = torch.arange(1 << 20, dtype=torch.int32, device=DEV)
    b = torch.zeros_like(a)
    assert L.szc_stream(2, a.data_ptr(), b.data_ptr(), a.numel() * 4, None,
                        torch.cuda.current_stream(DEV).cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_small_call_floor():
    flushes = []
    f = bench.floor_leg(DEV, 64 << 20, lambda: flushes.append(1), reps=3)
    assert len(flushes) == 2 * 5
    # a 16-byte launch against a copy of 64 MiB (reads and writes 128 MiB in all)
    assert 0 < f["one_tile_launch_us"] < f["copy_input_us"] < 10_000
    assert f["copy_bytes"] == 2 * (64 << 20)
