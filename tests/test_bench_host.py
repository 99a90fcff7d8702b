"""Host-side checks of bench.py (no GPU): the algorithmic byte counts that every roofline
figure divides by, the roofline record, the HBM-traffic lookup keyed by the kernel code
hash, and the refusal of more than one GPU."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_bf16():
    # n = 49157 words at C = 1024: 49 chunks, 4 pack tiles of 16384 words, E = 100.
    # Stream sections: sm 49157 + codes 24579 + offsets 8 * 50 = 400 + escapes 3 * 100 = 300.
    alg = bench.algorithmic_bytes([49157], [100], 1024)
    assert alg["encode"] == alg["decode"] == 2 * 49157 + 74436
    # pack: reads 2n, writes sm, codes, 49 tile-local offsets, 100 four-byte scratch
    # escapes and 4 tile counts
    assert alg["encode_pack"] == 98314 + 49157 + 24579 + 392 + 400 + 16
    # sums: 4 tile counts, one 2048-tile block total
    assert alg["encode_sums"] == 16 + 8
    # place (and finish): counts, scratch escapes read and written as 3 B, offsets read and
    # written, E
    assert alg["encode_place"] == alg["encode_finish"] == 16 + 400 + 300 + 784 + 8
    # the one-pass launch: exactly the encode's bytes
    assert alg["encode_onepass"] == alg["encode"]


def test_algorithmic_bytes_e5m2_and_batches():
    # n = 65543 E5M2 bytes at C = 1024: 65 chunks, 3 pack tiles of 32768, E = 10;
    # field stream ceil(3n / 8) = 24579, codes 32772, offsets 8 * 66 = 528, escapes 30
    alg = bench.algorithmic_bytes([65543], [10], 1024, e5m2=True)
    assert alg["encode"] == alg["decode"] == 65543 + 24579 + 32772 + 528 + 30
    # a batch adds up its segments; an empty segment still has its one chunk offset
    two = bench.algorithmic_bytes([49157, 0], [100, 0], 1024)
    one = bench.algorithmic_bytes([49157], [100], 1024)
    assert two["encode"] == one["encode"] + 8
    assert two["encode_pack"] == one["encode_pack"] + 4


def test_roofline_record():
    r = bench.roofline("decode", 8_000_000_000, 2.0, "no_such_workload")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["achieved"] == 4000.0 and r["frac"] == 0.5
    assert r["traffic"] is None and r["avg_launch_ms"] == 2.0


def test_traffic_lookup_needs_the_same_kernel_code(tmp_path, monkeypatch):
    src = bench.kernel_source_hash()
    assert len(src) == 16 and src == bench.kernel_source_hash()
    f = tmp_path / "pmc_traffic.txt"
    f.write_text("# comment\n"
                 f"decode wl {src} 1000 2000\n"
                 f"decode wl {'0' * 16} 5 5\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("decode", "wl") == {"fetch_bytes": 1000, "write_bytes": 2000,
                                                      "total_bytes": 3000}
    assert bench.measured_traffic("decode", "other") is None
    assert bench.measured_traffic("encode_pack", "wl") is None


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert p.returncode == 2
    assert "one GPU" in json.loads(p.stdout.strip().splitlines()[-1])["error"]


def test_input_digests_and_host_record():
    import hashlib

    import numpy as np
    a = np.arange(1000, dtype=np.uint16)
    b = np.arange(7, dtype=np.uint16)[::-1]
    assert bench.sha256_words([a, b]) == hashlib.sha256(a.tobytes() + b.copy().tobytes()).hexdigest()
    info = bench.host_info()
    assert info["nproc"] == os.cpu_count() and 1 <= info["usable_cores"] <= info["nproc"]


def test_ceiling_fraction():
    # 6 GB read at 6000 GB/s (1 ms) then 4 GB written at 4000 GB/s (1 ms): 2 ms of model
    # time against a 4 ms kernel
    ceil = {"read_GBps": 6000.0, "write_GBps": 4000.0}
    assert bench.ceiling_fraction(6_000_000_000, 4_000_000_000, 4.0, ceil) == 0.5


def test_saved_inputs_load_without_executing_anything(tmp_path):
    import numpy as np
    import pytest
    import torch
    from safetensors.torch import save_file
    k = torch.randn(4, 8, 16).to(torch.bfloat16)
    v = torch.randn(4, 8, 16).to(torch.bfloat16)
    words = lambda t: t.reshape(-1).view(torch.int16).numpy().view(np.uint16)
    save_file({"k": k, "v": v}, str(tmp_path / "kv.safetensors"))
    torch.save({"k": k, "v": v}, str(tmp_path / "kv.pt"))
    np.save(str(tmp_path / "k.npy"), words(k))
    for f in ("kv.safetensors", "kv.pt"):
        got = dict(bench.load_saved(str(tmp_path / f), "bf16"))
        assert set(got) == {"k", "v"}
        assert np.array_equal(got["k"], words(k)) and np.array_equal(got["v"], words(v))
    (name, arr), = bench.load_saved(str(tmp_path / "k.npy"), "bf16")
    assert np.array_equal(arr, words(k))
    # E5M2 tensors for the E5M2 codec; a float32 tensor is refused for either
    e = torch.randn(100).to(torch.float8_e5m2)
    torch.save(e, str(tmp_path / "e.pt"))
    (_, b8), = bench.load_saved(str(tmp_path / "e.pt"), "e5m2")
    assert np.array_equal(b8, e.view(torch.uint8).numpy())
    torch.save(torch.randn(10), str(tmp_path / "f.pt"))
    with pytest.raises(SystemExit):
        bench.load_saved(str(tmp_path / "f.pt"), "bf16")
    with pytest.raises(SystemExit):
        bench.load_saved(str(tmp_path / "kv.pt"), "e5m2")
    # a saved object outside the weights-only allowlist is refused by the loader
    import datetime
    torch.save({"k": datetime.date(2020, 1, 1)}, str(tmp_path / "obj.pt"))
    with pytest.raises(Exception) as ei:
        bench.load_saved(str(tmp_path / "obj.pt"), "bf16")
    assert "weights" in str(ei.value).lower() or "unpickl" in str(ei.value).lower()


def test_saved_workload_calibrates_on_the_given_tensors(tmp_path):
    import argparse

    import numpy as np
    import torch
    from safetensors.torch import save_file
    save_file({"a": torch.randn(64).to(torch.bfloat16), "b": torch.randn(32).to(torch.bfloat16)},
              str(tmp_path / "x.safetensors"))
    save_file({"c": torch.randn(48).to(torch.bfloat16)}, str(tmp_path / "cal.safetensors"))
    args = argparse.Namespace(input=str(tmp_path / "x.safetensors"), calibration_input="",
                              elem="bf16", chunk_size=1024)
    wl, names = bench.saved_workload(args)
    assert names == ["a", "b"] and [s.size for s in wl.segments] == [64, 32]
    assert wl.calibration.size == 96
    args.calibration_input = str(tmp_path / "cal.safetensors")
    wl, _ = bench.saved_workload(args)
    assert wl.calibration.size == 48 and wl.chunk_size == 1024
