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
