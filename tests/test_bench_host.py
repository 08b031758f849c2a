"""Host-side logic of bench.py (no GPU): the single-GPU refusal, the roofline
and step-record arithmetic, the weight-copy rotation, the host description
and the counter records' keying to the kernel sources."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test",
                                                  os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in out["error"]


def test_roofline_fractions(bench):
    h = bench.hbm_roof(8.0e9, 1000.0, "k", [])  # 8 GB in 1 ms: 8 TB/s
    assert h["bound"] == "hbm" and h["unit"] == "GB/s" and h["peak"] == 8000.0
    assert h["achieved"] == pytest.approx(8000.0) and h["frac"] == pytest.approx(1.0)
    m = bench.mfma_roof(2.5e12, 1000.0, "k", [])  # 2.5 T ops in 1 ms: 2.5 POP/s
    assert m["bound"] == "mfma" and m["peak"] == 5000.0
    assert m["achieved"] == pytest.approx(2500.0) and m["frac"] == pytest.approx(0.5)


class _Runner:
    def __init__(self, M):
        self.M, self.copies, self.lins = M, 2, [object()] * 3

    def bytes_step(self):
        return 4_000_000_000

    def ops_step(self):
        return 1_000_000_000_000


def test_step_record_units(bench):
    r = bench.step_record(_Runner(4), 1.0, 1.1, "hbm")  # 4 GB per 1 ms step
    assert r["unit"] == "GB/s" and r["value"] == pytest.approx(4000.0)
    assert r["frac_of_hbm_peak"] == pytest.approx(0.5)
    assert r["us_per_step"] == pytest.approx(1000.0) and r["us_per_token"] == pytest.approx(250.0)
    assert r["linears_per_step"] == 3 and r["weight_copies_rotated"] == 2
    t = bench.step_record(_Runner(512), 0.5, 0.5, "tops")  # 1 T ops per 0.5 ms
    assert t["unit"] == "TOPS" and t["value"] == pytest.approx(2000.0)
    assert t["frac_of_int8_peak"] == pytest.approx(0.4)


def test_weight_copies_stream_past_the_infinity_cache(bench):
    for nbytes in (4_423_680, 8_918_024, 521_011_200, 1_620_000_000):
        c = bench.weight_copies(nbytes)
        assert 2 <= c <= 64
        # the sets together exceed twice the 256 MB cache, unless capped at 64
        assert c == 64 or c * nbytes >= 2 * bench.MALL_BYTES


def test_host_description(bench):
    model, affinity, threads = bench.host_description()
    assert affinity == len(os.sched_getaffinity(0))
    assert 1 <= threads <= affinity


def test_counter_records_keyed_to_sources(bench):
    # A record counts only for the kernel source it was taken on: the lookup
    # returns its bytes for the recorded hash and nothing for any other.
    data = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert data
    for key, ent in data.items():
        # calibrated HBM bytes: 2 x FETCH_SIZE + 1 x WRITE_SIZE, in KiB
        calibrated = 1024 * (ent["fetch_factor"] * ent["fetch_kib"] +
                             ent["write_factor"] * ent["write_kib"])
        assert abs(ent["hbm_bytes_per_launch"] - calibrated) <= 2048, key
        assert bench.traffic_from_profile(ent["source_sha1"], key) == ent["hbm_bytes_per_launch"]
        assert bench.traffic_from_profile("0" * 40, key) is None
    assert bench.traffic_from_profile(next(iter(data.values()))["source_sha1"],
                                      "no_such_kernel") is None


def test_source_hash_ignores_comments_only(bench, tmp_path, monkeypatch):
    csrc = tmp_path / "w1_a8_matmul_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text("int f() { return 1; }  // one\n/* block */\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.source_hash(["a.hip"])
    (csrc / "a.hip").write_text("// another comment\nint f() {\n  return 1;\n}\n")
    assert bench.source_hash(["a.hip"]) == h1
    (csrc / "a.hip").write_text("int f() { return 2; }\n")
    assert bench.source_hash(["a.hip"]) != h1
