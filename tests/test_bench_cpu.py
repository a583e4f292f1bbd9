"""bench.py host-side behaviour (no GPU needed)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_only_for_matching_kernel_source(monkeypatch):
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.recorded_traffic("b256_h48_pool512_null32") is None


def test_traffic_record_parses():
    text = open(bench.TRAFFIC_FILE).read()
    assert "traffic_bytes_per_launch:" in text
    assert "kernel_source_sha256_16:" in text


def test_kernel_hash_covers_only_the_single_token_kernel():
    """Host code after the kernel does not change the hash; a change inside
    the kernel's region does."""
    import bench
    text = open(bench.KERNEL_SRC, encoding="utf-8").read()
    h = bench.kernel_hash(text)
    assert bench.kernel_hash(text + "\n// host-side addition\n") == h
    i = text.index("namespace {") + len("namespace {")
    assert bench.kernel_hash(text[:i] + "\n// edit\n" + text[i:]) != h


def test_recorded_traffic_matches_this_kernel():
    import bench
    t = bench.recorded_traffic("b256_h48_pool512_null32")
    assert t is not None and abs(t / 1478831616 - 1) < 0.01
    assert bench.recorded_traffic("b64_h24_pool128") is None


def test_cpu_baseline_reports_threads_model_and_single_thread_rate():
    """The oracle baseline object carries the fields the bench line states:
    the median rate of three runs, unit, the threads used (every CPU the
    process may run on, capped only by OMP_NUM_THREADS), the host facts,
    kind, the sample, and a one-thread rate."""
    from linear_attention_decode_02_amd import synth

    w = synth.small("cpu_fields", batch=3, heads=12, num_slots=6, seed=1,
                    null_every=3)
    inp = synth.make_inputs(w)
    units = w.units(inp["state_idx"])
    r = bench.cpu_baseline(w, inp, 0.3, 1000, units)
    assert r["kind"] == "oracle" and r["unit"] == "updates/s"
    runs = r["runs_updates_per_s"]
    assert len(runs) == 3 and r["value"] == runs[1] > 0
    host = r["host"]
    allowed = len(os.sched_getaffinity(0))
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    assert r["cores"] == (min(allowed, omp) if omp else allowed)
    assert host["nproc"] == os.cpu_count()
    assert host["affinity_cpus"] == allowed and host["model"]
    assert f"({units} updates)" in r["sample"]
    st = r["single_thread"]
    assert st["value"] > 0 and st["calls"] >= 1


def test_cpu_threads_follow_omp_num_threads(monkeypatch):
    allowed = len(os.sched_getaffinity(0))
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.cpu_threads()[0] == 1
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.cpu_threads()[0] == allowed
