"""bench.py's command-line contract, checked without a GPU: it measures one GPU only and says so
for --gpus above 1, and the helpers behind its JSON line (token order, kernel hash) behave as its
numbers assume."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_token_order_skips_the_cold_start_and_wraps():
    import bench
    assert bench.token_ids(1, 5, 6) == [1, 2, 3, 4, 5]
    assert bench.token_ids(4, 5, 6) == [4, 5, 1, 2, 3]
    assert 0 not in bench.token_ids(1, 100, 7)


def test_kernel_hash_ignores_comments_but_not_code():
    import bench
    a = "int f(int x) { return x + 1; } // one\n/* two */"
    b = "int f(int x) {\n  return x + 1;  // changed comment\n}"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()


def test_stored_traffic_is_tied_to_kernel_and_workload():
    import json
    import bench
    rec = json.load(open(os.path.join(ROOT, "profiles", "k_sparse_ffn_llama7b_traffic.json")))
    traffic, note = bench.stored_traffic(37.6e6, rec["config"] + 1)
    assert traffic is None and "not this one" in note
    if rec["kernel_hash"] == bench.kernel_source_hash():
        traffic, _ = bench.stored_traffic(37.6e6, rec["config"])
        assert traffic == rec["traffic_bytes_per_launch"]
