"""Host-side pieces of bench.py (CPU only): byte counts, sweep resume and sharding, the one-GPU
guard."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_dense_algorithmic_bytes():
    # W once, X once, R read, Y written (bf16): 51 380 224 + 35 840 M at N = 7168, K = 3584
    for M in (1, 4, 16, 256):
        assert bench.algorithmic_bytes(M) == 51380224 + 35840 * M


def test_kbit_algorithmic_bytes():
    # k plane words and one scale byte per 32 weights, the codebook, X, R, Y
    assert bench.kbit_algorithmic_bytes(1, 7168, 3584, 4) == 7168 * 112 * 17 + 64 + 2 * 3584 + 4 * 7168
    assert bench.kbit_algorithmic_bytes(2, 64, 64, 2) == 64 * 2 * 9 + 16 + 2 * 2 * 64 + 4 * 2 * 64


def test_kda_algorithmic_bytes():
    B, T, H, HV, K, V = 2, 4, 1, 1, 128, 16
    dim = 2 * H * K + HV * V
    base = B * T * dim * 2 + B * 3 * dim * 2 + dim * 5 * 2 + B * T * 3 * dim * 2 \
        + B * T * HV * K * 2 + B * T * HV * 2 + HV * K * 4 + HV * 4 + B * T * HV * V * 2
    state = B * HV * V * K * 4
    assert bench.kda_algorithmic_bytes(B, T, H, HV, K, V, False) == base + state * (1 + T)
    ring = B * HV * T * V * 2 + B * H * T * K * 2 + B * HV * T * K * 4 + B * HV * T * 4
    assert bench.kda_algorithmic_bytes(B, T, H, HV, K, V, True) == base + state + ring


def test_done_rows_skips_valid_rows_only(tmp_path):
    f = tmp_path / "rows.jsonl"
    rows = [{"m": 4, "n": 7168, "k": 3584, "config": {"path": 0, "block_size": 448}},
            {"m": 8, "n": 7168, "k": 3584, "config": {"path": 1}, "valid": False}]
    f.write_text("\n".join(json.dumps(r) for r in rows) + "\nnot json\n")
    done = bench.done_rows(str(f))
    assert done == {(4, 7168, 3584, json.dumps({"block_size": 448, "path": 0}, sort_keys=True))}
    assert bench.done_rows(str(tmp_path / "missing.jsonl")) == set()


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2 and "one GPU only" in p.stderr


def test_traffic_lookup_is_keyed_by_kernel_code():
    """A measured byte count applies only to the kernel instance and machine code it was taken
    on: the committed M = 4 entry resolves for its kernel and hash, and reads None for another
    hash (a rebuilt kernel), another kernel, or another shape."""
    entries = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))["entries"]
    e = [x for x in entries if x["M"] == 4][0]

    class FakeLib:
        def __init__(self, name, code):
            self.k = {"name": name, "code_sha256": code}

        def config_kernel(self, cfg):
            return self.k
    t = bench.lookup_traffic(FakeLib(e["kernel_mangled"], e["code_sha256"]), {}, 4)
    assert t["bytes"] == e["traffic_bytes"] == e["fetch_bytes"] + e["write_bytes"]
    assert bench.lookup_traffic(FakeLib(e["kernel"], e["code_sha256"]), {}, 4)["bytes"] == e["traffic_bytes"]
    assert bench.lookup_traffic(FakeLib(e["kernel_mangled"], "0" * 64), {}, 4) is None
    assert bench.lookup_traffic(FakeLib("other", e["code_sha256"]), {}, 4) is None
    assert bench.lookup_traffic(FakeLib(e["kernel_mangled"], e["code_sha256"]), {}, 5) is None


def test_config_shards_cover_the_candidates_once():
    import types
    cands = [{"i": i} for i in range(23)]
    for n in (1, 2, 3, 7):
        parts = [bench.config_shard(types.SimpleNamespace(config_shard=i, num_config_shards=n), cands)
                 for i in range(n)]
        seen = sorted(c["i"] for p in parts for c in p)
        assert seen == list(range(23))
        assert max(map(len, parts)) - min(map(len, parts)) <= 1


def test_bad_config_shard_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--mode", "sweep", "--config-shard", "2",
                        "--num-config-shards", "2"], capture_output=True, text=True, timeout=120)
    assert p.returncode == 2 and "--config-shard" in p.stderr


def test_bad_kda_layout_is_refused():
    p = subprocess.run([sys.executable, "-c", "import sys, types; sys.argv = ['bench.py']; import bench; "
                        "bench.run_kda(types.SimpleNamespace(ms='1', layouts='ring,bogus', out=None), None)"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert p.returncode != 0 and "--layouts" in p.stderr
