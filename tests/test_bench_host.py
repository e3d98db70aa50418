"""Host logic of bench.py, on the CPU: the one-GPU guard, the rule that HBM
traffic is read only from a counter summary taken on the current kernel
source, the stored size of a row from its C value, and the decode kernel
each workload reports (whose committed counter summaries must exist)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()
    r = run_bench([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_only_from_a_summary_of_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    current = bench.kernel_source_hash()
    assert len(current) == 16

    def write(name, text):
        (tmp_path / name).write_text(text)

    write("decode_rows_kernel_a_pmc.txt",
          f"header\nkernel_source_sha256_16: {current}\ntraffic_bytes_per_launch: 123456789\n")
    write("decode_rows_kernel_b_pmc.txt",
          "kernel_source_sha256_16: 0000000000000000\ntraffic_bytes_per_launch: 5\n")
    write("decode_rows_kernel_c_pmc.txt", f"kernel_source_sha256_16: {current}\n")
    assert bench.traffic_from_profiles("decode_rows_kernel", "a") == 123456789.0
    assert bench.traffic_from_profiles("decode_rows_kernel", "b") is None   # other source
    assert bench.traffic_from_profiles("decode_rows_kernel", "c") is None   # no figure
    assert bench.traffic_from_profiles("decode_rows_kernel", "d") is None   # no file


def test_stored_bytes_per_row():
    # rows of 1024 bytes (256 words, 8192 raw bits): a compressed row keeps
    # its whole stream words, a row with C >= 8192 is stored raw
    c = np.array([256, 257, 288, 289, 8191, 8192, 9000], dtype=np.uint32)
    got = bench.stored_bytes_per_row(c, 1024)
    assert got.tolist() == [32, 36, 36, 40, 1024, 1024, 1024]


def test_decode_kernel_names_and_committed_profiles():
    name = bench.decode_kernel_name
    cases = {  # (kernel, workload) as the benchmark reports them
        ("decode_batch_kernel", "llm_weights"): name(8192, batched=True, invariant_bits=8),
        ("decode_rows_kernel", "sparse_gnn"): name(2048, invariant_bits=32),
        ("decode_pipe_kernel", "dense_gnn"): name(1024, invariant_bits=5),
        ("decode_pipe_kernel", "dlrm_emb"): name(512, invariant_bits=4),
        ("decode_rows_kernel", "llm_kv"): name(4096, invariant_bits=10),
        ("decode_pos_pipe_kernel", "llm_kv"): name(4096, positional=True),
        ("decode_pos_pipe_kernel", "sparse_gnn"): name(2048, positional=True),
    }
    for (kernel, workload), got in cases.items():
        assert got == kernel, (workload, got)
        path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
        assert os.path.exists(path), path
    assert name(8192, host_image=True, invariant_bits=8) == "decode_segments_kernel"
    assert name(1024, width=64) == "decode_pipe64_kernel"
    assert name(8192, width=16, batched=True) == "decode_wide_batch_kernel"
