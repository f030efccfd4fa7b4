"""Host-side checks of bench.py: the one-GPU contract, the algorithmic work
counts the roofline divides by, and the source hash that decides whether the
stored HBM-traffic figure still describes the attention kernel.  No GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402  (standard library only at import time)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_work_counts_dsv3_decode():
    # 64 rows of 4096 cached tokens, 128 heads, bf16.  Each (row, head, token)
    # costs 2 * 576 FLOP for the score and 2 * 512 for the weighted sum; the
    # bytes are every 1152-byte cache row once plus, per (row, head), the
    # 1152-byte query read, the 1024-byte output and the 4-byte lse written.
    flop, nbytes = bench.work_counts(64, 128, [4096] * 64)["decode"]
    assert flop == 2176 * 64 * 128 * 4096 == 73014444032
    assert nbytes == 64 * 4096 * 1152 + 64 * 128 * (1152 + 1024 + 4) == 319848448


def test_work_counts_causal_query_tokens():
    # two new tokens at the end of a row of 10 cached rows: the first sees 9
    # rows, the second all 10
    assert bench.work_counts(1, 1, [10], q_len=2)["decode"][0] == 2176 * (9 + 10)
    # a row shorter than the query tokens: only the last token sees anything
    assert bench.work_counts(1, 1, [1], q_len=3)["decode"][0] == 2176 * 1
    # the cache is still read once per row, whatever the number of query tokens
    assert (bench.work_counts(1, 1, [10], q_len=2)["decode"][1]
            == 10 * 1152 + 2 * (1152 + 1024 + 4))


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    plain = tmp_path / "plain.hip"
    commented = tmp_path / "commented.hip"
    changed = tmp_path / "changed.hip"
    plain.write_text("int f() { return 1; }\n")
    commented.write_text("// a note\n\nint f() { return 1; }  // trailing note\n")
    changed.write_text("int f() { return 2; }\n")
    hashes = []
    for path in (plain, commented, changed):
        monkeypatch.setattr(bench, "KERNEL_SRCS", [str(path)])
        hashes.append(bench.kernel_source_hash())
    assert hashes[0] == hashes[1] != hashes[2]


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_profile_summary_per_workload(tmp_path):
    """Five fake rocprofv3 output directories for the few-heads workload: the
    summary lands under its own name, its traffic entry sits beside the other
    workloads' entries, and the bench's lookup finds it only for the kernel
    it was taken from."""
    kern = "void mla355::(anonymous namespace)::decode_bf16_kernel<16, 1, 2, 32, 2, false>(mla355::DecodeParams)"
    copy = "void at::native::copy_kernel"
    d = {k: tmp_path / k for k in ("trace", "fetch", "write", "cfetch", "cwrite")}
    _write_csv(str(d["trace"] / "x" / "trace_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [[kern, 13, 2.8e6, 219000.0, 80.0, 210000.0, 230000.0]])
    # two dispatches, each counted over two hardware instances
    cnt = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(str(d["fetch"] / "x" / "fetch_counter_collection.csv"), cnt,
               [[1, kern, "FETCH_SIZE", 50000.0], [1, kern, "FETCH_SIZE", 50000.0],
                [2, kern, "FETCH_SIZE", 60000.0], [2, kern, "FETCH_SIZE", 40000.0]])
    _write_csv(str(d["write"] / "x" / "write_counter_collection.csv"), cnt,
               [[1, kern, "WRITE_SIZE", 1000.0], [2, kern, "WRITE_SIZE", 1000.0]])
    _write_csv(str(d["cfetch"] / "x" / "cfetch_counter_collection.csv"), cnt,
               [[7, copy, "FETCH_SIZE", 131072.0]])
    _write_csv(str(d["cwrite"] / "x" / "cwrite_counter_collection.csv"), cnt,
               [[7, copy, "WRITE_SIZE", 262144.0]])
    out = tmp_path / "profiles"
    out.mkdir()
    # an entry of another workload already there is kept
    (out / "decode_traffic.json").write_text('{"other_workload": {"kernel": "k"}}\n')
    bench.summarize_profiles([str(d[k]) for k in ("trace", "fetch", "write", "cfetch", "cwrite")],
                             cid=3, out_dir=str(out))
    md = (out / "decode_bf16_kernel_few_heads_b128_h16_T8192.md").read_text()
    assert "--config 3" in md and "219.0" in md
    import json
    table = json.loads((out / "decode_traffic.json").read_text())
    assert set(table) == {"other_workload", "few_heads_b128_h16_T8192"}
    e = table["few_heads_b128_h16_T8192"]
    # FETCH_SIZE: 100000 KiB per dispatch x (256 MiB / 131072 KiB) = 2; WRITE_SIZE x 1
    assert e["hbm_bytes_per_launch"] == (100000 * 2 + 1000) * 1024
    name = "decode_bf16_kernel<16, 1, 2, 32, 2, false>"
    assert e["kernel"] == name
    path = str(out / "decode_traffic.json")
    assert bench.load_traffic("few_heads_b128_h16_T8192", name, path) == e["hbm_bytes_per_launch"]
    assert bench.load_traffic("few_heads_b128_h16_T8192", "decode_wide_kernel<4, 2, false>", path) is None
    assert bench.load_traffic("dsv3_decode_b64_h128_T4096", name, path) is None
