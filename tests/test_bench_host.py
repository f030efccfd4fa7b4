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
