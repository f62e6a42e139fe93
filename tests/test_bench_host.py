"""Host logic of bench.py (CPU): the algorithmic work model behind the
roofline figures, pinned by hand counts and by the oracle's page rules; the
gate that reports measured traffic only for the sources it was measured on;
the longest-first deal of the CPU baseline; and the single-GPU refusal."""

import json
import os
import re
import shutil
import subprocess
import sys

import numpy as np
import pytest

import bench
from oracle import slots as oslots

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_bytes_by_hand():
    # one token, one head: q, k, v, o of 128 bf16 (4 x 256 B) + g, beta fp32 (8 B)
    assert bench.prefill_bytes(1, 1, 1, 0) == 1032
    # q and k are per q/k head, v, o, g and beta per v-head
    assert bench.prefill_bytes(10, 4, 2, 0) == 10 * (2 * 2 * 256 + 2 * 4 * 256 + 4 * 8)
    # each state row read or stored moves H fp32 [128, 128] states
    assert bench.prefill_bytes(0, 3, 3, 5) == 5 * 3 * 128 * 128 * 4


def test_decode_bytes_by_hand():
    # the state read and written (2 x 64 KiB per head) plus one token's q, k, v, o, g, beta
    assert bench.decode_bytes(1, 1, 1) == 2 * 65536 + 1032
    assert bench.decode_bytes(256, 32, 16) == 256 * (2 * 32 * 65536 + 2 * 16 * 256 + 2 * 32 * 256 + 32 * 8)


def test_prefill_flops_by_hand():
    # per token and head: three d x d products across chunks (6 d^2) and five
    # C x d products within the chunk (10 C d), C = 64, d = 128
    assert bench.prefill_flops(1, 1) == 6 * 128 * 128 + 10 * 64 * 128
    assert bench.prefill_flops(64, 32) == 64 * 32 * (6 * 128 * 128 + 10 * 64 * 128)


@pytest.mark.parametrize("seed", range(20))
def test_state_rows_follow_the_page_rules(seed):
    """The rows the byte model counts are the oracle's read and written pages
    of every sequence with new tokens, plus one more store where the final
    state lands on a page end (the last boundary page and the final page are
    then the same row, stored twice)."""
    rng = np.random.default_rng(seed)
    ps = int(rng.choice([64, 128, 896, 1024]))
    B = int(rng.integers(1, 12))
    prefix = [int(rng.choice([0, ps, 2 * ps, rng.integers(0, 5 * ps)])) for _ in range(B)]
    new = [int(rng.choice([0, 1, ps - 1, ps, rng.integers(0, 4 * ps)])) for _ in range(B)]
    expect = 0
    for p, L in zip(prefix, new):
        if p + L == 0:
            continue
        n = (p + L + ps - 1) // ps
        pages = list(range(100, 100 + n))
        reads, writes = oslots.touched_rows(pages, p + L - (n - 1) * ps, ps, new_len=L)
        if L > 0:  # a sequence without new tokens loads and stores nothing
            expect += len(reads) + len(writes) + ((p + L) % ps == 0)
    assert bench._state_rows_prefill(prefix, new, ps) == expect


def test_lpt_deal():
    assert bench._lpt([5.0], 4) == 5.0
    # the greedy deal, not the optimum (3 + 3 | 2 + 2 + 2 would take 6)
    assert bench._lpt([3.0, 3.0, 2.0, 2.0, 2.0], 2) == 7.0
    assert bench._lpt([1.0] * 8, 3) == 3.0
    xs = list(np.random.default_rng(3).uniform(0, 1, size=40))
    t = bench._lpt(xs, 5)
    assert max(xs) <= t <= sum(xs) / 5 + max(xs)


def _copy_sources(dst):
    src = os.path.join(ROOT, "paged_recurrent_state_amd", "csrc")
    os.makedirs(os.path.join(dst, "paged_recurrent_state_amd"))
    shutil.copytree(src, os.path.join(dst, "paged_recurrent_state_amd", "csrc"))
    return os.path.join(dst, "paged_recurrent_state_amd", "csrc")


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    d0 = bench.kernel_sources_digest()
    assert len(d0) == 16 and int(d0, 16) >= 0
    csrc = _copy_sources(str(tmp_path))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_sources_digest() == d0
    f = os.path.join(csrc, "gdn_prefill.hip")
    text = open(f).read()
    open(f, "w").write("// a new comment line\n/* and a block\n comment */\n" + text.replace("\n", "\n  ", 3))
    assert bench.kernel_sources_digest() == d0
    open(f, "w").write(text.replace("kChunk", "kChunk ", 1) + "\nconstexpr int kUnused = 1;\n")
    assert bench.kernel_sources_digest() != d0


def test_traffic_only_for_the_measured_sources(monkeypatch):
    text = open(bench.COUNTERS_MD).read()
    m = re.search(r"bench-traffic: sources=([0-9a-f]+) prefill_path_bytes=(\d+) decode_bytes=(\d+)", text)
    assert m, "the counters summary records its sources and byte counts"
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: m.group(1))
    t = bench.measured_traffic()
    assert t == {"prefill": int(m.group(2)), "decode": int(m.group(3))}
    monkeypatch.setattr(bench, "kernel_sources_digest", lambda: "0" * 16)
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "COUNTERS_MD", os.path.join(ROOT, "no", "such", "file.md"))
    assert bench.measured_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
