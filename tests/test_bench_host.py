"""Host logic of bench.py (no GPU): the algorithmic byte accounting of a
decode step, the refusal of more than one GPU, and the code digest that keys
the stored traffic counters."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_step_bytes_at_batch_8_by_64k():
    """Per sequence at L = 65,536, D = 512, Di = 128, H = 64, K = 2048, each
    term worked out by hand:
      index_topk     65,408 candidates x 128 key bytes = 8,372,224
                     + 128 (query) + 4 x 2048 (indices) = 8,380,544
                     + 4 x 1022 page-table entries + 4 (count) = 8,384,636
      sparse_decode  2048 rows x (288 + 4) = 598,016, + 128 x 512 x 2 (window)
                     = 131,072, + 64 x 512 x 2 (queries) = 65,536, + 64 x 512 x 4
                     (output) = 131,072: 925,696; + 4 x 64 (LSE) + 4 (count)
                     = 925,956
      append         in 2 x 512 + 128 + 8 = 1,160, out 288 + 2 x 512 + 128 = 1,440
    """
    nb = bench.algorithmic_bytes(1, 65536, 64, 512, 128, 2048)
    assert nb == {"append": 2600, "index_topk": 8_384_636, "sparse_decode": 925_956}
    nb8 = bench.algorithmic_bytes(8, 65536, 64, 512, 128, 2048)
    assert sum(nb8.values()) == 74_505_536 == 8 * (2600 + 8_384_636 + 925_956)


def test_step_bytes_short_and_window_only_contexts():
    # L <= 128: no candidates, only the query of the indexer and the K slots
    nb = bench.algorithmic_bytes(1, 100, 16, 128, 64, 256)
    assert nb["index_topk"] == 64 + 4 * 256 + 4
    # D = 128: 72-byte rows
    assert nb["sparse_decode"] == 256 * 76 + 128 * 128 * 2 + 16 * 128 * 6 + 4 * 16 + 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_code_digest_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* fast */ }\n"
    b = "int f(int x) { return 2 * x; }"
    c = "int f(int x) { return 3 * x; }"
    assert bench._code_tokens(a) == bench._code_tokens(b) != bench._code_tokens(c)
    assert len(bench.source_digest()) == 16
