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


def test_trace_summary_finds_each_step(tmp_path):
    """A hand-made kernel trace: two b8_64k steps back to back (the second
    with a 1 µs gap before its decode), an unrelated kernel between them, and
    a b128 decode; the summary reports the medians of each sequence."""
    hdr = ("Kind,Agent_Id,Queue_Id,Stream_Id,Thread_Id,Dispatch_Id,Kernel_Id,Kernel_Name,"
           "Correlation_Id,Start_Timestamp,End_Timestamp,Grid_Size_X,Grid_Size_Y,Grid_Size_Z")
    rows, t = [], 0

    def k(name, dur_ns, grid_y=1, gap_ns=0):
        nonlocal t
        t += gap_ns
        rows.append(f'K,1,1,0,1,{len(rows)},1,"void csa2::{name}(int)",1,{t},{t + dur_ns},1,{grid_y},1')
        t += dur_ns

    for gap in (0, 1000):
        k("append_score_kernel<512, 128, 16>", 13000, grid_y=9)
        k("select_filter_kernel<csa2::IntKeys>", 5000)
        k("select_final_kernel<4, csa2::IntKeys, false>", 6000)
        k("sparse_decode_kernel<512, 16, true>", 13000, gap_ns=gap)
        k("sparse_combine_kernel<512, 16, 1>", 5000)
        k("fill_zero_kernel", 2000)
    k("sparse_decode64_kernel<512>", 70000)
    k("sparse_combine_kernel<512, 64, 4>", 15000)
    path = tmp_path / "trace.csv"
    path.write_text(hdr + "\n" + "\n".join(rows) + "\n")
    out = bench.trace_summary(str(path))
    assert "b8_64k step: csa2_append_index_topk + csa2_sparse_decode: 2 runs" in out
    assert "| `sparse_decode_kernel<512, 16, true>` | 13.00 | 0.50 |" in out
    assert "| whole run | 42.50 | |" in out
    assert "b128_rag csa2_sparse_decode: 1 runs" in out
    assert "| whole run | 85.00 | |" in out
    assert "b1_1m step: csa2_append_index_topk + csa2_sparse_decode: 0 runs" in out
