"""Host-side logic of the benchmark (no GPU): the single-GPU refusal, the
algorithmic-byte accounting behind the roofline figure, and the source files
that key the stored traffic counts."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_layer_pair():
    """Per-call bytes from the shapes: 1M context, batch 4, 64 heads x 512,
    580-byte FP8 records (448 E4M3 codes + 64 bf16 RoPE dims + f32 scale),
    FP4 indexer rows of 32 code bytes + 2 scale bytes, top-1024, window 128,
    projection 32768 -> 7168 in 8 groups of bf16 weights."""
    a = bench.algorithmic_bytes()
    assert bench.REC_ALGO == 448 + 2 * 64 + 4
    n_csa, n_hca = (1 << 20) // 4, (1 << 20) // 128
    # the indexer reads every key row once: 4 x 262,144 x 34 bytes (+ queries, weights, the output)
    assert a["csa_indexer_topk"] == 4 * n_csa * 34 + 4 * 4 * (32 + 2 + 4) + 4 * 1024 * 4
    # HCA attention: every compressed record of each sequence once, plus window, q, o
    assert a["hca_dense_mqa_attn"] == 2 * 4 * 64 * 512 * 2 + 4 * n_hca * 580 + 4 * 128 * 580
    # the projection streams its weights once: 8 x 896 x 4096 bf16
    assert a["csa_out_proj"] == 8 * 896 * 4096 * 2 + 4 * 32768 * 2 + 4 * 7168 * 2
    assert round(sum(a.values()) / 1e6, 2) == 177.35


def test_traffic_sources_exist_and_hash():
    for f in bench.TRAFFIC_SRC:
        assert os.path.isfile(os.path.join(ROOT, f)), f
    h = bench.src_hash()
    assert len(h) == 16 and all(c in "0123456789abcdef" for c in h)
