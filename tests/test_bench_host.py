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
    # per-token compression: the new token (bf16) and the block's pooling
    # state (d + 2 floats) in, the window entry and the finished block out
    assert a["hca_compress_kv"] == 4 * (512 * 2 + 514 * 4) + 2 * 4 * 580
    assert a["csa_compress_kv"] == 4 * (512 * 2 + 514 * 4 + 64 * 2 + 66 * 4) + 2 * 4 * 580 + 4 * 34
    assert round(sum(a.values()) / 1e6, 2) == 176.82


def test_traffic_sources_exist_and_hash():
    for f in bench.TRAFFIC_SRC:
        assert os.path.isfile(os.path.join(ROOT, f)), f
    h = bench.src_hash()
    assert len(h) == 16 and all(c in "0123456789abcdef" for c in h)


def test_prefill_trace_summary(tmp_path, capsys):
    """The prefill-section summary groups a kernel trace by call: the
    indexer's k_idxp_* launches summed per call, the two attention calls told
    apart by order (CSA launches first, then HCA), the projection's launches."""
    import sqlite3
    db = tmp_path / "run" / "trace_results.db"
    db.parent.mkdir()
    c = sqlite3.connect(db)
    c.execute("create table kernels (name text, start integer, end integer)")
    t = [0]

    def k(name, us):
        c.execute("insert into kernels values (?, ?, ?)", (name, t[0], t[0] + int(us * 1000)))
        t[0] += int(us * 1000) + 500

    for _ in range(3):                                 # decode steps before the section are ignored
        k("csa::k_idxd_filter(csa::IndexerArgs)", 2.5)
        k("csa::k_idxd_select(csa::IndexerArgs)", 5.0)
        k("void csa::k_attn_mfma<512, 64, true, unsigned short>(csa::AttnArgs)", 20.0)
    k("void at::native::fill(float)", 5.0)             # framework kernels are ignored
    for i in range(4):
        k("csa::k_idxp_thresh(csa::IndexerArgs, int, int)", 100.0 + i)
        k("csa::k_idxp_filter(csa::IndexerArgs)", 2000.0 + i)
        k("csa::k_idxp_select(csa::IndexerArgs)", 400.0 + i)
        k("csa::k_idxp_exact(csa::IndexerArgs)", 7.0)
    for us in (3000.0, 3010.0, 3020.0, 3030.0, 17600.0, 17610.0, 17620.0, 17630.0):
        k("void csa::k_attn_mfma<512, 64, true, unsigned short>(csa::AttnArgs)", us)
    for _ in range(4):
        k("void csa::k_proj_mfma<unsigned short>(csa::ProjArgs)", 550.0)
    # the decode workloads measured after the section are ignored
    k("void csa::k_compress<unsigned short>(csa::CompressArgs)", 30.0)
    k("void csa::k_attn_mfma<512, 64, true, unsigned short>(csa::AttnArgs)", 40.0)
    k("void csa::k_proj_mfma<unsigned short>(csa::ProjArgs)", 50.0)
    c.commit()
    c.close()
    bench.summarize_prefill(str(tmp_path))
    out = capsys.readouterr().out
    rows = {ln.split("|")[1].strip(): [x.strip() for x in ln.split("|")[2:5]] for ln in out.splitlines()
            if ln.startswith("| ") and not ln.startswith("| kernel") and not ln.startswith("| call")}
    assert rows["k_idxp_filter"] == ["4", "2001.5", "2000.0"]
    assert rows["csa_indexer_topk (k_idxp_*)"] == ["4", "2511.5", "2507.0"]   # 2507 + 3 i per launch
    assert rows["csa_sparse_mqa_attn"] == ["4", "3015.0", "3000.0"]
    assert rows["hca_dense_mqa_attn"] == ["4", "17615.0", "17600.0"]
    assert rows["attn_out_proj_grouped"] == ["4", "550.0", "550.0"]


def test_launch_summary_by_grid(tmp_path, capsys):
    """The per-launch summary keeps launches of one kernel over different grid
    sizes apart, takes durations from the trace run only and joins the
    counter run's values on the dispatch id (summed over instances; the
    largest instance for GRBM_GUI_ACTIVE)."""
    import sqlite3
    cols = "name text, grid_x integer, grid_y integer, grid_z integer, workgroup_x integer, dispatch_id integer, " \
           "start integer, end integer"

    def mk(sub, pmc):
        db = tmp_path / sub / "run_results.db"
        db.parent.mkdir()
        c = sqlite3.connect(db)
        c.execute(f"create table kernels ({cols})")
        c.execute("create table pmc_events (counter_name text, counter_value real, dispatch_id integer)")
        did = 0
        for rep in range(3):
            for gx, us in ((448 * 256, 55.0 + rep), (112 * 256, 12.0)):
                did += 1
                c.execute("insert into kernels values (?,?,?,?,?,?,?,?)",
                          ("void csa::k_lin8_stream<1, 4>(csa::LinArgs)", gx, 1, 1, 256, did, 0, int(us * 1000)))
                if pmc:
                    for inst in range(2):      # two instances of each counter
                        c.execute("insert into pmc_events values (?,?,?)", ("FETCH_SIZE", gx / 256 + inst, did))
                        c.execute("insert into pmc_events values (?,?,?)", ("GRBM_GUI_ACTIVE", 100.0 * (inst + 1), did))
            did += 1
            c.execute("insert into kernels values (?,?,?,?,?,?,?,?)", ("at::native::fill", 64, 1, 1, 64, did, 0, 5000))
        c.commit()
        c.close()
        return str(db.parent)

    bench.summarize_launches([mk("trace", False), mk("pmc", True)])
    out = capsys.readouterr().out.splitlines()
    assert out[0].split("|")[6:8] == [" FETCH_SIZE ", " GRBM_GUI_ACTIVE "]
    rows = {ln.split("|")[2].strip(): [x.strip() for x in ln.split("|")[3:8]] for ln in out[2:]}
    assert len(rows) == 2                                  # framework kernels are left out
    assert rows["448x1x1 wg of 256"] == ["3", "56.00", "55.00", "897", "200"]
    assert rows["112x1x1 wg of 256"] == ["3", "12.00", "12.00", "225", "200"]


def test_pmc_dispatch_summary(tmp_path, capsys):
    """Per-dispatch counter sums of one kernel, in dispatch order, one column
    per counter run (instances of a dispatch summed, other kernels ignored)."""
    import sqlite3
    for sub, cn, base in (("f", "FETCH_SIZE", 100.0), ("w", "WRITE_SIZE", 10.0)):
        (tmp_path / sub).mkdir()
        c = sqlite3.connect(tmp_path / sub / "run_results.db")
        c.execute("create table pmc_events (name text, counter_name text, counter_value real, dispatch_id integer)")
        for did in (3, 1, 2):
            for _ in range(2):
                c.execute("insert into pmc_events values (?, ?, ?, ?)",
                          ("void csa::k_attn_mfma<512, 64, true, unsigned short, 2, false>(csa::AttnArgs)", cn,
                           base * did, did))
            c.execute("insert into pmc_events values (?, ?, ?, ?)", ("csa::k_idxp_filter(csa::IndexerArgs)", cn, 1.0, 9))
        c.commit()
        c.close()
    bench.summarize_pmc_dispatches([str(tmp_path / "f"), str(tmp_path / "w")])
    rows = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("| ") and not ln.startswith("| launch")]
    assert rows == ["| 0 | 200.0 | 20.0 |", "| 1 | 400.0 | 40.0 |", "| 2 | 600.0 | 60.0 |"]
