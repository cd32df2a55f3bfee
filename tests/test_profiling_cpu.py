"""Host logic of the rocprofv3 helpers: counter scaling, traffic records and their invalidation."""
import csv
import os

from scaled_dot_product_tiled_amd import profiling


def _counter_csv(d, rows):
    os.makedirs(os.path.join(d, "host", "vm"), exist_ok=True)
    with open(os.path.join(d, "host", "vm", "1_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_record_scales_by_copy_and_tracks_source(tmp_path, monkeypatch):
    monkeypatch.setattr(profiling, "ROOT", str(tmp_path))
    src = tmp_path / "kern.hip"
    src.write_text("kernel v1\n")
    mib = 4
    # the copy moved 4 MiB: FETCH_SIZE read 2048 units (2 KiB each), WRITE_SIZE 4096 (1 KiB each)
    _counter_csv(tmp_path / "cf", [("copy", "FETCH_SIZE", 2048.0), ("fill", "FETCH_SIZE", 3.0)])
    _counter_csv(tmp_path / "cw", [("copy", "WRITE_SIZE", 4096.0), ("fill", "WRITE_SIZE", 4096.0)])
    _counter_csv(tmp_path / "f", [("void k<1>(A)", "FETCH_SIZE", 100.0), ("void k<1>(A)", "FETCH_SIZE", 300.0),
                                  ("void other(A)", "FETCH_SIZE", 7.0)])
    _counter_csv(tmp_path / "w", [("void k<1>(A)", "WRITE_SIZE", 10.0)])
    rec = profiling.traffic_record("k<1>", str(src), str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
                                   str(tmp_path / "cw"), mib)
    summary = tmp_path / "summary.txt"
    summary.write_text("text\n" + rec + "\n")
    got = profiling.read_traffic(str(summary), "k<1>")
    assert got == {"fetch_bytes": 200.0 * 2048, "write_bytes": 10.0 * 1024, "bytes": 200.0 * 2048 + 10.0 * 1024}
    assert profiling.read_traffic(str(summary), "other") is None        # no record for it
    src.write_text("kernel v2\n")                                       # the kernel changed: stale
    assert profiling.read_traffic(str(summary), "k<1>") is None
    assert profiling.read_traffic(str(tmp_path / "missing.txt"), "k<1>") is None


def test_committed_records_parse():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pdir = os.path.join(root, "profiles")
    for fn in os.listdir(pdir):
        for line in open(os.path.join(pdir, fn)):
            if line.startswith("record:"):
                kv = dict(t.split("=", 1) for t in line[len("record:"):].split())
                assert os.path.exists(os.path.join(root, kv["source"])), fn
                assert float(kv["fetch_scale"]) > 0 and float(kv["write_scale"]) > 0


def test_sq_table_derives_busy_fraction_and_lds_rate(tmp_path, monkeypatch):
    """One kernel active 1000 clocks on each of the 8 XCDs (GRBM_GUI_ACTIVE summed to 8000): MFMA
    busy 512000 SIMD-cycles of 1024 SIMDs is 50%; 4000 64-byte LDS units over 256 CUs x 1000 clocks
    is 1 byte per clock per CU; conflicts 10 of 200 active LDS cycles is 5%.  Kernels that are not
    the library's (here "other") are left out."""
    vals = {"GRBM_GUI_ACTIVE": 8000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 512000.0, "SQ_INSTS_LDS_LOAD_BANDWIDTH": 4000.0,
            "SQ_LDS_BANK_CONFLICT": 10.0, "SQ_LDS_IDX_ACTIVE": 200.0, "SQ_LDS_DATA_FIFO_FULL": 0.0,
            "SQ_BUSY_CU_CYCLES": 256000.0, "SQ_WAIT_INST_LDS": 2560.0, "SQ_LDS_ADDR_CONFLICT": 0.0}
    rows = [("void attn::fwd_kernel<1, 2>(A)", c, v) for c, v in vals.items()] + [("void other(A)", c, 1.0)
                                                                                  for c in vals]
    _counter_csv(tmp_path / "sq", rows)
    table = profiling.sq_table(str(tmp_path / "sq")).splitlines()
    assert len(table) == 2
    f = table[1].split()
    assert f[0] == "fwd_kernel<1,2>" and f[1] == "1000" and f[2] == "50.0%" and f[3] == "1.0" and f[4] == "5.00%"
    assert f[5] == "0.00%" and f[6] == "1.0%"   # 4 x 2560 wave-cycles of 4 x 1000 x 256
