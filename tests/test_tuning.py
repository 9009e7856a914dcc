"""Host-side checks of the plan-table generator and of the tables compiled in."""
import json
import os
import subprocess
import sys

from fp8_block_scaled_grouped_amd.tuning import make_tables as mt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rec(M, N, K, rule_us, plans):
    return {"sweep": "dense", "layer": "x", "M": M, "N": N, "K": K, "default_us": 1e9,
            "rule": [16, 128, 1, rule_us], "plans": plans}


def test_dense_rows_margin_ranges_and_scratch_cap():
    recs = [
        _rec(1, 2048, 7168, 10.0, [[16, 128, 8, 9.0], [16, 256, 16, 9.5]]),  # 10% faster: kept
        _rec(16, 2048, 7168, 10.0, [[16, 128, 8, 9.9]]),  # within the margin: rule stays
        _rec(64, 2048, 7168, 20.0, [[32, 128, 4, 15.0]]),
        # a split whose partials exceed the static scratch is skipped for the next best
        _rec(256, 18432, 7168, 100.0, [[128, 256, 4, 50.0], [128, 256, 1, 80.0]]),
    ]
    rows = mt.dense_rows(recs)
    assert [(r[0], r[1], r[2], r[3], r[4], r[5], r[6]) for r in rows] == [
        (1, 1, 2048, 7168, 16, 128, 8), (17, 64, 2048, 7168, 32, 128, 4), (1, 256, 18432, 7168, 128, 256, 1)]


def test_kb_per_split_matches_the_library_rule():
    # 56 K blocks in 24 runs -> runs of 3 blocks, 19 of them; one run when K fits
    assert mt.kb_per_split(7168, 24) == (3, 19)
    assert mt.kb_per_split(7168, 1) == (56, 1)
    assert mt.kb_per_split(1040, 100) == (1, 9)


def test_block_m_rows_pick_fastest_and_merge():
    recs = []
    for T, times in [(1, {16: 1.0, 32: 1.1}), (8, {16: 1.0, 32: 1.2}), (256, {16: 3.0, 32: 2.0}),
                     (8192, {32: 9.0, 128: 8.0})]:
        for bm, ms in times.items():
            recs.append({"sweep": "block_m", "tokens": T, "block_m": bm, "ms": ms, "topk": 8, "experts": 256})
    rows = mt.block_m_rows(recs)
    assert [(r[0], r[1]) for r in rows] == [(8 * 8 / 256, 16), (256 * 8 / 256, 32), (8192 * 8 / 256, 128)]


def test_written_headers_parse_back(tmp_path):
    mt.write_dense([(1, 64, 2048, 7168, 16, 128, 8, 9.0, 10.0)], "t", str(tmp_path))
    mt.write_block_m([(2.0, 16, 1.0, {16: 1.0})], "t", str(tmp_path))
    d = (tmp_path / "dense_tuned.h").read_text()
    assert "{1, 64, 2048, 7168, 16, 128, 8}" in d
    b = (tmp_path / "block_m_tuned.h").read_text()
    assert "{2, 16}" in b


def test_committed_tables_are_the_generators_output(tmp_path):
    # the headers in csrc/ are what make_tables writes from the committed sweep records
    tdir = os.path.join(ROOT, "fp8_block_scaled_grouped_amd", "tuning")
    csrc = os.path.join(ROOT, "fp8_block_scaled_grouped_amd", "csrc")
    subprocess.check_call([sys.executable, "-m", "fp8_block_scaled_grouped_amd.tuning.make_tables", "--out-dir",
                           str(tmp_path)], cwd=ROOT)
    for name, sweep in (("dense_tuned.h", "dense_sweep.jsonl"), ("block_m_tuned.h", "block_m_sweep.jsonl")):
        if os.path.exists(os.path.join(tdir, sweep)):
            with open(os.path.join(csrc, name)) as f:
                assert (tmp_path / name).read_text() == f.read(), name


def test_library_plans_follow_the_dense_table():
    # where the table holds a tiling, the workspace the library asks for at both ends of
    # the entry's M range is that tiling's split-K partials; elsewhere the rule's
    from fp8_block_scaled_grouped_amd import moe355
    path = os.path.join(ROOT, "fp8_block_scaled_grouped_amd", "tuning", "dense_sweep.jsonl")
    if not os.path.exists(path):
        return
    rows = mt.dense_rows(mt.read(path, "dense"))
    assert rows
    for m0, m1, n, k, bm, bnb, sp, us, dus in rows:
        runs = 1 if bnb == 16 else mt.kb_per_split(k, sp)[1]
        for M in (m0, m1):
            want = runs * M * n * 4 + 256 if runs > 1 else 0
            assert moe355.gemm_fp8_blockscale_workspace(M, n, k) == want, (M, n, k, sp)


def test_rocprof_summary_roles_and_traffic_scaling(tmp_path):
    from fp8_block_scaled_grouped_amd.tuning import rocprof_summary as rs
    g1u1 = "void moe355::(anonymous namespace)::bs_gemm_kernel<moe355::(anonymous namespace)::Cfg<1, 128, 256, 8, 2, 3>, 1, false, false>(moe355::GemmArgs)"
    assert rs.role(g1u1) == ("g1u1", "g1u1 (BM 128, B rows 256, 8 waves, 3 stages)")
    assert rs.role("big_gemm_kernel<2, false>")[0] == "down"
    small = "void moe355::(anonymous namespace)::dense_small_kernel<1, false>(moe355::DenseSmallArgs)"
    assert rs.role(small) == ("dense", "dense small-M (1 row tiles, 8 waves, plain B)")
    assert rs.role("__amd_rocclr_copyBuffer")[0] == "copy"
    assert rs.role("at::native::elementwise_kernel<...>")[0] is None
    # counters: two g1u1 dispatches and three calibration copies; bytes = KiB * copy bytes / copy KiB
    for counter, kib, copy_kib in (("FETCH_SIZE", (100.0, 300.0), 512.0), ("WRITE_SIZE", (10.0, 30.0), 1024.0)):
        d = tmp_path / counter / "host" / "1"
        d.mkdir(parents=True)
        lines = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
        lines += ['%d,"%s",%s,%f' % (i, g1u1, counter, v) for i, v in enumerate(kib)]
        lines += ["%d,__amd_rocclr_copyBuffer,%s,%f" % (10 + i, counter, copy_kib) for i in range(3)]
        (d / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")
    out = tmp_path / "t.json"
    subprocess.check_call([sys.executable, "-m", "fp8_block_scaled_grouped_amd.tuning.rocprof_summary", "traffic",
                           "--fetch-dir", str(tmp_path / "FETCH_SIZE"), "--write-dir", str(tmp_path / "WRITE_SIZE"),
                           "--workload", "w", "--copy-bytes", str(1 << 20), "--command-fetch", "f",
                           "--command-write", "w", "--out", str(out)], cwd=ROOT)
    k = json.loads(out.read_text())["kernels"]["g1u1"]
    assert k["fetch_bytes"] == 200.0 * (1 << 20) / 512.0
    assert k["write_bytes"] == 20.0 * (1 << 20) / 1024.0
    assert k["dispatches"] == 2


def test_rocprof_summary_memory_counters(tmp_path):
    """The memory-side summary: latency = LEVEL / reads, in flight = LEVEL / (GUI / 8), stall
    shares over 128 L2 channels, averaged over a kernel's dispatches."""
    from fp8_block_scaled_grouped_amd.tuning import rocprof_summary as rs
    down = "void moe355::(anonymous namespace)::bs_gemm_kernel<moe355::(anonymous namespace)::Cfg<2, 128, 256, 8, 2, 3>, 2, false, false>(moe355::GemmArgs)"
    d = tmp_path / "mem" / "host"
    d.mkdir(parents=True)
    vals = {"TCC_EA0_RDREQ_sum": 1000.0, "TCC_EA0_RDREQ_LEVEL_sum": 500000.0, "GRBM_GUI_ACTIVE": 8 * 2000.0,
            "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum": 128 * 2000.0 * 0.25, "TCC_EA0_RDREQ_GMI_CREDIT_STALL_sum": 0.0}
    lines = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp"]
    for disp in (1, 2):
        lines += ['%d,"%s",%s,%f,0,1000' % (disp, down, k, v) for k, v in vals.items()]
    lines += ['3,"at::native::elementwise_kernel<...>",TCC_EA0_RDREQ_sum,5,0,10']
    (d / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")
    r = rs.mem_rows(str(tmp_path / "mem"))
    assert list(r) == ["down (BM 128, B rows 256, 8 waves, 3 stages)"]
    x = r["down (BM 128, B rows 256, 8 waves, 3 stages)"]
    assert x["calls"] == 2 and x["reads"] == 1000.0
    assert x["latency_cycles"] == 500.0 and x["in_flight"] == 250.0
    assert abs(x["dram_stall"] - 0.25) < 1e-12 and x["gmi_stall"] == 0.0
    assert abs(x["clock_ghz"] - 2.0) < 1e-12
