"""Host-side logic of bench.py, without a GPU: rocprofv3 counter-CSV reduction, the copy
calibration of the byte counters, the kernel-source gate on committed traffic figures, the
MFMA-utilization reduction, and the refusal of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

import bench

HDR = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size",'
       '"Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count",'
       '"Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"')
GEMM = "void convrot::(anonymous namespace)::gemm_kernel<8, 1, true, 1>(unsigned char const*)"
RQ = "void convrot::(anonymous namespace)::rotate_quant_kernel<1, 8, 1>(void const*)"
COPY = "void at::native::elementwise_copy_kernel(int)"


def _counters(path, rows):
    """rows: (dispatch, grid, kernel, counter, value) -> a counter_collection.csv."""
    with open(path, "w") as fh:
        fh.write(HDR + "\n")
        for i, (d, g, k, c, v) in enumerate(rows):
            fh.write('%d,%d,"Agent 1",1,1,1,%d,1,"%s",256,0,0,0,0,0,"%s",%f,0,0\n' % (i, d, g, k, c, v))
    return str(path)


def test_counter_rows_of_one_dispatch_are_summed(tmp_path):
    # A counter reported per hardware instance arrives as several rows of one dispatch.
    p = _counters(tmp_path / "c.csv", [(7, 1024, GEMM, "FETCH_SIZE", 10.0), (7, 1024, GEMM, "FETCH_SIZE", 5.5),
                                       (8, 1024, GEMM, "FETCH_SIZE", 1.0)])
    got = bench._read_counter_csv(p)
    assert got[7][2]["FETCH_SIZE"] == 15.5 and got[8][2]["FETCH_SIZE"] == 1.0
    assert got[7][1] == 1024 and "gemm_kernel" in got[7][0]


def test_pmc_summary_scales_by_the_copy_and_takes_the_largest_launch(tmp_path):
    gib_kib = (1 << 30) / 1024.0
    # the copy reads 1 GiB and writes 1 GiB, but FETCH_SIZE reports half of it: scale 2
    cf = _counters(tmp_path / "cf.csv", [(1, 4096, COPY, "FETCH_SIZE", gib_kib / 2)])
    cw = _counters(tmp_path / "cw.csv", [(1, 4096, COPY, "WRITE_SIZE", gib_kib)])
    # two GEMM shapes (grids 1000 and 3000) and one rotate+quantize; medians over dispatches
    f = _counters(tmp_path / "f.csv", [(1, 3000, GEMM, "FETCH_SIZE", 100.0), (2, 3000, GEMM, "FETCH_SIZE", 300.0),
                                       (3, 3000, GEMM, "FETCH_SIZE", 200.0), (4, 1000, GEMM, "FETCH_SIZE", 9999.0),
                                       (5, 500, RQ, "FETCH_SIZE", 50.0)])
    w = _counters(tmp_path / "w.csv", [(1, 3000, GEMM, "WRITE_SIZE", 400.0), (4, 1000, GEMM, "WRITE_SIZE", 1.0),
                                       (5, 500, RQ, "WRITE_SIZE", 25.0)])
    out = tmp_path / "pmc.json"
    doc = bench.pmc_summary("wl", f, w, cf, cw, out_path=str(out))
    g = doc["workloads"]["wl"]["gemm"]
    assert g["grid_threads"] == 3000 and g["dispatches"] == 3
    assert g["fetch_bytes"] == round(200.0 * 1024 * 2) and g["write_bytes"] == round(400.0 * 1024)
    assert g["bytes"] == g["fetch_bytes"] + g["write_bytes"]
    r = doc["workloads"]["wl"]["rotate_quant"]
    assert r["fetch_bytes"] == round(50.0 * 1024 * 2) and r["write_bytes"] == round(25.0 * 1024)
    assert doc["kernel_source_hash"] == bench.kernel_source_hash()
    assert json.load(open(out)) == doc


def test_committed_traffic_is_used_only_for_the_same_kernel_sources(tmp_path, monkeypatch):
    entry = {"bytes": 123}
    p = tmp_path / "pmc.json"
    p.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(),
                             "workloads": {"wl": {"gemm": entry}}}))
    monkeypatch.setattr(bench, "PMC_FILE", str(p))
    assert bench.traffic_from_counters("wl", "gemm") == entry
    assert bench.traffic_from_counters("wl", "rotate_quant") is None
    p.write_text(json.dumps({"kernel_source_hash": "0" * 16, "workloads": {"wl": {"gemm": entry}}}))
    assert bench.traffic_from_counters("wl", "gemm") is None
    monkeypatch.setattr(bench, "PMC_FILE", str(tmp_path / "absent.json"))
    assert bench.traffic_from_counters("wl", "gemm") is None


def test_mfma_summary_reduces_busy_cycles_ops_and_clock(tmp_path):
    # one launch of 100 us: 2 GHz x 100 us = 200 000 active cycles per XCD (8 XCDs summed)
    c = _counters(tmp_path / "m.csv", [(1, 995328, GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 50000.0),
                                       (1, 995328, GEMM, "SQ_INSTS_VALU_MFMA_MOPS_I8", 1e9),
                                       (1, 995328, GEMM, "GRBM_GUI_ACTIVE", 8 * 200000.0),
                                       (1, 995328, GEMM, "MfmaUtil", 25.0)])
    t = tmp_path / "t.csv"
    t.write_text('"Dispatch_Id","Start_Timestamp","End_Timestamp"\n1,1000,101000\n')
    doc = bench.mfma_summary(c, str(t))
    assert doc["mfma_busy_cycles_per_simd_median"] == 50000.0
    assert doc["gui_active_cycles_per_xcd_median"] == 200000.0
    assert doc["implied_clock_GHz"] == 2.0
    assert doc["int8_mfma_ops_median"] == 512e9
    assert doc["duration_us_median"] == 100.0 and doc["MfmaUtil_pct_median"] == 25.0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_gemm_kernel_names_are_recognised():
    for name in (GEMM, "void convrot::(anonymous namespace)::gemm_xr_kernel<1, 16>(unsigned char const*)",
                 "void convrot::(anonymous namespace)::gemm_rw_kernel<1, 96, 0>(unsigned char const*)",
                 "void convrot::(anonymous namespace)::gemm_n2_kernel<8, 2, true>(unsigned char const*)",
                 "convrot::(anonymous namespace)::gemm_wide_kernel<4, 1>(unsigned char const*)",
                 "void convrot::(anonymous namespace)::gemm_fp6_kernel<1, 1>(unsigned char const*)"):
        assert bench._is_gemm(name), name
    for name in (RQ, COPY, "void convrot::(anonymous namespace)::weight_quant_mse_kernel(float const*)"):
        assert not bench._is_gemm(name), name


def test_gemm_kernel_label_follows_the_launch_rule():
    from w4a4_integer_quantized_amd import binding as rq
    T, R = rq.RQ_X_TILED, rq.RQ_X_ROWS
    # The shapes the GPU parity tests send to each kernel.
    assert bench.gemm_kernel_name(41472, 3072, 1024, 8, T) == "gemm_rw_kernel"
    assert bench.gemm_kernel_name(41472, 3072, 1024, 8, T, s32=True) == "gemm_rw_kernel"
    assert bench.gemm_kernel_name(4033, 3072, 1024, 8, T) == "gemm_rw_kernel"
    assert bench.gemm_kernel_name(4032, 3072, 1024, 8, T) == "gemm_xr_kernel"
    assert bench.gemm_kernel_name(41472, 1024, 1024, 8, T) == "gemm_xr_kernel"
    assert bench.gemm_kernel_name(8193, 1024, 1024, 8, T) == "gemm_xr_kernel"
    assert bench.gemm_kernel_name(8128, 1024, 1024, 8, T).startswith("gemm_kernel (8 waves")
    assert bench.gemm_kernel_name(4100, 2064, 1024, 8, T) == "gemm_xr_kernel"
    assert bench.gemm_kernel_name(4100, 2064, 1024, 8, T, s32=True) == "gemm_xr_kernel"   # same kernel for int32
    assert bench.gemm_kernel_name(4100, 2064, 2048, 4, T) == "gemm_kernel"        # int4: Kb = 1024
    assert bench.gemm_kernel_name(4100, 2064, 1024, 8, R) == "gemm_kernel"
    assert bench.gemm_kernel_name(1000, 1040, 1024, 8, T).startswith("gemm_kernel (8 waves")
    assert bench.gemm_kernel_name(4100, 2080, 3072, 8, T) == "gemm_n2_kernel"
    assert bench.gemm_kernel_name(8192, 1536, 6144, 8, T) == "gemm_n2_kernel"
    assert bench.gemm_kernel_name(2048, 6144, 1536, 8, R) == "gemm_wide_kernel"
    assert bench.gemm_kernel_name(2048, 6144, 1536, 8, R, act=1) == "gemm_kernel"
    assert bench.gemm_kernel_name(257, 512, 4096, 4, rq.RQ_X_FP6, rq.RQ_W_FP6) == "gemm_fp6_kernel"


def test_rotate_quant_kernel_label_follows_the_launch_rule():
    # nb = K / 128 blocks: G * NI with G in {1, 2, 4, 8, 12, 16}, NI <= 4 -> the coalesced kernel
    for K in (128, 256, 512, 1024, 1536, 2048, 3072, 4096, 6144, 8192):
        assert bench.rq_kernel_name(K) == "rotate_quant_coalesced_kernel", K
    for K in (640, 896, 1152, 1280, 1408, 1664, 1792, 1920):   # nb = 5, 7, 9, 10, 11, 13, 14, 15
        assert bench.rq_kernel_name(K) == "rotate_quant_kernel", K
    assert bench.rq_kernel_name(17 * 128) == "rotate_quant_generic_kernel"
    assert bench.rq_kernel_name(1024, fp6=True) == "rotate_quant_kernel"
    assert bench.rq_kernel_name(80 * 128) == "rotate_quant_generic_kernel"


def test_summaries_pick_the_dominant_gemm_kernel_by_name(tmp_path):
    # The persistent resident-weight GEMM has a smaller grid than the other linear's GEMM: the
    # dominant launch is chosen by kernel name, not by grid size.
    assert bench.dominant_gemm_kernel("vit_attn") == "gemm_rw_kernel"
    rw = "void convrot::(anonymous namespace)::gemm_rw_kernel<1, 96, 0>(unsigned char const*)"
    xr = "void convrot::(anonymous namespace)::gemm_xr_kernel<1, 16>(unsigned char const*)"
    gib_kib = (1 << 30) / 1024.0
    cf = _counters(tmp_path / "cf.csv", [(1, 4096, COPY, "FETCH_SIZE", gib_kib)])
    cw = _counters(tmp_path / "cw.csv", [(1, 4096, COPY, "WRITE_SIZE", gib_kib)])
    f = _counters(tmp_path / "f.csv", [(1, 131072, rw, "FETCH_SIZE", 100.0), (2, 331776, xr, "FETCH_SIZE", 7.0)])
    w = _counters(tmp_path / "w.csv", [(1, 131072, rw, "WRITE_SIZE", 200.0), (2, 331776, xr, "WRITE_SIZE", 9.0)])
    doc = bench.pmc_summary("wl", f, w, cf, cw, out_path=str(tmp_path / "p.json"), gemm_kernel="gemm_rw_kernel")
    assert doc["workloads"]["wl"]["gemm"]["grid_threads"] == 131072
    doc = bench.pmc_summary("wl", f, w, cf, cw, out_path=str(tmp_path / "q.json"))
    assert doc["workloads"]["wl"]["gemm"]["grid_threads"] == 331776
    assert not bench._matches(rw, "gemm_kernel") and bench._matches(GEMM, "gemm_kernel")
