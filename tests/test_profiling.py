"""The rocprofv3 summaries behind profiles/ (chunked_prefill_hybrid_layer_amd.profiling),
on small synthetic trace and counter files: forwards are cut at each RMSNorm
launch followed by a QKV projection, a step's launches are listed in order
with their median durations, phases sum the middle pass, and the HBM traffic
is scaled by what the counters read for the calibration copy.  CPU only."""
import csv

from chunked_prefill_hybrid_layer_amd import profiling as P

QKV = "void hb::gemm_kernel<0, hb::Tile<128, 96, 64, 4, 2, 4>, false>(hb::GemmArgs)"
NORM = "hb::rmsnorm_kernel(float const*, unsigned short const*, void*, int, float, float)"
ATTN = "void hb::attn_chunk_kernel<128, false>(hb::AttnArgs, float)"
O_PROJ = "void hb::gemm_kernel<1, hb::Tile<128, 128, 64, 4, 2, 4>, false>(hb::GemmArgs)"
GATE_UP = "void hb::gemm_specw_kernel<2, hb::SpecWTile<256, 224> >(hb::GemmArgs)"
DOWN = "void hb::gemm_spec_kernel<1, hb::SpecTile<256, 128, 3> >(hb::GemmArgs)"
FILL = "void at::native::vectorized_elementwise_kernel<8, at::native::FillFunctor<float> >"


def _trace(path, launches):
    """launches: (kernel name, duration ns) in time order."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        for name, d in launches:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + d})
            t += d + 500


def _forward(scale=1):
    return [(NORM, 5000 * scale), (QKV, 40000 * scale), (ATTN, 30000 * scale), (O_PROJ, 25000 * scale),
            (GATE_UP, 100000 * scale), (DOWN, 57000 * scale)]


def test_forwards_are_cut_at_norm_then_qkv_and_foreign_kernels_are_dropped(tmp_path):
    p = tmp_path / "run_kernel_trace.csv"
    _trace(p, [(FILL, 9000)] + _forward() + [(FILL, 9000)] + _forward(2))
    fw = P.forwards(str(p))
    assert len(fw) == 2
    assert [k for k, _, _ in fw[0]] == ["rmsnorm", "qkv_rope_append", "attn_chunk", "o_proj / down (residual)",
                                        "gate_up_swiglu", "o_proj / down (residual)"]
    assert [d for _, d, _ in fw[1]] == [10.0, 80.0, 60.0, 50.0, 200.0, 114.0]


def test_sequence_lists_launches_in_order_with_their_medians(tmp_path):
    p = tmp_path / "run_kernel_trace.csv"
    _trace(p, _forward(1) + _forward(3) + _forward(2))
    out = P.sequence(str(p))
    assert out.startswith("3 of 3 forwards")
    rows = [ln for ln in out.splitlines() if ln.startswith("| ") and ln[2].isdigit()]
    # the median of 1x, 3x, 2x is 2x; O comes before down (same short name, order tells them apart)
    assert [r.split("|")[3].strip() for r in rows] == ["10.00", "80.00", "60.00", "50.00", "200.00", "114.00"]
    assert out.splitlines()[-1].split("|")[3].strip() == "514.00"


def test_sequence_without_a_forward_says_so(tmp_path):
    p = tmp_path / "run_kernel_trace.csv"
    _trace(p, [(FILL, 1000), (ATTN, 2000)])
    assert P.sequence(str(p)).startswith("no layer forward")


def test_phases_sum_the_middle_pass(tmp_path):
    p = tmp_path / "run_kernel_trace.csv"
    _trace(p, _forward(1) + _forward(1) + _forward(5) + _forward(5) + _forward(9) + _forward(9))
    _, res = P.phases(str(p), [("x", 2, 3)])
    assert res["x"]["attn_chunk"] == 2 * 5 * 30.0


def _counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_is_scaled_by_the_calibration_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # the copy moves 256 MiB each way; FETCH_SIZE reads half of it, WRITE_SIZE all of it (KiB)
    _counters(fetch, [(copy, "FETCH_SIZE", 128 * 1024), (copy, "FETCH_SIZE", 10), (QKV, "FETCH_SIZE", 1000),
                      (QKV, "FETCH_SIZE", 3000)])
    _counters(write, [(copy, "WRITE_SIZE", 256 * 1024), (copy, "WRITE_SIZE", 10), (QKV, "WRITE_SIZE", 500)])
    res, cal = P.traffic(str(fetch), str(write))
    assert cal["copy_kernel"] == copy and abs(cal["fetch_factor"] - 2.0) < 1e-12 and cal["write_factor"] == 1.0
    q = res[QKV]
    assert q["read_bytes"] == 2000 * 1024 * 2.0 and q["write_bytes"] == 500 * 1024
    assert q["bytes_per_launch"] == q["read_bytes"] + q["write_bytes"] and q["launches"] == 2
