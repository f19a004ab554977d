"""bench.py's rocprofv3 summaries (the files under profiles/): kernel symbols
to layer stages, and the per-stage averages of a trace and of counters, on
small hand-written CSV files of rocprofv3's format."""

import csv
import os

import bench


def test_stage_of_kernel_mangled_and_demangled():
    cases = {
        "_ZN4lmoe11gemm_kernelIDF16bLi256ELi256ELi4ELi2ELi2ELb1ELi1ELi1ELb0ELi0ELi64EEEvNS_10GemmParamsE":
            "grouped_gemm1_relu2",
        "_ZN4lmoe11gemm_kernelIDF16bLi32ELi64ELi1ELi2ELi2ELb1ELi1ELi2ELb1ELi0ELi0EEEvNS_10GemmParamsE":
            "grouped_gemm2",
        "_ZN4lmoe11gemm_kernelIDF16bLi256ELi256ELi4ELi2ELi2ELb0ELi1ELi0ELb0ELi0ELi0EEEvNS_10GemmParamsE":
            "gemm_x_router_down_shared1",
        "_ZN4lmoe18skinny_gemm_kernelIDF16bLi2ELi8ELi16ELi0EEEvNS_10GemmParamsE": "gemm_x_router_down_shared1",
        "_ZN4lmoe19fewrow_split_kernelIDF16bLi2ELi1ELi8ELi3EEEvNS_10GemmParamsE": "gemm_up_shared2",
        "void lmoe::gemm_kernel<__hip_bfloat16, 128, 128, 2, 2, 2, true, 1, 2, false, 0, 0>(lmoe::GemmParams)":
            "grouped_gemm2",
        "void lmoe::fewrow_split_kernel<__hip_bfloat16, 2, 1, 8, 3>(lmoe::GemmParams)": "gemm_up_shared2",
        "_ZN4lmoe17route_tiny_kernelILi4EEEvNS_15TinyRouteParamsE.kd": "router_select",
        "void lmoe::dispatch_small_kernel(int const*, int, int const*, int const*, int, int, int, int, int, int, int, "
        "int*, int*, int*, HIP_vector_type<int, 4u>*, int*, int*, int*)": "dispatch_finalize",
        "void lmoe::router_select_kernel<4, 4, false>(float const*, int, int, int, int*, float*, int*, int*, int)":
            "router_select",
        "_ZN4lmoe17expert_mlp_kernelILi128ELi512ELi128ELi32ELi4ELi4ELi2ELi2ELi4ELb0ELi8EEEvNS_9MlpParamsE":
            "expert_mlp",
        "_ZN4lmoe14combine_kernelIDF16bEEvPKT_PKiPKfiiiPS1_l": "combine",
        "_ZN4lmoe14gemm_tn_kernelILi6EEEvNS_10GemmParamsE.kd": "backward_wgrad_experts",
        "void lmoe::gemm_tn_kernel<5>(lmoe::GemmParams)": "backward_wgrad",
        "_ZN4lmoe13retile_kernelIDF16bLi64EEEvPKT_iiPS1_.kd": "backward_retile",
        "_ZN12_GLOBAL__N_118gather_rows_kernelIDF16bEEvPKT_lPKiliPS1_": "backward_gather_rows",
    }
    for name, stage in cases.items():
        assert bench.stage_of_kernel(name) == stage, name


def _write(path, rows, fields):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


GEMM_X = "_ZN4lmoe11gemm_kernelIDF16bLi256ELi256ELi4ELi2ELi2ELb0ELi1ELi0ELb0ELi0ELi0EEEvNS_10GemmParamsE"
COMBINE = "_ZN4lmoe14combine_kernelIDF16bEEvPKT_PKiPKfiiiPS1_l"
ADD = "void at::native::vectorized_elementwise_kernel<4, at::native::CUDAFunctor_add<float>>(int)"


def test_trace_summary(tmp_path):
    f = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows = [{"Kernel_Name": GEMM_X, "Start_Timestamp": 1000, "End_Timestamp": 11000},
            {"Kernel_Name": GEMM_X, "Start_Timestamp": 20000, "End_Timestamp": 50000},
            {"Kernel_Name": COMBINE, "Start_Timestamp": 0, "End_Timestamp": 2000}]
    _write(str(tmp_path / "t" / "trace_kernel_trace.csv"), rows, f)
    lines = bench.summarize_trace(str(tmp_path / "t")).splitlines()
    x = [ln for ln in lines if ln.startswith("gemm_x_router_down_shared1")][0].split()
    assert x[1:] == ["2", "20.00", "10.00", "30.00"]
    c = [ln for ln in lines if ln.startswith("combine")][0].split()
    assert c[1:] == ["1", "2.00", "2.00", "2.00"]


def test_traffic_summary_scales_by_the_copy_calibration(tmp_path):
    f = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    # the calibration add reads 256 MiB and writes 256 MiB; its counters read half and all of it
    fetch = [{"Dispatch_Id": 1, "Kernel_Name": ADD, "Counter_Name": "FETCH_SIZE", "Counter_Value": 131072.0,
              "Start_Timestamp": 0, "End_Timestamp": 1},
             {"Dispatch_Id": 2, "Kernel_Name": COMBINE, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1024.0,
              "Start_Timestamp": 0, "End_Timestamp": 1}]
    write = [{"Dispatch_Id": 1, "Kernel_Name": ADD, "Counter_Name": "WRITE_SIZE", "Counter_Value": 262144.0,
              "Start_Timestamp": 0, "End_Timestamp": 1},
             {"Dispatch_Id": 2, "Kernel_Name": COMBINE, "Counter_Name": "WRITE_SIZE", "Counter_Value": 512.0,
              "Start_Timestamp": 0, "End_Timestamp": 1}]
    _write(str(tmp_path / "f" / "fetch_counter_collection.csv"), fetch, f)
    _write(str(tmp_path / "w" / "write_counter_collection.csv"), write, f)
    out = bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    assert "fetch_factor: 2.0000" in out and "write_factor: 1.0000" in out
    # 1024 KiB counted -> 2 MiB read; 512 KiB written
    assert f"traffic_bytes[combine]: {2 * 1024 * 1024 + 512 * 1024}" in out
