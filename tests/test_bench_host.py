"""Host logic of bench.py (no GPU): kernel-name classification for the counter ingestion and
the traffic scaling against the calibration copy."""
import csv
import json
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


@pytest.mark.parametrize("name,kind", [
    ("void nsg::gemm256h_kernel<0, true, false>(nsg::GemmArgs)", "gemm_nt_sym"),
    ("void nsg::gemm256h_kernel<0, true, true>(nsg::GemmArgs)", "gemm_nt_sym"),
    ("void nsg::gemm256h_kernel<1, false, true>(nsg::GemmArgs)", "gemm_nt"),
    ("void nsg::gemm256h_kernel<0, false, false>(nsg::GemmArgs)", "gemm_nt"),
    ("void nsg::gemm256_kernel<2, true, 4>(nsg::GemmArgs)", "gemm_nt_sym"),
    ("void nsg::gemm256_kernel<2, false, 4>(nsg::GemmArgs)", "gemm_nt"),
    ("void nsg::gemm_nt_kernel<2, 128, 128, 2, 2, true>(nsg::GemmArgs)", "gemm_nt_sym"),
    ("void nsg::gemm_nt_kernel<0, 128, 128, 2, 2, false>(nsg::GemmArgs)", "gemm_nt"),
    ("void nsg::scale_cast_transpose16_kernel<__bf16, _Float16, true>(nsg::ScaleArgs)", "scale_cast_transpose"),
    ("void nsg::scale_cast_transpose_kernel<float, float, false>(nsg::ScaleArgs)", "scale_cast_transpose"),
    ("void nsg::norm_reduce_kernel<__bf16, true>(nsg::NormReduceArgs)", "norm_reduce"),
    ("nsg::copy_kernel(uint4 const*, uint4*, unsigned long)", "copy"),
    ("void nsg::topk_kernel(nsg::TopkArgs)", None),
])
def test_kernel_kind(name, kind):
    assert bench.kernel_kind(name) == kind


def _write_pmc(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_ingest_scales_by_the_copy(tmp_path, monkeypatch):
    # the copy of COPY_BYTES reads 2x and writes 0.5x by the raw counters: a kernel's raw
    # counts are scaled by 1/2 and 2 respectively, and averaged over its dispatches
    gib_kib = bench.COPY_BYTES / 1024.0
    sym = "void nsg::gemm256h_kernel<0, true, true>(nsg::GemmArgs)"
    sym2 = "void nsg::gemm256h_kernel<0, true, false>(nsg::GemmArgs)"
    gen = "void nsg::gemm256h_kernel<0, false, false>(nsg::GemmArgs)"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_pmc(fetch, "FETCH_SIZE", [("nsg::copy_kernel(uint4 const*, uint4*, unsigned long)", 2 * gib_kib),
                                     (sym, 1000.0), (sym2, 3000.0), (gen, 4000.0)])
    _write_pmc(write, "WRITE_SIZE", [("nsg::copy_kernel(uint4 const*, uint4*, unsigned long)", 0.5 * gib_kib),
                                     (sym, 10.0), (sym2, 30.0), (gen, 40.0)])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    bench.ingest_pmc(str(fetch), str(write), "wl")
    tr = json.load(open(tmp_path / "traffic.json"))["wl"]
    assert tr["gemm_nt_sym"]["dispatches"] == 2
    assert tr["gemm_nt_sym"]["read_bytes_per_launch"] == pytest.approx(1024.0 * 2000.0 / 2)
    assert tr["gemm_nt_sym"]["write_bytes_per_launch"] == pytest.approx(1024.0 * 20.0 * 2)
    assert tr["gemm_nt"]["read_bytes_per_launch"] == pytest.approx(1024.0 * 4000.0 / 2)
    assert tr["calibration"]["fetch_scale"] == pytest.approx(0.5)
    assert tr["calibration"]["write_scale"] == pytest.approx(2.0)
