"""The HBM-traffic summary behind bench.py's roofline "traffic" field:
calibration against the copy kernel, the per-dispatch averages, and that
the figures go stale when the compiled library changes (CPU only, synthetic
counter files in rocprofv3's csv layout)."""

from __future__ import annotations

import csv
import os

import pytest

from ulysses_sequence_parallelism_seq_amd import traffic

KERNEL_NAMES = {
    "__amd_rocclr_copyBuffer": "__amd_rocclr_copyBuffer",
    "permute_seq_to_head": "(anonymous namespace)::permute_seq_to_head(HIP_vector_type<unsigned int, 4u> const*)",
    "permute_head_to_seq": "(anonymous namespace)::permute_head_to_seq(HIP_vector_type<unsigned int, 4u> const*)",
    "attn_dkdv_bf16_kernel<128,false>": "void (anonymous namespace)::attn_dkdv_bf16_kernel<128, false>((anonymous namespace)::BwdArgs)",
    "attn_dq_bf16_kernel<128,false>": "void (anonymous namespace)::attn_dq_bf16_kernel<128, false>((anonymous namespace)::BwdArgs)",
    "delta_bf16_kernel<128>": "void (anonymous namespace)::delta_bf16_kernel<128>(__bf16 const*, float*)",
}


def _counter_dir(path, counter, per_kernel):
    """One csv row per dispatch; per_kernel maps short name -> list of per-dispatch KiB
    (or (grid size, KiB) pairs)."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        disp = 0
        for short, values in per_kernel.items():
            for v in values:
                grid, v = v if isinstance(v, tuple) else (1024, v)
                disp += 1
                w.writerow({"Dispatch_Id": disp, "Grid_Size": grid, "Kernel_Name": KERNEL_NAMES[short],
                            "Counter_Name": counter, "Counter_Value": v})
                w.writerow({"Dispatch_Id": disp, "Grid_Size": grid, "Kernel_Name": KERNEL_NAMES[short],
                            "Counter_Name": "OTHER", "Counter_Value": 1e12})


@pytest.fixture
def fake_library(tmp_path, monkeypatch):
    lib = tmp_path / "libulysses.so"
    lib.write_bytes(b"compiled code, version 1")
    monkeypatch.setattr(traffic, "LIBRARY", str(lib))
    return lib


def test_calibrated_bytes_and_staleness(tmp_path, fake_library):
    gib = 1 << 30
    # the 1 GiB copies read and write 1 GiB; FETCH_SIZE reports half of that, WRITE_SIZE all
    # of it; a small copy of another grid size does not enter the calibration
    fetch = {"__amd_rocclr_copyBuffer": [(131072, 524288.0), (131072, 524288.0), (64, 3.0)],
             # a launch of three tensors (three times the grid) does not enter the per-tensor figure
             "permute_seq_to_head": [524300.0, 524300.0, (3072, 3 * 524300.0)],
             "permute_head_to_seq": [524290.0, (3072, 3 * 524290.0)],
             "attn_dkdv_bf16_kernel<128,false>": [900.0, 1100.0],
             "attn_dq_bf16_kernel<128,false>": [500.0], "delta_bf16_kernel<128>": [50.0]}
    write = {"__amd_rocclr_copyBuffer": [(131072, 1048576.0), (64, 9.0)],
             "permute_seq_to_head": [1048580.0, (3072, 3 * 1048580.0)],
             "permute_head_to_seq": [1048576.0, (3072, 3 * 1048576.0)],
             "attn_dkdv_bf16_kernel<128,false>": [10.0],
             "attn_dq_bf16_kernel<128,false>": [5.0], "delta_bf16_kernel<128>": [1.0]}
    _counter_dir(tmp_path / "fetch", "FETCH_SIZE", fetch)
    _counter_dir(tmp_path / "write", "WRITE_SIZE", write)
    out = tmp_path / "traffic.txt"
    traffic.write_traffic(str(tmp_path / "fetch"), str(tmp_path / "write"), str(out), "the commands", gib)

    rec = traffic.read_traffic(str(out))
    assert rec is not None
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    # per-dispatch averages (dK/dV: 1000 KiB), fetch doubled, write as counted
    want_kib = 2.0 * (1000.0 + 500.0 + 50.0) + (10.0 + 5.0 + 1.0)
    assert rec["bytes"] == pytest.approx(want_kib * 1024.0)
    assert rec["permute"]["permute_seq_to_head"] == pytest.approx((2.0 * 524300.0 + 1048580.0) * 1024.0)
    assert rec["permute"]["permute_head_to_seq"] == pytest.approx((2.0 * 524290.0 + 1048576.0) * 1024.0)

    # a different compiled library makes the figures stale
    fake_library.write_bytes(b"compiled code, version 2")
    assert traffic.read_traffic(str(out)) is None


def test_missing_file_or_library_is_stale(tmp_path, fake_library):
    assert traffic.read_traffic(str(tmp_path / "absent.txt")) is None
    out = tmp_path / "traffic.txt"
    out.write_text("library_sha256 0123\ncopy __amd_rocclr_copyBuffer bytes=1 fetch_kib=1 write_kib=1\n")
    assert traffic.read_traffic(str(out)) is None
    os.remove(fake_library)
    assert traffic.library_sha256() is None
