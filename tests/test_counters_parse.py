"""The counter summaries' parsing, on the CPU, over a small hand-written
rocprofv3 counter_collection.csv: the calibration copy is the run's first copy
dispatch (later copies are input conversions, not calibrations), a kernel's
dispatches are found by name and kept apart from other kernels, and a pass
that lacks the copy or the kernel is refused."""
import os

import pytest

from shared_base_residual_amd import counters as C

HEADER = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"


def _write(tmp_path, rows):
    d = tmp_path / "pass"
    (d / "host").mkdir(parents=True)
    (d / "host" / "run_counter_collection.csv").write_text(HEADER + "".join(f"{r}\n" for r in rows))
    return str(d)


def test_calibration_is_the_first_copy_and_kernels_by_name(tmp_path):
    d = _write(tmp_path, [
        "1,__amd_rocclr_copyBuffer,FETCH_SIZE,131072.0",
        "2,void rattn::decode_split_kernel<bf16>(DecodeParams),FETCH_SIZE,70000.0",
        "3,void rattn::combine_kernel<bf16>(DecodeParams),FETCH_SIZE,1500.0",
        "4,__amd_rocclr_copyBuffer,FETCH_SIZE,999.0",
        "5,void rattn::decode_split_kernel<bf16>(DecodeParams),FETCH_SIZE,71000.0",
        "6,void rattn::decode_split_kernel<bf16>(DecodeParams),WRITE_SIZE,2368.0",
    ])
    copy, kern = C._per_dispatch(d, "FETCH_SIZE", ["decode_split_kernel", "combine_kernel"])
    assert copy == 131072.0
    assert kern == {"decode_split_kernel": [70000.0, 71000.0], "combine_kernel": [1500.0]}
    # bytes per launch: counter KiB x 1024 x (copy bytes / counted copy bytes)
    scale = C.COPY_BYTES / (copy * 1024.0)
    assert scale == pytest.approx(2.0)
    assert sum(kern["decode_split_kernel"]) / 2 * 1024.0 * scale == pytest.approx(70500 * 2048)


def test_missing_copy_or_kernel_is_refused(tmp_path):
    d = _write(tmp_path, ["2,void rattn::decode_split_kernel<bf16>(DecodeParams),FETCH_SIZE,70000.0"])
    with pytest.raises(SystemExit):
        C._per_dispatch(d, "FETCH_SIZE", ["decode_split_kernel"])
    d2 = _write(tmp_path / "b", ["1,__amd_rocclr_copyBuffer,FETCH_SIZE,131072.0"])
    with pytest.raises(SystemExit):
        C._per_dispatch(d2, "FETCH_SIZE", ["decode_split_kernel"])
    with pytest.raises(SystemExit):
        C._per_dispatch(str(tmp_path / "empty"), "FETCH_SIZE", ["decode_split_kernel"])
