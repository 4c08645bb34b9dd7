"""Host logic of bench.py (no GPU): the HBM-traffic derivation from rocprofv3 counter files."""
import csv
import os

import pytest

import bench


def _write_pass(root, counter, rows):
    d = os.path.join(root, counter)
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Value"])
        w.writeheader()
        for did, name, val in rows:
            w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Value": val})


def _step_rows(scale):
    """One calibration copy, then two steps: act_quant before every projection, QKV as two GEMM
    dispatches (256x256 then 256x128 tiles), O, gate+up and down as one each.  Values in KiB."""
    rows = [(1, "__amd_rocclr_copyBuffer", 1 << 19)]  # reads half of 1 GiB, as FETCH_SIZE does
    did = 2
    for _ in range(2):
        for parts in ([100, 50], [70], [900], [300]):
            rows.append((did, "fgb::act_quant_kernel(...)", 999))
            did += 1
            for v in parts:
                rows.append((did, "void fgb::gemm_prefill_kernel<...>(...)", v * scale))
                did += 1
    return rows


def test_derive_traffic_groups_dispatches_into_projection_calls(tmp_path):
    _write_pass(str(tmp_path), "FETCH_SIZE", _step_rows(1))
    _write_pass(str(tmp_path), "WRITE_SIZE", _step_rows(2))
    t = bench.derive_traffic(str(tmp_path), names=("qkv", "o", "gate_up", "down"))
    assert t["fetch_size_copy_factor"] == pytest.approx(2.0)
    # WRITE_SIZE's copy dispatch reads the same 2^19 KiB, so its factor is also 2
    kib = 1024 * 2.0
    pp = t["per_projection"]
    assert pp["qkv"]["dispatches"] == 2 and pp["o"]["dispatches"] == 1
    assert pp["qkv"]["fetch_size_bytes"] == round(150 * kib)
    assert pp["qkv"]["write_size_bytes"] == round(300 * kib)
    assert pp["gate_up"]["fetch_size_bytes"] == round(900 * kib)
    assert pp["down"]["write_size_bytes"] == round(600 * kib)
    per_call = (150 + 70 + 900 + 300) * kib / 4 * 3  # fetch + twice that written
    assert t["gemm_prefill_hbm_bytes_per_call"] == round(per_call)
    assert t["kernel_source_hash"] == bench.kernel_source_hash()


def test_derive_traffic_rejects_a_partial_step(tmp_path):
    rows = _step_rows(1)[:-2]  # the second step loses its down projection (act_quant and GEMM)
    _write_pass(str(tmp_path), "FETCH_SIZE", rows)
    _write_pass(str(tmp_path), "WRITE_SIZE", rows)
    with pytest.raises(SystemExit):
        bench.derive_traffic(str(tmp_path), names=("qkv", "o", "gate_up", "down"))
