"""The committed HBM-traffic summaries that bench.py reports as
``roofline.traffic``: each record's total follows from its own counters and
scales, and a record taken on another kernel source is never reported."""

import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

NAMES = ["paged_decode_b16_ctx8k", "paged_decode_int8_b16_ctx8k", "paged_decode_c3_mix_b16"]


@pytest.mark.parametrize("name", NAMES)
def test_traffic_record_total_follows_from_counters(name):
    with open(os.path.join(ROOT, "profiles", name + "_traffic.json")) as f:
        rec = json.load(f)
    total = (rec["fetch_kib_per_dispatch"] * rec["fetch_scale"]
             + rec["write_kib_per_dispatch"] * rec["write_scale"]) * 1024
    assert abs(total - rec["hbm_bytes_per_launch"]) < 1024
    # FETCH_SIZE's calibration on a plain copy: the counter reads half the bytes.
    assert 1.99 < rec["fetch_scale"] < 2.01 and rec["write_scale"] == 1.0
    assert len(rec["kernel_source_sha256_16"]) == 16


@pytest.mark.parametrize("name", NAMES)
def test_traffic_reported_only_for_its_kernel_source(name):
    with open(os.path.join(ROOT, "profiles", name + "_traffic.json")) as f:
        rec = json.load(f)
    assert bench.measured_traffic(name, rec["kernel_source_sha256_16"]) == rec["hbm_bytes_per_launch"]
    assert bench.measured_traffic(name, "0" * 16) is None
    assert bench.measured_traffic(None, rec["kernel_source_sha256_16"]) is None
    assert bench.measured_traffic("no_such_profile", rec["kernel_source_sha256_16"]) is None
