"""The benchmark's host-side accounting, checked on the CPU.

The algorithmic byte counts that the roofline fractions divide by are held against the sizes of the
arrays the seeded generator actually builds (so a wrong scale-group size or a dropped scale array in
the accounting fails here), the counter scaling against its copy calibration, and the stored
traffic readings against the workloads the benchmark looks them up for, and the rocprofv3 summary
parsers against small CSV files of the same columns.
"""
import json
import os
import subprocess
import sys

import pytest
import torch

import bench
import moe_inputs as mi
from sparse_moe_expert_router_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

FORMATS = [mi.FMT_Q8_0, mi.FMT_I8_ROW, mi.FMT_FP8_ROW, mi.FMT_E2M1]


def _small(fmt, act=None):
    w = mi.workload("tiny", fmt=fmt, E=4, d_model=128, d_ff=256)
    return w if act is None else mi.workload("tiny", fmt=fmt, E=4, d_model=128, d_ff=256, act=act)


def _per_expert(layer, *names):
    ex = layer["experts"]
    NE = ex["E"] + ex["n_shared"]
    total = sum(ex[n].numel() * ex[n].element_size() for n in names)
    assert total % NE == 0
    return total // NE


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("act", [mi.ACT_SWIGLU, mi.ACT_RELU2])
def test_expert_bytes_match_the_generated_arrays(fmt, act):
    w = _small(fmt, act)
    lay = mi.make_layer(w, 0)
    assert bench.expert_gateup_bytes(w) == _per_expert(lay, "gate_up", "gate_up_scales")
    assert bench.expert_down_bytes(w) == _per_expert(lay, "down", "down_scales")
    assert mi.expert_bytes(w) == _per_expert(lay, "gate_up", "gate_up_scales", "down", "down_scales")


def test_e2m1_group_bytes_match_one_16_neuron_group():
    w = _small(mi.FMT_E2M1)
    lay = mi.make_layer(w, 0)
    ex = lay["experts"]
    NE = ex["E"] + ex["n_shared"]
    groups = NE * (w.d_ff // 16)
    c = bench.Case.__new__(bench.Case)
    c.w = w
    assert c.group_bytes() * groups == (ex["down"].numel() * ex["down"].element_size()
                                        + ex["down_scales"].numel() * ex["down_scales"].element_size())


@pytest.mark.parametrize("xtype", [mi.X_F32, mi.X_BF16])
def test_algorithmic_bytes_of_a_decode_call(xtype):
    # two instances touching 3 and 5 experts: the average, 4 experts' weights, plus x, router, out
    w = mi.workload("tiny", xtype=xtype)
    lay = mi.make_layer(w, 0)
    x = mi.make_x(w, 0)
    c = bench.Case.__new__(bench.Case)
    c.w, c.flags, c.distinct, c.active_groups = w, 0, [3, 5], None
    gu, layer = c.algorithmic_bytes()
    xb = x.numel() * x.element_size()
    gu_w = 4 * _per_expert(lay, "gate_up", "gate_up_scales")
    dn_w = 4 * _per_expert(lay, "down", "down_scales")
    router = lay["w_router"].numel() * lay["w_router"].element_size()
    out = w.T * w.d_model * 4
    assert gu == pytest.approx(gu_w + xb)
    assert layer == pytest.approx(gu_w + xb + dn_w + router + out)


def test_algorithmic_bytes_with_zero_skip_count_only_live_groups():
    w = mi.workload("tiny", fmt=mi.FMT_E2M1, act=mi.ACT_RELU2)
    c = bench.Case.__new__(bench.Case)
    c.w, c.flags, c.distinct, c.active_groups = w, 1, [2, 2], [10, 30]
    gu, layer = c.algorithmic_bytes()
    xb = w.T * w.d_model * 4
    dn = 20 * c.group_bytes()
    assert layer == pytest.approx(gu + dn + w.E * w.d_model * 4 + w.T * w.d_model * 4)
    assert gu == pytest.approx(2 * bench.expert_gateup_bytes(w) + xb)


def test_prefill_flops_count_each_pairs_contractions():
    c = bench.Case.__new__(bench.Case)
    c.w = w = mi.workload("gemma_prefill", T=16)
    # gate, up (d_model -> d_ff each) and down (d_ff -> d_model), 2 ops per multiply-add, per pair
    assert c.algorithmic_ops() == 2 * (2 * w.d_model * w.d_ff + w.d_ff * w.d_model) * w.T * w.k
    c.w = w = mi.workload("gemma_prefill", T=16, act=mi.ACT_RELU2)
    assert c.algorithmic_ops() == 2 * (w.d_model * w.d_ff + w.d_ff * w.d_model) * w.T * w.k


def test_counter_scaling_maps_the_copy_back_to_its_size():
    calib = {"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30,
             "fetch_kib": 524288.0 * 1.001, "write_kib": 1048576.0}
    got = profiling.scaled_traffic(calib["fetch_kib"], calib["write_kib"], calib)
    assert got == pytest.approx(2 * (1 << 30))
    assert profiling.scaled_traffic(0.0, 0.0, calib) == 0.0
    half = profiling.scaled_traffic(calib["fetch_kib"] / 2, 0.0, calib)
    assert half == pytest.approx((1 << 30) / 2)


def test_traffic_keys_name_the_workload():
    w = mi.workload("gemma_decode", T=8)
    assert bench.traffic_key(w, 0, True) == "gemma_decode:T=8:q8_0:tiled:flags=0"
    assert bench.traffic_key(w, 0, False) == "gemma_decode:T=8:q8_0:plain:flags=0"
    e = mi.workload("gemma_decode", T=8, fmt=mi.FMT_E2M1)
    assert bench.traffic_key(e, 0, True).endswith(":e2m1:plain:flags=0")
    s = mi.workload("gemma_decode", T=8, n_shared=1)
    assert bench.traffic_key(s, 0, True).endswith(":shared=1")


def test_stored_traffic_readings_are_well_formed():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        db = json.load(fh)
    assert db
    for key, ent in db.items():
        kernel, wl = key.split("|")
        assert kernel in ("gateup_int8", "up_e2m1", "ggemm_gateup_i8"), key
        assert ent["bytes_per_launch"] > 0
        cal = ent["calibration"]
        assert cal["fetch_kib"] > 0 and cal["write_kib"] > 0
        assert ent["command"].startswith("rocprofv3 --pmc ")
        assert len(ent["source_hash"]) == 16


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _dominant_kernel(w, flags):
    if flags & (4 | 8):
        return "ggemm_gateup_i8"
    return "up_e2m1" if w.fmt == mi.FMT_E2M1 else "gateup_int8"


def test_every_timed_workload_has_a_stored_traffic_reading():
    # the headline (Gemma-shaped decode, T = 8, Q8_0, tiled) and every variant with a roofline
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        db = json.load(fh)
    cases = [(mi.workload("gemma_decode", T=8), 0, True)]
    cases += [(w, f, "plain" not in label) for w, _, f, label in bench.variant_specs()]
    hashes = set()
    for w, flags, tiled in cases:
        key = f"{_dominant_kernel(w, flags)}|{bench.traffic_key(w, flags, tiled)}"
        assert key in db, key
        hashes.add(db[key]["source_hash"])
    assert len(hashes) == 1, "readings taken from different sources"


def test_kernel_stats_and_counter_means_parse_rocprofv3_csv(tmp_path):
    stats = tmp_path / "run_kernel_stats.csv"
    stats.write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void moe::gateup_int8_kernel<0, 1>(int const*, float*)",176,6988960,39710.0,55.1,38000,41000,100.0\n'
        '"moe::combine_rows4_kernel(float const*, int)",88,381920,4340.0,3.0,4100,4600,10.0\n')
    st = profiling.kernel_stats(str(stats))
    assert set(st) == {"moe::gateup_int8_kernel<0, 1>", "moe::combine_rows4_kernel"}
    g = st["moe::gateup_int8_kernel<0, 1>"]
    assert g["calls"] == 176 and g["avg_ns"] == 39710.0 and g["min_ns"] == 38000 and g["max_ns"] == 41000
    cnt = tmp_path / "run_counter_collection.csv"
    cnt.write_text(
        '"Kernel_Name","Counter_Name","Counter_Value"\n'
        '"void moe::gateup_int8_kernel<0, 1>(int const*, float*)","FETCH_SIZE",100.0\n'
        '"void moe::gateup_int8_kernel<0, 1>(int const*, float*)","FETCH_SIZE",300.0\n'
        '"void moe::gateup_int8_kernel<0, 1>(int const*, float*)","WRITE_SIZE",7.0\n'
        '"moe::combine_rows4_kernel(float const*, int)","FETCH_SIZE",50.0\n')
    m = profiling.counter_means(str(cnt), "FETCH_SIZE")
    assert m == {"moe::gateup_int8_kernel<0, 1>": (2, 200.0), "moe::combine_rows4_kernel": (1, 50.0)}
    assert profiling.counter_means(str(cnt), "WRITE_SIZE") == {"moe::gateup_int8_kernel<0, 1>": (1, 7.0)}


def test_traffic_lookup_checks_the_source_hash(tmp_path):
    key = "gateup_int8|gemma_decode:T=8:q8_0:tiled:flags=0"
    db = {key: {"bytes_per_launch": 123.0, "source_hash": profiling.source_hash()},
          "up_e2m1|x": {"bytes_per_launch": 5.0, "source_hash": "0" * 16}}
    (tmp_path / "traffic.json").write_text(json.dumps(db))
    kernel, wl = key.split("|")
    assert profiling.load_traffic(str(tmp_path), kernel, wl) == 123.0
    assert profiling.load_traffic(str(tmp_path), "up_e2m1", "x") is None        # older sources
    assert profiling.load_traffic(str(tmp_path), "gateup_int8", "absent") is None
    assert profiling.load_traffic(str(tmp_path / "none"), kernel, wl) is None


def test_profile_summaries_match_the_stored_readings():
    # every kernel summary names the command that made it and was taken at the same sources as
    # the traffic readings; the dominant kernel's traffic line agrees with traffic.json
    import glob
    import re
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        db = json.load(fh)
    hashes = {ent["source_hash"] for ent in db.values()}
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    assert len(paths) == len(db)
    for p in paths:
        txt = open(p).read()
        assert "rocprofv3 --kernel-trace --stats" in txt and "python3 bench.py" in txt, p
        m = re.search(r"HIP source hash at collection: `([0-9a-f]{16})`", txt)
        assert m and m.group(1) in hashes, p
        t = re.search(r"`(\w+)`: ([0-9.]+) MB of HBM traffic per launch vs ([0-9.]+) MB algorithmic", txt)
        assert t, p
        kernel, mb = t.group(1), float(t.group(2))
        near = [e["bytes_per_launch"] for k, e in db.items() if k.startswith(kernel + "|")]
        assert any(abs(b / 1e6 - mb) < 0.01 for b in near), p
