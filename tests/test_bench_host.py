"""Host-side checks of bench.py (no GPU): the one-GPU refusal, the byte
models behind the roofline line, and the counters lookup that turns the
traffic figure off when the kernel sources change."""
import json
import os
import subprocess
import sys

import bench
from dlrm_embedding_bag_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr, r.stderr
    assert r.stdout.strip() == "", "no JSON line for a refused run"


def test_fused_bytes_per_sample_at_the_benchmark_shape():
    # B = 2048, K = 32, D = 64, L = 20: rows 32*20*64*4 = 163840, indices
    # 32*20*4 = 2560, dense 256, output (64 + 528)*4 = 2368 -> 169024 B.
    assert bench.emb_interact_bytes_per_sample(32, 64, 20) == 169024
    assert 2048 * bench.emb_interact_bytes_per_sample(32, 64, 20) == 346161152


def test_general_form_bytes_reduce_to_the_f32_model():
    w = inputs.WORKLOADS["nc32"]
    assert bench.pool_bytes_per_sample(w, 32, 32 * 20) == \
        bench.emb_interact_bytes_per_sample(32, 64, 20)
    bf = inputs.WORKLOADS["nc32-bf16"]
    # bf16 rows are half as wide: 640 rows x 128 B less
    assert bench.pool_bytes_per_sample(bf, 32, 640) == 169024 - 640 * 128
    wt = inputs.WORKLOADS["nc32-weighted"]
    assert bench.pool_bytes_per_sample(wt, 32, 640) == 169024 + 640 * 4


def test_traffic_is_dropped_when_the_kernel_sources_change(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    p = tmp_path / "counters.json"
    p.write_text(json.dumps({"nc32": {"kernel_source_hash": h,
                                      "hbm_bytes_per_launch": 123.0}}))
    monkeypatch.setattr(bench, "COUNTERS_JSON", str(p))
    assert bench.read_traffic(h, "nc32")["hbm_bytes_per_launch"] == 123.0
    assert bench.read_traffic("0" * 16, "nc32") is None
    assert bench.read_traffic(h, "nc32-bf16") is None


def test_roofline_counts_served_bytes_and_stays_below_peak():
    """The roofline's achieved rate uses measured memory-side bytes when a
    counter record matches, else the compulsory bytes; the logical rate
    (repeated rows counted each time) is reported apart and may exceed the
    peak without touching frac."""
    logical, comp, ms = 346_161_152, 130_000_000, 0.040
    r = bench.hbm_roofline(logical, comp, ms, {"hbm_bytes_per_launch": 190e6}, None)
    assert r["achieved"] == 190e6 / 40e-6 / 1e9 and r["traffic"] == 190e6
    assert r["frac"] == r["achieved"] / 8000.0 and r["frac"] <= 1.0
    assert "measured" in r["byte_model"]
    assert r["logical_gbps"] > 8000.0          # L2-assisted: above the HBM peak
    r = bench.hbm_roofline(logical, comp, ms, None, {"gbps": 6000.0})
    assert r["traffic"] is None and "compulsory" in r["byte_model"]
    assert r["achieved"] == comp / 40e-6 / 1e9
    assert r["frac_of_practical_peak"] == r["achieved"] / 6000.0


def _pmc_dir(root, name, counter, rows):
    """A rocprofv3 --pmc output directory holding one counter_collection.csv
    with (dispatch id, kernel name, per-dimension value) rows."""
    d = os.path.join(root, name, "host", "1")
    os.makedirs(d)
    with open(os.path.join(d, "p_counter_collection.csv"), "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for disp, kern, val in rows:
            f.write(f'"{disp}","{kern}","{counter}","{val}"\n')


def test_record_counters_scales_by_known_reads_and_copies(tmp_path, monkeypatch):
    root = str(tmp_path)
    k = "void dlrm::interact_kernel<float, 4, 0, false, 16, false>(...)"
    # per-dispatch totals are summed over rows of one dispatch; the median
    # over dispatches is taken (100 KiB fetched, 10 KiB written per launch)
    _pmc_dir(root, "pmc_w_FETCH_SIZE", "FETCH_SIZE",
             [(1, k, 60), (1, k, 40), (2, k, 100), (3, k, 500), (4, "other", 7)])
    _pmc_dir(root, "pmc_w_WRITE_SIZE", "WRITE_SIZE", [(1, k, 10), (2, k, 10)])
    # the 1 GiB streaming read reads back half its size on FETCH_SIZE; the
    # 1 GiB copy all of it on WRITE_SIZE
    _pmc_dir(root, "pmc_read_FETCH_SIZE", "FETCH_SIZE",
             [(9, "dlrm::stream_read_kernel(...)", 524288)])
    _pmc_dir(root, "pmc_copy_WRITE_SIZE", "WRITE_SIZE", [(9, "__amd_rocclr_copyBuffer", 1048576)])
    out = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS_JSON", str(out))
    e = bench.record_counters(root, "w")
    assert e["fetch_size_kib_per_dispatch"] == 100 and e["write_size_kib_per_dispatch"] == 10
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    assert e["hbm_bytes_per_launch"] == 100 * 1024 * 2 + 10 * 1024
    assert "dram_bytes_per_launch" not in e
    assert e["kernel_source_hash"] == bench.kernel_source_hash()
    assert bench.read_traffic(bench.kernel_source_hash(), "w")["hbm_bytes_per_launch"] == \
        e["hbm_bytes_per_launch"]
    # the exact-unit DRAM request counters, when recorded (32-byte units)
    d = os.path.join(root, "pmc_w_DRAM", "host", "1")
    os.makedirs(d)
    with open(os.path.join(d, "p_counter_collection.csv"), "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        f.write(f'"1","{k}","TCC_EA0_RDREQ_DRAM_32B_sum","1000"\n')
        f.write(f'"1","{k}","TCC_EA0_WRREQ_WRITE_DRAM_32B_sum","50"\n')
    e = bench.record_counters(root, "w")
    assert e["dram_bytes_per_launch"] == 1050 * 32
