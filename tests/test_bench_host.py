"""bench.py's host logic (no GPU): the one-GPU rule, the algorithmic work of
each workload written out from its definition, and the rocprofv3 summary
arithmetic on synthetic counter files."""

import importlib.util
import json
import os
import subprocess
import sys

import pytest

from linear_attention_recurrence_forward_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""


# Bytes each workload must move once, written out term by term: state read and
# written, q and k once per key head, v and output once, g and beta once,
# capture once (elements x bytes).
def expected_bytes(d_k, d_v, hk, hv, t, s, capture=False, io=4):
    state = d_k * d_v * hv * s
    return (4 * 2 * state + io * t * s * (d_k * hk) * 2 + io * t * s * (d_v * hv) * 2
            + 4 * t * s * hv * 2 + (4 * t * state if capture else 0))


@pytest.mark.parametrize("name,shape,capture,total", [
    ("decode", (128, 128, 16, 48, 1, 1), False, 6_357_376),
    ("batched_decode", (128, 128, 16, 32, 1, 64), False, 271_597_568),
    ("spec_verify", (128, 128, 8, 8, 4, 8), True, 25_692_160),
    ("prefill", (128, 128, 16, 48, 512, 4), False, 160_169_984),
])
def test_algorithmic_bytes(bench, name, shape, capture, total):
    w, kernel, alg, _ = bench.workload_info(name)
    assert (w.d_k, w.d_v, w.n_k_heads, w.n_v_heads, w.n_tokens, w.n_seqs) == shape
    assert alg == expected_bytes(*shape, capture=capture) == total
    want = ("gdn_decode" if shape[4] == 1 else
            "gdn_short" if shape[4] <= 8 else "gdn_recurrent")
    assert kernel == want
    _, _, alg16, _ = bench.workload_info(name, "bf16")
    assert alg16 == expected_bytes(*shape, capture=capture, io=2)


@pytest.mark.parametrize("shape,capture,kernel", [
    ((128, 128, 16, 48, 1, 1), False, "gdn_decode"),
    ((128, 128, 8, 8, 2, 8), True, "gdn_short"),
    ((32, 32, 1, 2, 8, 1), False, "gdn_short"),
    ((128, 128, 8, 8, 12, 8), False, "gdn_short"),      # 8,192 rows
    ((128, 128, 8, 8, 12, 8), True, "gdn_recurrent"),   # D_k = 128 capture past 8
    ((64, 64, 8, 8, 16, 8), True, "gdn_short"),
    ((128, 128, 8, 136, 9, 1), False, "gdn_recurrent"),  # 17,408 rows
    ((128, 128, 8, 8, 17, 8), False, "gdn_recurrent"),
])
def test_kernel_of_a_workload(bench, shape, capture, kernel):
    """The kernel a bench line names follows the library's choice: one token
    the one-token kernel, 2 to 8 tokens the short kernel, 9 to 16 the short
    kernel on grids of at most 16,384 rows (not with capture at D_k = 128),
    longer the general one."""
    dk, dv, hk, hv, t, s = shape
    WORKLOADS["kernel_probe"] = WORKLOADS["spec_verify"].with_(
        name="kernel_probe", d_k=dk, d_v=dv, n_k_heads=hk, n_v_heads=hv, n_tokens=t,
        n_seqs=s, capture=capture)
    try:
        assert bench.workload_info("kernel_probe")[1] == kernel
    finally:
        del WORKLOADS["kernel_probe"]


def test_rollback_bytes(bench):
    w, kernel, alg, _ = bench.workload_info("rollback")
    state = w.d_k * w.d_v * w.n_v_heads * w.n_seqs
    assert kernel == "gdn_rollback_kernel"
    assert alg == 4 * 2 * state + 4 * w.n_seqs  # slice read, state written, indexes


def test_flops():
    w = WORKLOADS["prefill"]
    # one multiply and three multiply-adds per state cell per token
    assert w.flops() == 7 * 128 * 128 * 48 * 512 * 4 == 11_274_289_152


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(f'"{v}"' for v in r) + "\n")


def test_summarize_rocprof(bench, tmp_path):
    """Counters scaled by what they read for the calibration copy: FETCH_SIZE
    reads half (factor 2), WRITE_SIZE all (factor 1) in this fixture."""
    src, out = tmp_path / "prof", tmp_path / "profiles"
    wl, digest = "decode", "abc123"
    for log in (f"kt_{wl}.log", f"pmc_FETCH_SIZE_{wl}.log", f"pmc_WRITE_SIZE_{wl}.log"):
        os.makedirs(src, exist_ok=True)
        with open(src / log, "w") as f:
            f.write("noise\n" + json.dumps({"kernel_digest": digest}) + "\n")
    write_csv(str(src / f"kt_{wl}" / "run_kernel_stats.csv"),
              ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
              [["void gdn::gdn_decode<128>", 220, 3650.0, 2800.0, 7000.0, 30.0],
               ["__amd_rocclr_copyBuffer", 10, 3000.0, 2000.0, 9000.0, 70.0]])
    # per-dispatch durations 2.8, 3.0, 3.2 and 7.0 us: median 3.10 us
    write_csv(str(src / f"kt_{wl}" / "run_kernel_trace.csv"),
              ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
              [["void gdn::gdn_decode<128>", 1000 * i, 1000 * i + d]
               for i, d in enumerate((2800, 3200, 7000, 3000))])
    calib_mib = 1024
    for ctr, copy_kib, ours in (("FETCH_SIZE", 524288.0, [1600.0, 1700.0]),
                                ("WRITE_SIZE", 1048576.0, [3000.0, 3000.0])):
        write_csv(str(src / f"pmc_{ctr}_{wl}" / "run_counter_collection.csv"),
                  ["Kernel_Name", "Counter_Value"],
                  [["__amd_rocclr_copyBuffer", 10.0], ["__amd_rocclr_copyBuffer", copy_kib]]
                  + [["void gdn::gdn_decode<128>", v] for v in ours])
    md = bench.summarize_rocprof(str(src), wl, calib_mib,
                                 dict(kt="kt-cmd", fetch="fetch-cmd", write="write-cmd"),
                                 out_dir=str(out))
    with open(out / f"gdn_decode_{wl}_hbm_traffic.json") as f:
        rec = json.load(f)
    fetch = 1650.0 * 2 * 1024
    write = 3000.0 * 1 * 1024
    assert rec["kernel_digest"] == digest
    assert rec["fetch_bytes"] == pytest.approx(fetch)
    assert rec["write_bytes"] == pytest.approx(write)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(fetch + write)
    text = open(md).read()
    assert "kt-cmd" in text and "fetch-cmd" in text and "write-cmd" in text
    # average, median, p10 / p90 (nearest rank of 2.8, 3.0, 3.2, 7.0), min, max
    assert "| 220 | 3.65 | 3.10 | 2.80 / 7.00 | 2.80 | 7.00 |" in text
    assert f"ratio {(fetch + write) / 6_357_376:.3f}" in text
    assert bench.traffic_from_profiles(wl, digest, "gdn_decode", profiles=str(out)) == \
        pytest.approx(fetch + write)
    assert bench.traffic_from_profiles(wl, "other-build", "gdn_decode",
                                       profiles=str(out)) is None
    assert bench.traffic_from_profiles("prefill", digest, profiles=str(out)) is None


def test_summarize_rocprof_refuses_mixed_builds(bench, tmp_path):
    src = tmp_path / "prof"
    os.makedirs(src)
    for i, log in enumerate(("kt_decode.log", "pmc_FETCH_SIZE_decode.log",
                             "pmc_WRITE_SIZE_decode.log")):
        with open(src / log, "w") as f:
            f.write(json.dumps({"kernel_digest": f"build{i % 2}"}) + "\n")
    with pytest.raises(SystemExit, match="disagree"):
        bench.summarize_rocprof(str(src), "decode", 1024, {}, out_dir=str(tmp_path / "o"))


def test_summarize_valu_counters(bench, tmp_path):
    """Clock, per-token instruction counts and dual-issue share from two
    synthetic counter runs of the prefill workload."""
    src, out = tmp_path / "pmc", tmp_path / "profiles"
    os.makedirs(out)
    waves, toks = 3072, 512
    cycles = 400_000 * 8  # 2.0 GHz over 200 us, summed over 8 XCDs
    valu = waves * toks * 64.0
    dual = 1024 * 16_000.0  # quad-cycles issuing two, summed over 1024 SIMDs
    counters = {
        "sq1": dict(SQ_WAVES=waves, SQ_INSTS_VALU=valu, SQ_INSTS_SALU=1.0,
                    SQ_INSTS_VMEM_RD=1.0, GRBM_GUI_ACTIVE=cycles),
        "sq2": dict(SQ_WAVES=waves, SQ_ACTIVE_INST_VALU2=dual,
                    SQ_INSTS_VALU_FMA_F32=waves * toks * 48.0,
                    SQ_INSTS_VALU_MUL_F32=waves * toks * 4.0,
                    SQ_INSTS_VALU_ADD_F32=waves * toks * 6.0,
                    SQ_INSTS_VALU_FLOPS_FP32=11e9 / 64, SQ_INSTS_LDS=1.0,
                    GRBM_GUI_ACTIVE=cycles),
    }
    for p, cs in counters.items():
        rows = []
        for disp in (1, 2, 3):
            for name, v in cs.items():
                rows.append([disp, "void gdn::gdn_recurrent<128>", name, v,
                             1_000_000, 1_000_000 + 200_000])
        rows.append([9, "__amd_rocclr_copyBuffer", "SQ_WAVES", 5.0, 0, 10])
        write_csv(str(src / p / "run_counter_collection.csv"),
                  ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                   "Start_Timestamp", "End_Timestamp"], rows)
    with open(src / "sq1.log", "w") as f:
        f.write("noise\n" + json.dumps({"kernel_digest": "feed"}) + "\n")
    text = open(bench.summarize_valu_counters(str(src), out_dir=str(out))).read()
    assert "`feed`" in text
    assert "**2.00 GHz**" in text
    assert "per wave-token: 64.0" in text and "FP32 FMA 48.0" in text
    # 64 VALU per wave-token x 3 waves per SIMD x 512 tokens = 98.3 k per SIMD,
    # 16 k quad-cycles issue two: 32.6% dual-issued
    assert "98.3 k VALU instructions in 100.0 k quad-cycles" in text
    assert "(33% of VALU instructions are dual-issued)" in text
    assert "11.00 GFLOP per call" in text
    for cmd in bench.VALU_PASSES:
        assert cmd in text


def test_stale_build_is_refused(bench, monkeypatch, tmp_path):
    """The bench times the library it loads: when the build stamp next to
    libgdn.so differs from the current sources (or is missing) it exits with
    status 3 before touching the GPU; a matching stamp is returned as the
    digest the line reports."""
    from linear_attention_recurrence_forward_amd import build
    monkeypatch.setattr(build, "LIBDIR", str(tmp_path))
    monkeypatch.setattr(build, "source_digest", lambda: "current-sources")
    with pytest.raises(SystemExit) as e:
        bench.check_build()  # no stamp at all
    assert e.value.code == 3
    (tmp_path / "libgdn.digest").write_text("older-sources\n")
    with pytest.raises(SystemExit) as e:
        bench.check_build()
    assert e.value.code == 3
    (tmp_path / "libgdn.digest").write_text("current-sources\n")
    assert bench.check_build() == "current-sources"


def test_host_cpu(bench):
    cpu = bench.host_cpu()
    assert cpu["nproc"] >= 1 and 1 <= cpu["threads"] <= bench.MAX_WORKER_THREADS
    assert cpu["threads"] <= cpu["usable"] and isinstance(cpu["model"], str)


def test_cpu_baseline_fields(bench):
    """Every CPU baseline names the CPU and carries a one-core and an all-core
    rate of the oracle in the workload's unit."""
    w = WORKLOADS["tiny"]
    cpu = bench.cpu_baseline(w, 0.2)
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s"
    assert cpu["single_core"]["cores"] == 1 and cpu["single_core"]["value"] > 0
    assert cpu["value"] > 0 and cpu["cores"] == min(bench.host_cpu()["threads"], 2)
    assert cpu["cpu_model"] and cpu["nproc"] >= 1
    rb = bench.cpu_baseline(WORKLOADS["spec_verify"].with_(n_seqs=2), 0.2, rollback=True)
    assert rb["unit"] == "GB/s" and rb["single_core"]["value"] > 0


def test_summarize_default_trace(bench, tmp_path):
    """The default bench line's kernel trace: per-kernel statistics, the
    profiled build's digest and the bench line's kernel times, read from a
    gzip-compressed trace."""
    import gzip
    src, out = tmp_path / "prof", tmp_path / "profiles"
    write_csv(str(src / "kt_default" / "run_kernel_stats.csv"),
              ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
              [["void gdn::gdn_decode<128>", 3, 3000.0, 2000.0, 4000.0, 60.0]])
    rows = [["void gdn::gdn_decode<128>", 0, d] for d in (2000, 3000, 4000)]
    with gzip.open(src / "kt_default" / "run_kernel_trace.csv.gz", "wt") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for r in rows:
            f.write(",".join(f'"{v}"' for v in r) + "\n")
    line = {"kernel_digest": "cafe", "kernel_us": 2.8,
            "prefill": {"kernel_us": 180.0}, "rollback": {"kernel_us": 2.9}}
    with open(src / "kt_default.log", "w") as f:
        f.write("bench: progress\n" + json.dumps(line) + "\n")
    text = open(bench.summarize_default_trace(str(src), "the-command", str(out))).read()
    assert "`cafe`" in text and "the-command" in text
    assert "| 3 | 3.00 | 3.00 | 2.00 | 60.0 |" in text
    assert "| decode | 2.800 |" in text and "| prefill | 180.000 |" in text


def test_state_copy_bytes(bench):
    """The decode call's floor: the rollback kernel on the decode shape moves
    the state once each way (and reads one index)."""
    w, kernel, alg, _ = bench.workload_info("state_copy")
    assert (w.d_k, w.d_v, w.n_v_heads, w.n_tokens, w.n_seqs) == (128, 128, 48, 1, 1)
    assert kernel == "gdn_rollback_kernel"
    assert alg == 2 * 4 * 128 * 128 * 48 + 4
