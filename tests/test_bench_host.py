"""Host-side arithmetic of bench.py (no GPU): useful FLOPs, algorithmic GEMM bytes, the MXFP8
step's per-GEMM work table, and the reading of the committed counter summary."""
import json
import os

import numpy as np
import pytest

import bench
import moe_inputs as mi


def test_useful_flops_dsv3():
    w = mi.WORKLOADS["dsv3"]
    # 2 m d 2f (gate/up) + 2 m f d (down) per routed row, the same for the shared rows
    want = 6.0 * w.T * w.k * w.d * w.f + 6.0 * w.T * w.d * w.shared_f
    assert bench.useful_flops(w, None) == want
    assert abs(want - 6.494e12) / 6.494e12 < 1e-3          # 5.772 routed + 0.722 shared TFLOP


def test_useful_flops_no_shared():
    w = mi.WORKLOADS["mixtral"]
    assert bench.useful_flops(w, None) == 6.0 * w.T * w.k * w.d * w.f


def test_gemm1_bytes_counts_each_operand_once():
    w = mi.WORKLOADS["dsv3"]
    counts = np.ones(w.E, dtype=np.int64)
    counts[:10] = 0                                        # empty groups fetch no weights
    rows = w.T * w.k + w.T
    fused = bench.gemm1_bytes(w, counts, True)
    mat = bench.gemm1_bytes(w, counts, False)
    wbytes = (w.E - 10) * 2 * w.f * w.d * 2 + 2 * w.shared_f * w.d * 2   # + the shared expert's gate/up
    assert fused == wbytes + w.T * w.d * 2 + rows * w.f * 2 + rows * 4
    assert mat - fused == rows * w.d * 2 - w.T * w.d * 2   # x_perm instead of x


def test_mx_gemm_work_flops_sum_to_step():
    w = mi.WORKLOADS["dsv3_mxfp8"]
    rows = w.T * w.k + w.T
    work = bench.mx_gemm_work(w, rows, w.E + 1)
    total = sum(fl for _, fl in work.values())
    assert total == pytest.approx(18.0 * rows * w.d * w.f, rel=1e-12)
    # weight-gradient outputs: every group's full dW in bf16
    G = w.E + 1
    assert work["wgrad1"][0] >= G * 2 * w.f * w.d * 2
    assert work["wgrad2"][0] >= G * w.f * w.d * 2


def test_pmc_traffic_follows_source_hash(tmp_path, monkeypatch):
    # the committed summary is used only while the GEMM sources hash to its recorded value
    path = os.path.join(bench.ROOT, "profiles", "gemm1_swiglu_dsv3_pmc.md")
    if not os.path.exists(path):
        pytest.skip("no committed counter summary")
    got = bench.pmc_traffic("dsv3")
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") == bench.gemm_source_digest():
        assert got == int(fields["traffic_bytes_per_launch"])
    else:
        assert got is None
    monkeypatch.setattr(bench, "gemm_source_digest", lambda: "0" * 64)
    assert bench.pmc_traffic("dsv3") is None
    assert bench.pmc_traffic("no_such_workload") is None


def test_gpus_above_one_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().out


@pytest.mark.parametrize("name", ["dsv3_ep8", "mixtral", "qwen3"])
def test_held_workloads_refused(monkeypatch, capsys, name):
    monkeypatch.setattr("sys.argv", ["bench.py", "--workload", name])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 3
    assert "held" in json.loads(capsys.readouterr().out.strip())["error"]


def test_spread_and_host_info():
    sp = bench.spread([1.0, 2.0, 3.0, 4.0, 5.0])
    assert sp["median"] == 3.0 and sp["p10"] == pytest.approx(1.4) and sp["p90"] == pytest.approx(4.6)
    info = bench.host_info()
    assert set(info) == {"cpu_model", "blas", "cpus_available"}
    assert info["cpus_available"] >= 1
