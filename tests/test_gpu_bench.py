"""bench.py's JSON line on the GPU, run in this process on the 64^3 config with
few steps: every field of the contract is present, typed and consistent (the
roofline fraction is achieved / peak, the CPU baseline is the oracle's)."""
import json
import os
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_contract(capsys, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--config", "S", "--steps", "3", "--warmup", "1",
                                      "--no-variants", "--no-chain", "--also", "T", "--cpu-seconds", "0.2",
                                      "--gemm-reps", "3"])
    bench.main()
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key, typ in [("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict),
                     ("cpu_baseline", dict)]:
        assert isinstance(d[key], typ), key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["data"] == "synthetic"
    assert isinstance(d["config"]["workload"], str)
    r = d["roofline"]
    assert r["bound"] in ("hbm", "mfma", "alu") and r["unit"] in ("GB/s", "TFLOP/s")
    assert r["achieved"] > 0 and r["peak"] > 0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert r["traffic"] is None or r["traffic"] > 0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
    assert isinstance(c["unit"], str) and isinstance(c["sample"], str) and isinstance(c["cpu_model"], str)
    # every config measured the same way: phases, steady forward, effective TFLOP/s and its fraction
    assert set(d["configs"]) == {"S", "T"}
    for name, rec in d["configs"].items():
        assert rec["effective_tflops"] > 0 and rec["voxels_per_s_forward"] > 0
        assert abs(rec["frac_peak"] - rec["effective_tflops"] / rec["peak_tflops"]) < 1e-9
        for conv in ("block_table", "per_voxel_table"):
            assert rec["hash_map_hbm"][conv]["gbs"] > 0
    assert d["configs"]["T"]["peak_tflops"] == 157.3 and d["configs"]["S"]["peak_tflops"] == 2500.0
    ce = d["ceilings"]
    assert 0.5 < ce["mfma_bf16_tflops"]["frac_of_spec"] < 1.05
    assert 0.2 < ce["hbm_gbs"]["frac_of_spec"] < 1.05
    assert abs(r["frac_of_measured_peak"] * r["measured_peak"] - r["achieved"]) < 1e-6 * r["achieved"]
