"""Host logic of bench.py (no GPU): the one-GPU guard, and the HBM-traffic
ingest that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings (KiB per
dispatch) by what the same counters read for a plain copy of known size."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                       # no JSON line


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, name, vals in rows:
            for v in vals:                      # one row per XCD / instance, summed by the ingest
                w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_ingest_scales_by_the_copy_probe(tmp_path):
    gib_kib = bench.COPY_PROBE_BYTES / 1024.0
    q = "void rptq::(anonymous namespace)::qgemm_kernel<4, 4, false, TileCfg<128, 128, 4, 4, 2> >(...)"
    ln = "void rptq::(anonymous namespace)::ln_reorder_quant_kernel<4, 0, 5, 0>(...)"
    kv = "void rptq::(anonymous namespace)::kv_quant_pack_kernel<3, 3, true>(...)"
    cp = "__amd_rocclr_copyBuffer"
    # the counters read half of the copy's true bytes (fetch) and exactly them (write)
    fetch = [(1, ln, [10.0, 20.0]), (2, q, [100.0]), (3, q, [200.0]), (4, q, [300.0]), (5, q, [400.0]),
             (6, kv, [50.0]), (7, kv, [70.0]), (8, cp, [gib_kib / 4, gib_kib / 4])]
    write = [(1, ln, [3.0]), (2, q, [7.0]), (3, q, [8.0]), (4, q, [9.0]), (5, q, [10.0]),
             (6, kv, [5.0]), (7, kv, [5.0]), (8, cp, [gib_kib])]
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f, "FETCH_SIZE", fetch)
    _counter_csv(w, "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    res = bench.ingest_pmc(str(f), str(w), out_path=str(out))
    assert json.load(open(out)) == json.loads(json.dumps(res))
    assert res["qgemm"]["scale_fetch"] == pytest.approx(2.0) and res["qgemm"]["scale_write"] == pytest.approx(1.0)
    # qgemm takes the third-from-last W4A4 dispatch, the quantized-output one the second-from-last
    assert res["qgemm"]["fetch_bytes"] == pytest.approx(200.0 * 1024 * 2)
    assert res["qgemm"]["write_bytes"] == pytest.approx(8.0 * 1024)
    assert res["qgemm_quant_out"]["fetch_bytes"] == pytest.approx(300.0 * 1024 * 2)
    # per-instance rows of one dispatch are summed; the last matching dispatch is taken
    assert res["ln_reorder_quant"]["fetch_bytes"] == pytest.approx(30.0 * 1024 * 2)
    assert res["ln_reorder_quant"]["bytes_per_launch"] == pytest.approx(30.0 * 1024 * 2 + 3.0 * 1024)
    # KV pack: the mean over its dispatches
    assert res["kv_quant_pack"]["fetch_bytes"] == pytest.approx(60.0 * 1024 * 2)
    # a result is valid only for the source it was taken on
    assert bench.measured_traffic("qgemm", 0.0, path=str(out)) == pytest.approx(res["qgemm"]["bytes_per_launch"])
    stale = dict(res)
    stale["qgemm"] = dict(res["qgemm"], source_hash="0" * 16)
    json.dump(stale, open(out, "w"))
    assert bench.measured_traffic("qgemm", 0.0, path=str(out)) is None


def test_ingest_needs_the_copy_probe(tmp_path):
    q = "qgemm_kernel<4, 4, false, TileCfg<128, 128, 4, 4, 2> >"
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(f, "FETCH_SIZE", [(1, q, [1.0])])
    _counter_csv(w, "WRITE_SIZE", [(1, q, [1.0])])
    with pytest.raises(SystemExit, match="copy"):
        bench.ingest_pmc(str(f), str(w), out_path=str(tmp_path / "t.json"))
