"""Host-side logic of bench.py, without a GPU: the one-GPU refusal, the HBM
traffic record built from rocprofv3 counter CSVs (calibration by a plain
copy of known size), and the record being dropped once the product kernels'
sources differ from the ones the counters were taken on."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
GEMM = "void fp8lin::gemm_detail::gemm_pp_kernel<true, true, 0, 0, 0, false>(fp8lin::GemmProblem, int, int)"
OTHER = "void fp8lin::(anonymous namespace)::amax_bf16_kernel<true>(HIP_vector_type<unsigned int, 4u> const*)"
COPY = "__amd_rocclr_copyBuffer"


def write_csv(d, sub, rows):
    os.makedirs(os.path.join(d, sub, "host"), exist_ok=True)
    with open(os.path.join(d, sub, "host", "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, FIELDS)
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i + 1, "Dispatch_Id": i + 1, "Kernel_Name": kernel,
                        "Grid_Size": 512 if kernel == GEMM else 256, "Counter_Name": counter,
                        "Counter_Value": value})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT)
    assert r.returncode != 0
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_traffic_record_from_counter_csvs(tmp_path):
    d = str(tmp_path)
    kib = 1024.0
    copy_kib = bench.COPY_BYTES / kib
    # the copy: FETCH_SIZE reads half the copied bytes, WRITE_SIZE all of them
    write_csv(d, "copy_fetch", [(COPY, "FETCH_SIZE", copy_kib / 2), (COPY, "FETCH_SIZE", 1.0)])
    write_csv(d, "copy_write", [(COPY, "WRITE_SIZE", copy_kib)])
    # three product dispatches after another kernel (ignored by the record);
    # the two runs are the same program, so their dispatch ids match
    write_csv(d, "fetch", [(OTHER, "FETCH_SIZE", 5e6), (GEMM, "FETCH_SIZE", 1000.0),
                           (GEMM, "FETCH_SIZE", 2000.0), (GEMM, "FETCH_SIZE", 3000.0)])
    write_csv(d, "write", [(OTHER, "WRITE_SIZE", 7.0), (GEMM, "WRITE_SIZE", 400.0),
                           (GEMM, "WRITE_SIZE", 800.0)])
    out = str(tmp_path / "traffic.json")
    bench.record_traffic(d, out=out)
    rec = json.load(open(out))
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    assert rec["launches_fetch"] == 3 and rec["launches_write"] == 2
    assert rec["fetch_bytes_per_launch"] == round(2000.0 * kib * 2.0)
    assert rec["write_bytes_per_launch"] == round(600.0 * kib)
    assert rec["bytes_per_launch"] == round(2000.0 * kib * 2.0 + 600.0 * kib)
    assert rec["source_sha256"] == bench.sources_sha(bench.GEMM_SOURCES)
    assert bench.traffic_record(rec["workload"], path=out)["bytes_per_launch"] == rec["bytes_per_launch"]
    # the per-kernel table beside it: the products one row each, in step order
    table = open(tmp_path / "quant_gemm_llama70b_infer_hbm_bytes.txt").read().splitlines()
    rows = {" ".join(l.split()[:-4]): l.split()[-4:] for l in table if l.startswith(("amax", "gemm"))}
    assert rows["amax_bf16_kernel<true>"] == ["256", "1", f"{5e6 * kib * 2.0 / 1e6:.1f}", f"{7.0 * kib / 1e6:.1f}"]
    assert rows["gemm_pp_kernel<true, true, 0, 0, 0, false> qkv"][2] == f"{1000.0 * kib * 2.0 / 1e6:.1f}"
    assert rows["gemm_pp_kernel<true, true, 0, 0, 0, false> o"][3] == f"{800.0 * kib / 1e6:.1f}"
    assert rows["gemm_pp_kernel<true, true, 0, 0, 0, false> gate"][2] == f"{3000.0 * kib * 2.0 / 1e6:.1f}"
    # another workload, or other kernel sources: no record
    assert bench.traffic_record("another-workload", path=out) is None
    rec["source_sha256"] = "0" * 64
    json.dump(rec, open(out, "w"))
    assert bench.traffic_record(rec["workload"], path=out) is None



def test_parity_of_the_step_against_the_oracle_sample(orc):
    """bench.parity on workload 1 (full outputs): outputs equal to the
    oracle's pass; a code, a bias or a product output outside the tolerance
    is reported.  The 'GPU' side here is the oracle's own results on the host."""
    import numpy as np
    import torch

    import synth
    w = synth.WORKLOADS[1]
    host = {t.name: synth.workload_tensor(w, t.name) for t in w.tensors}
    res = {}
    line = bench.cpu_baseline(w, host, 1 << 31, 1 << 31, results=res)
    assert line["gemm_extrapolated"] is False
    q, outs = {}, {}
    for t in w.tensors:
        if t.name in res["quant"]:
            a, b, c = res["quant"][t.name]
            amax = torch.tensor([a], dtype=torch.int64).to(torch.int32).view(torch.float32)
            q[t.name] = (torch.from_numpy(np.array(c).reshape(t.shape)), torch.tensor([b], dtype=torch.int32),
                         amax, t.fmt)
    for key, (ref, bound) in res["gemm"].items():
        outs[key] = torch.from_numpy(ref.astype(np.float32))
    p = bench.parity(None, w, q, outs, res)
    assert p["quantisation_bit_exact"] and p["gemm_within_tolerance"], p
    assert p["gemm_outputs_checked"] == 128 * 256 and p["gemm_worst_err_over_sum_ab"] < 1e-6
    # one output off by twice the tolerance
    key = next(iter(outs))
    ref, bound = res["gemm"][key]
    outs[key][3, 5] = float(ref[3, 5] + 2e-5 * bound[3, 5])
    assert bench.parity(None, w, q, outs, res)["gemm_within_tolerance"] is False
    outs[key][3, 5] = float(ref[3, 5])
    # one code changed
    name = next(iter(q))
    q[name][0].view(-1)[7] ^= 1
    assert bench.parity(None, w, q, outs, res)["quantisation_bit_exact"] is False
