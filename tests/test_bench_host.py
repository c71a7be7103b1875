"""Host logic of the benchmark (no GPU): which stage a kernel belongs to, and
how counter folders become per-call HBM bytes."""
import csv
import json
import os

import bench


def test_kernel_stage_names():
    ks = bench.kernel_stage
    assert ks("void akv::k_obs_pipe<2, 1, 64, 2, 2, 3, true>(akv::ObsArgs)") == "obs_util"
    assert ks("void akv::k_obs_pipe<0, 1, 64, 2, 1, 2, false>(akv::ObsArgs)") == "obs_stats"
    assert ks("void akv::k_obs<2, 1, 1>(akv::ObsArgs)") == "obs_score"
    assert ks("void akv::k_assign_res<false, 8>(akv::AssignArgs)") == "assign"
    assert ks("void akv::k_dec_stream<1, 3, 3, 1, 4>(akv::DecArgs)") == "dec_stream"
    assert ks("akv::k_dec_merge(HIP_vector_type<float, 2u> const*, float const*)") == "dec_stream"
    assert ks("akv::k_dec_tail_bf16(void const*)") == "dec_tail"
    assert ks("__amd_rocclr_copyBuffer") is None


def _write(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for n, v in rows:
            w.writerow([n, counter, v])


def test_traffic_summary_counts_one_decode_call_per_stream_dispatch(tmp_path):
    """Two calls (warm-up + step): every compress stage once per call, the
    decode as stream + merge per call.  Counters in KiB; the copy probe reads
    half its bytes on FETCH_SIZE, so fetches scale by 2."""
    hdr = "void akv::k_headers(akv::UnitHeader)"
    util = "void akv::k_obs_pipe<2, 1, 64, 2, 2, 3, true>(akv::ObsArgs)"
    dec = "void akv::k_dec_stream<1, 3, 3, 1, 4>(akv::DecArgs)"
    mrg = "akv::k_dec_merge(HIP_vector_type<float, 2u> const*)"
    call = [(hdr, 1.0), (util, 1000.0), (dec, 100.0), (mrg, 10.0)]
    _write(str(tmp_path / "f"), "FETCH_SIZE", call * 2)
    _write(str(tmp_path / "w"), "WRITE_SIZE", [(n, v / 10) for n, v in call] * 2)
    copy = "__amd_rocclr_copyBuffer"
    _write(str(tmp_path / "cf"), "FETCH_SIZE", [(copy, bench.COPY_PROBE_BYTES / 1024 / 2)])
    _write(str(tmp_path / "cw"), "WRITE_SIZE", [(copy, bench.COPY_PROBE_BYTES / 1024)])
    out = str(tmp_path / "t.json")
    bench.traffic_summary("x", str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                          [], path=out)
    st = json.load(open(out))["stages"]
    assert st["obs_util"]["fetch_bytes"] == 2 * 1000.0 * 1024   # per call, fetch scale 2
    assert st["obs_util"]["write_bytes"] == 100.0 * 1024
    assert st["dec_stream"]["fetch_bytes"] == 2 * 110.0 * 1024  # stream + merge of one call
    assert st["dec_stream"]["dispatches_per_call"] == 2.0
