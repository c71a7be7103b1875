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


def test_stage_work_and_roofline_by_hand():
    """Algorithmic work of the assignment at the 8B shape, worked by hand, and
    the roofline choosing the bound with the longer time at peak."""
    import kv_cache_compression_snapkv_amd as akv
    import kvsynth
    w = kvsynth.WORKLOADS["llama8b_32k"]
    p = akv.plan(w.units, w.kv_heads, w.q_per_kv, w.n_tokens, w.head_dim, w.n_obs, akv.BF16, w.theta, w.window)
    flops, byts = bench.stage_work(p, "assign")
    assert flops == 512 * 8 * 2 * 2.0 * 32768 * p.A * 128          # 2 sides x 2 N A D per head
    x = 512 * 8 * 32768 * 128 * 2                                  # one side's inputs
    assert byts == 2 * x + 2 * 512 * 8 * p.A * 128 * 2 + 512 * 2 * 8 * 32768 * 4
    # A = 288 flop per byte of input is below the ridge (2.5e15 / 8e12 = 312.5):
    # HBM time at peak is the longer one
    r = bench.roofline(p, "assign", 20.0)                          # 20 ms
    assert r["bound"] == "hbm" and abs(r["frac"] - byts / 20e-3 / 8e12) < 1e-12
    w70 = kvsynth.WORKLOADS["llama70b_128k"]                        # A = 1056: above the ridge
    p70 = akv.plan(w70.units, w70.kv_heads, w70.q_per_kv, w70.n_tokens, w70.head_dim, w70.n_obs, akv.BF16,
                   w70.theta, w70.window)
    f70 = bench.stage_work(p70, "assign")[0]
    r = bench.roofline(p70, "assign", 50.0)
    assert r["bound"] == "mfma" and abs(r["frac"] - f70 / 50e-3 / 2.5e15) < 1e-12
    r = bench.roofline(p, "obs_stats", 10.0)                       # Q K^T only: HBM-bound
    assert r["bound"] == "hbm"
    assert abs(r["achieved"] - bench.stage_work(p, "obs_stats")[1] / 10e-3 / 1e9) < 1e-6
