"""GPU parity of the HIP compress / decode path against the CPU oracle.

Inputs are seeded synthetic workloads (kvsynth) generated on the GPU and
copied to the host for the oracle.  Sizes are chosen so the oracle finishes
in seconds while spanning several tiles and ragged tails.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import kvsynth
from oracle import anchorkv_oracle as O
from tests.parity import compare_unit, oracle_arrays

pytestmark = pytest.mark.gpu

W_ = kvsynth.WORKLOADS
SMALL = {
    # several 64/256/1024-token tiles and a ragged tail
    "bf16_ragged": W_["llama3b_8k"].scaled(seqs=1, layers=2, kv_heads=2, n_tokens=2000, n_obs=16, window=16,
                                          n_dirs=16, lognormal=True),
    # the tiny f32 workload at full size
    "f32_tiny": W_["tiny_f32"],
    # 8B-shaped heads, shorter context
    "bf16_8b_short": W_["llama8b_32k"].scaled(seqs=1, layers=1, n_tokens=4096),
    # stress features (outlier channels, isotropic tokens, Student-t values), shorter context
    "bf16_stress_short": W_["stress_64k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=3000, theta=0.05),
    # more observation queries than window tokens: causal mask reaches non-window keys
    "bf16_obs_gt_window": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=2, q_per_kv=2, n_tokens=1500,
                                                 n_obs=40, window=8, theta=0.15, n_dirs=8),
    # every token an anchor: decode is exact attention
    "bf16_all_anchors": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=2, q_per_kv=2, n_tokens=256, n_obs=8,
                                               window=256, theta=1.5, n_dirs=8),
    # more anchors than one LDS part (512): the assignment walks two parts
    "bf16_multi_part": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=2, q_per_kv=2, n_tokens=2048, n_obs=16,
                                              window=600, theta=0.5, n_dirs=8),
    # kv_heads * n_tokens > 65536: top-R streams the utilities instead of holding them in registers
    "bf16_long_topr": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=3, q_per_kv=2, n_tokens=22000, n_obs=16,
                                             window=32, theta=0.1, n_dirs=16),
    # 151..300 residual records per 1024-token tile: the decode's middle staging size
    "bf16_mid_staging": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=3000, n_obs=16, theta=0.07,
                                               n_dirs=16),
    # budget leaves no residual slots
    "bf16_no_residuals": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=1, q_per_kv=2, n_tokens=256, n_obs=8,
                                                window=32, theta=0.144, n_dirs=8),
}


def _flush(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make_inputs(w, device="cuda"):
    Ks, Vs, Qs = [], [], []
    for u in range(w.units):
        s, l = kvsynth.unit_index(w, u)
        K, V, Q = kvsynth.unit_inputs(w, s, l, device=device)
        Ks.append(K); Vs.append(V); Qs.append(Q)
    return torch.stack(Ks).contiguous(), torch.stack(Vs).contiguous(), torch.stack(Qs).contiguous()


def plan_for(akv, w):
    return akv.plan(w.units, w.kv_heads, w.q_per_kv, w.n_tokens, w.head_dim, w.n_obs,
                    akv.BF16 if w.dtype == "bf16" else akv.F32, w.theta, w.window)


def ws_view(ws, off, count, dtype=torch.float32):
    nbytes = count * torch.empty(0, dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype)


@pytest.fixture(scope="module")
def akv():
    import kv_cache_compression_snapkv_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("name", list(SMALL))
def test_compress_decode_parity(akv, name):
    w = SMALL[name]
    _flush(f"[parity] {name}: U={w.units} H={w.kv_heads} G={w.q_per_kv} N={w.n_tokens} dtype={w.dtype}")
    K, V, Q = make_inputs(w)
    p = plan_for(akv, w)
    cache, ws, dws = akv.alloc(p, "cuda")
    akv.compress(p, K, V, Q, cache, ws)
    q = kvsynth.decode_queries(w, 0, device="cuda").contiguous()
    o = torch.empty(w.units, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.float32, device="cuda")
    akv.decode_attn(p, cache, q, o, dws)
    torch.cuda.synchronize()
    offs = akv.workspace_offsets(p)
    U, H, N = w.units, w.kv_heads, w.n_tokens
    score = ws_view(ws, offs["score"], U * H * N).reshape(U, H, N).cpu().numpy().astype(np.float64)
    util = ws_view(ws, offs["util"], U * 2 * H * N).reshape(U, 2, H, N).cpu().numpy().astype(np.float64)
    cache_h = cache.cpu().numpy()
    K64, V64, Q64 = (kvsynth.to_f64(t) for t in (K, V, Q))
    q64, o_h = kvsynth.to_f64(q), o.cpu().numpy().astype(np.float64)
    for u in range(U):
        unit = cache_h[u * p.unit_stride: u * p.unit_stride + p.unit_bytes].tobytes()
        arr = akv.unpack_unit(p, unit)
        rep = compare_unit(K64[u], V64[u], Q64[u], w.q_per_kv, w.n_obs, w.theta, w.window, w.elem_bytes, arr,
                           taps=dict(score=score[u], util=util[u]), q=q64[u], o_gpu=o_h[u])
        _flush(f"[parity] {name} unit {u}: {rep}")


@pytest.mark.parametrize("name", ["bf16_ragged", "f32_tiny", "bf16_stress_short"])
def test_decode_on_host_packed_oracle_cache(akv, name):
    """Decode alone: the oracle's compressed representation, packed on the
    host into the cache layout, decoded on the GPU."""
    w = SMALL[name]
    _flush(f"[decode-packed] {name}")
    K, V, Q = make_inputs(w)
    p = plan_for(akv, w)
    K64, V64, Q64 = (kvsynth.to_f64(t) for t in (K, V, Q))
    dtype_code = 1 if w.dtype == "bf16" else 2
    cache_h = np.zeros(p.cache_bytes, dtype=np.uint8)
    comps = []
    for u in range(w.units):
        c = O.compress_unit(K64[u], V64[u], Q64[u], w.q_per_kv, w.n_obs, w.theta, w.window, w.elem_bytes)
        comps.append(c)
        unit = akv.pack_unit(p, oracle_arrays(c, dtype_code))
        cache_h[u * p.unit_stride: u * p.unit_stride + p.unit_bytes] = np.frombuffer(unit, np.uint8)
    cache = torch.from_numpy(cache_h).cuda()
    _, _, dws = akv.alloc(p, "cuda")
    for step in range(3):
        q = kvsynth.decode_queries(w, step, device="cuda").contiguous()
        o = torch.empty(w.units, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.float32, device="cuda")
        akv.decode_attn(p, cache, q, o, dws)
        torch.cuda.synchronize()
        q64, o_h = kvsynth.to_f64(q), o.cpu().numpy().astype(np.float64)
        for u in range(w.units):
            ref = O.decode_unit(comps[u], q64[u])
            err = np.linalg.norm(o_h[u] - ref, axis=1) / np.linalg.norm(ref, axis=1)
            assert err.max() <= 1e-3, (step, u, err.max())
    _flush(f"[decode-packed] {name}: ok")


def test_compress_is_deterministic_and_header_roundtrips(akv):
    w = SMALL["bf16_8b_short"]
    _flush("[determinism] bf16_8b_short")
    K, V, Q = make_inputs(w)
    p = plan_for(akv, w)
    c1, ws, _ = akv.alloc(p, "cuda")
    c2 = torch.empty_like(c1)
    akv.compress(p, K, V, Q, c1, ws)
    ws.fill_(0xAB)
    akv.compress(p, K, V, Q, c2, ws)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    hdr = c1[:256].cpu().numpy().tobytes()
    p2 = akv.plan_from_header(hdr, w.units)
    assert p2.as_dict() == p.as_dict()
