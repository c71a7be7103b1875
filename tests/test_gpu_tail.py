"""GPU parity of decode with an exact tail of tokens appended after the
one-shot compression (AnchorKV-adapted page, "Adaptation notes") against the
CPU oracle.

The compressed part is the oracle's own representation packed on the host
into the cache layout, so only decode is under test.  Tail keys, values and
the decode queries are seeded synthetic draws in the cache dtype.
"""
import sys

import numpy as np
import pytest
import torch

import kvsynth
from oracle import anchorkv_oracle as O
from tests.parity import oracle_arrays, oracle_params
from tests.test_gpu_parity import SMALL, make_inputs, plan_for

pytestmark = pytest.mark.gpu

W_ = kvsynth.WORKLOADS
CASES = {
    "bf16_ragged": SMALL["bf16_ragged"],
    "f32_tiny": SMALL["f32_tiny"],
    "bf16_8b_short": SMALL["bf16_8b_short"],
    # eight q-heads per KV head (one 8-wave workgroup per CU in the stream kernel)
    "bf16_g8": W_["llama70b_128k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=3000, n_dirs=16),
    # the paper's codec (Hadamard rotation + Lloyd-Max), 8 q-heads, two units
    "bf16_hlm_g8": W_["llama70b_128k"].scaled(seqs=1, layers=2, kv_heads=2, n_tokens=2500, n_dirs=16),
    # keys stored before the rotary embedding (the tail's keys are given rotated)
    "bf16_rope_g8": W_["llama70b_128k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=3000, n_obs=16, n_dirs=16),
    "f32_rope": W_["tiny_f32"].scaled(n_tokens=1300),
}
PARAMS = {"bf16_hlm_g8": dict(codec=1), "bf16_rope_g8": dict(rope=1), "f32_rope": dict(rope=1, rope_theta=10000.0)}
TAILS = [0, 1, 37, 300, 600]


def _flush(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def akv():
    import kv_cache_compression_snapkv_amd as m
    m.lib()
    return m


def packed_oracle_cache(akv, w, p, params=None):
    K, V, Q = make_inputs(w)
    K64, V64, Q64 = (kvsynth.to_f64(t) for t in (K, V, Q))
    code = 1 if w.dtype == "bf16" else 2
    cache_h = np.zeros(p.cache_bytes, dtype=np.uint8)
    comps = []
    for u in range(w.units):
        c = O.compress_unit(K64[u], V64[u], Q64[u], w.q_per_kv, w.n_obs, w.theta, w.window, w.elem_bytes,
                            **oracle_params(params))
        comps.append(c)
        cache_h[u * p.unit_stride: u * p.unit_stride + p.unit_bytes] = np.frombuffer(
            akv.pack_unit(p, oracle_arrays(c, code)), np.uint8)
    return torch.from_numpy(cache_h).cuda(), comps


def tail_inputs(w, cap, seed):
    g = torch.Generator().manual_seed(seed)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    shape = (w.units, w.kv_heads, cap, w.head_dim)
    Kt = torch.randn(shape, generator=g).to(dt)
    Vt = torch.randn(shape, generator=g).to(dt)
    return Kt, Vt


@pytest.mark.parametrize("name", list(CASES))
def test_decode_tail_parity(akv, name):
    w = CASES[name]
    _flush(f"[tail] {name}: U={w.units} H={w.kv_heads} G={w.q_per_kv} N={w.n_tokens} dtype={w.dtype}")
    prm = PARAMS.get(name, {})
    p = plan_for(akv, w, prm)
    cache, comps = packed_oracle_cache(akv, w, p, prm)
    _, _, dws = akv.alloc(p, "cuda")
    q = kvsynth.decode_queries(w, 0, device="cuda").contiguous()
    q64 = kvsynth.to_f64(q)
    cap = max(TAILS) + 5
    Kt, Vt = tail_inputs(w, cap, 0xA7C4 + len(name))
    # rows past n_tail hold NaN: they must never be read
    Kt_d, Vt_d = Kt.clone(), Vt.clone()
    o_plain = torch.empty(w.units, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.float32, device="cuda")
    akv.decode_attn(p, cache, q, o_plain, dws)
    for n in TAILS:
        Kt_d[:, :, n:] = float("nan")
        Vt_d[:, :, n:] = float("nan")
        Kt_d[:, :, :n] = Kt[:, :, :n]
        Vt_d[:, :, :n] = Vt[:, :, :n]
        Kg, Vg = Kt_d.cuda().contiguous(), Vt_d.cuda().contiguous()
        o = torch.empty_like(o_plain)
        akv.decode_attn_tail(p, cache, q, Kg, Vg, n, o, dws)
        torch.cuda.synchronize()
        o_h = o.cpu().numpy().astype(np.float64)
        if n == 0:   # the same launches as decode_attn
            assert torch.allclose(o, o_plain, rtol=1e-5, atol=1e-6), "empty tail must reproduce decode_attn"
        worst = 0.0
        K64t, V64t = kvsynth.to_f64(Kt[:, :, :n]), kvsynth.to_f64(Vt[:, :, :n])
        for u in range(w.units):
            ref = O.decode_unit_tail(comps[u], q64[u], K64t[u], V64t[u])
            err = np.linalg.norm(o_h[u] - ref, axis=1) / np.linalg.norm(ref, axis=1)
            worst = max(worst, float(err.max()))
        _flush(f"[tail] {name} n_tail={n}: max rel err {worst:.3g}")
        assert np.isfinite(o_h).all() and worst <= 1e-3, (n, worst)


def test_decode_argument_errors(akv):
    w = CASES["bf16_ragged"]
    p = plan_for(akv, w)
    cache, _, dws = akv.alloc(p, "cuda")
    q = torch.zeros(w.units, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.bfloat16, device="cuda")
    o = torch.empty(w.units, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.float32, device="cuda")
    Kt = torch.zeros(w.units, w.kv_heads, 4, w.head_dim, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(akv.AnchorKVError):
        akv.decode_attn_tail(p, cache, q, Kt, Kt, 5, o, dws)   # n_tail > tail_cap
    with pytest.raises(akv.AnchorKVError):
        akv.decode_attn_tail(p, cache, q, Kt, Kt, -1, o, dws)
    # shapes / dtypes that the kernels would index past: refused before any launch
    with pytest.raises(ValueError):
        akv.decode_attn_tail(p, cache, q[:, :1].contiguous(), Kt, Kt, 2, o, dws)
    with pytest.raises(ValueError):
        akv.decode_attn_tail(p, cache, q, Kt[:, :1].contiguous(), Kt[:, :1].contiguous(), 2, o, dws)
    with pytest.raises(ValueError):
        akv.decode_attn(p, cache, q.float(), o, dws)
    with pytest.raises(ValueError):
        akv.decode_attn(p, cache, q, o[:, :1].contiguous(), dws)
