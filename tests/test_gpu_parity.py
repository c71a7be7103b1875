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
from tests.parity import compare_unit, oracle_arrays, oracle_params

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
    # the method's fixed parameters away from the pages' values: pooling width
    # 5, half the non-window anchors scored, k = N/64
    "bf16_params": W_["llama8b_32k"].scaled(seqs=1, layers=2, kv_heads=2, n_tokens=4000, n_dirs=32),
    "f32_params": W_["tiny_f32"].scaled(n_tokens=1200),
    # one ranking of key and value token-sides under both budgets together
    "bf16_joint": W_["llama8b_32k"].scaled(seqs=1, layers=2, kv_heads=2, n_tokens=3000, n_dirs=32),
    "bf16_joint_stress": W_["stress_64k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=3000, theta=0.06),
    "f32_joint": W_["tiny_f32"],
    # the paper's residual codec (Hadamard rotation + Lloyd-Max codebook)
    "bf16_hlm": W_["llama8b_32k"].scaled(seqs=1, layers=2, kv_heads=2, n_tokens=3000, n_dirs=32),
    "bf16_hlm_g8": W_["llama70b_128k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=4500, theta=0.08),
    "bf16_hlm_stress": W_["stress_64k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=3000, theta=0.05),
    "f32_hlm": W_["tiny_f32"].scaled(n_tokens=1500),
    "bf16_hlm_joint": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=2500, n_obs=16, window=16),
    # other query-group sizes through the whole path
    "bf16_g6": W_["llama8b_32k"].scaled(seqs=1, layers=1, kv_heads=2, q_per_kv=6, n_tokens=2800, n_dirs=16),
    "f32_g3": W_["tiny_f32"].scaled(kv_heads=2, q_per_kv=3, n_tokens=1400),
    # four anchors per head: many tokens have a negative cosine with every
    # anchor, and the anchors fill a quarter of one 16-anchor block
    "bf16_few_anchors": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=2, q_per_kv=2, n_tokens=700, n_obs=4,
                                               window=2, n_dirs=8),
    # 529 anchors: a second part of 17 (one block with a single anchor)
    "bf16_a529": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=2, q_per_kv=2, n_tokens=2048, n_obs=16,
                                        window=513, theta=0.5, n_dirs=8),
    # 1040 anchors: three parts, the last one a single block
    "bf16_a1040": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=2, q_per_kv=2, n_tokens=3000, n_obs=16,
                                         window=1017, theta=0.5, n_dirs=8),
    # coverage-optimised anchors (furthest-point picks in batched rounds)
    "bf16_cover": W_["llama8b_32k"].scaled(seqs=1, layers=2, kv_heads=2, n_tokens=3000, n_dirs=32),
    "f32_cover": W_["tiny_f32"].scaled(n_tokens=1500),
    "bf16_cover_fps": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=2, q_per_kv=2, n_tokens=2500, n_obs=16,
                                             window=16, n_dirs=8),
    "bf16_cover_g8": W_["llama70b_128k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=4500, theta=0.08),
    # keys stored before the rotary embedding, rotated wherever they meet a query
    "bf16_rope": W_["llama8b_32k"].scaled(seqs=1, layers=2, kv_heads=2, n_tokens=3000, n_dirs=32),
    "bf16_rope_base1e4": W_["llama3b_8k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=2500, n_dirs=16),
    "f32_rope": W_["tiny_f32"].scaled(n_tokens=1500),
    "bf16_rope_g8": W_["llama70b_128k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=4500, n_obs=16, theta=0.08),
    "bf16_rope_joint": W_["llama8b_32k"].scaled(seqs=1, layers=1, kv_heads=2, n_tokens=3000, n_dirs=32),
    # more than 128 observation queries per KV head: two query groups per key range whose score
    # and key-utility partials are added (the 70B shape's 8 x 32; 6 x 32 leaves the second
    # group half empty)
    "bf16_rope_q256": W_["llama70b_128k"].scaled(seqs=1, layers=2, kv_heads=2, n_tokens=4500, theta=0.08),
    "bf16_rope_q192": W_["llama8b_32k"].scaled(seqs=1, layers=1, kv_heads=2, q_per_kv=6, n_tokens=3300,
                                               n_dirs=32),
    # one 8B-shaped head at its full 32K tokens: 32 chunks of phase recurrence per decode range
    "bf16_rope_long": W_["llama8b_32k"].scaled(seqs=1, layers=1, kv_heads=1),
    # pre-RoPE decode with a large [q-head][anchor] weight table (8 x 865, 55 KB of LDS) and, past
    # the table's limit, the decode that rebuilds every value row (8 x 1462 anchors)
    "bf16_rope_wide": W_["llama70b_128k"].scaled(seqs=1, layers=1, kv_heads=1, n_tokens=5000, n_obs=16, n_dirs=16,
                                                 theta=0.25),
    "bf16_rope_bigA": W_["llama70b_128k"].scaled(seqs=1, layers=1, kv_heads=1, n_tokens=8000, n_obs=16, n_dirs=16,
                                                 theta=0.2),
}
# non-default method parameters of some cases (anchorkv_params)
PARAMS = {"bf16_params": dict(pool=5, rho=0.5, anchor_div=64), "f32_params": dict(pool=3, rho=0.9, anchor_div=40),
          "bf16_joint": dict(pool_kv_jointly=1), "bf16_joint_stress": dict(pool_kv_jointly=1),
          "f32_joint": dict(pool_kv_jointly=1),
          "bf16_hlm": dict(codec=1), "bf16_hlm_g8": dict(codec=1), "bf16_hlm_stress": dict(codec=1),
          "f32_hlm": dict(codec=1), "bf16_hlm_joint": dict(codec=1, pool_kv_jointly=1),
          "bf16_few_anchors": dict(anchor_div=300),
          "bf16_cover": dict(anchor_mode=1, cover_rounds=4), "f32_cover": dict(anchor_mode=1, cover_rounds=3),
          # one pick per round: plain furthest-point sampling
          "bf16_cover_fps": dict(anchor_mode=1, cover_rounds=1024, anchor_div=100),
          "bf16_cover_g8": dict(anchor_mode=1),
          "bf16_rope": dict(rope=1), "bf16_rope_base1e4": dict(rope=1, rope_theta=10000.0),
          "f32_rope": dict(rope=1, rope_theta=10000.0), "bf16_rope_g8": dict(rope=1),
          "bf16_rope_joint": dict(rope=1, pool_kv_jointly=1), "bf16_rope_q256": dict(rope=1),
          "bf16_rope_q192": dict(rope=1, rope_theta=10000.0), "bf16_rope_long": dict(rope=1, rope_theta=10000.0),
          "bf16_rope_wide": dict(rope=1, anchor_div=6), "bf16_rope_bigA": dict(rope=1, anchor_div=4)}


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


def plan_for(akv, w, params=None):
    return akv.plan(w.units, w.kv_heads, w.q_per_kv, w.n_tokens, w.head_dim, w.n_obs,
                    akv.BF16 if w.dtype == "bf16" else akv.F32, w.theta, w.window, **(params or {}))


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
    prm = PARAMS.get(name, {})
    K, V, Q = make_inputs(w)
    p = plan_for(akv, w, prm)
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
                           taps=dict(score=score[u], util=util[u]), q=q64[u], o_gpu=o_h[u], params=prm)
        _flush(f"[parity] {name} unit {u}: {rep}")


@pytest.mark.parametrize("name", ["bf16_ragged", "f32_tiny", "bf16_stress_short", "bf16_joint", "bf16_hlm_g8",
                                  "f32_hlm", "bf16_hlm_stress", "bf16_rope", "f32_rope", "bf16_rope_g8",
                                  "bf16_rope_joint", "bf16_rope_long", "bf16_rope_wide", "bf16_rope_bigA"])
def test_decode_on_host_packed_oracle_cache(akv, name):
    """Decode alone: the oracle's compressed representation, packed on the
    host into the cache layout, decoded on the GPU."""
    w = SMALL[name]
    prm = PARAMS.get(name, {})
    _flush(f"[decode-packed] {name}")
    K, V, Q = make_inputs(w)
    p = plan_for(akv, w, prm)
    K64, V64, Q64 = (kvsynth.to_f64(t) for t in (K, V, Q))
    dtype_code = 1 if w.dtype == "bf16" else 2
    cache_h = np.zeros(p.cache_bytes, dtype=np.uint8)
    comps = []
    for u in range(w.units):
        c = O.compress_unit(K64[u], V64[u], Q64[u], w.q_per_kv, w.n_obs, w.theta, w.window, w.elem_bytes,
                            **oracle_params(prm))
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


@pytest.mark.parametrize("name", ["bf16_rope_q256", "bf16_rope_g8", "bf16_rope", "bf16_cover_g8"])
def test_compress_on_a_dirty_workspace(akv, name):
    """A workspace full of garbage gives the same cache, bit for bit, as a
    clean one; with pre-RoPE keys and 256 observation queries per KV head the
    two query groups add their score and key-utility partials onto words
    cleared inside compress."""
    w = SMALL[name]
    _flush(f"[determinism] {name}: U={w.units}")
    K, V, Q = make_inputs(w)
    p = plan_for(akv, w, PARAMS[name])
    c1, ws, _ = akv.alloc(p, "cuda")
    c2 = torch.empty_like(c1)
    ws.zero_()
    akv.compress(p, K, V, Q, c1, ws)
    ws.fill_(0xAB)
    akv.compress(p, K, V, Q, c2, ws)
    torch.cuda.synchronize()
    # each unit's bytes (the padding up to the unit stride is not written)
    for u in range(w.units):
        a, b = u * p.unit_stride, u * p.unit_stride + p.unit_bytes
        assert torch.equal(c1[a:b], c2[a:b]), u


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


def test_decode_of_a_cache_written_under_another_plan_gives_nan(akv):
    """Every decode workgroup checks its unit's header against the plan it was
    given: a cache compressed under another plan (here another theta, so other
    residual counts and section offsets) decodes to NaN, and only the unit
    headers are read (the buffer is as large as either plan's cache)."""
    w = SMALL["bf16_ragged"]
    _flush("[header-check] bf16_ragged, theta 0.1 cache decoded with a theta 0.2 plan")
    K, V, Q = make_inputs(w)
    p1 = plan_for(akv, w)
    p2 = plan_for(akv, w.scaled(theta=0.2))
    assert p1.R_K != p2.R_K
    cache = torch.zeros(max(p1.cache_bytes, p2.cache_bytes), dtype=torch.uint8, device="cuda")
    _, ws, dws1 = akv.alloc(p1, "cuda")
    akv.compress(p1, K, V, Q, cache[:p1.cache_bytes], ws)
    _, _, dws2 = akv.alloc(p2, "cuda")
    q = kvsynth.decode_queries(w, 0, device="cuda").contiguous()
    o = torch.zeros(w.units, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.float32, device="cuda")
    akv.decode_attn(p2, cache, q, o, dws2)
    torch.cuda.synchronize()
    assert torch.isnan(o).all()
    akv.decode_attn(p1, cache, q, o, dws1)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()


def test_save_restore_decodes_bitwise_identically(akv, tmp_path):
    """A compressed cache written to a file and read back into a fresh device
    buffer decodes, under the plan rebuilt from its own header, to outputs
    bitwise equal to those of the original buffer (the cache is position
    independent: offsets inside it are relative to the unit)."""
    w = SMALL["bf16_multi_part"].scaled(layers=3)
    _flush("[save-restore] bf16_multi_part, 3 units")
    K, V, Q = make_inputs(w)
    p = plan_for(akv, w)
    cache, ws, dws = akv.alloc(p, "cuda")
    akv.compress(p, K, V, Q, cache, ws)
    q = kvsynth.decode_queries(w, 2, device="cuda").contiguous()
    o1 = torch.empty(w.units, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.float32, device="cuda")
    akv.decode_attn(p, cache, q, o1, dws)
    torch.cuda.synchronize()
    f = tmp_path / "cache.bin"
    f.write_bytes(cache.cpu().numpy().tobytes())
    del cache
    raw = np.frombuffer(f.read_bytes(), dtype=np.uint8)
    p2 = akv.plan_from_header(raw[:256].tobytes(), w.units)
    assert p2.as_dict() == p.as_dict()
    # restored at another device address (offset by 4 KiB inside a larger buffer)
    big = torch.zeros(raw.size + 4096, dtype=torch.uint8, device="cuda")
    restored = big[4096:]
    restored.copy_(torch.from_numpy(raw.copy()))
    _, _, dws2 = akv.alloc(p2, "cuda")
    o2 = torch.full_like(o1, float("nan"))
    akv.decode_attn(p2, restored, q, o2, dws2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# decode instances for every q_per_kv the kernels are built for (1..8), both
# codecs and both element types, on host-packed oracle caches: short contexts
# with ragged tails, 8- and 16-wave workgroups (the 16-wave ones where the
# weight tables of many anchors do not leave room for two workgroups per CU)
DECODE_SHAPES = [(g, dt, codec, n_tok, window)
                 for g in (1, 2, 3, 5, 6, 7)
                 for dt, codec, n_tok, window in (("bf16", 0, 2600, 32), ("bf16", 1, 2100, 32),
                                                  ("f32", 0, 1800, 16), ("f32", 1, 1300, 16))] + \
                [(5, "bf16", 0, 9000, 800), (7, "bf16", 1, 9000, 800), (6, "f32", 0, 6000, 800)]


@pytest.mark.parametrize("G,dt,codec,n_tok,window", DECODE_SHAPES)
def test_decode_instances_on_packed_oracle_cache(akv, G, dt, codec, n_tok, window):
    base = W_["llama8b_32k"] if dt == "bf16" else W_["tiny_f32"]
    w = base.scaled(seqs=1, layers=1, kv_heads=2, q_per_kv=G, n_tokens=n_tok, n_obs=16, window=window,
                    theta=0.12 if window < 100 else 0.3, n_dirs=16)
    prm = dict(codec=codec)
    _flush(f"[decode-inst] G={G} {dt} codec={codec} N={n_tok} W={window}")
    K, V, Q = make_inputs(w)
    p = plan_for(akv, w, prm)
    K64, V64, Q64 = (kvsynth.to_f64(t) for t in (K, V, Q))
    c = O.compress_unit(K64[0], V64[0], Q64[0], G, w.n_obs, w.theta, w.window, w.elem_bytes, **prm)
    assert c.flag.any()
    cache_h = np.zeros(p.cache_bytes, dtype=np.uint8)
    cache_h[:p.unit_bytes] = np.frombuffer(akv.pack_unit(p, oracle_arrays(c, 1 if dt == "bf16" else 2)), np.uint8)
    cache = torch.from_numpy(cache_h).cuda()
    _, _, dws = akv.alloc(p, "cuda")
    for step in range(2):
        q = kvsynth.decode_queries(w, step, device="cuda").contiguous()
        o = torch.empty(1, 2 * G, w.head_dim, dtype=torch.float32, device="cuda")
        akv.decode_attn(p, cache, q, o, dws)
        torch.cuda.synchronize()
        ref = O.decode_unit(c, kvsynth.to_f64(q)[0])
        err = np.linalg.norm(o[0].cpu().numpy().astype(np.float64) - ref, axis=1) / np.linalg.norm(ref, axis=1)
        assert err.max() <= 1e-3, (step, err.max())
