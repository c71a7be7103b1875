"""Full-size parity: every workload at its real shape, compressed and decoded
in the launch configuration the benchmark times (all units in one compress
call, one decode step over all units).

The 3B-shaped workload is small enough for whole-unit comparisons against
the oracle (first and last unit).  For the larger workloads the oracle cannot
redo a whole unit in seconds, so the test checks the last unit (the unit
stride is exercised), every head of it, each stage against the oracle,
conditioned on the GPU's earlier decisions where they are within the stated
tie margins:

* observation score (all tokens) and the anchor set;
* stored anchors equal the input rows;
* nearest anchor, fp16 gamma and residual on a sample of tokens (oracle
  assignment against the GPU's anchors);
* utilities of the sampled tokens and of every token near the residual cut;
* the residual ids of the whole unit: the GPU's set is top-R of its own
  utilities (exact), and against the oracle's top-R a differing id must lie
  within the 1e-5 margin of the oracle's cut (oracle utilities, conditioned
  on the GPU's anchors and assignments, for every token within 1e-3 of the
  cut; tokens further away keep their side since the utilities agree to
  1e-4);
* 2-bit codes, scales and zeros of the checked flagged tokens;
* decode outputs of all q-heads against attention over the reconstruction of
  the GPU cache, and (adversarial workload) the Theorem-1 output-error bound
  for every q-head.
"""
import copy
import sys

import numpy as np
import pytest
import torch

import kvsynth
from oracle import anchorkv_oracle as O
from tests.parity import (MARGIN, OUT_RTOL, check_anchor_set, compare_unit, f16_bits_to_f64,
                          fp16_midpoint_distance, storage_to_f64)

pytestmark = pytest.mark.gpu

SAMPLE_TOKENS = 3072


def _flush(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def akv():
    import kv_cache_compression_snapkv_amd as m
    m.lib()
    return m


def ws_view(ws, off, count, dtype=torch.float32):
    nbytes = count * torch.empty(0, dtype=dtype).element_size()
    return ws[off:off + nbytes].view(dtype)


def run_workload(akv, w, step=0, params=None):
    """Inputs generated in place on the GPU, then compress (all units, one call)
    and one decode step (all units), as the benchmark launches them."""
    dev = "cuda"
    dt = akv.BF16 if w.dtype == "bf16" else akv.F32
    p = akv.plan(w.units, w.kv_heads, w.q_per_kv, w.n_tokens, w.head_dim, w.n_obs, dt, w.theta, w.window,
                 **(params or {}))
    K = torch.empty(w.units, w.kv_heads, w.n_tokens, w.head_dim, dtype=w.torch_dtype, device=dev)
    V = torch.empty_like(K)
    Q = torch.empty(w.units, w.kv_heads * w.q_per_kv, w.n_obs, w.head_dim, dtype=w.torch_dtype, device=dev)
    for u in range(w.units):
        s, l = kvsynth.unit_index(w, u)
        k, v, q = kvsynth.unit_inputs(w, s, l, device=dev)
        K[u].copy_(k); V[u].copy_(v); Q[u].copy_(q)
        del k, v, q
    cache, ws, dws = akv.alloc(p, dev)
    q = kvsynth.decode_queries(w, step, device=dev).contiguous()
    o = torch.empty(w.units, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.float32, device=dev)
    akv.compress(p, K, V, Q, cache, ws)
    akv.decode_attn(p, cache, q, o, dws)
    torch.cuda.synchronize()
    return p, K, V, Q, cache, ws, q, o


def plan_for_units(akv, w, units):
    dt = akv.BF16 if w.dtype == "bf16" else akv.F32
    return akv.plan(units, w.kv_heads, w.q_per_kv, w.n_tokens, w.head_dim, w.n_obs, dt, w.theta, w.window)


def unit_taps(akv, p, ws, u):
    offs = akv.workspace_offsets(p)
    U, H, N = p.units, p.H, p.N
    score = ws_view(ws, offs["score"], U * H * N).view(U, H, N)[u].cpu().numpy().astype(np.float64)
    util = ws_view(ws, offs["util"], U * 2 * H * N).view(U, 2, H, N)[u].cpu().numpy().astype(np.float64)
    return score, util


def unit_arrays(akv, p, cache, u):
    unit = cache[u * p.unit_stride: u * p.unit_stride + p.unit_bytes].cpu().numpy().tobytes()
    return akv.unpack_unit(p, unit)


def test_fullsize_llama3b_8k_whole_units(akv):
    """3B-shaped workload at full size (28 units x 8 heads x 8192 tokens):
    whole-unit comparison of the first and the last unit."""
    w = kvsynth.WORKLOADS["llama3b_8k"]
    _flush(f"[fullsize] {w.name}: units={w.units} N={w.n_tokens}")
    p, K, V, Q, cache, ws, q, o = run_workload(akv, w)
    for u in (0, w.units - 1):
        score, util = unit_taps(akv, p, ws, u)
        arr = unit_arrays(akv, p, cache, u)
        K64, V64, Q64 = (kvsynth.to_f64(t[u]) for t in (K, V, Q))
        rep = compare_unit(K64, V64, Q64, w.q_per_kv, w.n_obs, w.theta, w.window, w.elem_bytes, arr,
                           taps=dict(score=score, util=util), q=kvsynth.to_f64(q[u]),
                           o_gpu=o[u].cpu().numpy().astype(np.float64))
        _flush(f"[fullsize] {w.name} unit {u}: {rep}")


def _sampled_tokens(rng, N, A_pos, n):
    """Sample of token positions: the first and last 64, anchors-adjacent
    positions and uniform picks (sorted, unique)."""
    picks = [np.arange(min(64, N)), np.arange(max(0, N - 64), N), rng.choice(A_pos, size=min(64, A_pos.size)) + 1,
             rng.integers(0, N, size=n)]
    t = np.unique(np.clip(np.concatenate(picks), 0, N - 1))
    return t


UTIL_BAND = 1e-3   # tokens within this relative distance of the GPU's cut get oracle utilities
UTIL_RTOL = 1e-4   # GPU utilities against the oracle's (conditioned on the GPU's assignment)


def _near_cut(util_g, R):
    """Per side: the GPU's cut value and the mask [H, N] of eligible tokens
    whose GPU utility lies within UTIL_BAND of it, and of those above it."""
    out = []
    for s in range(2):
        ug = np.where(util_g[s] >= 0, util_g[s], -np.inf)
        c = O.cut_value(ug, R[s])
        if c is None:
            out.append((None, np.zeros(ug.shape, bool), np.zeros(ug.shape, bool)))
            continue
        near = np.isfinite(ug) & (np.abs(ug - c) <= UTIL_BAND * abs(c))
        above = np.isfinite(ug) & (ug > c + UTIL_BAND * abs(c))
        out.append((c, near, above))
    return out


def _oracle_residual_ids(ug, c_g, near, above, u_near, R):
    """The oracle's top-R set of one side, from oracle utilities on the tokens
    near the GPU's cut: a token further than UTIL_BAND from the cut keeps its
    side of it in the oracle while the GPU utilities are within UTIL_RTOL
    (checked on every near token and on the sampled ones), so the oracle's
    top-R is the tokens above the band plus the best near ones.  Returns the
    oracle mask and the oracle's cut value."""
    H, N = ug.shape
    uo = np.full((H, N), -np.inf)
    uo[above] = 1e300            # certainly selected (ties among them resolve by head, position)
    uo[near] = u_near
    sel = O.allocate(uo, R)
    rem = R - int(above.sum())
    c_o = np.sort(u_near)[::-1][rem - 1] if 0 < rem <= u_near.size else None
    return sel, c_o


def check_sampled_unit(akv, w, p, K, V, Q, cache, ws, q, o, u, seed=0):
    """Every head of unit u: observation score and anchor set; stored anchors;
    on sampled tokens the nearest anchor, fp16 gamma, utilities and codes;
    the decode outputs of all q-heads; the Theorem-1 bound for every q-head
    (adversarial workload).  Then the residual ids of the whole unit against
    the oracle under the 1e-5 rule (oracle utilities, conditioned on the GPU's
    anchors and assignments, for every token near the cut)."""
    rng = np.random.default_rng(seed)
    H, N, D, G, W = w.kv_heads, w.n_tokens, w.head_dim, w.q_per_kv, w.window
    e = w.elem_bytes
    dtype_code = 1 if e == 2 else 2
    op = O.plan(H, N, D, e, w.theta, W)
    assert (op.A, op.R_K, op.R_V) == (p.A, p.R_K, p.R_V)
    score_g, util_g = unit_taps(akv, p, ws, u)
    arr = unit_arrays(akv, p, cache, u)
    gpos = arr["positions"].astype(np.int64)
    gidx = arr["idx"].astype(np.int64)
    gflag = arr["flag"].astype(bool)
    rep = {}

    # residual selection over the whole unit: the oracle's allocation applied
    # to the GPU's own utilities must give exactly the GPU's residual set
    R = (p.R_K, p.R_V)
    for s in range(2):
        ug = np.where(util_g[s] >= 0, util_g[s], -np.inf)
        sel = O.allocate(ug, R[s])
        assert np.array_equal(sel, gflag[s]), f"side {s}: residual set differs from top-R of the GPU utilities"
        assert gflag[s].sum() == R[s]
    cuts = _near_cut(util_g, R)
    u_near = [np.full(int(cuts[s][1].sum()), np.nan) for s in range(2)]
    near_slot = [np.full((H, N), -1, np.int64) for s in range(2)]
    for s in range(2):
        near_slot[s][cuts[s][1]] = np.arange(u_near[s].size)
    rep["near_cut"] = [int(x.size) for x in u_near]

    o_g = o[u].cpu().numpy().astype(np.float64)
    q64 = kvsynth.to_f64(q[u])
    A = gpos.shape[1]
    worst_util = 0.0
    for h in range(H):
        Kh = kvsynth.to_f64(K[u, h])
        Vh = kvsynth.to_f64(V[u, h])
        Qh = kvsynth.to_f64(Q[u, h * G:(h + 1) * G]).reshape(G * w.n_obs, D)
        # observation attention, score, anchor set
        P, Oh = O.obs_attention(Qh, Kh, Vh, w.n_obs)
        score, pooled = O.anchor_score(P, W)
        s_err = np.max(np.abs(score_g[h] - score) / np.maximum(score, score.max() * 1e-6))
        assert s_err < 1e-4, f"head {h}: score mismatch {s_err}"
        ok, why = check_anchor_set(pooled, gpos[h], N, W, op.k_s, op.k_u)
        assert ok, f"head {h}: anchor set {why}"
        rep[f"h{h}_anchors"] = why
        # stored anchors are the input rows
        for s, X in enumerate((Kh, Vh)):
            ga = storage_to_f64(arr["anchors_k" if s == 0 else "anchors_v"][h], dtype_code)
            assert np.array_equal(ga, X[gpos[h]]), f"head {h} side {s}: stored anchors differ"
        is_anchor = np.zeros(N, bool)
        is_anchor[gpos[h]] = True
        anchor_rank = np.full(N, -1)
        anchor_rank[gpos[h]] = np.arange(A)
        # tokens checked on this head: a sample, plus every token near either cut
        near_t = np.nonzero(cuts[0][1][h] | cuts[1][1][h])[0]
        ts = np.union1d(_sampled_tokens(rng, N, gpos[h], SAMPLE_TOKENS), near_t)
        res = {}
        for s, X in enumerate((Kh, Vh)):
            # the oracle's assignment against the GPU's anchors (rows 0..A-1 of
            # the small problem are the anchors themselves)
            Xs = np.concatenate([X[gpos[h]], X[ts]])
            a_free = O.assign(Xs, np.arange(A))
            g_s = gidx[s, h, ts]
            o_s = np.where(is_anchor[ts], anchor_rank[ts], a_free["idx"][A:])
            mism = (g_s != o_s) & ~is_anchor[ts]
            bad = mism & (a_free["margin"][A:] >= MARGIN)
            assert not bad.any(), f"head {h} side {s}: {int(bad.sum())} assignments differ outside the margin"
            assert np.all(g_s[is_anchor[ts]] == anchor_rank[ts][is_anchor[ts]]), "anchor tokens not self-assigned"
            rep[f"h{h}_s{s}_assign_excused"] = int(mism.sum())
            # continue from the GPU's assignment
            a_c = O.assign(Xs, np.arange(A), idx_override=np.concatenate([np.arange(A), g_s]))
            gam, r = a_c["gamma"][A:], a_c["r"][A:]
            r[is_anchor[ts]] = 0.0
            gam = np.where(is_anchor[ts], 1.0, gam)
            g16 = f16_bits_to_f64(arr["gamma16"][s, h, ts])
            want16 = O.fp16_rne(gam)
            near16 = fp16_midpoint_distance(gam) < 1e-3
            assert not ((g16 != want16) & ~near16).any(), f"head {h} side {s}: fp16 gammas differ"
            res[s] = r
        # utilities of the checked tokens (oracle, conditioned on the GPU's assignment)
        uK, uV = O.utilities(P[:, ts], Oh, Qh, Vh[ts], res[0], res[1], ~is_anchor[ts])
        for s, uo in enumerate((uK, uV)):
            el = np.isfinite(uo)
            if el.any():
                rel = np.abs(util_g[s, h, ts][el] - uo[el]) / np.maximum(np.abs(uo[el]), 1e-30)
                worst_util = max(worst_util, float(rel.max()))
                assert rel.max() < UTIL_RTOL, f"head {h} side {s}: utility error {rel.max()}"
            assert np.all(util_g[s, h, ts][~el] < 0), "anchor tokens must be ineligible"
            slot = near_slot[s][h, ts]
            u_near[s][slot[slot >= 0]] = uo[slot >= 0]
        # codes of the checked flagged tokens
        for s in range(2):
            fl = gflag[s, h, ts]
            if not fl.any():
                continue
            r = res[s][fl]
            codes_o, sc_o, ze_o = O.quantize(r)
            lo = r.reshape(r.shape[0], -1, 32).min(-1)
            hi = r.reshape(r.shape[0], -1, 32).max(-1)
            safe_g = (fp16_midpoint_distance(lo) > 1e-3) & (fp16_midpoint_distance((hi - lo) / 3) > 1e-3)
            sc_g = f16_bits_to_f64(arr["scale16"][s, h, ts][fl])
            ze_g = f16_bits_to_f64(arr["zero16"][s, h, ts][fl])
            assert np.all((sc_g == sc_o) | ~safe_g), f"head {h} side {s}: scales differ"
            assert np.all((ze_g == ze_o) | ~safe_g), f"head {h} side {s}: zeros differ"
            safe_e = (O.code_margin(r, sc_o, ze_o) > 1e-3) & np.repeat(safe_g, 32, axis=1)
            bad = (arr["codes"][s, h, ts][fl] != codes_o) & safe_e
            assert not bad.any(), f"head {h} side {s}: {int(bad.sum())} codes differ"
            rep[f"h{h}_s{s}_codes_checked"] = int(safe_e.sum())
        # decode of this head's q-heads over the reconstruction of the GPU cache
        c = O.Compressed(plan=op, G=G, anchor_pos=gpos[h:h + 1], idx=gidx[:, h:h + 1], gamma=None,
                         gamma16=f16_bits_to_f64(arr["gamma16"][:, h:h + 1]), resid=None,
                         flag=gflag[:, h:h + 1],
                         codes=np.where(gflag[:, h:h + 1, :, None], arr["codes"][:, h:h + 1], 0).astype(np.uint8),
                         scale=f16_bits_to_f64(arr["scale16"][:, h:h + 1]),
                         zero=f16_bits_to_f64(arr["zero16"][:, h:h + 1]),
                         anchors=np.stack([Kh[gpos[h]][None], Vh[gpos[h]][None]]), score=None, pooled=None)
        Khat, Vhat = O.reconstruct(c)
        qh = q64[h * G:(h + 1) * G]
        ref = O.attention(qh, Khat[0], Vhat[0])
        err = np.linalg.norm(o_g[h * G:(h + 1) * G] - ref, axis=1) / np.linalg.norm(ref, axis=1)
        rep[f"h{h}_decode_err"] = float(err.max())
        assert err.max() <= OUT_RTOL, f"head {h}: decode error {err.max()}"
        if w.stress:
            # Theorem 1 [Pith review, "What would settle it"] for every q-head
            worst = 0.0
            for g in range(G):
                t = O.theorem1_terms(qh[g], Kh, Vh, Khat[0], Vhat[0])
                lhs, bound, bound2 = t[0], t[1] + t[2], t[3] + t[4]
                tol = 1e-12 * (1.0 + np.linalg.norm(Vh, axis=1).max())
                assert lhs <= bound + tol and lhs <= bound2 + tol, f"head {h} q {g}: Theorem-1 bound violated"
                worst = max(worst, lhs / max(bound, 1e-300))
            rep[f"h{h}_thm1_ratio_max"] = worst
        del P
    rep["util_err_max"] = worst_util
    assert not any(np.isnan(x).any() for x in u_near), "a token near the cut got no oracle utility"

    # residual ids of the whole unit against the oracle: a token the two sides
    # select differently must lie within MARGIN of the oracle's cut
    for s in range(2):
        c_g, near, above = cuts[s]
        if c_g is None:
            continue
        ug = np.where(util_g[s] >= 0, util_g[s], -np.inf)
        sel_o, c_o = _oracle_residual_ids(ug, c_g, near, above, u_near[s], R[s])
        # the construction holds while the oracle's cut stays well inside the
        # band: tokens beyond it are then on the same side of both cuts
        assert c_o is None or abs(c_o - c_g) <= 0.5 * UTIL_BAND * abs(c_g), f"side {s}: cuts {c_o} vs {c_g}"
        diff = sel_o != gflag[s]
        assert not (diff & ~near).any(), f"side {s}: a residual id differs away from the cut"
        if diff.any():
            assert c_o is not None
            ud = u_near[s][near_slot[s][diff]]
            rel = np.abs(ud - c_o) / abs(c_o)
            assert rel.max() <= MARGIN, f"side {s}: {int((rel > MARGIN).sum())} residual ids differ outside the margin"
        rep[f"s{s}_residual_ids_excused"] = int(diff.sum())
    return rep


@pytest.mark.parametrize("wname", ["llama8b_32k", "llama70b_128k", "stress_64k"])
def test_fullsize_sampled(akv, wname):
    w = kvsynth.WORKLOADS[wname]
    _flush(f"[fullsize] {wname}: units={w.units} H={w.kv_heads} G={w.q_per_kv} N={w.n_tokens}")
    p, K, V, Q, cache, ws, q, o = run_workload(akv, w)
    _flush(f"[fullsize] {wname}: compressed and decoded; checking unit {w.units - 1}")
    rep = check_sampled_unit(akv, w, p, K, V, Q, cache, ws, q, o, w.units - 1)
    _flush(f"[fullsize] {wname}: {rep}")
    # one unit per launch (the per-layer call): its plan splits every head into
    # many more token ranges, merged by the range-merge kernel; the outputs
    # equal those of the full-cache launch up to the order of the sums
    p1 = plan_for_units(akv, w, 1)
    assert p1.decode_splits > p.decode_splits
    _, _, dws1 = akv.alloc(p1, "cuda")
    o1 = torch.empty(1, w.kv_heads * w.q_per_kv, w.head_dim, dtype=torch.float32, device="cuda")
    akv.decode_attn(p1, cache[:p1.cache_bytes], q[:1].contiguous(), o1, dws1)
    torch.cuda.synchronize()
    d = (torch.linalg.norm(o1[0] - o[0], dim=-1) / torch.linalg.norm(o[0], dim=-1)).max().item()
    _flush(f"[fullsize] {wname}: one-unit launch ({p1.decode_splits} ranges per head) vs full launch "
           f"({p.decode_splits}): {d:.3g}")
    assert d <= 1e-5
    del K, V, Q, cache, ws
    torch.cuda.empty_cache()


def test_fullsize_llama3b_8k_rope_last_unit(akv):
    """3B-shaped workload at full size with the keys taken as pre-RoPE
    (28 units x 8 heads x 8192 tokens, rotary base 500000): whole-unit
    comparison of the last unit (rotated observation attention, utilities,
    residual ids, codes, decode over 8 chunks per head)."""
    w = kvsynth.WORKLOADS["llama3b_8k"]
    prm = dict(rope=1)
    _flush(f"[fullsize] {w.name} pre-RoPE: units={w.units} N={w.n_tokens}")
    p, K, V, Q, cache, ws, q, o = run_workload(akv, w, params=prm)
    u = w.units - 1
    score, util = unit_taps(akv, p, ws, u)
    arr = unit_arrays(akv, p, cache, u)
    rep = compare_unit(kvsynth.to_f64(K[u]), kvsynth.to_f64(V[u]), kvsynth.to_f64(Q[u]), w.q_per_kv, w.n_obs,
                       w.theta, w.window, w.elem_bytes, arr, taps=dict(score=score, util=util),
                       q=kvsynth.to_f64(q[u]), o_gpu=o[u].cpu().numpy().astype(np.float64), params=prm)
    _flush(f"[fullsize] {w.name} pre-RoPE unit {u}: {rep}")
