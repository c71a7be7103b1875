"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks an oracle function against something other than itself: a
library routine, a closed form, a hand-worked golden fixture, brute force on
tiny inputs, finite differences, or an invariant stated on the pages.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import anchorkv_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def clustered(r, H, N, D, ndir=8, noise=0.3):
    dirs = r.standard_normal((H, ndir, D))
    dirs /= np.linalg.norm(dirs, axis=-1, keepdims=True)
    cl = r.integers(0, ndir, (H, N))
    X = dirs[np.arange(H)[:, None], cl] + noise / math.sqrt(D) * r.standard_normal((H, N, D))
    return X * np.exp(0.5 * r.standard_normal((H, N)))[..., None]


def bf16_exact(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


# ---------------------------------------------------------------- rounding
def _fp16_bruteforce(x):
    allv = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
    bits = np.arange(65536, dtype=np.uint16)
    ok = np.isfinite(allv)
    allv, bits = allv[ok], bits[ok]
    out = []
    for v in x:
        d = np.abs(allv - v)
        best = d.min()
        cand = np.nonzero(d == best)[0]
        if cand.size > 1:   # tie: even mantissa (lowest bit 0)
            cand = [c for c in cand if bits[c] & 1 == 0] or list(cand)
        out.append(allv[cand[0]])
    return np.array(out)


def test_fp16_rne_matches_bruteforce():
    r = rng(1)
    x = np.concatenate([r.standard_normal(300) * 10.0 ** r.integers(-7, 5, 300),
                        np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2049.0, 2051.0, -0.5 - 2 ** -12, 6.1e-5, 1e-8])])
    x = x[np.abs(x) < 65504]
    np.testing.assert_array_equal(O.fp16_rne(x), _fp16_bruteforce(x))
    assert O.fp16_rne(np.array([1e6, -1e6])).tolist() == [65504.0, -65504.0]


# ---------------------------------------------------------------- byte plan
def test_plan_matches_hand_worked_counts():
    cases = json.load(open(os.path.join(GOLD, "plan_workloads.json")))["cases"]
    for c in cases:
        p = O.plan(c["H"], c["N"], c["D"], c["e"], c["theta"], c["W"])
        assert (p.A, p.k_s, p.k_u, p.R_K, p.R_V) == (c["A"], c["k_s"], c["k_u"], c["R"], c["R"]), c["name"]


@pytest.mark.parametrize("H,N,D,e,theta,W", [
    (8, 8192, 128, 2, 0.1, 32), (1, 512, 128, 4, 0.1, 32), (3, 5000, 64, 2, 0.07, 16),
    (2, 300, 32, 2, 0.9, 8), (4, 2048, 128, 2, 2.0, 32), (8, 65536, 128, 2, 0.02, 64)])
def test_plan_byte_invariant_and_tightness(H, N, D, e, theta, W):
    """Per side, the bytes used stay within theta*H*N*D*e and no further
    residual would fit unless every eligible token already has one."""
    p = O.plan(H, N, D, e, theta, W)
    rec = D // 4 + D // 8
    used = O.side_bytes(p, p.R_K)
    assert used <= float(np.float32(theta)) * H * N * D * e
    assert p.R_K == H * (N - p.A) or used + rec > p.budget_unit
    assert p.A - W == p.k_s + p.k_u and p.A <= N


def test_plan_budget_errors():
    with pytest.raises(ValueError):
        O.plan(8, 1024, 128, 2, 0.01, 32)     # window + pointers exceed the budget
    with pytest.raises(ValueError):
        O.plan(1, 100, 100, 2, 0.1, 8)        # D not a multiple of 32


def test_plan_residual_floor_at_short_context():
    """Velox, "The one setting worth tuning": at short contexts and small theta
    the anchors and their pointers use (nearly) the whole budget, leaving very
    few or zero residual slots.  When the anchor count is capped by the budget,
    what is left per head is less than one more anchor, so R < H*(D*e+2)/rec."""
    for N, theta in [(256, 0.15), (512, 0.08), (300, 0.2)]:
        p = O.plan(8, N, 128, 2, theta, 32)
        if p.A - 32 < N // 128:
            assert p.R_K < 8 * (128 * 2 + 2) / 48
    assert O.plan(8, 256, 128, 2, 0.15, 32).R_K <= 2
    assert O.plan(1, 256, 128, 2, 0.144, 32).R_K == 0


# ---------------------------------------------------------------- obs attention
def test_obs_attention_matches_sdpa_with_offset_causal_mask():
    r = rng(2)
    G, n_obs, N, D = 3, 5, 40, 32
    Q = r.standard_normal((G * n_obs, D))
    K = r.standard_normal((N, D))
    V = r.standard_normal((N, D))
    P, Oo = O.obs_attention(Q, K, V, n_obs)
    j = np.arange(G * n_obs) % n_obs
    mask = torch.from_numpy(np.arange(N)[None, :] <= (N - n_obs + j)[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None], attn_mask=mask[None])
    np.testing.assert_allclose(Oo, ref[0].numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(P.sum(1), 1.0, rtol=1e-13)
    assert np.all(P[~mask.numpy()] == 0)


# ---------------------------------------------------------------- score & anchors
@pytest.mark.parametrize("pool", [7, 1, 3, 5, 15])
def test_pooling_is_zero_padded_window_sum(pool):
    """Library routine: numpy's centred convolution with a box of the pooling
    width over the non-window scores; width 1 is no pooling."""
    r = rng(3)
    P = r.random((6, 50))
    score, pooled = O.anchor_score(P, 10) if pool == 7 else O.anchor_score(P, 10, pool)
    np.testing.assert_allclose(score, P.sum(0), rtol=1e-15)
    ref = np.convolve(score[:40], np.ones(pool), mode="same")
    np.testing.assert_allclose(pooled, ref, rtol=1e-13)
    if pool == 1:
        np.testing.assert_array_equal(pooled, score[:40])


def test_plan_anchor_parameters_hand_worked():
    """k = floor(N/anchor_div) non-window anchors, floor(rho k) of them scored,
    worked by hand at budgets that do not cap k: N = 8192 gives 64 at the
    pages' 128, 128 at 64; rho 0.7 of 64 is 44, 0.5 of 128 is 64, rho 1 keeps no
    uniform picks and rho 0 no scored ones."""
    for kw, (k, ks) in [({}, (64, 44)), (dict(anchor_div=64), (128, 89)), (dict(anchor_div=64, rho=0.5), (128, 64)),
                        (dict(rho=1.0), (64, 64)), (dict(rho=0.0), (64, 0)), (dict(anchor_div=1000), (8, 5))]:
        p = O.plan(8, 8192, 128, 2, 0.1, 32, **kw)
        assert (p.A - 32, p.k_s, p.k_u) == (k, ks, k - ks), kw


def _bruteforce_anchors(pooled, N, W, k_s, k_u):
    L = N - W
    scored = [t for t in range(L)
              if sum(1 for u in range(L) if pooled[u] > pooled[t] or (pooled[u] == pooled[t] and u < t)) < k_s]
    rest = [t for t in range(L) if t not in scored]
    M = len(rest)
    # pick i = the candidate at the midpoint of the i-th of k_u equal strata
    uni = [rest[math.floor(Fraction(2 * i + 1, 2) * Fraction(M, k_u))] for i in range(k_u)]
    return sorted(scored + uni + list(range(L, N)))


@pytest.mark.parametrize("seed", range(6))
def test_select_anchors_bruteforce(seed):
    r = rng(10 + seed)
    N, W = int(r.integers(20, 60)), int(r.integers(1, 8))
    pooled = r.integers(0, 6, N - W).astype(float)   # many ties
    k_s, k_u = int(r.integers(0, 6)), int(r.integers(1, 6))
    pos = O.select_anchors(pooled, N, W, k_s, k_u)
    assert pos.tolist() == _bruteforce_anchors(pooled, N, W, k_s, k_u)
    assert len(set(pos.tolist())) == W + k_s + k_u
    assert set(range(N - W, N)) <= set(pos.tolist())


# ---------------------------------------------------------------- coverage-optimised anchors
def _greedy_fps(X, base, L, k):
    """Furthest-point sampling one pick at a time, written with explicit
    loops: the candidate (t < L, not an anchor) whose largest cosine to the
    current anchors is smallest, the lower position on ties."""
    cur = list(base)
    out = []
    norm = [math.sqrt(float(np.dot(x, x))) for x in X]
    for _ in range(k):
        best_t, best_v = None, None
        for t in range(L):
            if t in cur:
                continue
            v = -math.inf
            for a in cur:
                den = norm[t] * norm[a]
                c = float(np.dot(X[t], X[a])) / den if den > 0 else 0.0
                v = max(v, c)
            if best_v is None or v < best_v:
                best_t, best_v = t, v
        out.append(best_t)
        cur.append(best_t)
    return out


@pytest.mark.parametrize("seed", range(4))
def test_cover_picks_one_per_round_is_furthest_point_sampling(seed):
    r = rng(40 + seed)
    N, D, W = int(r.integers(20, 45)), 8, int(r.integers(1, 4))
    X = r.standard_normal((N, D))
    X[int(r.integers(0, N - W))] = 0.0            # a zero-norm token: cosine 0 with everything
    L = N - W
    base = sorted(set(r.integers(0, L, 3).tolist())) + list(range(L, N))
    k = int(r.integers(1, 7))
    picks, margins = O.cover_picks(X, np.array(base), L, k, rounds=k)
    assert picks.tolist() == _greedy_fps(X, base, L, k)
    assert margins.shape == (k,)


def test_cover_picks_hand_worked():
    # exact cosines: tokens (0,-1), (1,1), (-1,0), (0,1) and the window anchor
    # (1,0).  The opposite token (-1,0) (cosine -1) comes first; then (0,-1)
    # and (0,1) both have largest cosine 0 and the lower position wins the
    # tie; (1,1) stays (largest cosine 1/sqrt(2)).
    X = np.zeros((5, 4))
    X[0, :2], X[1, :2], X[2, :2], X[3, :2], X[4, :2] = (0, -1), (1, 1), (-1, 0), (0, 1), (1, 0)
    picks, margins = O.cover_picks(X, np.array([4]), 4, 2, rounds=2)
    assert picks.tolist() == [2, 0]
    assert margins[0] == 1.0 and margins[1] == 0.0   # a clear first pick, an exact tie second


@pytest.mark.parametrize("seed", range(3))
def test_cover_picks_rounds_and_invariants(seed):
    r = rng(50 + seed)
    N, D, W = 80, 16, 5
    X = r.standard_normal((N, D))
    L = N - W
    base = list(range(0, L, 17)) + list(range(L, N))
    for k, R in ((10, 8), (3, 8), (12, 5), (7, 1)):
        sizes = O.cover_rounds_of(k, R)
        assert sum(sizes) == k and len(sizes) == min(R, k) and min(sizes) >= 1
        picks, margins = O.cover_picks(X, np.array(base), L, k, rounds=R)
        assert len(picks) == k == len(set(picks.tolist()))
        assert all(0 <= t < L and t not in base for t in picks.tolist())
        assert margins.shape == (len(sizes),) and (margins >= 0).all()
        # the first round's picks are the k-lowest maxima over the base set
        c, _ = O.cosine_table(X[:L], X[np.array(base)])
        mx = c.max(axis=1)
        cand = [t for t in range(L) if t not in base]
        first = sorted(cand, key=lambda t: (mx[t], t))[:sizes[0]]
        assert picks[:sizes[0]].tolist() == first
    # one round takes the k worst-covered candidates at once; k rounds are
    # greedy furthest-point sampling, which re-evaluates after every pick
    p1, _ = O.cover_picks(X, np.array(base), L, 6, rounds=1)
    c, _ = O.cosine_table(X[:L], X[np.array(base)])
    mx = c.max(axis=1)
    assert p1.tolist() == sorted([t for t in range(L) if t not in base], key=lambda t: (mx[t], t))[:6]


def test_select_anchors_cover_mode():
    r = rng(60)
    N, D, W, k_s, k_u = 70, 8, 4, 5, 6
    X = r.standard_normal((N, D))
    pooled = r.random(N - W)
    pos = O.select_anchors(pooled, N, W, k_s, k_u, mode=O.ANCHORS_COVER, X=X, rounds=3)
    scored = sorted(np.argsort(-pooled, kind="stable")[:k_s].tolist())
    base = scored + list(range(N - W, N))
    picks, _ = O.cover_picks(X, np.array(base), N - W, k_u, rounds=3)
    assert pos.tolist() == sorted(base + picks.tolist())
    assert len(set(pos.tolist())) == W + k_s + k_u


# ---------------------------------------------------------------- assignment & projection
def test_projection_hand_worked_example():
    g = json.load(open(os.path.join(GOLD, "projection_example.json")))
    D = 32
    pad = lambda v: np.array(list(v) + [0] * (D - len(v)), dtype=float)
    X = np.stack([pad(a) for a in g["anchors"]] + [pad(t["x"]) for t in g["tokens"]])
    res = O.assign(X, np.arange(3))
    for i, t in enumerate(g["tokens"]):
        k = 3 + i
        assert res["idx"][k] == t["idx"]
        assert res["gamma"][k] == pytest.approx(t["gamma"], abs=1e-15)
        np.testing.assert_allclose(res["r"][k], pad(t["r"]), atol=1e-15)
        c, _ = O.cosine_table(X[k:k + 1], X[:3])
        assert c[0, t["idx"]] == pytest.approx(t["cos"], abs=1e-15)
    # anchors reconstruct exactly with coefficient 1 and zero residual (Velox, "Evidence")
    assert res["idx"][:3].tolist() == [0, 1, 2] and np.all(res["gamma"][:3] == 1) and np.all(res["r"][:3] == 0)


def test_assign_bruteforce_and_projection_identities():
    r = rng(4)
    N, D, A = 120, 32, 9
    X = bf16_exact(clustered(r, 1, N, D, ndir=4)[0])
    X[7] = 0.0                                       # zero token: cosine 0 everywhere -> index 0
    pos = np.sort(r.choice(N, A, replace=False))
    res = O.assign(X, pos)
    for t in range(N):
        if t in pos:
            continue
        cs = []
        for a in range(A):
            xa = X[pos[a]]
            num = math.fsum(float(u) * float(v) for u, v in zip(X[t], xa))
            den = math.sqrt(math.fsum(float(u) ** 2 for u in X[t])) * math.sqrt(math.fsum(float(v) ** 2 for v in xa))
            cs.append(num / den if den > 0 else 0.0)
        best = max(range(A), key=lambda a: (cs[a], -a))
        if res["margin"][t] > 1e-12:
            assert res["idx"][t] == best, t
        xa = X[pos[res["idx"][t]]]
        rr = res["r"][t]
        # orthogonal decomposition (Velox "Evidence"; Pith "What carries the argument")
        np.testing.assert_allclose(res["gamma"][t] * xa + rr, X[t], atol=1e-12)
        assert abs(rr @ xa) <= 1e-12 * (np.linalg.norm(X[t]) * np.linalg.norm(xa) + 1e-300)
        # relative residual norm sqrt(1 - c^2) (Pith "Referee Report", minor 5)
        c = cs[res["idx"][t]]
        assert np.linalg.norm(rr) == pytest.approx(np.linalg.norm(X[t]) * math.sqrt(max(0.0, 1 - c * c)), abs=1e-10)
    assert res["idx"][7] == 0 and res["gamma"][7] == 0


# ---------------------------------------------------------------- utility (finite differences)
def _attn(q, K, V):
    s = K @ q / math.sqrt(q.size)
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ V


def test_utility_equals_first_order_output_change():
    """Key channel: moving k_t by eps*r changes logit t by eps<q,r>/sqrt(D), and by
    d alpha_t/d s_u = alpha_t(delta_tu - alpha_u) the output moves by
    eps * alpha_t <q,r>/sqrt(D) (v_t - o) to first order.  Value channel:
    y changes by exactly alpha_t * dv.  Summed norms over the observation
    queries must equal the oracle's utilities (Pith, "Assumptions & free
    parameters")."""
    r = rng(5)
    N, D, GQ = 24, 32, 4
    K = r.standard_normal((N, D))
    V = r.standard_normal((N, D))
    Q = r.standard_normal((GQ, D))
    rK = r.standard_normal((N, D)) * 0.3
    rV = r.standard_normal((N, D)) * 0.3
    P, Oo = O.obs_attention(Q, K, V, n_obs=1)   # every row sits at N-1: all keys visible
    uK, uV = O.utilities(P, Oo, Q, V, rK, rV, np.ones(N, bool))
    eps = 1e-6
    for t in range(N):
        fdK = fdV = 0.0
        for j in range(GQ):
            Kp, Km = K.copy(), K.copy()
            Kp[t] += eps * rK[t]
            Km[t] -= eps * rK[t]
            fdK += np.linalg.norm((_attn(Q[j], Kp, V) - _attn(Q[j], Km, V)) / (2 * eps))
            Vp = V.copy()
            Vp[t] += rV[t]
            fdV += np.linalg.norm(_attn(Q[j], K, Vp) - _attn(Q[j], K, V))
        assert uK[t] == pytest.approx(fdK, rel=1e-6)
        assert uV[t] == pytest.approx(fdV, rel=1e-10)


# ---------------------------------------------------------------- allocation
def test_allocation_is_optimal_subset_bruteforce():
    r = rng(6)
    H, N, R = 2, 6, 4
    u = r.random((H, N))
    u[0, 2] = -np.inf                        # an anchor: ineligible
    mask = O.allocate(u, R)
    items = [(h, t) for h in range(H) for t in range(N) if np.isfinite(u[h, t])]
    best = max(itertools.combinations(items, R), key=lambda s: sum(u[h, t] for h, t in s))
    assert sorted(zip(*np.nonzero(mask))) == sorted(best)


def test_allocation_ties_lower_head_then_position():
    u = np.ones((3, 4))
    mask = O.allocate(u, 5)
    assert [tuple(x) for x in np.argwhere(mask)] == [(0, 0), (0, 1), (0, 2), (0, 3), (1, 0)]


def test_allocation_pools_across_heads():
    """Velox, "Evidence": the budget favours the head with higher utility
    instead of splitting evenly."""
    r = rng(7)
    u = r.random((2, 100))
    u[1] *= 10
    mask = O.allocate(u, 60)
    assert mask[1].sum() > mask[0].sum()
    assert mask.sum() == 60


# ---------------------------------------------------------------- codec
def test_codec_nearest_level_bruteforce():
    r = rng(8)
    x = r.standard_normal((50, 64)) * np.exp(r.standard_normal((50, 1)))
    codes, sc, ze = O.quantize(x)
    margin = O.code_margin(x, sc, ze)
    for i in range(50):
        for d in range(64):
            g = d // 32
            levels = [ze[i, g] + sc[i, g] * c for c in range(4)]
            dist = [abs(x[i, d] - L) for L in levels]
            best = min(range(4), key=lambda c: (dist[c], c % 2, c))
            if margin[i, d] > 1e-9:
                assert codes[i, d] == best
    rt = O.dequantize(codes, sc, ze)
    # inside the covered range the error is at most half a step
    inside = (x >= np.repeat(ze, 32, 1)) & (x <= np.repeat(ze + 3 * sc, 32, 1))
    assert np.all(np.abs(x - rt)[inside] <= np.repeat(sc, 32, 1)[inside] / 2 * (1 + 1e-12))
    # and the grid spans the group up to the fp16 rounding of zero and scale
    assert np.all(np.abs(x - rt) <= np.repeat(sc, 32, 1) / 2 + 2 ** -10 * np.repeat(np.abs(ze) + 3 * sc, 32, 1))


def test_codec_reduces_error_in_aggregate():
    """Velox, "Evidence": the quantised residual is closer than storing nothing.
    For this codec it holds in aggregate, not per vector (30 zeros and +-1 give
    error^2 3.33 against ||r||^2 = 2)."""
    r = rng(9)
    x = r.standard_normal((500, 128))
    codes, sc, ze = O.quantize(x)
    assert (np.linalg.norm(x - O.dequantize(codes, sc, ze)) ** 2) < 0.2 * (np.linalg.norm(x) ** 2)
    v = np.zeros((1, 32))
    v[0, 0], v[0, 1] = 1.0, -1.0
    c, s, z = O.quantize(v)
    assert np.sum((v - O.dequantize(c, s, z)) ** 2) > np.sum(v ** 2)


def test_codec_zero_scale_group():
    x = np.full((1, 32), 0.25)
    c, s, z = O.quantize(x)
    assert s[0, 0] == 0 and np.all(c == 0) and np.all(O.dequantize(c, s, z) == 0.25)


# ---------------------------------------------------------------- whole pass, decode, Theorem 1
def small_unit(seed, H=2, G=2, N=600, D=64, n_obs=8, W=8):
    r = rng(seed)
    K = bf16_exact(clustered(r, H, N, D))
    V = bf16_exact(r.standard_normal((H, N, D)))
    Q = bf16_exact(r.standard_normal((H * G, n_obs, D)))
    return K, V, Q


def test_compress_invariants_and_determinism():
    K, V, Q = small_unit(11)
    c = O.compress_unit(K, V, Q, 2, 8, 0.1, 8, 2)
    c2 = O.compress_unit(K, V, Q, 2, 8, 0.1, 8, 2)
    p = c.plan
    for a, b in [(c.anchor_pos, c2.anchor_pos), (c.idx, c2.idx), (c.flag, c2.flag), (c.codes, c2.codes)]:
        np.testing.assert_array_equal(a, b)
    H, N = 2, 600
    # no token dropped: every position keeps a pointer into [0, A) (Velox, "Evidence")
    assert c.idx.shape == (2, H, N) and c.idx.min() >= 0 and c.idx.max() < p.A
    # window always kept exactly (Pith, "Assumptions & free parameters")
    for h in range(H):
        assert set(range(N - 8, N)) <= set(c.anchor_pos[h].tolist())
    assert c.flag[0].sum() == p.R_K and c.flag[1].sum() == p.R_V
    assert not np.any(c.flag[:, np.arange(H)[:, None], c.anchor_pos])
    # residuals are given to the highest utilities
    for s in range(2):
        cut = O.cut_value(c.u[s], p.R_K)
        assert np.all(c.u[s][c.flag[s]] >= cut) and np.all(c.u[s][~c.flag[s]] <= cut)
    # residual orthogonal to its anchor before quantisation
    for s, X in enumerate((K, V)):
        for h in range(H):
            xa = c.anchors[s, h][c.idx[s, h]]
            dots = (c.resid[s, h] * xa).sum(1)
            assert np.all(np.abs(dots) <= 1e-11 * (np.linalg.norm(X[h], axis=1) * np.linalg.norm(xa, axis=1) + 1e-300))
    assert O.side_bytes(p, p.R_K) <= 0.1 * H * N * 64 * 2


def test_decode_matches_sdpa_over_reconstruction():
    K, V, Q = small_unit(12)
    c = O.compress_unit(K, V, Q, 2, 8, 0.1, 8, 2)
    q = bf16_exact(rng(13).standard_normal((4, 64)))
    o = O.decode_unit(c, q)
    Kh, Vh = O.reconstruct(c)
    for h in range(2):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h * 2:(h + 1) * 2])[None], torch.from_numpy(Kh[h])[None], torch.from_numpy(Vh[h])[None])
        np.testing.assert_allclose(o[h * 2:(h + 1) * 2], ref[0].numpy(), rtol=1e-11, atol=1e-12)


def test_all_anchor_cache_is_exact_attention():
    """With W = N every token is an anchor stored exactly, so decode equals
    plain attention over K, V."""
    r = rng(14)
    H, G, N, D = 2, 2, 64, 32
    K = bf16_exact(r.standard_normal((H, N, D)))
    V = bf16_exact(r.standard_normal((H, N, D)))
    Q = bf16_exact(r.standard_normal((H * G, 4, D)))
    c = O.compress_unit(K, V, Q, G, 4, 1.5, N, 2)
    assert c.plan.A == N and c.flag.sum() == 0
    q = bf16_exact(r.standard_normal((H * G, D)))
    o = O.decode_unit(c, q)
    for h in range(H):
        np.testing.assert_allclose(o[h * G:(h + 1) * G], O.attention(q[h * G:(h + 1) * G], K[h], V[h]), rtol=1e-12)


def test_decode_tail_pins():
    """Decode with an exact tail appended after compression: an empty tail is
    plain decode; with every token an anchor it is attention over the
    concatenated sequence (library routine); a tail key aligned with the query
    and far larger than the rest takes the whole softmax."""
    r = rng(15)
    H, G, N, D, T = 2, 3, 96, 32, 7
    K = bf16_exact(clustered(r, H, N, D))
    V = bf16_exact(r.standard_normal((H, N, D)))
    Q = bf16_exact(r.standard_normal((H * G, 8, D)))
    q = bf16_exact(r.standard_normal((H * G, D)))
    Kt = bf16_exact(r.standard_normal((H, T, D)))
    Vt = bf16_exact(r.standard_normal((H, T, D)))
    c = O.compress_unit(K, V, Q, G, 8, 0.2, 8, 2)
    np.testing.assert_array_equal(O.decode_unit_tail(c, q, Kt[:, :0], Vt[:, :0]), O.decode_unit(c, q))
    # all anchors: exact attention over [K; K_tail]
    ca = O.compress_unit(K, V, Q, G, 8, 1.5, N, 2)
    assert ca.plan.A == N
    o = O.decode_unit_tail(ca, q, Kt, Vt)
    for h in range(H):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h * G:(h + 1) * G])[None], torch.from_numpy(np.concatenate([K[h], Kt[h]]))[None],
            torch.from_numpy(np.concatenate([V[h], Vt[h]]))[None])
        np.testing.assert_allclose(o[h * G:(h + 1) * G], ref[0].numpy(), rtol=1e-11, atol=1e-12)
    # one dominant tail key per head (aligned with the head's first query)
    Kd = Kt.copy()
    for h in range(H):
        Kd[h, 3] = 400.0 * q[h * G] / np.linalg.norm(q[h * G])
    o = O.decode_unit_tail(c, q, Kd, Vt)
    for h in range(H):
        np.testing.assert_allclose(o[h * G], Vt[h, 3], rtol=1e-9, atol=1e-9)


def test_theorem1_bound_holds():
    """Pith, "What carries the argument": ||y - y^|| <= attention-weighted
    value error + 2 V_max tanh(||q|| Delta_K / sqrt(D)); both the a^- and
    the a-weighted forms, on compressed caches and on random reconstructions."""
    K, V, Q = small_unit(15)
    c = O.compress_unit(K, V, Q, 2, 8, 0.1, 8, 2)
    Kh, Vh = O.reconstruct(c)
    r = rng(16)
    cases = [(K[h], V[h], Kh[h], Vh[h]) for h in range(2)]
    for _ in range(40):
        N, D = 30, 32
        Kx, Vx = r.standard_normal((N, D)), r.standard_normal((N, D))
        cases.append((Kx, Vx, Kx + r.standard_normal((N, D)) * r.random(), Vx + r.standard_normal((N, D)) * r.random()))
    for Kx, Vx, Khx, Vhx in cases:
        for _ in range(5):
            q = r.standard_normal(Kx.shape[1]) * 3
            err, val, key, val2, key2 = O.theorem1_terms(q, Kx, Vx, Khx, Vhx)
            tol = 1e-12 * (1 + np.linalg.norm(Vx))
            assert err <= val + key + tol
            assert err <= val2 + key2 + tol


def test_worked_example_density_cross_check():
    """Pith, "Referee Report": 91,056 residuals in the worked example and 17.3 %
    residual density at 20x; consistent with one 8-head layer at S = 32768 with
    two sides (the example's own byte costs are not printed)."""
    assert 91056 / (8 * 32768 * 2) == pytest.approx(0.173, abs=1e-3)


# ---------------------------------------------------------------- reconstruction, code margin, cut value
def _independent_reconstruction(c, K, V):
    """K^, V^ of a compressed unit built element by element from the stored
    fields, without the oracle's reconstruct / dequantize: x^_t = h(gamma_t)
    x_a(t) + [t flagged] (zero_g + scale_g code_d) (Pith, "What carries the
    argument": x^ = gamma x_a + r~), with h() the fp16 rounding done by numpy's
    float16 cast and gamma recomputed from the projection formula."""
    H, N, D = K.shape
    out = []
    for s, X in enumerate((K, V)):
        Xh = np.zeros((H, N, D))
        for h in range(H):
            pos = c.anchor_pos[h]
            for t in range(N):
                a = int(c.idx[s, h, t])
                xa = X[h, pos[a]]
                na2 = float(sum(v * v for v in xa))
                g = 1.0 if t == pos[a] else (float(sum(X[h, t, d] * xa[d] for d in range(D))) / na2 if na2 > 0 else 0.0)
                g16 = float(np.float16(g))
                for d in range(D):
                    val = g16 * xa[d]
                    if c.flag[s, h, t]:
                        grp = d // 32
                        val += c.zero[s, h, t, grp] + c.scale[s, h, t, grp] * int(c.codes[s, h, t, d])
                    Xh[h, t, d] = val
        out.append(Xh)
    return out


def _tiny_flagged_unit(seed):
    r = rng(seed)
    H, G, N, D, n_obs, W = 2, 2, 160, 32, 4, 4
    K = bf16_exact(clustered(r, H, N, D, ndir=4))
    V = bf16_exact(r.standard_normal((H, N, D)) + 1.0)
    Q = bf16_exact(r.standard_normal((H * G, n_obs, D)))
    c = O.compress_unit(K, V, Q, G, n_obs, 0.2, W, 2)
    assert 0 < c.flag[0].sum() < H * (N - c.plan.A) and 0 < c.flag[1].sum()
    return c, K, V, G


def test_reconstruct_matches_elementwise_definition():
    """Unflagged tokens reconstruct to exactly fp16(gamma) x_a; flagged tokens
    to fp16(gamma) x_a + dequantised codes, on both sides (a dropped residual,
    a residual added to unflagged tokens, the unrounded gamma or swapped sides
    all fail here)."""
    c, K, V, _ = _tiny_flagged_unit(21)
    Kh, Vh = O.reconstruct(c)
    Ki, Vi = _independent_reconstruction(c, K, V)
    np.testing.assert_array_equal(Kh, Ki)
    np.testing.assert_array_equal(Vh, Vi)
    # the stored fp16 gammas are not all exact: the rounding matters here
    assert np.any(c.gamma16 != c.gamma)


def test_reconstruct_error_bound():
    """||x - x^|| <= ||r - r~|| + |gamma - fp16(gamma)| ||x_a|| for flagged
    tokens and ||r|| + |gamma - fp16(gamma)| ||x_a|| for the rest, since
    x - x^ = (r - [flag] r~) + (gamma - fp16(gamma)) x_a."""
    c, K, V, _ = _tiny_flagged_unit(22)
    for s, (X, Xh) in enumerate(zip((K, V), O.reconstruct(c))):
        for h in range(X.shape[0]):
            xa = X[h, c.anchor_pos[h]][c.idx[s, h]]
            err = np.linalg.norm(X[h] - Xh[h], axis=1)
            rt = c.zero[s, h][:, np.arange(X.shape[2]) // 32] + c.scale[s, h][:, np.arange(X.shape[2]) // 32] * c.codes[s, h]
            kept = np.where(c.flag[s, h][:, None], rt, 0.0)
            bound = np.linalg.norm(c.resid[s, h] - kept, axis=1) + np.abs(c.gamma[s, h] - c.gamma16[s, h]) * np.linalg.norm(xa, axis=1)
            assert np.all(err <= bound * (1 + 1e-12) + 1e-300)
            # and a flagged residual does better than nothing in aggregate
            fl = c.flag[s, h]
            if fl.any():
                assert np.sum(err[fl] ** 2) < np.sum(np.linalg.norm(c.resid[s, h][fl], axis=1) ** 2)


def test_decode_matches_sdpa_over_independent_reconstruction():
    """decode_unit equals library attention (torch SDPA, fp64) over K^, V^
    built without the oracle's reconstruct."""
    c, K, V, G = _tiny_flagged_unit(23)
    Ki, Vi = _independent_reconstruction(c, K, V)
    q = bf16_exact(rng(24).standard_normal((K.shape[0] * G, K.shape[2])) * 2.0)
    o = O.decode_unit(c, q)
    for h in range(K.shape[0]):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h * G:(h + 1) * G])[None], torch.from_numpy(Ki[h])[None], torch.from_numpy(Vi[h])[None])
        np.testing.assert_allclose(o[h * G:(h + 1) * G], ref[0].numpy(), rtol=1e-11, atol=1e-12)


def test_code_margin_hand_values():
    """Distance of (r - zero)/scale from the nearest rounding midpoint k + 1/2,
    worked by hand; +inf where the scale is 0."""
    r = np.zeros((3, 32))
    r[0, :4] = [0.5, 1.4999, 2.0, 0.1]       # zero 0, scale 1
    r[1, :3] = [-0.75, -0.5, 0.25]           # zero -1, scale 0.5: y = 0.5, 1.0, 2.5
    scale = np.array([[1.0], [0.5], [0.0]])
    zero = np.array([[0.0], [-1.0], [3.0]])
    m = O.code_margin(r, scale, zero)
    np.testing.assert_allclose(m[0, :4], [0.0, 1e-4, 0.5, 0.4], atol=1e-12)
    np.testing.assert_allclose(m[1, :3], [0.0, 0.5, 0.0], atol=1e-12)
    assert np.all(np.isinf(m[2]))


def test_cut_value_hand_values():
    """The R-th largest eligible utility, ties counted with multiplicity;
    ineligible (-inf) items never count; R beyond the eligible items gives the
    smallest eligible one; R = 0 gives None."""
    u = np.array([[3.0, 1.0, 2.0], [2.0, -np.inf, 5.0]])
    assert [O.cut_value(u, R) for R in (1, 2, 3, 4, 5, 9)] == [5.0, 3.0, 2.0, 2.0, 1.0, 1.0]
    assert O.cut_value(u, 0) is None
    assert O.cut_value(np.full((2, 2), -np.inf), 3) is None
    # consistent with the allocation: flagged >= cut >= unflagged, and exactly R flagged
    for R in range(1, 6):
        mask = O.allocate(u, R)
        cut = O.cut_value(u, R)
        assert mask.sum() == R and np.all(u[mask] >= cut) and np.all(u[~mask & np.isfinite(u)] <= cut)


# ---------------------------------------------------------------- joint ranking of token-sides
def test_joint_plan_budget_and_tightness():
    """Both sides together stay within 2 floor(theta H N D e) and no further
    record would fit; pooling the two remainders never loses a slot."""
    for H, N, D, e, theta, W in [(8, 8192, 128, 2, 0.1, 32), (8, 32768, 128, 2, 0.05, 32), (3, 5000, 64, 2, 0.07, 16),
                                 (1, 512, 128, 4, 0.1, 32), (8, 65536, 128, 2, 0.02, 64)]:
        p = O.plan(H, N, D, e, theta, W, pool_kv_jointly=True)
        rec = D // 4 + D // 8
        used = 2 * p.fixed_per_side + rec * p.R_total
        assert used <= 2 * p.budget_unit
        assert p.R_total == 2 * H * (N - p.A) or used + rec > 2 * p.budget_unit
        assert p.R_total >= p.R_K + p.R_V and p.R_total <= p.R_K + p.R_V + 1


def test_joint_allocation_bruteforce():
    """With equal record costs the best R_total token-sides are the top
    R_total utilities over both sides: brute force over every subset of a
    tiny unit, and ties go to K before V, then head, then position."""
    r = rng(31)
    H, N, R = 2, 4, 5
    u = r.random((2, H, N))
    u[0, 1, 2] = -np.inf                     # an anchor
    u[1, 1, 2] = -np.inf
    flag = O.allocate(u.reshape(2 * H, N), R).reshape(2, H, N)
    items = [(s, h, t) for s in range(2) for h in range(H) for t in range(N) if np.isfinite(u[s, h, t])]
    best = max(itertools.combinations(items, R), key=lambda c: sum(u[i] for i in c))
    assert sorted(zip(*np.nonzero(flag))) == sorted(best)
    tied = np.ones((2, H, N))
    flag = O.allocate(tied.reshape(2 * H, N), 3).reshape(2, H, N)
    assert [tuple(x) for x in np.argwhere(flag)] == [(0, 0, 0), (0, 0, 1), (0, 0, 2)]
    flag = O.allocate(tied.reshape(2 * H, N), 2 * H * N - 1).reshape(2, H, N)
    assert not flag[1, H - 1, N - 1] and flag.sum() == 2 * H * N - 1


def test_joint_allocation_follows_the_larger_utilities():
    """Pooling across sides: with the value utilities scaled up, the value
    side takes more than its separate share of the records, the total stays
    the pooled slot count, and the compressed unit decodes like any other."""
    K, V, Q = small_unit(32)
    c = O.compress_unit(K, V * 8.0, Q, 2, 8, 0.1, 8, 2, pool_kv_jointly=True)
    p = c.plan
    assert p.joint and c.flag.sum() == p.R_total
    assert c.flag[1].sum() > p.R_V
    cut = O.cut_value(c.u.reshape(4, -1), p.R_total)
    assert np.all(c.u[c.flag] >= cut) and np.all(c.u[~c.flag & np.isfinite(c.u)] <= cut)
    q = bf16_exact(rng(33).standard_normal((4, 64)))
    Kh, Vh = O.reconstruct(c)
    o = O.decode_unit(c, q)
    np.testing.assert_allclose(o[:2], O.attention(q[:2], Kh[0], Vh[0]), rtol=1e-12)


# ---------------------------------------------------------------- the paper's codec (Hadamard + Lloyd-Max)
def test_splitmix64_published_vector():
    """SplitMix64 from seed 1234567 gives 6457827717110365317 then
    3203168211198807973 (the generator's published reference outputs); the
    default sign words are its first two outputs from the fixed seed."""
    st, a = O.splitmix64(1234567)
    st, b = O.splitmix64(st)
    assert (a, b) == (6457827717110365317, 3203168211198807973)
    st, x = O.splitmix64(O.SIGN_SEED)
    st, y = O.splitmix64(st)
    assert O.default_sign_words() == [x & 0xFFFFFFFF, x >> 32, y & 0xFFFFFFFF, y >> 32]
    s = O.signs_from_words(O.default_sign_words(), 128)
    assert set(np.unique(s)) == {-1.0, 1.0} and 40 < (s < 0).sum() < 88


@pytest.mark.parametrize("D", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_matches_library(D):
    """The orthonormal Sylvester matrix equals scipy's Hadamard matrix / sqrt(D),
    is symmetric and orthogonal."""
    from scipy.linalg import hadamard
    Hm = O.hadamard_matrix(D)
    np.testing.assert_array_equal(Hm * math.sqrt(D), hadamard(D).astype(np.float64))
    np.testing.assert_allclose(Hm @ Hm.T, np.eye(D), atol=1e-14)
    np.testing.assert_array_equal(Hm, Hm.T)


def test_rotation_definition_and_inverse():
    """rotate = H diag(s) r with the library Hadamard matrix, norm preserving,
    and unrotate inverts it; an all-zero sign word is the plain transform."""
    from scipy.linalg import hadamard
    r = rng(31).standard_normal((5, 128))
    words = O.default_sign_words()
    s = np.array([-1.0 if (words[i // 32] >> (i % 32)) & 1 else 1.0 for i in range(128)])
    ref = np.array([hadamard(128) @ (s * x) for x in r]) / math.sqrt(128)
    y = O.rotate(r, words)
    np.testing.assert_allclose(y, ref, atol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(r, axis=1), rtol=1e-13)
    np.testing.assert_allclose(O.unrotate(y, words), r, atol=1e-13)
    np.testing.assert_allclose(O.rotate(r, [0, 0, 0, 0]), r @ hadamard(128).T / math.sqrt(128), atol=1e-13)


def test_lloyd_max_conditions_by_quadrature():
    """The four-level codebook satisfies the Lloyd-Max conditions, checked by
    numerical integration of the Gaussian (not the closed forms the oracle
    iterates): each level is its cell's conditional mean and the threshold the
    midpoint; it matches Max's published values (0.4528, 1.510, 0.9816) and
    its mean squared error is Max's 0.1175."""
    from scipy import integrate
    lv, t = O.lloyd_max_gaussian4()
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    cells = [(-np.inf, -t), (-t, 0.0), (0.0, t), (t, np.inf)]
    for k, (a, b) in enumerate(cells):
        m0 = integrate.quad(pdf, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        m1 = integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(m1 / m0 - lv[k]) < 1e-10
    assert abs(t - 0.5 * (lv[2] + lv[3])) < 1e-15 and lv[1] == -lv[2] and lv[0] == -lv[3]
    assert abs(lv[2] - 0.4528) < 5e-5 and abs(lv[3] - 1.510) < 5e-4 and abs(t - 0.9816) < 5e-5
    mse = sum(integrate.quad(lambda x: (x - lv[k]) ** 2 * pdf(x), a, b, epsabs=1e-14)[0]
              for k, (a, b) in enumerate(cells))
    assert abs(mse - 0.1175) < 5e-5


def test_lloyd_max_is_the_mse_minimum():
    """Brute force: no symmetric four-level quantiser on a grid of (t, l1, l2)
    around the codebook has a smaller Gaussian MSE."""
    from scipy.stats import norm
    lv, t0 = O.lloyd_max_gaussian4()

    def mse(t, l1, l2):
        # 2 * [int_0^t (x - l1)^2 phi + int_t^inf (x - l2)^2 phi], closed form via scipy.stats moments
        def part(a, b, c):
            m0 = norm.cdf(b) - norm.cdf(a)
            m1 = norm.pdf(a) - norm.pdf(b)
            m2 = m0 + (a * norm.pdf(a) if np.isfinite(a) else 0) - (b * norm.pdf(b) if np.isfinite(b) else 0)
            return m2 - 2 * c * m1 + c * c * m0
        return 2 * (part(0, t, l1) + part(t, np.inf, l2))
    best = mse(t0, lv[2], lv[3])
    for dt, d1, d2 in itertools.product(np.linspace(-0.01, 0.01, 5), repeat=3):
        assert mse(t0 + dt, lv[2] + d1, lv[3] + d2) >= best - 1e-15


def test_hlm_codes_are_nearest_level_bruteforce():
    """Each code is the level nearest to y / sigma (the Lloyd-Max cells are the
    nearest-level cells); sigma = fp16(||r|| / sqrt(D)); a zero residual gets
    scale 0 and codes 0."""
    r = rng(32).standard_normal((40, 128)) * rng(33).uniform(0.01, 3.0, (40, 1))
    r[3] = 0.0
    words = O.default_sign_words()
    codes, sigma = O.quantize_hlm(r, words)
    lv, _ = O.lloyd_max_gaussian4()
    y = O.rotate(r, words)
    for i in range(r.shape[0]):
        assert sigma[i] == O.fp16_rne(np.linalg.norm(r[i]) / math.sqrt(128))
        if sigma[i] == 0:
            assert not codes[i].any()
            continue
        for d in range(128):
            u = y[i, d] / sigma[i]
            assert codes[i, d] == int(np.argmin(np.abs(u - lv)))
    assert sigma[3] == 0


def test_hlm_dequantize_elementwise():
    """r~_i = s_i * sum_j H[i, j] sigma level[c_j] / sqrt(D), by explicit loops
    over a small D with scipy's Hadamard matrix."""
    from scipy.linalg import hadamard
    D = 16
    words = [0b1010011100011101, 0, 0, 0]
    codes = rng(34).integers(0, 4, (3, D)).astype(np.uint8)
    sigma = np.array([0.5, 1.25, 0.0])
    lv, _ = O.lloyd_max_gaussian4()
    Hd = hadamard(D)
    out = O.dequantize_hlm(codes, sigma, words)
    for n in range(3):
        for i in range(D):
            s_i = -1.0 if (words[0] >> i) & 1 else 1.0
            acc = sum(Hd[i, j] * sigma[n] * lv[codes[n, j]] for j in range(D))
            assert abs(out[n, i] - s_i * acc / math.sqrt(D)) < 1e-14


def test_hlm_distortion_matches_the_gaussian_model():
    """For Gaussian residuals the relative squared error of the codec is the
    Lloyd-Max distortion 0.1175 (per coordinate, in units of sigma^2), within
    sampling error, whatever the signs."""
    r = rng(35).standard_normal((4000, 128))
    for words in (O.default_sign_words(), [0, 0, 0, 0]):
        codes, sigma = O.quantize_hlm(r, words)
        rt = O.dequantize_hlm(codes, sigma, words)
        rel = np.sum((r - rt) ** 2) / np.sum(r ** 2)
        assert abs(rel - 0.1175) < 0.004


def test_hlm_code_margin_hand_values():
    """Distance of y / sigma from the nearest of -t, 0, t, by hand through the
    inverse rotation: a residual whose rotation is sigma * (0.1, t + 0.02,
    -t - 0.3, 2.0, ...) with sigma = 1."""
    _, t = O.lloyd_max_gaussian4()
    words = [0x5, 0, 0, 0]
    D = 8
    u = np.array([0.1, t + 0.02, -t - 0.3, 2.0, -0.45, 0.0, 1.0, -2.0])
    u = u * math.sqrt(D) / np.linalg.norm(u)          # ||r|| / sqrt(D) = 1 exactly representable scale
    r = O.unrotate(u[None], words)
    sigma = np.array([1.0])
    m = O.hlm_code_margin(r, sigma, words)[0]
    want = np.minimum(np.minimum(np.abs(u + t), np.abs(u)), np.abs(u - t))
    np.testing.assert_allclose(m, want, atol=1e-13)
    assert np.all(np.isinf(O.hlm_code_margin(r, np.array([0.0]), words)))


def test_hlm_plan_hand_worked():
    """Records of the paper's codec cost D/4 + 4 = 36 bytes at D = 128, so with
    the fixed part of the affine plan R = floor((budget - fixed) / 36)."""
    pa = O.plan(8, 32768, 128, 2, 0.05, 32)
    ph = O.plan(8, 32768, 128, 2, 0.05, 32, codec=O.CODEC_HLM)
    assert O.rec_bytes(128, O.CODEC_HLM) == 36 and O.rec_bytes(128) == 48
    assert (ph.A, ph.fixed_per_side) == (pa.A, pa.fixed_per_side)
    assert ph.R_K == (ph.budget_unit - ph.fixed_per_side) // 36
    assert pa.R_K == (pa.budget_unit - pa.fixed_per_side) // 48
    assert O.side_bytes(ph, ph.R_K) <= ph.budget_unit < O.side_bytes(ph, ph.R_K + 1)
    with pytest.raises(ValueError):
        O.plan(8, 1024, 96, 2, 0.2, 32, codec=O.CODEC_HLM)


def _independent_reconstruction_hlm(c, K, V):
    from scipy.linalg import hadamard
    H, N, D = K.shape
    lv, _ = O.lloyd_max_gaussian4()
    s = np.array([-1.0 if (c.sign_words[i // 32] >> (i % 32)) & 1 else 1.0 for i in range(D)])
    Hd = hadamard(D) / math.sqrt(D)
    out = []
    for side, X in enumerate((K, V)):
        Xh = np.zeros_like(X)
        for h in range(H):
            anc = X[h, c.anchor_pos[h]]
            for t in range(N):
                v = c.gamma16[side, h, t] * anc[c.idx[side, h, t]]
                if c.flag[side, h, t]:
                    v = v + s * (Hd @ (c.sigma[side, h, t] * lv[c.codes[side, h, t].astype(int)]))
                Xh[h, t] = v
        out.append(Xh)
    return out


def test_hlm_compress_reconstruct_and_decode():
    """With the paper's codec the compressed unit's flagged tokens carry the
    codes and scale of their unquantised residual, the reconstruction equals
    an element-wise build, and decode equals SDPA over that build."""
    r = rng(38)
    H, N, D, G, n_obs, W = 2, 384, 128, 2, 16, 16
    K = bf16_exact(clustered(r, H, N, D))
    V = bf16_exact(r.standard_normal((H, N, D)) + 1.0)
    Q = bf16_exact(r.standard_normal((H * G, n_obs, D)))
    c = O.compress_unit(K, V, Q, G, n_obs, 0.2, W, 2, codec=O.CODEC_HLM)
    assert c.plan.codec == O.CODEC_HLM and 0 < c.flag[0].sum() and 0 < c.flag[1].sum()
    words = O.default_sign_words()
    codes, sigma = O.quantize_hlm(c.resid, words)
    np.testing.assert_array_equal(c.codes, np.where(c.flag[..., None], codes, 0))
    np.testing.assert_array_equal(c.sigma, np.where(c.flag, sigma, 0.0))
    Kh, Vh = O.reconstruct(c)
    Ki, Vi = _independent_reconstruction_hlm(c, K, V)
    np.testing.assert_allclose(Kh, Ki, atol=1e-12)
    np.testing.assert_allclose(Vh, Vi, atol=1e-12)
    q = bf16_exact(rng(39).standard_normal((H * G, D)))
    o = O.decode_unit(c, q)
    for h in range(H):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h * G:(h + 1) * G])[None], torch.from_numpy(Ki[h])[None], torch.from_numpy(Vi[h])[None])
        np.testing.assert_allclose(o[h * G:(h + 1) * G], ref[0].numpy(), rtol=1e-11, atol=1e-12)


def test_cover_set_check_accepts_the_oracle_and_rejects_a_swap():
    # the parity helper's round replay: the oracle's own coverage set passes
    # as exact; swapping a pick for a well-covered token fails
    from tests.parity import check_cover_set
    r = rng(70)
    N, D, W, k_s, k_u, R = 90, 16, 6, 6, 8, 3
    X = r.standard_normal((N, D))
    pooled = r.random(N - W)
    pos = O.select_anchors(pooled, N, W, k_s, k_u, mode=O.ANCHORS_COVER, X=X, rounds=R)
    ok, why = check_cover_set(X, pooled, pos, N, W, k_s, k_u, R)
    assert ok and why == "exact", why
    scored = set(np.argsort(-pooled, kind="stable")[:k_s].tolist())
    picks = [t for t in pos.tolist() if t < N - W and t not in scored]
    c, _ = O.cosine_table(X[:N - W], X[pos])
    mx = c.max(axis=1)
    outside = [t for t in range(N - W) if t not in set(pos.tolist())]
    best_covered = max(outside, key=lambda t: mx[t])
    bad = np.sort(np.array([t for t in pos.tolist() if t != picks[0]] + [best_covered]))
    ok, why = check_cover_set(X, pooled, bad, N, W, k_s, k_u, R)
    assert not ok, why


# ---------------------------------------------------------------- pre-RoPE key storage
def _rot_complex(X, base, positions):
    """R_t X_t through complex numbers: coordinate pair (i, i + D/2) as
    z = x_i + 1j x_{i+D/2}, turned by exp(1j t base^(-2i/D)) (a route
    independent of the oracle's cos/sin form)."""
    N, D = X.shape
    h = D // 2
    z = X[:, :h] + 1j * X[:, h:]
    w = np.exp(-(2.0 * np.arange(h) / D) * math.log(base))
    z = z * np.exp(1j * np.asarray(positions, dtype=np.float64)[:, None] * w[None, :])
    return np.concatenate([z.real, z.imag], axis=1)


@pytest.mark.parametrize("D,base", [(128, 500000.0), (64, 10000.0), (8, 50.0)])
def test_rope_is_an_orthogonal_rotation(D, base):
    """Pith, "Assumptions & free parameters": R_t is a per-position orthogonal
    linear map.  The rotation equals the complex-number form, preserves norms
    and inner products at one position, is the identity at position 0, and its
    matrix (from the images of the unit vectors) is orthogonal with
    determinant 1."""
    r = rng(40)
    N = 37
    X = r.standard_normal((N, D))
    pos = r.integers(0, 200000, N)
    Y = O.rope(X, base, pos)
    np.testing.assert_allclose(Y, _rot_complex(X, base, pos), rtol=0, atol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(Y, axis=1), np.linalg.norm(X, axis=1), rtol=1e-13)
    np.testing.assert_array_equal(O.rope(X, base, np.zeros(N)), X)
    for t in (1, 977, 131071):
        Rt = O.rope(np.eye(D), base, np.full(D, t)).T     # column k = R_t e_k
        np.testing.assert_allclose(Rt.T @ Rt, np.eye(D), atol=1e-12)
        assert np.linalg.det(Rt) == pytest.approx(1.0, abs=1e-9)


def test_rope_closed_forms():
    """The first pair turns by t radians (theta_0 = 1) and the pair D/4 by
    t / sqrt(base) (theta_{D/4} = base^(-1/2)); default keys sit at
    positions 0..N-1."""
    D, base, N = 16, 10000.0, 9
    X = np.zeros((N, D))
    X[:, 0] = 1.0
    X[:, D // 4] = 1.0
    Y = O.rope(X, base)
    t = np.arange(N)
    np.testing.assert_allclose(Y[:, 0], np.cos(t), atol=1e-15)
    np.testing.assert_allclose(Y[:, D // 2], np.sin(t), atol=1e-15)
    np.testing.assert_allclose(Y[:, D // 4], np.cos(t / 100.0), atol=1e-15)
    np.testing.assert_allclose(Y[:, D // 4 + D // 2], np.sin(t / 100.0), atol=1e-15)


def test_rope_depends_on_relative_position_only():
    """<R_m q, R_t k> = <q, R_{t-m} k>: the logit of a rotated query and key
    depends on their offset alone."""
    r = rng(41)
    D, base = 64, 500000.0
    for _ in range(20):
        q, k = r.standard_normal((1, D)), r.standard_normal((1, D))
        m, t = r.integers(0, 100000, 2)
        lhs = float((O.rope(q, base, [m]) @ O.rope(k, base, [t]).T)[0, 0])
        rhs = float((q @ O.rope(k, base, [t - m]).T)[0, 0])
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9)


def _rope_unit(seed, H=2, G=2, N=300, D=32, n_obs=6, W=6):
    r = rng(seed)
    K = bf16_exact(clustered(r, H, N, D, ndir=6))
    V = bf16_exact(r.standard_normal((H, N, D)) + 0.5)
    Q = bf16_exact(r.standard_normal((H * G, n_obs, D)) * 2.0)
    return K, V, Q


def test_rope_compress_attends_rotated_keys_and_stores_prerope_ones():
    """Pre-RoPE storage: the observation-window attention (score, p, o) is the
    one over the rotated keys, while the anchors, the assignment, gamma and the
    residual are those of the stored keys (the same as without rotation for the
    same anchors); the key utility uses the residual rotated at the token's
    position."""
    K, V, Q = _rope_unit(42)
    base, G, n_obs, W = 10000.0, 2, 6, 6
    c = O.compress_unit(K, V, Q, G, n_obs, 0.3, W, 2, rope_theta=base)
    Krot = np.stack([_rot_complex(K[h], base, np.arange(K.shape[1])) for h in range(K.shape[0])])
    post = O.compress_unit(Krot, V, Q, G, n_obs, 0.3, W, 2)
    np.testing.assert_allclose(c.score, post.score, rtol=1e-9, atol=1e-15)
    np.testing.assert_array_equal(c.anchor_pos, post.anchor_pos)
    plain = O.compress_unit(K, V, Q, G, n_obs, 0.3, W, 2, anchor_override=c.anchor_pos)
    for a, b in [(c.idx, plain.idx), (c.gamma, plain.gamma), (c.resid, plain.resid)]:
        np.testing.assert_array_equal(a, b)
    # the stored anchors are the pre-RoPE rows
    np.testing.assert_array_equal(c.anchors[0], K[np.arange(2)[:, None], c.anchor_pos])
    # key utility: sum_j p_jt |<q_j, R_t r_t>| / sqrt(D) ||v_t - o_j||, with
    # R_t r_t built through the complex form
    D = K.shape[2]
    for h in range(2):
        Qh = Q[h * G:(h + 1) * G].reshape(G * n_obs, D)
        Rr = _rot_complex(c.resid[0, h], base, np.arange(K.shape[1]))
        P, Oo = c.P[h], c.O[h]
        for t in (3, 50, 151):
            if not np.isfinite(c.u[0, h, t]):
                continue
            want = sum(P[j, t] * abs(Qh[j] @ Rr[t]) / math.sqrt(D) * np.linalg.norm(V[h, t] - Oo[j])
                       for j in range(G * n_obs))
            assert c.u[0, h, t] == pytest.approx(want, rel=1e-10)


def test_rope_utility_equals_first_order_output_change():
    """With pre-RoPE storage the attention sees R_t k_t: moving the stored k_t
    by eps*r moves logit t by eps<q, R_t r>/sqrt(D), so the first-order output
    change is eps alpha_t <q, R_t r>/sqrt(D) (v_t - o); its norm summed over the
    observation queries is the key utility."""
    r = rng(43)
    N, D, GQ, base = 20, 16, 3, 100.0
    K = r.standard_normal((N, D))
    V = r.standard_normal((N, D))
    Qo = r.standard_normal((GQ, D))
    rK = r.standard_normal((N, D)) * 0.3
    P, Oo = O.obs_attention(Qo, O.rope(K, base), V, n_obs=1)
    uK, _ = O.utilities(P, Oo, Qo, V, O.rope(rK, base), rK, np.ones(N, bool))
    eps = 1e-6
    for t in range(N):
        fd = 0.0
        for j in range(GQ):
            Kp, Km = K.copy(), K.copy()
            Kp[t] += eps * rK[t]
            Km[t] -= eps * rK[t]
            fd += np.linalg.norm((_attn(Qo[j], _rot_complex(Kp, base, np.arange(N)), V) -
                                  _attn(Qo[j], _rot_complex(Km, base, np.arange(N)), V)) / (2 * eps))
        assert uK[t] == pytest.approx(fd, rel=1e-6)


def test_rope_decode_distributes_over_the_decomposition():
    """Pith, "Referee Report" (RoPE distributing over the decomposition): decode
    over a pre-RoPE cache attends R_t(h(gamma) k_a + r~_t) = h(gamma) R_t k_a
    + R_t r~_t, the anchor turned at the token's position (not the anchor's);
    checked against SDPA over keys built that way element by element."""
    r = rng(44)
    H, G, N, D, n_obs, W, base = 2, 2, 160, 32, 4, 4, 10000.0
    K = bf16_exact(clustered(r, H, N, D, ndir=4))
    V = bf16_exact(r.standard_normal((H, N, D)) + 1.0)
    Q = bf16_exact(r.standard_normal((H * G, n_obs, D)))
    c = O.compress_unit(K, V, Q, G, n_obs, 0.2, W, 2, rope_theta=base)
    assert 0 < c.flag[0].sum()
    Ki, Vi = _independent_reconstruction(c, K, V)
    q = bf16_exact(r.standard_normal((H * G, D)) * 2.0)
    o = O.decode_unit(c, q)
    for h in range(H):
        xa = K[h, c.anchor_pos[h]][c.idx[0, h]]
        rt = Ki[h] - c.gamma16[0, h][:, None] * xa
        Kr = c.gamma16[0, h][:, None] * _rot_complex(xa, base, np.arange(N)) + _rot_complex(rt, base, np.arange(N))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[h * G:(h + 1) * G])[None], torch.from_numpy(Kr)[None], torch.from_numpy(Vi[h])[None])
        np.testing.assert_allclose(o[h * G:(h + 1) * G], ref[0].numpy(), rtol=1e-10, atol=1e-12)


def test_rope_all_anchor_cache_is_exact_rotary_attention_and_tail_as_given():
    """Every token an anchor: decode equals attention over the rotated keys; a
    tail appended after compression is attended as given (its keys already
    rotated)."""
    r = rng(45)
    H, G, N, D, T, base = 2, 2, 64, 32, 5, 500000.0
    K = bf16_exact(r.standard_normal((H, N, D)))
    V = bf16_exact(r.standard_normal((H, N, D)))
    Q = bf16_exact(r.standard_normal((H * G, 4, D)))
    c = O.compress_unit(K, V, Q, G, 4, 1.5, N, 2, rope_theta=base)
    assert c.plan.A == N and c.flag.sum() == 0
    q = bf16_exact(r.standard_normal((H * G, D)) * 3.0)
    Kt = bf16_exact(r.standard_normal((H, T, D)))
    Vt = bf16_exact(r.standard_normal((H, T, D)))
    o = O.decode_unit(c, q)
    ot = O.decode_unit_tail(c, q, Kt, Vt)
    for h in range(H):
        Kr = _rot_complex(K[h], base, np.arange(N))
        np.testing.assert_allclose(o[h * G:(h + 1) * G], O.attention(q[h * G:(h + 1) * G], Kr, V[h]), rtol=1e-9)
        np.testing.assert_allclose(ot[h * G:(h + 1) * G],
                                   O.attention(q[h * G:(h + 1) * G], np.concatenate([Kr, Kt[h]]),
                                               np.concatenate([V[h], Vt[h]])), rtol=1e-9)


def test_rope_theorem1_bound_holds():
    """Theorem 1 with the rotated keys: ||R_t K_t - R_t K^_t|| = ||K_t - K^_t||,
    so the bound holds with the stored-space key error."""
    K, V, Q = _rope_unit(46, N=400)
    base = 10000.0
    c = O.compress_unit(K, V, Q, 2, 6, 0.15, 6, 2, rope_theta=base)
    Kh, Vh = O.reconstruct(c)
    r = rng(47)
    for h in range(2):
        Kr = O.rope(K[h], base)
        Khr = O.rope(Kh[h], base)
        np.testing.assert_allclose(np.linalg.norm(Kr - Khr, axis=1), np.linalg.norm(K[h] - Kh[h], axis=1),
                                   rtol=1e-9, atol=1e-12)
        for _ in range(10):
            q = r.standard_normal(K.shape[2]) * 3
            err, val, key, val2, key2 = O.theorem1_terms(q, Kr, V[h], Khr, Vh[h])
            tol = 1e-12 * (1 + np.linalg.norm(V[h]))
            assert err <= val + key + tol and err <= val2 + key2 + tol
