"""Helpers for comparing the HIP path with the CPU oracle (tests only).

The comparison is conditioned: where the GPU takes a discrete decision that
differs from the oracle's (anchor set, nearest anchor, residual selection),
the difference is first checked against the stated tie margins (1e-5
relative on the pooled score, the top-2 cosine and the utility cut) and the
oracle then continues from the GPU's decision, so later stages are compared
on the same footing.
"""
from __future__ import annotations

import copy
import itertools
import math

import numpy as np
import torch

from oracle import anchorkv_oracle as O

MARGIN = 1e-5      # relative tie margin for discrete decisions
OUT_RTOL = 1e-3    # decode output: ||o_gpu - o_ref|| <= 1e-3 ||o_ref|| per (unit, q-head)


def oracle_params(params):
    """The library's method parameters as the oracle's keyword arguments:
    pre-RoPE keys (rope = 1, rope_theta) become rope_theta (the rotary base,
    500000 by default), everything else is passed through."""
    prm = dict(params or {})
    rope = prm.pop("rope", 0)
    base = prm.pop("rope_theta", 500000.0)
    if rope:
        prm["rope_theta"] = float(np.float32(base))
    return prm


def bits_f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_bits_to_f64(b):
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def anchors_to_storage(x, dtype_code):
    x32 = np.asarray(x, dtype=np.float32)
    if dtype_code == 1:
        return (x32.view(np.uint32) >> 16).astype(np.uint16)
    return x32


def storage_to_f64(a, dtype_code):
    if dtype_code == 1:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def oracle_arrays(c: O.Compressed, dtype_code):
    """Oracle compressed unit -> arrays for the host packer (the Hadamard /
    Lloyd-Max codec's scale goes in entry 0 of each token's scale16)."""
    scale16, zero16 = bits_f16(c.scale), bits_f16(c.zero)
    if c.codec == O.CODEC_HLM:
        scale16 = np.zeros(c.scale.shape, np.uint16)
        scale16[..., 0] = bits_f16(c.sigma)
        zero16 = np.zeros(c.zero.shape, np.uint16)
    return dict(positions=c.anchor_pos.astype(np.int32),
                anchors_k=anchors_to_storage(c.anchors[0], dtype_code),
                anchors_v=anchors_to_storage(c.anchors[1], dtype_code),
                idx=c.idx.astype(np.int32), gamma16=bits_f16(c.gamma16), flag=c.flag.astype(np.uint8),
                codes=c.codes.astype(np.uint8), scale16=scale16, zero16=zero16)


def fp16_midpoint_distance(x):
    """Distance of x from the nearest fp16 rounding midpoint, in units of the
    fp16 spacing at x (0.5 = exactly on a representable value)."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -24)))
    e = np.maximum(e, -14)
    ulp = 2.0 ** (e - 10)
    frac = ax / ulp - np.floor(ax / ulp)
    return np.abs(frac - 0.5)


def check_anchor_set(pooled, gpu_pos, N, W, k_s, k_u):
    """True if gpu_pos equals the oracle anchor set, or differs only by scored
    picks inside the tie band around the k_s-th largest pooled score."""
    orc = O.select_anchors(pooled, N, W, k_s, k_u)
    if np.array_equal(orc, np.sort(gpu_pos)):
        return True, "exact"
    if k_s == 0:
        return False, "uniform/window mismatch"
    L = N - W
    cut = np.sort(pooled)[::-1][k_s - 1]
    band = np.nonzero(np.abs(pooled - cut) <= MARGIN * abs(cut))[0]
    certain = np.nonzero(pooled > cut + MARGIN * abs(cut))[0]
    need = k_s - certain.size
    gset = set(np.asarray(gpu_pos).tolist())
    cand = [t for t in band.tolist() if t in gset]
    if need < 0 or len(cand) > 12:
        return False, "band too large"
    for sub in itertools.combinations(cand, need):
        scored = np.sort(np.concatenate([certain, np.array(sub, dtype=np.int64)]))
        taken = np.zeros(L, bool)
        taken[scored] = True
        rest = np.nonzero(~taken)[0]
        M = rest.size
        uni = np.array([rest[((2 * i + 1) * M) // (2 * k_u)] for i in range(k_u)], dtype=np.int64)
        full = np.sort(np.concatenate([scored, uni, np.arange(L, N)]))
        if np.array_equal(full, np.sort(gpu_pos)):
            return True, "tie-band"
    return False, "no tie-band explanation"


def check_cover_set(X, pooled, gpu_pos, N, W, k_s, k_u, rounds):
    """Coverage anchors of one head (reading R23): the GPU set must hold the
    window, the scored set (the k_s largest pooled scores, inside the tie band
    at the cut) and k_u picks that replay round by round: in each round the
    GPU's picks are the b lowest largest-cosines among its remaining picks,
    and no candidate left out has a largest cosine below the round's highest
    pick by more than the tie margin (relative).  X: the head's keys.
    Returns (ok, why)."""
    L = N - W
    g = np.sort(np.asarray(gpu_pos, dtype=np.int64))
    if not np.array_equal(g[g >= L], np.arange(L, N)):
        return False, "window"
    nonw = g[g < L]
    if nonw.size != k_s + k_u:
        return False, "count"
    order = np.lexsort((np.arange(L), -pooled))
    scored = set(order[:k_s].tolist())
    if k_s > 0 and not scored <= set(nonw.tolist()):
        # scored decisions inside the tie band: the GPU's scored set is the
        # k_s of its anchors with the largest pooled scores
        cut = pooled[order[k_s - 1]]
        miss = [t for t in scored if t not in set(nonw.tolist())]
        if any(abs(pooled[t] - cut) > MARGIN * abs(cut) for t in miss):
            return False, "scored set outside the tie band"
        gs = nonw[np.lexsort((nonw, -pooled[nonw]))][:k_s]
        scored = set(gs.tolist())
    cur = sorted(scored) + list(range(L, N))
    remaining = sorted(set(nonw.tolist()) - scored)
    exact_rounds = True
    for b in O.cover_rounds_of(k_u, rounds):
        c, _ = O.cosine_table(X[:L], X[np.asarray(cur, dtype=np.int64)])
        mx = c.max(axis=1)
        rem = np.asarray(remaining, dtype=np.int64)
        chosen = rem[np.lexsort((rem, mx[rem]))][:b]
        top = mx[chosen].max()
        cand = np.ones(L, dtype=bool)
        cand[np.asarray([t for t in cur if t < L], dtype=np.int64)] = False
        cand[chosen] = False
        if cand.any():
            low = mx[cand].min()
            if low < top - MARGIN * max(abs(top), 1e-30):
                return False, f"round pick above a left-out candidate ({top} vs {low})"
        pos_c = np.nonzero(~np.isin(np.arange(L), np.asarray(cur)))[0]
        want = pos_c[np.lexsort((pos_c, mx[pos_c]))][:b]
        exact_rounds &= set(want.tolist()) == set(chosen.tolist())
        cur += chosen.tolist()
        remaining = [t for t in remaining if t not in set(chosen.tolist())]
    return True, "exact" if exact_rounds else "tie-band"


def compare_unit(K, V, Q, G, n_obs, theta, W, e, gpu, taps=None, q=None, o_gpu=None, report=None, params=None):
    """Compare one unit.  K, V, Q: float64 inputs; gpu: unpacked GPU arrays;
    taps: optional dict of GPU workspace arrays for this unit (score [H,N],
    util [2,H,N]); q [H*G, D] float64 and o_gpu [H*G, D] for decode;
    params: the method's parameters other than theta and window (anchor_div,
    rho, pool) when they differ from the pages' values."""
    rep = {} if report is None else report
    prm = oracle_params(params)
    H, N, D = K.shape
    dtype_code = 1 if e == 2 else 2
    p = O.plan(H, N, D, e, theta, W,
               **{k: v for k, v in prm.items() if k in ("anchor_div", "rho", "pool_kv_jointly", "codec")})
    hlm = prm.get("codec", O.CODEC_AFFINE) == O.CODEC_HLM
    words = tuple(prm.get("sign_words", O.default_sign_words()))
    # 1. anchors (per head), from the oracle's own pooled score
    first = O.compress_unit(K, V, Q, G, n_obs, theta, W, e, **prm)
    if taps is not None and "score" in taps:
        s_err = np.max(np.abs(taps["score"] - first.score) / np.maximum(first.score, 1e-30 + first.score.max() * 1e-6))
        rep["score_max_rel_err"] = float(s_err)
        assert s_err < 1e-4, f"score mismatch {s_err}"
    gpos = gpu["positions"].astype(np.int64)
    # anchors are stored exactly: the cache rows equal the inputs at the positions
    for s_, X in enumerate((K, V)):
        ga = storage_to_f64(gpu["anchors_k" if s_ == 0 else "anchors_v"], dtype_code)
        want = X[np.arange(H)[:, None], gpos]
        bad = np.nonzero(np.any(ga != want, axis=-1))
        assert bad[0].size == 0, f"side {s_}: {bad[0].size} stored anchor rows differ, first (head, idx) {bad[0][:3], bad[1][:3]}"
    exact = 0
    cover = prm.get("anchor_mode", O.ANCHORS_UNIFORM) == O.ANCHORS_COVER
    for h in range(H):
        if cover:
            ok, why = check_cover_set(K[h], first.pooled[h], gpos[h], N, W, p.k_s, p.k_u,
                                      prm.get("cover_rounds", O.COVER_ROUNDS))
        else:
            ok, why = check_anchor_set(first.pooled[h], gpos[h], N, W, p.k_s, p.k_u)
        assert ok, f"anchor set head {h}: {why}"
        exact += why == "exact"
    rep["anchor_heads_exact"] = exact
    # 2. assignments (conditioned on the GPU anchors)
    second = O.compress_unit(K, V, Q, G, n_obs, theta, W, e, anchor_override=gpos, **prm)
    gidx = gpu["idx"].astype(np.int64)
    mism = gidx != second.idx
    if mism.any():
        bad = mism & (second.margin >= MARGIN)
        assert not bad.any(), f"{int(bad.sum())} assignments differ outside the tie margin"
    rep["assign_mismatch_excused"] = int(mism.sum())
    # 3. gamma (fp16), utilities and residual choice (conditioned on GPU assignments)
    third = O.compress_unit(K, V, Q, G, n_obs, theta, W, e, anchor_override=gpos, idx_override=gidx, **prm)
    g16 = f16_bits_to_f64(gpu["gamma16"])
    near = fp16_midpoint_distance(third.gamma) < 1e-3
    diff = (g16 != third.gamma16) & ~near
    assert not diff.any(), f"{int(diff.sum())} fp16 gammas differ away from rounding midpoints"
    if taps is not None and "util" in taps:
        u_o = np.where(np.isfinite(third.u), third.u, -1.0)
        u_g = taps["util"]
        scale = np.maximum(np.abs(u_o), 1e-30)
        rel = np.abs(u_g - u_o) / scale
        elig = u_o >= 0
        rep["util_max_rel_err"] = float(rel[elig].max()) if elig.any() else 0.0
    gflag = gpu["flag"].astype(bool)
    # the rankings: per side, or one over both sides (joint)
    lists = [(third.u.reshape(2 * H, N), third.flag.reshape(2 * H, N), gflag.reshape(2 * H, N), p.R_total, "joint")] \
        if p.joint else [(third.u[s], third.flag[s], gflag[s], R, str(s)) for s, R in enumerate((p.R_K, p.R_V))]
    for u_l, of_l, gf_l, R, name in lists:
        cut = O.cut_value(u_l, R)
        dif = gf_l != of_l
        if dif.any():
            uu = u_l[dif]
            assert cut is not None and np.all(np.abs(uu - cut) <= MARGIN * abs(cut)), \
                f"ranking {name}: {int(dif.sum())} residual ids differ outside the utility margin"
        rep[f"flag_mismatch_excused_{name}"] = int(dif.sum())
        assert gf_l.sum() == R
    # 4. codes, scales, zeros on the GPU's residual set
    fourth = O.compress_unit(K, V, Q, G, n_obs, theta, W, e, anchor_override=gpos, idx_override=gidx,
                             flag_override=gflag, **prm)
    for s in range(2):
        fl = gflag[s]
        r = fourth.resid[s][fl]                       # [R, D]
        if r.shape[0] == 0:
            continue
        if hlm:
            # scale fp16(||r|| / sqrt(D)) away from fp16 rounding midpoints;
            # codes where the rotated coordinate is away from the thresholds
            codes_o, sg_o = O.quantize_hlm(r, words)
            safe_s = fp16_midpoint_distance(np.linalg.norm(r, axis=1) / math.sqrt(D)) > 1e-3
            sg_g = f16_bits_to_f64(gpu["scale16"][s][fl][:, 0])
            assert np.all((sg_g == sg_o) | ~safe_s), f"side {s}: scales differ"
            assert not gpu["zero16"][s][fl].any() and not gpu["scale16"][s][fl][:, 1:].any()
            safe_e = (O.hlm_code_margin(r, sg_o, words) > 1e-3) & safe_s[:, None]
            bad = (gpu["codes"][s][fl] != codes_o) & safe_e
            assert not bad.any(), f"side {s}: {int(bad.sum())} codes differ away from thresholds"
            rep[f"codes_checked_{s}"] = int(safe_e.sum())
            continue
        codes_o, sc_o, ze_o = O.quantize(r)
        lo = r.reshape(r.shape[0], -1, 32).min(-1)
        hi = r.reshape(r.shape[0], -1, 32).max(-1)
        safe_g = (fp16_midpoint_distance(lo) > 1e-3) & (fp16_midpoint_distance((hi - lo) / 3) > 1e-3)
        sc_g = f16_bits_to_f64(gpu["scale16"][s][fl])
        ze_g = f16_bits_to_f64(gpu["zero16"][s][fl])
        assert np.all((sc_g == sc_o) | ~safe_g), f"side {s}: scales differ"
        assert np.all((ze_g == ze_o) | ~safe_g), f"side {s}: zeros differ"
        margin = O.code_margin(r, sc_o, ze_o)
        safe_e = (margin > 1e-3) & np.repeat(safe_g, 32, axis=1)
        cg = gpu["codes"][s][fl]
        bad = (cg != codes_o) & safe_e
        assert not bad.any(), f"side {s}: {int(bad.sum())} codes differ away from boundaries"
        rep[f"codes_checked_{s}"] = int(safe_e.sum())
    # 5. decode.  The reference continues from the representation the GPU
    # stored (its fp16 gammas, codes, scales and zeros, all validated above
    # against the oracle within the rounding-boundary rules), so that an
    # excused one-step code flip is not charged to the decode kernel.
    if q is not None and o_gpu is not None:
        o_own = O.decode_unit(fourth, q)
        err_own = np.linalg.norm(o_gpu - o_own, axis=1) / np.maximum(np.linalg.norm(o_own, axis=1), 1e-30)
        rep["decode_err_vs_oracle_repr"] = float(err_own.max())
        cond = copy.copy(fourth)
        cond.gamma16 = f16_bits_to_f64(gpu["gamma16"])
        cond.codes = np.where(gflag[..., None], gpu["codes"], 0).astype(np.uint8)
        cond.scale = f16_bits_to_f64(gpu["scale16"])
        cond.zero = f16_bits_to_f64(gpu["zero16"])
        if hlm:
            cond.sigma = np.where(gflag, f16_bits_to_f64(gpu["scale16"][..., 0]), 0.0)
        o_ref = O.decode_unit(cond, q)
        err = np.linalg.norm(o_gpu - o_ref, axis=1) / np.maximum(np.linalg.norm(o_ref, axis=1), 1e-30)
        rep["decode_max_rel_err"] = float(err.max())
        assert err.max() <= OUT_RTOL, f"decode error {err.max()}"
        # The unconditioned error against the oracle's own representation is
        # the kernel's error plus the effect of the stored words that differ
        # from the oracle's, every one of which was checked above to sit at a
        # rounding boundary (fp16 gamma / scale / zero near a midpoint, a code
        # near a threshold): count them and bound the excess by their effect.
        n_g16 = int(np.sum(cond.gamma16 != fourth.gamma16))
        n_codes = int(np.sum((cond.codes != fourth.codes) & gflag[..., None]))
        n_words = int(np.sum((cond.scale != fourth.scale) & gflag[..., None]) +
                      np.sum((cond.zero != fourth.zero) & gflag[..., None])) if not hlm else \
            int(np.sum((cond.sigma != fourth.sigma) & gflag))
        repr_eff = np.linalg.norm(o_ref - o_own, axis=1) / np.maximum(np.linalg.norm(o_own, axis=1), 1e-30)
        rep["repr_diffs"] = dict(gamma16=n_g16, codes=n_codes, scales=n_words)
        rep["repr_effect"] = float(repr_eff.max())
        ratio = np.linalg.norm(o_ref, axis=1) / np.maximum(np.linalg.norm(o_own, axis=1), 1e-30)
        assert np.all(err_own <= (err * ratio + repr_eff) * (1 + 1e-9) + 1e-12)
        if n_g16 == 0 and n_codes == 0 and n_words == 0:
            assert np.array_equal(o_ref, o_own)
    return rep
