"""CPU oracle of the anchor-residual KV-cache hot path (AnchorKV).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP path
and imports nothing from it.

Plain NumPy in float64, one unit (one layer of one sequence, all of its KV
heads) at a time, dense and unblocked, in the order the method states its steps.
Inputs are the exact bf16 / f32 values, upcast to float64.

Sources (web pages on the method; cited by page title and section):
  [Pith] "Pith review of AnchorKV: Anchor-Residual KV Cache Compression"
         (pith.science), sections "What carries the argument", "What would
         settle it", "Referee Report", "Assumptions & free parameters".
  [Velox] "AnchorKV-adapted - Anchor-Residual Compression, No Eviction"
         (VeloxQuant-MLX docs), sections "The problem this solves", "The one
         setting worth tuning: anchorkv_theta", "Adaptation notes", "Evidence".
Where the pages are silent the reading taken is stated at the step (readings
R1..R20, listed together in the design notes of the repository).

Implementation contract (not on the pages, fixed for this implementation): the
default residual codec is 2-bit group-affine with one fp16 scale and one fp16
zero per 32 contiguous coordinates (residual records of D/4 + D/8 bytes); the
paper's codec (randomized Hadamard rotation + 4-level Lloyd-Max, one fp16
scale per residual, records of D/4 + 4 bytes) is the alternative; anchors cost
D*e bytes, pointers 4 bytes (2-byte index + 2-byte fp16 coefficient); decode
logits are gamma * <q, k_anchor> + <q, r~> with no RoPE by default, and with
pre-RoPE key storage (rope_theta given) <q, R_t(gamma k_anchor + r~)>.

Parity status: every function here is pinned by tests under tests/ (library
routines, closed forms, brute force, finite differences, invariants), except
the readings that no printed example fixes (R2-R8, R14-R18), which are pinned
only by being written once here and checked by brute force against this text.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

POOL = 7            # kappa, positional pooling width [Pith, "Assumptions & free parameters"]
RHO = 0.7           # scored share of non-window anchors [Pith, same]
ANCHOR_DIV = 128    # k = S/128 non-window anchors [Pith, same]
GROUP = 32          # codec group size (implementation contract)
HEADER_PER_SIDE = 128
CHUNK = 1024        # tokens per residual-offset chunk
MAX_ANCHORS = 32767  # anchor index is 15 bits (bit 15 flags a residual)
FP16_MAX = 65504.0
CODEC_AFFINE = 0    # 2-bit group-affine residual codec (implementation contract)
CODEC_HLM = 1       # the paper's codec: randomized Hadamard rotation + 4-level Lloyd-Max
SIGN_SEED = 0x416E63686F724B56   # seed of the default rotation signs (reading R22)
ANCHORS_UNIFORM = 0   # the non-scored anchors are stratified uniform picks (reading R5)
ANCHORS_COVER = 1     # coverage-optimised picks: batched furthest-point sampling (reading R23)
COVER_ROUNDS = 8      # rounds of the coverage picks (R = k_u is plain furthest-point sampling)
ROPE_THETA = 500000.0  # default base of the rotary embedding with pre-RoPE keys (reading R24)


# --------------------------------------------------------------------------
# Rounding helpers
# --------------------------------------------------------------------------
def fp16_rne(x):
    """Round float64 to the nearest fp16 value (ties to even), saturating to
    +-65504 instead of overflowing to infinity (reading R12).  Returned as
    float64.  numpy's double->half conversion is correctly rounded; the tests
    pin it against a brute-force search over all 65536 half values."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        y = x.astype(np.float16).astype(np.float64)
    return np.where(np.isinf(y) & np.isfinite(x), np.sign(x) * FP16_MAX, y)


# --------------------------------------------------------------------------
# Byte plan [Pith, "What carries the argument" (per-layer byte accounting, theta
# the only knob) and "Assumptions & free parameters" (theta, k = S/128, rho,
# W, b_a = b_gamma = 2 bytes)]; [Velox, "The one setting worth tuning"].
# --------------------------------------------------------------------------
@dataclass
class Plan:
    H: int
    N: int
    D: int
    e: int
    theta: float
    W: int
    A: int
    k_s: int
    k_u: int
    R_K: int
    R_V: int
    budget_unit: int        # floor(theta * H * N * D * e) bytes per side per unit
    fixed_per_side: int     # header share + anchors + pointers + positions + chunk offsets
    n_chunks: int
    joint: bool = False     # one residual ranking over both sides (reading R18b)
    R_total: int = 0        # residual slots of both sides together when joint
    codec: int = CODEC_AFFINE


def rec_bytes(D, codec=CODEC_AFFINE):
    """Bytes of one residual record: D/4 bytes of 2-bit codes plus, for the
    group-affine codec, an fp16 scale and zero per 32 coordinates (D/8 bytes),
    for the Hadamard / Lloyd-Max codec one fp16 scale and 2 bytes of padding
    (reading R22)."""
    return D // 4 + (D // 8 if codec == CODEC_AFFINE else 4)


def plan(H, N, D, e, theta, W, anchor_div=ANCHOR_DIV, rho=RHO, pool_kv_jointly=False, codec=CODEC_AFFINE):
    """Anchor and residual counts of one unit.

    anchor_div and rho are the method's k = S/128 and 0.7 [Pith, "Assumptions
    & free parameters"], exposed as parameters (defaults are the pages' values).

    theta is taken at float32 precision (the value the C ABI receives) and all
    byte arithmetic is done in float64 then floored.
    Per head and side the budget is B = theta * N * D * e bytes.  Anchors cost
    D*e bytes plus 2 bytes of position each (the int32 position is shared by the
    two sides), every token costs a 4-byte pointer, every 1024-token chunk a
    4-byte residual offset, and the unit header 128 bytes per side, spread over
    the H heads:
        A_max = floor((B - 4N - 4*ceil(N/1024) - 128/H) / (D*e + 2)).
    Reading R2: k = floor(N/anchor_div) non-window anchors, capped so the
    anchors fit the budget and so that there are enough non-window tokens:
        k_nw = max(0, min(floor(N/anchor_div), A_max - W, N - W)).
    Reading R3: the window is not part of k: A = W + k_nw.
    Reading R4: k_s = floor(rho * k_nw) scored (float64), k_u = k_nw - k_s uniform.
    Residual slots per side per unit (pooled over heads; reading R16):
        R = min(H*(N-A), floor((floor(theta*H*N*D*e) - fixed) / rec)),
    rec = rec_bytes(D, codec) (D/4 + D/8 for the group-affine codec).
    With pool_kv_jointly (reading R18b: residuals go to the best token-sides,
    [Pith] "Referee Report", 17.3 % of token-sides) the two sides share what
    their budgets leave after the fixed parts:
        R_total = min(2*H*(N-A), floor(2*(floor(theta*H*N*D*e) - fixed) / rec)).
    """
    if not (N >= 1 and 1 <= W <= N and D % GROUP == 0 and H >= 1):
        raise ValueError("bad shape")
    th = float(np.float32(theta))
    C = -(-N // CHUNK)
    B = th * float(N * D * e)
    A_max = math.floor((B - 4.0 * N - 4.0 * C - HEADER_PER_SIDE / H) / (D * e + 2))
    if A_max < W:
        raise ValueError("budget too small for the window anchors and pointers")
    k_nw = max(0, min(N // anchor_div, A_max - W, N - W))
    k_s = math.floor(rho * k_nw)
    k_u = k_nw - k_s
    A = W + k_nw
    if A > MAX_ANCHORS:
        raise ValueError("too many anchors for a 15-bit index")
    budget_unit = math.floor(th * float(H * N * D * e))
    fixed = HEADER_PER_SIDE + H * (A * D * e + 4 * N + 2 * A + 4 * C)
    if codec not in (CODEC_AFFINE, CODEC_HLM) or (codec == CODEC_HLM and D & (D - 1)):
        raise ValueError("bad codec")
    rec = rec_bytes(D, codec)
    R = max(0, min(H * (N - A), (budget_unit - fixed) // rec))
    R_total = max(0, min(2 * H * (N - A), (2 * (budget_unit - fixed)) // rec)) if pool_kv_jointly else 0
    return Plan(H, N, D, e, th, W, A, k_s, k_u, R, R, budget_unit, fixed, C, bool(pool_kv_jointly), R_total, codec)


def side_bytes(p: Plan, R: int) -> int:
    """Bytes one side of one unit occupies: fixed part + R residual records."""
    return p.fixed_per_side + R * rec_bytes(p.D, p.codec)


def unit_bytes(p: Plan, R_K: int, R_V: int) -> int:
    """Bytes of both sides of one unit with R_K and R_V residual records."""
    return side_bytes(p, R_K) + side_bytes(p, R_V)


# --------------------------------------------------------------------------
# Step 1: observation-window attention [Pith, "What carries the argument"
# (SnapKV observation-window score) and "Assumptions & free parameters"
# (last W tokens' attention pooled over GQA query heads)].
# --------------------------------------------------------------------------
def obs_attention(Qh, Kh, Vh, n_obs):
    """Causal softmax attention of one KV head's observation queries.

    Qh: [GQ, D] rows ordered (q-head g, obs index j) -> row g*n_obs + j.
    Query j sits at position N - n_obs + j and sees keys t <= N - n_obs + j
    (reading R8).  Returns P [GQ, N] (probabilities), O = P @ V [GQ, D].
    """
    GQ, D = Qh.shape
    N = Kh.shape[0]
    S = (Qh @ Kh.T) / math.sqrt(D)
    j = np.arange(GQ) % n_obs
    visible = np.arange(N)[None, :] <= (N - n_obs + j)[:, None]
    S = np.where(visible, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    P = E / E.sum(axis=1, keepdims=True)
    return P, P @ Vh


# --------------------------------------------------------------------------
# Step 2: anchor score and positional pooling [Pith, "What carries the
# argument"; "Assumptions & free parameters" (pooling width kappa = 7, pooled
# over GQA query heads)].
# --------------------------------------------------------------------------
def anchor_score(P, W, pool=POOL):
    """score_t = sum over the head's observation queries of P[:, t] (reading R7),
    for every t; pooled_t = sum of score_u over |u - t| <= pool // 2 and
    u < N - W (reading R6: windowed sum = zero-padded mean over the odd width
    pool, 7 on the pages), for t < N - W."""
    N = P.shape[1]
    score = P.sum(axis=0)
    L = N - W
    half = pool // 2
    pooled = np.zeros(L)
    for t in range(L):
        lo, hi = max(0, t - half), min(L, t + half + 1)
        pooled[t] = score[lo:hi].sum()
    return score, pooled


def cover_rounds_of(k_u, rounds):
    """Round sizes of the coverage picks: R = min(rounds, k_u) rounds, round r
    takes floor(k_u (r+1) / R) - floor(k_u r / R) picks."""
    R = max(1, min(rounds, k_u))
    return [k_u * (r + 1) // R - k_u * r // R for r in range(R)] if k_u > 0 else []


def cover_picks(X, base_pos, L, k_u, rounds=COVER_ROUNDS, picks_override=None):
    """Coverage-optimised anchor picks [Pith, "Reading between the lines":
    anchors placed for coverage, by k-means or furthest-point picks, in place
    of the uniform ones], read as batched furthest-point sampling on the key
    side (reading R23): starting from the anchors base_pos, round r adds the
    b_r positions t < L that are not anchors yet with the lowest maximum signed
    cosine to the current anchors (cosine_table: 0 where a norm is 0), ties to
    the lower position.  With rounds >= k_u every round adds one position:
    plain furthest-point sampling.

    Returns (picks in round order, per-round margins): the margin of a round
    is (m_(b+1) - m_(b)) / max(|m_(b+1)|, |m_(b)|) for the b-th and (b+1)-th
    lowest maxima of that round (inf when no candidate is left out), the gap
    the tie rule compares with 1e-5.
    picks_override: the picks of another implementation in round order; each
    round then continues from those (a parity test checks them first).
    """
    cur = [int(t) for t in base_pos]
    picks, margins = [], []
    k = 0
    for b in cover_rounds_of(k_u, rounds):
        c, _ = cosine_table(X[:L], X[np.asarray(cur, dtype=np.int64)])
        mx = c.max(axis=1)
        cand = np.ones(L, dtype=bool)
        cur_a = np.asarray(cur, dtype=np.int64)
        cand[cur_a[cur_a < L]] = False
        pos = np.nonzero(cand)[0]
        order = pos[np.lexsort((pos, mx[pos]))]         # by (max cosine, position)
        new = order[:b]
        if order.size > b:
            m0, m1 = mx[order[b - 1]], mx[order[b]]
            den = max(abs(m0), abs(m1))
            margins.append((m1 - m0) / den if den > 0 else 0.0)
        else:
            margins.append(np.inf)
        if picks_override is not None:
            new = np.asarray(picks_override[k:k + b], dtype=np.int64)
        k += b
        picks.extend(int(t) for t in new)
        cur.extend(int(t) for t in new)
    return np.asarray(picks, dtype=np.int64), np.asarray(margins)


def select_anchors(pooled, N, W, k_s, k_u, mode=ANCHORS_UNIFORM, X=None, rounds=COVER_ROUNDS, picks_override=None):
    """Anchor positions, ascending (reading R9: the anchor index is the rank).

    * window: the last W positions [Pith, "Assumptions & free parameters"];
    * scored: the k_s largest pooled scores, ties to the lower position;
    * uniform (reading R5): with c the remaining non-window positions in
      ascending order (M of them), take c[floor((2i+1) * M / (2 k_u))], i < k_u;
    * or, with mode ANCHORS_COVER, k_u coverage picks over the keys X
      (cover_picks, starting from the scored and window anchors).
    """
    L = N - W
    order = np.lexsort((np.arange(L), -pooled))   # by (-pooled, position)
    scored = np.sort(order[:k_s])
    if mode == ANCHORS_COVER:
        base = np.concatenate([scored, np.arange(L, N)])
        picks, _ = cover_picks(X, base, L, k_u, rounds, picks_override)
        return np.sort(np.concatenate([base, picks])).astype(np.int64)
    taken = np.zeros(L, dtype=bool)
    taken[scored] = True
    rest = np.nonzero(~taken)[0]
    M = rest.size
    uni = np.array([rest[((2 * i + 1) * M) // (2 * k_u)] for i in range(k_u)], dtype=np.int64)
    pos = np.concatenate([scored, uni, np.arange(L, N)])
    return np.sort(pos).astype(np.int64)


# --------------------------------------------------------------------------
# Steps 5-6: nearest-anchor assignment and projection [Pith, "What carries the
# argument": gamma_i = <x_i, x_a>/||x_a||^2, x^_i = gamma_i x_a + r~_i; nearest
# anchor by cosine similarity]; [Velox, "Evidence" (anchors reconstruct with
# coefficient 1 and zero residual; projection + residual is exact)].
# --------------------------------------------------------------------------
def cosine_table(X, anchors_x):
    """c[t, a] = <x_t, x_a> / (||x_t|| ||x_a||), 0 where a norm is 0."""
    dots = X @ anchors_x.T
    nx = np.linalg.norm(X, axis=1)
    na = np.linalg.norm(anchors_x, axis=1)
    den = nx[:, None] * na[None, :]
    with np.errstate(invalid="ignore", divide="ignore"):
        c = np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)
    return c, dots


def assign(X, anchor_pos, idx_override=None):
    """Per token: anchor index a(t), float64 gamma, fp16 gamma, residual r.

    Non-anchor tokens take the highest signed cosine (reading R11), lowest
    anchor index on ties.  Anchor tokens are forced onto themselves with
    gamma = 1 and r = 0 (reading R10).  gamma = 0 when ||x_a|| = 0.
    r = x - gamma * x_a uses the unrounded gamma (reading R13); the stored
    coefficient is fp16(gamma), ties to even (reading R12).
    idx_override: an externally chosen assignment to continue from (used by
    the parity tests after they have checked it is within the tie margin).
    Returns dict(idx, gamma, gamma16, r, margin) where margin is the relative
    gap (c1 - c2)/|c1| between the best and second-best cosine.
    """
    N, D = X.shape
    A = anchor_pos.size
    ax = X[anchor_pos]
    c, dots = cosine_table(X, ax)
    idx = np.argmax(c, axis=1)            # first maximum = lowest index
    if A > 1:
        part = np.sort(c, axis=1)
        c1, c2 = part[:, -1], part[:, -2]
        with np.errstate(invalid="ignore", divide="ignore"):
            margin = np.where(np.abs(c1) > 0, (c1 - c2) / np.abs(np.where(c1 == 0, 1, c1)), 0.0)
    else:
        margin = np.full(N, np.inf)
    is_anchor = np.full(N, -1, dtype=np.int64)
    is_anchor[anchor_pos] = np.arange(A)
    if idx_override is not None:
        idx = np.asarray(idx_override, dtype=np.int64).copy()
    idx = np.where(is_anchor >= 0, is_anchor, idx)
    margin = np.where(is_anchor >= 0, np.inf, margin)
    xa = ax[idx]
    na2 = (xa * xa).sum(axis=1)
    d = (X * xa).sum(axis=1)
    gamma = np.where(na2 > 0, d / np.where(na2 > 0, na2, 1.0), 0.0)
    gamma = np.where(is_anchor >= 0, 1.0, gamma)
    r = X - gamma[:, None] * xa
    r[is_anchor >= 0] = 0.0
    return dict(idx=idx, gamma=gamma, gamma16=fp16_rne(gamma), r=r, margin=margin,
                is_anchor=is_anchor >= 0)


# --------------------------------------------------------------------------
# Step 7: first-order attention-output error utility [Pith, "What carries the
# argument" (key-induced and value-induced channels), "Assumptions & free
# parameters" (first-order softmax expansion, d alpha_t/d s_u =
# alpha_t (delta_tu - alpha_u); incoherence model making it additive)].
# Key channel p * |<q, dk>| / sqrt(D) * ||v - o||, value channel p * ||dv||,
# summed over the observation queries; dk, dv = the residuals a token would
# lose without a residual slot (reading R15).
# --------------------------------------------------------------------------
def utilities(P, O, Qh, V, rK, rV, eligible):
    GQ, D = Qh.shape
    qr = (Qh @ rK.T) / math.sqrt(D)                              # [GQ, N]
    vo = np.empty_like(P)                                        # ||v_t - o_j||
    for j in range(GQ):
        vo[j] = np.linalg.norm(V - O[j][None, :], axis=1)
    uK = (P * np.abs(qr) * vo).sum(axis=0)
    uV = P.sum(axis=0) * np.linalg.norm(rV, axis=1)
    uK = np.where(eligible, uK, -np.inf)
    uV = np.where(eligible, uV, -np.inf)
    return uK, uV


# --------------------------------------------------------------------------
# Steps 8-9: residual allocation under the byte budget [Pith, "What carries the
# argument" (residuals where reconstruction error most changes the output);
# Figure 11 (budget share per KV head); Velox, "Evidence" (budget pooled across
# heads)].  Greedy by utility, which is optimal for equal-cost additive items.
# --------------------------------------------------------------------------
def allocate(u, R):
    """u: [H, N] with -inf for ineligible items.  Returns a bool mask [H, N] of
    the R items with the largest u, ties to the lower head, then the lower
    position (reading R16)."""
    H, N = u.shape
    flat = u.reshape(-1)
    hh = np.repeat(np.arange(H), N)
    tt = np.tile(np.arange(N), H)
    order = np.lexsort((tt, hh, -flat))
    order = order[np.isfinite(flat[order])][:R]
    mask = np.zeros(H * N, dtype=bool)
    mask[order] = True
    return mask.reshape(H, N)


def cut_value(u, R):
    """The R-th largest eligible utility (the selection threshold), or None."""
    flat = u.reshape(-1)
    flat = flat[np.isfinite(flat)]
    if R == 0 or flat.size == 0:
        return None
    return np.sort(flat)[::-1][min(R, flat.size) - 1]


# --------------------------------------------------------------------------
# Step 10: 2-bit group-affine residual codec (implementation contract: one fp16
# scale and one fp16 zero per 32-element group; reading R14 for the details).
# --------------------------------------------------------------------------
def quantize(r):
    """r: [..., D].  Per group of 32 contiguous coordinates:
    zero = fp16(min), scale = fp16((max - min)/3),
    code = clamp(round_half_even((r - zero)/scale), 0, 3), code = 0 if scale = 0.
    Returns (codes uint8 [..., D], scale [..., D/32], zero [..., D/32]) with
    scale and zero as float64 values of the fp16 numbers."""
    sh = r.shape
    D = sh[-1]
    g = r.reshape(sh[:-1] + (D // GROUP, GROUP))
    lo = g.min(axis=-1)
    hi = g.max(axis=-1)
    zero = fp16_rne(lo)
    scale = fp16_rne((hi - lo) / 3.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.rint((g - zero[..., None]) / np.where(scale > 0, scale, 1.0)[..., None])
    q = np.clip(q, 0, 3)
    q = np.where((scale > 0)[..., None], q, 0)
    return q.reshape(sh).astype(np.uint8), scale, zero


def dequantize(codes, scale, zero):
    sh = codes.shape
    D = sh[-1]
    g = codes.reshape(sh[:-1] + (D // GROUP, GROUP)).astype(np.float64)
    return (zero[..., None] + scale[..., None] * g).reshape(sh)


def code_margin(r, scale, zero):
    """Distance of (r - zero)/scale from the nearest rounding boundary (x.5);
    +inf where scale = 0.  Used to skip boundary cases in parity checks."""
    sh = r.shape
    D = sh[-1]
    g = r.reshape(sh[:-1] + (D // GROUP, GROUP))
    with np.errstate(invalid="ignore", divide="ignore"):
        y = (g - zero[..., None]) / np.where(scale > 0, scale, 1.0)[..., None]
    f = np.abs((y - np.floor(y)) - 0.5)
    f = np.where((scale > 0)[..., None], f, np.inf)
    return f.reshape(sh)


# --------------------------------------------------------------------------
# Step 10, the paper's codec [Pith, "Referee Report" Summary (2-bit
# Hadamard-rotated, Lloyd-Max-quantised residuals) and "Assumptions & free
# parameters" (four-level Lloyd-Max codebook for a unit Gaussian, randomized
# Hadamard rotation with a shared fixed seed; after the rotation a residual's
# coordinates are modelled as Gaussian with variance ||r||^2 / D)].
# Reading R22 for the details: rotation y = (1/sqrt(D)) H_D diag(s) r with the
# Sylvester Hadamard matrix and a fixed sign vector s; scale sigma =
# fp16(||r|| / sqrt(D)); code of coordinate i from u_i = y_i / sigma against
# the Lloyd-Max thresholds -t, 0, t (a value on a threshold takes the upper
# cell); reconstruction r~ = diag(s) (1/sqrt(D)) H_D (sigma * level[code]).
# --------------------------------------------------------------------------
def splitmix64(state):
    """One step of the SplitMix64 generator (Steele, Lea and Flood, "Fast
    splittable pseudorandom number generators", 2014): returns (new state,
    output), all arithmetic modulo 2^64."""
    M = (1 << 64) - 1
    state = (state + 0x9E3779B97F4A7C15) & M
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M
    return state, z ^ (z >> 31)


def default_sign_words(seed=SIGN_SEED):
    """The default rotation signs as four 32-bit words (bit i % 32 of word
    i // 32 set means s_i = -1): the first two SplitMix64 outputs from the
    seed, low word first."""
    st, a = splitmix64(seed)
    st, b = splitmix64(st)
    return [a & 0xFFFFFFFF, a >> 32, b & 0xFFFFFFFF, b >> 32]


def signs_from_words(words, D):
    """s [D] in {+1, -1} from the sign words."""
    bits = np.array([(words[i // 32] >> (i % 32)) & 1 for i in range(D)])
    return np.where(bits == 1, -1.0, 1.0)


def hadamard_matrix(D):
    """Orthonormal Sylvester-Hadamard matrix (1/sqrt(D)) H_D with
    H_D[i, j] = (-1)^popcount(i & j); D a power of two."""
    i = np.arange(D)
    par = np.array([[bin(a & b).count("1") & 1 for b in i] for a in i])
    return np.where(par == 1, -1.0, 1.0) / math.sqrt(D)


def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def _Phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def lloyd_max_gaussian4(iters=200):
    """Four-level Lloyd-Max quantiser of a unit Gaussian (Lloyd 1982, Max
    1960), by Lloyd's iteration on the symmetric cells (-inf, -t), [-t, 0),
    [0, t), [t, inf): each level is the conditional mean of its cell and the
    inner threshold t the midpoint of the two positive levels.  Returns
    (levels [-l2, -l1, l1, l2], t)."""
    l1, l2 = 0.5, 1.5
    for _ in range(iters):
        t = 0.5 * (l1 + l2)
        l1 = (_phi(0.0) - _phi(t)) / (_Phi(t) - 0.5)     # E[X | 0 <= X < t]
        l2 = _phi(t) / (1.0 - _Phi(t))                     # E[X | X >= t]
    t = 0.5 * (l1 + l2)
    return np.array([-l2, -l1, l1, l2]), t


def rotate(r, words):
    """y = (1/sqrt(D)) H_D diag(s) r over the last axis."""
    D = r.shape[-1]
    return (r * signs_from_words(words, D)) @ hadamard_matrix(D).T


def unrotate(y, words):
    """r = diag(s) (1/sqrt(D)) H_D y (the inverse of rotate: the orthonormal
    Sylvester matrix is symmetric and its own inverse)."""
    D = y.shape[-1]
    return (y @ hadamard_matrix(D).T) * signs_from_words(words, D)


def quantize_hlm(r, words):
    """r: [..., D].  Returns (codes uint8 [..., D], sigma [...]) with sigma the
    float64 value of fp16(||r|| / sqrt(D)); codes 0 where sigma = 0."""
    D = r.shape[-1]
    lv, t = lloyd_max_gaussian4()
    sigma = fp16_rne(np.linalg.norm(r, axis=-1) / math.sqrt(D))
    y = rotate(r, words)
    with np.errstate(invalid="ignore", divide="ignore"):
        u = y / np.where(sigma > 0, sigma, 1.0)[..., None]
    codes = (u >= -t).astype(np.uint8) + (u >= 0.0) + (u >= t)
    codes = np.where((sigma > 0)[..., None], codes, 0)
    return codes.astype(np.uint8), sigma


def dequantize_hlm(codes, sigma, words):
    lv, _ = lloyd_max_gaussian4()
    return unrotate(sigma[..., None] * lv[codes.astype(np.int64)], words)


def hlm_code_margin(r, sigma, words):
    """Distance of u = y / sigma from the nearest threshold (-t, 0, t); +inf
    where sigma = 0.  Used to skip boundary cases in parity checks."""
    _, t = lloyd_max_gaussian4()
    y = rotate(r, words)
    with np.errstate(invalid="ignore", divide="ignore"):
        u = y / np.where(sigma > 0, sigma, 1.0)[..., None]
    m = np.minimum(np.minimum(np.abs(u + t), np.abs(u)), np.abs(u - t))
    return np.where((sigma > 0)[..., None], m, np.inf)


# --------------------------------------------------------------------------
# Pre-RoPE key storage [Pith, "Assumptions & free parameters" (RoPE is a
# per-position orthogonal linear map R_t, so R_t K_t = R_t K~_t + R_t r_t and
# ||R_t r_t|| = ||r_t||, which justifies storing keys before the rotation and
# rotating at decode time) and "Referee Report" (pre-RoPE key storage with
# RoPE distributing over the decomposition)].  The pages fix neither the
# pairing nor the frequencies; reading R24: the rotate-half pairing of the
# Llama models the pages evaluate, coordinates i and i + D/2 turned by the
# angle t * theta_i with theta_i = base^(-2i/D), the key at position t.
# --------------------------------------------------------------------------
def rope_freqs(D, base):
    """theta_i = base^(-2i/D) for i < D/2 (reading R24)."""
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / D)


def rope(X, base, positions=None):
    """R_t X_t for rows X [N, D] at positions (default 0..N-1): coordinate
    pairs (i, i + D/2) rotated by t * theta_i (reading R24)."""
    N, D = X.shape
    pos = np.arange(N, dtype=np.float64) if positions is None else np.asarray(positions, dtype=np.float64)
    ang = pos[:, None] * rope_freqs(D, base)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    h = D // 2
    x0, x1 = X[:, :h], X[:, h:]
    return np.concatenate([x0 * c - x1 * s, x0 * s + x1 * c], axis=1)


# --------------------------------------------------------------------------
# The whole compression pass of one unit [Pith, "What carries the argument";
# Velox, "Adaptation notes" (one-shot compression at the end of prefill)].
# --------------------------------------------------------------------------
@dataclass
class Compressed:
    plan: Plan
    G: int
    anchor_pos: np.ndarray        # [H, A] int
    idx: np.ndarray               # [2, H, N] anchor index per side (0 = K, 1 = V)
    gamma: np.ndarray             # [2, H, N] float64 (unrounded)
    gamma16: np.ndarray           # [2, H, N] float64 value of the fp16 coefficient
    resid: np.ndarray             # [2, H, N, D] float64 residual (unquantised)
    flag: np.ndarray              # [2, H, N] bool: residual stored
    codes: np.ndarray             # [2, H, N, D] uint8 (valid where flag)
    scale: np.ndarray             # [2, H, N, D/32]
    zero: np.ndarray              # [2, H, N, D/32]
    anchors: np.ndarray           # [2, H, A, D] exact anchor vectors
    score: np.ndarray             # [H, N]
    pooled: np.ndarray            # [H, N - W]
    P: list = field(repr=False, default=None)   # per head [GQ, N]
    O: np.ndarray = None          # [H, GQ, D]
    u: np.ndarray = None          # [2, H, N] utilities (-inf ineligible)
    margin: np.ndarray = None     # [2, H, N] top-2 cosine margin
    codec: int = CODEC_AFFINE
    sigma: np.ndarray = None      # [2, H, N] fp16 scale of the Hadamard / Lloyd-Max codec
    sign_words: tuple = None      # rotation signs of that codec
    rope_theta: float = None      # pre-RoPE keys: the rotary base (None: keys attended as stored)


def compress_unit(K, V, Q, G, n_obs, theta, W, e,
                  anchor_override=None, idx_override=None, flag_override=None,
                  anchor_div=ANCHOR_DIV, rho=RHO, pool=POOL, pool_kv_jointly=False,
                  codec=CODEC_AFFINE, sign_words=None, anchor_mode=ANCHORS_UNIFORM, cover_rounds=COVER_ROUNDS,
                  picks_override=None, rope_theta=None):
    """K, V: [H, N, D] float64; Q: [H*G, n_obs, D] float64.

    anchor_div, rho, pool: the method's fixed parameters (see plan and
    anchor_score), the pages' values by default.  pool_kv_jointly: one
    ranking of the key and value utilities of every (side, head, token) under
    the combined budget, ties to K before V, then lower head, then lower
    position (reading R18b); otherwise each side ranks its own items.
    codec: CODEC_AFFINE (group-affine, scale and zero per 32 coordinates) or
    CODEC_HLM (randomized Hadamard rotation with the signs sign_words, the
    default ones when None, and the Lloyd-Max codebook; reading R22).
    anchor_mode: ANCHORS_UNIFORM (stratified picks) or ANCHORS_COVER
    (coverage picks over the keys in cover_rounds rounds, reading R23).
    rope_theta: None, or the rotary base when K holds pre-RoPE keys (reading
    R25): the observation-window attention (and with it the score, p and o)
    sees the rotated keys R_t K_t, and the key channel of the utility the
    rotated residual R_t r_t of each token at its own position; the anchors,
    the nearest-anchor assignment, gamma, the residuals and their codes stay
    in the stored (pre-RoPE) space.

    The *_override arguments let a parity test continue from decisions the GPU
    took where the oracle's own decision was within the stated tie margin:
    anchor_override [H, A] positions, idx_override [2, H, N], flag_override
    [2, H, N] bool, picks_override [H] lists of coverage picks in round order.
    The test checks the overrides before passing them.
    """
    H, N, D = K.shape
    p = plan(H, N, D, e, theta, W, anchor_div, rho, pool_kv_jointly, codec)
    A = p.A
    GQ = G * n_obs
    anchor_pos = np.zeros((H, A), dtype=np.int64)
    idx = np.zeros((2, H, N), dtype=np.int64)
    gamma = np.zeros((2, H, N))
    gamma16 = np.zeros((2, H, N))
    resid = np.zeros((2, H, N, D))
    margin = np.zeros((2, H, N))
    eligible = np.zeros((H, N), dtype=bool)
    score = np.zeros((H, N))
    pooled = np.zeros((H, N - W))
    u = np.zeros((2, H, N))
    Ps, Os = [], np.zeros((H, GQ, D))
    for h in range(H):
        Qh = Q[h * G:(h + 1) * G].reshape(GQ, D)
        Ka = K[h] if rope_theta is None else rope(K[h], rope_theta)
        P, O = obs_attention(Qh, Ka, V[h], n_obs)
        Ps.append(P)
        Os[h] = O
        score[h], pooled[h] = anchor_score(P, W, pool)
        pos = select_anchors(pooled[h], N, W, p.k_s, p.k_u, anchor_mode, K[h], cover_rounds,
                             None if picks_override is None else picks_override[h])
        if anchor_override is not None:
            pos = np.sort(np.asarray(anchor_override[h], dtype=np.int64))
        anchor_pos[h] = pos
        for s, X in enumerate((K[h], V[h])):
            io = None if idx_override is None else idx_override[s, h]
            a = assign(X, pos, io)
            idx[s, h], gamma[s, h], gamma16[s, h] = a["idx"], a["gamma"], a["gamma16"]
            resid[s, h], margin[s, h] = a["r"], a["margin"]
            eligible[h] = ~a["is_anchor"]
        rK = resid[0, h] if rope_theta is None else rope(resid[0, h], rope_theta)
        u[0, h], u[1, h] = utilities(P, O, Qh, V[h], rK, resid[1, h], eligible[h])
    flag = np.zeros((2, H, N), dtype=bool)
    if p.joint:
        # the stacked (side, head) rows rank by (-u, side, head, position)
        flag = allocate(u.reshape(2 * H, N), p.R_total).reshape(2, H, N)
    else:
        for s, R in enumerate((p.R_K, p.R_V)):
            flag[s] = allocate(u[s], R)
    if flag_override is not None:
        flag = np.asarray(flag_override, dtype=bool).copy()
    sigma = None
    words = None
    if codec == CODEC_HLM:
        words = tuple(default_sign_words() if sign_words is None else sign_words)
        codes, sigma = quantize_hlm(resid, words)
        sigma = np.where(flag, sigma, 0.0)
        sc = np.zeros((2, H, N, D // GROUP))
        ze = np.zeros((2, H, N, D // GROUP))
    else:
        codes, sc, ze = quantize(resid)
    codes = np.where(flag[..., None], codes, 0).astype(np.uint8)
    anchors = np.stack([K[np.arange(H)[:, None], anchor_pos], V[np.arange(H)[:, None], anchor_pos]])
    return Compressed(p, G, anchor_pos, idx, gamma, gamma16, resid, flag, codes, sc, ze,
                      anchors, score, pooled, Ps, Os, u, margin, codec, sigma, words, rope_theta)


def reconstruct(c: Compressed):
    """K^, V^ [H, N, D]: fp16(gamma) * x_a + [flag] * dequantised residual
    [Pith, "What carries the argument"], with the cache's codec, in the stored
    space (pre-RoPE keys when c.rope_theta is set; see attended_keys)."""
    out = []
    H = c.anchor_pos.shape[0]
    for s in range(2):
        xa = c.anchors[s][np.arange(H)[:, None], c.idx[s]]
        if c.codec == CODEC_HLM:
            rt = dequantize_hlm(c.codes[s], c.sigma[s], c.sign_words)
        else:
            rt = dequantize(c.codes[s], c.scale[s], c.zero[s])
        out.append(c.gamma16[s][..., None] * xa + np.where(c.flag[s][..., None], rt, 0.0))
    return out[0], out[1]


def attention(q, K, V):
    """softmax(q K^T / sqrt(D)) V for q [M, D], K, V [N, D]; no mask."""
    D = q.shape[-1]
    s = (q @ K.T) / math.sqrt(D)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    return (p @ V) / p.sum(axis=-1, keepdims=True)


def attended_keys(c: Compressed, Kh):
    """The keys decode attends to: the reconstruction itself, or with pre-RoPE
    storage R_t K^_t at each token's position (reading R26)."""
    if c.rope_theta is None:
        return Kh
    return np.stack([rope(Kh[h], c.rope_theta) for h in range(Kh.shape[0])])


def decode_unit(c: Compressed, q):
    """Decode attention over the compressed cache of one unit.
    q: [H*G, D] float64 (post-RoPE when the keys are stored pre-RoPE); q-head
    h*G + g reads KV head h.  Returns o [H*G, D]."""
    Kh, Vh = reconstruct(c)
    Kh = attended_keys(c, Kh)
    H = Kh.shape[0]
    G = c.G
    o = np.zeros_like(q)
    for h in range(H):
        o[h * G:(h + 1) * G] = attention(q[h * G:(h + 1) * G], Kh[h], Vh[h])
    return o


def decode_unit_tail(c: Compressed, q, K_tail, V_tail):
    """Decode attention over the compressed cache of one unit followed by a
    tail of tokens appended after the one-shot compression and kept exact
    (AnchorKV-adapted page, "Adaptation notes": tokens produced during decode
    are appended at full precision and never re-anchored).  One softmax per
    q-head over the N reconstructed tokens and the tail of its KV head.
    q: [H*G, D]; K_tail, V_tail: [H, T, D] float64, T >= 0, tail keys attended
    as given (already rotated with pre-RoPE storage, reading R27).
    Returns o [H*G, D]."""
    Kh, Vh = reconstruct(c)
    Kh = attended_keys(c, Kh)
    H = Kh.shape[0]
    G = c.G
    o = np.zeros_like(q)
    for h in range(H):
        K = np.concatenate([Kh[h], K_tail[h]], axis=0)
        V = np.concatenate([Vh[h], V_tail[h]], axis=0)
        o[h * G:(h + 1) * G] = attention(q[h * G:(h + 1) * G], K, V)
    return o


# --------------------------------------------------------------------------
# Theorem 1 output-error bound [Pith, "What carries the argument" and
# "Referee Report" (E_K = 2 V_max tanh(mu), mu = ||q|| Delta_K / sqrt(D),
# Delta_K = max_t ||K_t - K^_t||)] (reading R20 for the exact form).
# --------------------------------------------------------------------------
def theorem1_terms(q, K, V, Kh, Vh):
    """Returns (||y - y^||, value term, key term, mirror value term, mirror key term)
    for one query: value term = sum_t a^_t ||V_t - V^_t|| (a^ from K^), key term =
    2 max_t ||V_t|| tanh(mu); the mirror form uses a (from K) and max ||V^_t||."""
    D = q.size
    y = attention(q[None], K, V)[0]
    yh = attention(q[None], Kh, Vh)[0]
    s = (Kh @ q) / math.sqrt(D)
    ah = np.exp(s - s.max()); ah /= ah.sum()
    s0 = (K @ q) / math.sqrt(D)
    a0 = np.exp(s0 - s0.max()); a0 /= a0.sum()
    dv = np.linalg.norm(V - Vh, axis=1)
    dK = np.linalg.norm(K - Kh, axis=1).max()
    mu = np.linalg.norm(q) * dK / math.sqrt(D)
    return (np.linalg.norm(y - yh), float(ah @ dv), 2 * np.linalg.norm(V, axis=1).max() * math.tanh(mu),
            float(a0 @ dv), 2 * np.linalg.norm(Vh, axis=1).max() * math.tanh(mu))
