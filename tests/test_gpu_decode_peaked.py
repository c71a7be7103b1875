"""GPU decode on hand-built compressed caches whose softmax is peaked.

An attention sink or a retrieval head puts one to a few keys 12-20 nats above
a long flat background.  The value side then adds up many tiny weights p * gamma
next to a few large ones, and any absolute rounding of those terms biases the
output once the values have a nonzero mean.  These caches are built directly
in the compressed representation (random anchors, pointers, coefficients and
2-bit residual records, packed on the host), with the peak keys aligned to the
decode queries, coefficients below and above 8 (and negative), and values with
a mean offset of 1.  The oracle's decode (dense attention over the explicit
reconstruction, fp64) is the reference; the bound is 1e-3 relative per q-head.
"""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import anchorkv_oracle as O
from tests.parity import anchors_to_storage, bits_f16, f16_bits_to_f64, storage_to_f64

pytestmark = pytest.mark.gpu

D = 128


def _flush(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def akv():
    import kv_cache_compression_snapkv_amd as m
    m.lib()
    return m


def bf16_round(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def peaked_unit(p, G, seed, peaks_nats, big_gamma):
    """Arrays of one unit (host packer layout) and its oracle view, plus the
    decode query [H*G, D] (bf16 values as float64).  Every q-head g of KV head
    h has its own peak anchor, aligned with its query, reached by 1-3 tokens
    with gamma 1; the background anchors are small, so background logits are
    within a few hundredths of a nat of 0."""
    r = np.random.default_rng(seed)
    H, N, A = p.H, p.N, p.A
    q = bf16_round(r.standard_normal((H * G, D)))
    ak = bf16_round(r.standard_normal((H, A, D)) * 0.05)
    av = bf16_round(r.standard_normal((H, A, D)) + 1.0)          # values with a mean offset
    peak_anchor = np.zeros((H, G), np.int64)
    for h in range(H):
        for g in range(G):
            a = g * 7 + 3
            peak_anchor[h, g] = a
            qg = q[h * G + g]
            nats = peaks_nats[(h * G + g) % len(peaks_nats)]
            ak[h, a] = bf16_round(qg / np.linalg.norm(qg) * nats * math.sqrt(D) / np.linalg.norm(qg))
    pos = np.sort(r.choice(N - p.window, A - p.window, replace=False))
    pos = np.concatenate([pos, np.arange(N - p.window, N)]).astype(np.int32)
    pos = np.tile(pos, (H, 1))
    bg = np.setdiff1d(np.arange(A), peak_anchor.reshape(-1))
    idx = r.choice(bg, size=(2, H, N)).astype(np.int32)
    g16 = r.uniform(0.5, 1.5, (2, H, N))
    if big_gamma:
        # coefficients of 8 and more (the general fixed-point path) and negative ones on both sides
        sel = r.random((2, H, N))
        g16 = np.where(sel < 0.1, r.uniform(8.0, 40.0, (2, H, N)), g16)
        g16 = np.where((sel >= 0.1) & (sel < 0.15), -r.uniform(0.2, 3.0, (2, H, N)), g16)
    for h in range(H):
        for g in range(G):
            n_pk = 1 + (h + g) % 3
            t = r.choice(N - p.window, n_pk, replace=False)
            idx[0, h, t] = peak_anchor[h, g]
            g16[0, h, t] = 1.0
    # anchor tokens point at themselves with gamma 1
    for h in range(H):
        idx[:, h, pos[h]] = np.arange(A)
        g16[:, h, pos[h]] = 1.0
    g16 = O.fp16_rne(g16)
    flag = np.zeros((2, H, N), np.uint8)
    for s, R in enumerate((p.R_K, p.R_V)):
        elig = np.ones((H, N), bool)
        for h in range(H):
            elig[h, pos[h]] = False
        cand = np.flatnonzero(elig.reshape(-1))
        flag[s].reshape(-1)[r.choice(cand, R, replace=False)] = 1
    codes = r.integers(0, 4, (2, H, N, D)).astype(np.uint8) * flag[..., None]
    scale = O.fp16_rne(r.uniform(0.01, 0.2, (2, H, N, D // 32))) * flag[..., None]
    zero = O.fp16_rne(-1.5 * scale - r.uniform(-0.02, 0.02, (2, H, N, D // 32))) * flag[..., None]
    arrays = dict(positions=pos, anchors_k=anchors_to_storage(ak, 1), anchors_v=anchors_to_storage(av, 1),
                  idx=idx, gamma16=bits_f16(g16), flag=flag, codes=codes, scale16=bits_f16(scale),
                  zero16=bits_f16(zero))
    c = O.Compressed(plan=None, G=G, anchor_pos=pos.astype(np.int64), idx=idx.astype(np.int64), gamma=g16,
                     gamma16=g16, resid=None, flag=flag.astype(bool), codes=codes, scale=scale, zero=zero,
                     anchors=np.stack([storage_to_f64(arrays["anchors_k"], 1), storage_to_f64(arrays["anchors_v"], 1)]),
                     score=None, pooled=None)
    return arrays, c, q


CASES = [
    # (kv_heads, q_per_kv, n_tokens, big_gamma, units).  The unit is replicated
    # `units` times so that the launch splits each head into as few token ranges
    # as a full cache does (one range per head: one running maximum over all of
    # a head's tokens, the case where small weights meet a large maximum).
    (2, 4, 32768, False, 256),
    (2, 4, 32768, True, 1),
    (2, 8, 32768, True, 128),
    (1, 8, 131072, False, 256),
    (1, 8, 131072, True, 128),
]


@pytest.mark.parametrize("H,G,N,big_gamma,U", CASES)
def test_decode_peaked_softmax(akv, H, G, N, big_gamma, U):
    _flush(f"[peaked] H={H} G={G} N={N} big_gamma={big_gamma} units={U}")
    p = akv.plan(U, H, G, N, D, 32, akv.BF16, 0.05, 32)
    arrays, c, q64 = peaked_unit(p, G, seed=N + 17 * G + H + (1000 if big_gamma else 0),
                                 peaks_nats=[12.0, 13.5, 15.0, 16.5, 18.0, 20.0], big_gamma=big_gamma)
    unit = torch.from_numpy(np.frombuffer(akv.pack_unit(p, arrays), np.uint8).copy()).cuda()
    cache = torch.zeros(int(p.cache_bytes), dtype=torch.uint8, device="cuda")
    cache.view(U, int(p.unit_stride))[:, :unit.numel()] = unit
    _, _, dws = akv.alloc(p, "cuda")
    qd = torch.from_numpy(q64.astype(np.float32)).to(torch.bfloat16).reshape(1, H * G, D).cuda()
    qd = qd.expand(U, H * G, D).contiguous()
    o = torch.empty(U, H * G, D, dtype=torch.float32, device="cuda")
    akv.decode_attn(p, cache, qd, o, dws)
    torch.cuda.synchronize()
    ref = O.decode_unit(c, q64)
    for u in sorted({0, U - 1}):
        got = o[u].cpu().numpy().astype(np.float64)
        err = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
        _flush(f"[peaked] H={H} G={G} N={N} big_gamma={big_gamma} units={U} ranges/head={p.decode_splits} "
               f"unit {u}: max rel err {err.max():.3e} (per q-head {np.array2string(err, precision=2)})")
        assert err.max() <= 1e-3
