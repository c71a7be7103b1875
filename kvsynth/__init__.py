"""Seeded synthetic KV-cache inputs.

This module only draws random tensors with the shapes, value distributions and
structure of the workloads described for the anchor-residual KV-cache method
(AnchorKV).  It contains none of the method's arithmetic: it is shared by the
CPU oracle's tests, the GPU parity tests and the benchmark so that all of them
see the same inputs.

Workloads (per-layer KV shapes of the models the paper evaluates: 8 KV heads,
head dim 128; "Pith review of AnchorKV", "Core claim" and "Assumptions & free
parameters"), with synthetic stand-ins for the prompts of the RULER /
LongBench / needle benchmarks, which are not used or reproduced:

* keys: a per-head dictionary of unit directions; each token picks one
  direction uniformly, adds a perturbation of norm 0.3 (0.3 * z / sqrt(D)),
  and is scaled by a log-normal(0, 0.5) factor (or 1);
* values: N(0, 1) per coordinate (Student-t with 3 degrees of freedom for the
  adversarial workload);
* observation queries and decode queries: N(0, I).

The adversarial workload additionally scales 4 seeded key channels by 20 on the
clustered 95 % of tokens and replaces the other 5 % by isotropic directions
(s_t * z / ||z||, no outlier scaling).

Everything is drawn in float32 with a torch.Generator seeded from
(0xA7C4, workload, sequence, layer) and then cast to the workload dtype with
round-to-nearest-even.  A given (workload, sequence, layer, device type) always
gives the same tensors.  CPU and GPU generators are different streams, so a GPU
test that checks against the oracle copies the GPU-generated inputs to the host.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

SEED_TAG = 0xA7C4
DECODE_TAG = 0xDEC


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # workload id used in the seed
    seqs: int                  # independent sequences
    layers: int                # layers per sequence; units = seqs * layers
    kv_heads: int
    q_per_kv: int
    n_tokens: int
    head_dim: int
    dtype: str                 # "bf16" or "f32"
    n_obs: int                 # observation queries per q-head
    theta: float
    window: int
    n_dirs: int                # key directions per head
    lognormal: bool            # log-normal(0, 0.5) key norms (else 1)
    decode_steps: int
    stress: bool = False       # outlier channels + isotropic tokens + Student-t values

    @property
    def units(self) -> int:
        return self.seqs * self.layers

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def scaled(self, **kw) -> "Workload":
        """A copy with some fields replaced (smaller parity-test instances)."""
        return dataclasses.replace(self, **kw)


# The five workloads, full size.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 1, 1, 1, 512, 128, "f32", 32, 0.1, 32, 16, True, 8),
    "llama3b_8k": Workload("llama3b_8k", 2, 1, 28, 8, 3, 8192, 128, "bf16", 32, 0.1, 32, 64, False, 128),
    "llama8b_32k": Workload("llama8b_32k", 3, 16, 32, 8, 4, 32768, 128, "bf16", 32, 0.05, 32, 256, True, 256),
    "llama70b_128k": Workload("llama70b_128k", 4, 1, 80, 8, 8, 131072, 128, "bf16", 32, 0.05, 32, 1024, False, 256),
    "stress_64k": Workload("stress_64k", 5, 4, 32, 8, 4, 65536, 128, "bf16", 64, 0.02, 64, 256, True, 64, stress=True),
}
WORKLOAD_ORDER = ["tiny_f32", "llama3b_8k", "llama8b_32k", "llama70b_128k", "stress_64k"]


def _seed(*parts: int) -> int:
    st = np.random.SeedSequence([int(p) for p in parts]).generate_state(2, np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def _gen(device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _keys(w: Workload, g: torch.Generator, device, iso_out: Optional[list] = None) -> torch.Tensor:
    H, N, D = w.kv_heads, w.n_tokens, w.head_dim
    dirs = torch.randn(H, w.n_dirs, D, generator=g, device=device)
    dirs = dirs / dirs.norm(dim=-1, keepdim=True)
    cl = torch.randint(0, w.n_dirs, (H, N), generator=g, device=device)
    z = torch.randn(H, N, D, generator=g, device=device)
    base = torch.gather(dirs, 1, cl.unsqueeze(-1).expand(H, N, D))
    k = base + (0.3 / math.sqrt(D)) * z
    if w.lognormal:
        s = torch.exp(0.5 * torch.randn(H, N, generator=g, device=device))
    else:
        s = torch.ones(H, N, device=device)
    if w.stress:
        ch = torch.stack([torch.randperm(D, generator=g, device=device)[:4] for _ in range(H)])  # [H,4]
        scale = torch.ones(H, D, device=device)
        scale.scatter_(1, ch, 20.0)
        iso = torch.rand(H, N, generator=g, device=device) < 0.05
        ziso = torch.randn(H, N, D, generator=g, device=device)
        ziso = ziso / ziso.norm(dim=-1, keepdim=True)
        k = torch.where(iso.unsqueeze(-1), ziso, k * scale.unsqueeze(1))
        if iso_out is not None:
            iso_out.append(iso)
    return k * s.unsqueeze(-1)


def _values(w: Workload, g: torch.Generator, device) -> torch.Tensor:
    H, N, D = w.kv_heads, w.n_tokens, w.head_dim
    z = torch.randn(H, N, D, generator=g, device=device)
    if not w.stress:
        return z
    c = torch.randn(3, H, N, D, generator=g, device=device)
    chi2 = (c * c).sum(0)
    return z / torch.sqrt(chi2 / 3.0)


def unit_inputs(w: Workload, seq: int, layer: int, device="cpu"):
    """K, V [H, N, D] and Q_obs [H*G, n_obs, D] of one (sequence, layer) unit, in w's dtype."""
    g = _gen(device, SEED_TAG, w.index, seq, layer)
    K = _keys(w, g, device)
    V = _values(w, g, device)
    Q = torch.randn(w.kv_heads * w.q_per_kv, w.n_obs, w.head_dim, generator=g, device=device)
    dt = w.torch_dtype
    return K.to(dt), V.to(dt), Q.to(dt)


def stress_isotropic_check(w: Workload, seq: int = 0, layer: int = 0, device="cpu", stride: int = 128):
    """Self-check of the adversarial workload's structure: the isotropic 5 %
    of the keys must be the worst-covered tokens.  For each head, every
    token's largest cosine to a reference dictionary (every stride-th token,
    the token itself excluded) is computed; returns, per head, the fraction of
    the isotropic tokens that fall among the |iso| lowest such cosines, and
    the largest isotropic / smallest clustered max-cosine."""
    assert w.stress
    g = _gen(device, SEED_TAG, w.index, seq, layer)
    iso_l: list = []
    K = _keys(w, g, device, iso_out=iso_l).to(w.torch_dtype).to(torch.float64)
    iso = iso_l[0]
    out = []
    for h in range(w.kv_heads):
        x = K[h] / K[h].norm(dim=-1, keepdim=True)
        ref = torch.arange(0, w.n_tokens, stride, device=device)
        c = x @ x[ref].T
        c[ref, torch.arange(ref.numel(), device=device)] = -2.0    # not the token itself
        mc = c.max(dim=1).values
        m = iso[h]
        n = int(m.sum())
        low = torch.argsort(mc)[:n]
        frac = float(m[low].float().mean()) if n else 1.0
        out.append(dict(iso=n, frac_lowest=frac, iso_max=float(mc[m].max()), clustered_min=float(mc[~m].min())))
    return out


def decode_queries(w: Workload, step: int, units: Optional[int] = None, device="cpu") -> torch.Tensor:
    """Decode-step queries [U, H*G, D] in w's dtype (one per q-head per unit)."""
    U = w.units if units is None else units
    g = _gen(device, SEED_TAG, w.index, DECODE_TAG, step)
    q = torch.randn(U, w.kv_heads * w.q_per_kv, w.head_dim, generator=g, device=device)
    return q.to(w.torch_dtype)


def unit_index(w: Workload, u: int):
    """(sequence, layer) of flat unit u (units are sequence-major)."""
    return divmod(u, w.layers)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16 / f32 tensor."""
    return t.detach().to("cpu", torch.float64).numpy()
