"""Seeded synthetic inputs for the Gated DeltaNet token-mixer hot path.

This module only draws numbers: shapes, lengths and value distributions of
the five benchmark workloads and of the small test cases.  It contains none
of the method's arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it.

Recipe (every tensor, in this fixed draw order from
``numpy.random.default_rng(seed)``): sequence lengths, x, conv weight, conv
bias (if any), the beta normals, the g normals, initial state, halo, upstream
output gradient, upstream final-state gradient.  Normals are drawn as
float32, scaled, and rounded to the activation dtype by round-to-nearest-even
(torch's float32 -> bfloat16 cast).  beta = sigmoid(n) and
g = -softplus(n) = -log1p(exp(n)) are evaluated in float64 from the float32
normal and rounded to float32; they are per token and per value head.

Layouts: x [T, C] with channels [Q heads | K heads | V heads]
(C = 2*Hk*dk + Hv*dv); conv weight [C, K]; halo [K-1, C]; g, beta [T, Hv];
states [N, Hv, dk, dv] float32; upstream output gradient [T, Hv, dv].
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

ACT_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Spec:
    """One workload.  ``lengths`` are the global sequence lengths; when
    ``world_size`` > 1 the processed tokens are shard ``rank`` of their
    concatenation (the consumer localises the global cu_seqlens itself)."""
    name: str
    lengths: Optional[Sequence[int]]      # None: drawn by ``length_rule``
    Hk: int
    Hv: int
    dk: int
    dv: int
    act: str = "bf16"
    K: int = 4
    seed: int = 0
    length_rule: Optional[str] = None     # "uniform:lo:hi:n" | "lognormal:total"
    h0_std: Optional[float] = None        # None: zero initial state
    halo: bool = False
    n_halo: int = 0                       # halo rows valid without a shard split
    bias: bool = False
    world_size: int = 1
    rank: int = 0
    backward: bool = False
    g_scale: float = 1.0                  # stress variants scale g
    beta_one_g_zero: bool = False         # stress variant beta = 1, g = 0

    @property
    def C(self) -> int:
        return 2 * self.Hk * self.dk + self.Hv * self.dv


def _bf(a: np.ndarray, act: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(ACT_DTYPES[act])


def _normal(rng, shape, std=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _normal_big(rng, rows, cols, std=1.0, act="bf16", block=8192):
    """Row blocks of a large [rows, cols] normal draw, rounded as they come,
    so peak host memory stays near the rounded tensor's size."""
    out = torch.empty((rows, cols), dtype=ACT_DTYPES[act])
    for r0 in range(0, rows, block):
        r1 = min(rows, r0 + block)
        out[r0:r1] = _bf(_normal(rng, (r1 - r0, cols), std), act)
    return out


def _draw_lengths(rng, rule: str):
    kind, *args = rule.split(":")
    if kind == "uniform":
        lo, hi, n = (int(a) for a in args)
        return [int(x) for x in rng.integers(lo, hi + 1, size=n)]
    if kind == "lognormal":
        total = int(args[0])
        out, acc = [], 0
        while acc < total:
            ln = int(np.clip(np.round(rng.lognormal(np.log(2048.0), 1.0)), 16, 16384))
            ln = min(ln, total - acc)
            out.append(ln)
            acc += ln
        return out
    raise ValueError(rule)


def shard_condition(lengths, world_size, rank):
    """Plain interval test used only to pick the sharded workload's seed: at
    least two sequences overlap the shard and the shard's first token does
    not start its sequence (the shard carries in a state)."""
    total = sum(lengths)
    part = total // world_size
    lo, hi = part * rank, part * (rank + 1)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    ends = np.cumsum(lengths)
    overlapping = [(s, e) for s, e in zip(starts, ends) if e > s and s < hi and e > lo]
    return len(overlapping) >= 2 and overlapping[0][0] < lo


def make(spec: Spec) -> dict:
    """Draws every input of ``spec``; returns CPU tensors and host metadata.

    Keys: cu_global (int64 numpy), T (tokens processed), x, w, bias, g, beta,
    h0, halo, do, dht (torch CPU tensors or None), cap (number of state slots:
    the global sequence count, an upper bound on the local count)."""
    rng = np.random.default_rng(spec.seed)
    lengths = list(spec.lengths) if spec.lengths is not None else _draw_lengths(rng, spec.length_rule)
    cu_global = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    total = int(cu_global[-1])
    T = total // spec.world_size if spec.world_size > 1 else total
    cap = len(lengths)
    C, Hv = spec.C, spec.Hv
    x = _normal_big(rng, T, C, act=spec.act)
    w = _bf(_normal(rng, (C, spec.K), std=1.0 / np.sqrt(spec.K)), spec.act)
    bias = _bf(_normal(rng, (C,)), spec.act) if spec.bias else None
    bn = _normal(rng, (T, Hv)).astype(np.float64)
    an = _normal(rng, (T, Hv)).astype(np.float64)
    if spec.beta_one_g_zero:
        beta = np.ones((T, Hv))
        g = np.zeros((T, Hv))
    else:
        beta = 1.0 / (1.0 + np.exp(-bn))
        g = -np.log1p(np.exp(an)) * spec.g_scale
    beta_t = torch.from_numpy(beta.astype(np.float32))
    g_t = torch.from_numpy(g.astype(np.float32))
    h0 = None
    if spec.h0_std is not None:
        if spec.world_size > 1:
            # only the state carried into the shard's first sequence is
            # random; sequences that start inside the shard start from zero
            h = np.zeros((cap, Hv, spec.dk, spec.dv), dtype=np.float32)
            h[0] = _normal(rng, (Hv, spec.dk, spec.dv), std=spec.h0_std)
        else:
            h = _normal(rng, (cap, Hv, spec.dk, spec.dv), std=spec.h0_std)
        h0 = torch.from_numpy(h)
    halo = _bf(_normal(rng, (spec.K - 1, C)), spec.act) if spec.halo and spec.K > 1 else None
    do = dht = None
    if spec.backward:
        do = _normal_big(rng, T, Hv * spec.dv, act=spec.act).view(T, Hv, spec.dv)
        dht = torch.from_numpy(_normal(rng, (cap, Hv, spec.dk, spec.dv), std=0.01))
    return dict(cu_global=cu_global, T=T, cap=cap, x=x, w=w, bias=bias, g=g_t, beta=beta_t,
                h0=h0, halo=halo, do=do, dht=dht, lengths=lengths)


def _sharded_seed(first: int = 2, world_size: int = 8, rank: int = 3) -> int:
    s = first
    while True:
        rng = np.random.default_rng(s)
        if shard_condition(_draw_lengths(rng, "lognormal:32768"), world_size, rank):
            return s
        s += 1


def configs() -> list:
    """The five benchmark workloads, in order."""
    return [
        Spec("single_t256_h2_d32_f32", [256], Hk=2, Hv=2, dk=32, dv=32, act="f32", seed=0,
             backward=True),
        Spec("varlen8_h16_d128_bf16", None, Hk=16, Hv=16, dk=128, dv=128, seed=1,
             length_rule="uniform:64:2048:8", h0_std=0.02),
        Spec("shard3of8_32k_h16_d128_bf16", None, Hk=16, Hv=16, dk=128, dv=128,
             seed=_sharded_seed(), length_rule="lognormal:32768", h0_std=0.02, halo=True,
             world_size=8, rank=3),
        Spec("long131k_hk16_hv32_d128_bf16", [131072], Hk=16, Hv=32, dk=128, dv=128, seed=3),
        Spec("fwdbwd_4x4096_h16_d128_bf16", [4096] * 4, Hk=16, Hv=16, dk=128, dv=128, seed=4,
             h0_std=0.02, halo=True, n_halo=3, backward=True),
    ]


def config(name_or_index) -> Spec:
    cs = configs()
    if isinstance(name_or_index, int):
        return cs[name_or_index]
    for c in cs:
        if c.name == name_or_index:
            return c
    raise KeyError(name_or_index)
