"""Seeded synthetic inputs for OAL causal attention (grouped positive quadratic kernel).

This module only draws numbers. It holds none of the method's arithmetic: no score,
kernel, state or readout is computed here. Both the CPU oracle and the GPU path read
what it returns, so that the two sides see bit-identical inputs.

The pages measure on real post-RoPE Qwen2.5-0.5B activations (daiwk reproduction notes,
section "原论文关键图", Figure 2(a): 64 QK dims per head, 60 bulk dims sharing one group
and a high-contribution tail split into small groups; section "数据协议": 4096-token
sequences). Those activations are not available, so the recipes below stand in for them:

* cfg1: one head, B=1, T=256, fp32; q,k ~ N(0,1) with dims 60..63 scaled x8, v ~ N(0,1);
  groups g0 = dims 0..59, g1 = {60,61}, g2 = {62}, g3 = {63}; L 5x5 lower-triangular with
  entries N(0, 0.3^2) and diagonal |.|+0.1; eps = 1e-3; seed 0.
* cfg2-5: 14 query heads over 2 KV heads, d = 64, bf16 q/k/v; per KV head 2..6 outlier dims
  scaled by U[4,10] in k and (own factor per head) in each of its query heads; RoPE with
  theta = 1e6 (rotate-half pairs (r, r+32)) applied in fp64 after the outlier scaling, then
  rounded to bf16 (round to nearest even); per query head n_tail in [2,5] tail groups over
  the outlier dims (padded with random extra dims when fewer than n_tail), the rest is the
  bulk group g0; L ~ N(0, 0.3^2) lower-triangular with diagonal |.|+0.1; eps = 1e-3.

Arrays are float32 numpy arrays whose values are exactly representable in the stated
input dtype; ``bf16_bits`` gives the raw 16-bit patterns for device upload.
Layouts: q [B, Hq, T, d]; k, v [B, Hkv, T, d]; group_of_dim [Hq, d] uint8 (config group
id g, which is entry g+1 of s-bar); L [Hq, g_max+1, g_max+1] float32 (row/col 0 = the
constant entry of s-bar); eps [Hq] float32; n_groups [Hq] int32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D_H = 64
ROPE_THETA = 1.0e6


@dataclass
class HeadParams:
    """Per-query-head kernel parameters: the group map and the PSD factor (L, eps)."""
    n_groups: np.ndarray      # [Hq] int32, G per head (1..d)
    group_of_dim: np.ndarray  # [Hq, d] uint8, config group id in [0, G)
    L: np.ndarray             # [Hq, g_max+1, g_max+1] float32, lower triangle used
    eps: np.ndarray           # [Hq] float32

    @property
    def g_max(self) -> int:
        return int(self.L.shape[1]) - 1

    @property
    def n_q_heads(self) -> int:
        return int(self.n_groups.shape[0])


@dataclass
class Inputs:
    """One synthetic workload: q, k, v plus the per-head parameters."""
    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    params: HeadParams
    dtype: str                # "f32" or "bf16": the dtype the arrays are exact in
    seed: int
    meta: dict = field(default_factory=dict)

    @property
    def dims(self):
        B, Hq, T, d = self.q.shape
        return B, Hq, int(self.k.shape[1]), T, d, int(self.v.shape[-1])


# ---------------------------------------------------------------------------------------
# rounding helpers (data plumbing only)

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to the nearest bf16 (ties to even); return float32."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(f)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of bf16-exact float32 values."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any((u & 0xFFFF) != 0):
        raise ValueError("values are not bf16-exact")
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------------------
# parameter draws

def draw_L(rng: np.random.Generator, G: int, g_max: int) -> np.ndarray:
    """Lower-triangular (G+1)x(G+1) factor: N(0, 0.3^2) entries, diagonal |.|+0.1, zero-padded."""
    L = np.zeros((g_max + 1, g_max + 1), dtype=np.float32)
    for a in range(G + 1):
        for b in range(a + 1):
            x = rng.normal(0.0, 0.3)
            L[a, b] = abs(x) + 0.1 if a == b else x
    return L


def random_params(rng: np.random.Generator, n_q_heads: int, d: int = D_H, g_min: int = 1,
                  g_hi: int = 4, eps: float = 1e-3, g_max: int | None = None,
                  allow_empty: bool = False) -> HeadParams:
    """Random group maps (any partition) and L per head, for tests on small shapes."""
    Gs = rng.integers(g_min, g_hi + 1, size=n_q_heads).astype(np.int32)
    Gs = np.minimum(Gs, d)
    gm = int(Gs.max()) if g_max is None else int(g_max)
    gamma = np.zeros((n_q_heads, d), dtype=np.uint8)
    Ls = np.zeros((n_q_heads, gm + 1, gm + 1), dtype=np.float32)
    for h in range(n_q_heads):
        G = int(Gs[h])
        if allow_empty:
            lab = rng.integers(0, G, size=d)
        else:
            lab = np.concatenate([np.arange(G), rng.integers(0, G, size=d - G)])
            rng.shuffle(lab)
        gamma[h] = lab.astype(np.uint8)
        Ls[h] = draw_L(rng, G, gm)
    return HeadParams(Gs, gamma, Ls, np.full(n_q_heads, eps, dtype=np.float32))


def per_dim_params(seed: int, n_heads: int, eps: float = 1e-3) -> HeadParams:
    """The per-dimension variant: G = 64 on every head, dimension r of head h in group
    perm_h[r] (a random permutation); L_h lower triangular 65 x 65 with N(0, 0.3^2) entries
    and diagonal |.| + 0.1."""
    rng = np.random.default_rng(seed)
    G = 64
    L = np.zeros((n_heads, G + 1, G + 1), np.float32)
    for h in range(n_heads):
        L[h] = np.tril(rng.normal(0.0, 0.3, (G + 1, G + 1)))
        np.fill_diagonal(L[h], np.abs(np.diag(L[h])) + 0.1)
    gamma = np.stack([rng.permutation(64) for _ in range(n_heads)]).astype(np.uint8)
    return HeadParams(np.full(n_heads, G, np.int32), gamma, L, np.full(n_heads, eps, np.float32))


# ---------------------------------------------------------------------------------------
# configs

def cfg1(seed: int = 0) -> Inputs:
    """Single head, batch 1, T=256, fp32, 4 groups over dims {0..59},{60,61},{62},{63}."""
    rng = np.random.default_rng(seed)
    T, d = 256, D_H
    q = rng.standard_normal((1, 1, T, d))
    k = rng.standard_normal((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, d))
    q[..., 60:64] *= 8.0
    k[..., 60:64] *= 8.0
    gamma = np.zeros((1, d), dtype=np.uint8)
    gamma[0, 60:62] = 1
    gamma[0, 62] = 2
    gamma[0, 63] = 3
    L = draw_L(rng, 4, 4)[None]
    params = HeadParams(np.array([4], np.int32), gamma, L, np.array([1e-3], np.float32))
    return Inputs("cfg1", q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                  params, "f32", seed)


def _rope(x: np.ndarray, pos0: int = 0) -> np.ndarray:
    """Rotate-half RoPE over the last axis (pairs (r, r+d/2)), positions pos0.. along axis -2."""
    d = x.shape[-1]
    half = d // 2
    T = x.shape[-2]
    inv = ROPE_THETA ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.arange(pos0, pos0 + T, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def qwen_like(B: int, T: int, seed: int, n_q_heads: int = 14, n_kv_heads: int = 2,
              name: str = "qwen_like", q_zero: bool = False, per_seq_seeds: list | None = None,
              pos0: int = 0, structure_seed: int | None = None) -> Inputs:
    """Qwen2.5-0.5B-shaped layer (d=64, GQA n_q_heads:n_kv_heads), bf16 inputs.

    Draw order: q, k, v, then the outlier structure and parameters (from ``structure_seed``
    when given, else from the same generator). ``per_seq_seeds`` gives each batch row its
    own generator for q, k, v. ``q_zero`` leaves q at zero (used for state-building
    prefixes whose outputs are not read).
    """
    d = D_H
    n_rep = n_q_heads // n_kv_heads
    qshape = (B, n_q_heads, T, d)
    if per_seq_seeds is None:
        rng = np.random.default_rng(seed)
        q = None if q_zero else rng.standard_normal(qshape)
        k = rng.standard_normal((B, n_kv_heads, T, d))
        v = rng.standard_normal((B, n_kv_heads, T, d))
        prng = rng if structure_seed is None else np.random.default_rng(structure_seed)
    else:
        q = None if q_zero else np.zeros(qshape)
        k = np.zeros((B, n_kv_heads, T, d))
        v = np.zeros((B, n_kv_heads, T, d))
        for b, s in enumerate(per_seq_seeds):
            r = np.random.default_rng(s)
            if not q_zero:
                q[b] = r.standard_normal((n_q_heads, T, d))
            k[b] = r.standard_normal((n_kv_heads, T, d))
            v[b] = r.standard_normal((n_kv_heads, T, d))
        prng = np.random.default_rng(seed if structure_seed is None else structure_seed)
    gamma = np.zeros((n_q_heads, d), dtype=np.uint8)
    Gs = np.zeros(n_q_heads, dtype=np.int32)
    Ls = np.zeros((n_q_heads, 7, 7), dtype=np.float32)   # G <= 6
    outliers = []
    for kv in range(n_kv_heads):
        n_out = int(prng.integers(2, 7))
        dims = np.sort(prng.choice(d, size=n_out, replace=False))
        outliers.append(dims.tolist())
        k[:, kv, :, dims] *= prng.uniform(4.0, 10.0, size=n_out)[:, None, None]
        for j in range(n_rep):
            h = kv * n_rep + j
            qf = prng.uniform(4.0, 10.0, size=n_out)
            if q is not None:
                q[:, h, :, dims] *= qf[:, None, None]
            n_tail = int(prng.integers(2, 6))
            tail = list(dims)
            if len(tail) < n_tail:
                rest = np.setdiff1d(np.arange(d), dims)
                tail += list(prng.choice(rest, size=n_tail - len(tail), replace=False))
            tail = np.array(tail)
            prng.shuffle(tail)
            # random partition of the tail into n_tail non-empty groups (ids 1..n_tail)
            lab = np.concatenate([np.arange(n_tail), prng.integers(0, n_tail, size=len(tail) - n_tail)])
            prng.shuffle(lab)
            gamma[h, tail] = (lab + 1).astype(np.uint8)
            Gs[h] = n_tail + 1
            Ls[h] = draw_L(prng, n_tail + 1, 6)
    # q left at zero is a read-only broadcast view (no memory)
    q = round_bf16(_rope(q, pos0)) if q is not None else np.broadcast_to(np.float32(0.0), qshape)
    k = round_bf16(_rope(k, pos0))
    v = round_bf16(v)
    params = HeadParams(Gs, gamma, Ls, np.full(n_q_heads, 1e-3, dtype=np.float32))
    return Inputs(name, q, k, v, params, "bf16", seed, {"outlier_dims": outliers})


def cfg2(seed: int = 2) -> Inputs:
    """B=1, T=4096, 14q/2kv, bf16 (the prefill headline workload)."""
    return qwen_like(1, 4096, seed, name="cfg2")


def cfg3(seed: int = 3) -> Inputs:
    """B=8 x T=4096, sequence b drawn from seed 3*1000+b; shared head structure."""
    return qwen_like(8, 4096, seed, name="cfg3",
                     per_seq_seeds=[seed * 1000 + b for b in range(8)])


def cfg4(seed: int = 4) -> Inputs:
    """B=1, T=32768 long context."""
    return qwen_like(1, 32768, seed, name="cfg4")


def cfg5_prefix(seed: int = 5, n_seq: int = 64, T: int = 4096) -> Inputs:
    """Decode workload prefix: n_seq sequences of T tokens (q left at zero: only k, v build the state)."""
    return qwen_like(n_seq, T, seed, name="cfg5_prefix", q_zero=True,
                     per_seq_seeds=[seed * 1000 + b for b in range(n_seq)])


def cfg5_steps(seed: int = 5, n_seq: int = 64, steps: int = 256, T0: int = 4096) -> Inputs:
    """Decode workload tokens: `steps` new tokens per sequence at positions T0.., same head structure
    (structure drawn from the cfg5 prefix seed so groups and L match the prefix)."""
    return qwen_like(n_seq, steps, seed, name="cfg5_steps",
                     per_seq_seeds=[seed * 1000 + 500 + b for b in range(n_seq)],
                     pos0=T0, structure_seed=seed)


def small(seed: int, B: int, Hq: int, Hkv: int, T: int, dtype: str = "bf16", d: int = D_H,
          g_hi: int = 6, outlier_scale: float = 6.0, allow_empty: bool = False) -> Inputs:
    """Small random case for parity tests: arbitrary grouping, a few outlier dims."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, d))
    k = rng.standard_normal((B, Hkv, T, d))
    v = rng.standard_normal((B, Hkv, T, d))
    nout = min(4, d)
    dims = rng.choice(d, size=nout, replace=False)
    q[..., dims] *= outlier_scale
    k[..., dims] *= outlier_scale
    params = random_params(rng, Hq, d, g_hi=g_hi, allow_empty=allow_empty)
    if dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    else:
        q, k, v = q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)
    return Inputs(f"small_s{seed}", q, k, v, params, dtype, seed)
