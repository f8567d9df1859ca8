"""Seeded synthetic inputs for the APB per-host prefill path.

This module only draws random tensors: it holds none of the method's arithmetic
(no scoring, selection, gathering or attention).  The HIP path's tests and
benchmark and the CPU oracle both consume exactly what it returns, so the two
sides always see identical bits.

Workload shapes follow the four backbones whose retaining heads the juejin.cn
APB explainer lists (section "如何运行 APB", retaining-heads table: Llama-3.1-8B,
Qwen-2.5-14B, Yi-34B-200K, Llama-3-8B-1M) split evenly over 8 hosts (section
"APB 的主要功能", even split of the input across hosts), with the anchor at 1/8
or 1/4 of a block (section "APB 的技术原理", smaller anchor block).  Planted
high-norm keys stand in for the needle of the pages' NIAH example.

Recipe (every tensor):
  * stream = numpy PCG64 seeded by SeedSequence(seed, spawn_key=(config_id, host, tensor_id)),
    tensor ids q=0, k=1, v=2, needle positions=3, scorer weights=4
    (host 0 for the global tensors 3 and 4);
  * q, k, v: fp32 standard normals times sigma, rounded once to bf16 (round to nearest even);
  * needles: per kv head, `needles` positions drawn without replacement over the whole
    sequence [0, n_hosts * local_len); the k rows at those positions are multiplied by 8
    (exact in bf16);
  * scorer: W1 [Hkv, Hs, (g+2)d] ~ N(0, 0.1^2) rounded to bf16, b1 [Hkv, Hs], w2 [Hkv, Hs],
    b2 [Hkv] ~ N(0, 0.1^2) kept in fp32.
Arrays are returned as float32 holding bf16-representable values; `bf16_bits`
gives the 16-bit patterns for device upload.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

T_Q, T_K, T_V, T_NEEDLE, T_SCORER = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    """One evaluated host of an evenly split long-context prefill."""

    name: str
    config_id: int
    n_hosts: int
    local_len: int          # L: tokens per host block
    anchor_len: int         # A: first A tokens of the sequence, prepended on the evaluated host
    pass_per_host: int      # l: tokens kept per kv head per earlier host
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    hidden: int             # scorer hidden width Hs
    sigma: float
    needles: int            # planted high-norm keys per kv head over the whole sequence
    seed: int = 0
    host_index: int = -1    # evaluated host; -1 means the last one

    @property
    def host(self) -> int:
        return self.n_hosts - 1 if self.host_index < 0 else self.host_index

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def pass_len(self) -> int:
        return self.host * self.pass_per_host

    @property
    def seq_len(self) -> int:
        return self.n_hosts * self.local_len

    @property
    def scorer_in(self) -> int:
        return (self.group + 2) * self.head_dim

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 1024 tokens over 4 hosts of 256, anchor 64, 32 kept per earlier host.
    "tiny": Workload("tiny", 0, 4, 256, 64, 32, 2, 1, 64, 32, 1.0, 0),
    # Llama-3.1-8B layer, last of 8 hosts at 128K.
    "llama8b": Workload("llama8b", 1, 8, 16384, 2048, 1024, 32, 8, 128, 256, 0.5, 16),
    # Qwen-2.5-14B layer, last of 8 hosts at 128K, anchor 1/4 of a block.
    "qwen14b": Workload("qwen14b", 2, 8, 16384, 4096, 2048, 40, 8, 128, 256, 0.5, 16),
    # Yi-34B-200K layer, last of 8 hosts at 200K.
    "yi34b": Workload("yi34b", 3, 8, 25600, 3200, 1600, 56, 8, 128, 256, 0.5, 0),
    # Llama-3-8B-1M layer, last of 8 hosts at 1M.
    "llama1m": Workload("llama1m", 4, 8, 131072, 16384, 4096, 32, 8, 128, 256, 0.5, 64),
}


def rng_for(w: Workload, host: int, tensor_id: int) -> np.random.Generator:
    ss = np.random.SeedSequence(w.seed, spawn_key=(w.config_id, host, tensor_id))
    return np.random.Generator(np.random.PCG64(ss))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """16-bit patterns of float32 values that are exactly bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("array holds values that are not bf16-representable")
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(sigma)
    return bf16_round(x)


def needle_positions(w: Workload) -> np.ndarray:
    """int64 [Hkv, needles]: global token positions of the planted keys, per kv head."""
    rng = rng_for(w, 0, T_NEEDLE)
    out = np.zeros((w.n_kv_heads, w.needles), dtype=np.int64)
    for h in range(w.n_kv_heads):
        if w.needles:
            out[h] = np.sort(rng.choice(w.seq_len, size=w.needles, replace=False))
    return out


def host_block(w: Workload, host: int):
    """(q [L,Hq,d], k [L,Hkv,d], v [L,Hkv,d]) of host `host`'s block, bf16 values in float32."""
    L, d = w.local_len, w.head_dim
    q = _normal_bf16(rng_for(w, host, T_Q), (L, w.n_q_heads, d), w.sigma)
    k = _normal_bf16(rng_for(w, host, T_K), (L, w.n_kv_heads, d), w.sigma)
    v = _normal_bf16(rng_for(w, host, T_V), (L, w.n_kv_heads, d), w.sigma)
    if w.needles:
        pos = needle_positions(w)
        lo, hi = host * L, (host + 1) * L
        for h in range(w.n_kv_heads):
            for t in pos[h]:
                if lo <= t < hi:
                    k[t - lo, h, :] *= np.float32(8.0)
    return q, k, v


def anchor_kv(w: Workload):
    """(k_anchor, v_anchor) [A,Hkv,d]: the first A tokens of the sequence (host 0's block)."""
    if w.anchor_len > w.local_len:
        raise ValueError("anchor longer than a host block")
    _, k0, v0 = host_block(w, 0)
    return (np.ascontiguousarray(k0[: w.anchor_len]),
            np.ascontiguousarray(v0[: w.anchor_len]))


def scorer_weights(w: Workload):
    """Random stand-in for the retaining heads: dict of w1 (bf16 values), b1, w2, b2 (fp32)."""
    rng = rng_for(w, 0, T_SCORER)
    Hkv, Hs = w.n_kv_heads, w.hidden
    w1 = _normal_bf16(rng, (Hkv, Hs, w.scorer_in), 0.1)
    b1 = (rng.standard_normal((Hkv, Hs), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    w2 = (rng.standard_normal((Hkv, Hs), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    b2 = (rng.standard_normal((Hkv,), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    return {"w1": w1, "b1": b1, "w2": w2, "b2": b2}


def tie_heavy_scores(n_heads: int, n: int, seed: int, specials: bool = True) -> np.ndarray:
    """fp32 [n_heads, n] scores drawn from a small value set so that ties are common.

    With `specials`, the set includes -inf, +inf, -0.0, +0.0 and NaN.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(99,))))
    vals = [-2.0, -1.0, -0.5, 0.25, 0.5, 1.0, 3.0]
    if specials:
        vals += [-np.inf, np.inf, -0.0, 0.0, np.nan]
    vals = np.array(vals, dtype=np.float32)
    return vals[rng.integers(0, len(vals), size=(n_heads, n))]


def default_head_map(n_q_heads: int, n_kv_heads: int) -> np.ndarray:
    g = n_q_heads // n_kv_heads
    return (np.arange(n_q_heads) // g).astype(np.int32)


def random_bf16(shape, seed: int, sigma: float = 1.0, stream: int = 0) -> np.ndarray:
    """Seeded N(0, sigma^2) draws rounded to bf16 (float32 array), for arbitrary shapes."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(77, stream))))
    return _normal_bf16(rng, shape, sigma)
