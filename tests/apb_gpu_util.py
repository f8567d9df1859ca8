"""Helpers shared by the GPU parity tests: device upload and the parity bars.

Bars (fixed before any kernel ran):
  * scores: |s - s_ref| <= 1e-4 * (1 + |s_ref|)  (bf16 products are exact in fp32;
    only the fp32 summation order differs from the float64 oracle);
  * indices, compressed blocks, passing block: bit-exact;
  * attention output: max |o - o_ref| <= 2e-2 and sum|o - o_ref| / sum|o_ref| <= 1e-2
    (bf16 inputs and output, fp32 accumulation);
  * log-sum-exp: |lse - lse_ref| <= 1e-3 * max(1, |lse_ref|).
"""
import numpy as np
import pytest
import torch

SCORE_RTOL = 1e-4
ATTN_MAX_ABS = 2e-2
ATTN_REL_L1 = 1e-2
LSE_TOL = 1e-3


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    from sparse_block_attention_amd import binding
    binding.lib()  # raises if the HIP library is missing


def check_scores(got: np.ndarray, ref: np.ndarray, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bound = SCORE_RTOL * (1 + np.abs(ref))
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} scores off, worst {err.max():.3e}"


def check_attention(o_got: np.ndarray, o_ref: np.ndarray, lse_got=None, lse_ref=None, what=""):
    o_got = np.asarray(o_got, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    assert np.isfinite(o_got).all(), f"{what}: non-finite output"
    diff = np.abs(o_got - o_ref)
    max_abs = diff.max() if diff.size else 0.0
    rel = diff.sum() / max(np.abs(o_ref).sum(), 1e-300)
    assert max_abs <= ATTN_MAX_ABS, f"{what}: max abs {max_abs:.3e}"
    assert rel <= ATTN_REL_L1, f"{what}: rel L1 {rel:.3e}"
    if lse_got is not None:
        lse_got = np.asarray(lse_got, np.float64)
        lse_ref = np.asarray(lse_ref, np.float64)
        e = np.abs(lse_got - lse_ref)
        assert (e <= LSE_TOL * np.maximum(1, np.abs(lse_ref))).all(), f"{what}: lse err {e.max():.3e}"
    return max_abs, rel


def sample_rows(L: int, n: int, seed: int = 0, tile: int = 128) -> np.ndarray:
    """First/last rows, rows at tile edges, and a seeded spread over [0, L)."""
    fixed = {0, 1, L - 1, L // 2}
    for t in (tile - 1, tile, 2 * tile - 1, L - tile, L - tile - 1):
        if 0 <= t < L:
            fixed.add(t)
    rng = np.random.default_rng(seed)
    extra = rng.choice(L, size=min(L, max(0, n - len(fixed))), replace=False)
    return np.array(sorted(fixed | set(int(x) for x in extra)), dtype=np.int64)
