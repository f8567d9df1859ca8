"""Attention in parts and the merge of partial results: HIP path vs the oracle.

The passing block is the only attention input that waits for the exchange
between hosts, so a host can attend over anchor + local first, over the passing
block later, and merge.  Checked here: every non-empty subset of key segments
against the oracle's subset attention, the two-phase result (two launches +
merge) against the oracle's one-pass attention, the merge kernel against the
oracle's merge (including empty sides, lse = -inf, and merging in place), and
the full-size Llama-3.1-8B host-7 shape on sampled rows.  Bars in apb_gpu_util;
the merge kernel's own bar is derived in test_merge_kernel_matches_oracle_merge.
"""
import numpy as np
import pytest
import torch

from oracle import apb_oracle as orc
from sparse_block_attention_amd import binding as B
from sparse_block_attention_amd import synth
from sparse_block_attention_amd.tensors import from_device_bf16, to_device_bf16, to_device_f32

from apb_gpu_util import check_attention, require_gpu, sample_rows

pytestmark = pytest.mark.gpu

SEG_NAMES = {B.APB_SEG_ANCHOR: "anchor", B.APB_SEG_PASSING: "passing", B.APB_SEG_LOCAL: "local"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _names(mask):
    return tuple(n for bit, n in SEG_NAMES.items() if mask & bit)


def _inputs(L, A, p, l, Hq, Hkv, d, seed, sigma=1.0):
    P = p * l
    shapes = [(L, Hq, d), (A, Hkv, d), (A, Hkv, d), (P, Hkv, d), (P, Hkv, d), (L, Hkv, d), (L, Hkv, d)]
    host = [synth.random_bf16(s, seed + i, sigma=sigma, stream=L) for i, s in enumerate(shapes)]
    dev = [to_device_bf16(x) if x.shape[0] else None for x in host]
    return B.Problem(Hq, Hkv, d, L, A, l, p, p + 1, None), host, dev


SHAPES = [
    # L, A, p, l, Hq, Hkv, d: ragged tails, several tiles per segment, both head sizes
    (200, 70, 3, 33, 4, 2, 128),
    (129, 17, 2, 40, 6, 3, 64),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"L{s[0]}_d{s[6]}")
@pytest.mark.parametrize("mask", range(1, 8), ids=lambda m: "+".join(_names(m)))
def test_segment_subset_all_rows(shape, mask):
    pr, host, dev = _inputs(*shape, seed=10 * mask)
    out, lse = B.apb_block_attention_segments(pr, mask, *dev, softmax_scale=0.09)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.block_attention(*host, scale=0.09, segments=_names(mask))
    check_attention(from_device_bf16(out), o_ref, lse.cpu().numpy(), lse_ref, f"segments {_names(mask)}")


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"L{s[0]}_d{s[6]}")
def test_two_phases_then_merge_equal_one_pass(shape):
    """anchor + local, then passing, merged (out of place and in place) vs the oracle's one pass."""
    pr, host, dev = _inputs(*shape, seed=100)
    o1, l1 = B.apb_block_attention_segments(pr, B.APB_SEG_ANCHOR | B.APB_SEG_LOCAL, *dev)
    o2, l2 = B.apb_block_attention_segments(pr, B.APB_SEG_PASSING, *dev)
    om, lm = B.apb_merge_attention(pr, o1, l1, o2, l2)
    o_whole, l_whole = B.apb_block_attention(pr, *dev)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.block_attention(*host)
    check_attention(from_device_bf16(om), o_ref, lm.cpu().numpy(), lse_ref, "merged two phases")
    check_attention(from_device_bf16(o_whole), o_ref, l_whole.cpu().numpy(), lse_ref, "one pass")
    # in place into phase 1's buffers: same bits as out of place
    om_bits, lm_bits = om.clone(), lm.clone()
    B.apb_merge_attention(pr, o1, l1, o2, l2, out=o1, lse=l1)
    torch.cuda.synchronize()
    assert torch.equal(o1, om_bits) and torch.equal(l1, lm_bits)


def test_passing_only_without_passing_rows_is_empty():
    """Host 0 has no passing block: attending over it alone sees nothing (O = 0, lse = -inf)."""
    pr, host, dev = _inputs(70, 5, 0, 0, 2, 1, 128, seed=200)
    out = torch.full((70, 2, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    out, lse = B.apb_block_attention_segments(pr, B.APB_SEG_PASSING, *dev, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0).item()
    assert torch.all(lse == float("-inf")).item()


@pytest.mark.parametrize("L,Hq,d", [(37, 5, 128), (64, 3, 64), (1, 1, 64)])
def test_merge_kernel_matches_oracle_merge(L, Hq, d):
    """Random partial results, including empty sides and far-apart lse values.

    Bar: both sides merge the same bf16 inputs; the kernel computes in fp32 and
    rounds once to bf16 (relative error <= 2^-9), fp32 steps add a few 2^-24, so
    |o - o_ref| <= 2^-8 |o_ref| + 1e-6 per element; lse within 1e-6 relative.
    Empty rows must be exactly O = 0, lse = -inf.
    """
    rng = np.random.default_rng(L * 1000 + Hq)
    oa = synth.random_bf16((L, Hq, d), 300 + L, stream=1)
    ob = synth.random_bf16((L, Hq, d), 301 + L, stream=2)
    la = (rng.standard_normal((Hq, L)) * 30).astype(np.float32)
    lb = (rng.standard_normal((Hq, L)) * 30).astype(np.float32)
    kind = rng.integers(0, 5, size=(Hq, L))
    la[kind == 1] = -np.inf                       # a empty
    lb[kind == 2] = -np.inf                       # b empty
    la[kind == 3] = -np.inf                       # both empty
    lb[kind == 3] = -np.inf
    la[0, 0] = 88.0                               # exp(lse) alone would overflow fp32
    lb[0, 0] = -90.0
    pr = B.Problem(Hq, 1, d, L, 0, 0, 0, 1, None)
    o, lse = B.apb_merge_attention(pr, to_device_bf16(oa), to_device_f32(la), to_device_bf16(ob),
                                   to_device_f32(lb))
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.merge_attention(oa, la, ob, lb)
    o_got = from_device_bf16(o).astype(np.float64)
    lse_got = lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_got), empty)
    assert np.all(o_got[empty.T] == 0.0)
    assert np.all(np.abs(o_got - o_ref) <= 2.0 ** -8 * np.abs(o_ref) + 1e-6)
    fin = ~empty
    assert np.all(np.abs(lse_got[fin] - lse_ref[fin]) <= 1e-6 * np.maximum(1.0, np.abs(lse_ref[fin])))


def test_llama8b_two_phases_sampled_rows():
    """Llama-3.1-8B host 7 of 8 at 128K (L 16384, A 2048, P 7168, 32/8 heads, d 128)."""
    L, A, p, l, Hq, Hkv, d = 16384, 2048, 7, 1024, 32, 8, 128
    pr, host, dev = _inputs(L, A, p, l, Hq, Hkv, d, seed=400, sigma=0.5)
    o1, l1 = B.apb_block_attention_segments(pr, B.APB_SEG_ANCHOR | B.APB_SEG_LOCAL, *dev)
    o2, l2 = B.apb_block_attention_segments(pr, B.APB_SEG_PASSING, *dev)
    om, lm = B.apb_merge_attention(pr, o1, l1, o2, l2)
    torch.cuda.synchronize()
    rows = sample_rows(L, 40, seed=3)
    o_ref, lse_ref = orc.block_attention(*host, rows=rows)
    check_attention(from_device_bf16(om)[rows], o_ref, lm.cpu().numpy()[:, rows], lse_ref, "llama8b merged")


@pytest.mark.parametrize("mode", ["star", "full_causal"])
def test_baseline_modes_full_size_sampled_rows(mode):
    """The baselines the pages compare with, on the same kernel at the Llama-3.1-8B shape:
    Star Attention (anchor = a whole 16384-token block, no passing) and full causal attention
    of host 7 of 8 (all 114688 earlier tokens visible as one passing block, no anchor)."""
    L, Hq, Hkv, d, p = 16384, 32, 8, 128, 7
    if mode == "star":
        pr, host, dev = _inputs(L, L, p, 0, Hq, Hkv, d, seed=500, sigma=0.5)
    else:
        pr, host, dev = _inputs(L, 0, p, L, Hq, Hkv, d, seed=600, sigma=0.5)
    out, lse = B.apb_block_attention(pr, *dev)
    torch.cuda.synchronize()
    rows = sample_rows(L, 24, seed=4)
    o_ref, lse_ref = orc.block_attention(*host, rows=rows)
    check_attention(from_device_bf16(out)[rows], o_ref, lse.cpu().numpy()[:, rows], lse_ref, mode)
