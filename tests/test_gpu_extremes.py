"""Extreme-value and maximum-size parity cases, checked against the oracle.

* Attention whose scores grow along the key order by more than 32 (log2 units) per
  64-key tile, so that the running softmax reference must move on every tile; scores
  that fall along the keys, so that later tiles underflow to zero; and huge scores of
  random sign (exponents in the hundreds).  A kernel that skipped a rescale would
  overflow or lose the dominant keys; the oracle subtracts the exact row maximum in
  float64 (plain definition of softmax).
* The whole path (score, top-l, gather, passing, attention) at the largest head
  count the boundary accepts (256 q heads), with GQA groups of 32 and of 256 q heads
  per kv head.
Bars are those of apb_gpu_util.
"""
import numpy as np
import pytest
import torch

from oracle import apb_oracle as orc
from sparse_block_attention_amd import binding as B
from sparse_block_attention_amd import synth
from sparse_block_attention_amd.tensors import from_device_bf16, to_device_bf16, to_device_f32

from apb_gpu_util import check_attention, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _segments(t_of_key, L, A, P, Hkv, d, seed):
    """K rows whose every entry is t (the key's position value), V random; split into
    anchor, passing and local segments in key order."""
    rng = np.random.default_rng(seed)
    k = _bf16(np.repeat(np.repeat(t_of_key[:, None, None], Hkv, 1), d, 2))
    v = _bf16(rng.uniform(-1, 1, size=(A + P + L, Hkv, d)))
    return (k[:A], v[:A]), (k[A:A + P], v[A:A + P]), (k[A + P:], v[A + P:])


def _run_attention(q, anc, pas, loc, p, l, Hq, Hkv, d, scale):
    L, A, P = q.shape[0], anc[0].shape[0], pas[0].shape[0]
    pr = B.Problem(Hq, Hkv, d, L, A, l, p, p + 1, None)
    dv = lambda x: to_device_bf16(x) if x.shape[0] else None
    out, lse = B.apb_block_attention(pr, to_device_bf16(q), dv(anc[0]), dv(anc[1]), dv(pas[0]), dv(pas[1]),
                                     to_device_bf16(loc[0]), to_device_bf16(loc[1]), softmax_scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = orc.block_attention(q, anc[0], anc[1], pas[0], pas[1], loc[0], loc[1], scale=scale)
    return from_device_bf16(out), lse.cpu().numpy(), o_ref, lse_ref


@pytest.mark.parametrize("direction", ["growing", "falling"])
@pytest.mark.parametrize("d", [128, 64])
def test_attention_scores_move_every_tile(direction, d):
    """q is all ones, every entry of key j is t_j = 0.01 j (growing) or 0.01 (n - j)
    (falling), softmax scale 1: s = d t_j, so consecutive 64-key tiles differ by
    64 * 0.01 * d * log2(e) > 32 in log2 units, and the row maxima reach ~1e3."""
    L, A, p, l, Hq, Hkv = 600, 70, 2, 100, 4, 2
    P = p * l
    n = A + P + L
    j = np.arange(n, dtype=np.float64)
    t = 0.01 * j if direction == "growing" else 0.01 * (n - 1 - j)
    anc, pas, loc = _segments(t, L, A, P, Hkv, d, seed=d)
    q = np.ones((L, Hq, d), np.float32)
    o, lse, o_ref, lse_ref = _run_attention(q, anc, pas, loc, p, l, Hq, Hkv, d, scale=1.0)
    assert np.isfinite(lse).all()
    check_attention(o, o_ref, lse, lse_ref, f"{direction} d={d}")


@pytest.mark.parametrize("d", [128, 64])
def test_attention_huge_random_scores(d):
    """Entries of q and k are +-8 with random signs (scores up to 8*8*d), default scale:
    softmax exponents in the hundreds, dominated by a few keys per row."""
    L, A, p, l, Hq, Hkv = 333, 65, 1, 130, 6, 3
    P = p * l
    rng = np.random.default_rng(7 + d)
    sgn = lambda shape: _bf16(8.0 * rng.choice([-1.0, 1.0], size=shape))
    q = sgn((L, Hq, d))
    anc = (sgn((A, Hkv, d)), _bf16(rng.uniform(-1, 1, (A, Hkv, d))))
    pas = (sgn((P, Hkv, d)), _bf16(rng.uniform(-1, 1, (P, Hkv, d))))
    loc = (sgn((L, Hkv, d)), _bf16(rng.uniform(-1, 1, (L, Hkv, d))))
    o, lse, o_ref, lse_ref = _run_attention(q, anc, pas, loc, p, l, Hq, Hkv, d, scale=None)
    check_attention(o, o_ref, lse, lse_ref, f"huge scores d={d}")


@pytest.mark.parametrize("Hq,Hkv,d,L,A,l,H,hidden", [
    (256, 8, 64, 300, 40, 50, 3, 32),      # 256 q heads, groups of 32
    (256, 1, 64, 130, 16, 20, 2, 64),      # one kv head for 256 q heads
])
def test_path_at_max_heads(Hq, Hkv, d, L, A, l, H, hidden):
    """Scores (all tokens), top-l and gather (bit-exact), passing (bit-exact) and
    attention (all rows) of the last host, at 256 q heads."""
    w = synth.Workload(f"maxheads_{Hkv}", 300 + Hkv, H, L, A, l, Hq, Hkv, d, hidden, 1.0, 2)
    wts = synth.scorer_weights(w)
    sc = {"w1": to_device_bf16(wts["w1"]), "b1": to_device_f32(wts["b1"]), "w2": to_device_f32(wts["w2"]),
          "b2": to_device_f32(wts["b2"])}
    ka, va = synth.anchor_kv(w)
    kcs, vcs, kc_np, vc_np = [], [], [], []
    for j in range(H):
        q, k, v = synth.host_block(w, j)
        pr = B.Problem(Hq, Hkv, d, L, A, l, j, H, None)
        qd, kd, vd = to_device_bf16(q), to_device_bf16(k), to_device_bf16(v)
        scores = B.apb_score_kv(pr, sc, qd, kd, vd)
        idx, kc, vc = B.apb_topk_gather(pr, scores, kd, vd)
        torch.cuda.synchronize()
        s_np = scores.cpu().numpy()
        s_ref = orc.score_kv(q, k, v, wts["w1"], wts["b1"], wts["w2"], wts["b2"])
        assert np.all(np.abs(s_np - s_ref) <= 1e-4 * (1 + np.abs(s_ref))), f"host {j} scores"
        idx_np = idx.cpu().numpy()
        assert np.array_equal(idx_np, orc.topl(s_np, l)), f"host {j} top-l"
        kr, vr = orc.gather(k, v, idx_np)
        assert np.array_equal(from_device_bf16(kc), kr) and np.array_equal(from_device_bf16(vc), vr)
        if j < H - 1:
            kcs.append(kc)
            vcs.append(vc)
            kc_np.append(kr)
            vc_np.append(vr)
            continue
        kp, vp = B.apb_build_passing(pr, kcs, vcs)
        kp_ref, vp_ref = orc.build_passing(kc_np, vc_np)
        kp_np, vp_np = from_device_bf16(kp), from_device_bf16(vp)
        assert np.array_equal(kp_np, kp_ref) and np.array_equal(vp_np, vp_ref), "passing"
        out, lse = B.apb_block_attention(pr, qd, to_device_bf16(ka), to_device_bf16(va), kp, vp, kd, vd)
        torch.cuda.synchronize()
        o_ref, lse_ref = orc.block_attention(q, ka, va, kp_np, vp_np, k, v)
        check_attention(from_device_bf16(out), o_ref, lse.cpu().numpy(), lse_ref, f"max heads Hkv={Hkv}")
