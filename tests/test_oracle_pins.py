"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test states what fixes the expected value: a hand derivation, a closed
form, a special case that reduces to a library routine (torch's
scaled_dot_product_attention / logsumexp in float64 on the CPU), an invariant,
or brute force on tiny inputs.  Sources are the APB pages: the arXiv abstract
(mlsanity.com/paper/2502.12085) and the juejin.cn explainer, sections
"APB 的主要功能" and "APB 的技术原理".
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

from oracle import apb_oracle as orc
from sparse_block_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa_causal(q, k, v, head_map, scale):
    """torch SDPA (float64, causal) over a full sequence; K/V expanded per q head."""
    T, Hq, d = q.shape
    kx = np.stack([k[:, head_map[i], :] for i in range(Hq)], axis=1)
    vx = np.stack([v[:, head_map[i], :] for i in range(Hq)], axis=1)
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(kx.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(vx.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    logits = torch.matmul(tq, tk.transpose(-1, -2)) * scale
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
    return o[0].numpy().transpose(1, 0, 2), lse[0].numpy()


# --------------------------------------------------------------------------- attention


def test_hand_worked_example():
    """Exact weights w**q via keys ln(w): values derived by hand (tests/golden)."""
    with open(os.path.join(GOLDEN, "attention_hand_example.json")) as f:
        g = json.load(f)
    x = g["inputs"]
    q = np.array(x["q"], dtype=np.float64)                       # [L=2, Hq=2, d=1]
    col = lambda a: np.array(a, dtype=np.float64).reshape(-1, 1, 1)
    o, lse = orc.block_attention(
        q, np.log(col(x["k_anchor_log_of"])), col(x["v_anchor"]),
        np.log(col(x["k_pass_log_of"])), col(x["v_pass"]),
        np.log(col(x["k_local_log_of"])), col(x["v_local"]),
        scale=x["scale"], kv_head_of_q=x["kv_head_of_q"])
    nd = np.array(g["expected"]["out_num_den"], dtype=np.float64)
    np.testing.assert_allclose(o[:, :, 0], nd[..., 0] / nd[..., 1], rtol=1e-13)
    np.testing.assert_allclose(lse, np.log(np.array(g["expected"]["lse_log_of"], float)), rtol=1e-13)


def test_anchor_only_equals_causal_attention():
    """P = 0 and anchor = sequence start: the last L rows of causal attention over [anchor; local]."""
    A, L, Hq, Hkv, d = 24, 40, 4, 2, 16
    hm = np.array([1, 0, 1, 0])
    q = _rand((A + L, Hq, d), 1)
    k = _rand((A + L, Hkv, d), 2)
    v = _rand((A + L, Hkv, d), 3)
    scale = 0.3
    o, lse = orc.block_attention(q[A:], k[:A], v[:A], None, None, k[A:], v[A:],
                                 scale=scale, kv_head_of_q=hm)
    o_ref, lse_ref = _sdpa_causal(q, k, v, hm, scale)
    np.testing.assert_allclose(o, o_ref[A:], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref[:, A:], rtol=1e-12, atol=1e-12)


def test_all_earlier_tokens_passed_equals_full_causal_attention():
    """A = 0 and l = L: host p's outputs equal rows [pL,(p+1)L) of full causal attention.

    Runs the oracle's whole chain (score, top-l, gather, build, attention).
    """
    w = synth.Workload("pin", 101, 3, 32, 0, 32, 4, 2, 16, 8, 1.0, 2)
    blocks = [synth.host_block(w, j) for j in range(w.n_hosts)]
    wts = synth.scorer_weights(w)
    kc, vc = [], []
    for j in range(w.host):
        _, idx, a, b = orc.compress_host(*blocks[j], wts, w.pass_per_host)
        assert np.array_equal(idx, np.tile(np.arange(w.local_len), (w.n_kv_heads, 1)))
        kc.append(a)
        vc.append(b)
    kp, vp = orc.build_passing(kc, vc)
    q, k, v = blocks[w.host]
    o, lse = orc.block_attention(q, None, None, kp, vp, k, v)
    Q = np.concatenate([b[0] for b in blocks]).astype(np.float64)
    K = np.concatenate([b[1] for b in blocks]).astype(np.float64)
    V = np.concatenate([b[2] for b in blocks]).astype(np.float64)
    o_ref, lse_ref = _sdpa_causal(Q, K, V, np.arange(4) // 2, 1 / np.sqrt(16))
    lo = w.host * w.local_len
    np.testing.assert_allclose(o, o_ref[lo:], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref[:, lo:], rtol=1e-12, atol=1e-12)


def test_zero_query_gives_mean_of_visible_values():
    """q = 0: uniform weights, so O[r] = mean of the A + P + r + 1 visible V rows."""
    A, P, L, Hq, Hkv, d = 5, 7, 9, 2, 1, 8
    va, vp, vl = _rand((A, Hkv, d), 4), _rand((P, Hkv, d), 5), _rand((L, Hkv, d), 6)
    ka, kp, kl = _rand((A, Hkv, d), 7), _rand((P, Hkv, d), 8), _rand((L, Hkv, d), 9)
    o, lse = orc.block_attention(np.zeros((L, Hq, d)), ka, va, kp, vp, kl, vl)
    allv = np.concatenate([va, vp, vl])[:, 0]
    for r in range(L):
        n = A + P + r + 1
        for i in range(Hq):
            np.testing.assert_allclose(o[r, i], allv[:n].mean(axis=0), rtol=1e-13, atol=1e-14)
            assert abs(lse[i, r] - np.log(n)) < 1e-13


def test_permuting_anchor_or_passing_rows_changes_nothing():
    A, P, L, Hq, Hkv, d = 11, 13, 17, 3, 1, 8
    q = _rand((L, Hq, d), 10)
    ka, va = _rand((A, Hkv, d), 11), _rand((A, Hkv, d), 12)
    kp, vp = _rand((P, Hkv, d), 13), _rand((P, Hkv, d), 14)
    kl, vl = _rand((L, Hkv, d), 15), _rand((L, Hkv, d), 16)
    o, lse = orc.block_attention(q, ka, va, kp, vp, kl, vl)
    pa, pp = np.random.default_rng(0).permutation(A), np.random.default_rng(1).permutation(P)
    o2, lse2 = orc.block_attention(q, ka[pa], va[pa], kp[pp], vp[pp], kl, vl)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)
    # ... while permuting local rows does change it (the causal mask is position-based).
    pl = np.random.default_rng(2).permutation(L)
    o3, _ = orc.block_attention(q, ka, va, kp, vp, kl[pl], vl[pl])
    assert not np.allclose(o3, o)


def test_single_local_token_without_anchor_or_passing():
    """L = 1, A = P = 0: o = v0 and lse = scale * <q, k0>."""
    q, k, v = _rand((1, 2, 16), 20), _rand((1, 1, 16), 21), _rand((1, 1, 16), 22)
    o, lse = orc.block_attention(q, None, None, None, None, k, v, scale=0.37)
    np.testing.assert_allclose(o[0, 0], v[0, 0], rtol=1e-15)
    np.testing.assert_allclose(o[0, 1], v[0, 0], rtol=1e-15)
    np.testing.assert_allclose(lse[:, 0], 0.37 * (q[0] @ k[0, 0]), rtol=1e-13)


def test_duplicated_key_counts_twice():
    """A key present in both anchor and passing gets weight 2*exp(logit): logit + ln 2."""
    d, L = 8, 3
    q = _rand((L, 1, d), 30)
    kdup, vdup = _rand((1, 1, d), 31), _rand((1, 1, d), 32)
    kl, vl = _rand((L, 1, d), 33), _rand((L, 1, d), 34)
    o, lse = orc.block_attention(q, kdup, vdup, kdup, vdup, kl, vl, scale=1.0)
    for r in range(L):
        logit = [q[r, 0] @ kdup[0, 0] + np.log(2.0)] + [q[r, 0] @ kl[c, 0] for c in range(r + 1)]
        vals = [vdup[0, 0]] + [vl[c, 0] for c in range(r + 1)]
        wts = np.exp(np.array(logit))
        np.testing.assert_allclose(o[r, 0], (wts[:, None] * np.array(vals)).sum(0) / wts.sum(),
                                   rtol=1e-12)
        np.testing.assert_allclose(lse[0, r], np.log(wts.sum()), rtol=1e-12)


def test_row_subset_matches_all_rows():
    q = _rand((50, 2, 8), 40)
    ka, va = _rand((3, 1, 8), 41), _rand((3, 1, 8), 42)
    kl, vl = _rand((50, 1, 8), 43), _rand((50, 1, 8), 44)
    o, lse = orc.block_attention(q, ka, va, None, None, kl, vl, chunk=7)
    rows = np.array([49, 0, 17, 33])
    o2, lse2 = orc.block_attention(q, ka, va, None, None, kl, vl, rows=rows, heads=[1])
    np.testing.assert_allclose(o2[:, 0], o[rows, 1], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2[0], lse[1, rows], rtol=1e-13)


# ------------------------------------------------------------- attention in parts + merge


def _sdpa_masked(q, K, V, visible, head_map, scale):
    """torch SDPA (float64) of q [R, Hq, d] over keys K, V [n, Hkv, d] with a boolean
    visibility mask [R, n]; also the log-sum-exp from torch.logsumexp."""
    R, Hq, d = q.shape
    kx = np.stack([K[:, head_map[i], :] for i in range(Hq)], axis=0)[None]   # [1, Hq, n, d]
    vx = np.stack([V[:, head_map[i], :] for i in range(Hq)], axis=0)[None]
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk, tv = torch.from_numpy(kx), torch.from_numpy(vx)
    mask = torch.from_numpy(visible)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    logits = torch.matmul(tq, tk.transpose(-1, -2)) * scale
    lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
    return o[0].numpy().transpose(1, 0, 2), lse[0].numpy()


def _parts_problem(seed=60, A=6, P=10, L=13, Hq=4, Hkv=2, d=8):
    r = lambda shape, s: _rand(shape, seed + s)
    return (r((L, Hq, d), 0), r((A, Hkv, d), 1), r((A, Hkv, d), 2), r((P, Hkv, d), 3),
            r((P, Hkv, d), 4), r((L, Hkv, d), 5), r((L, Hkv, d), 6))


SEGMENT_SUBSETS = [s for n in (1, 2, 3) for s in itertools.combinations(orc.SEGMENTS_ALL, n)]


@pytest.mark.parametrize("segments", SEGMENT_SUBSETS, ids=lambda s: "+".join(s))
def test_segment_subset_equals_masked_sdpa(segments):
    """Any subset of the key segments: SDPA over the chosen keys, the local ones causal."""
    q, ka, va, kp, vp, kl, vl = _parts_problem()
    hm = np.array([1, 0, 0, 1])
    L = q.shape[0]
    Ks, Vs, vis = [], [], []
    for name, K, V in (("anchor", ka, va), ("passing", kp, vp)):
        if name in segments:
            Ks.append(K)
            Vs.append(V)
            vis.append(np.ones((L, K.shape[0]), dtype=bool))
    if "local" in segments:
        Ks.append(kl)
        Vs.append(vl)
        vis.append(np.tril(np.ones((L, L), dtype=bool)))
    o_ref, lse_ref = _sdpa_masked(q, np.concatenate(Ks), np.concatenate(Vs), np.concatenate(vis, axis=1),
                                  hm, 0.4)
    o, lse = orc.block_attention(q, ka, va, kp, vp, kl, vl, scale=0.4, kv_head_of_q=hm,
                                 segments=segments, chunk=5)
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("split", [(("anchor", "local"), ("passing",)),
                                   (("anchor",), ("passing", "local")),
                                   (("local",), ("anchor", "passing"))],
                         ids=["al|p", "a|pl", "l|ap"])
def test_merge_of_two_parts_equals_whole(split):
    """Softmax over a disjoint union: merging the parts gives the one-pass result."""
    q, ka, va, kp, vp, kl, vl = _parts_problem(seed=70)
    o_all, lse_all = orc.block_attention(q, ka, va, kp, vp, kl, vl)
    oa, la = orc.block_attention(q, ka, va, kp, vp, kl, vl, segments=split[0])
    ob, lb = orc.block_attention(q, ka, va, kp, vp, kl, vl, segments=split[1])
    o, lse = orc.merge_attention(oa, la, ob, lb)
    np.testing.assert_allclose(o, o_all, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lse_all, rtol=1e-13, atol=1e-13)
    o2, lse2 = orc.merge_attention(ob, lb, oa, la)           # symmetric
    np.testing.assert_allclose(o2, o, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=1e-15)


def test_merge_closed_forms():
    """Empty side (lse = -inf) is the identity; a part merged with itself keeps O and
    adds ln 2 to lse; two empty sides stay empty (O = 0, lse = -inf)."""
    o = _rand((5, 3, 4), 80)
    lse = _rand((3, 5), 81)
    empty_o, empty_l = np.full_like(o, 7.0), np.full_like(lse, -np.inf)
    m, ml = orc.merge_attention(o, lse, empty_o, empty_l)
    assert np.array_equal(m, o) and np.array_equal(ml, lse)
    m, ml = orc.merge_attention(o, lse, o, lse)
    np.testing.assert_allclose(m, o, rtol=1e-15)
    np.testing.assert_allclose(ml, lse + np.log(2.0), rtol=1e-15, atol=1e-15)
    m, ml = orc.merge_attention(empty_o, empty_l, empty_o, empty_l)
    assert np.all(m == 0.0) and np.all(ml == -np.inf)


def test_rows_with_no_visible_key():
    """Passing only with P = 0: nothing to attend, O = 0 and lse = -inf."""
    q, ka, va, kp, vp, kl, vl = _parts_problem(P=0)
    o, lse = orc.block_attention(q, ka, va, kp, vp, kl, vl, segments=("passing",))
    assert np.all(o == 0.0) and np.all(lse == -np.inf)


# --------------------------------------------------------------------------- QKV projection


def test_qkv_projection_reads_the_weight_rows():
    """One-hot weight rows copy single input features into chosen output slots; zero rows give
    zero; the output is linear in x (brute-force dot products on a tiny case)."""
    rows, hidden, Hq, Hkv, d = 3, 8, 2, 1, 4
    x = _rand((rows, hidden), 95)
    wq = np.zeros((Hq * d, hidden))
    wq[5, 2] = 1.0                                   # q head 1, dim 1 <- feature 2
    wk = np.zeros((Hkv * d, hidden))
    wk[3, 7] = -2.0                                  # k dim 3 <- -2 * feature 7
    wv = _rand((Hkv * d, hidden), 96)
    q, k, v = orc.qkv_projection(x, wq, wk, wv, Hq, Hkv)
    assert q.shape == (rows, Hq, d) and k.shape == (rows, Hkv, d)
    np.testing.assert_array_equal(q[:, 1, 1], x[:, 2])
    assert np.count_nonzero(q) == np.count_nonzero(x[:, 2])
    np.testing.assert_array_equal(k[:, 0, 3], -2.0 * x[:, 7])
    for r in range(rows):
        for c in range(d):
            assert abs(v[r, 0, c] - sum(x[r, i] * wv[c, i] for i in range(hidden))) < 1e-12
    q2, _, _ = orc.qkv_projection(3.0 * x, wq, wk, wv, Hq, Hkv)
    np.testing.assert_allclose(q2, 3.0 * q, rtol=1e-15)


# --------------------------------------------------------------------------- rotary embedding


def test_rope_hand_values_and_position_zero():
    """d = 2, theta_0 = 1: (1, 0) and (0, 1) at position 1 turn by one radian; position 0 is the identity."""
    x = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])                      # rows at positions 1 and 2
    o = orc.rope(x, 1, 10000.0)
    np.testing.assert_allclose(o[0, 0], [np.cos(1.0), np.sin(1.0)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[1, 0], [-np.sin(2.0), np.cos(2.0)], rtol=0, atol=1e-15)
    y = _rand((3, 2, 8), 90)
    assert np.array_equal(orc.rope(y[:1], 0, 500000.0), y[:1])


def test_rope_frequency_schedule_hand_values():
    """The frequency of pair i is base^(-2i/d).  With base 10^4: d = 4 gives frequencies
    1 and 10^-2, so at position 100 pair (0, 2) turns by 100 rad and pair (1, 3) by exactly
    1 rad; d = 8 gives 1, 10^-1, 10^-2, 10^-3, so at position 1000 pairs 0..3 turn by
    1000, 100, 10 and 1 rad.  The angles are written out by hand: another schedule (for
    example base^(-i/d), which gives 10^-1 at d = 4) moves every pair but the first."""
    for d, pos, angles in [(4, 100, [100.0, 1.0]), (8, 1000, [1000.0, 100.0, 10.0, 1.0])]:
        half = d // 2
        for i, a in enumerate(angles):
            e_lo = np.zeros((1, 1, d))
            e_lo[0, 0, i] = 1.0                      # first element of pair i
            e_hi = np.zeros((1, 1, d))
            e_hi[0, 0, i + half] = 1.0               # second element of pair i
            want_lo = np.zeros(d)
            want_lo[i], want_lo[i + half] = np.cos(a), np.sin(a)
            want_hi = np.zeros(d)
            want_hi[i], want_hi[i + half] = -np.sin(a), np.cos(a)
            np.testing.assert_allclose(orc.rope(e_lo, pos, 10000.0)[0, 0], want_lo, rtol=0, atol=1e-12)
            np.testing.assert_allclose(orc.rope(e_hi, pos, 10000.0)[0, 0], want_hi, rtol=0, atol=1e-12)
    # base 500000 (Llama 3) at d = 4: pair (1, 3) turns by sqrt(1 / 500000) rad per position
    e = np.zeros((1, 1, 4))
    e[0, 0, 1] = 1.0
    a = 7.0 / np.sqrt(500000.0)
    np.testing.assert_allclose(orc.rope(e, 7, 500000.0)[0, 0], [0, np.cos(a), 0, np.sin(a)], rtol=0, atol=1e-14)


def test_rope_is_a_rotation_by_relative_position():
    """Pair norms are kept; <R(p) q, R(p') k> depends on p - p' only; R(a) then R(b) is R(a + b)."""
    q, k = _rand((1, 1, 64), 91), _rand((1, 1, 64), 92)
    base = 10000.0
    rq = orc.rope(np.repeat(q, 40, axis=0), 0, base)                # q at positions 0..39
    rk = orc.rope(np.repeat(k, 40, axis=0), 0, base)
    for p, pk in [(5, 2), (17, 14), (39, 36)]:                      # all three differ by 3
        np.testing.assert_allclose(rq[p, 0] @ rk[pk, 0], rq[5, 0] @ rk[2, 0], rtol=1e-12)
    x = _rand((4, 3, 128), 93)
    o = orc.rope(x, 1000, 500000.0)
    norm = lambda t: t[..., :64] ** 2 + t[..., 64:] ** 2
    np.testing.assert_allclose(norm(o), norm(x), rtol=1e-12)
    # composition: a row at position 7 turned again by 5 equals the row at position 12
    x1 = x[:1]
    np.testing.assert_allclose(orc.rope(orc.rope(x1, 7, 500000.0), 5, 500000.0), orc.rope(x1, 12, 500000.0),
                               rtol=1e-9, atol=1e-12)


# --------------------------------------------------------------------------- scorer


def _scorer_problem(seed=0, L=6, Hq=4, Hkv=2, d=8, Hs=5):
    q, k, v = _rand((L, Hq, d), seed), _rand((L, Hkv, d), seed + 1), _rand((L, Hkv, d), seed + 2)
    return q, k, v


def test_scorer_zero_w1_is_bias_path():
    q, k, v = _scorer_problem()
    Hkv, Hs, din = 2, 5, 4 * 8
    b1, w2, b2 = _rand((Hkv, Hs), 3), _rand((Hkv, Hs), 4), _rand((Hkv,), 5)
    s = orc.score_kv(q, k, v, np.zeros((Hkv, Hs, din)), b1, w2, b2)
    for h in range(Hkv):
        expect = np.float32(np.maximum(b1[h], 0) @ w2[h] + b2[h])
        assert np.all(s[h] == expect)


@pytest.mark.parametrize("head_map", [[0, 0, 1, 1], [1, 0, 0, 1]])
def test_scorer_input_layout_one_hot(head_map):
    """A one-hot W1 row reads one coordinate of x = [q of G_h (ascending); k_h; v_h]."""
    L, Hq, Hkv, d, Hs = 6, 4, 2, 8, 3
    q, k, v = _scorer_problem(L=L, Hq=Hq, Hkv=Hkv, d=d, Hs=Hs)
    hm = np.array(head_map)
    g = Hq // Hkv
    b1, b2 = np.zeros((Hkv, Hs)), np.zeros(Hkv)
    w2 = np.zeros((Hkv, Hs))
    w2[:, 0] = 1.0
    for h in range(Hkv):
        grp = [i for i in range(Hq) if hm[i] == h]
        # (position in x, source column)
        picks = [(j * d + e, q[:, grp[j], e]) for j in range(g) for e in (0, d - 1)]
        picks += [(g * d + 3, k[:, h, 3]), ((g + 1) * d + 5, v[:, h, 5])]
        for pos, src in picks:
            w1 = np.zeros((Hkv, Hs, (g + 2) * d))
            w1[h, 0, pos] = 1.0
            s = orc.score_kv(q, k, v, w1, b1, w2, b2, kv_head_of_q=hm)
            np.testing.assert_array_equal(s[h], np.maximum(src, 0).astype(np.float32))
            other = 1 - h
            np.testing.assert_array_equal(s[other], np.zeros(L, np.float32))


def test_scorer_matches_per_token_loop():
    """Second coding of the scorer definition: scalar loops, no matrix products."""
    L, Hq, Hkv, d, Hs = 3, 4, 2, 4, 3
    q, k, v = _scorer_problem(L=L, Hq=Hq, Hkv=Hkv, d=d, Hs=Hs)
    w1 = _rand((Hkv, Hs, 4 * d), 6)
    b1, w2, b2 = _rand((Hkv, Hs), 7), _rand((Hkv, Hs), 8), _rand((Hkv,), 9)
    s = orc.score_kv(q, k, v, w1, b1, w2, b2)
    for h in range(Hkv):
        for t in range(L):
            x = list(q[t, 2 * h]) + list(q[t, 2 * h + 1]) + list(k[t, h]) + list(v[t, h])
            acc = b2[h]
            for u in range(Hs):
                z = b1[h, u] + sum(w1[h, u, c] * x[c] for c in range(len(x)))
                acc += w2[h, u] * max(z, 0.0)
            assert abs(float(s[h, t]) - acc) <= 1e-6 * (1 + abs(acc))
            assert s.dtype == np.float32


# --------------------------------------------------------------------------- top-l

_SPECIAL = np.array([-np.inf, -1.0, -0.0, 0.0, 0.5, 1.0, np.nan], dtype=np.float32)


def _brute_select(s, l):
    """Rank definition: rank_i = #{j that strictly precede i}; keep rank_i < l."""
    s = np.asarray(s, dtype=np.float32)
    n = len(s)
    nan = np.isnan(s)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    si, sj = s[:, None], s[None, :]
    ni, nj = nan[:, None], nan[None, :]
    with np.errstate(invalid="ignore"):
        num_beats = (~ni & ~nj) & ((sj > si) | ((sj == si) & (j < i)))
    beats = num_beats | (ni & ~nj) | (ni & nj & (j < i))
    rank = beats.sum(axis=1)
    return np.nonzero(rank < l)[0].astype(np.int32)


def test_topl_exhaustive_small():
    for n in range(0, 5):
        for combo in itertools.product(range(len(_SPECIAL)), repeat=n):
            s = _SPECIAL[list(combo)]
            for l in range(n + 1):
                got = orc.topl_one(s, l)
                assert np.array_equal(got, _brute_select(s, l)), (s, l, got)


@pytest.mark.parametrize("n,seed", [(37, 1), (256, 2), (1000, 3), (4096, 4)])
def test_topl_random_against_rank_definition(n, seed):
    rng = np.random.default_rng(seed)
    rows = [synth.tie_heavy_scores(1, n, seed)[0],
            rng.standard_normal(n).astype(np.float32)]
    for s in rows:
        for l in sorted({0, 1, n // 3, n // 2, n - 1, n}):
            got = orc.topl_one(s, l)
            assert np.array_equal(got, _brute_select(s, l))
            assert len(got) == l and np.all(np.diff(got) > 0)


def test_topl_selected_dominate_unselected():
    s = synth.tie_heavy_scores(1, 2000, 7)[0]
    sel = orc.topl_one(s, 700)
    mask = np.zeros(len(s), bool)
    mask[sel] = True
    key = np.where(np.isnan(s), -np.inf, s)
    # every kept number is >= every dropped number; NaN only kept once numbers run out
    assert key[mask].min() >= key[~mask & ~np.isnan(s)].max()
    assert not (np.isnan(s[mask]).any() and (~mask & ~np.isnan(s)).any())


def test_topl_rejects_bad_l():
    with pytest.raises(ValueError):
        orc.topl_one(np.zeros(4, np.float32), 5)


# --------------------------------------------------------------------------- gather / build


def test_gather_rows_decode_to_their_indices():
    L, Hkv, d = 40, 3, 4
    t = np.arange(L, dtype=np.float32)[:, None, None]
    h = np.arange(Hkv, dtype=np.float32)[None, :, None]
    k = np.broadcast_to(t + 1000 * h, (L, Hkv, d)).copy()
    v = np.broadcast_to(-t - 1000 * h, (L, Hkv, d)).copy()
    idx = np.stack([np.sort(np.random.default_rng(hh).choice(L, 9, replace=False))
                    for hh in range(Hkv)]).astype(np.int32)
    kc, vc = orc.gather(k, v, idx)
    for hh in range(Hkv):
        assert np.array_equal(kc[:, hh, 0] - 1000 * hh, idx[hh])
        assert np.array_equal(-vc[:, hh, 2] - 1000 * hh, idx[hh])


def test_build_passing_is_host_major():
    p, l, Hkv, d = 4, 5, 2, 3
    kc = [np.full((l, Hkv, d), 0.0) + (100 * j + np.arange(l))[:, None, None] for j in range(p)]
    vc = [-x for x in kc]
    kp, vp = orc.build_passing(kc, vc)
    assert kp.shape == (p * l, Hkv, d)
    for j in range(p):
        for s in range(l):
            assert np.all(kp[j * l + s] == 100 * j + s) and np.all(vp[j * l + s] == -(100 * j + s))
    assert orc.build_passing([], []) == (None, None)


# --------------------------------------------------------------------------- generator


def test_generator_deterministic_and_bf16():
    w = synth.WORKLOADS["tiny"]
    a = synth.host_block(w, 2)
    b = synth.host_block(w, 2)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
        assert not np.any(x.view(np.uint32) & 0xFFFF)
    c = synth.host_block(w, 1)
    assert not np.array_equal(a[0], c[0])
    assert abs(float(a[0].std()) - w.sigma) < 0.05


def test_generator_needles_scale_k_rows_by_eight():
    w = synth.Workload("n", 102, 4, 64, 8, 4, 2, 2, 16, 8, 0.5, 5)
    w0 = w.with_(needles=0)
    pos = synth.needle_positions(w)
    for j in range(w.n_hosts):
        _, k, _ = synth.host_block(w, j)
        _, k0, _ = synth.host_block(w0, j)
        expect = k0.copy()
        for h in range(w.n_kv_heads):
            for t in pos[h]:
                if j * 64 <= t < (j + 1) * 64:
                    expect[t - j * 64, h] *= 8
        assert np.array_equal(k, expect)
    assert sum(((pos >= j * 64) & (pos < (j + 1) * 64)).sum() for j in range(4)) == 10


def test_bf16_round_ties_to_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20],
                 dtype=np.float32)
    np.testing.assert_array_equal(synth.bf16_round(x),
                                  np.array([1.0, 1.0 + 2 ** -6, -1.0, 1.0 + 2 ** -7], np.float32))
