"""Every output of every entry point, written inside guard bands.

Each output tensor is a view into a larger buffer whose every element first holds
a sentinel bit pattern (a NaN payload for floating point, -12345 for indices).
After the call: every element of the view has been overwritten (no sentinel left),
the guard elements before and after it still hold the sentinel (nothing written
past either end), the values match the oracle, and a second call gives the same
bits.  Sizes are ragged, so the last tile, chunk or workgroup of each kernel is
partial.  The top-l workspace is filled with garbage before the calls: its
contents on entry must not matter.
"""
import numpy as np
import pytest
import torch

from oracle import apb_oracle as orc
from sparse_block_attention_amd import binding as B
from sparse_block_attention_amd import synth
from sparse_block_attention_amd.tensors import from_device_bf16, to_device_bf16, to_device_f32

from apb_gpu_util import check_attention, check_scores, require_gpu

pytestmark = pytest.mark.gpu

G = 96  # guard elements on each side

SENTINEL = {torch.bfloat16: (torch.int16, 0x7FA5), torch.float32: (torch.int32, 0x7FC0DEAD),
            torch.int32: (torch.int32, -12345)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


class Guarded:
    """A device tensor of `shape` inside a sentinel-filled buffer with G guard elements each side."""

    def __init__(self, shape, dtype):
        self.n = int(np.prod(shape))
        self.dtype = dtype
        self.backing = torch.empty(self.n + 2 * G, dtype=dtype, device="cuda")
        ity, val = SENTINEL[dtype]
        self.bits = self.backing.view(ity)
        self.val = val
        self.bits.fill_(val)
        self.t = self.backing[G:G + self.n].view(*shape)

    def check(self, what):
        torch.cuda.synchronize()
        b = self.bits.cpu().numpy()
        assert (b[:G] == self.val).all(), f"{what}: written before the start"
        assert (b[G + self.n:] == self.val).all(), f"{what}: written past the end"
        body = b[G:G + self.n]
        assert not (body == self.val).any(), f"{what}: {(body == self.val).sum()} elements not written"

    def bits_copy(self):
        torch.cuda.synchronize()
        return self.bits.clone()


def _dev_scorer(wts):
    return {"w1": to_device_bf16(wts["w1"]), "b1": to_device_f32(wts["b1"]),
            "w2": to_device_f32(wts["w2"]), "b2": to_device_f32(wts["b2"])}


@pytest.mark.parametrize("L,Hq,Hkv,d,Hs", [(300, 4, 2, 128, 48), (16385, 4, 2, 64, 16), (257, 6, 3, 128, 256),
                                           (513, 2, 1, 64, 112)])
def test_score_kv_guarded(L, Hq, Hkv, d, Hs):
    """Scores of every token, ragged L (a partial last token tile), hidden widths that are
    multiples of 16 but not of 32 (48, 16, 112) and of 32 (256)."""
    w = synth.Workload("score_guard", 300 + L % 97, 1, L, 0, 1, Hq, Hkv, d, Hs, 1.0, 0)
    q, k, v = synth.host_block(w, 0)
    wts = synth.scorer_weights(w)
    s = Guarded((Hkv, L), torch.float32)
    args = (B.Problem(Hq, Hkv, d, L, 0, 1, 0, 1, None), _dev_scorer(wts), to_device_bf16(q), to_device_bf16(k),
            to_device_bf16(v))
    B.apb_score_kv(*args, scores=s.t)
    s.check("scores")
    ref = orc.score_kv(q, k, v, wts["w1"], wts["b1"], wts["w2"], wts["b2"])
    check_scores(s.t.cpu().numpy(), ref, "scores")
    first = s.bits_copy()
    B.apb_score_kv(*args, scores=s.t)
    assert torch.equal(s.bits_copy(), first), "scores differ between two calls"


@pytest.mark.parametrize("L,l,Hkv,d", [(300, 37, 2, 128), (16385, 1024, 3, 64), (256, 256, 1, 128),
                                       (40000, 4096, 2, 64), (1, 1, 2, 128)])
def test_topk_gather_guarded_with_garbage_workspace(L, l, Hkv, d):
    """idx, k_comp and v_comp written exactly; the workspace is filled with 0xFF bytes for
    the first call and random bytes for the second, with identical results."""
    rng = np.random.default_rng(L + l)
    s = rng.standard_normal((Hkv, L)).astype(np.float32)
    s[:, ::5] = np.round(s[:, ::5] * 4) / 4                   # some ties
    k = synth.random_bf16((L, Hkv, d), 30, stream=L)
    v = synth.random_bf16((L, Hkv, d), 31, stream=L)
    pr = B.Problem(Hkv, Hkv, d, L, 0, l, 1, 2, None)
    idx = Guarded((Hkv, l), torch.int32)
    kc = Guarded((l, Hkv, d), torch.bfloat16)
    vc = Guarded((l, Hkv, d), torch.bfloat16)
    ws = B.topk_workspace(pr)
    ws.fill_(0xFF)
    sd, kd, vd = to_device_f32(s), to_device_bf16(k), to_device_bf16(v)
    B.apb_topk_gather(pr, sd, kd, vd, idx=idx.t, k_comp=kc.t, v_comp=vc.t, workspace=ws)
    for g, name in ((idx, "idx"), (kc, "k_comp"), (vc, "v_comp")):
        g.check(name)
    idx_ref = orc.topl(s, l)
    assert np.array_equal(idx.t.cpu().numpy(), idx_ref)
    kr, vr = orc.gather(k, v, idx_ref)
    assert np.array_equal(from_device_bf16(kc.t), kr) and np.array_equal(from_device_bf16(vc.t), vr)
    first = [g.bits_copy() for g in (idx, kc, vc)]
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda"))
    B.apb_topk_gather(pr, sd, kd, vd, idx=idx.t, k_comp=kc.t, v_comp=vc.t, workspace=ws)
    for g, f, name in zip((idx, kc, vc), first, ("idx", "k_comp", "v_comp")):
        assert torch.equal(g.bits_copy(), f), f"{name} differs with other workspace contents"


def test_build_passing_guarded():
    p, l, Hkv, d = 5, 37, 3, 128
    blocks = [(synth.random_bf16((l, Hkv, d), 32, stream=j), synth.random_bf16((l, Hkv, d), 33, stream=j))
              for j in range(p)]
    pr = B.Problem(Hkv, Hkv, d, 64, 0, l, p, p + 1, None)
    kp = Guarded((p * l, Hkv, d), torch.bfloat16)
    vp = Guarded((p * l, Hkv, d), torch.bfloat16)
    B.apb_build_passing(pr, [to_device_bf16(b[0]) for b in blocks], [to_device_bf16(b[1]) for b in blocks],
                        k_pass=kp.t, v_pass=vp.t)
    kp.check("k_pass")
    vp.check("v_pass")
    kr, vr = orc.build_passing([b[0] for b in blocks], [b[1] for b in blocks])
    assert np.array_equal(from_device_bf16(kp.t), kr) and np.array_equal(from_device_bf16(vp.t), vr)


@pytest.mark.parametrize("segments", [B.APB_SEG_ANCHOR | B.APB_SEG_LOCAL, B.APB_SEG_PASSING, B.APB_SEG_ALL])
def test_segment_attention_guarded(segments):
    L, A, l, p, Hq, Hkv, d = 333, 70, 41, 2, 6, 3, 64
    P = p * l
    x = [synth.random_bf16(s, 40 + i, stream=segments) for i, s in enumerate(
        [(L, Hq, d), (A, Hkv, d), (A, Hkv, d), (P, Hkv, d), (P, Hkv, d), (L, Hkv, d), (L, Hkv, d)])]
    pr = B.Problem(Hq, Hkv, d, L, A, l, p, p + 1, None)
    out = Guarded((L, Hq, d), torch.bfloat16)
    lse = Guarded((Hq, L), torch.float32)
    dev = [to_device_bf16(t) for t in x]
    B.apb_block_attention_segments(pr, segments, *dev, out=out.t, lse=lse.t)
    out.check("out")
    lse.check("lse")
    names = [n for n, bit in (("anchor", B.APB_SEG_ANCHOR), ("passing", B.APB_SEG_PASSING),
                              ("local", B.APB_SEG_LOCAL)) if segments & bit]
    o_ref, lse_ref = orc.block_attention(*x, segments=names)
    check_attention(from_device_bf16(out.t), o_ref, lse.t.cpu().numpy(), lse_ref, f"segments {segments}")
    first = out.bits_copy(), lse.bits_copy()
    B.apb_block_attention_segments(pr, segments, *dev, out=out.t, lse=lse.t)
    assert torch.equal(out.bits_copy(), first[0]) and torch.equal(lse.bits_copy(), first[1])


def test_anchor_attention_guarded():
    A, Hq, Hkv, d = 201, 4, 2, 128
    q = synth.random_bf16((A, Hq, d), 50, sigma=0.5)
    k = synth.random_bf16((A, Hkv, d), 51, sigma=0.5)
    v = synth.random_bf16((A, Hkv, d), 52)
    pr = B.Problem(Hq, Hkv, d, 512, A, 8, 1, 2, None)
    out = Guarded((A, Hq, d), torch.bfloat16)
    lse = Guarded((Hq, A), torch.float32)
    B.apb_anchor_attention(pr, to_device_bf16(q), to_device_bf16(k), to_device_bf16(v), out=out.t, lse=lse.t)
    out.check("out")
    lse.check("lse")
    o_ref, lse_ref = orc.block_attention(q, None, None, None, None, k, v)
    check_attention(from_device_bf16(out.t), o_ref, lse.t.cpu().numpy(), lse_ref, "anchor attention")


@pytest.mark.parametrize("in_place", [False, True])
def test_merge_attention_guarded(in_place):
    """Merge of two partial results over disjoint key sets, into fresh buffers or over side a."""
    L, A, l, p, Hq, Hkv, d = 190, 50, 30, 2, 4, 2, 128
    P = p * l
    x = [synth.random_bf16(s, 60 + i) for i, s in enumerate(
        [(L, Hq, d), (A, Hkv, d), (A, Hkv, d), (P, Hkv, d), (P, Hkv, d), (L, Hkv, d), (L, Hkv, d)])]
    pr = B.Problem(Hq, Hkv, d, L, A, l, p, p + 1, None)
    dev = [to_device_bf16(t) for t in x]
    oa = Guarded((L, Hq, d), torch.bfloat16)
    la = Guarded((Hq, L), torch.float32)
    B.apb_block_attention_segments(pr, B.APB_SEG_ANCHOR | B.APB_SEG_LOCAL, *dev, out=oa.t, lse=la.t)
    ob, lb = B.apb_block_attention_segments(pr, B.APB_SEG_PASSING, *dev)
    if in_place:
        out, lse = oa, la
    else:
        out, lse = Guarded((L, Hq, d), torch.bfloat16), Guarded((Hq, L), torch.float32)
    B.apb_merge_attention(pr, oa.t, la.t, ob, lb, out=out.t, lse=lse.t)
    out.check("merged out")
    lse.check("merged lse")
    o_ref, lse_ref = orc.block_attention(*x)
    check_attention(from_device_bf16(out.t), o_ref, lse.t.cpu().numpy(), lse_ref, "merge")


@pytest.mark.parametrize("rows,heads,d,in_place", [(37, 5, 128, False), (37, 5, 128, True), (300, 3, 64, False)])
def test_rope_guarded(rows, heads, d, in_place):
    x = synth.random_bf16((rows, heads, d), 70, stream=rows)
    pos0, base = 9000, 500000.0
    o = Guarded((rows, heads, d), torch.bfloat16)
    if in_place:
        o.t.copy_(to_device_bf16(x))
        B.apb_rope(o.t, pos0, base, out=o.t)
    else:
        B.apb_rope(to_device_bf16(x), pos0, base, out=o.t)
    o.check("rope out")
    ref = orc.rope(x, pos0, base)
    got = from_device_bf16(o.t).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)


@pytest.mark.parametrize("rows,hidden", [(300, 96), (257, 64), (1, 32)])
def test_qkv_projection_guarded(rows, hidden):
    """Ragged token tiles and a K that ends in a half chunk (96 = 64 + 32)."""
    Hq, Hkv, d = 4, 2, 64
    x = synth.random_bf16((rows, hidden), 71, stream=rows)
    ws = [synth.random_bf16((n * d, hidden), 72 + i, sigma=hidden ** -0.5, stream=rows)
          for i, n in enumerate((Hq, Hkv, Hkv))]
    pr = B.Problem(Hq, Hkv, d, 64, 0, 0, 0, 1, None)
    outs = [Guarded((rows, n, d), torch.bfloat16) for n in (Hq, Hkv, Hkv)]
    B.apb_qkv_projection(pr, to_device_bf16(x), *[to_device_bf16(w) for w in ws], q=outs[0].t, k=outs[1].t,
                         v=outs[2].t)
    refs = orc.qkv_projection(x, *ws, Hq, Hkv)
    bounds = orc.qkv_projection(np.abs(x), *[np.abs(w) for w in ws], Hq, Hkv)
    for name, g, ref, bnd in zip("qkv", outs, refs, bounds):
        g.check(name)
        got = from_device_bf16(g.t).astype(np.float64)
        tol = 2.0 ** -8 * np.abs(ref) + 4 * np.sqrt(hidden) * 2.0 ** -24 * bnd
        assert np.all(np.abs(got - ref) <= tol), name
