"""The steps either side of the attention step in one layer on a host: the
anchor's own causal attention, rotary position embedding and the QKV
projection, HIP path vs oracle."""
import numpy as np
import pytest
import torch

from oracle import apb_oracle as orc
from sparse_block_attention_amd import binding as B
from sparse_block_attention_amd import synth
from sparse_block_attention_amd.tensors import from_device_bf16, to_device_bf16

from apb_gpu_util import check_attention, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("A,Hq,Hkv,d,hm", [(1, 2, 1, 128, None), (300, 6, 3, 128, [2, 0, 1, 1, 0, 2]),
                                            (2048, 32, 8, 128, None), (129, 4, 2, 64, None),
                                            (4095, 64, 8, 128, None)])  # 1024 items of 256 rows
def test_anchor_attention(A, Hq, Hkv, d, hm):
    q = synth.random_bf16((A, Hq, d), 1, sigma=0.5, stream=A)
    k = synth.random_bf16((A, Hkv, d), 2, sigma=0.5, stream=A)
    v = synth.random_bf16((A, Hkv, d), 3, stream=A)
    pr = B.Problem(Hq, Hkv, d, 4096, A, 16, 3, 4, hm)
    out, lse = B.apb_anchor_attention(pr, to_device_bf16(q), to_device_bf16(k), to_device_bf16(v))
    torch.cuda.synchronize()
    rows = np.arange(A) if A <= 300 else np.unique(np.r_[0, 1, 63, 64, 127, 128, A // 2, A - 1,
                                                          np.random.default_rng(A).integers(0, A, 40)])
    o_ref, lse_ref = orc.block_attention(q, None, None, None, None, k, v, kv_head_of_q=hm, rows=rows)
    check_attention(from_device_bf16(out)[rows], o_ref, lse.cpu().numpy()[:, rows], lse_ref, "anchor attention")


@pytest.mark.parametrize("rows,heads,d,pos0,base", [
    (5, 3, 128, 0, 10000.0), (300, 8, 64, 123456, 500000.0), (17, 2, 128, (1 << 26) - 17, 500000.0),
    (2048, 40, 128, 7 * 16384, 1000000.0), (17, 2, 128, (1 << 31) - 17, 500000.0),
    (7, 100, 64, 5, 10000.0), (9, 1, 128, 3, 10000.0)])
def test_rope_matches_oracle(rows, heads, d, pos0, base):
    """Bar: the kernel rounds an fp32 rotation once to bf16 (half an ulp, 2^-9 relative) after
    fp32 sin/cos of an angle reduced in double: |o - o_ref| <= 2^-8 |o_ref| + 1e-5."""
    x = synth.random_bf16((rows, heads, d), 4, stream=rows)
    xd = to_device_bf16(x)
    o = B.apb_rope(xd, pos0, base)
    torch.cuda.synchronize()
    ref = orc.rope(x, pos0, base)
    got = from_device_bf16(o).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)
    # in place gives the same bits
    B.apb_rope(xd, pos0, base, out=xd)
    torch.cuda.synchronize()
    assert torch.equal(xd, o)


@pytest.mark.parametrize("rows,hidden,Hq,Hkv,d", [(1, 32, 2, 1, 64), (300, 96, 4, 2, 64),
                                                  (513, 160, 3, 1, 64), (700, 512, 6, 3, 128),
                                                  (16384, 4096, 32, 8, 128)])
def test_qkv_projection_matches_oracle(rows, hidden, Hq, Hkv, d):
    """Ragged token and output tiles, K from one chunk to 4096.  Bar: one bf16 rounding of an
    fp32 sum (half an ulp, 2^-9 relative) plus fp32 summation error, bounded by
    4 sqrt(K) 2^-24 sum|x_i w_i|:  |o - o_ref| <= 2^-8 |o_ref| + 4 sqrt(K) 2^-24 sum|x_i w_i|."""
    x = synth.random_bf16((rows, hidden), 5, stream=rows)
    ws = [synth.random_bf16((n * d, hidden), 6 + i, sigma=hidden ** -0.5, stream=rows)
          for i, n in enumerate((Hq, Hkv, Hkv))]
    pr = B.Problem(Hq, Hkv, d, 64, 0, 0, 0, 1, None)
    q, k, v = B.apb_qkv_projection(pr, to_device_bf16(x), *[to_device_bf16(w) for w in ws])
    torch.cuda.synchronize()
    sample = np.arange(rows) if rows <= 1024 else np.unique(np.r_[0, 255, 256, rows - 1,
                                                                  np.random.default_rng(0).integers(0, rows, 60)])
    refs = orc.qkv_projection(x[sample], *ws, Hq, Hkv)
    bounds = orc.qkv_projection(np.abs(x[sample]), *[np.abs(w) for w in ws], Hq, Hkv)
    for name, got, ref, bnd in zip("qkv", (q, k, v), refs, bounds):
        g = from_device_bf16(got)[sample].astype(np.float64)
        tol = 2.0 ** -8 * np.abs(ref) + 4 * np.sqrt(hidden) * 2.0 ** -24 * bnd
        assert np.all(np.abs(g - ref) <= tol), (name, float(np.max(np.abs(g - ref) - tol)))
