"""Full-size parity for the other layer shapes: Qwen-2.5-14B, Yi-34B-200K and
Llama-3-8B-1M, the last of 8 hosts, in the launch configuration bench.py uses.

Every stage runs at full size through the C ABI and is checked against the
oracle fed the GPU's previous-stage output:
  * scores on sampled tokens (bar in apb_gpu_util);
  * top-l indices of every kv head over the whole block, bit-exact;
  * the compressed block (gather), bit-exact;
  * the passing block built from seeded compressed blocks of the 7 earlier
    hosts, bit-exact (those blocks are inputs of the passing assembly; drawing them
    directly saves compressing 7 more full-size host blocks);
  * attention on sampled rows of every q head.
"""
import numpy as np
import pytest
import torch

from oracle import apb_oracle as orc
from sparse_block_attention_amd import binding as B
from sparse_block_attention_amd import synth
from sparse_block_attention_amd.tensors import from_device_bf16, to_device_bf16, to_device_f32

from apb_gpu_util import check_attention, check_scores, require_gpu, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("name", ["qwen14b", "yi34b", "llama1m"])
def test_config_full_size_sampled(name):
    w = synth.WORKLOADS[name]
    print(f"\n[{name}] L={w.local_len} A={w.anchor_len} l={w.pass_per_host} Hq/Hkv={w.n_q_heads}/{w.n_kv_heads}",
          flush=True)
    pr = B.Problem(w.n_q_heads, w.n_kv_heads, w.head_dim, w.local_len, w.anchor_len, w.pass_per_host,
                   w.host, w.n_hosts, None)
    q, k, v = synth.host_block(w, w.host)
    wts = synth.scorer_weights(w)
    sc = {"w1": to_device_bf16(wts["w1"]), "b1": to_device_f32(wts["b1"]),
          "w2": to_device_f32(wts["w2"]), "b2": to_device_f32(wts["b2"])}
    qd, kd, vd = to_device_bf16(q), to_device_bf16(k), to_device_bf16(v)

    # score
    scores = B.apb_score_kv(pr, sc, qd, kd, vd)
    torch.cuda.synchronize()
    s_np = scores.cpu().numpy()
    tr = sample_rows(w.local_len, 200, seed=7)
    s_ref = orc.score_kv(q[tr], k[tr], v[tr], wts["w1"], wts["b1"], wts["w2"], wts["b2"])
    check_scores(s_np[:, tr], s_ref, f"{name} scores")

    # top-l + gather
    idx, kc, vc = B.apb_topk_gather(pr, scores, kd, vd)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    assert np.array_equal(idx_np, orc.topl(s_np, w.pass_per_host)), f"{name} top-l"
    kr, vr = orc.gather(k, v, idx_np)
    assert np.array_equal(from_device_bf16(kc), kr) and np.array_equal(from_device_bf16(vc), vr), f"{name} gather"
    del kc, vc, kr, vr

    # passing block from the earlier hosts' compressed blocks
    shape = (w.pass_per_host, w.n_kv_heads, w.head_dim)
    comps = [(synth.random_bf16(shape, 30, sigma=0.5, stream=j), synth.random_bf16(shape, 31, sigma=0.5, stream=j))
             for j in range(w.host)]
    kp, vp = B.apb_build_passing(pr, [to_device_bf16(c[0]) for c in comps], [to_device_bf16(c[1]) for c in comps])
    torch.cuda.synchronize()
    kp_ref, vp_ref = orc.build_passing([c[0] for c in comps], [c[1] for c in comps])
    kp_np, vp_np = from_device_bf16(kp), from_device_bf16(vp)
    assert np.array_equal(kp_np, kp_ref) and np.array_equal(vp_np, vp_ref), f"{name} passing"

    # attention
    ka, va = synth.anchor_kv(w)
    out, lse = B.apb_block_attention(pr, qd, to_device_bf16(ka), to_device_bf16(va), kp, vp, kd, vd)
    torch.cuda.synchronize()
    rows = sample_rows(w.local_len, 24, seed=8)
    o_ref, lse_ref = orc.block_attention(q, ka, va, kp_np, vp_np, k, v, rows=rows)
    rows_t = torch.from_numpy(rows).to(out.device)
    check_attention(from_device_bf16(out.index_select(0, rows_t)), o_ref, lse.cpu().numpy()[:, rows], lse_ref,
                    f"{name} attention")
