"""The allocation-free top-l entry point against the one with a caller workspace.

apb_topk_gather_noalloc keeps its workspace in a static per-GPU array.  Two calls
in a row, the second on a smaller problem, must give the same bits as
apb_topk_gather (and the oracle's selection): the array keeps the first call's
contents, which the second must not depend on.
"""
import numpy as np
import pytest
import torch

from oracle import apb_oracle as orc
from sparse_block_attention_amd import binding as B
from sparse_block_attention_amd import synth
from sparse_block_attention_amd.tensors import to_device_bf16, to_device_f32

from apb_gpu_util import require_gpu

pytestmark = pytest.mark.gpu


def _case(L, l, Hkv, d, seed):
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((Hkv, L)).astype(np.float32)
    s[:, ::7] = np.round(s[:, ::7] * 8) / 8                    # ties
    k = synth.random_bf16((L, Hkv, d), 80, stream=seed)
    v = synth.random_bf16((L, Hkv, d), 81, stream=seed)
    pr = B.Problem(Hkv, Hkv, d, L, 0, l, 1, 2, None)
    return pr, s, to_device_f32(s), to_device_bf16(k), to_device_bf16(v)


def test_noalloc_topk_matches_workspace_entry_on_two_calls():
    require_gpu()
    for L, l, Hkv, d, seed in [(16384, 1024, 8, 128, 1), (3001, 77, 3, 64, 2)]:
        pr, s, sd, kd, vd = _case(L, l, Hkv, d, seed)
        assert B.apb_topk_workspace_size(pr) <= B.NOALLOC_TOPK_WORKSPACE_BYTES
        outs = [torch.full((Hkv, l), -1, dtype=torch.int32, device="cuda"),
                torch.zeros((l, Hkv, d), dtype=torch.bfloat16, device="cuda"),
                torch.zeros((l, Hkv, d), dtype=torch.bfloat16, device="cuda")]
        B.apb_topk_gather_noalloc(pr, sd, kd, vd, *outs)
        ref = B.apb_topk_gather(pr, sd, kd, vd)
        torch.cuda.synchronize()
        for a, b, name in zip(outs, ref, ("idx", "k_comp", "v_comp")):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (L, name)
        assert np.array_equal(outs[0].cpu().numpy(), orc.topl(s, l)), L
