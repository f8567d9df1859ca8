"""Host-side checks of bench.py's accounting (no GPU).

* attention_flops: 4 d Hq times the visible (row, key) pairs.  The pair count is
  taken from the oracle itself: with q = 0 every visible key gets the same
  weight, so exp(lse) of a row is its number of visible keys.
* attention_bytes: q, the anchor/passing/local K and V, O and LSE, each once, as
  the arrays a launch reads and writes; stage_bytes likewise for the scorer,
  top-l + gather and the passing build.
* the traffic record is only used for its own workload, and bench refuses more
  than one GPU before touching a device.
"""
import importlib.util
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import apb_oracle as orc
from sparse_block_attention_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _small(L, A, l, host, Hq, Hkv, d):
    return synth.Workload("acct", 900, host + 1, L, A, l, Hq, Hkv, d, 32, 1.0, 0)


@pytest.mark.parametrize("L,A,l,host,Hq,Hkv,d", [
    (37, 5, 3, 2, 2, 1, 64), (64, 0, 4, 1, 4, 2, 128), (20, 9, 0, 3, 3, 3, 64), (1, 1, 1, 1, 2, 2, 128),
])
def test_attention_flops_count_the_oracles_visible_pairs(bench, L, A, l, host, Hq, Hkv, d):
    w = _small(L, A, l, host, Hq, Hkv, d)
    P = w.pass_len
    rng = np.random.default_rng(L + A)
    q = np.zeros((L, Hq, d))
    kv = lambda n: (rng.standard_normal((n, Hkv, d)), rng.standard_normal((n, Hkv, d)))
    (ka, va), (kp, vp), (kl, vl) = kv(A), kv(P), kv(L)
    _, lse = orc.block_attention(q, ka, va, kp, vp, kl, vl)
    pairs_per_head = np.exp(lse).sum(axis=1)            # visible keys summed over rows, per q head
    assert np.allclose(pairs_per_head, pairs_per_head[0])
    assert bench.attention_flops(w) == pytest.approx(4.0 * d * Hq * pairs_per_head[0], rel=1e-12)


def test_attention_bytes_are_the_arrays_of_one_launch(bench):
    w = synth.WORKLOADS["llama8b"]
    L, A, P, Hq, Hkv, d = w.local_len, w.anchor_len, w.pass_len, w.n_q_heads, w.n_kv_heads, w.head_dim
    bf16, f32 = 2, 4
    reads = L * Hq * d * bf16 + 2 * (A + P + L) * Hkv * d * bf16   # q, K and V of three segments
    writes = L * Hq * d * bf16 + Hq * L * f32                       # O and LSE
    assert bench.attention_bytes(w) == reads + writes
    assert bench.attention_flops(w) == pytest.approx(4.673058635776e12, rel=1e-12)


def test_traffic_record_is_used_only_for_its_workload(bench):
    assert bench.measured_traffic("qwen14b") is None
    assert bench.measured_traffic("tiny") is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU only" in r.stderr


def test_stage_bytes_are_the_arrays_each_step_moves(bench):
    """Scorer: q, k, v of the block and the fp32 scores (the scorer weights, L2-resident,
    are reported apart); top-l + gather: scores, K and V rows read and written, indices;
    passing: the earlier hosts' compressed blocks read and written.  Sizes from the
    generator's arrays."""
    w = synth.Workload("acct_stage", 901, 3, 40, 8, 6, 4, 2, 64, 32, 1.0, 0)
    q, k, v = synth.host_block(w, w.host)
    wts = synth.scorer_weights(w)
    scores = np.zeros((w.n_kv_heads, w.local_len), np.float32)
    idx = np.zeros((w.n_kv_heads, w.pass_per_host), np.int32)
    bf16 = lambda a: a.size * 2
    kv_row = w.n_kv_heads * w.head_dim * 2
    b = bench.stage_bytes(w)
    assert b["a1_score"] == bf16(q) + bf16(k) + bf16(v) + scores.nbytes
    assert bench.scorer_weight_bytes(w) == (bf16(wts["w1"]) + wts["b1"].size * 4 + wts["w2"].size * 4
                                            + wts["b2"].size * 4)
    assert b["a2a3_topl_gather"] == scores.nbytes + 2 * 2 * w.pass_per_host * kv_row + idx.nbytes
    assert b["a5_passing"] == 2 * 2 * w.host * w.pass_per_host * kv_row
