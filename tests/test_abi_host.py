"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before launching anything.

No call here reaches a kernel launch: every call carries at least one argument
that the host-side checks reject, or a size for which the entry point has
nothing to do (l == 0, P == 0).
"""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_block_attention_amd import binding as B
from sparse_block_attention_amd import build as build_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "apb.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        build_mod.build()
    return B.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(apb_[a-z_0-9]+)\s*\(", text)))


def _problem(**kw):
    base = dict(n_q_heads=4, n_kv_heads=2, head_dim=128, local_len=256, anchor_len=32,
                pass_per_host=16, host_index=3, n_hosts=4, kv_head_of_q=None)
    base.update(kw)
    return B.Problem(**base)


def test_header_declares_the_four_steps():
    names = _declared_functions()
    for n in ("apb_score_kv", "apb_topk_gather", "apb_build_passing", "apb_block_attention"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (apb_\w+)", out))
    assert set(names) <= exported, set(names) - exported


def test_abi_version_and_status_strings(lib):
    assert B.apb_abi_version() == 5
    assert B.apb_status_string(B.APB_OK) == "APB_OK"
    assert B.apb_status_string(B.APB_ERR_UNSUPPORTED) == "APB_ERR_UNSUPPORTED"
    assert B.apb_status_string(99) == "APB_ERR_UNKNOWN"


def test_status_values_match_the_header(lib):
    """The enum values are part of the ABI: read them from include/apb.h and compare with the
    binding's constants and the library's names for them."""
    text = open(HEADER).read()
    body = text[text.index("typedef enum"):text.index("} apb_status;")]
    values = {m.group(1): int(m.group(2)) for m in re.finditer(r"(APB_\w+)\s*=\s*(\d+)", body)}
    assert values == {"APB_OK": 0, "APB_ERR_INVALID_ARGUMENT": 1, "APB_ERR_UNSUPPORTED": 2,
                      "APB_ERR_WORKSPACE_TOO_SMALL": 3, "APB_ERR_HIP": 4, "APB_ERR_INTERNAL": 5}
    for name, v in values.items():
        assert getattr(B, name) == v
        assert B.apb_status_string(v) == name


def test_head_map_of_the_wrong_length_is_refused_before_the_call():
    """The library reads n_q_heads entries of kv_head_of_q; a shorter list would be read past
    its end and a longer one silently cut, so the binding refuses both."""
    for bad in ([0, 1, 1], [0, 0, 1, 1, 0]):
        with pytest.raises(ValueError, match="kv_head_of_q"):
            _problem(kv_head_of_q=bad).to_c()
    _problem(kv_head_of_q=[0, 1, 1, 0]).to_c()


@pytest.mark.parametrize("kw,code,needle", [
    ({}, B.APB_OK, ""),
    ({"n_kv_heads": 0}, B.APB_ERR_INVALID_ARGUMENT, "n_kv_heads"),
    ({"n_q_heads": 5}, B.APB_ERR_INVALID_ARGUMENT, "multiple"),
    ({"n_q_heads": 512, "n_kv_heads": 2}, B.APB_ERR_UNSUPPORTED, "n_q_heads"),
    ({"head_dim": 96}, B.APB_ERR_UNSUPPORTED, "head_dim"),
    ({"local_len": 0}, B.APB_ERR_INVALID_ARGUMENT, "local_len"),
    ({"local_len": (1 << 26) + 1}, B.APB_ERR_UNSUPPORTED, "local_len"),
    ({"anchor_len": -1}, B.APB_ERR_INVALID_ARGUMENT, "anchor_len"),
    ({"n_hosts": 0, "host_index": 0}, B.APB_ERR_INVALID_ARGUMENT, "n_hosts"),
    ({"host_index": 4}, B.APB_ERR_INVALID_ARGUMENT, "host_index"),
    ({"host_index": -1}, B.APB_ERR_INVALID_ARGUMENT, "host_index"),
    ({"pass_per_host": 257}, B.APB_ERR_INVALID_ARGUMENT, "pass_per_host"),
    ({"pass_per_host": -1}, B.APB_ERR_INVALID_ARGUMENT, "pass_per_host"),
    ({"kv_head_of_q": [0, 0, 1, 2]}, B.APB_ERR_INVALID_ARGUMENT, "kv_head_of_q"),
    ({"kv_head_of_q": [0, 0, 0, 1]}, B.APB_ERR_INVALID_ARGUMENT, "exactly 2"),
    ({"kv_head_of_q": [1, 0, 0, 1]}, B.APB_OK, ""),
    ({"local_len": 1, "pass_per_host": 1, "anchor_len": 0}, B.APB_OK, ""),
    ({"n_hosts": 1 << 20, "host_index": (1 << 20) - 1, "pass_per_host": 256}, B.APB_ERR_UNSUPPORTED, "passing"),
])
def test_validate_problem(lib, kw, code, needle):
    st = B.apb_validate_problem(_problem(**kw))
    assert st == code, (st, B.apb_last_error())
    assert needle in B.apb_last_error()


def _call_attention(lib, pr, q=0x1000, ka=0x2000, va=0x3000, kp=0x4000, vp=0x5000, kl=0x6000,
                    vl=0x7000, scale=0.125, out=0x8000, lse=None):
    cp, keep = pr.to_c()
    return lib.apb_block_attention(ctypes.byref(cp), q, ka, va, kp, vp, kl, vl, ctypes.c_float(scale),
                                   out, lse, None)


@pytest.mark.parametrize("override,code,needle", [
    ({"q": None}, B.APB_ERR_INVALID_ARGUMENT, "q_local"),
    ({"q": 0x1001}, B.APB_ERR_INVALID_ARGUMENT, "aligned"),
    ({"ka": None}, B.APB_ERR_INVALID_ARGUMENT, "k_anchor"),
    ({"vp": None}, B.APB_ERR_INVALID_ARGUMENT, "v_pass"),
    ({"out": None}, B.APB_ERR_INVALID_ARGUMENT, "out"),
    ({"lse": 0x9004}, B.APB_ERR_INVALID_ARGUMENT, "lse"),
    ({"scale": 0.0}, B.APB_ERR_INVALID_ARGUMENT, "softmax_scale"),
    ({"scale": float("inf")}, B.APB_ERR_INVALID_ARGUMENT, "softmax_scale"),
    ({"scale": float("nan")}, B.APB_ERR_INVALID_ARGUMENT, "softmax_scale"),
])
def test_attention_rejects_bad_arguments(lib, override, code, needle):
    st = _call_attention(lib, _problem(), **override)
    assert st == code
    assert needle in B.apb_last_error()


def test_attention_rejects_bad_problem(lib):
    assert _call_attention(lib, _problem(head_dim=80)) == B.APB_ERR_UNSUPPORTED
    assert _call_attention(lib, _problem(n_q_heads=3)) == B.APB_ERR_INVALID_ARGUMENT
    assert lib.apb_block_attention(None, 0x1000, 0, 0, 0, 0, 0x2000, 0x3000, ctypes.c_float(1.0),
                                   0x4000, None, None) == B.APB_ERR_INVALID_ARGUMENT


def _call_segments(lib, pr, segments, q=0x1000, ka=0x2000, va=0x3000, kp=0x4000, vp=0x5000, kl=0x6000,
                   vl=0x7000, scale=0.125, out=0x8000, lse=None):
    cp, keep = pr.to_c()
    return lib.apb_block_attention_segments(ctypes.byref(cp), segments, q, ka, va, kp, vp, kl, vl,
                                            ctypes.c_float(scale), out, lse, None)


@pytest.mark.parametrize("segments,override,code,needle", [
    (0, {}, B.APB_ERR_INVALID_ARGUMENT, "segments"),
    (8, {}, B.APB_ERR_INVALID_ARGUMENT, "segments"),
    (B.APB_SEG_ALL | 16, {}, B.APB_ERR_INVALID_ARGUMENT, "segments"),
    (B.APB_SEG_LOCAL, {"kl": None}, B.APB_ERR_INVALID_ARGUMENT, "k_local"),
    (B.APB_SEG_ANCHOR, {"va": 0x3008}, B.APB_ERR_INVALID_ARGUMENT, "v_anchor"),
    (B.APB_SEG_PASSING, {"kp": None}, B.APB_ERR_INVALID_ARGUMENT, "k_pass"),
    # segments left out: their pointers are not looked at (the bad q still stops the call)
    (B.APB_SEG_PASSING, {"ka": None, "kl": None, "vl": 0x7001, "q": None}, B.APB_ERR_INVALID_ARGUMENT,
     "q_local"),
    (B.APB_SEG_ANCHOR | B.APB_SEG_LOCAL, {"kp": None, "vp": None, "out": None}, B.APB_ERR_INVALID_ARGUMENT,
     "out"),
    (B.APB_SEG_ALL, {"scale": -1.0}, B.APB_ERR_INVALID_ARGUMENT, "softmax_scale"),
])
def test_segment_attention_rejects_bad_arguments(lib, segments, override, code, needle):
    st = _call_segments(lib, _problem(), segments, **override)
    assert st == code
    assert needle in B.apb_last_error()


def test_merge_rejects_bad_arguments(lib):
    cp, keep = _problem().to_c()
    good = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000]
    names = ["out_a", "lse_a", "out_b", "lse_b", "out"]
    for i, name in enumerate(names):
        for bad in (None, good[i] + 4):
            args = list(good)
            args[i] = bad
            assert lib.apb_merge_attention(ctypes.byref(cp), *args, None) == B.APB_ERR_INVALID_ARGUMENT
            assert name in B.apb_last_error()
    args = list(good[:5]) + [0x6004]
    assert lib.apb_merge_attention(ctypes.byref(cp), *args, None) == B.APB_ERR_INVALID_ARGUMENT
    assert "lse" in B.apb_last_error()
    cp, keep = _problem(head_dim=96).to_c()
    assert lib.apb_merge_attention(ctypes.byref(cp), *good, None) == B.APB_ERR_UNSUPPORTED


def test_anchor_attention_and_rope_reject_bad_arguments(lib):
    cp, keep = _problem(anchor_len=0).to_c()
    assert lib.apb_anchor_attention(ctypes.byref(cp), 0x1000, 0x2000, 0x3000, ctypes.c_float(0.1), 0x4000,
                                    None, None) == B.APB_ERR_INVALID_ARGUMENT
    assert "anchor_len" in B.apb_last_error()
    cp, keep = _problem().to_c()
    assert lib.apb_anchor_attention(ctypes.byref(cp), 0x1000, None, 0x3000, ctypes.c_float(0.1), 0x4000,
                                    None, None) == B.APB_ERR_INVALID_ARGUMENT
    assert "k_local" in B.apb_last_error()    # the anchor runs as a local block
    good = dict(x=0x1000, out=0x2000, rows=4, heads=2, d=128, pos0=0, base=10000.0)
    for bad, code, needle in [({"x": None}, B.APB_ERR_INVALID_ARGUMENT, "x"),
                              ({"out": 0x2008}, B.APB_ERR_INVALID_ARGUMENT, "out"),
                              ({"rows": 0}, B.APB_ERR_INVALID_ARGUMENT, "rows"),
                              ({"heads": 5000}, B.APB_ERR_INVALID_ARGUMENT, "heads"),
                              ({"d": 96}, B.APB_ERR_UNSUPPORTED, "head_dim"),
                              ({"pos0": -1}, B.APB_ERR_INVALID_ARGUMENT, "pos0"),
                              ({"pos0": (1 << 31) - 3}, B.APB_ERR_INVALID_ARGUMENT, "pos0"),
                              ({"base": 1.0}, B.APB_ERR_INVALID_ARGUMENT, "theta_base"),
                              ({"base": float("inf")}, B.APB_ERR_INVALID_ARGUMENT, "theta_base")]:
        a = dict(good, **bad)
        st = lib.apb_rope(a["x"], a["out"], a["rows"], a["heads"], a["d"], a["pos0"], ctypes.c_float(a["base"]),
                          None)
        assert st == code and needle in B.apb_last_error(), (bad, st, B.apb_last_error())


def test_qkv_projection_rejects_bad_arguments(lib):
    cp, keep = _problem().to_c()
    good = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000]
    assert lib.apb_qkv_projection(ctypes.byref(cp), 0, 64, *good, None) == B.APB_ERR_INVALID_ARGUMENT
    assert "rows" in B.apb_last_error()
    assert lib.apb_qkv_projection(ctypes.byref(cp), 4, 48, *good, None) == B.APB_ERR_UNSUPPORTED
    assert "hidden" in B.apb_last_error()
    for i, name in enumerate(["x", "wq", "wk", "wv", "q", "k", "v"]):
        args = list(good)
        args[i] = None if i % 2 else good[i] + 8
        assert lib.apb_qkv_projection(ctypes.byref(cp), 4, 64, *args, None) == B.APB_ERR_INVALID_ARGUMENT
        assert name in B.apb_last_error()


def test_score_rejects_bad_scorer(lib):
    cp, keep = _problem().to_c()
    good = dict(hidden=64, w1=0x1000, b1=0x2000, w2=0x3000, b2=0x4000)
    for bad, code in [({"hidden": 40}, B.APB_ERR_UNSUPPORTED), ({"hidden": 272}, B.APB_ERR_UNSUPPORTED),
                      ({"hidden": 8}, B.APB_ERR_UNSUPPORTED), ({"hidden": 512}, B.APB_ERR_UNSUPPORTED),
                      ({"w1": None}, B.APB_ERR_INVALID_ARGUMENT), ({"b2": 0x4008}, B.APB_ERR_INVALID_ARGUMENT)]:
        s = dict(good, **bad)
        sc = B._Scorer(s["hidden"], s["w1"], s["b1"], s["w2"], s["b2"])
        assert lib.apb_score_kv(ctypes.byref(cp), ctypes.byref(sc), 0x5000, 0x6000, 0x7000, 0x8000,
                                None) == code
    sc = B._Scorer(64, 0x1000, 0x2000, 0x3000, 0x4000)
    assert lib.apb_score_kv(ctypes.byref(cp), None, 0x5000, 0x6000, 0x7000, 0x8000,
                            None) == B.APB_ERR_INVALID_ARGUMENT
    assert lib.apb_score_kv(ctypes.byref(cp), ctypes.byref(sc), 0x5000, None, 0x7000, 0x8000,
                            None) == B.APB_ERR_INVALID_ARGUMENT


def _ws_size(lib, pr):
    cp, keep = pr.to_c()
    return lib.apb_topk_workspace_size(ctypes.byref(cp))


def test_topk_workspace_size(lib):
    """8 bytes of selection state per kv head plus 8 bytes per 256-token chunk per kv head,
    rounded up to 256 bytes; 0 for l == 0 and for an invalid problem."""
    for L, Hkv in [(256, 2), (257, 2), (16384, 8), (131072, 8), (1, 1), (1 << 26, 8)]:
        pr = _problem(local_len=L, n_kv_heads=Hkv, n_q_heads=2 * Hkv, pass_per_host=1, anchor_len=0)
        chunks = -(-L // 256)
        want = Hkv * 8 + Hkv * chunks * 8
        want = -(-want // 256) * 256
        assert _ws_size(lib, pr) == want, (L, Hkv)
        assert B.apb_topk_workspace_size(pr) == want
    assert _ws_size(lib, _problem(pass_per_host=0)) == 0
    assert _ws_size(lib, _problem(head_dim=96)) == 0
    assert "head_dim" in B.apb_last_error()


def test_topk_rejects_a_small_or_missing_workspace(lib):
    pr = _problem()
    need = _ws_size(lib, pr)
    cp, keep = pr.to_c()
    ptrs = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000]
    st = lib.apb_topk_gather(ctypes.byref(cp), *ptrs, 0x7000, need - 1, None)
    assert st == B.APB_ERR_WORKSPACE_TOO_SMALL
    assert str(need) in B.apb_last_error()
    st = lib.apb_topk_gather(ctypes.byref(cp), *ptrs, None, 0, None)
    assert st == B.APB_ERR_WORKSPACE_TOO_SMALL
    st = lib.apb_topk_gather(ctypes.byref(cp), *ptrs, None, need, None)
    assert st == B.APB_ERR_INVALID_ARGUMENT and "workspace" in B.apb_last_error()
    st = lib.apb_topk_gather(ctypes.byref(cp), *ptrs, 0x7008, need, None)
    assert st == B.APB_ERR_INVALID_ARGUMENT and "workspace" in B.apb_last_error()


def test_noalloc_topk_rejects_problems_beyond_its_static_workspace(lib):
    """The allocation-free top-l refuses, before any launch, a problem whose workspace exceeds
    the static array, and does nothing for l == 0."""
    ptrs = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000]
    big = _problem(local_len=1 << 26, n_kv_heads=8, n_q_heads=16, pass_per_host=1, anchor_len=0)
    assert _ws_size(lib, big) > B.NOALLOC_TOPK_WORKSPACE_BYTES
    cp, keep = big.to_c()
    assert lib.apb_topk_gather_noalloc(ctypes.byref(cp), *ptrs, None) == B.APB_ERR_UNSUPPORTED
    assert "static workspace" in B.apb_last_error()
    cp, keep = _problem(pass_per_host=0).to_c()
    assert lib.apb_topk_gather_noalloc(ctypes.byref(cp), None, None, None, None, None, None, None) == B.APB_OK
    cp, keep = _problem().to_c()
    assert lib.apb_topk_gather_noalloc(ctypes.byref(cp), None, *ptrs[1:], None) == B.APB_ERR_INVALID_ARGUMENT
    text = open(HEADER).read()
    assert "#define APB_NOALLOC_TOPK_WORKSPACE_BYTES ((size_t)4 << 20)" in text
    assert B.NOALLOC_TOPK_WORKSPACE_BYTES == 4 << 20


def test_topk_and_build_have_nothing_to_do_for_empty_sizes(lib):
    # l == 0: nothing selected, nothing launched, NULL outputs and workspace allowed.
    cp, keep = _problem(pass_per_host=0).to_c()
    assert lib.apb_topk_gather(ctypes.byref(cp), None, None, None, None, None, None, None, 0, None) == B.APB_OK
    assert lib.apb_build_passing(ctypes.byref(cp), None, None, None, None, None) == B.APB_OK
    # host 0: no preceding hosts, empty passing block.
    cp, keep = _problem(host_index=0).to_c()
    assert lib.apb_build_passing(ctypes.byref(cp), None, None, None, None, None) == B.APB_OK


def test_topk_and_build_reject_bad_pointers(lib):
    cp, keep = _problem().to_c()
    assert lib.apb_topk_gather(ctypes.byref(cp), 0x1000, 0x2000, 0x3000, None, 0x5000, 0x6000,
                               0x7000, 1 << 20, None) == B.APB_ERR_INVALID_ARGUMENT
    arr = (ctypes.c_void_p * 3)(0x1000, 0x2000, 0x3008)
    arr_ok = (ctypes.c_void_p * 3)(0x1000, 0x2000, 0x3000)
    assert lib.apb_build_passing(ctypes.byref(cp), arr_ok, arr, 0x4000, 0x5000, None) \
        == B.APB_ERR_INVALID_ARGUMENT
    assert "v_comp_hosts[2]" in B.apb_last_error()
    assert lib.apb_build_passing(ctypes.byref(cp), arr_ok, None, 0x4000, 0x5000, None) \
        == B.APB_ERR_INVALID_ARGUMENT
    assert lib.apb_build_passing(ctypes.byref(cp), arr_ok, arr_ok, None, 0x5000, None) \
        == B.APB_ERR_INVALID_ARGUMENT


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()
