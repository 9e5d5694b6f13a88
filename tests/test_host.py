"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every entry point `include/rpa.h` declares, validates configurations and
checks metadata without touching a device."""

import ctypes
import os
import re

import numpy as np
import pytest

import ragged_paged_gqa_amd as rpa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "rpa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rpa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = rpa.lib()
    names = _declared()
    assert "rpa_forward" in names and "rpa_workspace_bytes" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(rpa.EXPORTS)


def test_status_strings():
    for code, text in rpa.STATUS.items():
        assert rpa.status_string(code) == text
    assert rpa.status_string(99) == "unknown status"


def _cfg(**kw):
    base = dict(num_q_tokens=8, num_q_heads=8, num_kv_heads=2, head_dim=128, total_num_pages=16,
                page_size=16, max_num_seqs=4, pages_per_seq=4, sm_scale=0.1)
    base.update(kw)
    return rpa.Config(**base)


def _ws_status(cfg):
    c = cfg.to_c()
    n = ctypes.c_size_t(0)
    return rpa.lib().rpa_workspace_bytes(ctypes.byref(c), ctypes.byref(n))


@pytest.mark.parametrize("kw,code", [
    (dict(num_q_heads=6, num_kv_heads=4), 1),        # G not an integer
    (dict(num_kv_heads=0), 1),
    (dict(num_q_tokens=-1), 1),
    (dict(total_num_pages=0), 1),
    (dict(sliding_window=-3), 1),
    (dict(soft_cap=-1.0), 1),
    (dict(sm_scale=float("nan")), 1),
    (dict(k_scale=float("inf")), 1),
    (dict(is_causal=2), 1),
    (dict(head_dim=96), 2),                          # not built
    (dict(page_size=24), 2),
    (dict(page_size=2048, pages_per_seq=2), 2),
    (dict(kv_dtype=7), 2),
    (dict(q_dtype=rpa.DTYPE_F32, kv_dtype=rpa.DTYPE_F16), 2),   # f32 q runs on the bf16 path
    (dict(q_dtype=rpa.DTYPE_F32, kv_dtype=rpa.DTYPE_F32), 2),   # no f32 cache
    (dict(q_dtype=rpa.DTYPE_INT8, kv_dtype=rpa.DTYPE_INT8), 2),  # int8 is a K/V type only
    (dict(q_dtype=rpa.DTYPE_F16, kv_dtype=rpa.DTYPE_BF16), 2),  # 16-bit K/V in the q type
])
def test_invalid_configs_rejected_before_any_device_call(kw, code):
    cfg = _cfg(**kw)
    if "is_causal" in kw:
        c = cfg.to_c()
        c.is_causal = kw["is_causal"]
        n = ctypes.c_size_t(0)
        assert rpa.lib().rpa_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == code
        return
    assert _ws_status(cfg) == code


def test_forward_rejects_null_pointers_without_device():
    c = _cfg().to_c()
    st = rpa.lib().rpa_forward(ctypes.byref(c), None, None, None, None, None, None, None, None, None, 0, None)
    assert st == 1


def test_null_config_rejected():
    n = ctypes.c_size_t(0)
    assert rpa.lib().rpa_workspace_bytes(None, ctypes.byref(n)) == 1


def _meta():
    cfg = _cfg(num_q_tokens=10, max_num_seqs=3, pages_per_seq=4, total_num_pages=12)
    kv_lens = np.array([5, 33, 64], np.int32)
    pi = np.array([[0, 0, 0, 0], [1, 2, 3, 0], [4, 5, 6, 7]], np.int32)
    cu = np.array([0, 1, 4, 10], np.int32)
    return cfg, kv_lens, pi, cu


def test_check_metadata_accepts_valid():
    cfg, kvl, pi, cu = _meta()
    assert rpa.check_metadata(cfg, kvl, pi, cu, 3) == 0
    assert rpa.check_metadata(cfg, kvl, pi, cu, 2) == 0


@pytest.mark.parametrize("mutate", [
    lambda kvl, pi, cu: kvl.__setitem__(0, 0),            # q_len 1 > kv_len 0
    lambda kvl, pi, cu: kvl.__setitem__(2, 65),           # beyond pages_per_seq * page_size
    lambda kvl, pi, cu: pi.__setitem__((1, 2), 12),       # page id out of range
    lambda kvl, pi, cu: pi.__setitem__((2, 0), -1),
    lambda kvl, pi, cu: cu.__setitem__(2, 0),             # decreasing cu_q_lens
    lambda kvl, pi, cu: cu.__setitem__(3, 11),            # beyond num_q_tokens
])
def test_check_metadata_rejects_broken_preconditions(mutate):
    cfg, kvl, pi, cu = _meta()
    mutate(kvl, pi, cu)
    assert rpa.check_metadata(cfg, kvl, pi, cu, 3) == 5


def test_check_metadata_ignores_unused_table_entries():
    cfg, kvl, pi, cu = _meta()
    pi[0, 1:] = 10 ** 6     # sequence 0 has one page; the rest is never read
    assert rpa.check_metadata(cfg, kvl, pi, cu, 3) == 0
    assert rpa.check_metadata(cfg, kvl, pi, cu, 4) == 5   # num_seqs > max_num_seqs


@pytest.mark.parametrize("which,offset", [("q", 2), ("kv", 8), ("out", 4), ("lse", 2), ("sinks", 1)])
def test_forward_rejects_misaligned_pointers_without_device(which, offset):
    # q, K/V and out travel in 16-byte pieces, lse and sinks as f32: a pointer
    # off those boundaries is an invalid argument, found before any device call
    # (the buffers here are host memory that the library never dereferences)
    c = _cfg().to_c()
    buf = np.zeros(1 << 16, np.uint8)
    base = (buf.ctypes.data + 255) & ~255
    ptr = {k: base + 4096 * i for i, k in enumerate(("q", "kv", "kvl", "pi", "cu", "ns", "sinks", "out", "lse", "ws"))}
    ptr[which] += offset
    L = rpa.lib()
    st = L.rpa_forward_sinks(ctypes.byref(c), ptr["q"], ptr["kv"], ptr["kvl"], ptr["pi"], ptr["cu"], ptr["ns"],
                             ptr["sinks"], ptr["out"], ptr["lse"], ptr["ws"], 1 << 20, None)
    assert st == 1
