"""fp8 e5m2 K/V caches on the GPU against the oracle (the page's `Cfg` lists
f8e5m2 among the KV dtypes). The e5m2 path shares every step with e4m3fn but
the code decode (v_cvt_scalef32_pk_bf16_bf8, exact into bf16) and, for the
append, the rounding (saturating at +-57344). Cases: small ragged batches in
both kernel classes and head sizes, soft-cap, windows, non-causal; split-KV
merges in both classes; the fp8 decode workload's shape at full size on
sampled rows; the append over every finite bf16 value; append then attend.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import Device, assert_parity, check_sampled
from test_gpu_append import _append, _check, _kv_host
from test_gpu_parity import MEDIUM, _compare_all


pytestmark = pytest.mark.gpu

E5 = wl.KV_E5M2

SMALL_E5 = [
    # (seed, head_dim, causal, window, soft_cap, G, page)
    (401, 64, True, None, None, None, 16),
    (402, 128, True, None, None, None, 16),
    (403, 256, True, None, None, 2, 64),
    (404, 128, True, 17, 50.0, 4, 16),
    (405, 128, False, None, None, None, 32),
    (406, 64, True, 3, None, 8, 16),
    (407, 256, False, 9, 2.0, 3, 32),
    (408, 128, True, None, None, 16, 48),
]


@pytest.mark.parametrize("seed,D,causal,window,cap,G,page", SMALL_E5)
def test_e5m2_small_random(seed, D, causal, window, cap, G, page):
    w = wl.random_small(seed, max_seqs=5, head_dim=D, kv_dtype=E5, causal=causal, window=window,
                        soft_cap=cap, G=G, page_size=page, max_q=40, max_extra_kv=120)
    _compare_all(w, f"e5m2 small seed {seed}")


@pytest.mark.parametrize("case", MEDIUM[:3], ids=[c["name"] for c in MEDIUM[:3]])
def test_e5m2_split_kv(case):
    kw = dict(num_q_heads=case["Hq"], num_kv_heads=case["Hkv"], head_dim=case["D"], page_size=case["page"],
              pages_per_seq=None, sm_scale=1.0 / np.sqrt(case["D"]), kv_dtype=E5, k_scale=0.05, v_scale=0.05)
    pages = sum((k + case["page"] - 1) // case["page"] for k in case["kv_lens"])
    w = wl.build(case["name"] + "-e5m2", kw, case["q_lens"], case["kv_lens"], 100, total_num_pages=pages + 3,
                 max_num_seqs=len(case["q_lens"]) + 1, num_q_tokens=sum(case["q_lens"]) + 2)
    _compare_all(w, case["name"] + " e5m2")


def test_e5m2_fp8_decode_workload_shape_full_size():
    """The fp8 decode workload's lengths, heads, soft-cap and window with an
    e5m2 cache, at full size, on sampled rows."""
    rng = np.random.Generator(np.random.PCG64(4))
    q, kv = wl.lengths(4, rng)
    kw = dict(wl.cfg_kw(4), kv_dtype=E5)
    print("[e5m2] fp8 decode shape: generating", flush=True)
    w = wl.build("cfg4-e5m2", kw, q, kv, 4, rng=rng)
    d = Device(w)
    check_sampled(w, d, "cfg4 e5m2")
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("ks,vs", [(0.05, 0.05), (1.0, 3.0), (1 / 3, 2.0 ** -10)])
def test_e5m2_append_every_finite_bf16_value(ks, vs):
    pats = wl.finite_bf16_patterns()
    kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=128, page_size=16, sm_scale=0.1,
              kv_dtype=E5, k_scale=ks, v_scale=vs)
    w = wl.build("rounding-e5m2", kw, [255], [272], 21, total_num_pages=20)
    rng = np.random.Generator(np.random.PCG64(22))
    _check(w, pats.reshape(255, 2, 128), rng.permutation(pats).reshape(255, 2, 128), f"e5m2 all bf16 k/{ks} v/{vs}")


def test_e5m2_append_nan_stays_nan():
    kw = dict(num_q_heads=2, num_kv_heads=1, head_dim=64, page_size=16, sm_scale=0.1,
              kv_dtype=E5, k_scale=0.5, v_scale=0.5)
    w = wl.build("nan-e5m2", kw, [2], [2], 23, total_num_pages=1)
    k_new, v_new = wl.new_kv(w, 24)
    k_new[0, 0, :4] = [0x7FC0, 0xFFC0, 0x7F81, 0xFF81]
    dev = Device(w)
    _append(dev, k_new, v_new)
    got = _kv_host(dev)
    g = got[0, 0, 0, :4]
    assert (((g >> 2) & 31) == 31).all() and ((g & 3) != 0).all()
    ref, _ = oracle.kv_append(w, k_new, v_new)
    got[0, 0, 0, :4] = ref[0, 0, 0, :4]
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("seed,D", [(450, 128), (451, 64), (452, 256)])
def test_e5m2_append_then_attend(seed, D):
    w = wl.random_small(seed, max_seqs=5, head_dim=D, kv_dtype=E5, max_q=48, max_extra_kv=150)
    k_new, v_new = wl.new_kv(w, seed, std=1.5)
    dev = Device(w)
    _append(dev, k_new, v_new)
    out, lse = dev.run()
    w.kv_pages, _ = oracle.kv_append(w, k_new, v_new)
    ref_out, ref_lse = oracle.forward(w)
    T = w.valid_tokens()
    assert_parity(out.float().cpu().numpy()[:T], lse.cpu().numpy()[:T], ref_out[:T], ref_lse[:T],
                  f"e5m2 append+attend seed {seed}")
