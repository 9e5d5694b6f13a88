"""int8 K/V caches on the GPU against the oracle (the page's `Cfg` lists i8
among the KV dtypes; a code reads as code x scale). The int8 path shares the
one-byte path of the fp8 kinds but the widening (sign-extended bytes, exact in
bf16 and f16) and, for the append, the rounding (nearest integer, ties to
even, saturating at -128/127, NaN to 0). Cases: small ragged batches with bf16
and f16 q in both kernel classes; split-KV merges; the fp8 decode workload's
shape with an int8 cache at full size on sampled rows; the append over every
finite bf16 value; append then attend.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import Device, assert_parity, check_sampled
from test_gpu_append import _append, _check
from test_gpu_parity import MEDIUM, _compare_all


pytestmark = pytest.mark.gpu

I8 = wl.KV_I8

SMALL_I8 = [
    # (seed, head_dim, q_dtype, causal, window, soft_cap, G, page)
    (601, 64, wl.Q_BF16, True, None, None, None, 16),
    (602, 128, wl.Q_BF16, True, 17, 50.0, 4, 16),
    (603, 256, wl.Q_BF16, False, None, None, 2, 64),
    (604, 128, wl.Q_F16, True, None, None, None, 32),
    (605, 64, wl.Q_F16, True, 3, 30.0, 8, 16),
    (606, 256, wl.Q_F16, True, None, None, 16, 48),
]


@pytest.mark.parametrize("seed,D,qd,causal,window,cap,G,page", SMALL_I8)
def test_int8_small_random(seed, D, qd, causal, window, cap, G, page):
    w = wl.random_small(seed, max_seqs=5, head_dim=D, kv_dtype=I8, q_dtype=qd, causal=causal, window=window,
                        soft_cap=cap, G=G, page_size=page, max_q=40, max_extra_kv=120)
    _compare_all(w, f"int8 small seed {seed}")


@pytest.mark.parametrize("case", MEDIUM[:3], ids=[c["name"] for c in MEDIUM[:3]])
def test_int8_split_kv(case):
    kw = dict(num_q_heads=case["Hq"], num_kv_heads=case["Hkv"], head_dim=case["D"], page_size=case["page"],
              pages_per_seq=None, sm_scale=1.0 / np.sqrt(case["D"]), kv_dtype=I8, k_scale=0.05, v_scale=0.05)
    pages = sum((k + case["page"] - 1) // case["page"] for k in case["kv_lens"])
    w = wl.build(case["name"] + "-int8", kw, case["q_lens"], case["kv_lens"], 100, total_num_pages=pages + 3,
                 max_num_seqs=len(case["q_lens"]) + 1, num_q_tokens=sum(case["q_lens"]) + 2)
    _compare_all(w, case["name"] + " int8")


def test_int8_fp8_decode_workload_shape_full_size():
    print("[int8] fp8 decode shape: generating", flush=True)
    w = wl.named(4, kv_dtype=I8)
    d = Device(w)
    check_sampled(w, d, "cfg4 int8")
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("ks,vs", [(0.05, 0.05), (1.0, 3.0), (1 / 3, 2.0 ** -10)])
def test_int8_append_every_finite_bf16_value(ks, vs):
    pats = wl.finite_bf16_patterns()
    kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=128, page_size=16, sm_scale=0.1,
              kv_dtype=I8, k_scale=ks, v_scale=vs)
    w = wl.build("rounding-int8", kw, [255], [272], 21, total_num_pages=20)
    rng = np.random.Generator(np.random.PCG64(22))
    _check(w, pats.reshape(255, 2, 128), rng.permutation(pats).reshape(255, 2, 128), f"int8 all bf16 k/{ks} v/{vs}")


def test_int8_append_nan_and_ties():
    kw = dict(num_q_heads=2, num_kv_heads=1, head_dim=64, page_size=16, sm_scale=0.1,
              kv_dtype=I8, k_scale=1.0, v_scale=1.0)
    w = wl.build("ties-int8", kw, [2], [2], 23, total_num_pages=1)
    k_new, v_new = wl.new_kv(w, 24)
    vals = np.float32([0.5, 1.5, 2.5, -0.5, -1.5, 127.5, -128.5, 300.0, np.nan, -np.inf, np.inf, 126.5])
    k_new[0, 0, :len(vals)] = wl.to_bf16_bits(vals)
    _check(w, k_new, v_new, "int8 ties / NaN / saturation")


@pytest.mark.parametrize("qd", [wl.Q_BF16, wl.Q_F16])
def test_int8_append_then_attend(qd):
    w = wl.random_small(650, max_seqs=5, head_dim=128, kv_dtype=I8, q_dtype=qd, max_q=48, max_extra_kv=150)
    k_new, v_new = wl.new_kv(w, 650, std=1.5)
    dev = Device(w)
    _append(dev, k_new, v_new)
    out, lse = dev.run()
    w.kv_pages, _ = oracle.kv_append(w, k_new, v_new)
    ref_out, ref_lse = oracle.forward(w)
    T = w.valid_tokens()
    assert_parity(out.float().cpu().numpy()[:T], lse.cpu().numpy()[:T], ref_out[:T], ref_lse[:T],
                  f"int8 append+attend q {qd}")
