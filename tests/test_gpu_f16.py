"""f16 q/out (the page's `Cfg` q_dtype) on the GPU against the oracle, with
f16 K/V or fp8 K/V widened to f16 (exact). The f16 path runs the same kernels
with f16 MFMAs, f16 P and f16 output rounding; prefill P is kept below f16's
largest finite value by a one-step smaller rescale slack, which the
sharpened cases (Q x 8) exercise. Cases: small ragged batches in both kernel
classes and head sizes, soft-cap, windows, non-causal; split-KV merges in both
classes; the long-context and fp8 decode workloads' shapes at full size on
sampled rows; the append of f16 rows into f16 and fp8 caches.
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

F16 = wl.Q_F16

SMALL_F16 = [
    # (seed, head_dim, kv_dtype, causal, window, soft_cap, G, page)
    (501, 64, wl.KV_F16, True, None, None, None, 16),
    (502, 128, wl.KV_F16, True, None, None, None, 16),
    (503, 256, wl.KV_F16, True, None, None, 2, 64),
    (504, 128, wl.KV_F16, True, 17, 50.0, 4, 16),
    (505, 128, wl.KV_F16, False, None, None, None, 32),
    (506, 64, wl.KV_F16, True, 3, None, 8, 16),
    (507, 128, wl.KV_FP8, True, None, 30.0, 4, 16),
    (508, 256, wl.KV_E5M2, False, 9, 2.0, 3, 32),
    (509, 64, wl.KV_FP8, True, None, None, 16, 48),
]


def _small(seed, D, kvd, causal, window, cap, G, page):
    return wl.random_small(seed, max_seqs=5, head_dim=D, kv_dtype=kvd, q_dtype=F16, causal=causal,
                           window=window, soft_cap=cap, G=G, page_size=page, max_q=40, max_extra_kv=120)


@pytest.mark.parametrize("seed,D,kvd,causal,window,cap,G,page", SMALL_F16)
def test_f16_small_random(seed, D, kvd, causal, window, cap, G, page):
    _compare_all(_small(seed, D, kvd, causal, window, cap, G, page), f"f16 small seed {seed}")


@pytest.mark.parametrize("seed,D,kvd,causal,window,cap,G,page", SMALL_F16[:6])
def test_f16_small_random_sharpened(seed, D, kvd, causal, window, cap, G, page):
    w = _small(seed, D, kvd, causal, window, cap, G, page)
    w.q = wl.to_f16_bits(w.q.view(np.float16).astype(np.float32) * 8.0)
    _compare_all(w, f"f16 small seed {seed} x8")


@pytest.mark.parametrize("case", MEDIUM[:4], ids=[c["name"] for c in MEDIUM[:4]])
@pytest.mark.parametrize("q_mult", [1.0, 8.0])
def test_f16_split_kv(case, q_mult):
    kw = dict(num_q_heads=case["Hq"], num_kv_heads=case["Hkv"], head_dim=case["D"], page_size=case["page"],
              pages_per_seq=None, sm_scale=1.0 / np.sqrt(case["D"]), kv_dtype=wl.KV_F16, q_dtype=F16,
              sliding_window=case.get("window"))
    pages = sum((k + case["page"] - 1) // case["page"] for k in case["kv_lens"])
    w = wl.build(case["name"] + "-f16", kw, case["q_lens"], case["kv_lens"], 100, total_num_pages=pages + 3,
                 max_num_seqs=len(case["q_lens"]) + 1, num_q_tokens=sum(case["q_lens"]) + 2, q_mult=q_mult)
    _compare_all(w, case["name"] + f" f16 x{q_mult:g}")


@pytest.mark.parametrize("number", [5, 4])
def test_f16_named_workload_shapes_full_size(number):
    """The long-context workload with f16 q and K/V, the fp8 decode workload
    with f16 q over its e4m3fn cache; full size, sampled rows."""
    print(f"[f16] cfg{number}: generating", flush=True)
    w = wl.named(number, q_dtype=F16)
    d = Device(w)
    check_sampled(w, d, f"cfg{number} f16")
    del d
    torch.cuda.empty_cache()


def test_f16_append_every_finite_f16_value_into_f16_cache():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    pats = b[(b & 0x7C00) != 0x7C00][:63488]          # 63488 finite f16 patterns = 248 x 2 x 128
    kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=128, page_size=16, sm_scale=0.1,
              kv_dtype=wl.KV_F16, q_dtype=F16, k_scale=0.37, v_scale=3.0)
    w = wl.build("rounding-f16", kw, [248], [260], 21, total_num_pages=20)
    rng = np.random.Generator(np.random.PCG64(23))
    _check(w, pats.reshape(248, 2, 128), rng.permutation(pats).reshape(248, 2, 128), "f16 rows -> f16 cache")


@pytest.mark.parametrize("kvd", [wl.KV_F16, wl.KV_FP8, wl.KV_E5M2])
def test_f16_rows_append_then_attend(kvd):
    w = wl.random_small(520, max_seqs=5, head_dim=128, kv_dtype=kvd, q_dtype=F16, max_q=48, max_extra_kv=150)
    k_new, v_new = wl.new_kv(w, 520, std=1.5)
    dev = Device(w)
    _append(dev, k_new, v_new)
    out, lse = dev.run()
    w.kv_pages, _ = oracle.kv_append(w, k_new, v_new)
    ref_out, ref_lse = oracle.forward(w)
    T = w.valid_tokens()
    assert_parity(out.float().cpu().numpy()[:T], lse.cpu().numpy()[:T], ref_out[:T], ref_lse[:T],
                  f"f16 rows append+attend {kvd}")
