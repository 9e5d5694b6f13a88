"""f32 q/out (the page's `Cfg` q_dtype of packing 1) on the GPU against the
oracle. The kernels carry each q element as a bf16 pair hi + lo and take both
in the scores, over bf16 or one-byte K/V; out is written in f32. Cases: small
ragged batches in both kernel classes and all head sizes, soft-cap, windows,
non-causal, every K/V kind; split-KV merges in both classes; the mixed and fp8
decode workloads at full size on sampled rows; an LSE bound ten times tighter
than the parity bar, which a q rounded to bf16 misses by far (so the low half
of each f32 is used); the append of f32 rows into bf16, fp8 and int8 caches,
bit-exact.
"""

import copy

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import Device, assert_parity, check_sampled, run_numpy
from test_gpu_append import _append, _check
from test_gpu_parity import MEDIUM, _compare_all


pytestmark = pytest.mark.gpu

F32 = wl.Q_F32

SMALL_F32 = [
    # (seed, head_dim, kv_dtype, causal, window, soft_cap, G, page)
    (611, 64, wl.KV_BF16, True, None, None, None, 16),
    (612, 128, wl.KV_BF16, True, None, None, None, 16),
    (613, 256, wl.KV_BF16, True, None, None, 2, 64),
    (614, 128, wl.KV_BF16, True, 17, 50.0, 4, 16),
    (615, 128, wl.KV_BF16, False, None, None, None, 32),
    (616, 128, wl.KV_FP8, True, None, 30.0, 4, 16),
    (617, 256, wl.KV_E5M2, False, 9, 2.0, 3, 32),
    (618, 64, wl.KV_I8, True, 3, None, 8, 16),
    (619, 256, wl.KV_FP8, True, None, None, 1, 48),
]


def _small(seed, D, kvd, causal, window, cap, G, page):
    return wl.random_small(seed, max_seqs=5, head_dim=D, kv_dtype=kvd, q_dtype=F32, causal=causal,
                           window=window, soft_cap=cap, G=G, page_size=page, max_q=40, max_extra_kv=120)


@pytest.mark.parametrize("seed,D,kvd,causal,window,cap,G,page", SMALL_F32)
def test_f32_small_random(seed, D, kvd, causal, window, cap, G, page):
    _compare_all(_small(seed, D, kvd, causal, window, cap, G, page), f"f32 small seed {seed}")


@pytest.mark.parametrize("seed,D,kvd", [(621, 128, wl.KV_BF16), (622, 64, wl.KV_FP8), (623, 256, wl.KV_BF16),
                                        (624, 128, wl.KV_I8)])
def test_f32_lse_takes_the_low_bits(seed, D, kvd):
    """q x 4: the kernel's LSE is within 1e-4 of the oracle, while the oracle
    with the same q rounded to bf16 is off by more than 1e-3 somewhere."""
    w = wl.random_small(seed, max_seqs=5, head_dim=D, kv_dtype=kvd, q_dtype=F32, max_q=40, max_extra_kv=200)
    w.q = wl.to_q_bits(w.q.view(np.float32) * np.float32(4.0), F32)
    T = w.valid_tokens()
    ref_out, ref_lse = oracle.forward(w)
    wb = copy.copy(w)
    wb.q = wl.to_bf16_bits(w.q.view(np.float32)).astype(np.uint32) << 16
    _, lse_b = oracle.forward(wb)
    fin = np.isfinite(ref_lse[:T])
    assert np.max(np.abs(lse_b[:T][fin] - ref_lse[:T][fin])) > 1e-3
    out, lse = run_numpy(w)
    assert_parity(out[:T], lse[:T], ref_out[:T], ref_lse[:T], f"f32 x4 seed {seed}")
    d = np.abs(lse[:T][fin] - ref_lse[:T][fin])
    assert np.max(d) <= 1e-4, f"max lse error {np.max(d):.3e}"
    assert np.array_equal(np.isfinite(lse[:T]), fin)


@pytest.mark.parametrize("case", MEDIUM[:4], ids=[c["name"] for c in MEDIUM[:4]])
@pytest.mark.parametrize("kvd", [wl.KV_BF16, wl.KV_FP8])
def test_f32_split_kv(case, kvd):
    kw = dict(num_q_heads=case["Hq"], num_kv_heads=case["Hkv"], head_dim=case["D"], page_size=case["page"],
              pages_per_seq=None, sm_scale=1.0 / np.sqrt(case["D"]), kv_dtype=kvd, q_dtype=F32,
              sliding_window=case.get("window"))
    if wl.is_fp8(kvd):
        kw.update(k_scale=0.05, v_scale=0.05)
    pages = sum((k + case["page"] - 1) // case["page"] for k in case["kv_lens"])
    w = wl.build(case["name"] + "-f32", kw, case["q_lens"], case["kv_lens"], 100, total_num_pages=pages + 3,
                 max_num_seqs=len(case["q_lens"]) + 1, num_q_tokens=sum(case["q_lens"]) + 2)
    _compare_all(w, case["name"] + f" f32 q {kvd}")


@pytest.mark.parametrize("number", [3, 4])
def test_f32_named_workload_shapes_full_size(number):
    """The mixed workload (bf16 cache) and the fp8 decode workload (e4m3fn
    cache) with an f32 q; full size, sampled rows."""
    print(f"[f32] cfg{number}: generating", flush=True)
    w = wl.named(number, q_dtype=F32)
    d = Device(w)
    check_sampled(w, d, f"cfg{number} f32")
    del d
    torch.cuda.empty_cache()


def _finite_f32_bits(n, seed):
    """Seeded f32 bit patterns over every exponent (zeros and subnormals
    included), infinities and NaN excluded."""
    rng = np.random.Generator(np.random.PCG64(seed))
    b = rng.integers(0, 1 << 32, size=2 * n, dtype=np.uint64).astype(np.uint32)
    b = b[(b & 0x7F800000) != 0x7F800000][:n]
    assert b.size == n
    b[:4] = [0x00000000, 0x80000000, 0x00000001, 0x807FFFFF]
    return b


@pytest.mark.parametrize("kvd,ks,vs", [(wl.KV_BF16, 1.0, 1.0), (wl.KV_BF16, 0.3, 7.0), (wl.KV_FP8, 0.05, 0.05),
                                       (wl.KV_E5M2, 1.0, 3.0), (wl.KV_I8, 0.05, 2.0 ** -10)])
def test_f32_rows_append_bit_exact(kvd, ks, vs):
    """New rows in f32: random finite patterns of every magnitude, and a
    N(0, 9) batch, stored as the oracle's rounding of x / scale."""
    kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=128, page_size=16, sm_scale=0.1,
              kv_dtype=kvd, q_dtype=F32, k_scale=ks, v_scale=vs)
    w = wl.build("rounding-f32", kw, [248], [260], 31, total_num_pages=20)
    pats = _finite_f32_bits(2 * 248 * 2 * 128, 32 + int(1000 * ks))
    _check(w, pats[: 248 * 256].reshape(248, 2, 128), pats[248 * 256:].reshape(248, 2, 128),
           f"f32 rows -> {kvd} patterns")
    k_new, v_new = wl.new_kv(w, 33, std=3.0)
    _check(w, k_new, v_new, f"f32 rows -> {kvd} N(0,9)")


@pytest.mark.parametrize("kvd", [wl.KV_BF16, wl.KV_FP8, wl.KV_I8])
def test_f32_rows_append_then_attend(kvd):
    w = wl.random_small(630, max_seqs=5, head_dim=128, kv_dtype=kvd, q_dtype=F32, max_q=48, max_extra_kv=150)
    k_new, v_new = wl.new_kv(w, 630, std=1.5)
    dev = Device(w)
    _append(dev, k_new, v_new)
    out, lse = dev.run()
    assert out.dtype == torch.float32
    w.kv_pages, _ = oracle.kv_append(w, k_new, v_new)
    ref_out, ref_lse = oracle.forward(w)
    T = w.valid_tokens()
    assert_parity(out.cpu().numpy()[:T], lse.cpu().numpy()[:T], ref_out[:T], ref_lse[:T],
                  f"f32 rows append+attend {kvd}")
