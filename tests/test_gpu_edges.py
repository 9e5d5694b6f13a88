"""Edge cases of the attention path on the GPU against the oracle: no
sequence at all, the largest page size (1024 keys), pure prompts (q_len =
kv_len, ragged tails), single-key sequences, more sequences than one planner
tile (512), a window wider than every sequence, and negative and zero score
scales.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import Device, assert_parity
from test_gpu_parity import _compare_all

pytestmark = pytest.mark.gpu


def test_no_sequences_leaves_every_row_untouched():
    kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, pages_per_seq=None, sm_scale=0.08)
    w = wl.build("none", kw, [3, 5], [40, 60], 61, total_num_pages=10, num_q_tokens=8)
    w.num_seqs[0] = 0
    d = Device(w)
    out = torch.full((8, 8, 128), 5.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((8, 8), -7.0, dtype=torch.float32, device="cuda")
    out, lse = d.run(out=out, lse=lse)
    assert torch.all(out == 5.0) and torch.all(lse == -7.0)


@pytest.mark.parametrize("D,kvd", [(128, wl.KV_BF16), (256, wl.KV_BF16), (128, wl.KV_FP8), (64, wl.KV_I8)])
def test_largest_page_size(D, kvd):
    """page_size 1024, both kernel classes, split chunks inside one page: the
    window starts the 20000-key sequence's key range at key 9952, so its two
    chunks meet at key 18144, inside page 17."""
    kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=D, page_size=1024, pages_per_seq=None,
              sm_scale=1.0 / np.sqrt(D), kv_dtype=kvd, sliding_window=10000)
    if wl.is_fp8(kvd):
        kw.update(k_scale=0.05, v_scale=0.05)
    q_lens, kv_lens = [1, 40, 2, 300], [3000, 20000, 1024, 4000]
    pages = sum((k + 1023) // 1024 for k in kv_lens)
    w = wl.build("page1024", kw, q_lens, kv_lens, 62, total_num_pages=pages + 1, num_q_tokens=sum(q_lens) + 1)
    _compare_all(w, f"page 1024 D {D} {kvd}")


@pytest.mark.parametrize("q_mult", [1.0, 8.0])
def test_pure_prompts(q_mult):
    """q_len = kv_len: a sequence's queries start at key 0 (ragged tails, lengths
    off the 16-key grid)."""
    kw = dict(num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=32, pages_per_seq=None, sm_scale=0.09)
    lens = [1, 17, 130, 333, 1]
    w = wl.build("prompts", kw, lens, lens, 63, q_mult=q_mult)
    _compare_all(w, f"pure prompts x{q_mult:g}")


def test_single_key_sequences():
    kw = dict(num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16, pages_per_seq=None, sm_scale=0.3)
    w = wl.build("onekey", kw, [1, 1, 1], [1, 1, 1], 64)
    out, lse = Device(w).run()
    ref_out, ref_lse = oracle.forward(w)
    assert_parity(out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, "single key")


def test_more_sequences_than_one_planner_tile():
    """1300 sequences (three tiles of 512): mostly decodes, some short prefills."""
    rng = np.random.Generator(np.random.PCG64(65))
    S = 1300
    q_lens = np.where(rng.random(S) < 0.9, 1, rng.integers(2, 40, size=S))
    kv_lens = q_lens + rng.integers(0, 200, size=S)
    kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16, pages_per_seq=None, sm_scale=0.125)
    w = wl.build("many", kw, q_lens, kv_lens, 65, rng=rng, max_num_seqs=S + 3, num_q_tokens=int(q_lens.sum()) + 2)
    out, lse = Device(w).run()
    T = w.valid_tokens()
    toks = np.sort(rng.choice(T, size=min(T, 600), replace=False))
    heads = np.tile(np.arange(8), len(toks))
    ref_out, ref_lse, _ = oracle.rows(w, np.repeat(toks, 8), heads)
    o = out.float().cpu().numpy()[np.repeat(toks, 8), heads]
    l = lse.cpu().numpy()[np.repeat(toks, 8), heads]
    assert_parity(o, l, ref_out, ref_lse, "1300 sequences")


def test_window_wider_than_every_sequence():
    kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, pages_per_seq=None, sm_scale=0.09,
              sliding_window=100000)
    w = wl.build("widewin", kw, [1, 50, 3], [700, 900, 64], 66)
    _compare_all(w, "window wider than kv_len")


@pytest.mark.parametrize("q_dtype,kvd,scale,cap", [
    (wl.Q_BF16, wl.KV_BF16, -0.09, None),
    (wl.Q_BF16, wl.KV_FP8, -0.09, 30.0),
    (wl.Q_F16, wl.KV_F16, -0.09, None),
    (wl.Q_F32, wl.KV_BF16, -0.09, None),
    (wl.Q_F32, wl.KV_I8, -0.09, 20.0),
    (wl.Q_BF16, wl.KV_BF16, 0.0, None),
    (wl.Q_F32, wl.KV_E5M2, 0.0, None),
])
def test_negative_and_zero_score_scale(q_dtype, kvd, scale, cap):
    """sm_scale < 0 (the kernels flip q's sign and use |scale|) and sm_scale = 0
    (every visible key weighs the same: out is the mean of the visible V),
    in both kernel classes."""
    kw = dict(num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=32, pages_per_seq=None, sm_scale=scale,
              soft_cap=cap, kv_dtype=kvd, q_dtype=q_dtype)
    if wl.is_fp8(kvd):
        kw.update(k_scale=0.05, v_scale=0.05)
    w = wl.build("scale", kw, [1, 1, 40, 130], [300, 17, 200, 130], 65)
    _compare_all(w, f"sm_scale {scale} q {q_dtype} kv {kvd} cap {cap}")
