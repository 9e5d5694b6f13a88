"""The algorithmic work bench.py divides by kernel time (the roofline's
`achieved`), checked against hand counts on tiny workloads: flops = 4·D per
(q head, visible key); bytes = each sequence's K/V span once per kv head, plus
q, out (in the q type) and the LSE per query row; a sequence is decode-class
when its packed rows fit one 16-row tile."""

import workloads as wl
import bench


def _w(q_lens, kv_lens, **kw):
    base = dict(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, pages_per_seq=None, sm_scale=0.1)
    base.update(kw)
    return wl.build("acct", base, q_lens, kv_lens, 5)


def test_decode_class_counts_bf16():
    # seq 0: 1 token at position 4 sees 5 keys; seq 1: 3 tokens at 4, 5, 6 see 5 + 6 + 7
    r = bench.algorithmic_work(_w([1, 3], [5, 7]))
    assert r["decode"][0] == 4 * 4 * 64 * (5 + 18)
    # K/V: Hkv * 2 * D * 2 B over spans 5 and 7; per query token Hq * (2 * 2 * D + 4)
    assert r["decode"][1] == 2 * 2 * 64 * 2 * (5 + 7) + 4 * 4 * (4 * 64 + 4)
    assert r["decode"][2] == 4 and r["prefill"] == [0.0, 0.0, 0]


def test_f32_q_and_one_byte_cache_bytes():
    r = bench.algorithmic_work(_w([1, 3], [5, 7], q_dtype=wl.Q_F32))
    assert r["decode"][1] == 2 * 2 * 64 * 2 * (5 + 7) + 4 * 4 * (2 * 4 * 64 + 4)
    r = bench.algorithmic_work(_w([1, 3], [5, 7], kv_dtype=wl.KV_FP8, k_scale=0.05, v_scale=0.05))
    assert r["decode"][1] == 2 * 2 * 64 * 1 * (5 + 7) + 4 * 4 * (4 * 64 + 4)


def test_window_and_prefill_class():
    # window 3: the token at position 4 sees keys 2..4
    r = bench.algorithmic_work(_w([1], [5], sliding_window=3))
    assert r["decode"][0] == 4 * 4 * 64 * 3
    assert r["decode"][1] == 2 * 2 * 64 * 2 * 3 + 4 * (4 * 64 + 4)
    # 9 tokens x G = 2 is 18 packed rows: prefill class; positions 3..11 see 4..12 keys
    r = bench.algorithmic_work(_w([9], [12]))
    assert r["prefill"][0] == 4 * 4 * 64 * sum(range(4, 13))
    assert r["prefill"][1] == 2 * 2 * 64 * 2 * 12 + 9 * 4 * (4 * 64 + 4)
    assert r["prefill"][2] == 9 and r["decode"] == [0.0, 0.0, 0]
