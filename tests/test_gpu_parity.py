"""GPU parity of the HIP path against the f64 CPU oracle (needs an MI355X).

Small ragged workloads are compared row for row over every valid (token, q
head); they span several 32-key steps, ragged tails, split and unsplit units,
both attention kernels (<= 16 packed rows per sequence and kv head go to the
decode kernel, more to the prefill kernel) and the split merge.
"""

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_gqa_amd as rpa
import workloads as wl
from gpu_util import Device, assert_parity, run_numpy

pytestmark = pytest.mark.gpu


def _compare_all(w, what):
    print(f"[parity] {what}", flush=True)
    out, lse = run_numpy(w)
    ref_out, ref_lse = oracle.forward(w)
    T = w.valid_tokens()
    return assert_parity(out[:T], lse[:T], ref_out[:T], ref_lse[:T], what)


def test_fp8_conversion_matches_oracle_table():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    got = rpa.decode_fp8(codes).cpu().numpy().astype(np.float64)
    ref = oracle.e4m3fn_to_f64(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_tiny_named_workload():
    _compare_all(wl.named(1), "tiny")


def test_tiny_named_workload_sharpened():
    _compare_all(wl.named(1, q_mult=8.0), "tiny x8")


SMALL = [
    # (seed, head_dim, kv_dtype, causal, window, soft_cap, G, page)
    (1, 64, wl.KV_BF16, True, None, None, None, 16),
    (2, 128, wl.KV_BF16, True, None, None, None, 16),
    (3, 256, wl.KV_BF16, True, None, None, None, 64),
    (4, 128, wl.KV_FP8, True, None, None, None, 16),
    (5, 128, wl.KV_BF16, False, None, None, None, 32),
    (6, 64, wl.KV_BF16, True, 7, None, None, 16),
    (7, 128, wl.KV_BF16, True, None, 5.0, None, 16),
    (8, 128, wl.KV_FP8, True, 17, 50.0, 4, 16),
    (9, 64, wl.KV_BF16, True, 1, None, 1, 16),
    (10, 256, wl.KV_FP8, False, 9, 2.0, 3, 32),
    (11, 64, wl.KV_BF16, True, None, None, 8, 16),
    (12, 128, wl.KV_BF16, True, None, None, 16, 48),
    (13, 64, wl.KV_FP8, True, 3, None, 2, 16),
    (14, 256, wl.KV_BF16, True, 40, 30.0, 2, 16),
]


@pytest.mark.parametrize("seed,D,kvd,causal,window,cap,G,page", SMALL)
def test_small_random(seed, D, kvd, causal, window, cap, G, page):
    w = wl.random_small(seed, max_seqs=5, head_dim=D, kv_dtype=kvd, causal=causal, window=window,
                        soft_cap=cap, G=G, page_size=page, max_q=40, max_extra_kv=120)
    _compare_all(w, f"small seed {seed}")


@pytest.mark.parametrize("seed,D,kvd,causal,window,cap,G,page", SMALL[:8])
def test_small_random_sharpened(seed, D, kvd, causal, window, cap, G, page):
    w = wl.random_small(seed, max_seqs=5, head_dim=D, kv_dtype=kvd, causal=causal, window=window,
                        soft_cap=cap, G=G, page_size=page, max_q=40, max_extra_kv=120)
    w.q = wl.to_bf16_bits(wl.bf16_bits_to_f32(w.q) * 8.0)
    _compare_all(w, f"small seed {seed} x8")


MEDIUM = [
    # decode-class rows with long KV (split chunks), prefill-class rows with long KV
    dict(name="dec-split", q_lens=[1, 1, 2, 1], kv_lens=[3000, 257, 1900, 40], Hq=8, Hkv=2, D=128, page=16),
    # (prefill chunks are at least 8192 keys: these units take 2 and 3)
    dict(name="pf-split", q_lens=[40, 3, 70], kv_lens=[20000, 1500, 9000], Hq=8, Hkv=2, D=128, page=32),
    dict(name="pf-split-d256", q_lens=[24, 9], kv_lens=[18000, 9000], Hq=16, Hkv=2, D=256, page=64),
    dict(name="mixed-window", q_lens=[33, 1, 1, 5], kv_lens=[2100, 2000, 700, 1300], Hq=8, Hkv=4, D=64,
         page=16, window=300),
    dict(name="fp8-cap-window", q_lens=[1, 1, 1], kv_lens=[4000, 2500, 1000], Hq=32, Hkv=8, D=128, page=16,
         fp8=True, cap=50.0, window=1024),
    dict(name="noncausal-long", q_lens=[50, 2], kv_lens=[1200, 2222], Hq=4, Hkv=1, D=128, page=16,
         causal=False),
    # one-byte K/V: decode units of two kv heads, with an odd head count (the
    # last unit has one head) and with a single head
    dict(name="fp8-odd-heads", q_lens=[1, 2, 1, 1], kv_lens=[3100, 900, 2047, 33], Hq=12, Hkv=3, D=128, page=16,
         fp8=True),
    dict(name="fp8-one-head", q_lens=[1, 1, 3], kv_lens=[2900, 40, 1500], Hq=4, Hkv=1, D=128, page=16, fp8=True),
]


def _medium(case, seed=100, q_mult=1.0):
    kw = dict(num_q_heads=case["Hq"], num_kv_heads=case["Hkv"], head_dim=case["D"],
              page_size=case["page"], pages_per_seq=None, sm_scale=1.0 / np.sqrt(case["D"]),
              is_causal=case.get("causal", True), sliding_window=case.get("window"),
              soft_cap=case.get("cap"))
    if case.get("fp8"):
        kw.update(kv_dtype=wl.KV_FP8, k_scale=0.05, v_scale=0.05)
    pages = sum((k + case["page"] - 1) // case["page"] for k in case["kv_lens"])
    return wl.build(case["name"], kw, case["q_lens"], case["kv_lens"], seed, total_num_pages=pages + 3,
                    max_num_seqs=len(case["q_lens"]) + 1, num_q_tokens=sum(case["q_lens"]) + 2, q_mult=q_mult)


@pytest.mark.parametrize("case", MEDIUM, ids=[c["name"] for c in MEDIUM])
def test_medium_with_split_kv(case):
    _compare_all(_medium(case), case["name"])


@pytest.mark.parametrize("case", MEDIUM, ids=[c["name"] for c in MEDIUM])
def test_medium_with_split_kv_sharpened(case):
    _compare_all(_medium(case, q_mult=8.0), case["name"] + " x8")


@pytest.mark.parametrize("case", MEDIUM[:3], ids=[c["name"] for c in MEDIUM[:3]])
def test_medium_cases_split(case):
    """The split cases do split: prefill units of more than one chunk (merged
    by the last finisher) or decode units over more than one wave (merged by
    the combine kernel), whatever the planner's chunk and wave rules."""
    w = _medium(case)
    d = Device(w)
    ws = rpa.plan(d.kv_lens, d.cu_q_lens, d.num_seqs, d.cfg)
    torch.cuda.synchronize()
    offs, lim = rpa.plan_layout(d.cfg)
    host = ws.cpu().numpy()
    hdr = host[offs[0]:offs[0] + 256].view(np.int32)
    n_split_pf, Tb, W = int(hdr[6]), int(hdr[7]), int(hdr[8])
    if case["name"].startswith("pf"):
        assert n_split_pf > 0
    else:
        # some unit's blocks fall into the ranges of two to four waves (the
        # combine kernel's one-pass merge) and some into more (its batched one)
        ds = host[offs[1]:offs[1] + 32 * int(hdr[2])].view(np.int32).reshape(-1, 8)
        wave = lambda b: np.searchsorted((Tb * np.arange(W + 1, dtype=np.int64)) // W, b, side="right") - 1
        parts = [wave(int(r[6]) + (h + 1) * int(r[7]) - 1) - wave(int(r[6]) + h * int(r[7])) + 1
                 for r in ds if int(r[7]) > 0 for h in range(case["Hkv"])]
        assert any(2 <= n <= 4 for n in parts), parts
        assert any(n > 4 for n in parts), parts


def test_padding_rows_untouched_and_empty_sequences():
    # q_len 0 sequences, num_seqs < max_num_seqs, padding tokens after the last one
    kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, pages_per_seq=None, sm_scale=0.08)
    w = wl.build("pad", kw, [3, 0, 17, 0, 1], [50, 20, 300, 5, 999], 31, total_num_pages=120,
                 max_num_seqs=7, num_q_tokens=30)
    d = Device(w)
    sentinel_out = torch.full((30, 8, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    sentinel_lse = torch.full((30, 8), 123.0, dtype=torch.float32, device="cuda")
    out, lse = d.run(out=sentinel_out, lse=sentinel_lse)
    T = w.valid_tokens()
    assert T == 21
    assert torch.all(out[T:] == 7.0) and torch.all(lse[T:] == 123.0)
    ref_out, ref_lse = oracle.forward(w)
    assert_parity(out[:T].float().cpu().numpy(), lse[:T].cpu().numpy(), ref_out[:T], ref_lse[:T], "padding")


def test_lse_optional():
    w = wl.random_small(41, max_seqs=4)
    d = Device(w)
    out1, _ = d.run(want_lse=False)
    out2, lse2 = d.run()
    assert lse2 is not None and torch.equal(out1, out2)


@pytest.mark.parametrize("case", [MEDIUM[0], MEDIUM[1], MEDIUM[4]], ids=["dec", "pf", "fp8"])
def test_bitwise_deterministic(case):
    w = _medium(case, seed=7)
    d = Device(w)
    T = w.valid_tokens()
    o1, l1 = d.run()
    o1, l1 = o1[:T].clone(), l1[:T].clone()
    for _ in range(2):
        o2, l2 = d.run()
        # bit patterns, so that equal NaNs would also compare equal
        assert torch.equal(o1.view(torch.int16), o2[:T].view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2[:T].view(torch.int32))


@pytest.mark.parametrize("kvd", [wl.KV_BF16, wl.KV_FP8])
def test_poison_in_unread_memory_is_ignored(kvd):
    kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, pages_per_seq=None, sm_scale=0.09,
              sliding_window=200)
    if kvd == wl.KV_FP8:
        kw.update(kv_dtype=wl.KV_FP8, k_scale=0.05, v_scale=0.05)
    q_lens, kv_lens = [20, 1, 3], [1000, 717, 45]
    pages = sum((k + 15) // 16 for k in kv_lens)
    w = wl.build("poison", kw, q_lens, kv_lens, 3, total_num_pages=pages + 5, max_num_seqs=4, num_q_tokens=24)
    d = Device(w)
    o1, l1 = d.run()
    o1, l1 = o1.clone(), l1.clone()
    nan = 0x7FC0 if kvd == wl.KV_BF16 else 0x7F
    used = set()
    for s in range(w.n_seqs):
        n = (kv_lens[s] + 15) // 16
        used.update(int(p) for p in w.page_indices[s, :n])
        if kv_lens[s] % 16:
            w.kv_pages[w.page_indices[s, n - 1], kv_lens[s] % 16:] = nan
        w.page_indices[s, n:] = 1 << 29
    for p in range(w.cfg.total_num_pages):
        if p not in used:
            w.kv_pages[p] = nan
    w.page_indices[w.n_seqs:] = -7
    w.kv_lens[w.n_seqs:] = 1 << 30
    d2 = Device(w)
    o2, l2 = d2.run()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
