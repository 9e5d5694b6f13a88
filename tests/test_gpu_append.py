"""KV-cache append on the GPU (rpa_kv_append) against the oracle, bit for bit.

The append is integer/byte work once the f32 quotient is fixed, so the bar is
bit-exact equality of the whole cache (written slots and untouched ones):

* rounding: every finite bf16 value through every cache mode (bf16 bit copy,
  bf16 with scales, e4m3fn with several scales, saturation, subnormals);
* placement: random ragged batches (empty sequences, q_len = kv_len,
  page-crossing runs, padding tokens, spare table rows) at D 64/128/256;
* broken tables write nothing for the affected tokens;
* the named workloads at full size (written slots plus the untouched rest,
  compared on the device against the oracle's values scattered into a copy);
* append then attend: rpa_forward over the appended cache matches the oracle's
  attention over the oracle's appended cache.
"""

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_gqa_amd as rpa
import workloads as wl
from gpu_util import Device, assert_parity

pytestmark = pytest.mark.gpu


def _kv_host(dev):
    kv = dev.kv.cpu()
    return kv.numpy() if kv.dtype == torch.uint8 else kv.view(torch.int16).numpy().view(np.uint16)


def _bits_dev(a):
    """Row bits of the q dtype on the device: uint32 (f32) as float32, 16-bit as a 2-byte tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.float32)).cuda()
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def _append(dev, k_new, v_new):
    rpa.kv_append(_bits_dev(k_new), _bits_dev(v_new), dev.kv, dev.kv_lens, dev.page_indices, dev.cu_q_lens,
                  dev.num_seqs, dev.cfg)
    torch.cuda.synchronize()


def _assert_same_cache(got, ref, what):
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{what}: {len(bad)} cache elements differ; first at {bad[0].tolist()}: "
                             f"got {got[tuple(bad[0])]:#x}, want {ref[tuple(bad[0])]:#x}")


def _check(w, k_new, v_new, what):
    print(f"[append] {what}", flush=True)
    dev = Device(w)
    _append(dev, k_new, v_new)
    ref, _ = oracle.kv_append(w, k_new, v_new)
    _assert_same_cache(_kv_host(dev), ref, what)


# ------------------------------------------------------------- rounding

MODES = [
    (wl.KV_BF16, None, None),      # bit copy
    (wl.KV_BF16, 0.3, 7.0),
    (wl.KV_FP8, 0.05, 0.05),
    (wl.KV_FP8, 1.0, 3.0),
    (wl.KV_FP8, 1 / 3, 2.0 ** -10),
]


@pytest.mark.parametrize("kv_dtype,ks,vs", MODES)
def test_every_finite_bf16_value(kv_dtype, ks, vs):
    pats = wl.finite_bf16_patterns()               # 65280 = 255 tokens x 2 heads x 128
    kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=128, page_size=16, sm_scale=0.1,
              kv_dtype=kv_dtype, k_scale=ks, v_scale=vs)
    w = wl.build("rounding", kw, [255], [272], 21, total_num_pages=20)
    rng = np.random.Generator(np.random.PCG64(22))
    k_new = pats.reshape(255, 2, 128)
    v_new = rng.permutation(pats).reshape(255, 2, 128)
    _check(w, k_new, v_new, f"all bf16 values {kv_dtype} k/{ks} v/{vs}")


@pytest.mark.parametrize("kv_dtype", [wl.KV_BF16, wl.KV_FP8])
def test_nan_stays_nan(kv_dtype):
    kw = dict(num_q_heads=2, num_kv_heads=1, head_dim=64, page_size=16, sm_scale=0.1,
              kv_dtype=kv_dtype, k_scale=0.5, v_scale=0.5)
    w = wl.build("nan", kw, [2], [2], 23, total_num_pages=1)
    k_new, v_new = wl.new_kv(w, 24)
    k_new[0, 0, :8] = [0x7FC0, 0xFFC0, 0x7F81, 0xFF81, 0x7FFF, 0xFFFF, 0x7FC0, 0xFFC0]
    dev = Device(w)
    _append(dev, k_new, v_new)
    ref, _ = oracle.kv_append(w, k_new, v_new)
    got = _kv_host(dev)
    if kv_dtype == wl.KV_FP8:
        assert ((got[0, 0, 0, :8] & 0x7F) == 0x7F).all()
    else:
        g = got[0, 0, 0, :8]
        assert ((g & 0x7F80) == 0x7F80).all() and ((g & 0x7F) != 0).all()
    got[0, 0, 0, :8] = ref[0, 0, 0, :8]
    _assert_same_cache(got, ref, "NaN rows aside")


# ------------------------------------------------------------- placement

RAGGED = [(seed, D, kvd) for seed, (D, kvd) in enumerate(
    [(64, wl.KV_BF16), (128, wl.KV_BF16), (256, wl.KV_BF16), (64, wl.KV_FP8), (128, wl.KV_FP8),
     (256, wl.KV_FP8), (128, wl.KV_BF16), (128, wl.KV_FP8), (64, wl.KV_BF16), (256, wl.KV_FP8)], start=300)]


@pytest.mark.parametrize("seed,D,kvd", RAGGED)
def test_random_ragged_batches(seed, D, kvd):
    w = wl.random_small(seed, max_seqs=6, head_dim=D, kv_dtype=kvd, page_size=16 * (1 + seed % 3),
                        max_q=40, max_extra_kv=100)
    k_new, v_new = wl.new_kv(w, seed, std=2.0)
    _check(w, k_new, v_new, f"ragged seed {seed} D {D} {kvd}")


def test_hand_placement_case():
    from test_oracle_append import golden_rows, placement_case
    w = placement_case()
    k_new, v_new = wl.new_kv(w, 31)
    dev = Device(w)
    _append(dev, k_new, v_new)
    got = _kv_host(dev)
    for t, s, pos, page, slot in golden_rows():
        assert np.array_equal(got[page, slot, 0::2], k_new[t]) and np.array_equal(got[page, slot, 1::2], v_new[t])
    ref, _ = oracle.kv_append(w, k_new, v_new)
    _assert_same_cache(got, ref, "hand placement")


def test_many_sequences_search():
    """3000 sequences (several rounds of the 64-way sequence search), mixed
    q_len 0..3, some sequences with q_len = kv_len."""
    rng = np.random.Generator(np.random.PCG64(40))
    S = 3000
    q_lens = rng.integers(0, 3, size=S, endpoint=True)
    kv_lens = q_lens + rng.integers(0, 40, size=S) * (rng.random(S) < 0.8)
    kv_lens = np.maximum(kv_lens, 1)
    kw = dict(num_q_heads=2, num_kv_heads=1, head_dim=64, page_size=16, sm_scale=0.1)
    w = wl.build("many", kw, q_lens, kv_lens, 41, rng=rng, max_num_seqs=S + 5,
                 num_q_tokens=int(q_lens.sum()) + 3)
    k_new, v_new = wl.new_kv(w, 42)
    _check(w, k_new, v_new, "3000 sequences")


def test_broken_entries_write_nothing():
    from test_oracle_append import placement_case
    w = placement_case(wl.KV_FP8, k_scale=0.5, v_scale=0.5)
    k_new, v_new = wl.new_kv(w, 32)
    w.page_indices[1, 2] = 12        # out of range for 12 pages
    w.page_indices[3, 3] = -1
    w.kv_lens[0] = 0                 # q_len 1 > kv_len 0
    ref, skipped = oracle.kv_append(w, k_new, v_new)
    assert skipped == 1 + 3 + 16
    dev = Device(w)
    _append(dev, k_new, v_new)
    _assert_same_cache(_kv_host(dev), ref, "broken table")


def test_no_sequences_writes_nothing():
    from test_oracle_append import placement_case
    w = placement_case()
    w.num_seqs[0] = 0
    k_new, v_new = wl.new_kv(w, 33)
    dev = Device(w)
    _append(dev, k_new, v_new)
    _assert_same_cache(_kv_host(dev), w.kv_pages, "num_seqs 0")


def test_rejects_bad_arguments():
    from test_oracle_append import placement_case
    w = placement_case()
    dev = Device(w)
    k_new, v_new = wl.new_kv(w, 34)
    k, v = _bits_dev(k_new), _bits_dev(v_new)
    L = rpa.lib()
    c = dev.cfg.to_c()
    import ctypes
    args = [dev.kv_lens.data_ptr(), dev.page_indices.data_ptr(), dev.cu_q_lens.data_ptr(), dev.num_seqs.data_ptr(),
            None]
    assert L.rpa_kv_append(ctypes.byref(c), None, v.data_ptr(), dev.kv.data_ptr(), *args) == 1
    assert L.rpa_kv_append(ctypes.byref(c), k.data_ptr() + 2, v.data_ptr(), dev.kv.data_ptr(), *args) == 1
    c.k_scale = 0.0
    assert L.rpa_kv_append(ctypes.byref(c), k.data_ptr(), v.data_ptr(), dev.kv.data_ptr(), *args) == 1
    torch.cuda.synchronize()
    _assert_same_cache(_kv_host(dev), w.kv_pages, "rejected calls")


# ------------------------------------------------------------- full size

@pytest.mark.parametrize("number", [2, 3, 4, 5])
def test_named_workloads_full_size(number):
    w = wl.named(number)
    print(f"[append] named workload {number}", flush=True)
    k_new, v_new = wl.new_kv(w, 100 + number, std=1.0)
    c = w.cfg
    # oracle values of the written slots only (the cache copy would be large)
    seq = np.repeat(np.arange(w.n_seqs), w.q_lens())
    t = np.arange(w.valid_tokens())
    q0 = w.cu_q_lens[seq]
    pos = w.kv_lens[seq] - w.q_lens()[seq] + (t - q0)
    page = w.page_indices[seq, pos // c.page_size]
    slot = page.astype(np.int64) * c.page_size + pos % c.page_size
    small = wl.Workload(name="slots", cfg=wl.Config(
        num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads, head_dim=c.head_dim, page_size=1,
        total_num_pages=len(t), pages_per_seq=1, max_num_seqs=len(t), num_q_tokens=len(t),
        kv_dtype=c.kv_dtype, sm_scale=c.sm_scale, k_scale=c.k_scale, v_scale=c.v_scale),
        q=w.q[:len(t)], kv_pages=np.zeros((len(t), 1, 2 * c.num_kv_heads, c.head_dim), w.kv_pages.dtype),
        kv_lens=np.ones(len(t), np.int32), page_indices=np.arange(len(t), dtype=np.int32)[:, None],
        cu_q_lens=np.arange(len(t) + 1, dtype=np.int32), num_seqs=np.array([len(t)], np.int32))
    # the same tokens, one per sequence of one slot: the oracle's rounding, placed at `slot`
    ref_rows, skipped = oracle.kv_append(small, k_new[:len(t)], v_new[:len(t)])
    assert skipped == 0
    dev = Device(w)
    flat = dev.kv.view(-1, 2 * c.num_kv_heads, c.head_dim)
    expect = flat.clone()
    rows = torch.from_numpy(ref_rows.reshape(len(t), 2 * c.num_kv_heads, c.head_dim).view(
        np.int16 if ref_rows.dtype == np.uint16 else np.uint8)).cuda()
    if ref_rows.dtype == np.uint16:
        rows = rows.view(torch.bfloat16)
    expect[torch.from_numpy(slot).cuda()] = rows
    _append(dev, k_new, v_new)
    same = torch.equal(flat.view(torch.uint8) if flat.dtype == torch.uint8 else flat.view(torch.int16),
                       expect.view(torch.uint8) if expect.dtype == torch.uint8 else expect.view(torch.int16))
    assert same, f"named workload {number}: cache differs from the oracle's appended values"


# ------------------------------------------------------------- append, then attend

@pytest.mark.parametrize("seed,kvd,D", [(50, wl.KV_BF16, 128), (51, wl.KV_FP8, 128), (52, wl.KV_BF16, 64),
                                        (53, wl.KV_FP8, 256)])
def test_append_then_attend(seed, kvd, D):
    w = wl.random_small(seed, max_seqs=5, head_dim=D, kv_dtype=kvd, max_q=48, max_extra_kv=150)
    k_new, v_new = wl.new_kv(w, seed, std=1.5)
    dev = Device(w)
    _append(dev, k_new, v_new)
    out, lse = dev.run()
    kv_ref, _ = oracle.kv_append(w, k_new, v_new)
    w.kv_pages = kv_ref
    ref_out, ref_lse = oracle.forward(w)
    T = w.valid_tokens()
    assert_parity(out.float().cpu().numpy()[:T], lse.cpu().numpy()[:T], ref_out[:T], ref_lse[:T],
                  f"append+attend seed {seed}")
