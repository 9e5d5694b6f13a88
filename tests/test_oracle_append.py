"""Pins of the oracle's kv-cache append against things other than itself (no GPU).

* placement      - a hand-derived table of (token -> page, slot) in tests/golden/,
                   following the ragged paged attention kernel page's row ids
                   (query token i at key position kv_len - q_len + i) and its
                   page gather; every slot not listed keeps its bits
* K/V heads      - K of kv head h lands in combined head 2h, V in 2h+1 (the
                   page's `stridedLoadKv` layout), checked with distinct markers
* e4m3fn rounding - brute force: the nearest finite e4m3fn value (ties to the
                   even code, saturation at +-448) over every finite bf16 value
                   and over the midpoints between adjacent e4m3fn values; and
                   torch's float8_e4m3fn cast after clamping
* e5m2 rounding  - the same brute force over the finite e5m2 codes (saturation
                   at +-57344) and torch's float8_e5m2 cast
* int8 rounding  - numpy's rint (ties to even) and clip to [-128, 127] over every
                   finite bf16 value and the half-integers around the range
* f16 rounding   - numpy's float32 -> float16 cast (random patterns, midpoints,
                   the overflow edge); rows in f16 (f16 q) into f16 and fp8 caches
* bf16 rounding  - torch's float32 -> bfloat16 cast on random bit patterns,
                   subnormals and values next to the overflow threshold
* the quotient   - the appended code is the brute-force nearest code of
                   numpy's IEEE float32 quotient x / scale
* broken tables  - tokens whose page or position is out of range are skipped
"""

import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_append_placement.txt")


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def placement_case(kv_dtype=wl.KV_BF16, k_scale=None, v_scale=None):
    kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, sm_scale=0.125,
              kv_dtype=kv_dtype, k_scale=k_scale, v_scale=v_scale)
    return wl.from_tables(kw, [1, 5, 0, 16], [8, 35, 20, 64], [[3], [7, 1, 10], [5, 6], [2, 9, 4, 11]], 11,
                          total_num_pages=12, max_num_seqs=5, num_q_tokens=24, pages_per_seq=4)


def golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(tuple(int(x) for x in line.split()))
    return rows


def _f32(bits_u16):
    return (np.asarray(bits_u16, dtype=np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- placement

def test_placement_matches_hand_derived_table():
    w = placement_case()
    k_new, v_new = wl.new_kv(w, 5)
    kv, skipped = oracle.kv_append(w, k_new, v_new)
    assert skipped == 0
    rows = golden_rows()
    assert [r[0] for r in rows] == list(range(22))
    written = np.zeros(kv.shape[:2], dtype=bool)
    for t, s, pos, page, slot in rows:
        assert w.page_indices[s, pos // 16] == page and pos % 16 == slot  # the table itself is consistent
        for h in range(2):
            assert np.array_equal(kv[page, slot, 2 * h], k_new[t, h])
            assert np.array_equal(kv[page, slot, 2 * h + 1], v_new[t, h])
        written[page, slot] = True
    assert np.array_equal(kv[~written], w.kv_pages[~written])


def test_k_and_v_heads_land_in_even_and_odd_combined_heads():
    w = placement_case()
    T, Hkv, D = 24, 2, 64
    # markers: small integers, exact in bf16
    k = np.zeros((T, Hkv, D), np.float32)
    v = np.zeros((T, Hkv, D), np.float32)
    for t in range(T):
        for h in range(Hkv):
            k[t, h] = 1 + t + 32 * h
            v[t, h] = -(1 + t + 32 * h)
    kv, _ = oracle.kv_append(w, wl.to_bf16_bits(k), wl.to_bf16_bits(v))
    vals = _f32(kv)
    for t, s, pos, page, slot in golden_rows():
        for h in range(Hkv):
            assert (vals[page, slot, 2 * h] == 1 + t + 32 * h).all()
            assert (vals[page, slot, 2 * h + 1] == -(1 + t + 32 * h)).all()


def test_broken_table_entries_are_skipped():
    w = placement_case()
    k_new, v_new = wl.new_kv(w, 6)
    w.page_indices[1, 2] = 12          # tokens 3..5 of seq 1 -> page out of range
    w.kv_lens[0] = 0                   # seq 0: q_len 1 > kv_len 0 -> position -1
    kv, skipped = oracle.kv_append(w, k_new, v_new)
    assert skipped == 4
    assert np.array_equal(kv[3, 7], w.kv_pages[3, 7])
    assert np.array_equal(kv[1, 14, 0], k_new[1, 0])  # the rest of seq 1 still lands


def test_bf16_unit_scale_is_a_bit_copy():
    w = placement_case()
    bits = wl.finite_bf16_patterns()
    rng = np.random.Generator(np.random.PCG64(3))
    k = rng.choice(bits, size=(24, 2, 64))
    v = rng.choice(bits, size=(24, 2, 64))
    kv, _ = oracle.kv_append(w, k, v)
    for t, s, pos, page, slot in golden_rows():
        assert np.array_equal(kv[page, slot, 0::2], k[t])
        assert np.array_equal(kv[page, slot, 1::2], v[t])


# ---------------------------------------------------------------- rounding

def _e4m3fn_table():
    """(values f64, codes) of every finite e4m3fn code, decoded by torch."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return vals, codes


def brute_e4m3fn(x):
    """Nearest finite e4m3fn code of each f32 in x: same sign, ties to the even code,
    saturating at +-448. Brute force over the 254 finite codes."""
    vals, codes = _e4m3fn_table()
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), 448.0)
    pos_mask = (codes & 0x80) == 0
    pv, pc = vals[pos_mask], codes[pos_mask]
    d = np.abs(a[:, None] - pv[None, :])
    best = d.min(axis=1, keepdims=True)
    tie = d == best
    # among tied candidates prefer the even code
    pick = np.where(tie & ((pc[None, :] & 1) == 0), 1, 0) + tie
    idx = np.argmax(pick, axis=1)
    out = pc[idx].astype(np.uint8)
    return np.where(neg, out | 0x80, out).astype(np.uint8)


def _e4m3fn_midpoints():
    vals, codes = _e4m3fn_table()
    pv = np.sort(vals[(codes & 0x80) == 0])
    mids = (pv[1:] + pv[:-1]) / 2
    mids = np.concatenate([mids, [448.0, 456.0, 464.0, 480.0, 1e6, 2.0 ** -10, 2.0 ** -11]])
    m32 = mids.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mids)  # every midpoint is an f32
    up = np.nextafter(m32, np.float32(np.inf))
    dn = np.nextafter(m32, np.float32(0))
    x = np.concatenate([m32, up, dn])
    return np.concatenate([x, -x])


def test_e4m3fn_rounding_matches_brute_force_on_all_bf16_values():
    x = _f32(wl.finite_bf16_patterns())
    assert np.array_equal(oracle.f32_to_e4m3fn(x), brute_e4m3fn(x))


def test_e4m3fn_rounding_at_midpoints_and_saturation():
    x = _e4m3fn_midpoints()
    got = oracle.f32_to_e4m3fn(x)
    assert np.array_equal(got, brute_e4m3fn(x))
    # saturation: everything at or past 448 in magnitude is the largest finite code
    big = np.abs(x) >= 448
    assert ((got[big] & 0x7F) == 0x7E).all()


def test_e4m3fn_rounding_matches_torch_cast_after_clamp():
    rng = np.random.Generator(np.random.PCG64(9))
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * np.float32(s)
                        for s in (1e-3, 0.1, 1.0, 30.0, 300.0)])
    x = np.concatenate([x, _e4m3fn_midpoints()])
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.f32_to_e4m3fn(x), ref)


def _e5m2_table():
    codes = np.array([c for c in range(256) if ((c >> 2) & 31) != 31], dtype=np.uint8)
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e5m2).to(torch.float64).numpy()
    return vals, codes


def brute_e5m2(x):
    """Nearest finite e5m2 code (same sign, ties to the even code, saturating at
    +-57344), by brute force over the finite codes."""
    vals, codes = _e5m2_table()
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    a = np.minimum(np.abs(x), 57344.0)
    pos = (codes & 0x80) == 0
    pv, pc = vals[pos], codes[pos]
    d = np.abs(a[:, None] - pv[None, :])
    tie = d == d.min(axis=1, keepdims=True)
    idx = np.argmax(np.where(tie & ((pc[None, :] & 1) == 0), 1, 0) + tie, axis=1)
    out = pc[idx].astype(np.uint8)
    return np.where(neg, out | 0x80, out).astype(np.uint8)


def test_e5m2_rounding_matches_brute_force_and_torch():
    x = _f32(wl.finite_bf16_patterns())
    vals, codes = _e5m2_table()
    pv = np.sort(vals[(codes & 0x80) == 0])
    mids = ((pv[1:] + pv[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
                        -mids, np.float32([57344, 61440, 65536, 1e9])])
    got = oracle.f32_to_e5m2(x)
    assert np.array_equal(got, brute_e5m2(x))
    ref = torch.from_numpy(np.clip(x, -57344, 57344)).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e5m2_append_is_the_nearest_code_of_the_f32_quotient():
    w = placement_case(wl.KV_E5M2, k_scale=0.01, v_scale=7.0)
    k_new, v_new = wl.new_kv(w, 9, std=5.0)
    kv, _ = oracle.kv_append(w, k_new, v_new)
    for t, s_, pos, page, slot in golden_rows():
        assert np.array_equal(kv[page, slot, 0::2], brute_e5m2(_f32(k_new[t]).ravel() / np.float32(0.01)).reshape(2, 64))
        assert np.array_equal(kv[page, slot, 1::2], brute_e5m2(_f32(v_new[t]).ravel() / np.float32(7.0)).reshape(2, 64))


def test_f16_rounding_matches_numpy_cast():
    rng = np.random.Generator(np.random.PCG64(14))
    bits = rng.integers(0, 1 << 32, size=60000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]
    x = bits.view(np.float32)
    # f16 midpoints (exact in f32) and their neighbours, subnormals, the overflow edge
    h = np.arange(0, 0x7C00, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[1:] + h[:-1]) / 2).astype(np.float32)
    edge = np.float32([65504, 65519, 65520, 65535, 65536, 1e6, 2.0 ** -25, 3 * 2.0 ** -26])
    x = np.concatenate([x, mids, np.nextafter(mids, np.float32(np.inf)), edge, -edge])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16(x), ref)


def test_f16_rows_append_into_f16_and_fp8_caches():
    """New rows in f16 (f16 q): an f16 cache takes RN_f16(x / scale), an
    e4m3fn cache the nearest code of the f32 quotient."""
    for kvd, ks in ((wl.KV_F16, 0.5), (wl.KV_FP8, 0.05)):
        kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, sm_scale=0.125,
                  kv_dtype=kvd, q_dtype=wl.Q_F16, k_scale=ks, v_scale=2.0)
        w = wl.from_tables(kw, [1, 5, 0, 16], [8, 35, 20, 64], [[3], [7, 1, 10], [5, 6], [2, 9, 4, 11]], 12,
                           total_num_pages=12, max_num_seqs=5, num_q_tokens=24, pages_per_seq=4)
        k_new, v_new = wl.new_kv(w, 15, std=3.0)
        kv, skipped = oracle.kv_append(w, k_new, v_new)
        assert skipped == 0
        xk = k_new.view(np.float16).astype(np.float32)
        xv = v_new.view(np.float16).astype(np.float32)
        for t, s_, pos, page, slot in golden_rows():
            qk = xk[t].ravel() / np.float32(ks)
            qv = xv[t].ravel() / np.float32(2.0)
            if kvd == wl.KV_F16:
                assert np.array_equal(kv[page, slot, 0::2].ravel(), qk.astype(np.float16).view(np.uint16))
                assert np.array_equal(kv[page, slot, 1::2].ravel(), qv.astype(np.float16).view(np.uint16))
            else:
                assert np.array_equal(kv[page, slot, 0::2].ravel(), brute_e4m3fn(qk))
                assert np.array_equal(kv[page, slot, 1::2].ravel(), brute_e4m3fn(qv))


def test_f32_rows_append_into_bf16_fp8_and_int8_caches():
    """New rows in f32 (f32 q): each cache takes its rounding of the f32
    quotient x / scale, with every bit of x read (a bf16 cache: torch's RNE
    cast; e4m3fn: the brute-force nearest code; int8: numpy's rint and clip)."""
    for kvd, ks in ((wl.KV_BF16, 0.5), (wl.KV_FP8, 0.05), (wl.KV_I8, 0.05)):
        kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16, sm_scale=0.125,
                  kv_dtype=kvd, q_dtype=wl.Q_F32, k_scale=ks, v_scale=2.0)
        w = wl.from_tables(kw, [1, 5, 0, 16], [8, 35, 20, 64], [[3], [7, 1, 10], [5, 6], [2, 9, 4, 11]], 12,
                           total_num_pages=12, max_num_seqs=5, num_q_tokens=24, pages_per_seq=4)
        k_new, v_new = wl.new_kv(w, 16, std=3.0)
        assert k_new.dtype == np.uint32 and np.any(k_new & 0xFFFF)
        kv, skipped = oracle.kv_append(w, k_new, v_new)
        assert skipped == 0
        xk = k_new.view(np.float32)
        xv = v_new.view(np.float32)
        for t, s_, pos, page, slot in golden_rows():
            for comb, x, sc in ((0, xk, ks), (1, xv, 2.0)):
                qx = x[t].ravel() / np.float32(sc)
                got = kv[page, slot, comb::2].ravel()
                if kvd == wl.KV_BF16:
                    ref = torch.from_numpy(qx.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                elif kvd == wl.KV_FP8:
                    ref = brute_e4m3fn(qx)
                else:
                    ref = np.clip(np.rint(qx), -128, 127).astype(np.int8).view(np.uint8)
                assert np.array_equal(got, ref), (kvd, t, comb)


def test_i8_rounding_matches_numpy_rint_and_clip():
    x = _f32(wl.finite_bf16_patterns())
    halves = np.arange(-140, 140, dtype=np.float32) + np.float32(0.5)   # ties: to even
    x = np.concatenate([x, halves, np.nextafter(halves, np.float32(np.inf)), np.nextafter(halves, np.float32(-np.inf))])
    ref = np.clip(np.rint(x.astype(np.float64)), -128, 127).astype(np.int8)
    assert np.array_equal(oracle.f32_to_i8(x), ref)
    assert oracle.f32_to_i8(np.float32([np.nan]))[0] == 0


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.Generator(np.random.PCG64(10))
    bits = rng.integers(0, 1 << 32, size=60000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]                    # finite
    sub = rng.integers(0, 1 << 23, size=2000, dtype=np.uint32)        # subnormals
    near_max = np.arange(0x7F7F0000, 0x7F7FFFFF, 97, dtype=np.uint32)  # next to overflow
    ties = (rng.integers(0, 1 << 15, size=2000, dtype=np.uint32) << 16) | 0x8000
    ties = ties[(ties & 0x7F800000) != 0x7F800000]
    allb = np.concatenate([bits, sub, near_max, ties, ties | 0x80000000])
    x = allb.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(x), ref)


def test_fp8_append_is_the_nearest_code_of_the_f32_quotient():
    rng = np.random.Generator(np.random.PCG64(12))
    xs = _f32(rng.choice(wl.finite_bf16_patterns(), size=40000))
    for s in (np.float32(0.05), np.float32(3.0), np.float32(1 / 3)):
        with np.errstate(over="ignore"):
            q32 = xs / s                                        # IEEE float32 division
        assert np.array_equal(oracle.f32_to_e4m3fn(q32), brute_e4m3fn(q32))
    w = placement_case(wl.KV_FP8, k_scale=0.05, v_scale=3.0)
    k_new, v_new = wl.new_kv(w, 8, std=4.0)
    kv, _ = oracle.kv_append(w, k_new, v_new)
    for t, s_, pos, page, slot in golden_rows():
        assert np.array_equal(kv[page, slot, 0::2], brute_e4m3fn(_f32(k_new[t]).ravel() / np.float32(0.05)).reshape(2, 64))
        assert np.array_equal(kv[page, slot, 1::2], brute_e4m3fn(_f32(v_new[t]).ravel() / np.float32(3.0)).reshape(2, 64))


def test_bf16_scaled_append_rounds_the_f32_quotient():
    w = placement_case(wl.KV_BF16, k_scale=0.3, v_scale=7.0)
    k_new, v_new = wl.new_kv(w, 13, std=3.0)
    kv, _ = oracle.kv_append(w, k_new, v_new)
    tb = lambda x: torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for t, s_, pos, page, slot in golden_rows():
        assert np.array_equal(kv[page, slot, 0::2], tb(_f32(k_new[t]) / np.float32(0.3)))
        assert np.array_equal(kv[page, slot, 1::2], tb(_f32(v_new[t]) / np.float32(7.0)))


def test_nan_input_gives_nan_code():
    assert (oracle.f32_to_e4m3fn(np.array([np.nan, -np.nan], np.float32)) & 0x7F == 0x7F).all()
    b = oracle.f32_to_bf16(np.array([np.nan], np.float32))
    assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0
