"""Pins of the CPU oracle against things other than itself (no GPU).

Every part of the oracle is tied here to a closed form, an invariant, or a
library routine, so that a plausible slip in it (a dropped term, a swapped K/V
head, a wrong causal offset or GQA index) fails at least one test:

* dtype decode          - torch's own casts (numpy's for f16), plus printed
                          e4m3fn, e5m2 and binary16 values; fp8 and int8
                          caches and f16 q / K/V end to end against sdpa over
                          those decodes (int8: numpy's signed byte x scale)
* softmax/PV/GQA/scale  - torch.scaled_dot_product_attention in f64
* causal offsets        - Q = 0 closed form: lse = ln(#visible keys)
* window boundary       - window 1 returns V at the query position exactly;
                          shift invariance; Q = 0 counts
* soft-cap              - tanh from the math library; the logistic form of
                          the spatial-compiler page (`capped`); a closed form
                          end to end
* page gather           - page-table permutation invariance; poison in pages,
                          slots and table entries the method never reads
* raggedness            - each sequence alone reproduces its slice
* dequant scales        - linearity
* attention sinks       - closed forms (Q = 0; a single visible key), the
                          log-sum-exp identity against the same rows without
                          sinks, and sinks at -inf changing nothing
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _seq_kv(w, s, comb):
    """Contiguous f64 keys (comb=0) or values (comb=1) of sequence s, per kv head,
    read through the page table: [Hkv, kv_len, D]."""
    c = w.cfg
    kvl = int(w.kv_lens[s])
    idx = np.arange(kvl)
    phys = w.page_indices[s, idx // c.page_size]
    slot = idx % c.page_size
    bits = w.kv_pages[phys, slot]  # [kv_len, 2Hkv, D]
    if c.kv_dtype == wl.KV_I8:
        vals = bits.view(np.int8).astype(np.float64) * (c.k_scale if comb == 0 else c.v_scale)
    elif wl.is_fp8(c.kv_dtype):
        tdt = torch.float8_e4m3fn if c.kv_dtype == wl.KV_FP8 else torch.float8_e5m2
        vals = torch.from_numpy(bits.copy()).view(tdt).to(torch.float64).numpy()
        scale = (c.k_scale if comb == 0 else c.v_scale)
        vals = vals * scale
    elif c.kv_dtype == wl.KV_F16:
        vals = bits.view(np.float16).astype(np.float64)
    else:
        vals = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    return np.transpose(vals[:, comb::2, :], (1, 0, 2))


def _q_f64(w):
    if w.cfg.q_dtype == wl.Q_F32:
        return w.q.view(np.float32).astype(np.float64)
    if w.cfg.q_dtype == wl.Q_F16:
        return w.q.view(np.float16).astype(np.float64)
    return torch.from_numpy(w.q.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


# ----------------------------------------------------------------------------- decode

def test_e4m3fn_all_codes_match_torch_cast():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # NaN only at S.1111.111
    assert set(np.flatnonzero(np.isnan(mine))) == {0x7F, 0xFF}


def test_e4m3fn_printed_values():
    # OCP FP8 E4M3: largest finite 448, smallest subnormal 2^-9, smallest normal 2^-6.
    table = {0x00: 0.0, 0x38: 1.0, 0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9,
             0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9, 0x40: 2.0, 0x3C: 1.5}
    for code, val in table.items():
        assert oracle.e4m3fn_to_f64(np.array([code], np.uint8))[0] == val
    assert math.copysign(1.0, oracle.e4m3fn_to_f64(np.array([0x80], np.uint8))[0]) == -1.0


def test_e5m2_all_codes_match_torch_cast():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e5m2_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # NaN at exponent 31 with a non-zero mantissa, infinities at S.11111.00
    assert set(np.flatnonzero(np.isnan(mine))) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}
    assert mine[0x7C] == np.inf and mine[0xFC] == -np.inf


def test_e5m2_printed_values():
    # OCP FP8 E5M2: largest finite 57344, smallest subnormal 2^-16, smallest normal 2^-14.
    table = {0x00: 0.0, 0x3C: 1.0, 0x7B: 57344.0, 0xFB: -57344.0, 0x01: 2.0 ** -16,
             0x04: 2.0 ** -14, 0x03: 3 * 2.0 ** -16, 0x40: 2.0, 0x3E: 1.5}
    for code, val in table.items():
        assert oracle.e5m2_to_f64(np.array([code], np.uint8))[0] == val
    assert math.copysign(1.0, oracle.e5m2_to_f64(np.array([0x80], np.uint8))[0]) == -1.0


def test_f16_all_patterns_match_numpy_cast():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    # IEEE binary16: largest finite 65504, smallest subnormal 2^-24
    assert mine[0x7BFF] == 65504.0 and mine[0x0001] == 2.0 ** -24 and mine[0x7C00] == np.inf


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # drop inf/NaN patterns
    mine = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(mine, ref)


# ----------------------------------------------------------------------------- soft-cap

@pytest.mark.parametrize("c", [1.0, 30.0, 50.0])
def test_soft_cap_matches_math_tanh_and_logistic_form(c):
    for x in [-1e4, -200.0, -3.7, -1e-3, 0.0, 2.5e-7, 0.9, 49.0, 51.0, 1e5]:
        s = oracle.soft_cap(x, c)
        assert s == pytest.approx(c * math.tanh(x / c), rel=1e-15, abs=1e-300)
        # 2c*sigma(2x/c) - c with sigma(z) = 1/(1+exp(-z)): one exp, one reciprocal
        z = 2 * x / c
        logistic = 2 * c / (1 + math.exp(-z)) - c if z > -700 else -c
        assert s == pytest.approx(logistic, rel=1e-12, abs=1e-12 * c)
        assert abs(s) <= c
    assert oracle.soft_cap(1e-6, 50.0) == pytest.approx(1e-6, rel=1e-9)


# ----------------------------------------------------------------------------- library pin

def _sdpa_case(seed, G, Hkv, D, kv_len, causal, page_size=16, perm_table=True):
    q_len = kv_len  # square: top-left and bottom-right causal alignment agree
    kw = dict(num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=page_size,
              pages_per_seq=None, sm_scale=0.37, is_causal=causal)
    w = wl.build("sdpa", kw, [q_len], [kv_len], seed)
    if not perm_table:
        n = w.page_indices.shape[1]
        w.page_indices[0, :n] = np.arange(n)
    return w


@pytest.mark.parametrize("G,Hkv,D,kv_len,causal", [
    (1, 1, 16, 37, False), (2, 2, 32, 50, True), (4, 2, 64, 64, True), (3, 3, 16, 21, False),
])
def test_matches_torch_sdpa_square(G, Hkv, D, kv_len, causal):
    w = _sdpa_case(11 + G + D, G, Hkv, D, kv_len, causal)
    out, lse = oracle.forward(w)
    q = torch.from_numpy(_q_f64(w)).permute(1, 0, 2)[None]          # [1, Hq, T, D]
    k = torch.from_numpy(_seq_kv(w, 0, 0).copy())[None]                # [1, Hkv, kv, D]
    v = torch.from_numpy(_seq_kv(w, 0, 1).copy())[None]
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=w.cfg.sm_scale,
                                         enable_gqa=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # lse against torch.logsumexp of the library's own scaled scores
    kk = k.repeat_interleave(G, dim=1)
    scores = (q @ kk.transpose(-1, -2)) * w.cfg.sm_scale
    if causal:
        scores = scores.masked_fill(torch.ones(kv_len, kv_len, dtype=torch.bool).triu(1), float("-inf"))
    ref_lse = torch.logsumexp(scores, dim=-1)[0].permute(1, 0).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kv_dtype", [wl.KV_FP8, wl.KV_E5M2, wl.KV_I8])
def test_fp8_cache_matches_torch_sdpa_on_decoded_values(kv_dtype):
    """fp8 K/V (each kind) are read as code * scale: the oracle equals sdpa in
    f64 over torch's own decode of the same codes, scaled."""
    G, Hkv, D, kv_len = 2, 2, 32, 40
    kw = dict(num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=16, pages_per_seq=None,
              sm_scale=0.3, is_causal=True, kv_dtype=kv_dtype, k_scale=0.25, v_scale=3.0)
    w = wl.build("fp8sdpa", kw, [kv_len], [kv_len], 17)
    out, _ = oracle.forward(w)
    q = torch.from_numpy(_q_f64(w)).permute(1, 0, 2)[None]
    k = torch.from_numpy(_seq_kv(w, 0, 0).copy())[None]
    v = torch.from_numpy(_seq_kv(w, 0, 1).copy())[None]
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.cfg.sm_scale,
                                         enable_gqa=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kv_dtype", [wl.KV_F16, wl.KV_FP8, wl.KV_E5M2, wl.KV_I8])
def test_f16_q_matches_torch_sdpa_on_decoded_values(kv_dtype):
    """f16 q (the page's `Cfg` q_dtype) with f16 or fp8 K/V: sdpa in f64 over
    numpy's / torch's decode of the same bits."""
    G, Hkv, D, kv_len = 2, 2, 32, 40
    kw = dict(num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=16, pages_per_seq=None,
              sm_scale=0.3, is_causal=True, kv_dtype=kv_dtype, q_dtype=wl.Q_F16)
    if wl.is_fp8(kv_dtype):
        kw.update(k_scale=0.25, v_scale=3.0)
    w = wl.build("f16sdpa", kw, [kv_len], [kv_len], 18)
    out, _ = oracle.forward(w)
    q = torch.from_numpy(_q_f64(w)).permute(1, 0, 2)[None]
    k = torch.from_numpy(_seq_kv(w, 0, 0).copy())[None]
    v = torch.from_numpy(_seq_kv(w, 0, 1).copy())[None]
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.cfg.sm_scale,
                                         enable_gqa=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kv_dtype", [wl.KV_BF16, wl.KV_FP8, wl.KV_E5M2, wl.KV_I8])
def test_f32_q_matches_torch_sdpa_on_decoded_values(kv_dtype):
    """f32 q (the page's `Cfg` q_dtype, packing 1): every f32 bit of q counts;
    sdpa in f64 over numpy's reading of the same bits."""
    G, Hkv, D, kv_len = 2, 2, 32, 40
    kw = dict(num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=16, pages_per_seq=None,
              sm_scale=0.3, is_causal=True, kv_dtype=kv_dtype, q_dtype=wl.Q_F32)
    if wl.is_fp8(kv_dtype):
        kw.update(k_scale=0.25, v_scale=3.0)
    w = wl.build("f32sdpa", kw, [kv_len], [kv_len], 19)
    assert w.q.dtype == np.uint32
    # the generated q is not bf16-representable: the low 16 bits are used
    assert np.any(w.q & 0xFFFF)
    out, lse = oracle.forward(w)
    q = torch.from_numpy(_q_f64(w)).permute(1, 0, 2)[None]
    k = torch.from_numpy(_seq_kv(w, 0, 0).copy())[None]
    v = torch.from_numpy(_seq_kv(w, 0, 1).copy())[None]
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.cfg.sm_scale,
                                         enable_gqa=True)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_f32_q_of_bf16_values_equals_bf16_q():
    """An f32 q that holds bf16 values gives exactly the bf16-q result; with
    its low bits kept the result moves (the f32 bits are read, not truncated)."""
    kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=32, page_size=16, pages_per_seq=None,
              sm_scale=0.3, is_causal=True)
    wb = wl.build("qbf16", dict(kw, q_dtype=wl.Q_BF16), [6, 1], [30, 17], 23)
    wf = wl.build("qf32", dict(kw, q_dtype=wl.Q_F32), [6, 1], [30, 17], 23)
    # same draw: the f32 q rounds to the bf16 q
    assert np.array_equal(wl.to_bf16_bits(wf.q.view(np.float32)), wb.q)
    ob, lb = oracle.forward(wb)
    of, lf = oracle.forward(wf)
    assert not np.allclose(lf, lb, rtol=0, atol=1e-9)
    wf.q = (wb.q.astype(np.uint32) << 16)  # exactly the bf16 values, as f32
    o2, l2 = oracle.forward(wf)
    assert np.array_equal(o2, ob) and np.array_equal(l2, lb)


def test_bottom_right_causal_equals_suffix_of_square_problem():
    """A sequence's q_len queries are the LAST q_len positions of its keys:
    the result equals the bottom rows of the square causal problem (library)."""
    G, Hkv, D, kv_len, q_len = 2, 2, 32, 45, 7
    kw = dict(num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, page_size=16,
              pages_per_seq=None, sm_scale=0.2, is_causal=True)
    w = wl.build("suffix", kw, [q_len], [kv_len], 5)
    out, lse = oracle.forward(w)
    k = torch.from_numpy(_seq_kv(w, 0, 0).copy())[None]
    v = torch.from_numpy(_seq_kv(w, 0, 1).copy())[None]
    qfull = torch.zeros(1, G * Hkv, kv_len, D, dtype=torch.float64)
    qfull[0, :, kv_len - q_len:] = torch.from_numpy(_q_f64(w)).permute(1, 0, 2)
    ref = F.scaled_dot_product_attention(qfull, k, v, is_causal=True, scale=w.cfg.sm_scale,
                                         enable_gqa=True)[0, :, kv_len - q_len:].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- closed forms

def _zero_q(w):
    w.q[:] = 0
    return w


@pytest.mark.parametrize("window", [None, 1, 5, 40])
@pytest.mark.parametrize("causal", [True, False])
def test_zero_q_lse_counts_visible_keys(window, causal):
    w = _zero_q(wl.random_small(3, max_seqs=4, window=window, causal=causal, max_q=20, max_extra_kv=60))
    out, lse = oracle.forward(w)
    for s in range(w.n_seqs):
        q0 = int(w.cu_q_lens[s]); ql = int(w.cu_q_lens[s + 1]) - q0; kvl = int(w.kv_lens[s])
        v = _seq_kv(w, s, 1)
        G = w.cfg.num_q_heads // w.cfg.num_kv_heads
        for i in range(ql):
            p = kvl - ql + i
            hi = p + 1 if causal else kvl
            lo = max(0, p - window + 1) if window else 0
            n_vis = hi - lo
            assert np.all(lse[q0 + i] == math.log(n_vis)), (s, i)
            for n in range(w.cfg.num_q_heads):
                np.testing.assert_allclose(out[q0 + i, n], v[n // G, lo:hi].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_window_one_returns_value_at_query_position():
    w = wl.random_small(8, max_seqs=4, window=1, causal=True)
    out, lse = oracle.forward(w)
    G = w.cfg.num_q_heads // w.cfg.num_kv_heads
    q = _q_f64(w)
    for s in range(w.n_seqs):
        q0 = int(w.cu_q_lens[s]); ql = int(w.cu_q_lens[s + 1]) - q0; kvl = int(w.kv_lens[s])
        k = _seq_kv(w, s, 0); v = _seq_kv(w, s, 1)
        for i in range(ql):
            p = kvl - ql + i
            for n in range(w.cfg.num_q_heads):
                assert np.array_equal(out[q0 + i, n], v[n // G, p])
                x = float(np.dot(q[q0 + i, n], k[n // G, p])) * w.cfg.sm_scale
                assert lse[q0 + i, n] == pytest.approx(x, rel=1e-13, abs=1e-13)


def test_window_equals_dropping_keys_before_it():
    """Shift invariance: a window that starts at key lo for every query gives the
    same rows as the same sequence with keys [lo, kv_len) and no window."""
    D, page = 32, 16
    kw = dict(num_q_heads=4, num_kv_heads=2, head_dim=D, page_size=page, pages_per_seq=None,
              sm_scale=0.25, is_causal=True, sliding_window=None)
    kv_len, q_len, lo = 64, 1, 32   # lo is page aligned
    w_full = wl.build("full", dict(kw, sliding_window=kv_len - lo), [q_len], [kv_len], 21)
    w_cut = wl.build("cut", kw, [q_len], [kv_len - lo], 21)
    # same Q; the cut sequence reads the full sequence's last pages
    w_cut.q[:] = w_full.q
    w_cut.kv_pages = w_full.kv_pages
    w_cut.cfg.total_num_pages = w_full.cfg.total_num_pages
    w_cut.page_indices = np.ascontiguousarray(w_full.page_indices[:, lo // page:])
    w_cut.cfg.pages_per_seq = w_cut.page_indices.shape[1]
    o1, l1 = oracle.forward(w_full)
    o2, l2 = oracle.forward(w_cut)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-14, atol=1e-15)


def test_equal_scores_give_mean_of_visible_values():
    w = wl.random_small(12, max_seqs=3, causal=True)
    # every key row identical -> every visible score equal
    kv = w.kv_pages.reshape(-1, w.cfg.page_size, w.cfg.num_kv_heads, 2, w.cfg.head_dim)
    kv[:, :, :, 0, :] = kv[0:1, 0:1, :, 0, :]
    out, lse = oracle.forward(w)
    G = w.cfg.num_q_heads // w.cfg.num_kv_heads
    for s in range(w.n_seqs):
        q0 = int(w.cu_q_lens[s]); ql = int(w.cu_q_lens[s + 1]) - q0; kvl = int(w.kv_lens[s])
        v = _seq_kv(w, s, 1)
        for i in range(ql):
            p = kvl - ql + i
            for n in range(w.cfg.num_q_heads):
                np.testing.assert_allclose(out[q0 + i, n], v[n // G, :p + 1].mean(axis=0), rtol=1e-12, atol=1e-14)


def test_gqa_map_constant_values_per_kv_head():
    w = wl.random_small(14, max_seqs=3, G=3)
    Hkv = w.cfg.num_kv_heads
    consts = wl.to_bf16_bits(np.arange(1, Hkv + 1, dtype=np.float32) * 0.5)
    kv = w.kv_pages.reshape(-1, w.cfg.page_size, Hkv, 2, w.cfg.head_dim)
    for h in range(Hkv):
        kv[:, :, h, 1, :] = consts[h]
    out, _ = oracle.forward(w)
    T = w.valid_tokens()
    for n in range(w.cfg.num_q_heads):
        assert np.all(out[:T, n] == 0.5 * (n // 3 + 1))


def test_soft_cap_closed_form_end_to_end():
    """Q = a*e0 and every K row b*e0: every score x = a*b*sm_scale, so the row is
    uniform, out = mean V and lse = c*tanh(x/c) + ln(#visible)."""
    c = 3.0
    w = wl.random_small(15, max_seqs=3, soft_cap=c, causal=True)
    D = w.cfg.head_dim
    a, b = 6.0, 8.0
    w.q[:] = 0
    w.q[:, :, 0] = wl.to_bf16_bits(np.array([a], np.float32))[0]
    kv = w.kv_pages.reshape(-1, w.cfg.page_size, w.cfg.num_kv_heads, 2, D)
    kv[:, :, :, 0, :] = 0
    kv[:, :, :, 0, 0] = wl.to_bf16_bits(np.array([b], np.float32))[0]
    out, lse = oracle.forward(w)
    x = a * b * w.cfg.sm_scale
    for s in range(w.n_seqs):
        q0 = int(w.cu_q_lens[s]); ql = int(w.cu_q_lens[s + 1]) - q0; kvl = int(w.kv_lens[s])
        for i in range(ql):
            n_vis = kvl - ql + i + 1
            np.testing.assert_allclose(lse[q0 + i], c * math.tanh(x / c) + math.log(n_vis), rtol=1e-14)


# ----------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("kv_dtype", [wl.KV_BF16, wl.KV_FP8, wl.KV_E5M2, wl.KV_F16, wl.KV_I8])
def test_page_permutation_invariance(kv_dtype):
    w = wl.random_small(21, max_seqs=4, kv_dtype=kv_dtype, window=9,
                        q_dtype=wl.Q_F16 if kv_dtype == wl.KV_F16 else wl.Q_BF16)
    o1, l1 = oracle.forward(w)
    rng = np.random.default_rng(7)
    P = w.cfg.total_num_pages
    perm = rng.permutation(P)          # new location of old page p is perm[p]
    new_kv = np.empty_like(w.kv_pages)
    new_kv[perm] = w.kv_pages
    w.kv_pages = new_kv
    used = np.zeros_like(w.page_indices, dtype=bool)
    for s in range(w.n_seqs):
        used[s, :(int(w.kv_lens[s]) + w.cfg.page_size - 1) // w.cfg.page_size] = True
    w.page_indices = np.where(used, perm[w.page_indices], w.page_indices).astype(np.int32)
    o2, l2 = oracle.forward(w)
    assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(l1, l2, equal_nan=True)


@pytest.mark.parametrize("kv_dtype", [wl.KV_BF16, wl.KV_FP8])
def test_poison_in_unread_memory_is_ignored(kv_dtype):
    w = wl.random_small(22, max_seqs=4, kv_dtype=kv_dtype)
    o1, l1 = oracle.forward(w)
    c = w.cfg
    nan = 0x7FC0 if kv_dtype == wl.KV_BF16 else 0x7F
    used_pages = set()
    for s in range(w.n_seqs):
        kvl = int(w.kv_lens[s]); n = (kvl + c.page_size - 1) // c.page_size
        used_pages.update(int(p) for p in w.page_indices[s, :n])
        w.page_indices[s, n:] = 2 ** 30            # never dereferenced
        if kvl % c.page_size:
            w.kv_pages[w.page_indices[s, n - 1], kvl % c.page_size:] = nan   # tail slots
    for p in range(c.total_num_pages):
        if p not in used_pages:
            w.kv_pages[p] = nan
    w.page_indices[w.n_seqs:] = -5
    o2, l2 = oracle.forward(w)
    assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(l1, l2, equal_nan=True)


def test_each_sequence_alone_reproduces_its_slice():
    w = wl.random_small(23, max_seqs=4)
    o_all, l_all = oracle.forward(w)
    for s in range(w.n_seqs):
        q0 = int(w.cu_q_lens[s]); q1 = int(w.cu_q_lens[s + 1])
        ws = wl.Workload(w.name, w.cfg, w.q, w.kv_pages, w.kv_lens.copy(), w.page_indices.copy(),
                         w.cu_q_lens.copy(), w.num_seqs.copy())
        # sequence s becomes the only sequence, keeping its tokens in place
        ws.kv_lens[:] = 0; ws.kv_lens[0] = w.kv_lens[s]
        ws.page_indices[0] = w.page_indices[s]
        ws.cu_q_lens[:] = q1; ws.cu_q_lens[0] = q0
        ws.num_seqs = np.array([1], np.int32)
        o, l = oracle.forward(ws)
        assert np.array_equal(o[q0:q1], o_all[q0:q1]) and np.array_equal(l[q0:q1], l_all[q0:q1])


def test_value_scale_is_linear_and_key_scale_folds_into_sm_scale():
    w = wl.random_small(24, max_seqs=3, kv_dtype=wl.KV_FP8, soft_cap=None)
    o1, l1 = oracle.forward(w)
    w.cfg.v_scale = w.cfg.v_scale * 2.0
    o2, l2 = oracle.forward(w)
    T = w.valid_tokens()
    assert np.array_equal(o2[:T], 2.0 * o1[:T]) and np.array_equal(l2[:T], l1[:T])
    w.cfg.v_scale /= 2.0
    ks = w.cfg.k_scale
    w.cfg.k_scale = 1.0
    w.cfg.sm_scale = w.cfg.sm_scale * ks
    o3, l3 = oracle.forward(w)
    np.testing.assert_allclose(o3[:T], o1[:T], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l3[:T], l1[:T], rtol=1e-12, atol=1e-14)


def test_rows_entry_matches_forward():
    w = wl.random_small(25, max_seqs=4, window=7)
    o, l = oracle.forward(w)
    T = w.valid_tokens()
    toks = np.repeat(np.arange(w.cfg.num_q_tokens), w.cfg.num_q_heads)
    heads = np.tile(np.arange(w.cfg.num_q_heads), w.cfg.num_q_tokens)
    o2, l2, st = oracle.rows(w, toks, heads)
    assert np.all(st[: T * w.cfg.num_q_heads] == 0) and np.all(st[T * w.cfg.num_q_heads:] == 1)
    n = T * w.cfg.num_q_heads
    assert np.array_equal(o2[:n], o[:T].reshape(n, -1)) and np.array_equal(l2[:n], l[:T].reshape(n))


def test_named_tiny_workload_shape_and_finiteness():
    w = wl.named(1)
    assert w.cfg.num_q_tokens == 22 and list(w.cu_q_lens) == [0, 1, 6, 22]
    assert w.cfg.total_num_pages == 32 and w.page_indices.shape == (3, 4)
    o, l = oracle.forward(w)
    assert np.isfinite(o).all() and np.isfinite(l).all()


# ----------------------------------------------------------------------------- attention sinks

def test_sinks_zero_q_closed_form():
    """Q = 0: every visible score is 0, so out = mean(V) * n / (n + e^sink) and
    lse = log(n + e^sink)."""
    w = _zero_q(wl.with_sinks(wl.random_small(5, max_seqs=4, causal=True, max_q=12, max_extra_kv=40), 5))
    out, lse = oracle.forward(w)
    G = w.cfg.num_q_heads // w.cfg.num_kv_heads
    for s in range(w.n_seqs):
        q0 = int(w.cu_q_lens[s]); ql = int(w.cu_q_lens[s + 1]) - q0; kvl = int(w.kv_lens[s])
        v = _seq_kv(w, s, 1)
        for i in range(ql):
            n_vis = kvl - ql + i + 1
            for n in range(w.cfg.num_q_heads):
                sk = float(w.sinks[n])
                want = v[n // G, :n_vis].mean(axis=0) * n_vis / (n_vis + math.exp(sk))
                np.testing.assert_allclose(out[q0 + i, n], want, rtol=1e-12, atol=1e-15)
                assert lse[q0 + i, n] == pytest.approx(np.logaddexp(math.log(n_vis), sk), rel=1e-13, abs=1e-13)


def test_sinks_single_visible_key():
    """Window 1: one visible key with score x, so out = V * sigmoid(x - sink)
    and lse = logaddexp(x, sink)."""
    w = wl.with_sinks(wl.random_small(8, max_seqs=4, window=1, causal=True), 8)
    out, lse = oracle.forward(w)
    G = w.cfg.num_q_heads // w.cfg.num_kv_heads
    q = _q_f64(w)
    for s in range(w.n_seqs):
        q0 = int(w.cu_q_lens[s]); ql = int(w.cu_q_lens[s + 1]) - q0; kvl = int(w.kv_lens[s])
        k = _seq_kv(w, s, 0); v = _seq_kv(w, s, 1)
        for i in range(ql):
            p = kvl - ql + i
            for n in range(w.cfg.num_q_heads):
                x = float(np.dot(q[q0 + i, n], k[n // G, p])) * w.cfg.sm_scale
                sk = float(w.sinks[n])
                np.testing.assert_allclose(out[q0 + i, n], v[n // G, p] / (1.0 + math.exp(sk - x)),
                                           rtol=1e-12, atol=1e-15)
                assert lse[q0 + i, n] == pytest.approx(np.logaddexp(x, sk), rel=1e-13, abs=1e-13)


@pytest.mark.parametrize("kv_dtype,cap", [(wl.KV_BF16, None), (wl.KV_FP8, 30.0)])
def test_sinks_logsumexp_identity(kv_dtype, cap):
    """With a sink the row is the same softmax over one more logit that carries
    no value: lse' = logaddexp(lse, sink) and out' = out * e^(lse - lse')."""
    base = wl.random_small(14, max_seqs=4, causal=True, kv_dtype=kv_dtype, soft_cap=cap, max_q=16)
    o0, l0 = oracle.forward(base)
    w = wl.with_sinks(wl.random_small(14, max_seqs=4, causal=True, kv_dtype=kv_dtype, soft_cap=cap, max_q=16),
                      14, mean=0.0, std=3.0)
    o1, l1 = oracle.forward(w)
    T = w.valid_tokens()
    sk = w.sinks.astype(np.float64)[None, :]
    l_want = np.logaddexp(l0[:T], sk)
    np.testing.assert_allclose(l1[:T], l_want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(o1[:T], o0[:T] * np.exp(l0[:T] - l_want)[..., None], rtol=1e-12, atol=1e-15)


def test_sinks_at_minus_infinity_change_nothing():
    base = wl.random_small(16, max_seqs=4, causal=True)
    o0, l0 = oracle.forward(base)
    w = wl.random_small(16, max_seqs=4, causal=True)
    w.sinks = np.full(w.cfg.num_q_heads, -np.inf, dtype=np.float32)
    o1, l1 = oracle.forward(w)
    T = w.valid_tokens()
    assert np.array_equal(o0[:T], o1[:T]) and np.array_equal(l0[:T], l1[:T])
