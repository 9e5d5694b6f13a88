"""Exact checks of the planning kernel's tile list (needs an MI355X).

The plan is copied back from the workspace and checked against the metadata,
with no second implementation of the planner: every packed query row of every
sequence is owned by exactly one unit of the right class, each unit's key range
covers exactly the keys its rows can see (rounded down to 16 at the start),
the items of each prefill unit tile that range in chunks with no gap or
overlap, and the decode sequence table carries each decode sequence once, in
order, with its block count and stream-K position.
"""

import numpy as np
import pytest
import torch

import ragged_paged_gqa_amd as rpa
import workloads as wl
from gpu_util import lib_config

pytestmark = pytest.mark.gpu


def _plan(w):
    cfg = lib_config(w)
    ws = rpa.plan(torch.from_numpy(w.kv_lens).cuda(), torch.from_numpy(w.cu_q_lens).cuda(),
                  torch.from_numpy(w.num_seqs).cuda(), cfg)
    torch.cuda.synchronize()
    offs, lim = rpa.plan_layout(cfg)
    host = ws.cpu().numpy()
    hdr = host[offs[0]:offs[0] + 256].view(np.int32)
    n_du, n_pu, n_ds, n_pi, _, pch = (int(x) for x in hdr[:6])
    # decode sequence records: seq, q0, ql, kvl, lo16, hi, blk0, nb
    ds = host[offs[1]:offs[1] + 32 * n_ds].view(np.int32).reshape(n_ds, 8)
    pu = host[offs[2]:offs[2] + 32 * n_pu].view(np.int32).reshape(n_pu, 8)
    pi = host[offs[4]:offs[4] + 8 * n_pi].view(np.int32).reshape(n_pi, 2)
    qbase, qcount, qnext = hdr[16:24].copy(), hdr[24:32].copy(), hdr[32:40].copy()
    ql = host[offs[5]:offs[5] + 4 * 8 * int(lim[3])].view(np.int32)
    return dict(n_du=n_du, ds=ds, pu=pu, pi=pi, pch=pch, lim=lim, qbase=qbase, qcount=qcount, qnext=qnext,
                qlist=ql, W=int(lim[6]), dec_blocks=int(hdr[7]), W_used=int(hdr[8]))


def _visible_range(c, G, kvl, ql, r0, nr):
    """[lo rounded down to 16, hi): the keys rows r0 .. r0 + nr - 1 of a
    sequence can see, from the causal and window rules."""
    firsts, lasts = [], []
    for r in range(r0, r0 + nr):
        p = kvl - ql + r // G
        last = p if c.is_causal else kvl - 1
        first = max(0, p - c.sliding_window + 1) if c.sliding_window else 0
        firsts.append(first)
        lasts.append(min(last, kvl - 1))
    return (min(firsts) // 16) * 16, max(lasts) + 1


def _check_decode(P, w, owner):
    """One record per decode sequence, in sequence order, with the metadata,
    the visible key range of all its rows, its 16-key block count and the
    exclusive scan of Hkv * blocks; the header's stream-K totals. Then the
    split itself (start(w) = floor(Tb * w / W)): every wave's range holds at
    most one part that continues a unit from the previous range and at most
    one first part of a unit that runs on, so the two partial slots of a
    wave are never shared."""
    c = w.cfg
    G = c.num_q_heads // c.num_kv_heads
    Hkv = c.num_kv_heads
    cap = c.pages_per_seq * c.page_size
    # keys per stream-K block: 32 for one-byte K/V, else 16
    bk = 32 if wl.is_fp8(c.kv_dtype) else 16
    dec = [s for s in range(int(w.num_seqs[0]))
           if 0 < int(w.cu_q_lens[s + 1]) - int(w.cu_q_lens[s]) and
           (int(w.cu_q_lens[s + 1]) - int(w.cu_q_lens[s])) * G <= P["lim"][4]]
    ds = P["ds"]
    assert len(ds) == len(dec) and P["n_du"] == len(dec) * Hkv
    blk = 0
    for k, s in enumerate(dec):
        q0 = int(w.cu_q_lens[s]); ql = int(w.cu_q_lens[s + 1]) - q0; kvl = min(int(w.kv_lens[s]), cap)
        lo, hi = _visible_range(c, G, kvl, ql, 0, ql * G)
        nb = -(-max(hi - lo, 0) // bk)
        assert tuple(int(x) for x in ds[k]) == (s, q0, ql, kvl, lo, hi, blk, nb), (k, s)
        blk += Hkv * nb
        for h in range(Hkv):
            for r in range(ql * G):
                assert (s, h, r) not in owner
                owner[(s, h, r)] = "dec"
    Tb, W = P["dec_blocks"], P["W"]
    assert Tb == blk
    Wu = P["W_used"]
    c = w.cfg
    two_group = (c.head_dim == 256 and c.kv_dtype in (wl.KV_BF16, wl.KV_F16)
                 and c.q_dtype in (wl.Q_BF16, wl.Q_F16))
    if two_group:
        # the decode class has a launch of its own: all its waves get work
        assert Wu == max(1, min(W, Tb))
    else:
        # one launch holds both classes: the decode work may go to fewer
        # whole workgroups (4 waves each) than the launch has
        assert 1 <= Wu <= max(1, min(W, Tb)) and (Wu == max(1, min(W, Tb)) or Wu % 4 == 0)
    if Tb == 0:
        return
    starts = (Tb * np.arange(Wu + 1, dtype=np.int64)) // Wu
    assert np.all(np.diff(starts) >= 1)
    unit_b0 = np.array([int(r[6]) + h * int(r[7]) for r in ds for h in range(Hkv)], np.int64)
    unit_nb = np.array([int(r[7]) for r in ds for h in range(Hkv)], np.int64)
    for wv in range(Wu):
        a, b = starts[wv], starts[wv + 1]
        inside = (unit_b0 < b) & (unit_b0 + unit_nb > a)
        cont = inside & (unit_b0 < a)
        first_split = inside & (unit_b0 >= a) & (unit_b0 + unit_nb > b)
        assert cont.sum() <= 1 and first_split.sum() <= 1
        assert unit_nb[inside].sum() >= 1


def _check_queues(P, n_kv_heads):
    """Each prefill item sits in exactly one of the 8 queues, the one of its
    (sequence, kv head); queue x starts at x * max_pf_items and starts empty;
    within a queue, one (sequence, kv head)'s items come chunk-major."""
    n_pi = len(P["pi"])
    max_pi = P["lim"][3]
    assert np.all(P["qnext"] == 0)
    assert int(P["qcount"].sum()) == n_pi
    assert np.all(P["qbase"] == np.arange(8) * max_pi)
    entries = []
    for x in range(8):
        q = P["qlist"][x * max_pi:x * max_pi + int(P["qcount"][x])]
        entries.append(q)
        last = {}
        for it in q:
            ui, c = P["pi"][it]
            s, h, r0 = P["pu"][ui][:3]
            assert (s * n_kv_heads + h) % 8 == x
            key = (c, r0)
            if (s, h) in last:
                assert key > last[(s, h)]
            last[(s, h)] = key
    allq = np.concatenate(entries) if entries else np.zeros(0, np.int32)
    assert np.array_equal(np.sort(allq), np.arange(n_pi))
    # within a queue the sequences come heaviest first (the visible keys of
    # their units of one kv head; ties by sequence index) while the plan has
    # one tile of sequences
    work = {}
    for s_, h_, r0_, nr_, lo_, hi_, nch_, it0_ in P["pu"]:
        if h_ == 0:
            work[int(s_)] = work.get(int(s_), 0) + max(int(hi_) - int(lo_), 0)
    if len(P["pu"]) and max(work) < 512:
        for q in entries:
            order = []
            for it in q:
                s_ = int(P["pu"][P["pi"][it][0]][0])
                if not order or order[-1] != s_:
                    order.append(s_)
            keys = [(-work[s_], s_) for s_ in order]
            assert keys == sorted(keys)


def _check(w):
    P = _plan(w)
    c = w.cfg
    G = c.num_q_heads // c.num_kv_heads
    dec_rows, pf_rows, ch = P["lim"][4], P["lim"][5], P["pch"]
    owner = {}
    _check_decode(P, w, owner)
    units, items = P["pu"], P["pi"]
    seen_items = np.zeros(len(items), dtype=int)
    for ui, (s, h, r0, nr, lo, hi, nch, it0) in enumerate(units):
        q0 = int(w.cu_q_lens[s]); ql = int(w.cu_q_lens[s + 1]) - q0; kvl = int(w.kv_lens[s])
        assert ql * G > dec_rows
        assert 1 <= nr <= pf_rows
        for r in range(r0, r0 + nr):
            assert (s, h, r) not in owner
            owner[(s, h, r)] = "pf"
        assert (lo, hi) == _visible_range(c, G, kvl, ql, r0, nr)
        # items tile [lo, hi) exactly
        assert nch == max(1, -(-(hi - lo) // ch))
        for k in range(nch):
            seen_items[it0 + k] += 1
            assert tuple(items[it0 + k]) == (ui, k)
            a, b = lo + k * ch, min(hi, lo + (k + 1) * ch)
            assert a < b or (nch == 1 and hi <= lo)
    assert np.all(seen_items == 1)
    _check_queues(P, c.num_kv_heads)
    for s in range(w.n_seqs):
        ql = int(w.cu_q_lens[s + 1]) - int(w.cu_q_lens[s])
        for h in range(c.num_kv_heads):
            for r in range(ql * G):
                assert (s, h, r) in owner


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_plan_small(seed):
    _check(wl.random_small(seed, max_seqs=6, max_q=50, max_extra_kv=3000, window=None if seed != 2 else 300))


def test_plan_named_tiny():
    _check(wl.named(1))


@pytest.mark.parametrize("number", [2, 3, 4, 5])
def test_plan_named_lengths(number):
    # lengths of the large workloads, with a 1-page cache: the plan reads metadata only
    rng = np.random.Generator(np.random.PCG64(number))
    q_lens, kv_lens = wl.lengths(number, rng)
    kw = dict(wl.cfg_kw(number))
    page = kw["page_size"]
    S = len(q_lens)
    pps = kw["pages_per_seq"]
    cfg = wl.Config(total_num_pages=1, max_num_seqs=S, num_q_tokens=int(np.sum(q_lens)),
                    **{k: v for k, v in kw.items() if k != "pages_per_seq"}, pages_per_seq=pps)
    cu = np.zeros(S + 1, np.int32)
    cu[1:] = np.cumsum(q_lens)
    w = wl.Workload("lens", cfg, np.zeros((1, 1, 1), np.uint16), np.zeros((1,), np.uint16),
                    np.asarray(kv_lens, np.int32), np.zeros((S, pps), np.int32), cu, np.array([S], np.int32))
    _check(w)
    _ = page
