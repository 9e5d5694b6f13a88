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
    # item records: unit, chunk, the unit's record (8 ints), q0, ql, kvl, 3 pad
    pi = host[offs[4]:offs[4] + 64 * n_pi].view(np.int32).reshape(n_pi, 16)
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


def _snake(g):
    r, k = divmod(g, 8)
    return 7 - k if r & 1 else k


def _check_queues(P, n_kv_heads):
    """The queue lists, entry for entry. Each tile of 512 sequences ranks its
    prefill sequences heaviest first (visible keys of one kv head's units;
    ties by sequence index) and deals its (sequence, kv head) groups to the
    8 queues back and forth: group g = rank * Hkv + h goes to queue 0..7,
    7..0, ... In each queue the tile's entries are every chunk but the units'
    last ones, groups in rank order, then the last chunks, groups by the size
    class of their last chunks (16 * keys // chunk, at most 15; the largest
    over the group's units) larger first, ties by rank; inside a part a
    group's entries are chunk-major (chunk, then row block). Queue x starts
    at x * max_pf_items and starts empty."""
    n_pi = len(P["pi"])
    max_pi = P["lim"][3]
    C = P["pch"]
    assert np.all(P["qnext"] == 0)
    assert int(P["qcount"].sum()) == n_pi
    assert np.all(P["qbase"] == np.arange(8) * max_pi)
    groups = {}
    for ui, (s_, h_, r0_, nr_, lo_, hi_, nch_, it0_) in enumerate(P["pu"]):
        groups.setdefault((int(s_), int(h_)), []).append(
            (int(r0_), int(lo_), int(hi_), int(nch_), int(it0_)))
    seqs = sorted({s_ for s_, _ in groups})
    expect = [[] for _ in range(8)]
    for tile in sorted({s_ // 512 for s_ in seqs}):
        ts = [s_ for s_ in seqs if s_ // 512 == tile]
        work = {s_: sum(max(hi - lo, 0) for _, lo, hi, _, _ in groups[(s_, 0)]) for s_ in ts}
        cls = {s_: max(min(15, 16 * max((hi - lo) - (nch - 1) * C, 0) // C) for _, lo, hi, nch, _ in groups[(s_, 0)])
               for s_ in ts}
        by_work = sorted(ts, key=lambda s_: (-work[s_], s_))
        rank = {s_: r for r, s_ in enumerate(by_work)}
        by_cls = sorted(ts, key=lambda s_: (-cls[s_], rank[s_]))
        part_a = [[] for _ in range(8)]
        part_b = [[] for _ in range(8)]
        for order, part, last in ((by_work, part_a, False), (by_cls, part_b, True)):
            for s_ in order:
                for h in range(n_kv_heads):
                    ents = []
                    for r0, lo, hi, nch, it0 in groups[(s_, h)]:
                        for c in range(nch):
                            if (c == nch - 1) == last:
                                ents.append((c, r0, it0 + c))
                    part[_snake(rank[s_] * n_kv_heads + h)] += [e[2] for e in sorted(ents)]
        for x in range(8):
            expect[x] += part_a[x] + part_b[x]
    entries = []
    for x in range(8):
        q = P["qlist"][x * max_pi:x * max_pi + int(P["qcount"][x])]
        assert list(q) == expect[x], f"queue {x}"
        entries.append(q)
    allq = np.concatenate(entries) if entries else np.zeros(0, np.int32)
    assert np.array_equal(np.sort(allq), np.arange(n_pi))


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
            rec = items[it0 + k]
            assert tuple(rec[:2]) == (ui, k)
            # the copy of the unit's record and of the sequence's metadata
            assert tuple(rec[2:10]) == (s, h, r0, nr, lo, hi, nch, it0)
            assert tuple(rec[10:13]) == (q0, ql, kvl)
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
    # the decode waves given work, by the rule for each workload: the decode
    # batches (2, 4) use half the launch's 4-wave workgroups (two fit on a
    # CU at head_dim 128); the mixed batch (3), whose estimated prefill time
    # is well above half its decode time, a quarter; the long context (5)
    # has no decode work
    P = _plan(w)
    W, Tb, Wu = P["W"], P["dec_blocks"], P["W_used"]
    expect = {2: (W // 8) * 4, 3: (W // 16) * 4, 4: (W // 8) * 4, 5: 1}[number]
    assert Wu == min(expect, max(Tb, 1)), (Wu, expect, Tb)
