"""Exact checks of the planning kernel's tile list (needs an MI355X).

The plan is copied back from the workspace and checked against the metadata,
with no second implementation of the planner: every packed query row of every
sequence is owned by exactly one unit of the right class, each unit's key range
covers exactly the keys its rows can see (rounded down to 16 at the start),
and the items of each unit tile that range in chunks with no gap or overlap.
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
    n_du, n_pu, n_di, n_pi, dch, pch = (int(x) for x in hdr[:6])
    du = host[offs[1]:offs[1] + 32 * n_du].view(np.int32).reshape(n_du, 8)
    pu = host[offs[2]:offs[2] + 32 * n_pu].view(np.int32).reshape(n_pu, 8)
    # decode items are full descriptors: seq, kv_head, c_lo, c_hi, kvl, q0, ql,
    # row0, nrows, nch, unit, chunk, 4 x pad
    di = host[offs[3]:offs[3] + 64 * n_di].view(np.int32).reshape(n_di, 16)
    pi = host[offs[4]:offs[4] + 8 * n_pi].view(np.int32).reshape(n_pi, 2)
    qbase, qcount, qnext = hdr[16:24].copy(), hdr[24:32].copy(), hdr[32:40].copy()
    ql = host[offs[5]:offs[5] + 4 * 8 * int(lim[3])].view(np.int32)
    W = int(lim[6])
    wfirst = host[offs[6]:offs[6] + 4 * W].view(np.int32)
    return dict(du=du, pu=pu, di=di, pi=pi, dch=dch, pch=pch, lim=lim, qbase=qbase, qcount=qcount,
                qnext=qnext, qlist=ql, W=W, wfirst=wfirst, dec_blocks=int(hdr[7]), W_used=int(hdr[8]))


def _check_stream_k(P):
    """Decode items run in stream-K order: the units' 16-key blocks laid end
    to end are split into W equal contiguous ranges; each wave's items are
    consecutive, cover exactly its range and start at wfirst[wave]."""
    di, W, Tb, Wu = P["di"], P["W"], P["dec_blocks"], P["W_used"]
    assert Wu == max(1, min(W, Tb))
    waves = di[:, 12]
    assert np.all(np.diff(waves) >= 0)
    assert np.all((waves >= 0) & (waves < Wu))
    blocks = np.zeros(Wu, np.int64)
    for d in di:
        blocks[d[12]] += -(-(int(d[3]) - int(d[2])) // 16)
    starts = (Tb * np.arange(Wu + 1, dtype=np.int64)) // Wu
    assert np.array_equal(blocks, np.diff(starts))
    for w in range(W):
        idx = np.nonzero(waves == w)[0]
        if len(idx) == 0:
            assert P["wfirst"][w] == np.iinfo(np.int32).max
        else:
            assert P["wfirst"][w] == idx[0]
            assert np.array_equal(idx, np.arange(idx[0], idx[0] + len(idx)))


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


def _check(w):
    P = _plan(w)
    c = w.cfg
    G = c.num_q_heads // c.num_kv_heads
    dec_rows, pf_rows = P["lim"][4], P["lim"][5]
    owner = {}
    for cls, units, items, ch in (("dec", P["du"], P["di"], P["dch"]), ("pf", P["pu"], P["pi"], P["pch"])):
        seen_items = np.zeros(len(items), dtype=int)
        for ui, (s, h, r0, nr, lo, hi, nch, it0) in enumerate(units):
            q0 = int(w.cu_q_lens[s]); ql = int(w.cu_q_lens[s + 1]) - q0; kvl = int(w.kv_lens[s])
            rows = ql * G
            assert (rows <= dec_rows) == (cls == "dec")
            assert 1 <= nr <= (dec_rows if cls == "dec" else pf_rows)
            for r in range(r0, r0 + nr):
                assert (s, h, r) not in owner
                owner[(s, h, r)] = cls
            # visible key range of the unit's rows
            firsts, lasts = [], []
            for r in range(r0, r0 + nr):
                p = kvl - ql + r // G
                last = p if c.is_causal else kvl - 1
                first = max(0, p - c.sliding_window + 1) if c.sliding_window else 0
                firsts.append(first); lasts.append(min(last, kvl - 1))
            assert lo == (min(firsts) // 16) * 16
            assert hi == max(lasts) + 1
            # items tile [lo, hi) exactly (a decode unit with no key has none)
            if cls == "pf":
                assert nch == max(1, -(-(hi - lo) // ch))
            else:
                assert nch >= (1 if hi > lo else 0) and (nch == 0) == (hi <= lo)
            for k in range(nch):
                seen_items[it0 + k] += 1
                if cls == "pf":
                    assert tuple(items[it0 + k]) == (ui, k)
                    a, b = lo + k * ch, min(hi, lo + (k + 1) * ch)
                    assert a < b or (nch == 1 and hi <= lo)
                    continue
                d = items[it0 + k]
                assert (d[10], d[11]) == (ui, k)
                assert (d[0], d[1], d[7], d[8], d[9]) == (s, h, r0, nr, nch)
                assert (d[4], d[5], d[6]) == (kvl, q0, ql)
                # consecutive, 16-aligned boundaries, on consecutive waves
                a, b = int(d[2]), int(d[3])
                assert a == (lo if k == 0 else int(items[it0 + k - 1][3]))
                assert (a - lo) % 16 == 0 and (b == max(hi, lo) if k == nch - 1 else (b - lo) % 16 == 0)
                assert a < b
                if k > 0:
                    assert d[12] == items[it0 + k - 1][12] + 1
        assert np.all(seen_items == 1), cls
    _check_queues(P, c.num_kv_heads)
    _check_stream_k(P)
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


@pytest.mark.parametrize("number", [2, 3, 5])
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
