"""rpa_forward on several streams, from several threads and under graph
capture (needs an MI355X).

Each call enqueues its launches on the caller's stream only, with no state
kept between calls but the workspace the caller passes. These tests check
that results do not depend on what else is in flight: calls on two streams
of one thread, calls from two threads, and a captured call replayed several
times with other work between the replays. The kernels are deterministic for
a given batch, so results are compared bit for bit, and a sample of rows
against the oracle.
"""

import threading

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_gqa_amd as rpa
import workloads as wl
from gpu_util import Device, assert_parity, sample_rows

pytestmark = pytest.mark.gpu


def _mixed(seed, head_dim, G=4, Hkv=4):
    # prefill chunks with prior context beside many decode sequences
    rng = np.random.Generator(np.random.PCG64(seed))
    n_pf, n_dec = 4, 64
    prior = rng.integers(0, 3000, size=n_pf)
    q_lens = np.concatenate([np.full(n_pf, 160), np.ones(n_dec, np.int64)])
    kv_lens = np.concatenate([prior + 160, rng.integers(1000, 6000, size=n_dec, endpoint=True)])
    page = 16
    kw = dict(num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=head_dim, page_size=page,
              pages_per_seq=int((kv_lens.max() + page - 1) // page), sm_scale=1.0 / np.sqrt(head_dim))
    return wl.build(f"streams{seed}", kw, q_lens, kv_lens, seed, rng=rng)


def _forward(d, stream=None):
    # out and lse are made on the stream the call runs on
    with torch.cuda.stream(stream or torch.cuda.current_stream()):
        return rpa.forward(d.q, d.kv, d.kv_lens, d.page_indices, d.cu_q_lens, d.num_seqs, d.cfg,
                           workspace=d.workspace, stream=stream)


def _same(a, b, n, what):
    """the rows of the n valid tokens, bit for bit"""
    (oa, la), (ob, lb) = a, b
    assert torch.equal(oa[:n].view(torch.int16), ob[:n].view(torch.int16)), what
    assert torch.equal(la[:n], lb[:n]), what


def _oracle_sample(w, out, lse, what):
    tokens, heads = sample_rows(w, n_random=96)
    t = torch.from_numpy(tokens).cuda()
    h = torch.from_numpy(heads).cuda()
    ref_o, ref_l, st = oracle.rows(w, tokens, heads)
    assert np.all(st == 0)
    assert_parity(out[t, h].float().cpu().numpy(), lse[t, h].cpu().numpy(), ref_o, ref_l, what)


def test_calls_on_two_streams_of_one_thread():
    wa, wb = _mixed(31, 128), _mixed(32, 64)
    da, db = Device(wa), Device(wb)
    print("[streams] references, one call at a time", flush=True)
    ref_a = tuple(x.clone() for x in da.run())
    ref_b = tuple(x.clone() for x in db.run())
    _oracle_sample(wa, *ref_a, "head_dim 128 batch vs oracle")
    _oracle_sample(wb, *ref_b, "head_dim 64 batch vs oracle")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    print("[streams] two streams, back to back", flush=True)
    got = []
    for _ in range(2):
        got.append((_forward(da, sa), _forward(db, sb)))
    torch.cuda.synchronize()
    for a, b in got:
        _same(a, ref_a, wa.valid_tokens(), "stream a")
        _same(b, ref_b, wb.valid_tokens(), "stream b")


def test_calls_from_two_threads():
    ws = [_mixed(41, 128), _mixed(42, 128, G=8, Hkv=2)]
    ds = [Device(w) for w in ws]
    print("[streams] references", flush=True)
    refs = [tuple(x.clone() for x in d.run()) for d in ds]
    results = [[], []]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.default_stream())
            for _ in range(3):
                results[i].append(_forward(ds[i], s))
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    print("[streams] two threads, three calls each", flush=True)
    th = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        assert len(results[i]) == 3
        for r in results[i]:
            _same(r, refs[i], ws[i].valid_tokens(), f"thread {i}")


def test_graph_capture_replays():
    w = _mixed(51, 128)
    d = Device(w)
    c = d.cfg
    T, Hq, D = c.num_q_tokens, c.num_q_heads, c.head_dim
    n = w.valid_tokens()
    print("[streams] eager reference", flush=True)
    ref = tuple(x.clone() for x in d.run())
    _oracle_sample(w, *ref, "eager vs oracle")
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        rpa.forward(d.q, d.kv, d.kv_lens, d.page_indices, d.cu_q_lens, d.num_seqs, c, out=out, lse=lse,
                    workspace=d.workspace, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    print("[streams] capture", flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rpa.forward(d.q, d.kv, d.kv_lens, d.page_indices, d.cu_q_lens, d.num_seqs, c, out=out, lse=lse,
                    workspace=d.workspace)
    torch.cuda.synchronize()
    for i in range(3):
        print(f"[streams] replay {i}", flush=True)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        _forward(d)  # an eager call between the replays, on the same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same((out, lse), ref, n, f"replay {i}")
