"""Parity at the full sizes of the named workloads, in the launch
configuration the benchmark times (needs an MI355X).

The oracle computes the compared rows one by one; every case also runs on a
sharpened copy (Q x 8, exact in bf16) that makes the softmax peaky, so that
|out| ~ 1 and the absolute tolerance cannot hide an error:

* decode batch and fp8 decode: every row (all q heads of every token);
* mixed batch: every row of the 56 decode sequences and of two whole
  448-token prefill chunks (sharpened: the decode rows and one chunk);
* long context: all q heads of 128 seeded random tokens, and every row of two
  whole 128-token sequences, the longest and the shortest context (sharpened:
  all q heads of the first and last token of two sequences and 192 random
  (token, head) pairs);
* attention sinks at full size: the decode batch with seeded sinks, every row.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import Device, assert_parity

pytestmark = pytest.mark.gpu


def _all_heads(w, tokens):
    tokens = np.asarray(tokens, dtype=np.int64)
    Hq = w.cfg.num_q_heads
    return np.repeat(tokens, Hq), np.tile(np.arange(Hq), len(tokens))


def _seq_tokens(w, s):
    return np.arange(int(w.cu_q_lens[s]), int(w.cu_q_lens[s + 1]))


def _check_rows(w, d, tokens, heads, what):
    print(f"[workload] {what}: running GPU", flush=True)
    out, lse = d.run()
    t = torch.from_numpy(np.asarray(tokens)).cuda()
    h = torch.from_numpy(np.asarray(heads)).cuda()
    got_o = out[t, h].float().cpu().numpy()
    got_l = lse[t, h].cpu().numpy()
    print(f"[workload] {what}: oracle on {len(tokens)} rows", flush=True)
    ref_o, ref_l, st = oracle.rows(w, tokens, heads)
    assert np.all(st == 0)
    stats = assert_parity(got_o, got_l, ref_o, ref_l, what)
    print(f"[workload] {what}: ok {stats}", flush=True)


def _sharpen(w, d):
    w.q = wl.to_bf16_bits(wl.bf16_bits_to_f32(w.q) * 8.0)
    d.q = torch.from_numpy(w.q.view(np.int16)).cuda().view(torch.bfloat16)


def _done(d):
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("number", [2, 4])
def test_decode_workload_every_row(number):
    print(f"[workload] cfg{number}: generating", flush=True)
    w = wl.named(number)
    d = Device(w)
    tokens, heads = _all_heads(w, np.arange(w.valid_tokens()))
    _check_rows(w, d, tokens, heads, f"cfg{number} every row")
    _sharpen(w, d)
    _check_rows(w, d, tokens, heads, f"cfg{number} x8 every row")
    _done(d)


def test_mixed_workload_decode_sequences_and_two_prefill_chunks():
    print("[workload] cfg3: generating", flush=True)
    w = wl.named(3)
    d = Device(w)
    q_lens = w.q_lens()
    prefill = [s for s in range(w.n_seqs) if q_lens[s] > 1]
    decode = [s for s in range(w.n_seqs) if q_lens[s] == 1]
    assert len(prefill) == 8 and len(decode) == 56
    dec_tokens = np.concatenate([_seq_tokens(w, s) for s in decode])
    # the chunks with the shortest and the longest prior context
    prior = [int(w.kv_lens[s]) - int(q_lens[s]) for s in prefill]
    chunks = [prefill[int(np.argmin(prior))], prefill[int(np.argmax(prior))]]
    tokens, heads = _all_heads(w, np.concatenate([dec_tokens] + [_seq_tokens(w, s) for s in chunks]))
    _check_rows(w, d, tokens, heads, "cfg3 decode sequences + two prefill chunks")
    _sharpen(w, d)
    tokens, heads = _all_heads(w, np.concatenate([dec_tokens, _seq_tokens(w, chunks[1])]))
    _check_rows(w, d, tokens, heads, "cfg3 x8 decode sequences + one prefill chunk")
    _done(d)


def test_long_context_random_tokens_all_heads():
    print("[workload] cfg5: generating", flush=True)
    w = wl.named(5)
    d = Device(w)
    rng = np.random.default_rng(5)
    tokens, heads = _all_heads(w, np.sort(rng.choice(w.valid_tokens(), size=128, replace=False)))
    _check_rows(w, d, tokens, heads, "cfg5 all heads of 128 random tokens")
    # the sequence with the shortest context, whole
    s = int(np.argmin(w.kv_lens[:w.n_seqs]))
    tokens, heads = _all_heads(w, _seq_tokens(w, s))
    _check_rows(w, d, tokens, heads, f"cfg5 every row of sequence {s}")
    _done(d)


def test_long_context_whole_sequence_and_sharpened_sample():
    print("[workload] cfg5: generating", flush=True)
    w = wl.named(5)
    d = Device(w)
    # the sequence with the longest context: its rows span the most chunks
    s = int(np.argmax(w.kv_lens[:w.n_seqs]))
    tokens, heads = _all_heads(w, _seq_tokens(w, s))
    _check_rows(w, d, tokens, heads, f"cfg5 every row of sequence {s}")
    _sharpen(w, d)
    rng = np.random.default_rng(0)
    mid = w.n_seqs // 2
    ends = [int(w.cu_q_lens[0]), w.valid_tokens() - 1, int(w.cu_q_lens[mid]), int(w.cu_q_lens[mid + 1]) - 1]
    t0, h0 = _all_heads(w, ends)
    rt = rng.integers(0, w.valid_tokens(), size=192)
    rh = rng.integers(0, w.cfg.num_q_heads, size=192)
    _check_rows(w, d, np.concatenate([t0, rt]), np.concatenate([h0, rh]), "cfg5 x8 sample")
    _done(d)


def test_decode_workload_with_sinks_every_row():
    print("[workload] cfg2 + sinks: generating", flush=True)
    w = wl.with_sinks(wl.named(2), 2)
    d = Device(w)
    tokens, heads = _all_heads(w, np.arange(w.valid_tokens()))
    _check_rows(w, d, tokens, heads, "cfg2 with sinks every row")
    _done(d)
