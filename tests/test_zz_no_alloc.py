"""rpa_forward_noalloc, the entry point for callers that cannot allocate
(needs an MI355X): called through the C ABI twice in a row, the second time
on a smaller batch, each result checked against rpa_forward_sinks on the
same inputs (bit for bit, and at the parity bar) and against the oracle; a
configuration whose workspace exceeds the scratch array is refused before
anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import ragged_paged_gqa_amd as rpa
import workloads as wl
from gpu_util import Device, assert_parity

pytestmark = pytest.mark.gpu


def _split_batch():
    # prefill-class rows with long KV (split chunks, merged by the last
    # finisher) beside decode-class rows with long KV (split, merged by the
    # combine kernel), with attention sinks
    kw = dict(num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=32, pages_per_seq=None, sm_scale=0.088)
    q_lens, kv_lens = [40, 1, 70, 1, 2], [20000, 3000, 900, 257, 1900]
    pages = sum((k + 31) // 32 for k in kv_lens)
    w = wl.build("noalloc-split", kw, q_lens, kv_lens, 77, total_num_pages=pages + 3, max_num_seqs=6,
                 num_q_tokens=sum(q_lens) + 2)
    return wl.with_sinks(w, 77)


def _noalloc(d):
    c = d.cfg
    out = torch.full((c.num_q_tokens, c.num_q_heads, c.head_dim), float("nan"), dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((c.num_q_tokens, c.num_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    rpa.forward_noalloc(d.q, d.kv, d.kv_lens, d.page_indices, d.cu_q_lens, d.num_seqs, c, out=out, lse=lse,
                        sinks=d.sinks)
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    for w in (_split_batch(), wl.named(1)):  # the second batch is the smaller one
        print(f"[noalloc] {w.name}", flush=True)
        d = Device(w)
        ref_out, ref_lse = d.run()  # rpa_forward / rpa_forward_sinks with a torch workspace
        out, lse = _noalloc(d)
        T = w.valid_tokens()
        assert torch.equal(out[:T].view(torch.int16), ref_out[:T].view(torch.int16)), w.name
        assert torch.equal(lse[:T], ref_lse[:T]), w.name
        assert_parity(out[:T].float().cpu().numpy(), lse[:T].cpu().numpy(), ref_out[:T].float().cpu().numpy(),
                      ref_lse[:T].cpu().numpy(), f"{w.name} vs workspace entry point")
        o_out, o_lse = oracle.forward(w)
        assert_parity(out[:T].float().cpu().numpy(), lse[:T].cpu().numpy(), o_out[:T], o_lse[:T],
                      f"{w.name} vs oracle")


def test_noalloc_refuses_a_workspace_beyond_its_array():
    # the long-context workload's shapes need more than the 256 MiB array; the
    # call must return "workspace too small" without touching the pointers
    w = wl.named(1)
    d = Device(w)
    cfg = rpa.Config(num_q_tokens=2048, num_q_heads=32, num_kv_heads=2, head_dim=256, total_num_pages=24576,
                     page_size=64, max_num_seqs=16, pages_per_seq=2048, sm_scale=1 / 16)
    assert rpa.workspace_bytes(cfg) > rpa.NOALLOC_SCRATCH_BYTES
    c = cfg.to_c()
    p = d.q.data_ptr()
    st = rpa.lib().rpa_forward_noalloc(ctypes.byref(c), p, p, p, p, p, p, None, p, None, None)
    assert st == 3
    torch.cuda.synchronize()
