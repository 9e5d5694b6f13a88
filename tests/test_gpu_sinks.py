"""Attention sinks on the GPU (rpa_forward_sinks) against the oracle.

One logit per q head joins each row's softmax and carries no value (the
spatial-compiler page's `flat_softmax_rows_at` with `sinks`). A whole row takes
its sink where it is normalised; split rows take it once, in the merge. The
cases cover both kernel classes, fp8 K/V, the soft-cap, windows, split-KV
merges in both classes, and sinks that dominate the row.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import Device, assert_parity, run_numpy

pytestmark = pytest.mark.gpu

from test_gpu_parity import MEDIUM, SMALL, _medium  # noqa: E402


def _compare(w, what):
    out, lse = run_numpy(w)
    ref_out, ref_lse = oracle.forward(w)
    T = w.valid_tokens()
    assert_parity(out[:T], lse[:T], ref_out[:T], ref_lse[:T], what)


@pytest.mark.parametrize("seed,D,kvd,causal,window,cap,G,page", SMALL[:10])
def test_sinks_small_random(seed, D, kvd, causal, window, cap, G, page):
    w = wl.random_small(seed, max_seqs=5, head_dim=D, kv_dtype=kvd, causal=causal, window=window,
                        soft_cap=cap, G=G, page_size=page, max_q=40, max_extra_kv=120)
    _compare(wl.with_sinks(w, seed), f"sinks small seed {seed}")


@pytest.mark.parametrize("case", MEDIUM[:5], ids=[c["name"] for c in MEDIUM[:5]])
def test_sinks_split_kv(case):
    """Split units: the sink joins the merge, once, not the chunks' partials."""
    _compare(wl.with_sinks(_medium(case), 7), case["name"] + " sinks")


@pytest.mark.parametrize("case", [MEDIUM[0], MEDIUM[1]], ids=["dec", "pf"])
def test_sinks_dominant(case):
    """Sinks well above every score: the rows shrink towards 0 and the LSE
    follows the sink."""
    w = wl.with_sinks(_medium(case, q_mult=4.0), 9, mean=12.0, std=2.0)
    _compare(w, case["name"] + " dominant sinks")


def test_sinks_at_minus_infinity_equal_plain_forward():
    w = wl.random_small(23, max_seqs=5, head_dim=128, max_q=30, max_extra_kv=200)
    d = Device(w)
    out0, lse0 = d.run()
    d.sinks = torch.full((w.cfg.num_q_heads,), -float("inf"), dtype=torch.float32, device="cuda")
    out1, lse1 = d.run()
    T = w.valid_tokens()
    assert torch.equal(out0[:T], out1[:T]) and torch.equal(lse0[:T], lse1[:T])
