"""Shared helpers of the GPU parity tests: upload a seeded workload, run the
HIP path through the C ABI, compare with the oracle at the stated bar."""

from __future__ import annotations

import numpy as np
import torch

import ragged_paged_gqa_amd as rpa
import workloads as wl

# Parity bar: bf16 outputs within |d| <= ATOL + RTOL*|ref| of the f64 oracle,
# per-row LSE within LSE_TOL (natural log units).
ATOL = 2e-2
RTOL = 2e-2
LSE_TOL = 1e-3
# Additional, stricter check on the whole compared set: relative RMS error.
REL_RMS_TOL = 2e-2


def lib_config(w: wl.Workload) -> rpa.Config:
    c = w.cfg
    return rpa.Config(
        num_q_tokens=c.num_q_tokens, num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
        head_dim=c.head_dim, total_num_pages=c.total_num_pages, page_size=c.page_size,
        max_num_seqs=c.max_num_seqs, pages_per_seq=c.pages_per_seq,
        kv_dtype={wl.KV_FP8: rpa.DTYPE_FP8_E4M3FN, wl.KV_E5M2: rpa.DTYPE_FP8_E5M2,
                  wl.KV_F16: rpa.DTYPE_F16, wl.KV_I8: rpa.DTYPE_INT8}.get(c.kv_dtype, rpa.DTYPE_BF16),
        q_dtype={wl.Q_F16: rpa.DTYPE_F16, wl.Q_F32: rpa.DTYPE_F32}.get(c.q_dtype, rpa.DTYPE_BF16),
        sm_scale=c.sm_scale, soft_cap=c.soft_cap or 0.0,
        k_scale=1.0 if c.k_scale is None else c.k_scale,
        v_scale=1.0 if c.v_scale is None else c.v_scale,
        is_causal=c.is_causal, sliding_window=c.sliding_window or 0)


def upload_q_bits(bits: np.ndarray, q_dtype: str, device="cuda") -> torch.Tensor:
    """Bits of the q dtype (workloads.to_q_bits) -> a device tensor of that dtype."""
    if q_dtype == wl.Q_F32:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.float32)).to(device)
    t16 = torch.float16 if q_dtype == wl.Q_F16 else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(t16)


class Device:
    """A workload's inputs resident on the GPU."""

    def __init__(self, w: wl.Workload, device="cuda"):
        self.w = w
        self.cfg = lib_config(w)
        t16 = torch.float16 if w.cfg.q_dtype == wl.Q_F16 else torch.bfloat16
        self.q = upload_q_bits(w.q, w.cfg.q_dtype, device)
        if wl.is_fp8(w.cfg.kv_dtype):
            self.kv = torch.from_numpy(w.kv_pages).to(device)
        else:
            self.kv = torch.from_numpy(w.kv_pages.view(np.int16)).to(device).view(t16)
        self.kv_lens = torch.from_numpy(w.kv_lens).to(device)
        self.page_indices = torch.from_numpy(w.page_indices).to(device)
        self.cu_q_lens = torch.from_numpy(w.cu_q_lens).to(device)
        self.num_seqs = torch.from_numpy(w.num_seqs).to(device)
        self.sinks = None if w.sinks is None else torch.from_numpy(np.ascontiguousarray(w.sinks)).to(device)
        self.workspace = rpa.alloc_workspace(self.cfg)

    def run(self, out=None, lse=None, want_lse=True):
        out, lse = rpa.forward(self.q, self.kv, self.kv_lens, self.page_indices, self.cu_q_lens,
                               self.num_seqs, self.cfg, out=out, lse=lse, workspace=self.workspace,
                               want_lse=want_lse, sinks=self.sinks)
        torch.cuda.synchronize()
        return out, lse


def run_numpy(w: wl.Workload):
    d = Device(w)
    out, lse = d.run()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def assert_parity(out, lse, ref_out, ref_lse, what=""):
    """out/ref_out [..., D]; lse/ref_lse [...]; only rows given are compared."""
    out = np.asarray(out, np.float64)
    ref_out = np.asarray(ref_out, np.float64)
    assert np.isfinite(ref_out).all(), f"{what}: oracle produced non-finite values"
    diff = np.abs(out - ref_out)
    bound = ATOL + RTOL * np.abs(ref_out)
    bad = ~(diff <= bound)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outputs outside the bar; "
                           f"max |d| {np.nanmax(diff):.3e}")
    rms_ref = float(np.sqrt(np.mean(ref_out ** 2)))
    rel_rms = float(np.sqrt(np.mean((out - ref_out) ** 2))) / max(rms_ref, 1e-30)
    assert rel_rms <= REL_RMS_TOL, f"{what}: relative RMS error {rel_rms:.3e}"
    if lse is not None:
        dl = np.abs(np.asarray(lse, np.float64) - np.asarray(ref_lse, np.float64))
        badl = ~(dl <= LSE_TOL)
        assert not badl.any(), f"{what}: {int(badl.sum())} lse values off; max |d| {np.nanmax(dl):.3e}"
    return dict(max_abs=float(np.max(diff)) if diff.size else 0.0, rel_rms=rel_rms)


def sample_rows(w: wl.Workload, n_random: int = 192, seed: int = 0):
    """A seeded sample of (token, q head) rows of a large workload: every q
    head of the first and last token of the batch and of a middle sequence,
    plus n_random random pairs."""
    rng = np.random.default_rng(seed)
    T = w.valid_tokens()
    Hq = w.cfg.num_q_heads
    s = w.n_seqs // 2
    toks = [int(w.cu_q_lens[0]), T - 1, int(w.cu_q_lens[s]), int(w.cu_q_lens[s + 1]) - 1]
    tokens = np.repeat(np.array(toks), Hq)
    heads = np.tile(np.arange(Hq), len(toks))
    rt = rng.integers(0, T, size=n_random)
    rh = rng.integers(0, Hq, size=n_random)
    return np.concatenate([tokens, rt]), np.concatenate([heads, rh])


def check_sampled(w: wl.Workload, d, what: str):
    """Runs the HIP path on device workload d and compares the sampled rows
    with the oracle, computed one by one."""
    import oracle

    print(f"[workload] {what}: running GPU", flush=True)
    out, lse = d.run()
    tokens, heads = sample_rows(w)
    t = torch.from_numpy(tokens).cuda()
    h = torch.from_numpy(heads).cuda()
    got_o = out[t, h].float().cpu().numpy()
    got_l = lse[t, h].cpu().numpy()
    print(f"[workload] {what}: oracle on {len(tokens)} rows", flush=True)
    ref_o, ref_l, st = oracle.rows(w, tokens, heads)
    assert np.all(st == 0)
    stats = assert_parity(got_o, got_l, ref_o, ref_l, what)
    print(f"[workload] {what}: ok {stats}", flush=True)
