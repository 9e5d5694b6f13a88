"""Seeded synthetic inputs for ragged paged GQA attention.

This module only draws inputs: sequence lengths, a page table, Q and the
paged K/V cache, stored as the raw bits the kernels read (bf16 as uint16,
fp8 e4m3fn as uint8). It holds none of the attention arithmetic, and both
the CPU oracle and the GPU path consume what it produces.

Layouts follow the operand list of the ragged paged attention kernel page
(zml ``platforms/tpu/ragged_paged.zig``, ``run``: operands and ``Cfg``):

* ``q``            [num_q_tokens, num_q_heads, head_dim]
* ``kv_pages``     [total_num_pages, page_size, 2*num_kv_heads, head_dim],
                   K of kv head h at combined head 2h, V at 2h+1
* ``kv_lens``      [max_num_seqs] int32
* ``page_indices`` [max_num_seqs, pages_per_seq] int32
* ``cu_q_lens``    [max_num_seqs + 1] int32
* ``num_seqs``     [1] int32

Recipe (all five named workloads): ``np.random.Generator(PCG64(seed))`` with
the workload's number as seed; draw order lengths -> page permutation -> Q
-> K/V. Sequence s owns ``ceil(kv_len_s / page_size)`` consecutive entries of
the permutation; unused page-table entries hold 0 (or a poison value).
Q/K/V values are N(0,1) rounded to bf16 (round to nearest even); fp8 K/V are
N(0,1)/scale rounded to e4m3fn (saturated at +-448) or to e5m2 (saturated at
+-57344); int8 K/V are N(0,1)/scale rounded to the nearest integer (saturated
at -128 / 127). K/V pages are drawn in
chunks of ``PAGE_CHUNK`` pages, each from its own spawned PCG64 stream, so
large caches are generated in parallel yet identically on every machine.
"""

from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os

import numpy as np
import torch

PAGE_CHUNK = 256

KV_BF16 = "bf16"
KV_FP8 = "fp8_e4m3fn"
KV_E5M2 = "fp8_e5m2"
KV_F16 = "f16"
KV_I8 = "int8"
Q_BF16 = "bf16"
Q_F16 = "f16"
Q_F32 = "f32"
FP8_KINDS = (KV_FP8, KV_E5M2)
ONE_BYTE_KINDS = (KV_FP8, KV_E5M2, KV_I8)


def is_fp8(kv_dtype: str) -> bool:
    """One-byte K/V codes with a scale (e4m3fn, e5m2 or int8)."""
    return kv_dtype in ONE_BYTE_KINDS


@dataclasses.dataclass
class Config:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    total_num_pages: int
    pages_per_seq: int
    max_num_seqs: int
    num_q_tokens: int
    kv_dtype: str = KV_BF16
    q_dtype: str = Q_BF16     # q, out and the append's new K/V rows
    sm_scale: float = 1.0
    soft_cap: float | None = None
    k_scale: float | None = None
    v_scale: float | None = None
    is_causal: bool = True
    sliding_window: int | None = None

    def __post_init__(self):
        # Scales reach the kernels as f32; keep the f32-rounded values so that
        # every consumer sees the same numbers.
        f32 = lambda v: None if v is None else float(np.float32(v))
        self.sm_scale = f32(self.sm_scale)
        self.soft_cap = f32(self.soft_cap)
        self.k_scale = f32(self.k_scale)
        self.v_scale = f32(self.v_scale)


@dataclasses.dataclass
class Workload:
    name: str
    cfg: Config
    q: np.ndarray             # bits of the q dtype [T, Hq, D]: uint16 (bf16, f16) or uint32 (f32)
    kv_pages: np.ndarray      # uint16 (bf16, f16) or uint8 (e4m3fn, e5m2) bits [P, page, 2*Hkv, D]
    kv_lens: np.ndarray       # int32 [max_num_seqs]
    page_indices: np.ndarray  # int32 [max_num_seqs, pages_per_seq]
    cu_q_lens: np.ndarray     # int32 [max_num_seqs + 1]
    num_seqs: np.ndarray      # int32 [1]
    sinks: np.ndarray | None = None  # float32 [Hq] attention-sink logits, or none

    @property
    def n_seqs(self) -> int:
        return int(self.num_seqs[0])

    def q_lens(self) -> np.ndarray:
        n = self.n_seqs
        return (self.cu_q_lens[1:n + 1] - self.cu_q_lens[:n]).astype(np.int64)

    def valid_tokens(self) -> int:
        return int(self.cu_q_lens[self.n_seqs])


# ----------------------------------------------------------------------------
# value encoders (library casts only)

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (torch's CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_e4m3fn_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> fp8 e4m3fn bits, saturated at +-448 then rounded to nearest even."""
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bits, round to nearest even (numpy's cast)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_q_bits(x: np.ndarray, q_dtype: str) -> np.ndarray:
    """Values -> bits of the q dtype: uint16 for bf16 / f16, uint32 for f32."""
    if q_dtype == Q_F32:
        return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return to_f16_bits(x) if q_dtype == Q_F16 else to_bf16_bits(x)


def to_i8_codes(x: np.ndarray) -> np.ndarray:
    """float32 -> int8 codes: nearest integer (ties to even), saturated at -128 / 127."""
    return np.clip(np.rint(np.ascontiguousarray(x, dtype=np.float32)), -128, 127).astype(np.int8).view(np.uint8)


def to_e5m2_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> fp8 e5m2 bits, saturated at +-57344 then rounded to nearest even."""
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -57344.0, 57344.0)
    t = torch.from_numpy(x).to(torch.float8_e5m2)
    return t.view(torch.uint8).numpy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# generation

def _fill_kv(kv: np.ndarray, seed: int, kv_dtype: str, scale: float | None,
             threads: int | None = None) -> None:
    P = kv.shape[0]
    n_chunks = (P + PAGE_CHUNK - 1) // PAGE_CHUNK
    children = np.random.SeedSequence([seed, 0x5EED]).spawn(n_chunks)
    per_page = int(np.prod(kv.shape[1:]))

    def work(c):
        p0, p1 = c * PAGE_CHUNK, min(P, (c + 1) * PAGE_CHUNK)
        rng = np.random.Generator(np.random.PCG64(children[c]))
        z = rng.standard_normal((p1 - p0) * per_page, dtype=np.float32)
        if kv_dtype == KV_FP8:
            kv[p0:p1] = to_e4m3fn_bits(z / np.float32(scale)).reshape(kv[p0:p1].shape)
        elif kv_dtype == KV_E5M2:
            kv[p0:p1] = to_e5m2_bits(z / np.float32(scale)).reshape(kv[p0:p1].shape)
        elif kv_dtype == KV_F16:
            kv[p0:p1] = to_f16_bits(z).reshape(kv[p0:p1].shape)
        elif kv_dtype == KV_I8:
            kv[p0:p1] = to_i8_codes(z / np.float32(scale)).reshape(kv[p0:p1].shape)
        else:
            kv[p0:p1] = to_bf16_bits(z).reshape(kv[p0:p1].shape)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if n_chunks == 1 or threads <= 1:
        for c in range(n_chunks):
            work(c)
    else:
        torch_threads = torch.get_num_threads()
        torch.set_num_threads(1)
        try:
            with _cf.ThreadPoolExecutor(threads) as ex:
                list(ex.map(work, range(n_chunks)))
        finally:
            torch.set_num_threads(torch_threads)


def build(name: str, cfg_kw: dict, q_lens, kv_lens, seed: int, *, rng=None,
          total_num_pages: int | None = None, max_num_seqs: int | None = None,
          num_q_tokens: int | None = None, page_table: str = "perm",
          unused_entry: int = 0, q_mult: float = 1.0) -> Workload:
    """Assemble a workload from explicit lengths.

    ``rng`` continues an existing stream (lengths already drawn from it);
    otherwise a fresh PCG64(seed) is used. ``page_table='perm'`` gives each
    sequence consecutive entries of a seeded permutation of all pages.
    ``q_mult`` scales Q before rounding (sharpened softmax variants).
    """
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    q_lens = np.asarray(q_lens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    S = len(q_lens)
    page = cfg_kw["page_size"]
    pages_needed = (kv_lens + page - 1) // page
    if total_num_pages is None:
        total_num_pages = max(1, int(pages_needed.sum()))
    if max_num_seqs is None:
        max_num_seqs = S
    pps = cfg_kw.get("pages_per_seq") or max(1, int(pages_needed.max(initial=1)))
    T_valid = int(q_lens.sum())
    if num_q_tokens is None:
        num_q_tokens = max(1, T_valid)
    cfg = Config(total_num_pages=total_num_pages, max_num_seqs=max_num_seqs,
                 num_q_tokens=num_q_tokens,
                 **{k: v for k, v in cfg_kw.items() if k != "pages_per_seq"},
                 pages_per_seq=pps)
    assert pages_needed.sum() <= total_num_pages
    assert (pages_needed <= pps).all()

    perm = rng.permutation(total_num_pages).astype(np.int32)
    page_indices = np.full((max_num_seqs, pps), unused_entry, dtype=np.int32)
    off = 0
    for s in range(S):
        n = int(pages_needed[s])
        page_indices[s, :n] = perm[off:off + n]
        off += n

    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    qz = rng.standard_normal((num_q_tokens, Hq, D), dtype=np.float32)
    if q_mult != 1.0:
        qz *= np.float32(q_mult)
    q = to_q_bits(qz, cfg.q_dtype)

    kv_np_dtype = np.uint8 if is_fp8(cfg.kv_dtype) else np.uint16
    kv = np.empty((total_num_pages, page, 2 * Hkv, D), dtype=kv_np_dtype)
    _fill_kv(kv, seed, cfg.kv_dtype, cfg.k_scale if is_fp8(cfg.kv_dtype) else None)

    kv_lens_arr = np.zeros(max_num_seqs, dtype=np.int32)
    kv_lens_arr[:S] = kv_lens
    cu = np.zeros(max_num_seqs + 1, dtype=np.int32)
    cu[1:S + 1] = np.cumsum(q_lens)
    cu[S + 1:] = cu[S]
    return Workload(name=name, cfg=cfg, q=q, kv_pages=kv, kv_lens=kv_lens_arr,
                    page_indices=page_indices, cu_q_lens=cu,
                    num_seqs=np.array([S], dtype=np.int32))


# ----------------------------------------------------------------------------
# the five named workloads

WORKLOADS = {
    1: "tiny ragged: 3 seqs, q_lens [1,5,16], kv_lens [8,37,64], 4/2 heads, D 64, page 16",
    2: "decode: 256 seqs x 1 token, kv U[512,8192], 32/8 heads, D 128, page 16, bf16",
    3: "mixed: 8 x 448-token chunks (prior U[0,8192]) + 56 decodes (kv U[1024,16384]), 64/8 heads, D 128, page 32",
    4: "fp8 decode: 128 seqs x 1 token, kv U[4096,32768], 32/8 heads, D 128, page 16, e4m3fn, softcap 50, window 4096",
    5: "long context: 16 seqs x 128 tokens, kv U[65536,131072], 32/2 heads, D 256, page 64, bf16",
}


def lengths(number: int, rng) -> tuple[np.ndarray, np.ndarray]:
    """The (q_lens, kv_lens) draw of a named workload, first in its stream."""
    if number == 1:
        return np.array([1, 5, 16]), np.array([8, 37, 64])
    if number == 2:
        kv = rng.integers(512, 8192, size=256, endpoint=True)
        return np.ones(256, dtype=np.int64), kv
    if number == 3:
        prior = rng.integers(0, 8192, size=8, endpoint=True)
        dec = rng.integers(1024, 16384, size=56, endpoint=True)
        q = np.concatenate([np.full(8, 448), np.ones(56, dtype=np.int64)])
        return q, np.concatenate([prior + 448, dec])
    if number == 4:
        kv = rng.integers(4096, 32768, size=128, endpoint=True)
        return np.ones(128, dtype=np.int64), kv
    if number == 5:
        kv = rng.integers(65536, 131072, size=16, endpoint=True)
        return np.full(16, 128), kv
    raise ValueError(number)


def cfg_kw(number: int) -> dict:
    if number == 1:
        return dict(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                    pages_per_seq=4, sm_scale=1.0 / 8)
    if number == 2:
        return dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    pages_per_seq=512, sm_scale=1.0 / math.sqrt(128))
    if number == 3:
        return dict(num_q_heads=64, num_kv_heads=8, head_dim=128, page_size=32,
                    pages_per_seq=512, sm_scale=1.0 / math.sqrt(128))
    if number == 4:
        return dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                    pages_per_seq=2048, sm_scale=1.0 / math.sqrt(128),
                    kv_dtype=KV_FP8, k_scale=0.05, v_scale=0.05,
                    soft_cap=50.0, sliding_window=4096)
    if number == 5:
        return dict(num_q_heads=32, num_kv_heads=2, head_dim=256, page_size=64,
                    pages_per_seq=2048, sm_scale=1.0 / 16)
    raise ValueError(number)


def named(number: int, *, q_mult: float = 1.0, unused_entry: int = 0,
          seed: int | None = None, kv_dtype: str | None = None, q_dtype: str | None = None) -> Workload:
    """A named workload; `kv_dtype` swaps its K/V type (fp8 kinds take the fp8
    decode workload's scales, 0.05, when the workload has none) and `q_dtype`
    its q/out type (with f16 q a bf16 cache becomes f16; f32 q keeps the cache)."""
    seed = number if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    q_lens, kv_lens = lengths(number, rng)
    kw = dict(q_mult=q_mult, unused_entry=unused_entry)
    if number == 1:
        kw["total_num_pages"] = 32
    ckw = cfg_kw(number)
    if q_dtype == Q_F32:
        ckw["q_dtype"] = Q_F32
    if q_dtype == Q_F16:
        ckw["q_dtype"] = Q_F16
        if kv_dtype is None and ckw.get("kv_dtype", KV_BF16) == KV_BF16:
            kv_dtype = KV_F16
    if kv_dtype is not None:
        ckw["kv_dtype"] = kv_dtype
        if is_fp8(kv_dtype):
            ckw.setdefault("k_scale", 0.05)
            ckw.setdefault("v_scale", 0.05)
        else:
            ckw.pop("k_scale", None)
            ckw.pop("v_scale", None)
    return build(f"cfg{number}", ckw, q_lens, kv_lens, seed, rng=rng, **kw)


def with_sinks(w: Workload, seed: int, mean: float = 1.0, std: float = 2.0) -> Workload:
    """w with seeded attention-sink logits, one per q head (N(mean, std^2), f32)."""
    rng = np.random.Generator(np.random.PCG64([seed, 0x51A7]))
    w.sinks = rng.normal(mean, std, size=w.cfg.num_q_heads).astype(np.float32)
    return w


def random_small(seed: int, *, max_seqs: int = 4, head_dim: int = 64,
                 kv_dtype: str = KV_BF16, q_dtype: str = Q_BF16, causal: bool = True,
                 window: int | None = None, soft_cap: float | None = None,
                 G: int | None = None, page_size: int = 16,
                 max_q: int = 24, max_extra_kv: int = 80) -> Workload:
    """Small ragged workload with random lengths, for property tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    S = int(rng.integers(1, max_seqs, endpoint=True))
    q_lens = rng.integers(0, max_q, size=S, endpoint=True)
    kv_lens = q_lens + rng.integers(0, max_extra_kv, size=S, endpoint=True)
    kv_lens = np.maximum(kv_lens, 1)
    Hkv = int(rng.integers(1, 3, endpoint=True))
    G = int(rng.integers(1, 5, endpoint=True)) if G is None else G
    kw = dict(num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=head_dim,
              page_size=page_size, pages_per_seq=None,
              sm_scale=1.0 / math.sqrt(head_dim), kv_dtype=kv_dtype, q_dtype=q_dtype,
              is_causal=causal, sliding_window=window, soft_cap=soft_cap)
    if is_fp8(kv_dtype):
        kw.update(k_scale=0.05, v_scale=0.05)
    pages_needed = int(((kv_lens + page_size - 1) // page_size).sum())
    return build(f"rand{seed}", kw, q_lens, kv_lens, seed, rng=rng,
                 total_num_pages=pages_needed + int(rng.integers(0, 4)),
                 max_num_seqs=S + int(rng.integers(0, 2)),
                 num_q_tokens=int(q_lens.sum()) + int(rng.integers(0, 3)) or 1)


# ----------------------------------------------------------------------------
# inputs of the kv-cache append

def from_tables(cfg_kw: dict, q_lens, kv_lens, tables, seed: int, *, total_num_pages: int,
                max_num_seqs: int | None = None, num_q_tokens: int | None = None,
                pages_per_seq: int | None = None) -> Workload:
    """A workload with an explicit page table (one list of page ids per sequence);
    Q and the cache are drawn from PCG64(seed) as in ``build``."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    S = len(q_lens)
    max_num_seqs = S if max_num_seqs is None else max_num_seqs
    pps = pages_per_seq or max(len(t) for t in tables)
    kw = dict(cfg_kw, pages_per_seq=pps)
    w = build("tables", kw, q_lens, kv_lens, seed, total_num_pages=total_num_pages,
              max_num_seqs=max_num_seqs, num_q_tokens=num_q_tokens)
    w.page_indices[:] = 0
    for s, t in enumerate(tables):
        w.page_indices[s, :len(t)] = np.asarray(t, dtype=np.int32)
    return w


def new_kv(w: Workload, seed: int, std: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    """Seeded new K and V rows for every query token: bits of the q dtype
    [T, Hkv, D], N(0, std^2)."""
    c = w.cfg
    rng = np.random.Generator(np.random.PCG64([seed, 0xA11E]))
    shape = (c.num_q_tokens, c.num_kv_heads, c.head_dim)
    k = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    v = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    return to_q_bits(k, c.q_dtype), to_q_bits(v, c.q_dtype)


def finite_bf16_patterns() -> np.ndarray:
    """Every bf16 bit pattern that encodes a finite value (uint16, ascending)."""
    b = np.arange(1 << 16, dtype=np.uint32)
    return b[(b & 0x7F80) != 0x7F80].astype(np.uint16)
