"""CPU f64 oracle for ragged paged GQA attention and its KV-cache append —
test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP library
(``ragged_paged_gqa_amd``) and never imports it. The arithmetic lives in
``rpa_oracle.c`` (plain C, f64, OpenMP over rows); this module only builds
it with gcc and marshals numpy arrays.

Pins: the tests in ``tests/test_oracle.py`` and ``tests/test_oracle_append.py``
tie every part of the oracle to something other than itself (closed forms,
invariants, library routines, brute force, a hand-derived placement table).
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rpa_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
# RPA_ORACLE_LIB may name another build of the same source (the sanitizer test's)
_LIB = os.environ.get("RPA_ORACLE_LIB") or os.path.join(_BUILD, "librpa_oracle.so")

KV_CODES = {"bf16": 0, "fp8_e4m3fn": 1, "fp8_e5m2": 2, "f16": 3, "int8": 4}
Q_CODES = {"bf16": 0, "f16": 3, "f32": 5}


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("num_q_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("total_num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_num_seqs", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("is_causal", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32),
        ("has_soft_cap", ctypes.c_int32),
        ("sm_scale", ctypes.c_double),
        ("soft_cap", ctypes.c_double),
        ("k_scale", ctypes.c_double),
        ("v_scale", ctypes.c_double),
        ("sinks", ctypes.c_void_p),
        ("q_dtype", ctypes.c_int32),
    ]


def build(force: bool = True) -> str:
    """Compile rpa_oracle.c with gcc (no fast-math) into _build/."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    os.makedirs(_BUILD, exist_ok=True)
    tmp = _LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_e4m3fn_to_f64.restype = ctypes.c_double
        L.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_e5m2_to_f64.restype = ctypes.c_double
        L.oracle_e5m2_to_f64.argtypes = [ctypes.c_uint8]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_i8.restype = ctypes.c_int8
        L.oracle_f32_to_i8.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_e5m2.restype = ctypes.c_uint8
        L.oracle_f32_to_e5m2.argtypes = [ctypes.c_float]
        L.oracle_soft_cap.restype = ctypes.c_double
        L.oracle_soft_cap.argtypes = [ctypes.c_double, ctypes.c_double]
        L.oracle_f32_to_e4m3fn.restype = ctypes.c_uint8
        L.oracle_f32_to_e4m3fn.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        P = ctypes.c_void_p
        L.oracle_forward.restype = ctypes.c_int
        L.oracle_forward.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, ctypes.c_int32, P, P, ctypes.c_int]
        L.oracle_kv_append.restype = ctypes.c_int64
        L.oracle_kv_append.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, P, ctypes.c_int32]
        L.oracle_rows.restype = ctypes.c_int
        L.oracle_rows.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, ctypes.c_int32, P, P, ctypes.c_int64,
                                  P, P, P, ctypes.c_int]
        _lib = L
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _cfg(w) -> _Cfg:
    c = w.cfg
    sinks = getattr(w, "sinks", None)
    cfg = _Cfg(
        num_q_tokens=c.num_q_tokens, num_q_heads=c.num_q_heads, num_kv_heads=c.num_kv_heads,
        head_dim=c.head_dim, total_num_pages=c.total_num_pages, page_size=c.page_size,
        max_num_seqs=c.max_num_seqs, pages_per_seq=c.pages_per_seq, kv_dtype=KV_CODES[c.kv_dtype],
        is_causal=int(bool(c.is_causal)), sliding_window=int(c.sliding_window or 0),
        has_soft_cap=int(c.soft_cap is not None), sm_scale=float(c.sm_scale),
        soft_cap=float(c.soft_cap or 0.0),
        k_scale=1.0 if c.k_scale is None else float(c.k_scale),
        v_scale=1.0 if c.v_scale is None else float(c.v_scale), sinks=None,
        q_dtype=Q_CODES[getattr(c, "q_dtype", "bf16")])
    if sinks is not None:
        # f64 copy of the f32 sink logits, kept alive with the struct
        cfg._sinks = np.ascontiguousarray(np.asarray(sinks, dtype=np.float32), dtype=np.float64)
        assert cfg._sinks.shape == (c.num_q_heads,)
        cfg.sinks = cfg._sinks.ctypes.data
    return cfg


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _inputs(w):
    arrs = [np.ascontiguousarray(w.q), np.ascontiguousarray(w.kv_pages),
            np.ascontiguousarray(w.kv_lens, dtype=np.int32),
            np.ascontiguousarray(w.page_indices, dtype=np.int32),
            np.ascontiguousarray(w.cu_q_lens, dtype=np.int32)]
    # q: bits of the q dtype (uint16 for bf16 / f16, uint32 for f32)
    assert arrs[0].dtype == (np.uint32 if getattr(w.cfg, "q_dtype", "bf16") == "f32" else np.uint16)
    return arrs


def forward(w, nthreads: int | None = None):
    """All rows. Returns (out [T, Hq, D] f64, lse [T, Hq] f64); padding rows are NaN."""
    c = w.cfg
    out = np.full((c.num_q_tokens, c.num_q_heads, c.head_dim), np.nan)
    lse = np.full((c.num_q_tokens, c.num_q_heads), np.nan)
    q, kv, kvl, pi, cu = _inputs(w)
    cfg = _cfg(w)
    rc = lib().oracle_forward(ctypes.byref(cfg), _ptr(q), _ptr(kv), _ptr(kvl), _ptr(pi), _ptr(cu),
                              int(w.num_seqs[0]), _ptr(out), _ptr(lse), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_forward rejected the inputs (code {rc})")
    return out, lse


def rows(w, tokens, heads, nthreads: int | None = None):
    """Selected rows. Returns (out [n, D] f64, lse [n] f64, status [n] int32).

    status 0 = computed, 1 = padding token (row left NaN)."""
    c = w.cfg
    tokens = np.ascontiguousarray(tokens, dtype=np.int64)
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    n = len(tokens)
    out = np.full((n, c.head_dim), np.nan)
    lse = np.full(n, np.nan)
    status = np.zeros(n, dtype=np.int32)
    q, kv, kvl, pi, cu = _inputs(w)
    cfg = _cfg(w)
    rc = lib().oracle_rows(ctypes.byref(cfg), _ptr(q), _ptr(kv), _ptr(kvl), _ptr(pi), _ptr(cu),
                           int(w.num_seqs[0]), _ptr(tokens), _ptr(heads), n, _ptr(out), _ptr(lse),
                           _ptr(status), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_rows rejected the inputs (code {rc})")
    return out, lse, status


def bf16_to_f64(bits) -> np.ndarray:
    L = lib()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.oracle_bf16_to_f64(int(x)) for x in b]).reshape(np.shape(bits))


def e4m3fn_to_f64(codes) -> np.ndarray:
    L = lib()
    b = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.oracle_e4m3fn_to_f64(int(x)) for x in b]).reshape(np.shape(codes))


def e5m2_to_f64(codes) -> np.ndarray:
    L = lib()
    b = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([L.oracle_e5m2_to_f64(int(x)) for x in b]).reshape(np.shape(codes))


def f16_to_f64(bits) -> np.ndarray:
    L = lib()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.oracle_f16_to_f64(int(x)) for x in b]).reshape(np.shape(bits))


def f32_to_i8(x) -> np.ndarray:
    """Element-wise f32 -> int8 code (nearest integer, ties to even, saturating; NaN -> 0)."""
    f = lib().oracle_f32_to_i8
    a = np.asarray(x, dtype=np.float32)
    return np.array([f(float(v)) for v in a.ravel()], dtype=np.int8).reshape(a.shape)


def f32_to_f16(x) -> np.ndarray:
    """Element-wise f32 -> f16 bits (nearest even; overflow to +-inf)."""
    f = lib().oracle_f32_to_f16
    a = np.asarray(x, dtype=np.float32)
    return np.array([f(float(v)) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)


def soft_cap(x: float, c: float) -> float:
    return lib().oracle_soft_cap(float(x), float(c))


def kv_append(w, k_new, v_new):
    """The cache after writing k_new / v_new ([T, Hkv, D] bits of the q dtype) of every
    query token of w into a copy of w.kv_pages. Returns (kv_pages, skipped):
    skipped counts tokens whose slot falls outside the page table."""
    c = w.cfg
    shape = (c.num_q_tokens, c.num_kv_heads, c.head_dim)
    if getattr(w.cfg, "q_dtype", "bf16") == "f32":
        # f32 rows: float32 values or their uint32 bits
        k_new = np.ascontiguousarray(k_new).view(np.uint32)
        v_new = np.ascontiguousarray(v_new).view(np.uint32)
    else:
        k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
        v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
    assert k_new.shape == shape and v_new.shape == shape
    kv = np.array(w.kv_pages, copy=True, order="C")
    _, _, kvl, pi, cu = _inputs(w)
    cfg = _cfg(w)
    n = lib().oracle_kv_append(ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(kv), _ptr(kvl), _ptr(pi),
                               _ptr(cu), int(w.num_seqs[0]))
    if n < 0:
        raise ValueError("oracle_kv_append rejected the inputs")
    return kv, int(n)


def f32_to_e4m3fn(x) -> np.ndarray:
    """Element-wise f32 -> e4m3fn code (nearest even, saturating at +-448)."""
    f = lib().oracle_f32_to_e4m3fn
    a = np.asarray(x, dtype=np.float32)
    return np.array([f(float(v)) for v in a.ravel()], dtype=np.uint8).reshape(a.shape)


def f32_to_e5m2(x) -> np.ndarray:
    """Element-wise f32 -> e5m2 code (nearest even, saturating at +-57344)."""
    f = lib().oracle_f32_to_e5m2
    a = np.asarray(x, dtype=np.float32)
    return np.array([f(float(v)) for v in a.ravel()], dtype=np.uint8).reshape(a.shape)


def f32_to_bf16(x) -> np.ndarray:
    """Element-wise f32 -> bf16 bits (nearest even)."""
    f = lib().oracle_f32_to_bf16
    a = np.asarray(x, dtype=np.float32)
    return np.array([f(float(v)) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)
