"""Ragged paged GQA attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI in ``include/rpa.h`` (library
``_build/librpa.so``, built by ``ragged_paged_gqa_amd.build``). Every step of
the computation runs in the library's HIP kernels; this module only checks
tensor shapes/dtypes, passes device pointers and the current HIP stream, and
allocates outputs/workspace with torch when the caller does not pass them.
There is no fallback: if the library is missing, importing the entry points
raises.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# RPA_LIB_PATH may name another build of the same sources (e.g. a tuning variant).
LIB_PATH = os.environ.get("RPA_LIB_PATH") or os.path.join(_HERE, "_build", "librpa.so")

DTYPE_BF16 = 0
DTYPE_FP8_E4M3FN = 1
DTYPE_FP8_E5M2 = 2
DTYPE_F16 = 3
DTYPE_INT8 = 4
DTYPE_F32 = 5

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration", 3: "workspace too small",
          4: "HIP runtime error", 5: "metadata violates a precondition"}


class RpaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, 'unknown')} (status {status})")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [
        ("num_q_tokens", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("total_num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_num_seqs", ctypes.c_int32),
        ("pages_per_seq", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("soft_cap", ctypes.c_float),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("is_causal", ctypes.c_int32),
        ("sliding_window", ctypes.c_int32),
    ]


@dataclasses.dataclass
class Config:
    """Shapes and numeric knobs (the kernel page's `Cfg`)."""
    num_q_tokens: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    total_num_pages: int
    page_size: int
    max_num_seqs: int
    pages_per_seq: int
    kv_dtype: int = DTYPE_BF16
    sm_scale: float = 1.0
    soft_cap: float = 0.0        # 0: off
    k_scale: float = 1.0
    v_scale: float = 1.0
    is_causal: bool = True
    sliding_window: int = 0      # 0: off
    q_dtype: int = DTYPE_BF16    # q and out: DTYPE_BF16, DTYPE_F16 or DTYPE_F32

    def to_c(self) -> _Config:
        return _Config(
            num_q_tokens=self.num_q_tokens, num_q_heads=self.num_q_heads, num_kv_heads=self.num_kv_heads,
            head_dim=self.head_dim, total_num_pages=self.total_num_pages, page_size=self.page_size,
            max_num_seqs=self.max_num_seqs, pages_per_seq=self.pages_per_seq, q_dtype=self.q_dtype,
            kv_dtype=self.kv_dtype, sm_scale=self.sm_scale, soft_cap=self.soft_cap or 0.0,
            k_scale=1.0 if self.k_scale is None else self.k_scale,
            v_scale=1.0 if self.v_scale is None else self.v_scale,
            is_causal=int(bool(self.is_causal)), sliding_window=int(self.sliding_window or 0))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run python -m ragged_paged_gqa_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        CP = ctypes.POINTER(_Config)
        L.rpa_workspace_bytes.argtypes = [CP, ctypes.POINTER(ctypes.c_size_t)]
        L.rpa_forward.argtypes = [CP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.rpa_forward_sinks.argtypes = [CP, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.rpa_forward_noalloc.argtypes = [CP, P, P, P, P, P, P, P, P, P, P]
        L.rpa_status_string.argtypes = [ctypes.c_int]
        L.rpa_status_string.restype = ctypes.c_char_p
        L.rpa_check_metadata.argtypes = [CP, P, P, P, ctypes.c_int32]
        L.rpa_plan.argtypes = [CP, P, P, P, P, ctypes.c_size_t, P]
        L.rpa_plan_layout.argtypes = [CP, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_int32)]
        L.rpa_kv_append.argtypes = [CP, P, P, P, P, P, P, P, P]
        L.rpa_debug_decode_fp8.argtypes = [P, P, ctypes.c_int32, P]
        L.rpa_profile_begin.argtypes = [ctypes.c_int32]
        L.rpa_profile_end.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)]
        for f in ("rpa_workspace_bytes", "rpa_forward", "rpa_forward_sinks", "rpa_forward_noalloc",
                  "rpa_check_metadata", "rpa_plan",
                  "rpa_plan_layout", "rpa_kv_append",
                  "rpa_debug_decode_fp8", "rpa_profile_begin", "rpa_profile_end"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


EXPORTS = ("rpa_workspace_bytes", "rpa_forward", "rpa_forward_sinks", "rpa_forward_noalloc", "rpa_status_string",
           "rpa_check_metadata",
           "rpa_plan", "rpa_plan_layout", "rpa_kv_append", "rpa_debug_decode_fp8", "rpa_profile_begin", "rpa_profile_end")

# rpa_profile_end's slots: the plan, the tile launch (both classes), the
# merge of split decode units, the whole call.
KERNELS = ("plan", "tiles", "combine", "call")


def _check(status: int, what: str) -> None:
    if status != 0:
        raise RpaError(status, what)


def status_string(status: int) -> str:
    return lib().rpa_status_string(status).decode()


def workspace_bytes(cfg: Config) -> int:
    c = cfg.to_c()
    n = ctypes.c_size_t(0)
    _check(lib().rpa_workspace_bytes(ctypes.byref(c), ctypes.byref(n)), "rpa_workspace_bytes")
    return int(n.value)


def plan_layout(cfg: Config):
    c = cfg.to_c()
    offs = (ctypes.c_size_t * 8)()
    lim = (ctypes.c_int32 * 8)()
    _check(lib().rpa_plan_layout(ctypes.byref(c), offs, lim), "rpa_plan_layout")
    return list(offs), list(lim)


def check_metadata(cfg: Config, kv_lens, page_indices, cu_q_lens, num_seqs: int) -> int:
    """Host-side precondition check; returns the status code (0 = ok)."""
    c = cfg.to_c()
    kvl = np.ascontiguousarray(kv_lens, dtype=np.int32)
    pi = np.ascontiguousarray(page_indices, dtype=np.int32)
    cu = np.ascontiguousarray(cu_q_lens, dtype=np.int32)
    return lib().rpa_check_metadata(ctypes.byref(c), kvl.ctypes.data, pi.ctypes.data, cu.ctypes.data,
                                    int(num_seqs))


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _dev_i32(t: torch.Tensor, name: str, numel: int) -> None:
    if not (t.is_cuda and t.dtype == torch.int32 and t.is_contiguous() and t.numel() >= numel):
        raise ValueError(f"{name}: expected a contiguous int32 CUDA tensor of >= {numel} elements")


def _q_torch_dtype(cfg: Config):
    return {DTYPE_F16: torch.float16, DTYPE_F32: torch.float32}.get(cfg.q_dtype, torch.bfloat16)


def _q_size(cfg: Config) -> int:
    return 4 if cfg.q_dtype == DTYPE_F32 else 2


def _check_inputs(cfg: Config, q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs):
    T, Hq, D = cfg.num_q_tokens, cfg.num_q_heads, cfg.head_dim
    if not (q.is_cuda and q.is_contiguous() and q.element_size() == _q_size(cfg) and q.numel() == T * Hq * D):
        raise ValueError(f"q: expected a contiguous {_q_size(cfg)}-byte (q dtype) CUDA tensor "
                         "[num_q_tokens, num_q_heads, head_dim]")
    eb = 1 if cfg.kv_dtype in (DTYPE_FP8_E4M3FN, DTYPE_FP8_E5M2, DTYPE_INT8) else 2
    kv_numel = cfg.total_num_pages * cfg.page_size * 2 * cfg.num_kv_heads * D
    if not (kv_pages.is_cuda and kv_pages.is_contiguous() and kv_pages.element_size() == eb
            and kv_pages.numel() == kv_numel):
        raise ValueError("kv_pages: expected a contiguous CUDA tensor "
                         "[total_num_pages, page_size, 2*num_kv_heads, head_dim] of the kv dtype")
    _dev_i32(kv_lens, "kv_lens", cfg.max_num_seqs)
    _dev_i32(page_indices, "page_indices", cfg.max_num_seqs * cfg.pages_per_seq)
    _dev_i32(cu_q_lens, "cu_q_lens", cfg.max_num_seqs + 1)
    _dev_i32(num_seqs, "num_seqs", 1)


def alloc_workspace(cfg: Config, device=None) -> torch.Tensor:
    n = workspace_bytes(cfg)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device or "cuda")


def forward(q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, cfg: Config, *, out=None, lse=None,
            workspace=None, want_lse: bool = True, stream=None, sinks=None):
    """Ragged paged attention. Returns (out, lse) as torch tensors on the device.

    q [T, Hq, D] bf16, f16 or f32 (cfg.q_dtype, also out's type); kv_pages
    [P, page, 2*Hkv, D] in the q type or fp8 e4m3fn / e5m2 (uint8 storage); kv_lens [S], page_indices [S, pps], cu_q_lens [S+1],
    num_seqs [1]: int32 device tensors. Rows of padding tokens keep whatever
    `out`/`lse` held. `sinks`: optional float32 device tensor [Hq] of
    attention-sink logits (rpa_forward_sinks).
    """
    _check_inputs(cfg, q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs)
    T, Hq, D = cfg.num_q_tokens, cfg.num_q_heads, cfg.head_dim
    if out is None:
        out = torch.zeros((T, Hq, D), dtype=_q_torch_dtype(cfg), device=q.device)
    elif not (out.is_cuda and out.is_contiguous() and out.element_size() == _q_size(cfg)
              and out.numel() == T * Hq * D):
        raise ValueError(f"out: expected a contiguous {_q_size(cfg)}-byte (q dtype) CUDA tensor [T, Hq, D]")
    if want_lse and lse is None:
        lse = torch.full((T, Hq), float("nan"), dtype=torch.float32, device=q.device)
    if lse is not None and not (lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32
                                and lse.numel() == T * Hq):
        raise ValueError("lse: expected a contiguous float32 CUDA tensor [T, Hq]")
    if workspace is None:
        workspace = alloc_workspace(cfg, q.device)
    c = cfg.to_c()
    if sinks is None:
        st = lib().rpa_forward(ctypes.byref(c), q.data_ptr(), kv_pages.data_ptr(), kv_lens.data_ptr(),
                               page_indices.data_ptr(), cu_q_lens.data_ptr(), num_seqs.data_ptr(), out.data_ptr(),
                               lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream_ptr(stream))
        _check(st, "rpa_forward")
    else:
        if not (sinks.is_cuda and sinks.is_contiguous() and sinks.dtype == torch.float32 and sinks.numel() == Hq):
            raise ValueError("sinks: expected a contiguous float32 CUDA tensor [Hq]")
        st = lib().rpa_forward_sinks(ctypes.byref(c), q.data_ptr(), kv_pages.data_ptr(), kv_lens.data_ptr(),
                                     page_indices.data_ptr(), cu_q_lens.data_ptr(), num_seqs.data_ptr(),
                                     sinks.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
                                     workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     _stream_ptr(stream))
        _check(st, "rpa_forward_sinks")
    return out, lse


def forward_noalloc(q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, cfg: Config, *, out, lse=None,
                    sinks=None, stream=None):
    """rpa_forward_noalloc: as `forward`, with the library's own scratch array
    as the workspace (nothing is allocated; `out` must be given). Calls that
    overlap on one GPU share that array and race."""
    _check_inputs(cfg, q, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs)
    T, Hq, D = cfg.num_q_tokens, cfg.num_q_heads, cfg.head_dim
    if not (out.is_cuda and out.is_contiguous() and out.element_size() == _q_size(cfg) and out.numel() == T * Hq * D):
        raise ValueError(f"out: expected a contiguous {_q_size(cfg)}-byte (q dtype) CUDA tensor [T, Hq, D]")
    if lse is not None and not (lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32
                                and lse.numel() == T * Hq):
        raise ValueError("lse: expected a contiguous float32 CUDA tensor [T, Hq]")
    if sinks is not None and not (sinks.is_cuda and sinks.is_contiguous() and sinks.dtype == torch.float32
                                  and sinks.numel() == Hq):
        raise ValueError("sinks: expected a contiguous float32 CUDA tensor [Hq]")
    c = cfg.to_c()
    st = lib().rpa_forward_noalloc(ctypes.byref(c), q.data_ptr(), kv_pages.data_ptr(), kv_lens.data_ptr(),
                                   page_indices.data_ptr(), cu_q_lens.data_ptr(), num_seqs.data_ptr(),
                                   sinks.data_ptr() if sinks is not None else None, out.data_ptr(),
                                   lse.data_ptr() if lse is not None else None, _stream_ptr(stream))
    _check(st, "rpa_forward_noalloc")
    return out, lse


# Size of rpa_forward_noalloc's scratch array: the largest workspace it serves.
NOALLOC_SCRATCH_BYTES = 256 << 20


def kv_append(k_new, v_new, kv_pages, kv_lens, page_indices, cu_q_lens, num_seqs, cfg: Config, *,
              stream=None):
    """Write every query token's new K and V rows into kv_pages, in place (rpa_kv_append).

    k_new, v_new [T, Hkv, D] CUDA tensors of the q type; the rest as in `forward`.
    Returns kv_pages.
    """
    T, Hkv, D = cfg.num_q_tokens, cfg.num_kv_heads, cfg.head_dim
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if not (t.is_cuda and t.is_contiguous() and t.element_size() == _q_size(cfg) and t.numel() == T * Hkv * D):
            raise ValueError(f"{name}: expected a contiguous {_q_size(cfg)}-byte (q dtype) CUDA tensor "
                             "[num_q_tokens, num_kv_heads, head_dim]")
    eb = 1 if cfg.kv_dtype in (DTYPE_FP8_E4M3FN, DTYPE_FP8_E5M2, DTYPE_INT8) else 2
    if not (kv_pages.is_cuda and kv_pages.is_contiguous() and kv_pages.element_size() == eb
            and kv_pages.numel() == cfg.total_num_pages * cfg.page_size * 2 * Hkv * D):
        raise ValueError("kv_pages: expected a contiguous CUDA tensor "
                         "[total_num_pages, page_size, 2*num_kv_heads, head_dim] of the kv dtype")
    _dev_i32(kv_lens, "kv_lens", cfg.max_num_seqs)
    _dev_i32(page_indices, "page_indices", cfg.max_num_seqs * cfg.pages_per_seq)
    _dev_i32(cu_q_lens, "cu_q_lens", cfg.max_num_seqs + 1)
    _dev_i32(num_seqs, "num_seqs", 1)
    c = cfg.to_c()
    st = lib().rpa_kv_append(ctypes.byref(c), k_new.data_ptr(), v_new.data_ptr(), kv_pages.data_ptr(),
                             kv_lens.data_ptr(), page_indices.data_ptr(), cu_q_lens.data_ptr(), num_seqs.data_ptr(),
                             _stream_ptr(stream))
    _check(st, "rpa_kv_append")
    return kv_pages


def plan(kv_lens, cu_q_lens, num_seqs, cfg: Config, workspace=None, stream=None):
    """Run only the planning kernel; returns the workspace tensor holding the plan."""
    _dev_i32(kv_lens, "kv_lens", cfg.max_num_seqs)
    _dev_i32(cu_q_lens, "cu_q_lens", cfg.max_num_seqs + 1)
    _dev_i32(num_seqs, "num_seqs", 1)
    if workspace is None:
        workspace = alloc_workspace(cfg, kv_lens.device)
    c = cfg.to_c()
    st = lib().rpa_plan(ctypes.byref(c), kv_lens.data_ptr(), cu_q_lens.data_ptr(), num_seqs.data_ptr(),
                        workspace.data_ptr(), workspace.numel(), _stream_ptr(stream))
    _check(st, "rpa_plan")
    return workspace


def decode_fp8(codes: torch.Tensor, stream=None) -> torch.Tensor:
    """fp8 e4m3fn codes (uint8 CUDA tensor) -> float32, with the kernels' conversion."""
    if not (codes.is_cuda and codes.dtype == torch.uint8 and codes.is_contiguous()):
        raise ValueError("codes: expected a contiguous uint8 CUDA tensor")
    out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _check(lib().rpa_debug_decode_fp8(codes.data_ptr(), out.data_ptr(), codes.numel(), _stream_ptr(stream)),
           "rpa_debug_decode_fp8")
    return out


def profile_begin(max_calls: int) -> None:
    """Record HIP events around the kernels of the next `max_calls` forward calls."""
    _check(lib().rpa_profile_begin(int(max_calls)), "rpa_profile_begin")


def profile_end():
    """Wait for the recorded events; returns ({kernel: summed ms}, n_calls)."""
    ms = (ctypes.c_float * len(KERNELS))()
    n = ctypes.c_int32(0)
    _check(lib().rpa_profile_end(ms, ctypes.byref(n)), "rpa_profile_end")
    return dict(zip(KERNELS, (float(x) for x in ms))), int(n.value)
