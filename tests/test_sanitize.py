"""The oracle and the host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; errors are fatal):

* the host logic that touches no device (configuration checks, workspace
  layout, metadata check, status strings: ragged_paged_gqa_amd/csrc/
  rpa_host.cpp) is built with g++ into tests/sanitize_host.cpp's harness and
  run over a grid of configurations and random and broken tables;
* the oracle (oracle/rpa_oracle.c) is built with gcc as a shared library and
  driven from a Python process with the sanitizer runtimes preloaded, over
  ragged workloads of every K/V and q type, sampled rows, poisoned tables and
  the KV-cache append.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "ragged_paged_gqa_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs gcc and g++ with the sanitizer runtimes")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return os.path.realpath(path) if os.path.isabs(path) and os.path.exists(path) else None


def test_host_c_abi_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_checks")
    subprocess.run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(CSRC, "rpa_host.cpp"), os.path.join(ROOT, "tests", "sanitize_host.cpp"),
                    "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "host checks passed" in r.stdout


ORACLE_DRIVER = r"""
import numpy as np
import oracle
import workloads as wl

cases = [
    dict(seed=1, head_dim=64),
    dict(seed=2, head_dim=128, kv_dtype=wl.KV_FP8, window=7, soft_cap=30.0),
    dict(seed=3, head_dim=64, kv_dtype=wl.KV_E5M2, causal=False),
    dict(seed=4, head_dim=64, kv_dtype=wl.KV_I8, G=3),
    dict(seed=5, head_dim=64, kv_dtype=wl.KV_F16, q_dtype=wl.Q_F16, window=1),
    dict(seed=6, head_dim=128, q_dtype=wl.Q_F32, page_size=32),
]
for kw in cases:
    seed = kw.pop("seed")
    w = wl.random_small(seed, max_seqs=4, max_q=12, max_extra_kv=40, **kw)
    out, lse = oracle.forward(w)
    T = w.valid_tokens()
    assert np.isfinite(out[:T]).all() and np.isfinite(lse[:T]).all(), seed
    # sampled rows, padding tokens included
    toks = np.arange(w.cfg.num_q_tokens).repeat(2)
    heads = np.tile([0, w.cfg.num_q_heads - 1], w.cfg.num_q_tokens)
    ro, rl, st = oracle.rows(w, toks, heads)
    ok = st == 0
    assert np.array_equal(ro[ok], out[toks[ok], heads[ok]]), seed
    # unused table entries poisoned with an out-of-range page id
    w2 = wl.random_small(seed, max_seqs=4, max_q=12, max_extra_kv=40, **kw)
    for s in range(w2.n_seqs):
        used = -(-int(w2.kv_lens[s]) // w2.cfg.page_size)
        w2.page_indices[s, used:] = 10 ** 6
    o2, l2 = oracle.forward(w2)
    assert np.array_equal(o2[:T], out[:T]), seed
    # the append of new rows into a copy of the cache
    k_new, v_new = wl.new_kv(w, 100 + seed)
    kv, skipped = oracle.kv_append(w, k_new, v_new)
    assert kv.shape == w.kv_pages.shape
for x in np.linspace(-500, 500, 2001, dtype=np.float32):
    oracle.f32_to_e4m3fn(np.array([x], np.float32))
    oracle.f32_to_e5m2(np.array([x], np.float32))
    oracle.f32_to_i8(np.array([x], np.float32))
oracle.e4m3fn_to_f64(np.arange(256, dtype=np.uint8))
oracle.e5m2_to_f64(np.arange(256, dtype=np.uint8))
oracle.f16_to_f64(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16))
oracle.bf16_to_f64(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16))
print("oracle checks passed")
"""


def test_oracle_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not found")
    lib = str(tmp_path / "librpa_oracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-fopenmp", "-fPIC", "-shared", *SAN, "-fno-fast-math", "-o", lib,
                    os.path.join(ROOT, "oracle", "rpa_oracle.c"), "-lm"], check=True)
    driver = tmp_path / "drive.py"
    driver.write_text(ORACLE_DRIVER)
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", RPA_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2",
               PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, str(driver)], env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "oracle checks passed" in r.stdout
