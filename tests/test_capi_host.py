"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any GPU work (CPU only: no compute calls)."""
import ctypes
import os
import re

import pytest

from dsa_sparse_attention_lightning_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if not f.endswith(".h"):
            continue
        src = open(os.path.join(inc, f)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M):
            if m.group(1) not in ("if", "while", "for", "sizeof"):
                names.append(m.group(1))
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    return _lib.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_attn", "indexcache_run_stack",
                 "dsa_last_error", "dsa_topk_workspace_size", "dsa_sparse_attn_workspace_size",
                 "indexcache_stack_workspace_size", "dsa_version"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_version(lib):
    assert b"gfx950" in lib.dsa_version()


def _err(lib):
    return lib.dsa_last_error().decode()


def test_topk_rejects_bad_k(lib):
    st = lib.dsa_topk(16, 4096, 16, 1, 1, 4096, 0, 16, None, 0, None)
    assert st == _lib.DSA_ERR_INVALID_ARG and "k must be" in _err(lib)
    st = lib.dsa_topk(16, 4096, 16, 1, 1, 4096, 20000, 16, None, 0, None)
    assert st == _lib.DSA_ERR_UNSUPPORTED


def test_topk_rejects_null_and_misaligned(lib):
    assert lib.dsa_topk(None, 4096, 16, 1, 1, 4096, 8, 16, None, 0, None) == 1
    assert "scores is NULL" in _err(lib)
    assert lib.dsa_topk(18, 4096, 16, 1, 1, 4096, 8, 16, None, 0, None) == 1
    assert "aligned" in _err(lib)
    assert lib.dsa_topk(16, 4094, 16, 1, 1, 4094, 8, 16, None, 0, None) == 1  # ld % 4


def test_indexer_rejects_unsupported(lib):
    f = lib.dsa_indexer_scores
    assert f(16, 0, None, 16, 16, None, 16, 1, 1, 64, 96, 128, 16, 128, None) == 2   # D = 96
    assert f(16, 0, None, 16, 16, None, 16, 1, 1, 65, 128, 128, 16, 128, None) == 2  # H = 65
    assert f(16, 1, None, 16, 16, None, 16, 1, 1, 64, 128, 128, 16, 128, None) == 1  # fp8 no scale
    assert "scale" in _err(lib)
    assert f(16, 0, 16, 16, 16, None, 16, 1, 1, 64, 128, 128, 16, 128, None) == 1   # bf16 + scale
    assert f(16, 7, None, 16, 16, None, 16, 1, 1, 64, 128, 128, 16, 128, None) == 1  # dtype
    assert f(16, 0, None, 16, 16, None, 16, 1, 200, 64, 128, 128, 16, 128, None) == 1  # T > Lmax


def test_attn_rejects_unsupported(lib):
    f = lib.dsa_sparse_attn
    assert f(16, 16, 16, 16, 1, 1, 128, 100, 8, 512, 512, 0.1, 16, None, None, 0, None) == 2
    assert f(16, 16, 16, 16, 1, 1, 100, 100, 8, 576, 512, 0.1, 16, None, None, 0, None) == 2
    assert f(16, 16, 16, 16, 1, 1, 128, 100, 8, 576, 512, -1.0, 16, None, None, 0, None) == 1
    need = ctypes.c_size_t()
    assert lib.dsa_sparse_attn_workspace_size(8, 1, 128, 2048, 512, ctypes.byref(need)) == 0
    if need.value:
        assert f(16, 16, 16, 16, 8, 1, 128, 4096, 2048, 576, 512, 0.1, 16, None, None, 0,
                 None) == _lib.DSA_ERR_WORKSPACE


def test_limits_are_enforced_on_the_host(lib):
    """Shapes past what the kernels address are rejected before any launch."""
    f = lib.dsa_indexer_scores
    # one sequence's bf16 keys above 2^31 bytes (buffer-resource range)
    assert f(16, 0, None, 16, 16, None, 16, 1, 1, 64, 128, 1 << 23, 16, 1 << 23, None) == 2
    assert "per sequence" in _err(lib) or "bytes" in _err(lib)
    # B * T above 65535 indexer rows
    assert f(16, 0, None, 16, 16, None, 16, 300, 300, 64, 128, 4096, 16, 4096, None) == 2
    a = lib.dsa_sparse_attn
    assert a(16, 16, 16, 16, 1, 1, 1040, 100, 8, 576, 512, 0.1, 16, None, None, 0, None) == 2
    assert "Hq" in _err(lib)
    assert a(16, 16, 16, 16, 1, 1, 128, 1 << 17, 65537, 576, 512, 0.1, 16, None, None, 0,
             None) == 2
    assert "k must be" in _err(lib)
    # latent rows of one sequence above 2^31 bytes
    assert a(16, 16, 16, 16, 1, 1, 128, 1 << 21, 2048, 576, 512, 0.1, 16, None, None, 0,
             None) == 2
    assert "per sequence" in _err(lib)
    assert a(16, 16, 16, 16, 1, 9, 128, 8, 8, 576, 512, 0.1, 16, None, None, 0, None) == 1
    assert "exceeds Lmax" in _err(lib)
    need = ctypes.c_size_t()
    assert lib.dsa_topk_workspace_size(1, 1, 4096, 16, None) == 1
    assert lib.dsa_sparse_attn_workspace_size(1, 1, 100, 16, 512, ctypes.byref(need)) == 1
    assert lib.indexcache_stack_workspace_size(None, ctypes.byref(need)) == 1


def _stack_args(pattern, n):
    layers = (_lib.Layer * n)()
    for i in range(n):
        layers[i] = _lib.Layer(16, None, 16, 16, None, 16, 16, 16, None)
    shape = _lib.StackShape(1, 1, 64, 128, 4096, 2048, 128, 576, 512, 0, 0.1)
    return pattern.encode(), n, layers, shape


@pytest.mark.parametrize("pattern,n,msg", [("SFFF", 4, "start with 'F'"), ("FSX", 3, "neither"),
                                           ("FSS", 4, "length"), ("FSSSS", 4, "length")])
def test_stack_rejects_bad_patterns(lib, pattern, n, msg):
    p, n, layers, shape = _stack_args(pattern, n)
    st = lib.indexcache_run_stack(p, n, layers, ctypes.byref(shape), 16, 16, 16, 4096, 16,
                                  1 << 30, None, None)
    assert st == _lib.DSA_ERR_INVALID_ARG
    assert msg in _err(lib)


def test_stack_rejects_small_workspace(lib):
    p, n, layers, shape = _stack_args("FSSS", 4)
    need = ctypes.c_size_t()
    assert lib.indexcache_stack_workspace_size(ctypes.byref(shape), ctypes.byref(need)) == 0
    if need.value == 0:
        pytest.skip("no workspace needed at this shape")
    st = lib.indexcache_run_stack(p, n, layers, ctypes.byref(shape), 16, 16, 16, 4096, 16,
                                  need.value - 1, None, None)
    assert st == _lib.DSA_ERR_WORKSPACE


def test_kv_append_rejects_bad_arguments(lib):
    f = lib.dsa_kv_append
    # (kv_new, k_new, ctx, B, T, Lmax, d_qk, D, dtype, kv_cache, k_cache, k_scale, stream)
    assert f(None, None, 16, 1, 1, 64, 576, 128, 1, None, None, None, None) == 1
    assert "nothing to append" in _err(lib)
    assert f(16, None, 16, 1, 1, 64, 576, 128, 1, None, None, None, None) == 1   # no kv_cache
    assert "together" in _err(lib)
    assert f(None, 16, 16, 1, 1, 64, 576, 128, 1, None, 16, None, None) == 1     # fp8, no scale
    assert "k_scale" in _err(lib)
    assert f(None, 16, 16, 1, 1, 64, 576, 128, 0, None, 16, 16, None) == 1       # bf16 + scale
    assert f(16, None, 16, 1, 1, 64, 576, 128, 0, 16, None, 16, None) == 1       # scale, no keys
    assert f(16, None, 16, 1, 1, 64, 574, 128, 0, 16, None, None, None) == 2     # d_qk % 4
    assert f(None, 16, 16, 1, 1, 64, 576, 512, 1, None, 16, 16, None) == 2       # D > 256
    assert f(None, 16, 16, 1, 1, 64, 576, 128, 5, None, 16, 16, None) == 1       # dtype
    assert f(16, 16, 16, 1, 100, 64, 576, 128, 1, 16, 16, 16, None) == 1        # T > Lmax
    assert f(16, 16, None, 1, 1, 64, 576, 128, 1, 16, 16, 16, None) == 1        # no ctx_len
    assert f(16, 16, 16, 1, 1, 64, 576, 128, 1, 16, 18, 16, None) == 1          # misaligned
    assert "aligned" in _err(lib)



def test_stream_probe_rejects_bad_arguments(lib):
    f = lib.dsa_probe_stream_read
    # (src, bytes, workgroups, form, sink, stream)
    assert f(None, 8192, 256, 0, 16, None) == 1
    assert "src is NULL" in _err(lib)
    assert f(16, 8192, 256, 0, None, None) == 1
    assert "sink is NULL" in _err(lib)
    assert f(16, 8000, 256, 0, 16, None) == 1              # not whole 8 KB tiles
    assert "multiple of 8192" in _err(lib)
    assert f(16, 0, 256, 0, 16, None) == 1
    assert f(16, 8192, 0, 0, 16, None) == 1                # no workgroups
    assert f(16, 8192, 65537, 1, 16, None) == 1
    assert f(16, 8192, 256, 2, 16, None) == 1              # unknown form
    assert "form" in _err(lib)
    assert f(24, 8192, 256, 0, 16, None) == 1              # misaligned
    assert "aligned" in _err(lib)
    assert f(16, 1 << 32, 1, 0, 16, None) == 2             # one run of 4 GiB
    assert "2^31" in _err(lib)

C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "dsa_indexcache.h"

int main(void) {
  /* a validation error comes back as a status and a message, nothing launched */
  if (dsa_topk(NULL, 4096, NULL, 1, 1, 4096, 8, NULL, NULL, 0, NULL) != DSA_ERR_INVALID_ARG)
    return 1;
  if (strstr(dsa_last_error(), "NULL") == NULL) return 2;
  /* host-only pattern search on a 4-layer cost matrix */
  double c[16] = {0};
  c[1 * 4 + 0] = 0.5;
  c[2 * 4 + 0] = 0.9; c[2 * 4 + 1] = 0.1;
  c[3 * 4 + 0] = 0.8; c[3 * 4 + 1] = 0.7; c[3 * 4 + 2] = 0.2;
  char pats[3 * 5];
  double tot[3];
  if (indexcache_greedy_search(c, 4, 3, pats, tot) != DSA_OK) return 3;
  double one = 0.0;
  if (indexcache_pattern_cost(c, 4, "FFSS", &one) != DSA_OK) return 4;
  dsa_stack_shape_t shape = {1, 1, 64, 128, 4096, 2048, 128, 576, 512, DSA_FP8_E4M3, 0.07f, 0};
  size_t need = 0;
  if (indexcache_stack_workspace_size(&shape, &need) != DSA_OK) return 5;
  printf("%s %s %s %.3f %.3f %zu\n", pats, pats + 5, pats + 10, tot[2], one, need);
  return 0;
}
"""


def test_header_is_plain_c_and_links(lib, tmp_path):
    """The C ABI header compiles as C99 with warnings as errors, and a C program
    linked against the library gets statuses, messages and host-only search
    results through it (no GPU work)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or ROCm headers not available")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src), "-o",
           str(exe), "-L", libdir, "-ldsa_indexcache", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    words = r.stdout.split()
    assert words[:3] == ["FFSF", "FFSS", "FSSS"]
    assert abs(float(words[3]) - 2.2) < 1e-9 and abs(float(words[4]) - 0.8) < 1e-9
    assert int(words[5]) > 0


def test_fused_indexer_topk_host_checks(lib):
    """The fused indexer + top-k takes one-query-row shapes whose rows split
    into at most 1024 workgroup runs, sizes its workspace like the chunked
    top-k (one chunk per workgroup), and rejects bad calls on the host."""
    need = ctypes.c_size_t()
    ws = lib.dsa_indexer_topk_workspace_size
    assert ws(8, 1, 64, 128, _lib.DSA_FP8_E4M3, 131072, 2048, ctypes.byref(need)) == 0
    rows, L, chunks = 8, 131072, 32   # one chunk per workgroup: 8 waves x 8 tiles of 64 keys
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert need.value == (a(rows * 4096 * 4) + a(rows * 12) + a(rows * chunks * 4)
                          + 2 * a(rows * L * 4))
    # 8388608 fp8 keys of D = 128 are 1024 workgroups of 128 tiles; one more
    # tile is not taken
    assert ws(1, 1, 64, 128, _lib.DSA_FP8_E4M3, 8388608, 2048, ctypes.byref(need)) == 0
    assert ws(1, 1, 64, 128, _lib.DSA_FP8_E4M3, 8388608 + 64, 2048,
              ctypes.byref(need)) == _lib.DSA_ERR_UNSUPPORTED
    # several query rows per sequence: the prefill form, candidate lists of
    # Lmax keys and positions per row plus a count per row
    assert ws(1, 16, 64, 128, _lib.DSA_FP8_E4M3, 8192, 2048, ctypes.byref(need)) == 0
    assert need.value == 2 * a(16 * 8192 * 4) + a(16 * 4)
    # the stack fuses decode shapes only, unless told not to
    fz = ctypes.c_int(-1)
    dec = _lib.StackShape(8, 1, 64, 128, 131072, 2048, 0, 576, 512, _lib.DSA_FP8_E4M3, 0.1)
    assert lib.indexcache_stack_fuses_topk(ctypes.byref(dec), ctypes.byref(fz)) == 0
    assert fz.value == 1
    dec.flags = _lib.DSA_STACK_UNFUSED_TOPK
    assert lib.indexcache_stack_fuses_topk(ctypes.byref(dec), ctypes.byref(fz)) == 0
    assert fz.value == 0
    pre = _lib.StackShape(1, 8192, 64, 128, 65536, 2048, 0, 576, 512, _lib.DSA_FP8_E4M3, 0.1)
    assert lib.indexcache_stack_fuses_topk(ctypes.byref(pre), ctypes.byref(fz)) == 0
    assert fz.value == 0
    f = lib.dsa_indexer_topk
    # fp8 without scales; NULL output; workspace too small
    assert f(16, _lib.DSA_FP8_E4M3, None, 16, 16, None, 16, 1, 1, 64, 128, 4096, 64, 16, 16,
             1 << 30, None) == _lib.DSA_ERR_INVALID_ARG
    assert f(16, _lib.DSA_BF16, None, 16, 16, None, 16, 1, 1, 64, 128, 4096, 64, None, 16,
             1 << 30, None) == _lib.DSA_ERR_INVALID_ARG
    assert f(16, _lib.DSA_BF16, None, 16, 16, None, 16, 1, 1, 64, 128, 4096, 64, 16, 16, 8,
             None) == _lib.DSA_ERR_WORKSPACE
    # a stack shape with unknown flags is refused
    p, n, layers, shape = _stack_args("FSSS", 4)
    shape.flags = 6
    st = lib.indexcache_run_stack(p, n, layers, ctypes.byref(shape), 16, 16, 16, 4096, 16,
                                  1 << 30, None, None)
    assert st == _lib.DSA_ERR_INVALID_ARG and "flags" in _err(lib)
