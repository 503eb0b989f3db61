"""The host-side pattern search of the C ABI against the oracle (CPU only:
these entry points take host memory and launch nothing)."""
import math
import os

import numpy as np
import pytest

import oracle
import dsa_sparse_attention_lightning_amd as dsa
from dsa_sparse_attention_lightning_amd import _lib


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    return _lib.load()


def _matrix(r, n, ties=0.0, infs=0.0):
    C = np.tril(r.uniform(0, 1, (n, n)), -1)
    if ties:
        C = np.round(C * 4) / 4                       # few distinct values: many equal costs
    if infs:
        C[np.tril(r.uniform(size=(n, n)) < infs, -1)] = math.inf
    return C


@pytest.mark.parametrize("n", [1, 2, 3, 8, 17, 48])
@pytest.mark.parametrize("kind", ["plain", "ties", "inf", "diag"])
def test_greedy_equals_oracle(lib, n, kind):
    r = np.random.default_rng(100 + n)
    C = _matrix(r, n, ties=kind == "ties", infs=0.1 if kind == "inf" else 0.0)
    if kind == "diag":                                 # arbitrary matrices: diagonal counts too
        C = C + np.diag(r.uniform(0, 1, n))
    for m in sorted({0, 1, n // 2, n - 1} & set(range(n))):
        assert dsa.greedy_search(C, m) == oracle.greedy_pattern_search(C, m)


def test_pattern_cost_equals_oracle(lib):
    r = np.random.default_rng(7)
    C = _matrix(r, 12)
    for _ in range(50):
        p = "F" + "".join(r.choice(["F", "S"], 11))
        assert dsa.pattern_cost(C, p) == oracle.pattern_cost(p, C)


def test_search_rejects_bad_arguments(lib):
    C = np.zeros((4, 4))
    with pytest.raises(dsa.DSAError, match="n_shared"):
        dsa.greedy_search(C, 4)
    with pytest.raises(dsa.DSAError, match="start with"):
        dsa.pattern_cost(C, "SFFF")
    with pytest.raises(dsa.DSAError, match="length"):
        dsa.pattern_cost(C, "FFF")
    C[2, 1] = math.nan
    with pytest.raises(dsa.DSAError, match="NaN"):
        dsa.greedy_search(C, 1)


def test_reuse_costs_rejects_bad_arguments(lib):
    import ctypes
    shape = _lib.StackShape(1, 1, 64, 128, 4096, 2048, 0, 576, 512, 0, 0.1)
    need = ctypes.c_size_t()
    # the output proxy needs attention heads
    assert lib.indexcache_reuse_costs_workspace_size(ctypes.byref(shape), 4, 0,
                                                     ctypes.byref(need)) == 1
    assert lib.indexcache_reuse_costs_workspace_size(ctypes.byref(shape), 4, 1,
                                                     ctypes.byref(need)) == 0
    assert lib.indexcache_reuse_costs_workspace_size(ctypes.byref(shape), 4, 9,
                                                     ctypes.byref(need)) == 1
    big = _lib.StackShape(1, 1, 64, 128, 65536, 16384, 0, 576, 512, 0, 0.1)
    assert lib.indexcache_reuse_costs_workspace_size(ctypes.byref(big), 4, 1,
                                                     ctypes.byref(need)) == 2   # k > 8192
    assert lib.indexcache_reuse_costs_workspace_size(ctypes.byref(shape), 4, 1,
                                                     ctypes.byref(need)) == 0
    layers = (_lib.Layer * 4)()
    st = lib.indexcache_reuse_costs(4, layers, ctypes.byref(shape), 16, 1, 16, 16, 4096, 16,
                                    need.value - 1, None)
    assert st == _lib.DSA_ERR_WORKSPACE
