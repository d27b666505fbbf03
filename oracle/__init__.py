"""fp64 CPU oracle for batched draft-token verification (ctypes wrapper).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  It never imports the GPU
library and the GPU library never imports it.

The arithmetic lives in ``oracle.c`` (plain C, double precision); this module
only builds that file with gcc when its shared library is missing and converts
numpy arrays to pointers.  Input dictionaries are the ones produced by the
``workloads`` generators.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BAND_EPS = 1e-5

MUT_NONE = 0
MUT_SAMPLE_TARGET_AT_MISMATCH = 1
MUT_RESIDUAL_SWAPPED = 2
MUT_ROWS_SHIFTED = 3
MUT_ACCEPT_INVERTED = 4
MUT_ARGMAX_LAST = 5
MUT_TREE_TIE_HIGHEST = 6
MUT_TREE_STALE_RESIDUAL = 7


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _lib.svo_set_mutation.argtypes = [ctypes.c_int]
        _lib.svo_set_num_threads.argtypes = [ctypes.c_int]
        _lib.svo_verify_chain.argtypes = (
            [ctypes.c_int] * 4 + [ctypes.c_void_p] * 10 + [ctypes.c_double])
        _lib.svo_verify_greedy.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 4
        _lib.svo_verify_tree.argtypes = (
            [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2 + [ctypes.c_int] * 2 + [ctypes.c_void_p] * 4)
        _lib.svo_verify_tree_sampled.argtypes = (
            [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2 + [ctypes.c_int] * 2 + [ctypes.c_void_p] * 9 +
            [ctypes.c_double])
        _lib.svo_row_logz.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 3
        _lib.svo_row_argmax.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 2
        _lib.svo_commit_tokens.argtypes = ([ctypes.c_int] * 2 + [ctypes.c_void_p] * 4 + [ctypes.c_int] +
                                           [ctypes.c_void_p] * 3)
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    return np.ascontiguousarray(a, dtype=dtype) if a is not None else None


def set_mutation(m: int) -> None:
    """Plant one of the MUT_* mistakes (tests of test power only)."""
    lib().svo_set_mutation(int(m))


def set_num_threads(n: int) -> None:
    lib().svo_set_num_threads(int(n))


def max_threads() -> int:
    return int(lib().svo_max_threads())


def verify_chain(inp: dict, band_eps: float = BAND_EPS) -> dict:
    B, k, V, dt = inp["B"], inp["k"], inp["V"], inp["dtype"]
    x = _c(inp["draft_tokens"], np.int32)
    d = _c(inp["draft_logits"])
    t = _c(inp["target_logits"])
    T = _c(inp["temperature"], np.float32)
    u = _c(inp["uniforms"], np.float32)
    acc = np.empty(B, np.int32)
    em = np.empty((B, k + 1), np.int32)
    ap = np.empty((B, k), np.float64)
    band = np.empty(B, np.int32)
    W = np.empty(B, np.float64)
    rc = lib().svo_verify_chain(B, k, V, dt, _ptr(x), _ptr(d), _ptr(t), _ptr(T), _ptr(u),
                                _ptr(acc), _ptr(em), _ptr(ap), _ptr(band), _ptr(W), float(band_eps))
    if rc != 0:
        raise ValueError(f"svo_verify_chain returned {rc}")
    return dict(accepted_len=acc, emitted=em, accept_prob=ap, band=band.astype(bool), final_mass=W)


def verify_greedy(inp: dict) -> dict:
    B, k, V, dt = inp["B"], inp["k"], inp["V"], inp["dtype"]
    x = _c(inp["draft_tokens"], np.int32)
    t = _c(inp["target_logits"])
    acc = np.empty(B, np.int32)
    em = np.empty((B, k + 1), np.int32)
    rc = lib().svo_verify_greedy(B, k, V, dt, _ptr(x), _ptr(t), _ptr(acc), _ptr(em))
    if rc != 0:
        raise ValueError(f"svo_verify_greedy returned {rc}")
    return dict(accepted_len=acc, emitted=em)


def verify_tree(inp: dict) -> dict:
    B, N, V, dt = inp["B"], inp["N"], inp["V"], inp["dtype"]
    par = _c(inp["parent"], np.int32)
    stride = 0 if par.ndim == 1 else par.shape[1]
    md = int(inp["max_depth"])
    tok = _c(inp["node_tokens"], np.int32)
    t = _c(inp["target_logits"])
    acc = np.empty(B, np.int32)
    em = np.empty((B, md + 1), np.int32)
    nodes = np.empty((B, md + 1), np.int32)
    rc = lib().svo_verify_tree(B, N, V, dt, _ptr(tok), _ptr(par), stride, md, _ptr(t),
                               _ptr(acc), _ptr(em), _ptr(nodes))
    if rc != 0:
        raise ValueError(f"svo_verify_tree returned {rc}")
    return dict(accepted_len=acc, emitted=em, accepted_nodes=nodes)


def verify_tree_sampled(inp: dict, band_eps: float = BAND_EPS) -> dict:
    """Multi-step speculative sampling over a draft tree (see oracle.c)."""
    B, N, V, dt = inp["B"], inp["N"], inp["V"], inp["dtype"]
    par = _c(inp["parent"], np.int32)
    stride = 0 if par.ndim == 1 else par.shape[1]
    md = int(inp["max_depth"])
    tok = _c(inp["node_tokens"], np.int32)
    d = _c(inp["draft_logits"])
    t = _c(inp["target_logits"])
    T = _c(inp["temperature"], np.float32)
    u = _c(inp["uniforms"], np.float32)
    acc = np.empty(B, np.int32)
    em = np.empty((B, md + 1), np.int32)
    nodes = np.empty((B, md + 1), np.int32)
    band = np.empty(B, np.int32)
    mass = np.empty(B, np.float64)
    rc = lib().svo_verify_tree_sampled(B, N, V, dt, _ptr(tok), _ptr(par), stride, md, _ptr(d), _ptr(t), _ptr(T),
                                       _ptr(u), _ptr(acc), _ptr(em), _ptr(nodes), _ptr(band), _ptr(mass),
                                       float(band_eps))
    if rc != 0:
        raise ValueError(f"svo_verify_tree_sampled returned {rc}")
    return dict(accepted_len=acc, emitted=em, accepted_nodes=nodes, band=band.astype(bool), final_mass=mass)


def row_logz(logits: np.ndarray, dtype: int, temperature) -> np.ndarray:
    """log sum_v exp(l_v / T) for every row of ``logits[..., V]``."""
    V = logits.shape[-1]
    rows = _c(logits.reshape(-1, V))
    n = rows.shape[0]
    T = np.broadcast_to(np.asarray(temperature, np.float32), (n,)).copy()
    out = np.empty(n, np.float64)
    if lib().svo_row_logz(n, V, dtype, _ptr(rows), _ptr(T), _ptr(out)) != 0:
        raise ValueError("svo_row_logz failed")
    return out.reshape(logits.shape[:-1])


def row_argmax(logits: np.ndarray, dtype: int) -> np.ndarray:
    V = logits.shape[-1]
    rows = _c(logits.reshape(-1, V))
    out = np.empty(rows.shape[0], np.int32)
    if lib().svo_row_argmax(rows.shape[0], V, dtype, _ptr(rows), _ptr(out)) != 0:
        raise ValueError("svo_row_argmax failed")
    return out.reshape(logits.shape[:-1])


def commit_tokens(accepted_len, emitted, seq_len, history=None) -> dict:
    """Returns the updated seq_len and history and the packed layout."""
    acc = _c(accepted_len, np.int32)
    em = _c(emitted, np.int32)
    B, width = em.shape
    sl = np.array(seq_len, dtype=np.int32, copy=True)
    hist = None if history is None else np.array(history, dtype=np.int32, copy=True)
    stride = 0 if hist is None else hist.shape[1]
    offs = np.empty(B + 1, np.int32)
    packed = np.full(B * width, -7, np.int32)
    status = np.empty(B, np.int32)
    rc = lib().svo_commit_tokens(B, width, _ptr(acc), _ptr(em), _ptr(sl), _ptr(hist), stride, _ptr(offs),
                                 _ptr(packed), _ptr(status))
    if rc != 0:
        raise ValueError(f"svo_commit_tokens returned {rc}")
    return dict(seq_len=sl, history=hist, packed_offsets=offs, packed=packed[:offs[B]], status=status)
