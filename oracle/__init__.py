"""fp64 CPU oracle for exact attention and its gradient (ctypes over liboracle.so).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the GPU library, and the GPU library never calls it.

Every function takes numpy arrays shaped ``[..., N, d]`` (any leading batch and
head dimensions), converts them to contiguous float64 and evaluates the plain
definition slice by slice in C (see ``oracle.c`` for the formulas and the
passages of the pages they follow).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    lib.oracle_fwd_rows.argtypes = [ctypes.c_int, _ip, _dp, ctypes.c_int, _dp, _dp,
                                    ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                    _dp, _dp, _dp]
    lib.oracle_fwd_rows.restype = ctypes.c_int
    lib.oracle_fwd.argtypes = [ctypes.c_int, _dp, _dp, _dp, ctypes.c_int,
                               ctypes.c_double, ctypes.c_int, _dp, _dp]
    lib.oracle_fwd.restype = ctypes.c_int
    lib.oracle_bwd.argtypes = [ctypes.c_int, _dp, _dp, _dp, _dp, ctypes.c_int,
                               ctypes.c_double, ctypes.c_int, _dp, _dp, _dp, _dp,
                               _dp, _dp]
    lib.oracle_bwd.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_lse_merge.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp,
                                     _dp]
    lib.oracle_lse_merge.restype = ctypes.c_int
    lib.oracle_set_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a):
    return a.ctypes.data_as(_dp)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def num_threads() -> int:
    """OpenMP threads the oracle uses."""
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> int:
    return _load().oracle_set_num_threads(int(n))


def attention_fwd(q, k, v, scale, causal):
    """O = softmax(scale*Q K^T [+ causal mask]) V and LSE per row, in fp64.

    q, k, v: [..., N, d]. Returns (o [..., N, d], lse [..., N])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, N, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    lib = _load()
    qs, ks, vs = q.reshape(-1, N, d), k.reshape(-1, N, d), v.reshape(-1, N, d)
    o = np.empty_like(qs)
    lse = np.empty(qs.shape[:2], dtype=np.float64)
    for s in range(qs.shape[0]):
        _check(lib.oracle_fwd(N, _p(qs[s]), _p(ks[s]), _p(vs[s]), d, float(scale),
                              int(bool(causal)), _p(o[s]), _p(lse[s])), "fwd")
    return o.reshape(*lead, N, d), lse.reshape(*lead, N)


def attention_fwd_rows(q_rows, qpos, k, v, scale, causal, return_p=False):
    """Forward for selected query rows of ONE slice.

    q_rows: [M, d] query vectors; qpos: [M] their positions (for the causal
    mask); k, v: [N, d]. Returns (o [M, d], lse [M]) and P [M, N] if asked."""
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    qpos = np.ascontiguousarray(np.asarray(qpos, dtype=np.int32))
    M, d = q_rows.shape
    N = k.shape[0]
    o = np.empty((M, d), dtype=np.float64)
    lse = np.empty(M, dtype=np.float64)
    P = np.empty((M, N), dtype=np.float64) if return_p else None
    rc = _load().oracle_fwd_rows(M, qpos.ctypes.data_as(_ip), _p(q_rows), N, _p(k),
                                 _p(v), d, float(scale), int(bool(causal)), _p(o),
                                 _p(lse), _p(P) if return_p else None)
    _check(rc, "fwd_rows")
    return (o, lse, P) if return_p else (o, lse)


def lse_merge(o_parts, lse_parts):
    """Merge partial attention results over disjoint key sets, in fp64.

    o_parts: [P, rows, d] normalised partial outputs; lse_parts: [P, rows]
    their log-normalisers (-inf for a part with no visible key). Returns
    (o [rows, d], lse [rows])."""
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    P, rows, d = o_parts.shape
    assert lse_parts.shape == (P, rows)
    o = np.empty((rows, d), dtype=np.float64)
    lse = np.empty(rows, dtype=np.float64)
    _check(_load().oracle_lse_merge(P, rows, d, _p(o_parts), _p(lse_parts), _p(o), _p(lse)),
           "lse_merge")
    return o, lse


def attention_bwd(q, k, v, do, scale, causal, return_ds=False):
    """Gradients of the attention forward with upstream gradient dO, in fp64.

    Returns dict with dq, dk, dv ([..., N, d]), D = rowsum(dP o P) and
    Dprime = rowsum(dO o O) ([..., N]), and dS ([..., N, N]) if asked."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    *lead, N, d = q.shape
    lib = _load()
    qs, ks, vs, gs = (x.reshape(-1, N, d) for x in (q, k, v, do))
    nb = qs.shape[0]
    dq, dk, dv = np.empty_like(qs), np.empty_like(qs), np.empty_like(qs)
    D = np.empty((nb, N)); Dp = np.empty((nb, N))
    dS = np.empty((nb, N, N)) if return_ds else None
    for s in range(nb):
        rc = lib.oracle_bwd(N, _p(qs[s]), _p(ks[s]), _p(vs[s]), _p(gs[s]), d,
                            float(scale), int(bool(causal)), _p(dq[s]), _p(dk[s]),
                            _p(dv[s]), _p(D[s]), _p(Dp[s]),
                            _p(dS[s]) if return_ds else None)
        _check(rc, "bwd")
    out = {"dq": dq.reshape(*lead, N, d), "dk": dk.reshape(*lead, N, d),
           "dv": dv.reshape(*lead, N, d), "D": D.reshape(*lead, N),
           "Dprime": Dp.reshape(*lead, N)}
    if return_ds:
        out["dS"] = dS.reshape(*lead, N, N)
    return out
