"""ctypes front end of the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It never touches the GPU library and the
GPU library never touches it.  Inputs are widened to fp64 here (bf16 and fp32
values widen exactly); every result is fp64 unless stated otherwise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

FAR_FIXED_OFFSET = 0
FAR_UNROTATED = 1
ENOTSPD = -4

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_lp = ctypes.POINTER(ctypes.c_int64)
_up = ctypes.POINTER(ctypes.c_uint16)
_i64 = ctypes.c_int64


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.orc_second_moment.argtypes = [_dp, _i64, _i64, ctypes.c_double, _dp]
        L.orc_cholesky.argtypes = [_dp, _i64, _dp]
        L.orc_assign_h.argtypes = [_dp, _i64, _i64, _dp, _i64, _dp, _ip, _dp, _dp]
        L.orc_assign_cosine.argtypes = [_dp, _i64, _i64, _dp, _i64, _dp, _i64, ctypes.c_double,
                                        _ip, _dp, _dp]
        L.orc_retrieval_count.argtypes = [_i64, ctypes.c_double]
        L.orc_retrieval_count.restype = _i64
        L.orc_select_retrieval.argtypes = [_dp, _i64, _i64, _dp, ctypes.c_double, _ip, _ip, _dp]
        L.orc_reconstruct.argtypes = [_up, _ip, _i64, _i64, _dp, _i64, _i64, _i64, _i64,
                                      ctypes.c_int, ctypes.c_double, _dp, _lp]
        L.orc_rope_at.argtypes = [_dp, _i64, _i64, ctypes.c_double, ctypes.c_double, _dp]
        L.orc_kmeans_update.argtypes = [_dp, _i64, _i64, _ip, _i64, _dp, _dp, _lp]
        L.orc_kmeans.argtypes = [_dp, _i64, _i64, _i64, _dp, ctypes.c_int, _dp, _ip]
        L.orc_kmeans_init.argtypes = [_dp, _i64, _i64, _i64, _dp, ctypes.POINTER(ctypes.c_uint64), _ip]
        L.orc_topk_codes.argtypes = [_dp, _i64, _up, _i64, _dp, _i64, _i64, _ip, _dp]
        L.orc_round_bf16.argtypes = [_dp, _i64, _up]
        for f in (L.orc_second_moment, L.orc_cholesky, L.orc_assign_h, L.orc_assign_cosine,
                  L.orc_select_retrieval, L.orc_reconstruct, L.orc_rope_at,
                  L.orc_kmeans_update, L.orc_kmeans, L.orc_kmeans_init, L.orc_topk_codes):
            f.restype = ctypes.c_int
        L.orc_round_bf16.restype = None
        L.orc_threads.argtypes, L.orc_threads.restype = [], ctypes.c_int
        _LIB = L
    return _LIB


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, t):
    return a.ctypes.data_as(t) if a is not None else None


class OracleError(RuntimeError):
    def __init__(self, status):
        super().__init__("oracle status %d" % status)
        self.status = status


def _check(st):
    if st != 0:
        raise OracleError(st)


# ----------------------------------------------------------------- calibrate
def second_moment(q, ridge=1e-4):
    q = _f64(q)
    m, d = q.shape
    h = np.empty((d, d))
    _check(lib().orc_second_moment(_ptr(q, _dp), m, d, float(ridge), _ptr(h, _dp)))
    return h


def cholesky(h):
    h = _f64(h)
    d = h.shape[0]
    l = np.empty((d, d))
    _check(lib().orc_cholesky(_ptr(h, _dp), d, _ptr(l, _dp)))
    return l


def calibrate(queries, ridge=1e-4):
    """Per head: H in fp64 rounded to fp32 (the array a2ats_query_second_moment returns),
    then L = cholesky(that fp32 H) in fp64, rounded to fp32."""
    queries = np.asarray(queries)
    heads = queries.shape[0]
    d = queries.shape[2]
    H = np.empty((heads, d, d), np.float32)
    L = np.empty((heads, d, d), np.float32)
    for h in range(heads):
        H[h] = second_moment(queries[h], ridge).astype(np.float32)
        L[h] = cholesky(H[h]).astype(np.float32)
    return H, L


# ----------------------------------------------------------------- encode
def assign_h(x, cb, l=None):
    """x [n,d], cb [c,d], l [d,d] or None -> (code int32 [n], d1 [n], d2 [n])."""
    x = _f64(x)
    cb = _f64(cb)
    n, d = x.shape
    c = cb.shape[0]
    lf = _f64(l) if l is not None else None
    code = np.empty(n, np.int32)
    d1 = np.empty(n)
    d2 = np.empty(n)
    _check(lib().orc_assign_h(_ptr(x, _dp), n, d, _ptr(cb, _dp), c, _ptr(lf, _dp),
                              _ptr(code, _ip), _ptr(d1, _dp), _ptr(d2, _dp)))
    return code, d1, d2


def assign_cosine(x, q, cb, beta):
    """x [n,d], q [nq,d] (nq in {1,n}) or [d], cb [c,d] -> (code, s1, s2)."""
    x = _f64(x)
    q = _f64(q)
    if q.ndim == 1:
        q = q[None, :]
    cb = _f64(cb)
    n, d = x.shape
    code = np.empty(n, np.int32)
    s1 = np.empty(n)
    s2 = np.empty(n)
    _check(lib().orc_assign_cosine(_ptr(x, _dp), n, d, _ptr(q, _dp), q.shape[0], _ptr(cb, _dp),
                                   cb.shape[0], float(beta), _ptr(code, _ip), _ptr(s1, _dp),
                                   _ptr(s2, _dp)))
    return code, s1, s2


# ----------------------------------------------------------------- split
def retrieval_count(n, fraction):
    return int(lib().orc_retrieval_count(int(n), float(fraction)))


def select_retrieval(keys, q, fraction):
    """keys [n,d], q [d] -> (retrieval_idx ascending, bulk_idx ascending, cosine [n])."""
    keys = _f64(keys)
    q = _f64(q).reshape(-1)
    n, d = keys.shape
    nr = retrieval_count(n, fraction)
    if nr < 0:
        raise OracleError(-1)
    ret = np.empty(max(nr, 0), np.int32)
    bulk = np.empty(n - nr, np.int32)
    cosv = np.empty(n)
    _check(lib().orc_select_retrieval(_ptr(keys, _dp), n, d, _ptr(q, _dp), float(fraction),
                                      _ptr(ret, _ip), _ptr(bulk, _ip), _ptr(cosv, _dp)))
    return ret, bulk, cosv


# ----------------------------------------------------------------- reconstruct
def reconstruct(codes, positions, cb, cur, window, far_b=2048, far_mode=FAR_FIXED_OFFSET,
                base=10000.0):
    """codes [n] uint16, positions [n] int32, cb [c,d] -> (out fp64 [n,d], far_count)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint16)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    cb = _f64(cb)
    n = codes.shape[0]
    c, d = cb.shape
    out = np.empty((n, d))
    far = np.zeros(1, np.int64)
    _check(lib().orc_reconstruct(_ptr(codes, _up), _ptr(pos, _ip), n, d, _ptr(cb, _dp), c,
                                 int(cur), int(window), int(far_b), int(far_mode), float(base),
                                 _ptr(out, _dp), _ptr(far, _lp)))
    return out, int(far[0])


def rope_at(x, position, base=10000.0):
    """Rows of x [rows, d] rotated as tokens at `position` (the query-side R_b of Eq. 11 when
    position = b) -> fp64 [rows, d]."""
    x = _f64(x)
    rows, d = x.shape
    out = np.empty((rows, d))
    _check(lib().orc_rope_at(_ptr(x, _dp), rows, d, float(position), float(base), _ptr(out, _dp)))
    return out


def kmeans_update(x, code, cb):
    """x [n,d], code [n] (int), cb [k,d] -> (new cb fp64 [k,d], counts int64 [k])."""
    x = _f64(x)
    cb = _f64(cb)
    code = np.ascontiguousarray(code, dtype=np.int32)
    n, d = x.shape
    k = cb.shape[0]
    out = np.empty((k, d))
    cnt = np.empty(k, np.int64)
    _check(lib().orc_kmeans_update(_ptr(x, _dp), n, d, _ptr(code, _ip), k, _ptr(cb, _dp),
                                   _ptr(out, _dp), _ptr(cnt, _lp)))
    return out, cnt


def kmeans(x, cb, l=None, iters=5):
    """Lloyd's iterations from cb (H-weighted with l) -> (cb fp64 [k,d], final code [n])."""
    x = _f64(x)
    cb = _f64(cb).copy()
    n, d = x.shape
    k = cb.shape[0]
    lf = _f64(l) if l is not None else None
    code = np.empty(n, np.int32)
    _check(lib().orc_kmeans(_ptr(x, _dp), n, d, k, _ptr(lf, _dp), int(iters), _ptr(cb, _dp),
                            _ptr(code, _ip)))
    return cb, code


def kmeans_init(x, k, r, l=None):
    """k-means++ seeding in z-space: x [n,d], k centers, r [k] uint64 draws, l [d,d] or None
    -> idx int32 [k] (the rows chosen as centers, in order)."""
    x = _f64(x)
    n, d = x.shape
    r = np.ascontiguousarray(r, dtype=np.uint64)
    if r.shape != (k,):
        raise ValueError("r must hold k draws")
    lf = _f64(l) if l is not None else None
    idx = np.empty(k, np.int32)
    _check(lib().orc_kmeans_init(_ptr(x, _dp), n, d, int(k), _ptr(lf, _dp),
                                 r.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), _ptr(idx, _ip)))
    return idx


def topk_codes(qb, codes, cb, k):
    """qb [d] (= q R_b), codes [n] uint16, cb [c,d], k -> (idx int32 [k] ascending,
    score fp64 [k])."""
    qb = _f64(qb).reshape(-1)
    codes = np.ascontiguousarray(codes, dtype=np.uint16)
    cb = _f64(cb)
    n = codes.shape[0]
    c, d = cb.shape
    idx = np.empty(k, np.int32)
    sc = np.empty(k)
    _check(lib().orc_topk_codes(_ptr(qb, _dp), d, _ptr(codes, _up), n, _ptr(cb, _dp), c, int(k),
                                _ptr(idx, _ip), _ptr(sc, _dp)))
    return idx, sc


def round_bf16(x):
    """fp64 -> raw bf16 bits (nearest, ties to even), same shape."""
    x = _f64(x)
    out = np.empty(x.shape, np.uint16)
    lib().orc_round_bf16(_ptr(x.reshape(-1), _dp), x.size, _ptr(out.reshape(-1), _up))
    return out


def threads() -> int:
    return int(lib().orc_threads())
