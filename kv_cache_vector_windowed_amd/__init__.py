"""A2ATS key-cache hot path on MI355X (gfx950): Python binding of liba2ats.so.

Every function here only marshals arguments: it checks tensor placement, dtypes and shapes,
allocates outputs and the workspace with torch on the same device, and calls the C ABI
declared in include/a2ats.h on torch's current HIP stream.  All computation happens in the
library's kernels.  If the library has not been built, the functions raise.

Operations (see include/a2ats.h for the exact contracts):
    calibrate(queries, ridge)            -> (H, L)
    encode(keys, codebook, chol, ...)    -> codes [, dist]
    assign_cosine(x, query, codebook, beta) -> codes
    select_retrieval(keys, query, fraction) -> (retrieval_idx, bulk_idx)
    reconstruct(codes, positions, codebook, cur_pos, window, ...) -> rotated keys
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liba2ats.so")

F32, BF16 = 0, 1
FAR_FIXED_OFFSET, FAR_UNROTATED = 0, 1
HEAD_DIM = 128
STATUS = {0: "ok", -1: "EINVAL", -2: "EDTYPE", -3: "EWORKSPACE", -4: "ENOTSPD", -5: "EHIP",
          -6: "ESCRATCH"}
NOALLOC_TABLE_ROWS = 8192  # A2ATS_NOALLOC_TABLE_ROWS: windows up to 8191 tokens

_lib = None


class A2ATSError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, STATUS.get(status, "?"), status))


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("liba2ats.so is not built (run __graft_entry__.build() or "
                               "python kv_cache_vector_windowed_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, sz, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t, ctypes.c_double
        L.a2ats_strerror.argtypes, L.a2ats_strerror.restype = [i32], ctypes.c_char_p
        L.a2ats_version.argtypes, L.a2ats_version.restype = [], i32
        L.a2ats_retrieval_count.argtypes, L.a2ats_retrieval_count.restype = [i64, dbl], i64
        L.a2ats_calibrate_workspace.argtypes, L.a2ats_calibrate_workspace.restype = [i64, i64, i64], sz
        L.a2ats_calibrate.argtypes = [p, i64, i64, i64, dbl, p, p, p, sz, p]
        L.a2ats_encode_workspace.argtypes, L.a2ats_encode_workspace.restype = [i64, i64, i64, i64], sz
        L.a2ats_encode.argtypes = [p, i32, i64, i64, i64, p, i64, p, i64, p, p, p, p, p, sz, p]
        L.a2ats_encode_prepare.argtypes = [p, i64, p, i64, i64, i64, p, sz, p]
        L.a2ats_encode_prepared.argtypes = [p, i32, i64, i64, i64, p, i64, i64, p, p, p, p, p, sz, p]
        L.a2ats_merge_codes.argtypes = [p, p, i64, i64, i64, p, p]
        L.a2ats_assign_cosine_workspace.argtypes = [i64, i64, i64]
        L.a2ats_assign_cosine_workspace.restype = sz
        L.a2ats_assign_cosine.argtypes = [p, i32, i64, i64, i64, p, i64, p, i64, dbl, p, p, sz, p]
        L.a2ats_select_retrieval_workspace.argtypes = [i64, i64]
        L.a2ats_select_retrieval_workspace.restype = sz
        L.a2ats_select_retrieval.argtypes = [p, i32, i64, i64, i64, p, dbl, p, p, p, sz, p]
        L.a2ats_reconstruct_workspace.argtypes = [i64, i64, i64, i64, i64, i32]
        L.a2ats_reconstruct_workspace.restype = sz
        L.a2ats_pq_reconstruct_workspace.argtypes = [i64, i64, i64]
        L.a2ats_pq_reconstruct_workspace.restype = sz
        L.a2ats_reconstruct.argtypes = [p, p, i64, i64, i64, i64, p, i64, i64, i64, i64, i32, dbl,
                                        p, i32, p, sz, p]
        L.a2ats_reconstruct_noalloc.argtypes = [p, p, i64, i64, i64, i64, p, i64, i64, i64, i64,
                                                i32, dbl, p, i32, p]
        L.a2ats_reconstruct_update.argtypes = [p, p, i64, i64, i64, i64, p, i64, i64, i64, i64,
                                               i64, dbl, p, i32, p]
        L.a2ats_far_query_rope.argtypes = [p, i32, i64, i64, i64, dbl, p, i32, p]
        L.a2ats_pq_encode.argtypes = [p, i32, i64, i64, i64, i64, p, i64, p, i64, p, p, i64, dbl, p, p]
        L.a2ats_pq_reconstruct.argtypes = [p, p, i64, i64, i64, i64, i64, p, i64, i64, i64, i64, i32,
                                           dbl, p, i32, p, sz, p]
        L.a2ats_pq_accounting.argtypes = [i64, i64, i64, i64, i32, p, p, p, p, p]
        L.a2ats_pq_accounting.restype = i32
        L.a2ats_kmeans_update_workspace.argtypes = [i64, i64, i64]
        L.a2ats_kmeans_update_workspace.restype = sz
        L.a2ats_kmeans_update.argtypes = [p, i32, i64, i64, i64, p, i32, i64, p, p, p, p, sz, p]
        L.a2ats_kmeans_workspace.argtypes = [i64, i64, i64, i64]
        L.a2ats_kmeans_workspace.restype = sz
        L.a2ats_kmeans.argtypes = [p, i32, i64, i64, i64, i64, p, i32, p, p, p, sz, p]
        L.a2ats_kmeans_init_workspace.argtypes = [i64, i64, i64, i64]
        L.a2ats_kmeans_init_workspace.restype = sz
        L.a2ats_kmeans_init.argtypes = [p, i32, i64, i64, i64, i64, p, p, p, p, p, sz, p]
        L.a2ats_topk_workspace.argtypes = [i64, i64, i64]
        L.a2ats_topk_workspace.restype = sz
        L.a2ats_topk_codes.argtypes = [p, i32, i64, i64, i64, i64, p, i64, p, i64, i64, p, p, p,
                                       sz, p]
        L.a2ats_profile_enable.argtypes, L.a2ats_profile_enable.restype = [i32], i32
        L.a2ats_profile_reset.argtypes, L.a2ats_profile_reset.restype = [], i32
        L.a2ats_profile_read.argtypes, L.a2ats_profile_read.restype = [ctypes.c_char_p, sz], i64
        for f in ("a2ats_calibrate", "a2ats_encode", "a2ats_encode_prepare", "a2ats_encode_prepared",
                  "a2ats_assign_cosine",
                  "a2ats_select_retrieval", "a2ats_reconstruct", "a2ats_reconstruct_noalloc",
                  "a2ats_reconstruct_update",
                  "a2ats_far_query_rope", "a2ats_pq_encode", "a2ats_pq_reconstruct",
                  "a2ats_kmeans_update", "a2ats_kmeans", "a2ats_kmeans_init", "a2ats_topk_codes"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        raise A2ATSError(status, what)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("expected float32 or bfloat16, got %s" % t.dtype)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns blocks aligned to at least 512 bytes
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def retrieval_count(n: int, fraction: float) -> int:
    """ceil(fraction * n) in fp64; -1 for an invalid fraction."""
    return int(lib().a2ats_retrieval_count(int(n), float(fraction)))


def calibrate(queries: torch.Tensor, ridge: float = 1e-4):
    """queries [heads, m, d] fp32 -> (H [heads, d, d], L [heads, d, d]) fp32.  Waits."""
    _dev(queries, "queries")
    if queries.dtype != torch.float32 or queries.dim() != 3:
        raise ValueError("queries must be [heads, m, d] float32")
    heads, m, d = queries.shape
    h = torch.empty((heads, d, d), dtype=torch.float32, device=queries.device)
    l = torch.empty_like(h)
    ws = _workspace(lib().a2ats_calibrate_workspace(heads, m, d), queries.device)
    _check(lib().a2ats_calibrate(_ptr(queries), heads, m, d, float(ridge), _ptr(h), _ptr(l),
                                 _ptr(ws), ws.numel(), _stream(queries.device)), "calibrate")
    return h, l


def encode(keys: torch.Tensor, codebook: torch.Tensor, chol: torch.Tensor | None = None,
           idx: torch.Tensor | None = None, codes: torch.Tensor | None = None,
           want_dist: bool = False, stats: torch.Tensor | None = None,
           dist: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Nearest-centroid codes under H = L L^T (plain when chol is None).

    keys [heads, n, d] fp32/bf16, codebook [heads, c, d] fp32, chol [heads, d, d] fp32,
    idx [heads, n_idx] int32 rows to encode (others of `codes` untouched), codes [heads, n]
    uint16 to write into (allocated when None).  Returns codes, or (codes, dist) with
    want_dist (dist [heads, n] fp32 is written into `dist` when given).  stats: optional
    int32 tensor of 8 elements receiving a2ats_encode_stats.  workspace: an optional uint8
    device tensor of at least encode_workspace_bytes() bytes (allocated when None).
    """
    _dev(keys, "keys")
    _dev(codebook, "codebook")
    heads, n, d = keys.shape
    c = codebook.shape[1]
    if codebook.dtype != torch.float32 or codebook.shape != (heads, c, d):
        raise ValueError("codebook must be [heads, c, d] float32")
    if chol is not None:
        _dev(chol, "chol")
        if chol.dtype != torch.float32 or chol.shape != (heads, d, d):
            raise ValueError("chol must be [heads, d, d] float32")
    n_idx = 0
    if idx is not None:
        _dev(idx, "idx")
        if idx.dtype != torch.int32 or idx.dim() != 2 or idx.shape[0] != heads:
            raise ValueError("idx must be [heads, n_idx] int32")
        n_idx = idx.shape[1]
    if codes is None:
        codes = torch.zeros((heads, n), dtype=torch.uint16, device=keys.device)
    else:
        _dev(codes, "codes")
    if dist is not None:
        _dev(dist, "dist")
        if dist.dtype != torch.float32 or dist.shape != (heads, n):
            raise ValueError("dist must be [heads, n] float32")
        want_dist = True
    elif want_dist:
        dist = torch.zeros((heads, n), dtype=torch.float32, device=keys.device)
    if stats is not None:
        _dev(stats, "stats")
    need = lib().a2ats_encode_workspace(heads, n, d, c)
    if workspace is None:
        ws = _workspace(need, keys.device)
    else:
        ws = _dev(workspace, "workspace")
        if ws.dtype != torch.uint8 or ws.numel() < need:
            raise ValueError("workspace must be uint8 with at least %d bytes" % need)
    _check(lib().a2ats_encode(_ptr(keys), _dtype_code(keys), heads, n, d, _ptr(idx), n_idx,
                              _ptr(codebook), c, _ptr(chol), _ptr(codes), _ptr(dist),
                              _ptr(stats), _ptr(ws), ws.numel(), _stream(keys.device)), "encode")
    return (codes, dist) if want_dist else codes


class PreparedCodebook:
    """A codebook (and optional L) prepared for encoding `n` keys per head: the workspace of
    a2ats_encode_prepare, reused by every encode_prepared call.  Keep the object alive while
    work that uses it is queued on any stream."""

    def __init__(self, codebook: torch.Tensor, chol: torch.Tensor | None, n: int):
        _dev(codebook, "codebook")
        heads, c, d = codebook.shape
        self.heads, self.c, self.d, self.n = heads, c, d, int(n)
        self.ws = _workspace(lib().a2ats_encode_workspace(heads, self.n, d, c), codebook.device)
        self.prepare(codebook, chol)

    def prepare(self, codebook: torch.Tensor, chol: torch.Tensor | None):
        """(Re)run the codebook side into this workspace, on the current stream."""
        _dev(codebook, "codebook")
        if codebook.dtype != torch.float32 or codebook.shape != (self.heads, self.c, self.d):
            raise ValueError("codebook must be [%d, %d, %d] float32" % (self.heads, self.c, self.d))
        if chol is not None:
            _dev(chol, "chol")
            if chol.dtype != torch.float32 or chol.shape != (self.heads, self.d, self.d):
                raise ValueError("chol must be [heads, d, d] float32")
        self.chol = chol
        _check(lib().a2ats_encode_prepare(_ptr(codebook), self.c, _ptr(chol), self.heads, self.n,
                                          self.d, _ptr(self.ws), self.ws.numel(),
                                          _stream(codebook.device)), "encode_prepare")
        return self


def encode_prepare(codebook: torch.Tensor, chol: torch.Tensor | None, n: int) -> PreparedCodebook:
    """Codebook side of encode (depends on codebook and L only), on the current stream."""
    return PreparedCodebook(codebook, chol, n)


def encode_workspace_bytes(heads: int, n: int, c: int, d: int = HEAD_DIM) -> int:
    """Bytes of the caller workspace that encode() needs for these sizes."""
    return int(lib().a2ats_encode_workspace(heads, n, d, c))


def encode_prepared(keys: torch.Tensor, prep: PreparedCodebook, idx: torch.Tensor | None = None,
                    codes: torch.Tensor | None = None, want_dist: bool = False,
                    stats: torch.Tensor | None = None, dist: torch.Tensor | None = None):
    """Key side of encode with a prepared codebook (keys [heads, n, d], n == prep.n); the
    other arguments and the result as for encode()."""
    _dev(keys, "keys")
    heads, n, d = keys.shape
    if (heads, n, d) != (prep.heads, prep.n, prep.d):
        raise ValueError("keys must be [%d, %d, %d]" % (prep.heads, prep.n, prep.d))
    n_idx = 0
    if idx is not None:
        _dev(idx, "idx")
        if idx.dtype != torch.int32 or idx.dim() != 2 or idx.shape[0] != heads:
            raise ValueError("idx must be [heads, n_idx] int32")
        n_idx = idx.shape[1]
    if codes is None:
        codes = torch.zeros((heads, n), dtype=torch.uint16, device=keys.device)
    else:
        _dev(codes, "codes")
    if dist is not None:
        _dev(dist, "dist")
        if dist.dtype != torch.float32 or dist.shape != (heads, n):
            raise ValueError("dist must be [heads, n] float32")
        want_dist = True
    elif want_dist:
        dist = torch.zeros((heads, n), dtype=torch.float32, device=keys.device)
    if stats is not None:
        _dev(stats, "stats")
    _check(lib().a2ats_encode_prepared(_ptr(keys), _dtype_code(keys), heads, n, d, _ptr(idx), n_idx,
                                       prep.c, _ptr(prep.chol), _ptr(codes), _ptr(dist),
                                       _ptr(stats), _ptr(prep.ws), prep.ws.numel(),
                                       _stream(keys.device)), "encode_prepared")
    return (codes, dist) if want_dist else codes


def assign_cosine(x: torch.Tensor, query: torch.Tensor, codebook: torch.Tensor, beta: float):
    """x [heads, n, d], query [heads, nq, d] (nq in {1, n}), codebook [heads, c, d] -> codes."""
    _dev(x, "x")
    _dev(query, "query")
    _dev(codebook, "codebook")
    heads, n, d = x.shape
    if query.dtype != x.dtype or query.dim() != 3 or query.shape[0] != heads:
        raise ValueError("query must be [heads, nq, d] in the dtype of x")
    codes = torch.zeros((heads, n), dtype=torch.uint16, device=x.device)
    ws = _workspace(lib().a2ats_assign_cosine_workspace(heads, n, codebook.shape[1]), x.device)
    _check(lib().a2ats_assign_cosine(_ptr(x), _dtype_code(x), heads, n, d, _ptr(query),
                                     query.shape[1], _ptr(codebook), codebook.shape[1],
                                     float(beta), _ptr(codes), _ptr(ws), ws.numel(),
                                     _stream(x.device)), "assign_cosine")
    return codes


def merge_codes(codes: torch.Tensor, src: torch.Tensor, idx: torch.Tensor) -> torch.Tensor:
    """codes [heads, n] uint16 (updated in place), src [heads, n] uint16, idx [heads, n_idx]
    int32: codes[h, idx[h, i]] = src[h, idx[h, i]].  Returns codes."""
    _dev(codes, "codes")
    _dev(src, "src")
    _dev(idx, "idx")
    if codes.dtype != torch.uint16 or src.dtype != torch.uint16 or idx.dtype != torch.int32:
        raise ValueError("codes and src must be uint16, idx int32")
    if codes.dim() != 2 or src.shape != codes.shape or idx.dim() != 2 or idx.shape[0] != codes.shape[0]:
        raise ValueError("codes, src [heads, n] and idx [heads, n_idx]")
    heads, n = codes.shape
    _check(lib().a2ats_merge_codes(_ptr(src), _ptr(idx), heads, n, idx.shape[1], _ptr(codes),
                                   _stream(codes.device)), "merge_codes")
    return codes


def select_retrieval(keys: torch.Tensor, query: torch.Tensor, fraction: float):
    """keys [heads, n, d], query [heads, d] -> (retrieval_idx [heads, n_r], bulk [heads, n-n_r])."""
    _dev(keys, "keys")
    _dev(query, "query")
    heads, n, d = keys.shape
    if query.dtype != keys.dtype or query.shape != (heads, d):
        raise ValueError("query must be [heads, d] in the dtype of keys")
    n_r = retrieval_count(n, fraction)
    if n_r < 0:
        raise A2ATSError(-1, "select_retrieval")
    ret = torch.empty((heads, n_r), dtype=torch.int32, device=keys.device)
    bulk = torch.empty((heads, n - n_r), dtype=torch.int32, device=keys.device)
    ws = _workspace(lib().a2ats_select_retrieval_workspace(heads, n), keys.device)
    _check(lib().a2ats_select_retrieval(_ptr(keys), _dtype_code(keys), heads, n, d, _ptr(query),
                                        float(fraction), _ptr(ret), _ptr(bulk), _ptr(ws),
                                        ws.numel(), _stream(keys.device)), "select_retrieval")
    return ret, bulk


def reconstruct(codes: torch.Tensor, positions: torch.Tensor, codebook: torch.Tensor,
                cur_pos: int, window: int, far_offset: int = 2048,
                far_mode: int = FAR_FIXED_OFFSET, rope_base: float = 10000.0,
                out_dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None):
    """codes [batch, heads, n] uint16, positions [batch, n] int32, codebook [heads, c, d]
    -> out [batch, heads, n, d] (out_dtype)."""
    _dev(codes, "codes")
    _dev(positions, "positions")
    _dev(codebook, "codebook")
    batch, heads, n = codes.shape
    c, d = codebook.shape[1], codebook.shape[2]
    if positions.dtype != torch.int32 or positions.shape != (batch, n):
        raise ValueError("positions must be [batch, n] int32")
    if out is None:
        out = torch.empty((batch, heads, n, d), dtype=out_dtype, device=codes.device)
    else:
        _dev(out, "out")
    ws = _workspace(lib().a2ats_reconstruct_workspace(heads, c, d, int(cur_pos), int(window),
                                                      _dtype_code(out)), codes.device)
    _check(lib().a2ats_reconstruct(_ptr(codes), _ptr(positions), batch, heads, n, d,
                                   _ptr(codebook), c, int(cur_pos), int(window), int(far_offset),
                                   int(far_mode), float(rope_base), _ptr(out), _dtype_code(out),
                                   _ptr(ws), ws.numel(), _stream(codes.device)), "reconstruct")
    return out


def reconstruct_noalloc(codes: torch.Tensor, positions: torch.Tensor, codebook: torch.Tensor,
                        cur_pos: int, window: int, out: torch.Tensor, far_offset: int = 2048,
                        far_mode: int = FAR_FIXED_OFFSET, rope_base: float = 10000.0):
    """reconstruct() into the caller's `out` without allocating device memory: the rope
    table lives in a fixed per-GPU array of the library (min(max(window, 0), cur_pos + 1) + 1
    <= NOALLOC_TABLE_ROWS).  Calls on one GPU whose work overlaps race on that array."""
    _dev(codes, "codes")
    _dev(positions, "positions")
    _dev(codebook, "codebook")
    _dev(out, "out")
    batch, heads, n = codes.shape
    c, d = codebook.shape[1], codebook.shape[2]
    if positions.dtype != torch.int32 or positions.shape != (batch, n):
        raise ValueError("positions must be [batch, n] int32")
    if out.shape != (batch, heads, n, d):
        raise ValueError("out must be [batch, heads, n, d]")
    _check(lib().a2ats_reconstruct_noalloc(_ptr(codes), _ptr(positions), batch, heads, n, d,
                                           _ptr(codebook), c, int(cur_pos), int(window),
                                           int(far_offset), int(far_mode), float(rope_base),
                                           _ptr(out), _dtype_code(out), _stream(codes.device)),
           "reconstruct_noalloc")
    return out


def reconstruct_update(codes: torch.Tensor, positions: torch.Tensor, codebook: torch.Tensor,
                       n_prev: int, cur_prev: int, cur_pos: int, window: int, out: torch.Tensor,
                       rope_base: float = 10000.0):
    """Advance `out` (a FAR_UNROTATED reconstruct of the first n_prev tokens at cur_prev) to
    the FAR_UNROTATED reconstruct of all n tokens at cur_pos, rewriting only the rows that
    change.  codes [batch, heads, n] uint16, positions [batch, n] int32, out [batch, heads,
    n, d] fp32 or bf16."""
    _dev(codes, "codes")
    _dev(positions, "positions")
    _dev(codebook, "codebook")
    _dev(out, "out")
    batch, heads, n = codes.shape
    c, d = codebook.shape[1], codebook.shape[2]
    if positions.dtype != torch.int32 or positions.shape != (batch, n):
        raise ValueError("positions must be [batch, n] int32")
    if out.shape != (batch, heads, n, d):
        raise ValueError("out must be [batch, heads, n, d]")
    _check(lib().a2ats_reconstruct_update(_ptr(codes), _ptr(positions), batch, heads, n, d,
                                          _ptr(codebook), c, int(n_prev), int(cur_prev),
                                          int(cur_pos), int(window), float(rope_base), _ptr(out),
                                          _dtype_code(out), _stream(codes.device)),
           "reconstruct_update")
    return out


def far_query_rope(q: torch.Tensor, far_offset: int = 2048, rope_base: float = 10000.0,
                   out: torch.Tensor | None = None, out_dtype: torch.dtype | None = None):
    """q [..., d] -> q R_b: every row rotated as a token at position far_offset (Eq. 11's
    query-side far rotation).  out may be q itself."""
    _dev(q, "q")
    d = q.shape[-1]
    rows = q.numel() // d if d else 0
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    else:
        _dev(out, "out")
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    _check(lib().a2ats_far_query_rope(_ptr(q), _dtype_code(q), rows, d, int(far_offset),
                                      float(rope_base), _ptr(out), _dtype_code(out),
                                      _stream(q.device)), "far_query_rope")
    return out


def pq_encode(x: torch.Tensor, codebook: torch.Tensor, sub_dim: int = 8,
              chol: torch.Tensor | None = None, query: torch.Tensor | None = None,
              beta: float = 0.5, idx: torch.Tensor | None = None,
              codes: torch.Tensor | None = None):
    """Sub-vector codes: x [heads, n, d] (fp32/bf16), codebook [k, sub_dim] fp32 shared by
    every sub-space and head, chol [sub_dim, sub_dim] (H-weighted) or query [heads, nq, d]
    (cosine blend) or neither (plain) -> codes [heads, n, d // sub_dim] uint8 (only the idx
    rows are written when idx is given)."""
    _dev(x, "x")
    _dev(codebook, "codebook")
    heads, n, d = x.shape
    k = codebook.shape[0]
    if codebook.shape[1] != sub_dim:
        raise ValueError("codebook must be [k, sub_dim]")
    if codes is None:
        codes = torch.zeros((heads, n, d // sub_dim), dtype=torch.uint8, device=x.device)
    n_idx = 0
    if idx is not None:
        _dev(idx, "idx")
        if idx.dtype != torch.int32 or idx.dim() != 2 or idx.shape[0] != heads:
            raise ValueError("idx must be [heads, n_idx] int32")
        n_idx = idx.shape[1]
    nq = 0
    if query is not None:
        _dev(query, "query")
        nq = query.shape[1]
    _check(lib().a2ats_pq_encode(_ptr(x), _dtype_code(x), heads, n, d, sub_dim, _ptr(idx), n_idx,
                                 _ptr(codebook), k, _ptr(chol), _ptr(query), nq, float(beta),
                                 _ptr(codes), _stream(x.device)), "pq_encode")
    return codes


def pq_reconstruct(codes: torch.Tensor, positions: torch.Tensor, codebook: torch.Tensor,
                   cur_pos: int, window: int, far_offset: int = 2048,
                   far_mode: int = FAR_FIXED_OFFSET, rope_base: float = 10000.0,
                   out_dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None):
    """codes [batch, heads, n, m] uint8, positions [batch, n] int32, codebook [k, sub_dim]
    -> out [batch, heads, n, m * sub_dim].  Values: window=0, far_mode=FAR_UNROTATED."""
    _dev(codes, "codes")
    _dev(positions, "positions")
    _dev(codebook, "codebook")
    batch, heads, n, m = codes.shape
    k, sub = codebook.shape
    d = m * sub
    if positions.dtype != torch.int32 or positions.shape != (batch, n):
        raise ValueError("positions must be [batch, n] int32")
    if out is None:
        out = torch.empty((batch, heads, n, d), dtype=out_dtype, device=codes.device)
    else:
        _dev(out, "out")
    ws = _workspace(lib().a2ats_pq_reconstruct_workspace(d, int(cur_pos), int(window)), codes.device)
    _check(lib().a2ats_pq_reconstruct(_ptr(codes), _ptr(positions), batch, heads, n, d, sub,
                                      _ptr(codebook), k, int(cur_pos), int(window), int(far_offset),
                                      int(far_mode), float(rope_base), _ptr(out), _dtype_code(out),
                                      _ptr(ws), ws.numel(), _stream(codes.device)), "pq_reconstruct")
    return out


def pq_accounting(tokens: int, heads: int, d: int = 128, sub_dim: int = 8, bits: int = 8) -> dict:
    """The compression the settings decide: bits per number, ratio against fp16, table bytes,
    packed code bytes and fp16 bytes for `tokens` tokens of `heads` heads (host only)."""
    bpn, ratio = ctypes.c_double(), ctypes.c_double()
    table, comp, fp16 = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().a2ats_pq_accounting(tokens, heads, d, sub_dim, bits, ctypes.byref(bpn),
                                     ctypes.byref(ratio), ctypes.byref(table), ctypes.byref(comp),
                                     ctypes.byref(fp16)), "pq_accounting")
    return {"bits_per_number": bpn.value, "ratio_vs_fp16": ratio.value, "table_bytes": table.value,
            "compressed_bytes": comp.value, "fp16_bytes": fp16.value}


def kmeans_update(x: torch.Tensor, codes: torch.Tensor, codebook: torch.Tensor,
                  out: torch.Tensor | None = None, want_counts: bool = False):
    """x [heads, n, d], codes [heads, n] uint16 or uint8, codebook [heads, k, d] fp32 ->
    new codebook (cluster member means; empty clusters unchanged) [, counts int32]."""
    _dev(x, "x")
    _dev(codes, "codes")
    _dev(codebook, "codebook")
    heads, n, d = x.shape
    k = codebook.shape[-2]
    if out is None:
        out = torch.empty_like(codebook)
    counts = torch.empty((heads, k), dtype=torch.int32, device=x.device) if want_counts else None
    cbytes = 2 if codes.dtype == torch.uint16 else 1
    ws = _workspace(lib().a2ats_kmeans_update_workspace(heads, n, k), x.device)
    _check(lib().a2ats_kmeans_update(_ptr(x), _dtype_code(x), heads, n, d, _ptr(codes), cbytes, k,
                                     _ptr(codebook), _ptr(out), _ptr(counts), _ptr(ws), ws.numel(),
                                     _stream(x.device)), "kmeans_update")
    return (out, counts) if want_counts else out


def kmeans(x: torch.Tensor, codebook: torch.Tensor, chol: torch.Tensor | None = None,
           iters: int = 10):
    """Lloyd's k-means from `codebook` (updated in place).  x [heads, n, 128] with codebook
    [heads, k, 128] (codes uint16 [heads, n]), or pooled sub-vectors x [n, d] (d 4 or 8) with
    one codebook [k, d] (codes uint8 [n]).  Returns (codebook, codes)."""
    _dev(x, "x")
    _dev(codebook, "codebook")
    if x.dim() == 2:
        heads, (n, d) = 1, x.shape
        codes = torch.empty(n, dtype=torch.uint8, device=x.device)
    else:
        heads, n, d = x.shape
        codes = torch.empty((heads, n), dtype=torch.uint16, device=x.device)
    k = codebook.shape[-2]
    ws = _workspace(lib().a2ats_kmeans_workspace(heads, n, d, k), x.device)
    _check(lib().a2ats_kmeans(_ptr(x), _dtype_code(x), heads, n, d, k, _ptr(chol), int(iters),
                              _ptr(codebook), _ptr(codes), _ptr(ws), ws.numel(), _stream(x.device)),
           "kmeans")
    return codebook, codes


def kmeans_init(x: torch.Tensor, k: int, draws: torch.Tensor, chol: torch.Tensor | None = None,
                want_idx: bool = False):
    """k-means++ seeding in z-space.  x [heads, n, d] (or pooled sub-vectors [n, d], one
    codebook), draws [heads, k] (or [k]) uint64 held in an int64 tensor, chol [heads, d, d]
    (or [d, d]) or None -> codebook [heads, k, d] (or [k, d]) fp32 [, idx int32]."""
    _dev(x, "x")
    _dev(draws, "draws")
    pooled = x.dim() == 2
    xv = x[None] if pooled else x
    heads, n, d = xv.shape
    if draws.dtype != torch.int64 or draws.numel() != heads * k:
        raise ValueError("draws must hold heads * k 64-bit values (int64 tensor)")
    if chol is not None:
        _dev(chol, "chol")
        if chol.dtype != torch.float32 or chol.numel() != heads * d * d:
            raise ValueError("chol must be [heads, d, d] float32")
    cb = torch.empty((heads, k, d), dtype=torch.float32, device=x.device)
    idx = torch.empty((heads, k), dtype=torch.int32, device=x.device) if want_idx else None
    ws = _workspace(lib().a2ats_kmeans_init_workspace(heads, n, d, k), x.device)
    _check(lib().a2ats_kmeans_init(_ptr(xv), _dtype_code(x), heads, n, d, int(k), _ptr(chol),
                                   _ptr(draws), _ptr(cb), _ptr(idx), _ptr(ws), ws.numel(),
                                   _stream(x.device)), "kmeans_init")
    if pooled:
        cb = cb[0]
        idx = idx[0] if idx is not None else None
    return (cb, idx) if want_idx else cb


def topk_codes(qb: torch.Tensor, codes: torch.Tensor, codebook: torch.Tensor, k: int,
               want_scores: bool = True):
    """Top-k tokens by the approximate score (q R_b) . c_code.  qb [batch, hq, d] (fp32/bf16,
    already rotated by far_query_rope), codes [batch, hkv, n] uint16, codebook [hkv, c, d]
    fp32 -> idx [batch, hq, k] int32 ascending (and scores [batch, hq, k] fp32)."""
    _dev(qb, "qb")
    _dev(codes, "codes")
    _dev(codebook, "codebook")
    if qb.dim() != 3 or codes.dim() != 3 or codebook.dim() != 3:
        raise ValueError("qb [batch, hq, d], codes [batch, hkv, n], codebook [hkv, c, d]")
    if codes.dtype != torch.uint16 or codebook.dtype != torch.float32:
        raise ValueError("codes must be uint16 and codebook fp32")
    batch, hq, d = qb.shape
    _, hkv, n = codes.shape
    c = codebook.shape[1]
    if codes.shape[0] != batch or codebook.shape[0] != hkv or codebook.shape[2] != d:
        raise ValueError("qb, codes and codebook shapes disagree")
    idx = torch.empty((batch, hq, k), dtype=torch.int32, device=qb.device)
    sc = torch.empty((batch, hq, k), dtype=torch.float32, device=qb.device) if want_scores else None
    ws = _workspace(lib().a2ats_topk_workspace(batch, hq, c), qb.device)
    _check(lib().a2ats_topk_codes(_ptr(qb), _dtype_code(qb), batch, hq, hkv, d, _ptr(codes), n,
                                  _ptr(codebook), c, int(k), _ptr(idx), _ptr(sc), _ptr(ws),
                                  ws.numel(), _stream(qb.device)), "topk_codes")
    return (idx, sc) if want_scores else idx


# ----------------------------------------------------------------- kernel timing
def profile_enable(on: bool = True):
    lib().a2ats_profile_enable(1 if on else 0)


def profile_reset():
    lib().a2ats_profile_reset()


def profile_read() -> dict:
    """{kernel name: (launches, total_ms)} for kernels launched while profiling was on."""
    n = lib().a2ats_profile_read(None, 0)
    buf = ctypes.create_string_buffer(int(n) + 16)
    lib().a2ats_profile_read(buf, len(buf))
    out = {}
    for line in buf.value.decode().splitlines():
        name, cnt, ms = line.split("\t")
        out[name] = (int(cnt), float(ms))
    return out
