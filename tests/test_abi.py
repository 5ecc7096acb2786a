"""The C ABI: the library loads, exports every function include/a2ats.h declares, and every
host-side validation path returns its status without touching a device (runs on CPU)."""
import ctypes
import json
import math
import os
import re
import subprocess

import pytest

import kv_cache_vector_windowed_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "a2ats.h")

EINVAL, EDTYPE, EWORKSPACE = -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(a2ats_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kv.LIB_PATH):
        pytest.skip("library not built")
    return kv.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) >= 15
    out = subprocess.check_output(["nm", "-D", "--defined-only", kv.LIB_PATH], text=True)
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(L, n)


def test_version_and_strerror(L):
    assert L.a2ats_version() == 1
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert L.a2ats_strerror(st).decode() not in ("", "unknown status")
    assert L.a2ats_strerror(42).decode() == "unknown status"


@pytest.mark.parametrize("n,f,want", [(4096, 0.1, 410), (32768, 0.1, 3277), (131072, 0.05, 6554),
                                      (10, 0.3, 3), (100, 0.07, 8), (1, 0.2, 1), (1, 0.0, 0),
                                      (0, 0.5, 0), (5, 1.0, 5), (10, 1.5, -1), (10, -0.1, -1),
                                      (-1, 0.5, -1)])
def test_retrieval_count(L, n, f, want):
    assert L.a2ats_retrieval_count(n, f) == want
    assert L.a2ats_retrieval_count(10, math.nan) == -1


FAKE = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation first
FAKE2 = ctypes.c_void_p(8192)  # a second distinct pointer, also never dereferenced


def test_encode_validation(L):
    ws_need = L.a2ats_encode_workspace(2, 100, 128, 50)
    assert ws_need > 0
    assert L.a2ats_encode_workspace(2, 100, 64, 50) == 0
    args = dict(keys=FAKE, dt=1, heads=2, n=100, d=128, idx=None, n_idx=0, cb=FAKE, c=50,
                chol=None, codes=FAKE, dist=None, stats=None, ws=FAKE, wsb=ws_need, s=None)

    def call(**kw):
        a = dict(args, **kw)
        return L.a2ats_encode(a["keys"], a["dt"], a["heads"], a["n"], a["d"], a["idx"], a["n_idx"],
                              a["cb"], a["c"], a["chol"], a["codes"], a["dist"], a["stats"],
                              a["ws"], a["wsb"], a["s"])

    assert call(dt=5) == EDTYPE
    assert call(d=64) == EINVAL
    assert call(d=127) == EINVAL
    assert call(c=0) == EINVAL
    assert call(c=65537) == EINVAL
    assert call(heads=0) == EINVAL
    assert call(n=-1) == EINVAL
    assert call(idx=FAKE, n_idx=101) == EINVAL
    assert call(idx=FAKE, n_idx=-1) == EINVAL
    assert call(keys=None) == EINVAL
    assert call(codes=None) == EINVAL
    assert call(keys=ctypes.c_void_p(4098)) == EINVAL          # not 16-byte aligned
    assert call(wsb=ws_need - 1) == EWORKSPACE
    assert call(ws=None) == EWORKSPACE
    assert call(ws=ctypes.c_void_p(4096 + 64)) == EWORKSPACE   # not 256-byte aligned
    assert call(n=0) == 0                                       # nothing to do
    assert call(idx=FAKE, n_idx=0) == 0


def test_encode_prepare_validation(L):
    ws_need = L.a2ats_encode_workspace(2, 100, 128, 50)

    def prep(cb=FAKE, c=50, heads=2, n=100, d=128, wsb=ws_need):
        return L.a2ats_encode_prepare(cb, c, None, heads, n, d, FAKE, wsb, None)

    assert prep(cb=None) == EINVAL
    assert prep(c=0) == EINVAL
    assert prep(c=65537) == EINVAL
    assert prep(d=64) == EINVAL
    assert prep(heads=0) == EINVAL
    assert prep(n=-1) == EINVAL
    assert prep(wsb=ws_need - 1) == EWORKSPACE

    def run(keys=FAKE, dt=1, n=100, d=128, idx=None, n_idx=0, c=50, codes=FAKE, wsb=ws_need):
        return L.a2ats_encode_prepared(keys, dt, 2, n, d, idx, n_idx, c, None, codes, None, None,
                                       FAKE, wsb, None)

    assert run(dt=5) == EDTYPE
    assert run(d=64) == EINVAL
    assert run(c=0) == EINVAL
    assert run(idx=FAKE, n_idx=101) == EINVAL
    assert run(keys=None) == EINVAL
    assert run(codes=None) == EINVAL
    assert run(keys=ctypes.c_void_p(4098)) == EINVAL
    assert run(wsb=ws_need - 1) == EWORKSPACE
    assert run(n=0) == 0                   # nothing to encode: no launch
    assert run(idx=FAKE, n_idx=0) == 0


def test_assign_cosine_validation(L):
    def call(dt=0, heads=1, n=4, d=128, nq=1, c=8, beta=0.5, x=FAKE, ws=FAKE, wsb=1 << 30):
        return L.a2ats_assign_cosine(x, dt, heads, n, d, FAKE, nq, FAKE, c, beta, FAKE, ws, wsb,
                                     None)

    need = L.a2ats_assign_cosine_workspace(1, 4, 8)
    assert need >= 2 * 4 * 8 * 8
    # a large input is batched: the workspace stays bounded
    assert L.a2ats_assign_cosine_workspace(8, 32768, 1024) <= 2 * (64 << 20) + 4096
    assert call(ws=None, wsb=0) == EWORKSPACE
    assert call(wsb=need - 1) == EWORKSPACE

    assert call(dt=3) == EDTYPE
    for beta in (-0.01, 1.01, math.nan):
        assert call(beta=beta) == EINVAL
    assert call(nq=2) == EINVAL
    assert call(d=257) == EINVAL
    assert call(c=0) == EINVAL
    assert call(c=65537) == EINVAL
    assert call(x=None) == EINVAL
    assert call(n=0) == 0


def test_merge_codes_validation(L):
    def call(heads=2, n=100, n_idx=10, src=FAKE, idx=FAKE, codes=FAKE2):
        return L.a2ats_merge_codes(src, idx, heads, n, n_idx, codes, None)

    assert call(heads=0) == EINVAL
    assert call(n=-1) == EINVAL
    assert call(n_idx=101) == EINVAL
    assert call(n_idx=-1) == EINVAL
    assert call(src=None) == EINVAL
    assert call(idx=None) == EINVAL
    assert call(codes=None) == EINVAL
    assert call(n_idx=0, src=None, idx=None, codes=None) == 0  # nothing to merge
    assert call(codes=FAKE) == 0                              # src == codes: nothing changes


def test_select_validation(L):
    need = L.a2ats_select_retrieval_workspace(2, 1000)
    assert need > 0

    def call(dt=1, heads=2, n=1000, d=128, f=0.1, ws=FAKE, wsb=need, keys=FAKE):
        return L.a2ats_select_retrieval(keys, dt, heads, n, d, FAKE, f, FAKE, FAKE, ws, wsb, None)

    assert call(dt=2) == EDTYPE
    assert call(d=64) == EINVAL
    assert call(f=1.5) == EINVAL
    assert call(f=math.nan) == EINVAL
    assert call(keys=None) == EINVAL
    assert call(wsb=need - 1) == EWORKSPACE
    assert call(n=0) == 0


def test_reconstruct_validation(L):
    need = L.a2ats_reconstruct_workspace(2, 10, 128, 16384, 256, 0)
    assert need >= (256 + 1) * 64 * 16 + 2 * 10 * 128 * 4  # table + far rows
    assert L.a2ats_reconstruct_workspace(2, 10, 128, 10, 1 << 40, 1) >= 11 * 64 * 16 + 2 * 10 * 128 * 2
    assert L.a2ats_reconstruct_workspace(2, 10, 128, 10, 5, 7) == 0  # dtype
    assert L.a2ats_pq_reconstruct_workspace(128, 10, 1 << 40) >= 11 * 64 * 16  # rows capped at cur+1

    def call(out_dt=0, d=128, cur=100, window=16, far_mode=0, base=10000.0, c=10, n=50,
             wsb=None, codes=FAKE):
        wsb = need if wsb is None else wsb
        return L.a2ats_reconstruct(codes, FAKE, 1, 2, n, d, FAKE, c, cur, window, 2048, far_mode,
                                   base, FAKE, out_dt, FAKE, wsb, None)

    assert call(out_dt=7) == EDTYPE
    assert call(d=64) == EINVAL
    assert call(cur=-1) == EINVAL
    assert call(far_mode=2) == EINVAL
    assert call(base=0.0) == EINVAL
    assert call(base=math.inf) == EINVAL
    assert call(c=0) == EINVAL
    assert call(codes=None) == EINVAL
    assert call(wsb=0) == EWORKSPACE
    assert call(n=0) == 0


def test_reconstruct_noalloc_validation(L):
    # every failing case returns before the library touches a device
    def call(out_dt=0, d=128, cur=100, window=16, far_mode=0, base=10000.0, c=10, n=50,
             codes=FAKE):
        return L.a2ats_reconstruct_noalloc(codes, FAKE, 1, 2, n, d, FAKE, c, cur, window, 2048,
                                           far_mode, base, FAKE, out_dt, None)

    ESCRATCH = -6
    assert call(out_dt=7) == EDTYPE
    assert call(d=64) == EINVAL
    assert call(cur=-1) == EINVAL
    assert call(far_mode=2) == EINVAL
    assert call(base=0.0) == EINVAL
    assert call(c=0) == EINVAL
    assert call(codes=None) == EINVAL
    assert call(n=0) == 0
    # the fixed table holds A2ATS_NOALLOC_TABLE_ROWS rows: min(max(W, 0), cur + 1) near rows + 1
    rows = kv.NOALLOC_TABLE_ROWS
    assert call(cur=10 ** 6, window=rows) == ESCRATCH
    assert call(cur=10 ** 6, window=10 ** 9) == ESCRATCH
    assert call(cur=rows - 1, window=10 ** 9) == ESCRATCH   # cur + 1 = rows near rows
    assert "scratch" in L.a2ats_strerror(ESCRATCH).decode()
    text = open(HEADER).read()
    assert "#define A2ATS_NOALLOC_TABLE_ROWS %d" % rows in text


def test_reconstruct_update_validation(L):
    def call(out_dt=0, d=128, n=50, n_prev=40, cur_prev=99, cur=100, base=10000.0, c=10,
             codes=FAKE):
        return L.a2ats_reconstruct_update(codes, FAKE, 1, 2, n, d, FAKE, c, n_prev, cur_prev, cur,
                                          16, base, FAKE, out_dt, None)

    assert call(out_dt=3) == EDTYPE
    assert call(d=256) == EINVAL
    assert call(n_prev=-1) == EINVAL
    assert call(n_prev=51) == EINVAL
    assert call(cur_prev=-1) == EINVAL
    assert call(cur=-2) == EINVAL
    assert call(base=-1.0) == EINVAL
    assert call(c=65537) == EINVAL
    assert call(codes=None) == EINVAL
    assert call(n=0, n_prev=0) == 0


def test_far_query_rope_validation(L):
    def call(q=FAKE, qdt=0, rows=4, d=128, base=10000.0, out=ctypes.c_void_p(1 << 20), odt=0):
        return L.a2ats_far_query_rope(q, qdt, rows, d, 2048, base, out, odt, None)

    assert call(qdt=2) == EDTYPE
    assert call(odt=5) == EDTYPE
    assert call(d=64) == EINVAL
    assert call(rows=-1) == EINVAL
    assert call(base=math.nan) == EINVAL
    assert call(q=None) == EINVAL
    assert call(rows=0) == 0
    # partial overlap, or the same buffer with another dtype, is refused before any launch
    assert call(out=ctypes.c_void_p(4096 + 256)) == EINVAL
    assert call(out=FAKE, odt=1) == EINVAL


def test_pq_accounting_matches_pages_table(L):
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pq_compression.json")))
    for case in g["cases"]:
        r = kv.pq_accounting(4096, 8, 128, case["sub_dim"], case["bits"])
        assert r["bits_per_number"] == case["bits_per_number"]
        assert r["ratio_vs_fp16"] == case["smaller_by"]
        assert r["table_bytes"] == case["table_kb"] * 1024
        assert r["fp16_bytes"] == 4096 * 8 * 128 * 2
        assert r["compressed_bytes"] * case["smaller_by"] == r["fp16_bytes"]
    assert L.a2ats_pq_accounting(10, 1, 128, 12, 8, None, None, None, None, None) == EINVAL
    assert L.a2ats_pq_accounting(10, 1, 128, 8, 0, None, None, None, None, None) == EINVAL


def test_pq_validation(L):
    def enc(dt=1, d=128, sub=8, k=256, n=10, beta=0.5, nq=1, q=None, chol=None, x=FAKE):
        return L.a2ats_pq_encode(x, dt, 2, n, d, sub, None, 0, FAKE, k, chol, q, nq, beta, FAKE,
                                 None)

    assert enc(dt=9) == EDTYPE
    assert enc(d=64) == EINVAL
    assert enc(sub=16) == EINVAL
    assert enc(k=257) == EINVAL
    assert enc(k=0) == EINVAL
    assert enc(q=FAKE, beta=1.5) == EINVAL
    assert enc(q=FAKE, nq=3) == EINVAL
    assert enc(x=None) == EINVAL
    assert enc(n=0) == 0

    def rec(odt=0, sub=8, k=256, n=10, wsb=1 << 20, mode=0, cur=5):
        return L.a2ats_pq_reconstruct(FAKE, FAKE, 1, 2, n, 128, sub, FAKE, k, cur, 4, 2048, mode,
                                      10000.0, FAKE, odt, FAKE, wsb, None)

    assert rec(odt=4) == EDTYPE
    assert rec(sub=2) == EINVAL
    assert rec(k=300) == EINVAL
    assert rec(mode=3) == EINVAL
    assert rec(cur=-1) == EINVAL
    assert rec(wsb=0) == EWORKSPACE
    assert rec(n=0) == 0


def test_kmeans_validation(L):
    need = L.a2ats_kmeans_update_workspace(2, 1000, 64)
    assert need > 0

    def upd(dt=0, d=128, cb=2, k=64, n=1000, wsb=None, x=FAKE):
        wsb = need if wsb is None else wsb
        return L.a2ats_kmeans_update(x, dt, 2, n, d, FAKE, cb, k, FAKE, FAKE, None, FAKE, wsb, None)

    assert upd(dt=5) == EDTYPE
    assert upd(cb=4) == EDTYPE
    assert upd(d=12) == EINVAL
    assert upd(k=5000) == EINVAL
    assert upd(cb=1, k=300) == EINVAL
    assert upd(x=None) == EINVAL
    assert upd(wsb=16) == EWORKSPACE

    def km(d=128, heads=1, n=1024, k=64, iters=3, wsb=1 << 30):
        return L.a2ats_kmeans(FAKE, 0, heads, n, d, k, None, iters, FAKE, FAKE, FAKE, wsb, None)

    assert km(d=16) == EINVAL          # the driver trains whole vectors or 4/8 sub-vectors
    assert km(d=8, heads=2) == EINVAL  # one shared sub-vector codebook
    assert km(d=8, n=1000) == EINVAL   # 1000 sub-vectors do not fill whole 128-wide rows
    assert km(d=8, k=512) == EINVAL
    assert km(iters=-1) == EINVAL
    assert km(wsb=8) == EWORKSPACE
    assert km(n=0) == 0


def test_kmeans_init_validation(L):
    need = L.a2ats_kmeans_init_workspace(2, 1000, 128, 16)
    assert need >= 2 * 1000 * 128 * 4 + 2 * 2 * 1000 * 8
    assert L.a2ats_kmeans_init_workspace(1, 10, 128, 11) == 0  # k > n

    def call(dt=1, heads=2, n=1000, d=128, k=16, x=FAKE, draws=FAKE, cb=FAKE, wsb=None):
        wsb = need if wsb is None else wsb
        return L.a2ats_kmeans_init(x, dt, heads, n, d, k, None, draws, cb, None, FAKE, wsb, None)

    assert call(dt=5) == EDTYPE
    assert call(d=12) == EINVAL
    assert call(d=256) == EINVAL
    assert call(k=0) == EINVAL
    assert call(k=1001) == EINVAL
    assert call(n=0) == EINVAL
    assert call(heads=0) == EINVAL
    assert call(x=None) == EINVAL
    assert call(draws=None) == EINVAL
    assert call(cb=None) == EINVAL
    assert call(wsb=need - 1) == EWORKSPACE


def test_topk_codes_validation(L):
    need = L.a2ats_topk_workspace(2, 6, 16)
    assert need >= 2 * 6 * 16 * 4 and need % 256 == 0
    assert L.a2ats_topk_workspace(0, 6, 16) == 0 and L.a2ats_topk_workspace(2, 6, 4097) == 0

    def call(qdt=0, batch=2, hq=6, hkv=2, d=128, n=64, c=16, k=8, qb=FAKE, idx=FAKE, ws=FAKE,
             wsb=None, cb=FAKE):
        return L.a2ats_topk_codes(qb, qdt, batch, hq, hkv, d, FAKE, n, cb, c, k, idx, None,
                                  ws, need if wsb is None else wsb, None)

    assert call(qdt=2) == EDTYPE
    assert call(d=64) == EINVAL
    assert call(hq=5) == EINVAL          # hq not a multiple of hkv
    assert call(batch=0) == EINVAL
    assert call(c=0) == EINVAL
    assert call(c=4097) == EINVAL
    assert call(k=65) == EINVAL          # k > n
    assert call(k=-1) == EINVAL
    assert call(qb=None) == EINVAL
    assert call(idx=None) == EINVAL
    assert call(cb=None) == EINVAL
    assert call(qb=ctypes.c_void_p(4100)) == EINVAL  # queries not 16-byte aligned
    assert call(batch=1 << 28, hq=8) == EINVAL       # batch * hq >= 2^31
    assert call(ws=None) == EWORKSPACE
    assert call(wsb=need - 1) == EWORKSPACE
    assert call(k=0) == 0                # nothing to select: no launch
    assert call(n=0, k=0) == 0


def test_calibrate_validation(L):
    need = L.a2ats_calibrate_workspace(2, 100, 128)
    assert need > 0 and L.a2ats_calibrate_workspace(2, 100, 129) == 0

    def call(heads=2, m=100, d=128, ridge=1e-4, wsb=need, q=FAKE):
        return L.a2ats_calibrate(q, heads, m, d, ridge, FAKE, FAKE, FAKE, wsb, None)

    assert call(d=129) == EINVAL
    assert call(m=0) == EINVAL
    assert call(ridge=-1.0) == EINVAL
    assert call(ridge=math.nan) == EINVAL
    assert call(q=None) == EINVAL
    assert call(wsb=need - 1) == EWORKSPACE


def test_binding_fails_loudly_without_device_tensors():
    import torch
    with pytest.raises(ValueError):
        kv.calibrate(torch.zeros(1, 4, 128))


def test_bench_refuses_more_than_one_gpu():
    # the benchmark is for one GPU: --gpus above 1 exits with a message before touching a device
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
