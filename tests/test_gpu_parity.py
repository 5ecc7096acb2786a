"""GPU parity: every call of the C ABI against the fp64 CPU oracle on seeded inputs.

Small cases are compared element by element (several MFMA tiles, ragged tails); the
workloads at full size are compared on sampled rows the oracle computes one by one.  All
calls go through the C ABI (via the ctypes binding) on cuda:0.
"""
import numpy as np
import pytest
import torch

import kv_cache_vector_windowed_amd as kv
import oracle
from kv_cache_vector_windowed_amd import synth

from parity import (DEV, bf16_to_np_bits, check_codes, check_dist, check_rotation,
                    check_rounded_once, check_split,
                    f32_to_dev, keys_to_dev, u16_to_dev, u16_to_np)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def oracle_L(cfg, heads, m):
    return oracle.calibrate(synth.queries(cfg, heads, m), 1e-4)[1]


def z2_of(x, l):
    x = np.asarray(x, np.float64)
    return ((x @ l.astype(np.float64)) ** 2).sum(-1) if l is not None else (x ** 2).sum(-1)


# ====================================================================== calibrate
class TestCalibrate:
    @pytest.mark.parametrize("name", ["tiny", "layer", "encode_stress"])
    def test_workload(self, name):
        w = W[name]
        q = synth.queries(w.cfg, w.heads, w.m)
        H, L = kv.calibrate(f32_to_dev(q), 1e-4)
        Ho, Lo = oracle.calibrate(q, 1e-4)
        H, L = H.cpu().numpy(), L.cpu().numpy()
        for h in range(w.heads):
            assert np.abs(H[h] - Ho[h]).max() <= 1e-5 * np.abs(Ho[h]).max()
            assert np.abs(L[h] - Lo[h]).max() <= 1e-5 * np.abs(Lo[h]).max()
            assert np.all(np.triu(L[h], 1) == 0)

    def test_small_odd_dimension(self):
        q = synth.queries(100, 3, 77, d=5)
        H, L = kv.calibrate(f32_to_dev(q), 0.25)
        Ho, Lo = oracle.calibrate(q, 0.25)
        np.testing.assert_allclose(H.cpu().numpy(), Ho, rtol=0, atol=1e-5 * np.abs(Ho).max())
        np.testing.assert_allclose(L.cpu().numpy(), Lo, rtol=0, atol=1e-5 * np.abs(Lo).max())

    def test_not_positive_definite(self):
        q = synth.queries(101, 1, 64, d=8)
        q[:, :, 3] = 0.0  # zero column, no ridge: exact zero pivot
        with pytest.raises(kv.A2ATSError) as e:
            kv.calibrate(f32_to_dev(q), 0.0)
        assert e.value.status == -4


# ====================================================================== encode
def run_encode(name_or_w, n_sample=None, use_h=True, seed=0):
    w = W[name_or_w] if isinstance(name_or_w, str) else name_or_w
    keys = synth.keys(w.cfg, w.heads, w.n, w.key_dtype)
    cb = synth.codebook(w.cfg, w.heads, w.c)
    L = oracle_L(w.cfg, w.heads, w.m) if use_h else None
    stats = torch.zeros(8, dtype=torch.int32, device=DEV)
    codes, dist = kv.encode(keys_to_dev(keys), f32_to_dev(cb), f32_to_dev(L) if use_h else None,
                            want_dist=True, stats=stats)
    codes = u16_to_np(codes)
    dist = dist.cpu().numpy()
    rng = np.random.default_rng(seed)
    ties = []
    for h in range(w.heads):
        rows = np.arange(w.n) if n_sample is None else np.sort(rng.choice(w.n, n_sample, replace=False))
        x = keys.values[h][rows]
        lh = L[h] if use_h else None
        code, d1, d2 = oracle.assign_h(x, cb[h], lh)
        tie, _ = check_codes(codes[h][rows], code, d1, d2, "%s head %d" % (w.name, h))
        check_dist(dist[h][rows], d1, z2_of(x, lh), "%s head %d" % (w.name, h))
        ties.append(tie)
    st = stats.cpu().numpy()
    assert st[0] == w.heads * w.n
    assert st[1] + st[2] + st[3] + st[4] == st[0]
    return float(np.mean(ties)), st


class TestEncode:
    @pytest.mark.parametrize("use_h", [False, True])
    def test_tiny_all_rows(self, use_h):
        tie, st = run_encode("tiny", use_h=use_h)
        print("tiny use_h=%s tie rate %.2e stats %s" % (use_h, tie, st[:5]))

    def test_ragged_shapes_and_index_subset(self):
        w = synth.Workload("ragged", 110, 3, 1000, 100, "bf16", m=300)
        keys = synth.keys(w.cfg, w.heads, w.n, "bf16")
        cb = synth.codebook(w.cfg, w.heads, w.c)
        L = oracle_L(w.cfg, w.heads, w.m)
        rng = np.random.default_rng(3)
        idx = np.stack([np.sort(rng.choice(w.n, 333, replace=False)) for _ in range(w.heads)]).astype(np.int32)
        codes0 = u16_to_dev(np.full((w.heads, w.n), 0xFFFF, np.uint16))
        out = kv.encode(keys_to_dev(keys), f32_to_dev(cb), f32_to_dev(L),
                        idx=torch.from_numpy(idx).to(DEV), codes=codes0)
        out = u16_to_np(out)
        for h in range(w.heads):
            code, d1, d2 = oracle.assign_h(keys.values[h][idx[h]], cb[h], L[h])
            check_codes(out[h][idx[h]], code, d1, d2, "ragged head %d" % h)
            untouched = np.setdiff1d(np.arange(w.n), idx[h])
            assert np.all(out[h][untouched] == 0xFFFF)

    def test_layer_sampled(self):
        tie, st = run_encode("layer", n_sample=768)
        print("layer tie rate %.2e stats %s" % (tie, st[:5]))

    def test_encode_stress_sampled(self):
        # 4096 of the 131072 rows of every head: at the measured ~1.2% rescan rate about 50
        # keys a head that went through the rescan
        tie, st = run_encode("encode_stress", n_sample=4096)
        print("encode_stress tie rate %.2e stats %s" % (tie, st[:5]))

    @pytest.mark.parametrize("c", [4097, 16384, 65536])
    @pytest.mark.parametrize("use_h", [False, True])
    def test_large_codebooks(self, c, use_h):
        # C beyond the workloads' 4096 up to the uint16 limit: the tile index packed into the
        # scores' low bits widens (13 bits at 65536), so the packing slack grows and more
        # keys go to the rerank, the rescan, candidate-list overflow and the full scan;
        # every row is checked, with distances and the decision counts
        w = synth.Workload("bigc", 160 + c % 89, 2, 700, c, "bf16", m=512)
        tie, st = run_encode(w, use_h=use_h)
        print("C=%d use_h=%s tie rate %.2e stats %s" % (c, use_h, tie, st[:5]))

    @pytest.mark.parametrize("use_h", [False, True])
    def test_candidate_list_overflow(self, use_h):
        # 48 copies of one centroid (perturbed by 2^-26 relative, which fp32 mostly rounds
        # away) and every third key drawn around it: those keys' rescan collects more
        # candidates than a key's list holds (32), so the decide pass gives them the fp64 scan
        # of the whole codebook; equal scores resolve to the lowest index
        heads, n, c = 2, 600, 256
        keys = synth.keys(131, heads, n, "f32")
        cb = synth.codebook(131, heads, c)
        rng = np.random.default_rng(131)
        near = np.arange(0, n, 3)
        for h in range(heads):
            base = cb[h, 40].astype(np.float64)
            for j in range(40, 88):
                cb[h, j] = (base * (1.0 + rng.uniform(-2.0 ** -26, 2.0 ** -26, 128))).astype(np.float32)
            noise = rng.standard_normal((len(near), 128)) * 0.05 * np.abs(base).mean()
            keys.values[h, near] = (base + noise).astype(np.float32)
        L = oracle_L(131, heads, 256) if use_h else None
        stats = torch.zeros(8, dtype=torch.int32, device=DEV)
        codes, dist = kv.encode(keys_to_dev(keys), f32_to_dev(cb), f32_to_dev(L) if use_h else None,
                                want_dist=True, stats=stats)
        codes, dist = u16_to_np(codes), dist.cpu().numpy()
        for h in range(heads):
            lh = L[h] if use_h else None
            code, d1, d2 = oracle.assign_h(keys.values[h], cb[h], lh)
            check_codes(codes[h], code, d1, d2, "overflow head %d" % h)
            check_dist(dist[h], d1, z2_of(keys.values[h], lh), "overflow head %d" % h)
        st = stats.cpu().numpy()
        print("candidate overflow use_h=%s stats %s" % (use_h, st[:5]))
        assert st[0] == heads * n and st[1] + st[2] + st[3] + st[4] == st[0]
        assert st[4] > 0  # the full scans ran

    def test_large_codebook_fp32_keys(self):
        w = synth.Workload("bigc32", 171, 1, 900, 4097, "f32", m=512)
        tie, st = run_encode(w, use_h=True)
        print("C=4097 fp32 keys tie rate %.2e stats %s" % (tie, st[:5]))

    def test_single_centroid_and_duplicate_centroids(self):
        keys = synth.keys(120, 2, 300, "f32")
        cb1 = synth.codebook(120, 2, 1)
        out = u16_to_np(kv.encode(keys_to_dev(keys), f32_to_dev(cb1), None))
        assert np.all(out == 0)
        cb = synth.codebook(121, 2, 40)
        cb[:, 20] = cb[:, 5]  # exact duplicate rows: ties resolve to the lower index
        cb[:, 39] = cb[:, 5]
        L = oracle_L(121, 2, 256)
        for chol in (None, L):
            out = u16_to_np(kv.encode(keys_to_dev(keys), f32_to_dev(cb),
                                      f32_to_dev(chol) if chol is not None else None))
            assert not np.any(out == 20) and not np.any(out == 39)
            for h in range(2):
                code, d1, d2 = oracle.assign_h(keys.values[h], cb[h], None if chol is None else chol[h])
                check_codes(out[h], code, d1, d2, "duplicates")

    def test_keys_outside_fp16_range(self):
        keys = synth.keys(122, 1, 200, "f32")
        keys.values[0, ::7, 3] *= 1e4  # some elements beyond 65504 (first half of a lane pair)
        keys.values[0, 2::9, 12] *= 1e4  # and in the second half
        cb = synth.codebook(122, 1, 64) * 1e2
        out, dist = kv.encode(keys_to_dev(keys), f32_to_dev(cb), None, want_dist=True)
        code, d1, d2 = oracle.assign_h(keys.values[0], cb[0], None)
        check_codes(u16_to_np(out)[0], code, d1, d2, "large keys")
        check_dist(dist.cpu().numpy()[0], d1, z2_of(keys.values[0], None), "large keys")

    @pytest.mark.parametrize("use_h", [False, True])
    def test_bf16_keys_outside_fp16_normal_range(self, use_h):
        # bf16 elements beyond fp16's range, below its normal range (down to bf16's own
        # subnormals) and exact zeros, spread over several 32-key blocks and both lane halves
        w = synth.Workload("bf16edge", 123, 2, 700, 96, "bf16", m=300)
        vals = synth.keys(w.cfg, w.heads, w.n, "f32").values.astype(np.float32)
        vals[:, ::11, 5] *= 1e5          # beyond 65504
        vals[:, 3::13, 70] *= 1e-6       # below 2^-14
        vals[:, 5::17, 100] = 3e-39      # bf16 subnormal
        vals[:, 7::19, :] *= 1e-7        # whole keys below 2^-14
        vals[:, 9::23, 64:] = 0.0        # zero halves
        vals[:, 1::29, 2] = -vals[:, 1::29, 2] * 1e-6
        bits = synth.f32_to_bf16_bits(vals)
        keys = synth.Keys(synth.bf16_bits_to_f32(bits), "bf16", bits)
        cb = synth.codebook(w.cfg, w.heads, w.c)
        L = oracle_L(w.cfg, w.heads, w.m) if use_h else None
        out, dist = kv.encode(keys_to_dev(keys), f32_to_dev(cb),
                              f32_to_dev(L) if use_h else None, want_dist=True)
        out, dist = u16_to_np(out), dist.cpu().numpy()
        for h in range(w.heads):
            code, d1, d2 = oracle.assign_h(keys.values[h], cb[h], None if L is None else L[h])
            check_codes(out[h], code, d1, d2, "bf16 edge head %d" % h)
            check_dist(dist[h], d1, z2_of(keys.values[h], None if L is None else L[h]), "bf16 edge")

    @pytest.mark.parametrize("use_h", [False, True])
    def test_prepared_runs_match_one_shot(self, use_h):
        # one prepare, two runs (all rows, then a subset of other keys): each equals encode()
        w = synth.Workload("prepared", 120, 2, 1500, 300, "bf16", m=400)
        cb = f32_to_dev(synth.codebook(w.cfg, w.heads, w.c))
        L = f32_to_dev(oracle_L(w.cfg, w.heads, w.m)) if use_h else None
        prep = kv.encode_prepare(cb, L, w.n)
        k1 = keys_to_dev(synth.keys(w.cfg, w.heads, w.n, "bf16"))
        k2 = keys_to_dev(synth.keys(w.cfg + 1, w.heads, w.n, "bf16"))
        rng = np.random.default_rng(5)
        idx = torch.from_numpy(np.stack([np.sort(rng.choice(w.n, 700, replace=False))
                                         for _ in range(w.heads)]).astype(np.int32)).to(DEV)
        for keys, ix in ((k1, None), (k2, idx)):
            a = kv.encode_prepared(keys, prep, idx=ix, want_dist=True)
            b = kv.encode(keys, cb, L, idx=ix, want_dist=True)
            assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
            assert torch.equal(a[1], b[1])

    @pytest.mark.parametrize("use_h", [False, True])
    def test_prepared_runs_leave_state_clear(self, use_h):
        # one prepare, then runs with and without statistics, all keys and subsets: every run
        # starts from the state the previous one left (cleared), so each equals a one-shot call
        w = synth.Workload("prepared_runs", 124, 2, 1500, 300, "bf16", m=400)
        cb = f32_to_dev(synth.codebook(w.cfg, w.heads, w.c))
        L = f32_to_dev(oracle_L(w.cfg, w.heads, w.m)) if use_h else None
        prep = kv.encode_prepare(cb, L, w.n)
        k1 = keys_to_dev(synth.keys(w.cfg, w.heads, w.n, "bf16"))
        k2 = keys_to_dev(synth.keys(w.cfg + 1, w.heads, w.n, "bf16"))
        rng = np.random.default_rng(7)
        idx = torch.from_numpy(np.stack([np.sort(rng.choice(w.n, 600, replace=False))
                                         for _ in range(w.heads)]).astype(np.int32)).to(DEV)
        for keys, ix, with_stats in ((k1, None, True), (k2, idx, False), (k1, None, False),
                                     (k2, idx, True), (k2, None, True)):
            sa = torch.zeros(8, dtype=torch.int32, device=DEV) if with_stats else None
            sb = torch.zeros(8, dtype=torch.int32, device=DEV) if with_stats else None
            a = kv.encode_prepared(keys, prep, idx=ix, want_dist=True, stats=sa)
            b = kv.encode(keys, cb, L, idx=ix, want_dist=True, stats=sb)
            assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
            assert torch.equal(a[1], b[1])
            if with_stats:
                assert torch.equal(sa, sb)
                assert int(sa[0]) == (w.heads * w.n if ix is None else ix.numel())

    def test_deterministic(self):
        w = W["tiny"]
        keys = keys_to_dev(synth.keys(w.cfg, 1, w.n, w.key_dtype))
        cb = f32_to_dev(synth.codebook(w.cfg, 1, w.c))
        L = f32_to_dev(oracle_L(w.cfg, 1, w.m))
        a = kv.encode(keys, cb, L, want_dist=True)
        b = kv.encode(keys, cb, L, want_dist=True)
        assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
        assert torch.equal(a[1], b[1])


# ====================================================================== cosine blend
class TestAssignCosine:
    @pytest.mark.parametrize("beta", [1.0, 0.7, 0.0])
    def test_tiny_retrieval_rows(self, beta):
        w = W["tiny"]
        keys = synth.keys(w.cfg, 1, w.n, w.key_dtype)
        cb = synth.codebook(w.cfg, 1, w.c)
        nr = oracle.retrieval_count(w.n, w.fraction)
        rows = np.arange(w.n - nr, w.n)  # any 410 rows; the proxy query is the last key
        x = keys.values[:, rows]
        q = keys.values[:, -1:]
        out = u16_to_np(kv.assign_cosine(f32_to_dev(x), f32_to_dev(q), f32_to_dev(cb), beta))
        code, s1, s2 = oracle.assign_cosine(x[0], q[0], cb[0], beta)
        bad = (s1 - s2 > 1e-5) & (out[0] != code)
        assert not bad.any(), np.nonzero(bad)[0][:5]

    def test_decode_new_keys(self):
        w = W["decode"]
        x = synth.new_keys(w.cfg, w.heads, w.batch)  # [heads, 32 sequences, d]
        cb = synth.codebook(w.cfg, w.heads, w.c)
        beta = w.betas[0]
        out = u16_to_np(kv.assign_cosine(f32_to_dev(x), f32_to_dev(x), f32_to_dev(cb), beta))
        for h in range(w.heads):
            code, s1, s2 = oracle.assign_cosine(x[h], x[h], cb[h], beta)
            bad = (s1 - s2 > 1e-5) & (out[h] != code)
            assert not bad.any()

    @pytest.mark.parametrize("heads,n,d,c,nq,dtype", [
        (3, 7, 100, 300, "n", "f32"),     # partial slices, row blocks and centroid tiles
        (2, 33, 8, 9, "1", "bf16"),       # one short slice, tiny codebook
        (1, 2, 256, 1, "n", "f32"),       # the largest d, a single centroid
        (1, 100, 8, 65536, "1", "f32")])  # several workspace batches
    def test_shapes_and_batches(self, heads, n, d, c, nq, dtype):
        rng = np.random.default_rng(heads * 7 + n + d + c)
        x = rng.standard_normal((heads, n, d)).astype(np.float32)
        q = rng.standard_normal((heads, n if nq == "n" else 1, d)).astype(np.float32)
        if dtype == "bf16":
            x, q = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)), synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(q))
        cb = rng.standard_normal((heads, c, d)).astype(np.float32)
        xd, qd = torch.from_numpy(x).to(DEV), torch.from_numpy(q).to(DEV)
        if dtype == "bf16":
            xd, qd = xd.to(torch.bfloat16), qd.to(torch.bfloat16)  # exact: on the bf16 grid
        if c == 65536:
            assert kv.lib().a2ats_assign_cosine_workspace(heads, n, c) < 2 * heads * n * c * 8
        out = u16_to_np(kv.assign_cosine(xd, qd, f32_to_dev(cb), 0.6))
        for h in range(heads):
            code, s1, s2 = oracle.assign_cosine(x[h], q[h] if nq == "n" else q[h, 0], cb[h], 0.6)
            bad = (s1 - s2 > 1e-5) & (out[h] != code)
            assert not bad.any(), (h, np.nonzero(bad)[0][:5])

    def test_bf16_rows_and_beta_one_matches_plain_encode(self):
        k = synth.keys(130, 2, 150, "bf16")
        cb = synth.codebook(130, 2, 70)
        xd = keys_to_dev(k)
        out = kv.assign_cosine(xd, xd[:, -1:].contiguous(), f32_to_dev(cb), 1.0)
        plain = kv.encode(xd, f32_to_dev(cb), None)
        for h in range(2):
            code, d1, d2 = oracle.assign_h(k.values[h], cb[h], None)
            check_codes(u16_to_np(out)[h], code, d1, d2, "beta=1")
            check_codes(u16_to_np(plain)[h], code, d1, d2, "plain")


# ====================================================================== retrieval split
def run_split(keys: synth.Keys, q: np.ndarray, f: float, what: str):
    ret, bulk = kv.select_retrieval(keys_to_dev(keys), q_to_dev(q, keys.dtype), f)
    ret, bulk = ret.cpu().numpy(), bulk.cpu().numpy()
    heads, n, _ = keys.values.shape
    band = 0
    for h in range(heads):
        ro, bo, cosv = oracle.select_retrieval(keys.values[h], q_exact(q, keys.dtype)[h], f)
        band += check_split(ret[h], bulk[h], n, cosv, ro, "%s head %d" % (what, h))
    return band


def q_to_dev(q, dtype):
    if dtype == "bf16":
        return torch.from_numpy(synth.f32_to_bf16_bits(q).view(np.int16)).to(DEV).view(torch.bfloat16)
    return f32_to_dev(q)


def q_exact(q, dtype):
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(q)) if dtype == "bf16" else q


class TestSelectRetrieval:
    @pytest.mark.parametrize("name", ["tiny", "layer", "long_context"])
    def test_workload(self, name):
        w = W[name]
        keys = synth.keys(w.cfg, w.heads, w.n, w.key_dtype)
        q = keys.values[:, -1].copy()  # proxy query: the last key of each head
        band = run_split(keys, q, w.fraction, name)
        print("%s: %d indices in the tie band" % (name, band))

    @pytest.mark.parametrize("f", [0.0, 1.0, 0.5, 0.07])
    def test_fractions_ragged(self, f):
        keys = synth.keys(140, 2, 5000, "bf16")
        run_split(keys, keys.values[:, 17].copy(), f, "f=%g" % f)

    def test_degenerate_inputs(self):
        keys = synth.keys(141, 3, 4500, "f32")
        keys.values[0, 100:200] = 0.0          # zero-norm keys score 0
        keys.values[1] = keys.values[1, :1]    # every key identical: all ties, lowest indices win
        q = keys.values[:, 3].copy()
        q[2] = 0.0                             # zero query: every score 0
        run_split(keys, q, 0.3, "degenerate")
        ret, _ = kv.select_retrieval(keys_to_dev(keys), f32_to_dev(q), 0.3)
        nr = oracle.retrieval_count(4500, 0.3)
        assert np.array_equal(ret.cpu().numpy()[1], np.arange(nr))
        assert np.array_equal(ret.cpu().numpy()[2], np.arange(nr))

    @pytest.mark.parametrize("n", [20000, 40000])
    def test_many_candidates_in_one_bin(self, n):
        # 2500 keys that are power-of-two multiples of one key: the same cosine to a query
        # along that key, the largest of all, so the cut falls inside one tie group of
        # 2500 (a sort of the bin's candidates on one path, a radix select on the other)
        keys = synth.keys(143, 1, n, "f32")
        k0 = keys.values[0, 0].copy()
        keys.values[0, :2500] = k0[None, :] * (2.0 ** (np.arange(2500) % 8 - 4))[:, None]
        f = 1000.0 / n
        run_split(keys, k0[None, :].copy(), f, "tie group n=%d" % n)
        ret, _ = kv.select_retrieval(keys_to_dev(keys), f32_to_dev(k0[None, :].copy()), f)
        nr = oracle.retrieval_count(n, f)
        assert np.array_equal(ret.cpu().numpy()[0], np.arange(nr))

    def test_many_small_heads(self):
        # 200 heads of 777 keys: one partial histogram and one block a head, so every launch's
        # head index comes from the workgroup index alone
        keys = synth.keys(147, 200, 777, "bf16")
        run_split(keys, keys.values[:, 3].copy(), 0.13, "200 heads")

    @pytest.mark.parametrize("n", [100_001, 262_144, 300_000])
    def test_large_heads(self, n):
        # 100001: a ragged head of unaligned rows; 262144 and 300000: 500 to 1000 keys in the
        # cut's bin (rank counting one thread a candidate)
        keys = synth.keys(145, 1, n, "bf16")
        band = run_split(keys, keys.values[:, -1].copy(), 0.05, "n=%d" % n)
        print("n=%d: %d indices in the tie band" % (n, band))

    @pytest.mark.parametrize("n", [40_000, 300_000])
    def test_tie_group_and_identical_keys_both_paths(self, n):
        # a tie group of 2500 around the cut (sorted in LDS), and a head of identical keys (all
        # ties, lowest indices win; a radix select over the candidates in global memory)
        keys = synth.keys(146, 2, n, "f32")
        k0 = keys.values[0, 0].copy()
        keys.values[0, :2500] = k0[None, :] * (2.0 ** (np.arange(2500) % 8 - 4))[:, None]
        keys.values[1] = keys.values[1, :1]
        q = np.stack([k0, keys.values[1, 7]])
        f = 1000.0 / n
        run_split(keys, q, f, "ties n=%d" % n)
        ret, bulk = kv.select_retrieval(keys_to_dev(keys), f32_to_dev(q), f)
        nr = oracle.retrieval_count(n, f)
        assert np.array_equal(ret.cpu().numpy()[0], np.arange(nr))
        assert np.array_equal(ret.cpu().numpy()[1], np.arange(nr))
        assert np.array_equal(bulk.cpu().numpy()[1], np.arange(nr, n))

    def test_one_head_beyond_lds_offsets(self):
        # more than 4096 blocks of 1024 scores in one head (n > 4,194,304): the threshold pass
        # takes the candidates' block offsets from global memory instead of LDS
        n = 4_194_304 + 300_001
        rng = np.random.default_rng(77)
        x = rng.standard_normal((1, n, 128), dtype=np.float32)
        bits = synth.f32_to_bf16_bits(x)
        del x
        vals = synth.bf16_bits_to_f32(bits)
        kd = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
        ret, bulk = kv.select_retrieval(kd, kd[:, -1].contiguous(), 0.05)
        ro, _, cosv = oracle.select_retrieval(vals[0], vals[0, -1], 0.05)
        near = check_split(ret.cpu().numpy()[0], bulk.cpu().numpy()[0], n, cosv, ro, "4.5M keys")
        print("one head of %d keys: %d indices inside the tie band" % (n, near))

    def test_degenerate_long(self):
        # every key identical beyond the one-workgroup size: all ties, lowest indices win
        keys = synth.keys(144, 1, 40000, "f32")
        keys.values[0] = keys.values[0, :1]
        q = keys.values[:, 5].copy()
        ret, bulk = kv.select_retrieval(keys_to_dev(keys), f32_to_dev(q), 0.3)
        nr = oracle.retrieval_count(40000, 0.3)
        assert np.array_equal(ret.cpu().numpy()[0], np.arange(nr))
        assert np.array_equal(bulk.cpu().numpy()[0], np.arange(nr, 40000))

    def test_single_token(self):
        keys = synth.keys(142, 1, 1, "bf16")
        ret, bulk = kv.select_retrieval(keys_to_dev(keys), q_to_dev(keys.values[:, 0], "bf16"), 0.2)
        assert ret.cpu().numpy().tolist() == [[0]] and bulk.shape == (1, 0)


# ====================================================================== reconstruct
def oracle_rows(codes, pos, cb, w_cur, window, far_b, far_mode):
    out, _ = oracle.reconstruct(codes, pos, cb, w_cur, window, far_b, far_mode)
    return out


class TestReconstruct:
    def test_tiny_fp32_all_tokens(self):
        w = W["tiny"]
        cb = synth.codebook(w.cfg, 1, w.c)
        codes = synth.uniform_codes(w.cfg, (1, 1, w.n), w.c)
        pos = np.arange(w.n, dtype=np.int32)[None]
        out = kv.reconstruct(u16_to_dev(codes), torch.from_numpy(pos).to(DEV), f32_to_dev(cb),
                             w.cur_pos, w.window).cpu().numpy()
        ref = oracle_rows(codes[0, 0], pos[0], cb[0], w.cur_pos, w.window, w.far_b, 0)
        err, n_big = check_rotation(out[0, 0], ref, cb[0][codes[0, 0]].astype(np.float64), "f32", "tiny")
        print("tiny reconstruct max err %g, >1e-5: %d" % (err, n_big))

    def test_decode_sampled(self):
        w = W["decode"]
        cb = synth.codebook(w.cfg, w.heads, w.c)
        codes = synth.uniform_codes(w.cfg, (w.batch, w.heads, w.n), w.c)
        pos = np.tile(np.arange(w.n, dtype=np.int32), (w.batch, 1))
        out = kv.reconstruct(u16_to_dev(codes), torch.from_numpy(pos).to(DEV), f32_to_dev(cb),
                             w.cur_pos, w.window)
        rng = np.random.default_rng(5)
        b = rng.integers(0, w.batch, 4000)
        h = rng.integers(0, w.heads, 4000)
        t = np.concatenate([rng.integers(0, w.n, 3000), rng.integers(w.n - w.window - 4, w.n, 1000)])
        got = out[torch.from_numpy(b).to(DEV), torch.from_numpy(h).to(DEV),
                  torch.from_numpy(t).to(DEV)].cpu().numpy()
        for hh in range(w.heads):
            m = h == hh
            ref = oracle_rows(codes[b[m], hh, t[m]], pos[b[m], t[m]], cb[hh], w.cur_pos, w.window,
                              w.far_b, 0)
            check_rotation(got[m], ref, cb[hh][codes[b[m], hh, t[m]]].astype(np.float64), "f32",
                           "decode head %d" % hh)

    @pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
    def test_more_items_than_staged(self, out_dtype):
        # one head of 1027 work items (64 tokens each): the grid of 256 workgroups gives some
        # workgroup five items, one more than it stages in LDS (that one is read in the loop)
        w = W["long_context"]
        n = 1027 * 64
        cb = synth.codebook(w.cfg, 1, 256)
        codes = synth.uniform_codes(w.cfg, (1, 1, n), 256)
        pos = np.arange(n, dtype=np.int32)[None]
        dt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        out = kv.reconstruct(u16_to_dev(codes), torch.from_numpy(pos).to(DEV), f32_to_dev(cb),
                             n - 1, 300, out_dtype=dt)
        got = out[0, 0].cpu()
        got = got.numpy() if out_dtype == "f32" else synth.bf16_bits_to_f32(bf16_to_np_bits(got))
        ref = oracle_rows(codes[0, 0], pos[0], cb[0], n - 1, 300, 2048, 0)
        check_rotation(got, ref, cb[0][codes[0, 0]].astype(np.float64), out_dtype,
                       "five items a workgroup")

    def test_long_context_bf16_sampled(self):
        w = W["long_context"]
        cb = synth.codebook(w.cfg, w.heads, w.c)
        codes = synth.uniform_codes(w.cfg, (1, w.heads, w.n), w.c)
        pos = np.arange(w.n, dtype=np.int32)[None]
        out = kv.reconstruct(u16_to_dev(codes), torch.from_numpy(pos).to(DEV), f32_to_dev(cb),
                             w.cur_pos, w.window, out_dtype=torch.bfloat16)
        rng = np.random.default_rng(6)
        t = np.concatenate([rng.integers(0, w.n, 3000), np.arange(w.n - w.window - 8, w.n)])
        for hh in range(w.heads):
            got = bf16_to_np_bits(out[0, hh, torch.from_numpy(t).to(DEV)])
            ref = oracle_rows(codes[0, hh, t], pos[0, t], cb[hh], w.cur_pos, w.window, w.far_b, 0)
            check_rotation(synth.bf16_bits_to_f32(got), ref, cb[hh][codes[0, hh, t]].astype(np.float64),
                           "bf16", "long_context head %d" % hh)

    @pytest.mark.parametrize("window,far_mode,far_b", [(0, 0, 2048), (-5, 1, 2048), (10 ** 9, 0, 2048),
                                                       (300, 1, 0), (300, 0, 77), (1, 0, 5000)])
    def test_windows_and_modes(self, window, far_mode, far_b):
        cb = synth.codebook(150, 2, 90)
        codes = synth.uniform_codes(150, (2, 2, 1777), 90)
        pos = np.tile(np.arange(1777, dtype=np.int32), (2, 1))
        cur = 1800
        out = kv.reconstruct(u16_to_dev(codes), torch.from_numpy(pos).to(DEV), f32_to_dev(cb), cur,
                             window, far_offset=far_b, far_mode=far_mode).cpu().numpy()
        for b in range(2):
            for h in range(2):
                ref = oracle_rows(codes[b, h], pos[b], cb[h], cur, window, far_b, far_mode)
                check_rotation(out[b, h], ref, cb[h][codes[b, h]].astype(np.float64), "f32", "modes")

    def test_invalid_code_or_position_is_nan_and_window_is_bitwise_exact(self):
        cb = synth.codebook(151, 1, 50)
        codes = synth.uniform_codes(151, (1, 1, 600), 50)
        codes[0, 0, 7] = 50
        pos = np.arange(600, dtype=np.int32)[None].copy()
        pos[0, 9] = -3
        out = kv.reconstruct(u16_to_dev(codes), torch.from_numpy(pos).to(DEV), f32_to_dev(cb), 599, 64)
        o = out.cpu().numpy()[0, 0]
        assert np.all(np.isnan(o[7])) and np.all(np.isnan(o[9])) and np.isfinite(o[10]).all()
        exact = kv.reconstruct(u16_to_dev(codes), torch.from_numpy(pos).to(DEV), f32_to_dev(cb), 599,
                               10 ** 6).cpu().numpy()[0, 0]
        assert np.array_equal(o[536:], exact[536:])  # inside the window: identical to exact RoPE


# ====================================================================== pipeline
# ====================================================================== far keys unrotated
def ulp(v, dtype):
    """Spacing of the output format at |v| (fp32: 24 significant bits, bf16: 8)."""
    bits = 24 if dtype == "f32" else 8
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - (bits - 1))


def widen(t):
    return t.float().cpu().numpy().astype(np.float64)


class TestFarQueryRope:
    @pytest.mark.parametrize("rows,b", [(1, 2048), (3, 0), (1000, 2048), (777, 131071), (64, -5)])
    @pytest.mark.parametrize("dt_in,dt_out", [("f32", "f32"), ("bf16", "bf16"), ("f32", "bf16"),
                                              ("bf16", "f32")])
    def test_matches_oracle(self, rows, b, dt_in, dt_out):
        rng = np.random.default_rng(rows + 7 * abs(b))
        x = (rng.standard_normal((rows, 128)) * 3).astype(np.float32)
        if dt_in == "bf16":
            x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
        xd = torch.from_numpy(x).to(DEV)
        if dt_in == "bf16":
            xd = xd.to(torch.bfloat16)  # exact: x is already on the bf16 grid
        odt = torch.float32 if dt_out == "f32" else torch.bfloat16
        got = widen(kv.far_query_rope(xd, b, out_dtype=odt))
        ref = oracle.rope_at(x.astype(np.float64), b)
        # fp64 rotation rounded once: within one unit of the output format, and the single
        # nearest-even rounding of the oracle's value outside the angle band
        err = np.abs(got - ref)
        assert np.all(err <= ulp(ref, dt_out)), err.max()
        mag = np.abs(x) + np.abs(np.concatenate([x[:, 64:], x[:, :64]], axis=1))
        check_rounded_once(got, ref, mag.astype(np.float64), dt_out, abs(b) + 1, "far query rope")

    def test_in_place_and_batched_shape(self):
        rng = np.random.default_rng(3)
        x = (rng.standard_normal((2, 24, 5, 128))).astype(np.float32)
        xd = torch.from_numpy(x).to(DEV)
        want = kv.far_query_rope(xd.clone(), 2048)
        kv.far_query_rope(xd, 2048, out=xd)
        assert torch.equal(xd, want)
        ref = oracle.rope_at(x.reshape(-1, 128).astype(np.float64), 2048).reshape(x.shape)
        assert np.abs(xd.cpu().numpy() - ref).max() <= 2.0 ** -22 * np.abs(ref).max()

    def test_eq11_logits_against_fixed_offset_keys(self):
        # logits of one query against far keys: (q R_b) . k with unrotated keys (GPU) equal
        # RoPE(q, cur) . RoPE(k, cur - b), the fixed-offset form (oracle, fp64)
        w = W["decode"]
        cb = synth.codebook(w.cfg, 1, w.c)[0]
        rng = np.random.default_rng(11)
        n, cur, win, b = 4000, 5000, 256, 2048
        codes = rng.integers(0, w.c, n).astype(np.uint16)
        pos = np.arange(n, dtype=np.int32)
        q = rng.standard_normal((1, 128)).astype(np.float32)
        keys = kv.reconstruct(u16_to_dev(codes[None, None]), torch.from_numpy(pos[None]).to(DEV),
                              f32_to_dev(cb[None]), cur, win, far_mode=kv.FAR_UNROTATED)
        qb = kv.far_query_rope(torch.from_numpy(q).to(DEV), b)
        logits = (keys[0, 0].double() @ qb[0].double()).cpu().numpy()
        fixed, far = oracle.reconstruct(codes, pos, cb, cur, win, far_b=b)
        assert far == n
        ref = fixed @ oracle.rope_at(q.astype(np.float64), cur)[0]
        scale = np.abs(cb[codes]).sum(1) * np.abs(q).sum()
        assert np.all(np.abs(logits - ref) <= 1e-6 * scale)


class TestReconstructUpdate:
    @staticmethod
    def setup_case(batch, heads, n, c, seed, out_dtype):
        rng = np.random.default_rng(seed)
        cb = (rng.standard_normal((heads, c, 128)) * 2).astype(np.float32)
        codes = rng.integers(0, c, (batch, heads, n)).astype(np.uint16)
        pos = np.tile(np.arange(n, dtype=np.int32), (batch, 1))
        return (u16_to_dev(codes), torch.from_numpy(pos).to(DEV), f32_to_dev(cb),
                torch.float32 if out_dtype == "f32" else torch.bfloat16, codes, pos, cb)

    @staticmethod
    def full(codes, pos, cb, cur, win, odt):
        return kv.reconstruct(codes, pos, cb, cur, win, far_mode=kv.FAR_UNROTATED, out_dtype=odt)

    @pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
    @pytest.mark.parametrize("win", [64, 1, 0, -3, 100000])
    def test_steps_match_full_reconstruct(self, out_dtype, win):
        batch, heads, n, c = 2, 3, 3000, 70
        cd, pd, cbd, odt, codes, pos, cb = self.setup_case(batch, heads, n, c, 5, out_dtype)
        # decode steps: one token appended per step, the window slides by one; rows of
        # tokens not yet appended hold a sentinel until their first update writes them
        n_prev, cur = n - 10, n - 11
        out = self.full(cd, pd, cbd, cur, win, odt)
        out[:, :, n_prev:] = 7.0
        for step in range(10):
            kv.reconstruct_update(cd, pd, cbd, n_prev, cur, cur + 1, win, out)
            n_prev, cur = n_prev + 1, cur + 1
            assert torch.equal(out, self.full(cd, pd, cbd, cur, win, odt)), step
        # a jump of many positions at once
        kv.reconstruct_update(cd, pd, cbd, n, cur, cur + 150, win, out)
        assert torch.equal(out, self.full(cd, pd, cbd, cur + 150, win, odt))

    @pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
    def test_writes_only_changed_rows(self, out_dtype):
        batch, heads, n, c, win = 2, 2, 1500, 40, 100
        cd, pd, cbd, odt, codes, pos, cb = self.setup_case(batch, heads, n, c, 6, out_dtype)
        cur0, cur1, n_prev = 1200, 1260, 1490
        out = self.full(cd, pd, cbd, cur0, win, odt)
        # sentinels: one row whose status is unchanged (must survive), rows that crossed the
        # window edge and appended rows (must be rewritten)
        keep_t, cross_t, leave_t = 500, 1230, 1120
        out[:, :, keep_t] = 3.0
        out[:, :, cross_t] = 3.0   # far at cur0 (1230 > 1200: not yet seen), near at cur1
        out[:, :, leave_t] = 3.0   # near at cur0 (delta 80), far at cur1 (delta 140)
        out[:, :, n_prev:] = 3.0
        kv.reconstruct_update(cd, pd, cbd, n_prev, cur0, cur1, win, out)
        ref = self.full(cd, pd, cbd, cur1, win, odt)
        assert torch.all(out[:, :, keep_t] == 3.0)
        out[:, :, keep_t] = ref[:, :, keep_t]
        assert torch.equal(out, ref)

    def test_backwards_invalid_codes_and_positions(self):
        batch, heads, n, c, win = 1, 2, 800, 30, 50
        cd, pd, cbd, odt, codes, pos, cb = self.setup_case(batch, heads, n, c, 7, "f32")
        pos[0, 10] = -4
        codes[0, 1, 700] = 31  # >= c
        pd = torch.from_numpy(pos).to(DEV)
        cd = u16_to_dev(codes)
        out = self.full(cd, pd, cbd, 790, win, odt)
        kv.reconstruct_update(cd, pd, cbd, n, 790, 720, win, out)  # moving back in time
        ref = self.full(cd, pd, cbd, 720, win, odt)
        assert torch.equal(torch.nan_to_num(out, nan=-9.0), torch.nan_to_num(ref, nan=-9.0))
        assert torch.isnan(out[0, 1, 700]).all() and torch.isnan(out[0, :, 10]).all()

    def test_decode_shape_step_against_oracle(self):
        # the decode workload: 32 sequences x 8 heads x 16384 tokens, fp32, W=256; one step
        w = W["decode"]
        cb = synth.codebook(w.cfg, w.heads, w.c)
        codes = synth.uniform_codes(w.cfg, (w.batch, w.heads, w.n), w.c)
        pos = np.tile(np.arange(w.n, dtype=np.int32), (w.batch, 1))
        cd, pd, cbd = u16_to_dev(codes), torch.from_numpy(pos).to(DEV), f32_to_dev(cb)
        cur = w.n - 1
        out = kv.reconstruct(cd, pd, cbd, cur - 1, w.window, far_mode=kv.FAR_UNROTATED)
        kv.reconstruct_update(cd, pd, cbd, w.n - 1, cur - 1, cur, w.window, out)
        full = kv.reconstruct(cd, pd, cbd, cur, w.window, far_mode=kv.FAR_UNROTATED)
        assert torch.equal(out, full)
        # the rows the step changed, against the oracle
        for t in (cur - w.window, w.n - 1, cur - w.window + 1, 0):
            for hh in (0, 5):
                got = out[:, hh, t].cpu().numpy()
                ref, _ = oracle.reconstruct(codes[:, hh, t], pos[:, t], cb[hh], cur, w.window,
                                            far_mode=oracle.FAR_UNROTATED)
                check_rotation(got, ref, cb[hh][codes[:, hh, t]].astype(np.float64), "f32",
                               "decode step token %d head %d" % (t, hh))


# ====================================================================== sub-vector codes
def sub_rows(x, sub):
    """[.., n, d] -> [.. * n * d/sub, sub] (row-major: sub-spaces of a row consecutive)."""
    return np.ascontiguousarray(x.reshape(-1, sub))


class TestPQ:
    @staticmethod
    def inputs(n, sub, k, dtype, seed):
        keys = synth.keys(200 + seed, 2, n, dtype)
        cb = synth.pq_codebook(200 + seed, 2, k, sub)
        q = synth.queries(200 + seed, 2, 512)
        l = oracle.cholesky(oracle.second_moment(sub_rows(q, sub), 1e-4))
        return keys, cb, l

    @pytest.mark.parametrize("sub,k", [(8, 256), (4, 256), (8, 16)])
    @pytest.mark.parametrize("dtype", ["bf16", "f32"])
    @pytest.mark.parametrize("mode", ["plain", "h"])
    def test_encode_matches_oracle(self, sub, k, dtype, mode):
        keys, cb, l = self.inputs(700, sub, k, dtype, 1)
        lt = f32_to_dev(l.astype(np.float32)) if mode == "h" else None
        got = kv.pq_encode(keys_to_dev(keys), f32_to_dev(cb), sub, chol=lt).cpu().numpy()
        # the oracle sees the same fp32 factor the kernel does
        lref = l.astype(np.float32).astype(np.float64) if mode == "h" else None
        code, d1, d2 = oracle.assign_h(sub_rows(keys.values, sub), cb, lref)
        check_codes(got.reshape(-1).astype(np.int64), code, d1, d2, "pq %s sub %d k %d" % (mode, sub, k))

    @pytest.mark.parametrize("sub", [8, 4])
    @pytest.mark.parametrize("beta", [0.5, 1.0, 0.0])
    def test_blend_matches_oracle(self, sub, beta):
        keys, cb, _ = self.inputs(300, sub, 256, "bf16", 2)
        xd = keys_to_dev(keys)
        got = kv.pq_encode(xd, f32_to_dev(cb), sub, query=xd[:, -1:].contiguous(), beta=beta)
        got = got.cpu().numpy()
        m = 128 // sub
        for h in range(2):
            x = keys.values[h]
            for s_ in range(m):
                sl = slice(s_ * sub, (s_ + 1) * sub)
                code, s1, s2 = oracle.assign_cosine(x[:, sl], x[-1, sl], cb, beta)
                bad = (s1 - s2 > 1e-5) & (got[h, :, s_] != code)
                assert not bad.any(), (h, s_, np.nonzero(bad)[0][:5])

    def test_idx_rows_only_and_layer_shape_sampled(self):
        w = W["pq_layer"]
        keys = synth.keys(w.cfg, w.heads, w.n, w.key_dtype)
        cb = synth.pq_codebook(w.cfg, w.heads, w.c, 8)
        q = synth.queries(w.cfg, w.heads, w.m)
        hq, lq = kv.calibrate(f32_to_dev(sub_rows(q, 8)[None]), 1e-4)  # one 8x8 H, pooled
        kd = keys_to_dev(keys)
        ret, bulk = kv.select_retrieval(kd, kd[:, -1].contiguous(), w.fraction)
        codes = torch.full((w.heads, w.n, 16), 255, dtype=torch.uint8, device=DEV)
        kv.pq_encode(kd, f32_to_dev(cb), 8, idx=bulk, codes=codes)
        kv.pq_encode(kd, f32_to_dev(cb), 8, chol=lq[0], idx=ret, codes=codes)
        got = codes.cpu().numpy()
        ret, bulk = ret.cpu().numpy(), bulk.cpu().numpy()
        lref = lq[0].cpu().numpy().astype(np.float64)
        rng = np.random.default_rng(3)
        for h in range(w.heads):
            for rows, lf in ((rng.choice(ret[h], 300, replace=False), lref),
                             (rng.choice(bulk[h], 300, replace=False), None)):
                code, d1, d2 = oracle.assign_h(sub_rows(keys.values[h, rows], 8), cb, lf)
                check_codes(got[h, rows].reshape(-1).astype(np.int64), code, d1, d2, "head %d" % h)
        # a row selected by neither list keeps its initial bytes: every row is in one list
        assert (got != 255).any(axis=2).all()

    @pytest.mark.parametrize("sub", [8, 4])
    @pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
    def test_reconstruct_matches_oracle(self, sub, out_dtype):
        rng = np.random.default_rng(9)
        batch, heads, n, k, m = 2, 3, 1100, 200, 128 // sub
        cb = synth.pq_codebook(210, 2, k, sub)
        codes = rng.integers(0, k, (batch, heads, n, m)).astype(np.uint8)
        pos = np.tile(np.arange(n, dtype=np.int32), (batch, 1))
        cur, win, b = n - 1, 100, 2048
        odt = torch.float32 if out_dtype == "f32" else torch.bfloat16
        out = kv.pq_reconstruct(torch.from_numpy(codes).to(DEV), torch.from_numpy(pos).to(DEV),
                                f32_to_dev(cb), cur, win, b, out_dtype=odt)
        for bb in range(batch):
            for h in range(heads):
                full = cb[codes[bb, h]].reshape(n, 128).astype(np.float64)  # concatenated
                ref, _ = oracle.reconstruct(np.arange(n, dtype=np.uint16), pos[bb], full, cur,
                                            win, b)
                if out_dtype == "f32":
                    check_rotation(out[bb, h].cpu().numpy(), ref, full, "f32", "pq %d %d" % (bb, h))
                else:
                    check_rotation(out[bb, h].float().cpu().numpy(), ref, full, "bf16", "pq")

    def test_values_are_a_plain_gather_and_invalid_codes_nan(self):
        rng = np.random.default_rng(10)
        n, k = 500, 64
        cb = synth.pq_codebook(211, 1, k, 8)
        codes = rng.integers(0, k, (1, 2, n, 16)).astype(np.uint8)
        codes[0, 1, 7, 3] = 200  # >= k
        pos = np.arange(n, dtype=np.int32)[None].copy()
        pos[0, 9] = -1
        out = kv.pq_reconstruct(torch.from_numpy(codes).to(DEV), torch.from_numpy(pos).to(DEV),
                                f32_to_dev(cb), n - 1, 0, far_mode=kv.FAR_UNROTATED).cpu().numpy()
        want = cb[np.minimum(codes, k - 1)].reshape(1, 2, n, 128)
        ok = np.ones((1, 2, n), bool)
        ok[0, 1, 7] = False
        ok[0, :, 9] = False
        assert np.array_equal(out[ok], want[ok])
        assert np.isnan(out[~ok]).all()


# ====================================================================== codebook training
def f32_ulp(v):
    return np.spacing(np.abs(np.asarray(v, np.float32))).astype(np.float64)


class TestKmeans:
    @pytest.mark.parametrize("d,dtype", [(128, "bf16"), (128, "f32"), (8, "f32"), (4, "bf16")])
    def test_update_matches_oracle(self, d, dtype):
        rng = np.random.default_rng(50 + d)
        heads, n, k = 2, 3072, 64
        keys = synth.keys(60 + d, heads, n * d // 128, dtype)
        x = keys.values.reshape(heads, n, d)
        codes = rng.integers(0, k + 3, (heads, n))  # k .. k+2: ignored
        codes[codes == 7] = 8                       # cluster 7 empty in both heads
        cb = rng.standard_normal((heads, k, d)).astype(np.float32)
        xd = torch.from_numpy(x).to(DEV)
        if dtype == "bf16":
            xd = xd.to(torch.bfloat16)  # exact: the values are on the bf16 grid
        ct = torch.uint16 if d == 128 else torch.uint8
        cd = torch.from_numpy(codes.astype(np.uint16 if d == 128 else np.uint8)).to(DEV)
        out, cnt = kv.kmeans_update(xd, cd, f32_to_dev(cb), want_counts=True)
        out, cnt = out.cpu().numpy(), cnt.cpu().numpy()
        for h in range(heads):
            ref, rc = oracle.kmeans_update(x[h], codes[h], cb[h])
            assert np.array_equal(cnt[h], rc)
            ref32 = ref.astype(np.float32)
            if d == 128:  # members summed in ascending row order, as the oracle does
                assert np.array_equal(out[h], ref32)
            else:         # interleaved member subsets: within one fp32 unit
                assert np.all(np.abs(out[h] - ref32) <= f32_ulp(ref32))
            assert np.array_equal(out[h, 7], cb[h, 7])

    def test_update_layer_shape(self):
        # the codebook-training update at the layer workload's size (8 heads x 32768 bf16
        # keys, k = 1024 per head; uniform codes: ~32 members a cluster, so every sum runs in
        # ascending row order and the result is bitwise the oracle's), plus a large cluster
        # (more than 256 members: segmented sums, within one fp32 unit)
        w = W["layer"]
        keys = synth.keys(w.cfg, w.heads, w.n, "bf16")
        codes = synth.uniform_codes(w.cfg, (w.heads, w.n), w.c).astype(np.int64)
        codes[:, :4000] = 5  # cluster 5: 4000+ members in every head
        cb = synth.codebook(w.cfg, w.heads, w.c)
        out, cnt = kv.kmeans_update(keys_to_dev(keys), torch.from_numpy(codes.astype(np.uint16)).to(DEV),
                                    f32_to_dev(cb), want_counts=True)
        out, cnt = out.cpu().numpy(), cnt.cpu().numpy()
        for h in range(w.heads):
            ref, rc = oracle.kmeans_update(keys.values[h], codes[h], cb[h])
            assert np.array_equal(cnt[h], rc)
            ref32 = ref.astype(np.float32)
            small = rc <= 256
            assert np.array_equal(out[h][small], ref32[small])
            assert np.all(np.abs(out[h] - ref32) <= f32_ulp(ref32))

    def test_update_is_deterministic(self):
        keys = synth.keys(70, 2, 5000, "bf16")
        xd = keys_to_dev(keys)
        codes = torch.from_numpy(np.random.default_rng(1).integers(0, 300, (2, 5000)).astype(np.uint16)).to(DEV)
        cb = f32_to_dev(np.zeros((2, 300, 128), np.float32))
        a = kv.kmeans_update(xd, codes, cb)
        b = kv.kmeans_update(xd, codes, cb)
        assert torch.equal(a, b)

    @pytest.mark.parametrize("use_h", [True, False])
    def test_lloyd_whole_vectors_matches_oracle(self, use_h):
        w = W["layer"]
        heads, n, k = 2, 4096, 64
        keys = synth.keys(w.cfg, heads, n, "bf16")
        cb0 = keys.values[:, ::n // k][:, :k].copy()  # k spread rows as the initial codebook
        lt = None
        if use_h:
            _, lt = kv.calibrate(f32_to_dev(synth.queries(w.cfg, heads, 1024)), 1e-4)
        cbd = f32_to_dev(cb0)
        cbd, codes = kv.kmeans(keys_to_dev(keys), cbd, lt, iters=4)
        got_cb, got_code = cbd.cpu().numpy(), codes.cpu().numpy()
        for h in range(heads):
            lref = lt[h].cpu().numpy().astype(np.float64) if use_h else None
            ref_cb, ref_code = oracle.kmeans(keys.values[h], cb0[h], lref, iters=4)
            assert np.array_equal(got_code[h], ref_code)
            assert np.array_equal(got_cb[h], ref_cb.astype(np.float32))

    def test_lloyd_pooled_sub_vectors(self):
        # Round by round: the GPU's assignment of the GPU's current codebook against the
        # oracle's assignment of that same codebook (bit-exact outside the 1e-5 tie band),
        # then the GPU's update of those codes against the oracle's update of the same codes
        # (a cluster's members are summed in interleaved subsets: within one fp32 unit).  The
        # driver's rounds equal the same rounds taken one call at a time, bit for bit.
        w = W["pq_layer"]
        keys = synth.keys(w.cfg, 1, 2048, "f32")
        x = np.ascontiguousarray(keys.values[0].reshape(-1, 8))  # the pages' reshape(-1, sub_dim)
        cb0 = x[::x.shape[0] // 256][:256].copy()
        q = synth.queries(w.cfg, 1, 512)
        _, lt = kv.calibrate(f32_to_dev(np.ascontiguousarray(q.reshape(1, -1, 8))), 1e-4)
        l0 = lt[0].contiguous()
        lref = l0.cpu().numpy().astype(np.float64)
        xd = f32_to_dev(x)
        cb = f32_to_dev(cb0)
        rounds = 3
        for r in range(rounds + 1):
            _, codes = kv.kmeans(xd, cb.clone(), l0, iters=0)  # assignment of the current codebook
            got_code = codes.cpu().numpy().astype(np.int64)
            cur = cb.cpu().numpy()
            code, d1, d2 = oracle.assign_h(x, cur, lref)
            check_codes(got_code, code, d1, d2, "pooled round %d" % r)
            if r == rounds:
                break
            new = kv.kmeans_update(xd[None], codes[None], cb[None])[0]
            ref, _ = oracle.kmeans_update(x, got_code, cur)
            ref32 = ref.astype(np.float32)
            assert np.all(np.abs(new.cpu().numpy() - ref32) <= f32_ulp(ref32)), r
            cb = new.contiguous()
        cbd, codes = kv.kmeans(xd, f32_to_dev(cb0), l0, iters=rounds)
        assert torch.equal(cbd, cb)
        assert np.array_equal(codes.cpu().numpy().astype(np.int64), got_code)
        # the H-weighted objective of the trained codebook is no worse than the initial one
        _, d_init, _ = oracle.assign_h(x, cb0, lref)
        _, d_fin, _ = oracle.assign_h(x, cbd.cpu().numpy(), lref)
        assert d_fin.sum() < d_init.sum()


def draws_u64(seed, shape):
    return np.random.default_rng(seed).integers(0, 2 ** 64, size=shape, dtype=np.uint64)


def u64_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int64)).to(DEV)


class TestKmeansInit:
    """k-means++ seeding in z-space: the chosen rows equal the oracle's, bit for bit."""

    def test_layer_shape_h_weighted(self):
        # 2 heads of the layer workload (32768 bf16 keys each), k = 1024, L from calibration
        w = W["layer"]
        heads = 2
        keys = synth.keys(w.cfg, heads, w.n, "bf16")
        _, lt = kv.calibrate(f32_to_dev(synth.queries(w.cfg, heads, w.m)), 1e-4)
        r = draws_u64(60, (heads, w.c))
        cb, idx = kv.kmeans_init(keys_to_dev(keys), w.c, u64_to_dev(r), lt, want_idx=True)
        idx, cb = idx.cpu().numpy(), cb.cpu().numpy()
        lref = lt.cpu().numpy().astype(np.float64)
        for h in range(heads):
            want = oracle.kmeans_init(keys.values[h], w.c, r[h], lref[h])
            assert np.array_equal(idx[h], want), (h, np.nonzero(idx[h] != want)[0][:5])
            assert np.array_equal(cb[h], keys.values[h][want])
            assert len(np.unique(want)) == w.c

    def test_pooled_sub_vectors(self):
        # the pages' shared sub-vector codebook: keys pooled as [-1, 8] (131072 sub-vectors of
        # 8192 keys), k = 256, one 8x8 L from the pooled query sub-vectors
        w = W["pq_layer"]
        keys = synth.keys(w.cfg, 1, 8192, "bf16")
        x = np.ascontiguousarray(keys.values[0].reshape(-1, 8))
        xb = keys_to_dev(keys).reshape(-1, 8)
        q = synth.queries(w.cfg, 1, 1024)
        _, lt = kv.calibrate(f32_to_dev(np.ascontiguousarray(q.reshape(1, -1, 8))), 1e-4)
        r = draws_u64(61, 256)
        cb, idx = kv.kmeans_init(xb, 256, u64_to_dev(r), lt[0].contiguous(), want_idx=True)
        want = oracle.kmeans_init(x, 256, r, lt[0].cpu().numpy().astype(np.float64))
        assert np.array_equal(idx.cpu().numpy(), want)
        assert np.array_equal(cb.cpu().numpy(), x[want])

    @pytest.mark.parametrize("n,d,k,dtype,use_h", [(1000, 128, 37, "f32", True),
                                                   (3000, 8, 300, "bf16", False),
                                                   (777, 4, 777, "f32", True),
                                                   (5, 16, 1, "bf16", True),
                                                   (2049, 32, 64, "bf16", True)])
    def test_shapes(self, n, d, k, dtype, use_h):
        rng = np.random.default_rng(n + d)
        x = (rng.standard_normal((2, n, d)) * rng.uniform(0.3, 3.0, d)).astype(np.float32)
        if dtype == "bf16":
            x = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
        xd = torch.from_numpy(x).to(DEV)
        if dtype == "bf16":
            xd = xd.to(torch.bfloat16)  # exact: x is on the bf16 grid
        l = None
        if use_h:
            l = np.stack([np.tril(rng.standard_normal((d, d)) * 0.2) + np.diag(rng.uniform(0.5, 2.0, d))
                          for _ in range(2)]).astype(np.float32)
        r = draws_u64(n * 7 + k, (2, k))
        cb, idx = kv.kmeans_init(xd, k, u64_to_dev(r), f32_to_dev(l) if use_h else None, want_idx=True)
        idx, cb = idx.cpu().numpy(), cb.cpu().numpy()
        for h in range(2):
            want = oracle.kmeans_init(x[h], k, r[h], None if l is None else l[h].astype(np.float64))
            assert np.array_equal(idx[h], want), (h, np.nonzero(idx[h] != want)[0][:5])
            assert np.array_equal(cb[h], x[h][want])

    def test_duplicates_fall_back_to_uniform_draws(self):
        # 3 distinct rows repeated: after the three are chosen every weight is 0
        base = np.array([[1.0, 2.0, 0.5, -1.0], [4.0, 0.0, 1.0, 2.0], [-3.0, 1.0, 1.0, 0.0]],
                        np.float32)
        x = np.repeat(base, 700, axis=0)[None]
        r = draws_u64(62, (1, 10))
        cb, idx = kv.kmeans_init(torch.from_numpy(x).to(DEV), 10, u64_to_dev(r), want_idx=True)
        want = oracle.kmeans_init(x[0], 10, r[0])
        assert np.array_equal(idx.cpu().numpy()[0], want)
        assert len({tuple(v) for v in x[0][want[:3]]}) == 3


class TestPipeline:
    def test_two_streams_prepared_equals_sequential(self):
        # the benchmark's step: prepares and the H-weighted encode on a second stream
        w = W["layer"]
        keys = synth.keys(w.cfg, w.heads, w.n, w.key_dtype)
        kd, cbd = keys_to_dev(keys), f32_to_dev(synth.codebook(w.cfg, w.heads, w.c))
        H, L = kv.calibrate(f32_to_dev(synth.queries(w.cfg, w.heads, w.m)), 1e-4)
        proxy = kd[:, -1].contiguous()
        ret, bulk = kv.select_retrieval(kd, proxy, w.fraction)
        seq = kv.encode(kd, cbd, None)
        seq = kv.encode(kd, cbd, L, idx=ret, codes=seq)
        aux = torch.cuda.Stream(device=DEV)
        main = torch.cuda.current_stream(DEV)
        codes = torch.zeros((w.heads, w.n), dtype=torch.uint16, device=DEV)
        for _ in range(3):  # repeated steps reuse nothing but the tensors above
            aux.wait_event(main.record_event())
            with torch.cuda.stream(aux):
                pp = kv.encode_prepare(cbd, None, w.n)
                plain_ready = aux.record_event()
                ph = kv.encode_prepare(cbd, L, w.n)
            r2, b2 = kv.select_retrieval(kd, proxy, w.fraction)
            split_done = main.record_event()
            main.wait_event(plain_ready)
            kv.encode_prepared(kd, pp, idx=b2, codes=codes)
            aux.wait_event(split_done)
            with torch.cuda.stream(aux):
                kv.encode_prepared(kd, ph, idx=r2, codes=codes)
            main.wait_event(aux.record_event())
            torch.cuda.synchronize()
            assert torch.equal(codes.view(torch.int16), seq.view(torch.int16))
            del pp, ph

    def test_graph_replays_match_eager(self):
        # the benchmark's step captured in a HIP graph: every replay, with eager work and
        # synchronisations between replays, gives the eager step's codes and keys bit for bit
        w = W["layer"]
        keys = synth.keys(w.cfg, w.heads, w.n, w.key_dtype)
        kd, cbd = keys_to_dev(keys), f32_to_dev(synth.codebook(w.cfg, w.heads, w.c))
        H, L = kv.calibrate(f32_to_dev(synth.queries(w.cfg, w.heads, w.m)), 1e-4)
        proxy = kd[:, -1].contiguous()
        pos = torch.arange(w.n, dtype=torch.int32, device=DEV)[None]
        codes = torch.zeros((w.heads, w.n), dtype=torch.uint16, device=DEV)
        out = torch.empty((1, w.heads, w.n, 128), dtype=torch.bfloat16, device=DEV)
        aux = torch.cuda.Stream(device=DEV)
        pp, ph = kv.encode_prepare(cbd, None, w.n), kv.encode_prepare(cbd, L, w.n)

        def step():
            main = torch.cuda.current_stream(DEV)
            aux.wait_event(main.record_event())
            with torch.cuda.stream(aux):
                pp.prepare(cbd, None)
                plain_ready = aux.record_event()
                ph.prepare(cbd, L)
            ret, bulk = kv.select_retrieval(kd, proxy, w.fraction)
            split_done = main.record_event()
            main.wait_event(plain_ready)
            kv.encode_prepared(kd, pp, idx=bulk, codes=codes)
            aux.wait_event(split_done)
            with torch.cuda.stream(aux):
                kv.encode_prepared(kd, ph, idx=ret, codes=codes)
            main.wait_event(aux.record_event())
            kv.reconstruct(codes[None], pos, cbd, w.cur_pos, w.window, out=out)

        step()
        torch.cuda.synchronize()
        ref_codes, ref_out = codes.clone(), out.view(torch.int16).clone()
        side = torch.cuda.Stream(device=DEV)
        side.wait_stream(torch.cuda.current_stream(DEV))
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream(DEV).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(4):
            codes.fill_(7)
            out.fill_(1.0)
            step()  # eager work between replays
            torch.cuda.synchronize()
            codes.fill_(7)
            out.fill_(1.0)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(codes, ref_codes)
            assert torch.equal(out.view(torch.int16), ref_out)

    def test_merge_codes(self):
        rng = np.random.default_rng(11)
        heads, n = 3, 5000
        base = rng.integers(0, 65536, (heads, n), dtype=np.uint16)
        src = rng.integers(0, 65536, (heads, n), dtype=np.uint16)
        idx = np.stack([np.sort(rng.choice(n, 700, replace=False)) for _ in range(heads)]).astype(np.int32)
        idx[1, 5] = -3      # skipped
        idx[2, 9] = n + 4   # skipped
        want = base.copy()
        for h in range(heads):
            ok = (idx[h] >= 0) & (idx[h] < n)
            want[h, idx[h][ok]] = src[h, idx[h][ok]]
        codes = u16_to_dev(base)
        kv.merge_codes(codes, u16_to_dev(src), torch.from_numpy(idx).to(DEV))
        assert np.array_equal(u16_to_np(codes), want)

    def test_all_plain_then_merge_equals_split_passes(self):
        # the pages' order (plain codes for every key, query-aware codes at the retrieval
        # indices) run as two independent passes plus the merge, against bulk + retrieval
        w = W["layer"]
        keys = synth.keys(w.cfg, w.heads, w.n, w.key_dtype)
        kd, cbd = keys_to_dev(keys), f32_to_dev(synth.codebook(w.cfg, w.heads, w.c))
        H, L = kv.calibrate(f32_to_dev(synth.queries(w.cfg, w.heads, w.m)), 1e-4)
        ret, bulk = kv.select_retrieval(kd, kd[:, -1].contiguous(), w.fraction)
        ref = kv.encode(kd, cbd, None, idx=bulk)
        ref = kv.encode(kd, cbd, L, idx=ret, codes=ref)
        allp = kv.encode(kd, cbd, None)
        hcodes = kv.encode(kd, cbd, L, idx=ret)
        kv.merge_codes(allp, hcodes, ret)
        assert torch.equal(allp.view(torch.int16), ref.view(torch.int16))

    @pytest.mark.parametrize("name", ["layer", "long_context"])
    def test_split_encode_reconstruct(self, name):
        w = W[name]
        keys = synth.keys(w.cfg, w.heads, w.n, w.key_dtype)
        cb = synth.codebook(w.cfg, w.heads, w.c)
        q = synth.queries(w.cfg, w.heads, w.m)
        kd, cbd = keys_to_dev(keys), f32_to_dev(cb)
        H, L = kv.calibrate(f32_to_dev(q), 1e-4)
        ret, bulk = kv.select_retrieval(kd, kd[:, -1].contiguous(), w.fraction)
        codes = kv.encode(kd, cbd, None)
        codes = kv.encode(kd, cbd, L, idx=ret, codes=codes)
        out = kv.reconstruct(codes[None].contiguous(), torch.arange(w.n, dtype=torch.int32, device=DEV)[None],
                             cbd, w.cur_pos, w.window, out_dtype=torch.bfloat16)
        Lh = L.cpu().numpy()
        codes_np = u16_to_np(codes)
        ret_np = ret.cpu().numpy()
        rng = np.random.default_rng(7)
        for h in range(w.heads):
            r = ret_np[h][rng.choice(ret_np.shape[1], 256, replace=False)]
            code, d1, d2 = oracle.assign_h(keys.values[h][r], cb[h], Lh[h])
            check_codes(codes_np[h][r], code, d1, d2, "%s retrieval rows" % name)
            b = np.setdiff1d(rng.choice(w.n, 600, replace=False), ret_np[h])[:256]
            code, d1, d2 = oracle.assign_h(keys.values[h][b], cb[h], None)
            check_codes(codes_np[h][b], code, d1, d2, "%s bulk rows" % name)
            t = np.concatenate([b, np.arange(w.n - 16, w.n)])
            got = synth.bf16_bits_to_f32(bf16_to_np_bits(out[0, h, torch.from_numpy(t).to(DEV)]))
            ref = oracle_rows(codes_np[h][t], t.astype(np.int32), cb[h], w.cur_pos, w.window, w.far_b, 0)
            check_rotation(got, ref, cb[h][codes_np[h][t]].astype(np.float64), "bf16", name)


# --------------------------------------------------------------------------- top-K over codes
def topk_case(qb, codes, cb, k, qdt="f32"):
    """GPU top-K of qb [batch, hq, 128] fp32 (on the bf16 grid when qdt is bf16) against the
    oracle row by row: indices bit-exact, scores bit-exact (as values: -0 == +0)."""
    batch, hq, _ = qb.shape
    hkv = codes.shape[1]
    qd = torch.from_numpy(np.ascontiguousarray(qb)).to(DEV)
    if qdt == "bf16":
        qd = qd.to(torch.bfloat16)  # exact: qb is already on the bf16 grid
    idx, sc = kv.topk_codes(qd, u16_to_dev(codes), f32_to_dev(cb), k)
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy().astype(np.float64)
    g = hq // hkv
    for b in range(batch):
        for h in range(hq):
            ri, rs = oracle.topk_codes(qb[b, h].astype(np.float64), codes[b, h // g], cb[h // g], k)
            assert np.array_equal(idx[b, h], ri), (b, h, np.flatnonzero(idx[b, h] != ri)[:5])
            assert np.array_equal(sc[b, h], rs), (b, h)
    return idx, sc


def bf16_grid(x):
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(x, np.float32)))


class TestTopkCodes:
    # (batch, hq, hkv, n, c, k): every group size the kernel templates on (1..4), groups split
    # over workgroups (8 = 4 + 4, 5 = 4 + 1 partial), ragged token counts, partial codebook
    # tiles, several tiles (c = 4096), rows too long for LDS (n > 32768), and more of a key
    # head's queries than one table workgroup takes (96): 100 = 96 + 4 and 320 = 3 x 96 + 32
    @pytest.mark.parametrize("batch,hq,hkv,n,c,k", [
        (2, 6, 2, 3000, 256, 300), (1, 3, 3, 1000, 1000, 1), (3, 4, 2, 4097, 1024, 4097),
        (1, 8, 2, 5000, 300, 777), (2, 4, 1, 2048, 4096, 1500), (1, 5, 1, 999, 64, 100),
        (1, 2, 1, 40000, 1024, 4000), (1, 1, 1, 1, 1, 1), (2, 2, 2, 65, 7, 64),
        (1, 3, 1, 3000, 1500, 700), (50, 4, 2, 600, 300, 50), (40, 8, 1, 300, 100, 30)])
    @pytest.mark.parametrize("qdt", ["f32", "bf16"])
    def test_matches_oracle(self, batch, hq, hkv, n, c, k, qdt):
        rng = np.random.default_rng(batch * 1000 + hq * 100 + n + c)
        cb = (rng.standard_normal((hkv, c, 128)) * 2).astype(np.float32)
        codes = rng.integers(0, c, (batch, hkv, n)).astype(np.uint16)
        qb = rng.standard_normal((batch, hq, 128)).astype(np.float32)
        if qdt == "bf16":
            qb = bf16_grid(qb)
        topk_case(qb, codes, cb, k, qdt)

    @pytest.mark.parametrize("k", [1, 37, 500, 1999, 2000])
    def test_ties_invalid_codes_and_signed_zero(self, k):
        # a codebook of four values (one repeated) over 2000 tokens: the cut falls inside runs
        # of equal scores; codes >= c score -inf; a zero query ties every valid token at 0
        rng = np.random.default_rng(k)
        base = rng.standard_normal((3, 128)).astype(np.float32)
        cb = np.stack([base[0], base[1], base[0], base[2]])[None]  # entries 0 and 2 equal
        codes = rng.integers(0, 6, (1, 1, 2000)).astype(np.uint16)  # 4, 5 are invalid
        qb = np.stack([rng.standard_normal(128), np.zeros(128), -np.zeros(128)])[None]
        qb = qb.astype(np.float32)
        idx, sc = topk_case(qb, codes, cb, k)
        # the zero queries take the lowest-indexed valid tokens, then invalid ones at -inf
        valid = np.flatnonzero(codes[0, 0] < 4)
        want = np.sort(np.concatenate([valid, np.flatnonzero(codes[0, 0] >= 4)])[:k])
        assert np.array_equal(idx[0, 1], want) and np.array_equal(idx[0, 2], want)

    def test_clustered_scores_several_passes(self):
        # q = e_0 makes score_j = cb[j, 0] exactly: 1500 entries spread over [-100, 100] and
        # a run of 500 consecutive fp32 values at 1.0 (two groups of 24 equal to members of the
        # run), so the first select pass's bin holding the cut has far more than 64 entries
        # and a second pass over the run's range splits them (C = 2048: two entries a thread)
        rng = np.random.default_rng(11)
        c, n = 2048, 20000
        cb = rng.standard_normal((1, c, 128)).astype(np.float32)
        run = np.float32(1.0) + np.arange(500, dtype=np.float32) * np.float32(2.0 ** -23)
        v = rng.uniform(-100, 100, c).astype(np.float32)
        v[:500] = run
        v[500:524] = run[100]
        v[524:548] = run[300]
        cb[0, :, 0] = rng.permutation(v)
        qb = np.zeros((1, 2, 128), np.float32)
        qb[0, :, 0] = 1.0
        qb[0, 1, 0] = 2.0  # the same order at twice the scale
        codes = rng.integers(0, c, (1, 1, n)).astype(np.uint16)
        s = cb[0, codes[0, 0], 0]
        above = int(np.sum(s > run[250]))
        for k in (above, above + 1, above + 37, int(np.sum(s >= run[100]))):
            topk_case(qb, codes, cb, k)

    def test_table_sum_order_under_cancellation(self):
        # every table entry is a score (each code once, k = n); the terms of dimensions 64..127
        # are those of 0..63 negated, with magnitudes over 80 binades, so each entry is the
        # rounding left over by the fp64 sum in dimension order: another order (a pairwise tree,
        # checked here on the CPU) changes most entries, and bit-exact scores pin the order
        rng = np.random.default_rng(21)
        c, batch, hq = 4096, 2, 4

        def wide(shape):
            return (rng.uniform(1, 2, shape) * np.exp2(rng.integers(-20, 21, shape))
                    * rng.choice([-1, 1], shape)).astype(np.float32)
        half = wide((1, c, 64))
        cb = np.concatenate([half, half], axis=2)
        qh = wide((batch, hq, 64))
        qb = np.concatenate([qh, -qh], axis=2)
        qb[:, :, 0] = 1.0
        cb[0, :, 0] = rng.standard_normal(c).astype(np.float32)
        terms = cb[0].astype(np.float64) * qb[0, 0].astype(np.float64)  # exact products
        seq = np.zeros(c)
        for a in range(128):
            seq = seq + terms[:, a]
        changed = np.sum(seq.astype(np.float32) != np.sum(terms, axis=1).astype(np.float32))
        assert changed > c // 2, changed
        codes = np.stack([rng.permutation(c) for _ in range(batch)])[:, None].astype(np.uint16)
        topk_case(qb, codes, cb, c)

    @pytest.mark.parametrize("k", [1, 400, 1000, 4990])
    def test_infinite_scores(self, k):
        # scores beyond the fp32 range round to +inf or -inf, so the select bins by shifts of
        # the order key; hundreds of tokens tie at +inf, and -inf scores tie with the invalid
        # codes (codes >= c)
        rng = np.random.default_rng(12)
        c, n = 600, 5000
        cb = rng.standard_normal((1, c, 128)).astype(np.float32)
        cb[0, :100, 0] = 3e38
        cb[0, 100:200, 0] = -3e38
        qb = np.zeros((1, 2, 128), np.float32)
        qb[0, :, 0] = 10.0
        qb[0, 1, 1:] = rng.standard_normal(127)
        codes = rng.integers(0, c + 3, (1, 1, n)).astype(np.uint16)
        topk_case(qb, codes, cb, k)

    def test_decode_shape(self):
        # 32 sequences x 24 query heads over 8 key heads, 16384 uniform codes, C = 1024,
        # k = 10%: every row checked (qb = oracle's q R_b rounded to fp32)
        w = W["topk_decode"]
        cb = synth.codebook(w.cfg, w.heads, w.c)
        codes = synth.uniform_codes(w.cfg, (w.batch, w.heads, w.n), w.c)
        q = synth.queries(w.cfg, w.q_heads, w.batch).transpose(1, 0, 2)
        qb = oracle.rope_at(q.reshape(-1, 128).astype(np.float64), w.far_b)
        qb = qb.astype(np.float32).reshape(q.shape)
        topk_case(qb, codes, cb, int(np.ceil(w.fraction * w.n)))

    def test_after_far_query_rope(self):
        # the composed decode path: GPU far rotation of the raw query, then top-K; the
        # oracle's rotation agrees to one fp32 unit, so the picked sets agree up to near-ties
        w = W["topk_decode"]
        batch, n, c, k = 4, 4096, w.c, 400
        cb = synth.codebook(w.cfg, w.heads, c)
        codes = synth.uniform_codes(w.cfg, (batch, w.heads, n), c)
        q = np.ascontiguousarray(synth.queries(w.cfg, w.q_heads, batch).transpose(1, 0, 2))
        qb = kv.far_query_rope(torch.from_numpy(q).to(DEV), w.far_b)
        idx = kv.topk_codes(qb, u16_to_dev(codes), f32_to_dev(cb), k, want_scores=False).cpu().numpy()
        qr = oracle.rope_at(q.reshape(-1, 128).astype(np.float64), w.far_b).reshape(q.shape)
        g = w.q_heads // w.heads
        for b in range(batch):
            for h in range(w.q_heads):
                s = cb[h // g].astype(np.float64)[codes[b, h // g]] @ qr[b, h]
                kth = np.sort(s)[::-1][k - 1]
                slack = 1e-5 * np.abs(cb[h // g]).sum(1).max() * np.abs(qr[b, h]).max()
                assert np.all(s[idx[b, h]] >= kth - slack)
                assert np.all(np.diff(idx[b, h]) > 0)
