"""Helpers shared by the GPU parity tests: device transfer and the comparison rules.

Comparison rules (the oracle is fp64; each bound covers the GPU path's own rounding):
  codes      bit-exact wherever the oracle's (d2 - d1) / d1 > 1e-5; the rest is the tie band
  distances  |gpu - d1| <= 1e-4 d1 + 1e-6 ||z||^2
  blend      bit-exact wherever the oracle's best-minus-second score > 1e-5
  split      equal sets except indices whose oracle cosine lies within 1e-5 of the cosine at
             the n_r-th place; both outputs ascending and together a cover of 0..n-1
  rotation   fp32: |gpu - ref| <= 1e-5 + 2^-21 (|x_i| + |x_partner|)
             bf16: |gpu - ref| <= 2e-2 |ref| + 2^-21 (|x_i| + |x_partner|)
             and both: bit-exact equality with the single nearest-even rounding of the
             oracle's fp64 value, except where that value lies within
             delta = (pmax 2^-51 + 2^-50)(|x_i| + |x_partner|) of a rounding midpoint (the two
             sides' fp64 angles p theta come from different pow / cos / sin implementations,
             each within an ulp or two of the exact function, for |p| <= pmax); there the GPU
             value must be one of the two values next to that midpoint
"""
import numpy as np
import torch

from kv_cache_vector_windowed_amd import synth

DEV = "cuda:0"


def keys_to_dev(k: synth.Keys) -> torch.Tensor:
    if k.dtype == "bf16":
        return torch.from_numpy(k.bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(k.values)).to(DEV)


def f32_to_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def u16_to_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(DEV).view(torch.uint16)


def u16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_np_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_codes(gpu, code, d1, d2, what=""):
    """Bit-exact outside the tie band; returns (tie rate, mismatches inside the band)."""
    gpu = np.asarray(gpu).astype(np.int64)
    code = np.asarray(code).astype(np.int64)
    gap = (d2 - d1) / np.maximum(d1, 1e-300)
    decided = gap > 1e-5
    bad = np.nonzero(decided & (gpu != code))[0]
    assert bad.size == 0, "%s: %d codes differ outside the tie band, e.g. rows %s gpu %s oracle %s" % (
        what, bad.size, bad[:5], gpu[bad[:5]], code[bad[:5]])
    return float((~decided).mean()), int(((~decided) & (gpu != code)).sum())


def check_dist(gpu, d1, z2, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    tol = 1e-4 * d1 + 1e-6 * z2
    err = np.abs(gpu - d1)
    worst = np.argmax(err - tol)
    assert np.all(err <= tol), "%s: dist error %g > tol %g at %d" % (what, err[worst], tol[worst], worst)
    return float((err / np.maximum(d1, 1e-300)).max())


def check_split(ret, bulk, n, cosv, oracle_ret, what=""):
    ret = np.asarray(ret).astype(np.int64)
    bulk = np.asarray(bulk).astype(np.int64)
    nr = len(oracle_ret)
    assert len(ret) == nr and len(bulk) == n - nr, what
    assert np.all(np.diff(ret) > 0) and np.all(np.diff(bulk) > 0), what + ": not ascending"
    assert np.array_equal(np.sort(np.concatenate([ret, bulk])), np.arange(n)), what + ": not a cover"
    if nr == 0 or nr == n:
        return 0
    thr = np.sort(cosv)[::-1][nr - 1]
    diff = np.setxor1d(ret, np.asarray(oracle_ret))
    outside = diff[np.abs(cosv[diff] - thr) > 1e-5]
    assert outside.size == 0, "%s: %d indices differ outside the tie band" % (what, outside.size)
    return int(diff.size)


def check_rounded_once(gpu, ref, mag, dtype, pmax=2 ** 18, what=""):
    """gpu: fp32 values (bf16 outputs widened, which is exact), ref: the oracle's fp64 values,
    mag: |x_i| + |x_partner| per element.  Returns the number of elements inside the band."""
    g32 = np.ascontiguousarray(gpu, dtype=np.float32)
    ref = np.asarray(ref, dtype=np.float64)
    nan_g, nan_r = np.isnan(g32), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), "%s: NaN rows differ" % what
    if dtype == "bf16":
        gb = synth.f32_to_bf16_bits(g32).astype(np.int64)
        assert np.array_equal(synth.bf16_bits_to_f32(gb.astype(np.uint16)).view(np.uint32),
                              g32.view(np.uint32)), "%s: not bf16 values" % what
        import oracle
        wb = oracle.round_bf16(np.where(nan_r, 0.0, ref)).astype(np.int64)
        wv = synth.bf16_bits_to_f32(wb.astype(np.uint16)).astype(np.float64)
    else:
        gb = g32.view(np.uint32).astype(np.int64)
        w32 = np.where(nan_r, 0.0, ref).astype(np.float32)  # nearest even
        wb = w32.view(np.uint32).astype(np.int64)
        wv = w32.astype(np.float64)
    bad = (gb != wb) & ~nan_r
    if not bad.any():
        return 0
    delta = (pmax * 2.0 ** -51 + 2.0 ** -50) * np.asarray(mag, np.float64)
    gv = g32.astype(np.float64)
    adjacent = (np.abs(gb - wb) == 1) & (np.signbit(gv) == np.signbit(wv))
    mid = 0.5 * (gv + wv)
    ok = adjacent & (np.abs(ref - mid) <= delta)
    worst = np.nonzero(bad & ~ok)[0] if bad.ndim == 1 else np.argwhere(bad & ~ok)
    assert np.all(ok[bad]), "%s: %d elements are not the single rounding of the oracle's value, " \
        "e.g. at %s: gpu %r oracle %r" % (what, int((bad & ~ok).sum()), worst[:3],
                                          gv[bad & ~ok][:3], ref[bad & ~ok][:3])
    return int(bad.sum())


def check_rotation(gpu, ref, src, dtype, what="", pmax=2 ** 18):
    """gpu: fp32 values (bf16 widened), ref: fp64 oracle, src: the fp64 pre-RoPE rows.  The
    tolerance rule, then the single-rounding rule (check_rounded_once)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    h = src.shape[-1] // 2
    partner = np.concatenate([src[..., h:], src[..., :h]], axis=-1)
    mag = np.abs(src) + np.abs(partner)
    if dtype == "f32":
        tol = 1e-5 + 2.0 ** -21 * mag
    else:
        tol = 2e-2 * np.abs(ref) + 2.0 ** -21 * mag
    nan = np.isnan(ref)
    err = np.where(nan, 0.0, np.abs(gpu - ref))
    ok = err <= tol
    assert np.all(ok), "%s: %d elements out of tolerance, max err %g" % (what, (~ok).sum(), err.max())
    check_rounded_once(gpu, ref, mag, dtype, pmax, what)
    return float(err.max()), int((err > 1e-5).sum())
