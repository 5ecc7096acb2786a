"""Helpers shared by the GPU parity tests: device transfer and the comparison rules.

Comparison rules (the oracle is fp64; each bound covers the GPU path's own rounding):
  codes      bit-exact wherever the oracle's (d2 - d1) / d1 > 1e-5; the rest is the tie band
  distances  |gpu - d1| <= 1e-4 d1 + 1e-6 ||z||^2
  blend      bit-exact wherever the oracle's best-minus-second score > 1e-5
  split      equal sets except indices whose oracle cosine lies within 1e-5 of the cosine at
             the n_r-th place; both outputs ascending and together a cover of 0..n-1
  rotation   fp32: |gpu - ref| <= 1e-5 + 2^-21 (|x_i| + |x_partner|)
             bf16: |gpu - ref| <= 2e-2 |ref| + 2^-21 (|x_i| + |x_partner|)
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


def check_rotation(gpu, ref, src, dtype, what=""):
    """gpu: fp32 values (bf16 widened), ref: fp64 oracle, src: the fp64 pre-RoPE rows."""
    gpu = np.asarray(gpu, dtype=np.float64)
    h = src.shape[-1] // 2
    partner = np.concatenate([src[..., h:], src[..., :h]], axis=-1)
    mag = np.abs(src) + np.abs(partner)
    if dtype == "f32":
        tol = 1e-5 + 2.0 ** -21 * mag
    else:
        tol = 2e-2 * np.abs(ref) + 2.0 ** -21 * mag
    err = np.abs(gpu - ref)
    ok = err <= tol
    assert np.all(ok), "%s: %d elements out of tolerance, max err %g" % (what, (~ok).sum(), err.max())
    return float(err.max()), int((err > 1e-5).sum())
