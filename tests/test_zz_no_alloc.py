"""The allocation-free reconstruct, a2ats_reconstruct_noalloc, called through the C ABI and
compared bit for bit with a2ats_reconstruct (the existing entry point with a caller
workspace) on two calls in a row, the second with a smaller input: the fixed table keeps the
first call's rows beyond the second call's, which the second call must not read."""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_vector_windowed_amd as kv
from parity import DEV, f32_to_dev, u16_to_dev

pytestmark = pytest.mark.gpu


def noalloc(codes, pos, cb, cur, window, far_b, far_mode, out):
    batch, heads, n = codes.shape
    return kv.lib().a2ats_reconstruct_noalloc(
        ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(pos.data_ptr()), batch, heads, n, 128,
        ctypes.c_void_p(cb.data_ptr()), cb.shape[1], cur, window, far_b, far_mode, 10000.0,
        ctypes.c_void_p(out.data_ptr()), 0 if out.dtype == torch.float32 else 1,
        ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))


def inputs(seed, batch, heads, n, c):
    rng = np.random.default_rng(seed)
    cb = f32_to_dev((rng.standard_normal((heads, c, 128)) * 2).astype(np.float32))
    codes = u16_to_dev(rng.integers(0, c, (batch, heads, n)).astype(np.uint16))
    pos = torch.from_numpy(np.tile(np.arange(n, dtype=np.int32), (batch, 1))).to(DEV)
    return codes, pos, cb


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_equals_reconstruct_on_two_calls(out_dtype):
    bits = torch.int32 if out_dtype == torch.float32 else torch.int16
    rows = kv.NOALLOC_TABLE_ROWS
    # (batch, heads, n, c, cur, window, far mode): the first call fills the whole table
    # (rows - 1 near rows and the far row), the second is smaller in every dimension
    cases = [(2, 3, rows + 500, 300, rows + 499, rows - 1, kv.FAR_FIXED_OFFSET),
             (1, 2, 1200, 90, 1199, 64, kv.FAR_UNROTATED)]
    for i, (batch, heads, n, c, cur, win, mode) in enumerate(cases):
        codes, pos, cb = inputs(40 + i, batch, heads, n, c)
        out = torch.full((batch, heads, n, 128), 7.0, dtype=out_dtype, device=DEV)
        assert noalloc(codes, pos, cb, cur, win, 2048, mode, out) == 0
        ref = kv.reconstruct(codes, pos, cb, cur, win, far_offset=2048, far_mode=mode,
                             out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(out.view(bits), ref.view(bits)), "call %d" % i


def test_noalloc_rejects_a_window_beyond_the_table():
    codes, pos, cb = inputs(50, 1, 1, 100, 10)
    out = torch.empty((1, 1, 100, 128), dtype=torch.float32, device=DEV)
    rows = kv.NOALLOC_TABLE_ROWS
    assert noalloc(codes, pos, cb, 10 ** 6, rows, 2048, 0, out) == -6
    assert noalloc(codes, pos, cb, 10 ** 6, rows - 1, 2048, 0, out) == 0
    torch.cuda.synchronize()
