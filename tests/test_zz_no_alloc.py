"""dp_grad_sqnorm_noalloc (the entry point that allocates nothing) through the
C ABI, against dp_grad_sqnorm with a caller-provided workspace."""

import ctypes

import numpy as np
import pytest
import torch

import gradient_reduce_zero_amd as grz
from gradient_reduce_zero_amd import _native as N

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _with_workspace(parts, max_norm):
    n = parts.numel()
    ws = torch.empty(max(grz.dp_grad_sqnorm_workspace(n) // 8, 1), dtype=torch.float64,
                     device=DEV)
    sq = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    sc = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    assert grz.lib().dp_grad_sqnorm(_ptr(parts), n, max_norm, _ptr(ws), _ptr(sq), _ptr(sc),
                                    _stream()) == N.GRZ_OK
    return sq, sc


def _no_alloc(parts, max_norm):
    sq = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    sc = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    assert grz.lib().dp_grad_sqnorm_noalloc(_ptr(parts), parts.numel(), max_norm, _ptr(sq),
                                            _ptr(sc), _stream()) == N.GRZ_OK
    return sq, sc


def _bits(t):
    return t.cpu().numpy().view(np.uint64 if t.dtype == torch.float64 else np.uint32)


def test_no_alloc_norm_equals_the_workspace_norm_on_two_calls_in_a_row():
    # Largest first, then smaller: the second call must not see the first's
    # scratch contents.  Sizes: two tree levels (4096 * 4097 + 3 pieces), one
    # level (7B one-rank plan: 1,645,121 pieces), and a single block (3000).
    g = torch.Generator(device=DEV).manual_seed(5)
    for npieces, max_norm in ((4096 * 4097 + 3, 1.0), (1_645_121, 30.0), (3000, 0.0)):
        parts = torch.rand(npieces, dtype=torch.float64, device=DEV, generator=g) * 1e-3
        want_sq, want_sc = _with_workspace(parts, max_norm)
        got_sq, got_sc = _no_alloc(parts, max_norm)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(got_sq), _bits(want_sq)), npieces
        assert np.array_equal(_bits(got_sc), _bits(want_sc)), npieces
        assert got_sq.item() > 0


def test_no_alloc_norm_refuses_a_tree_beyond_its_scratch():
    # 8191 * 4096 pieces need 8191 + 2 level sums: more than 65536 bytes.  The
    # call is refused on the host before anything is launched.
    sq = torch.zeros(1, dtype=torch.float64, device=DEV)
    parts = torch.zeros(1, dtype=torch.float64, device=DEV)
    n = 8191 * 4096
    assert grz.dp_grad_sqnorm_workspace(n) > N.GRZ_NOALLOC_SCRATCH_BYTES
    assert grz.lib().dp_grad_sqnorm_noalloc(_ptr(parts), n, 1.0, _ptr(sq), None,
                                            _stream()) == N.GRZ_ERANGE
    assert grz.lib().dp_grad_sqnorm_noalloc(_ptr(parts), -1, 1.0, _ptr(sq), None,
                                            _stream()) == N.GRZ_EINVAL
    assert grz.dp_grad_sqnorm_workspace(8190 * 4096) <= N.GRZ_NOALLOC_SCRATCH_BYTES
