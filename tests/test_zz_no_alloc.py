"""GPU test of lp_fp8_cast_current_noalloc, the current-scaling entry point that allocates nothing
(its partial maxima live in a static device array): called through the C ABI, its codes and
descale equal lp_fp8_cast_current's (the workspace variant) bit for bit, on two calls in a row,
the second on a smaller input, so the array's contents from the first call cannot leak into the
second."""
import ctypes

import numpy as np
import pytest
import torch

import precision_attention_mxfp8_amd as lp
from precision_attention_mxfp8_amd import _lib

pytestmark = pytest.mark.gpu


def _both(x: torch.Tensor):
    lib = _lib.load()
    t, h, _ = x.shape
    dt = _lib.DTYPE_BF16 if x.dtype == torch.bfloat16 else _lib.DTYPE_FP32
    stream = torch.cuda.current_stream().cuda_stream
    work = torch.empty((257,), dtype=torch.float32, device=x.device)
    y_ref = torch.empty((t, h, 128), dtype=torch.uint8, device=x.device)
    s_ref = torch.empty((1, 1), dtype=torch.float32, device=x.device)
    rc = lib.lp_fp8_cast_current(x.data_ptr(), dt, x.stride(0), x.stride(1), t, h, 128, work.data_ptr(),
                                 y_ref.data_ptr(), s_ref.data_ptr(), stream)
    assert rc == 0, lib.lpfa_last_error()
    y = torch.full((t, h, 128), 0x55, dtype=torch.uint8, device=x.device)
    s = torch.full((1, 1), -1.0, dtype=torch.float32, device=x.device)
    rc = lib.lp_fp8_cast_current_noalloc(x.data_ptr(), dt, x.stride(0), x.stride(1), t, h, 128,
                                         y.data_ptr(), s.data_ptr(), stream)
    assert rc == 0, lib.lpfa_last_error()
    torch.cuda.synchronize()
    return y, s, y_ref, s_ref, work[0].item()


def test_noalloc_matches_workspace_entry_twice_shrinking():
    dev = torch.device("cuda")
    rng = np.random.default_rng(1300)
    # first call: large FP32 tensor (all 256 amax workgroups), its maximum planted near the end
    x1 = (rng.standard_normal((4099, 8, 128)) * 3.0).astype(np.float32)
    x1[4090, 5, 77] = -9000.0
    # second call: a small BF16 tensor whose maximum (12.5) is far below the first one's, handled by
    # fewer amax workgroups; a stale partial maximum from the first call would show in its descale
    x2 = (rng.standard_normal((37, 3, 128)) * 2.0).astype(np.float32)
    x2[5, 1, 3] = 12.5
    t1 = torch.from_numpy(x1).to(dev)
    t2 = torch.from_numpy(x2).to(dev).to(torch.bfloat16)
    y, s, y_ref, s_ref, amax = _both(t1)
    assert amax == 9000.0
    assert torch.equal(y, y_ref) and torch.equal(s, s_ref) and s.item() == np.float32(9000.0) / np.float32(448.0)
    y, s, y_ref, s_ref, amax = _both(t2)
    assert amax == 12.5
    assert torch.equal(y, y_ref) and torch.equal(s, s_ref) and s.item() == np.float32(12.5) / np.float32(448.0)
    # the Python binding of the same entry point, with caller-provided outputs
    out = torch.empty((37, 3, 128), dtype=torch.uint8, device=dev)
    d = torch.empty((1, 1), dtype=torch.float32, device=dev)
    lp.cast_e4m3_current_noalloc(t2, out, d)
    torch.cuda.synchronize()
    assert torch.equal(out, y_ref) and torch.equal(d, s_ref)


def test_noalloc_rejects_bad_arguments():
    lib = _lib.load()
    x = torch.zeros((4, 2, 128), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((4, 2, 128), dtype=torch.uint8, device="cuda")
    assert lib.lp_fp8_cast_current_noalloc(x.data_ptr(), 0, 256, 128, 4, 2, 128, y.data_ptr(), None, None) == _lib.LPFA_EINVAL
    assert lib.lp_fp8_cast_current_noalloc(x.data_ptr(), 0, 256, 128, 4, 2, 64, y.data_ptr(), y.data_ptr(), None) == _lib.LPFA_ENOTSUP
