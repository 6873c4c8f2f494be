"""The MFMA-only reference kernels bench.py times (libpkv_bench.so): each
must issue exactly iters x chains MFMAs of its shape per wave, or the FLOP
rate it reports would be for work it did not do.  With every operand 1/8
(exact in fp16) each accumulator element gains K/64 per MFMA (K the
contraction length), exactly, so a thread's sum of its accumulators is a
closed form: chains x elements x K/64 x iters = 16 x iters for both shapes
(8 chains x 4 elements x 32/64, 4 chains x 16 elements x 16/64)."""
import ctypes

import numpy as np
import pytest

import bench


def _fn():
    lib = ctypes.CDLL(bench.BENCH_LIB)
    fn = lib.pkvb_mfma_rate
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_float, ctypes.c_float, ctypes.c_void_p]
    return fn


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("blocks,iters", [(1, 1), (3, 7), (512, 1024)])
def test_mfma_rate_does_all_its_work(shape, blocks, iters):
    import torch
    out = torch.full((blocks * 256,), -1.0, dtype=torch.float32, device="cuda:0")
    print(f"mfma rate: shape {shape} blocks {blocks} iters {iters}", flush=True)
    rc = _fn()(out.data_ptr(), shape, blocks, iters, 0.125, 0.125, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    np.testing.assert_array_equal(out.cpu().numpy(), np.full(blocks * 256, 16.0 * iters, np.float32))


@pytest.mark.gpu
def test_mfma_rate_rejects_bad_arguments():
    import torch
    out = torch.zeros(256, dtype=torch.float32, device="cuda:0")
    fn = _fn()
    s = torch.cuda.current_stream().cuda_stream
    assert fn(out.data_ptr(), 2, 1, 1, 0.125, 0.125, s) != 0     # no such shape
    assert fn(out.data_ptr(), 0, 0, 1, 0.125, 0.125, s) != 0     # no workgroups
    assert fn(out.data_ptr(), 0, 1, 0, 0.125, 0.125, s) != 0     # no iterations
    assert fn(None, 0, 1, 1, 0.125, 0.125, s) != 0
