"""The streaming-read reference kernel bench.py times (libpkv_bench.so):
it must read every 16-byte chunk of the buffer, or the bandwidth it reports
would be for fewer bytes than it claims."""
import ctypes

import numpy as np
import pytest

import bench

MAGIC = 0x9E3779B9


def _fn():
    lib = ctypes.CDLL(bench.BENCH_LIB)
    fn = lib.pkvb_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_void_p]
    return fn


@pytest.mark.gpu
@pytest.mark.parametrize("chunks,grid,at", [(1, 1, 0), (2, 1, 1), (3, 1, 2), (4096, 8, 4095),
                                            (4096, 8, 1234), (1 << 20, 2048, (1 << 20) - 1),
                                            (1 << 20, 2048, 524287), (1 << 20, 2048, 524288),
                                            (1000003, 4096, 999999), (1000003, 4096, 1000002),
                                            (1000003, 4096, 500001)])
def test_stream_read_reaches_every_chunk(chunks, grid, at):
    """A zero buffer with the kernel's magic word planted in one chunk: the
    one thread that reads it writes the sink, wherever the chunk sits (either
    half, body of the unrolled loop or its tail, the odd last chunk)."""
    import torch
    dev = torch.device("cuda:0")
    words = np.zeros(chunks * 4, dtype=np.uint32)
    words[4 * at + 2] = MAGIC
    buf = torch.from_numpy(words.view(np.int32)).to(dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    print(f"stream read: chunks {chunks} grid {grid} magic at {at}", flush=True)
    rc = _fn()(buf.data_ptr(), chunks * 16, sink.data_ptr(), grid,
               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == MAGIC


@pytest.mark.gpu
def test_stream_read_rejects_bad_arguments():
    import torch
    buf = torch.zeros(64, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    fn = _fn()
    s = torch.cuda.current_stream().cuda_stream
    assert fn(buf.data_ptr(), 17, sink.data_ptr(), 1, s) != 0       # not a multiple of 16
    assert fn(buf.data_ptr() + 4, 64, sink.data_ptr(), 1, s) != 0   # misaligned
    assert fn(buf.data_ptr(), 64, sink.data_ptr(), 0, s) != 0       # no workgroups
    assert fn(None, 64, sink.data_ptr(), 1, s) != 0
