"""pkv_time_next_call and pkv_read_probe on the GPU.

Kernel-level timing: the events passed for the next device call take its
kernels' start and end (a positive span that covers the kernel), and the
setting is consumed by that call alone: a later call leaves the events as
they were.  The read probe runs in order and gathered through a permutation,
leaving the sink untouched for a zero-filled buffer.
"""

import numpy as np
import pytest

from paged_kv_cache_244_amd import _lib

pytestmark = pytest.mark.gpu


def test_time_next_call_spans_the_kernel_and_is_consumed():
    import torch

    print("\n[case] pkv_time_next_call on pkv_read_probe", flush=True)
    stream = torch.cuda.current_stream()
    tiles = 1 << 16                                # 256 MiB
    buf = torch.zeros(tiles * 4096, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    order = torch.from_numpy(np.random.default_rng(5).permutation(tiles).astype(np.int32)).cuda()
    timer = _lib.KernelTimer()
    torch.cuda.synchronize()
    for order_ptr in (None, order.data_ptr()):
        _lib.time_next_call(timer)
        assert _lib.lib().pkv_read_probe(buf.data_ptr(), tiles, order_ptr, sink.data_ptr(), 2048,
                                         stream.cuda_stream) == _lib.PKV_OK
        ms = timer.ms()
        # 256 MiB cannot be read in under ~20 us, nor should it take 100 ms
        assert 0.02 < ms < 100.0, ms
        # the setting was consumed: an untimed call leaves both events as they were
        _lib.lib().pkv_read_probe(buf.data_ptr(), tiles, order_ptr, sink.data_ptr(), 2048,
                                  stream.cuda_stream)
        torch.cuda.synchronize()
        assert timer.ms() == ms
    assert int(sink.item()) == 0
