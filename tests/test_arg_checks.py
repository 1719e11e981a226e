"""kv_swap_blocks, pkv_upload_write, pkv_read_probe, pkv_check_tables and
pkv_wave_timeline_read argument checks that need no GPU.

Every call here is refused (or is a no-op) before the library touches the HIP
runtime: bad sizes, geometry that is not built, nothing to copy, NULL pools and
too many pairs.  The copies themselves are checked on the GPU
(tests/test_gpu_swap.py).
"""

import ctypes

import numpy as np

from paged_kv_cache_244_amd import _lib


def _arr(*ptrs):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def _call(dst_blocks=4, src_blocks=4, layers=1, pairs=1, hkv=2, d=64, bs=16, pools=None, pair_ptr=8):
    pools = pools if pools is not None else [_arr(16)] * 4
    return _lib.lib().kv_swap_blocks(pools[0], pools[1], dst_blocks, pools[2], pools[3], src_blocks,
                                     layers, pair_ptr, pairs, hkv, d, bs, None)


def test_sizes_and_geometry_are_checked_first():
    assert _call(dst_blocks=0) == _lib.PKV_ERR_INVALID_ARG
    assert _call(src_blocks=-1) == _lib.PKV_ERR_INVALID_ARG
    assert _call(layers=-1) == _lib.PKV_ERR_INVALID_ARG
    assert _call(pairs=-1) == _lib.PKV_ERR_INVALID_ARG
    assert _call(hkv=0) == _lib.PKV_ERR_INVALID_ARG
    assert _call(d=96) == _lib.PKV_ERR_UNSUPPORTED
    assert _call(bs=12) == _lib.PKV_ERR_UNSUPPORTED


def test_nothing_to_copy_is_a_no_op():
    assert _call(pairs=0, pools=[None] * 4, pair_ptr=None) == _lib.PKV_OK
    assert _call(layers=0, pools=[None] * 4, pair_ptr=None) == _lib.PKV_OK


def test_null_pointers_and_too_many_pairs():
    assert _call(pools=[None, _arr(16), _arr(16), _arr(16)]) == _lib.PKV_ERR_INVALID_ARG
    assert _call(pair_ptr=None) == _lib.PKV_ERR_INVALID_ARG
    assert _call(pairs=65536) == _lib.PKV_ERR_INVALID_ARG
    assert b"65535" in _lib.lib().pkv_last_error()


def test_upload_write_arguments_checked_before_any_launch():
    """pkv_upload_write refuses bad sizes, geometry and alignment, and does nothing
    when both parts are empty, without touching the HIP runtime."""
    lib = _lib.lib()

    def call(bytes_=0, ntok=0, nb=4, hkv=2, d=64, bs=16, dst=None, src=None):
        return lib.pkv_upload_write(dst, src, bytes_, None, None, nb, None, None, None, ntok, hkv,
                                    d, bs, None)

    assert call() == _lib.PKV_OK
    assert call(ntok=-1) == _lib.PKV_ERR_INVALID_ARG
    assert call(nb=0) == _lib.PKV_ERR_INVALID_ARG
    assert call(d=96) == _lib.PKV_ERR_UNSUPPORTED
    assert call(bs=24) == _lib.PKV_ERR_UNSUPPORTED
    assert call(bytes_=24, dst=16, src=16) == _lib.PKV_ERR_INVALID_ARG          # size % 16
    assert call(bytes_=32, dst=8, src=16) == _lib.PKV_ERR_INVALID_ARG           # alignment
    assert call(bytes_=32) == _lib.PKV_ERR_INVALID_ARG                          # NULL buffers
    assert call(ntok=4) == _lib.PKV_ERR_INVALID_ARG                             # NULL pools


def test_read_probe_arguments_checked_on_the_host():
    lib = _lib.lib()
    assert lib.pkv_read_probe(None, -1, None, None, 64, None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_read_probe(None, 4, None, None, 0, None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_read_probe(None, 4, None, None, 64, None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_read_probe(8, 4, None, None, 64, None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_read_probe(24, 4, None, 16, 64, None) == _lib.PKV_ERR_INVALID_ARG  # misaligned
    assert b"aligned" in lib.pkv_last_error()
    assert lib.pkv_read_probe(None, 0, None, None, 64, None) == _lib.PKV_OK           # nothing



def test_event_helpers_refuse_null():
    lib = _lib.lib()
    assert lib.pkv_event_create(None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_event_destroy(None) == _lib.PKV_OK
    import ctypes
    ms = ctypes.c_float()
    assert lib.pkv_event_elapsed_ms(None, None, ctypes.byref(ms)) == _lib.PKV_ERR_INVALID_ARG


def test_check_tables_arguments_checked_on_the_host():
    lib = _lib.lib()
    result = 4096   # never dereferenced: every call below fails its argument checks
    assert lib.pkv_check_tables(None, 4, None, 2, 16, 10, None, None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_check_tables(None, 4, None, -1, 16, 10, result, None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_check_tables(None, 4, None, 2, 0, 10, result, None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_check_tables(None, -1, None, 2, 16, 10, result, None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_check_tables(None, 4, 64, 2, 16, 10, result, None) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_check_tables(64, 4, None, 2, 16, -3, result, None) == _lib.PKV_ERR_INVALID_ARG


def test_wave_timeline_reader_in_the_product_library():
    """libpagedkv.so records no per-wave timeline: the reader says so without a
    device call; bad arguments are refused first."""
    lib = _lib.lib()
    buf = np.zeros(6, dtype=np.uint64)
    ptr = buf.ctypes.data
    assert lib.pkv_wave_timeline_read(3, ptr, buf.nbytes, 0) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_wave_timeline_read(-1, ptr, buf.nbytes, 0) == _lib.PKV_ERR_INVALID_ARG
    assert lib.pkv_wave_timeline_read(_lib.PKV_TIMELINE_VALU, None, 48, 0) == _lib.PKV_ERR_INVALID_ARG
    for kind in (_lib.PKV_TIMELINE_VALU, _lib.PKV_TIMELINE_MFMA, _lib.PKV_TIMELINE_PREFILL):
        assert lib.pkv_wave_timeline_read(kind, ptr, buf.nbytes, 1) == _lib.PKV_ERR_UNSUPPORTED
        assert b"timeline" in lib.pkv_last_error()
